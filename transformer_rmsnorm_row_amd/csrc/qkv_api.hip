// C ABI of the fused attention-input library: plan management, argument
// validation and kernel selection.  Declarations and the contract of every entry
// point are in include/qkv.h.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <unordered_set>

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include "qkv.h"
#include "launch.h"
#include "backward.h"
#include "prefill_pre.h"
#include "unfused.h"

// Device scratch of qkv_forward_noalloc (layout and size next to that entry point).
constexpr size_t kNoAllocScratchBytes = 4096 + (size_t)256 * (128 * 128 + 128) * sizeof(float);
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr uint64_t kPlanMagic = 0x514b564d49333535ull;  // "QKVMI355"

struct Plan {
  uint64_t magic;
  qkv_plan_desc desc;
  int device;
  int N, Nq, Nkv;
  bool bf16;
  bool prefill_ok;
  bool decode_ok;   // shape supported by the decode kernel (for T <= its token capacity)
  float* inv_rms;     // [max_tokens]
  double* rev_freq;   // [head_dim/2]
  float* partials;    // decode partial sums
  uint32_t* counters; // decode arrival counters
  float* kpart;       // split-K prefill: partial tiles
  uint32_t* kcount;   // split-K prefill: per-tile arrival counters
  int kpart_units;    // partial tiles kpart holds
  void* xw;           // QKV_PLAN_PREFILL_PREPASS: bf16(x * w_norm) from the pre-pass, max_tokens rounded up to 256 rows
  // backward scratch, allocated by the first qkv_backward through the plan
  void* bwd_gy;         // [max_tokens, N] plan dtype
  void* bwd_ga;         // [max_tokens, H] plan dtype
  float* bwd_partial;   // [kBackwardPartials, H] fp32
  rocblas_handle blas;  // the unfused forward's GEMM (created on its first call)
};

std::mutex g_mu;
std::unordered_set<const void*> g_live;

bool is_live(const void* p) {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_live.count(p) != 0;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxBytes = (int64_t)1 << 31;  // 32-bit byte offsets in every kernel

qkv_status check_desc(const qkv_plan_desc* d) {
  if (!d) return QKV_ERR_INVALID_ARG;
  if (d->max_tokens < 1) return QKV_ERR_INVALID_ARG;
  if (d->hidden < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 2) return QKV_ERR_INVALID_ARG;
  if (d->head_dim % 2 != 0) return QKV_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return QKV_ERR_INVALID_ARG;
  if (d->dtype != QKV_F32 && d->dtype != QKV_BF16) return QKV_ERR_INVALID_ARG;
  if (d->has_bias != 0 && d->has_bias != 1) return QKV_ERR_INVALID_ARG;
  if (!std::isfinite(d->eps) || d->eps < 0.0) return QKV_ERR_INVALID_ARG;
  if (!std::isfinite(d->rope_theta) || d->rope_theta <= 0.0) return QKV_ERR_INVALID_ARG;
  if ((d->flags & ~QKV_PLAN_PREFILL_PREPASS) != 0) return QKV_ERR_INVALID_ARG;
  if (d->hidden % 8 != 0) return QKV_ERR_UNSUPPORTED;
  if (d->head_dim % 8 != 0) return QKV_ERR_UNSUPPORTED;
  const int64_t elem = d->dtype == QKV_BF16 ? 2 : 4;
  const int64_t N = (int64_t)(d->num_q_heads + 2 * (int64_t)d->num_kv_heads) * d->head_dim;
  if (N >= kMaxBytes) return QKV_ERR_UNSUPPORTED;
  const int64_t widest = N > d->hidden ? N : d->hidden;
  if (d->max_tokens >= kMaxBytes / (widest * elem)) return QKV_ERR_UNSUPPORTED;
  if ((int64_t)d->hidden * N * elem >= kMaxBytes) return QKV_ERR_UNSUPPORTED;
  // The pre-pass buffer holds bf16 rows padded to whole 256-row panels.
  if ((d->flags & QKV_PLAN_PREFILL_PREPASS) != 0 &&
      (d->max_tokens + 255) / 256 * 256 * (int64_t)d->hidden * 2 >= kMaxBytes)
    return QKV_ERR_UNSUPPORTED;
  return QKV_OK;
}

Plan* as_plan(qkv_plan p) {
  if (!p || !is_live(p)) return nullptr;
  Plan* pl = reinterpret_cast<Plan*>(p);
  return pl->magic == kPlanMagic ? pl : nullptr;
}

qkv_status check_device(const Plan* pl) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QKV_ERR_HIP;
  return dev == pl->device ? QKV_OK : QKV_ERR_INVALID_ARG;
}

void free_scratch(Plan* pl) {
  if (pl->inv_rms) (void)hipFree(pl->inv_rms);
  if (pl->rev_freq) (void)hipFree(pl->rev_freq);
  if (pl->partials) (void)hipFree(pl->partials);
  if (pl->counters) (void)hipFree(pl->counters);
  if (pl->kpart) (void)hipFree(pl->kpart);
  if (pl->kcount) (void)hipFree(pl->kcount);
  if (pl->xw) (void)hipFree(pl->xw);
  if (pl->bwd_gy) (void)hipFree(pl->bwd_gy);
  if (pl->bwd_ga) (void)hipFree(pl->bwd_ga);
  if (pl->bwd_partial) (void)hipFree(pl->bwd_partial);
  if (pl->blas) (void)rocblas_destroy_handle(pl->blas);
  pl->inv_rms = nullptr;
  pl->rev_freq = nullptr;
  pl->partials = nullptr;
  pl->counters = nullptr;
  pl->kpart = nullptr;
  pl->xw = nullptr;
  pl->kcount = nullptr;
  pl->bwd_gy = nullptr;
  pl->bwd_ga = pl->bwd_partial = nullptr;
  pl->blas = nullptr;
}

// The GEMM library handle, created on the first call that needs it.
qkv_status ensure_blas_locked(Plan* pl) {
  if (pl->blas) return QKV_OK;
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success) return QKV_ERR_HIP;
  pl->blas = h;
  return QKV_OK;
}

qkv_status ensure_blas(Plan* pl) {
  std::lock_guard<std::mutex> lk(g_mu);
  return ensure_blas_locked(pl);
}

// First backward through a plan: its scratch.
qkv_status ensure_backward_scratch(Plan* pl) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (pl->bwd_partial) return QKV_OK;
  const size_t T = (size_t)pl->desc.max_tokens, H = (size_t)pl->desc.hidden, N = (size_t)pl->N;
  const size_t elem = pl->bf16 ? 2 : 4;
  // each buffer is allocated once: a call after a failed allocation keeps what succeeded
  const size_t tp = (size_t)qkv::backward_token_pitch((int)T);
  bool ok = (pl->bwd_gy || hipMalloc(&pl->bwd_gy, tp * N * elem) == hipSuccess) &&
            (pl->bwd_ga || hipMalloc(&pl->bwd_ga, T * H * elem) == hipSuccess) &&
            hipMalloc(&pl->bwd_partial, (size_t)qkv::kBackwardPartials * H * sizeof(float)) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    return QKV_ERR_OUT_OF_MEMORY;
  }
  return QKV_OK;
}

// Token counts the decode kernel takes, run over consecutive chunks of kDecodeTokens.
// The prefill kernel's few 256 x 256 tiles leave most compute units idle at these
// sizes, each walking the whole hidden dimension.  Its split-K form doubles the
// workgroups, and on the GQA decode shape it overtakes two decode launches once the
// second launch needs the 128-token form (193+ tokens); without a split form the decode
// kernel keeps up to two full 128-token launches.
constexpr int64_t kDecodeMaxTokens = qkv::kDecodeTokens + 64;
constexpr int64_t kDecodeMaxTokensUnsplit = 2 * qkv::kDecodeTokens;

int choose_variant(const Plan* pl, int64_t T) {
  const bool split = pl->bf16 && pl->prefill_ok && pl->kpart &&
                     qkv::prefill_split_count((int)T, pl->desc.hidden, pl->N, pl->kpart_units) > 1;
  if (pl->bf16 && pl->decode_ok && T <= (split ? kDecodeMaxTokens : kDecodeMaxTokensUnsplit) &&
      qkv::decode_supports((int)std::min<int64_t>(T, qkv::kDecodeTokens), pl->desc.hidden, pl->N, pl->Nq, pl->Nkv,
                           pl->desc.head_dim))
    return QKV_VARIANT_DECODE;
  if (pl->bf16 && pl->prefill_ok) return split ? QKV_VARIANT_PREFILL_SPLIT : QKV_VARIANT_PREFILL;
  return QKV_VARIANT_GENERIC;
}

// Validation shared by both forward entry points, then the launch of the variant.
// k and v are dense [T, Nkv] outputs, or caches of cache_rows rows when slots is set.
qkv_status launch_forward(Plan* pl, int64_t num_tokens, const void* x, const void* w_norm, const void* w_qkv,
                          const void* bias, const int32_t* pos, void* q, void* k, void* v, const int32_t* slots,
                          int cache_rows, void* stream) {
  if (!x || !w_norm || !w_qkv || !pos || !q) return QKV_ERR_INVALID_ARG;
  if ((bias != nullptr) != (pl->desc.has_bias == 1)) return QKV_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w_norm, 16) || !aligned(w_qkv, 16) || !aligned(q, 16) || !aligned(pos, 4) ||
      (bias && !aligned(bias, 16)))
    return QKV_ERR_INVALID_ARG;
  qkv_status st = check_device(pl);
  if (st != QKV_OK) return st;

  qkv::ForwardArgs a{};
  a.x = x;
  a.w_norm = w_norm;
  a.w = w_qkv;
  a.bias = bias;
  a.pos = pos;
  a.q = q;
  a.k = k;
  a.v = v;
  a.inv_rms = pl->inv_rms;
  a.rev_freq = pl->rev_freq;
  a.partials = pl->partials;
  a.counters = pl->counters;
  a.kpart = pl->kpart;
  a.kcount = pl->kcount;
  a.kpart_units = pl->kpart_units;
  a.slots = slots;
  a.cache_rows = slots ? cache_rows : (int)num_tokens;
  a.T = (int)num_tokens;
  a.H = pl->desc.hidden;
  a.N = pl->N;
  a.Nq = pl->Nq;
  a.Nkv = pl->Nkv;
  a.d = pl->desc.head_dim;
  a.eps = (float)pl->desc.eps;
  a.bf16 = pl->bf16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  hipError_t e;
  switch (choose_variant(pl, num_tokens)) {
    case QKV_VARIANT_PREFILL:
      if (pl->xw) {
        // pre-pass form (QKV_PLAN_PREFILL_PREPASS): bf16(x * w_norm) and 1/rms per row
        // into plan scratch; the MFMA kernel then streams the activations like the weight
        e = qkv::launch_prenorm(x, w_norm, pl->xw, pl->inv_rms, a.T, a.H, a.eps, s);
        if (e != hipSuccess) break;
        a.x = pl->xw;
        a.prenormed = true;
        e = qkv::launch_prefill_pre(a, s);  // takes every shape of the plain prefill variant
      } else if (qkv::prefill_wide_supports(a.H, a.N, a.Nq, a.Nkv, a.d)) {
        e = qkv::launch_prefill_wide(a, s);  // one launch, normalise-on-load
      } else {
        e = qkv::launch_prefill(a, s);  // one launch, the 256 x 256 kernel's normalise-on-load form
      }
      break;
    case QKV_VARIANT_PREFILL_SPLIT:  // the launcher makes the same split choice
      e = qkv::launch_prefill(a, s);
      break;
    case QKV_VARIANT_DECODE: {
      // one launch per chunk of up to kDecodeTokens tokens, in order on the stream:
      // the launches share the plan's partial sums and arrival counters
      const int64_t elem = 2;  // bf16
      e = hipSuccess;
      for (int64_t t0 = 0; t0 < num_tokens && e == hipSuccess; t0 += qkv::kDecodeTokens) {
        qkv::ForwardArgs c = a;
        c.T = (int)std::min<int64_t>(qkv::kDecodeTokens, num_tokens - t0);
        c.x = static_cast<const char*>(x) + t0 * a.H * elem;
        c.pos = pos + t0;
        c.q = static_cast<char*>(q) + t0 * a.Nq * elem;
        if (slots) {
          c.slots = slots + t0;  // k and v are the caches, addressed by slot
        } else {
          c.k = static_cast<char*>(k) + t0 * a.Nkv * elem;
          c.v = static_cast<char*>(v) + t0 * a.Nkv * elem;
          c.cache_rows = c.T;
        }
        e = qkv::launch_decode(c, s);
      }
      break;
    }
    default:
      e = qkv::launch_generic(a, s);
      break;
  }
  return e == hipSuccess ? QKV_OK : QKV_ERR_HIP;
}

// ---- no-allocation forward: its scratch is a file-scope device array ----
//
// Layout of `scratch` (one copy per GPU, kept until the process ends):
//   [0, 2 KB)        rotary frequency table, up to 256 doubles (head_dim <= 512)
//   [2 KB, 3 KB)     decode arrival counters, one per 128-column head (up to 256)
//   [4 KB, end)      decode partial sums: at most 256 units of 128 tokens x 128 columns
//                    plus 128 sums of squares each (the decode kernel runs at most one unit
//                    per CU, so every supported shape fits)
constexpr size_t kNoAllocRevOffset = 0, kNoAllocRevMax = 256;
constexpr size_t kNoAllocCountOffset = 2048, kNoAllocMaxHeads = 256;
constexpr size_t kNoAllocPartOffset = 4096;
constexpr size_t kNoAllocPartFloats = 256 * (128 * 128 + 128);
constexpr size_t kNoAllocBytes = kNoAllocPartOffset + kNoAllocPartFloats * sizeof(float);
static_assert(kNoAllocRevOffset + kNoAllocRevMax * sizeof(double) <= kNoAllocCountOffset, "table fits");
static_assert(kNoAllocCountOffset + kNoAllocMaxHeads * sizeof(uint32_t) <= kNoAllocPartOffset, "counters fit");
static_assert(kNoAllocBytes == kNoAllocScratchBytes, "the array holds the layout");

struct RevTable {
  double rev[kNoAllocRevMax];
};

// One workgroup: writes the call's rotary table and zeroes the decode counters, in
// stream order before the forward's kernels (a kernel, not a memset, so the call can
// be captured into a graph).
__global__ __launch_bounds__(256) void noalloc_setup_kernel(RevTable tbl, int half, uint8_t* base) {
  double* rev = reinterpret_cast<double*>(base + kNoAllocRevOffset);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(base + kNoAllocCountOffset);
  const int i = (int)threadIdx.x;
  if (i < half) rev[i] = tbl.rev[i];
  if (i < (int)kNoAllocMaxHeads) cnt[i] = 0u;
}

constexpr int kNoAllocMaxDevices = 64;
std::mutex g_noalloc_mu;
uint8_t* g_noalloc_ptr[kNoAllocMaxDevices];

// The device address of `scratch` on device `dev` (current), looked up once per device.
// In host code the array's name is only a handle for the runtime, never an address.
qkv_status noalloc_scratch(int dev, uint8_t** out) {
  if (dev < 0 || dev >= kNoAllocMaxDevices) return QKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return QKV_ERR_HIP;
    }
    g_noalloc_ptr[dev] = static_cast<uint8_t*>(p);
    (void)qkv::persistent_grid(1);  // the persistent kernels' CU count, once per device
  }
  *out = g_noalloc_ptr[dev];
  return QKV_OK;
}

}  // namespace

extern "C" {

qkv_status qkv_plan_create(const qkv_plan_desc* desc, qkv_plan* out_plan) {
  if (!out_plan) return QKV_ERR_INVALID_ARG;
  *out_plan = nullptr;
  qkv_status st = check_desc(desc);
  if (st != QKV_OK) return st;

  Plan* pl = new (std::nothrow) Plan();
  if (!pl) return QKV_ERR_OUT_OF_MEMORY;
  std::memset(pl, 0, sizeof(*pl));
  pl->magic = kPlanMagic;
  pl->desc = *desc;
  pl->Nq = desc->num_q_heads * desc->head_dim;
  pl->Nkv = desc->num_kv_heads * desc->head_dim;
  pl->N = pl->Nq + 2 * pl->Nkv;
  pl->bf16 = desc->dtype == QKV_BF16;
  pl->prefill_ok = pl->bf16 && qkv::prefill_supports(desc->hidden, pl->N, pl->Nq, pl->Nkv, desc->head_dim);
  pl->decode_ok = pl->bf16 && qkv::decode_supports(1, desc->hidden, pl->N, pl->Nq, pl->Nkv, desc->head_dim);

  if (hipGetDevice(&pl->device) != hipSuccess) {
    delete pl;
    return QKV_ERR_HIP;
  }
  // the persistent kernels' CU count, looked up here once per device, outside any graph
  // capture a later forward may run under
  (void)qkv::persistent_grid(1);
  const int half = desc->head_dim / 2;
  bool ok = hipMalloc(&pl->inv_rms, sizeof(float) * (size_t)desc->max_tokens) == hipSuccess &&
            hipMalloc(&pl->rev_freq, sizeof(double) * (size_t)half) == hipSuccess;
  if (ok && pl->decode_ok) {
    // per-head partial sums of the decode kernel and its arrival counters (zeroed once;
    // the kernel leaves them at zero after every forward)
    const size_t nheads = (size_t)pl->N / 128;
    ok = hipMalloc(&pl->partials, sizeof(float) * qkv::decode_scratch_floats(desc->hidden, pl->N)) == hipSuccess &&
         hipMalloc(&pl->counters, sizeof(uint32_t) * nheads) == hipSuccess &&
         hipMemset(pl->counters, 0, sizeof(uint32_t) * nheads) == hipSuccess &&
         hipDeviceSynchronize() == hipSuccess;
  }
  if (ok && pl->prefill_ok) {
    // partial tiles of the split-K prefill form (used when the tiles alone would leave
    // most CUs idle) and one arrival counter per tile (zeroed once; the kernel leaves
    // them at zero after every forward)
    pl->kpart_units = qkv::prefill_split_units((int)desc->max_tokens, pl->N);
    ok = ((desc->flags & QKV_PLAN_PREFILL_PREPASS) == 0 ||
          hipMalloc(&pl->xw, (size_t)(desc->max_tokens + 255) / 256 * 256 * desc->hidden * 2) == hipSuccess) &&
         hipMalloc(&pl->kpart, sizeof(float) * qkv::prefill_split_floats(pl->kpart_units)) == hipSuccess &&
         hipMalloc(&pl->kcount, sizeof(uint32_t) * qkv::kPrefillSplitMaxTiles) == hipSuccess &&
         hipMemset(pl->kcount, 0, sizeof(uint32_t) * qkv::kPrefillSplitMaxTiles) == hipSuccess &&
         hipDeviceSynchronize() == hipSuccess;
  }
  if (!ok) {
    free_scratch(pl);
    delete pl;
    (void)hipGetLastError();
    return QKV_ERR_OUT_OF_MEMORY;
  }
  // Rotary frequencies theta^(-2i/d), stored in revolutions per position so the
  // kernels can reduce the angle exactly with a rounding of the turn count.
  double host_rev[1024];
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < half && i < 1024; ++i)
    host_rev[i] = std::pow(desc->rope_theta, -2.0 * (double)i / (double)desc->head_dim) / two_pi;
  if (half > 1024 ||
      hipMemcpy(pl->rev_freq, host_rev, sizeof(double) * (size_t)half, hipMemcpyHostToDevice) != hipSuccess) {
    free_scratch(pl);
    delete pl;
    return half > 1024 ? QKV_ERR_UNSUPPORTED : QKV_ERR_HIP;
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.insert(pl);
  }
  *out_plan = reinterpret_cast<qkv_plan>(pl);
  return QKV_OK;
}

qkv_status qkv_plan_variant(qkv_plan plan, int64_t num_tokens, int32_t* variant) {
  Plan* pl = as_plan(plan);
  if (!pl || !variant || num_tokens < 1 || num_tokens > pl->desc.max_tokens) return QKV_ERR_INVALID_ARG;
  *variant = choose_variant(pl, num_tokens);
  return QKV_OK;
}

qkv_status qkv_forward(qkv_plan plan, int64_t num_tokens, const void* x, const void* w_norm, const void* w_qkv,
                       const void* bias, const int32_t* pos, void* q, void* k, void* v, void* stream) {
  Plan* pl = as_plan(plan);
  if (!pl) return QKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return QKV_OK;
  if (num_tokens < 0 || num_tokens > pl->desc.max_tokens) return QKV_ERR_INVALID_ARG;
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16)) return QKV_ERR_INVALID_ARG;
  return launch_forward(pl, num_tokens, x, w_norm, w_qkv, bias, pos, q, k, v, nullptr, 0, stream);
}

qkv_status qkv_forward_kv_cache(qkv_plan plan, int64_t num_tokens, const void* x, const void* w_norm,
                                const void* w_qkv, const void* bias, const int32_t* pos, const int32_t* slots,
                                int64_t cache_rows, void* q, void* k_cache, void* v_cache, void* stream) {
  Plan* pl = as_plan(plan);
  if (!pl) return QKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return QKV_OK;
  if (num_tokens < 0 || num_tokens > pl->desc.max_tokens) return QKV_ERR_INVALID_ARG;
  if (!slots || !aligned(slots, 4) || cache_rows < 1) return QKV_ERR_INVALID_ARG;
  if (!k_cache || !v_cache || !aligned(k_cache, 16) || !aligned(v_cache, 16)) return QKV_ERR_INVALID_ARG;
  const int64_t elem = pl->bf16 ? 2 : 4;
  if (cache_rows >= kMaxBytes / ((int64_t)pl->Nkv * elem)) return QKV_ERR_UNSUPPORTED;
  return launch_forward(pl, num_tokens, x, w_norm, w_qkv, bias, pos, q, k_cache, v_cache, slots, (int)cache_rows,
                        stream);
}

qkv_status qkv_forward_noalloc(const qkv_plan_desc* desc, int64_t num_tokens, const void* x, const void* w_norm,
                               const void* w_qkv, const void* bias, const int32_t* pos, void* q, void* k, void* v,
                               void* stream) {
  qkv_status st = check_desc(desc);
  if (st != QKV_OK) return st;
  if (desc->flags != 0) return QKV_ERR_UNSUPPORTED;  // the pre-pass form needs plan scratch
  if (num_tokens == 0) return QKV_OK;
  if (num_tokens < 0 || num_tokens > desc->max_tokens) return QKV_ERR_INVALID_ARG;
  if (!x || !w_norm || !w_qkv || !pos || !q || !k || !v) return QKV_ERR_INVALID_ARG;
  if ((bias != nullptr) != (desc->has_bias == 1)) return QKV_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w_norm, 16) || !aligned(w_qkv, 16) || !aligned(q, 16) || !aligned(k, 16) ||
      !aligned(v, 16) || !aligned(pos, 4) || (bias && !aligned(bias, 16)))
    return QKV_ERR_INVALID_ARG;
  const int half = desc->head_dim / 2;
  if ((size_t)half > kNoAllocRevMax) return QKV_ERR_UNSUPPORTED;  // table larger than its slot
  const int Nq = desc->num_q_heads * desc->head_dim, Nkv = desc->num_kv_heads * desc->head_dim;
  const int N = Nq + 2 * Nkv, H = desc->hidden, d = desc->head_dim;
  const bool bf16 = desc->dtype == QKV_BF16;
  const int64_t T = num_tokens;
  // Kernel choice as for a plan without the split-K prefill form (whose partial tiles
  // would not fit): the decode kernel up to two launches of 128 tokens when its partial
  // sums fit the array, else the single-launch normalise-on-load prefill kernel, else
  // the generic kernel.
  const bool decode_fits = bf16 && qkv::decode_supports(1, H, N, Nq, Nkv, d) && (size_t)(N / 128) <= kNoAllocMaxHeads &&
                           qkv::decode_scratch_floats(H, N) <= kNoAllocPartFloats;
  int variant = QKV_VARIANT_GENERIC;
  if (decode_fits && T <= kDecodeMaxTokensUnsplit &&
      qkv::decode_supports((int)std::min<int64_t>(T, qkv::kDecodeTokens), H, N, Nq, Nkv, d))
    variant = QKV_VARIANT_DECODE;
  else if (bf16 && qkv::prefill_supports(H, N, Nq, Nkv, d))
    variant = QKV_VARIANT_PREFILL;
  if (variant == QKV_VARIANT_DECODE && qkv::decode_scratch_floats(H, N) > kNoAllocPartFloats)
    return QKV_ERR_UNSUPPORTED;  // never reached for supported shapes; kept as the size guard

  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QKV_ERR_HIP;
  uint8_t* base = nullptr;
  st = noalloc_scratch(dev, &base);
  if (st != QKV_OK) return st;

  RevTable tbl{};
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < half; ++i) tbl.rev[i] = std::pow(desc->rope_theta, -2.0 * (double)i / (double)d) / two_pi;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  noalloc_setup_kernel<<<dim3(1), dim3(256), 0, s>>>(tbl, half, base);
  if (hipGetLastError() != hipSuccess) return QKV_ERR_HIP;

  qkv::ForwardArgs a{};
  a.x = x;
  a.w_norm = w_norm;
  a.w = w_qkv;
  a.bias = bias;
  a.pos = pos;
  a.q = q;
  a.k = k;
  a.v = v;
  a.rev_freq = reinterpret_cast<const double*>(base + kNoAllocRevOffset);
  a.counters = reinterpret_cast<uint32_t*>(base + kNoAllocCountOffset);
  a.partials = reinterpret_cast<float*>(base + kNoAllocPartOffset);
  a.cache_rows = (int)T;
  a.T = (int)T;
  a.H = H;
  a.N = N;
  a.Nq = Nq;
  a.Nkv = Nkv;
  a.d = d;
  a.eps = (float)desc->eps;
  a.bf16 = bf16;
  hipError_t e = hipSuccess;
  if (variant == QKV_VARIANT_DECODE) {
    const int64_t elem = 2;
    for (int64_t t0 = 0; t0 < T && e == hipSuccess; t0 += qkv::kDecodeTokens) {
      qkv::ForwardArgs c = a;
      c.T = (int)std::min<int64_t>(qkv::kDecodeTokens, T - t0);
      c.x = static_cast<const char*>(x) + t0 * H * elem;
      c.pos = pos + t0;
      c.q = static_cast<char*>(q) + t0 * Nq * elem;
      c.k = static_cast<char*>(k) + t0 * Nkv * elem;
      c.v = static_cast<char*>(v) + t0 * Nkv * elem;
      c.cache_rows = c.T;
      e = qkv::launch_decode(c, s);
    }
  } else if (variant == QKV_VARIANT_PREFILL) {
    // one launch: the plans' plain prefill kernel where the shape allows it, else the
    // 256 x 256 kernel's normalise-on-load form (no split-K scratch, no pre-pass)
    e = qkv::prefill_wide_supports(H, N, Nq, Nkv, d) ? qkv::launch_prefill_wide(a, s) : qkv::launch_prefill(a, s);
  } else {
    e = qkv::launch_generic(a, s);
  }
  return e == hipSuccess ? QKV_OK : QKV_ERR_HIP;
}

qkv_status qkv_rms_inv(qkv_plan plan, int64_t num_tokens, const void* x, float* inv_rms, void* stream) {
  Plan* pl = as_plan(plan);
  if (!pl) return QKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return QKV_OK;
  if (num_tokens < 0 || num_tokens > pl->desc.max_tokens) return QKV_ERR_INVALID_ARG;
  if (!x || !inv_rms || !aligned(x, 16) || !aligned(inv_rms, 4)) return QKV_ERR_INVALID_ARG;
  qkv_status st = check_device(pl);
  if (st != QKV_OK) return st;
  hipError_t e = qkv::launch_inv_rms(x, inv_rms, (int)num_tokens, pl->desc.hidden, (float)pl->desc.eps, pl->bf16,
                                     reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QKV_OK : QKV_ERR_HIP;
}

qkv_status qkv_rms_norm(qkv_plan plan, int64_t num_tokens, const void* x, const void* w_norm, void* xn,
                        void* stream) {
  Plan* pl = as_plan(plan);
  if (!pl) return QKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return QKV_OK;
  if (num_tokens < 0 || num_tokens > pl->desc.max_tokens) return QKV_ERR_INVALID_ARG;
  if (!x || !w_norm || !xn || !aligned(x, 16) || !aligned(w_norm, 16) || !aligned(xn, 16)) return QKV_ERR_INVALID_ARG;
  qkv_status st = check_device(pl);
  if (st != QKV_OK) return st;
  const hipError_t e = qkv::launch_rms_norm(x, w_norm, xn, (int)num_tokens, pl->desc.hidden, (float)pl->desc.eps,
                                            pl->bf16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QKV_OK : QKV_ERR_HIP;
}

qkv_status qkv_rope(qkv_plan plan, int64_t num_tokens, const void* bias, const int32_t* pos, void* y, void* stream) {
  Plan* pl = as_plan(plan);
  if (!pl) return QKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return QKV_OK;
  if (num_tokens < 0 || num_tokens > pl->desc.max_tokens) return QKV_ERR_INVALID_ARG;
  if ((bias != nullptr) != (pl->desc.has_bias == 1)) return QKV_ERR_INVALID_ARG;
  if (!pos || !y || !aligned(pos, 4) || !aligned(y, 16) || (bias && !aligned(bias, 16))) return QKV_ERR_INVALID_ARG;
  qkv_status st = check_device(pl);
  if (st != QKV_OK) return st;
  const hipError_t e = qkv::launch_rope(y, bias, pos, pl->rev_freq, (int)num_tokens, pl->N, pl->Nq, pl->Nkv,
                                        pl->desc.head_dim, pl->bf16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QKV_OK : QKV_ERR_HIP;
}

qkv_status qkv_head_norm_rope(qkv_plan plan, int64_t num_tokens, const void* w_qnorm, const void* w_knorm,
                              const int32_t* pos, void* y, void* stream) {
  Plan* pl = as_plan(plan);
  if (!pl) return QKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return QKV_OK;
  if (num_tokens < 0 || num_tokens > pl->desc.max_tokens) return QKV_ERR_INVALID_ARG;
  if (!w_qnorm || !w_knorm || !pos || !y || !aligned(w_qnorm, 16) || !aligned(w_knorm, 16) || !aligned(pos, 4) ||
      !aligned(y, 16))
    return QKV_ERR_INVALID_ARG;
  if (pl->desc.head_dim > 256) return QKV_ERR_UNSUPPORTED;
  qkv_status st = check_device(pl);
  if (st != QKV_OK) return st;
  const hipError_t e =
      qkv::launch_head_norm_rope(y, w_qnorm, w_knorm, pos, pl->rev_freq, (int)num_tokens, pl->N, pl->Nq, pl->Nkv,
                                 pl->desc.head_dim, (float)pl->desc.eps, pl->bf16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QKV_OK : QKV_ERR_HIP;
}

qkv_status qkv_forward_unfused(qkv_plan plan, int64_t num_tokens, const void* x, const void* w_norm,
                               const void* w_qkv, const void* bias, const int32_t* pos, void* xn, void* y,
                               void* stream) {
  Plan* pl = as_plan(plan);
  if (!pl) return QKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return QKV_OK;
  if (num_tokens < 0 || num_tokens > pl->desc.max_tokens) return QKV_ERR_INVALID_ARG;
  if ((bias != nullptr) != (pl->desc.has_bias == 1)) return QKV_ERR_INVALID_ARG;
  if (!x || !w_norm || !w_qkv || !pos || !xn || !y) return QKV_ERR_INVALID_ARG;
  for (const void* p : {x, w_norm, w_qkv, (const void*)xn, (const void*)y})
    if (!aligned(p, 16)) return QKV_ERR_INVALID_ARG;
  if (!aligned(pos, 4) || (bias && !aligned(bias, 16))) return QKV_ERR_INVALID_ARG;
  qkv_status st = check_device(pl);
  if (st != QKV_OK) return st;
  st = ensure_blas(pl);
  if (st != QKV_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int T = (int)num_tokens, H = pl->desc.hidden, N = pl->N;
  if (qkv::launch_rms_norm(x, w_norm, xn, T, H, (float)pl->desc.eps, pl->bf16, s) != hipSuccess) return QKV_ERR_HIP;
  // Row-major y [T, N] = xn [T, H] W [H, N]  <=>  column-major (N x T) = W (N x H) * xn (H x T),
  // fp32 accumulation, output in the plan dtype.
  if (rocblas_set_stream(pl->blas, s) != rocblas_status_success) return QKV_ERR_HIP;
  const rocblas_datatype io = pl->bf16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const float one = 1.0f, zero = 0.0f;
  if (rocblas_gemm_ex(pl->blas, rocblas_operation_none, rocblas_operation_none, N, T, H, &one, w_qkv, io, N, xn, io,
                      H, &zero, y, io, N, y, io, N, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                      0) != rocblas_status_success)
    return QKV_ERR_HIP;
  const hipError_t e =
      qkv::launch_rope(y, bias, pos, pl->rev_freq, T, N, pl->Nq, pl->Nkv, pl->desc.head_dim, pl->bf16, s);
  return e == hipSuccess ? QKV_OK : QKV_ERR_HIP;
}

qkv_status qkv_plan_destroy(qkv_plan plan) {
  if (!plan) return QKV_OK;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_live.erase(plan)) return QKV_ERR_INVALID_ARG;
  }
  Plan* pl = reinterpret_cast<Plan*>(plan);
  int prev = -1;
  bool switched = hipGetDevice(&prev) == hipSuccess && prev != pl->device && hipSetDevice(pl->device) == hipSuccess;
  (void)hipDeviceSynchronize();
  free_scratch(pl);
  if (switched) (void)hipSetDevice(prev);
  pl->magic = 0;
  delete pl;
  return QKV_OK;
}

qkv_status qkv_swiglu_forward(int64_t num_tokens, int32_t hidden, int32_t intermediate, int32_t dtype, double eps,
                              const void* x, const void* w_norm, const void* w_gate_up, void* out, void* stream) {
  if (num_tokens < 0 || hidden < 1 || intermediate < 1) return QKV_ERR_INVALID_ARG;
  if (dtype != QKV_F32 && dtype != QKV_BF16) return QKV_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.0) return QKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return QKV_OK;
  if (!x || !w_norm || !w_gate_up || !out) return QKV_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w_norm, 16) || !aligned(w_gate_up, 16) || !aligned(out, 16))
    return QKV_ERR_INVALID_ARG;
  if (dtype != QKV_BF16 || !qkv::swiglu_supports(hidden, intermediate)) return QKV_ERR_UNSUPPORTED;
  const int64_t H = hidden, I = intermediate;
  if (num_tokens * H * 2 >= kMaxBytes || H * 2 * I * 2 >= kMaxBytes || num_tokens * I * 2 >= kMaxBytes)
    return QKV_ERR_UNSUPPORTED;
  qkv::ForwardArgs a{};
  a.x = x;
  a.w_norm = w_norm;
  a.w = w_gate_up;
  a.q = out;
  a.T = (int)num_tokens;
  a.H = hidden;
  a.N = 2 * intermediate;
  a.Nq = intermediate;
  a.d = 128;
  a.eps = (float)eps;
  a.bf16 = true;
  const hipError_t e = qkv::launch_swiglu(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QKV_OK : QKV_ERR_HIP;
}

qkv_status qkv_backward(qkv_plan plan, int64_t num_tokens, const void* x, const void* w_norm, const void* w_qkv,
                        const int32_t* pos, const void* dq, const void* dk, const void* dv, void* dx, void* dw_norm,
                        void* dw_qkv, void* dbias, void* stream) {
  Plan* pl = as_plan(plan);
  if (!pl) return QKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return QKV_OK;
  if (num_tokens < 0 || num_tokens > pl->desc.max_tokens) return QKV_ERR_INVALID_ARG;
  if (!x || !w_norm || !w_qkv || !pos || !dq || !dk || !dv || !dx || !dw_norm || !dw_qkv)
    return QKV_ERR_INVALID_ARG;
  if ((dbias != nullptr) != (pl->desc.has_bias == 1)) return QKV_ERR_INVALID_ARG;
  for (const void* p : {x, w_norm, w_qkv, dq, dk, dv, (const void*)dx, (const void*)dw_norm, (const void*)dw_qkv})
    if (!aligned(p, 16)) return QKV_ERR_INVALID_ARG;
  if (!aligned(pos, 4) || (dbias && !aligned(dbias, 16))) return QKV_ERR_INVALID_ARG;
  // the transposed gradient [N, T rounded up to 32] is addressed with 32-bit byte offsets
  if ((int64_t)qkv::backward_token_pitch((int)num_tokens) * pl->N * (pl->bf16 ? 2 : 4) >= kMaxBytes)
    return QKV_ERR_UNSUPPORTED;
  qkv_status st = check_device(pl);
  if (st != QKV_OK) return st;
  st = ensure_backward_scratch(pl);
  if (st != QKV_OK) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  qkv::BackwardArgs b{};
  b.x = x;
  b.w_norm = w_norm;
  b.w = w_qkv;
  b.pos = pos;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.dx = dx;
  b.dw_norm = dw_norm;
  b.dbias = dbias;
  b.gy = pl->bwd_gy;
  b.ga = pl->bwd_ga;
  b.inv_rms = pl->inv_rms;
  b.partial = pl->bwd_partial;
  b.rev_freq = pl->rev_freq;
  b.T = (int)num_tokens;
  b.H = pl->desc.hidden;
  b.N = pl->N;
  b.Nq = pl->Nq;
  b.Nkv = pl->Nkv;
  b.d = pl->desc.head_dim;
  b.eps = (float)pl->desc.eps;
  b.bf16 = pl->bf16;
  if (qkv::launch_backward_pre_gemm(b, s) != hipSuccess) return QKV_ERR_HIP;

  // dW = diag(w_norm) x^T g straight into the caller's dw_qkv, G = g W^T into plan scratch
  if (qkv::launch_backward_gemms(b, dw_qkv, s) != hipSuccess) return QKV_ERR_HIP;
  return qkv::launch_backward_post_gemm(b, s) == hipSuccess ? QKV_OK : QKV_ERR_HIP;
}

const char* qkv_status_string(qkv_status status) {
  switch (status) {
    case QKV_OK: return "ok";
    case QKV_ERR_INVALID_ARG: return "invalid argument";
    case QKV_ERR_UNSUPPORTED: return "unsupported shape or configuration";
    case QKV_ERR_HIP: return "HIP runtime error";
    case QKV_ERR_OUT_OF_MEMORY: return "out of device memory";
  }
  return "unknown status";
}

const char* qkv_variant_name(int32_t variant) {
  switch (variant) {
    case QKV_VARIANT_GENERIC: return "generic";
    case QKV_VARIANT_PREFILL: return "prefill";
    case QKV_VARIANT_DECODE: return "decode";
    case QKV_VARIANT_PREFILL_SPLIT: return "prefill_split";
  }
  return "unknown";
}

}  // extern "C"
