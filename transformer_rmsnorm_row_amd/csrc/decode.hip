// Decode kernel for gfx950: the whole chain for a small batch of tokens (T <= 64,
// one new token per sequence), streaming the QKV weight from HBM exactly once.
//
// Same method as the prefill kernel -- the fused RMSNorm + QKV projection + RoPE of
// the page "Liger-Kernel底层优化：新一代内核级推理加速引擎介绍" (fused-kernel listing in
// section "融合内核是如何工作的？来看一段简化版实现") -- in the regime that page's
// section on the system stack singles out: per-query efficiency, where a layer step
// is a handful of tokens and the weight read dominates.  With 64 tokens the weight
// (H x N bf16) is ~97% of all bytes, so the kernel is bound by HBM bandwidth and is
// organised to keep every byte of W in flight once:
//
//   * 4 workgroups per head, each owning columns 16q..16q+15 and 64+16q..64+16q+15 of
//     one head, so both members of every rotation pair stay in one lane; the four
//     workgroups of a head are numbered onto the same XCD, so each 128-byte weight
//     line is fetched into that XCD's L2 once and read by all four.
//   * 8 waves per workgroup split K; each wave streams its 32-row weight slices
//     global -> LDS (buffer_load ... lds) through an 8-deep ring, and reads them back
//     as MFMA B fragments with ds_read_b64_tr_b16.  Activations (x, 64 x 32 per step)
//     come into registers 4 steps ahead, are multiplied by the norm weight and
//     rounded once to bf16 (normalise-on-load), and their squares are summed on the
//     way, so the RMS row reduction needs no separate pass over x.
//   * v_mfma_f32_16x16x32_bf16 over 4 token blocks x 2 column blocks per step.
//   * Partial sums of the 8 waves are added in LDS in a fixed order (deterministic);
//     then 1/rms, bias, rotation with in-kernel cos/sin, one bf16 store.
// All vector-memory instructions are issued as inline assembly and every wait is an
// exact, compile-time vmcnt, so the compiler never drains the pipeline.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace qkv {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStepK = 32;                     // k rows per step
constexpr int kRing = 8;                       // weight steps in flight per wave
constexpr int kXDepth = 4;                     // activation steps in flight per wave
constexpr int kStepBytes = kStepK * 64;        // 32 rows x 32 columns x 2 B
constexpr int kWaveRing = kRing * kStepBytes;  // 16 KB
constexpr int kLds = kWaves * kWaveRing;       // 128 KB
constexpr int kTokens = 64;                    // token capacity (4 blocks of 16)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int S, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (S < E) {
    f(std::integral_constant<int, S>{});
    static_for<S + 1, E>(f);
  }
}

// Issue order of vector-memory instructions (per wave):
//   prologue: weight slices 0..kRing-1 (2 instructions each), then activation steps
//             0..kXDepth-1 (5 each: 4 token blocks + the norm weight);
//   step s:   activation step s+kXDepth, then weight slice s+kRing (when they exist).
// These helpers count that sequence so each wait can name exactly how many younger
// instructions may stay outstanding.
template <int NS>
struct Issue {
  static constexpr int wops(int s) { return s < NS ? 2 : 0; }
  static constexpr int xops(int s) { return s < NS ? 5 : 0; }
  // index one past the last instruction of weight slice s / activation step s
  static constexpr int w_end(int s) {
    if (s < kRing) {
      int n = 0;
      for (int t = 0; t <= s; ++t) n += wops(t);
      return n;
    }
    return step_begin(s - kRing) + xops(s - kRing + kXDepth) + wops(s);
  }
  static constexpr int x_end(int s) {
    if (s < kXDepth) {
      int n = 0;
      for (int t = 0; t < kRing; ++t) n += wops(t);
      for (int t = 0; t <= s; ++t) n += xops(t);
      return n;
    }
    return step_begin(s - kXDepth) + xops(s);
  }
  // instructions issued before step s starts issuing
  static constexpr int step_begin(int s) {
    int n = 0;
    for (int t = 0; t < kRing; ++t) n += wops(t);
    for (int t = 0; t < kXDepth; ++t) n += xops(t);
    for (int t = 0; t < s; ++t) n += xops(t + kXDepth) + wops(t + kRing);
    return n;
  }
  // outstanding instructions allowed at the start of step s
  static constexpr int wait_at(int s) {
    const int need = w_end(s) > x_end(s) ? w_end(s) : x_end(s);
    const int v = step_begin(s) - need;
    return v > 62 ? 62 : v;
  }
};

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ u32x4 asm_load16(uint32_t voff, const u32x4& rsrc) {
  u32x4 v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rsrc));
  return v;
}

template <int NSTEPS>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(ForwardArgs a, int nheads) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  using I = Issue<NSTEPS>;

  // ---- workgroup -> (head, quarter); the 4 quarters of a head share an XCD
  const int b = blockIdx.x;
  int head, q;
  if ((nheads & 7) == 0) {
    const int xcd = b & 7, local = b >> 3;
    q = local & 3;
    head = (local >> 2) * 8 + xcd;
  } else {
    head = b >> 2;
    q = b & 3;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, N = a.N, T = a.T;
  const int c0 = head * 128 + 16 * q;  // first column of segment 0; segment 1 is c0 + 64
  const int kbeg = wave * (NSTEPS * kStepK);

  auto rsrc_of = [](const void* p, uint32_t bytes) {
    const uint64_t base = reinterpret_cast<uint64_t>(p);
    return u32x4{(uint32_t)base, (uint32_t)(base >> 32), bytes, (uint32_t)kBufferWord3};
  };
  const u32x4 w_rsrc = rsrc_of(a.w, (uint32_t)H * (uint32_t)N * 2u);
  const u32x4 x_rsrc = rsrc_of(a.x, (uint32_t)T * (uint32_t)H * 2u);  // tokens >= T read as 0
  const u32x4 n_rsrc = rsrc_of(a.w_norm, (uint32_t)H * 2u);

  // ---- weight DMA: instruction i of a step covers rows 16i + lane/4 of the slice.
  // LDS row (64 B) = 4 chunks [seg0 0-7 | seg0 8-15 | seg1 0-7 | seg1 8-15], chunk
  // index XOR (row/8 mod 4) so the transpose reads of the four k-groups spread
  // over the banks.
  const uint32_t lds0 =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem + wave * kWaveRing;
  uint32_t d_voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t row = 16u * i + (lane >> 2);
    const uint32_t lc = (uint32_t)(lane & 3) ^ ((row >> 3) & 3u);  // logical chunk held by this lane
    d_voff[i] = ((uint32_t)(kbeg + row) * N + c0 + 64u * (lc >> 1) + 8u * (lc & 1)) * 2u;
  }
  auto dma = [&](int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + (s % kRing) * kStepBytes + i * 1024);
      const uint32_t voff = d_voff[i] + (uint32_t)(s * kStepK) * (uint32_t)N * 2u;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(dst), "v"(voff),
                   "s"(w_rsrc)
                   : "m0", "memory");
    }
  };
  // ---- B fragments: 16-lane group g reads k rows 8g + 4h + 0..3 of column block cb
  const uint32_t tg = lane >> 4, tj = lane & 15;
  uint32_t t_off[2][2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t row = 8u * tg + 4u * h + (tj >> 2);
      const uint32_t col = 16u * cb + 4u * (tj & 3);
      const uint32_t pc = (col >> 3) ^ ((row >> 3) & 3u);
      t_off[cb][h] = row * 64u + pc * 16u + (col & 7u) * 2u;
    }

  // ---- activations: lane -> token tb*16 + lane%16, k = 8 * (lane/16) .. + 7
  const uint32_t x_voff = ((uint32_t)(lane & 15) * H + kbeg + 8u * (lane >> 4)) * 2u;
  const uint32_t n_voff = (uint32_t)(kbeg + 8 * (lane >> 4)) * 2u;
  u32x4 xr[kXDepth][4], nr[kXDepth];
  auto xload = [&](int s) {
    const int set = s % kXDepth;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      xr[set][tb] = asm_load16(x_voff + (uint32_t)(tb * 16) * H * 2u + (uint32_t)(s * kStepK) * 2u, x_rsrc);
    nr[set] = asm_load16(n_voff + (uint32_t)(s * kStepK) * 2u, n_rsrc);
  };

  f32x4 acc[4][2];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[tb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[4] = {0.f, 0.f, 0.f, 0.f};

  // ---- prologue
#pragma unroll
  for (int s = 0; s < kRing; ++s)
    if (s < NSTEPS) dma(s);
#pragma unroll
  for (int s = 0; s < kXDepth; ++s)
    if (s < NSTEPS) xload(s);

  static_for<0, NSTEPS>([&](auto sc) {
    constexpr int s = decltype(sc)::value;
    constexpr int set = s % kXDepth;
    vm_wait<I::wait_at(s)>();
    // make the activation registers of this step depend on the wait
    asm volatile("" : "+v"(xr[set][0]), "+v"(xr[set][1]), "+v"(xr[set][2]), "+v"(xr[set][3]), "+v"(nr[set]));
    const uint8_t* slot = smem + wave * kWaveRing + (s % kRing) * kStepBytes;
    bf16x8 fb[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(slot + t_off[cb][0]));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(slot + t_off[cb][1]));
      fb[cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    float wf[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      wf[2 * c] = bf16_lo(nr[set][c]);
      wf[2 * c + 1] = bf16_hi(nr[set][c]);
    }
    bf16x8 fa[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      u32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float lo = bf16_lo(xr[set][tb][c]), hi = bf16_hi(xr[set][tb][c]);
        ss[tb] = fmaf(lo, lo, fmaf(hi, hi, ss[tb]));
        o[c] = pack_bf16x2(lo * wf[2 * c], hi * wf[2 * c + 1]);
      }
      fa[tb] = __builtin_bit_cast(bf16x8, o);
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[tb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[tb], fb[cb], acc[tb][cb], 0, 0, 0);
    // the slot just read is refilled below: its transpose reads must have returned
    // (they have, since the MFMAs consumed them; the wait makes it explicit)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if constexpr (s + kXDepth < NSTEPS) xload(s + kXDepth);
    if constexpr (s + kRing < NSTEPS) dma(s + kRing);
  });

  // ---- cross-wave reduction in LDS (fixed order), then the epilogue
  __syncthreads();  // all rings consumed; the LDS is reused below
  float* red = reinterpret_cast<float*>(smem);                      // [wave][tb][cb][4][64]
  float* red_ss = reinterpret_cast<float*>(smem + kWaves * 8192);   // [wave][64 tokens]
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(((wave * 4 + tb) * 2 + cb) * 4 + r) * 64 + lane] = acc[tb][cb][r];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    float v = ss[tb];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (lane < 16) red_ss[wave * 64 + tb * 16 + lane] = v;
  }
  __syncthreads();
  if (wave >= 4) return;
  const int tb = wave;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int col = c0 + (lane & 15);  // segment-0 column; its rotation partner is col + 64
  void* out;
  int width, ocol;
  if (head * 128 < Nq) {
    out = a.q; width = Nq; ocol = col;
  } else if (head * 128 < Nq + Nkv) {
    out = a.k; width = Nkv; ocol = col - Nq;
  } else {
    out = a.v; width = Nkv; ocol = col - Nq - Nkv;
  }
  const bool rotate = head * 128 < Nq + Nkv;
  float b0 = 0.f, b1 = 0.f;
  if (a.bias) {
    b0 = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.bias)[col]);
    b1 = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.bias)[col + 64]);
  }
  const double rev = a.rev_freq[16 * q + (lane & 15)];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = tb * 16 + (lane >> 4) * 4 + r;
    float y0 = 0.f, y1 = 0.f, sq = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      y0 += red[(((w * 4 + tb) * 2 + 0) * 4 + r) * 64 + lane];
      y1 += red[(((w * 4 + tb) * 2 + 1) * 4 + r) * 64 + lane];
      sq += red_ss[w * 64 + t];
    }
    if (t >= T) continue;
    const float rinv = rsqrtf(sq / (float)H + a.eps);
    y0 = fmaf(y0, rinv, b0);
    y1 = fmaf(y1, rinv, b1);
    if (rotate) {
      float cs, sn;
      rope_cos_sin(a.pos[t], rev, cs, sn);
      const float u = y0, v = y1;
      y0 = u * cs - v * sn;
      y1 = v * cs + u * sn;
    }
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + (size_t)t * width + ocol;
    o[0] = f32_to_bf16(y0);
    o[64] = f32_to_bf16(y1);
  }
}

}  // namespace

bool decode_supports(int T, int H, int N, int Nq, int Nkv, int d) {
  return T >= 1 && T <= kTokens && d == 128 && Nq % 128 == 0 && Nkv % 128 == 0 && N % 128 == 0 &&
         (H == kWaves * kStepK * 16 || H == kWaves * kStepK * 8 || H == kWaves * kStepK * 32);
}

hipError_t launch_decode(const ForwardArgs& a, hipStream_t stream) {
  const int nheads = a.N / 128;
  const int steps = a.H / (kWaves * kStepK);
  dim3 grid(nheads * 4), block(kThreads);
  if (steps == 16)
    decode_kernel<16><<<grid, block, 0, stream>>>(a, nheads);
  else if (steps == 8)
    decode_kernel<8><<<grid, block, 0, stream>>>(a, nheads);
  else if (steps == 32)
    decode_kernel<32><<<grid, block, 0, stream>>>(a, nheads);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace qkv
