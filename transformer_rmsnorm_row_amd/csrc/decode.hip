// Decode kernel for gfx950: the whole chain for a small batch of tokens (T <= 128,
// one new token per sequence), streaming the QKV weight from HBM exactly once.
// Two forms: up to 64 tokens and up to 128; per token they compute the same sums in
// the same order, so a token's result does not depend on which form ran it.
//
// Same method as the prefill kernel -- the fused RMSNorm + QKV projection + RoPE of
// the page "Liger-Kernel底层优化：新一代内核级推理加速引擎介绍" (fused-kernel listing in
// section "融合内核是如何工作的？来看一段简化版实现") -- in the regime that page's
// discussion of where the library sits in the stack singles out: per-query
// efficiency, where a step is a handful of tokens and the weight read dominates.
// With 64 tokens the weight (H x N bf16) is ~97% of all bytes, so the kernel is
// bound by HBM bandwidth and is laid out so that every weight byte is read once,
// in full 256-byte rows, while the activations stay cheap:
//
//   * Work unit = one head (128 output columns, so both members of every rotation
//     pair are in the unit) x one of S slices of the hidden dimension, S as large
//     as keeps one unit per CU (5 for 48 heads: 240 units).  Each CU sustains a
//     fixed amount of loads in flight, so the weight streams faster the more CUs
//     take part; splitting K also keeps the per-unit share of x small.  When S
//     divides 8, units of the same K slice are numbered onto the same XCDs and
//     share their x slice in L2.
//   * 4 waves per unit split its K slice (runtime step counts, as even as the 32-row
//     steps allow); each wave streams 32-row steps of the weight (32 x 128 bf16)
//     and of x (64 or 128 x 32 bf16) global -> LDS with buffer_load ... lds through
//     a 3-deep (64 tokens) or 2-deep (128 tokens) ring.  B fragments (weight) come
//     back with ds_read_b64_tr_b16, A fragments (x) with ds_read_b128; each A
//     element is multiplied by its norm weight in fp32 (exact product) and rounded
//     once to bf16 (normalise-on-load), and the squares of the raw values are
//     summed for the RMS row reduction.
//   * v_mfma_f32_32x32x16_bf16, 2 or 4 token blocks x 4 column blocks per 16-wide k
//     (the 128-token form's 256 accumulator registers fill the AGPR file).
//   * The 4 waves add their partial sums in LDS (64 tokens per pass); each unit
//     writes its fp32 partial (tokens x 128) and its partial sums of squares to
//     plan scratch and bumps the head's arrival counter.  The unit that arrives
//     last adds the S partials in a fixed order (so results are deterministic),
//     applies 1/rms, bias and the rotation with in-kernel cos/sin, stores bf16, and
//     resets the counter.
// All vector-memory instructions in the streaming loop are inline assembly with
// exact, compile-time vmcnt waits, so the compiler never drains the pipeline.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace qkv {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kStepK = 32;                        // k rows per step
constexpr int kCols = 128;                        // one head
constexpr int kWBytes = kStepK * kCols * 2;       // 8 KB weight per step
constexpr int kLds = 144 * 1024;
constexpr int kMaxSplit = 5;                      // K slices per head, at most
constexpr int kMaxTokens = kDecodeTokens;         // largest token capacity instantiated (128)

// Layout for a launch of up to kTok tokens (64 or 128): kTok / 32 MFMA token blocks;
// a ring of 3 (64 tokens: 12 KB slots) or 2 (128 tokens: 16 KB slots) steps per wave;
// weight DMA (8) + x DMA (kTok / 16) + 2 norm-weight loads per step; the cross-wave
// reduction in passes of 64 tokens, so one pass of wave partials fits in LDS.
template <int kTok>
struct Cfg {
  static_assert(kTok == 64 || kTok == 128, "token capacities of the decode kernel");
  static constexpr int kTB = kTok / 32;
  static constexpr int kRing = kTok == 64 ? 3 : 2;
  static constexpr int kXBytes = kTok * kStepK * 2;
  static constexpr int kSlot = kWBytes + kXBytes;
  static constexpr int kWaveRing = kRing * kSlot;
  static constexpr int kXOps = kTok / 16;
  static constexpr int kOpsPerStep = 8 + kXOps + 2;
  static constexpr int kPasses = kTok / 64;
  static_assert(kWaves * kWaveRing <= kLds, "the rings fit in LDS");
  static_assert(kWaves * 64 * kCols * 4 + kWaves * kTok * 4 <= kLds, "one pass of wave partials fits in LDS");
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Vector-memory issue order per wave: steps 0..kRing-1 in the prologue, then
// step s + kRing right after step s has been consumed, kOpsPerStep instructions
// each; at the start of step s the loads of the min(kRing, nsteps - s) - 1 later
// steps may still be outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void dma16(uint32_t lds_dst, uint32_t voff, const u32x4& rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_dst), "v"(voff), "s"(rsrc)
               : "m0", "memory");
}

__device__ __forceinline__ u32x4 asm_load16(uint32_t voff, const u32x4& rsrc) {
  u32x4 v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rsrc));
  return v;
}


__device__ __forceinline__ u32x4 rsrc_of(const void* p, uint32_t bytes) {
  const uint64_t base = reinterpret_cast<uint64_t>(p);
  return u32x4{(uint32_t)base, (uint32_t)(base >> 32), bytes, (uint32_t)kBufferWord3};
}

// Weight slot: [32 k][128 n] (256-byte rows); 16-byte chunk c of row k sits at
// chunk c ^ 4*(k mod 4) so a transpose read's 4-row x 16-column blocks hit
// distinct banks.  Activation slot: [kTok tokens][32 k] (64-byte rows); chunk c of
// token t sits at c ^ ((t / 4) mod 4).
__device__ __forceinline__ uint32_t wchunk(uint32_t k, uint32_t c) { return c ^ ((k & 3u) << 2); }
__device__ __forceinline__ uint32_t xchunk(uint32_t t, uint32_t c) { return c ^ ((t >> 2) & 3u); }

template <int P>
using Int = std::integral_constant<int, P>;

template <int kTok>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(ForwardArgs a, int nheads, int nsplit) {
  using C = Cfg<kTok>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  __shared__ int s_last;

  // ---- unit -> (head, K slice); units of one K slice share XCDs
  const int b = blockIdx.x;
  int head, kq;
  const int per = 8 / nsplit;  // XCDs per K slice
  if (nsplit <= 8 && 8 % nsplit == 0 && nheads % per == 0) {
    const int xcd = b & 7, local = b >> 3;
    kq = xcd / per;
    head = (xcd % per) * (nheads / per) + local;
  } else {
    head = b / nsplit;
    kq = b % nsplit;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, N = a.N, T = a.T;
  const int n0 = head * kCols;
  // K slice kq of the head = 32-row steps [gs0, gs1) of the H / 32; its 4 waves split
  // them as evenly as possible (every wave gets at least one: H / 32 >= 4 nsplit)
  const int nst = H / kStepK;
  const int gs0 = nst * kq / nsplit, gs1 = nst * (kq + 1) / nsplit;
  const int ws0 = gs0 + (gs1 - gs0) * wave / kWaves, ws1 = gs0 + (gs1 - gs0) * (wave + 1) / kWaves;
  const int nsteps = ws1 - ws0;
  const int kbeg = ws0 * kStepK;

  const u32x4 w_rsrc = rsrc_of(a.w, (uint32_t)H * (uint32_t)N * 2u);
  const u32x4 x_rsrc = rsrc_of(a.x, (uint32_t)T * (uint32_t)H * 2u);  // tokens >= T read as 0
  const u32x4 n_rsrc = rsrc_of(a.w_norm, (uint32_t)H * 2u);
  const uint32_t ring0 =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem + wave * C::kWaveRing;

  // weight DMA: instruction i covers rows 4i..4i+3; lane -> row 4i + lane/16,
  // physical chunk lane%16, i.e. logical chunk wchunk(row, lane%16)
  const uint32_t w_voff = (((uint32_t)kbeg + (lane >> 4)) * N + n0 + 8u * wchunk(lane >> 4, lane & 15)) * 2u;
  // x DMA: instruction i covers tokens 16i..16i+15; lane -> token 16i + lane/4,
  // physical chunk lane%4, i.e. logical chunk xchunk(token, lane%4)
  const uint32_t x_voff = (((uint32_t)(lane >> 2)) * H + kbeg + 8u * xchunk(lane >> 2, lane & 3)) * 2u;
  auto issue_step = [&](int s, int sl) {
    const uint32_t slot = __builtin_amdgcn_readfirstlane(ring0 + sl * C::kSlot);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma16(slot + i * 1024, w_voff + ((uint32_t)(s * kStepK + 4 * i)) * (uint32_t)N * 2u, w_rsrc);
#pragma unroll
    for (int i = 0; i < C::kXOps; ++i)
      dma16(slot + kWBytes + i * 1024, x_voff + ((uint32_t)(16 * i) * H + s * kStepK) * 2u, x_rsrc);
  };
  // norm weight of the lane's k values: k = 16*ks + 8*(lane/32) + 0..7
  const uint32_t nw_voff = ((uint32_t)kbeg + 8u * (lane >> 5)) * 2u;
  u32x4 nw[C::kRing][2];
  auto issue_nw = [&](int s, int sl) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) nw[sl][ks] = asm_load16(nw_voff + (uint32_t)(s * kStepK + 16 * ks) * 2u, n_rsrc);
  };

  // fragment read offsets within a slot
  const uint32_t fl = lane & 31, fh = lane >> 5;
  uint32_t a_off[C::kTB][2];  // [token block][k half]
#pragma unroll
  for (int tb = 0; tb < C::kTB; ++tb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t t = 32u * tb + fl;
      a_off[tb][ks] = kWBytes + t * 64u + xchunk(t, 2u * ks + fh) * 16u;
    }
  const uint32_t tg = lane >> 4, tj = lane & 15;
  uint32_t b_off[4];  // [column block]; + ks*16 rows, + 4 rows for the second half
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const uint32_t krow = 8u * (tg >> 1) + (tj >> 2);
    const uint32_t col = cb * 32u + 16u * (tg & 1) + 4u * (tj & 3);
    b_off[cb] = krow * 256u + wchunk(krow, col >> 3) * 16u + (col & 7u) * 2u;
  }

  f32x16 acc[C::kTB][4];
  float ss[C::kTB];
#pragma unroll
  for (int tb = 0; tb < C::kTB; ++tb) {
    ss[tb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tb][cb][r] = 0.f;
  }

  // ---- prologue: up to kRing steps in flight
#pragma unroll
  for (int s = 0; s < C::kRing; ++s)
    if (s < nsteps) {
      issue_step(s, s);
      issue_nw(s, s);
    }

  // one step s (s % kRing == SL: ring slots and registers are compile-time); the loads
  // of the min(kRing, nsteps - s) - 1 later steps may stay outstanding
  auto step = [&](auto SLc, int s) {
    constexpr int slot_i = decltype(SLc)::value;
    const int later = min(C::kRing - 1, nsteps - 1 - s);  // wave-uniform
    if (later >= 2)
      vm_wait<2 * C::kOpsPerStep>();
    else if (later == 1)
      vm_wait<C::kOpsPerStep>();
    else
      vm_wait<0>();
    asm volatile("" : "+v"(nw[slot_i][0]), "+v"(nw[slot_i][1]));
    const uint8_t* slot = smem + wave * C::kWaveRing + slot_i * C::kSlot;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float wf[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        wf[2 * c] = bf16_lo(nw[slot_i][ks][c]);
        wf[2 * c + 1] = bf16_hi(nw[slot_i][ks][c]);
      }
      bf16x8 fa[C::kTB], fb[4];
#pragma unroll
      for (int tb = 0; tb < C::kTB; ++tb) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(slot + a_off[tb][ks]);
        u32x4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float lo = bf16_lo(raw[c]), hi = bf16_hi(raw[c]);
          ss[tb] = fmaf(lo, lo, fmaf(hi, hi, ss[tb]));
          o[c] = pack_bf16x2(lo * wf[2 * c], hi * wf[2 * c + 1]);
        }
        fa[tb] = __builtin_bit_cast(bf16x8, o);
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const uint8_t* p = slot + b_off[cb] + ks * 16 * 256;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 256));
        fb[cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int tb = 0; tb < C::kTB; ++tb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          acc[tb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tb], fb[cb], acc[tb][cb], 0, 0, 0);
    }
    // the slot is refilled next: all its LDS reads must have returned
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (s + C::kRing < nsteps) {
      issue_step(s + C::kRing, slot_i);
      issue_nw(s + C::kRing, slot_i);
    }
  };
  if constexpr (C::kRing == 3) {
    for (int s = 0; s < nsteps; s += 3) {
      step(Int<0>{}, s);
      if (s + 1 < nsteps) step(Int<1>{}, s + 1);
      if (s + 2 < nsteps) step(Int<2>{}, s + 2);
    }
  } else {
    // whole step pairs, then an odd last step: no merge inside the loop body
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
      step(Int<0>{}, s);
      step(Int<1>{}, s + 1);
    }
    if (s < nsteps) step(Int<0>{}, s);
  }

  // ---- the 4 waves' partial sums, added in LDS in a fixed order, 64 tokens (two
  // blocks) per pass.  LDS layout red[wave][tb % 2][cb][r/4][lane][r%4]: the 4
  // accumulator registers r%4 = 0..3 of a lane are 4 consecutive tokens of one column,
  // kept together so both the write and the cross-wave read are 16-byte operations.
  __syncthreads();  // every ring consumed: the LDS is reused below
  f32x4* red = reinterpret_cast<f32x4*>(smem);
  float* red_ss = reinterpret_cast<float*>(smem + kWaves * 64 * kCols * 4);  // [wave][kTok]
#pragma unroll
  for (int tb = 0; tb < C::kTB; ++tb) {
    const float v = ss[tb] + __shfl_xor(ss[tb], 32, 64);
    if (lane < 32) red_ss[wave * kTok + 32 * tb + lane] = v;
  }
  // Unit partial in plan scratch: [kTok / 4 token quads][128 columns][4 tokens] fp32,
  // then [kTok] sums of squares.  Written with agent-scope (sc1) stores, which go to
  // the device-wide coherence point rather than this XCD's L2; the unit that
  // arrives last reads them back the same way.  This avoids the full-L2
  // writeback and invalidate a device-wide fence costs when each XCD has its own
  // L2.
  const size_t unit = (size_t)head * nsplit + kq;
  const uint32_t part_floats = (uint32_t)nheads * nsplit * (kTok * kCols + kTok);
  const u32x4 p_rsrc = rsrc_of(a.partials, part_floats * 4u);
  const uint32_t part_off = (uint32_t)(unit * (kTok * kCols)) * 4u;
  const uint32_t ss_off = (uint32_t)((size_t)nheads * nsplit * (kTok * kCols) + unit * kTok) * 4u;
#pragma unroll
  for (int pass = 0; pass < C::kPasses; ++pass) {
    if (pass > 0) __syncthreads();  // the previous pass's cross-wave reads are done
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x16& ac = acc[2 * pass + tl][cb];
          red[(((wave * 2 + tl) * 4 + cb) * 4 + rq) * 64 + lane] =
              f32x4{ac[4 * rq], ac[4 * rq + 1], ac[4 * rq + 2], ac[4 * rq + 3]};
        }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int item = tid + kThreads * it;  // 2048 (token quad, column) cells of the pass
      const int tq = item >> 7, c = item & 127;
      const int tl = tq >> 3, rq = (tq & 7) >> 1, half = tq & 1;
      const int cb = c >> 5, ln = half * 32 + (c & 31);
      f32x4 v = red[(((0 * 2 + tl) * 4 + cb) * 4 + rq) * 64 + ln];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += red[(((w * 2 + tl) * 4 + cb) * 4 + rq) * 64 + ln];
      asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen sc1" ::"v"(__builtin_bit_cast(u32x4, v)),
                   "v"(part_off + (uint32_t)((16 * pass + tq) * kCols + c) * 16u), "s"(p_rsrc)
                   : "memory");
    }
  }
  if (tid < kTok) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red_ss[w * kTok + tid];
    __hip_atomic_store(&a.partials[ss_off / 4 + tid], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // every wave's stores complete before the unit is counted in
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&a.counters[head], 1u) == (unsigned)(nsplit - 1);
  __syncthreads();
  if (!s_last) return;

  // ---- last unit of the head: sum the S partials in K-slice order, then epilogue,
  // 64 tokens per pass.  Thread -> token quad tq (of the pass) and rotation pairs
  // j0 + 16i (i < 4): every load of a pass is issued before any is used.
  const int j0 = tid & 15;
  const uint32_t head_off = (uint32_t)((size_t)head * nsplit * (kTok * kCols)) * 4u;
  const uint32_t head_ss = (uint32_t)((size_t)nheads * nsplit * (kTok * kCols) + (size_t)head * nsplit * kTok) * 4u;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const bool rotate = n0 < Nq + Nkv;
  double frq[4];
  float bcol[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    frq[i] = a.rev_freq[j0 + 16 * i];
    bcol[i][0] = a.bias ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.bias)[n0 + j0 + 16 * i]) : 0.f;
    bcol[i][1] = a.bias ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.bias)[n0 + j0 + 16 * i + 64]) : 0.f;
  }
  void* out;
  int width, ocol0;
  if (n0 < Nq) {
    out = a.q; width = Nq; ocol0 = n0;
  } else if (n0 < Nq + Nkv) {
    out = a.k; width = Nkv; ocol0 = n0 - Nq;
  } else {
    out = a.v; width = Nkv; ocol0 = n0 - Nq - Nkv;
  }
  const bool to_cache = a.slots != nullptr && n0 >= Nq;  // K/V rows go to cache slots
#pragma unroll 1
  for (int pass = 0; pass < C::kPasses; ++pass) {
    const int tq = (tid >> 4) + 16 * pass;  // token quad of the unit block
    if (4 * tq >= T) break;                 // uniform per 16 lanes; no barrier follows
    // per-row inputs of the epilogue, requested before the partials so their
    // latency overlaps
    int32_t prow[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) prow[rr] = (rotate && 4 * tq + rr < T) ? a.pos[4 * tq + rr] : 0;
    u32x4 pv[4][kMaxSplit][2], sv[kMaxSplit];
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      if (s >= nsplit) break;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // unit block = kTok * kCols floats = kTok * kCols / 4 16-byte cells
          const uint32_t off = head_off + (uint32_t)(s * (kTok * kCols / 4) + tq * kCols + j0 + 16 * i + 64 * h) * 16u;
          asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen sc1" : "=v"(pv[i][s][h]) : "v"(off), "s"(p_rsrc) : "memory");
        }
      asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen sc1" : "=v"(sv[s]) : "v"(head_ss + (uint32_t)(s * kTok + 4 * tq) * 4u), "s"(p_rsrc) : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    f32x4 y[4][2], sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) y[i][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      if (s >= nsplit) break;
      asm volatile("" : "+v"(sv[s]));
      sq += __builtin_bit_cast(f32x4, sv[s]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          asm volatile("" : "+v"(pv[i][s][h]));
          y[i][h] += __builtin_bit_cast(f32x4, pv[i][s][h]);
        }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int t = 4 * tq + rr;
      if (t >= T) break;
      int row = t;
      if (to_cache) {
        row = a.slots[t];
        if (row < 0 || row >= a.cache_rows) continue;
      }
      const float rinv = rsqrtf(sq[rr] / (float)H + a.eps);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 16 * i;
        const float y0r = fmaf(y[i][0][rr], rinv, bcol[i][0]), y1r = fmaf(y[i][1][rr], rinv, bcol[i][1]);
        float y0 = y0r, y1 = y1r;
        if (rotate) {
          float cs, sn;
          rope_cos_sin(prow[rr], frq[i], cs, sn);
          const float u = y0, v = y1;
          y0 = u * cs - v * sn;
          y1 = v * cs + u * sn;
        }
        uint16_t* o = reinterpret_cast<uint16_t*>(out) + (size_t)row * width + ocol0 + j;
        o[0] = f32_to_bf16(y0);
        o[64] = f32_to_bf16(y1);
      }
    }
  }
  if (tid == 0) a.counters[head] = 0u;  // ready for the next forward on this plan
}

int pick_split(int nheads, int H) {
  // as many K slices per head as keep one unit per CU (256 CUs), at most kMaxSplit,
  // with at least one 32-row step per wave
  if (H % kStepK != 0 || nheads < 1) return 0;
  const int nst = H / kStepK;
  int s = min(kMaxSplit, 256 / nheads);
  s = min(s, nst / kWaves);
  return s >= 1 ? s : 0;
}

}  // namespace

bool decode_supports(int T, int H, int N, int Nq, int Nkv, int d) {
  return T >= 1 && T <= kMaxTokens && d == 128 && Nq % 128 == 0 && Nkv % 128 == 0 && N % 128 == 0 &&
         pick_split(N / 128, H) > 0;
}

size_t decode_scratch_floats(int H, int N) {
  const int nheads = N / 128;
  const int s = pick_split(nheads, H);
  return (size_t)nheads * s * (kMaxTokens * kCols + kMaxTokens);
}

hipError_t launch_decode(const ForwardArgs& a, hipStream_t stream) {
  const int nheads = a.N / 128;
  const int nsplit = pick_split(nheads, a.H);
  if (nsplit < 1) return hipErrorInvalidValue;
  if (a.T <= 64)
    decode_kernel<64><<<dim3(nheads * nsplit), dim3(kThreads), 0, stream>>>(a, nheads, nsplit);
  else
    decode_kernel<128><<<dim3(nheads * nsplit), dim3(kThreads), 0, stream>>>(a, nheads, nsplit);
  return hipGetLastError();
}

}  // namespace qkv

