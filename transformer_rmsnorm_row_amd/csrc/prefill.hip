// bf16 MFMA prefill kernel for gfx950: normalise-on-load QKV projection with the
// bias and rotate-half rotary embedding applied in registers, Q/K/V written once.
//
// The method is the fused RMSNorm + QKV projection + RoPE kernel of the page
// "Liger-Kernel底层优化：新一代内核级推理加速引擎介绍" (section
// "融合内核是如何工作的？来看一段简化版实现", and the fused-kernel list that names
// "Fused RMSNorm + QKV Projection + RoPE"): the normalised activations exist only
// inside the kernel, the bias is added to each dot product, and each rotation pair
// (i, i + head_dim/2) is turned by the position's angle before the single store.
//
// gfx950 design (the listing's one-thread-per-feature loop is not used):
//   * 256 x 256 output tile per 256-thread workgroup, 4 waves in a 2 x 2 grid, each
//     wave a 128 x 128 block = 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32
//     per lane).  A wave's 128 columns are one head (head_dim 128), so both halves of
//     every rotation pair sit in the same lane and the same accumulator register.
//   * K advances 64 at a time through double-buffered LDS tiles (2 x 64 KB); the
//     next slice's 16-byte global loads are issued before the current slice's 64
//     MFMAs and land in LDS after them, one barrier per slice.
//   * Normalise-on-load: each x element is multiplied by its norm weight in fp32
//     and rounded once to bf16 as it is written to LDS.  The per-token factor
//     1/rms is applied to the accumulator rows in the epilogue, which is the same
//     product (diag(r) X diag(w) W = diag(r) (X diag(w)) W); the normalised
//     activations never reach HBM.
//   * The weight tile [k][n] is transposed in registers (v_perm) into [n][k] so
//     both MFMA operands are read from LDS with one 16-byte read per fragment.
//     LDS rows are 128 B with the 16-byte chunk index XOR-swizzled by the row.
//   * Tiles are numbered so that the ~32 workgroups running at once on one XCD
//     (workgroups go round-robin over the 8 XCDs) cover 4 row panels x 8 column
//     panels and share them in that XCD's L2.
//   * Epilogue: y = acc * r[t] + bias; Q and K pairs rotated with cos/sin of
//     pos * theta^(-2i/d) (turn count reduced in fp64, hardware sin/cos on the
//     fraction of a turn); bf16 results staged through LDS and stored with
//     16-byte coalesced writes.
#include "device_common.h"
#include "launch.h"

namespace qkv {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kTile = BM * BK * 2;                 // bytes of one [256][64] bf16 tile
constexpr int kStagePitch = 272;                   // 128 bf16 + 16 B pad per staged output row
constexpr int kStageBytes = 128 * kStagePitch;     // one wave's 128 x 128 output block
constexpr int kMainBytes = 4 * kStageBytes > 4 * kTile ? 4 * kStageBytes : 4 * kTile;
constexpr int kLds = kMainBytes + BM * 8;          // + per-row pos and 1/rms
constexpr int kGroupM = 4;

// LDS address of 16-byte chunk `chunk` (0..7) of row `row` in a [256][64] bf16 tile.
__device__ __forceinline__ uint32_t tile_off(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ ((row ^ (row >> 3)) & 7u)) << 4);
}

__device__ __forceinline__ u32x4 lds_read16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(uint8_t* base, uint32_t off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}

__device__ __forceinline__ float turn_fraction(int32_t pos, double rev) {
  double t = (double)pos * rev;
  return (float)(t - floor(t));
}

// Interleave the 16 MFMAs of a K substep with the VALU, LDS and VMEM work issued
// alongside them, so the matrix pipe is not left waiting behind the rest.
template <int kValuPerMfma, int kDsReads, int kDsWrites, int kVmemReads>
__device__ __forceinline__ void sched_substep() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (kValuPerMfma > 0) __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    if (i < kDsReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (i >= 4 && i - 4 < kDsWrites) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if (i >= 6 && i - 6 < kVmemReads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

__global__ __launch_bounds__(256, 1) void prefill_kernel(ForwardArgs a, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  int32_t* s_pos = reinterpret_cast<int32_t*>(smem + kMainBytes);
  float* s_rinv = reinterpret_cast<float*>(smem + kMainBytes + BM * 4);

  // ---- tile selection: XCD-contiguous numbering, then groups of kGroupM row panels
  const int G = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int q8 = G >> 3, r8 = G & 7;
  const int L = (xcd < r8) ? xcd * (q8 + 1) + local : r8 * (q8 + 1) + (xcd - r8) * q8 + local;
  const int group = L / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int idx = L - group * kGroupM * tiles_n;
  const int tm = first_m + idx % gm;
  const int tn = idx / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int wm = wave >> 1, wn = wave & 1;
  const int H = a.H, N = a.N, T = a.T;

  {
    int t = m0 + tid;
    s_pos[tid] = t < T ? a.pos[t] : 0;
    s_rinv[tid] = t < T ? a.inv_rms[t] : 0.f;
  }

  const auto rx = make_rsrc(a.x, (uint32_t)T * (uint32_t)H * 2u);
  const auto rwn = make_rsrc(a.w_norm, (uint32_t)H * 2u);
  const auto rw = make_rsrc(a.w, (uint32_t)H * (uint32_t)N * 2u);

  // ---- per-thread global load coordinates
  const uint32_t kc = tid & 7, ar = tid >> 3;             // A: chunk kc of rows ar + 32j
  const uint32_t bc = tid & 31, bg = tid >> 5;            // B: cols 8bc.., rows 8bg + j
  const uint32_t a_goff = ((uint32_t)(m0 + ar) * H + kc * 8u) * 2u;
  const uint32_t a_gstep = 32u * H * 2u;
  const uint32_t b_goff = (8u * bg * N + n0 + 8u * bc) * 2u;
  const uint32_t b_gstep = (uint32_t)N * 2u;

  uint32_t a_soff[8], b_soff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a_soff[j] = tile_off(ar + 32u * j, kc);
    b_soff[j] = tile_off(8u * bc + j, bg);
  }
  // ---- per-lane fragment read offsets
  const uint32_t fl = lane & 31, fh = lane >> 5;
  uint32_t a_roff[4][4], b_roff[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      a_roff[rb][ks] = tile_off(wm * 128u + rb * 32u + fl, ks * 2u + fh);
      b_roff[rb][ks] = tile_off(wn * 128u + rb * 32u + fl, ks * 2u + fh);
    }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ga[8], gb[8], gw;
  // Loads of a K slice.  Past the end of K they read zeros (out of the buffer's
  // range) or rows that are never used, so the loop body needs no branch.
  auto gload_a = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) ga[j] = buf_load16(rx, a_goff + j * a_gstep + (uint32_t)k0 * 2u);
    gw = buf_load16(rwn, ((uint32_t)k0 + kc * 8u) * 2u);
  };
  auto gload_b = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) gb[j] = buf_load16(rw, b_goff + ((uint32_t)k0 + j) * b_gstep);
  };
  // x rows j0..j1-1 of the slice: scale by the norm weight in fp32, round to bf16.
  auto lstore_a = [&](uint8_t* As, int j0, int j1) {
    float wf[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      wf[2 * c] = bf16_lo(gw[c]);
      wf[2 * c + 1] = bf16_hi(gw[c]);
    }
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      u32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = pack_bf16x2(bf16_lo(ga[j][c]) * wf[2 * c], bf16_hi(ga[j][c]) * wf[2 * c + 1]);
      lds_write16(As, a_soff[j], o);
    }
  };
  // weight columns 8bc + jj (jj0..jj1-1) of the slice, transposed to [n][k].
  auto lstore_b = [&](uint8_t* Bs, int jj0, int jj1) {
#pragma unroll
    for (int jj = jj0; jj < jj1; ++jj) {
      const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) o[qd] = __builtin_amdgcn_perm(gb[2 * qd + 1][jj >> 1], gb[2 * qd][jj >> 1], sel);
      lds_write16(Bs, b_soff[jj], o);
    }
  };
  bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
  auto read_frags = [&](const uint8_t* As, const uint8_t* Bs, int ks, bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = __builtin_bit_cast(bf16x8, lds_read16(As, a_roff[i][ks]));
      fb[i] = __builtin_bit_cast(bf16x8, lds_read16(Bs, b_roff[i][ks]));
    }
  };
  auto mfmas = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  uint8_t* const A0 = smem;
  uint8_t* const B0 = smem + kTile;
  uint8_t* const A1 = smem + 2 * kTile;
  uint8_t* const B1 = smem + 3 * kTile;

  // One K slice from (Ac, Bc) while slice kt+1 goes from registers into (An, Bn)
  // and slice kt+2 is fetched into the registers.
  auto body = [&](const uint8_t* Ac, const uint8_t* Bc, uint8_t* An, uint8_t* Bn, int kt) {
    read_frags(Ac, Bc, 1, fa1, fb1);
    mfmas(fa0, fb0);
    lstore_a(An, 0, 4);
    sched_substep<5, 8, 4, 0>();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(Ac, Bc, 2, fa0, fb0);
    mfmas(fa1, fb1);
    lstore_a(An, 4, 8);
    gload_a((kt + 2) * BK);
    sched_substep<5, 8, 4, 9>();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(Ac, Bc, 3, fa1, fb1);
    mfmas(fa0, fb0);
    lstore_b(Bn, 0, 4);
    sched_substep<1, 8, 4, 0>();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa1, fb1);
    lstore_b(Bn, 4, 8);
    gload_b((kt + 2) * BK);
    sched_substep<1, 0, 4, 8>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_frags(An, Bn, 0, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nk = H / BK;  // even
  gload_a(0);
  gload_b(0);
  lstore_a(A0, 0, 8);
  lstore_b(B0, 0, 8);
  gload_a(BK);
  gload_b(BK);
  __syncthreads();
  read_frags(A0, B0, 0, fa0, fb0);
  for (int kt = 0; kt < nk; kt += 2) {
    body(A0, B0, A1, B1, kt);
    body(A1, B1, A0, B0, kt + 1);
  }
  __syncthreads();

  // ---- epilogue: scale, bias, rotate, stage as bf16, store
  const int col0 = n0 + wn * 128;  // first column of this wave's head
  const bool rotate = col0 < a.Nq + a.Nkv;
  void* out;
  uint32_t width, ocol;
  if (col0 < a.Nq) {
    out = a.q; width = a.Nq; ocol = col0;
  } else if (col0 < a.Nq + a.Nkv) {
    out = a.k; width = a.Nkv; ocol = col0 - a.Nq;
  } else {
    out = a.v; width = a.Nkv; ocol = col0 - a.Nq - a.Nkv;
  }
  float bcol[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    bcol[cb] = a.bias ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.bias)[col0 + cb * 32 + fl]) : 0.f;
  const double f0 = a.rev_freq[fl], f1 = a.rev_freq[32 + fl];

  uint8_t* stage = smem + wave * kStageBytes;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int rbase = rb * 32 + rg * 8 + (int)fh * 4;
      const f32x4 ri4 = *reinterpret_cast<const f32x4*>(s_rinv + wm * 128 + rbase);
      const i32x4 p4 = *reinterpret_cast<const i32x4*>(s_pos + wm * 128 + rbase);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float y[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) y[cb] = fmaf(acc[rb][cb][rg * 4 + rr], ri4[rr], bcol[cb]);
        if (rotate) {
          const float t0 = turn_fraction(p4[rr], f0), t1 = turn_fraction(p4[rr], f1);
          const float c0 = __builtin_amdgcn_cosf(t0), s0 = __builtin_amdgcn_sinf(t0);
          const float c1 = __builtin_amdgcn_cosf(t1), s1 = __builtin_amdgcn_sinf(t1);
          const float u0 = y[0], v0 = y[2], u1 = y[1], v1 = y[3];
          y[0] = u0 * c0 - v0 * s0;
          y[2] = v0 * c0 + u0 * s0;
          y[1] = u1 * c1 - v1 * s1;
          y[3] = v1 * c1 + u1 * s1;
        }
        uint16_t* srow = reinterpret_cast<uint16_t*>(stage + (rbase + rr) * kStagePitch);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) srow[cb * 32 + fl] = f32_to_bf16(y[cb]);
      }
    }
  }
  __syncthreads();
  const auto ro = make_rsrc(out, (uint32_t)T * width * 2u);
  const uint32_t ch = lane & 15;
#pragma unroll 8
  for (int it = 0; it < 32; ++it) {
    const uint32_t row = (lane >> 4) + 4u * it;
    const u32x4 v = lds_read16(stage, row * kStagePitch + ch * 16u);
    const uint32_t grow = (uint32_t)(m0 + wm * 128) + row;
    buf_store16(v, ro, (grow * width + ocol + ch * 8u) * 2u);
  }
}

}  // namespace

bool prefill_supports(int H, int N, int Nq, int Nkv, int d) {
  return d == 128 && H % (2 * BK) == 0 && N % BN == 0 && Nq % 128 == 0 && Nkv % 128 == 0;
}

hipError_t launch_prefill(const ForwardArgs& a, hipStream_t stream) {
  hipError_t e = launch_inv_rms(a.x, a.inv_rms, a.T, a.H, a.eps, true, stream);
  if (e != hipSuccess) return e;
  const int tiles_m = (a.T + BM - 1) / BM, tiles_n = a.N / BN;
  prefill_kernel<<<dim3(tiles_m * tiles_n), dim3(256), 0, stream>>>(a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace qkv
