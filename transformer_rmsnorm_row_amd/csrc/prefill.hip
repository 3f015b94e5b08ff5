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
constexpr int kTile = BM * BK * 2;                 // bytes of one [256][64] bf16 tile (A or B)
constexpr int kBStages = 3;                        // weight slices in flight (global -> LDS directly)
constexpr int kAStages = 2;                        // converted activation slices
constexpr int kBBase = 0;
constexpr int kABase = kBStages * kTile;
constexpr int kLds = (kBStages + kAStages) * kTile;  // 160 KB
constexpr int kStagePitch = 272;                   // 128 bf16 + 16 B pad per staged output row
constexpr int kStageBytes = 128 * kStagePitch;     // one wave's 128 x 128 output block
constexpr int kRowInfo = 4 * kStageBytes;          // per-row pos and 1/rms after the staging area
static_assert(kRowInfo + BM * 8 <= kLds, "epilogue staging must fit in the tile memory");
constexpr int kGroupM = 4;

// LDS address of 16-byte chunk `chunk` (0..7) of row `row` in a [256][64] bf16
// activation tile (row = token, 64 k per row).
__device__ __forceinline__ uint32_t tile_off(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ ((row ^ (row >> 3)) & 7u)) << 4);
}
// The weight slice stays [64 k][256 n] (512 B rows) as loaded; 16-byte chunk c of
// row k sits at chunk c ^ 4*(k mod 4), which spreads the 4-row x 16-column blocks
// of a transpose read over all banks.
__device__ __forceinline__ uint32_t wchunk(uint32_t k, uint32_t c) { return c ^ ((k & 3u) << 2); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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


  // ---- activation slice (registers -> LDS): thread owns chunk kc of rows ar + 32j
  const uint32_t kc = tid & 7, ar = tid >> 3;
  const uint32_t a_goff = ((uint32_t)(m0 + ar) * H + kc * 8u) * 2u;
  const uint32_t a_gstep = 32u * H * 2u;
  uint32_t a_soff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a_soff[j] = kABase + tile_off(ar + 32u * j, kc);

  // ---- weight slice (global -> LDS directly): wave loads rows 16*wave + 2i (+1),
  // each instruction one 1 KB run of LDS = two 512 B rows; lane l fills physical
  // chunk l % 32 of row 2i + l / 32, i.e. logical chunk wchunk(row, l % 32).
  uint32_t b_voff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const uint32_t krow = 2u * par + (lane >> 5);  // row within the 4-row swizzle period
    b_voff[par] = ((16u * wave + krow) * N + n0 + 8u * wchunk(krow, lane & 31)) * 2u;
  }
  // Issued as inline assembly: the compiler cannot tell that a stage being
  // filled is never the one being read, and would otherwise drain every load
  // before each LDS read.  The waits are explicit (wait_vmcnt before barriers).
  const uint64_t wbase = reinterpret_cast<uint64_t>(a.w);
  const u32x4 w_rsrc = {(uint32_t)wbase, (uint32_t)(wbase >> 32), (uint32_t)H * (uint32_t)N * 2u,
                        (uint32_t)kBufferWord3};
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  auto dma_b = [&](int k0, int stage) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + kBBase + stage * kTile + (16 * wave + 2 * i) * 512);
      // the whole offset goes in the per-lane operand so the buffer's range check
      // (zero fill past the end of the weight) sees all of it
      const uint32_t voff = b_voff[i & 1] + ((uint32_t)k0 + 2u * (i & ~1)) * (uint32_t)N * 2u;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(dst), "v"(voff), "s"(w_rsrc)
                   : "m0");
    }
  };

  // ---- fragment read offsets
  const uint32_t fl = lane & 31, fh = lane >> 5;
  uint32_t a_roff[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a_roff[rb][ks] = kABase + tile_off(wm * 128u + rb * 32u + fl, ks * 2u + fh);
  // transpose reads of the weight: 16-lane group g covers k rows 8(g/2) + 4h + 0..3
  // and columns 16(g%2) + 0..15 of a 32-column block; lane j of the group points at
  // row j/4, columns 4(j%4)..+3.
  const uint32_t tg = lane >> 4, tj = lane & 15;
  uint32_t b_roff[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const uint32_t krow = 8u * (tg >> 1) + (tj >> 2);
    const uint32_t col = wn * 128u + cb * 32u + 16u * (tg & 1) + 4u * (tj & 3);
    b_roff[cb] = krow * 512u + wchunk(krow, col >> 3) * 16u + (col & 7u) * 2u;
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ga[2][8], gw[2];
  // Loads past the end of K read zeros (outside the buffer's range) or rows that
  // are never used, so the loop body needs no branch.  Like the weight DMA they are
  // inline assembly, so that every vector-memory instruction is invisible to the
  // compiler's wait insertion and the waits below can count them exactly.
  const uint64_t xbase = reinterpret_cast<uint64_t>(a.x), nbase = reinterpret_cast<uint64_t>(a.w_norm);
  const u32x4 x_rsrc = {(uint32_t)xbase, (uint32_t)(xbase >> 32), (uint32_t)T * (uint32_t)H * 2u, (uint32_t)kBufferWord3};
  const u32x4 n_rsrc = {(uint32_t)nbase, (uint32_t)(nbase >> 32), (uint32_t)H * 2u, (uint32_t)kBufferWord3};
  auto asm_load16 = [](uint32_t voff, const u32x4& rsrc) {
    u32x4 v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rsrc));
    return v;
  };
  auto gload_rows = [&](int set, int k0, int j0, int j1) {
#pragma unroll
    for (int j = j0; j < j1; ++j) ga[set][j] = asm_load16(a_goff + j * a_gstep + (uint32_t)k0 * 2u, x_rsrc);
  };
  auto gload_w = [&](int set, int k0) { gw[set] = asm_load16(((uint32_t)k0 + kc * 8u) * 2u, n_rsrc); };
  // the activation registers of a set become usable only after an explicit wait
  auto tie_set = [&](int set) {
    asm volatile("" : "+v"(ga[set][0]), "+v"(ga[set][1]), "+v"(ga[set][2]), "+v"(ga[set][3]), "+v"(ga[set][4]),
                 "+v"(ga[set][5]), "+v"(ga[set][6]), "+v"(ga[set][7]), "+v"(gw[set]));
  };
  // rows j0..j1-1 of a slice: x * norm weight in fp32, rounded once to bf16, into LDS
  auto convert_rows = [&](int set, int stage, int j0, int j1) {
    float wf[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      wf[2 * c] = bf16_lo(gw[set][c]);
      wf[2 * c + 1] = bf16_hi(gw[set][c]);
    }
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      u32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        o[c] = pack_bf16x2(bf16_lo(ga[set][j][c]) * wf[2 * c], bf16_hi(ga[set][j][c]) * wf[2 * c + 1]);
      lds_write16(smem, a_soff[j] + stage * kTile, o);
    }
  };

  bf16x8 fa[2][4], fb[2][4];
  auto read_frags = [&](int astage, uint32_t bbase, int ks, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[buf][i] = __builtin_bit_cast(bf16x8, lds_read16(smem, a_roff[i][ks] + astage * kTile));
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const uint8_t* p = smem + bbase + b_roff[cb] + ks * 16 * 512;
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 512));
      fb[buf][cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
  };

  // One K slice kt: MFMAs from A stage (kt % 2) and B stage bcur; meanwhile the
  // weight slice kt+2 streams into B stage bnext2, activation slice kt+1 (register
  // set `cs`) is converted into A stage (kt+1) % 2, and activation slice kt+3 is
  // loaded into the freed register set.
  auto body = [&](int kt, int as, int cs, uint32_t bcur, int bnext2) {
    dma_b((kt + 2) * BK, bnext2);
    // Vector-memory order per slice i: weight DMA of slice i+2 (8), then the
    // activation loads of slice i+3 (9).  The activation set converted now (slice
    // kt+1, loaded during slice kt-2) is complete once at most the 17 instructions
    // of slice kt-1 and the 8 just issued remain.
    wait_vmcnt<25>();
    tie_set(cs);
    read_frags(as, bcur, 1, 1);
    mfmas(0);
    convert_rows(cs, as ^ 1, 0, 2);
    gload_rows(cs, (kt + 3) * BK, 0, 2);
    sched_substep<3, 12, 2, 10>();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(as, bcur, 2, 0);
    mfmas(1);
    convert_rows(cs, as ^ 1, 2, 4);
    gload_rows(cs, (kt + 3) * BK, 2, 4);
    sched_substep<3, 12, 2, 2>();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(as, bcur, 3, 1);
    mfmas(0);
    convert_rows(cs, as ^ 1, 4, 6);
    gload_rows(cs, (kt + 3) * BK, 4, 6);
    sched_substep<3, 12, 2, 2>();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
    convert_rows(cs, as ^ 1, 6, 8);
    gload_rows(cs, (kt + 3) * BK, 6, 8);
    gload_w(cs, (kt + 3) * BK);
    sched_substep<3, 0, 2, 3>();
    __builtin_amdgcn_sched_barrier(0);
    // the weight slice read next (issued one slice ago) must have landed: that
    // slice's 9 activation loads and this slice's 17 instructions came after it
    wait_vmcnt<26>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nk = H / BK;  // even
  // prologue: weight slices 0 and 1 in flight, activation slices 0..2 loaded,
  // slice 0 converted
  dma_b(0, 0);
  dma_b(BK, 1);
  gload_rows(0, 0, 0, 8);
  gload_w(0, 0);
  gload_rows(1, BK, 0, 8);
  gload_w(1, BK);
  wait_vmcnt<9>();  // slice 0 of x (and both weight slices) landed; slice 1 of x may be in flight
  tie_set(0);
  convert_rows(0, 0, 0, 8);
  gload_rows(0, 2 * BK, 0, 8);
  gload_w(0, 2 * BK);
  // slice 1 of x (converted in the first slice) must be in before the steady-state
  // counts apply; only slice 2's 9 loads may remain
  wait_vmcnt<9>();
  __syncthreads();

  uint32_t bcur = kBBase, bn1 = kBBase + kTile, bn2i = 2;
  for (int kt = 0; kt < nk; kt += 2) {
    read_frags(0, bcur, 0, 0);
    body(kt, 0, 1, bcur, bn2i);
    {  // rotate the three weight stages
      uint32_t t = bcur; bcur = bn1; bn1 = kBBase + bn2i * kTile; (void)t;
      bn2i = (bn2i == 2) ? 0 : bn2i + 1;
    }
    read_frags(1, bcur, 0, 0);
    body(kt + 1, 1, 0, bcur, bn2i);
    {
      bcur = bn1; bn1 = kBBase + bn2i * kTile;
      bn2i = (bn2i == 2) ? 0 : bn2i + 1;
    }
  }
  // Drain the loads that ran past the end of K before the tile memory is reused.
  // The activation registers they target are never read again, so the compiler
  // would hand them to the epilogue: tying them to the wait keeps them reserved
  // until the late loads have landed.
  asm volatile("s_waitcnt vmcnt(0)"
               : "+v"(ga[0][0]), "+v"(ga[0][1]), "+v"(ga[0][2]), "+v"(ga[0][3]), "+v"(ga[0][4]), "+v"(ga[0][5]),
                 "+v"(ga[0][6]), "+v"(ga[0][7]), "+v"(gw[0]), "+v"(ga[1][0]), "+v"(ga[1][1]), "+v"(ga[1][2]),
                 "+v"(ga[1][3]), "+v"(ga[1][4]), "+v"(ga[1][5]), "+v"(ga[1][6]), "+v"(ga[1][7]), "+v"(gw[1])
               :
               : "memory");
  __syncthreads();
  int32_t* s_pos = reinterpret_cast<int32_t*>(smem + kRowInfo);
  float* s_rinv = reinterpret_cast<float*>(smem + kRowInfo + BM * 4);
  {
    int t = m0 + tid;
    s_pos[tid] = t < T ? a.pos[t] : 0;
    s_rinv[tid] = t < T ? a.inv_rms[t] : 0.f;
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
