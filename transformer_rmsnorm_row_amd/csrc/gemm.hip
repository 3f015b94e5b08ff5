// The two plain GEMMs of the backward (dW = a^T gy and ga = gy W^T) on the matrix cores
// of gfx950, and a plain fp32-FMA GEMM for fp32 plans and shapes outside the MFMA form.
//
// The backward of the fused chain (the page "Liger-Kernel底层优化：新一代内核级推理加速
// 引擎介绍", fused-kernel list, "Fused RMSNorm + QKV Projection + RoPE", differentiated
// by the chain rule) needs the weight gradient dW = a^T gy over the tokens and the
// activation gradient ga = gy W^T over the projection's columns, with a the normalised
// activations and gy the unrotated upstream gradient.
//
// MFMA form (bf16 operands, fp32 accumulation):
//   * 256 x 256 output tile per 512-thread workgroup (8 waves, two per SIMD); wave
//     (g, s) owns rows 128g..+127 and columns 64s..+63: 8 x 4 accumulators of
//     v_mfma_f32_16x16x32_bf16 (128 fp32 per lane).  With no conversion in the loop the
//     16-cycle 16 x 16 x 32 shape, which moves half the accumulator bytes per flop of
//     the 32 x 32 x 16 one, is the faster of the two at the chip's power limit.
//   * Each operand is one of two layouts in memory:
//       kRowK  [rows][K], k contiguous: a step of 32 k is 64 bytes of each of the tile's
//              256 rows, staged as [256][64 B] with the 16-byte chunks XOR-ed by bits
//              1..2 of the row, read as fragments with ds_read_b128;
//       kKRow  [K][cols], cols contiguous: a step is 32 rows of 512 bytes, staged as
//              loaded with chunk c of k row r at c ^ 2 ((r mod 4) + 4 ((r / 8) mod 4)),
//              read as fragments with the transpose read ds_read_b64_tr_b16.
//     Both GEMMs take A as kKRow and B as kRowK, the pairing measured fastest (one
//     operand of each kind: 623-633 us on 8192 x 4096 x 12288, against 650 us with both
//     kKRow and 838 us with both kRowK): dW takes a [T, H] and gy^T [N, Tp], ga takes
//     gy^T and W [H, N].  The unrotated gradient is written transposed for this.  Both
//     results are rounded once to the plan dtype.
//   * Both operands go global -> LDS by DMA (buffer_load ... lds), three steps ahead
//     into 4-deep rings (2 x 64 KB), 1 KB per instruction, two instructions per
//     operand, wave and step.
//   * Ping-pong: waves 0-3 and 4-7 are one phase apart.  A memory phase reads the
//     wave's fragments of step t, issues step t + 3 and waits until its own part of
//     step t + 1 has landed; a compute phase runs the step's 32 MFMAs.  Barriers
//     separate the phases, so on every SIMD one wave feeds the matrix pipe while the
//     other reads LDS.
//   * Tails: loads outside an operand's buffer read zeros (K past the end for kKRow,
//     rows past the end for kRowK); kRowK steps that start at or past K are sent outside
//     the buffer, and a kRowK operand whose K is not a multiple of 32 must carry zeros
//     in its rows from K to the next multiple of 32 (its last step reads them); stores
//     outside the M x N result are dropped.
//   * Tiles are numbered XCD-contiguously in groups of 8 row panels, so the ~32
//     workgroups resident on one XCD share their operand steps in its L2.
//   * Epilogue: each wave stages its 128 x 64 results, rounded once to bf16, through LDS
//     and stores 16-byte row pieces (whole 128-byte lines).
#include <type_traits>

#include "device_common.h"
#include "backward.h"
#include "prefill_pre.h"

namespace qkv {

namespace {

constexpr int GM = 256, GN = 256, GK = 32;
constexpr int kGThreads = 512;
constexpr int kGStep = 256 * GK * 2;  // bytes of one operand's step: [256][32] or [32][256] bf16
constexpr int kGStages = 4;
constexpr int kGABase = 0;
constexpr int kGBBase = kGStages * kGStep;
constexpr int kGLds = 2 * kGStages * kGStep;  // 128 KB
// Row panels per tile group.  The backward's products, measured on the whole backward of the
// Llama-7B shape: 2 / 4 / 8 / 16 panels -> 1472-1492 / 1428-1451 / 1421-1436 / 1452-1470 us,
// and on another box 3 / 5 / 6 / 8 / 12 -> 1493-1518 / 1487-1505 / 1466-1487 / 1452-1473 /
// 1476-1494 us.  The pre-pass form's kernel, same box (Qwen-7B, Llama-7B pairs): 3 / 5 / 6 / 8 /
// 12 -> 1190 / 1185-1186 / 1189-1191 / 1190-1191 / 1211-1212 us and 617 / 612-613 / 612-615 /
// 621-623 / 619-623 us.
constexpr int kGGroupM = 8, kGPreGroupM = 5;
constexpr uint32_t kOutside = 0x80000000u;  // a byte offset past every operand (all are < 2^31 bytes)

// kTiled: the pre-pass's bf16(x * w_norm), stored per 256-row panel and 32-wide k step
// in exactly the kRowK staging order ([panels][K / 32][256 rows][64 B], chunk c of row r
// at c ^ ((r >> 1) & 3)), so each DMA instruction reads 1 KB of consecutive bytes.
constexpr int kRowK = 0, kKRow = 1, kTiled = 2;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int N>
__device__ __forceinline__ void gwait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// [256][64 B] staging of a kRowK step: chunk c of row r at c ^ ((r >> 1) & 3).  Bits 1-2
// of the row leave the 16 x 16 x 32 fragment reads (lane l: row l % 16, chunk l / 16)
// free of bank conflicts; bits 2-3 cost about 4 conflict cycles per read (measured:
// 19.9% of the pre-normalised kernel's CU cycles).
__device__ __forceinline__ uint32_t rowk_off(uint32_t row, uint32_t chunk) {
  return row * 64u + ((chunk ^ ((row >> 1) & 3u)) << 4);
}
// [32][512 B] staging of a kKRow step: chunk c of k row r at c ^ 2 ((r mod 4) + 4 ((r / 8)
// mod 4)), so the 16 k rows of one transpose read (4 per 16-lane group, groups 8 rows
// apart) fall on distinct banks
__device__ __forceinline__ uint32_t krow_chunk(uint32_t k, uint32_t c) {
  return c ^ (((k & 3u) | (((k >> 3) & 3u) << 2)) << 1);
}

// One operand of the MFMA GEMM: its DMA offsets and fragment reads.  `org` is the
// tile's first row (kRowK) or column (kKRow) of this operand, `ld` its row pitch in
// elements, `len` the rows (kRowK) or K (kKRow) the buffer holds.
template <int kLayout>
struct Operand {
  u32x4 rsrc;
  uint32_t voff[2];   // per DMA instruction, for k = 0
  uint32_t ld2;       // row pitch in bytes
  uint32_t kbytes;    // kRowK: K in bytes (steps at or past it are sent outside the buffer)

  __device__ void init(const void* p, int org, int ld, int len, int K, int wave, int lane) {
    const uint64_t base = reinterpret_cast<uint64_t>(p);
    rsrc = u32x4{(uint32_t)base, (uint32_t)(base >> 32), (uint32_t)len * (uint32_t)ld * 2u, (uint32_t)kBufferWord3};
    ld2 = (uint32_t)ld * 2u;
    kbytes = (uint32_t)K * 2u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (kLayout == kRowK) {
        // instruction i of wave w fills rows 32w + 16i .. +15; lane l physical chunk l % 4
        // of row 32w + 16i + l / 4
        const uint32_t r = 32u * wave + 16u * i + (lane >> 2);
        const uint32_t c = ((uint32_t)lane & 3u) ^ ((r >> 1) & 3u);
        voff[i] = ((uint32_t)org + r) * ld2 + c * 16u;
      } else if constexpr (kLayout == kTiled) {
        // the panel of rows org .. org + 255 (org a multiple of 256), then the same 1 KB
        // as in LDS: instruction i of wave w, 16 bytes per lane
        voff[i] = (uint32_t)(org / 256) * (uint32_t)K * 512u + (32u * wave + 16u * i) * 64u + 16u * (uint32_t)lane;
      } else {
        // instruction i of wave w fills k rows 4w + 2i, +1; lane l physical chunk l % 32
        // of row 4w + 2i + l / 32
        const uint32_t k = 4u * wave + 2u * i + (lane >> 5);
        const uint32_t c = krow_chunk(k, (uint32_t)lane & 31u);
        voff[i] = k * ld2 + ((uint32_t)org + 8u * c) * 2u;
      }
    }
  }

  // DMA of step t into ring slot `stage` at LDS byte `lds_base` (wave-uniform parts in
  // scalar registers; the whole per-lane offset in the vector operand so the buffer's
  // range check sees all of it)
  __device__ __forceinline__ void issue(int t, int stage, uint32_t lds_base, int wave) {
    const uint32_t k0 = (uint32_t)t * GK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t dst, off;
      if constexpr (kLayout == kRowK) {
        dst = lds_base + (uint32_t)stage * kGStep + (32u * wave + 16u * i) * 64u;
        off = k0 * 2u < kbytes ? voff[i] + k0 * 2u : kOutside;
      } else if constexpr (kLayout == kTiled) {
        dst = lds_base + (uint32_t)stage * kGStep + (32u * wave + 16u * i) * 64u;
        off = voff[i] + (uint32_t)t * (uint32_t)kGStep;
      } else {
        dst = lds_base + (uint32_t)stage * kGStep + (4u * wave + 2u * i) * 512u;
        off = voff[i] + k0 * ld2;
      }
      dst = __builtin_amdgcn_readfirstlane(dst);
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(dst), "v"(off), "s"(rsrc)
                   : "m0");
    }
  }
};

// Fragment of a 16-wide block (rows or columns blk..blk+15 of the operand's 256) for
// the step's 32 k: lane l gets index blk + l % 16, k 8 (l / 16) .. +7, the operand layout
// of v_mfma_f32_16x16x32_bf16 for A rows and B columns alike.
template <int kLayout>
__device__ __forceinline__ bf16x8 read_frag(const uint8_t* stage_base, uint32_t blk, int lane) {
  if constexpr (kLayout == kRowK || kLayout == kTiled) {
    const uint32_t row = blk + ((uint32_t)lane & 15u), chunk = (uint32_t)lane >> 4;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(stage_base + rowk_off(row, chunk)));
  } else {
    // transpose reads: 16-lane group g covers k rows 8 g + 0..3 (+4 for the second read)
    // and the block's 16 indices; lane j of the group points at k row j / 4, indices
    // 4 (j % 4) .. +3, and receives index j's four k values
    const uint32_t tg = (uint32_t)lane >> 4, tj = (uint32_t)lane & 15u;
    const uint32_t k = 8u * tg + (tj >> 2);
    const uint32_t col = blk + 4u * (tj & 3u);
    const uint8_t* p = stage_base + k * 512u + krow_chunk(k, col >> 3) * 16u + (col & 7u) * 2u;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 512));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

template <int N>
using GInt = std::integral_constant<int, N>;

// Tile (m0, n0) that workgroup `bid` of a grid of one workgroup per tile owns: XCD-contiguous numbering, then groups of
// kGroup row panels, so the ~32 workgroups resident on one XCD share operand steps
// in its L2.
template <int kGroup>
__device__ __forceinline__ void gemm_tile(int tiles_m, int tiles_n, int bid, int& m0, int& n0) {
  const int G = tiles_m * tiles_n;
  const int xcd = bid & 7, local = bid >> 3;
  const int q8 = G >> 3, r8 = G & 7;
  const int L = (xcd < r8) ? xcd * (q8 + 1) + local : r8 * (q8 + 1) + (xcd - r8) * q8 + local;
  const int group = L / (kGroup * tiles_n);
  const int first_m = group * kGroup;
  const int gm = min(tiles_m - first_m, kGroup);
  const int idx = L - group * kGroup * tiles_n;
  m0 = (first_m + idx % gm) * GM;
  n0 = (idx / gm) * GN;
}

// The K loop of one 256 x 256 tile: wave (g = wave / 4) accumulates rows 128 g .. +127 of
// the tile against the four 16-column blocks of B that start at tile columns bcol[0..3],
// as 8 x 4 accumulators of v_mfma_f32_16x16x32_bf16.  `hook` runs once, after the last
// load has landed (t = nk - 2), to request the epilogue's inputs under the last two steps.
// On return every load has landed and every fragment read has returned.
template <int kLA, int kLB, class Hook>
__device__ __forceinline__ void mfma_loop(Operand<kLA>& opa, Operand<kLB>& opb, uint8_t* smem, int nk, int wave,
                                          int lane, const uint32_t (&bcol)[4], f32x4 (&acc)[8][4], Hook&& hook) {
  const int grp = wave >> 2;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 fa[8], fb[4];
  auto read_frags = [&](int stage) {
    const uint8_t* sa = smem + kGABase + stage * kGStep;
    const uint8_t* sb = smem + kGBBase + stage * kGStep;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) fa[rb] = read_frag<kLA>(sa, 128u * grp + 16u * rb, lane);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) fb[cb] = read_frag<kLB>(sb, bcol[cb], lane);
  };
  auto issue = [&](int t, int stage) {
    opa.issue(t, stage, lds0 + kGABase, wave);
    opb.issue(t, stage, lds0 + kGBBase, wave);
  };
  constexpr int kOps = 4;  // vector-memory instructions per wave and step
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  // end of a memory phase: this wave's fragment reads have returned (the other group
  // issues DMA into the ring slot this wave read one step earlier right after it),
  // while its DMA stays in flight
  auto raw_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Step t (t % 4 == P).  Memory phase: fragments of step t from slot P; issue step
  // t + 3 into slot (t + 3) % 4, which held step t - 1: this group read it in its
  // previous memory phase and the other group in the memory phase that ended at the
  // last barrier.  Per wave the DMA order is ..., t + 1, t + 2, t + 3, so this wave's
  // part of step t + 1 has landed once at most 2 kOps instructions are outstanding, and
  // every wave's part has before the barrier after which step t + 1 is first read.
  // Mode: 0 issue t + 3; 1 nothing to issue (t = nk - 3); 2 wait for the last step
  // (t = nk - 2); 3 the last step.
  auto step = [&](auto Pc, int t, auto ModeC) {
    constexpr int P = decltype(Pc)::value;
    constexpr int kMode = decltype(ModeC)::value;
    read_frags(P);
    if constexpr (kMode == 0) {
      issue(t + 3, (P + 3) & 3);
      gwait_vmcnt<2 * kOps>();
    } else if constexpr (kMode == 1) {
      gwait_vmcnt<kOps>();
    } else if constexpr (kMode == 2) {
      gwait_vmcnt<0>();
      hook();
    }
    raw_barrier();
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int rb = i >> 2, cb = i & 3;
      acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[rb], fb[cb], acc[rb][cb], 0, 0, 0);
    }
    barrier();
  };

  // prologue: steps 0..2 issued, this wave's part of step 0 landed
#pragma unroll
  for (int s = 0; s < 3; ++s) issue(s, s);
  gwait_vmcnt<2 * kOps>();
  barrier();
  // waves 4-7 start one phase late
  if (grp == 1) barrier();
  int t = 0;
  for (; t < nk - 4; t += 4) {
    step(GInt<0>{}, t, GInt<0>{});
    step(GInt<1>{}, t + 1, GInt<0>{});
    step(GInt<2>{}, t + 2, GInt<0>{});
    step(GInt<3>{}, t + 3, GInt<0>{});
  }
  step(GInt<0>{}, t, GInt<0>{});
  step(GInt<1>{}, t + 1, GInt<1>{});
  step(GInt<2>{}, t + 2, GInt<2>{});
  step(GInt<3>{}, t + 3, GInt<3>{});
  if (grp == 0) barrier();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The thread index of a tile body passes through an empty asm, so that nothing derived
// from it is hoisted out of the persistent tile loop and kept live across tiles.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

template <int kLA, int kLB>
__device__ __forceinline__ void gemm_mfma_tile(const GemmArgs& g, int tiles_m, int tiles_n, int nk, int bid) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kGLds];
  int m0, n0;
  gemm_tile<kGGroupM>(tiles_m, tiles_n, bid, m0, n0);
  const int tid = opaque_tid(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, slot = wave & 3;

  Operand<kLA> opa;
  Operand<kLB> opb;
  // A: rows m of the result; kRowK holds them as rows of length K, kKRow as columns
  opa.init(g.a, m0, g.lda, kLA == kRowK ? g.M : g.K, g.K, wave, lane);
  opb.init(g.b, n0, g.ldb, kLB == kRowK ? g.N : g.K, g.K, wave, lane);
  // wave (g, s) owns columns 64 s .. +63
  const uint32_t bcol[4] = {64u * slot, 64u * slot + 16u, 64u * slot + 32u, 64u * slot + 48u};
  f32x4 acc[8][4];
  mfma_loop(opa, opb, smem, nk, wave, lane, bcol, acc, [] {});

  // ---- epilogue through LDS: the rings are free (every wave's last fragment reads
  // returned before the last barrier).  Accumulator register i of lane l is row
  // 4 (l / 16) + i, column l % 16 of its 16 x 16 block.  Each wave stages its 128 x 64
  // results, rounded once to bf16, in a private 16 KB region (128-byte rows), column bits
  // 4-5 XOR-ed with bits 2-3 of the row (the four 16-lane groups write rows 4 apart,
  // which then land on different banks), reads them back as 16-byte row pieces and
  // stores those: whole 128-byte lines.
  uint8_t* ws = smem + wave * 16384;
  const uint32_t swz = ((uint32_t)lane >> 4) << 4;  // 16 ((row >> 2) & 3) of every row this lane writes
  const auto c_rsrc = make_rsrc(g.c, (uint32_t)g.M * (uint32_t)g.ldc * 2u);
  // row scales of the lane's 32 rows (1 without row_scale; rows past M read 0)
  float rsc[8][4];
  if (g.row_scale) {
    const auto s_rsrc = make_rsrc(g.row_scale, (uint32_t)g.M * 2u);
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t grow = (uint32_t)(m0 + 128 * grp) + 16u * rb + 4u * ((uint32_t)lane >> 4) + i;
        rsc[rb][i] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(s_rsrc, (int)(grow * 2u), 0, 0));
      }
  } else {
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) rsc[rb][i] = 1.f;
  }
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t row = 16u * rb + 4u * ((uint32_t)lane >> 4) + i;
        const uint32_t col = (16u * cb + ((uint32_t)lane & 15u)) ^ swz;
        // the element is copied out as a float first (a bit cast taken straight from a
        // vector element has been miscompiled); then scaled in fp32 and rounded once
        const float v = acc[rb][cb][i] * rsc[rb][i];
        *reinterpret_cast<uint16_t*>(ws + row * 128u + col * 2u) = f32_to_bf16(v);
      }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t row = 8u * j + ((uint32_t)lane >> 3), q = (uint32_t)lane & 7u;
    const uint32_t pc = (8u * q) ^ (((row >> 2) & 3u) << 4);
    const u32x4 v = *reinterpret_cast<const u32x4*>(ws + row * 128u + pc * 2u);
    const int grow = m0 + 128 * grp + (int)row, gcol = n0 + 64 * slot + 8 * (int)q;
    // rows past M fall outside the buffer's range; columns past N are sent outside it
    const uint32_t off = gcol < g.N ? ((uint32_t)grow * (uint32_t)g.ldc + (uint32_t)gcol) * 2u : kOutside;
    // non-temporal: measured on the Llama-7B backward (A/B, 6 calls each), 1451-1470 against
    // 1458-1487 us
    buf_store16_nt(v, c_rsrc, off);
  }
}

// Persistent over tiles, as the single-launch prefill kernel: at most one workgroup per CU
// (a multiple of 8) takes the tiles a grid of one workgroup per tile would start, in that
// order; no workgroup waits for another.
template <int kLA, int kLB>
__global__ __launch_bounds__(kGThreads, 1) void gemm_mfma_kernel(GemmArgs g, int tiles_m, int tiles_n, int nk) {
  const int G = tiles_m * tiles_n;
  for (int vb = blockIdx.x; vb < G; vb += (int)gridDim.x) {
    gemm_mfma_tile<kLA, kLB>(g, tiles_m, tiles_n, nk, vb);
    __syncthreads();  // the next tile's first steps overwrite the output staging
  }
}

// ---- the pre-normalised QKV forward on the same loop (the opt-in pre-pass form): A is
// the pre-pass's tiled bf16(x * w_norm) [T_pad, H], B the weight [H, N].  Wave (g, s)
// holds rows 128 g .. +127 and two 32-column halves d/2 apart, so both members of every
// rotation pair sit in the same lane and register of accumulator blocks cb and cb + 2.
// Epilogue: y = acc * r[t] + bias, Q and K pairs rotated with cos/sin of
// pos * theta^(-2i/d) (turn count in fp64, hardware sin/cos on the fraction of a turn),
// rounded once to bf16, staged per wave through LDS and stored as 16-byte row pieces;
// K and V rows optionally to key/value-cache slots.
template <int kD>
__device__ __forceinline__ int pre_first_half(int s) {
  static_assert(kD == 64 || kD == 128 || kD == 256, "head sizes of the kernel");
  return kD == 128 ? 128 * (s >> 1) + 32 * (s & 1) : (kD == 256 ? 32 * s : 64 * s);
}

template <int kD>
__device__ __forceinline__ void prefill_pre_tile(const ForwardArgs& a, int tiles_m, int tiles_n, int nk, int bid) {
  // the rings, then (epilogue) 8 per-wave staging regions over them and the row information
  __shared__ __attribute__((aligned(16))) uint8_t smem[kGLds + 3 * GM * 4];
  static_assert(8 * 16384 <= kGLds, "staging regions inside the rings");
  int m0, n0;
  gemm_tile<kGPreGroupM>(tiles_m, tiles_n, bid, m0, n0);
  const int tid = opaque_tid(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, slot = wave & 3;
  const int H = a.H, N = a.N, T = a.T;
  const int T_pad = tiles_m * GM;

  Operand<kTiled> opa;
  Operand<kKRow> opb;
  opa.init(a.x, m0, H, T_pad, H, wave, lane);
  opb.init(a.w, n0, N, H, H, wave, lane);
  const int fb = pre_first_half<kD>(slot);
  const uint32_t bcol[4] = {(uint32_t)fb, (uint32_t)fb + 16u, (uint32_t)(fb + kD / 2), (uint32_t)(fb + kD / 2 + 16)};

  // The epilogue's inputs, requested once the last load has landed: 1/rms, position and
  // cache slot of row tid (tid < 256), the bias of the lane's four columns and the
  // rotation frequencies of its two pairs.  Range-checked loads need no branch (rows
  // past T read 0, a plan without bias reads 0 through an empty range).
  float rinv_pref = 0.f;
  int32_t pos_pref = 0, slot_pref = -1;
  uint16_t braw[4] = {0, 0, 0, 0};
  uint64_t rev_bits[2] = {0, 0};
  auto prefetch = [&]() {
    const int row = (int)((uint32_t)(m0 + (tid & (GM - 1))) * 4u);
    rinv_pref = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.inv_rms, (uint32_t)T * 4u), row, 0, 0));
    pos_pref = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.pos, (uint32_t)T * 4u), row, 0, 0);
    slot_pref = __builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(a.slots ? a.slots : a.pos, a.slots ? (uint32_t)T * 4u : 0u), row, 0, 0);
    const auto b_rsrc = make_rsrc(a.bias ? a.bias : a.w, a.bias ? (uint32_t)N * 2u : 0u);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      braw[cb] = __builtin_amdgcn_raw_buffer_load_b16(b_rsrc, (int)((uint32_t)(n0 + (int)bcol[cb] + (lane & 15)) * 2u), 0, 0);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      rev_bits[cb] = __builtin_bit_cast(
          uint64_t, __builtin_amdgcn_raw_buffer_load_b64(make_rsrc(a.rev_freq, (kD / 2) * 8u),
                                                         (int)((uint32_t)(fb % kD + 16 * cb + (lane & 15)) * 8u), 0, 0));
  };
  f32x4 acc[8][4];
  mfma_loop(opa, opb, smem, nk, wave, lane, bcol, acc, prefetch);

  // ---- epilogue (the rings are free: every fragment read returned before the loop's
  // last barrier).  Row information of the tile's 256 rows after the 8 staging regions.
  __syncthreads();
  float* s_rinv = reinterpret_cast<float*>(smem + 8 * 16384);
  int32_t* s_pos = reinterpret_cast<int32_t*>(smem + 8 * 16384 + GM * 4);
  int32_t* s_slot = reinterpret_cast<int32_t*>(smem + 8 * 16384 + GM * 8);
  if (tid < GM) {
    s_rinv[tid] = rinv_pref;
    s_pos[tid] = pos_pref;
    s_slot[tid] = m0 + tid < T ? slot_pref : -1;  // rows past T write nothing
  }
  __syncthreads();
  float bv[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) bv[cb] = bf16_to_f32(braw[cb]);
  const double rev[2] = {__builtin_bit_cast(double, rev_bits[0]), __builtin_bit_cast(double, rev_bits[1])};
  // the wave's head lies in one of Q, K, V (their column counts are multiples of the head
  // size): Q and K heads are rotated, V heads not
  const int hcol = n0 + fb;
  const bool rotate = hcol < a.Nq + a.Nkv;
  // Staging: the wave's 128 x 64 results (columns 0-31 the first half, 32-63 the second)
  // in a private 16 KB region of 128-byte rows, column bits 4-5 XOR-ed with bits 2-3 of
  // the row (the four 16-lane groups write rows 4 apart, which then land on different
  // banks).  Accumulator register i of lane l is row 4 (l / 16) + i, column l % 16 of its
  // 16 x 16 block.
  uint8_t* ws = smem + wave * 16384;
  const uint32_t swz = ((uint32_t)lane >> 4) << 4;
  auto scale_rotate_stage = [&](auto RotC) {
    constexpr bool kRot = decltype(RotC)::value;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lrow = 16u * rb + 4u * ((uint32_t)lane >> 4) + i;
          const int trow = 128 * grp + (int)lrow;
          const float ri = s_rinv[trow];
          float y0 = fmaf(acc[rb][cb][i], ri, bv[cb]);
          float y1 = fmaf(acc[rb][cb + 2][i], ri, bv[cb + 2]);
          if constexpr (kRot) {
            double t = (double)s_pos[trow] * rev[cb];
            const float tf = (float)(t - floor(t));
            const float c = __builtin_amdgcn_cosf(tf), s = __builtin_amdgcn_sinf(tf);
            const float u0 = y0, v0 = y1;
            y0 = u0 * c - v0 * s;
            y1 = v0 * c + u0 * s;
          }
          const uint32_t c0 = (16u * cb + ((uint32_t)lane & 15u)) ^ swz, c1 = (32u + 16u * cb + ((uint32_t)lane & 15u)) ^ swz;
          *reinterpret_cast<uint16_t*>(ws + lrow * 128u + c0 * 2u) = f32_to_bf16(y0);
          *reinterpret_cast<uint16_t*>(ws + lrow * 128u + c1 * 2u) = f32_to_bf16(y1);
        }
      }
    }
  };
  if (rotate)
    scale_rotate_stage(std::true_type{});
  else
    scale_rotate_stage(std::false_type{});

  void* out;
  uint32_t width, ocol;
  if (hcol < a.Nq) {
    out = a.q; width = a.Nq; ocol = hcol;
  } else if (hcol < a.Nq + a.Nkv) {
    out = a.k; width = a.Nkv; ocol = hcol - a.Nq;
  } else {
    out = a.v; width = a.Nkv; ocol = hcol - a.Nq - a.Nkv;
  }
  const bool to_cache = a.slots != nullptr && hcol >= a.Nq;
  const uint32_t out_rows = to_cache ? (uint32_t)a.cache_rows : (uint32_t)T;
  const auto ro = make_rsrc(out, out_rows * width * 2u);
  // 16-byte pieces: 8 per 128-byte staged row, pieces 0-3 to the first half's columns
  // and 4-7 to the second half's (d/2 further)
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t lrow = 8u * j + ((uint32_t)lane >> 3), q = (uint32_t)lane & 7u;
    const uint32_t pc = (8u * q) ^ (((lrow >> 2) & 3u) << 4);
    const u32x4 v = *reinterpret_cast<const u32x4*>(ws + lrow * 128u + pc * 2u);
    const int trow = 128 * grp + (int)lrow;
    uint32_t orow = (uint32_t)(m0 + trow);
    if (to_cache) {
      const int32_t sr = s_slot[trow];
      orow = sr >= 0 && sr < a.cache_rows ? (uint32_t)sr : out_rows;
    } else if (m0 + trow >= T) {
      orow = out_rows;  // past the buffer's range: dropped
    }
    const uint32_t col = ocol + (q < 4 ? 8u * q : (uint32_t)(kD / 2) + 8u * (q - 4));
    buf_store16_nt(v, ro, (orow * width + col) * 2u);
  }
}

template <int kD>
__global__ __launch_bounds__(kGThreads, 1) void prefill_pre_kernel(ForwardArgs a, int tiles_m, int tiles_n, int nk) {
  const int G = tiles_m * tiles_n;
  for (int vb = blockIdx.x; vb < G; vb += (int)gridDim.x) {
    prefill_pre_tile<kD>(a, tiles_m, tiles_n, nk, vb);
    __syncthreads();  // the next tile's first steps overwrite the output staging
  }
}

// ---- plain FMA GEMM: 64 x 64 tile per 256-thread block, 4 x 4 results per thread,
// K in chunks of 16 staged in LDS as fp32; results in the operands' dtype.
template <bool BF16>
__device__ __forceinline__ float gload(const void* p, size_t i) {
  if constexpr (BF16)
    return bf16_to_f32(((const uint16_t*)p)[i]);
  else
    return ((const float*)p)[i];
}

template <int kLA, int kLB, bool BF16>
__global__ __launch_bounds__(256) void gemm_fma_kernel(GemmArgs g) {
  __shared__ float sa[16][64 + 4];
  __shared__ float sb[16][64 + 4];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tm = tid >> 4, tn = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = tid + 256 * e;  // 1024 elements of each 64 x 16 tile
      const int kk = i & 15, mm = i >> 4;
      const int k = k0 + kk;
      const int m = m0 + mm, n = n0 + mm;
      float va = 0.f, vb = 0.f;
      if (k < g.K && m < g.M)
        va = gload<BF16>(g.a, kLA == kRowK ? (size_t)m * g.lda + k : (size_t)k * g.lda + m);
      if (k < g.K && n < g.N)
        vb = gload<BF16>(g.b, kLB == kRowK ? (size_t)n * g.ldb + k : (size_t)k * g.ldb + n);
      sa[kk][mm] = va;
      sb[kk][mm] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = sa[kk][tm + 16 * i];
        bv[i] = sb[kk][tn + 16 * i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + tm + 16 * i, n = n0 + tn + 16 * j;
      if (m < g.M && n < g.N) {
        const float v = g.row_scale ? acc[i][j] * gload<BF16>(g.row_scale, m) : acc[i][j];
        // the operands' dtype, rounded once for bf16
        if constexpr (BF16)
          ((uint16_t*)g.c)[(size_t)m * g.ldc + n] = f32_to_bf16(v);
        else
          ((float*)g.c)[(size_t)m * g.ldc + n] = v;
      }
    }
}

template <int kLA, int kLB>
hipError_t run_mfma(const GemmArgs& g, hipStream_t s) {
  const int tiles_m = (g.M + GM - 1) / GM, tiles_n = (g.N + GN - 1) / GN;
  const int nk = ((g.K + GK - 1) / GK + 3) / 4 * 4;  // whole groups of 4 steps; the extra read zeros
  gemm_mfma_kernel<kLA, kLB><<<dim3(persistent_grid(tiles_m * tiles_n)), dim3(kGThreads), 0, s>>>(g, tiles_m, tiles_n,
                                                                                                  nk);
  return hipGetLastError();
}

template <int kLA, int kLB>
hipError_t run_fma(const GemmArgs& g, bool bf16, hipStream_t s) {
  const dim3 grid((g.N + 63) / 64, (g.M + 63) / 64), block(256);
  if (bf16)
    gemm_fma_kernel<kLA, kLB, true><<<grid, block, 0, s>>>(g);
  else
    gemm_fma_kernel<kLA, kLB, false><<<grid, block, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace

bool prefill_pre_supports(int H, int N, int d) {
  return (d == 64 || d == 128 || d == 256) && N % GN == 0 && H % 128 == 0 && H >= 128;
}

hipError_t launch_prefill_pre(const ForwardArgs& a, hipStream_t s) {
  if (!a.prenormed || !prefill_pre_supports(a.H, a.N, a.d)) return hipErrorInvalidValue;
  const int tiles_m = (a.T + GM - 1) / GM, tiles_n = a.N / GN, nk = a.H / GK;
  const dim3 grid(persistent_grid(tiles_m * tiles_n)), block(kGThreads);
  if (a.d == 64)
    prefill_pre_kernel<64><<<grid, block, 0, s>>>(a, tiles_m, tiles_n, nk);
  else if (a.d == 256)
    prefill_pre_kernel<256><<<grid, block, 0, s>>>(a, tiles_m, tiles_n, nk);
  else
    prefill_pre_kernel<128><<<grid, block, 0, s>>>(a, tiles_m, tiles_n, nk);
  return hipGetLastError();
}

hipError_t launch_backward_gemms(const BackwardArgs& b, void* dw, hipStream_t s) {
  const int tp = backward_token_pitch(b.T);
  // dW [H, N] (plan dtype) = diag(w_norm) x^T g: M = H, N = N, K = T; x [T, H] is
  // [K][cols] and its buffer range ends at row T (the last step's rows past it read
  // zeros), g^T [N, Tp] is [rows][K] with a zero pad from T to Tp (the last step reads it
  // in whole 32-wide k pieces); w_norm scales the result rows
  GemmArgs w{};
  w.a = b.x;
  w.b = b.gy;
  w.c = dw;
  w.row_scale = b.w_norm;
  w.M = b.H;
  w.N = b.N;
  w.K = b.T;
  w.lda = b.H;
  w.ldb = tp;
  w.ldc = b.N;
  // G [T, H] (plan dtype) = g W^T: M = T, N = H, K = N; g^T [N, Tp] is [K][cols], W
  // [H, N] is [rows][K]
  GemmArgs a{};
  a.a = b.gy;
  a.b = b.w;
  a.c = b.ga;
  a.M = b.T;
  a.N = b.H;
  a.K = b.N;
  a.lda = tp;
  a.ldb = b.N;
  a.ldc = b.H;
  hipError_t e;
  if (b.bf16) {
    e = run_mfma<kKRow, kRowK>(w, s);
    if (e != hipSuccess) return e;
    // W's rows are read in whole 32-wide k steps
    if (b.N % GK == 0) return run_mfma<kKRow, kRowK>(a, s);
    return run_fma<kKRow, kRowK>(a, true, s);
  }
  e = run_fma<kKRow, kRowK>(w, false, s);
  if (e != hipSuccess) return e;
  return run_fma<kKRow, kRowK>(a, false, s);
}

}  // namespace qkv
