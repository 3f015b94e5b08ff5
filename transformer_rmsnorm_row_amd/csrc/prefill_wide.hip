// Single-launch bf16 prefill kernel for gfx950: RMS row reduction, normalise-on-load
// QKV projection, bias and rotate-half rotary embedding, Q/K/V written once.
//
// The method is the fused RMSNorm + QKV projection + RoPE kernel of the page
// "Liger-Kernel底层优化：新一代内核级推理加速引擎介绍" (section
// "融合内核是如何工作的？来看一段简化版实现", and the fused-kernel list that names
// "Fused RMSNorm + QKV Projection + RoPE"): the sum of squares over the hidden size
// gives each token's 1/rms, the normalised activations exist only in registers and
// LDS (never in HBM), the bias is added to each dot product, and each rotation pair
// (i, i + head_dim/2) is turned by the position's angle before the single store.
//
// gfx950 design:
//   * 128 x 512 output tile per 512-thread workgroup (8 waves, two per SIMD).  Every
//     wave owns all 128 rows and 64 columns: two 32-column halves kD/2 apart, so both
//     members of every rotation pair sit in the same lane and register index of two
//     accumulators.  32 v_mfma_f32_16x16x32_bf16 accumulators (8 row blocks x 4 column
//     blocks of 16 x 16) = 128 fp32 per lane.
//   * Why 512 columns: the activations are normalised on load, and each row's conversion
//     (x times the norm weight in fp32, one rounding to bf16, the squares summed for the
//     row reduction) is shared by every column of its tile.  Twice the columns of a
//     256 x 256 tile halve the conversion per matrix instruction, which leaves the
//     VALU issue slots that the 16-cycle 16 x 16 x 32 MFMA (half the accumulator traffic
//     per flop of the 32 x 32 x 16 form) needs free.  The register file caps the tile at
//     64K accumulators per workgroup, so the rows go down to 128.
//   * Ping-pong schedule: K advances 32 per step.  Waves 0-3 (columns 0-255, one per
//     SIMD) and waves 4-7 (columns 256-511) are offset by one phase: a memory phase
//     (LDS -> fragment registers, load issue, waits) and a compute phase (32 MFMAs with
//     the conversion of a later step woven in), separated by workgroup barriers, so each
//     SIMD's matrix pipe is fed by one wave while the other reads its fragments.
//   * Weight steps [32 k][512 n] (1 KB rows) go global -> LDS directly (buffer_load ...
//     lds), issued three steps ahead into a 4-deep ring; 16-byte chunk c of k row r sits
//     at chunk c ^ s(r), s(r) = 2 ((r mod 4) + 4 ((r / 8) mod 4)), so the 16 rows of a
//     transpose read (ds_read_b64_tr_b16) fall on distinct 32-byte bank groups.
//   * Normalise-on-load: each group converts half of the tile's rows of step t + 2 in
//     its compute phase of step t (x and the norm weight loaded three steps ahead, 16
//     bytes per thread), into a 4-deep ring of [128 rows][32 k] activation steps (64-byte
//     rows, 16-byte chunks XOR-ed with bits 1-2 of the row).  1/rms scales the
//     accumulator rows in the epilogue, which is the same product
//     (diag(r) X diag(w) W = diag(r) (X diag(w)) W).
//   * All vector-memory instructions of the loop are inline assembly with waits counted
//     at compile time, so prefetches stay in flight across barriers.
//   * Persistent over tiles: one workgroup per CU walks its tiles in turn, so a tile's
//     start does not wait for a new workgroup to be dispatched.
//   * Tiles are numbered so that the ~32 workgroups running at once on one XCD
//     (workgroups go round-robin over the 8 XCDs) cover 6 row panels x 5-6 column panels
//     (8 x 4 for narrow projections) and share their x and W steps in that XCD's L2.
//   * Epilogue: y = acc * r[t] + bias; Q and K pairs rotated with cos/sin of
//     pos * theta^(-2i/d) (turn count reduced in fp64, hardware sin/cos on the fraction
//     of a turn); bf16 results staged through LDS and stored with 16-byte writes, K and V
//     rows optionally to key/value-cache slots.
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace qkv {

namespace {

constexpr int WM = 128;                      // rows per tile
constexpr int WN = 512;                      // columns per tile
constexpr int WK = 32;                       // k per step
constexpr int kThreads = 512;
constexpr int kStages = 4;                   // both rings: loads issued 3 steps ahead
constexpr int kAStep = WM * WK * 2;          // 8 KB: one [128][32] bf16 activation step
constexpr int kWStep = WK * WN * 2;          // 32 KB: one [32][512] bf16 weight step
constexpr int kWRing = 0;
constexpr int kARing = kStages * kWStep;     // 128 KB
constexpr int kLoopLds = kARing + kStages * kAStep;
constexpr int kStagePitch = 272;             // 128 bf16 + 16 B pad per staged output row
constexpr int kStageBlock = WM * kStagePitch;
constexpr int kRowInfo = 4 * kStageBlock;    // per-row pos, 1/rms, cache slot after the stages
constexpr int kEpiLds = kRowInfo + WM * 12;
constexpr int kLds = kLoopLds > kEpiLds ? kLoopLds : kEpiLds;
static_assert(kLds <= 160 * 1024, "LDS budget of one workgroup");
// Row panels per tile group (the tiles of a group are numbered row panel fastest): 6 for
// projections of 24 or more column tiles, 8 for narrower ones.  Measured, single launch, us
// per forward, groups of 2 / 3 / 4 / 6 row panels on one box, then 4 / 5 / 6 / 7 / 8 / 12 /
// 16 on a slower one: Qwen-7B 1417 / 1394 / 1363 / 1351, then 1403 / 1404 / 1391 / 1389-1398 /
// 1416 / 1393 / 1395; Llama-7B 731 / 714 / 699 / 692, then 719 / 714 / 713 / 712 / 716 / 710 /
// 720.  The 12-column-tile GQA shape: 366 us with groups of 8 or 16, 369 with 4 or 6.
constexpr int kGroupMWide = 6, kGroupMNarrow = 8;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// LDS byte offset of 16-byte chunk `chunk` (0..3) of row `row` of an activation step.
// The chunk index is XOR-ed with bits 1-2 of the row: measured on gfx950, this layout
// leaves both the 16 x 16 x 32 A-fragment reads (lane l: row l % 16, chunk l / 16) and
// the conversion writes (four lanes per row) free of bank conflicts, while XOR-ing with
// bits 2-3 (the 32 x 32 x 16 kernel's layout) costs about four conflict cycles per read.
__device__ __forceinline__ uint32_t a_off(uint32_t row, uint32_t chunk) {
  return row * 64u + ((chunk ^ ((row >> 1) & 3u)) << 4);
}
// Physical 16-byte chunk of logical chunk c in k row r of a weight step (1 KB rows).
__device__ __forceinline__ uint32_t w_swz(uint32_t r) { return ((r & 3u) | (((r >> 3) & 3u) << 2)) << 1; }

__device__ __forceinline__ u32x4 lds_read16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(uint8_t* base, uint32_t off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}
__device__ __forceinline__ u32x4 asm_load16(uint32_t voff, const u32x4& rsrc) {
  u32x4 v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rsrc));
  return v;
}
__device__ __forceinline__ float turn_fraction(int32_t pos, double rev) {
  double t = (double)pos * rev;
  return (float)(t - floor(t));
}

template <int P>
using Int = std::integral_constant<int, P>;

// Tile column of the first of wave w's two 32-column halves for head size kD; the
// second, at + kD/2, holds the rotation partners of the first.  The 16 halves of the
// tile belong to the 8 waves one to one, and waves 0-3 own columns 0-255.
template <int kD>
__device__ __forceinline__ int first_half(int w) {
  static_assert(kD == 64 || kD == 128 || kD == 256, "head sizes of the kernel");
  return kD == 128 ? 128 * (w >> 1) + 32 * (w & 1) : (kD == 256 ? 256 * (w >> 2) + 32 * (w & 3) : 64 * w);
}

// kGlu: the gated MLP on the same loop (post-attention RMSNorm, then [gate | up] and
// SiLU(gate) * up).  A tile covers 256 features: each 128-column "head" h holds gate
// features 64 h .. +63 and the same up features 64 columns to the right, so a wave's two
// halves (d/2 = 64 apart) are the gate and up sums of the same features.
// One output tile: the tile that workgroup `bid` of a grid of tiles_m * tiles_n would own.
template <int kD, bool kGlu>
__device__ __forceinline__ void wide_tile(const ForwardArgs& a, int tiles_m, int tiles_n, int bid) {
  static_assert(!kGlu || kD == 128, "gated MLP: 64-feature halves");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];

  // ---- tile selection: XCD-contiguous numbering, then groups of kGroupM row panels
  const int G = tiles_m * tiles_n;
  const int xcd = bid & 7, local = bid >> 3;
  const int q8 = G >> 3, r8 = G & 7;
  const int L = (xcd < r8) ? xcd * (q8 + 1) + local : r8 * (q8 + 1) + (xcd - r8) * q8 + local;
  const int kGroupM = tiles_n >= 24 ? kGroupMWide : kGroupMNarrow;
  const int group = L / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int idx = L - group * kGroupM * tiles_n;
  const int tm = first_m + idx % gm;
  const int tn = idx / gm;
  const int m0 = tm * WM, n0 = tn * WN;

  // The thread index is made opaque to the compiler, so that nothing derived from it
  // is hoisted out of the caller's tile loop and kept live (in spilled registers)
  // across tiles.
  int tid_opaque = threadIdx.x;
  asm volatile("" : "+v"(tid_opaque));
  const int tid = tid_opaque;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int grp = wave >> 2;
  const int fb = first_half<kD>(wave);  // tile column of the wave's first 32-column half
  const int H = a.H, N = a.N, T = a.T;
  const int nk = H / WK;  // multiple of 4, at least 4

  // ---- activation staging: thread u of its group converts 16-byte chunk kc of row
  // 64 grp + u / 4 of each step
  const uint32_t u = tid & 255, kc = u & 3;
  const uint32_t crow = 64u * grp + (u >> 2);
  const uint32_t x_voff = ((uint32_t)(m0 + crow) * H + kc * 8u) * 2u;
  const uint32_t a_woff = kARing + a_off(crow, kc);

  // ---- weight DMA: wave w fills k rows 4w .. 4w + 3 of each step, one 1 KB row per
  // instruction; lane l writes physical chunk l of the row, i.e. logical chunk l ^ s(row)
  uint32_t b_voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t kr = 4u * wave + i;
    uint32_t col = n0 + 8u * (lane ^ w_swz(kr));
    if constexpr (kGlu) {
      // logical chunk c: head c / 16, column 8 (c % 16) of it, gate below 64, up above
      const uint32_t c = lane ^ w_swz(kr), wi = (c & 15u) * 8u;
      const uint32_t f = 256u * (uint32_t)tn + 64u * (c >> 4) + (wi & 63u);
      col = wi < 64u ? f : (uint32_t)(N / 2) + f;
    }
    b_voff[i] = (kr * N + col) * 2u;
  }
  const uint64_t wbase = reinterpret_cast<uint64_t>(a.w);
  const u32x4 w_rsrc = {(uint32_t)wbase, (uint32_t)(wbase >> 32), (uint32_t)H * (uint32_t)N * 2u,
                        (uint32_t)kBufferWord3};
  const uint64_t xbase = reinterpret_cast<uint64_t>(a.x), nbase = reinterpret_cast<uint64_t>(a.w_norm);
  const u32x4 x_rsrc = {(uint32_t)xbase, (uint32_t)(xbase >> 32), (uint32_t)T * (uint32_t)H * 2u,
                        (uint32_t)kBufferWord3};
  const u32x4 n_rsrc = {(uint32_t)nbase, (uint32_t)(nbase >> 32), (uint32_t)H * 2u, (uint32_t)kBufferWord3};
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  // ---- fragment read offsets.  A (16 x 32 per row block): lane l reads row l % 16,
  // chunk l / 16.  B (32 x 16 per column block) by transpose reads: 16-lane group g
  // covers k rows 8g + 4h + 0..3 and the block's 16 columns; lane j of the group points
  // at row j / 4, columns 4 (j % 4) .. + 3, and receives column j's four k values.
  const uint32_t a_roff = kARing + a_off(lane & 15, lane >> 4);
  const uint32_t tg = lane >> 4, tj = lane & 15;
  uint32_t b_roff[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const uint32_t krow = 8u * tg + (tj >> 2);
    const uint32_t col = (uint32_t)(fb + (cb < 2 ? 16 * cb : kD / 2 + 16 * (cb - 2))) + 4u * (tj & 3);
    b_roff[cb] = kWRing + krow * 1024u + (((col >> 3) ^ w_swz(krow)) << 4) + (col & 7u) * 2u;
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;

  // Two register sets of staged x and norm weight: step s lives in set s % 2 from its
  // load (issued in the memory phase of step s - 3) until its conversion (in the compute
  // phase of step s - 2).  Loads past the end of the activations read zeros.
  u32x4 gx[2], gw[2];

  // Vector-memory work of one step: the activation part (x and norm weight, 2
  // instructions) into register set `set`, then the weight part (4 DMA instructions) into
  // ring slot `wstage`.  The waits below count these instructions.
  auto issue_x = [&](int t, int set) {
    const uint32_t k0 = (uint32_t)t * WK;
    gx[set] = asm_load16(x_voff + k0 * 2u, x_rsrc);
    gw[set] = asm_load16((k0 + kc * 8u) * 2u, n_rsrc);
  };
  auto issue_w = [&](int t, int wstage) {
    const uint32_t k0 = (uint32_t)t * WK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t dst =
          __builtin_amdgcn_readfirstlane(lds0 + kWRing + wstage * kWStep + (4 * wave + i) * 1024);
      // the whole offset goes in the per-lane operand so the buffer's range check sees it
      const uint32_t voff = b_voff[i] + k0 * (uint32_t)N * 2u;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(dst), "v"(voff), "s"(w_rsrc)
                   : "m0");
    }
  };
  // per step and wave: 2 activation + 4 weight instructions
  constexpr int kXOps = 2, kWOps = 4;
  auto tie_set = [&](int set) { asm volatile("" : "+v"(gx[set]), "+v"(gw[set])); };

  // x times the norm weight in fp32 (exact products), rounded once to bf16; the raw
  // squares go into the row sum
  auto convert = [&](int set, float* wf, int c) {
    const float lo = bf16_lo(gx[set][c]), hi = bf16_hi(gx[set][c]);
    ss = fmaf(lo, lo, fmaf(hi, hi, ss));
    return pack_bf16x2(lo * wf[2 * c], hi * wf[2 * c + 1]);
  };
  auto unpack_w = [&](int set, float* wf) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      wf[2 * c] = bf16_lo(gw[set][c]);
      wf[2 * c + 1] = bf16_hi(gw[set][c]);
    }
  };

  bf16x8 fa[8], fbr[4];
  auto read_frags = [&](int stage) {
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
      fa[rb] = __builtin_bit_cast(bf16x8, lds_read16(smem, a_roff + stage * kAStep + rb * 1024));
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const uint8_t* p = smem + b_roff[cb] + stage * kWStep;
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 1024));
      fbr[cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // Compute phase: the 32 MFMAs of one step from registers, with the conversion of
  // register set `set` into activation slot `astage` spread over the first 18 (two VALU
  // instructions under each 16-cycle MFMA) and its LDS write placed so that the last
  // MFMAs cover its latency before the barrier.
  auto compute = [&](int set, int astage, bool conv) {
    float wf[8];
    if (conv) unpack_w(set, wf);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int rb = i >> 2, cb = i & 3;
      acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[rb], fbr[cb], acc[rb][cb], 0, 0, 0);
      if (conv && i < 4) {
        o[i] = convert(set, wf, i);
        if (i == 3) lds_write16(smem, a_woff + astage * kAStep, o);
      }
    }
    if (conv) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
        if (i < 20) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);     // VALU
        if (i == 21) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);    // LDS write
      }
    }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // The epilogue's per-row and per-column inputs -- position (and cache slot) of row
  // tid, bias of this lane's four columns, rotation frequencies of its two pairs -- are
  // requested in the compute phase of step K/32 - 2, after the last loop wait, so they
  // hold no registers during the loop and their latency hides under the last two steps.
  // Range-checked buffer loads need no branch (rows past T read position 0, a plan
  // without bias reads 0 through an empty range).
  int32_t pos_pref = 0, slot_pref = -1;
  uint16_t braw[4] = {0, 0, 0, 0};
  uint64_t rev_bits[2] = {0, 0};
  auto prefetch_epilogue = [&]() {
    if constexpr (kGlu) return;  // the gated MLP needs only 1/rms
    pos_pref = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.pos, (uint32_t)T * 4u),
                                                    (int)((uint32_t)(m0 + (tid & (WM - 1))) * 4u), 0, 0);
    slot_pref = __builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(a.slots ? a.slots : a.pos, a.slots ? (uint32_t)T * 4u : 0u),
        (int)((uint32_t)(m0 + (tid & (WM - 1))) * 4u), 0, 0);
    const auto b_rsrc = make_rsrc(a.bias ? a.bias : a.w, a.bias ? (uint32_t)N * 2u : 0u);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = fb + (cb < 2 ? 16 * cb : kD / 2 + 16 * (cb - 2)) + (lane & 15);
      braw[cb] = __builtin_amdgcn_raw_buffer_load_b16(b_rsrc, (int)((uint32_t)(n0 + col) * 2u), 0, 0);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      rev_bits[cb] = __builtin_bit_cast(
          uint64_t, __builtin_amdgcn_raw_buffer_load_b64(make_rsrc(a.rev_freq, (kD / 2) * 8u),
                                                         (int)((uint32_t)(fb % kD + 16 * cb + (lane & 15)) * 8u), 0,
                                                         0));
  };

  // One step t (t % 4 == P).  Waves 0-3 run the memory phase of step t while waves
  // 4-7 run the compute phase of step t - 1, and the other way round one phase later.
  // Memory phase: read this wave's fragments of step t (activation and weight slot
  // t % 4), issue x(t + 3) into register set (t + 1) % 2 and W(t + 3) into weight slot
  // (t + 3) % 4, and wait until this wave's part of W(t + 1) has landed.  Per wave the
  // vector-memory order is ..., x(t + 1), W(t + 1), x(t + 2), W(t + 2), x(t + 3),
  // W(t + 3), so that wait is vmcnt(12).  Compute phase: wait for x(t + 2) (vmcnt(10)),
  // run the MFMAs of step t and convert this group's rows of step t + 2 into activation
  // slot (t + 2) % 4.  Both phases end at a barrier that waits for this wave's LDS
  // reads and writes but not for its loads.
  // Slot reuse: weight slot (t + 3) % 4 and activation slot (t + 2) % 4 held steps
  // t - 1 and t - 2, read in memory phases that ended (reads returned) before the
  // phases that overwrite them; register set (t + 1) % 2 was converted in the compute
  // phase of step t - 1.  Every wave has its part of W(t + 1) complete before the
  // barrier that ends its memory phase t, both groups' rows of step t + 2 are in LDS
  // before the barrier that ends the second group's compute phase t, and the first
  // reads of either come after those barriers.
  // Mode: 0 issue x(t + 3) and W(t + 3); 1 issue nothing (t = K/32 - 3); 2 no
  // conversion left (t = K/32 - 2); 3 the last step.
  auto step = [&](auto Pc, int t, auto ModeC) {
    constexpr int P = decltype(Pc)::value;
    constexpr int kMode = decltype(ModeC)::value;
    read_frags(P);
    if constexpr (kMode == 0) {
      issue_x(t + 3, (P + 1) & 1);
      issue_w(t + 3, (P + 3) & 3);
      wait_vmcnt<2 * (kXOps + kWOps)>();
    } else if constexpr (kMode == 1) {
      wait_vmcnt<kXOps + kWOps>();
    } else if constexpr (kMode == 2) {
      wait_vmcnt<0>();
    }
    barrier();
    if constexpr (kMode == 2) prefetch_epilogue();
    if constexpr (kMode == 0) {
      wait_vmcnt<kWOps + kXOps + kWOps>();
      tie_set(P & 1);
    } else if constexpr (kMode == 1) {
      wait_vmcnt<kWOps>();
      tie_set(P & 1);
    }
    compute(P & 1, (P + 2) & 3, kMode <= 1);
    barrier();
  };

  // ---- prologue: x(0), W(0), x(1), W(1) issued; x(0) converted into activation slot
  // 0; x(2), W(2) issued; x(1) converted into slot 1
  issue_x(0, 0);
  issue_w(0, 0);
  issue_x(1, 1);
  issue_w(1, 1);
  wait_vmcnt<kWOps + kXOps + kWOps>();
  tie_set(0);
  {
    float wf[8];
    unpack_w(0, wf);
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = convert(0, wf, c);
    lds_write16(smem, a_woff, o);
  }
  issue_x(2, 0);
  issue_w(2, 2);
  wait_vmcnt<kWOps + kXOps + kWOps>();
  tie_set(1);
  {
    float wf[8];
    unpack_w(1, wf);
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = convert(1, wf, c);
    lds_write16(smem, a_woff + kAStep, o);
  }
  barrier();
  // waves 4-7 start one phase late: their memory phase runs under the compute phase of
  // waves 0-3 and the other way round
  if (grp == 1) barrier();

  int t = 0;
  for (; t < nk - 4; t += 4) {
    step(Int<0>{}, t, Int<0>{});
    step(Int<1>{}, t + 1, Int<0>{});
    step(Int<2>{}, t + 2, Int<0>{});
    step(Int<3>{}, t + 3, Int<0>{});
  }
  step(Int<0>{}, t, Int<0>{});
  step(Int<1>{}, t + 1, Int<1>{});
  step(Int<2>{}, t + 2, Int<2>{});
  step(Int<3>{}, t + 3, Int<3>{});
  if (grp == 0) barrier();

  // Every load has landed by now; the wait, tied to the staging registers, keeps the
  // compiler from handing those registers to the epilogue ahead of it.
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(gx[0]), "+v"(gw[0]), "+v"(gx[1]), "+v"(gw[1]) : : "memory");
  __syncthreads();
  int32_t* s_pos = reinterpret_cast<int32_t*>(smem + kRowInfo);
  float* s_rinv = reinterpret_cast<float*>(smem + kRowInfo + WM * 4);
  int32_t* s_slot = reinterpret_cast<int32_t*>(smem + kRowInfo + WM * 8);
  {
    // the four lanes holding the chunks of a row are adjacent (kc = lane % 4)
    float v = ss;
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    if (kc == 0) s_rinv[crow] = rsqrtf(v / (float)H + a.eps);
    if (tid < WM) {
      s_pos[tid] = pos_pref;
      s_slot[tid] = m0 + tid < T ? slot_pref : -1;  // rows past T write nothing
    }
  }
  __syncthreads();

  if constexpr (kGlu) {
    // ---- gated-MLP epilogue: out = SiLU(g) * u with g, u the gate and up sums scaled by
    // 1/rms; staged as bf16 in two 128-feature blocks, stored with 16-byte writes to
    // out [T, N / 2]
    const int fbase = 64 * (wave >> 1) + 32 * (wave & 1);  // the wave's first feature in the tile
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      const int rbase = 16 * rb + 4 * (lane >> 4);
      const f32x4 ri4 = *reinterpret_cast<const f32x4*>(s_rinv + rbase);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int fc = fbase + 16 * cb + (lane & 15);
        uint8_t* st = smem + (fc >> 7) * kStageBlock + (fc & 127) * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[rb][cb][i] * ri4[i], up = acc[rb][cb + 2][i] * ri4[i];
          const float o = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * up;
          *reinterpret_cast<uint16_t*>(st + (rbase + i) * kStagePitch) = f32_to_bf16(o);
        }
      }
    }
    __syncthreads();
    // wave w stores rows 32 (w % 4) .. + 31 of feature block w / 4: 16 lanes of 16 bytes
    // per 256-byte row; rows past T fall outside the buffer's range
    const uint32_t I = (uint32_t)N / 2u;
    const auto ro = make_rsrc(a.q, (uint32_t)T * I * 2u);
    const int blk = wave >> 2;
    const uint8_t* stage = smem + blk * kStageBlock;
    const uint32_t ch = lane & 15;
    const uint32_t fcol = 256u * (uint32_t)tn + 128u * (uint32_t)blk;
#pragma unroll 4
    for (int it = 0; it < 8; ++it) {
      const uint32_t row = 32u * (wave & 3) + 4u * it + (lane >> 4);
      const u32x4 v = lds_read16(stage, row * kStagePitch + ch * 16u);
      buf_store16_nt(v, ro, (((uint32_t)m0 + row) * I + fcol + ch * 8u) * 2u);
    }
  } else {
  // ---- epilogue: scale, bias, rotate, stage as bf16 per 128-column block, store
  float bcol[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) bcol[cb] = bf16_to_f32(braw[cb]);
  const double rev[2] = {__builtin_bit_cast(double, rev_bits[0]), __builtin_bit_cast(double, rev_bits[1])};
  // the wave's head lies in one of Q, K, V (their column counts are multiples of the
  // head size): Q and K heads are rotated, V heads not
  const bool rotate = n0 + fb < a.Nq + a.Nkv;
  auto scale_rotate_stage = [&](auto RotC) {
    constexpr bool kRot = decltype(RotC)::value;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      const int rbase = 16 * rb + 4 * (lane >> 4);
      const f32x4 ri4 = *reinterpret_cast<const f32x4*>(s_rinv + rbase);
      const i32x4 p4 = *reinterpret_cast<const i32x4*>(s_pos + rbase);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int c0 = fb + 16 * cb + (lane & 15), c1 = c0 + kD / 2;
        uint8_t* st0 = smem + (c0 >> 7) * kStageBlock + (c0 & 127) * 2;
        uint8_t* st1 = smem + (c1 >> 7) * kStageBlock + (c1 & 127) * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float y0 = fmaf(acc[rb][cb][i], ri4[i], bcol[cb]);
          float y1 = fmaf(acc[rb][cb + 2][i], ri4[i], bcol[cb + 2]);
          if constexpr (kRot) {
            const float tf = turn_fraction(p4[i], rev[cb]);
            const float c = __builtin_amdgcn_cosf(tf), s = __builtin_amdgcn_sinf(tf);
            const float u0 = y0, v0 = y1;
            y0 = u0 * c - v0 * s;
            y1 = v0 * c + u0 * s;
          }
          *reinterpret_cast<uint16_t*>(st0 + (rbase + i) * kStagePitch) = f32_to_bf16(y0);
          *reinterpret_cast<uint16_t*>(st1 + (rbase + i) * kStagePitch) = f32_to_bf16(y1);
        }
      }
    }
  };
  if (rotate)
    scale_rotate_stage(std::true_type{});
  else
    scale_rotate_stage(std::false_type{});
  __syncthreads();

  // wave w stores rows 64 (w % 2) .. + 63 of 128-column block w / 2: 16 lanes of 16
  // bytes per 256-byte row.  K and V rows go to their cache slots when the forward has
  // them; a row index of out_rows or more lies past the buffer's range, so that store
  // is dropped.
  const int blk = wave >> 1;
  const int hcol = n0 + 128 * blk;
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
  const uint8_t* stage = smem + blk * kStageBlock;
  const uint32_t ch = lane & 15;
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
    const uint32_t row = 64u * (wave & 1) + 4u * it + (lane >> 4);
    const u32x4 v = lds_read16(stage, row * kStagePitch + ch * 16u);
    uint32_t orow = (uint32_t)m0 + row;
    if (to_cache) {
      const int32_t sr = s_slot[row];
      orow = sr >= 0 && sr < a.cache_rows ? (uint32_t)sr : out_rows;
    }
    buf_store16_nt(v, ro, (orow * width + ocol + ch * 8u) * 2u);
  }
  }
}

// Persistent over tiles: a grid of at most one workgroup per CU (a multiple of 8, so a
// workgroup's XCD is the same for all its tiles) walks the tiles in the order a grid of
// one workgroup per tile would start them, so the workgroups running at once on an XCD
// still share a tile group.  No workgroup waits for another.  Against one workgroup per
// tile (measured, outputs bit-identical; two boxes): Qwen-7B 1368-1369 -> 1343-1344 and
// 1333-1334 -> 1317-1318 us, Llama-7B 698-700 -> 684-686 and 683-684 -> 666-667 us, the
// GQA shape 371 -> 364 and 362 -> 355.5 us, the Llama-7B gated MLP 1241-1243 -> 1217-1218
// and 1209-1212 -> 1185-1190 us.
template <int kD, bool kGlu = false>
__global__ __launch_bounds__(kThreads, 1) void prefill_wide_kernel(ForwardArgs a, int tiles_m, int tiles_n) {
  const int G = tiles_m * tiles_n;
  for (int vb = blockIdx.x; vb < G; vb += (int)gridDim.x) {
    wide_tile<kD, kGlu>(a, tiles_m, tiles_n, vb);
    __syncthreads();  // the next tile's first weight steps overwrite the output staging
  }
}


}  // namespace

int persistent_grid(int tiles) {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return tiles;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) return tiles;
    c = n - n % 8;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return tiles < c ? tiles : c;
}

bool prefill_wide_supports(int H, int N, int Nq, int Nkv, int d) {
  return (d == 64 || d == 128 || d == 256) && H % (4 * WK) == 0 && N % WN == 0 && Nq % 128 == 0 &&
         Nkv % 128 == 0 && Nq % d == 0 && Nkv % d == 0;
}

bool swiglu_wide_supports(int H, int I) { return H % (4 * WK) == 0 && (2 * I) % WN == 0; }

hipError_t launch_swiglu_wide(const ForwardArgs& a, hipStream_t stream) {
  // a.N = 2I columns of [gate | up]; the output (a.q) is [T, I]
  if (!swiglu_wide_supports(a.H, a.N / 2)) return hipErrorInvalidValue;
  const int tiles_m = (a.T + WM - 1) / WM, tiles_n = a.N / WN;
  prefill_wide_kernel<128, true><<<dim3(persistent_grid(tiles_m * tiles_n)), dim3(kThreads), 0, stream>>>(a, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_prefill_wide(const ForwardArgs& a, hipStream_t stream) {
  const int tiles_m = (a.T + WM - 1) / WM, tiles_n = a.N / WN;
  const dim3 grid(persistent_grid(tiles_m * tiles_n)), block(kThreads);
  if (a.d == 64)
    prefill_wide_kernel<64><<<grid, block, 0, stream>>>(a, tiles_m, tiles_n);
  else if (a.d == 256)
    prefill_wide_kernel<256><<<grid, block, 0, stream>>>(a, tiles_m, tiles_n);
  else
    prefill_wide_kernel<128><<<grid, block, 0, stream>>>(a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace qkv
