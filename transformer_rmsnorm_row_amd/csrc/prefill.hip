// bf16 MFMA prefill kernel for gfx950 on 256 x 256 tiles: RMS row reduction,
// normalise-on-load QKV projection, bias and rotate-half rotary embedding, Q/K/V
// written once.  It serves the prefill shapes the 128 x 512 kernel of prefill_wide.hip
// does not take, the split-K form for token counts too small to fill the chip, and the
// gated MLP epilogue.
//
// The method is the fused RMSNorm + QKV projection + RoPE kernel of the page
// "Liger-Kernel底层优化：新一代内核级推理加速引擎介绍" (section
// "融合内核是如何工作的？来看一段简化版实现", and the fused-kernel list that names
// "Fused RMSNorm + QKV Projection + RoPE"): the sum of squares over the hidden size
// gives each token's 1/rms, the bias is added to each dot product, and each rotation pair
// (i, i + head_dim/2) is turned by the position's angle before the single store.  The
// normalised activations exist only inside the kernel.
//
// gfx950 design (the listing's one-thread-per-feature loop is not used):
//   * 256 x 256 output tile per 512-thread workgroup (8 waves, two per SIMD).  Wave
//     (g, s) owns rows 128g..128g+127 and, of head s/2 of the tile, the 32-column
//     blocks starting at 32(s%2) and 32(s%2) + 64: both halves of every rotation pair
//     sit in the same lane, in the same register of two accumulators.  8 x
//     v_mfma_f32_32x32x16_bf16 accumulators = 128 fp32 per lane.
//   * Ping-pong schedule: K advances 32 per step; waves 0-3 (one per SIMD) and
//     waves 4-7 alternate between a memory phase (LDS -> fragment registers, load
//     issue, waits) and a compute phase (16 MFMAs from registers with the staging
//     arithmetic woven in), separated by workgroup barriers, so each SIMD's matrix
//     pipe is fed by one wave while the other wave reads its next fragments.
//   * Weight steps [32 k][256 n] go global -> LDS directly (buffer_load ... lds),
//     issued three steps ahead into a 4-deep ring, 16-byte chunks XOR-swizzled by
//     k mod 4 so that the MFMA B fragments are read conflict-free with
//     ds_read_b64_tr_b16 (LDS transpose reads).
//   * Normalise-on-load: x is loaded into registers two steps ahead, multiplied by
//     its norm weight in fp32 (exact products), rounded once to bf16 and written to
//     a 2-deep activation ring; the same registers give the row sums of squares, so
//     1/rms needs no separate pass.  1/rms scales the accumulator rows in the
//     epilogue, which is the same product (diag(r) X diag(w) W = diag(r) (X diag(w)) W).
//   * All vector-memory instructions of the loop are inline assembly with waits
//     counted at compile time, so prefetches stay in flight across barriers.
//   * Tiles are numbered so that the ~32 workgroups running at once on one XCD
//     (workgroups go round-robin over the 8 XCDs) cover 4 row panels x 8 column
//     panels and share them in that XCD's L2.
//   * Epilogue: y = acc * r[t] + bias; Q and K pairs rotated with cos/sin of
//     pos * theta^(-2i/d) (turn count reduced in fp64, hardware sin/cos on the
//     fraction of a turn); bf16 results staged through LDS and stored with 16-byte
//     writes.
//   * Split-K form (kSplit = 2), for token counts whose tiles number at most 128 and
//     would leave most CUs idle: the two halves of a tile's K range run in two
//     workgroups; each stores its fp32 partial tile and partial row sums of squares to
//     plan scratch and counts itself in, and the second to arrive adds the other's
//     partial to its own registers (two terms commute, so the result does not depend
//     on the arrival order) before the same epilogue.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace qkv {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;
constexpr int kThreads = 512;
constexpr int kStep = BM * BK * 2;                  // bytes of one [256][32] or [32][256] bf16 step
constexpr int kWStages = 4;                         // weight steps: DMA issued 3 steps ahead
constexpr int kAStages = 2;                         // converted activation steps
constexpr int kWBase = 0;
constexpr int kABase = kWStages * kStep;
constexpr int kStagePitch = 272;                    // 128 bf16 + 16 B pad per staged output row
constexpr int kBlockStage = 128 * kStagePitch;      // one group's 128 rows x one head
constexpr int kRowInfo = 4 * kBlockStage;           // per-row pos, 1/rms, cache slot after the staging area
constexpr int kLds = kRowInfo + BM * 12;
static_assert(kABase + kAStages * kStep <= kLds, "loop rings must fit");
static_assert(kLds <= 160 * 1024, "LDS budget of one workgroup");
// Row panels per tile group (2 was slower for the 6144-column GQA shape and for the
// gated MLP).
constexpr int kGroupM = 4;

// LDS byte offset of 16-byte chunk `chunk` (0..3) of row `row` in a [256][32] bf16
// activation step (64 B rows).  The chunk index is XOR-ed with bits 2..3 of the row,
// so the 16 rows read by 16 lanes of a fragment read cover all banks.
__device__ __forceinline__ uint32_t a_off(uint32_t row, uint32_t chunk) {
  return row * 64u + ((chunk ^ ((row >> 2) & 3u)) << 4);
}
// The weight step stays [32 k][256 n] (512 B rows) as loaded; 16-byte chunk c of
// row k sits at chunk c ^ 4*(k mod 4), which spreads the 4-row x 16-column blocks
// of a transpose read over all banks.
__device__ __forceinline__ uint32_t wchunk(uint32_t k, uint32_t c) { return c ^ ((k & 3u) << 2); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

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

// Epilogues sharing the normalise-on-load GEMM: the attention-input chain (bias,
// rotary embedding, Q/K/V stores) and the gated MLP (SiLU(gate) * up).
constexpr int kEpiQkv = 0, kEpiSwiglu = 1;

// Tile column of the first of a wave's two 32-column blocks for head size kD; the
// second block, at + kD/2, holds the rotation partners of the first.  Each 32-column
// block of the tile belongs to exactly one wave of a row group.
template <int kD>
__device__ __forceinline__ int pair_block(int slot) {
  static_assert(kD == 64 || kD == 128 || kD == 256, "head sizes of the MFMA kernel");
  return kD == 128 ? 128 * (slot >> 1) + 32 * (slot & 1) : (kD == 256 ? 32 * slot : 64 * slot);
}

// Floats of one partial tile of the split-K form: the 256 x 256 fp32 sums, then the
// 256 rows' partial sums of squares.
constexpr int kPartFloats = BM * BN + BM;

template <int kEpi, int kD, int kSplit>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(ForwardArgs a, int tiles_m, int tiles_n) {
  constexpr bool kSplitK = kSplit > 1;
  constexpr int nsplit = kSplit;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  __shared__ int s_last;

  // ---- tile selection: XCD-contiguous numbering, then groups of kGroupM row panels.
  // Split-K form: workgroup b takes K slice b % nsplit of tile b / nsplit.
  const int G = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  int L, ks = 0;
  if constexpr (kSplitK) {
    L = bid / nsplit;
    ks = bid % nsplit;
  } else {
    const int xcd = bid & 7, local = bid >> 3;
    const int q8 = G >> 3, r8 = G & 7;
    L = (xcd < r8) ? xcd * (q8 + 1) + local : r8 * (q8 + 1) + (xcd - r8) * q8 + local;
  }
  const int group_m = kGroupM;
  const int group = L / (group_m * tiles_n);
  const int first_m = group * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int idx = L - group * group_m * tiles_n;
  const int tm = first_m + idx % gm;
  const int tn = idx / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int grp = wave >> 2, slot = wave & 3;
  const int head = slot >> 1;          // which 128-column half of the tile this wave stores
  const int blk = pair_block<kD>(slot);  // tile column of the wave's first block
  const int c0 = blk % kD;             // first rotation-pair index of this wave
  const int H = a.H, N = a.N, T = a.T;
  // 32-row steps of this workgroup's K range: all of H, or slice ks of nsplit
  const int nk = kSplitK ? H / BK / nsplit : H / BK;  // multiple of 4, at least 4
  const uint32_t kofs = kSplitK ? (uint32_t)(ks * nk * BK) : 0u;  // first k of the range
  const uint32_t fl = lane & 31, fh = lane >> 5;

  // ---- activation staging: thread u of its group owns chunk kc of the group's rows
  // ar and ar + 64 (tile rows 128 grp + ar + 64 j)
  const uint32_t u = tid & 255, kc = u & 3, ar = u >> 2;
  const uint32_t arow = 128u * grp + ar;
  const uint32_t x_voff = ((uint32_t)(m0 + arow) * H + kofs + kc * 8u) * 2u;
  const uint32_t x_jstep = 64u * H * 2u;
  const uint32_t a_woff = kABase + a_off(arow, kc);  // row + 64 keeps the swizzle: + 4096

  // ---- weight DMA: wave w fills rows 4w + 2i (+1) of each step, i = 0, 1; each
  // instruction is one 1 KB run of LDS = two 512 B rows, lane l filling physical
  // chunk l % 32 of row 4w + 2i + l / 32, i.e. logical chunk wchunk(row, l % 32).
  uint32_t b_voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t krow = 2u * i + (lane >> 5);  // row within the 4-row swizzle period
    uint32_t col = n0 + 8u * wchunk(krow, lane & 31);
    if constexpr (kEpi == kEpiSwiglu) {
      // tile tn covers features 128 tn .. +127; its "head" h (128 columns) holds gate
      // features 64h .. +63 in columns 0-63 and the same up features in 64-127, so each
      // lane's column pair (j, j + 64) is (gate, up) of one feature
      const uint32_t lc = wchunk(krow, lane & 31), h = lc >> 4, wi = (lc & 15u) * 8u;
      const uint32_t f = 128u * (uint32_t)tn + 64u * h + (wi & 63u);
      col = wi < 64u ? f : (uint32_t)(N / 2) + f;
    }
    b_voff[i] = ((kofs + 4u * wave + krow) * N + col) * 2u;
  }
  const uint64_t wbase = reinterpret_cast<uint64_t>(a.w);
  const u32x4 w_rsrc = {(uint32_t)wbase, (uint32_t)(wbase >> 32), (uint32_t)H * (uint32_t)N * 2u,
                        (uint32_t)kBufferWord3};
  const uint64_t xbase = reinterpret_cast<uint64_t>(a.x), nbase = reinterpret_cast<uint64_t>(a.w_norm);
  const u32x4 x_rsrc = {(uint32_t)xbase, (uint32_t)(xbase >> 32), (uint32_t)T * (uint32_t)H * 2u, (uint32_t)kBufferWord3};
  const u32x4 n_rsrc = {(uint32_t)nbase, (uint32_t)(nbase >> 32), (uint32_t)H * 2u, (uint32_t)kBufferWord3};
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  // ---- fragment read offsets (stage and 32-row block offsets are immediates)
  const uint32_t a_roff0 = kABase + a_off(128u * grp + fl, fh);      // ks = 0
  const uint32_t a_roff1 = kABase + a_off(128u * grp + fl, 2u + fh); // ks = 1
  // transpose reads of the weight: 16-lane group g covers k rows 8(g/2) + 4h + 0..3
  // and columns 16(g%2) + 0..15 of a 32-column block; lane j of the group points at
  // row j/4, columns 4(j%4)..+3.
  const uint32_t tg = lane >> 4, tj = lane & 15;
  uint32_t b_roff[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const uint32_t krow = 8u * (tg >> 1) + (tj >> 2);
    const uint32_t col = (uint32_t)(blk + (kD / 2) * cb) + 16u * (tg & 1) + 4u * (tj & 3);
    b_roff[cb] = kWBase + krow * 512u + wchunk(krow, col >> 3) * 16u + (col & 7u) * 2u;
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  float ss[2] = {0.f, 0.f};

  // Two register sets of staged activations: step t lives in set t % 2 from its
  // load (issued in the memory phase of step t - 2) until it is converted (in the
  // compute phase of step t - 1).  Loads past the end of K read zeros (outside the
  // buffer's range) or rows that are never used, so the loop needs no branch.
  u32x4 gx[2][2], gw[2];

  // Vector-memory work of one step: the weight part is 2 DMA instructions into ring
  // slot `wstage`, the activation part 2 x loads and 1 norm-weight load into register
  // set `set`.  The waits below count these instructions.
  auto issue_w = [&](int t, int wstage) {
    const uint32_t k0 = (uint32_t)t * BK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + kWBase + wstage * kStep + (4 * wave + 2 * i) * 512);
      // the whole offset goes in the per-lane operand so the buffer's range check
      // (zero fill past the end of the weight) sees all of it
      const uint32_t voff = b_voff[i] + k0 * (uint32_t)N * 2u;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(dst), "v"(voff), "s"(w_rsrc)
                   : "m0");
    }
  };
  auto issue_x = [&](int t, int set) {
    const uint32_t k0 = (uint32_t)t * BK;
    gx[set][0] = asm_load16(x_voff + k0 * 2u, x_rsrc);
    gx[set][1] = asm_load16(x_voff + x_jstep + k0 * 2u, x_rsrc);
    gw[set] = asm_load16((kofs + k0 + kc * 8u) * 2u, n_rsrc);
  };
  constexpr int kWOps = 2, kXOps = 3;
  // the registers of a set become usable only after an explicit wait
  auto tie_set = [&](int set) { asm volatile("" : "+v"(gx[set][0]), "+v"(gx[set][1]), "+v"(gw[set])); };

  // One 16 x 8 element piece of the conversion: x * norm weight in fp32 (exact
  // products), rounded once to bf16; the raw squares go into the row sums.
  auto convert_dword = [&](int set, int j, int c, const float* wf) {
    const float lo = bf16_lo(gx[set][j][c]), hi = bf16_hi(gx[set][j][c]);
    ss[j] = fmaf(lo, lo, fmaf(hi, hi, ss[j]));
    return pack_bf16x2(lo * wf[2 * c], hi * wf[2 * c + 1]);
  };

  bf16x8 fa[4][2], fb[2][2];
  auto read_frags = [&](int astage, int wstage) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t ab = (ks ? a_roff1 : a_roff0) + astage * kStep;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) fa[rb][ks] = __builtin_bit_cast(bf16x8, lds_read16(smem, ab + rb * 2048));
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const uint8_t* p = smem + b_roff[cb] + wstage * kStep + ks * 16 * 512;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 512));
        fb[cb][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  // Compute phase: the 16 MFMAs of one step from registers, with the conversion of
  // register set `set` into activation slot `astage` spread over the first 13 (at most
  // 5 VALU instructions, 20 issue cycles, under each 32-cycle MFMA) and its two LDS
  // writes placed so that the last MFMAs cover their latency before the barrier.
  auto compute = [&](int set, int astage, bool conv) {
    float wf[8];
    if (conv) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        wf[2 * c] = bf16_lo(gw[set][c]);
        wf[2 * c + 1] = bf16_hi(gw[set][c]);
      }
    }
    u32x4 o[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ks = i >> 3, rb = (i >> 1) & 3, cb = i & 1;
      acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[rb][ks], fb[cb][ks], acc[rb][cb], 0, 0, 0);
      if (conv && i < 8) {
        const int j = i >> 2, c = i & 3;
        o[j][c] = convert_dword(set, j, c, wf);
        if (c == 3) lds_write16(smem, a_woff + 4096u * j + astage * kStep, o[j]);
      }
    }
    if (conv) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (i < 13) __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
        if (i == 7 || i == 12) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
      }
    }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  // End of a memory phase: this wave's fragment reads have returned (the other group
  // issues DMA into the ring slot it read one step earlier right after this barrier),
  // while its global loads and DMA stay in flight.
  auto raw_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // One step t (t % 4 == P).  Waves 0-3 run the memory phase of step t while waves
  // 4-7 run the compute phase of step t - 1, and the other way round one phase later.
  // Memory phase: read this wave's fragments of step t (activation slot t % 2, weight
  // slot t % 4), issue x(t + 2) into register set t % 2 and W(t + 3) into weight slot
  // (t + 3) % 4, and wait until this wave's part of W(t + 1) has landed.  Per wave the
  // vector-memory order is ..., W(t + 1), x(t + 1), W(t + 2), x(t + 2), W(t + 3), so
  // that wait is vmcnt(10).  The phase ends at a barrier that waits for this wave's
  // fragment reads but not for its loads: in the next phase the other group issues its
  // part of W(t + 3) into slot (t - 1) % 4, which this wave read in its previous memory
  // phase, and the DMA must not land before those reads have returned.  Compute phase:
  // wait for x(t + 1) (vmcnt(7)), the MFMAs
  // of step t and the conversion of x(t + 1) into activation slot (t + 1) % 2, closed
  // by a full barrier so the converted rows are in LDS before this group reads them.
  // Slot reuse is safe: weight slot (t + 3) % 4 held step t - 1, which both groups
  // read in memory phases that ended, reads returned, before this phase began; activation slot
  // (t + 1) % 2 held step t - 1 of this group's rows, read in its previous memory
  // phase; register set t % 2 was converted in the previous compute phase.  Every wave
  // has its part of W(t + 1) complete before the barrier that ends its memory phase t,
  // and the first reads of W(t + 1) come after that barrier.
  // Mode: 0 issue x(t + 2) and W(t + 3); 1 issue x(t + 2) only (t = K/32 - 3);
  // 2 issue nothing and wait for everything by its compute phase (t = K/32 - 2);
  // 3 the last step.
  auto step = [&](auto Pc, int t, auto ModeC) {
    constexpr int P = decltype(Pc)::value;
    constexpr int kMode = decltype(ModeC)::value;
    constexpr bool kLast = kMode == 3;
    read_frags(P & 1, P);
    // memory phase: only this wave's part of W(t + 1) has to be complete at its end
    if constexpr (kMode == 0) {
      issue_x(t + 2, P & 1);
      issue_w(t + 3, (P + 3) & 3);
      wait_vmcnt<2 * kWOps + 2 * kXOps>();
    } else if constexpr (kMode == 1) {
      issue_x(t + 2, P & 1);
      wait_vmcnt<kWOps + 2 * kXOps>();
    } else if constexpr (kMode == 2) {
      wait_vmcnt<kXOps>();
    }
    raw_barrier();
    // compute phase: x(t + 1) in registers before its conversion; the compiler waits
    // for each fragment register before the MFMA that reads it
    if constexpr (kMode == 0) wait_vmcnt<2 * kWOps + kXOps>();
    else if constexpr (kMode == 1) wait_vmcnt<kWOps + kXOps>();
    else if constexpr (kMode == 2) wait_vmcnt<0>();
    if constexpr (!kLast) tie_set((P + 1) & 1);
    compute((P + 1) & 1, (P + 1) & 1, !kLast);
    barrier();
  };

  // The epilogue's per-row and per-column inputs, requested now so that their latency
  // hides under the main loop: position (and cache slot) of row tid, bias of this
  // lane's two columns, rotation frequency of its pair.
  // Range-checked buffer loads need no branch (rows past T read position 0, a plan
  // without bias reads 0 through an empty range), so nothing waits for them before
  // their first use in the epilogue.
  const int hcol = n0 + head * 128;  // first column of the 128-column half this wave stores
  int32_t pos_pref = 0, slot_pref = -1;
  uint16_t braw[2] = {0, 0};
  uint64_t rev_bits = 0;
  if constexpr (kEpi == kEpiQkv) {
    pos_pref = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.pos, (uint32_t)T * 4u),
                                                    (int)((uint32_t)(m0 + (tid & (BM - 1))) * 4u), 0, 0);
    slot_pref = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.slots ? a.slots : a.pos, a.slots ? (uint32_t)T * 4u : 0u),
                                                     (int)((uint32_t)(m0 + (tid & (BM - 1))) * 4u), 0, 0);
    const auto b_rsrc = make_rsrc(a.bias ? a.bias : a.w, a.bias ? (uint32_t)N * 2u : 0u);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      braw[cb] = __builtin_amdgcn_raw_buffer_load_b16(b_rsrc, (int)((uint32_t)(n0 + blk + (kD / 2) * cb + fl) * 2u), 0, 0);
    rev_bits = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(make_rsrc(a.rev_freq, (kD / 2) * 8u),
                                                                                 (int)((uint32_t)(c0 + fl) * 8u), 0, 0));
  }
  // prologue: W(0..2) and x(0..1) issued, x(0) converted into activation slot 0
  issue_w(0, 0);
  issue_x(0, 0);
  issue_w(1, 1);
  issue_x(1, 1);
  issue_w(2, 2);
  wait_vmcnt<2 * kWOps + kXOps>();
  tie_set(0);
  {
    float wf[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      wf[2 * c] = bf16_lo(gw[0][c]);
      wf[2 * c + 1] = bf16_hi(gw[0][c]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = convert_dword(0, j, c, wf);
      lds_write16(smem, a_woff + 4096u * j, o);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();
  // waves 4-7 start one phase late: their memory phase runs under the compute
  // phase of waves 0-3 and the other way round
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

  // Every load has landed by now (step K/32 - 2 waited for all of them); the wait, tied
  // to the staging registers, keeps the compiler from handing those registers to the
  // epilogue ahead of it.
  asm volatile("s_waitcnt vmcnt(0)"
               : "+v"(gx[0][0]), "+v"(gx[0][1]), "+v"(gw[0]), "+v"(gx[1][0]), "+v"(gx[1][1]), "+v"(gw[1])
               :
               : "memory");
  __syncthreads();
  int32_t* s_pos = reinterpret_cast<int32_t*>(smem + kRowInfo);
  float* s_rinv = reinterpret_cast<float*>(smem + kRowInfo + BM * 4);
  int32_t* s_slot = reinterpret_cast<int32_t*>(smem + kRowInfo + BM * 8);
  {
    // the four lanes holding the chunks of a row are adjacent (kc = lane % 4)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float v = ss[j];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      // the split-K form keeps the raw partial sum until the slices are added
      if (kc == 0) s_rinv[arow + 64u * j] = kSplitK ? v : rsqrtf(v / (float)H + a.eps);
    }
    if (tid < BM) {
      s_pos[tid] = pos_pref;
      s_slot[tid] = m0 + tid < T ? slot_pref : -1;  // rows past T write nothing
    }
  }
  __syncthreads();

  if constexpr (kSplitK) {
    // ---- split-K: this workgroup's partial tile goes to plan scratch and is counted
    // in per tile; the workgroup that arrives last adds the other slice's partial tile to
    // its own, then runs the epilogue.  Partial tile layout: 16-byte chunk j (0..31) of thread tid at
    // j * 512 + tid, chunk j holding registers 4 (j % 4) .. + 3 of accumulator j / 4;
    // then the 256 row sums of squares.  Stores and loads are device-coherent (sc1),
    // since the slices of a tile run on different XCDs.
    const uint64_t pbase = reinterpret_cast<uint64_t>(a.kpart);
    const u32x4 p_rsrc = {(uint32_t)pbase, (uint32_t)(pbase >> 32), (uint32_t)a.kpart_units * kPartFloats * 4u,
                          (uint32_t)kBufferWord3};
    // byte offsets: a wave-uniform part (partial tile, chunk) in the scalar offset
    // operand, the thread's 16 or 4 bytes in the vector one
    const uint32_t own = (uint32_t)__builtin_amdgcn_readfirstlane((L * nsplit + ks) * kPartFloats * 4);
    const uint32_t t16 = (uint32_t)tid * 16u, t4 = (uint32_t)tid * 4u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int ai = j >> 2, q4 = j & 3;
      const f32x16& ac = acc[ai >> 1][ai & 1];
      const f32x4 v = {ac[4 * q4], ac[4 * q4 + 1], ac[4 * q4 + 2], ac[4 * q4 + 3]};
      asm volatile("buffer_store_dwordx4 %0, %1, %2, %3 offen sc1" ::"v"(__builtin_bit_cast(u32x4, v)), "v"(t16),
                   "s"(p_rsrc), "s"(own + (uint32_t)(j * kThreads * 16))
                   : "memory");
    }
    if (tid < BM)
      asm volatile("buffer_store_dword %0, %1, %2, %3 offen sc1" ::"v"(s_rinv[tid]), "v"(t4), "s"(p_rsrc),
                   "s"(own + (uint32_t)(BM * BN * 4))
                   : "memory");
    // every store of the workgroup complete before it is counted in
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&a.kcount[L], 1u) == (unsigned)(nsplit - 1);
    __syncthreads();
    if (!s_last) return;
    // Two slices: the sum is own + other, and floating-point addition is commutative, so
    // the result does not depend on which workgroup arrives last.  The other slice's
    // partial tile is read in 8-chunk batches (32 KB per workgroup), double-buffered:
    // the next batch is in flight while one is added in.
    static_assert(kSplit == 2, "the reduction below adds exactly two partial tiles");
    const uint32_t other = (uint32_t)__builtin_amdgcn_readfirstlane((L * nsplit + (1 - ks)) * kPartFloats * 4);
    u32x4 buf[2][8];
#pragma unroll
    for (int b = 0; b <= 4; ++b) {
      if (b < 4) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen sc1"
                       : "=v"(buf[b & 1][jj])
                       : "v"(t16), "s"(p_rsrc), "s"(other + (uint32_t)((8 * b + jj) * kThreads * 16))
                       : "memory");
      }
      if (b == 0) continue;
      // batch b - 1 has landed once at most the 8 loads of batch b are outstanding
      if (b < 4)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const int pb = b - 1;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        asm volatile("" : "+v"(buf[pb & 1][jj]));
        const int j = 8 * pb + jj, ai = j >> 2, q4 = j & 3;
        f32x16& ac = acc[ai >> 1][ai & 1];
        const f32x4 f = __builtin_bit_cast(f32x4, buf[pb & 1][jj]);
#pragma unroll
        for (int e = 0; e < 4; ++e) ac[4 * q4 + e] += f[e];
      }
      // the batch's adds happen here, not later: its registers are free for the next
      asm volatile("" : "+v"(acc[pb][0]), "+v"(acc[pb][1]));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (tid < BM) {
      uint32_t u;
      asm volatile("buffer_load_dword %0, %1, %2, %3 offen sc1\n\ts_waitcnt vmcnt(0)"
                   : "=v"(u)
                   : "v"(t4), "s"(p_rsrc), "s"(other + (uint32_t)(BM * BN * 4))
                   : "memory");
      s_rinv[tid] = rsqrtf((s_rinv[tid] + __uint_as_float(u)) / (float)H + a.eps);
    }
    __syncthreads();
    if (tid == 0) a.kcount[L] = 0u;  // ready for the next forward through the plan
  }

  if constexpr (kEpi == kEpiSwiglu) {
    // ---- epilogue: out = SiLU(g) * u with g, u the gate and up sums scaled by 1/rms;
    // staged as bf16 per (row half, head) block of 64 features, stored with 16-byte writes
    uint8_t* stage = smem + (grp * 2 + head) * kBlockStage;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int rbase = rb * 32 + rg * 8 + (int)fh * 4;  // row within the group's 128
        const f32x4 ri4 = *reinterpret_cast<const f32x4*>(s_rinv + grp * 128 + rbase);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float g = acc[rb][0][rg * 4 + rr] * ri4[rr];
          const float u = acc[rb][1][rg * 4 + rr] * ri4[rr];
          const float o = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
          reinterpret_cast<uint16_t*>(stage + (rbase + rr) * kStagePitch)[c0 + fl] = f32_to_bf16(o);
        }
      }
    }
    __syncthreads();
    // wave (grp, slot) stores rows 64 (slot % 2) .. +63 of its (group, head) block:
    // 8 lanes of 16 bytes per 128-byte row
    const uint32_t I = (uint32_t)N / 2u;
    const uint32_t fcol = 128u * (uint32_t)tn + 64u * (uint32_t)head;
    const auto ro = make_rsrc(a.q, (uint32_t)T * I * 2u);
    const uint32_t ch = lane & 7;
#pragma unroll 4
    for (int it = 0; it < 8; ++it) {
      const uint32_t row = 64u * (slot & 1) + 8u * it + (lane >> 3);
      const u32x4 v = lds_read16(stage, row * kStagePitch + ch * 16u);
      const uint32_t grow = (uint32_t)(m0 + 128 * grp) + row;
      buf_store16_nt(v, ro, (grow * I + fcol + ch * 8u) * 2u);
    }
  } else {
    // ---- epilogue: scale, bias, rotate, stage as bf16, store
    const float bcol[2] = {bf16_to_f32(braw[0]), bf16_to_f32(braw[1])};
    const double rev = __builtin_bit_cast(double, rev_bits);
    // (the head's tensor: both blocks of the wave and the half it stores lie in one of
    // Q, K, V, whose column counts are multiples of 128 and of the head size)
    const bool rotate = n0 + blk < a.Nq + a.Nkv;
    void* out;
    uint32_t width, ocol;
    if (hcol < a.Nq) {
      out = a.q; width = a.Nq; ocol = hcol;
    } else if (hcol < a.Nq + a.Nkv) {
      out = a.k; width = a.Nkv; ocol = hcol - a.Nq;
    } else {
      out = a.v; width = a.Nkv; ocol = hcol - a.Nq - a.Nkv;
    }

    uint8_t* stage = smem + (grp * 2 + head) * kBlockStage;
    // block cb goes to the stage of its 128-column half, at its column within that half
    uint8_t* const stg[2] = {smem + (grp * 2 + blk / 128) * kBlockStage,
                             smem + (grp * 2 + (blk + kD / 2) / 128) * kBlockStage};
    const int scol[2] = {blk % 128 + (int)fl, (blk + kD / 2) % 128 + (int)fl};
    // one instantiation per case, so the uniform test is not repeated (as a branch)
    // around every element and independent elements can overlap
    auto scale_rotate_stage = [&](auto RotC) {
      constexpr bool kRot = decltype(RotC)::value;
  #pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
  #pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int rbase = rb * 32 + rg * 8 + (int)fh * 4;  // row within the group's 128
          const f32x4 ri4 = *reinterpret_cast<const f32x4*>(s_rinv + grp * 128 + rbase);
          const i32x4 p4 = *reinterpret_cast<const i32x4*>(s_pos + grp * 128 + rbase);
  #pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            float y0 = fmaf(acc[rb][0][rg * 4 + rr], ri4[rr], bcol[0]);
            float y1 = fmaf(acc[rb][1][rg * 4 + rr], ri4[rr], bcol[1]);
            if constexpr (kRot) {
              const float tf = turn_fraction(p4[rr], rev);
              const float c = __builtin_amdgcn_cosf(tf), s = __builtin_amdgcn_sinf(tf);
              const float u0 = y0, v0 = y1;
              y0 = u0 * c - v0 * s;
              y1 = v0 * c + u0 * s;
            }
            reinterpret_cast<uint16_t*>(stg[0] + (rbase + rr) * kStagePitch)[scol[0]] = f32_to_bf16(y0);
            reinterpret_cast<uint16_t*>(stg[1] + (rbase + rr) * kStagePitch)[scol[1]] = f32_to_bf16(y1);
          }
        }
      }
    };
    if (rotate)
      scale_rotate_stage(std::true_type{});
    else
      scale_rotate_stage(std::false_type{});
    __syncthreads();
    // wave (grp, slot) stores rows 64 (slot % 2) .. +63 of its (group, head) block.
    // K and V rows go to their cache slots when the forward has them; a row index of
    // out_rows or more lies past the buffer's range, so that store is dropped.
    const bool to_cache = a.slots != nullptr && hcol >= a.Nq;
    const uint32_t out_rows = to_cache ? (uint32_t)a.cache_rows : (uint32_t)T;
    const auto ro = make_rsrc(out, out_rows * width * 2u);
    const uint32_t ch = lane & 15;
  #pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const uint32_t row = 64u * (slot & 1) + 4u * it + (lane >> 4);
      const u32x4 v = lds_read16(stage, row * kStagePitch + ch * 16u);
      uint32_t orow = (uint32_t)(m0 + 128 * grp) + row;
      if (to_cache) {
        const int32_t sr = s_slot[128 * grp + row];
        orow = sr >= 0 && sr < a.cache_rows ? (uint32_t)sr : out_rows;
      }
      buf_store16_nt(v, ro, (orow * width + ocol + ch * 8u) * 2u);
    }
  }
}

}  // namespace

bool prefill_supports(int H, int N, int Nq, int Nkv, int d) {
  return (d == 64 || d == 128 || d == 256) && H % (4 * BK) == 0 && N % BN == 0 && Nq % 128 == 0 &&
         Nkv % 128 == 0 && Nq % d == 0 && Nkv % d == 0;
}

// K slices per tile: 2 (the split-K form) when the tiles alone would leave at least half
// of the 256 CUs idle, else 1 (the plain form).  Each slice keeps at least 8 steps of 32
// rows and a multiple of 4 of them.  Four slices were measured too: each workgroup's
// loop is shorter, but the last-arriving one then reads four partial tiles, and the
// forward was 1-5% slower than with two.
int prefill_splits(const ForwardArgs& a, int tiles) {
  if (!a.kpart || !a.kcount) return 1;
  return prefill_split_count(a.T, a.H, a.N, a.kpart_units);
}

template <int kD>
hipError_t launch_prefill_d(const ForwardArgs& a, int tiles_m, int tiles_n, hipStream_t stream) {
  const int tiles = tiles_m * tiles_n, s = prefill_splits(a, tiles);
  if (s == 2)
    prefill_kernel<kEpiQkv, kD, 2><<<dim3(tiles * 2), dim3(kThreads), 0, stream>>>(a, tiles_m, tiles_n);
  else
    prefill_kernel<kEpiQkv, kD, 1><<<dim3(tiles), dim3(kThreads), 0, stream>>>(a, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_prefill(const ForwardArgs& a, hipStream_t stream) {
  if (a.prenormed) return hipErrorInvalidValue;  // the pre-pass form runs launch_prefill_pre
  const int tiles_m = (a.T + BM - 1) / BM, tiles_n = a.N / BN;
  if (a.d == 64) return launch_prefill_d<64>(a, tiles_m, tiles_n, stream);
  if (a.d == 256) return launch_prefill_d<256>(a, tiles_m, tiles_n, stream);
  return launch_prefill_d<128>(a, tiles_m, tiles_n, stream);
}

int prefill_split_count(int T, int H, int N, int units) {
  const int tiles = (T + BM - 1) / BM * (N / BN), nk = H / BK;
  if (tiles > kPrefillSplitMaxTiles) return 1;
  return tiles * 2 <= units && nk % 8 == 0 && nk / 2 >= 8 ? 2 : 1;
}

int prefill_split_units(int max_tokens, int N) {
  const int tiles = (max_tokens + BM - 1) / BM * (N / BN);
  return 2 * (tiles < kPrefillSplitMaxTiles ? tiles : kPrefillSplitMaxTiles);
}

size_t prefill_split_floats(int units) { return (size_t)units * kPartFloats; }

bool swiglu_supports(int H, int I) { return H % (4 * BK) == 0 && I % 128 == 0; }

hipError_t launch_swiglu(const ForwardArgs& a, hipStream_t stream) {
  // a.N = 2I columns of [gate | up]; the output (a.q) is [T, I]
  if (swiglu_wide_supports(a.H, a.N / 2)) return launch_swiglu_wide(a, stream);  // one 128 x 512 launch
  const int tiles_m = (a.T + BM - 1) / BM, tiles_n = a.N / BN;
  prefill_kernel<kEpiSwiglu, 128, 1><<<dim3(tiles_m * tiles_n), dim3(kThreads), 0, stream>>>(a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace qkv
