// Host-side launchers of the kernels behind the C ABI (internal; not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkv {

// Everything one forward needs, resolved by the host API after validation.
struct ForwardArgs {
  const void* x;
  const void* w_norm;
  const void* w;
  const void* bias;        // nullptr when the plan has no bias
  const int32_t* pos;
  void* q;
  void* k;
  void* v;
  float* inv_rms;          // scratch [T] fp32
  const double* rev_freq;  // [head_dim/2] rotary frequencies, revolutions per position
  float* partials;         // decode scratch
  uint32_t* counters;      // decode scratch
  // prefill with the hidden dimension split over several workgroups per tile (when the
  // tiles alone would leave most CUs idle): fp32 partial tiles and per-tile arrival
  // counters, or null when the plan has none
  float* kpart;
  uint32_t* kcount;
  int kpart_units;         // partial tiles kpart holds
  // KV-cache form: when non-null, K and V of token t go to row slots[t] of k and v,
  // which then hold cache_rows rows; tokens whose slot is outside [0, cache_rows)
  // write no K/V.  Q stays dense.
  const int32_t* slots;
  int cache_rows;
  int T, H, N, Nq, Nkv, d;
  float eps;
  bool bf16;
  // x holds bf16(x * w_norm) pre-tiled and inv_rms each row's 1/rms, written by
  // launch_prenorm: the opt-in pre-pass form's MFMA kernel (launch_prefill_pre) then loads
  // the activations like the weight, with no conversion
  bool prenormed;
};

// One pass over bf16 x [T, H]: xw = bf16(x * w_norm), tiled per 256-row panel and 32-wide
// k step in the LDS order of the pre-pass form's MFMA kernel (T rounded up to 256 rows, the
// extra rows zero), and inv_rms[t] = 1/rms of row t.
hipError_t launch_prenorm(const void* x, const void* w_norm, void* xw, float* inv_rms, int T, int H, float eps,
                          hipStream_t stream);
hipError_t launch_inv_rms(const void* x, float* inv_rms, int T, int H, float eps, bool bf16,
                          hipStream_t stream);
hipError_t launch_generic(const ForwardArgs& a, hipStream_t stream);
hipError_t launch_prefill(const ForwardArgs& a, hipStream_t stream);
bool prefill_supports(int H, int N, int Nq, int Nkv, int d);
// Single-launch normalise-on-load prefill on 128 x 512 tiles with 16 x 16 x 32 MFMAs
// (prefill_wide.hip): the plain prefill forward's kernel for head sizes 64/128/256, N a
// multiple of 512 and H of 128.
hipError_t launch_prefill_wide(const ForwardArgs& a, hipStream_t stream);
bool prefill_wide_supports(int H, int N, int Nq, int Nkv, int d);
// Workgroups of a tile-persistent launch over `tiles` tiles on the current device: one
// per CU (the CU count rounded down to a multiple of 8, so that a workgroup's XCD is the
// same for every tile it takes), or `tiles` if that is fewer.  The CU count is looked up
// once per device (an attribute query, no stream work, so a forward under graph capture
// may run it); should the query fail, every tile gets a workgroup of its own.
int persistent_grid(int tiles);
// The split-K form of the prefill kernel (two K slices per 256 x 256 tile, partial
// tiles added by the last-arriving workgroup) is used up to this many tiles, one arrival
// counter each.
constexpr int kPrefillSplitMaxTiles = 128;
// Partial tiles a plan of max_tokens tokens and N columns needs for the split-K form of
// the prefill kernel, and their fp32 element count.
int prefill_split_units(int max_tokens, int N);
// K slices per tile the prefill kernel uses for T tokens (1: the plain form), given a
// plan whose split scratch holds `units` partial tiles.
int prefill_split_count(int T, int H, int N, int units);
size_t prefill_split_floats(int units);
// Token capacity of one decode launch (batches of up to 64 tokens run a 64-token form
// of the kernel); larger batches run as consecutive launches of up to this many tokens.
constexpr int kDecodeTokens = 128;
hipError_t launch_decode(const ForwardArgs& a, hipStream_t stream);
// gated MLP on the prefill kernel: x, w_norm, w = [H, 2I] (gate | up), q = out [T, I],
// N = 2I, T, H, eps, bf16
hipError_t launch_swiglu(const ForwardArgs& a, hipStream_t stream);
bool swiglu_supports(int H, int I);
// the same on the 128 x 512 kernel of prefill_wide.hip, which launch_swiglu picks when 2I is
// a multiple of 512 (and H of 128)
hipError_t launch_swiglu_wide(const ForwardArgs& a, hipStream_t stream);
bool swiglu_wide_supports(int H, int I);
bool decode_supports(int T, int H, int N, int Nq, int Nkv, int d);
// fp32 elements of plan scratch the decode kernel needs (partials + sums of squares)
size_t decode_scratch_floats(int H, int N);

}  // namespace qkv
