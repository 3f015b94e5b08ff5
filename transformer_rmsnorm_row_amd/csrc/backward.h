// Host-side launchers of the backward's kernels behind the C ABI (internal; not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkv {

// Backward of the chain (see backward.hip): everything but the two GEMMs.
struct BackwardArgs {
  const void* x;
  const void* w_norm;
  const void* w;           // W_qkv [H, N]
  const int32_t* pos;
  const void* dq;
  const void* dk;
  const void* dv;
  void* dx;
  void* dw_norm;
  void* dbias;             // nullptr when the plan has no bias
  void* gy;                // scratch [N, Tp] plan dtype: r[t] times the unrotated upstream gradient, transposed
  void* ga;                // scratch [T, H] plan dtype: r[t] times the gradient of the activations
  float* inv_rms;          // scratch [T]: r
  float* partial;          // scratch [kBackwardPartials, H] fp32 column partial sums
  const double* rev_freq;  // [d/2]
  int T, H, N, Nq, Nkv, d;
  float eps;
  bool bf16;
};
constexpr int kBackwardChunks = 64;     // token chunks of the generic column sums
constexpr int kBackwardPartials = 2048; // partial rows of the fused norm-gradient pass (>= kBackwardChunks)
// Token pitch of the transposed gradient gy^T [N][Tp]: T rounded up to 32 (pad zero).
inline int backward_token_pitch(int T) { return (T + 31) / 32 * 32; }
// One plain GEMM C[M, N] = s[m] sum_k A(m, k) B(k, n), fp32 accumulation (gemm.hip), with
// s = row_scale (M values in the operands' dtype) or 1 when row_scale is null.  Each
// operand is [rows][K] (k contiguous) or [K][cols] per the GEMM's template; pitches in
// elements.
struct GemmArgs {
  const void* a;
  const void* b;
  void* c;
  const void* row_scale;
  int M, N, K;
  int lda, ldb, ldc;
};
// The backward's two GEMMs on this library's kernels: dw [H, N] (plan dtype) =
// diag(w_norm) x^T gy and b.ga [T, H] (plan dtype) = gy W^T, gy already scaled by r;
// bf16 plans on the matrix cores (ga there when N is a multiple of 32), fp32 plans and
// other shapes on fp32 FMA tiles.
hipError_t launch_backward_gemms(const BackwardArgs& b, void* dw, hipStream_t stream);
int backward_colsum_chunks(int T);
// r, unrotate (gy, scaled by r) and the bias gradient
hipError_t launch_backward_pre_gemm(const BackwardArgs& b, hipStream_t stream);
// dx and the norm-weight gradient, once ga = gy W^T is in b.ga
hipError_t launch_backward_post_gemm(const BackwardArgs& b, hipStream_t stream);

}  // namespace qkv
