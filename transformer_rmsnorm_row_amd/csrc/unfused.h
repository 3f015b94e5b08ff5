// Host-side launchers of the unfused steps (internal; not exported): the RMSNorm and
// the bias + rotation as kernels of their own, for comparison with the fused chain.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkv {

// xn [T, H] = x [T, H] * 1/rms(row) * w_norm [H], in the plan dtype (H % 8 == 0).
hipError_t launch_rms_norm(const void* x, const void* w_norm, void* xn, int T, int H, float eps, bool bf16,
                           hipStream_t stream);
// In place on y [T, N] (Q columns, then K, then V): + bias [N] when bias is non-null,
// then the rotate-half turn of every Q and K head by pos[t] times rev_freq[i] turns
// (d % 8 == 0, Nq and Nkv multiples of d).
hipError_t launch_rope(void* y, const void* bias, const int32_t* pos, const double* rev_freq, int T, int N, int Nq,
                       int Nkv, int d, bool bf16, hipStream_t stream);

// In place on y [T, N]: every Q head (weight wq [d]) and K head (weight wk [d]) divided
// by its own RMS over d (eps), multiplied by the weight, then turned like launch_rope;
// V untouched (d % 8 == 0, d <= 256).
hipError_t launch_head_norm_rope(void* y, const void* wq, const void* wk, const int32_t* pos,
                                 const double* rev_freq, int T, int N, int Nq, int Nkv, int d, float eps, bool bf16,
                                 hipStream_t stream);

}  // namespace qkv
