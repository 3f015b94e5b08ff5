// The opt-in pre-pass form's MFMA kernel (gemm.hip): internal launcher, not exported.
#pragma once

#include "launch.h"

namespace qkv {

// Whether the 256 x 256 16 x 16 x 32 kernel takes the pre-normalised forward of this
// shape: head size 64, 128 or 256, N a multiple of 256, H of 128.
bool prefill_pre_supports(int H, int N, int d);
// a.x holds the pre-pass's tiled bf16(x * w_norm) and a.inv_rms each row's 1/rms
// (launch_prenorm); Q, K, V as the other forwards write them.
hipError_t launch_prefill_pre(const ForwardArgs& a, hipStream_t stream);

}  // namespace qkv
