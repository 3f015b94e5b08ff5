// Row reduction of RMSNorm: inv_rms[t] = 1/sqrt(sum_k x[t,k]^2 / H + eps).
//
// Step 1 of the fused-kernel listing on the page "Liger-Kernel底层优化：新一代内核级
// 推理加速引擎介绍" (section "融合内核是如何工作的？来看一段简化版实现"): sum of squares
// over the whole hidden size, divided by the hidden size, eps inside the reciprocal
// square root.  There every thread of a token redoes the full sum; here one 64-lane
// wavefront owns one token row, streams it with 16-byte loads (HBM-bound: 2H bytes
// in, 4 bytes out per token) and combines the lane sums with cross-lane shuffles.
#include "device_common.h"
#include "launch.h"

namespace qkv {

template <bool BF16>
__global__ __launch_bounds__(256) void inv_rms_kernel(const void* __restrict__ x, float* __restrict__ out,
                                                      int T, int H, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  constexpr uint32_t kElem = BF16 ? 2u : 4u;
  const uint32_t row_bytes = (uint32_t)H * kElem;  // multiple of 16 (H % 8 == 0)
  const char* base = (const char*)x + (size_t)row * row_bytes;
  float ss0 = 0.f, ss1 = 0.f;
#pragma unroll 4
  for (uint32_t off = (uint32_t)lane * 16u; off < row_bytes; off += 64u * 16u) {
    u32x4 v = __builtin_nontemporal_load((const u32x4*)(base + off));
    if constexpr (BF16) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float lo = bf16_lo(v[c]), hi = bf16_hi(v[c]);
        ss0 = fmaf(lo, lo, ss0);
        ss1 = fmaf(hi, hi, ss1);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; c += 2) {
        float a = __uint_as_float(v[c]), b = __uint_as_float(v[c + 1]);
        ss0 = fmaf(a, a, ss0);
        ss1 = fmaf(b, b, ss1);
      }
    }
  }
  float ss = wave_sum(ss0 + ss1);
  if (lane == 0) out[row] = rsqrtf(ss / (float)H + eps);
}

// Pre-pass of the prefill kernel's pre-normalised form: the same row reduction, and
// the normalise-on-load product bf16(x * w_norm) written out so the GEMM can stream it
// global -> LDS like the weight.  One wavefront per row, 16-byte loads and stores.
__global__ __launch_bounds__(256) void prenorm_kernel(const void* __restrict__ x, const void* __restrict__ w,
                                                      void* __restrict__ xw, float* __restrict__ out, int T, int H,
                                                      float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const uint32_t row_bytes = (uint32_t)H * 2u;  // multiple of 16 (H % 8 == 0)
  const char* base = (const char*)x + (size_t)row * row_bytes;
  char* dst = (char*)xw + (size_t)row * row_bytes;
  float ss0 = 0.f, ss1 = 0.f;
#pragma unroll 4
  for (uint32_t off = (uint32_t)lane * 16u; off < row_bytes; off += 64u * 16u) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(base + off));
    const u32x4 g = *(const u32x4*)((const char*)w + off);
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float lo = bf16_lo(v[c]), hi = bf16_hi(v[c]);
      ss0 = fmaf(lo, lo, ss0);
      ss1 = fmaf(hi, hi, ss1);
      o[c] = pack_bf16x2(lo * bf16_lo(g[c]), hi * bf16_hi(g[c]));
    }
    *(u32x4*)(dst + off) = o;
  }
  const float ss = wave_sum(ss0 + ss1);
  if (lane == 0) out[row] = rsqrtf(ss / (float)H + eps);
}

hipError_t launch_prenorm(const void* x, const void* w_norm, void* xw, float* inv_rms, int T, int H, float eps,
                          hipStream_t stream) {
  prenorm_kernel<<<dim3((T + 3) / 4), dim3(256), 0, stream>>>(x, w_norm, xw, inv_rms, T, H, eps);
  return hipGetLastError();
}

hipError_t launch_inv_rms(const void* x, float* inv_rms, int T, int H, float eps, bool bf16,
                          hipStream_t stream) {
  dim3 grid((T + 3) / 4), block(256);
  if (bf16)
    inv_rms_kernel<true><<<grid, block, 0, stream>>>(x, inv_rms, T, H, eps);
  else
    inv_rms_kernel<false><<<grid, block, 0, stream>>>(x, inv_rms, T, H, eps);
  return hipGetLastError();
}

}  // namespace qkv
