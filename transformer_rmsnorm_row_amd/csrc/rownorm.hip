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

// Pre-pass of the opt-in pre-normalised form: the same row reduction, and
// the normalise-on-load product bf16(x * w_norm) written out pre-tiled in the order the
// kernel's LDS holds it, so that each of its activation DMA instructions reads 1 KB of
// consecutive bytes.  Tiled layout: [T_pad / 256 panels][H / 32 steps][256 rows][4 x 16 B],
// 16-byte chunk q (k = 8q .. 8q + 7 of the step) of row r stored at chunk q ^ ((r / 2) % 4).
// One wavefront per row (rows T .. T_pad - 1 of the last panel are written as zeros),
// 16-byte loads and stores.
__global__ __launch_bounds__(256) void prenorm_kernel(const void* __restrict__ x, const void* __restrict__ w,
                                                      void* __restrict__ xw, float* __restrict__ out, int T,
                                                      int T_pad, int H, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T_pad) return;
  const uint32_t row_bytes = (uint32_t)H * 2u;  // multiple of 16 (H % 8 == 0)
  const char* base = (const char*)x + (size_t)row * row_bytes;
  const uint32_t r = (uint32_t)row & 255u, swz = (r >> 1) & 3u;
  char* panel = (char*)xw + (size_t)(row >> 8) * 256u * row_bytes;
  float ss0 = 0.f, ss1 = 0.f;
#pragma unroll 4
  for (uint32_t off = (uint32_t)lane * 16u; off < row_bytes; off += 64u * 16u) {
    const uint32_t c = off >> 4, step = c >> 2, q = c & 3u;
    u32x4 o = {0u, 0u, 0u, 0u};
    if (row < T) {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)(base + off));
      const u32x4 g = *(const u32x4*)((const char*)w + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo(v[e]), hi = bf16_hi(v[e]);
        ss0 = fmaf(lo, lo, ss0);
        ss1 = fmaf(hi, hi, ss1);
        o[e] = pack_bf16x2(lo * bf16_lo(g[e]), hi * bf16_hi(g[e]));
      }
    }
    *(u32x4*)(panel + ((size_t)step * 256u + r) * 64u + ((q ^ swz) << 4)) = o;
  }
  if (row >= T) return;
  const float ss = wave_sum(ss0 + ss1);
  if (lane == 0) out[row] = rsqrtf(ss / (float)H + eps);
}

hipError_t launch_prenorm(const void* x, const void* w_norm, void* xw, float* inv_rms, int T, int H, float eps,
                          hipStream_t stream) {
  const int T_pad = (T + 255) / 256 * 256;
  prenorm_kernel<<<dim3((T_pad + 3) / 4), dim3(256), 0, stream>>>(x, w_norm, xw, inv_rms, T, T_pad, H, eps);
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
