// The chain's steps as separate kernels, for measuring what fusing them saves.
//
// The pages on Liger-Kernel ("Liger-Kernel底层优化：新一代内核级推理加速引擎介绍",
// sections on why fusion pays and on the fused kernel) credit the fused chain with
// fewer launches and one HBM round trip instead of several: unfused, the normalised
// activations go to HBM and come back for the projection, and the projection output
// goes to HBM, comes back for the bias and rotation, and goes out again.  These two
// kernels are that unfused form; between them the projection is a library GEMM.
//
//   rms_norm_kernel  xn[t,k] = x[t,k] * r[t] * w[k], r[t] = 1/sqrt(mean_k x[t,k]^2 + eps),
//                    fp32 arithmetic, one rounding to the output dtype.  One wavefront per
//                    row: a first pass sums the squares with 16-byte loads, a second pass
//                    re-reads the row (from L2) with the norm weight and writes xn.
//   rope_kernel      in place on the projection output y [T, N]: adds the bias to every
//                    column (when given) and turns each rotate-half pair (i, i + d/2) of the
//                    Q and K heads by pos[t] * theta^(-2i/d); V columns only get the bias.
//                    Each thread takes 4 consecutive pairs of one head.
//   head_norm_rope_kernel  the norm and the rotation in one pass, read as a per-head
//                    RMSNorm of every Q and K head of y (weights [d] for Q and for K,
//                    eps of the plan) followed by the turn of its pairs: one wavefront per
//                    (token, head) item at a time, about 8 items per wavefront in a grid
//                    stride, lane j holding the pair (j, j + d/2) (j + 64 for larger heads),
//                    the head's sum of squares reduced across the wave.
#include <algorithm>

#include "device_common.h"
#include "unfused.h"

namespace qkv {

namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void rms_norm_kernel(const void* __restrict__ x, const void* __restrict__ w,
                                                       void* __restrict__ y, int T, int H, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  constexpr uint32_t kElem = BF16 ? 2u : 4u;
  const uint32_t row_bytes = (uint32_t)H * kElem;  // multiple of 16 (H % 8 == 0)
  const char* xr = (const char*)x + (size_t)row * row_bytes;
  char* yr = (char*)y + (size_t)row * row_bytes;
  float ss0 = 0.f, ss1 = 0.f;
#pragma unroll 4
  for (uint32_t off = (uint32_t)lane * 16u; off < row_bytes; off += 64u * 16u) {
    const u32x4 v = *(const u32x4*)(xr + off);
    if constexpr (BF16) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float lo = bf16_lo(v[c]), hi = bf16_hi(v[c]);
        ss0 = fmaf(lo, lo, ss0);
        ss1 = fmaf(hi, hi, ss1);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; c += 2) {
        const float a = __uint_as_float(v[c]), b = __uint_as_float(v[c + 1]);
        ss0 = fmaf(a, a, ss0);
        ss1 = fmaf(b, b, ss1);
      }
    }
  }
  const float rinv = rsqrtf(wave_sum(ss0 + ss1) / (float)H + eps);
#pragma unroll 4
  for (uint32_t off = (uint32_t)lane * 16u; off < row_bytes; off += 64u * 16u) {
    const u32x4 v = *(const u32x4*)(xr + off);
    const u32x4 g = *(const u32x4*)((const char*)w + off);
    u32x4 o;
    if constexpr (BF16) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        o[c] = pack_bf16x2(bf16_lo(v[c]) * rinv * bf16_lo(g[c]), bf16_hi(v[c]) * rinv * bf16_hi(g[c]));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = __float_as_uint(__uint_as_float(v[c]) * rinv * __uint_as_float(g[c]));
    }
    *(u32x4*)(yr + off) = o;
  }
}

template <bool BF16>
__device__ __forceinline__ void load4(const void* p, size_t i, float* f) {
  if constexpr (BF16) {
    const uint2 v = *(const uint2*)((const uint16_t*)p + i);
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  } else {
    const float4 v = *(const float4*)((const float*)p + i);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void store4(void* p, size_t i, const float* f) {
  if constexpr (BF16) {
    *(uint2*)((uint16_t*)p + i) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
  } else {
    *(float4*)((float*)p + i) = make_float4(f[0], f[1], f[2], f[3]);
  }
}

// Work items of a row: first the rotated quads (4 pairs of one Q or K head each), then,
// with a bias, the V columns in groups of 4.
template <bool BF16>
__global__ __launch_bounds__(256) void rope_kernel(void* __restrict__ y, const void* __restrict__ bias,
                                                   const int32_t* __restrict__ pos,
                                                   const double* __restrict__ rev_freq, int N, int Nq, int Nkv,
                                                   int d, int rot_items, int items, int blocks_per_row) {
  const int row = blockIdx.x / blocks_per_row;
  const int item = (blockIdx.x % blocks_per_row) * 256 + threadIdx.x;
  if (item >= items) return;
  const size_t base = (size_t)row * N;
  float u[4], v[4];
  if (item < rot_items) {
    const int quads = d / 8;  // quads of pairs per head
    const int head = item / quads, i0 = (item % quads) * 4;
    const int c0 = head * d + i0, c1 = c0 + d / 2;
    load4<BF16>(y, base + c0, u);
    load4<BF16>(y, base + c1, v);
    if (bias) {
      float bu[4], bv[4];
      load4<BF16>(bias, c0, bu);
      load4<BF16>(bias, c1, bv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[e] += bu[e];
        v[e] += bv[e];
      }
    }
    const int32_t p = pos[row];
    float o0[4], o1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float cs, sn;
      rope_cos_sin(p, rev_freq[i0 + e], cs, sn);
      o0[e] = u[e] * cs - v[e] * sn;
      o1[e] = v[e] * cs + u[e] * sn;
    }
    store4<BF16>(y, base + c0, o0);
    store4<BF16>(y, base + c1, o1);
  } else {
    const int c = Nq + Nkv + (item - rot_items) * 4;
    float bv[4];
    load4<BF16>(y, base + c, u);
    load4<BF16>(bias, c, bv);
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] += bv[e];
    store4<BF16>(y, base + c, u);
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* p, size_t i) {
  if constexpr (BF16)
    return bf16_lo((uint32_t)((const uint16_t*)p)[i]);
  else
    return ((const float*)p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store1(void* p, size_t i, float v) {
  if constexpr (BF16)
    ((uint16_t*)p)[i] = f32_to_bf16(v);
  else
    ((float*)p)[i] = v;
}

// Pairs per lane: up to 2 (head_dim <= 256).
template <bool BF16>
__global__ __launch_bounds__(256) void head_norm_rope_kernel(void* __restrict__ y, const void* __restrict__ wq,
                                                             const void* __restrict__ wk,
                                                             const int32_t* __restrict__ pos,
                                                             const double* __restrict__ rev_freq, int T, int N,
                                                             int nq_heads, int rot_heads, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int half = d / 2;
  const int items = T * rot_heads, stride = gridDim.x * 4;
  // each wavefront walks (token, rotated head) items with a grid stride
  for (int item = blockIdx.x * 4 + (threadIdx.x >> 6); item < items; item += stride) {
    const int row = item / rot_heads, head = item % rot_heads;
    const void* w = head < nq_heads ? wq : wk;
    const size_t base = (size_t)row * N + (size_t)head * d;
    float u[2] = {0.f, 0.f}, v[2] = {0.f, 0.f}, ss = 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      if (i < half) {
        u[r] = load1<BF16>(y, base + i);
        v[r] = load1<BF16>(y, base + i + half);
        ss = fmaf(u[r], u[r], fmaf(v[r], v[r], ss));
      }
    }
    const float rinv = rsqrtf(wave_sum(ss) / (float)d + eps);
    const int32_t p = pos[row];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      if (i < half) {
        const float a = u[r] * rinv * load1<BF16>(w, i), b = v[r] * rinv * load1<BF16>(w, i + half);
        float cs, sn;
        rope_cos_sin(p, rev_freq[i], cs, sn);
        store1<BF16>(y, base + i, a * cs - b * sn);
        store1<BF16>(y, base + i + half, b * cs + a * sn);
      }
    }
  }
}

}  // namespace

hipError_t launch_head_norm_rope(void* y, const void* wq, const void* wk, const int32_t* pos,
                                 const double* rev_freq, int T, int N, int Nq, int Nkv, int d, float eps, bool bf16,
                                 hipStream_t stream) {
  const int nq_heads = Nq / d, rot_heads = (Nq + Nkv) / d;
  const int items = T * rot_heads;
  // about 8 items per wavefront, at least 4096 workgroups when there is that much work
  const int blocks = std::max(1, std::min((items + 3) / 4, std::max(4096, (items + 31) / 32)));
  dim3 grid((unsigned)blocks), block(256);
  if (bf16)
    head_norm_rope_kernel<true><<<grid, block, 0, stream>>>(y, wq, wk, pos, rev_freq, T, N, nq_heads, rot_heads, d,
                                                            eps);
  else
    head_norm_rope_kernel<false><<<grid, block, 0, stream>>>(y, wq, wk, pos, rev_freq, T, N, nq_heads, rot_heads,
                                                             d, eps);
  return hipGetLastError();
}

hipError_t launch_rms_norm(const void* x, const void* w_norm, void* xn, int T, int H, float eps, bool bf16,
                           hipStream_t stream) {
  dim3 grid((T + 3) / 4), block(256);
  if (bf16)
    rms_norm_kernel<true><<<grid, block, 0, stream>>>(x, w_norm, xn, T, H, eps);
  else
    rms_norm_kernel<false><<<grid, block, 0, stream>>>(x, w_norm, xn, T, H, eps);
  return hipGetLastError();
}

hipError_t launch_rope(void* y, const void* bias, const int32_t* pos, const double* rev_freq, int T, int N, int Nq,
                       int Nkv, int d, bool bf16, hipStream_t stream) {
  const int rot_items = (Nq + Nkv) / 8;  // (Nq + Nkv) / 2 pairs, 4 per item
  const int items = rot_items + (bias ? Nkv / 4 : 0);
  const int blocks_per_row = (items + 255) / 256;
  dim3 grid((unsigned)T * (unsigned)blocks_per_row), block(256);
  if (bf16)
    rope_kernel<true><<<grid, block, 0, stream>>>(y, bias, pos, rev_freq, N, Nq, Nkv, d, rot_items, items,
                                                  blocks_per_row);
  else
    rope_kernel<false><<<grid, block, 0, stream>>>(y, bias, pos, rev_freq, N, Nq, Nkv, d, rot_items, items,
                                                   blocks_per_row);
  return hipGetLastError();
}

}  // namespace qkv
