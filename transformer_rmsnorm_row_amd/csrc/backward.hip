// Backward of the fused attention-input chain: the elementwise and row/column
// reduction kernels around the two plain GEMMs (which rocBLAS runs, see qkv_api.hip).
//
// Chain rule of the forward (RMSNorm -> projection (+bias) -> rotate-half rotary
// embedding of Q and K) for upstream gradients dQ, dK, dV, with r[t] the token's
// inverse RMS and a = x r w the normalised activations:
//   gy   = the rotation by -angle of each (dQ, dK) pair, dV unchanged   (unrotate)
//   db   = sum over tokens of gy                                        (column sum)
//   dW   = a^T gy,  ga = gy W^T                                         (GEMMs)
//   dw   = sum over tokens of ga * x * r                                (column sum)
//   dx_j = r w_j ga_j - (r^3 / H) x_j sum_k ga_k w_k x_k                (row kernel)
// Column sums are two-pass (fixed chunks of tokens, then the chunks in order), so
// every result is deterministic.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace qkv {

namespace {

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, size_t i) {
  if constexpr (BF16)
    return bf16_to_f32(((const uint16_t*)p)[i]);
  else
    return ((const float*)p)[i];
}

template <bool BF16>
__device__ __forceinline__ void st(void* p, size_t i, float v) {
  if constexpr (BF16)
    ((uint16_t*)p)[i] = f32_to_bf16(v);
  else
    ((float*)p)[i] = v;
}

// 8 consecutive elements of a row as fp32 (one 16-byte load for bf16, two for fp32)
// and back.  Callers keep the offsets multiples of 8 elements (H % 8 == 0 and d % 16
// == 0 where used).
template <bool BF16>
__device__ __forceinline__ void ld8(const void* p, size_t i, float (&v)[8]) {
  if constexpr (BF16) {
    const u32x4 r = *reinterpret_cast<const u32x4*>((const uint16_t*)p + i);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[2 * c] = bf16_lo(r[c]);
      v[2 * c + 1] = bf16_hi(r[c]);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>((const float*)p + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>((const float*)p + i + 4);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[c] = a[c];
      v[4 + c] = b[c];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void st8(void* p, size_t i, const float (&v)[8]) {
  if constexpr (BF16) {
    u32x4 r;
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = pack_bf16x2(v[2 * c], v[2 * c + 1]);
    *reinterpret_cast<u32x4*>((uint16_t*)p + i) = r;
  } else {
    *reinterpret_cast<f32x4*>((float*)p + i) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>((float*)p + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// One thread per (token, 8 consecutive rotation pairs of one head): 16-byte loads of
// the u and v halves.  Used when d/2 is a multiple of 8.
template <bool BF16>
__global__ __launch_bounds__(256) void unrotate8_kernel(BackwardArgs b) {
  const int half = b.d / 2, units = b.N / 16;  // 8-pair groups per token
  const size_t total = (size_t)b.T * units;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(e / units), g = (int)(e % units);
    const int p0 = g * 8;                                 // first pair of the group
    const int c = (p0 / half) * b.d + (p0 % half);        // its first column
    const void* src;
    int width, oc;
    if (c < b.Nq) {
      src = b.dq; width = b.Nq; oc = c;
    } else if (c < b.Nq + b.Nkv) {
      src = b.dk; width = b.Nkv; oc = c - b.Nq;
    } else {
      src = b.dv; width = b.Nkv; oc = c - b.Nq - b.Nkv;
    }
    float gu[8], gv[8];
    ld8<BF16>(src, (size_t)t * width + oc, gu);
    ld8<BF16>(src, (size_t)t * width + oc + half, gv);
    if (c < b.Nq + b.Nkv) {
      const int i0 = p0 % half;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float cs, sn;
        rope_cos_sin(b.pos[t], b.rev_freq[i0 + j], cs, sn);
        const float u = gu[j], v = gv[j];
        gu[j] = u * cs + v * sn;
        gv[j] = v * cs - u * sn;
      }
    }
    st8<BF16>(b.gy, (size_t)t * b.N + c, gu);
    st8<BF16>(b.gy, (size_t)t * b.N + c + half, gv);
  }
}

// One thread per (token, rotation pair); pairs enumerate features i < d/2 of every
// head of Q, K and V (V pairs are copied unrotated).
template <bool BF16>
__global__ __launch_bounds__(256) void unrotate_kernel(BackwardArgs b) {
  const int half = b.d / 2, units = b.N / 2;
  const size_t total = (size_t)b.T * units;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(e / units), u = (int)(e % units);
    const int c = (u / half) * b.d + (u % half);
    const void* src;
    int width, oc;
    if (c < b.Nq) {
      src = b.dq; width = b.Nq; oc = c;
    } else if (c < b.Nq + b.Nkv) {
      src = b.dk; width = b.Nkv; oc = c - b.Nq;
    } else {
      src = b.dv; width = b.Nkv; oc = c - b.Nq - b.Nkv;
    }
    const float gu = ld<BF16>(src, (size_t)t * width + oc), gv = ld<BF16>(src, (size_t)t * width + oc + half);
    float y0 = gu, y1 = gv;
    if (c < b.Nq + b.Nkv) {
      float cs, sn;
      rope_cos_sin(b.pos[t], b.rev_freq[u % half], cs, sn);
      y0 = gu * cs + gv * sn;
      y1 = gv * cs - gu * sn;
    }
    st<BF16>(b.gy, (size_t)t * b.N + c, y0);
    st<BF16>(b.gy, (size_t)t * b.N + c + half, y1);
  }
}

// One wave per token: r[t] and the normalised activations a = x r w in the plan dtype.
// KIT > 0: H = 512 KIT, and the lane's KIT x 8 values of the row stay in registers
// between the two passes (same arithmetic, same order); KIT = 0: any H, row read twice.
template <bool BF16, int KIT>
__global__ __launch_bounds__(256) void activations_kernel(BackwardArgs b) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= b.T) return;
  const size_t row = (size_t)t * b.H;
  if constexpr (KIT > 0) {
    float v[KIT][8];
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < KIT; ++m) {
      ld8<BF16>(b.x, row + lane * 8 + 512 * m, v[m]);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(v[m][j], v[m][j], ss);
    }
    const float r = rsqrtf(wave_sum(ss) / (float)b.H + b.eps);
    if (lane == 0) b.inv_rms[t] = r;
#pragma unroll
    for (int m = 0; m < KIT; ++m) {
      float w[8];
      ld8<BF16>(b.w_norm, lane * 8 + 512 * m, w);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[m][j] = v[m][j] * r * w[j];
      st8<BF16>(b.act, row + lane * 8 + 512 * m, v[m]);
    }
    return;
  }
  float ss = 0.f;
  for (int k = lane * 8; k < b.H; k += 512) {
    float v[8];
    ld8<BF16>(b.x, row + k, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
  }
  const float r = rsqrtf(wave_sum(ss) / (float)b.H + b.eps);
  if (lane == 0) b.inv_rms[t] = r;
  for (int k = lane * 8; k < b.H; k += 512) {
    float v[8], w[8];
    ld8<BF16>(b.x, row + k, v);
    ld8<BF16>(b.w_norm, k, w);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * r * w[j];
    st8<BF16>(b.act, row + k, v);
  }
}

// One wave per token: dx from ga (fp32), x, w and r.  KIT as for the activations:
// the lane's ga and x values stay in registers between the inner product and dx.
template <bool BF16, int KIT>
__global__ __launch_bounds__(256) void norm_grad_kernel(BackwardArgs b) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= b.T) return;
  const size_t row = (size_t)t * b.H;
  if constexpr (KIT > 0) {
    float g[KIT][8], x[KIT][8];
    float inner = 0.f;
#pragma unroll
    for (int m = 0; m < KIT; ++m) {
      float w[8];
      ld8<false>(b.ga, row + lane * 8 + 512 * m, g[m]);
      ld8<BF16>(b.w_norm, lane * 8 + 512 * m, w);
      ld8<BF16>(b.x, row + lane * 8 + 512 * m, x[m]);
#pragma unroll
      for (int j = 0; j < 8; ++j) inner = fmaf(g[m][j] * w[j], x[m][j], inner);
    }
    inner = wave_sum(inner);
    const float r = b.inv_rms[t];
    const float c2 = r * r * r / (float)b.H * inner;
#pragma unroll
    for (int m = 0; m < KIT; ++m) {
      float w[8];
      ld8<BF16>(b.w_norm, lane * 8 + 512 * m, w);
#pragma unroll
      for (int j = 0; j < 8; ++j) g[m][j] = r * w[j] * g[m][j] - c2 * x[m][j];
      st8<BF16>(b.dx, row + lane * 8 + 512 * m, g[m]);
    }
    return;
  }
  float inner = 0.f;
  for (int k = lane * 8; k < b.H; k += 512) {
    float g[8], w[8], x[8];
    ld8<false>(b.ga, row + k, g);
    ld8<BF16>(b.w_norm, k, w);
    ld8<BF16>(b.x, row + k, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) inner = fmaf(g[j] * w[j], x[j], inner);
  }
  inner = wave_sum(inner);
  const float r = b.inv_rms[t];
  const float c2 = r * r * r / (float)b.H * inner;
  for (int k = lane * 8; k < b.H; k += 512) {
    float g[8], w[8], x[8];
    ld8<false>(b.ga, row + k, g);
    ld8<BF16>(b.w_norm, k, w);
    ld8<BF16>(b.x, row + k, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = r * w[j] * g[j] - c2 * x[j];
    st8<BF16>(b.dx, row + k, g);
  }
}

// Column sums over tokens, pass 1: block (column group, token chunk) -> fp32 partial.
// kMode 0: gy[t, c]; kMode 1: ga[t, c] * x[t, c] * r[t].
template <bool BF16, int kMode>
__global__ __launch_bounds__(256) void colsum_partial_kernel(BackwardArgs b, int ncols, int chunks) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= ncols) return;
  const int per = (b.T + chunks - 1) / chunks;
  const int t0 = blockIdx.y * per, t1 = min(b.T, t0 + per);
  float s = 0.f;
  // unrolled so that the loads of several tokens are in flight; the adds keep token order
#pragma unroll 8
  for (int t = t0; t < t1; ++t) {
    if constexpr (kMode == 0)
      s += ld<BF16>(b.gy, (size_t)t * ncols + c);
    else
      s = fmaf(b.ga[(size_t)t * ncols + c] * ld<BF16>(b.x, (size_t)t * ncols + c), b.inv_rms[t], s);
  }
  b.partial[(size_t)blockIdx.y * ncols + c] = s;
}

// Pass 2: the chunks of each column added in order.
template <bool BF16>
__global__ __launch_bounds__(256) void colsum_final_kernel(const float* partial, void* out, int ncols, int chunks) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= ncols) return;
  float s = 0.f;
  // unrolled so that the chunks' loads are in flight together; the adds keep chunk order
#pragma unroll 16
  for (int j = 0; j < chunks; ++j) s += partial[(size_t)j * ncols + c];
  st<BF16>(out, c, s);
}

template <bool BF16, int kMode>
hipError_t colsum(const BackwardArgs& b, int ncols, void* out, hipStream_t stream) {
  const int chunks = backward_colsum_chunks(b.T);
  colsum_partial_kernel<BF16, kMode><<<dim3((ncols + 255) / 256, chunks), dim3(256), 0, stream>>>(b, ncols, chunks);
  colsum_final_kernel<BF16><<<dim3((ncols + 255) / 256), dim3(256), 0, stream>>>(b.partial, out, ncols, chunks);
  return hipGetLastError();
}

template <bool BF16>
hipError_t pre_gemm(const BackwardArgs& b, hipStream_t stream) {
  if ((b.d / 2) % 8 == 0) {
    const size_t total = (size_t)b.T * (b.N / 16);
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
    unrotate8_kernel<BF16><<<dim3(blocks), dim3(256), 0, stream>>>(b);
  } else {
    const size_t total = (size_t)b.T * (b.N / 2);
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
    unrotate_kernel<BF16><<<dim3(blocks), dim3(256), 0, stream>>>(b);
  }
  const dim3 rows((b.T + 3) / 4), threads(256);
  switch (b.H) {
    case 1024: activations_kernel<BF16, 2><<<rows, threads, 0, stream>>>(b); break;
    case 2048: activations_kernel<BF16, 4><<<rows, threads, 0, stream>>>(b); break;
    case 4096: activations_kernel<BF16, 8><<<rows, threads, 0, stream>>>(b); break;
    default: activations_kernel<BF16, 0><<<rows, threads, 0, stream>>>(b); break;
  }
  if (b.dbias) return colsum<BF16, 0>(b, b.N, b.dbias, stream);
  return hipGetLastError();
}

template <bool BF16>
hipError_t post_gemm(const BackwardArgs& b, hipStream_t stream) {
  const dim3 rows((b.T + 3) / 4), threads(256);
  switch (b.H) {
    case 1024: norm_grad_kernel<BF16, 2><<<rows, threads, 0, stream>>>(b); break;
    case 2048: norm_grad_kernel<BF16, 4><<<rows, threads, 0, stream>>>(b); break;
    case 4096: norm_grad_kernel<BF16, 8><<<rows, threads, 0, stream>>>(b); break;
    default: norm_grad_kernel<BF16, 0><<<rows, threads, 0, stream>>>(b); break;
  }
  return colsum<BF16, 1>(b, b.H, b.dw_norm, stream);
}

}  // namespace

int backward_colsum_chunks(int T) { return T < kBackwardChunks ? T : kBackwardChunks; }

hipError_t launch_backward_pre_gemm(const BackwardArgs& b, hipStream_t stream) {
  return b.bf16 ? pre_gemm<true>(b, stream) : pre_gemm<false>(b, stream);
}

hipError_t launch_backward_post_gemm(const BackwardArgs& b, hipStream_t stream) {
  return b.bf16 ? post_gemm<true>(b, stream) : post_gemm<false>(b, stream);
}

}  // namespace qkv
