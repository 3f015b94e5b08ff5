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
template <bool BF16>
__global__ __launch_bounds__(256) void activations_kernel(BackwardArgs b) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= b.T) return;
  const size_t row = (size_t)t * b.H;
  float ss = 0.f;
  for (int k = lane; k < b.H; k += 64) {
    const float v = ld<BF16>(b.x, row + k);
    ss = fmaf(v, v, ss);
  }
  const float r = rsqrtf(wave_sum(ss) / (float)b.H + b.eps);
  if (lane == 0) b.inv_rms[t] = r;
  for (int k = lane; k < b.H; k += 64) st<BF16>(b.act, row + k, ld<BF16>(b.x, row + k) * r * ld<BF16>(b.w_norm, k));
}

// One wave per token: dx from ga (fp32), x, w and r.
template <bool BF16>
__global__ __launch_bounds__(256) void norm_grad_kernel(BackwardArgs b) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= b.T) return;
  const size_t row = (size_t)t * b.H;
  float inner = 0.f;
  for (int k = lane; k < b.H; k += 64) inner = fmaf(b.ga[row + k] * ld<BF16>(b.w_norm, k), ld<BF16>(b.x, row + k), inner);
  inner = wave_sum(inner);
  const float r = b.inv_rms[t];
  const float c2 = r * r * r / (float)b.H * inner;
  for (int k = lane; k < b.H; k += 64)
    st<BF16>(b.dx, row + k, r * ld<BF16>(b.w_norm, k) * b.ga[row + k] - c2 * ld<BF16>(b.x, row + k));
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
  const size_t total = (size_t)b.T * (b.N / 2);
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  unrotate_kernel<BF16><<<dim3(blocks), dim3(256), 0, stream>>>(b);
  activations_kernel<BF16><<<dim3((b.T + 3) / 4), dim3(256), 0, stream>>>(b);
  if (b.dbias) return colsum<BF16, 0>(b, b.N, b.dbias, stream);
  return hipGetLastError();
}

template <bool BF16>
hipError_t post_gemm(const BackwardArgs& b, hipStream_t stream) {
  norm_grad_kernel<BF16><<<dim3((b.T + 3) / 4), dim3(256), 0, stream>>>(b);
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
