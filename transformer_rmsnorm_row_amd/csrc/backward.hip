// Backward of the fused attention-input chain: the elementwise and row/column
// reduction kernels around the two plain GEMMs (gemm.hip).
//
// Chain rule of the forward (RMSNorm -> projection (+bias) -> rotate-half rotary
// embedding of Q and K) for upstream gradients dQ, dK, dV, with r[t] the token's
// inverse RMS and a = x r w the normalised activations:
//   gy   = the rotation by -angle of each (dQ, dK) pair, dV unchanged
//   db   = sum over tokens of gy
//   dW   = a^T gy,  ga = gy W^T
//   dw   = sum over tokens of ga * x * r
//   dx_j = r w_j ga_j - (r^3 / H) x_j sum_k ga_k w_k x_k
// Both r and w are folded out of the normalised activations, which are never formed:
// with g = r gy (each token's row scaled by its r, rounded once to the plan dtype) and
// G = g W^T = r ga,
//   dW   = diag(w) x^T g          (x itself is the GEMM operand; w scales the result rows)
//   db   = sum over tokens of g / r
//   dw   = sum over tokens of G * x
//   dx_j = w_j G_j - (r^2 / H) x_j sum_k G_k w_k x_k
// which is the same algebra (the page's operator-fusion section fuses the norm into the
// projection the same way).  g is stored transposed, g^T [N][Tp] with Tp = T rounded up
// to 32 and the pad zero: both GEMMs then take one operand with k contiguous and one with
// k as the row index, the pairing the MFMA GEMM runs fastest.  Column sums are two-pass
// (fixed chunks of tokens, then the chunks in order) and row sums one wave per row in a
// fixed order, so every result is deterministic.
#include <algorithm>

#include "device_common.h"
#include "backward.h"
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

// Unrotate, scale and transpose: block (64 tokens, 32 consecutive rotation pairs) reads
// the pairs' two columns from dq, dk or dv (Q and K pairs turned back by -angle, V pairs
// copied), multiplies them by the token's r, stages them in LDS as [64 columns][64
// tokens], and writes the 64 g^T rows' 64-token pieces.  Pairs enumerate features i < d/2 of every head of Q, K and V; pair u
// is column (u / half) d + u % half and its partner is half further.  Tokens in [T, Tp)
// are written as zeros.
template <bool BF16>
__global__ __launch_bounds__(256) void unrotate_t_kernel(BackwardArgs b, int tp) {
  __shared__ float s[64][65];
  const int half = b.d / 2, npairs = b.N / 2;
  const int t0 = blockIdx.x * 64, u0 = blockIdx.y * 32;
  for (int e = threadIdx.x; e < 64 * 32; e += 256) {
    const int t = e >> 5, j = e & 31, u = u0 + j, tt = t0 + t;
    float y0 = 0.f, y1 = 0.f;
    if (u < npairs && tt < b.T) {
      const float r = b.inv_rms[tt];  // requested first: its latency overlaps the gradient loads
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
      const float gu = ld<BF16>(src, (size_t)tt * width + oc), gv = ld<BF16>(src, (size_t)tt * width + oc + half);
      y0 = gu;
      y1 = gv;
      if (c < b.Nq + b.Nkv) {
        float cs, sn;
        rope_cos_sin(b.pos[tt], b.rev_freq[u % half], cs, sn);
        y0 = gu * cs + gv * sn;
        y1 = gv * cs - gu * sn;
      }
      y0 *= r;
      y1 *= r;
    }
    s[j][t] = y0;
    s[32 + j][t] = y1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int jc = e >> 6, t = e & 63, tt = t0 + t;
    const int u = u0 + (jc & 31);
    if (u >= npairs || tt >= tp) continue;
    const int c = (u / half) * b.d + (u % half) + (jc >= 32 ? half : 0);
    st<BF16>(b.gy, (size_t)c * tp + tt, s[jc][t]);
  }
}

// The same with 16-byte accesses, when d/2 is a multiple of 8: block (64 tokens, 64
// pairs) loads 8 pairs' u and v halves per thread and item, stages [128 columns][64
// tokens] in fp32, and stores 8-token pieces of the gy^T rows.
template <bool BF16>
__global__ __launch_bounds__(256) void unrotate_t8_kernel(BackwardArgs b, int tp) {
  __shared__ float s[128][65];
  const int half = b.d / 2, npairs = b.N / 2;
  const int t0 = blockIdx.x * 64, u0 = blockIdx.y * 64;
  for (int e = threadIdx.x; e < 64 * 8; e += 256) {
    const int gi = e & 7, t = e >> 3, tt = t0 + t, u = u0 + 8 * gi;
    float gu[8], gv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) gu[k] = gv[k] = 0.f;
    if (u < npairs && tt < b.T) {
      const int c = (u / half) * b.d + (u % half), i0 = u % half;
      const void* src;
      int width, oc;
      if (c < b.Nq) {
        src = b.dq; width = b.Nq; oc = c;
      } else if (c < b.Nq + b.Nkv) {
        src = b.dk; width = b.Nkv; oc = c - b.Nq;
      } else {
        src = b.dv; width = b.Nkv; oc = c - b.Nq - b.Nkv;
      }
      // every load of the item is issued before any is used (one memory round trip): r,
      // the position and frequencies (read for V pairs too, whose angles are unused), the
      // two halves
      const float r = b.inv_rms[tt];
      const int32_t p = b.pos[tt];
      double fr[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) fr[k] = b.rev_freq[i0 + k];
      ld8<BF16>(src, (size_t)tt * width + oc, gu);
      ld8<BF16>(src, (size_t)tt * width + oc + half, gv);
      const bool rot = c < b.Nq + b.Nkv;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float cs, sn;
        rope_cos_sin(p, fr[k], cs, sn);
        const float x0 = gu[k], x1 = gv[k];
        gu[k] = (rot ? x0 * cs + x1 * sn : x0) * r;
        gv[k] = (rot ? x1 * cs - x0 * sn : x1) * r;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      s[8 * gi + k][t] = gu[k];
      s[64 + 8 * gi + k][t] = gv[k];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 128 * 8; e += 256) {
    const int lc = e >> 3, tq = e & 7, tt = t0 + 8 * tq;
    const int u = u0 + (lc & 63);
    if (u >= npairs || tt >= tp) continue;
    const int c = (u / half) * b.d + (u % half) + (lc >= 64 ? half : 0);
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = s[lc][8 * tq + k];
    st8<BF16>(b.gy, (size_t)c * tp + tt, v);
  }
}

// db[n] = sum over tokens of g^T[n][t] / r[t]: one wave per row, lane partial sums over
// 8-token pieces in order, then a fixed shuffle tree.  Tokens of the zero pad (t >= T)
// add nothing.
template <bool BF16>
__global__ __launch_bounds__(256) void rowsum_kernel(BackwardArgs b, int tp) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= b.N) return;
  float acc = 0.f;
  for (int t = lane * 8; t < b.T; t += 512) {
    float v[8];
    ld8<BF16>(b.gy, (size_t)n * tp + t, v);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (t + j < b.T) acc += v[j] / b.inv_rms[t + j];
  }
  acc = wave_sum(acc);
  if (lane == 0) st<BF16>(b.dbias, n, acc);
}

// One wave per token: dx from G = r ga, x, w and r.  KIT > 0: H = 512 KIT, and the
// lane's KIT x 8 values of G and x stay in registers between the inner product and dx;
// KIT = 0: any H, rows read twice.
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
      ld8<BF16>(b.ga, row + lane * 8 + 512 * m, g[m]);
      ld8<BF16>(b.w_norm, lane * 8 + 512 * m, w);
      ld8<BF16>(b.x, row + lane * 8 + 512 * m, x[m]);
#pragma unroll
      for (int j = 0; j < 8; ++j) inner = fmaf(g[m][j] * w[j], x[m][j], inner);
    }
    inner = wave_sum(inner);
    const float r = b.inv_rms[t];
    const float c2 = r * r / (float)b.H * inner;
#pragma unroll
    for (int m = 0; m < KIT; ++m) {
      float w[8];
      ld8<BF16>(b.w_norm, lane * 8 + 512 * m, w);
#pragma unroll
      for (int j = 0; j < 8; ++j) g[m][j] = w[j] * g[m][j] - c2 * x[m][j];
      st8<BF16>(b.dx, row + lane * 8 + 512 * m, g[m]);
    }
    return;
  }
  float inner = 0.f;
  for (int k = lane * 8; k < b.H; k += 512) {
    float g[8], w[8], x[8];
    ld8<BF16>(b.ga, row + k, g);
    ld8<BF16>(b.w_norm, k, w);
    ld8<BF16>(b.x, row + k, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) inner = fmaf(g[j] * w[j], x[j], inner);
  }
  inner = wave_sum(inner);
  const float r = b.inv_rms[t];
  const float c2 = r * r / (float)b.H * inner;
  for (int k = lane * 8; k < b.H; k += 512) {
    float g[8], w[8], x[8];
    ld8<BF16>(b.ga, row + k, g);
    ld8<BF16>(b.w_norm, k, w);
    ld8<BF16>(b.x, row + k, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = w[j] * g[j] - c2 * x[j];
    st8<BF16>(b.dx, row + k, g);
  }
}

// dx as norm_grad_kernel, fused with the norm-weight gradient's column sums: each wave
// takes `tpw` consecutive tokens in order, keeps its lane's KIT x 8 column sums of
// G x in registers across them, and writes them as one row of `partial` (rows in
// wave order; the final pass adds them in that order).
template <bool BF16, int KIT>
__global__ __launch_bounds__(256) void norm_grad_fused_kernel(BackwardArgs b, int tpw, int nparts) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= nparts) return;
  float col[KIT][8];
#pragma unroll
  for (int m = 0; m < KIT; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) col[m][j] = 0.f;
  for (int q = 0; q < tpw; ++q) {
    const int t = wid * tpw + q;
    if (t >= b.T) break;
    const size_t row = (size_t)t * b.H;
    float g[KIT][8], x[KIT][8];
    float inner = 0.f;
#pragma unroll
    for (int m = 0; m < KIT; ++m) {
      float w[8];
      ld8<BF16>(b.ga, row + lane * 8 + 512 * m, g[m]);
      ld8<BF16>(b.w_norm, lane * 8 + 512 * m, w);
      ld8<BF16>(b.x, row + lane * 8 + 512 * m, x[m]);
#pragma unroll
      for (int j = 0; j < 8; ++j) inner = fmaf(g[m][j] * w[j], x[m][j], inner);
    }
    inner = wave_sum(inner);
    const float r = b.inv_rms[t];
    const float c2 = r * r / (float)b.H * inner;
#pragma unroll
    for (int m = 0; m < KIT; ++m) {
      float w[8], d[8];
      ld8<BF16>(b.w_norm, lane * 8 + 512 * m, w);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        d[j] = w[j] * g[m][j] - c2 * x[m][j];
        col[m][j] = fmaf(g[m][j], x[m][j], col[m][j]);
      }
      st8<BF16>(b.dx, row + lane * 8 + 512 * m, d);
    }
  }
#pragma unroll
  for (int m = 0; m < KIT; ++m) st8<false>(b.partial, (size_t)wid * b.H + lane * 8 + 512 * m, col[m]);
}

// Column sums over tokens, pass 1: block (column group, token chunk) -> fp32 partial
// of G[t, c] * x[t, c].
template <bool BF16>
__global__ __launch_bounds__(256) void colsum_partial_kernel(BackwardArgs b, int ncols, int chunks) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= ncols) return;
  const int per = (b.T + chunks - 1) / chunks;
  const int t0 = blockIdx.y * per, t1 = min(b.T, t0 + per);
  float s = 0.f;
  // unrolled so that the loads of several tokens are in flight; the adds keep token order
#pragma unroll 8
  for (int t = t0; t < t1; ++t) {
    s = fmaf(ld<BF16>(b.ga, (size_t)t * ncols + c), ld<BF16>(b.x, (size_t)t * ncols + c), s);
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

// Final pass over many partial rows: block = 16 columns x 16 slices of the rows; each
// thread adds its slice's rows in order, then the 16 slice sums of a column are added
// in slice order.
template <bool BF16>
__global__ __launch_bounds__(256) void colsum_final16_kernel(const float* partial, void* out, int ncols, int rows) {
  __shared__ float red[16][17];
  const int cl = threadIdx.x & 15, sl = threadIdx.x >> 4;
  const int c = blockIdx.x * 16 + cl;
  const int per = (rows + 15) / 16;
  const int r0 = sl * per, r1 = min(rows, r0 + per);
  float s = 0.f;
  if (c < ncols) {
#pragma unroll 16
    for (int j = r0; j < r1; ++j) s += partial[(size_t)j * ncols + c];
  }
  red[sl][cl] = s;
  __syncthreads();
  if (sl == 0 && c < ncols) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) v += red[k][cl];
    st<BF16>(out, c, v);
  }
}

template <bool BF16>
hipError_t colsum(const BackwardArgs& b, int ncols, void* out, hipStream_t stream) {
  const int chunks = backward_colsum_chunks(b.T);
  colsum_partial_kernel<BF16><<<dim3((ncols + 255) / 256, chunks), dim3(256), 0, stream>>>(b, ncols, chunks);
  colsum_final_kernel<BF16><<<dim3((ncols + 255) / 256), dim3(256), 0, stream>>>(b.partial, out, ncols, chunks);
  return hipGetLastError();
}

template <bool BF16>
hipError_t pre_gemm(const BackwardArgs& b, hipStream_t stream) {
  const int tp = backward_token_pitch(b.T);
  // r first: the unrotate kernel scales by it
  const hipError_t e = launch_inv_rms(b.x, b.inv_rms, b.T, b.H, b.eps, BF16, stream);
  if (e != hipSuccess) return e;
  if ((b.d / 2) % 8 == 0)
    unrotate_t8_kernel<BF16><<<dim3((tp + 63) / 64, (b.N / 2 + 63) / 64), dim3(256), 0, stream>>>(b, tp);
  else
    unrotate_t_kernel<BF16><<<dim3((tp + 63) / 64, (b.N / 2 + 31) / 32), dim3(256), 0, stream>>>(b, tp);
  if (b.dbias) rowsum_kernel<BF16><<<dim3((b.N + 3) / 4), dim3(256), 0, stream>>>(b, tp);
  return hipGetLastError();
}

template <bool BF16, int KIT>
hipError_t fused_post(const BackwardArgs& b, hipStream_t stream) {
  const int tpw = (b.T + kBackwardPartials - 1) / kBackwardPartials;
  const int nparts = (b.T + tpw - 1) / tpw;
  norm_grad_fused_kernel<BF16, KIT><<<dim3((nparts + 3) / 4), dim3(256), 0, stream>>>(b, tpw, nparts);
  colsum_final16_kernel<BF16><<<dim3((b.H + 15) / 16), dim3(256), 0, stream>>>(b.partial, b.dw_norm, b.H, nparts);
  return hipGetLastError();
}

template <bool BF16>
hipError_t post_gemm(const BackwardArgs& b, hipStream_t stream) {
  switch (b.H) {
    case 1024: return fused_post<BF16, 2>(b, stream);
    case 2048: return fused_post<BF16, 4>(b, stream);
    case 4096: return fused_post<BF16, 8>(b, stream);
    default: break;
  }
  norm_grad_kernel<BF16, 0><<<dim3((b.T + 3) / 4), dim3(256), 0, stream>>>(b);
  return colsum<BF16>(b, b.H, b.dw_norm, stream);
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
