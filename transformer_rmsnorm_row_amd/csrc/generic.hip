// Generic fused kernel: normalise-on-load, projection, bias and rotary epilogue with
// fp32 FMA tiles.  It runs every shape the plan accepts in both dtypes; it is the
// path of fp32 plans (whose tolerance needs true fp32 products) and of bf16 shapes
// the MFMA kernels do not take.
//
// What it computes follows the fused-kernel listing of the page "Liger-Kernel底层优化：
// 新一代内核级推理加速引擎介绍" (section "融合内核是如何工作的？来看一段简化版实现"):
// each input element enters the dot products scaled by the norm weight, the token's
// sum of squares is gathered from the same staged values and its inverse RMS scales
// the dot products (the normalised row never goes to memory, and no separate pass
// over x is needed), the bias is added to each dot product, and the rotation pairs
// feature i with i + head_dim/2.
// Unlike the listing (one thread per output feature re-reading the whole row and
// weight column), a 256-thread block computes a 32-token x 32-pair tile from LDS:
// each thread owns 4 tokens x one rotation pair (columns c and c + head_dim/2), so
// both halves of a pair sit in the same thread for the rotation.
#include "device_common.h"
#include "launch.h"

namespace qkv {

namespace {

constexpr int BT = 32;   // tokens per block
constexpr int BU = 32;   // rotation pairs (units) per block: 64 output columns
constexpr int BK = 32;   // reduction slice staged in LDS

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if constexpr (BF16)
    return bf16_to_f32(((const uint16_t*)p)[i]);
  else
    return ((const float*)p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* p, size_t i, float v) {
  if constexpr (BF16)
    ((uint16_t*)p)[i] = f32_to_bf16(v);
  else
    ((float*)p)[i] = v;
}

// Output column of the first member of rotation pair u (pairs enumerate, head by
// head, the features i < head_dim/2 of every head of Q, K and V).
__device__ __forceinline__ int pair_col(int u, int half, int d) { return (u / half) * d + (u % half); }

template <bool BF16>
__global__ __launch_bounds__(256) void generic_kernel(ForwardArgs a) {
  __shared__ float As[BK][BT + 1];
  __shared__ float Bs[BK][2 * BU + 1];

  const int tid = threadIdx.x;
  const int tx = tid % BU;         // pair within the tile
  const int ty = tid / BU;         // 0..7: tokens ty*4 .. ty*4+3
  const int t0 = blockIdx.x * BT;
  const int u0 = blockIdx.y * BU;
  const int half = a.d / 2;
  const int units = a.N / 2;

  float acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j][0] = acc[j][1] = 0.f;
  // sums of squares of the raw x values this thread stages (rows tid / 32 + 8 m); 1/rms
  // scales the accumulators in the epilogue: diag(r) (X diag(w)) W = (diag(r) X diag(w)) W
  float ssq[4] = {0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < a.H; k0 += BK) {
    // A slice: x[t,k] * w_norm[k], 32 x 32, 4 per thread (row tid / 32 + 8 m, column
    // tid % 32), and the squares of x into the row sums.
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      int e = tid + 256 * m;
      int r = e / BK, cc = e % BK;
      int t = t0 + r, kk = k0 + cc;
      float xv = 0.f, val = 0.f;
      if (t < a.T && kk < a.H) {
        xv = load_elem<BF16>(a.x, (size_t)t * a.H + kk);
        val = xv * load_elem<BF16>(a.w_norm, kk);
      }
      ssq[m] = fmaf(xv, xv, ssq[m]);
      As[cc][r] = val;
    }
    // B slice: the two columns of each pair, 32 x 64, 8 per thread.
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      int e = tid + 256 * m;
      int kk = e / (2 * BU), s = e % (2 * BU);
      int u = u0 + (s % BU);
      float val = 0.f;
      if (u < units && k0 + kk < a.H) {
        int col = pair_col(u, half, a.d) + (s / BU) * half;
        val = load_elem<BF16>(a.w, (size_t)(k0 + kk) * a.N + col);
      }
      Bs[kk][s] = val;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
      float b0 = Bs[kk][tx], b1 = Bs[kk][BU + tx];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float av = As[kk][ty * 4 + j];
        acc[j][0] = fmaf(av, b0, acc[j][0]);
        acc[j][1] = fmaf(av, b1, acc[j][1]);
      }
    }
    __syncthreads();
  }

  // 1/rms of the block's 32 rows: the 32 lanes staging a row add their sums
  __shared__ float s_rinv[BT];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float v = ssq[m];
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, 32);
    if ((tid & 31) == 0) s_rinv[tid / 32 + 8 * m] = rsqrtf(v / (float)a.H + a.eps);
  }
  __syncthreads();

  const int u = u0 + tx;
  if (u >= units) return;
  const int c = pair_col(u, half, a.d);
  const int cp = c + half;
  const int i = u % half;
  const bool rotate = c < a.Nq + a.Nkv;
  float b0 = 0.f, b1 = 0.f;
  if (a.bias) {
    b0 = load_elem<BF16>(a.bias, c);
    b1 = load_elem<BF16>(a.bias, cp);
  }
  void* out;
  int width, oc;
  if (c < a.Nq) {
    out = a.q; width = a.Nq; oc = c;
  } else if (c < a.Nq + a.Nkv) {
    out = a.k; width = a.Nkv; oc = c - a.Nq;
  } else {
    out = a.v; width = a.Nkv; oc = c - a.Nq - a.Nkv;
  }
  const bool to_cache = a.slots != nullptr && c >= a.Nq;  // K/V rows go to cache slots
  const double rev = a.rev_freq[i];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int t = t0 + ty * 4 + j;
    if (t >= a.T) break;
    const float rinv = s_rinv[ty * 4 + j];
    float y0 = fmaf(acc[j][0], rinv, b0), y1 = fmaf(acc[j][1], rinv, b1);
    if (rotate) {
      float cs, sn;
      rope_cos_sin(a.pos[t], rev, cs, sn);
      float r0 = y0 * cs - y1 * sn;
      float r1 = y1 * cs + y0 * sn;
      y0 = r0;
      y1 = r1;
    }
    int row = t;
    if (to_cache) {
      row = a.slots[t];
      if (row < 0 || row >= a.cache_rows) continue;
    }
    store_elem<BF16>(out, (size_t)row * width + oc, y0);
    store_elem<BF16>(out, (size_t)row * width + oc + half, y1);
  }
}

}  // namespace

hipError_t launch_generic(const ForwardArgs& a, hipStream_t stream) {
  dim3 grid((a.T + BT - 1) / BT, (a.N / 2 + BU - 1) / BU), block(256);
  if (a.bf16)
    generic_kernel<true><<<grid, block, 0, stream>>>(a);
  else
    generic_kernel<false><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qkv
