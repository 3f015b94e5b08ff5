// Device-side helpers shared by the kernels of the fused attention-input chain
// (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a gfx9-family buffer resource: 32-bit data format, raw (unswizzled)
// addressing.  With stride 0 the record count is a byte bound; loads beyond it
// return zero and stores beyond it are dropped.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kBufferWord3);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
  return __builtin_bit_cast(u32x4, v);
}

__device__ __forceinline__ void buf_store16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)byte_off, 0, 0);
}
// The same as a non-temporal (streaming) store, for a forward's final outputs, which no
// later step of the kernel reads: they do not displace the operand steps that the
// workgroups of an XCD share in its L2 (measured on the single-launch prefill, two boxes:
// Qwen-7B 1330-1333 -> 1307-1309 and 1323-1326 -> 1295-1302 us, the Llama-7B gated MLP
// 1199-1200 -> 1182-1186 us, the pre-pass form's Qwen-7B pair 1169 -> 1159-1163 us; the
// other prefill shapes unchanged).
__device__ __forceinline__ void buf_store16_nt(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)byte_off, 0, 2);
}

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even and keeps
// NaN a NaN (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 a = (__bf16)f;
  return __builtin_bit_cast(uint16_t, a);
}

// cos and sin of the rotary angle pos * theta^(-2i/d).  `rev` is that frequency in
// revolutions per position, theta^(-2i/d) / (2 pi), prepared in fp64 on the host.
// The product is formed in fp64 and reduced to the fraction of a turn there, so
// positions up to 2^31 keep their angle to ~1e-9 rad; the hardware sin/cos
// (v_sin_f32 / v_cos_f32, which take the angle in turns) evaluate the fraction to
// ~1.2e-7 absolute.
__device__ __forceinline__ void rope_cos_sin(int32_t pos, double rev, float& c, float& s) {
  const double turns = (double)pos * rev;
  const float frac = (float)(turns - floor(turns));  // [0, 1) turn
  s = __builtin_amdgcn_sinf(frac);
  c = __builtin_amdgcn_cosf(frac);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace qkv
