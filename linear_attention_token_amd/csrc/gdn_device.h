// Device-side helpers shared by the GDN kernels: bf16 <-> fp32, io loads/stores, MFMA operand
// types and wave reductions. gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kWave = 64;

// bf16 kept as raw 16-bit storage so every conversion is explicit.
struct bf16 {
  uint16_t x;
};

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with the hardware converter (v_cvt_pk_bf16_f32: round to nearest even, NaN kept).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two fp32 -> one dword of two bf16 (a in the low half), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Hardware reciprocal (v_rcp_f32, 1 ulp).
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Scalar io access for the two io types.
template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct io<bf16> {
  static __device__ __forceinline__ float ld(const bf16* p) { return bf2f(p->x); }
  static __device__ __forceinline__ void st(bf16* p, float v) { p->x = f2bf(v); }
};

// 16-byte vector access: VEC elements of the io type (8 bf16 or 4 fp32).
template <typename T> struct vec16;
template <> struct vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void cvt(const uint4& v, float* out) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ void ld(const float* p, float* out) {
    float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
  static __device__ __forceinline__ void st(float* p, const float* in) {
    *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
  }
};
template <> struct vec16<bf16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void cvt(const uint4& v, float* out) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void ld(const bf16* p, float* out) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void st(bf16* p, const float* in) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// MFMA operand / accumulator vectors.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16x16x32 bf16 MFMA, fp32 accumulate.  With lane l, i = l % 16, q = l / 16:
//   A operand: row i, 8 consecutive k starting at 8q;  B operand: column i, the same 8 k;
//   accumulator: rows 4q + r (r = 0..3), column i.
__device__ __forceinline__ f32x4 mfma16x16x32(const short8& a, const short8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16x4 fp32 MFMA. A: row i, k = q; B: column i, k = q; accumulator as above.
__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ short8 ld_short8(const void* p) {
  return *reinterpret_cast<const short8*>(p);
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Logistic function and SiLU on the hardware exp2 / reciprocal.
__device__ __forceinline__ float sigmoidf_(float z) { return frcp(1.0f + __expf(-z)); }
__device__ __forceinline__ float siluf_(float u) { return u * frcp(1.0f + __expf(-u)); }

}  // namespace gdn
