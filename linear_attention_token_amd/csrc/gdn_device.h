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

// Non-temporal 16-byte accesses, for streams touched once per step (read-once inputs, results
// read back only by a later kernel): they do not displace data that is reused soon from the
// caches.
typedef uint32_t u32x4nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldnt16(const void* p) {
  const u32x4nt t = __builtin_nontemporal_load(reinterpret_cast<const u32x4nt*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void stnt16(void* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4nt{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4nt*>(p));
}

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

// 32x32x16 bf16 MFMA, fp32 accumulate. With lane l, i = l % 32, q = l / 32:
//   A operand: row i, 8 consecutive k starting at 8q;  B operand: column i, the same 8 k;
//   accumulator element e: row 8 (e / 4) + 4q + e % 4, column i.
// One wave per SIMD keeps the matrix pipe busier with this shape than with 16x16x32.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32x32x16(const short8& a, const short8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// 16x16x4 fp32 MFMA. A: row i, k = q; B: column i, k = q; accumulator as above.
__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ short8 ld_short8(const void* p) {
  return *reinterpret_cast<const short8*>(p);
}

// 16x16x16 bf16 MFMA, fp32 accumulate. A: row i, 4 consecutive k starting at 4q; B: column i, the
// same 4 k; accumulator as above -- so an accumulator tile, rounded, is directly a B operand.
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16x16x16(const short4v& a, const short4v& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ short4v ld_short4(const void* p) {
  return *reinterpret_cast<const short4v*>(p);
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// The same sums without LDS traffic (group_sum's shuffles become ds_bpermute on this target):
// rotations inside each 16-lane row by DPP (row_ror 8, 4, 2, 1 leave every lane of the row with the
// row's sum), then gfx950's row swaps add row pairs (v_permlane16_swap: rows 0+1 and 2+3) and the two
// wave halves (v_permlane32_swap). Each step adds a lane's value to its partner's, so every lane of a
// group ends with bitwise the same sum.
template <int ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false));
}
// v + v of lane ^ 32 and v + v of lane ^ 16. The swaps are written as inline asm on two copies of v:
// this compiler folds the two results of its permlane-swap builtins into one register when both
// inputs are the same value (it then adds a result to itself). The s_nops cover the wait states
// between a VALU write and a permlane read, and between the swap and the next read.
__device__ __forceinline__ float half_pair_sum(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return a + b;
}
__device__ __forceinline__ float row_pair_sum(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return a + b;
}
template <int width>
__device__ __forceinline__ float wave_sum(float v) {
  static_assert(width == 16 || width == 32 || width == 64, "16, 32 or 64 lanes");
  v += dpp_f32<0x128>(v);  // row_ror:8
  v += dpp_f32<0x124>(v);  // row_ror:4
  v += dpp_f32<0x122>(v);  // row_ror:2
  v += dpp_f32<0x121>(v);  // row_ror:1
  if (width >= 32) v = row_pair_sum(v);
  if (width == 64) v = half_pair_sum(v);
  return v;
}

// ---- direct global -> LDS loads with explicit waits ----------------------------------------------
// The compiler's own wait insertion treats these loads conservatively (a full vmcnt(0) at barriers),
// so they are issued from inline asm and waited for with explicit vmcnt counts.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}
// 16 (dma16) or 4 (dma4) bytes per lane from gptr to LDS address lds + size * lane; `lds` must be
// the same in all lanes. M0 (the LDS base of these loads) is an output of the asm, so the compiler
// keeps no value of its own in M0 across it.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  int m0_out;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : "={m0}"(m0_out) : "v"(gptr), "s"(m0v) : "memory");
  (void)m0_out;
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  int m0_out;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" : "={m0}"(m0_out) : "v"(gptr), "s"(m0v) : "memory");
  (void)m0_out;
}
// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Row order pi used between the WY kernel and the chunk scan: inside every block of 32 rows,
// position 4q + r (q, r < 4) holds row 8q + r and position 16 + 4q + r holds row 8q + 4 + r. With
// it, accumulator tiles 2s and 2s + 1 of an MFMA lane (rows 4q + r) are together the 8 consecutive
// rows 32s + 8q .. +7 that an operand lane covers, so accumulators feed the next product directly.
__device__ __forceinline__ int pi32(int x) {
  const int b = x & ~31, y = x & 31;
  return b + ((y & 15) >> 2) * 8 + (y >> 4) * 4 + (y & 3);
}

// LDS transpose read (ds_read_b64_tr_b16): in each group of 16 lanes, lane i passes the address of
// row i / 4, columns 4 (i % 4) .. +3 of a 4 x 16 block of 16-bit elements, and receives column i of
// the block's four rows (element r = row r).
__device__ __forceinline__ short4v ld_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) short4v lds_short4v;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p));
}

// Two fp32 accumulator tiles (4 + 4 rows) -> one bf16 MFMA operand (8 k values).
__device__ __forceinline__ short8 pack8(const f32x4& a, const f32x4& b) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v v = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                    pack_bf16x2(b[2], b[3])};
  return __builtin_bit_cast(short8, v);
}

// Buffer loads: a wave-uniform base and size in SGPRs, a 32-bit byte offset per lane and a
// constant (SGPR) offset per access, so a run of loads at fixed distances needs one address
// register. Out-of-range accesses read zero.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// 16 bytes, non-temporal (streamed data that is read once).
__device__ __forceinline__ float4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}

// 16 bytes through the caches.
__device__ __forceinline__ float4 buf_ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Item of block b of n when each of the 8 XCDs (to which blocks are dispatched round robin) walks
// its own contiguous range of items: block b serves item (b % 8) (n / 8) + b / 8, for n a multiple
// of 8 (else item b).
__device__ __forceinline__ unsigned xcd_range_item(unsigned b, unsigned n) {
  return n % 8u == 0u ? (b % 8u) * (n / 8u) + b / 8u : b;
}

// One fp32 accumulator tile -> bf16 operand; two bf16 tiles -> one 16-byte piece.
__device__ __forceinline__ short4v pack4(const f32x4& a) {
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  const u32x2v v = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
  return __builtin_bit_cast(short4v, v);
}
__device__ __forceinline__ short8 join8(const short4v& a, const short4v& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Unit and position inside the unit of block b under the XCD-aware numbering (see xcd_blocks):
// block b = 8 * (per_unit * j + sub) + x serves unit 8 * j + x.
__device__ __forceinline__ void xcd_item(int b, int per_unit, int& unit, int& sub) {
  const int x = b & 7, k = b >> 3, j = k / per_unit;
  unit = 8 * j + x;
  sub = k - j * per_unit;
}

// One thread of the conv-cache tail (ConvTailArgs in gdn_internal.h): sequence n, channel group g.
template <typename IO, typename A>
__device__ __forceinline__ void conv_tail_piece(const A& a, int n, int64_t g) {
  constexpr int VEC = vec16<IO>::N;
  const int64_t c0 = g * VEC;
  if (n >= a.n_seqs || c0 >= a.C) return;
  const int64_t s0 = min<int64_t>(max<int64_t>(a.cu[n], 0), a.T);
  const int64_t s1 = min<int64_t>(max<int64_t>(a.cu[n + 1], s0), a.T);
  const IO* src;
  int64_t ld;
  if (c0 < a.qk_ch) { src = static_cast<const IO*>(a.q) + c0; ld = a.ld_q; }
  else if (c0 < 2 * a.qk_ch) { src = static_cast<const IO*>(a.k) + (c0 - a.qk_ch); ld = a.ld_k; }
  else { src = static_cast<const IO*>(a.v) + (c0 - 2 * a.qk_ch); ld = a.ld_v; }
  const IO* cin = static_cast<const IO*>(a.conv_in);
  IO* cout = static_cast<IO*>(a.conv_out);
  float r[3][VEC];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int64_t pos = s1 - 3 + j;
    if (pos >= s0) vec16<IO>::ld(src + pos * ld, r[j]);
    else if (cin != nullptr) vec16<IO>::ld(cin + (int64_t(n) * 3 + (3 + (pos - s0))) * a.C + c0, r[j]);
    else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) r[j][e] = 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) vec16<IO>::st(cout + (int64_t(n) * 3 + j) * a.C + c0, r[j]);
}

// Logistic function and SiLU on the hardware exp2 / reciprocal.
__device__ __forceinline__ float sigmoidf_(float z) { return frcp(1.0f + __expf(-z)); }
__device__ __forceinline__ float siluf_(float u) { return u * frcp(1.0f + __expf(-u)); }

}  // namespace gdn
