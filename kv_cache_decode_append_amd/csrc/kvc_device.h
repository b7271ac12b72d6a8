// Device-side helpers shared by the kvc kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));   // 4 x 16-bit MFMA operand

// Storage tag for bfloat16 elements (raw 16-bit patterns).
struct bf16_tag {};
// Storage tag for fp8 E4M3 codes with one fp32 scale per (token, kv head) row;
// the kernels compute on them in bf16 (every E4M3 value is a bf16 value).
struct fp8_tag {};

template <typename T> struct ElemBytes;
template <> struct ElemBytes<float> { static constexpr int value = 4; };
template <> struct ElemBytes<bf16_tag> { static constexpr int value = 2; };
template <> struct ElemBytes<fp8_tag> { static constexpr int value = 1; };

// ---------------------------------------------------------------------------
// Buffer resources. A raw (stride 0) buffer descriptor over [base, base+bytes):
// loads at offsets >= bytes return zero and touch no memory, so a descriptor of
// 0 bytes turns a load into a no-op. Word 3 = 0x00020000 selects the 32-bit
// raw data format on gfx9-family parts (CDNA included).
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}

// Same load with the non-temporal (nt) cache policy: for data read once per
// kernel, such as the K/V tiles of a decode step, so that it streams through
// the caches instead of displacing reused data.
constexpr int kCachePolicyNonTemporal = 2;
__device__ __forceinline__ u32x4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kCachePolicyNonTemporal);
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32), which rounds
// to nearest even in the default rounding mode (finite inputs).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---------------------------------------------------------------------------
// fp8 E4M3 (OCP: bias 7, largest finite 448, S.1111.111 = NaN)
// ---------------------------------------------------------------------------
constexpr float kE4M3Max = 448.f;
// Rows whose largest magnitude is below this are stored as zeros (scale 0), so
// that 448 / amax stays finite.
constexpr float kZeroRowAmax = 0x1p-100f;

// Code of a finite value: nearest E4M3 value, ties to the even code (the even
// mantissa), magnitudes above 448 clamped to 448; values that round to zero
// give +0.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const float a = fminf(fabsf(y), kE4M3Max);
  uint32_t code;
  if (a < 0.015625f) {
    // below 2^-6 the codes are the multiples of 2^-9 (scaling by 2^9 is exact)
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    // round the fp32 mantissa to 3 bits (ties to even), carrying into the
    // exponent; then rebias the exponent from 127 to 7
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  }
  return (y < 0.f && code != 0u) ? (code | 0x80u) : code;
}

// Eight codes (little-endian bytes of two words) to eight bf16 values in four
// words, exactly (the gfx950 conversion reads OCP E4M3).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(const u32x2& w) {
  return u32x4{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, true))};
}

// Eight bf16 values (four words) times inv, each coded to E4M3.
__device__ __forceinline__ u32x2 bf16x8_to_e4m3x8(const u32x4& v, float inv) {
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[2 * i] = f32_to_e4m3(__uint_as_float(v[i] << 16) * inv);
    c[2 * i + 1] = f32_to_e4m3(__uint_as_float(v[i] & 0xffff0000u) * inv);
  }
  return u32x2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
               c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
}

// Largest magnitude of eight bf16 values (four words).
__device__ __forceinline__ float bf16x8_amax(const u32x4& v) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    m = fmaxf(m, fmaxf(fabsf(__uint_as_float(v[i] << 16)),
                       fabsf(__uint_as_float(v[i] & 0xffff0000u))));
  return m;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------------------
// Cross-lane reductions with DPP inside a row of 16 lanes.
// All lanes of the group end with the group's result.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each 16

// Reduce over an aligned group of N lanes, N in {8, 16}.
template <int N>
__device__ __forceinline__ float group_max(float v) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  v = fmaxf(v, dpp_f<kQuadXor1>(v));
  v = fmaxf(v, dpp_f<kQuadXor2>(v));
  v = fmaxf(v, dpp_f<kRowHalfMirror>(v));
  if constexpr (N == 16) v = fmaxf(v, dpp_f<kRowMirror>(v));
  return v;
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  v += dpp_f<kQuadXor1>(v);
  v += dpp_f<kQuadXor2>(v);
  v += dpp_f<kRowHalfMirror>(v);
  if constexpr (N == 16) v += dpp_f<kRowMirror>(v);
  return v;
}

// Reduce across the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with the gfx950 row-swap permutes: swapping a value with itself across row
// pairs leaves each lane with its own and its partner's copy.
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ void flag_error(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

}  // namespace kvc
