// Device-side helpers shared by the gfx950 kernels: vector types, bf16 / E4M3 / E2M1 / fp16
// conversions with the exact rounding the layer's codes are defined by.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace svdq {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8_t;
typedef __attribute__((ext_vector_type(4))) int32_t i32x4_t;
typedef __attribute__((ext_vector_type(16))) int32_t i32x16_t;
typedef __attribute__((ext_vector_type(2))) uint16_t u16x2_t;

constexpr int NVFP4_BLOCK = 16;
constexpr int INT4_GROUP = 64;

// Raw (unstrided) buffer resource over `bytes` bytes from `base`.  A buffer load whose offset is
// at or past `bytes` returns zeros without touching memory, so a look-ahead load that has run
// past the data can still be issued, with kNoLoad as its offset: every path through a loop then
// issues the same loads, which keeps the compiler's wait counts exact instead of draining the
// loads in flight at the loop head.
constexpr uint32_t kNoLoad = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// Cache-policy operand of a streaming (nontemporal) buffer load.
constexpr int kNt = 2;

// s_waitcnt vmcnt(n) (other counters untouched), gfx9 encoding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// Non-negative fp32 magnitude -> E4M3 code, nearest even, satfinite at 448; *val receives the
// code's value.  Normal range: keep 3 mantissa bits of the fp32 pattern with RNE on the bits
// (a carry moves into the exponent); subnormal range (below 2^-6): quantum 2^-9.
__device__ __forceinline__ uint32_t e4m3_encode_pos(float q, float* val) {
  if (q >= 448.0f) {
    *val = 448.0f;
    return 0x7Eu;
  }
  if (q < 0.015625f) {
    float t = __builtin_rintf(q * 512.0f);  // exact scaling; rint rounds half to even
    *val = t * 0.001953125f;
    return (uint32_t)t;  // t == 8 is the smallest normal, code 0x08
  }
  uint32_t b = __float_as_uint(q);
  b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
  *val = __uint_as_float(b);
  return (b >> 20) - (120u << 3);
}

// Signed E4M3 element code: the magnitude as above (satfinite at 448), bit 7 the sign of q
// (also for zero).
__device__ __forceinline__ uint32_t e4m3_encode_signed(float q) {
  float v;
  return e4m3_encode_pos(fabsf(q), &v) | ((__float_as_uint(q) >> 31) << 7);
}

// Four fp32 values -> four E4M3 codes (value i in byte i), round to nearest even, saturating at
// ±448: the same codes as e4m3_encode_signed, from the hardware conversion after a clamp to
// ±448 (the conversion turns values beyond the format's range into NaN).  An in-bounds
// comparison over every code midpoint (and its fp32 neighbours), a 2^-12 grid over ±600 and a
// million random finite values found no difference.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const float lo = -448.0f, hi = 448.0f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, lo, hi),
                                          __builtin_amdgcn_fmed3f(b, lo, hi), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, lo, hi),
                                      __builtin_amdgcn_fmed3f(d, lo, hi), w, true);
  return (uint32_t)w;
}
// Two values -> two E4M3 codes in the low 16 bits (as e4m3_pack4).
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b) {
  const float lo = -448.0f, hi = 448.0f;
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, lo, hi),
                                                   __builtin_amdgcn_fmed3f(b, lo, hi), 0, false) &
         0xFFFFu;
}

// MX block exponent ("MiniMax-H3 — MXFP8 (weight-quantized, vLLM-Omni native layout)", section
// "Quant format": E8M0 scale per 32; block exponent by the OCP microscaling rule):
// floor(log2 a) − emax for a block maximum a > 0, −127 for a == 0, clamped to [−127, 127].
// frexp's exponent is floor(log2 a) + 1, subnormal a included.
__device__ __forceinline__ int mx_exponent(float a, int emax) {
  if (a == 0.0f) return -127;
  const int e = __builtin_amdgcn_frexp_expf(a) - 1 - emax;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// NVFP4 block scale: q = a / d6, s = E4M3(q), S = s·g, inv = 1/S (0 when S == 0).  The code
// comes from the hardware conversion (as e4m3_pack2) and its value from the exact hardware
// decode.
__device__ __forceinline__ uint32_t nvfp4_block_scale(float a, float g, float d6, float* inv) {
  const uint32_t code = e4m3_pack2(a / d6, 0.0f) & 0xFFu;
  const float sval = __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
  float S = sval * g;
  *inv = (S != 0.0f) ? 1.0f / S : 0.0f;
  return code;
}

// Two fp32 values (already multiplied by the block's inverse scale) -> two E2M1 nibbles written
// into byte `sel` of `old` (low nibble = first value).  The hardware conversion with scale 1.0
// rounds to nearest even, saturates at ±6 and keeps the sign of zero.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y0, y1, 1.0f, SEL);
}

// Eight fp32 values -> one dword of eight E2M1 nibbles (element i in nibble i).
__device__ __forceinline__ uint32_t e2m1_pack8(const float* y) {
  uint32_t w = 0;
  w = e2m1_pack2<0>(w, y[0], y[1]);
  w = e2m1_pack2<1>(w, y[2], y[3]);
  w = e2m1_pack2<2>(w, y[4], y[5]);
  w = e2m1_pack2<3>(w, y[6], y[7]);
  return w;
}

// int4 code from fp32 value times inverse scale: clamp(rint(v), -8, 7) as a nibble.
__device__ __forceinline__ uint32_t int4_code(float v) {
  int c = (int)__builtin_rintf(v);
  c = c < -8 ? -8 : (c > 7 ? 7 : c);
  return (uint32_t)c & 0xFu;
}

// Eight fp32 low-rank activations D[k0 .. k0+8), times `mul`, as an exact-to-2^-16 pair of bf16
// MFMA operands: hi = bf16(d), lo = bf16(d - hi) (d - hi is exact in fp32), so hi·u + lo·u
// carries d to 16 significant bits through a bf16 MFMA.  `valid` false gives zeros (rank
// padding).
__device__ __forceinline__ void lowrank_operand(const float* p, bool valid, float mul,
                                                bf16x8_t& hi, bf16x8_t& lo) {
  u32x4_t a = u32x4_t{0u, 0u, 0u, 0u}, b = u32x4_t{0u, 0u, 0u, 0u};
  if (valid) {
    a = reinterpret_cast<const u32x4_t*>(p)[0];
    b = reinterpret_cast<const u32x4_t*>(p)[1];
  }
  const float d[8] = {__uint_as_float(a[0]) * mul, __uint_as_float(a[1]) * mul,
                      __uint_as_float(a[2]) * mul, __uint_as_float(a[3]) * mul,
                      __uint_as_float(b[0]) * mul, __uint_as_float(b[1]) * mul,
                      __uint_as_float(b[2]) * mul, __uint_as_float(b[3]) * mul};
  u32x4_t vh, vl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t ph = pack_bf16x2(d[2 * j], d[2 * j + 1]);
    vh[j] = ph;
    vl[j] = pack_bf16x2(d[2 * j] - bf16_lo(ph), d[2 * j + 1] - bf16_hi(ph));
  }
  hi = __builtin_bit_cast(bf16x8_t, vh);
  lo = __builtin_bit_cast(bf16x8_t, vl);
}

// 8 E2M1 codes (one dword, element i in nibble i) times a block scale -> 8 exact fp16 values.
__device__ __forceinline__ f16x8_t dequant8(uint32_t codes, f16x2_t s2) {
  f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
  f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
  f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
  f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
  f16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Two E4M3 scale bytes (low byte first) -> fp16 pair, exactly: the E4M3 pattern without its
// sign, shifted into an fp16 exponent/mantissa, is the value times 2^-8 (subnormals included),
// and the multiply by 256 is exact.
__device__ __forceinline__ f16x2_t e4m3x2_to_f16x2(uint32_t x) {
  const uint32_t bits = ((x & 0x7Fu) << 7) | ((x & 0x7F00u) << 15);
  return __builtin_bit_cast(f16x2_t, bits) * f16x2_t{(_Float16)256.0f, (_Float16)256.0f};
}

// Exact values of stored element codes: an E2M1 nibble (sign in bit 3) and an E4M3 byte (sign in
// bit 7; normal (8 + m)·2^(e − 10), subnormal m·2^-9).
__device__ __forceinline__ double e2m1_value(uint32_t nib) {
  const uint32_t m = nib & 7u;
  const double mag = m < 4u ? 0.5 * (double)m : (m == 4u ? 2.0 : m == 5u ? 3.0 : m == 6u ? 4.0 : 6.0);
  return (nib & 8u) ? -mag : mag;
}
__device__ __forceinline__ double e4m3_value(uint32_t b) {
  const int e = (int)((b >> 3) & 15u), m = (int)(b & 7u);
  const double mag = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (b & 0x80u) ? -mag : mag;
}

// Running maximum of non-negative floats stored as their bit patterns (monotone for >= 0).
__device__ __forceinline__ void atomic_max_pos(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

}  // namespace svdq
