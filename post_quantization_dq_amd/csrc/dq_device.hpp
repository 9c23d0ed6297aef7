// Device-side numerics of the DualQuant solver for gfx950: element and scale rounding,
// scale projection, and the per-format block quantiser applied to one lane's chunk of 16
// consecutive elements of a row.
//
// Formats (conference entry: INT4, the MX family and NVFP4; news summary: INT4, MXINT4,
// MXFP4, NVFP4):
//   INT4    symmetric, group 64 or 128, bf16 scale s = bf16(amax/7), q = rint(v * (1/s)) in [-7,7]
//   MXINT4  32-element block, E8M0 exponent e = floor(log2 amax), q = rint(v * 2^(2-e)) in [-7,7]
//   MXFP4   32-element block, E8M0 exponent e = floor(log2 amax) - 2, q = E2M1(v * 2^-e)
//   NVFP4   16-element block, E4M3 scale sb = E4M3(amax * k6), d = sb * s_t, q = E2M1(v * (1/d))
// E2M1 rounding is to nearest with ties to the even mantissa bit, saturating at 6, keeping
// the sign of zero; it uses the gfx950 scaled FP4 conversions, whose scale operand only
// contributes its exponent field (a power-of-two division), exactly what the MX block
// exponent needs.  E4M3 uses the OCP FP8 conversion after clamping to 448 (the conversion
// itself overflows to NaN above 464).

#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dqk {

enum Fmt { INT4 = 0, MXINT4 = 1, MXFP4 = 2, NVFP4 = 3, INT8 = 4, MXINT8 = 5,
           MXFP8_E4M3 = 6, MXFP8_E5M2 = 7, MXFP6_E2M3 = 8, MXFP6_E3M2 = 9 };

// The OCP MX FP8 / FP6 element types (a minifloat under an E8M0 shared exponent).
template <int FMT>
constexpr bool mx_mini() { return FMT >= MXFP8_E4M3 && FMT <= MXFP6_E3M2; }
template <int FMT>
constexpr bool mx_fp6() { return FMT == MXFP6_E2M3 || FMT == MXFP6_E3M2; }
// Exponent of the element type's largest binade: the MX shared scale is
// 2^(floor(log2 amax) - emax).
template <int FMT>
constexpr int mini_emax() {
  return FMT == MXFP8_E4M3 ? 8 : FMT == MXFP8_E5M2 ? 15 : FMT == MXFP6_E2M3 ? 2 : 4;
}
template <int FMT>
constexpr float mini_max() {
  return FMT == MXFP8_E4M3 ? 448.0f : FMT == MXFP8_E5M2 ? 57344.0f : FMT == MXFP6_E2M3 ? 7.5f : 28.0f;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Global-memory views of the generic pointers the kernels receive: loads and stores through
// them compile to global_* instructions, which the wait counters track apart from LDS, so
// LDS reads do not wait for outstanding HBM loads.
#define DQ_GAS __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const DQ_GAS T* gp(const T* p) { return (const DQ_GAS T*)p; }
template <typename T>
__device__ __forceinline__ DQ_GAS T* gp(T* p) { return (DQ_GAS T*)p; }

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------- scalar rounding
// bf16 round-to-nearest-even of a finite fp32 (carry into the exponent is the correct
// rounding up to the next binade).
__device__ __forceinline__ float bf16_rne(float x) {
  uint32_t u = f2u(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u2f(u & 0xFFFF0000u);
}

// E4M3FN code of x >= 0 (finite), nearest with ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code_sat(float x) {
  x = fminf(x, 448.0f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0u, false) & 0xFFu;
}

// Value of a non-negative E4M3FN code (0..126): subnormals m * 2^-9, normals (8+m) * 2^(e-10).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  uint32_t e = (code >> 3) & 15u, m = code & 7u;
  return e ? ldexpf((float)(8u + m), (int)e - 10) : ldexpf((float)m, -9);
}

// floor(log2 a) for finite a > 0 (exact, also for subnormals).
__device__ __forceinline__ int floor_log2(float a) { return __builtin_amdgcn_frexp_expf(a) - 1; }

// fp32 operand whose exponent field encodes 2^e for the scaled FP4 conversions
// (valid for e in [-126, 127]; callers keep e >= -100).
__device__ __forceinline__ float pow2_operand(int e) { return u2f((uint32_t)(e + 127) << 23); }

// Nearest integer in [-7, 7], ties to even.
__device__ __forceinline__ float int4_round(float x) {
  return __builtin_amdgcn_fmed3f(__builtin_rintf(x), -7.0f, 7.0f);
}
// Nearest integer in [-127, 127], ties to even.
__device__ __forceinline__ float int8_round(float x) {
  return __builtin_amdgcn_fmed3f(__builtin_rintf(x), -127.0f, 127.0f);
}

// ---------------------------------------------------------------- scale projections
// Nearest admissible dual scale to x > 0 (conference entry: scales are projected onto the
// format's admissible set after each update; the nearest point is the exact minimiser of
// the 1-D quadratic each closed-form step solves).  NVFP4: E4M3 values.  INT and MX
// formats: bf16 values -- a power-of-two row scale would be absorbed exactly by the MX
// blocks' E8M0 exponents, so the MX dual scales live in bf16 like INT4's (the pages store
// their per-group scales in bf16); E8M0 is the block scale's set, inside the quantiser.
__device__ __forceinline__ float proj_e4m3(float x) {   // E4M3FN values in [2^-9, 448]
  uint32_t c = e4m3_code_sat(x);
  return e4m3_value(c ? c : 1u);
}
__device__ __forceinline__ float proj_bf16(float x) {   // bf16 values in [2^-126, max bf16]
  const float hi = u2f(0x7F7F0000u);
  float b = bf16_rne(fminf(x, hi));
  return fmaxf(u2f(0x00800000u), fminf(hi, b));
}
template <int FMT>
__device__ __forceinline__ float project(float x) {
  if (FMT == NVFP4) return proj_e4m3(x);
  return proj_bf16(x);   // INT4, INT8 and every MX format
}

// Wait for this wave's LDS writes, then a bare workgroup barrier.  Global loads issued
// earlier (later pipeline stages, the next row) stay in flight -- the fence of
// __syncthreads would wait for them too; the memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0), vmcnt and expcnt free
  asm volatile("s_barrier" ::: "memory");
}

// ---------------------------------------------------------------- cross-lane helpers
// Max over the L consecutive lanes that share a block (L in {1,2,4,8}).
template <int L>
__device__ __forceinline__ float block_max(float a) {
  if (L >= 2) a = fmaxf(a, __shfl_xor(a, 1));
  if (L >= 4) a = fmaxf(a, __shfl_xor(a, 2));
  if (L >= 8) a = fmaxf(a, __shfl_xor(a, 4));
  return a;
}

__device__ __forceinline__ double wave_sum(double x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// ---------------------------------------------------------------- format traits
template <int FMT> struct Traits;
template <> struct Traits<INT4> { static constexpr int DEF_G = 128; static constexpr int SCALE_BYTES = 2; };
template <> struct Traits<MXINT4> { static constexpr int DEF_G = 32; static constexpr int SCALE_BYTES = 1; };
template <> struct Traits<MXFP4> { static constexpr int DEF_G = 32; static constexpr int SCALE_BYTES = 1; };
template <> struct Traits<NVFP4> { static constexpr int DEF_G = 16; static constexpr int SCALE_BYTES = 1; };
template <> struct Traits<INT8> { static constexpr int DEF_G = 128; static constexpr int SCALE_BYTES = 2; };
template <> struct Traits<MXINT8> { static constexpr int DEF_G = 32; static constexpr int SCALE_BYTES = 1; };
template <> struct Traits<MXFP8_E4M3> { static constexpr int DEF_G = 32; static constexpr int SCALE_BYTES = 1; };
template <> struct Traits<MXFP8_E5M2> { static constexpr int DEF_G = 32; static constexpr int SCALE_BYTES = 1; };
template <> struct Traits<MXFP6_E2M3> { static constexpr int DEF_G = 32; static constexpr int SCALE_BYTES = 1; };
template <> struct Traits<MXFP6_E3M2> { static constexpr int DEF_G = 32; static constexpr int SCALE_BYTES = 1; };
// 32-bit words of element codes per 16-element chunk: 4-bit codes pack into 2, 6-bit into
// 3 (a bit stream), 8-bit into 4.
template <int FMT>
constexpr int code_words() {
  return (FMT == INT8 || FMT == MXINT8 || FMT == MXFP8_E4M3 || FMT == MXFP8_E5M2) ? 4
         : mx_fp6<FMT>()                                                          ? 3
                                                                                  : 2;
}
template <int FMT>
constexpr bool grouped_int() { return FMT == INT4 || FMT == INT8; }

// NVFP4 per-sweep tables: for every E4M3 code, d = fl(e4m3(code) * s_t) and id = fl(1/d).
struct NvTab {
  float d[128];
  float id[128];
};

// Everything a lane needs to quantise its chunk: the NVFP4 tensor-scale terms and table.
struct QCtx {
  float k6;        // NVFP4: fl(1 / fl(6 s_t)); 0 means "tensor scale zero: all blocks zero"
  const NvTab* tab;
};

// Result of quantising one chunk (16 elements): Qhat_k = p[k] * f, where p is the
// element-grid value (E2M1 value or integer) and f the block's dequantisation factor
// (NVFP4 d = e4m3(sb) * s_t, MXFP4 2^e, MXINT4 2^(e-2), MXINT8 2^(e-6), INT4/INT8 s).
struct Chunk {
  uint32_t code[4];   // 4-bit formats: 16 nibbles, element k in bits 4k..4k+3 of words 0-1;
                      // 6-bit formats: element k in bits 6k..6k+5 of words 0-2;
                      // 8-bit formats: 16 bytes, element k in byte k of words 0-3
  uint32_t scode;     // block scale code (bf16 bits, E8M0 byte or E4M3 byte)
  float f;            // block factor
  float p[16];        // grid values
  bool underflow;     // NVFP4: non-zero block whose scale rounded to zero
};

// E2M1 codes of x[0..15] (scale operand `sc` divides by a power of two) and their values.
__device__ __forceinline__ void fp4_encode16(const float (&x)[16], float sc, uint32_t& c0,
                                             uint32_t& c1) {
  c0 = 0u;
  c1 = 0u;
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, x[0], x[1], sc, 0);
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, x[2], x[3], sc, 1);
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, x[4], x[5], sc, 2);
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, x[6], x[7], sc, 3);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, x[8], x[9], sc, 0);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, x[10], x[11], sc, 1);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, x[12], x[13], sc, 2);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, x[14], x[15], sc, 3);
}
__device__ __forceinline__ void fp4_decode16(uint32_t c0, uint32_t c1, float (&p)[16]) {
  f32x2 t[8];
  t[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, 1.0f, 0);
  t[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, 1.0f, 1);
  t[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, 1.0f, 2);
  t[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, 1.0f, 3);
  t[4] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, 1.0f, 0);
  t[5] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, 1.0f, 1);
  t[6] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, 1.0f, 2);
  t[7] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, 1.0f, 3);
#pragma unroll
  for (int k = 0; k < 8; ++k) { p[2 * k] = t[k].x; p[2 * k + 1] = t[k].y; }
}
__device__ __forceinline__ void int4_decode16(uint32_t c0, uint32_t c1, float (&p)[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    uint32_t w = (k < 8) ? c0 : c1;
    p[k] = (float)(((int)(w << (28 - 4 * (k & 7)))) >> 28);   // sign-extended nibble
  }
}
__device__ __forceinline__ void int8_decode16(const uint32_t (&c)[4], float (&p)[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k)
    p[k] = (float)(((int)(c[k >> 2] << (24 - 8 * (k & 3)))) >> 24);   // sign-extended byte
}

// FP8 codes of x[0..15] (already within the type's finite range) and their values, with
// the hardware conversions (round to nearest even; OCP E4M3FN / E5M2 encodings).
template <int FMT>
__device__ __forceinline__ void fp8_encode16(const float (&x)[16], uint32_t (&c)[4], float (&p)[16]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t u = 0u;
    if (FMT == MXFP8_E4M3) {
      u = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w], x[4 * w + 1], u, false);
      u = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2], x[4 * w + 3], u, true);
    } else {
      u = __builtin_amdgcn_cvt_pk_bf8_f32(x[4 * w], x[4 * w + 1], u, false);
      u = __builtin_amdgcn_cvt_pk_bf8_f32(x[4 * w + 2], x[4 * w + 3], u, true);
    }
    c[w] = u;
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f32x2 lo, hi;
    if (FMT == MXFP8_E4M3) {
      lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[w], false);
      hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[w], true);
    } else {
      lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)c[w], false);
      hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)c[w], true);
    }
    p[4 * w] = lo.x; p[4 * w + 1] = lo.y; p[4 * w + 2] = hi.x; p[4 * w + 3] = hi.y;
  }
}
template <int FMT>
__device__ __forceinline__ void fp8_decode16(const uint32_t (&c)[4], float (&p)[16]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f32x2 lo, hi;
    if (FMT == MXFP8_E4M3) {
      lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[w], false);
      hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[w], true);
    } else {
      lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)c[w], false);
      hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)c[w], true);
    }
    p[4 * w] = lo.x; p[4 * w + 1] = lo.y; p[4 * w + 2] = hi.x; p[4 * w + 3] = hi.y;
  }
}

// FP6 codes of x[0..15] and their values with the hardware conversions.  The 2xpk16
// conversion writes its 32 results interleaved (field 2i from the first source's element i,
// field 2i+1 from the second's), so even elements go to the first source and odd elements
// to the second: the first three words then hold the chunk's codes in stream order.  The
// conversion rounds to nearest even (E2M3: bias 1, 3 mantissa bits; E3M2: bias 3, 2
// mantissa bits; subnormals below 2^(1-bias)), saturates at 7.5 / 28 and keeps the sign of
// a negative value that rounds to zero; this was checked element by element against a
// bit-level implementation of that rounding on every midpoint of both grids.
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
template <int FMT>
__device__ __forceinline__ void fp6_encode16_hw(const float (&x)[16], uint32_t (&c)[4], float (&p)[16]) {
  f32x16 a = {}, b = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) { a[i] = x[2 * i]; b[i] = x[2 * i + 1]; }
  u32x6 w = (FMT == MXFP6_E2M3) ? __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f)
                                : __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, 1.0f);
  c[0] = w[0]; c[1] = w[1]; c[2] = w[2]; c[3] = 0u;
  const u32x6 z = u32x6{w[0], w[1], w[2], 0u, 0u, 0u};
  const f32x32 d = (FMT == MXFP6_E2M3) ? __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(z, 1.0f)
                                       : __builtin_amdgcn_cvt_scalef32_pk32_f32_bf6(z, 1.0f);
#pragma unroll
  for (int k = 0; k < 16; ++k) p[k] = d[k];
}
template <int FMT>
__device__ __forceinline__ void fp6_decode16_hw(const uint32_t (&c)[4], float (&p)[16]) {
  const u32x6 z = u32x6{c[0], c[1], c[2], 0u, 0u, 0u};
  const f32x32 d = (FMT == MXFP6_E2M3) ? __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(z, 1.0f)
                                       : __builtin_amdgcn_cvt_scalef32_pk32_f32_bf6(z, 1.0f);
#pragma unroll
  for (int k = 0; k < 16; ++k) p[k] = d[k];
}

// Quantise one lane's 16 normalised values v (one chunk of a block of L*16).
template <int FMT, int L>
__device__ __forceinline__ void quantize_chunk(const float (&v)[16], const QCtx& ctx, Chunk& o) {
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) a = fmaxf(a, fabsf(v[k]));
  a = block_max<L>(a);
  o.underflow = false;
  if (FMT == NVFP4) {
    const uint32_t sbc = (ctx.k6 > 0.0f) ? e4m3_code_sat(a * ctx.k6) : 0u;
    o.scode = sbc;
    o.underflow = (sbc == 0u) && (a > 0.0f);
    const float id = ctx.tab->id[sbc];   // entry 0 holds 0
    o.f = ctx.tab->d[sbc];
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = v[k] * id;
    uint32_t c0, c1;
    fp4_encode16(x, 1.0f, c0, c1);
    if (sbc == 0u) { c0 = 0u; c1 = 0u; }
    o.code[0] = c0;
    o.code[1] = c1;
    fp4_decode16(c0, c1, o.p);
  } else if (FMT == MXFP4) {
    int e = (a > 0.0f) ? floor_log2(a) - 2 : -127;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    o.scode = (uint32_t)(e + 127);
    o.f = ldexpf(1.0f, e);
    uint32_t c0, c1;
    if (e >= -100) {        // the scale operand carries 2^e: the conversion divides exactly
      fp4_encode16(v, pow2_operand(e), c0, c1);
    } else {                // tiny blocks: scale by 2^-e first (exact), convert unscaled
      float x[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) x[k] = ldexpf(v[k], -e);
      fp4_encode16(x, 1.0f, c0, c1);
    }
    if (a == 0.0f) { c0 = 0u; c1 = 0u; }
    o.code[0] = c0;
    o.code[1] = c1;
    fp4_decode16(c0, c1, o.p);
  } else if (FMT == MXINT4) {
    int e = (a > 0.0f) ? floor_log2(a) : -127;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    o.scode = (uint32_t)(e + 127);
    o.f = ldexpf(1.0f, e - 2);
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float q = (a > 0.0f) ? int4_round(ldexpf(v[k], 2 - e)) : 0.0f;
      const uint32_t nib = (uint32_t)(int)q & 0xFu;
      if (k < 8) c0 |= nib << (4 * k); else c1 |= nib << (4 * (k - 8));
      o.p[k] = q;
    }
    o.code[0] = c0;
    o.code[1] = c1;
  } else if (mx_mini<FMT>()) {
    // OCP MX v1.0 FP8 / FP6 elements: shared exponent floor(log2 amax) - emax, elements
    // the nearest value of v * 2^-e (scaling by a power of two is exact), saturating
    int e = (a > 0.0f) ? floor_log2(a) - mini_emax<FMT>() : -127;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    o.scode = (uint32_t)(e + 127);
    o.f = ldexpf(1.0f, e);
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      x[k] = __builtin_amdgcn_fmed3f(ldexpf(v[k], -e), -mini_max<FMT>(), mini_max<FMT>());
    if (mx_fp6<FMT>()) {
      fp6_encode16_hw<FMT>(x, o.code, o.p);
    } else {
      fp8_encode16<FMT>(x, o.code, o.p);
    }
    if (a == 0.0f) {
#pragma unroll
      for (int w = 0; w < 4; ++w) o.code[w] = 0u;
#pragma unroll
      for (int k = 0; k < 16; ++k) o.p[k] = 0.0f;
    }
  } else if (FMT == MXINT8) {
    // OCP MX v1.0 MXINT8: elements q * 2^-6 with q in [-127, 127]; shared exponent
    // floor(log2 amax)
    int e = (a > 0.0f) ? floor_log2(a) : -127;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    o.scode = (uint32_t)(e + 127);
    o.f = ldexpf(1.0f, e - 6);
    uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float q = (a > 0.0f) ? int8_round(ldexpf(v[k], 6 - e)) : 0.0f;
      c[k >> 2] |= ((uint32_t)(int)q & 0xFFu) << (8 * (k & 3));
      o.p[k] = q;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) o.code[w] = c[w];
  } else if (FMT == INT8) {
    const float s = (a > 0.0f) ? bf16_rne(a / 127.0f) : 0.0f;
    o.scode = f2u(s) >> 16;
    o.f = s;
    const float is = (s > 0.0f) ? 1.0f / s : 0.0f;
    uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float q = (s > 0.0f) ? int8_round(v[k] * is) : 0.0f;
      c[k >> 2] |= ((uint32_t)(int)q & 0xFFu) << (8 * (k & 3));
      o.p[k] = q;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) o.code[w] = c[w];
  } else {  // INT4
    const float s = (a > 0.0f) ? bf16_rne(a / 7.0f) : 0.0f;
    o.scode = f2u(s) >> 16;
    o.f = s;
    const float is = (s > 0.0f) ? 1.0f / s : 0.0f;
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float q = (s > 0.0f) ? int4_round(v[k] * is) : 0.0f;
      const uint32_t nib = (uint32_t)(int)q & 0xFu;
      if (k < 8) c0 |= nib << (4 * k); else c1 |= nib << (4 * (k - 8));
      o.p[k] = q;
    }
    o.code[0] = c0;
    o.code[1] = c1;
  }
}

// Block factor of a stored scale code (NVFP4 uses the table of the tensor scale the codes
// were made with).
template <int FMT>
__device__ __forceinline__ float block_factor(uint32_t scode, const NvTab* tab) {
  if (FMT == NVFP4) return tab->d[scode & 127u];
  if (FMT == MXFP4) return ldexpf(1.0f, (int)scode - 127);
  if (FMT == MXINT4) return ldexpf(1.0f, (int)scode - 129);
  if (FMT == MXINT8) return ldexpf(1.0f, (int)scode - 133);
  if (mx_mini<FMT>()) return ldexpf(1.0f, (int)scode - 127);
  return u2f(scode << 16);   // INT4, INT8: bf16 scale
}

// Grid values of a stored chunk (code words as stored: 2 for 4-bit, 3 for 6-bit, 4 for 8-bit
// formats).
template <int FMT>
__device__ __forceinline__ void decode_grid(const uint32_t (&c)[4], float (&p)[16]) {
  if (FMT == NVFP4 || FMT == MXFP4) fp4_decode16(c[0], c[1], p);
  else if (FMT == INT8 || FMT == MXINT8) int8_decode16(c, p);
  else if (FMT == MXFP8_E4M3 || FMT == MXFP8_E5M2) fp8_decode16<FMT>(c, p);
  else if (mx_fp6<FMT>()) fp6_decode16_hw<FMT>(c, p);
  else int4_decode16(c[0], c[1], p);
}

}  // namespace dqk
