// DualQuant dual-scale BCD solver: plain, slow CPU oracle.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this
// file; only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
// shares no code, header, table or constant with the GPU library.
//
// What it computes (DualQuant, "Dual-scale Calibration-free Weight-and-Activation
// Quantization for LLMs"; the listing page's abstract, the conference entry's longer
// abstract, and the news summary's mechanism paragraph):
//   minimise  || W - diag(r) . Qhat . diag(c) ||_F^2
// over a row-scale vector r, a column-scale vector c (the activation rescaling beta)
// and the block fake-quantised matrix Qhat = FQ_f(W ./ (r c^T)), by block coordinate
// descent whose subproblems have closed forms, projecting each scale update onto the
// format's admissible set.  The pages print no equation; every reading taken where
// they are silent is restated next to the code that implements it.
//
// Style: brute-force nearest-grid rounding with explicit tie rules, fp64 accumulation,
// fixed summation order (results do not depend on the thread count).  The quantiser's
// own decisions are taken in fp32, the precision the block formats are defined in.
// Build with -ffp-contract=off and without fast-math.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

enum Fmt { FMT_INT4 = 0, FMT_MXINT4 = 1, FMT_MXFP4 = 2, FMT_NVFP4 = 3, FMT_INT8 = 4, FMT_MXINT8 = 5,
           FMT_MXFP8_E4M3 = 6, FMT_MXFP8_E5M2 = 7, FMT_MXFP6_E2M3 = 8, FMT_MXFP6_E3M2 = 9 };

bool is_mx_minifloat(int fmt) { return fmt >= FMT_MXFP8_E4M3 && fmt <= FMT_MXFP6_E3M2; }
// Element code width: 4 bits (two per byte), 6 bits (a packed bit stream) or 8 bits (one
// per byte).
int code_bits(int fmt) {
  if (fmt == FMT_INT8 || fmt == FMT_MXINT8 || fmt == FMT_MXFP8_E4M3 || fmt == FMT_MXFP8_E5M2) return 8;
  if (fmt == FMT_MXFP6_E2M3 || fmt == FMT_MXFP6_E3M2) return 6;
  return 4;
}
bool is_mx(int fmt) {
  return fmt == FMT_MXINT4 || fmt == FMT_MXFP4 || fmt == FMT_MXINT8 || is_mx_minifloat(fmt);
}
bool is_int_grouped(int fmt) { return fmt == FMT_INT4 || fmt == FMT_INT8; }
enum Dtype { DT_F32 = 0, DT_BF16 = 1 };
enum Status { OK = 0, ERR_NULL = -1, ERR_SHAPE = -2, ERR_FORMAT = -4, ERR_VALUE = -8 };

// ---------------------------------------------------------------- bit helpers
float f_of(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
uint32_t u_of(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
float bf16_to_f32(uint16_t h) { return f_of((uint32_t)h << 16); }

// ---------------------------------------------------------------- threading
int g_threads = 1;

template <class F>
void parallel_rows(int64_t n, F fn) {
  int nt = std::max(1, std::min<int>(g_threads, (int)std::max<int64_t>(1, n)));
  if (nt == 1) { fn((int64_t)0, n); return; }
  std::vector<std::thread> th;
  int64_t chunk = (n + nt - 1) / nt;
  for (int t = 0; t < nt; ++t) {
    int64_t b = t * chunk, e = std::min(n, b + chunk);
    if (b >= e) break;
    th.emplace_back([=] { fn(b, e); });
  }
  for (auto& x : th) x.join();
}

// ---------------------------------------------------------------- element grids
// E2M1 (OCP MX v1.0 FP4): 1 sign, 2 exponent, 1 mantissa bit.  The magnitude code k
// (0..7) encodes these values; the mantissa bit is k & 1.
const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

// Nearest E2M1 magnitude, ties to the even mantissa bit; anything beyond 6 saturates to
// 6 (the nearest finite point).  The sign bit is kept, so a negative input that rounds
// to zero encodes as 0b1000.
uint8_t e2m1_encode(float x) {
  // Above 7 the nearest grid point is 6 whatever the value; clamping there keeps the
  // distances below exact in fp64 for huge inputs.
  double ax = std::min(std::fabs((double)x), 7.0);
  int best = 0;
  double bestd = ax;
  for (int k = 1; k < 8; ++k) {
    double d = std::fabs(ax - kE2M1[k]);
    if (d < bestd || (d == bestd && (k % 2) == 0)) { best = k; bestd = d; }
  }
  return (uint8_t)((std::signbit(x) ? 8 : 0) | best);
}
double e2m1_decode(uint8_t code) {
  double m = kE2M1[code & 7];
  return (code & 8) ? -m : m;
}

// E4M3FN (OCP FP8): bias 7, no infinities, 0x7F is NaN; largest finite value 448.
double e4m3_value(int code) {
  int e = (code >> 3) & 15, m = code & 7;
  if (e == 0) return std::ldexp((double)m, -9);
  return std::ldexp(1.0 + m / 8.0, e - 7);
}
// Nearest non-negative E4M3FN value (codes 0..126) to x >= 0, ties to the even code;
// values beyond 448 saturate to 448.
int e4m3_encode_nonneg(float x, int lowest_code) {
  double ax = std::min((double)x, 480.0);  // beyond 480 the nearest value is 448 anyway
  int best = lowest_code;
  double bestd = std::fabs(ax - e4m3_value(lowest_code));
  for (int k = lowest_code + 1; k <= 126; ++k) {
    double d = std::fabs(ax - e4m3_value(k));
    if (d < bestd || (d == bestd && (k % 2) == 0)) { best = k; bestd = d; }
  }
  return best;
}

// The OCP MX v1.0 FP8 and FP6 element types: sign, ebits exponent bits with the given
// bias, mbits mantissa bits, subnormals when the exponent field is 0.  E4M3 keeps only
// the all-ones code as NaN (largest finite 448); E5M2 reserves the all-ones exponent for
// infinities and NaN (largest finite 57344); the FP6 types have no special codes (E2M3
// largest 7.5, E3M2 largest 28).  emax is the exponent of the largest binade, the offset
// the MX shared scale removes.
struct Minifloat {
  int ebits, mbits, bias, emax;
};
Minifloat minifloat_of(int fmt) {
  switch (fmt) {
    case FMT_MXFP8_E4M3: return {4, 3, 7, 8};
    case FMT_MXFP8_E5M2: return {5, 2, 15, 15};
    case FMT_MXFP6_E2M3: return {2, 3, 1, 2};
    default: return {3, 2, 3, 4};   // FMT_MXFP6_E3M2
  }
}
// Whether a magnitude code is a finite number.
bool mini_finite(int fmt, int mag) {
  const Minifloat m = minifloat_of(fmt);
  if (fmt == FMT_MXFP8_E4M3) return mag != 0x7F;
  if (fmt == FMT_MXFP8_E5M2) return (mag >> m.mbits) != (1 << m.ebits) - 1;
  return true;
}
// Value of a finite magnitude code, from the definition.
double mini_value(int fmt, int mag) {
  const Minifloat m = minifloat_of(fmt);
  const int e = mag >> m.mbits, f = mag & ((1 << m.mbits) - 1);
  if (e == 0) return std::ldexp((double)f, 1 - m.bias - m.mbits);
  return std::ldexp(1.0 + std::ldexp((double)f, -m.mbits), e - m.bias);
}
int mini_mag_codes(int fmt) {
  const Minifloat m = minifloat_of(fmt);
  return 1 << (m.ebits + m.mbits);
}
double mini_max(int fmt) {
  double best = 0.0;
  for (int k = 0; k < mini_mag_codes(fmt); ++k)
    if (mini_finite(fmt, k)) best = std::max(best, mini_value(fmt, k));
  return best;
}
// Nearest finite value of the type to x, ties to the even code (the code's low bit is the
// mantissa's low bit); magnitudes beyond the largest finite value saturate to it (the
// reading taken for every MX element type, as for E2M1).  The sign bit is kept, so a
// negative input that rounds to zero encodes as negative zero.
int mini_encode(int fmt, float x) {
  const double mx = mini_max(fmt);
  const double ax = std::min(std::fabs((double)x), 2.0 * mx);
  int best = 0;
  double bestd = ax;
  for (int k = 1; k < mini_mag_codes(fmt); ++k) {
    if (!mini_finite(fmt, k)) continue;
    const double d = std::fabs(ax - mini_value(fmt, k));
    if (d < bestd || (d == bestd && (k % 2) == 0)) { best = k; bestd = d; }
  }
  const Minifloat m = minifloat_of(fmt);
  return (std::signbit(x) ? (1 << (m.ebits + m.mbits)) : 0) | best;
}
double mini_decode(int fmt, int code) {
  const Minifloat m = minifloat_of(fmt);
  const int mag = code & ((1 << (m.ebits + m.mbits)) - 1);
  const double v = mini_value(fmt, mag);
  return (code >> (m.ebits + m.mbits)) & 1 ? -v : v;
}

// Nearest bfloat16 to a finite fp32 x, ties to even: the two candidates are x with its
// low 16 bits cleared and the next bf16 further from zero.
float bf16_round(float x) {
  uint32_t u = u_of(x);
  float lo = f_of(u & 0xFFFF0000u);
  float hi = f_of((u & 0xFFFF0000u) + 0x10000u);
  double dlo = std::fabs((double)x - (double)lo);
  double dhi = std::fabs((double)hi - (double)x);
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return ((u >> 16) & 1u) ? hi : lo;
}

// Nearest integer in [-qmax, qmax] to x, ties to even.
int int_round_clamp(float x, int qmax) {
  double ax = std::max(-(double)qmax - 1.0, std::min((double)x, (double)qmax + 1.0));
  int best = -qmax;
  double bestd = std::fabs(ax + qmax);
  for (int k = -qmax + 1; k <= qmax; ++k) {
    double d = std::fabs(ax - k);
    if (d < bestd || (d == bestd && (k % 2) == 0)) { best = k; bestd = d; }
  }
  return best;
}

// floor(log2 a) for a finite a > 0 (exact, from frexp).
int floor_log2(float a) {
  int k;
  std::frexp((double)a, &k);
  return k - 1;
}

// ---------------------------------------------------------------- scale projections
// After each closed-form update, the scale is projected onto the format's admissible
// set (the conference abstract: "projecting scales onto their format-specific admissible
// set after each update").  For a 1-D quadratic D (s - x)^2 the constrained minimiser is
// the admissible point nearest to x, so "projection" is the nearest point.
//   NVFP4:              positive E4M3FN values [2^-9, 448]; ties to the even code.
//   INT, MX formats:    positive bf16 values [2^-126, max bf16]; ties to even.
// The MX block scale itself stays an E8M0 power of two inside the quantiser.  The dual
// scales are not: a power-of-two row scale would be absorbed exactly by every block's E8M0
// exponent (same codes, same reconstruction), so the dual scales would change nothing for
// MX, against the conference abstract's "formally support MX" and the news summary's
// ablation in which row scales alone already help.  They multiply outside the block format
// (r on the layer output, c on the activations before their quantiser), in the bf16 the
// pages store their per-group weight scales in (listing page, Table 12).
float project(int fmt, float x) {
  if (fmt == FMT_NVFP4) return (float)e4m3_value(e4m3_encode_nonneg(x, 1));
  const float lo = std::ldexp(1.0f, -126);
  const float hi = f_of(0x7F7F0000u);
  float b = bf16_round(std::min(x, hi));
  return std::max(lo, std::min(hi, b));
}

// ---------------------------------------------------------------- block quantisers
// FQ_f on a normalised row-major matrix V (rows x cols); blocks of g consecutive
// elements along a row.  Outputs: packed codes (4-bit formats: two per byte, low nibble =
// even column; 8-bit formats: one byte per element), block scales (bf16 for INT4/INT8,
// E8M0 byte for MX, E4M3 byte for NVFP4), the NVFP4 fp32 tensor scale, and Qhat (the
// dequantised values, fp32).
struct FQOut {
  uint8_t* codes;      // rows * cols * bits / 8
  void* scales;        // rows * cols / g
  float* tscale;       // 1 (NVFP4)
  float* qhat;         // rows * cols (may be null)
  uint32_t flags;
};

void put_code(uint8_t* codes, int64_t idx, uint8_t nib) {
  uint8_t& b = codes[idx >> 1];
  if (idx & 1) b = (uint8_t)((b & 0x0F) | (nib << 4));
  else b = (uint8_t)((b & 0xF0) | (nib & 0x0F));
}

// 6-bit codes: element idx occupies bits 6*idx .. 6*idx+5 of the little-endian bit
// stream of the code buffer (four elements in three bytes).
void put_code6(uint8_t* codes, int64_t idx, int code) {
  for (int b = 0; b < 6; ++b) {
    const int64_t bit = 6 * idx + b;
    uint8_t& byte = codes[bit >> 3];
    const uint8_t mask = (uint8_t)(1u << (bit & 7));
    byte = (uint8_t)(((code >> b) & 1) ? (byte | mask) : (byte & ~mask));
  }
}
int get_code6(const uint8_t* codes, int64_t idx) {
  int code = 0;
  for (int b = 0; b < 6; ++b) {
    const int64_t bit = 6 * idx + b;
    code |= ((codes[bit >> 3] >> (bit & 7)) & 1) << b;
  }
  return code;
}

// Code of element idx at the format's width (two's complement for the integer formats).
void put_code_w(int bits, uint8_t* codes, int64_t idx, int q) {
  if (bits == 8) codes[idx] = (uint8_t)(q & 0xFF);
  else if (bits == 6) put_code6(codes, idx, q & 0x3F);
  else put_code(codes, idx, (uint8_t)(q & 0xF));
}

// Grouped symmetric integers (INT4: qmax 7; INT8: qmax 127): s = bf16(a / qmax),
// codes = clamp(rint(v * (1/s)), -qmax, qmax), Qhat = q * s.  An all-zero block stores
// scale 0.
void fq_int_row(int fmt, const float* v, int64_t row, int64_t cols, int g, FQOut& o) {
  const int qmax = (fmt == FMT_INT8) ? 127 : 7;
  const int bits = code_bits(fmt);
  uint16_t* sc = (uint16_t*)o.scales;
  for (int64_t b = 0; b < cols / g; ++b) {
    const float* x = v + b * g;
    float a = 0.0f;
    for (int k = 0; k < g; ++k) a = std::max(a, std::fabs(x[k]));
    float s = (a > 0.0f) ? bf16_round(a / (float)qmax) : 0.0f;
    sc[row * (cols / g) + b] = (uint16_t)(u_of(s) >> 16);
    float is = (s > 0.0f) ? 1.0f / s : 0.0f;
    for (int k = 0; k < g; ++k) {
      int q = (s > 0.0f) ? int_round_clamp(x[k] * is, qmax) : 0;
      int64_t idx = row * cols + b * g + k;
      put_code_w(bits, o.codes, idx, q);
      if (o.qhat) o.qhat[idx] = (float)q * s;
    }
  }
}

// MXINT4 (by analogy with OCP MXINT8): shared exponent e = floor(log2 amax), elements
// are 4-bit two's-complement integers with an implicit 2^-2, clamped symmetrically to
// [-7, 7]: q = clamp(rint(v * 2^(2-e)), -7, 7), Qhat = q * 2^(e-2).  Scale byte e+127.
// MXINT8 (OCP MX v1.0): 8-bit two's-complement elements with an implicit 2^-6, largest
// magnitude below 2 so the shared exponent is e = floor(log2 amax):
// q = clamp(rint(v * 2^(6-e)), -127, 127), Qhat = q * 2^(e-6).
// MXFP4 (OCP MX v1.0): e = floor(log2 amax) - 2, q = E2M1(v * 2^-e), Qhat = q * 2^e.
// MXFP8 (E4M3, E5M2) and MXFP6 (E2M3, E3M2), OCP MX v1.0: e = floor(log2 amax) - emax of
// the element type, q = nearest element value to v * 2^-e (saturating), Qhat = q * 2^e.
// Exponents clamp to [-127, 127]; an all-zero block stores scale byte 0 and codes 0.
void fq_mx_row(int fmt, const float* v, int64_t row, int64_t cols, int g, FQOut& o) {
  uint8_t* sc = (uint8_t*)o.scales;
  const int bits = code_bits(fmt);
  int off = 0;
  if (fmt == FMT_MXFP4) off = 2;
  if (is_mx_minifloat(fmt)) off = minifloat_of(fmt).emax;
  for (int64_t b = 0; b < cols / g; ++b) {
    const float* x = v + b * g;
    float a = 0.0f;
    for (int k = 0; k < g; ++k) a = std::max(a, std::fabs(x[k]));
    int e = -127;
    if (a > 0.0f) e = std::max(-127, std::min(127, floor_log2(a) - off));
    if (is_mx_minifloat(fmt)) {
      sc[row * (cols / g) + b] = (uint8_t)(e + 127);
      for (int k = 0; k < g; ++k) {
        const int64_t idx = row * cols + b * g + k;
        int code = 0;
        float qh = 0.0f;
        if (a > 0.0f) {
          code = mini_encode(fmt, std::ldexp(x[k], -e));
          qh = std::ldexp((float)mini_decode(fmt, code), e);
        }
        put_code_w(bits, o.codes, idx, code);
        if (o.qhat) o.qhat[idx] = qh;
      }
      continue;
    }
    sc[row * (cols / g) + b] = (uint8_t)(e + 127);
    for (int k = 0; k < g; ++k) {
      int64_t idx = row * cols + b * g + k;
      uint8_t nib = 0;
      float qh = 0.0f;
      if (a > 0.0f) {
        if (fmt == FMT_MXFP4) {
          nib = e2m1_encode(std::ldexp(x[k], -e));
          qh = std::ldexp((float)e2m1_decode(nib), e);
        } else if (fmt == FMT_MXINT8) {
          int q = int_round_clamp(std::ldexp(x[k], 6 - e), 127);
          nib = (uint8_t)(q & 0xFF);
          qh = std::ldexp((float)q, e - 6);
        } else {
          int q = int_round_clamp(std::ldexp(x[k], 2 - e), 7);
          nib = (uint8_t)(q & 0xF);
          qh = std::ldexp((float)q, e - 2);
        }
      }
      if (fmt == FMT_MXINT8) o.codes[idx] = nib;
      else put_code(o.codes, idx, nib);
      if (o.qhat) o.qhat[idx] = qh;
    }
  }
}

// NVFP4 (NVIDIA's public two-level scheme): A = max|V| over the matrix,
// s_t = A / 2688 (2688 = 6 * 448), k6 = 1 / (6 s_t); per 16-element block
// sb = E4M3(a * k6) (saturating), d = sb * s_t, q = E2M1(v * (1/d)), Qhat = q * d.
// A block whose scale rounds to zero is all zero (flag bit 8).
void fq_nvfp4_row(const float* v, int64_t row, int64_t cols, float s_t, float k6, FQOut& o,
                  uint32_t* flags) {
  uint8_t* sc = (uint8_t*)o.scales;
  const int g = 16;
  for (int64_t b = 0; b < cols / g; ++b) {
    const float* x = v + b * g;
    float a = 0.0f;
    for (int k = 0; k < g; ++k) a = std::max(a, std::fabs(x[k]));
    int sbc = (s_t > 0.0f) ? e4m3_encode_nonneg(a * k6, 0) : 0;
    if (sbc == 0 && a > 0.0f) *flags |= 8u;
    sc[row * (cols / g) + b] = (uint8_t)sbc;
    float d = (float)e4m3_value(sbc) * s_t;
    float id = (sbc > 0) ? 1.0f / d : 0.0f;
    for (int k = 0; k < g; ++k) {
      int64_t idx = row * cols + b * g + k;
      uint8_t nib = 0;
      float qh = 0.0f;
      if (sbc > 0) {
        nib = e2m1_encode(x[k] * id);
        qh = (float)e2m1_decode(nib) * d;
      }
      put_code(o.codes, idx, nib);
      if (o.qhat) o.qhat[idx] = qh;
    }
  }
}

int group_ok(int fmt, int g) {
  if (is_int_grouped(fmt)) return g == 64 || g == 128;
  if (is_mx(fmt)) return g == 32;
  if (fmt == FMT_NVFP4) return g == 16;
  return 0;
}

// FQ over a normalised matrix; returns the NVFP4 tensor scale through o.tscale.
void fq_matrix(int fmt, int g, const float* V, int64_t rows, int64_t cols, FQOut& o) {
  float s_t = 0.0f, k6 = 0.0f;
  if (fmt == FMT_NVFP4) {
    float A = 0.0f;
    for (int64_t i = 0; i < rows * cols; ++i) A = std::max(A, std::fabs(V[i]));
    s_t = A / 2688.0f;
    float six_st = 6.0f * s_t;
    k6 = (s_t > 0.0f) ? 1.0f / six_st : 0.0f;
    // The scheme divides twice: by 6 s_t for the block scales, and by each block factor
    // d = e4m3(sb) s_t for the elements.  Both reciprocals must be finite fp32 numbers for
    // every block scale that can occur, the smallest being 2^-9 (the least E4M3 subnormal).
    // When A is so small that 1 / fl(2^-9 s_t) overflows (s_t at or below about 2^-119) or
    // s_t underflows to 0, no block of the matrix can be encoded: it quantises to zero and
    // flag bit 16 says so.
    const float id_min = (s_t > 0.0f) ? 1.0f / ((float)e4m3_value(1) * s_t) : 0.0f;
    if (!(s_t > 0.0f) || !std::isfinite(k6) || !std::isfinite(id_min)) {
      if (A > 0.0f) o.flags |= 16u;
      s_t = 0.0f;
      k6 = 0.0f;
    }
    if (o.tscale) *o.tscale = s_t;
  }
  std::vector<uint32_t> fl(std::max<int64_t>(rows, 1), 0u);
  parallel_rows(rows, [&](int64_t b, int64_t e) {
    for (int64_t i = b; i < e; ++i) {
      const float* v = V + i * cols;
      if (is_int_grouped(fmt)) fq_int_row(fmt, v, i, cols, g, o);
      else if (fmt == FMT_NVFP4) fq_nvfp4_row(v, i, cols, s_t, k6, o, &fl[i]);
      else fq_mx_row(fmt, v, i, cols, g, o);
    }
  });
  // 4-bit and 6-bit codes of neighbouring columns of one row share bytes, and rows never
  // share bytes (cols is a multiple of the group, hence of 16), so the row-parallel
  // writes are safe.
  for (auto f : fl) o.flags |= f;
}

// Normalisation used by every quantiser call: ir = 1/r, ic = 1/c (fp32, correctly
// rounded), v = (W * ir) * ic, two fp32 multiplies in that order.
void normalise(const float* W, int64_t rows, int64_t cols, const float* r, const float* c,
               float* V) {
  std::vector<float> ic(cols);
  for (int64_t j = 0; j < cols; ++j) ic[j] = 1.0f / c[j];
  parallel_rows(rows, [&](int64_t b, int64_t e) {
    for (int64_t i = b; i < e; ++i) {
      float ir = 1.0f / r[i];
      for (int64_t j = 0; j < cols; ++j) {
        float t = W[i * cols + j] * ir;
        V[i * cols + j] = t * ic[j];
      }
    }
  });
}

void load_w(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld, float* out) {
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < cols; ++j)
      out[i * cols + j] = (dtype == DT_F32) ? ((const float*)W)[i * ld + j]
                                            : bf16_to_f32(((const uint16_t*)W)[i * ld + j]);
}

bool all_finite(const float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!std::isfinite(x[i])) return false;
  return true;
}

// F(r, c, Q) = sum_ij (W_ij - r_i Q_ij c_j)^2 in fp64, rows summed in order.
double recon_error(const float* W, const float* Q, const float* r, const float* c,
                   int64_t rows, int64_t cols) {
  std::vector<double> rowF(rows, 0.0);
  parallel_rows(rows, [&](int64_t b, int64_t e) {
    for (int64_t i = b; i < e; ++i) {
      double s = 0.0;
      for (int64_t j = 0; j < cols; ++j) {
        double d = (double)W[i * cols + j] - (double)r[i] * (double)Q[i * cols + j] * (double)c[j];
        s += d * d;
      }
      rowF[i] = s;
    }
  });
  double F = 0.0;
  for (double x : rowF) F += x;
  return F;
}

}  // namespace

extern "C" {

void o_set_threads(int n) { g_threads = std::max(1, n); }
int o_get_threads() { return g_threads; }

// ---- scalar rounding, vectorised for tests
void o_e2m1_encode(const float* x, uint8_t* code, int64_t n) {
  for (int64_t i = 0; i < n; ++i) code[i] = e2m1_encode(x[i]);
}
void o_e2m1_decode(const uint8_t* code, float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = (float)e2m1_decode(code[i]);
}
// x >= 0 expected; returns codes 0..126
void o_e4m3_encode(const float* x, uint8_t* code, int64_t n) {
  for (int64_t i = 0; i < n; ++i) code[i] = (uint8_t)e4m3_encode_nonneg(x[i], 0);
}
void o_e4m3_decode(const uint8_t* code, float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = (float)e4m3_value(code[i] & 0x7F);
}
// MX FP8 / FP6 element codes (sign bit above the magnitude bits) and their values.
int o_mini_encode(int fmt, const float* x, uint8_t* code, int64_t n) {
  if (!is_mx_minifloat(fmt)) return ERR_FORMAT;
  for (int64_t i = 0; i < n; ++i) code[i] = (uint8_t)mini_encode(fmt, x[i]);
  return OK;
}
int o_mini_decode(int fmt, const uint8_t* code, float* x, int64_t n) {
  if (!is_mx_minifloat(fmt)) return ERR_FORMAT;
  const Minifloat m = minifloat_of(fmt);
  const int mask = (1 << (m.ebits + m.mbits + 1)) - 1;
  for (int64_t i = 0; i < n; ++i) {
    const int c = code[i] & mask;
    x[i] = mini_finite(fmt, c & (mask >> 1)) ? (float)mini_decode(fmt, c) : std::nanf("");
  }
  return OK;
}

void o_bf16_round(const float* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = bf16_round(x[i]);
}
void o_int_round(const float* x, int8_t* q, int64_t n, int qmax) {
  for (int64_t i = 0; i < n; ++i) q[i] = (int8_t)int_round_clamp(x[i], qmax);
}
void o_project(int fmt, const float* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = project(fmt, x[i]);
}

// ---- FQ on an already-normalised matrix
int o_fq(int fmt, int g, const float* V, int64_t rows, int64_t cols, uint8_t* codes,
         void* scales, float* tscale, float* qhat, uint32_t* flags) {
  if (!V || !codes || !scales) return ERR_NULL;
  if (!group_ok(fmt, g)) return ERR_FORMAT;
  if (rows < 0 || cols < 0 || cols % g) return ERR_SHAPE;
  if (!all_finite(V, rows * cols)) return ERR_VALUE;
  FQOut o{codes, scales, tscale, qhat, 0u};
  if (fmt == FMT_NVFP4 && !tscale) return ERR_NULL;
  fq_matrix(fmt, g, V, rows, cols, o);
  if (flags) *flags = o.flags;
  return OK;
}

// ---- Qhat-step at given scales: FQ_f(W ./ (r c^T)).  r or c null means ones.
int o_quantize_weights(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       const float* r, const float* c, int fmt, int g, uint8_t* codes,
                       void* scales, float* tscale, float* qhat) {
  if (!W || !codes || !scales) return ERR_NULL;
  if (!group_ok(fmt, g)) return ERR_FORMAT;
  if (rows < 0 || cols < 0 || cols % g || ld < cols) return ERR_SHAPE;
  std::vector<float> Wf(rows * cols), V(rows * cols);
  load_w(W, dtype, rows, cols, ld, Wf.data());
  if (!all_finite(Wf.data(), rows * cols)) return ERR_VALUE;
  std::vector<float> rr(rows, 1.0f), cc(cols, 1.0f);
  if (r) std::copy(r, r + rows, rr.begin());
  if (c) std::copy(c, c + cols, cc.begin());
  normalise(Wf.data(), rows, cols, rr.data(), cc.data(), V.data());
  return o_fq(fmt, g, V.data(), rows, cols, codes, scales, tscale, qhat, nullptr);
}

// ---- dequantise codes + scales into Qhat values (fp32)
int o_dequantize(int fmt, int g, const uint8_t* codes, const void* scales, float tscale,
                 int64_t rows, int64_t cols, float* out) {
  if (!codes || !scales || !out) return ERR_NULL;
  if (!group_ok(fmt, g)) return ERR_FORMAT;
  if (cols % g) return ERR_SHAPE;
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < cols; ++j) {
      int64_t idx = i * cols + j;
      int64_t bi = i * (cols / g) + j / g;
      float v = 0.0f;
      if (is_mx_minifloat(fmt)) {
        const int code = code_bits(fmt) == 8 ? (int)codes[idx] : get_code6(codes, idx);
        const int e = (int)((const uint8_t*)scales)[bi] - 127;
        out[idx] = std::ldexp((float)mini_decode(fmt, code), e);
        continue;
      }
      if (code_bits(fmt) == 8) {
        const int q = (int)(int8_t)codes[idx];
        if (fmt == FMT_INT8) v = (float)q * bf16_to_f32(((const uint16_t*)scales)[bi]);
        else v = std::ldexp((float)q, (int)((const uint8_t*)scales)[bi] - 127 - 6);
        out[idx] = v;
        continue;
      }
      uint8_t nib = (codes[idx >> 1] >> ((idx & 1) * 4)) & 0xF;
      if (fmt == FMT_INT4) {
        float s = bf16_to_f32(((const uint16_t*)scales)[bi]);
        int q = (nib & 8) ? (int)nib - 16 : (int)nib;
        v = (float)q * s;
      } else if (fmt == FMT_MXINT4) {
        int e = (int)((const uint8_t*)scales)[bi] - 127;
        int q = (nib & 8) ? (int)nib - 16 : (int)nib;
        v = std::ldexp((float)q, e - 2);
      } else if (fmt == FMT_MXFP4) {
        int e = (int)((const uint8_t*)scales)[bi] - 127;
        v = std::ldexp((float)e2m1_decode(nib), e);
      } else {
        int sbc = ((const uint8_t*)scales)[bi];
        float d = (float)e4m3_value(sbc) * tscale;
        v = (sbc > 0) ? (float)e2m1_decode(nib) * d : 0.0f;
      }
      out[idx] = v;
    }
  return OK;
}

// ---- the BCD solve.
// Iteration order (a reading: the pages do not fix it): starting from r = c = 1 (or the
// given initial scales) and Q^0 = FQ(W ./ r c^T), each iteration t = 1..T does
//   r-step: for every row,    N = sum_j W_ij Q_ij c_j,  D = sum_j (Q_ij c_j)^2,
//           r_i <- Proj(fl32(N / D)) when D > 0 (else r_i is kept);
//   c-step: for every column, N = sum_i r_i W_ij Q_ij,  D = sum_i (r_i Q_ij)^2,
//           c_j <- Proj(fl32(N / D)) when D > 0, using the new r;
//   Q-step: candidate Qc = FQ(W ./ r c^T), kept only if it does not raise F at the
//           current scales (ties are kept); otherwise Q stays and the step counts as
//           rejected.  This safeguard makes the normalised MSE non-increasing, the
//           property the pages state as Theorem 1(i) (Fig. 2b, Fig. 3b).
//   stats:  nmse[t] = F(r, c, Q^t) / ||W||^2,
//           relchg[t] = ||Q^t - Q^{t-1}||_F / ||Q^{t-1}||_F   (0 when the denominator is 0).
// The two scale steps minimise F exactly over the admissible sets (each is a separable
// 1-D quadratic whose constrained minimiser is the projection of N/D).
// Outputs: final r, c; codes, block scales and tensor scale of Q^T; histories
// nmse[0..T], relchg[0..T] (relchg[0] = 0); rejected-step count; and, when given,
// traces of every iteration's unprojected closed-form values, r_trace [T][rows] and
// c_trace [T][cols] (NaN where D = 0).  tol > 0 stops after the first iteration whose
// relchg is <= tol (a rejected step has relchg 0); iters_run reports the count.
// Resuming: the solver's whole state is (r, c, kept Qhat).  When q_codes is given, the
// solve starts from r_init, c_init and the kept Qhat held in q_codes / q_scales /
// q_tscale (the outputs of an earlier solve) instead of FQ(W ./ r c^T): after a rejected
// step the kept Qhat is not the quantisation of W at the current scales, so the scales
// alone would not resume exactly.
int o_solve(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int g,
            int iters, float tol, const float* r_init, const float* c_init, float* r_out,
            float* c_out, uint8_t* codes, void* scales, float* tscale, double* nmse_hist,
            double* relchg_hist, int* rejected_out, int* iters_run, float* r_trace,
            float* c_trace, uint32_t* flags_out, int steps, const uint8_t* q_codes,
            const void* q_scales, float q_tscale) {
  if (!W || !r_out || !c_out || !codes || !scales) return ERR_NULL;
  if (steps < 0 || steps > 3) return ERR_SHAPE;
  if (!group_ok(fmt, g)) return ERR_FORMAT;
  if (rows < 0 || cols < 0 || cols % g || ld < cols || iters < 0) return ERR_SHAPE;
  if (fmt == FMT_NVFP4 && !tscale) return ERR_NULL;
  const int64_t N = rows * cols;
  const int64_t nblk = N / g;
  std::vector<float> Wf(N);
  load_w(W, dtype, rows, cols, ld, Wf.data());
  if (!all_finite(Wf.data(), N)) return ERR_VALUE;

  std::vector<float> r(rows, 1.0f), c(cols, 1.0f);
  if (r_init) std::copy(r_init, r_init + rows, r.begin());
  if (c_init) std::copy(c_init, c_init + cols, c.begin());

  double normW2 = 0.0;
  for (int64_t i = 0; i < N; ++i) normW2 += (double)Wf[i] * (double)Wf[i];

  const size_t sc_bytes = is_int_grouped(fmt) ? 2 : 1;
  const int64_t code_bytes = N * code_bits(fmt) / 8;
  std::vector<float> V(N), Q(N), Qc(N);
  std::vector<uint8_t> codesA(code_bytes), codesC(code_bytes);
  std::vector<uint8_t> scA(nblk * sc_bytes), scC(nblk * sc_bytes);
  float tsA = 0.0f, tsC = 0.0f;
  uint32_t flags = 0;

  if (q_codes) {
    if (!q_scales) return ERR_NULL;
    std::memcpy(codesA.data(), q_codes, codesA.size());
    std::memcpy(scA.data(), q_scales, scA.size());
    tsA = (fmt == FMT_NVFP4) ? q_tscale : 0.0f;
    int rc = o_dequantize(fmt, g, codesA.data(), scA.data(), tsA, rows, cols, Q.data());
    if (rc != OK) return rc;
  } else {
    normalise(Wf.data(), rows, cols, r.data(), c.data(), V.data());
    FQOut o{codesA.data(), scA.data(), &tsA, Q.data(), 0u};
    fq_matrix(fmt, g, V.data(), rows, cols, o);
    flags |= o.flags;
  }
  auto nmse_of = [&](double F) { return normW2 > 0.0 ? F / normW2 : 0.0; };
  if (nmse_hist) nmse_hist[0] = nmse_of(recon_error(Wf.data(), Q.data(), r.data(), c.data(), rows, cols));
  if (relchg_hist) relchg_hist[0] = 0.0;
  int rejected = 0, done = 0;

  std::vector<double> rowN(rows), rowD(rows), colN(cols), colD(cols);
  for (int t = 1; t <= iters; ++t) {
    // r-step (skipped, r kept, when the row scales are frozen)
    if (steps & 1) {
    parallel_rows(rows, [&](int64_t b, int64_t e) {
      for (int64_t i = b; i < e; ++i) {
        double n_ = 0.0, d_ = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
          double u = (double)Q[i * cols + j] * (double)c[j];
          n_ += (double)Wf[i * cols + j] * u;
          d_ += u * u;
        }
        rowN[i] = n_;
        rowD[i] = d_;
      }
    });
    for (int64_t i = 0; i < rows; ++i) {
      float x = std::numeric_limits<float>::quiet_NaN();
      if (rowD[i] > 0.0) {
        x = (float)(rowN[i] / rowD[i]);
        r[i] = project(fmt, x);
      }
      if (r_trace) r_trace[(int64_t)(t - 1) * rows + i] = x;
    }
    }
    // c-step (loop interchanged per column range; each column still sums rows in order);
    // skipped, c kept, when the column scales are frozen
    if (steps & 2) {
    parallel_rows(cols, [&](int64_t jb, int64_t je) {
      for (int64_t j = jb; j < je; ++j) { colN[j] = 0.0; colD[j] = 0.0; }
      for (int64_t i = 0; i < rows; ++i) {
        double ri = (double)r[i];
        for (int64_t j = jb; j < je; ++j) {
          double q = (double)Q[i * cols + j];
          colN[j] += ri * (double)Wf[i * cols + j] * q;
          double u = ri * q;
          colD[j] += u * u;
        }
      }
    });
    for (int64_t j = 0; j < cols; ++j) {
      float x = std::numeric_limits<float>::quiet_NaN();
      if (colD[j] > 0.0) {
        x = (float)(colN[j] / colD[j]);
        c[j] = project(fmt, x);
      }
      if (c_trace) c_trace[(int64_t)(t - 1) * cols + j] = x;
    }
    }
    // Q-step with safeguard
    normalise(Wf.data(), rows, cols, r.data(), c.data(), V.data());
    FQOut o{codesC.data(), scC.data(), &tsC, Qc.data(), 0u};
    fq_matrix(fmt, g, V.data(), rows, cols, o);
    flags |= o.flags;
    double Fc = recon_error(Wf.data(), Qc.data(), r.data(), c.data(), rows, cols);
    double Fp = recon_error(Wf.data(), Q.data(), r.data(), c.data(), rows, cols);
    double relv = 0.0;
    if (Fc <= Fp) {
      double num = 0.0, den = 0.0;
      for (int64_t i = 0; i < N; ++i) {
        double dq = (double)Qc[i] - (double)Q[i];
        num += dq * dq;
        den += (double)Q[i] * (double)Q[i];
      }
      relv = den > 0.0 ? std::sqrt(num) / std::sqrt(den) : 0.0;
      if (relchg_hist) relchg_hist[t] = relv;
      if (nmse_hist) nmse_hist[t] = nmse_of(Fc);
      Q.swap(Qc);
      codesA.swap(codesC);
      scA.swap(scC);
      tsA = tsC;
    } else {
      ++rejected;
      if (relchg_hist) relchg_hist[t] = 0.0;
      if (nmse_hist) nmse_hist[t] = nmse_of(Fp);
    }
    done = t;
    if (tol > 0.0f && relv <= (double)tol) break;
  }
  std::copy(r.begin(), r.end(), r_out);
  std::copy(c.begin(), c.end(), c_out);
  std::memcpy(codes, codesA.data(), codesA.size());
  std::memcpy(scales, scA.data(), scA.size());
  if (fmt == FMT_NVFP4) *tscale = tsA;
  if (rejected_out) *rejected_out = rejected;
  if (iters_run) *iters_run = done;
  if (flags_out) *flags_out = flags;
  return OK;
}

// ---- activation path: x' = x * c_j (fp32; exact for admissible c), then FQ_f per
// token row along the in-dimension.  c null means no rescaling (beta not applied).
int o_rescale_quantize_acts(const uint16_t* X, int64_t tokens, int64_t cols, int64_t ld,
                            const float* c, int fmt, int g, uint8_t* codes, void* scales,
                            float* tscale, float* xq_rescaled) {
  if (!X || !codes || !scales) return ERR_NULL;
  if (!group_ok(fmt, g)) return ERR_FORMAT;
  if (tokens < 0 || cols < 0 || cols % g || ld < cols) return ERR_SHAPE;
  std::vector<float> Xs(tokens * cols);
  for (int64_t t = 0; t < tokens; ++t)
    for (int64_t j = 0; j < cols; ++j) {
      float x = bf16_to_f32(X[t * ld + j]);
      Xs[t * cols + j] = c ? x * c[j] : x;
    }
  if (!all_finite(Xs.data(), tokens * cols)) return ERR_VALUE;
  return o_fq(fmt, g, Xs.data(), tokens, cols, codes, scales, tscale, xq_rescaled, nullptr);
}

// ---- activation SQNR in the activation domain: xhat = deq(FQ(x * c)) / c,
// SQNR = 10 log10( sum x^2 / sum (x - xhat)^2 ).  c null means ones.
double o_act_sqnr(const uint16_t* X, int64_t tokens, int64_t cols, int64_t ld, const float* c,
                  int fmt, int g, const uint8_t* codes, const void* scales, float tscale) {
  std::vector<float> deq(tokens * cols);
  if (o_dequantize(fmt, g, codes, scales, tscale, tokens, cols, deq.data()) != OK)
    return std::numeric_limits<double>::quiet_NaN();
  double sx = 0.0, se = 0.0;
  for (int64_t t = 0; t < tokens; ++t)
    for (int64_t j = 0; j < cols; ++j) {
      double x = (double)bf16_to_f32(X[t * ld + j]);
      double xh = (double)deq[t * cols + j] / (c ? (double)c[j] : 1.0);
      sx += x * x;
      se += (x - xh) * (x - xh);
    }
  if (se == 0.0) return std::numeric_limits<double>::infinity();
  return 10.0 * std::log10(sx / se);
}

// ---- quantised linear layer (the listing page's Table 11 "quantized linears" and
// Table 12's packed 4-bit weights; the news summary: beta folds into the activation
// quantiser, r into the layer's output).  With activations quantised as
// Aq = FQ(X diag(c)) (tokens x K) and weights W ~ diag(r) Q diag(c) (N x K),
//   Y = X W^T ~ Aq . Q^T . diag(r),   Y_tn = r_n * sum_k Aq_tk Q_nk,
// every element dequantised from its codes and block scales, products and sums in fp64.
// r may be null (ones).  Y is [M][N] fp64.  Sampled variant: only the entries (m[i], n[i]).
// NVFP4 elements are dequantised without their tensor scale (e2m1 * e4m3 is exact in fp32);
// the callers multiply each product by a_ts * b_ts in fp64, so every element stands for
// e2m1 * e4m3 * s_t exactly, as the format defines it.
static int linear_deq(int fmt, int g, const uint8_t* a_codes, const void* a_scales, int64_t M,
                      const uint8_t* b_codes, const void* b_scales, int64_t N, int64_t K,
                      std::vector<float>& A, std::vector<float>& B) {
  if (!a_codes || !a_scales || !b_codes || !b_scales) return ERR_NULL;
  if (!group_ok(fmt, g)) return ERR_FORMAT;
  if (M < 0 || N < 0 || K < 0 || K % g) return ERR_SHAPE;
  A.assign((size_t)M * K, 0.0f);
  B.assign((size_t)N * K, 0.0f);
  int rc = o_dequantize(fmt, g, a_codes, a_scales, 1.0f, M, K, A.data());
  if (rc != OK) return rc;
  return o_dequantize(fmt, g, b_codes, b_scales, 1.0f, N, K, B.data());
}

int o_quantized_linear(int fmt, int g, const uint8_t* a_codes, const void* a_scales, float a_ts,
                       int64_t M, const uint8_t* b_codes, const void* b_scales, float b_ts,
                       int64_t N, int64_t K, const float* r, double* Y) {
  if (!Y) return ERR_NULL;
  std::vector<float> A, B;
  int rc = linear_deq(fmt, g, a_codes, a_scales, M, b_codes, b_scales, N, K, A, B);
  if (rc != OK) return rc;
  const double ts = fmt == FMT_NVFP4 ? (double)a_ts * (double)b_ts : 1.0;
  parallel_rows(M, [&](int64_t b, int64_t e) {
    for (int64_t m = b; m < e; ++m)
      for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += (double)A[m * K + k] * (double)B[n * K + k] * ts;
        Y[m * N + n] = acc * (r ? (double)r[n] : 1.0);
      }
  });
  return OK;
}

// Entries (m[i], n[i]) of the same product, plus sum_k |Aq_mk Q_nk| |r_n| for error bounds.
int o_quantized_linear_entries(int fmt, int g, const uint8_t* a_codes, const void* a_scales,
                               float a_ts, int64_t M, const uint8_t* b_codes,
                               const void* b_scales, float b_ts, int64_t N, int64_t K,
                               const float* r, const int64_t* mi, const int64_t* ni,
                               int64_t count, double* y, double* absy) {
  if (!mi || !ni || !y || !absy) return ERR_NULL;
  std::vector<float> A, B;
  int rc = linear_deq(fmt, g, a_codes, a_scales, M, b_codes, b_scales, N, K, A, B);
  if (rc != OK) return rc;
  const double ts = fmt == FMT_NVFP4 ? (double)a_ts * (double)b_ts : 1.0;
  for (int64_t i = 0; i < count; ++i) {
    if (mi[i] < 0 || mi[i] >= M || ni[i] < 0 || ni[i] >= N) return ERR_SHAPE;
    double acc = 0.0, aa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double p = (double)A[mi[i] * K + k] * (double)B[ni[i] * K + k] * ts;
      acc += p;
      aa += std::fabs(p);
    }
    const double rn = r ? (double)r[ni[i]] : 1.0;
    y[i] = acc * rn;
    absy[i] = aa * std::fabs(rn);
  }
  return OK;
}

}  // extern "C"
