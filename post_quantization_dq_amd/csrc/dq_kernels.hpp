// HIP kernels of the DualQuant dual-scale BCD solver for gfx950.
//
// Each BCD iteration is three launches over all problems of a batch:
//   k_rowpass   one wave per row (no workgroup barriers in the row loop); c and 1/c of every
//               column sit in LDS.  It quantises the candidate Qc = FQ_f(W ./ r^s c^s^T)
//               (Qhat-step of iteration s) and stores its codes, measures F(r^s,c^s,Qc), the
//               change against the kept Qhat^{s-1} read back from its codes (relchg numerator,
//               and dF = F(Qc) - F(Qhat^{s-1}) accumulated per lane, so unchanged elements add
//               exactly 0 to the safeguard decision), and runs the r-step of iteration s+1
//               for both outcomes of the safeguard: from the candidate (kept if dF <= 0) and
//               from the kept Qhat^{s-1} (whole-row sums, fp64 across lanes).  The two differ
//               only on the chunks whose codes changed.
//   k_colpass   workgroups own 1024-column strips and a range of rows; each wave first
//               reduces the row pass's dF partials (a fixed order, so every workgroup and the
//               finalize reach the same decision), then, with the r of the outcome taken, it
//               accumulates the c-step sums N_j, D_j (and the NVFP4 column amax of W ./ r) of
//               that outcome's Qhat in registers and writes one partial per row range.
//   k_finalize  reduces the partials and projects c; its first workgroup per problem takes
//               the safeguard decision and writes the next sweep's state (after a rejection
//               it moves the kept-Qhat r-step into place).  Every sweep therefore completes
//               one iteration: a solve of T iterations is T + 1 sweeps, rejected steps or not.
// Lane l of a wave owns chunks of 16 consecutive columns; blocks of MX (32) and INT4/INT8
// (64/128) formats span 2..8 adjacent lanes.

#pragma once
#include <type_traits>

#include "dq_device.hpp"

namespace dqk {

enum Mode { MODE_INIT = 0, MODE_NORMAL = 1, MODE_DONE = 3 };

// Per-problem solver state.  It is double-buffered by sweep parity: the kernels of sweep sw
// read st[sw & 1], and the decision at the end of sweep sw (k_finalize) writes the whole of
// st[(sw + 1) & 1], so no kernel reads a state that is being written.
struct alignas(16) State {
  int32_t mode, it_done, acc, rs;
  int32_t cs, rejected, sweeps, needs_ts;   // needs_ts: NVFP4 tensor scale from fwp pending
  float st_cur, k6_cur, st_acc, pad2;
  double normW2, qn2_acc;
};

// A solve's report as it lands in the caller's device memory (the layout of dq_report).
struct ReportDev {
  int32_t iters_run, rejected_steps;
  uint32_t flags;
  int32_t sweeps;
};

struct ProbDev {
  const void* W;
  int64_t rows, cols, ld;
  float* r[3];      // row scales: the current slot (state rs) and one per outcome of the next
  float* ir[3];     // r-step, (rs + 1) % 3 from the candidate, (rs + 2) % 3 from the kept Qhat
  float* c[2];
  float* ic[2];
  uint8_t* codes[2];
  void* scales[2];
  void* colP;       // [rranges][NQ][cols] column partials (fp64 for INT4/INT8, else fp32)
  double* swp;      // [rowblocks][4]: F(Qc), dF, relchg numerator, ||Qc||^2
  float* fwp;       // [fin_wgs]: NVFP4 amax partials
  double* initp;    // [init_wgs][2]
  State* st;        // [2], by sweep parity
  uint32_t* flags;  // DQ_FLAG_* bits, set with atomics by any kernel
  double* nmse;     // [iters+1]
  double* relchg;   // [iters+1]
  float* x_alt;     // [rows]: unprojected kept-Qhat r-step values (NaN: no closed form)
  uint32_t* altz;   // nonzero: a row's kept-Qhat r-step had D = 0 in this sweep
  float* r_trace;   // [iters][rows] or null: unprojected r-step values
  float* c_trace;   // [iters][cols] or null: unprojected c-step values
  const float* r_init;
  const float* c_init;
  float* r_out;     // the caller's outputs: final r [rows], c [cols], NVFP4 tensor scale [1]
  float* c_out;
  float* ts_out;    // null outside NVFP4
  ReportDev* report;   // the caller's device report, or null
  int32_t rowblocks, rows_per_blk, fin_wgs, iters;   // row pass: blocks of rows per workgroup
  int32_t nstrips, rranges, rows_per_range, init_wgs; // column pass: 1024-column strips x row ranges
  int32_t dtype;
  float tol;
  int32_t steps;   // scale steps that run: bit 0 row scales, bit 1 column scales
  int32_t pad;
};

struct WgEntry {
  int32_t prob, idx;
};

// The solve's counter of problems still running is followed, kStatesOffset bytes on, by
// the two state slots of every problem of the call (problem k: slots 2k, 2k + 1), so a
// pass reaches its state from the launch-table entry alone, in parallel with the problem
// descriptor, instead of through the descriptor's pointer.
constexpr int kStatesOffset = 256;
__device__ __forceinline__ State* state_slots(const int32_t* live, int prob) {
  return (State*)((const char*)live + kStatesOffset) + 2 * prob;
}

// Flag bit of a solve whose state did not reach DONE within the sweeps that were queued
// (cannot happen: a solve of T iterations takes T + 1 sweeps).
constexpr uint32_t kFlagUnfinished = 32u;

// ---------------------------------------------------------------- loads and stores
// Codes of chunk l of row i: 8 bytes (4-bit formats), 12 bytes (6-bit) or 16 bytes (8-bit).
template <int FMT, int L>
__device__ __forceinline__ void store_chunk(uint8_t* codes, void* scales, int64_t i, int64_t n,
                                            int l, int g, const Chunk& ch) {
  if (code_words<FMT>() == 4) {
    *gp((u32x4*)(codes + i * n + 16 * (int64_t)l)) = u32x4{ch.code[0], ch.code[1], ch.code[2], ch.code[3]};
  } else if (code_words<FMT>() == 3) {
    DQ_GAS uint32_t* q = gp((uint32_t*)(codes + ((i * n * 3) >> 2) + 12 * (int64_t)l));
    q[0] = ch.code[0];
    q[1] = ch.code[1];
    q[2] = ch.code[2];
  } else
    *gp((u32x2*)(codes + ((i * n) >> 1) + 8 * (int64_t)l)) = u32x2{ch.code[0], ch.code[1]};
  if ((l % L) == 0) {
    int64_t bi = i * (n / g) + l / L;
    if (Traits<FMT>::SCALE_BYTES == 2) gp((uint16_t*)scales)[bi] = (uint16_t)ch.scode;
    else gp((uint8_t*)scales)[bi] = (uint8_t)ch.scode;
  }
}

template <int FMT, int L>
__device__ __forceinline__ void load_codes(const uint8_t* codes, const void* scales, int64_t i,
                                           int64_t n, int l, int g, uint32_t (&c)[4],
                                           uint32_t& sc) {
  if (code_words<FMT>() == 4) {
    const u32x4 cw = *gp((const u32x4*)(codes + i * n + 16 * (int64_t)l));
    c[0] = cw.x; c[1] = cw.y; c[2] = cw.z; c[3] = cw.w;
  } else if (code_words<FMT>() == 3) {
    const DQ_GAS uint32_t* q = gp((const uint32_t*)(codes + ((i * n * 3) >> 2) + 12 * (int64_t)l));
    c[0] = q[0]; c[1] = q[1]; c[2] = q[2]; c[3] = 0u;
  } else {
    const u32x2 cw = *gp((const u32x2*)(codes + ((i * n) >> 1) + 8 * (int64_t)l));
    c[0] = cw.x; c[1] = cw.y; c[2] = 0u; c[3] = 0u;
  }
  int64_t bi = i * (n / g) + l / L;
  sc = (Traits<FMT>::SCALE_BYTES == 2) ? (uint32_t)gp((const uint16_t*)scales)[bi]
                                       : (uint32_t)gp((const uint8_t*)scales)[bi];
}

__device__ __forceinline__ void build_nvtab(NvTab& tab, float s_t) {
  for (int k = threadIdx.x; k < 128; k += blockDim.x) {
    float d = e4m3_value((uint32_t)k) * s_t;
    tab.d[k] = (k > 0) ? d : 0.0f;
    tab.id[k] = (k > 0 && d > 0.0f) ? 1.0f / d : 0.0f;
  }
}

// NVFP4 tensor-scale terms from the normalised matrix's amax A: s_t = A / 2688 and
// k6 = 1 / (6 s_t).  The scheme divides by 6 s_t and by every block factor e4m3(sb) s_t,
// the smallest being 2^-9 s_t; when either reciprocal is not a finite fp32 number (s_t at
// or below about 2^-119) or s_t is 0, no block can be encoded and the matrix quantises to
// zero (`tiny`, flag bit 16 when A > 0).
__device__ __forceinline__ void nv_tensor_terms(float A, float& s_t, float& k6, bool& tiny) {
  s_t = A / 2688.0f;
  float six = 6.0f * s_t;
  k6 = (s_t > 0.0f) ? 1.0f / six : 0.0f;
  const float id_min = (s_t > 0.0f) ? 1.0f / (0x1p-9f * s_t) : 0.0f;
  tiny = false;
  if (!(s_t > 0.0f) || !isfinite(k6) || !isfinite(id_min)) {
    tiny = (A > 0.0f);
    s_t = 0.0f;
    k6 = 0.0f;
  }
}

// ---------------------------------------------------------------- setup / init
// Scales from the caller's initial values (or ones) and a fresh state.
__global__ void k_setup(const ProbDev* __restrict__ probs) {
  const ProbDev& P = probs[blockIdx.y];
  if (P.rows == 0 || P.cols == 0) return;   // empty problems have no buffers
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < P.rows) {
    float r = P.r_init ? gp(P.r_init)[k] : 1.0f;
    gp(P.r[0])[k] = r;
    gp(P.ir[0])[k] = 1.0f / r;
  }
  if (k < P.cols) {
    float c = P.c_init ? gp(P.c_init)[k] : 1.0f;
    gp(P.c[0])[k] = c;
    gp(P.ic[0])[k] = 1.0f / c;
  }
  if (k == 0) {
    State* s = P.st;
    s->mode = MODE_INIT;
    s->it_done = 0;
    s->acc = 0;
    s->rs = 0;
    s->cs = 0;
    s->rejected = 0;
    s->sweeps = 0;
    s->needs_ts = 0;
    s->st_cur = s->k6_cur = s->st_acc = 0.0f;
    s->normW2 = 0.0;
    s->qn2_acc = 0.0;
    *P.flags = 0u;
    *P.altz = 0u;
  }
}

// ||W||^2 (fp64), non-finite check, and for NVFP4 the amax of W ./ r c^T at the initial
// scales.  blockIdx.y = problem, blockIdx.x = block of rows.
template <int FMT, int DT>
__global__ __launch_bounds__(256) void k_init(const ProbDev* __restrict__ probs) {
  const ProbDev& P = probs[blockIdx.y];
  if (P.dtype != DT || P.rows == 0 || P.cols == 0 || (int)blockIdx.x >= P.init_wgs) return;
  const int64_t n = P.cols;
  const int64_t rpb = (P.rows + P.init_wgs - 1) / P.init_wgs;
  const int64_t r0 = (int64_t)blockIdx.x * rpb, r1 = min(P.rows, r0 + rpb);
  double s2 = 0.0;
  float amax = 0.0f;
  bool bad = false;
  constexpr int VEC = (DT == 1) ? 8 : 4;   // elements per 16-byte load
  constexpr int U = 4;                      // loads in flight per thread
  const int64_t nv = n / VEC;
  const int64_t rowbytes = P.ld * (DT == 1 ? 2 : 4);
  const DQ_GAS f32x4* ic4 = gp((const f32x4*)P.ic[0]);
  // with the default initial column scales (all 1) and a row scale of 1, (w * ir) * ic is w
  // exactly, so the NVFP4 amax needs no multiplies
  const bool unit_c = P.c_init == nullptr;
  for (int64_t i = r0; i < r1; ++i) {
    const float ir = gp(P.ir[0])[i];
    const bool unit = unit_c && ir == 1.0f;
    const DQ_GAS u32x4* rowp = gp((const u32x4*)((const char*)P.W + i * rowbytes));
    for (int64_t v0 = threadIdx.x; v0 < nv; v0 += (int64_t)blockDim.x * U) {
      u32x4 u[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int64_t v = v0 + (int64_t)q * blockDim.x;
        if (v < nv) u[q] = rowp[v];
        else u[q] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int64_t v = v0 + (int64_t)q * blockDim.x;
        if (v >= nv) break;
        float w[VEC];
        const uint32_t uu[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
        if (DT == 1) {
#pragma unroll
          for (int k = 0; k < 4; ++k) { w[2 * k] = u2f(uu[k] << 16); w[2 * k + 1] = u2f(uu[k] & 0xFFFF0000u); }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) w[k] = u2f(uu[k]);
        }
        // sum of squares: a bf16 square is exact in fp32 and eight of them are summed with
        // a relative error below 2^-21 before the fp64 accumulation; an fp32 input's four
        // squares round once each.  A partial that is not finite (a NaN or Inf element, or a
        // square beyond the fp32 range) or below 2^-100 (where squares may underflow) is
        // redone element by element in fp64.
        float p2 = 0.0f;
#pragma unroll
        for (int k = 0; k < VEC; ++k) p2 = fmaf(w[k], w[k], p2);
        if (isfinite(p2) && p2 >= 0x1p-100f) {
          s2 += (double)p2;
        } else {
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            bad |= !isfinite(w[k]);
            s2 += (double)w[k] * (double)w[k];
          }
        }
        if (FMT == NVFP4) {
          if (unit) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) amax = fmaxf(amax, fabsf(w[k]));
          } else {
            float icv[VEC];
#pragma unroll
            for (int k = 0; k < VEC / 4; ++k) {
              const f32x4 a = ic4[v * (VEC / 4) + k];
              icv[4 * k] = a.x; icv[4 * k + 1] = a.y; icv[4 * k + 2] = a.z; icv[4 * k + 3] = a.w;
            }
#pragma unroll
            for (int k = 0; k < VEC; ++k) amax = fmaxf(amax, fabsf((w[k] * ir) * icv[k]));
          }
        }
      }
    }
  }
  __shared__ double ss[4];
  __shared__ float sm[4];
  s2 = wave_sum(s2);
  amax = wave_max(amax);
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { ss[wv] = s2; sm[wv] = amax; }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    gp(P.initp)[2 * blockIdx.x] = ((ss[0] + ss[1]) + ss[2]) + ss[3];
    gp(P.initp)[2 * blockIdx.x + 1] = (double)fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    if (bad) atomicOr(P.flags, 1u);
  }
}

// Combines k_init's partials (one workgroup per problem): strided per thread, then in
// fixed order; sets ||W||^2 and the initial NVFP4 tensor-scale terms.
template <int FMT>
__global__ __launch_bounds__(256) void k_init_reduce(const ProbDev* __restrict__ probs) {
  const ProbDev& P = probs[blockIdx.x];
  if (P.rows == 0 || P.cols == 0) return;
  __shared__ double ss[4];
  __shared__ float sm[4];
  double tot = 0.0;
  float A = 0.0f;
  for (int b = threadIdx.x; b < P.init_wgs; b += blockDim.x) {
    tot += gp(P.initp)[2 * b];
    A = fmaxf(A, (float)gp(P.initp)[2 * b + 1]);
  }
  tot = wave_sum(tot);
  A = wave_max(A);
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { ss[wv] = tot; sm[wv] = A; }
  __syncthreads();
  if (threadIdx.x != 0) return;
  tot = ((ss[0] + ss[1]) + ss[2]) + ss[3];
  A = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  State* s = P.st;
  s->normW2 = tot;
  if (FMT == NVFP4) {
    float st_, k6_;
    bool tiny;
    nv_tensor_terms(A, st_, k6_, tiny);
    s->st_cur = st_;
    s->k6_cur = k6_;
    if (tiny) atomicOr(P.flags, 16u);
  }
}

// ---------------------------------------------------------------- raw rows
template <int DT>
struct RawRow;
template <>
struct RawRow<1> {   // bf16: 8 packed words per chunk
  uint32_t u[8];
  __device__ __forceinline__ void load(const void* base, int64_t i, int64_t ld, int j0) {
    const DQ_GAS u32x4* p = gp((const u32x4*)((const uint16_t*)base + i * ld + j0));
    const u32x4 a = p[0], b = p[1];
    u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w; u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int k = 0; k < 8; ++k) u[k] = 0u;
  }
  __device__ __forceinline__ void unpack(float (&w)[16]) const {
#pragma unroll
    for (int k = 0; k < 8; ++k) { w[2 * k] = u2f(u[k] << 16); w[2 * k + 1] = u2f(u[k] & 0xFFFF0000u); }
  }
};
template <>
struct RawRow<0> {   // fp32: 16 floats per chunk
  float f[16];
  __device__ __forceinline__ void load(const void* base, int64_t i, int64_t ld, int j0) {
    const DQ_GAS f32x4* p = gp((const f32x4*)((const float*)base + i * ld + j0));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 a = p[k];
      f[4 * k] = a.x; f[4 * k + 1] = a.y; f[4 * k + 2] = a.z; f[4 * k + 3] = a.w;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int k = 0; k < 16; ++k) f[k] = 0.0f;
  }
  __device__ __forceinline__ void unpack(float (&w)[16]) const {
#pragma unroll
    for (int k = 0; k < 16; ++k) w[k] = f[k];
  }
};

// 16 values of chunk ch from an LDS vector stored chunk-interleaved: float4 number q (0..3)
// of chunk ch at index q * nch + ch, so consecutive lanes read consecutive 16-byte words.
__device__ __forceinline__ void lds_load16(const f32x4* base, int nch, int ch, float (&x)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 a = base[q * nch + ch];
    x[4 * q] = a.x; x[4 * q + 1] = a.y; x[4 * q + 2] = a.z; x[4 * q + 3] = a.w;
  }
}

// 16 consecutive floats (vector loads when the base is 16-byte aligned).
__device__ __forceinline__ void load16_global(const float* p, bool aligned, float (&x)[16]) {
  if (aligned) {
    const DQ_GAS f32x4* q = gp((const f32x4*)p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 a = q[k];
      x[4 * k] = a.x; x[4 * k + 1] = a.y; x[4 * k + 2] = a.z; x[4 * k + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = gp(p)[k];
  }
}

// Which iteration a pass belongs to, read from the problem's state at kernel entry.
struct PassInfo {
  int mode, it, rs, cs, acc, cb, tr;
  bool stats, next, alt;
  __device__ __forceinline__ PassInfo(const State* st, int iters) {
    mode = st->mode;
    it = (mode == MODE_INIT) ? 0 : st->it_done + 1;
    stats = (mode == MODE_NORMAL);           // a kept Qhat exists: safeguard and relchg
    next = (it < iters);                     // the r/c steps of iteration it + 1 run now
    alt = stats && next;                     // ... for both outcomes of the safeguard
    rs = st->rs;
    cs = st->cs;
    acc = st->acc;
    cb = (mode == MODE_INIT) ? 0 : 1 - acc;  // buffer the candidate is written to
    tr = it;                                 // trace row of the r/c steps computed now
  }
};

// Row-scale slots written by a sweep whose current slot is rs: the r-step from the candidate
// and the one from the kept Qhat.
__device__ __forceinline__ int slot_next(int rs) { return rs == 2 ? 0 : rs + 1; }
__device__ __forceinline__ int slot_alt(int rs) { return rs == 0 ? 2 : rs - 1; }

// dF = F(Qc) - F(kept Qhat) summed over the row pass's workgroup partials in one fixed order
// (lane-strided, four partials per lane requested at once, then a butterfly whose result is
// the same in every lane), so the column pass's workgroups and the finalize's decision all
// reach the same value.  Every lane of the wave must take part in the butterfly.
__device__ __forceinline__ double rowpass_dF_part(const ProbDev& P) {
  const int lane = threadIdx.x & 63;
  double s = 0.0;
  for (int b0 = 0; b0 < P.rowblocks; b0 += 256) {
    double v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = b0 + 64 * u + lane;
      v[u] = b < P.rowblocks ? gp(P.swp)[4 * (size_t)b + 1] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) s += v[u];
  }
  return s;
}
__device__ __forceinline__ double rowpass_dF_sum(double part) { return wave_sum(part); }
__device__ __forceinline__ double rowpass_dF(const ProbDev& P) {
  return rowpass_dF_sum(rowpass_dF_part(P));
}

// Exact products of the grouped integer formats' kept-Qhat r-step sums, as doubles.  With
// projected (bf16) column scales, q = p c has at most 3 + 8 (INT4) or 7 + 8 (INT8) significant
// bits, so w q for a bf16 weight (8 bits) and q^2 for INT4 are exact in fp32 and one fp32
// multiply gives the same double as an fp64 multiply; the others are taken in fp64.
template <int FMT, int DT>
__device__ __forceinline__ double exact_wq(float w, float q) {
  if (DT == 1) return (double)(w * q);
  return (double)w * (double)q;
}
template <int FMT>
__device__ __forceinline__ double exact_qq(float q) {
  if (FMT == INT4) return (double)(q * q);
  return (double)q * (double)q;
}

// ---------------------------------------------------------------- row pass
// Words of one entry of the row pass's queue of changed chunks: the chunk index and block
// scale code in one word, then the candidate's code words; padded to 16 or 32 bytes.
template <int FMT>
constexpr int queue_words() { return code_words<FMT>() + 1 <= 4 ? 4 : 8; }
constexpr int kQueueLen = 64;   // entries per wave: one flush runs one entry per lane

// CG = 1 (matrices wider than the LDS holds): c and 1/c are read from global memory (they
// stay in L2) instead of LDS.
//
// Kept-Qhat work on changed chunks only: a chunk whose candidate codes and block scale code
// equal the kept ones (under equal block factors: always for the MX and integer formats,
// for NVFP4 when the two tensor scales are equal) has the same dequantised values, so it adds
// exactly 0 to the change of F and to the relchg numerator.  With `compact` set, a changed
// chunk adds its candidate error to dF at once and is queued (per wave, in LDS); at the end
// of the row, or when the queue is full, one lane per queued chunk reloads its W and kept
// codes, subtracts the kept Qhat's error and adds its relchg term.  On the pages' NVFP4
// weights a few percent of the chunks change per iteration.
template <int FMT, int DT, int L, int CG>
__global__ __launch_bounds__(1024) void k_rowpass(const ProbDev* __restrict__ probs,
                                                  const WgEntry* __restrict__ table, int sw,
                                                  const int32_t* __restrict__ live, int compact) {
  // the counter and the table entry are requested together (one round of latency)
  const int32_t nlive = *gp(live);
  const WgEntry we = table[blockIdx.x];
  if (nlive == 0) return;   // every problem finished: this queued sweep has nothing to do
  const ProbDev& P = probs[we.prob];
  State* st = state_slots(live, we.prob) + (sw & 1);
  if (st->mode == MODE_DONE) return;
  const PassInfo pi(st, P.iters);
  constexpr bool A64 = grouped_int<FMT>();   // INT4/INT8: exact products accumulated in fp64
  const int g = L * 16;
  const int64_t n = P.cols;
  const int nch = (int)(n >> 4);

  extern __shared__ float lds[];
  f32x4* s_c4 = (f32x4*)lds;           // c, chunk-interleaved (see lds_load16)
  f32x4* s_ic4 = s_c4 + 4 * nch;       // 1/c, same layout
  NvTab* tab_c = (NvTab*)(CG ? lds : lds + 2 * n);
  NvTab* tab_p = tab_c + 1;
  __shared__ double redw[16][4];
  // the wave index as a wave-uniform (scalar) value, so the row addresses derived from it are too
  const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63,
            nw = (int)(blockDim.x >> 6);
  constexpr int QW = queue_words<FMT>();
  uint32_t* queue = (uint32_t*)(tab_c + (FMT == NVFP4 ? 2 : 0)) + (size_t)wave * kQueueLen * QW;

  // NVFP4 tensor scale of this sweep's candidate.  After a kept step it follows from the
  // amax of W ./ r c^T at the new scales, i.e. from the finalize partials: every workgroup
  // derives the same value, and the first one records it for the later kernels of the sweep.
  float s_t = 0.0f, k6 = 0.0f;
  if (FMT == NVFP4) {
    s_t = st->st_cur;
    k6 = st->k6_cur;
    if (st->needs_ts) {
      __shared__ float sa[16];
      float a = 0.0f;
      for (int k = t; k < P.fin_wgs; k += blockDim.x) a = fmaxf(a, gp(P.fwp)[k]);
      a = wave_max(a);
      if (lane == 0) sa[wave] = a;
      __syncthreads();
      a = sa[0];
      for (int w = 1; w < nw; ++w) a = fmaxf(a, sa[w]);
      bool tiny;
      nv_tensor_terms(a, s_t, k6, tiny);
      if (we.idx == 0 && t == 0) {
        st->st_cur = s_t;
        st->k6_cur = k6;
        if (tiny) atomicOr(P.flags, 16u);
      }
    }
  }

  const float* cglob = P.c[pi.cs];
  const float* icglob = P.ic[pi.cs];
  {
    const DQ_GAS f32x4* c4 = gp((const f32x4*)cglob);
    const DQ_GAS f32x4* ic4 = gp((const f32x4*)icglob);
    for (int e = threadIdx.x; !CG && e < 4 * nch; e += blockDim.x) {
      const int ch = e >> 2, q = e & 3;
      s_c4[q * nch + ch] = c4[e];
      s_ic4[q * nch + ch] = ic4[e];
    }
    if (FMT == NVFP4) {
      build_nvtab(*tab_c, s_t);
      build_nvtab(*tab_p, st->st_acc);
    }
  }
  __syncthreads();

  const DQ_GAS float* rcur = gp(P.r[pi.rs]);
  const DQ_GAS float* ircur = gp(P.ir[pi.rs]);
  DQ_GAS float* rnext = gp(P.r[slot_next(pi.rs)]);
  DQ_GAS float* irnext = gp(P.ir[slot_next(pi.rs)]);
  uint8_t* ccodes = P.codes[pi.cb];
  void* cscales = P.scales[pi.cb];
  const uint8_t* acodes = P.codes[pi.acc];
  const void* ascales = P.scales[pi.acc];
  QCtx qc;
  qc.k6 = k6;
  qc.tab = tab_c;

  double aFc = 0.0, adF = 0.0, arel = 0.0, aqn = 0.0;
  bool uflow = false, zrow = false;
  const int64_t row0 = (int64_t)we.idx * P.rows_per_blk;
  const int64_t row1 = min(P.rows, row0 + P.rows_per_blk);
  const int nloop = (nch + 63) >> 6;
  // equal block factors for equal scale codes (NVFP4: equal tensor scales)
  const bool cq = compact && pi.stats && (FMT != NVFP4 || s_t == st->st_acc);
  const bool alt = pi.alt;

  // kept-Qhat r-step sums of the current row (the safeguard's other outcome)
  double Nk = 0.0, Dk = 0.0;
  // the kept Qhat's error, the relchg terms and the kept-Qhat r-step sums of the `count`
  // queued chunks of row i
  auto flush = [&](int64_t i, float r_, int count) {
    __builtin_amdgcn_wave_barrier();
    if (lane < count) {
      const uint32_t* e = queue + lane * QW;
      const int chq = (int)(e[0] & 0xFFFFu);
      const uint32_t scq = e[0] >> 16;
      uint32_t cw[4] = {e[1], code_words<FMT>() > 1 ? e[2] : 0u, code_words<FMT>() > 2 ? e[3] : 0u,
                        code_words<FMT>() > 3 ? e[4] : 0u};
      RawRow<DT> rq;
      rq.load(P.W, i, P.ld, 16 * chq);
      uint32_t kq[4] = {0u, 0u, 0u, 0u}, ksq = 0u;
      load_codes<FMT, L>(acodes, ascales, i, n, chq, g, kq, ksq);
      float w[16], cc[16], pq[16], pp[16];
      rq.unpack(w);
      if (CG) load16_global(cglob + 16 * (int64_t)chq, true, cc);
      else lds_load16(s_c4, nch, chq, cc);
      decode_grid<FMT>(cw, pq);
      decode_grid<FMT>(kq, pp);
      const float f = block_factor<FMT>(scq, tab_c);
      const float fp = block_factor<FMT>(ksq, tab_p);
      const float rfp = r_ * fp;
      float Fpl = 0.0f, rl = 0.0f, Nbk = 0.0f, Dbk = 0.0f;
      double Nbkd = 0.0, Dbkd = 0.0;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float ppc = pp[k] * cc[k];
        const float ep = fmaf(-rfp, ppc, w[k]);
        Fpl = fmaf(ep, ep, Fpl);
        const float df = pq[k] * f - pp[k] * fp;
        rl = fmaf(df, df, rl);
        if (alt) {   // the kept Qhat's r-step sums, as for the chunks computed inline
          if (A64) {
            Nbkd += exact_wq<FMT, DT>(w[k], ppc);
            Dbkd += exact_qq<FMT>(ppc);
          } else {
            Nbk = fmaf(w[k], ppc, Nbk);
            Dbk = fmaf(ppc, ppc, Dbk);
          }
        }
      }
      adF -= (double)Fpl;
      arel += (double)rl;
      if (alt) {
        if (A64) {
          Nk += (double)fp * Nbkd;
          Dk += ((double)fp * (double)fp) * Dbkd;
        } else {
          Nk += (double)fp * (double)Nbk;
          Dk += (double)(fp * fp) * (double)Dbk;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  for (int64_t i = row0 + wave; i < row1; i += nw) {
    const float r_ = rcur[i];
    const float ir_ = ircur[i];
    double Nrow = 0.0, Drow = 0.0;
    Nk = 0.0;
    Dk = 0.0;
    int qn = 0;   // queued chunks of this row (wave-uniform)
    for (int kk = 0; kk < nloop; ++kk) {
      const int chn = lane + 64 * kk;
      const bool valid = chn < nch;
      // Lanes past the row's end load and work on the row's first chunk: every load stays in
      // range, nothing needs zeroing or a branch, and none of their results is stored or summed.
      const int cl = valid ? chn : 0;
      RawRow<DT> raw;
      raw.load(P.W, i, P.ld, 16 * cl);
      uint32_t pk[4] = {0u, 0u, 0u, 0u}, ps = 0;
      if (!(pi.mode == MODE_INIT)) load_codes<FMT, L>(acodes, ascales, i, n, cl, g, pk, ps);
      float w[16];
      raw.unpack(w);
      float p[16];
      float Nb = 0.0f, Db = 0.0f;
      double Nbd = 0.0, Dbd = 0.0;
      float cc[16];
      float v[16];
      {
        float icc[16];
        if (CG) load16_global(icglob + 16 * (int64_t)cl, true, icc);
        else lds_load16(s_ic4, nch, cl, icc);
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = (w[k] * ir_) * icc[k];
      }
      Chunk ch;
      quantize_chunk<FMT, L>(v, qc, ch);
      // Every chunk is written, changed or not: skipping the unchanged ones (a few percent
      // change per iteration) leaves sparse 8-byte writes in partly written lines, and the
      // pass got slower (43.9 against 38.3 us on 4096 x 14336 NVFP4).
      if (valid) store_chunk<FMT, L>(ccodes, cscales, i, n, chn, g, ch);
      uflow |= ch.underflow && valid;
      const float f = ch.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) p[k] = ch.p[k];
      if (CG) load16_global(cglob + 16 * (int64_t)cl, true, cc);
      else lds_load16(s_c4, nch, cl, cc);
      const float rf = r_ * f;
      float Fl = 0.0f, ql = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float pc = p[k] * cc[k];
        const float e = fmaf(-rf, pc, w[k]);
        Fl = fmaf(e, e, Fl);
        if (A64) {
          Nbd = fma((double)w[k], (double)pc, Nbd);
          Dbd = fma((double)pc, (double)pc, Dbd);
        } else {
          Nb = fmaf(w[k], pc, Nb);
          Db = fmaf(pc, pc, Db);
        }
        ql = fmaf(p[k], p[k], ql);
      }
      float Fpl = 0.0f, rl = 0.0f;
      bool changed = false, queued = false;
      if (cq) {
#pragma unroll
        for (int w4 = 0; w4 < code_words<FMT>(); ++w4) changed |= ch.code[w4] != pk[w4];
        changed = valid && (changed || ch.scode != ps);
        const uint64_t mask = __ballot(changed);
        const int cnt = __popcll(mask);
        queued = qn + cnt <= kQueueLen;   // wave-uniform; a full queue falls back to inline
        if (queued && mask) {
          const int pos = qn + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
          if (changed) {
            uint32_t* e = queue + pos * QW;
            e[0] = (uint32_t)chn | (ch.scode << 16);
#pragma unroll
            for (int w4 = 0; w4 < code_words<FMT>(); ++w4) e[1 + w4] = ch.code[w4];
          }
          qn += cnt;
        }
      }
      // kept-Qhat r-step terms of this chunk: its own where they are computed inline (here),
      // the candidate's where the codes are unchanged (below), at the flush where queued
      double kN = 0.0, kD = 0.0;
      if (pi.stats && !queued) {
        float pp[16];
        decode_grid<FMT>(pk, pp);
        const float fp = block_factor<FMT>(ps, tab_p);
        const float rfp = r_ * fp;
        float Nbk = 0.0f, Dbk = 0.0f;
        double Nbkd = 0.0, Dbkd = 0.0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float ppc = pp[k] * cc[k];
          const float ep = fmaf(-rfp, ppc, w[k]);
          Fpl = fmaf(ep, ep, Fpl);
          // difference of the two dequantised values, each rounded to fp32 as the
          // values themselves are: exactly 0 where Qhat did not change
          const float df = p[k] * f - pp[k] * fp;
          rl = fmaf(df, df, rl);
          if (alt) {
            if (A64) {   // exact products, summed in fp64 as in the candidate's sums
              Nbkd += exact_wq<FMT, DT>(w[k], ppc);
              Dbkd += exact_qq<FMT>(ppc);
            } else {
              Nbk = fmaf(w[k], ppc, Nbk);
              Dbk = fmaf(ppc, ppc, Dbk);
            }
          }
        }
        if (A64) {
          kN = (double)fp * Nbkd;
          kD = ((double)fp * (double)fp) * Dbkd;
        } else {
          kN = (double)fp * (double)Nbk;
          kD = (double)(fp * fp) * (double)Dbk;
        }
      }
      if (valid) {
        aFc += (double)Fl;
        // queued chunks: the candidate's error now, the kept one's at the flush; unchanged
        // chunks under compaction add 0
        adF += queued ? (changed ? (double)Fl : 0.0) : (double)Fl - (double)Fpl;
        arel += (double)rl;
        aqn += (double)(f * f) * (double)ql;
        double cN, cD;
        if (A64) {
          cN = (double)f * Nbd;
          cD = ((double)f * (double)f) * Dbd;
        } else {
          cN = (double)f * (double)Nb;
          cD = (double)(f * f) * (double)Db;
        }
        Nrow += cN;
        Drow += cD;
        if (alt && !(queued && changed)) {
          Nk += queued ? cN : kN;
          Dk += queued ? cD : kD;
        }
      }
    }
    if (qn > 0) flush(i, r_, qn);   // wave-uniform
    if (pi.next) {
      // r-step of the next iteration from the whole row (fixed butterfly order in fp64), from
      // the candidate and, when a kept Qhat exists, from the kept one
      const double N = wave_sum(Nrow), D = wave_sum(Drow);
      double N2 = 0.0, D2 = 0.0;
      if (alt) {
        N2 = wave_sum(Nk);
        D2 = wave_sum(Dk);
      }
      if (lane == 0) {
        float x = __builtin_nanf(""), rnew = r_;
        if (!(P.steps & 1)) {
          // row scales frozen: r is kept and no closed form is recorded
        } else if (D > 0.0) {
          x = (float)(N / D);
          rnew = project<FMT>(x);
        } else {
          zrow = true;
        }
        rnext[i] = rnew;
        irnext[i] = 1.0f / rnew;
        if (P.r_trace) gp(P.r_trace)[(int64_t)pi.tr * P.rows + i] = x;
        if (alt) {
          // a row with D = 0 here is flagged by the finalize if this outcome is taken
          float x2 = __builtin_nanf(""), r2 = r_;
          if (!(P.steps & 1)) {
          } else if (D2 > 0.0) {
            x2 = (float)(N2 / D2);
            r2 = project<FMT>(x2);
          } else {
            atomicOr(P.altz, 1u);
          }
          gp(P.r[slot_alt(pi.rs)])[i] = r2;
          gp(P.ir[slot_alt(pi.rs)])[i] = 1.0f / r2;
          if (P.r_trace) gp(P.x_alt)[i] = x2;
        }
      }
    }
  }

  {
    const double a0 = wave_sum(aFc), a1 = wave_sum(adF), a2 = wave_sum(arel), a3 = wave_sum(aqn);
    if (lane == 0) { redw[wave][0] = a0; redw[wave][1] = a1; redw[wave][2] = a2; redw[wave][3] = a3; }
  }
  const bool anyu = __syncthreads_or(uflow);
  const bool anyz = __syncthreads_or(zrow);
  if (t == 0) {
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    for (int k = 0; k < nw; ++k) { s0 += redw[k][0]; s1 += redw[k][1]; s2 += redw[k][2]; s3 += redw[k][3]; }
    DQ_GAS double* o = gp(P.swp + 4 * (size_t)we.idx);
    o[0] = s0; o[1] = s1; o[2] = s2; o[3] = s3;
    const uint32_t fl = (anyu ? 8u : 0u) | (anyz ? 2u : 0u);
    if (fl) atomicOr(P.flags, fl);
  }
}

// ---------------------------------------------------------------- column pass
// Workgroup = 8 waves on one strip of 64 chunks (1024 columns) and one range of rows; wave
// w takes rows w, w+8, ... of the range.  The waves' accumulators are combined in LDS in
// fixed wave order and written as this range's partial.  fp32 accumulation keeps a wave
// within 128 VGPRs (two workgroups per CU); INT4/INT8's fp64 accumulators need the wider
// budget.
template <int FMT, int DT, int L>
__device__ __forceinline__ void colpass_body(const ProbDev* __restrict__ probs,
                                             const WgEntry* __restrict__ table, int sw,
                                             const int32_t* __restrict__ live) {
  const int32_t nlive = *gp(live);
  const WgEntry we = table[blockIdx.x];
  if (nlive == 0) return;
  const ProbDev& P = probs[we.prob];
  const State* st = state_slots(live, we.prob) + (sw & 1);
  if (st->mode == MODE_DONE) return;
  const PassInfo pi(st, P.iters);
  if (!pi.next) return;
  constexpr bool A64 = grouped_int<FMT>();
  typedef typename std::conditional<A64, double, float>::type acc_t;
  constexpr int NQ = (FMT == NVFP4) ? 3 : 2;
  const int g = L * 16;
  const int64_t n = P.cols;
  const int nch = (int)(n >> 4);
  const int strip = we.idx % P.nstrips, rr = we.idx / P.nstrips;
  const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int chn = strip * 64 + lane;
  // lanes past the matrix's last chunk work on its first chunk; their sums are never stored
  const int chl = chn < nch ? chn : 0;
  const int j0 = 16 * chl;
  // The outcome of the safeguard is the same in every wave and workgroup: a kept candidate
  // gives the sums over its codes with the r-step from it, a rejected one the sums over the
  // kept Qhat with the r-step from that.  Each wave requests the row pass's dF partials and,
  // alongside, its first rows with the candidate's codes (kept on most sweeps); it learns the
  // outcome before its first products and reloads those rows' codes and r after a rejection.
  const bool decide = pi.stats;
  int qb = pi.cb, rslot = slot_next(pi.rs);
  const uint8_t* qcodes = P.codes[qb];
  const void* qscales = P.scales[qb];
  const DQ_GAS float* rnew = gp(P.r[rslot]);
  const DQ_GAS float* irnew = gp(P.ir[rslot]);
  __shared__ NvTab tabs[2];   // [0]: the candidate's tensor scale, [1]: the kept Qhat's
  const NvTab* tab = &tabs[0];
  if (FMT == NVFP4) {
    build_nvtab(tabs[0], st->st_cur);
    if (decide) build_nvtab(tabs[1], st->st_acc);
    __syncthreads();
  }
  // requested after the barrier, which would otherwise wait for them
  double dpart = 0.0;
  if (decide) dpart = rowpass_dF_part(P);
  bool pending = decide;   // wave-uniform: the outcome is not applied yet

  acc_t cN[16], cD[16];
  float cM[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) { cN[k] = (acc_t)0; cD[k] = (acc_t)0; cM[k] = 0.0f; }
  const int64_t row0 = (int64_t)rr * P.rows_per_range;
  const int64_t row1 = min(P.rows, row0 + P.rows_per_range);
  constexpr int U = A64 ? 1 : 2;   // rows in flight per wave
  for (int64_t i0 = row0 + wave; i0 < row1; i0 += 8 * U) {
    RawRow<DT> raw[U];
    uint32_t cw[U][4], sc[U];
    float rr_[U], irn[U];
    int64_t ix[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // rows past the range load the range's last row (not summed): every row's loads are
      // issued on one path, so the compiler's wait before a row's products leaves the later
      // rows' loads in flight
      ix[u] = i0 + 8 * u < row1 ? i0 + 8 * u : row1 - 1;
      raw[u].load(P.W, ix[u], P.ld, j0);
      load_codes<FMT, L>(qcodes, qscales, ix[u], n, chl, g, cw[u], sc[u]);
      rr_[u] = rnew[ix[u]];
      irn[u] = (FMT == NVFP4) ? irnew[ix[u]] : 0.0f;
    }
    if (pending) {   // first trip of the wave
      pending = false;
      if (!(rowpass_dF_sum(dpart) <= 0.0)) {
        qb = pi.acc;
        rslot = slot_alt(pi.rs);
        qcodes = P.codes[qb];
        qscales = P.scales[qb];
        rnew = gp(P.r[rslot]);
        irnew = gp(P.ir[rslot]);
        tab = &tabs[1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          load_codes<FMT, L>(qcodes, qscales, ix[u], n, chl, g, cw[u], sc[u]);
          rr_[u] = rnew[ix[u]];
          irn[u] = (FMT == NVFP4) ? irnew[ix[u]] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + 8 * u >= row1) break;
      float w[16], p[16];
      // keep the scale code's use (and so the wait for it, which in order covers this row's
      // other loads) here, after the previous row's products
      asm volatile("" : "+v"(sc[u]));
      raw[u].unpack(w);
      decode_grid<FMT>(cw[u], p);
      const float f = block_factor<FMT>(sc[u], tab);
      const float rf = rr_[u] * f;
      const float rf2 = rf * rf;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (A64) {   // INT4/INT8: rf = r * s and rf * p are exact in fp32 (bf16 x bf16 x at
                     // most 7 bits); products exact in fp64
          cN[k] = fma((double)rf, (double)w[k] * (double)p[k], (double)cN[k]);
          const double rp = (double)(rf * p[k]);
          cD[k] = fma(rp, rp, (double)cD[k]);
        } else {
          cN[k] = fmaf(rf, w[k] * p[k], (float)cN[k]);
          cD[k] = fmaf(rf2, p[k] * p[k], (float)cD[k]);
        }
        if (FMT == NVFP4) cM[k] = fmaxf(cM[k], fabsf(w[k] * irn[u]));
      }
    }
  }
  // combine the 8 waves: one quantity per round, every wave stores its 16 values per lane in
  // LDS, then thread (lane chunk l, quad kq) sums the 8 waves in wave order and stores 4
  // consecutive columns, so a wave writes 1 KB of the partial contiguously
  typedef acc_t vec4 __attribute__((ext_vector_type(4)));
  extern __shared__ float xs[];
  vec4* xa = (vec4*)xs;                     // [8 waves][64 chunks][4 quads]
  DQ_GAS acc_t* base = gp((acc_t*)P.colP + (size_t)rr * NQ * (size_t)n + 16 * (size_t)strip * 64);
  const int ol = t >> 2, oq = t & 3;        // output chunk (0..127, only < 64 used) and quad
  for (int qi = 0; qi < NQ; ++qi) {
    if (qi) __syncthreads();
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      vec4 v;
      if (qi == 0) v = vec4{cN[4 * kq], cN[4 * kq + 1], cN[4 * kq + 2], cN[4 * kq + 3]};
      else if (qi == 1) v = vec4{cD[4 * kq], cD[4 * kq + 1], cD[4 * kq + 2], cD[4 * kq + 3]};
      else v = vec4{(acc_t)cM[4 * kq], (acc_t)cM[4 * kq + 1], (acc_t)cM[4 * kq + 2], (acc_t)cM[4 * kq + 3]};
      xa[(wave * 64 + lane) * 4 + kq] = v;
    }
    __syncthreads();
    if (ol < 64 && strip * 64 + ol < nch) {
      vec4 a = xa[ol * 4 + oq];
#pragma unroll
      for (int w = 1; w < 8; ++w) {
        const vec4 o = xa[(w * 64 + ol) * 4 + oq];
        if (qi < 2) a += o;
        else { a.x = fmaxf(a.x, o.x); a.y = fmaxf(a.y, o.y); a.z = fmaxf(a.z, o.z); a.w = fmaxf(a.w, o.w); }
      }
      *(DQ_GAS vec4*)(base + (size_t)qi * n + 16 * ol + 4 * oq) = a;
    }
  }
}

template <int FMT, int DT, int L>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_colpass(
    const ProbDev* __restrict__ probs, const WgEntry* __restrict__ table, int sw,
    const int32_t* __restrict__ live) {
  colpass_body<FMT, DT, L>(probs, table, sw, live);
}

template <int FMT, int DT, int L>
__global__ __launch_bounds__(512) void k_colpass_wide(const ProbDev* __restrict__ probs,
                                                      const WgEntry* __restrict__ table, int sw,
                                                      const int32_t* __restrict__ live) {
  colpass_body<FMT, DT, L>(probs, table, sw, live);
}

// ---------------------------------------------------------------- finalize
// Column reduction of the row-range partials, c-step projection and the per-workgroup amax
// for the next NVFP4 tensor scale.  A workgroup covers 64 columns with 4 threads per column;
// thread part p sums ranges p, p+4, ... (sixteen loads in flight), and the four parts are
// added in part order.  One more workgroup per problem takes the safeguard decision from
// the row pass's partials (written by an earlier kernel) and writes the state of the next
// sweep, alongside the column workgroups; the amax partials it does not wait for are
// reduced by the next row pass.
template <int FMT>
__global__ __launch_bounds__(256) void k_finalize(const ProbDev* __restrict__ probs,
                                                  const WgEntry* __restrict__ table, int sw,
                                                  int32_t* __restrict__ live) {
  // Once every problem is DONE the state slots are no longer read (the outputs kernel reads
  // the slot of the last sweep a problem ran, recorded in its state), so nothing is carried.
  const int32_t nlive = *gp(live);
  const WgEntry we = table[blockIdx.x];
  if (nlive == 0) return;
  const ProbDev& P = probs[we.prob];
  const State* st = state_slots(live, we.prob) + (sw & 1);
  State* sn = state_slots(live, we.prob) + ((sw + 1) & 1);
  const int mode = st->mode;
  // workgroups 0 .. fin_wgs-1 reduce columns; the one with index fin_wgs takes the
  // safeguard decision (it needs only the row pass's partials, so it runs alongside)
  const bool decider = (we.idx == P.fin_wgs);
  if (mode == MODE_DONE) {   // carry a finished state forward to the next sweep's slot
    if (decider && threadIdx.x == 0) *sn = *st;
    return;
  }
  const int it = (mode == MODE_INIT) ? 0 : st->it_done + 1;
  const bool next = (it < P.iters);
  const int cs = st->cs;
  const int64_t n = P.cols;

  __shared__ double sred[2][4][64];   // [quantity][part][column]
  __shared__ float smax[4][64];
  __shared__ float wmax[1];
  __shared__ double tr[4 * 256];

  const int t = threadIdx.x, col = t & 63, part = t >> 6;
  bool zcol = false;
  if (!decider) {
    if (next) {
      constexpr int NQ = (FMT == NVFP4) ? 3 : 2;
      typedef typename std::conditional<grouped_int<FMT>(), double, float>::type acc_t;
      const int64_t j = (int64_t)we.idx * 64 + col;
      double N = 0.0, D = 0.0;
      float M = 0.0f;
      if (j < n) {
        const int S = P.rranges;
        const DQ_GAS acc_t* b = gp((const acc_t*)P.colP + j);
        const size_t stride = (size_t)NQ * (size_t)n;
        for (int b0 = 0; b0 < S; b0 += 64) {
          acc_t vn[16], vd[16], vm[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {   // clamped index: every load is issued, unused ones dropped
            const int sr = min(b0 + part + 4 * u, S - 1);
            const DQ_GAS acc_t* q = b + (size_t)sr * stride;
            vn[u] = q[0];
            vd[u] = q[n];
            if (FMT == NVFP4) vm[u] = q[2 * n];
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            if (b0 + part + 4 * u < S) {
              N += (double)vn[u];
              D += (double)vd[u];
              if (FMT == NVFP4) M = fmaxf(M, (float)vm[u]);
            }
          }
        }
      }
      sred[0][part][col] = N;
      sred[1][part][col] = D;
      smax[part][col] = M;
      __syncthreads();
      float am = 0.0f;
      if (part == 0 && j < n) {
        N = ((sred[0][0][col] + sred[0][1][col]) + sred[0][2][col]) + sred[0][3][col];
        D = ((sred[1][0][col] + sred[1][1][col]) + sred[1][2][col]) + sred[1][3][col];
        M = fmaxf(fmaxf(smax[0][col], smax[1][col]), fmaxf(smax[2][col], smax[3][col]));
        float x = __builtin_nanf("");
        float cnew;
        if (!(P.steps & 2)) {   // column scales frozen: c is kept
          cnew = gp(P.c[cs])[j];
        } else if (D > 0.0) {
          x = (float)(N / D);
          cnew = project<FMT>(x);
        } else {
          cnew = gp(P.c[cs])[j];
          zcol = true;
        }
        const float icn = 1.0f / cnew;
        gp(P.c[1 - cs])[j] = cnew;
        gp(P.ic[1 - cs])[j] = icn;
        if (P.c_trace) gp(P.c_trace)[(int64_t)it * n + j] = x;
        if (FMT == NVFP4) am = M * icn;
      }
      if (FMT == NVFP4 && part == 0) {
        am = wave_max(am);
        if (t == 0) wmax[0] = am;
      }
    }
    zcol = __syncthreads_or(zcol);
    if (t == 0) {
      if (next && FMT == NVFP4) gp(P.fwp)[we.idx] = wmax[0];
      if (zcol) atomicOr(P.flags, 4u);
    }
    return;
  }

  // decision: dF in the column pass's order (the same outcome there and here); after a
  // rejection the next sweep takes the kept-Qhat r-step (its slot, its trace row, its flag)
  // statistics: fixed-order reductions of the row pass's partials, strided per thread, then
  // a pairwise tree over the 256 threads (F(Qc), relchg numerator, ||Qc||^2; dF as above)
  double f[4] = {0.0, 0.0, 0.0, 0.0};
  for (int s = t; s < P.rowblocks; s += 256) {
    const DQ_GAS double* o = gp(P.swp + 4 * (size_t)s);
    f[0] += o[0]; f[2] += o[2]; f[3] += o[3];
  }
  const double dF = rowpass_dF(P);
  if (mode == MODE_NORMAL && next && !(dF <= 0.0) && P.r_trace) {
    const int64_t m = P.rows;
    for (int64_t i = t; i < m; i += 256) gp(P.r_trace)[(int64_t)it * m + i] = gp(P.x_alt)[i];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) tr[q * 256 + t] = f[q];
  for (int w = 128; w >= 1; w >>= 1) {
    __syncthreads();
    if (t < w) {
#pragma unroll
      for (int q = 0; q < 4; ++q) tr[q * 256 + t] += tr[q * 256 + t + w];
    }
  }
  __syncthreads();
  if (t != 0) return;
  const double Fc = tr[0], rel = tr[512], qn = tr[768];
  const uint32_t az = *gp(P.altz);
  *gp(P.altz) = 0u;   // read by this decision only; the next row pass runs after it

  State ns = *st;
  const double nW = st->normW2;
  bool accepted = true;
  double relv = 0.0;
  if (mode == MODE_INIT) {
    if (P.nmse) P.nmse[0] = nW > 0.0 ? Fc / nW : 0.0;
    if (P.relchg) P.relchg[0] = 0.0;
    ns.acc = 0;
    ns.qn2_acc = qn;
    ns.st_acc = st->st_cur;
    ns.it_done = 0;
  } else if (mode == MODE_NORMAL) {
    accepted = (dF <= 0.0);
    if (accepted) {
      relv = st->qn2_acc > 0.0 ? sqrt(rel) / sqrt(st->qn2_acc) : 0.0;
      if (P.nmse) P.nmse[it] = nW > 0.0 ? Fc / nW : 0.0;
      ns.acc = 1 - st->acc;
      ns.qn2_acc = qn;
      ns.st_acc = st->st_cur;
    } else {
      ns.rejected += 1;
      if (P.nmse) P.nmse[it] = nW > 0.0 ? (Fc - dF) / nW : 0.0;
      if (az && next) atomicOr(P.flags, 2u);   // a row whose kept Qhat is all zero
    }
    if (P.relchg) P.relchg[it] = relv;
    ns.it_done = it;
  }
  const bool stop = it >= P.iters || (mode == MODE_NORMAL && P.tol > 0.0f && relv <= (double)P.tol);
  ns.needs_ts = 0;
  if (stop) {
    ns.mode = MODE_DONE;
    ns.sweeps += 1;
    *sn = ns;
    atomicSub(live, 1);   // after the state: a later sweep that sees 0 reads no state
    return;
  }
  // the r and c of the outcome taken (r moved into place above after a rejection); the kept
  // Qhat stays in its buffer after a rejection
  ns.rs = accepted ? slot_next(st->rs) : slot_alt(st->rs);
  ns.cs = 1 - st->cs;
  ns.needs_ts = (FMT == NVFP4) ? 1 : 0;   // from this finalize's amax partials
  ns.mode = MODE_NORMAL;
  ns.sweeps += 1;
  *sn = ns;
}

// ---------------------------------------------------------------- outputs
// After the queued sweeps: each problem's final r, c, NVFP4 tensor scale and, when its kept
// Qhat is in the second code buffer, its codes and block scales go to the caller's buffers,
// and its report to the caller's device report.  The final state is the slot whose mode is
// DONE (the decision that finished a problem wrote it; later sweeps that still ran for other
// problems copied it to the other slot too).  Grid: x = workgroups per problem, y = problem.
__device__ __forceinline__ void copy_bytes(uint8_t* dst, const uint8_t* src, int64_t bytes,
                                           int64_t tid, int64_t nthr) {
  const int64_t n16 = bytes >> 4;   // both buffers are 16-byte aligned
  const DQ_GAS u32x4* s4 = gp((const u32x4*)src);
  DQ_GAS u32x4* d4 = gp((u32x4*)dst);
  int64_t k = tid;
  for (; k + 3 * nthr < n16; k += 4 * nthr) {   // four loads in flight per thread
    const u32x4 v0 = s4[k], v1 = s4[k + nthr], v2 = s4[k + 2 * nthr], v3 = s4[k + 3 * nthr];
    d4[k] = v0;
    d4[k + nthr] = v1;
    d4[k + 2 * nthr] = v2;
    d4[k + 3 * nthr] = v3;
  }
  for (; k < n16; k += nthr) d4[k] = s4[k];
  for (int64_t b = 16 * n16 + tid; b < bytes; b += nthr) gp(dst)[b] = gp(src)[b];
}

__device__ __forceinline__ void write_report(ReportDev* rep, int32_t iters_run, int32_t rejected,
                                             uint32_t flags, int32_t sweeps) {
  DQ_GAS int32_t* q = gp((int32_t*)rep);   // 4-byte aligned: four word stores
  q[0] = iters_run;
  q[1] = rejected;
  q[2] = (int32_t)flags;
  q[3] = sweeps;
}

__global__ __launch_bounds__(256) void k_outputs(const ProbDev* __restrict__ probs,
                                                 int code_bits, int scale_bytes, int g) {
  const ProbDev& P = probs[blockIdx.y];
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  if (!P.st) {   // an empty problem: all iterations "run", nothing else to write
    if (tid == 0 && P.report) write_report(P.report, P.iters, 0, 0u, 0);
    return;
  }
  const bool d0 = P.st[0].mode == MODE_DONE, d1 = P.st[1].mode == MODE_DONE;
  const State s = P.st[(d0 || !d1) ? 0 : 1];
  if (tid == 0 && P.report) {
    const uint32_t fl = *gp(P.flags) | ((d0 || d1) ? 0u : kFlagUnfinished);
    write_report(P.report, s.it_done, s.rejected, fl, s.sweeps);
  }
  for (int64_t i = tid; i < P.rows; i += nthr) gp(P.r_out)[i] = gp(P.r[s.rs])[i];
  for (int64_t j = tid; j < P.cols; j += nthr) gp(P.c_out)[j] = gp(P.c[s.cs])[j];
  if (tid == 0 && P.ts_out) *gp(P.ts_out) = s.st_acc;
  if (s.acc == 1) {
    const int64_t n = P.rows * P.cols;
    copy_bytes(P.codes[0], P.codes[1], n * code_bits / 8, tid, nthr);
    copy_bytes((uint8_t*)P.scales[0], (const uint8_t*)P.scales[1], n / g * scale_bytes, tid, nthr);
  }
}

// ---------------------------------------------------------------- standalone quantiser
// MODEV = 0: weights, v = (W * (1/r_i)) * (1/c_j);  MODEV = 1: activations, v = x * c_j.
// Pass 1 (NVFP4 only): per-workgroup amax of v.  Rounding is monotone, so the amax of a
// column is fl(max_i |inner_ij| * s_j) with inner = fl(x * (1/r_i)) (weights) or x
// (activations) and s_j = 1/c_j or c_j: each thread keeps the running column maxima of the
// eight or four columns of one 16-byte vector over a range of rows and scales them once.
// Workgroup = 256 vectors x a range of rows; blockIdx.x = strip + nstrips * range.
template <int DT, int MODEV>
__global__ __launch_bounds__(256) void k_qamax(const void* __restrict__ X, int64_t rows,
                                               int64_t cols, int64_t ld,
                                               const float* __restrict__ r,
                                               const float* __restrict__ c,
                                               float* __restrict__ part, int nstrips,
                                               int rows_per_range) {
  constexpr int VEC = (DT == 1) ? 8 : 4;   // elements per 16-byte load
  constexpr int U = 16;                     // loads in flight per thread (a 16-row range: one round)
  const int strip = (int)(blockIdx.x % nstrips), rr = (int)(blockIdx.x / nstrips);
  const int64_t nv = cols / VEC;
  const int64_t v = (int64_t)strip * 256 + threadIdx.x;
  const int64_t r0 = (int64_t)rr * rows_per_range, r1 = min(rows, r0 + rows_per_range);
  const int64_t rowbytes = ld * (DT == 1 ? 2 : 4);
  float cm[VEC], cj[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) { cm[k] = 0.0f; cj[k] = 1.0f; }
  // this thread's column scales, requested before the rows so they arrive under them
  if (v < nv && c) {
#pragma unroll
    for (int k = 0; k < VEC; ++k) cj[k] = gp(c)[v * VEC + k];
  }
  if (v < nv) {
    for (int64_t i0 = r0; i0 < r1; i0 += U) {
      u32x4 u[U];
      float ir[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int64_t i = min(i0 + q, r1 - 1);   // clamped: a repeated row does not change a max
        u[q] = gp((const u32x4*)((const char*)X + i * rowbytes))[v];
        ir[q] = (MODEV == 0 && r) ? 1.0f / gp(r)[i] : 1.0f;
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const uint32_t uu[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
        float w[VEC];
        if (DT == 1) {
#pragma unroll
          for (int k = 0; k < 4; ++k) { w[2 * k] = u2f(uu[k] << 16); w[2 * k + 1] = u2f(uu[k] & 0xFFFF0000u); }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) w[k] = u2f(uu[k]);
        }
#pragma unroll
        for (int k = 0; k < VEC; ++k) cm[k] = fmaxf(cm[k], MODEV == 0 ? fabsf(w[k] * ir[q]) : fabsf(w[k]));
      }
    }
  }
  float m = 0.0f;
  if (v < nv) {
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      float sj = 1.0f;
      if (c) sj = (MODEV == 0) ? 1.0f / cj[k] : fabsf(cj[k]);
      m = fmaxf(m, (MODEV == 0) ? fabsf(cm[k] * sj) : cm[k] * sj);
    }
  }
  m = wave_max(m);
  __shared__ float sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) gp(part)[blockIdx.x] = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
}

// Pass 2: quantise; workgroup = H row slots x LPR lanes, one chunk per lane, looping over
// row groups so the tensor-scale table is built once per workgroup.  A launch covers chunks
// lbeg .. lbeg + LPR - 1 of every row (rows wider than 1024 chunks take several launches).
template <int FMT, int DT, int L, int MODEV>
__global__ __launch_bounds__(1024) void k_quant(const void* __restrict__ X, int64_t rows,
                                                int64_t cols, int64_t ld,
                                                const float* __restrict__ r,
                                                const float* __restrict__ c, uint8_t* codes,
                                                void* scales, float* tensor_scale,
                                                const float* __restrict__ part, int nparts,
                                                int lpr, int H, int lbeg) {
  __shared__ NvTab tab;
  __shared__ float sA;
  QCtx qc;
  qc.k6 = 0.0f;
  qc.tab = &tab;
  if (FMT == NVFP4) {
    __shared__ float smax[16];
    float a = 0.0f;
    for (int k = threadIdx.x; k < nparts; k += blockDim.x) a = fmaxf(a, gp(part)[k]);
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
      float A = 0.0f;
      for (int k = 0; k < (int)(blockDim.x >> 6); ++k) A = fmaxf(A, smax[k]);
      sA = A;
    }
    __syncthreads();
    float s_t, k6;
    bool tiny;
    nv_tensor_terms(sA, s_t, k6, tiny);
    qc.k6 = k6;
    build_nvtab(tab, s_t);
    if (blockIdx.x == 0 && threadIdx.x == 0) *gp(tensor_scale) = s_t;
    __syncthreads();
  }
  const int t = threadIdx.x;
  const int h = t / lpr, l = lbeg + (t - h * lpr);   // this lane's chunk of the row
  const bool lane_ok = l < (int)(cols >> 4);
  const int j0 = lane_ok ? l * 16 : 0;
  float cv[16];   // c (or its reciprocal for weights) of this lane's columns, for every row
  if (lane_ok && c) {
    load16_global(c + j0, ((uintptr_t)c & 15u) == 0, cv);
    if (MODEV == 0) {
#pragma unroll
      for (int k = 0; k < 16; ++k) cv[k] = 1.0f / cv[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) cv[k] = 1.0f;
  }
  // row groups of H rows, strided over the grid
  for (int64_t i = (int64_t)blockIdx.x * H + h; i - h < rows; i += (int64_t)gridDim.x * H) {
    const bool act = lane_ok && i < rows;
    float w[16], v[16];
    RawRow<DT> raw;
    if (act) raw.load(X, i, ld, j0); else raw.zero();
    raw.unpack(w);
    if (MODEV == 0) {
      const float ir = (act && r) ? 1.0f / gp(r)[i] : 1.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = (w[k] * ir) * cv[k];
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = c ? w[k] * cv[k] : w[k];
    }
    Chunk ch;
    quantize_chunk<FMT, L>(v, qc, ch);
    if (act) store_chunk<FMT, L>(codes, scales, i, cols, l, L * 16, ch);
  }
}

// ---------------------------------------------------------------- multi-output activations
// Several projections that read the same activations (q/k/v, gate/up), each with its own
// column scales: X is read once per pass and every output gets exactly what the
// single-output activation quantiser would produce for its c.
constexpr int kMaxMulti = 8;
struct MultiOut {
  const float* c[kMaxMulti];   // column scales of each output, or null (no rescaling)
  uint8_t* codes[kMaxMulti];
  void* scales[kMaxMulti];
  float* ts[kMaxMulti];
  int count;
};

// NVFP4 amax pre-pass: the column maxima of |x| are shared; each output scales them by its
// own |c| (rounding is monotone) and keeps one partial per workgroup: part[k][blockIdx.x].
template <int DT>
__global__ __launch_bounds__(256) void k_qamax_multi(const void* __restrict__ X, int64_t rows,
                                                     int64_t cols, int64_t ld, MultiOut mo,
                                                     float* __restrict__ part, int nstrips,
                                                     int rows_per_range) {
  constexpr int VEC = (DT == 1) ? 8 : 4;
  constexpr int U = 4;
  const int strip = (int)(blockIdx.x % nstrips), rr = (int)(blockIdx.x / nstrips);
  const int64_t nv = cols / VEC;
  const int64_t v = (int64_t)strip * 256 + threadIdx.x;
  const int64_t r0 = (int64_t)rr * rows_per_range, r1 = min(rows, r0 + rows_per_range);
  const int64_t rowbytes = ld * (DT == 1 ? 2 : 4);
  // every output's |c| of this lane's columns, requested before the rows stream in so the
  // loads complete under them
  float sj[kMaxMulti][VEC];
#pragma unroll
  for (int o = 0; o < kMaxMulti; ++o) {
    if (o < mo.count && mo.c[o] && v < nv && (((uintptr_t)mo.c[o] & 15u) == 0)) {
#pragma unroll
      for (int h = 0; h < VEC / 4; ++h) {
        const f32x4 q = gp((const f32x4*)(mo.c[o] + v * VEC))[h];
        sj[o][4 * h] = fabsf(q.x); sj[o][4 * h + 1] = fabsf(q.y);
        sj[o][4 * h + 2] = fabsf(q.z); sj[o][4 * h + 3] = fabsf(q.w);
      }
    } else {
#pragma unroll
      for (int k = 0; k < VEC; ++k)
        sj[o][k] = (o < mo.count && mo.c[o] && v < nv) ? fabsf(gp(mo.c[o])[v * VEC + k]) : 1.0f;
    }
  }
  float cm[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) cm[k] = 0.0f;
  if (v < nv) {
    for (int64_t i0 = r0; i0 < r1; i0 += U) {
      u32x4 u[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int64_t i = min(i0 + q, r1 - 1);
        u[q] = gp((const u32x4*)((const char*)X + i * rowbytes))[v];
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const uint32_t uu[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
        float w[VEC];
        if (DT == 1) {
#pragma unroll
          for (int k = 0; k < 4; ++k) { w[2 * k] = u2f(uu[k] << 16); w[2 * k + 1] = u2f(uu[k] & 0xFFFF0000u); }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) w[k] = u2f(uu[k]);
        }
#pragma unroll
        for (int k = 0; k < VEC; ++k) cm[k] = fmaxf(cm[k], fabsf(w[k]));
      }
    }
  }
  __shared__ float sm[kMaxMulti][4];
  // unrolled with constant indices so the pointer table stays in kernel-argument registers
#pragma unroll
  for (int o = 0; o < kMaxMulti; ++o) {
    if (o >= mo.count) break;
    float m = 0.0f;
    if (v < nv) {
#pragma unroll
      for (int k = 0; k < VEC; ++k) m = fmaxf(m, cm[k] * sj[o][k]);
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) sm[o][threadIdx.x >> 6] = m;
  }
  __syncthreads();
  if (threadIdx.x < (unsigned)mo.count) {
    const int o = threadIdx.x;
    gp(part)[(size_t)o * gridDim.x + blockIdx.x] =
        fmaxf(fmaxf(sm[o][0], sm[o][1]), fmaxf(sm[o][2], sm[o][3]));
  }
}

// c_lds: every output's c sits in dynamic LDS (count * cols floats, chunk-interleaved as in
// the row pass: float4 q of chunk ch of output o at (4 o + q) * nch + ch), so each row reads
// it from LDS instead of reloading it from memory; otherwise it is read from memory per row.
template <int FMT, int DT, int L>
__global__ __launch_bounds__(1024) void k_quant_multi(const void* __restrict__ X, int64_t rows,
                                                      int64_t cols, int64_t ld, MultiOut mo,
                                                      const float* __restrict__ part, int nparts,
                                                      int lpr, int H, int c_lds, int lbeg) {
  __shared__ NvTab tabs[kMaxMulti];
  __shared__ float sk6[kMaxMulti];
  extern __shared__ f32x4 cq[];
  const int nch = (int)(cols >> 4);
  if (c_lds) {
    for (int e = threadIdx.x; e < mo.count * nch; e += blockDim.x) {
      const int o = e / nch, ch = e - o * nch;
      float cv[16];
      if (mo.c[o]) load16_global(mo.c[o] + 16 * ch, ((uintptr_t)mo.c[o] & 15u) == 0, cv);
      else {
#pragma unroll
        for (int k = 0; k < 16; ++k) cv[k] = 1.0f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        cq[(4 * o + q) * nch + ch] = f32x4{cv[4 * q], cv[4 * q + 1], cv[4 * q + 2], cv[4 * q + 3]};
    }
    __syncthreads();
  }
  if (FMT == NVFP4) {
    // every output's partial maxima are requested together, then reduced and turned into
    // tables in one round (one round of load latency for all outputs, not one per output)
    __shared__ float smax[kMaxMulti][16];
    float a[kMaxMulti];
#pragma unroll
    for (int o = 0; o < kMaxMulti; ++o) a[o] = 0.0f;
    for (int k = threadIdx.x; k < nparts; k += blockDim.x) {
#pragma unroll
      for (int o = 0; o < kMaxMulti; ++o)
        if (o < mo.count) a[o] = fmaxf(a[o], gp(part)[(size_t)o * nparts + k]);
    }
#pragma unroll
    for (int o = 0; o < kMaxMulti; ++o) {
      if (o >= mo.count) break;
      const float w = wave_max(a[o]);
      if ((threadIdx.x & 63) == 0) smax[o][threadIdx.x >> 6] = w;
    }
    __syncthreads();
#pragma unroll
    for (int o = 0; o < kMaxMulti; ++o) {
      if (o >= mo.count) break;
      float A = 0.0f;
      for (int k = 0; k < (int)(blockDim.x >> 6); ++k) A = fmaxf(A, smax[o][k]);
      float s_t, k6;
      bool tiny;
      nv_tensor_terms(A, s_t, k6, tiny);
      build_nvtab(tabs[o], s_t);
      if (threadIdx.x == 0) sk6[o] = k6;
      if (blockIdx.x == 0 && threadIdx.x == 0) *gp(mo.ts[o]) = s_t;
    }
    __syncthreads();
  }
  const int t = threadIdx.x;
  const int h = t / lpr, l = lbeg + (t - h * lpr);   // this lane's chunk of the row
  const bool lane_ok = l < nch;
  const int j0 = lane_ok ? l * 16 : 0;
  for (int64_t i = (int64_t)blockIdx.x * H + h; i - h < rows; i += (int64_t)gridDim.x * H) {
    const bool act = lane_ok && i < rows;
    float w[16];
    RawRow<DT> raw;
    if (act) raw.load(X, i, ld, j0); else raw.zero();
    raw.unpack(w);
#pragma unroll
    for (int o = 0; o < kMaxMulti; ++o) {
      if (o >= mo.count) break;
      float v[16];
      if (c_lds && mo.c[o]) {
        float cv[16];
        lds_load16(cq + 4 * o * nch, nch, lane_ok ? l : 0, cv);
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = w[k] * cv[k];
      } else if (mo.c[o]) {
        float cv[16];
        load16_global(mo.c[o] + j0, ((uintptr_t)mo.c[o] & 15u) == 0, cv);
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = w[k] * cv[k];
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = w[k];
      }
      QCtx qc;
      qc.k6 = (FMT == NVFP4) ? sk6[o] : 0.0f;
      qc.tab = &tabs[o];
      Chunk ch;
      quantize_chunk<FMT, L>(v, qc, ch);
      if (act) store_chunk<FMT, L>(mo.codes[o], mo.scales[o], i, cols, l, L * 16, ch);
    }
  }
}

// ---------------------------------------------------------------- dequantise
template <int FMT, int L>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes,
                                                 const void* __restrict__ scales,
                                                 const float* __restrict__ tensor_scale,
                                                 int64_t rows, int64_t cols,
                                                 const float* __restrict__ r,
                                                 const float* __restrict__ c,
                                                 float* __restrict__ out) {
  __shared__ NvTab tab;
  if (FMT == NVFP4) {
    build_nvtab(tab, *tensor_scale);
    __syncthreads();
  }
  const int64_t nch = cols >> 4;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= rows * nch) return;
  const int64_t i = e / nch;
  const int l = (int)(e - i * nch);
  uint32_t cw[4], sc;
  load_codes<FMT, L>(codes, scales, i, cols, l, L * 16, cw, sc);
  float p[16], q[16];
  decode_grid<FMT>(cw, p);
  const float f = block_factor<FMT>(sc, &tab);
#pragma unroll
  for (int k = 0; k < 16; ++k) q[k] = p[k] * f;
  const float ri = r ? r[i] : 1.0f;
  float* o = out + i * cols + 16 * (int64_t)l;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    float y = q[k];
    if (r) y = ri * y;
    if (c) y = y * c[16 * (int64_t)l + k];
    o[k] = y;
  }
}

// ---------------------------------------------------------------- diagnostics
__global__ void k_debug_round(int fn, const float* __restrict__ x, void* out, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (fn == 0) {  // E2M1 code of a pair -> two bytes
    if (2 * e + 1 < n) {
      uint32_t b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[2 * e], x[2 * e + 1], 1.0f, 0);
      ((uint8_t*)out)[2 * e] = (uint8_t)(b & 0xFu);
      ((uint8_t*)out)[2 * e + 1] = (uint8_t)((b >> 4) & 0xFu);
    } else if (2 * e < n) {
      uint32_t b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[2 * e], 0.0f, 1.0f, 0);
      ((uint8_t*)out)[2 * e] = (uint8_t)(b & 0xFu);
    }
    return;
  }
  if (e >= n) return;
  const float v = x[e];
  switch (fn) {
    case 1: ((uint8_t*)out)[e] = (uint8_t)e4m3_code_sat(v); break;
    case 2: ((float*)out)[e] = bf16_rne(v); break;
    case 3: ((int8_t*)out)[e] = (int8_t)(int)int4_round(v); break;
    case 4: ((float*)out)[e] = project<MXFP4>(v); break;
    case 5: ((float*)out)[e] = project<NVFP4>(v); break;
    case 6: ((float*)out)[e] = project<INT4>(v); break;
    default: break;
  }
}

}  // namespace dqk
