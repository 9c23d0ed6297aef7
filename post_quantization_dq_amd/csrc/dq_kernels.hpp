// HIP kernels of the DualQuant dual-scale BCD solver for gfx950.
//
// One pass over W ("sweep") per BCD iteration.  Sweep s takes the scales (r^s, c^s) and
//   * quantises the candidate Qc = FQ_f(W ./ r^s c^s^T)       (Qhat-step of iteration s),
//   * measures F(r^s,c^s,Qc) and the change against the kept Qhat^{s-1} read back from its
//     stored codes: relchg numerator, and dF = F(Qc) - F(Qhat^{s-1}) accumulated per lane
//     and row (so unchanged elements contribute exactly 0 to the safeguard decision),
//   * assuming the candidate is kept, runs the r-step of iteration s+1 (row reduction over
//     the whole row inside the workgroup) and accumulates the c-step column sums with the
//     new r (per-lane registers, one partial per row strip).
// A small finalize kernel then reduces the column partials, projects c, and its last
// workgroup takes the safeguard decision and advances the per-problem state machine.  If
// the candidate is rejected the speculative r/c are discarded and the next sweep runs in
// FIXUP mode (r/c steps from the kept Qhat) before continuing.
//
// Layout: workgroup = H row slots x LPR lanes; lane l of a slot owns columns
// [16l, 16l+16) of its row ("chunk"), so a row of up to 16384 columns is held by one
// slot and the column accumulators stay in the lane's registers across the strip.

#pragma once
#include <type_traits>

#include "dq_device.hpp"

namespace dqk {

enum Mode { MODE_INIT = 0, MODE_NORMAL = 1, MODE_FIXUP = 2, MODE_DONE = 3 };

struct alignas(16) State {
  int32_t mode, it_done, acc, rs;
  int32_t cs, rejected, sweeps, pad0;
  uint32_t flags, counter, init_counter, pad1;
  float st_cur, k6_cur, st_acc, pad2;
  double normW2, qn2_acc;
};

struct ProbDev {
  const void* W;
  int64_t rows, cols, ld;
  float* r[2];
  float* ir[2];
  float* c[2];
  float* ic[2];
  uint8_t* codes[2];
  void* scales[2];
  void* colP;       // [strips][NQ][cols] column partials (fp64 for INT4, else fp32)
  double* swp;      // [strips][4]: F(Qc), dF, relchg numerator, ||Qc||^2
  float* fwp;       // [fin_wgs]: NVFP4 amax partials
  double* initp;    // [init_wgs][2]
  State* st;
  double* nmse;     // [iters+1]
  double* relchg;   // [iters+1]
  float* r_trace;   // [iters][rows] or null: unprojected r-step values
  float* c_trace;   // [iters][cols] or null: unprojected c-step values
  const float* r_init;
  const float* c_init;
  int32_t strips, rows_per_strip, fin_wgs, iters;
  int32_t lpr, hslots, init_wgs, dtype;
  float tol;
  int32_t pad[3];
};

struct WgEntry {
  int32_t prob, idx;
};

constexpr float kTinyTensorScale = 7.888609052210118e-31f;  // 2^-100

// ---------------------------------------------------------------- loads and stores
template <int FMT, int L>
__device__ __forceinline__ void store_chunk(uint8_t* codes, void* scales, int64_t i, int64_t n,
                                            int l, int g, const Chunk& ch) {
  uint2* cp = (uint2*)(codes + ((i * n) >> 1) + 8 * (int64_t)l);
  *cp = make_uint2(ch.code[0], ch.code[1]);
  if ((l % L) == 0) {
    int64_t bi = i * (n / g) + l / L;
    if (Traits<FMT>::SCALE_BYTES == 2) ((uint16_t*)scales)[bi] = (uint16_t)ch.scode;
    else ((uint8_t*)scales)[bi] = (uint8_t)ch.scode;
  }
}

template <int FMT, int L>
__device__ __forceinline__ void load_codes(const uint8_t* codes, const void* scales, int64_t i,
                                           int64_t n, int l, int g, uint32_t& c0, uint32_t& c1,
                                           uint32_t& sc) {
  uint2 cw = *(const uint2*)(codes + ((i * n) >> 1) + 8 * (int64_t)l);
  c0 = cw.x;
  c1 = cw.y;
  int64_t bi = i * (n / g) + l / L;
  sc = (Traits<FMT>::SCALE_BYTES == 2) ? (uint32_t)((const uint16_t*)scales)[bi]
                                       : (uint32_t)((const uint8_t*)scales)[bi];
}

__device__ __forceinline__ void build_nvtab(NvTab& tab, float s_t) {
  for (int k = threadIdx.x; k < 128; k += blockDim.x) {
    float d = e4m3_value((uint32_t)k) * s_t;
    tab.d[k] = (k > 0) ? d : 0.0f;
    tab.id[k] = (k > 0 && d > 0.0f) ? 1.0f / d : 0.0f;
  }
}

// NVFP4 tensor-scale terms from the normalised matrix's amax A.
__device__ __forceinline__ void nv_tensor_terms(float A, float& s_t, float& k6, bool& tiny) {
  s_t = A / 2688.0f;
  float six = 6.0f * s_t;
  k6 = (s_t > 0.0f) ? 1.0f / six : 0.0f;
  tiny = false;
  if (!(s_t >= kTinyTensorScale) || !isfinite(k6)) {
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
    float r = P.r_init ? P.r_init[k] : 1.0f;
    P.r[0][k] = r;
    P.ir[0][k] = 1.0f / r;
  }
  if (k < P.cols) {
    float c = P.c_init ? P.c_init[k] : 1.0f;
    P.c[0][k] = c;
    P.ic[0][k] = 1.0f / c;
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
    s->flags = 0;
    s->counter = 0;
    s->init_counter = 0;
    s->st_cur = s->k6_cur = s->st_acc = 0.0f;
    s->normW2 = 0.0;
    s->qn2_acc = 0.0;
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
  for (int64_t i = r0; i < r1; ++i) {
    float ir = P.ir[0][i];
    for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
      float w = (DT == 1) ? u2f((uint32_t)((const uint16_t*)P.W)[i * P.ld + j] << 16)
                          : ((const float*)P.W)[i * P.ld + j];
      bad |= !isfinite(w);
      s2 += (double)w * (double)w;
      if (FMT == NVFP4) amax = fmaxf(amax, fabsf((w * ir) * P.ic[0][j]));
    }
  }
  __shared__ double ss[4];
  __shared__ float sm[4];
  __shared__ int last;
  s2 = wave_sum(s2);
  amax = wave_max(amax);
  int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { ss[wv] = s2; sm[wv] = amax; }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    P.initp[2 * blockIdx.x] = ((ss[0] + ss[1]) + ss[2]) + ss[3];
    P.initp[2 * blockIdx.x + 1] = (double)fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    if (bad) atomicOr(&P.st->flags, 1u);
    __threadfence();
    unsigned prev = atomicAdd(&P.st->init_counter, 1u);
    last = (prev == (unsigned)P.init_wgs - 1);
  }
  __syncthreads();
  if (!last || threadIdx.x != 0) return;
  __threadfence();
  double tot = 0.0;
  float A = 0.0f;
  for (int b = 0; b < P.init_wgs; ++b) {
    tot += P.initp[2 * b];
    A = fmaxf(A, (float)P.initp[2 * b + 1]);
  }
  State* s = P.st;
  s->normW2 = tot;
  if (FMT == NVFP4) {
    float st_, k6_;
    bool tiny;
    nv_tensor_terms(A, st_, k6_, tiny);
    s->st_cur = st_;
    s->k6_cur = k6_;
    if (tiny) atomicOr(&s->flags, (uint32_t)16u);
  }
  s->init_counter = 0;
}

// ---------------------------------------------------------------- the sweep
// K = chunks of 16 columns per lane (chunk index l + k * lpr).  With K == 1 the row's
// values and grid values stay in registers for the column phase; with K == 2 they are
// re-derived from the raw row and the codes to keep the register file within budget.
template <int DT>
struct RawRow;
template <>
struct RawRow<1> {   // bf16: 8 packed words per chunk
  uint32_t u[8];
  __device__ __forceinline__ void load(const void* base, int64_t i, int64_t ld, int j0) {
    const uint4* p = (const uint4*)((const uint16_t*)base + i * ld + j0);
    uint4 a = p[0], b = p[1];
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
    const float4* p = (const float4*)((const float*)base + i * ld + j0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float4 a = p[k];
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

template <int FMT, int DT, int L, int K>
__global__ __launch_bounds__(512) void k_sweep(const ProbDev* __restrict__ probs,
                                               const WgEntry* __restrict__ table) {
  const WgEntry we = table[blockIdx.x];
  const ProbDev& P = probs[we.prob];
  State* st = P.st;
  const int mode = st->mode;
  if (mode == MODE_DONE) return;
  const int it = (mode == MODE_INIT) ? 0 : st->it_done + 1;
  const bool cand = (mode != MODE_FIXUP);
  const bool stats = (mode == MODE_NORMAL);
  const bool next = (mode == MODE_FIXUP) || (it < P.iters);
  const int rs = st->rs, cs = st->cs, acc = st->acc;
  const int cb = (mode == MODE_INIT) ? 0 : 1 - acc;
  const int g = L * 16;
  constexpr bool HOLD = (K == 1);
  // INT4 (fine bf16 scale grid) accumulates exact products in fp64 so that its projected
  // scales agree with an fp64 reference essentially always; the other formats use fp32
  // partials per lane and row strip with fp64 combines.
  constexpr bool A64 = (FMT == INT4);
  typedef typename std::conditional<A64, double, float>::type acc_t;
  constexpr int NQ = (FMT == NVFP4) ? 3 : 2;
  const int tr = (mode == MODE_FIXUP) ? it - 1 : it;   // trace row of the r-step computed here

  __shared__ NvTab tab_c, tab_p;
  __shared__ double red[2][8][2];
  __shared__ double redw[8][4];
  extern __shared__ float xs[];

  if (FMT == NVFP4) {
    build_nvtab(tab_c, st->st_cur);
    build_nvtab(tab_p, st->st_acc);
    __syncthreads();
  }

  const int t = threadIdx.x, lpr = P.lpr, H = P.hslots;
  const int h = t / lpr, l = t - h * lpr;
  const int64_t n = P.cols;
  const int nch = (int)(n >> 4);
  const int wave = t >> 6, wps = lpr >> 6;

  float cc[K][16], icc[K][16];
  acc_t colN[K][16], colD[K][16];
  float colM[K][16];
#pragma unroll
  for (int kc = 0; kc < K; ++kc) {
    const int ch = l + kc * lpr;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      cc[kc][k] = 0.0f; icc[kc][k] = 0.0f;
      colN[kc][k] = (acc_t)0; colD[kc][k] = (acc_t)0; colM[kc][k] = 0.0f;
    }
    if (ch < nch) {
      const float4* cp = (const float4*)(P.c[cs] + 16 * ch);
      const float4* icp = (const float4*)(P.ic[cs] + 16 * ch);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float4 a = cp[k], b = icp[k];
        cc[kc][4 * k] = a.x; cc[kc][4 * k + 1] = a.y; cc[kc][4 * k + 2] = a.z; cc[kc][4 * k + 3] = a.w;
        icc[kc][4 * k] = b.x; icc[kc][4 * k + 1] = b.y; icc[kc][4 * k + 2] = b.z; icc[kc][4 * k + 3] = b.w;
      }
    }
  }
  double aFc = 0.0, adF = 0.0, arel = 0.0, aqn = 0.0;
  bool uflow = false, zrow = false;

  const int64_t row0 = (int64_t)we.idx * P.rows_per_strip;
  const int64_t row1 = min(P.rows, row0 + P.rows_per_strip);
  const float* rcur = P.r[rs];
  const float* ircur = P.ir[rs];
  float* rnext = P.r[1 - rs];
  float* irnext = P.ir[1 - rs];
  uint8_t* ccodes = P.codes[cb];
  void* cscales = P.scales[cb];
  const uint8_t* acodes = P.codes[acc];
  const void* ascales = P.scales[acc];
  QCtx qc;
  qc.k6 = st->k6_cur;
  qc.tab = &tab_c;
  const int ngroups = (P.rows_per_strip + H - 1) / H;

  for (int gi = 0; gi < ngroups; ++gi) {
    const int64_t i = row0 + (int64_t)gi * H + h;
    const bool rowok = i < row1;
    const float r_ = rowok ? rcur[i] : 1.0f;
    const float ir_ = rowok ? ircur[i] : 1.0f;
    double Nrow = 0.0, Drow = 0.0;
    RawRow<DT> raw[K];
    uint32_t kc0[K], kc1[K];
    float kf[K];
    float wh[HOLD ? K : 1][16], ph[HOLD ? K : 1][16];
#pragma unroll
    for (int kc = 0; kc < K; ++kc) {
      const int chn = l + kc * lpr;
      const bool valid = rowok && (chn < nch);
      const int j0 = 16 * chn;
      if (valid) raw[kc].load(P.W, i, P.ld, j0); else raw[kc].zero();
      float w[16];
      raw[kc].unpack(w);
      float p[16];
      float f;
      float Nb = 0.0f, Db = 0.0f;
      double Nbd = 0.0, Dbd = 0.0;
      if (cand) {
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = (w[k] * ir_) * icc[kc][k];
        Chunk ch;
        quantize_chunk<FMT, L>(v, qc, ch);
        if (valid) store_chunk<FMT, L>(ccodes, cscales, i, n, chn, g, ch);
        uflow |= ch.underflow && valid;
        f = ch.f;
        kc0[kc] = ch.code[0];
        kc1[kc] = ch.code[1];
        const float rf = r_ * f;
        float Fl = 0.0f, ql = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          p[k] = ch.p[k];
          const float pc = p[k] * cc[kc][k];
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
        if (stats) {
          uint32_t p0 = 0, p1 = 0, ps = 0;
          if (valid) load_codes<FMT, L>(acodes, ascales, i, n, chn, g, p0, p1, ps);
          float pp[16];
          decode_grid<FMT>(p0, p1, pp);
          const float fp = block_factor<FMT>(ps, &tab_p);
          const float rfp = r_ * fp;
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const float ppc = pp[k] * cc[kc][k];
            const float ep = fmaf(-rfp, ppc, w[k]);
            Fpl = fmaf(ep, ep, Fpl);
            const float df = fmaf(p[k], f, -(pp[k] * fp));
            rl = fmaf(df, df, rl);
          }
        }
        if (valid) {
          aFc += (double)Fl;
          adF += (double)Fl - (double)Fpl;
          arel += (double)rl;
          aqn += (double)(f * f) * (double)ql;
        }
      } else {
        uint32_t p0 = 0, p1 = 0, ps = 0;
        if (valid) load_codes<FMT, L>(acodes, ascales, i, n, chn, g, p0, p1, ps);
        decode_grid<FMT>(p0, p1, p);
        f = block_factor<FMT>(ps, &tab_p);
        kc0[kc] = p0;
        kc1[kc] = p1;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float pc = p[k] * cc[kc][k];
          if (A64) {
            Nbd = fma((double)w[k], (double)pc, Nbd);
            Dbd = fma((double)pc, (double)pc, Dbd);
          } else {
            Nb = fmaf(w[k], pc, Nb);
            Db = fmaf(pc, pc, Db);
          }
        }
      }
      kf[kc] = f;
      if (valid) {
        if (A64) {
          Nrow += (double)f * Nbd;
          Drow += ((double)f * (double)f) * Dbd;
        } else {
          Nrow += (double)f * (double)Nb;
          Drow += (double)(f * f) * (double)Db;
        }
      }
      if (HOLD) {
#pragma unroll
        for (int k = 0; k < 16; ++k) { wh[HOLD ? kc : 0][k] = w[k]; ph[HOLD ? kc : 0][k] = p[k]; }
      }
    }
    if (next) {
      // r-step of the next iteration: whole-row sums, fp64 across lanes and waves
      const double Nd = wave_sum(Nrow), Dd = wave_sum(Drow);
      if ((t & 63) == 0) { red[gi & 1][wave][0] = Nd; red[gi & 1][wave][1] = Dd; }
      __syncthreads();
      double N = 0.0, D = 0.0;
      for (int k = 0; k < wps; ++k) {
        N += red[gi & 1][h * wps + k][0];
        D += red[gi & 1][h * wps + k][1];
      }
      float rnew = 1.0f, irn = 1.0f;
      if (rowok) {
        float x = __builtin_nanf("");
        if (D > 0.0) {
          x = (float)(N / D);
          rnew = project<FMT>(x);
        } else {
          rnew = r_;
          zrow = true;
        }
        irn = 1.0f / rnew;
        if (l == 0) {
          rnext[i] = rnew;
          irnext[i] = irn;
          if (P.r_trace) P.r_trace[(int64_t)tr * P.rows + i] = x;
        }
      }
#pragma unroll
      for (int kc = 0; kc < K; ++kc) {
        const int chn = l + kc * lpr;
        if (!(rowok && chn < nch)) continue;
        float w[16], p[16];
        if (HOLD) {
#pragma unroll
          for (int k = 0; k < 16; ++k) { w[k] = wh[HOLD ? kc : 0][k]; p[k] = ph[HOLD ? kc : 0][k]; }
        } else {
          raw[kc].unpack(w);
          decode_grid<FMT>(kc0[kc], kc1[kc], p);
        }
        const float rf = rnew * kf[kc];
        const float rf2 = rf * rf;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          if (A64) {   // INT4: rf = r * s and rf * p are exact in fp32; the products below are exact in fp64
            colN[kc][k] = fma((double)rf, (double)w[k] * (double)p[k], (double)colN[kc][k]);
            const double rp = (double)(rf * p[k]);
            colD[kc][k] = fma(rp, rp, (double)colD[kc][k]);
          } else {
            colN[kc][k] = fmaf(rf, w[k] * p[k], (float)colN[kc][k]);
            colD[kc][k] = fmaf(rf2, p[k] * p[k], (float)colD[kc][k]);
          }
          if (FMT == NVFP4) colM[kc][k] = fmaxf(colM[kc][k], fabsf(w[k] * irn));
        }
      }
    }
  }

  if (next) {
    // combine the row slots' column partials (fixed slot order), then write this strip's
    if (H > 1) {
      acc_t* xa = (acc_t*)xs;
      for (int qi = 0; qi < NQ; ++qi) {
        __syncthreads();
        if (h >= 1 && l < nch) {
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const acc_t v = (qi == 0) ? colN[0][k] : (qi == 1) ? colD[0][k] : (acc_t)colM[0][k];
            xa[(k * (H - 1) + (h - 1)) * lpr + l] = v;
          }
        }
        __syncthreads();
        if (h == 0 && l < nch) {
          for (int hh = 1; hh < H; ++hh) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
              const acc_t o = xa[(k * (H - 1) + (hh - 1)) * lpr + l];
              if (qi == 0) colN[0][k] += o;
              else if (qi == 1) colD[0][k] += o;
              else colM[0][k] = fmaxf(colM[0][k], (float)o);
            }
          }
        }
      }
    }
    if (h == 0) {
#pragma unroll
      for (int kc = 0; kc < K; ++kc) {
        const int chn = l + kc * lpr;
        if (chn >= nch) continue;
        acc_t* base = (acc_t*)P.colP + (size_t)we.idx * NQ * (size_t)n + 16 * chn;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          base[k] = colN[kc][k];
          base[n + k] = colD[kc][k];
          if (FMT == NVFP4) base[2 * n + k] = (acc_t)colM[kc][k];
        }
      }
    }
  }

  if (cand) {
    const double a0 = wave_sum(aFc), a1 = wave_sum(adF), a2 = wave_sum(arel), a3 = wave_sum(aqn);
    if ((t & 63) == 0) { redw[wave][0] = a0; redw[wave][1] = a1; redw[wave][2] = a2; redw[wave][3] = a3; }
  }
  const bool anyu = __syncthreads_or(uflow);
  const bool anyz = __syncthreads_or(zrow);
  if (t == 0) {
    if (cand) {
      double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
      const int nw = (int)(blockDim.x >> 6);
      for (int k = 0; k < nw; ++k) { s0 += redw[k][0]; s1 += redw[k][1]; s2 += redw[k][2]; s3 += redw[k][3]; }
      double* o = P.swp + 4 * (size_t)we.idx;
      o[0] = s0; o[1] = s1; o[2] = s2; o[3] = s3;
    }
    const uint32_t fl = (anyu ? 8u : 0u) | (anyz ? 2u : 0u);
    if (fl) atomicOr(&st->flags, fl);
  }
}

// ---------------------------------------------------------------- finalize
// Column reduction of the strip partials, c-step projection, next NVFP4 tensor scale, and
// (last workgroup of each problem) the safeguard decision and state update.
template <int FMT>
__global__ __launch_bounds__(256) void k_finalize(const ProbDev* __restrict__ probs,
                                                  const WgEntry* __restrict__ table) {
  const WgEntry we = table[blockIdx.x];
  const ProbDev& P = probs[we.prob];
  State* st = P.st;
  const int mode = st->mode;
  if (mode == MODE_DONE) return;
  const int it = (mode == MODE_INIT) ? 0 : st->it_done + 1;
  const bool next = (mode == MODE_FIXUP) || (it < P.iters);
  const int cs = st->cs;
  const int64_t n = P.cols;

  __shared__ double sN[4][64], sD[4][64];
  __shared__ float sM[4][64];
  __shared__ float wmax[4];
  __shared__ double sred[256][4];
  __shared__ int last;

  const int t = threadIdx.x;
  bool zcol = false;
  if (next) {
    const int part = t >> 6, cl = t & 63;
    const int64_t j = (int64_t)we.idx * 64 + cl;
    double N = 0.0, D = 0.0;
    float M = 0.0f;
    if (j < n) {
      const int S = P.strips;
      const int s0 = part * S / 4, s1 = (part + 1) * S / 4;
      constexpr int NQ = (FMT == NVFP4) ? 3 : 2;
      typedef typename std::conditional<FMT == INT4, double, float>::type acc_t;
      for (int s = s0; s < s1; ++s) {
        const acc_t* b = (const acc_t*)P.colP + (size_t)s * NQ * (size_t)n;
        N += (double)b[j];
        D += (double)b[n + j];
        if (FMT == NVFP4) M = fmaxf(M, (float)b[2 * n + j]);
      }
    }
    sN[part][cl] = N;
    sD[part][cl] = D;
    sM[part][cl] = M;
    __syncthreads();
    float am = 0.0f;
    if (part == 0 && j < n) {
      N = ((sN[0][cl] + sN[1][cl]) + sN[2][cl]) + sN[3][cl];
      D = ((sD[0][cl] + sD[1][cl]) + sD[2][cl]) + sD[3][cl];
      M = fmaxf(fmaxf(sM[0][cl], sM[1][cl]), fmaxf(sM[2][cl], sM[3][cl]));
      float x = __builtin_nanf("");
      float cnew;
      if (D > 0.0) {
        x = (float)(N / D);
        cnew = project<FMT>(x);
      } else {
        cnew = P.c[cs][j];
        zcol = true;
      }
      const float icn = 1.0f / cnew;
      P.c[1 - cs][j] = cnew;
      P.ic[1 - cs][j] = icn;
      if (P.c_trace) P.c_trace[(int64_t)((mode == MODE_FIXUP) ? it - 1 : it) * n + j] = x;
      if (FMT == NVFP4) am = M * icn;
    }
    if (FMT == NVFP4) {
      am = wave_max(am);
      if ((t & 63) == 0) wmax[t >> 6] = am;
    }
  }
  zcol = __syncthreads_or(zcol);
  if (t == 0) {
    if (next && FMT == NVFP4) P.fwp[we.idx] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    if (zcol) atomicOr(&st->flags, 4u);
    __threadfence();
    unsigned prev = atomicAdd(&st->counter, 1u);
    last = (prev == (unsigned)P.fin_wgs - 1);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();

  // fixed-order reductions of the sweep's strip partials and the amax partials
  double f0 = 0.0, f1 = 0.0, f2 = 0.0, f3 = 0.0;
  if (mode != MODE_FIXUP) {
    for (int s = t; s < P.strips; s += 256) {
      const double* o = P.swp + 4 * (size_t)s;
      f0 += o[0]; f1 += o[1]; f2 += o[2]; f3 += o[3];
    }
  }
  float A = 0.0f;
  if (next && FMT == NVFP4) {
    for (int k = t; k < P.fin_wgs; k += 256) A = fmaxf(A, P.fwp[k]);
  }
  sred[t][0] = f0; sred[t][1] = f1; sred[t][2] = f2; sred[t][3] = f3;
  A = wave_max(A);
  if ((t & 63) == 0) wmax[t >> 6] = A;
  __syncthreads();
  if (t != 0) return;
  double Fc = 0.0, dF = 0.0, rel = 0.0, qn = 0.0;
  for (int k = 0; k < 256; ++k) { Fc += sred[k][0]; dF += sred[k][1]; rel += sred[k][2]; qn += sred[k][3]; }
  A = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));

  const double nW = st->normW2;
  bool accepted = true;
  double relv = 0.0;
  if (mode == MODE_INIT) {
    if (P.nmse) P.nmse[0] = nW > 0.0 ? Fc / nW : 0.0;
    if (P.relchg) P.relchg[0] = 0.0;
    st->acc = 0;
    st->qn2_acc = qn;
    st->st_acc = st->st_cur;
    st->it_done = 0;
  } else if (mode == MODE_NORMAL) {
    accepted = (dF <= 0.0);
    if (accepted) {
      relv = st->qn2_acc > 0.0 ? sqrt(rel) / sqrt(st->qn2_acc) : 0.0;
      if (P.nmse) P.nmse[it] = nW > 0.0 ? Fc / nW : 0.0;
      st->acc = 1 - st->acc;
      st->qn2_acc = qn;
      st->st_acc = st->st_cur;
    } else {
      st->rejected += 1;
      if (P.nmse) P.nmse[it] = nW > 0.0 ? (Fc - dF) / nW : 0.0;
    }
    if (P.relchg) P.relchg[it] = relv;
    st->it_done = it;
  }
  const bool stop = (mode != MODE_FIXUP) &&
                    (it >= P.iters || (mode == MODE_NORMAL && P.tol > 0.0f && relv <= (double)P.tol));
  if (stop) {
    st->mode = MODE_DONE;
  } else if (accepted) {
    st->rs = 1 - st->rs;
    st->cs = 1 - st->cs;
    if (FMT == NVFP4) {
      float s_, k_;
      bool tiny;
      nv_tensor_terms(A, s_, k_, tiny);
      st->st_cur = s_;
      st->k6_cur = k_;
      if (tiny) st->flags |= 16u;
    }
    st->mode = MODE_NORMAL;
  } else {
    st->mode = MODE_FIXUP;
  }
  st->sweeps += 1;
  st->counter = 0;
}

// ---------------------------------------------------------------- standalone quantiser
// MODEV = 0: weights, v = (W * (1/r_i)) * (1/c_j);  MODEV = 1: activations, v = x * c_j.
// Pass 1 (NVFP4 only): per-workgroup amax of v.
template <int DT, int MODEV>
__global__ __launch_bounds__(256) void k_qamax(const void* __restrict__ X, int64_t rows,
                                               int64_t cols, int64_t ld,
                                               const float* __restrict__ r,
                                               const float* __restrict__ c,
                                               float* __restrict__ part) {
  float m = 0.0f;
  const int64_t total = rows * cols;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / cols, j = e - i * cols;
    float x = (DT == 1) ? u2f((uint32_t)((const uint16_t*)X)[i * ld + j] << 16)
                        : ((const float*)X)[i * ld + j];
    float v;
    if (MODEV == 0) {
      const float ir = r ? 1.0f / r[i] : 1.0f;
      const float ic = c ? 1.0f / c[j] : 1.0f;
      v = (x * ir) * ic;
    } else {
      v = c ? x * c[j] : x;
    }
    m = fmaxf(m, fabsf(v));
  }
  m = wave_max(m);
  __shared__ float sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
}

// Pass 2: quantise; workgroup = H row slots x LPR lanes, one chunk per lane.
template <int FMT, int DT, int L, int MODEV>
__global__ __launch_bounds__(1024) void k_quant(const void* __restrict__ X, int64_t rows,
                                                int64_t cols, int64_t ld,
                                                const float* __restrict__ r,
                                                const float* __restrict__ c, uint8_t* codes,
                                                void* scales, float* tensor_scale,
                                                const float* __restrict__ part, int nparts,
                                                int lpr, int H) {
  __shared__ NvTab tab;
  __shared__ float sA;
  QCtx qc;
  qc.k6 = 0.0f;
  qc.tab = &tab;
  if (FMT == NVFP4) {
    if (threadIdx.x == 0) {
      float A = 0.0f;
      for (int k = 0; k < nparts; ++k) A = fmaxf(A, part[k]);
      sA = A;
    }
    __syncthreads();
    float s_t, k6;
    bool tiny;
    nv_tensor_terms(sA, s_t, k6, tiny);
    qc.k6 = k6;
    build_nvtab(tab, s_t);
    if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = s_t;
    __syncthreads();
  }
  const int t = threadIdx.x;
  const int h = t / lpr, l = t - h * lpr;
  const int64_t i = (int64_t)blockIdx.x * H + h;
  const bool act = (l < (int)(cols >> 4)) && (i < rows);
  const int j0 = l * 16;
  float w[16], v[16];
  RawRow<DT> raw;
  if (act) raw.load(X, i, ld, j0); else raw.zero();
  raw.unpack(w);
  if (MODEV == 0) {
    const float ir = (act && r) ? 1.0f / r[i] : 1.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float ic = (act && c) ? 1.0f / c[j0 + k] : 1.0f;
      v[k] = (w[k] * ir) * ic;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = (act && c) ? w[k] * c[j0 + k] : w[k];
  }
  Chunk ch;
  quantize_chunk<FMT, L>(v, qc, ch);
  if (act) store_chunk<FMT, L>(codes, scales, i, cols, l, L * 16, ch);
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
  uint32_t c0, c1, sc;
  load_codes<FMT, L>(codes, scales, i, cols, l, L * 16, c0, c1, sc);
  float p[16], q[16];
  decode_grid<FMT>(c0, c1, p);
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
    case 4: ((float*)out)[e] = proj_pow2(v); break;
    case 5: ((float*)out)[e] = proj_e4m3(v); break;
    case 6: ((float*)out)[e] = proj_bf16(v); break;
    default: break;
  }
}

}  // namespace dqk
