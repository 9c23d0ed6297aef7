// C-ABI host layer of the DualQuant solver library (gfx950): argument validation,
// workspace layout, launch planning and the iteration loop.  See include/dq.h for the
// contract of every entry point.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/dq.h"
#include "dq_kernels.hpp"
#include "dq_linear.hpp"

using namespace dqk;

namespace {

constexpr int kMaxCols = 65536;
constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

int default_group(int fmt) {
  switch (fmt) {
    case DQ_FMT_INT4: return 128;
    case DQ_FMT_INT8: return 128;
    case DQ_FMT_MXINT8: return 32;
    case DQ_FMT_MXFP8_E4M3: return 32;
    case DQ_FMT_MXFP8_E5M2: return 32;
    case DQ_FMT_MXFP6_E2M3: return 32;
    case DQ_FMT_MXFP6_E3M2: return 32;
    case DQ_FMT_MXINT4: return 32;
    case DQ_FMT_MXFP4: return 32;
    case DQ_FMT_NVFP4: return 16;
    default: return 0;
  }
}

int resolve_group(const dq_quant_spec& s) {
  if (s.fmt < DQ_FMT_INT4 || s.fmt > DQ_FMT_MXFP6_E3M2) return -1;
  int g = s.group ? s.group : default_group(s.fmt);
  if ((s.fmt == DQ_FMT_INT4 || s.fmt == DQ_FMT_INT8) && g != 64 && g != 128) return -1;
  const bool mx = s.fmt == DQ_FMT_MXINT4 || s.fmt == DQ_FMT_MXFP4 || s.fmt == DQ_FMT_MXINT8 ||
                  (s.fmt >= DQ_FMT_MXFP8_E4M3 && s.fmt <= DQ_FMT_MXFP6_E3M2);
  if (mx && g != 32) return -1;
  if (s.fmt == DQ_FMT_NVFP4 && g != 16) return -1;
  return g;
}

bool grouped_int_fmt(int fmt) { return fmt == DQ_FMT_INT4 || fmt == DQ_FMT_INT8; }
int scale_bytes(int fmt) { return grouped_int_fmt(fmt) ? 2 : 1; }
// Bits per element code: 4 (two per byte), 6 (a bit stream) or 8.
int code_bits(int fmt) {
  if (fmt == DQ_FMT_INT8 || fmt == DQ_FMT_MXINT8 || fmt == DQ_FMT_MXFP8_E4M3 ||
      fmt == DQ_FMT_MXFP8_E5M2)
    return 8;
  if (fmt == DQ_FMT_MXFP6_E2M3 || fmt == DQ_FMT_MXFP6_E3M2) return 6;
  return 4;
}
size_t code_bytes(int fmt, int64_t rows, int64_t cols) {
  return (size_t)rows * (size_t)cols * (size_t)code_bits(fmt) / 8;
}
// Column partials per row range: N, D (and the NVFP4 column amax); fp64 for INT4.
size_t partial_bytes(int fmt, int64_t strips, int64_t cols) {
  const int nq = fmt == DQ_FMT_NVFP4 ? 3 : 2;
  const size_t el = grouped_int_fmt(fmt) ? sizeof(double) : sizeof(float);
  return (size_t)strips * nq * cols * el;
}
int elem_bytes(int dt) { return dt == DQ_F32 ? 4 : 2; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Checks shared by every entry point that reads a [rows][ld] matrix.
int check_matrix(const void* X, int32_t dt, int64_t rows, int64_t cols, int64_t ld, int g) {
  if (dt != DQ_F32 && dt != DQ_BF16) return DQ_ERR_FORMAT;
  if (rows < 0 || cols < 0 || ld < cols) return DQ_ERR_SHAPE;
  if (cols % g != 0 || cols > kMaxCols) return DQ_ERR_SHAPE;
  if (rows > 0 && cols > 0) {
    if (!X) return DQ_ERR_NULL;
    if (!aligned16(X) || ((ld * elem_bytes(dt)) % 16) != 0) return DQ_ERR_ALIGN;
  }
  return DQ_OK;
}

// Row pass: workgroups of 16 waves, one wave per row, one workgroup per CU (all registers).
constexpr int kRowWaves = 16;
constexpr int kRowWgs = 256;
constexpr int kTargetRowWaves = kRowWgs * kRowWaves;
// Column pass: workgroups of 8 waves on a 1024-column strip and a range of rows, two per CU
// (registers).  A matrix takes at most its share of 512 workgroups, rounded down, so a
// single matrix runs in one round: 4096 x 14336 gets 14 strips x 36 ranges = 504 (26.6 us
// per launch; 896 workgroups in 1.75 rounds took 29.9 us, and 518 in just over one round
// took 2.6 us more than that).
constexpr int kTargetColWgs = 512;
// The finalize pass reduces up to 64 row ranges per column with one round of loads.
constexpr int64_t kMaxRowRanges = 64;
// Caps for large batches: many workgroups of bounded size keep the last wave of workgroups
// short; a single projection-sized matrix stays below both.
constexpr int64_t kMaxRowsPerBlk = 256;
// Iterations per solve: the queued sweeps (T + 1) and the history buffers stay modest.
constexpr int kMaxIters = 1 << 16;
constexpr int64_t kMaxRowsPerRange = 512;
// Standalone quantiser geometry: one chunk per lane, up to 1024 threads; rows wider than
// 16384 columns take several passes of 1024 chunks.
int lanes_per_row(int64_t cols) {
  return (int)std::min<int64_t>(1024, std::max<int64_t>(64, (cols / 16 + 63) / 64 * 64));
}
int row_slots(int lpr) { return std::max(1, 1024 / lpr); }
// Rows per quantiser workgroup: as many as 1024 threads hold, halved while that leaves fewer
// row groups than the grid may take (a few tokens then spread over more CUs instead of
// stacking 4 rows of 256 lanes on one).  Each row's result does not depend on it.
int quant_rows_per_group(int lpr, int64_t rows, int64_t max_groups) {
  int H = row_slots(lpr);
  while (H > 1 && (rows + H - 1) / H < max_groups) H >>= 1;
  return H;
}
// LDS one workgroup may take on the current device (160 KiB on gfx950), read once per device.
int device_lds_limit() {
  static std::atomic<int> cache[64];   // 0: not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        v <= 0)
      v = -1;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return std::max(v, 0);
}
// The row pass keeps c and 1/c in LDS (8 bytes per column), always up to 16384 columns and
// beyond that while the queue of changed chunks still fits beside them; otherwise it reads
// them from global memory (L2-resident).  Without the queue every chunk would run the kept
// Qhat's work inline (3584 x 18944 NVFP4: 67.8 us with c in LDS and no queue).
constexpr int64_t kRowPassLdsCols = 16384;
size_t rowpass_tabs(int fmt) { return fmt == DQ_FMT_NVFP4 ? 2 * sizeof(NvTab) : 0; }
size_t rowpass_queue(int fmt);
bool rowpass_cg(int fmt, int64_t cols) {
  if (cols <= kRowPassLdsCols) return false;
  return 2 * sizeof(float) * (size_t)cols + rowpass_tabs(fmt) + rowpass_queue(fmt) >
         (size_t)device_lds_limit();
}
size_t rowpass_lds(int fmt, int64_t cols) {
  return (rowpass_cg(fmt, cols) ? 0 : 2 * sizeof(float) * (size_t)cols) + rowpass_tabs(fmt);
}
// The queue of changed chunks (kRowWaves waves x kQueueLen entries), when it fits beside the rest.
size_t rowpass_queue(int fmt) {
  const int words = code_bits(fmt) == 8 ? 8 : 4;   // queue_words<FMT>()
  return (size_t)kRowWaves * kQueueLen * words * sizeof(uint32_t);
}
bool rowpass_compact(int fmt, int64_t cols) {
  return rowpass_lds(fmt, cols) + rowpass_queue(fmt) <= (size_t)device_lds_limit();
}
size_t rowpass_lds_total(int fmt, int64_t cols) {
  return rowpass_lds(fmt, cols) + (rowpass_compact(fmt, cols) ? rowpass_queue(fmt) : 0);
}
size_t colpass_lds(int fmt) { return (size_t)8 * 64 * 16 * (grouped_int_fmt(fmt) ? 8 : 4); }

struct Plan {
  std::vector<ProbDev> dev;
  std::vector<int> group_of;   // launch group index, -1 for empty problems
  struct Group {               // problems sharing (dtype, cols) share the launches
    int dtype;
    int64_t cols;
    std::vector<WgEntry> row, col, fin;
    size_t row_off, col_off, fin_off;  // offsets of the tables in the workspace
  };
  std::vector<Group> groups;
  // [live_off, up_end): uploaded at once -- the live-problem counter, the problem
  // descriptors and every launch table (and the state slots between the counter and the
  // descriptors, which k_setup then writes)
  size_t live_off = 0, probs_off = 0, up_end = 0, total = 0;
  int32_t live = 0;   // problems with work (rows and cols > 0)
  std::vector<size_t> prob_off;
};

// Lays out the workspace and the launch tables (sizes only; pointers are bound later).
int make_plan(const dq_problem* p, int32_t count, int g, int fmt, int iters, Plan& pl) {
  pl.dev.assign(count, ProbDev{});
  pl.group_of.assign(count, -1);
  pl.prob_off.assign(count, 0);
  std::map<std::pair<int, int64_t>, int> gid;
  int64_t total_rows = 0;
  for (int k = 0; k < count; ++k) {
    if (p[k].rows == 0 || p[k].cols == 0) continue;
    total_rows += p[k].rows;
    auto key = std::make_pair((int)p[k].w_dtype, (int64_t)p[k].cols);
    auto it = gid.find(key);
    if (it == gid.end()) {
      Plan::Group G;
      G.dtype = p[k].w_dtype;
      G.cols = p[k].cols;
      it = gid.emplace(key, (int)pl.groups.size()).first;
      pl.groups.push_back(G);
    }
    pl.group_of[k] = it->second;
  }
  // Rows per row-pass workgroup.  A single matrix or a small batch takes the smallest block
  // that puts every block in one round of one workgroup per CU, so the CUs share the rows
  // evenly (5120 rows: 256 blocks of 20, not 160 blocks of 32 with 96 CUs idle; 1024 rows:
  // 256 blocks of 4, some waves idle, rather than 64 blocks of 16 on a quarter of the CUs).
  // Otherwise: 16 rows per wave-round, at most kMaxRowsPerBlk (a large batch splits into
  // many similar workgroups, balanced by the dispatcher).
  const int64_t rows_per_wave = std::max<int64_t>(1, (total_rows + kTargetRowWaves - 1) / kTargetRowWaves);
  int64_t rows_per_blk = std::min<int64_t>(kMaxRowsPerBlk, kRowWaves * rows_per_wave);
  {
    std::vector<int64_t> rows_of;
    for (int k = 0; k < count; ++k)
      if (pl.group_of[k] >= 0) rows_of.push_back(p[k].rows);
    if (!rows_of.empty() && rows_of.size() <= (size_t)kRowWgs) {
      for (int64_t b = std::max<int64_t>(1, (total_rows + kRowWgs - 1) / kRowWgs);
           b <= kMaxRowsPerBlk; ++b) {
        int64_t wgs = 0;
        for (int64_t m : rows_of) wgs += (m + b - 1) / b;
        if (wgs <= kRowWgs) {
          rows_per_blk = b;
          break;
        }
      }
    }
  }
  const int nq = fmt == DQ_FMT_NVFP4 ? 3 : 2;
  const size_t acc_bytes = grouped_int_fmt(fmt) ? 8 : 4;
  size_t off = 0;
  for (int k = 0; k < count; ++k) {
    ProbDev& d = pl.dev[k];
    d.rows = p[k].rows;
    d.cols = p[k].cols;
    d.ld = p[k].ld;
    d.iters = iters;
    d.dtype = p[k].w_dtype;
    if (pl.group_of[k] < 0) continue;
    Plan::Group& G = pl.groups[pl.group_of[k]];
    d.rows_per_blk = (int32_t)rows_per_blk;
    d.rowblocks = (int32_t)((d.rows + d.rows_per_blk - 1) / d.rows_per_blk);
    d.nstrips = (int32_t)((d.cols / 16 + 63) / 64);
    int64_t want = (kTargetColWgs * d.rows + total_rows - 1) / total_rows;   // this matrix's share
    int64_t rr = std::max<int64_t>(1, std::min<int64_t>(d.rows, want / d.nstrips));
    rr = std::min<int64_t>(rr, kMaxRowRanges);
    d.rows_per_range = (int32_t)std::min<int64_t>(kMaxRowsPerRange, (d.rows + rr - 1) / rr);
    d.rranges = (int32_t)((d.rows + d.rows_per_range - 1) / d.rows_per_range);
    d.fin_wgs = (int32_t)((d.cols + 63) / 64);
    d.init_wgs = (int32_t)std::min<int64_t>(1024, d.rows);
    pl.prob_off[k] = off;
    off = align_up(off + 2 * sizeof(uint32_t));                        // flags, altz
    off = align_up(off + 7 * sizeof(float) * d.rows);                  // r[3], ir[3], x_alt
    off = align_up(off + 4 * sizeof(float) * d.cols);                  // c[2], ic[2]
    off = align_up(off + code_bytes(fmt, d.rows, d.cols));             // codes buffer 1
    off = align_up(off + (size_t)d.rows * d.cols / g * scale_bytes(fmt));
    off = align_up(off + (size_t)d.rranges * nq * d.cols * acc_bytes);  // column partials
    off = align_up(off + (size_t)d.rowblocks * 4 * sizeof(double));
    off = align_up(off + (size_t)d.fin_wgs * sizeof(float));
    off = align_up(off + (size_t)d.init_wgs * 2 * sizeof(double));
    off = align_up(off + 2 * (size_t)(iters + 1) * sizeof(double));   // histories if caller has none
    for (int b = 0; b < d.rowblocks; ++b) G.row.push_back(WgEntry{k, b});
    for (int b = 0; b < d.nstrips * d.rranges; ++b) G.col.push_back(WgEntry{k, b});
    G.fin.push_back(WgEntry{k, d.fin_wgs});   // the decision workgroup, dispatched first
    for (int f = 0; f < d.fin_wgs; ++f) G.fin.push_back(WgEntry{k, f});
  }
  pl.live = 0;
  for (int k = 0; k < count; ++k) pl.live += pl.group_of[k] >= 0 ? 1 : 0;
  pl.live_off = off;   // the counter, then (kStatesOffset on) every problem's two state slots
  off = align_up(off + kStatesOffset + 2 * sizeof(State) * std::max(1, (int)count));
  pl.probs_off = off;
  off = align_up(off + sizeof(ProbDev) * std::max(1, (int)count));
  for (auto& G : pl.groups) {
    G.row_off = off;
    off = align_up(off + sizeof(WgEntry) * G.row.size());
    G.col_off = off;
    off = align_up(off + sizeof(WgEntry) * G.col.size());
    G.fin_off = off;
    off = align_up(off + sizeof(WgEntry) * G.fin.size());
  }
  pl.up_end = off;
  pl.total = off;
  return DQ_OK;
}

void bind_pointers(const dq_problem* p, int32_t count, int g, int fmt, int iters, char* ws,
                   Plan& pl) {
  static_assert(sizeof(ReportDev) == sizeof(dq_report) &&
                    offsetof(ReportDev, flags) == offsetof(dq_report, flags) &&
                    offsetof(ReportDev, sweeps) == offsetof(dq_report, sweeps),
                "device report layout differs from dq_report");
  for (int k = 0; k < count; ++k) {
    pl.dev[k].report = (ReportDev*)p[k].report;
    if (pl.group_of[k] < 0) continue;
    ProbDev& d = pl.dev[k];
    char* q = ws + pl.prob_off[k];
    auto take = [&](size_t bytes) { char* r = q; q += align_up(bytes); return r; };
    d.st = (State*)(ws + pl.live_off + kStatesOffset) + 2 * k;
    d.flags = (uint32_t*)take(2 * sizeof(uint32_t));
    d.altz = d.flags + 1;
    float* rr = (float*)take(7 * sizeof(float) * d.rows);
    for (int q = 0; q < 3; ++q) {
      d.r[q] = rr + q * d.rows;
      d.ir[q] = rr + (3 + q) * d.rows;
    }
    d.x_alt = rr + 6 * d.rows;
    float* cc = (float*)take(4 * sizeof(float) * d.cols);
    d.c[0] = cc; d.c[1] = cc + d.cols; d.ic[0] = cc + 2 * d.cols; d.ic[1] = cc + 3 * d.cols;
    d.codes[0] = p[k].codes;
    d.codes[1] = (uint8_t*)take(code_bytes(fmt, d.rows, d.cols));
    d.scales[0] = p[k].block_scales;
    d.scales[1] = take((size_t)d.rows * d.cols / g * scale_bytes(fmt));
    d.colP = take(partial_bytes(fmt, d.rranges, d.cols));
    d.swp = (double*)take((size_t)d.rowblocks * 4 * sizeof(double));
    d.fwp = (float*)take((size_t)d.fin_wgs * sizeof(float));
    d.initp = (double*)take((size_t)d.init_wgs * 2 * sizeof(double));
    double* hist = (double*)take(2 * (size_t)(iters + 1) * sizeof(double));
    d.nmse = p[k].nmse_hist ? p[k].nmse_hist : hist;
    d.relchg = p[k].relchg_hist ? p[k].relchg_hist : hist + (iters + 1);
    d.W = p[k].W;
    d.r_trace = p[k].r_trace;
    d.c_trace = p[k].c_trace;
    d.r_init = p[k].r_init;
    d.c_init = p[k].c_init;
    d.r_out = p[k].r;
    d.c_out = p[k].c;
    d.ts_out = fmt == DQ_FMT_NVFP4 ? p[k].tensor_scale : nullptr;
  }
}

// ---------------------------------------------------------------- template dispatch
template <int FMT>
constexpr int lanes_per_block(int g) { return g / 16; }

// Events attached to the next solver-pass launch (kernel begin / end timestamps, no extra
// stream packets); set by the iteration loop when per-kernel timing is requested.
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

template <typename K, typename... A>
void launch_timed(K kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t s, A... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, s, t_ev_start, t_ev_stop, 0u, args...);
  t_ev_start = nullptr;
  t_ev_stop = nullptr;
}

// Dynamic-LDS limit of a kernel that takes more than the default 64 KiB, set before each
// launch (on the current device; a cached flag would miss a second device).
bool lds_limit(const void* kernel, int bytes) {
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
}

#define DQ_HIP(call)                                   \
  do {                                                 \
    if ((call) != hipSuccess) return DQ_ERR_HIP;       \
  } while (0)

template <int FMT, int DT, int L>
int launch_passes(const Plan::Group& G, const ProbDev* probs, const WgEntry* rtab,
                  const WgEntry* ctab, hipStream_t s, int sw, int32_t* live) {
  const size_t rl = rowpass_lds_total(FMT, G.cols);
  const int compact = rowpass_compact(FMT, G.cols) ? 1 : 0;
  if (rowpass_cg(FMT, G.cols))
    launch_timed(k_rowpass<FMT, DT, L, 1>, dim3((unsigned)G.row.size()), dim3(kRowWaves * 64), rl,
                 s, probs, rtab, sw, (const int32_t*)live, compact);
  else
    launch_timed(k_rowpass<FMT, DT, L, 0>, dim3((unsigned)G.row.size()), dim3(kRowWaves * 64), rl,
                 s, probs, rtab, sw, (const int32_t*)live, compact);
  if (hipGetLastError() != hipSuccess) return DQ_ERR_HIP;
  return DQ_OK;
}

template <int FMT, int DT, int L>
int launch_colpass(const Plan::Group& G, const ProbDev* probs, const WgEntry* ctab, hipStream_t s,
                   int sw, int32_t* live) {
  if constexpr (grouped_int<FMT>())
    launch_timed(k_colpass_wide<FMT, DT, L>, dim3((unsigned)G.col.size()), dim3(512),
                 colpass_lds(FMT), s, probs, ctab, sw, (const int32_t*)live);
  else
    launch_timed(k_colpass<FMT, DT, L>, dim3((unsigned)G.col.size()), dim3(512), colpass_lds(FMT),
                 s, probs, ctab, sw, (const int32_t*)live);
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

template <int FMT, int L>
int launch_pass_dt(int which, const Plan::Group& G, const ProbDev* probs, const WgEntry* rtab,
                   const WgEntry* ctab, hipStream_t s, int sw, int32_t* live) {
  if (which == 0)
    return G.dtype == DQ_F32 ? launch_passes<FMT, 0, L>(G, probs, rtab, ctab, s, sw, live)
                             : launch_passes<FMT, 1, L>(G, probs, rtab, ctab, s, sw, live);
  return G.dtype == DQ_F32 ? launch_colpass<FMT, 0, L>(G, probs, ctab, s, sw, live)
                           : launch_colpass<FMT, 1, L>(G, probs, ctab, s, sw, live);
}

// Dynamic LDS limits of a group's pass kernels (set once per solve, before the launches).
template <int FMT, int DT, int L>
int prepare_passes(const Plan::Group& G) {
  const size_t rl = rowpass_lds_total(FMT, G.cols);
  if (rl > 64 * 1024 &&
      hipFuncSetAttribute(rowpass_cg(FMT, G.cols) ? (const void*)k_rowpass<FMT, DT, L, 1>
                                                  : (const void*)k_rowpass<FMT, DT, L, 0>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)rl) != hipSuccess)
    return DQ_ERR_HIP;
  if constexpr (grouped_int<FMT>()) {
    if (hipFuncSetAttribute((const void*)k_colpass_wide<FMT, DT, L>,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)colpass_lds(FMT)) != hipSuccess)
      return DQ_ERR_HIP;
  }
  return DQ_OK;
}

int prepare_passes_any(int fmt, int g, const Plan::Group& G) {
#define DQ_P(F, L) return G.dtype == DQ_F32 ? prepare_passes<F, 0, L>(G) : prepare_passes<F, 1, L>(G)
  switch (fmt) {
    case DQ_FMT_INT4:
      if (g == 64) { DQ_P(INT4, 4); }
      DQ_P(INT4, 8);
    case DQ_FMT_INT8:
      if (g == 64) { DQ_P(INT8, 4); }
      DQ_P(INT8, 8);
    case DQ_FMT_MXINT4: DQ_P(MXINT4, 2);
    case DQ_FMT_MXINT8: DQ_P(MXINT8, 2);
    case DQ_FMT_MXFP8_E4M3: DQ_P(MXFP8_E4M3, 2);
    case DQ_FMT_MXFP8_E5M2: DQ_P(MXFP8_E5M2, 2);
    case DQ_FMT_MXFP6_E2M3: DQ_P(MXFP6_E2M3, 2);
    case DQ_FMT_MXFP6_E3M2: DQ_P(MXFP6_E3M2, 2);
    case DQ_FMT_MXFP4: DQ_P(MXFP4, 2);
    default: DQ_P(NVFP4, 1);
  }
#undef DQ_P
}

// which = 0: row pass, 1: column pass
int launch_pass_any(int which, int fmt, int g, const Plan::Group& G, const ProbDev* probs,
                    const WgEntry* rtab, const WgEntry* ctab, hipStream_t s, int sw,
                    int32_t* live) {
  switch (fmt) {
    case DQ_FMT_INT4:
      return g == 64 ? launch_pass_dt<INT4, 4>(which, G, probs, rtab, ctab, s, sw, live)
                     : launch_pass_dt<INT4, 8>(which, G, probs, rtab, ctab, s, sw, live);
    case DQ_FMT_INT8:
      return g == 64 ? launch_pass_dt<INT8, 4>(which, G, probs, rtab, ctab, s, sw, live)
                     : launch_pass_dt<INT8, 8>(which, G, probs, rtab, ctab, s, sw, live);
    case DQ_FMT_MXINT4: return launch_pass_dt<MXINT4, 2>(which, G, probs, rtab, ctab, s, sw, live);
    case DQ_FMT_MXINT8: return launch_pass_dt<MXINT8, 2>(which, G, probs, rtab, ctab, s, sw, live);
    case DQ_FMT_MXFP8_E4M3: return launch_pass_dt<MXFP8_E4M3, 2>(which, G, probs, rtab, ctab, s, sw, live);
    case DQ_FMT_MXFP8_E5M2: return launch_pass_dt<MXFP8_E5M2, 2>(which, G, probs, rtab, ctab, s, sw, live);
    case DQ_FMT_MXFP6_E2M3: return launch_pass_dt<MXFP6_E2M3, 2>(which, G, probs, rtab, ctab, s, sw, live);
    case DQ_FMT_MXFP6_E3M2: return launch_pass_dt<MXFP6_E3M2, 2>(which, G, probs, rtab, ctab, s, sw, live);
    case DQ_FMT_MXFP4: return launch_pass_dt<MXFP4, 2>(which, G, probs, rtab, ctab, s, sw, live);
    default: return launch_pass_dt<NVFP4, 1>(which, G, probs, rtab, ctab, s, sw, live);
  }
}

int launch_finalize_any(int fmt, const Plan::Group& G, const ProbDev* probs,
                        const WgEntry* tab, hipStream_t s, int sw, int32_t* live) {
  dim3 grid((unsigned)G.fin.size()), block(256);
  switch (fmt) {
    case DQ_FMT_INT4: launch_timed(k_finalize<INT4>, grid, block, 0, s, probs, tab, sw, live); break;
    case DQ_FMT_INT8: launch_timed(k_finalize<INT8>, grid, block, 0, s, probs, tab, sw, live); break;
    case DQ_FMT_MXINT8: launch_timed(k_finalize<MXINT8>, grid, block, 0, s, probs, tab, sw, live); break;
    case DQ_FMT_MXFP8_E4M3: launch_timed(k_finalize<MXFP8_E4M3>, grid, block, 0, s, probs, tab, sw, live); break;
    case DQ_FMT_MXFP8_E5M2: launch_timed(k_finalize<MXFP8_E5M2>, grid, block, 0, s, probs, tab, sw, live); break;
    case DQ_FMT_MXFP6_E2M3: launch_timed(k_finalize<MXFP6_E2M3>, grid, block, 0, s, probs, tab, sw, live); break;
    case DQ_FMT_MXFP6_E3M2: launch_timed(k_finalize<MXFP6_E3M2>, grid, block, 0, s, probs, tab, sw, live); break;
    case DQ_FMT_MXINT4: launch_timed(k_finalize<MXINT4>, grid, block, 0, s, probs, tab, sw, live); break;
    case DQ_FMT_MXFP4: launch_timed(k_finalize<MXFP4>, grid, block, 0, s, probs, tab, sw, live); break;
    default: launch_timed(k_finalize<NVFP4>, grid, block, 0, s, probs, tab, sw, live); break;
  }
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

template <int FMT>
int launch_init_t(int dt, dim3 grid, const ProbDev* probs, hipStream_t s) {
  if (dt == DQ_F32) hipLaunchKernelGGL((k_init<FMT, 0>), grid, dim3(256), 0, s, probs);
  else hipLaunchKernelGGL((k_init<FMT, 1>), grid, dim3(256), 0, s, probs);
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

int launch_init_reduce_any(int fmt, int count, const ProbDev* probs, hipStream_t s) {
  dim3 grid((unsigned)count), block(256);
  switch (fmt) {
    case DQ_FMT_INT4: hipLaunchKernelGGL((k_init_reduce<INT4>), grid, block, 0, s, probs); break;
    case DQ_FMT_INT8: hipLaunchKernelGGL((k_init_reduce<INT8>), grid, block, 0, s, probs); break;
    case DQ_FMT_MXINT8: hipLaunchKernelGGL((k_init_reduce<MXINT8>), grid, block, 0, s, probs); break;
    case DQ_FMT_MXFP8_E4M3: hipLaunchKernelGGL((k_init_reduce<MXFP8_E4M3>), grid, block, 0, s, probs); break;
    case DQ_FMT_MXFP8_E5M2: hipLaunchKernelGGL((k_init_reduce<MXFP8_E5M2>), grid, block, 0, s, probs); break;
    case DQ_FMT_MXFP6_E2M3: hipLaunchKernelGGL((k_init_reduce<MXFP6_E2M3>), grid, block, 0, s, probs); break;
    case DQ_FMT_MXFP6_E3M2: hipLaunchKernelGGL((k_init_reduce<MXFP6_E3M2>), grid, block, 0, s, probs); break;
    case DQ_FMT_MXINT4: hipLaunchKernelGGL((k_init_reduce<MXINT4>), grid, block, 0, s, probs); break;
    case DQ_FMT_MXFP4: hipLaunchKernelGGL((k_init_reduce<MXFP4>), grid, block, 0, s, probs); break;
    default: hipLaunchKernelGGL((k_init_reduce<NVFP4>), grid, block, 0, s, probs); break;
  }
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

int launch_init_any(int fmt, int dt, dim3 grid, const ProbDev* probs, hipStream_t s) {
  switch (fmt) {
    case DQ_FMT_INT4: return launch_init_t<INT4>(dt, grid, probs, s);
    case DQ_FMT_INT8: return launch_init_t<INT8>(dt, grid, probs, s);
    case DQ_FMT_MXINT8: return launch_init_t<MXINT8>(dt, grid, probs, s);
    case DQ_FMT_MXFP8_E4M3: return launch_init_t<MXFP8_E4M3>(dt, grid, probs, s);
    case DQ_FMT_MXFP8_E5M2: return launch_init_t<MXFP8_E5M2>(dt, grid, probs, s);
    case DQ_FMT_MXFP6_E2M3: return launch_init_t<MXFP6_E2M3>(dt, grid, probs, s);
    case DQ_FMT_MXFP6_E3M2: return launch_init_t<MXFP6_E3M2>(dt, grid, probs, s);
    case DQ_FMT_MXINT4: return launch_init_t<MXINT4>(dt, grid, probs, s);
    case DQ_FMT_MXFP4: return launch_init_t<MXFP4>(dt, grid, probs, s);
    default: return launch_init_t<NVFP4>(dt, grid, probs, s);
  }
}

// Row ranges of the amax pre-pass: at most nparts workgroups in all, and at least
// kAmaxMinRows rows per thread so each workgroup's fixed work (column scales, reduction)
// is amortised over enough rows.
constexpr int64_t kAmaxMinRows = 16;
int64_t amax_ranges(int64_t rows, int nstrips, int nparts) {
  const int64_t by_rows = std::max<int64_t>(1, rows / kAmaxMinRows);
  return std::max<int64_t>(1, std::min<int64_t>(by_rows, nparts / nstrips));
}

// Standalone quantiser (weights: MODEV 0; activations: MODEV 1).  The quantiser grid is
// capped so each workgroup handles several row groups.
constexpr int64_t kQuantGroupsMax = 256;
template <int FMT, int DT, int L, int MODEV>
int launch_quant_t(const void* X, int64_t rows, int64_t cols, int64_t ld, const float* r,
                   const float* c, uint8_t* codes, void* scales, float* ts, float* part,
                   int nparts, hipStream_t s) {
  if (FMT == NVFP4) {
    const int64_t nv = cols / (DT == DQ_F32 ? 4 : 8);
    const int nstrips = (int)((nv + 255) / 256);
    const int64_t ranges = amax_ranges(rows, nstrips, nparts);
    const int rpr = (int)((rows + ranges - 1) / ranges);
    const int nwg = nstrips * (int)((rows + rpr - 1) / rpr);   // <= nparts
    nparts = nwg;
    hipLaunchKernelGGL((k_qamax<DT, MODEV>), dim3((unsigned)nwg), dim3(256), 0, s, X, rows, cols,
                       ld, r, c, part, nstrips, rpr);
  }
  const int lpr = lanes_per_row(cols), H = quant_rows_per_group(lpr, rows, kQuantGroupsMax);
  const int64_t groups = (rows + H - 1) / H;
  const unsigned grid = (unsigned)std::min<int64_t>(groups, kQuantGroupsMax);
  for (int lbeg = 0; lbeg < cols / 16; lbeg += lpr)   // one launch per 16384 columns
    hipLaunchKernelGGL((k_quant<FMT, DT, L, MODEV>), dim3(grid), dim3(lpr * H), 0, s, X, rows,
                       cols, ld, r, c, codes, scales, ts, part, nparts, lpr, H, lbeg);
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

template <int MODEV>
int launch_quant_any(int fmt, int g, int dt, const void* X, int64_t rows, int64_t cols,
                     int64_t ld, const float* r, const float* c, uint8_t* codes, void* scales,
                     float* ts, float* part, int nparts, hipStream_t s) {
#define DQ_Q(F, L)                                                                           \
  return dt == DQ_F32                                                                        \
             ? launch_quant_t<F, 0, L, MODEV>(X, rows, cols, ld, r, c, codes, scales, ts,    \
                                              part, nparts, s)                               \
             : launch_quant_t<F, 1, L, MODEV>(X, rows, cols, ld, r, c, codes, scales, ts,    \
                                              part, nparts, s)
  switch (fmt) {
    case DQ_FMT_INT4:
      if (g == 64) { DQ_Q(INT4, 4); }
      DQ_Q(INT4, 8);
    case DQ_FMT_INT8:
      if (g == 64) { DQ_Q(INT8, 4); }
      DQ_Q(INT8, 8);
    case DQ_FMT_MXINT4: DQ_Q(MXINT4, 2);
    case DQ_FMT_MXINT8: DQ_Q(MXINT8, 2);
    case DQ_FMT_MXFP8_E4M3: DQ_Q(MXFP8_E4M3, 2);
    case DQ_FMT_MXFP8_E5M2: DQ_Q(MXFP8_E5M2, 2);
    case DQ_FMT_MXFP6_E2M3: DQ_Q(MXFP6_E2M3, 2);
    case DQ_FMT_MXFP6_E3M2: DQ_Q(MXFP6_E3M2, 2);
    case DQ_FMT_MXFP4: DQ_Q(MXFP4, 2);
    default: DQ_Q(NVFP4, 1);
  }
#undef DQ_Q
}

constexpr int kQuantParts = 1024;

// ---------------------------------------------------------------- no-allocation scratch
// The scratch of dq_rescale_quantize_acts_noalloc: the NVFP4 amax pre-pass partials (one per
// pre-pass workgroup, at most kQuantParts).  Every GPU the library runs on holds its own
// copy until the process ends.  Host code never uses this name as an address: the kernels
// get the device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[kQuantParts];
static_assert(sizeof(scratch) == DQ_NOALLOC_SCRATCH_BYTES, "scratch size and header differ");
constexpr int kMaxScratchDevices = 64;

// Device address of `scratch` on the current device, looked up once per device.
int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxScratchDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return DQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DQ_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return DQ_OK;
}

// Quantised linear layer: dynamic LDS above 64 KiB is opted into once per instantiation.
// FP4 codes with K a multiple of 256 and FP8 codes with K a multiple of 128, with 4-byte
// aligned scale arrays, take the direct-to-LDS ring; everything else the register-staged
// kernel.
template <int FMT, int OB>
int launch_linear(dim3 grid, hipStream_t s, const LinArgs& p) {
  if constexpr (elem_bits<FMT>() != 6) {
    if (p.K % DmaGeom<FMT>::KS == 0 && ((uintptr_t)p.as & 3u) == 0 && ((uintptr_t)p.bs & 3u) == 0) {
      if (!lds_limit((const void*)k_linear_dma<FMT, OB>, DmaGeom<FMT>::LDS)) return DQ_ERR_HIP;
      hipLaunchKernelGGL((k_linear_dma<FMT, OB>), grid, dim3(256), DmaGeom<FMT>::LDS, s, p);
      return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
    }
  }
  if (!lds_limit((const void*)k_linear<FMT, OB>, LinGeom<FMT>::LDS)) return DQ_ERR_HIP;
  hipLaunchKernelGGL((k_linear<FMT, OB>), grid, dim3(256), LinGeom<FMT>::LDS, s, p);
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

template <int OB>
int launch_linear_nv(dim3 grid, hipStream_t s, const LinArgs& p) {
  // codes through LDS where K is a multiple of the 128-K stage and the scale arrays allow
  // 4-byte loads; otherwise dequantised into LDS (any K that is a multiple of 32)
  if (p.K % NvDmaGeom::KS == 0 && ((uintptr_t)p.as & 3u) == 0 && ((uintptr_t)p.bs & 3u) == 0) {
    hipLaunchKernelGGL((k_linear_nv_dma<OB>), grid, dim3(256), NvDmaGeom::LDS, s, p);   // 54 KiB
    return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
  }
  hipLaunchKernelGGL((k_linear_nv<OB>), grid, dim3(256), NvGeom::LDS, s, p);   // 64 KiB
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

template <int GS, int OB, int TM>
int launch_linear_i4(dim3 grid, hipStream_t s, const LinArgs& p) {
  if (!lds_limit((const void*)k_linear_i4<GS, OB, TM>, I4Geom<TM>::LDS)) return DQ_ERR_HIP;
  hipLaunchKernelGGL((k_linear_i4<GS, OB, TM>), grid, dim3(256), I4Geom<TM>::LDS, s, p);   // 72 / 45 KiB
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}
template <int GS, int OB>
int launch_linear_i4_tm(int tm_rows, dim3 grid, hipStream_t s, const LinArgs& p) {
  return tm_rows == 32 ? launch_linear_i4<GS, OB, 32>(grid, s, p) : launch_linear_i4<GS, OB, 128>(grid, s, p);
}

static_assert(kMaxMulti == DQ_MAX_MULTI, "kernel and header output limits differ");
// The fused activation quantiser keeps every output's column scales in LDS up to this size
// (q/k/v or gate/up of a 4096-wide model need 48 or 32 KiB); beyond it they are read from
// memory per row.
constexpr size_t kMultiCLds = 96 * 1024;

template <int FMT, int DT, int L>
int launch_quant_multi_t(const void* X, int64_t rows, int64_t cols, int64_t ld,
                         const MultiOut& mo, float* part, int nparts, hipStream_t s) {
  if (FMT == NVFP4) {
    const int64_t nv = cols / (DT == DQ_F32 ? 4 : 8);
    const int nstrips = (int)((nv + 255) / 256);
    const int64_t ranges = amax_ranges(rows, nstrips, nparts);
    const int rpr = (int)((rows + ranges - 1) / ranges);
    const int nwg = nstrips * (int)((rows + rpr - 1) / rpr);   // <= nparts
    nparts = nwg;
    hipLaunchKernelGGL((k_qamax_multi<DT>), dim3((unsigned)nwg), dim3(256), 0, s, X, rows, cols,
                       ld, mo, part, nstrips, rpr);
  }
  const int lpr = lanes_per_row(cols), H = quant_rows_per_group(lpr, rows, kQuantGroupsMax);
  const int64_t groups = (rows + H - 1) / H;
  const unsigned grid = (unsigned)std::min<int64_t>(groups, kQuantGroupsMax);
  const size_t c_bytes = (size_t)mo.count * cols * sizeof(float);
  // c is staged in LDS when it fits and every workgroup quantises two or more row groups;
  // with one group per workgroup (a few tokens) the staging is a round of load latency that
  // the rows do not pay back, and each row reads its c from L2 alongside its X instead
  const int64_t groups_per_wg = (groups + grid - 1) / grid;
  const int c_lds = (c_bytes <= kMultiCLds && groups_per_wg >= 2) ? 1 : 0;
  if (c_lds && c_bytes > 64 * 1024) {
    if (!lds_limit((const void*)k_quant_multi<FMT, DT, L>, (int)kMultiCLds)) return DQ_ERR_HIP;
  }
  for (int lbeg = 0; lbeg < cols / 16; lbeg += lpr)   // one launch per 16384 columns
    hipLaunchKernelGGL((k_quant_multi<FMT, DT, L>), dim3(grid), dim3(lpr * H),
                       c_lds ? c_bytes : 0, s, X, rows, cols, ld, mo, part, nparts, lpr, H, c_lds,
                       lbeg);
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

int launch_quant_multi_any(int fmt, int g, int dt, const void* X, int64_t rows, int64_t cols,
                           int64_t ld, const MultiOut& mo, float* part, int nparts,
                           hipStream_t s) {
#define DQ_Q(F, L)                                                                     \
  return dt == DQ_F32 ? launch_quant_multi_t<F, 0, L>(X, rows, cols, ld, mo, part, nparts, s) \
                      : launch_quant_multi_t<F, 1, L>(X, rows, cols, ld, mo, part, nparts, s)
  switch (fmt) {
    case DQ_FMT_INT4:
      if (g == 64) { DQ_Q(INT4, 4); }
      DQ_Q(INT4, 8);
    case DQ_FMT_INT8:
      if (g == 64) { DQ_Q(INT8, 4); }
      DQ_Q(INT8, 8);
    case DQ_FMT_MXINT4: DQ_Q(MXINT4, 2);
    case DQ_FMT_MXINT8: DQ_Q(MXINT8, 2);
    case DQ_FMT_MXFP8_E4M3: DQ_Q(MXFP8_E4M3, 2);
    case DQ_FMT_MXFP8_E5M2: DQ_Q(MXFP8_E5M2, 2);
    case DQ_FMT_MXFP6_E2M3: DQ_Q(MXFP6_E2M3, 2);
    case DQ_FMT_MXFP6_E3M2: DQ_Q(MXFP6_E3M2, 2);
    case DQ_FMT_MXFP4: DQ_Q(MXFP4, 2);
    default: DQ_Q(NVFP4, 1);
  }
#undef DQ_Q
}

}  // namespace

// ============================================================================ C ABI
extern "C" {

const char* dq_status_string(int status) {
  switch (status) {
    case DQ_OK: return "ok";
    case DQ_ERR_NULL: return "a required pointer is NULL";
    case DQ_ERR_SHAPE: return "invalid shape (rows/cols/ld, cols not a multiple of the group, or cols > 65536)";
    case DQ_ERR_ALIGN: return "base pointer or row pitch not 16-byte aligned";
    case DQ_ERR_FORMAT: return "unknown format, group or dtype";
    case DQ_ERR_WORKSPACE: return "workspace missing or too small";
    case DQ_ERR_HIP: return "HIP runtime error";
    case DQ_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

static int validate_solve(const dq_problem* p, int32_t count, dq_quant_spec spec,
                          const dq_solve_opts* o, int* g_out) {
  if (!p || !o) return DQ_ERR_NULL;
  if (count < 1 || count > 65535) return DQ_ERR_ARG;   // problems index the grid's y dimension
  int g = resolve_group(spec);
  if (g < 0) return DQ_ERR_FORMAT;
  if (o->iters < 0 || o->iters > kMaxIters || !(o->tol_relchg >= 0.0f)) return DQ_ERR_ARG;
  if (o->scale_steps < 0 || o->scale_steps > (DQ_STEP_ROW | DQ_STEP_COL)) return DQ_ERR_ARG;
  for (int k = 0; k < count; ++k) {
    int rc = check_matrix(p[k].W, p[k].w_dtype, p[k].rows, p[k].cols, p[k].ld, g);
    if (rc) return rc;
    if (p[k].report && ((uintptr_t)p[k].report & 3u)) return DQ_ERR_ALIGN;
    if (p[k].rows == 0 || p[k].cols == 0) continue;
    if (!p[k].r || !p[k].c || !p[k].codes || !p[k].block_scales) return DQ_ERR_NULL;
    if (spec.fmt == DQ_FMT_NVFP4 && !p[k].tensor_scale) return DQ_ERR_NULL;
    if (!aligned16(p[k].codes) || !aligned16(p[k].block_scales)) return DQ_ERR_ALIGN;
    if (p[k].r_init && !aligned16(p[k].r_init)) return DQ_ERR_ALIGN;
    if (p[k].c_init && !aligned16(p[k].c_init)) return DQ_ERR_ALIGN;
  }
  *g_out = g;
  return DQ_OK;
}

size_t dq_workspace_bytes(const dq_problem* problems, int32_t count, dq_quant_spec spec,
                          const dq_solve_opts* opts) {
  int g = 0;
  if (validate_solve(problems, count, spec, opts, &g) != DQ_OK) return 0;
  Plan pl;
  make_plan(problems, count, g, spec.fmt, opts->iters, pl);
  return pl.total;
}

// Sweeps a solve of T iterations queues: the INIT sweep and one per iteration.  Each sweep
// computes the next r and c steps for both outcomes of its safeguard, so a rejected step
// costs no extra sweep.
static int max_sweeps(int iters) { return iters + 1; }

// The solve, stream-ordered.  With `timed_sweeps` > 0, a begin/end event pair is attached to
// each pass's launches (row pass, column pass, finalize + decision, all groups) of the first
// `timed_sweeps` queued sweeps; the events are read later (dq_solve_timed_read), once the
// caller's stream has run them, so timing adds no wait to the stream.
//
// Those events are created once per device and kept for the process (six per sweep created
// on every call cost host time the GPU spent idle), with the number of sweeps the last timed
// solve on the device attached them to.  The lock guards that state; timed solves on one
// device must not overlap between their enqueue and their read.
static std::mutex g_timing_mu;
static std::vector<hipEvent_t> g_timing_events[64];
static int32_t g_timing_count[64];

static int solve_impl(const dq_problem* problems, int32_t count, dq_quant_spec spec,
                      const dq_solve_opts* opts, void* workspace, size_t workspace_bytes,
                      void* stream, int32_t timed_sweeps) {
  int g = 0;
  int rc = validate_solve(problems, count, spec, opts, &g);
  if (rc) return rc;
  Plan pl;
  make_plan(problems, count, g, spec.fmt, opts->iters, pl);
  if (!workspace) return DQ_ERR_WORKSPACE;
  if (workspace_bytes < pl.total) return DQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DQ_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  bind_pointers(problems, count, g, spec.fmt, opts->iters, ws, pl);
  for (auto& d : pl.dev) {
    d.tol = opts->tol_relchg;
    d.steps = opts->scale_steps ? opts->scale_steps : (DQ_STEP_ROW | DQ_STEP_COL);
  }
  const int iters = opts->iters;
  const int nsw = max_sweeps(iters);

  // the timing events, before anything is enqueued
  std::unique_lock<std::mutex> timing_lock(g_timing_mu, std::defer_lock);
  std::vector<hipEvent_t>* evp = nullptr;
  int32_t* timed_count = nullptr;
  if (timed_sweeps > 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DQ_ERR_HIP;
    timing_lock.lock();
    evp = &g_timing_events[dev];
    timed_count = &g_timing_count[dev];
    *timed_count = 0;
    const size_t need = 6 * (size_t)std::min(nsw, (int)timed_sweeps);
    while (evp->size() < need) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return DQ_ERR_HIP;
      evp->push_back(e);
    }
  }

  // empty problems: zero histories (their reports come from the outputs kernel)
  for (int k = 0; k < count; ++k) {
    if (pl.group_of[k] >= 0) continue;
    if (problems[k].nmse_hist)
      DQ_HIP(hipMemsetAsync(problems[k].nmse_hist, 0, sizeof(double) * (iters + 1), s));
    if (problems[k].relchg_hist)
      DQ_HIP(hipMemsetAsync(problems[k].relchg_hist, 0, sizeof(double) * (iters + 1), s));
  }

  // the live-problem counter, the problem descriptors and every launch table, in one upload
  // (the runtime stages pageable host memory before the call returns)
  ProbDev* dprobs = (ProbDev*)(ws + pl.probs_off);
  int32_t* live = (int32_t*)(ws + pl.live_off);
  std::vector<char> up(pl.up_end - pl.live_off);
  std::memcpy(up.data(), &pl.live, sizeof(int32_t));
  std::memcpy(up.data() + (pl.probs_off - pl.live_off), pl.dev.data(), sizeof(ProbDev) * count);
  for (auto& G : pl.groups) {
    std::memcpy(up.data() + (G.row_off - pl.live_off), G.row.data(), sizeof(WgEntry) * G.row.size());
    std::memcpy(up.data() + (G.col_off - pl.live_off), G.col.data(), sizeof(WgEntry) * G.col.size());
    std::memcpy(up.data() + (G.fin_off - pl.live_off), G.fin.data(), sizeof(WgEntry) * G.fin.size());
  }
  DQ_HIP(hipMemcpyAsync(live, up.data(), up.size(), hipMemcpyHostToDevice, s));

  if (!pl.groups.empty()) {
    int64_t maxdim = 1;
    int max_init = 1;
    for (int k = 0; k < count; ++k) {
      if (pl.group_of[k] < 0) continue;
      maxdim = std::max(maxdim, std::max(pl.dev[k].rows, pl.dev[k].cols));
      max_init = std::max(max_init, pl.dev[k].init_wgs);
    }
    hipLaunchKernelGGL(k_setup, dim3((unsigned)((maxdim + 255) / 256), (unsigned)count), dim3(256),
                       0, s, dprobs);
    DQ_HIP(hipGetLastError());
    for (int dt = 0; dt < 2; ++dt) {
      bool any = false;
      for (int k = 0; k < count; ++k) any |= (pl.group_of[k] >= 0 && problems[k].w_dtype == dt);
      if (!any) continue;
      rc = launch_init_any(spec.fmt, dt, dim3((unsigned)max_init, (unsigned)count), dprobs, s);
      if (rc) return rc;
    }
    rc = launch_init_reduce_any(spec.fmt, count, dprobs, s);
    if (rc) return rc;
    for (auto& G : pl.groups) {
      rc = prepare_passes_any(spec.fmt, g, G);
      if (rc) return rc;
    }
    // Every sweep a solve may need is queued now; a sweep whose problems are all finished
    // exits at its first instruction (the live counter), so nothing waits on the host.
    const size_t ng = pl.groups.size();
    for (int sw = 0; sw < nsw; ++sw) {
      const bool tm = timed_count && *timed_count < timed_sweeps;
      hipEvent_t e[6] = {};
      if (tm)
        for (int q = 0; q < 6; ++q) e[q] = (*evp)[6 * (size_t)*timed_count + q];
      for (int which = 0; which < 3; ++which) {
        for (size_t gi = 0; gi < ng; ++gi) {
          const auto& G = pl.groups[gi];
          if (tm) {
            t_ev_start = gi == 0 ? e[2 * which] : nullptr;
            t_ev_stop = gi + 1 == ng ? e[2 * which + 1] : nullptr;
          }
          rc = which < 2 ? launch_pass_any(which, spec.fmt, g, G, dprobs,
                                           (const WgEntry*)(ws + G.row_off),
                                           (const WgEntry*)(ws + G.col_off), s, sw, live)
                         : launch_finalize_any(spec.fmt, G, dprobs,
                                               (const WgEntry*)(ws + G.fin_off), s, sw, live);
          t_ev_start = t_ev_stop = nullptr;
          if (rc) return rc;
        }
      }
      if (tm) ++*timed_count;
    }
  }
  // outputs and device reports: workgroups per problem of the outputs kernel -- one 64-byte
  // slice per thread of the largest code copy, at most 2048 per problem and about 64 K over
  // the batch (a problem whose kept codes are already in the caller's buffer leaves them idle)
  int64_t max_copy = 1;
  for (int k = 0; k < count; ++k)
    if (pl.group_of[k] >= 0)
      max_copy = std::max<int64_t>(max_copy, (int64_t)code_bytes(spec.fmt, pl.dev[k].rows, pl.dev[k].cols));
  const int64_t out_x = std::max<int64_t>(
      1, std::min<int64_t>({(max_copy + 16383) / 16384, 2048, std::max<int64_t>(1, 65536 / count)}));
  hipLaunchKernelGGL(k_outputs, dim3((unsigned)out_x, (unsigned)count), dim3(256), 0, s, dprobs,
                     code_bits(spec.fmt), scale_bytes(spec.fmt), g);
  if (hipGetLastError() != hipSuccess) return DQ_ERR_HIP;
  return DQ_OK;
}

int dq_solve(const dq_problem* problems, int32_t count, dq_quant_spec spec,
             const dq_solve_opts* opts, void* workspace, size_t workspace_bytes, void* stream) {
  return solve_impl(problems, count, spec, opts, workspace, workspace_bytes, stream, 0);
}

int dq_solve_timed_enqueue(const dq_problem* problems, int32_t count, dq_quant_spec spec,
                           const dq_solve_opts* opts, void* workspace, size_t workspace_bytes,
                           void* stream, int32_t timed_sweeps) {
  if (timed_sweeps < 1) return DQ_ERR_ARG;
  return solve_impl(problems, count, spec, opts, workspace, workspace_bytes, stream, timed_sweeps);
}

int dq_solve_timed_read(float* pass_ms, int32_t pass_ms_capacity, int32_t* pass_ms_count) {
  if (!pass_ms || !pass_ms_count) return DQ_ERR_NULL;
  if (pass_ms_capacity < 0) return DQ_ERR_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_timing_mu);
  const std::vector<hipEvent_t>& ev = g_timing_events[dev];
  const int32_t n = std::min(g_timing_count[dev], pass_ms_capacity);
  for (int k = 0; k < n; ++k)
    for (int q = 0; q < 3; ++q) {
      float ms = 0.0f;
      // hipErrorNotReady: the stream has not run the timed launches yet
      if (hipEventElapsedTime(&ms, ev[6 * k + 2 * q], ev[6 * k + 2 * q + 1]) != hipSuccess)
        return DQ_ERR_HIP;
      pass_ms[3 * k + q] = ms;
    }
  *pass_ms_count = n;
  return DQ_OK;
}

int dq_solve_timed(const dq_problem* problems, int32_t count, dq_quant_spec spec,
                   const dq_solve_opts* opts, void* workspace, size_t workspace_bytes,
                   void* stream, float* pass_ms, int32_t pass_ms_capacity,
                   int32_t* pass_ms_count) {
  if (!pass_ms || !pass_ms_count) return DQ_ERR_NULL;
  if (pass_ms_capacity < 0) return DQ_ERR_ARG;
  int rc = pass_ms_capacity > 0
               ? solve_impl(problems, count, spec, opts, workspace, workspace_bytes, stream,
                            pass_ms_capacity)
               : solve_impl(problems, count, spec, opts, workspace, workspace_bytes, stream, 0);
  if (rc) return rc;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DQ_ERR_HIP;
  if (pass_ms_capacity == 0) {
    *pass_ms_count = 0;
    return DQ_OK;
  }
  return dq_solve_timed_read(pass_ms, pass_ms_capacity, pass_ms_count);
}

size_t dq_quantize_workspace_bytes(int64_t rows, int64_t cols, dq_quant_spec spec) {
  (void)rows;
  (void)cols;
  return spec.fmt == DQ_FMT_NVFP4 ? kQuantParts * sizeof(float) : 0;
}

static int quantize_common(int modev, const void* X, int32_t dt, int64_t rows, int64_t cols,
                           int64_t ld, const float* r, const float* c, dq_quant_spec spec,
                           uint8_t* codes, void* scales, float* ts, void* ws, size_t wsb,
                           void* stream) {
  int g = resolve_group(spec);
  if (g < 0) return DQ_ERR_FORMAT;
  int rc = check_matrix(X, dt, rows, cols, ld, g);
  if (rc) return rc;
  if (rows == 0 || cols == 0) return DQ_OK;
  if (!codes || !scales) return DQ_ERR_NULL;
  if (spec.fmt == DQ_FMT_NVFP4 && !ts) return DQ_ERR_NULL;
  if (!aligned16(codes) || !aligned16(scales)) return DQ_ERR_ALIGN;
  if (spec.fmt == DQ_FMT_NVFP4) {
    if (!ws) return DQ_ERR_WORKSPACE;
    if (wsb < dq_quantize_workspace_bytes(rows, cols, spec)) return DQ_ERR_WORKSPACE;
  }
  hipStream_t s = (hipStream_t)stream;
  if (modev == 0)
    return launch_quant_any<0>(spec.fmt, g, dt, X, rows, cols, ld, r, c, codes, scales, ts,
                               (float*)ws, kQuantParts, s);
  return launch_quant_any<1>(spec.fmt, g, dt, X, rows, cols, ld, nullptr, c, codes, scales, ts,
                             (float*)ws, kQuantParts, s);
}

int dq_quantize_weights(const void* W, int32_t w_dtype, int64_t rows, int64_t cols, int64_t ld,
                        const float* r, const float* c, dq_quant_spec spec, uint8_t* codes,
                        void* block_scales, float* tensor_scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return quantize_common(0, W, w_dtype, rows, cols, ld, r, c, spec, codes, block_scales,
                         tensor_scale, workspace, workspace_bytes, stream);
}

int dq_rescale_quantize_acts(const void* X, int32_t x_dtype, int64_t tokens, int64_t cols,
                             int64_t ld, const float* c, dq_quant_spec spec, uint8_t* codes,
                             void* block_scales, float* tensor_scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return quantize_common(1, X, x_dtype, tokens, cols, ld, nullptr, c, spec, codes, block_scales,
                         tensor_scale, workspace, workspace_bytes, stream);
}

int dq_rescale_quantize_acts_noalloc(const void* X, int32_t x_dtype, int64_t tokens,
                                     int64_t cols, int64_t ld, const float* c,
                                     dq_quant_spec spec, uint8_t* codes, void* block_scales,
                                     float* tensor_scale, void* stream) {
  // argument checks first, exactly as the workspace variant makes them
  int g = resolve_group(spec);
  if (g < 0) return DQ_ERR_FORMAT;
  int rc = check_matrix(X, x_dtype, tokens, cols, ld, g);
  if (rc) return rc;
  if (tokens == 0 || cols == 0) return DQ_OK;
  const size_t need = dq_quantize_workspace_bytes(tokens, cols, spec);
  if (need > sizeof(scratch)) return DQ_ERR_WORKSPACE;
  if (need == 0)   // this format's kernels use no scratch
    return quantize_common(1, X, x_dtype, tokens, cols, ld, nullptr, c, spec, codes,
                           block_scales, tensor_scale, nullptr, 0, stream);
  // the scratch is the current device's: the stream must run there
  int dev = -1;
  hipDevice_t sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DQ_ERR_HIP;
  if (stream) {
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return DQ_ERR_HIP;
    if (sdev != dev) return DQ_ERR_ARG;
  }
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return quantize_common(1, X, x_dtype, tokens, cols, ld, nullptr, c, spec, codes, block_scales,
                         tensor_scale, ws, sizeof(scratch), stream);
}

size_t dq_quantize_multi_workspace_bytes(int64_t tokens, int64_t cols, int32_t count,
                                         dq_quant_spec spec) {
  (void)tokens;
  (void)cols;
  if (count < 1 || count > DQ_MAX_MULTI) return 0;
  return spec.fmt == DQ_FMT_NVFP4 ? (size_t)count * kQuantParts * sizeof(float) : 0;
}

int dq_rescale_quantize_acts_multi(const void* X, int32_t x_dtype, int64_t tokens,
                                   int64_t cols, int64_t ld, int32_t count,
                                   const float* const* c, dq_quant_spec spec,
                                   uint8_t* const* codes, void* const* block_scales,
                                   float* const* tensor_scales, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (count < 1 || count > DQ_MAX_MULTI) return DQ_ERR_ARG;
  int g = resolve_group(spec);
  if (g < 0) return DQ_ERR_FORMAT;
  int rc = check_matrix(X, x_dtype, tokens, cols, ld, g);
  if (rc) return rc;
  if (tokens == 0 || cols == 0) return DQ_OK;
  if (!codes || !block_scales) return DQ_ERR_NULL;
  if (spec.fmt == DQ_FMT_NVFP4 && !tensor_scales) return DQ_ERR_NULL;
  MultiOut mo{};
  mo.count = count;
  for (int k = 0; k < count; ++k) {
    if (!codes[k] || !block_scales[k]) return DQ_ERR_NULL;
    if (!aligned16(codes[k]) || !aligned16(block_scales[k])) return DQ_ERR_ALIGN;
    if (spec.fmt == DQ_FMT_NVFP4 && !tensor_scales[k]) return DQ_ERR_NULL;
    mo.c[k] = c ? c[k] : nullptr;
    mo.codes[k] = codes[k];
    mo.scales[k] = block_scales[k];
    mo.ts[k] = (spec.fmt == DQ_FMT_NVFP4) ? tensor_scales[k] : nullptr;
  }
  if (spec.fmt == DQ_FMT_NVFP4) {
    if (!workspace) return DQ_ERR_WORKSPACE;
    if (workspace_bytes < dq_quantize_multi_workspace_bytes(tokens, cols, count, spec))
      return DQ_ERR_WORKSPACE;
  }
  return launch_quant_multi_any(spec.fmt, g, x_dtype, X, tokens, cols, ld, mo,
                                (float*)workspace, kQuantParts, (hipStream_t)stream);
}

// Rows of the INT4 layer's activation tile: 32 for a few tokens (up to 96: 82 tokens fill
// three tiles of 32 rather than one of 128), else 128.
static int i4_tile_m(int64_t M) { return M <= 96 ? 32 : 128; }
// Split K for the INT4 layer when its output tiles alone cannot fill the GPU twice over (few
// tokens): about two workgroups per CU, but no more splits than the stages of K, and partial
// sums at most twice the weight codes (K / 4M splits of M x N fp32 against N x K / 2
// bytes).  With 32-row tiles, whose stages are short, up to 511 tiles are split in two: a
// 14336-wide layer at 82 tokens (336 tiles) would otherwise run 16 stages back to back.
static void i4_split(int64_t M, int64_t N, int64_t K, int& ksplit, int& st_split) {
  const int tmr = i4_tile_m(M);
  const int64_t tiles = ((M + tmr - 1) / tmr) * ((N + kLinTile - 1) / kLinTile);
  const int64_t nst = (K / 64 + 3) / 4;   // stages of 256 K
  int64_t k = 1;
  if (tiles > 0 && tiles < (tmr == 32 ? 512 : 256) && nst > 1) {
    k = (512 + tiles - 1) / tiles;
    k = std::min<int64_t>(k, std::max<int64_t>(1, K / (4 * std::max<int64_t>(M, 1))));
    k = std::min<int64_t>(std::min<int64_t>(k, nst), 64);
  }
  const int64_t per = nst > 0 ? (nst + k - 1) / k : 0;
  st_split = (int)per;
  ksplit = per > 0 ? (int)((nst + per - 1) / per) : 1;
}
static int64_t i4_part_pitch(int64_t N) { return (N + 3) & ~(int64_t)3; }

size_t dq_quantized_linear_workspace_bytes(dq_quant_spec spec, int64_t M, int64_t N, int64_t K) {
  if (spec.fmt != DQ_FMT_INT4 || resolve_group(spec) < 0 || M <= 0 || N <= 0 || K <= 0) return 0;
  int ks = 1, per = 0;
  i4_split(M, N, K, ks, per);
  return ks > 1 ? (size_t)ks * (size_t)M * (size_t)i4_part_pitch(N) * sizeof(float) : 0;
}

int dq_quantized_linear(dq_quant_spec spec, const uint8_t* a_codes, const uint8_t* a_scales,
                        const float* a_tensor_scale, int64_t M, const uint8_t* b_codes,
                        const uint8_t* b_scales, const float* b_tensor_scale, int64_t N,
                        int64_t K, const float* r, void* y, int32_t y_dtype, int64_t ldy,
                        void* stream) {
  return dq_quantized_linear_ws(spec, a_codes, a_scales, a_tensor_scale, M, b_codes, b_scales,
                                b_tensor_scale, N, K, r, y, y_dtype, ldy, nullptr, 0, stream);
}

int dq_quantized_linear_ws(dq_quant_spec spec, const uint8_t* a_codes, const uint8_t* a_scales,
                           const float* a_tensor_scale, int64_t M, const uint8_t* b_codes,
                           const uint8_t* b_scales, const float* b_tensor_scale, int64_t N,
                           int64_t K, const float* r, void* y, int32_t y_dtype, int64_t ldy,
                           void* workspace, size_t workspace_bytes, void* stream) {
  const int g = resolve_group(spec);
  if (g < 0) return DQ_ERR_FORMAT;
  const int f = spec.fmt;
  const bool nv = f == DQ_FMT_NVFP4, i4 = f == DQ_FMT_INT4;
  if (f != DQ_FMT_MXFP4 && f != DQ_FMT_MXFP8_E4M3 && f != DQ_FMT_MXFP8_E5M2 &&
      f != DQ_FMT_MXFP6_E2M3 && f != DQ_FMT_MXFP6_E3M2 && !nv && !i4)
    return DQ_ERR_FORMAT;
  if (y_dtype != DQ_F32 && y_dtype != DQ_BF16) return DQ_ERR_FORMAT;
  if (M < 0 || N < 0 || K < 0 || K % (i4 ? g : 32) || ldy < N) return DQ_ERR_SHAPE;
  if (M == 0 || N == 0) return DQ_OK;
  if (!y) return DQ_ERR_NULL;
  if (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales)) return DQ_ERR_NULL;
  if (nv && (!a_tensor_scale || !b_tensor_scale)) return DQ_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(b_codes) || ((uintptr_t)y % (y_dtype == DQ_F32 ? 4 : 2)))
    return DQ_ERR_ALIGN;
  if (i4 && (((uintptr_t)a_scales | (uintptr_t)b_scales) & 1u)) return DQ_ERR_ALIGN;   // bf16
  const int tm_rows = i4 ? i4_tile_m(M) : kLinTile;   // rows of the activation tile
  const int64_t tm = (M + tm_rows - 1) / tm_rows, tn = (N + kLinTile - 1) / kLinTile;
  if (tm * tn > (int64_t)0x7FFFFFFF / 64) return DQ_ERR_SHAPE;
  LinArgs p{a_codes, a_scales, b_codes, b_scales, r, a_tensor_scale, b_tensor_scale, y,
            M, N, K, ldy, (int32_t)tm, (int32_t)tn, nullptr, 0, 1, (int32_t)((K / 64 + 3) / 4)};
  hipStream_t s = (hipStream_t)stream;
  dim3 grid((unsigned)(tm * tn)), block(256);
  if (nv) return y_dtype == DQ_BF16 ? launch_linear_nv<1>(grid, s, p) : launch_linear_nv<0>(grid, s, p);
  if (i4) {
    const size_t need = dq_quantized_linear_workspace_bytes(spec, M, N, K);
    if (workspace && need > 0) {
      if (workspace_bytes < need) return DQ_ERR_WORKSPACE;
      if (!aligned16(workspace)) return DQ_ERR_ALIGN;
      int ks = 1, per = 0;
      i4_split(M, N, K, ks, per);
      p.ksplit = ks;
      p.st_split = per;
      p.part = (float*)workspace;
      p.ldp = i4_part_pitch(N);
      grid = dim3((unsigned)(tm * tn * ks));
    }
    int rc;
    if (g == 64)
      rc = y_dtype == DQ_BF16 ? launch_linear_i4_tm<1, 1>(tm_rows, grid, s, p)
                              : launch_linear_i4_tm<1, 0>(tm_rows, grid, s, p);
    else
      rc = y_dtype == DQ_BF16 ? launch_linear_i4_tm<2, 1>(tm_rows, grid, s, p)
                              : launch_linear_i4_tm<2, 0>(tm_rows, grid, s, p);
    if (rc != DQ_OK || !p.part) return rc;
    const int64_t threads = M * ((N + 3) / 4);
    dim3 rg((unsigned)((threads + 255) / 256));
    if (y_dtype == DQ_BF16) hipLaunchKernelGGL((k_linear_i4_reduce<1>), rg, block, 0, s, p);
    else hipLaunchKernelGGL((k_linear_i4_reduce<0>), rg, block, 0, s, p);
    return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
  }
#define DQ_L(F)                                                                          \
  rc = (y_dtype == DQ_BF16) ? launch_linear<F, 1>(grid, s, p) : launch_linear<F, 0>(grid, s, p); \
  break
  int rc = DQ_OK;
  switch (f) {
    case DQ_FMT_MXFP4: DQ_L(MXFP4);
    case DQ_FMT_MXFP8_E4M3: DQ_L(MXFP8_E4M3);
    case DQ_FMT_MXFP8_E5M2: DQ_L(MXFP8_E5M2);
    case DQ_FMT_MXFP6_E2M3: DQ_L(MXFP6_E2M3);
    default: DQ_L(MXFP6_E3M2);
  }
#undef DQ_L
  return rc;
}

int dq_recode_mxint4_to_mxfp6(const uint8_t* codes, const uint8_t* block_scales, int64_t rows,
                              int64_t cols, uint8_t* out_codes, uint8_t* out_scales,
                              void* stream) {
  if (rows < 0 || cols < 0 || cols % 32) return DQ_ERR_SHAPE;
  if (rows == 0 || cols == 0) return DQ_OK;
  if (!codes || !block_scales || !out_codes || !out_scales) return DQ_ERR_NULL;
  if (!aligned16(codes) || ((uintptr_t)out_codes & 7u)) return DQ_ERR_ALIGN;
  const int64_t nb = rows * (cols / 32);
  hipLaunchKernelGGL(k_recode_mxint4_e2m3, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, codes, block_scales, nb, out_codes, out_scales);
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

int dq_dequantize(dq_quant_spec spec, const uint8_t* codes, const void* block_scales,
                  const float* tensor_scale, int64_t rows, int64_t cols, const float* r,
                  const float* c, float* out, void* stream) {
  int g = resolve_group(spec);
  if (g < 0) return DQ_ERR_FORMAT;
  if (rows < 0 || cols < 0 || cols % g) return DQ_ERR_SHAPE;
  if (rows == 0 || cols == 0) return DQ_OK;
  if (!codes || !block_scales || !out) return DQ_ERR_NULL;
  if (spec.fmt == DQ_FMT_NVFP4 && !tensor_scale) return DQ_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  int64_t nthreads = rows * (cols / 16);
  dim3 grid((unsigned)((nthreads + 255) / 256)), block(256);
  switch (spec.fmt) {
    case DQ_FMT_INT4:
      if (g == 64) hipLaunchKernelGGL((k_dequant<INT4, 4>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out);
      else hipLaunchKernelGGL((k_dequant<INT4, 8>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out);
      break;
    case DQ_FMT_INT8:
      if (g == 64) hipLaunchKernelGGL((k_dequant<INT8, 4>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out);
      else hipLaunchKernelGGL((k_dequant<INT8, 8>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out);
      break;
    case DQ_FMT_MXINT4: hipLaunchKernelGGL((k_dequant<MXINT4, 2>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out); break;
    case DQ_FMT_MXINT8: hipLaunchKernelGGL((k_dequant<MXINT8, 2>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out); break;
    case DQ_FMT_MXFP8_E4M3: hipLaunchKernelGGL((k_dequant<MXFP8_E4M3, 2>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out); break;
    case DQ_FMT_MXFP8_E5M2: hipLaunchKernelGGL((k_dequant<MXFP8_E5M2, 2>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out); break;
    case DQ_FMT_MXFP6_E2M3: hipLaunchKernelGGL((k_dequant<MXFP6_E2M3, 2>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out); break;
    case DQ_FMT_MXFP6_E3M2: hipLaunchKernelGGL((k_dequant<MXFP6_E3M2, 2>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out); break;
    case DQ_FMT_MXFP4: hipLaunchKernelGGL((k_dequant<MXFP4, 2>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out); break;
    default: hipLaunchKernelGGL((k_dequant<NVFP4, 1>), grid, block, 0, s, codes, block_scales, tensor_scale, rows, cols, r, c, out); break;
  }
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

int dq_debug_round(int32_t fn, const float* x, void* out, int64_t n, void* stream) {
  if (fn < DQ_ROUND_E2M1 || fn > DQ_PROJ_BF16) return DQ_ERR_ARG;
  if (n < 0) return DQ_ERR_SHAPE;
  if (n == 0) return DQ_OK;
  if (!x || !out) return DQ_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(k_debug_round, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (int)fn,
                     x, out, n);
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

}  // extern "C"
