// Quantised linear layer on the gfx950 block-scaled matrix cores.
//
// The layer that consumes what the solver and the activation quantiser produce (listing
// page Table 11, "quantized linears"; Table 12, packed 4-bit weights; news summary: the
// column scales fold into the activation quantiser and the row scales into the output):
//
//     Y = X W^T ~ Aq . Q^T . diag(r),    Aq = FQ(X diag(c)),   W ~ diag(r) Q diag(c),
//
// with Aq [M][K] and Q [N][K] in an MX format (32-element blocks along K, E8M0 scales).
// One V_MFMA_SCALE_F32_16X16X128_F8F6F4 multiplies a 16x128 tile of Aq by a 128x16 tile of
// Q^T, applying both operands' block scales; its operand layout (measured):
//   - lane l holds row (l % 16) of its tile and K-group g = l / 16;
//   - FP4 / FP6: the 32 consecutive K elements of block g, packed as in memory (nibbles low
//     first, or the 6-bit little-endian stream);
//   - FP8: bytes 0-15 hold K 16g .. 16g+15 and bytes 16-31 hold K 64+16g .. 64+16g+15;
//   - the lane's scale byte is the E8M0 scale of block g of its row;
//   - result: lane l, element v holds C[4 (l / 16) + v][l % 16].
// The codes are staged through LDS in their memory layout: whole-row global reads, then
// each lane reads its fragment (one to three LDS reads) with no repacking.  Two kernels:
// k_linear_dma (FP4 and FP8 with whole stages: global loads go straight into an LDS ring)
// and k_linear (every format and any K that is a multiple of 32: the loads are staged in
// registers, LDS rows are padded, and the last partial stage is masked).
#pragma once

#include <type_traits>

namespace dqk {

typedef int v8i __attribute__((ext_vector_type(8)));

template <int FMT>
constexpr int mfma_elem_fmt() {   // the instruction's element-format selector
  return FMT == MXFP8_E4M3 ? 0 : FMT == MXFP8_E5M2 ? 1 : FMT == MXFP6_E2M3 ? 2 : FMT == MXFP6_E3M2 ? 3 : 4;
}
template <int FMT>
constexpr int elem_bits() {
  return (FMT == MXFP8_E4M3 || FMT == MXFP8_E5M2) ? 8 : mx_fp6<FMT>() ? 6 : 4;
}

constexpr int kLinTile = 128;   // workgroup tile (M and N); four waves of 64 x 64
constexpr int kLinK = 128;      // K per instruction

struct LinArgs {
  const uint8_t* a;    // activation codes [M][K * bits / 8]
  const uint8_t* as;   // activation block scales [M][K / 32]
  const uint8_t* b;    // weight codes [N][K * bits / 8]
  const uint8_t* bs;   // weight block scales [N][K / 32]
  const float* r;      // row scales of the weights (output columns) [N], or null
  const float* ats;    // NVFP4: activation tensor scale [1]
  const float* bts;    // NVFP4: weight tensor scale [1]
  void* y;             // output [M][ldy], fp32 or bf16
  int64_t M, N, K, ldy;
  int32_t tiles_m, tiles_n;
  // split K (INT4): workgroups of one output tile take consecutive ranges of `st_split`
  // stages each and write unscaled fp32 partial sums to part [ksplit][M][ldp]; a second
  // kernel adds them in split order.  ksplit = 1 and part = null: no split.
  float* part;
  int64_t ldp;
  int32_t ksplit, st_split;
};

// Tile of this workgroup.  Workgroups are dispatched round-robin over the 8 XCDs; each XCD
// gets a contiguous range of tiles, ordered down the M tiles of one N column first, so the
// tiles that share weight rows (and, across columns, the activations) meet in one L2.
__device__ __forceinline__ int lin_item(int nitems) {
  const int bid = blockIdx.x, x = bid & 7, q = nitems >> 3, rem = nitems & 7;
  return x * q + (x < rem ? x : rem) + (bid >> 3);
}
__device__ __forceinline__ void lin_tile(int ntiles, int tiles_m, int& tm, int& tn) {
  const int t = lin_item(ntiles);
  tm = t % tiles_m;
  tn = t / tiles_m;
}

// Stores one wave's (16 BI) x (16 BJ) block of Y (64 x 64 by default) from accumulators of
// (B A^T) products (the weight fragment is the instruction's first operand): acc[i][j][v]
// holds Y[m0 + 16 i + lane % 16][n0 + 16 j + 4 (lane / 16) + v].  So each lane writes four
// consecutive columns of one row, one 8-byte (bf16) or 16-byte (fp32) store where the
// output's alignment and row pitch allow it, as (acc * s) * r[n].
template <int OUT_BF16, int BI = 4, int BJ = 4>
__device__ __forceinline__ void lin_store(const f32x4 (&acc)[BI][BJ], const LinArgs& p, int64_t m0,
                                          int64_t n0, float s) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const bool vec = (p.ldy & 3) == 0 && ((uintptr_t)p.y & (OUT_BF16 ? 7u : 15u)) == 0;
#pragma unroll
  for (int j = 0; j < BJ; ++j) {
    const int64_t n = n0 + 16 * j + 4 * g;
    float rn[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) rn[v] = (p.r && n + v < p.N) ? gp(p.r)[n + v] : 1.0f;
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int64_t m = m0 + 16 * i + r16;
      if (m >= p.M) continue;
      float yv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) yv[v] = (acc[i][j][v] * s) * rn[v];
      const int64_t o = m * p.ldy + n;
      if (vec && n + 3 < p.N) {
        if (OUT_BF16) {
          const uint32_t h0 = (f2u(bf16_rne(yv[0])) >> 16) | (f2u(bf16_rne(yv[1])) & 0xFFFF0000u);
          const uint32_t h1 = (f2u(bf16_rne(yv[2])) >> 16) | (f2u(bf16_rne(yv[3])) & 0xFFFF0000u);
          *gp((u32x2*)((uint16_t*)p.y + o)) = u32x2{h0, h1};
        } else {
          *gp((f32x4*)((float*)p.y + o)) = f32x4{yv[0], yv[1], yv[2], yv[3]};
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (n + v >= p.N) break;
          if (OUT_BF16) gp((uint16_t*)p.y)[o + v] = (uint16_t)(f2u(bf16_rne(yv[v])) >> 16);
          else gp((float*)p.y)[o + v] = yv[v];
        }
      }
    }
  }
}

// Staging geometry per element width: K per stage (one or two instructions), bytes of a
// row per stage, the global-load chunk, the padded LDS row pitch (consecutive rows start
// 36 or 28 banks apart, so the 16 rows a fragment read touches fall on distinct banks) and
// the scale bytes of a row per stage.
template <int FMT>
struct LinGeom {
  static constexpr int EB = elem_bits<FMT>();
  static constexpr int KS = (EB == 4) ? 256 : 128;
  static constexpr int NI = KS / kLinK;
  static constexpr int ROWB = KS * EB / 8;          // 128, 96, 128
  static constexpr int CH = (EB == 6) ? 8 : 16;     // FP6 blocks are 24 bytes
  static constexpr int CPR = ROWB / CH;             // chunks per row
  static constexpr int PITCH = ROWB + 16;
  static constexpr int SPR = KS / 32;               // blocks per row per stage
  static constexpr int BB = 4 * EB;                 // bytes per block
  static constexpr int TILE = kLinTile * PITCH;     // one operand's codes
  static constexpr int STILE = kLinTile * SPR;      // one operand's scales
  static constexpr int STAGE = 2 * TILE + 2 * STILE;
  static constexpr int LDS = 2 * STAGE;             // double buffered
  static constexpr int NCH = kLinTile * CPR / 256;  // global chunks per thread per operand
  static constexpr int NSC = kLinTile * SPR / 256;  // scale bytes per thread per operand
};

// Global -> registers -> LDS for one stage of one operand (rows r0 .. r0+127 of a [rows][K]
// code matrix): 256 threads read consecutive chunks, eight (or twelve) to a row, so each
// row's stage bytes come in as whole cache-line segments.  Rows past the end read the last
// row (their results are not stored); chunks at or beyond K read the row start and are
// written to LDS as zeros, so the selection waits for nothing the store does not need.
template <int FMT>
struct LinStage {
  using G = LinGeom<FMT>;
  typedef uint32_t chunk_t __attribute__((ext_vector_type(G::CH / 4)));
  chunk_t c[2][G::NCH];
  uint32_t sc[2][G::NSC];

  template <int OP>
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                       int64_t r0, int64_t K, int64_t st) {
    const int64_t rowbytes = K * G::EB / 8, nblk = K / 32;
#pragma unroll
    for (int j = 0; j < G::NCH; ++j) {
      const int q = threadIdx.x + 256 * j, rr = q / G::CPR, cc = q % G::CPR;
      int64_t row = r0 + rr;
      row = row < rows ? row : rows - 1;
      const int64_t blk = st * G::SPR + (cc * G::CH) / G::BB;
      const int64_t off = blk < nblk ? st * G::ROWB + cc * G::CH : 0;
      c[OP][j] = *gp((const chunk_t*)(codes + row * rowbytes + off));
    }
#pragma unroll
    for (int j = 0; j < G::NSC; ++j) {
      const int q = threadIdx.x + 256 * j, rr = q / G::SPR, bb = q % G::SPR;
      int64_t row = r0 + rr;
      row = row < rows ? row : rows - 1;
      int64_t blk = st * G::SPR + bb;
      blk = blk < nblk ? blk : 0;
      sc[OP][j] = gp(scales)[row * nblk + blk];
    }
  }
  template <int OP>
  __device__ __forceinline__ void store(uint8_t* lds, int64_t K, int64_t st) const {
    uint8_t* tile = lds + OP * G::TILE;
    uint8_t* stile = lds + 2 * G::TILE + OP * G::STILE;
    const int64_t nblk = K / 32;
#pragma unroll
    for (int j = 0; j < G::NCH; ++j) {
      const int q = threadIdx.x + 256 * j, rr = q / G::CPR, cc = q % G::CPR;
      const bool ok = st * G::SPR + (cc * G::CH) / G::BB < nblk;
      *(chunk_t*)(tile + rr * G::PITCH + cc * G::CH) = ok ? c[OP][j] : chunk_t(0u);
    }
#pragma unroll
    for (int j = 0; j < G::NSC; ++j) stile[threadIdx.x + 256 * j] = (uint8_t)sc[OP][j];
  }
};

// Fragment of instruction u of a stage from LDS: this lane's tile row `row` (0..127) and
// K-group g, as the instruction wants it (see the layout at the top of this file).
template <int FMT>
__device__ __forceinline__ void lin_frag(const uint8_t* tile, int row, int u, int g, v8i& v) {
  using G = LinGeom<FMT>;
  const uint8_t* rp = tile + row * G::PITCH;
  if (G::EB == 4) {
    const u32x4 x = *(const u32x4*)(rp + 64 * u + 16 * g);
    v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  } else if (G::EB == 6) {
    const u32x2* q = (const u32x2*)(rp + 24 * g);
    const u32x2 x0 = q[0], x1 = q[1], x2 = q[2];
    v = v8i{(int)x0.x, (int)x0.y, (int)x1.x, (int)x1.y, (int)x2.x, (int)x2.y, 0, 0};
  } else {
    const u32x4 x = *(const u32x4*)(rp + 16 * g);
    const u32x4 y = *(const u32x4*)(rp + 64 + 16 * g);
    v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  }
}

// One workgroup = a 128 x 128 tile of Y; four waves of 64 x 64 (4 x 4 instruction tiles).
// Per stage: the next stage's codes and scales are read from HBM into registers while this
// stage's products run from LDS; then they are written to the other LDS buffer and the
// workgroup synchronises once.
template <int FMT, int OUT_BF16>
__global__ __launch_bounds__(256) void k_linear(LinArgs p) {
  using G = LinGeom<FMT>;
  constexpr int F = mfma_elem_fmt<FMT>();
  extern __shared__ __align__(16) uint8_t lin_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int tm, tn;
  lin_tile(p.tiles_m * p.tiles_n, p.tiles_m, tm, tn);
  const int64_t mt0 = (int64_t)tm * kLinTile, nt0 = (int64_t)tn * kLinTile;
  const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
  const int g = lane >> 4, r16 = lane & 15;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t nst = (p.K + G::KS - 1) / G::KS;
  LinStage<FMT> stg;
  auto fetch = [&](int64_t st) {
    stg.template load<0>(p.a, p.as, p.M, mt0, p.K, st);
    stg.template load<1>(p.b, p.bs, p.N, nt0, p.K, st);
  };
  auto put = [&](int64_t st, uint8_t* buf) {
    stg.template store<0>(buf, p.K, st);
    stg.template store<1>(buf, p.K, st);
  };
  if (nst > 0) {
    fetch(0);
    put(0, lin_lds);
    __syncthreads();
  }
  for (int64_t st = 0; st < nst; ++st) {
    uint8_t* cur = lin_lds + (st & 1) * G::STAGE;
    uint8_t* nxt = lin_lds + ((st + 1) & 1) * G::STAGE;
    const bool more = st + 1 < nst;
    if (more) fetch(st + 1);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* ta = cur;
    const uint8_t* tb = cur + G::TILE;
    const uint8_t* sa_t = cur + 2 * G::TILE;
    const uint8_t* sb_t = sa_t + G::STILE;
#pragma unroll
    for (int u = 0; u < G::NI; ++u) {
      v8i a[4], b[4];
      int sa[4], sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lin_frag<FMT>(ta, wm + 16 * i + r16, u, g, a[i]);
        lin_frag<FMT>(tb, wn + 16 * i + r16, u, g, b[i]);
        sa[i] = sa_t[(wm + 16 * i + r16) * G::SPR + 4 * u + g];
        sb[i] = sb_t[(wn + 16 * i + r16) * G::SPR + 4 * u + g];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i], acc[i][j], F, F, 0,
                                                                        sb[j], 0, sa[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (more) put(st + 1, nxt);
    __syncthreads();
  }

  lin_store<OUT_BF16>(acc, p, mt0 + wm, nt0 + wn, 1.0f);   // Y[m][n] = acc * r[n]
}

// ---------------------------------------------------------------- direct-to-LDS variant
// For FP4 codes with K a multiple of 256 and FP8 codes with K a multiple of 128.  Global loads write LDS directly
// (global_load_lds_dwordx4: lane l's 16 bytes land at the wave's LDS address + 16 l), so
// no registers stage the tiles and a ring of D stages (128 K each) keeps D - 1 stages in
// flight while one is multiplied (D = 2: the next stage loads during this one's products,
// with no staging registers).  Rows are unpadded; within a row the 16-byte chunks are
// XOR-swizzled by row so that the 16 rows one fragment read touches hit distinct banks.
template <int FMT>
struct DmaGeom {
  static constexpr int EB = elem_bits<FMT>();
  static constexpr int KS = (EB == 4) ? 256 : 128;      // K per stage: rows of 128 bytes
  static constexpr int NI = KS / kLinK;                 // instructions per stage
  static constexpr int ROWB = KS * EB / 8;              // 128
  static constexpr int CPR = ROWB / 16;                 // chunks per row
  static constexpr int RPI = 64 / CPR;                  // rows per wave instruction
  static constexpr int SPR = KS / 32;                   // scale bytes per row per stage
  static constexpr int TILE = kLinTile * ROWB;
  static constexpr int STILE = kLinTile * SPR;
  static constexpr int STAGE = 2 * TILE + 2 * STILE;
  static constexpr int D = 2;                           // ring depth
  static constexpr int LDS = D * STAGE;                 // 68 KiB (FP4), 66 KiB (FP8)
  static constexpr int CODE_INSTS = kLinTile / RPI / 4; // per wave per operand per stage
  static constexpr int SC_INSTS = (SPR + 3) / 4;        // scale loads per wave per stage
  static constexpr int INSTS = 2 * CODE_INSTS + SC_INSTS;
};
// Swizzle of the 16-byte chunk positions of a 128-byte row r, so that the 16 rows one
// fragment read touches (one chunk each) hit 16 distinct 4-bank groups: a 128-byte row spans
// 32 banks, so rows of one parity share banks, and the chunk index is XOR-ed with
// (r >> 1) & 7.  (Stages of 128 K, 64-byte rows, in a four-deep ring were slower: 52 us
// against 36 us on 2048 x 4096 x 4096.)
__device__ __forceinline__ int swz128(int r) { return (r >> 1) & 7; }
template <int FMT>
__device__ __forceinline__ int dma_swz(int r) { return swz128(r); }

template <int FMT>
__device__ __forceinline__ void dma_stage(const LinArgs& p, int64_t mt0, int64_t nt0, int64_t st,
                                          uint8_t* buf) {
  using G = DmaGeom<FMT>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rowbytes = p.K * G::EB / 8, nblk = p.K / 32;
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    const uint8_t* codes = op ? p.b : p.a;
    const int64_t r0 = op ? nt0 : mt0, rows = op ? p.N : p.M;
    uint8_t* tile = buf + op * G::TILE;
#pragma unroll
    for (int ii = 0; ii < G::CODE_INSTS; ++ii) {
      const int rbase = (wave * G::CODE_INSTS + ii) * G::RPI;   // first tile row of this load
      const int r = rbase + lane / G::CPR, c = lane % G::CPR;
      int64_t row = r0 + r;
      row = row < rows ? row : rows - 1;
      const uint8_t* src = codes + row * rowbytes + st * G::ROWB + 16 * (c ^ dma_swz<FMT>(r));
      __builtin_amdgcn_global_load_lds((const DQ_GAS void*)src,
                                       (__attribute__((address_space(3))) void*)(tile + rbase * G::ROWB),
                                       16, 0, 0);
    }
  }
  // scales: each operand's [128][SPR] bytes in 256-byte pieces, dword q of a piece holding
  // bytes 4 (q % (SPR / 4)) .. +3 of row q / (SPR / 4)
#pragma unroll
  for (int j = 0; j < G::SC_INSTS; ++j) {
    const int q = wave * G::SC_INSTS + j;                  // 0 .. SPR - 1
    const int op = q / (G::SPR / 2), part = q % (G::SPR / 2);
    const int d = 64 * part + lane, r = d / (G::SPR / 4), word = d % (G::SPR / 4);
    const uint8_t* scales = op ? p.bs : p.as;
    const int64_t r0 = op ? nt0 : mt0, rows = op ? p.N : p.M;
    int64_t row = r0 + r;
    row = row < rows ? row : rows - 1;
    const uint8_t* src = scales + row * nblk + st * G::SPR + 4 * word;
    uint8_t* stile = buf + 2 * G::TILE + op * G::STILE + 256 * part;
    __builtin_amdgcn_global_load_lds((const DQ_GAS void*)src,
                                     (__attribute__((address_space(3))) void*)stile, 4, 0, 0);
  }
}

// s_waitcnt immediate that waits until at most `vm` vector-memory operations are
// outstanding and ignores the other counters (vmcnt in bits 3:0 and 15:14).
__device__ __forceinline__ void wait_vmcnt(int vm) {
  switch (vm) {
#define DQ_W(n) case n: __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
    DQ_W(0) DQ_W(1) DQ_W(2) DQ_W(3) DQ_W(4) DQ_W(5) DQ_W(6) DQ_W(7) DQ_W(8) DQ_W(9) DQ_W(10)
    DQ_W(11) DQ_W(12) DQ_W(13) DQ_W(14) DQ_W(15) DQ_W(16) DQ_W(17) DQ_W(18) DQ_W(19) DQ_W(20)
#undef DQ_W
    default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;
  }
}

template <int FMT, int OUT_BF16>
__global__ __launch_bounds__(256) void k_linear_dma(LinArgs p) {
  using G = DmaGeom<FMT>;
  constexpr int F = mfma_elem_fmt<FMT>();
  extern __shared__ __align__(16) uint8_t lin_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int tm, tn;
  lin_tile(p.tiles_m * p.tiles_n, p.tiles_m, tm, tn);
  const int64_t mt0 = (int64_t)tm * kLinTile, nt0 = (int64_t)tn * kLinTile;
  const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
  const int g = lane >> 4, r16 = lane & 15;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t nst = p.K / G::KS;
  for (int64_t s = 0; s < G::D - 1 && s < nst; ++s) dma_stage<FMT>(p, mt0, nt0, s, lin_lds + s * G::STAGE);
  for (int64_t st = 0; st < nst; ++st) {
    // this stage has landed once at most the later stages' loads are outstanding
    const int64_t later = min((int64_t)(G::D - 2), nst - 1 - st);
    wait_vmcnt((int)(later * G::INSTS));
    // A bare barrier: every wave has waited for its own loads of this stage, and its reads
    // of the buffer about to be refilled were consumed by its last products.  (The fence
    // of __syncthreads would wait for all outstanding loads, draining the ring.)  The
    // memory clobber keeps the compiler from moving LDS accesses across it.
    asm volatile("s_barrier" ::: "memory");
    if (st + G::D - 1 < nst)
      dma_stage<FMT>(p, mt0, nt0, st + G::D - 1, lin_lds + ((st + G::D - 1) % G::D) * G::STAGE);
    const uint8_t* cur = lin_lds + (st % G::D) * G::STAGE;
    const uint8_t* sa_t = cur + 2 * G::TILE;
    const uint8_t* sb_t = sa_t + G::STILE;
    // LDS reads of the stage: the scale words and the first instruction step's fragments,
    // which its products wait for in full; each later step's fragments are issued before the
    // products of the step before it, so those reads overlap products (never more than 15
    // reads outstanding, so the waits the compiler inserts count them exactly)
    v8i a[G::NI][4], b[G::NI][4];
    int sa[G::NI][4], sb[G::NI][4];
    uint64_t sw8s[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int op = 0; op < 2; ++op) {
        // the row's scale bytes of this stage in one read (the four lanes of a row share it)
        const uint8_t* srow = (op ? sb_t : sa_t) + ((op ? wn : wm) + 16 * i + r16) * G::SPR;
        sw8s[i][op] = (G::SPR == 8) ? *(const uint64_t*)srow : (uint64_t)*(const uint32_t*)srow;
      }
    }
    auto frags = [&](int u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int op = 0; op < 2; ++op) {
          const int r = (op ? wn : wm) + 16 * i + r16;
          const uint8_t* rp = cur + op * G::TILE + r * G::ROWB;
          const int sw = dma_swz<FMT>(r);
          v8i v;
          if (G::EB == 4) {
            const u32x4 x = *(const u32x4*)(rp + 16 * ((4 * u + g) ^ sw));
            v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
          } else {
            const u32x4 x = *(const u32x4*)(rp + 16 * (g ^ sw));
            const u32x4 y = *(const u32x4*)(rp + 16 * ((4 + g) ^ sw));
            v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
          }
          if (op) b[u][i] = v; else a[u][i] = v;
        }
      }
    };
    auto products = [&](int u) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[u][j], a[u][i], acc[i][j], F,
                                                                        F, 0, sb[u][j], 0, sa[u][i]);
    };
    frags(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < G::NI; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa[u][i] = (int)((sw8s[i][0] >> (8 * (4 * u + g))) & 0xFFu);
        sb[u][i] = (int)((sw8s[i][1] >> (8 * (4 * u + g))) & 0xFFu);
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 1; u < G::NI; ++u) {
      frags(u);
      __builtin_amdgcn_sched_barrier(0);
      products(u - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    products(G::NI - 1);
  }

  lin_store<OUT_BF16>(acc, p, mt0 + wm, nt0 + wn, 1.0f);
}

// ---------------------------------------------------------------- NVFP4 on the f16 cores
// NVFP4 scales (E4M3 per 16 elements, fp32 per tensor) have no block-scaled matrix-core
// form.  Within a tensor every element is e2m1(q) * e4m3(sb) * s_t, and e2m1(q) * e4m3(sb)
// has at most 6 significant bits and lies in [2^-10, 2688] (or is zero), so it is exact in
// fp16: the operands are dequantised to that product on the way into LDS (the hardware
// FP4 -> packed f16 conversion, then one packed f16 multiply by the block scale: one
// instruction per element), multiplied on the f16 cores (v_mfma_f32_16x16x32_f16: lane l
// holds row l % 16 and K 8 (l / 16) .. +7, measured), and the two tensor scales and r are
// applied to the fp32 result.  Stage = 64 K: a 128-byte f16 row per tile row.
struct NvGeom {
  static constexpr int KS = 64;
  static constexpr int ROWB = KS * 2;               // 128 bytes of f16
  static constexpr int TILE = kLinTile * ROWB;      // 16 KiB
  static constexpr int STAGE = 2 * TILE;
  static constexpr int LDS = 2 * STAGE;             // 64 KiB
};
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Eight e2m1 codes (one word, low nibble first) times s, as four packed f16 pairs: byte b
// of the word holds elements 2b (low nibble, low half) and 2b + 1.
__device__ __forceinline__ void fp4_f16_scaled8(uint32_t w, f16x2 s, uint32_t* h) {
  h[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s);
  h[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s);
  h[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s);
  h[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s);
}

// Tile row of thread t (the other half of the row's stage is thread t ^ 1).  Each group of
// 8 lanes takes four even or four odd rows whose swizzles differ, so the 16-byte chunks its
// LDS stores hit are 8 distinct bank groups (pairs of consecutive rows, which share a
// swizzle, in one group of 8 made every store a 2-way bank conflict).
__device__ __forceinline__ int nv_row(int t) {
  return 8 * (t >> 4) + 2 * ((t >> 1) & 3) + ((t >> 3) & 1);
}

// One thread's share of one stage of both operands: tile row nv_row(t), 32 elements (two
// NVFP4 blocks) starting at K 32 (t % 2) of the stage, as loaded (codes and the two scale
// bytes).
struct NvRaw {
  u32x4 code[2];
  uint32_t sc[2];
  template <int OP>
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                       int64_t r0, int64_t K, int64_t st) {
    const int rr = nv_row(threadIdx.x), half = threadIdx.x & 1;
    int64_t row = r0 + rr;
    row = row < rows ? row : rows - 1;
    int64_t k = st * NvGeom::KS + 32 * half;
    k = k < K ? k : 0;   // a chunk at or beyond K reads the row start; it is zeroed on store
    // K is a multiple of 32, so a chunk below K holds both of its blocks
    code[OP] = *gp((const u32x4*)(codes + row * (K / 2) + k / 2));
    const DQ_GAS uint8_t* sp = gp(scales + row * (K / 16) + k / 16);
    sc[OP] = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
  }
  // The two block scales of operand OP as f16 (E4M3 codes 0..126; the sign bits are
  // cleared, as the format stores non-negative scales); a chunk at or beyond K gets scale 0,
  // so it stores zeros.
  template <int OP>
  __device__ __forceinline__ f16x2 scales(int64_t K, int64_t st) const {
    const int64_t k0 = st * NvGeom::KS + 32 * (threadIdx.x & 1);
    const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[OP] & 0x7F7Fu, 1.0f, false);
    return k0 < K ? s01 : f16x2{(_Float16)0.0f, (_Float16)0.0f};
  }
  // Block BLK of operand OP dequantised to f16 with its scale, written into OP's LDS tile:
  // 16 f16 = two 16-byte chunks at K offset 32 half + 16 BLK, chunks 4 half + 2 BLK and +1.
  template <int OP, int BLK>
  __device__ __forceinline__ void store_blk(uint8_t* lds, f16x2 s01) const {
    const int rr = nv_row(threadIdx.x), half = threadIdx.x & 1;
    uint8_t* rp = lds + OP * NvGeom::TILE + rr * NvGeom::ROWB;
    const uint32_t w0 = BLK ? code[OP].z : code[OP].x, w1 = BLK ? code[OP].w : code[OP].y;
    const _Float16 sv = BLK ? s01.y : s01.x;
    const f16x2 s2 = {sv, sv};
    uint32_t h[8];
    fp4_f16_scaled8(w0, s2, h);
    fp4_f16_scaled8(w1, s2, h + 4);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = (4 * half + 2 * BLK + q) ^ swz128(rr);
      *(u32x4*)(rp + 16 * c) = u32x4{h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]};
    }
  }
};

// Y tile 128 x 128 per workgroup, four waves of 64 x 64 (as k_linear).  Stages of 64 K:
// raw codes are loaded into registers two stages ahead, dequantised into one of two f16
// LDS buffers one stage ahead, and multiplied from the other.
template <int OUT_BF16>
__global__ __launch_bounds__(256) void k_linear_nv(LinArgs p) {
  extern __shared__ __align__(16) uint8_t lin_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int tm, tn;
  lin_tile(p.tiles_m * p.tiles_n, p.tiles_m, tm, tn);
  const int64_t mt0 = (int64_t)tm * kLinTile, nt0 = (int64_t)tn * kLinTile;
  const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
  const int g = lane >> 4, r16 = lane & 15;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t nst = (p.K + NvGeom::KS - 1) / NvGeom::KS;
  uint8_t* const buf0 = lin_lds;
  uint8_t* const buf1 = lin_lds + NvGeom::STAGE;
  NvRaw ra, rb;
  auto fetch = [&](NvRaw& R, int64_t st) {
    R.template load<0>(p.a, p.as, p.M, mt0, p.K, st);
    R.template load<1>(p.b, p.bs, p.N, nt0, p.K, st);
  };
  auto frags = [&](const uint8_t* cur, int u, f16x8 (&a)[4], f16x8 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra_ = wm + 16 * i + r16, rb_ = wn + 16 * i + r16;
      a[i] = *(const f16x8*)(cur + ra_ * NvGeom::ROWB + 16 * ((4 * u + g) ^ swz128(ra_)));
      b[i] = *(const f16x8*)(cur + NvGeom::TILE + rb_ * NvGeom::ROWB +
                             16 * ((4 * u + g) ^ swz128(rb_)));
    }
  };
  auto mrow = [&](int i, const f16x8& a, const f16x8 (&b)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j], a, acc[i][j], 0, 0, 0);
  };
#define DQ_SB __builtin_amdgcn_sched_barrier(0)
  // The products of the stage in `cur` (two K-steps of 32, four rows of four products
  // each), with the dequantisation of the stage held in R (index sn) into `nb` cut into
  // four blocks and placed between them: the matrix cores take 16 cycles per product, in
  // which the wave issues the conversions of the next stage.
  auto half_trip = [&](const uint8_t* cur, const NvRaw& R, int64_t sn, uint8_t* nb) {
    f16x8 a0[4], b0[4], a1[4], b1[4];
    frags(cur, 0, a0, b0);
    const f16x2 s0 = R.template scales<0>(p.K, sn), s1 = R.template scales<1>(p.K, sn);
    mrow(0, a0[0], b0);
    DQ_SB;
    R.template store_blk<0, 0>(nb, s0);
    DQ_SB;
    mrow(1, a0[1], b0);
    DQ_SB;
    frags(cur, 1, a1, b1);
    DQ_SB;
    mrow(2, a0[2], b0);
    DQ_SB;
    R.template store_blk<0, 1>(nb, s0);
    DQ_SB;
    mrow(3, a0[3], b0);
    mrow(0, a1[0], b1);
    DQ_SB;
    R.template store_blk<1, 0>(nb, s1);
    DQ_SB;
    mrow(1, a1[1], b1);
    mrow(2, a1[2], b1);
    DQ_SB;
    R.template store_blk<1, 1>(nb, s1);
    DQ_SB;
    mrow(3, a1[3], b1);
  };
#undef DQ_SB

  // Two stages per trip, so that the two register sets keep fixed names.  The trip has no
  // branches: stages at or beyond K load in-range bytes and store zeros (their products add
  // nothing).
  if (nst > 0) {
    fetch(ra, 0);
    fetch(rb, 1);
    ra.template store_blk<0, 0>(buf0, ra.template scales<0>(p.K, 0));
    ra.template store_blk<0, 1>(buf0, ra.template scales<0>(p.K, 0));
    ra.template store_blk<1, 0>(buf0, ra.template scales<1>(p.K, 0));
    ra.template store_blk<1, 1>(buf0, ra.template scales<1>(p.K, 0));
    lds_barrier();
  }
  for (int64_t st = 0; st < nst; st += 2) {
    // stage st is in buf0; rb holds stage st + 1; buf1 is free
    fetch(ra, st + 2);
    half_trip(buf0, rb, st + 1, buf1);
    lds_barrier();
    // stage st + 1 is in buf1; ra holds stage st + 2; buf0 is free
    fetch(rb, st + 3);
    half_trip(buf1, ra, st + 2, buf0);
    lds_barrier();
  }

  lin_store<OUT_BF16>(acc, p, mt0 + wm, nt0 + wn, gp(p.ats)[0] * gp(p.bts)[0]);
}

// ---------------------------------------------------------------- NVFP4, codes through LDS
// The same layer with the raw codes and scales moved into LDS by the direct-to-LDS ring and
// dequantised in registers right before the products (LDS carries 4-bit codes, not f16
// values, and no wave stores to LDS).  A stage is 128 K: 64 bytes of codes and 8 scale
// bytes per tile row.  Within a stage lane group g takes blocks 2g and 2g + 1 (16
// contiguous bytes: one read per row fragment): K-step u of the instruction gets block
// 2g + u / 2, half u % 2.  Activations and weights use the same order, so the four
// K-steps sum the stage's 128 products of every output.  Rows of 64 bytes span 16 banks,
// so the chunk index is XOR-ed with (r >> 2) & 3 to give a fragment read's 16 rows
// distinct banks.
struct NvDmaGeom {
  static constexpr int KS = 128;
  static constexpr int ROWB = KS / 2;                    // 64 bytes of codes per row
  static constexpr int CPR = ROWB / 16;                  // 4 chunks
  static constexpr int RPI = 64 / CPR;                   // 16 rows per wave instruction
  static constexpr int SPR = KS / 16;                    // 8 scale bytes per row
  static constexpr int TILE = kLinTile * ROWB;           // 8 KiB
  static constexpr int STILE = kLinTile * SPR;           // 1 KiB
  static constexpr int STAGE = 2 * TILE + 2 * STILE;
  static constexpr int D = 3;                            // ring depth
  static constexpr int LDS = D * STAGE;                  // 54 KiB
  static constexpr int CODE_INSTS = kLinTile / RPI / 4;  // 2 per wave per operand
  static constexpr int SC_INSTS = 2 * kLinTile * SPR / 4 / 64 / 4;   // 2 per wave
  static constexpr int INSTS = 2 * CODE_INSTS + SC_INSTS;
};
__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ void nv_dma_stage(const LinArgs& p, int64_t mt0, int64_t nt0,
                                             int64_t st, uint8_t* buf) {
  using G = NvDmaGeom;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rowbytes = p.K / 2, nblk = p.K / 16;
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    const uint8_t* codes = op ? p.b : p.a;
    const int64_t r0 = op ? nt0 : mt0, rows = op ? p.N : p.M;
    uint8_t* tile = buf + op * G::TILE;
#pragma unroll
    for (int ii = 0; ii < G::CODE_INSTS; ++ii) {
      const int rbase = (wave * G::CODE_INSTS + ii) * G::RPI;
      const int r = rbase + lane / G::CPR, c = lane % G::CPR;
      int64_t row = r0 + r;
      row = row < rows ? row : rows - 1;
      const uint8_t* src = codes + row * rowbytes + st * G::ROWB + 16 * (c ^ swz64(r));
      __builtin_amdgcn_global_load_lds((const DQ_GAS void*)src,
                                       (__attribute__((address_space(3))) void*)(tile + rbase * G::ROWB),
                                       16, 0, 0);
    }
  }
  // scales: each operand's [128][8] bytes as four pieces of 64 dwords; dword d of an
  // operand holds bytes 4 (d % 2) .. +3 of row d / 2
#pragma unroll
  for (int j = 0; j < G::SC_INSTS; ++j) {
    const int q = wave * G::SC_INSTS + j;               // 0 .. 7
    const int op = q / 4, part = q % 4;
    const int d = 64 * part + lane, r = d / 2, word = d % 2;
    const uint8_t* scales = op ? p.bs : p.as;
    const int64_t r0 = op ? nt0 : mt0, rows = op ? p.N : p.M;
    int64_t row = r0 + r;
    row = row < rows ? row : rows - 1;
    const uint8_t* src = scales + row * nblk + st * G::SPR + 4 * word;
    uint8_t* stile = buf + 2 * G::TILE + op * G::STILE + 256 * part;
    __builtin_amdgcn_global_load_lds((const DQ_GAS void*)src,
                                     (__attribute__((address_space(3))) void*)stile, 4, 0, 0);
  }
}

// Row fragment of one operand for the stage: 16 bytes of codes (blocks 2g, 2g + 1 of the
// stage) and their two E4M3 scales as f16 (sign bits cleared, as in k_linear_nv).
struct NvFrag {
  u32x4 q;
  f16x2 s;
};
__device__ __forceinline__ NvFrag nv_frag(const uint8_t* tile, const uint8_t* stile, int r, int g) {
  NvFrag f;
  f.q = *(const u32x4*)(tile + r * NvDmaGeom::ROWB + 16 * (g ^ swz64(r)));
  const uint32_t sb = *(const uint16_t*)(stile + r * NvDmaGeom::SPR + 2 * g);
  f.s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb & 0x7F7Fu, 1.0f, false);
  return f;
}
// The eight f16 of K-step u: word u of the codes times the scale of block u / 2.
__device__ __forceinline__ f16x8 nv_expand(const NvFrag& f, int u) {
  const uint32_t w = u == 0 ? f.q.x : (u == 1 ? f.q.y : (u == 2 ? f.q.z : f.q.w));
  const _Float16 sv = (u < 2) ? f.s.x : f.s.y;
  uint32_t h[4];
  fp4_f16_scaled8(w, f16x2{sv, sv}, h);
  f16x8 v;
  __builtin_memcpy(&v, h, 16);
  return v;
}

template <int OUT_BF16>
__global__ __launch_bounds__(256) void k_linear_nv_dma(LinArgs p) {
  using G = NvDmaGeom;
  extern __shared__ __align__(16) uint8_t lin_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int tm, tn;
  lin_tile(p.tiles_m * p.tiles_n, p.tiles_m, tm, tn);
  const int64_t mt0 = (int64_t)tm * kLinTile, nt0 = (int64_t)tn * kLinTile;
  const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
  const int g = lane >> 4, r16 = lane & 15;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t nst = p.K / G::KS;
  for (int64_t s = 0; s < G::D - 1 && s < nst; ++s) nv_dma_stage(p, mt0, nt0, s, lin_lds + s * G::STAGE);
  for (int64_t st = 0; st < nst; ++st) {
    const int64_t later = min((int64_t)(G::D - 2), nst - 1 - st);
    wait_vmcnt((int)(later * G::INSTS));
    // bare barrier, as in k_linear_dma: this stage has landed for every wave, and the
    // buffer refilled next was last read before it
    asm volatile("s_barrier" ::: "memory");
    if (st + G::D - 1 < nst)
      nv_dma_stage(p, mt0, nt0, st + G::D - 1, lin_lds + ((st + G::D - 1) % G::D) * G::STAGE);
    const uint8_t* cur = lin_lds + (st % G::D) * G::STAGE;
    NvFrag fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = nv_frag(cur, cur + 2 * G::TILE, wm + 16 * i + r16, g);
      fb[i] = nv_frag(cur + G::TILE, cur + 2 * G::TILE + G::STILE, wn + 16 * i + r16, g);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = nv_expand(fa[i], u);
        b[i] = nv_expand(fb[i], u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
  }
  lin_store<OUT_BF16>(acc, p, mt0 + wm, nt0 + wn, gp(p.ats)[0] * gp(p.bts)[0]);
}

// ---------------------------------------------------------------- MXINT4 -> MXFP6 E2M3
// The matrix cores take no integer elements under E8M0 scales, but every MXINT4 element
// q * 2^(e-2) (q in [-7, 7]) is exactly an E2M3 value times an E8M0 scale: q itself under
// scale 2^(e-2), or q / 2^(2-(e+127)) under the smallest scale 2^-127 when e - 2 is below
// it (q / 2 and q / 4 are E2M3 values for every q).  One thread per 32-element block: read
// its 16 bytes of nibbles and its scale, write 24 bytes of 6-bit codes and the new scale.
__global__ __launch_bounds__(256) void k_recode_mxint4_e2m3(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t nblocks, uint8_t* out_codes,
                                                            uint8_t* out_scales) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4 w = gp((const u32x4*)codes)[b];
  const uint32_t sc = gp(scales)[b];
  const float f = sc >= 2u ? 1.0f : (sc == 1u ? 0.5f : 0.25f);
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  f32x16 ev = {}, od = {};
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int q = ((int)(ww[k >> 3] << (28 - 4 * (k & 7)))) >> 28;   // sign-extended nibble
    const float v = (float)q * f;                                       // exact
    if (k & 1) od[k >> 1] = v; else ev[k >> 1] = v;
  }
  // the 2xpk16 conversion interleaves its sources: even elements first source, odd second
  const u32x6 c = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
  DQ_GAS u32x2* o = gp((u32x2*)(out_codes + 24 * b));
  o[0] = u32x2{c[0], c[1]};
  o[1] = u32x2{c[2], c[3]};
  o[2] = u32x2{c[4], c[5]};
  gp(out_scales)[b] = (uint8_t)(sc >= 2u ? sc - 2u : 0u);
}

// ---------------------------------------------------------------- INT4 on the int8 cores
// INT4 (two's-complement nibbles, one bf16 scale per group of 64 or 128 elements along K)
// has no block-scaled matrix-core form: its scales are bf16 values, not powers of two.
// Within a group every product is an integer, so V_MFMA_I32_16X16X64_I8 sums a 64-element
// step exactly in int32: each lane gives 16 of the 64 elements of its row, and since the A
// and B lanes of one K-group pick the same 16, which 16 does not matter.  A nibble goes to
// the high half of its byte (the byte is 16 q, so no sign extension is needed) and the
// int32 sum is 256 P, P the group's integer dot product (|P| <= 64 * 64 per step).  Per
// output and group the wave then converts 256 P to fp32 (exact), multiplies the two bf16
// scales (an 8-bit by 8-bit significand product: exact in fp32) and adds P * sa * sb to the
// fp32 accumulator with one fma; 2^-8 and r are applied at the store.
//
// Those three vector operations per output and group, plus one per four elements to
// unpack the nibbles, outweigh the int8 cores' share (16 cycles per instruction of 16 x 16
// x 64 against 4 x 4 cycles for one wave-wide vector operation): the kernel is bound by the
// vector ALU, not by the matrix cores or HBM.
//
// Staging: a ring of two stages of 256 K (128 bytes of codes per tile row, as the FP4
// direct-to-LDS kernel, chunks XOR-swizzled by row); codes go to LDS by direct-to-LDS
// global loads, clamped to the row start past K (those steps are skipped); each thread
// loads its share of the stage's bf16 scales into registers and writes them to LDS as fp32
// after the products, so any K that is a multiple of the group runs in the one kernel.
// TM: rows of the activation tile.  128 (four waves of 64 x 64 over a 128 x 128 tile) for
// many tokens; 32 (four waves of 32 x 32 side by side over a 32 x 128 tile) for a few, so
// that 82 tokens fill 96 tile rows instead of 128 and three times as many tiles share the
// GPU.  The weight tile is 128 rows either way.
template <int TM>
struct I4Geom {
  static constexpr int KS = 256;                  // K per stage
  static constexpr int SUB = KS / 64;             // 64-element steps per stage
  static constexpr int ROWB = KS / 2;             // 128 bytes of codes per tile row
  static constexpr int CPR = ROWB / 16;           // 8 chunks
  static constexpr int RPI = 64 / CPR;            // 8 rows per wave load
  static constexpr int ATILE = TM * ROWB;         // activation codes: 16 or 4 KiB
  static constexpr int BTILE = kLinTile * ROWB;   // weight codes: 16 KiB
  static constexpr int ASTILE = SUB * TM * 4;     // fp32 scales [4 slots][TM rows]
  static constexpr int BSTILE = SUB * kLinTile * 4;   // fp32 scales [4 slots][128 rows]: 2 KiB
  static constexpr int STAGE = ATILE + BTILE + ASTILE + BSTILE;
  static constexpr int D = 2;                     // ring depth
  static constexpr int LDS = D * STAGE;           // 72 or 45 KiB
  static constexpr int A_INSTS = TM / RPI / 4;    // loads per wave: 4 or 1 (activations)
  static constexpr int B_INSTS = kLinTile / RPI / 4;   // 4 (weights)
  static constexpr int WM = TM == 128 ? 64 : 32;  // wave block
  static constexpr int WN = TM == 128 ? 64 : 32;
  static constexpr int BI = WM / 16, BJ = WN / 16;   // instruction tiles per wave block
};
typedef int v4i __attribute__((ext_vector_type(4)));

template <int TM>
__device__ __forceinline__ void i4_codes(const LinArgs& p, int64_t mt0, int64_t nt0, int64_t st,
                                         uint8_t* buf) {
  using G = I4Geom<TM>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rowbytes = p.K / 2;
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    const uint8_t* codes = op ? p.b : p.a;
    const int64_t r0 = op ? nt0 : mt0, rows = op ? p.N : p.M;
    uint8_t* tile = buf + op * G::ATILE;
    const int insts = op ? G::B_INSTS : G::A_INSTS;
#pragma unroll
    for (int ii = 0; ii < insts; ++ii) {
      const int rbase = (wave * insts + ii) * G::RPI;
      const int r = rbase + lane / G::CPR, c = lane % G::CPR;
      int64_t row = r0 + r;
      row = row < rows ? row : rows - 1;
      int64_t off = st * G::ROWB + 16 * (c ^ swz128(r));
      off = off < rowbytes ? off : 0;   // past K: the row's first chunk (never multiplied)
      __builtin_amdgcn_global_load_lds((const DQ_GAS void*)(codes + row * rowbytes + off),
                                       (__attribute__((address_space(3))) void*)(tile + rbase * G::ROWB),
                                       16, 0, 0);
    }
  }
}

// This thread's share of a stage's scales: tile row t / 2 of both operands (activation rows
// only below TM); with groups of 64 the two bf16 of steps 2 (t % 2) and +1, with groups of
// 128 the one bf16 of group t % 2 of the stage.  Past K the row's first scale is read (its
// steps are skipped).  The values stay as loaded until i4_scales_store, so nothing waits for
// these loads before the stage's products (combining the two halves here made every stage
// wait a round of load latency before requesting the next stage's codes).
template <int GS, int TM>
__device__ __forceinline__ void i4_scales_load(const LinArgs& p, int64_t mt0, int64_t nt0,
                                               int64_t st, uint32_t (&sv)[2][2]) {
  const int rr = threadIdx.x >> 1, h = threadIdx.x & 1;
  const int64_t ng = p.K / (64 * GS);
  sv[0][0] = sv[0][1] = 0u;
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    if (op == 0 && rr >= TM) continue;
    const uint16_t* sc = (const uint16_t*)(op ? p.bs : p.as);
    const int64_t r0 = op ? nt0 : mt0, rows = op ? p.N : p.M;
    int64_t row = r0 + rr;
    row = row < rows ? row : rows - 1;
    const DQ_GAS uint16_t* sr = gp(sc + row * ng);
    if (GS == 1) {
      int64_t g0 = 4 * st + 2 * h, g1 = g0 + 1;
      g0 = g0 < ng ? g0 : 0;
      g1 = g1 < ng ? g1 : 0;
      sv[op][0] = sr[g0];
      sv[op][1] = sr[g1];
    } else {
      int64_t g0 = 2 * st + h;
      g0 = g0 < ng ? g0 : 0;
      sv[op][0] = sr[g0];
    }
  }
}
// LDS scale tile of an operand: fp32 [4 slots][rows], slot k = the scale of the stage's k-th
// group (slots 2, 3 unused with groups of 128), so that the scales of four consecutive rows
// are one 16-byte read.
template <int GS, int TM>
__device__ __forceinline__ void i4_scales_store(uint8_t* buf, const uint32_t (&sv)[2][2]) {
  using G = I4Geom<TM>;
  const int rr = threadIdx.x >> 1, h = threadIdx.x & 1;
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    if (op == 0 && rr >= TM) continue;
    const int rows = op ? kLinTile : TM;
    float* t = (float*)(buf + G::ATILE + G::BTILE + op * G::ASTILE);
    if (GS == 1) {
      t[(2 * h) * rows + rr] = u2f(sv[op][0] << 16);
      t[(2 * h + 1) * rows + rr] = u2f(sv[op][1] << 16);
    } else {
      t[h * rows + rr] = u2f(sv[op][0] << 16);
    }
  }
}

// 16 nibbles (8 bytes, low nibble first) -> 16 bytes of 16 q for the int8 cores.  The byte
// order differs from the element order; A and B are unpacked alike.
__device__ __forceinline__ v4i i4_unpack(uint64_t x) {
  const uint32_t w0 = (uint32_t)x, w1 = (uint32_t)(x >> 32), m = 0xF0F0F0F0u;
  return v4i{(int)((w0 << 4) & m), (int)(w0 & m), (int)((w1 << 4) & m), (int)(w1 & m)};
}

template <int GS, int OUT_BF16, int TM>
__global__ __launch_bounds__(256) void k_linear_i4(LinArgs p) {
  using G = I4Geom<TM>;
  constexpr int BI = G::BI, BJ = G::BJ;
  extern __shared__ __align__(16) uint8_t lin_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // work item = (tile, split); the splits of one tile are consecutive items, so they run on
  // one XCD and share the activation tile in its L2
  const int item = lin_item(p.tiles_m * p.tiles_n * p.ksplit);
  const int tile = item / p.ksplit, split = item % p.ksplit;
  const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;
  const int64_t mt0 = (int64_t)tm * TM, nt0 = (int64_t)tn * kLinTile;
  const int wm = TM == 128 ? (wave & 1) * 64 : 0, wn = TM == 128 ? (wave >> 1) * 64 : wave * 32;
  const int g = lane >> 4, r16 = lane & 15;

  f32x4 acc[BI][BJ];
#pragma unroll
  for (int i = 0; i < BI; ++i)
#pragma unroll
    for (int j = 0; j < BJ; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t nsub = p.K / 64;
  const int64_t nst_all = (nsub + G::SUB - 1) / G::SUB;
  const int64_t st0 = (int64_t)split * p.st_split;                     // this split's stages
  const int64_t nst = st0 + p.st_split < nst_all ? st0 + p.st_split : nst_all;
  uint32_t sv[2][2];
  if (st0 < nst) {
    i4_scales_load<GS, TM>(p, mt0, nt0, st0, sv);
    i4_codes<TM>(p, mt0, nt0, st0, lin_lds);
    i4_scales_store<GS, TM>(lin_lds, sv);
  }
  for (int64_t st = st0; st < nst; ++st) {
    // This stage's codes (the only loads outstanding) have landed and every thread has
    // written its scales; the buffer refilled next was last read before this barrier.
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("s_barrier" ::: "memory");
    const bool more = st + 1 < nst;
    uint8_t* nxt = lin_lds + ((st - st0 + 1) & 1) * G::STAGE;
    if (more) {
      i4_scales_load<GS, TM>(p, mt0, nt0, st + 1, sv);
      i4_codes<TM>(p, mt0, nt0, st + 1, nxt);
    }
    const uint8_t* cur = lin_lds + ((st - st0) & 1) * G::STAGE;
    const float* sa_t = (const float*)(cur + G::ATILE + G::BTILE);
    const float* sb_t = (const float*)(cur + G::ATILE + G::BTILE + G::ASTILE);
#pragma unroll
    for (int k = 0; k < G::SUB / GS; ++k) {
      if (st * G::SUB + GS * k >= nsub) break;   // the same for the whole workgroup
      v4i P[BI][BJ];
#pragma unroll
      for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j) P[i][j] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < GS; ++h) {
        const int u = GS * k + h;   // 64-element step: chunks 2u, 2u + 1 of the row
        v4i a[BI], b[BJ];
#pragma unroll
        for (int i = 0; i < BI; ++i) {
          const int ra = wm + 16 * i + r16;
          const int ca = (2 * u + (g >> 1)) ^ swz128(ra);
          a[i] = i4_unpack(*(const uint64_t*)(cur + ra * G::ROWB + 16 * ca + 8 * (g & 1)));
        }
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
          const int rb = wn + 16 * j + r16;
          const int cb = (2 * u + (g >> 1)) ^ swz128(rb);
          b[j] = i4_unpack(*(const uint64_t*)(cur + G::ATILE + rb * G::ROWB + 16 * cb + 8 * (g & 1)));
        }
#pragma unroll
        for (int i = 0; i < BI; ++i)
#pragma unroll
          for (int j = 0; j < BJ; ++j)
            P[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b[j], a[i], P[i][j], 0, 0, 0);
      }
      // P[i][j][v] belongs to row wm + 16 i + r16 and column wn + 16 j + 4 g + v
      float sa[BI];
      f32x4 sb[BJ];
#pragma unroll
      for (int i = 0; i < BI; ++i) sa[i] = sa_t[k * TM + wm + 16 * i + r16];
#pragma unroll
      for (int j = 0; j < BJ; ++j) sb[j] = *(const f32x4*)(sb_t + k * kLinTile + wn + 16 * j + 4 * g);
#pragma unroll
      for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[i][j][v] = __builtin_fmaf((float)P[i][j][v], sa[i] * sb[j][v], acc[i][j][v]);
    }
    if (more) i4_scales_store<GS, TM>(nxt, sv);
  }

  if (p.part) {
    // unscaled partial sums of this split: acc[i][j][v] is the product at row
    // mt0 + wm + 16 i + lane % 16, column nt0 + wn + 16 j + 4 (lane / 16) + v
    float* base = p.part + (int64_t)split * p.M * p.ldp;
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int64_t m = mt0 + wm + 16 * i + r16;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        const int64_t n = nt0 + wn + 16 * j + 4 * g;
        if (n < p.N) *gp((f32x4*)(base + m * p.ldp + n)) = acc[i][j];   // ldp >= N rounded to 4
      }
    }
    return;
  }
  lin_store<OUT_BF16, BI, BJ>(acc, p, mt0 + wm, nt0 + wn, 1.0f / 256.0f);
}

// The split sums of k_linear_i4 added in split order, then scaled as the unsplit kernel
// scales its accumulator: Y[m][n] = ((sum_s part[s][m][n]) * 2^-8) * r[n].  One thread per
// four consecutive columns of a row.
template <int OUT_BF16>
__global__ __launch_bounds__(256) void k_linear_i4_reduce(LinArgs p) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = (p.N + 3) / 4;
  if (q >= p.M * per_row) return;
  const int64_t m = q / per_row, n = 4 * (q % per_row);
  f32x4 s = *gp((const f32x4*)(p.part + m * p.ldp + n));
  // eight splits' loads requested at once (clamped to the last split, not added), then
  // added in split order
  for (int k0 = 1; k0 < p.ksplit; k0 += 8) {
    f32x4 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u < p.ksplit ? k0 + u : p.ksplit - 1;
      t[u] = *gp((const f32x4*)(p.part + ((int64_t)k * p.M + m) * p.ldp + n));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < p.ksplit) s = f32x4{s.x + t[u].x, s.y + t[u].y, s.z + t[u].z, s.w + t[u].w};
  }
  float yv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (n + v >= p.N) break;
    const float rn = p.r ? gp(p.r)[n + v] : 1.0f;
    const float x = (yv[v] * (1.0f / 256.0f)) * rn;
    const int64_t o = m * p.ldy + n + v;
    if (OUT_BF16) gp((uint16_t*)p.y)[o] = (uint16_t)(f2u(bf16_rne(x)) >> 16);
    else gp((float*)p.y)[o] = x;
  }
}

}  // namespace dqk
