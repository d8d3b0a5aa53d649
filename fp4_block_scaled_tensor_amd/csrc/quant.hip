// Block-scaled FP4 quantizer kernels for gfx950 (HBM-bound).
//
// "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach (접근 방법):
// per-operand cached amax and scale target T set the tensor scale; block scales are
// nearest-even and saturating, a zero scale becomes one; the E2M1 payload is nearest-even
// (stochastic for dY); weights use 2D 16x16 blocks shared by the forward and backward views.
// "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs", methodology (방법론):
// transposed layouts are produced by a fused transpose + quantize pass through on-chip
// memory instead of a separate transpose in HBM.
// "技術概要：MXFP4 による大規模言語モデルの事前学習", method (手法): deterministic H16/H32
// Hadamard rotation of the weight-gradient operands, fused here into the transposed pass.
//
// Kernels:
//   k_quant_row_t ROW view on 8 x 1024 tiles: 8 elements per lane, a block's maximum over B/8
//                 lanes by DPP (any input whose in-tile offsets fit 32 bits).
//   k_quant_row   ROW view, general form and the tile-local (LOCAL) pass: one thread per
//                 B-element block along the row, two rows per thread with both rows' loads
//                 issued first; a workgroup covers several rows when a row has fewer than 256
//                 blocks; 16-byte loads.
//   k_quant_col   COL view: a 128-token x 64-feature tile staged in LDS (four workgroups fit a
//                 CU); each thread owns a 16/32-token run of one feature (optionally rotated by
//                 the FWHT), writes its payload to an LDS output tile, which is stored
//                 row-contiguously.
//   k_quant_2d    TILE2D: a 64x64 tile in LDS; tile amaxes by lane shuffles; both the forward
//                 payload (row segments) and the transposed payload (column segments).
//   k_amax_*      max|x| (plain, or along-token FWHT for Hadamard views): a workgroup max, then
//                 at most one atomicMax per workgroup on the float bits (non-negative floats
//                 order like unsigned integers), skipped when the result already holds more.
// The quantize kernels also write the operand's g (workgroup 0, thread 0) and, if asked,
// fold their block maxima into the observed amax (one atomic per workgroup).
#include <algorithm>
#include <type_traits>

#include "quant_common.hpp"

namespace fp4k {

// Tile order across the XCDs: consecutive workgroup ids land on the 8 XCDs in turn, each with
// its own L2. With xcd_tile, XCD k takes the k-th contiguous run of tiles instead, so
// neighbouring tiles, which write the two halves (or quarters) of the same 128-byte lines of
// the payload and scale arrays, complete those lines in one L2 before they are written back.
// (Used by the COL and TILE2D kernels, whose tiles write 64- and 32-byte pieces of the
// transposed payload rows: at 8192 x 4096 the COL view 32.6 -> 27.9 us, the 14336 x 4096
// weight 46.2 -> 43.0 us. The ROW kernel writes whole lines of payload and keeps the
// round-robin order: 17.7 against 18.9 us chunked.)
__device__ __forceinline__ uint32_t xcd_tile(uint32_t id, uint32_t total) {
  if ((total & 7) == 0) return (id & 7) * (total >> 3) + (id >> 3);
  return id;
}

// ---------------------------------------------------------------- ROW view
// Thread layout: TPR threads per row (a power of two, at most NT), NT / TPR rows per pass;
// block index b = blockIdx.x * TPR + (thread % TPR). Each thread does rows r and r + RPW/2
// of a group of RPW = 2 NT / TPR rows, both rows' loads issued before either is used.
template <int B, bool F32>
__device__ __forceinline__ void load_block(const void* x, int64_t elem, float (&v)[B]) {
#pragma unroll
  for (int j = 0; j < B / 8; ++j) load8<F32>(x, elem + 8 * j, v + 8 * j);
}

template <int FMT, int B, bool SR>
__device__ __forceinline__ float quant_block_row(const float (&v)[B], const TensorScales& ts, int64_t r, int64_t b,
                                                 int64_t cols, uint64_t seed, uint64_t offset, uint8_t* __restrict__ q,
                                                 uint8_t* __restrict__ s, Health& h) {
  float amax_b = 0.0f;
#pragma unroll
  for (int j = 0; j < B; ++j) amax_b = mag_max(amax_b, fabsf(v[j]));
  uint32_t code;
  float mult;
  block_scale<FMT>(amax_b, ts, code, mult, h);
  uint32_t words[B / 8];
  payload<B, SR>(v, mult, (uint64_t)(r * cols + b * B), seed, offset, words);
  uint8_t* qp = q + r * (cols / 2) + b * (B / 2);
  if constexpr (B == 16) out_u2<true>(qp, words[0], words[1]);
  else out_u4<true>(qp, words[0], words[1], words[2], words[3]);
  out_u8<true>(s + r * (cols / B) + b, (uint8_t)code);
  return amax_b;
}

// LOCAL (tile-local tensor scales): d_amax holds one amax per stripe of 2^stripe_log2 rows and
// row r uses the tensor scales of d_amax[r >> stripe_log2]; g is not written (the caller
// turns the stripe maxima into g afterwards) and d_amax_obs is not used.
template <int FMT, int B, bool SR, bool F32, bool LOCAL = false>
__global__ __launch_bounds__(NT) void k_quant_row(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                                                  int tpr_log2, const float* __restrict__ d_amax, float T,
                                                  uint64_t seed, uint64_t offset, uint8_t* __restrict__ q,
                                                  uint8_t* __restrict__ s, float* __restrict__ d_amax_obs,
                                                  float* __restrict__ d_g, int stripe_log2 = 0,
                                                  uint32_t* __restrict__ stats = nullptr) {
  const int tpr = 1 << tpr_log2;
  const int half_rows = NT >> tpr_log2;                // rows per pass
  const int64_t nbr = cols / B;
  const int64_t b = (int64_t)blockIdx.x * tpr + (threadIdx.x & (tpr - 1));
  TensorScales ts{1.0f, 1.0f, 1.0f};
  if constexpr (!LOCAL) {
    if constexpr (FMT != FMT_E8M0) ts = tensor_scales(d_amax, T);
    write_g<FMT>(d_g, ts);
  }
  float obs = 0.0f;
  Health h;
  if (b < nbr) {
    // row groups of 2 * half_rows rows, strided over the grid (one group per workgroup
    // unless the matrix has more than 65535 groups)
    for (int64_t rg = blockIdx.y; rg * 2 * half_rows < rows; rg += gridDim.y) {
      const int64_t r0 = rg * (2 * half_rows) + (threadIdx.x >> tpr_log2);
      const int64_t r1 = r0 + half_rows;
      const bool has0 = r0 < rows, has1 = r1 < rows;
      TensorScales ts0 = ts, ts1 = ts;
      if constexpr (LOCAL) {
        ts0 = tensor_scales_from(has0 ? d_amax[r0 >> stripe_log2] : 0.0f, T);
        ts1 = tensor_scales_from(has1 ? d_amax[r1 >> stripe_log2] : 0.0f, T);
      }
      float v0[B], v1[B];
      if (has0) load_block<B, F32>(x, r0 * ld + b * B, v0);
      if (has1) load_block<B, F32>(x, r1 * ld + b * B, v1);
      if (has0) obs = mag_max(obs, quant_block_row<FMT, B, SR>(v0, ts0, r0, b, cols, seed, offset, q, s, h));
      if (has1) obs = mag_max(obs, quant_block_row<FMT, B, SR>(v1, ts1, r1, b, cols, seed, offset, q, s, h));
    }
  }
  if (!LOCAL && d_amax_obs) wg_max_to(d_amax_obs, obs);
  if (!LOCAL) health_flush(stats, h);
}

// ROW view on QT x QF tiles (8 x 1024; with HBM-streamed inputs at 8192 x 4096: UE5M3 18.1 us
// against 19.3 for the per-block-thread form, MXFP4 18.0 either way): lane l of a pass loads
// the 8 elements [8(l%QL), 8(l%QL)+8) of token row l/QL (QL = QF/8 = 128 lanes read one 2 KB
// bf16 row segment), a block
// spans B/8 neighbouring lanes whose maxima combine by DPP, each lane stores its 4 payload
// bytes and the block's first lane the scale code. Raw buffer loads/stores: lanes outside the
// matrix use an out-of-range offset (the hardware drops them). Used when the in-tile offsets
// fit 32 bits (ld * elem_size <= 2^24 bytes, cols <= 2^25).
#ifndef FP4_ROW_TILE
#define FP4_ROW_TILE 8, 1024
#endif
// Stripe-maximum pieces of the two-pass tile-local quantizer: at most this many columns
// and at least 2^FP4_SAMAX_MIN_ROWS_LOG2 rows per workgroup, about FP4_SAMAX_WPC workgroups
// per CU, FP4_SAMAX_UL 16-byte loads in flight per thread. The tensor maximum's grid has about
// FP4_AMAX_WPC workgroups per CU. Both end in one atomic max per workgroup, and atomics on one
// address serialize across the chip: at 8192 x 4096 bf16 the tensor maximum takes 25.6 us with
// 2048 workgroups, 21.3 with 512, 17.8 with 768 (three per CU), and the 128-row stripe
// quantizer 49 us with 4 stripe-maximum workgroups per CU against 38 with one (and 8 loads in
// flight per thread).
#ifndef FP4_SAMAX_COLS
#define FP4_SAMAX_COLS 4096
#endif
#ifndef FP4_SAMAX_MIN_ROWS_LOG2
#define FP4_SAMAX_MIN_ROWS_LOG2 0
#endif
#ifndef FP4_AMAX_WPC
#define FP4_AMAX_WPC 3
#endif
#ifndef FP4_SAMAX_UL
#define FP4_SAMAX_UL 8
#endif
#ifndef FP4_SAMAX_WPC
#define FP4_SAMAX_WPC 1
#endif
static_assert(FP4_SAMAX_COLS % 8 == 0 && FP4_SAMAX_COLS >= 64 && FP4_SAMAX_COLS <= (1 << 20),
              "stripe-maximum chunk must be a multiple of 8 columns within [64, 2^20]");

#ifndef FP4_ROW_TILED
#define FP4_ROW_TILED 1
#endif
constexpr int ROW_TILE[2] = {FP4_ROW_TILE};
constexpr int QT = ROW_TILE[0], QF = ROW_TILE[1];
constexpr int QL = QF / 8, QPP = NT / QL, QPASSES = QT / QPP;
static_assert(QL <= NT && NT % QL == 0 && QPASSES >= 1 && QPASSES * QPP == QT, "row tile");

template <int FMT, int B, bool SR, bool F32>
__global__ __launch_bounds__(NT) void k_quant_row_t(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t ld, const float* __restrict__ d_amax, float T,
                                                    uint64_t seed, uint64_t offset, uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ s, float* __restrict__ d_amax_obs,
                                                    float* __restrict__ d_g, uint32_t* __restrict__ stats) {
  constexpr int LB = B / 8;                     // lanes per block
  constexpr int ESZ = F32 ? 4 : 2;
  const int64_t nft = (cols + QF - 1) / QF;
  const int64_t t0 = (int64_t)(blockIdx.x / nft) * QT, f0 = (int64_t)(blockIdx.x % nft) * QF;
  TensorScales ts{1.0f, 1.0f, 1.0f};
  if constexpr (FMT != FMT_E8M0) ts = tensor_scales(d_amax, T);
  write_g<FMT>(d_g, ts);
  const int lc = threadIdx.x % QL, lr = threadIdx.x / QL;
  const int rl = (int)min(rows - t0, (int64_t)QT), cl = (int)min(cols - f0, (int64_t)QF);
  const bool cok = lc * 8 < cl;
  const rsrc_t rx = make_rsrc(reinterpret_cast<const char*>(x) + (t0 * ld + f0) * ESZ);
  const uint32_t qcols = (uint32_t)(cols / 2), scols = (uint32_t)(cols / B);
  const rsrc_t rq = make_rsrc(q + t0 * (int64_t)qcols + f0 / 2);
  const rsrc_t rs = make_rsrc(s + t0 * (int64_t)scols + f0 / B);
  const uint32_t ld_b = (uint32_t)(ld * ESZ);
  Chunk8<F32> c[QPASSES];
#pragma unroll
  for (int p = 0; p < QPASSES; ++p) {
    const int r = p * QPP + lr;
    c[p].load(rx, (cok && r < rl) ? (uint32_t)r * ld_b + (uint32_t)(lc * 8 * ESZ) : OOB);
  }
  float obs = 0.0f;
  Health h;
#pragma unroll
  for (int p = 0; p < QPASSES; ++p) {
    const int r = p * QPP + lr;
    const bool ok = cok && r < rl;
    float v[8];
    c[p].to_float(v);
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = mag_max(am, fabsf(v[j]));
    am = group_max<LB>(am);
    uint32_t code;
    float mult;
    Health hb;
    block_scale<FMT>(am, ts, code, mult, hb);
    h.add_if(ok && (lc & (LB - 1)) == 0, hb);     // one count per block (its first lane)
    uint32_t w;
    payload<8, SR>(v, mult, SR ? (uint64_t)((t0 + r) * cols + f0 + lc * 8) : 0, seed, offset, &w);
    __builtin_amdgcn_raw_buffer_store_b32(w, rq, ok ? (uint32_t)r * qcols + (uint32_t)(lc * 4) : OOB, 0, ST_NT);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, rs,
                                         (ok && (lc & (LB - 1)) == 0) ? (uint32_t)r * scols + (uint32_t)(lc / LB) : OOB,
                                         0, ST_NT);
    if (ok) obs = mag_max(obs, am);
  }
  if (d_amax_obs) wg_max_to(d_amax_obs, obs);
  health_flush(stats, h);
}

// ---------------------------------------------------------------- COL view (wgrad operands)
constexpr int CT = 128;   // tokens per tile
constexpr int CF = 64;    // features per tile

template <int HN>
__device__ __forceinline__ void fwht_inplace(float* v) {
#pragma unroll
  for (int h = 1; h < HN; h <<= 1) {
#pragma unroll
    for (int i = 0; i < HN; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Stage a CT x CF tile of x (rows = tokens, cols = features) into LDS as float.
template <bool F32>
__device__ __forceinline__ void stage_tile(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                                           int64_t t0, int64_t f0, float (*tile)[CF + 1]) {
  // 8-element chunks: CT rows x (CF/8) chunks
  for (int c = threadIdx.x; c < CT * (CF / 8); c += NT) {
    const int rr = c / (CF / 8), cc = (c % (CF / 8)) * 8;
    float v[8];
    if (t0 + rr < rows && f0 + cc < cols) {
      load8<F32>(x, (t0 + rr) * ld + f0 + cc, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[rr][cc + j] = v[j];
  }
}

// COL-view quantization of one staged CT x CF tile (tokens x features): each thread owns a
// U-token run of one feature, the payload goes through the LDS output tile and is stored
// row-contiguously (feature rows of q). Returns the thread's largest block amax; adds the
// blocks of features inside the matrix to h.
template <int FMT, int B, bool SR, int HN>
__device__ __forceinline__ float col_tile(float (*tile)[CF + 1], uint32_t (*qout)[CT / 8 + 1], uint8_t (*sout)[CT / B],
                                          int64_t rows, int64_t cols, int64_t t0, int64_t f0, const TensorScales& ts,
                                          uint64_t seed, uint64_t offset, uint8_t* __restrict__ q,
                                          uint8_t* __restrict__ s, Health& h) {
  constexpr int U = (HN > B) ? HN : B;          // tokens per thread unit
  constexpr int UNITS = CT / U;                 // units per feature in a tile
  const int f = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  float obs = 0.0f;
  for (int u = w; u < UNITS; u += NT / 64) {
    if (t0 + (int64_t)u * U >= rows) break;
    float v[U];
#pragma unroll
    for (int i = 0; i < U; ++i) v[i] = tile[u * U + i][f];
    if constexpr (HN > 0) {
#pragma unroll
      for (int h0 = 0; h0 < U; h0 += HN) fwht_inplace<HN>(v + h0);   // every HN-token run of the unit
    }
#pragma unroll
    for (int bb = 0; bb < U / B; ++bb) {
      float amax_b = 0.0f;
#pragma unroll
      for (int i = 0; i < B; ++i) amax_b = mag_max(amax_b, fabsf(v[bb * B + i]));
      obs = mag_max(obs, amax_b);
      uint32_t code;
      float mult;
      Health hb;
      block_scale<FMT>(amax_b, ts, code, mult, hb);
      h.add_if(f0 + f < cols, hb);              // features past the matrix are zero padding
      uint32_t words[B / 8];
      const int tok = u * U + bb * B;           // token offset inside the tile
      payload<B, SR>(v + bb * B, mult, (uint64_t)((f0 + f) * rows + t0 + tok), seed, offset, words);
#pragma unroll
      for (int j = 0; j < B / 8; ++j) qout[f][tok / 8 + j] = words[j];
      sout[f][tok / B] = (uint8_t)code;
    }
  }
  __syncthreads();
  // store payload rows: feature f0+ff, bytes [t0/2, t0/2 + CT/2) in 8-byte pieces
  const int64_t qrow = rows / 2;
  for (int c = threadIdx.x; c < CF * (CT / 16); c += NT) {
    const int ff = c / (CT / 16), piece = c % (CT / 16);
    const int64_t tok = t0 + piece * 16;
    if (f0 + ff < cols && tok < rows) {
      out_u2<false>(q + (f0 + ff) * qrow + tok / 2, qout[ff][2 * piece], qout[ff][2 * piece + 1]);
    }
  }
  const int64_t srow = rows / B;
  for (int c = threadIdx.x; c < CF * (CT / B); c += NT) {
    const int ff = c / (CT / B), j = c % (CT / B);
    if (f0 + ff < cols && t0 + (int64_t)j * B < rows) out_u8<false>(s + (f0 + ff) * srow + t0 / B + j, sout[ff][j]);
  }
  return obs;
}

template <int FMT, int B, bool SR, bool F32, int HN>
__global__ __launch_bounds__(NT) void k_quant_col(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                                                  const float* __restrict__ d_amax, float T, uint64_t seed,
                                                  uint64_t offset, uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                                                  float* __restrict__ d_amax_obs, float* __restrict__ d_g,
                                                  uint32_t* __restrict__ stats) {
  __shared__ float tile[CT][CF + 1];
  __shared__ uint32_t qout[CF][CT / 8 + 1];     // 8 codes per dword
  __shared__ uint8_t sout[CF][CT / B];
  const uint32_t tid = xcd_tile(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
  const int64_t t0 = (int64_t)(tid % gridDim.x) * CT;
  const int64_t f0 = (int64_t)(tid / gridDim.x) * CF;
  stage_tile<F32>(x, rows, cols, ld, t0, f0, tile);
  __syncthreads();
  TensorScales ts{1.0f, 1.0f, 1.0f};
  if constexpr (FMT != FMT_E8M0) ts = tensor_scales(d_amax, T);
  write_g<FMT>(d_g, ts);
  Health h;
  const float obs = col_tile<FMT, B, SR, HN>(tile, qout, sout, rows, cols, t0, f0, ts, seed, offset, q, s, h);
  if (d_amax_obs) wg_max_to(d_amax_obs, obs);
  health_flush(stats, h);
}

// ---------------------------------------------------------------- ROW + COL views in one pass
// "Format-Aware Fusion for Fast FP4 Pretraining", abstract: the producer emits its consumers'
// layouts. One read of x gives the forward operand (ROW view) and the saved-for-backward
// operand (COL view, optionally Hadamard-rotated), each with its own cached amax, T and
// rounding.
//
// A workgroup owns a tile of RT tokens x RF features (RcTile below). Lane l of a pass loads
// the 8 elements [8(l%L), 8(l%L)+8) of token row l/L, L = RF/8 lanes per row (a nearest-even
// tile reads 512-byte bf16 row segments, which stream from HBM faster than narrower ones),
// so the ROW blocks are finished in registers: a block spans B/8 neighbouring lanes, whose
// maxima are combined with DPP quad permutes. The tile is then written to LDS in the
// input's own type for the COL view, whose payload is transposed through a small LDS tile as
// in the COL kernel. Workgroups are ordered so that each XCD walks the feature tiles of a
// token stripe in turn: the partial 128-byte lines each tile writes are completed in that
// XCD's L2 before they are written back.
// Tile shape (tokens x features): nearest-even tiles of 64 x 256 (512-byte row segments; the
// loads dominate, and wider segments stream faster from HBM); stochastic ones, bound by the
// Philox and rounding arithmetic, 128 x 64.
#ifndef FP4_RC_RT
#define FP4_RC_RT 64
#endif
#ifndef FP4_RC_RF
#define FP4_RC_RF 256
#endif
#ifndef FP4_RC_RT_SR
#define FP4_RC_RT_SR 128
#endif
#ifndef FP4_RC_RF_SR
#define FP4_RC_RF_SR 64
#endif
template <bool SR>
struct RcTile {
  static constexpr int T = SR ? FP4_RC_RT_SR : FP4_RC_RT;   // tokens per fused tile
  static constexpr int F = SR ? FP4_RC_RF_SR : FP4_RC_RF;   // features per fused tile
};

// Persistent: gridDim.x workgroups walk the tiles. When the tile count and the grid are
// multiples of 8, workgroup w (on XCD w % 8) takes tiles k*P + w/8 + i*(gridDim.x/8) of
// the contiguous run [k*P, (k+1)*P) of XCD k = w % 8 (P = tiles / 8). The next tile's
// loads are issued before the current tile is processed. Lane offsets are 32-bit: the host
// bounds ld, rows and cols so that no offset inside a tile reaches 2^31.
template <int FMT, int B, bool SRR, bool SRC, bool F32, int HN>
__global__ __launch_bounds__(NT) void k_quant_rowcol(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                     int64_t ld, const float* __restrict__ amax_r, float T_r,
                                                     uint64_t seed_r, uint64_t offset_r,
                                                     const float* __restrict__ amax_c, float T_c, uint64_t seed_c,
                                                     uint64_t offset_c, uint8_t* __restrict__ q,
                                                     uint8_t* __restrict__ s, float* __restrict__ g_r,
                                                     float* __restrict__ obs_r, uint8_t* __restrict__ qt,
                                                     uint8_t* __restrict__ st, float* __restrict__ g_c,
                                                     float* __restrict__ obs_c, uint32_t* __restrict__ stats_r,
                                                     uint32_t* __restrict__ stats_c) {
  constexpr int RT = RcTile<SRR || SRC>::T, RF = RcTile<SRR || SRC>::F;
  constexpr int U = (HN > B) ? HN : B;          // COL tokens per thread unit
  constexpr int UNITS = RT / U;
  static_assert(RF <= NT && NT % RF == 0 && RT % U == 0 && RT % 16 == 0, "COL units: whole features per thread");
  static_assert((RF * (RT / 16)) % NT == 0 && (RF * (RT / B)) % NT == 0, "COL stores: whole passes");
  static_assert(NT % (RF / 8) == 0 && RT % (NT / (RF / 8)) == 0, "ROW loads: whole passes");
  constexpr int LPR = RF / 8;                   // lanes per tile row (8 elements each)
  constexpr int RPP = NT / LPR;                 // token rows per load pass
  constexpr int PASSES = RT / RPP;
  constexpr int LB = B / 8;                     // lanes per ROW block
  constexpr int ESZ = F32 ? 4 : 2;
  using Elem = typename std::conditional<F32, float, uint16_t>::type;
  __shared__ __align__(16) Elem tile[RT][RF];
  __shared__ uint32_t qout[RF][RT / 8 + 1];
  __shared__ uint8_t sout[RF][RT / B];
  const uint32_t nft = (uint32_t)((cols + RF - 1) / RF);
  const uint32_t total = (uint32_t)((rows + RT - 1) / RT) * nft;
  const uint32_t G = gridDim.x;
  uint32_t id, stride, end;
  if ((total & 7) == 0 && (G & 7) == 0) {
    const uint32_t per = total >> 3, k = blockIdx.x & 7;
    id = k * per + (blockIdx.x >> 3);
    stride = G >> 3;
    end = (k + 1) * per;
  } else {
    id = blockIdx.x;
    stride = G;
    end = total;
  }

  TensorScales tr{1.0f, 1.0f, 1.0f}, tc{1.0f, 1.0f, 1.0f};
  if constexpr (FMT != FMT_E8M0) {
    tr = tensor_scales(amax_r, T_r);
    tc = tensor_scales(amax_c, T_c);
  }
  write_g<FMT>(g_r, tr);
  write_g<FMT>(g_c, tc);

  const int lc = threadIdx.x % LPR, lr = threadIdx.x / LPR;
  const int f = threadIdx.x % RF;
  const uint32_t ld_b = (uint32_t)(ld * ESZ);
  const uint32_t qcols = (uint32_t)(cols / 2), scols = (uint32_t)(cols / B);
  const uint32_t qrows = (uint32_t)(rows / 2), srows = (uint32_t)(rows / B);

  // loads of tile `tid` (all lanes OOB when tid is past the end: no traffic)
  auto load_tile = [&](uint32_t tid, Chunk8<F32> (&c)[PASSES]) {
    const bool any = tid < end;
    const uint32_t tt = any ? tid / nft : 0, ft = any ? tid - tt * nft : 0;
    const int64_t t0 = (int64_t)tt * RT, f0 = (int64_t)ft * RF;
    const rsrc_t rx = make_rsrc(reinterpret_cast<const char*>(x) + (t0 * ld + f0) * ESZ);
    const int rl = (int)min(rows - t0, (int64_t)RT), cl = (int)min(cols - f0, (int64_t)RF);   // valid rows, cols
    const bool cok = any && lc * 8 < cl;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = p * RPP + lr;
      c[p].load(rx, (cok && r < rl) ? (uint32_t)r * ld_b + (uint32_t)(lc * 8 * ESZ) : OOB);
    }
  };
  float orow = 0.0f, ocol = 0.0f;
  Health hrow, hcol;
  Chunk8<F32> cur[PASSES];
  load_tile(id, cur);
  // wait for the first tile here: inside the loop the current tile always comes from the
  // previous iteration's prefetch, whose wait counts are exact
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
#pragma unroll
    for (int h = 0; h < (F32 ? 2 : 1); ++h)
      asm volatile("" ::"v"(cur[p].w[h].x), "v"(cur[p].w[h].y), "v"(cur[p].w[h].z), "v"(cur[p].w[h].w));
  for (; id < end; id += stride) {
    Chunk8<F32> nxt[PASSES];
    load_tile(id + stride, nxt);
    const uint32_t tt = id / nft, ft = id - tt * nft;
    const int64_t t0 = (int64_t)tt * RT, f0 = (int64_t)ft * RF;
    const int rl = (int)min(rows - t0, (int64_t)RT), cl = (int)min(cols - f0, (int64_t)RF);
    const bool cok = lc * 8 < cl;

    // ROW view
    const rsrc_t rq = make_rsrc(q + t0 * qcols + f0 / 2);
    const rsrc_t rs = make_rsrc(s + t0 * scols + f0 / B);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = p * RPP + lr;
      const bool ok = cok && r < rl;
      float v[8];
      cur[p].to_float(v);
      float am = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) am = mag_max(am, fabsf(v[j]));
      am = group_max<LB>(am);
      uint32_t code;
      float mult;
      Health hb;
      block_scale<FMT>(am, tr, code, mult, hb);
      hrow.add_if(ok && (lc & (LB - 1)) == 0, hb);
      uint32_t w;
      payload<8, SRR>(v, mult, SRR ? (uint64_t)((t0 + r) * cols + f0 + lc * 8) : 0, seed_r, offset_r, &w);
      __builtin_amdgcn_raw_buffer_store_b32(w, rq, ok ? (uint32_t)r * qcols + (uint32_t)(lc * 4) : OOB, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, rs,
                                           (ok && (lc & (LB - 1)) == 0) ? (uint32_t)r * scols + (uint32_t)(lc / LB) : OOB,
                                           0, 0);
      if (ok) orow = mag_max(orow, am);
    }

    // stage the tile in the input's own type for the COL view
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      uint4* dst = reinterpret_cast<uint4*>(&tile[p * RPP + lr][lc * 8]);
#pragma unroll
      for (int h = 0; h < (F32 ? 2 : 1); ++h) dst[h] = cur[p].w[h];
    }
    __syncthreads();

    // COL view: thread -> (feature f, unit u) of U consecutive tokens
    for (int u = threadIdx.x / RF; u < UNITS; u += NT / RF) {
      if (u * U >= rl) break;                   // rows % U == 0: units are whole
      float c[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        if constexpr (F32) c[i] = tile[u * U + i][f];
        else c[i] = __uint_as_float((uint32_t)tile[u * U + i][f] << 16);
      }
      if constexpr (HN > 0) {
#pragma unroll
        for (int h0 = 0; h0 < U; h0 += HN) fwht_inplace<HN>(c + h0);
      }
#pragma unroll
      for (int bb = 0; bb < U / B; ++bb) {
        float amax_b = 0.0f;
#pragma unroll
        for (int i = 0; i < B; ++i) amax_b = mag_max(amax_b, fabsf(c[bb * B + i]));
        if (f < cl) ocol = mag_max(ocol, amax_b);
        uint32_t code;
        float mult;
        Health hb;
        block_scale<FMT>(amax_b, tc, code, mult, hb);
        hcol.add_if(f < cl, hb);
        uint32_t words[B / 8];
        const int tok = u * U + bb * B;
        payload<B, SRC>(c + bb * B, mult, SRC ? (uint64_t)((f0 + f) * rows + t0 + tok) : 0, seed_c, offset_c, words);
#pragma unroll
        for (int j = 0; j < B / 8; ++j) qout[f][tok / 8 + j] = words[j];
        sout[f][tok / B] = (uint8_t)code;
      }
    }
    __syncthreads();   // also: every COL read of `tile` is done before the next tile is staged
    const rsrc_t rqt = make_rsrc(qt + f0 * qrows + t0 / 2);
    const rsrc_t rst = make_rsrc(st + f0 * srows + t0 / B);
#pragma unroll
    for (int k = 0; k < RF * (RT / 16) / NT; ++k) {
      const int cc = threadIdx.x + k * NT;
      const int ff = cc / (RT / 16), piece = cc % (RT / 16);
      const bool ok = ff < cl && piece * 16 < rl;
      const v2u w2 = {qout[ff][2 * piece], qout[ff][2 * piece + 1]};
      __builtin_amdgcn_raw_buffer_store_b64(w2, rqt, ok ? (uint32_t)ff * qrows + (uint32_t)(piece * 8) : OOB, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < RF * (RT / B) / NT; ++k) {
      const int cc = threadIdx.x + k * NT;
      const int ff = cc / (RT / B), j = cc % (RT / B);
      const bool ok = ff < cl && j * B < rl;
      __builtin_amdgcn_raw_buffer_store_b8(sout[ff][j], rst, ok ? (uint32_t)ff * srows + (uint32_t)j : OOB, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) cur[p] = nxt[p];
  }
  if (obs_r) wg_max_to(obs_r, orow);
  if (obs_r && obs_c) __syncthreads();   // wg_max_to's partials array is reused
  if (obs_c) wg_max_to(obs_c, ocol);
  health_flush(stats_r, hrow);
  if (stats_r && stats_c) __syncthreads();   // health_flush's partials array is reused
  health_flush(stats_c, hcol);
}

// ---------------------------------------------------------------- ROW view, tile-local scales
// "Format-Aware Fusion for Fast FP4 Pretraining", abstract: a cooperative-thread-array-local
// NVFP4 scale domain. One workgroup owns a stripe of 2^stripe_log2 rows across all columns:
// it reduces the stripe's amax (current scaling, no global pass), derives the stripe's
// tensor scales from it with the global-scale arithmetic, then quantizes the stripe's
// blocks (the second read of the stripe is served by the L2).
template <int FMT, int B, bool SR, bool F32>
__global__ __launch_bounds__(NT) void k_quant_row_local(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                        int64_t ld, int stripe_log2, float T, uint64_t seed,
                                                        uint64_t offset, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ s, float* __restrict__ g_out,
                                                        float* __restrict__ amax_out) {
  __shared__ float part[NT / 64];
  const int64_t r0 = (int64_t)blockIdx.x << stripe_log2;
  const int64_t nr = min((int64_t)1 << stripe_log2, rows - r0);
  const int64_t chunks = cols / 8;                 // 8-element chunks per row
  // stripe amax: UL chunks per thread in flight per step
  constexpr int UL = 8;
  float m = 0.0f;
  const int64_t nch = nr * chunks;
  for (int64_t c0 = threadIdx.x; c0 < nch; c0 += UL * NT) {
    float v[UL][8];
#pragma unroll
    for (int u = 0; u < UL; ++u) {
      int64_t c = c0 + u * NT;
      c = c < nch ? c : nch - 1;                     // clamped: a repeated chunk does not change the max
      const int64_t r = c / chunks, k = (c - r * chunks) * 8;
      load8<F32>(x, (r0 + r) * ld + k, v[u]);
    }
#pragma unroll
    for (int u = 0; u < UL; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = mag_max(m, fabsf(v[u][j]));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  float A = part[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) A = mag_max(A, part[i]);
  const TensorScales ts = tensor_scales_from(A, T);
  if (threadIdx.x == 0) {
    g_out[blockIdx.x] = ts.g;
    if (amax_out) amax_out[blockIdx.x] = A;
  }
  // the stripe's blocks, UB per thread in flight per step
  constexpr int UB = 64 / B;
  const int64_t nb = cols / B, nblk = nr * nb;
  for (int64_t i0 = threadIdx.x; i0 < nblk; i0 += UB * NT) {
    float v[UB][B];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      int64_t i = i0 + u * NT;
      i = i < nblk ? i : nblk - 1;
      load_block<B, F32>(x, (r0 + i / nb) * ld + (i % nb) * B, v[u]);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int64_t i = i0 + u * NT;
      Health unused;
      if (i < nblk) quant_block_row<FMT, B, SR>(v[u], ts, r0 + i / nb, i % nb, cols, seed, offset, q, s, unused);
    }
  }
}

// Register-resident form for bf16 stripes of at most 65536 elements (e.g. 16 rows of 4096),
// 1024-thread workgroups: each thread loads up to 64 / B whole blocks of the stripe once
// (16-byte chunks, lanes on consecutive blocks), reduces the stripe maximum from the
// registers (the magnitude of a bf16 orders like its low 15 bits, so a packed 16-bit integer
// max gives it two elements at a time), then quantizes the same registers: the stripe is
// read from HBM once.
constexpr int NTL = 1024;
constexpr int LOCAL_REG_ELEMS = NTL * 64;
template <int FMT, int B, bool SR>
__global__ __launch_bounds__(NTL) void k_quant_row_local_reg(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                               int64_t ld, int stripe_log2, float T, uint64_t seed,
                                                               uint64_t offset, uint8_t* __restrict__ q,
                                                               uint8_t* __restrict__ s, float* __restrict__ g_out,
                                                               float* __restrict__ amax_out) {
  constexpr int BPT = 64 / B;    // blocks per thread
  constexpr int CPB = B / 8;     // 16-byte chunks per block
  __shared__ uint32_t part[NTL / 64];
  const int64_t r0 = (int64_t)blockIdx.x << stripe_log2;
  const int64_t nr = min((int64_t)1 << stripe_log2, rows - r0);
  const int64_t nb = cols / B, nblk = nr * nb;   // nblk <= BPT * NTL (checked by the launcher)
  uint4 raw[BPT][CPB];
#pragma unroll
  for (int u = 0; u < BPT; ++u) {
    // 32-bit index arithmetic: i < nblk <= 65536 / B
    const uint32_t i = (uint32_t)(u * NTL) + threadIdx.x, rr = i / (uint32_t)nb, bb = i - rr * (uint32_t)nb;
    if (i < (uint32_t)nblk) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + (r0 + rr) * ld + (int64_t)bb * B;
#pragma unroll
      for (int c = 0; c < CPB; ++c) raw[u][c] = *reinterpret_cast<const uint4*>(p + 8 * c);
    } else {
#pragma unroll
      for (int c = 0; c < CPB; ++c) raw[u][c] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  uint32_t mm = 0;
#pragma unroll
  for (int u = 0; u < BPT; ++u)
#pragma unroll
    for (int c = 0; c < CPB; ++c) {
      const uint4 w = raw[u][c];
      const uint32_t a = pk_max_u16(w.x & 0x7FFF7FFFu, w.y & 0x7FFF7FFFu);
      const uint32_t b = pk_max_u16(w.z & 0x7FFF7FFFu, w.w & 0x7FFF7FFFu);
      mm = pk_max_u16(mm, pk_max_u16(a, b));
    }
  uint32_t m = max(mm & 0xFFFFu, mm >> 16);   // bf16 magnitude bits
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, k));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t mb = part[0];
#pragma unroll
  for (int i = 1; i < NTL / 64; ++i) mb = max(mb, part[i]);
  const float A = __uint_as_float(mb << 16);
  const TensorScales ts = tensor_scales_from(A, T);
  if (threadIdx.x == 0) {
    g_out[blockIdx.x] = ts.g;
    if (amax_out) amax_out[blockIdx.x] = A;
  }
#pragma unroll
  for (int u = 0; u < BPT; ++u) {
    const uint32_t i = (uint32_t)(u * NTL) + threadIdx.x, rr = i / (uint32_t)nb, bb = i - rr * (uint32_t)nb;
    if (i < (uint32_t)nblk) {
      float v[B];
#pragma unroll
      for (int c = 0; c < CPB; ++c) {
        const uint4 w = raw[u][c];
        v[8 * c + 0] = bf16_lo(w.x); v[8 * c + 1] = bf16_hi(w.x); v[8 * c + 2] = bf16_lo(w.y); v[8 * c + 3] = bf16_hi(w.y);
        v[8 * c + 4] = bf16_lo(w.z); v[8 * c + 5] = bf16_hi(w.z); v[8 * c + 6] = bf16_lo(w.w); v[8 * c + 7] = bf16_hi(w.w);
      }
      Health unused;
      quant_block_row<FMT, B, SR>(v, ts, r0 + rr, (int64_t)bb, cols, seed, offset, q, s, unused);
    }
  }
}

// Two-pass form for stripes too few to fill the chip with one workgroup each: the stripe
// maxima are reduced by workgroups of (piece, stripe) into amax[stripe] (zeroed first; one
// atomic per workgroup), the row quantizer then reads them (LOCAL mode), and
// k_stripe_finalize turns each maximum into the stripe's g (and copies it out if asked).
// A piece is 2^piece_log2 rows of the stripe by chunk_cols columns; blockIdx.x enumerates
// (row piece, column chunk) with the chunk fastest. Whole-row pieces (chunk_cols = cols) read
// one contiguous span per workgroup.
template <bool F32>
__global__ __launch_bounds__(NT) void k_stripe_amax(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t ld, int stripe_log2, int piece_log2,
                                                    int64_t chunk_cols, float* __restrict__ amax) {
  const int64_t nck = (cols + chunk_cols - 1) / chunk_cols;
  const int64_t piece = (int64_t)blockIdx.x / nck, ck = (int64_t)blockIdx.x - piece * nck;
  const int64_t s0 = (int64_t)blockIdx.y << stripe_log2;
  const int64_t r0 = s0 + (piece << piece_log2);
  const int64_t rend = min(s0 + ((int64_t)1 << stripe_log2), rows);
  const int64_t nr = max((int64_t)0, min((int64_t)1 << piece_log2, rend - r0));   // 0 past a ragged stripe
  const int64_t c0 = ck * chunk_cols;
  const int64_t cw = min(chunk_cols, cols - c0) / 8;        // 8-element chunks per row of the piece
  // 32-bit index arithmetic: n <= 2^piece_log2 rows x chunk_cols / 8 (the launcher bounds it)
  const uint32_t n = (uint32_t)(nr * cw), cw32 = (uint32_t)cw;
  constexpr int UL = FP4_SAMAX_UL;
  float m = 0.0f;
  for (uint32_t i0 = threadIdx.x; i0 < n; i0 += UL * NT) {
    float v[UL][8];
#pragma unroll
    for (int u = 0; u < UL; ++u) {
      uint32_t i = i0 + u * NT;
      i = i < n ? i : n - 1;                                 // a repeated chunk does not change the max
      const uint32_t r = i / cw32, k = (i - r * cw32) * 8;
      load8<F32>(x, (r0 + r) * ld + c0 + k, v[u]);
    }
#pragma unroll
    for (int u = 0; u < UL; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = mag_max(m, fabsf(v[u][j]));
  }
  wg_max_to(amax + blockIdx.y, m);
}

__global__ void k_fill_n(float* __restrict__ p, float v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t run_fill(float* p, float v, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + NT - 1) / NT;
  hipLaunchKernelGGL(k_fill_n, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(NT), 0, stream, p, v, n);
  return hipGetLastError();
}

// g[i] holds stripe i's amax on entry and its decode scale g on exit.
__global__ void k_stripe_finalize(float* __restrict__ g, float* __restrict__ amax_out, int64_t n, float T) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float A = g[i];
    if (amax_out) amax_out[i] = A;
    g[i] = tensor_scales_from(A, T).g;
  }
}

// ---------------------------------------------------------------- TILE2D (weights)
constexpr int WT = 64;   // 64x64 weight tile per workgroup

template <int FMT, bool F32>
__global__ __launch_bounds__(NT) void k_quant_2d(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                                                 const float* __restrict__ d_amax, float T, uint8_t* __restrict__ q,
                                                 uint8_t* __restrict__ qt, uint8_t* __restrict__ s,
                                                 float* __restrict__ d_amax_obs, float* __restrict__ d_g,
                                                 uint32_t* __restrict__ stats) {
  __shared__ float tile[WT][WT + 1];
  __shared__ float mults[WT / 16][WT / 16];
  const uint32_t tid = xcd_tile(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
  const int64_t r0 = (int64_t)(tid / gridDim.x) * WT, c0 = (int64_t)(tid % gridDim.x) * WT;
  for (int c = threadIdx.x; c < WT * (WT / 8); c += NT) {
    const int rr = c / (WT / 8), cc = (c % (WT / 8)) * 8;
    float v[8];
    if (r0 + rr < rows && c0 + cc < cols) {
      load8<F32>(x, (r0 + rr) * ld + c0 + cc, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[rr][cc + j] = v[j];
  }
  __syncthreads();
  TensorScales ts = tensor_scales(d_amax, T);
  write_g<FMT>(d_g, ts);
  // forward view: thread = (row r, 16-col segment sg); lanes 4k+sg of a wave share a 16x16 tile
  const int r = threadIdx.x >> 2, sg = threadIdx.x & 3;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = tile[r][sg * 16 + i];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = mag_max(m, fabsf(v[i]));
  m = mag_max(m, __shfl_xor(m, 4, 64));
  m = mag_max(m, __shfl_xor(m, 8, 64));
  m = mag_max(m, __shfl_xor(m, 16, 64));
  m = mag_max(m, __shfl_xor(m, 32, 64));
  uint32_t code;
  float mult;
  Health hb, h;
  block_scale<FMT>(m, ts, code, mult, hb);
  const bool rvalid = (r0 + r) < rows && (c0 + sg * 16) < cols;
  h.add_if(rvalid && (r & 15) == 0, hb);        // one count per 16x16 tile
  if ((r & 15) == 0) {
    mults[r >> 4][sg] = mult;
    if (rvalid) out_u8<false>(s + ((r0 + r) >> 4) * (cols / 16) + ((c0 >> 4) + sg), (uint8_t)code);
  }
  uint32_t words[2];
  payload<16, false>(v, mult, 0, 0, 0, words);
  if (rvalid) out_u2<false>(q + (r0 + r) * (cols / 2) + (c0 + sg * 16) / 2, words[0], words[1]);
  __syncthreads();
  // transposed view: thread = (column cc, 16-row segment rs)
  const int cc = threadIdx.x >> 2, rs = threadIdx.x & 3;
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = tile[rs * 16 + i][cc];
  payload<16, false>(v, mults[rs][cc >> 4], 0, 0, 0, words);
  if ((c0 + cc) < cols && (r0 + rs * 16) < rows)
    out_u2<false>(qt + (c0 + cc) * (rows / 2) + (r0 + rs * 16) / 2, words[0], words[1]);
  if (d_amax_obs) wg_max_to(d_amax_obs, m);
  health_flush(stats, h);
}

// ---------------------------------------------------------------- amax
// Each thread reads P consecutive 8-element pieces (16 P contiguous bytes of bf16) of R
// adjacent rows per pass, all R * P = 8 loads issued before any is used. P is chosen so that
// NT * P pieces span about one row (no idle lanes on narrow rows), R = 8 / P.
template <bool F32, int P>
__global__ __launch_bounds__(NT) void k_amax_plain(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                                                   float* __restrict__ out) {
  constexpr int R = 8 / P;
  float m = 0.0f;
  const int64_t chunks = cols / 8;            // cols % 8 == 0 (validated)
  const int64_t ry = (int64_t)gridDim.y * R;
  for (int64_t p0 = ((int64_t)blockIdx.x * NT + threadIdx.x) * P; p0 < chunks; p0 += (int64_t)gridDim.x * NT * P) {
    for (int64_t r = (int64_t)blockIdx.y * R; r < rows; r += ry) {
      float v[R][P][8];
#pragma unroll
      for (int u = 0; u < R; ++u)
#pragma unroll
        for (int p = 0; p < P; ++p) {
          if (r + u < rows && p0 + p < chunks) {
            load8<F32>(x, (r + u) * ld + (p0 + p) * 8, v[u][p]);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[u][p][j] = 0.0f;
          }
        }
#pragma unroll
      for (int u = 0; u < R; ++u)
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int j = 0; j < 8; ++j) m = mag_max(m, fabsf(v[u][p][j]));
    }
  }
  wg_max_to(out, m);
}

template <bool F32, int P>
static void launch_amax(const void* x, int64_t rows, int64_t cols, int64_t ld, float* out, hipStream_t stream) {
  // a bounded grid (about FP4_AMAX_WPC workgroups per CU): one atomic per workgroup
  const int64_t chunks = cols / 8;
  const int64_t cx = (chunks + (int64_t)NT * P - 1) / ((int64_t)NT * P);
  const unsigned gx = (unsigned)(cx > 16 ? 16 : cx);
  const int64_t ry = (rows + 8 / P - 1) / (8 / P);
  const int64_t cap = std::max<int64_t>(1, (int64_t)FP4_AMAX_WPC * device_cu_count() / gx);
  const unsigned gy = (unsigned)(ry < cap ? ry : cap);
  hipLaunchKernelGGL((k_amax_plain<F32, P>), dim3(gx, gy), dim3(NT), 0, stream, x, rows, cols, ld, out);
}

template <bool F32, int HN>
__global__ __launch_bounds__(NT) void k_amax_hadamard(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                      int64_t ld, float* __restrict__ out) {
  __shared__ float tile[CT][CF + 1];
  const int64_t t0 = (int64_t)blockIdx.x * CT, f0 = (int64_t)blockIdx.y * CF;
  stage_tile<F32>(x, rows, cols, ld, t0, f0, tile);
  __syncthreads();
  const int f = threadIdx.x & 63, w = threadIdx.x >> 6;
  float m = 0.0f;
  for (int u = w; u < CT / HN; u += NT / 64) {
    float v[HN];
#pragma unroll
    for (int i = 0; i < HN; ++i) v[i] = tile[u * HN + i][f];
    fwht_inplace<HN>(v);
#pragma unroll
    for (int i = 0; i < HN; ++i) m = mag_max(m, fabsf(v[i]));   // padded rows/cols are zero
  }
  wg_max_to(out, m);
}

__global__ void k_fill_f32(float* p, float v) { *p = v; }

// health counts of a call start at zero (a kernel, not a memset: safe under graph capture)
__global__ void k_zero_stats(uint32_t* p) {
  if (threadIdx.x < FP4_STATS_WORDS) p[threadIdx.x] = 0u;
}

__global__ void k_write_g(const float* __restrict__ d_amax, float T, int fmt, float* __restrict__ d_g) {
  *d_g = (fmt == FMT_E8M0) ? 1.0f : tensor_scales(d_amax, T).g;
}

__global__ void k_cache_update(float* amax, int32_t* valid, int32_t D, int64_t step, const float* obs) {
  if (*valid == 0 || (step % D) == 0) {
    *amax = *obs;
    *valid = 1;
  }
}

__global__ void k_cache_reset(int32_t* valid) { *valid = 0; }

// Smallest and largest scale code of an operand: out[0] = min, out[1] = max (the caller's fill
// kernel sets them to 255 and 0 first); a workgroup reduction, then one atomic each.
__global__ __launch_bounds__(NT) void k_scale_range(const uint8_t* __restrict__ s, int64_t n, int32_t* out) {
  int lo = 255, hi = 0;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
    const int c = s[i];
    lo = min(lo, c);
    hi = max(hi, c);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o, 64));
    hi = max(hi, __shfl_xor(hi, o, 64));
  }
  __shared__ int part[2][NT / 64];
  if ((threadIdx.x & 63) == 0) {
    part[0][threadIdx.x >> 6] = lo;
    part[1][threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) {
      lo = min(lo, part[0][i]);
      hi = max(hi, part[1][i]);
    }
    atomicMin(out, lo);
    atomicMax(out + 1, hi);
  }
}

__global__ void k_range_init(int32_t* out) {
  out[0] = 255;
  out[1] = 0;
}

__global__ void k_debug_encode(const float* __restrict__ x, const uint16_t* __restrict__ u16, int64_t n, int which,
                               uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= n) return;
  const float v = x[i];
  uint32_t c = 0;
  if (which == 0) c = e2m1_pack2<0>(0u, v, 0.0f) & 15u;
  else if (which == 1) c = enc_scale3<FMT_UE5M3>(v);
  else if (which == 2) c = enc_scale3<FMT_E4M3>(v);
  else if (which == 3) c = e8m0_code(v);
  else c = e2m1_sr_pack2<0>(0u, e2m1_sr_twice(v, u16[i]), 0.0f) & 15u;
  out[i] = (uint8_t)c;
}

// ---------------------------------------------------------------- launchers

template <int FMT, int B, bool SR, bool F32>
static hipError_t launch_row(const QuantArgs& a) {
  const int64_t tiles = ((a.rows + QT - 1) / QT) * ((a.cols + QF - 1) / QF);
  if (FP4_ROW_TILED && a.ld * (F32 ? 4 : 2) <= (int64_t(1) << 24) && a.cols <= (int64_t(1) << 25) &&
      tiles < (int64_t(1) << 31)) {
    hipLaunchKernelGGL((k_quant_row_t<FMT, B, SR, F32>), dim3((unsigned)tiles), dim3(NT), 0, a.stream, a.x, a.rows,
                       a.cols, a.ld, a.d_amax, a.T, a.seed, a.offset, a.q, a.s, a.d_amax_obs, a.d_g, a.stats);
    return hipGetLastError();
  }
  const int64_t nbr = a.cols / B;
  int tpr_log2 = 0;
  while ((1 << tpr_log2) < nbr && (1 << tpr_log2) < NT) ++tpr_log2;     // threads per row
  const int64_t rows_per_wg = 2 * (NT >> tpr_log2);
  const int64_t groups = (a.rows + rows_per_wg - 1) / rows_per_wg;
  const unsigned gy = (unsigned)(groups < 65535 ? groups : 65535);     // the kernel strides over the rest
  dim3 grid((unsigned)((nbr + (1 << tpr_log2) - 1) >> tpr_log2), gy);
  hipLaunchKernelGGL((k_quant_row<FMT, B, SR, F32>), grid, dim3(NT), 0, a.stream, a.x, a.rows, a.cols, a.ld, tpr_log2,
                     a.d_amax, a.T, a.seed, a.offset, a.q, a.s, a.d_amax_obs, a.d_g, 0, a.stats);
  return hipGetLastError();
}

template <int FMT, int B, bool SR, bool F32, int HN>
static hipError_t launch_col(const QuantArgs& a) {
  dim3 grid((unsigned)((a.rows + CT - 1) / CT), (unsigned)((a.cols + CF - 1) / CF));
  hipLaunchKernelGGL((k_quant_col<FMT, B, SR, F32, HN>), grid, dim3(NT), 0, a.stream, a.x, a.rows, a.cols, a.ld,
                     a.d_amax, a.T, a.seed, a.offset, a.q, a.s, a.d_amax_obs, a.d_g, a.stats);
  return hipGetLastError();
}

template <int FMT, int B, bool SRR, bool SRC, bool F32, int HN>
static hipError_t launch_rowcol(const RowColArgs& a) {
  constexpr int RT = RcTile<SRR || SRC>::T, RF = RcTile<SRR || SRC>::F;
  const int64_t tiles = ((a.rows + RT - 1) / RT) * ((a.cols + RF - 1) / RF);
  // one resident wave of workgroups (rounded down to a multiple of 8 XCDs), or fewer
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_quant_rowcol<FMT, B, SRR, SRC, F32, HN>, NT, 0) !=
            hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  int64_t grid = (int64_t)per_cu * device_cu_count();
  if (grid > tiles) grid = tiles;
  if (grid >= 8) grid &= ~(int64_t)7;
  hipLaunchKernelGGL((k_quant_rowcol<FMT, B, SRR, SRC, F32, HN>), dim3((unsigned)grid), dim3(NT), 0, a.stream, a.x, a.rows, a.cols,
                     a.ld, a.amax_r, a.T_r, a.seed_r, a.offset_r, a.amax_c, a.T_c, a.seed_c, a.offset_c, a.q, a.s,
                     a.g_r, a.obs_r, a.qt, a.st, a.g_c, a.obs_c, a.stats_r, a.stats_c);
  return hipGetLastError();
}

template <int FMT, int B, bool SRR, bool SRC, bool F32>
static hipError_t rowcol_h(const RowColArgs& a) {
  if (a.hadamard_n == 16) return launch_rowcol<FMT, B, SRR, SRC, F32, 16>(a);
  if (a.hadamard_n == 32) return launch_rowcol<FMT, B, SRR, SRC, F32, 32>(a);
  return launch_rowcol<FMT, B, SRR, SRC, F32, 0>(a);
}

template <int FMT, int B, bool F32>
static hipError_t rowcol_sr(const RowColArgs& a) {
  if (a.sr_r) return a.sr_c ? rowcol_h<FMT, B, true, true, F32>(a) : rowcol_h<FMT, B, true, false, F32>(a);
  return a.sr_c ? rowcol_h<FMT, B, false, true, F32>(a) : rowcol_h<FMT, B, false, false, F32>(a);
}

template <bool F32>
static hipError_t rowcol_fmt(const RowColArgs& a) {
  if (a.fmt == FMT_E8M0) return rowcol_sr<FMT_E8M0, 32, F32>(a);
  if (a.fmt == FMT_UE5M3) return a.block == 16 ? rowcol_sr<FMT_UE5M3, 16, F32>(a) : rowcol_sr<FMT_UE5M3, 32, F32>(a);
  return a.block == 16 ? rowcol_sr<FMT_E4M3, 16, F32>(a) : rowcol_sr<FMT_E4M3, 32, F32>(a);
}

hipError_t run_quantize_rowcol(const RowColArgs& a) {
  hipError_t e = hipSuccess;
  for (float* o : {a.obs_r, a.obs_c}) {
    if (!o) continue;
    hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(1), 0, a.stream, o, 0.0f);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  for (uint32_t* h : {a.stats_r, a.stats_c}) {
    if (!h) continue;
    hipLaunchKernelGGL(k_zero_stats, dim3(1), dim3(64), 0, a.stream, h);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.rows == 0 || a.cols == 0) {
    if (a.g_r) {
      hipLaunchKernelGGL(k_write_g, dim3(1), dim3(1), 0, a.stream, a.amax_r, a.T_r, a.fmt, a.g_r);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.g_c) {
      hipLaunchKernelGGL(k_write_g, dim3(1), dim3(1), 0, a.stream, a.amax_c, a.T_c, a.fmt, a.g_c);
      e = hipGetLastError();
    }
    return e;
  }
  return a.f32 ? rowcol_fmt<true>(a) : rowcol_fmt<false>(a);
}

template <int FMT, int B, bool SR, bool F32>
static hipError_t launch_local(const LocalQuantArgs& a) {
  const int64_t stripes = (a.rows + ((int64_t)1 << a.stripe_log2) - 1) >> a.stripe_log2;
  if (stripes >= 2 * (int64_t)device_cu_count() && !F32 &&
      ((int64_t)1 << a.stripe_log2) * a.cols <= (int64_t)LOCAL_REG_ELEMS) {
    // enough stripes to fill the chip, each small enough to stay in registers: one read
    hipLaunchKernelGGL((k_quant_row_local_reg<FMT, B, SR>), dim3((unsigned)stripes), dim3(NTL), 0, a.stream, a.x,
                       a.rows, a.cols, a.ld, a.stripe_log2, a.T, a.seed, a.offset, a.q, a.s, a.g, a.amax);
    return hipGetLastError();
  }
  if (stripes >= 2 * (int64_t)device_cu_count()) {
    // enough stripes to fill the chip: one workgroup per stripe, one pass
    hipLaunchKernelGGL((k_quant_row_local<FMT, B, SR, F32>), dim3((unsigned)stripes), dim3(NT), 0, a.stream, a.x,
                       a.rows, a.cols, a.ld, a.stripe_log2, a.T, a.seed, a.offset, a.q, a.s, a.g, a.amax);
    return hipGetLastError();
  }
  // few large stripes: stripe maxima into g by (column chunk, stripe) workgroups, the row
  // quantizer with per-stripe scales, then g from the maxima
  hipError_t e;
  const unsigned fb = (unsigned)((stripes + NT - 1) / NT);
  hipLaunchKernelGGL(k_fill_n, dim3(fb), dim3(NT), 0, a.stream, a.g, 0.0f, stripes);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // Pieces for the stripe maxima: whole rows (at most FP4_SAMAX_COLS columns), as few rows
  // as it takes to have FP4_SAMAX_WPC workgroups per CU, then narrower column chunks (down
  // to 64).
  const int64_t want = FP4_SAMAX_WPC * (int64_t)device_cu_count();
  int64_t chunk = a.cols < FP4_SAMAX_COLS ? (a.cols + 7) / 8 * 8 : FP4_SAMAX_COLS;
  int piece_log2 = a.stripe_log2;
  auto pieces = [&]() { return stripes * ((int64_t)1 << (a.stripe_log2 - piece_log2)) * ((a.cols + chunk - 1) / chunk); };
  while (piece_log2 > FP4_SAMAX_MIN_ROWS_LOG2 && pieces() < want) --piece_log2;
  while (chunk > 64 && pieces() < want) chunk = (chunk / 2 + 7) / 8 * 8;
  const int64_t nx = ((int64_t)1 << (a.stripe_log2 - piece_log2)) * ((a.cols + chunk - 1) / chunk);
  if (nx >= (int64_t)1 << 31) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_stripe_amax<F32>), dim3((unsigned)nx, (unsigned)stripes), dim3(NT), 0, a.stream, a.x,
                     a.rows, a.cols, a.ld, a.stripe_log2, piece_log2, chunk, a.g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nbr = a.cols / B;
  int tpr_log2 = 0;
  while ((1 << tpr_log2) < nbr && (1 << tpr_log2) < NT) ++tpr_log2;
  const int64_t rows_per_wg = 2 * (NT >> tpr_log2);
  const int64_t groups = (a.rows + rows_per_wg - 1) / rows_per_wg;
  const unsigned gy = (unsigned)(groups < 65535 ? groups : 65535);
  dim3 grid((unsigned)((nbr + (1 << tpr_log2) - 1) >> tpr_log2), gy);
  hipLaunchKernelGGL((k_quant_row<FMT, B, SR, F32, true>), grid, dim3(NT), 0, a.stream, a.x, a.rows, a.cols, a.ld,
                     tpr_log2, a.g, a.T, a.seed, a.offset, a.q, a.s, nullptr, nullptr, a.stripe_log2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_stripe_finalize, dim3(fb), dim3(NT), 0, a.stream, a.g, a.amax, stripes, a.T);
  return hipGetLastError();
}

template <int FMT, int B>
static hipError_t local_types(const LocalQuantArgs& a) {
  if (a.stochastic) return a.f32 ? launch_local<FMT, B, true, true>(a) : launch_local<FMT, B, true, false>(a);
  return a.f32 ? launch_local<FMT, B, false, true>(a) : launch_local<FMT, B, false, false>(a);
}

hipError_t run_quantize_local(const LocalQuantArgs& a) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  if (a.fmt == FMT_UE5M3) return a.block == 16 ? local_types<FMT_UE5M3, 16>(a) : local_types<FMT_UE5M3, 32>(a);
  return a.block == 16 ? local_types<FMT_E4M3, 16>(a) : local_types<FMT_E4M3, 32>(a);
}

template <int FMT, bool F32>
static hipError_t launch_2d(const QuantArgs& a) {
  dim3 grid((unsigned)((a.cols + WT - 1) / WT), (unsigned)((a.rows + WT - 1) / WT));
  hipLaunchKernelGGL((k_quant_2d<FMT, F32>), grid, dim3(NT), 0, a.stream, a.x, a.rows, a.cols, a.ld, a.d_amax, a.T, a.q,
                     a.qt, a.s, a.d_amax_obs, a.d_g, a.stats);
  return hipGetLastError();
}

template <int FMT, int B, bool SR, bool F32>
static hipError_t dispatch_col_h(const QuantArgs& a) {
  if (a.hadamard_n == 16) return launch_col<FMT, B, SR, F32, 16>(a);
  if (a.hadamard_n == 32) return launch_col<FMT, B, SR, F32, 32>(a);
  return launch_col<FMT, B, SR, F32, 0>(a);
}

template <int FMT, int B, bool F32>
static hipError_t dispatch_view(const QuantArgs& a) {
  if (a.view == 0) return a.stochastic ? launch_row<FMT, B, true, F32>(a) : launch_row<FMT, B, false, F32>(a);
  if (a.view == 1) return a.stochastic ? dispatch_col_h<FMT, B, true, F32>(a) : dispatch_col_h<FMT, B, false, F32>(a);
  if constexpr (FMT != FMT_E8M0 && B == 16) return launch_2d<FMT, F32>(a);
  return hipErrorInvalidValue;
}

template <bool F32>
static hipError_t dispatch_fmt(const QuantArgs& a) {
  if (a.fmt == FMT_E8M0) return dispatch_view<FMT_E8M0, 32, F32>(a);
  if (a.fmt == FMT_UE5M3) return a.block == 16 ? dispatch_view<FMT_UE5M3, 16, F32>(a) : dispatch_view<FMT_UE5M3, 32, F32>(a);
  return a.block == 16 ? dispatch_view<FMT_E4M3, 16, F32>(a) : dispatch_view<FMT_E4M3, 32, F32>(a);
}

hipError_t run_quantize(const QuantArgs& a) {
  hipError_t e;
  if (a.d_amax_obs) {
    hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(1), 0, a.stream, a.d_amax_obs, 0.0f);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.stats) {
    hipLaunchKernelGGL(k_zero_stats, dim3(1), dim3(64), 0, a.stream, a.stats);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.rows == 0 || a.cols == 0) {
    // nothing to quantize: g is still defined by the tensor scale
    if (a.d_g) {
      hipLaunchKernelGGL(k_write_g, dim3(1), dim3(1), 0, a.stream, a.d_amax, a.T, a.fmt, a.d_g);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  return a.f32 ? dispatch_fmt<true>(a) : dispatch_fmt<false>(a);   // the kernel writes g
}

hipError_t run_amax(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld, int hadamard_n, float* out,
                    hipStream_t stream) {
  hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(1), 0, stream, out, 0.0f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows == 0 || cols == 0) return e;
  if (hadamard_n == 0) {
    const int64_t chunks = cols / 8;
    if (chunks >= 4 * NT) {
      if (f32) launch_amax<true, 4>(x, rows, cols, ld, out, stream);
      else launch_amax<false, 4>(x, rows, cols, ld, out, stream);
    } else if (chunks >= 2 * NT) {
      if (f32) launch_amax<true, 2>(x, rows, cols, ld, out, stream);
      else launch_amax<false, 2>(x, rows, cols, ld, out, stream);
    } else {
      if (f32) launch_amax<true, 1>(x, rows, cols, ld, out, stream);
      else launch_amax<false, 1>(x, rows, cols, ld, out, stream);
    }
    return hipGetLastError();
  }
  dim3 grid((unsigned)((rows + CT - 1) / CT), (unsigned)((cols + CF - 1) / CF));
  if (hadamard_n == 16) {
    if (f32) hipLaunchKernelGGL((k_amax_hadamard<true, 16>), grid, dim3(NT), 0, stream, x, rows, cols, ld, out);
    else hipLaunchKernelGGL((k_amax_hadamard<false, 16>), grid, dim3(NT), 0, stream, x, rows, cols, ld, out);
  } else {
    if (f32) hipLaunchKernelGGL((k_amax_hadamard<true, 32>), grid, dim3(NT), 0, stream, x, rows, cols, ld, out);
    else hipLaunchKernelGGL((k_amax_hadamard<false, 32>), grid, dim3(NT), 0, stream, x, rows, cols, ld, out);
  }
  return hipGetLastError();
}

hipError_t run_cache_update(float* amax, int32_t* valid, int32_t D, int64_t step, const float* obs, hipStream_t stream) {
  hipLaunchKernelGGL(k_cache_update, dim3(1), dim3(1), 0, stream, amax, valid, D, step, obs);
  return hipGetLastError();
}

hipError_t run_zero_stats(uint32_t* stats, hipStream_t stream) {
  hipLaunchKernelGGL(k_zero_stats, dim3(1), dim3(64), 0, stream, stats);
  return hipGetLastError();
}

hipError_t run_scale_range(const uint8_t* s, int64_t n, int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_range_init, dim3(1), dim3(1), 0, stream, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n == 0) return e;
  const int64_t want = (n + NT - 1) / NT, cap = 4 * (int64_t)device_cu_count();
  hipLaunchKernelGGL(k_scale_range, dim3((unsigned)(want < cap ? want : cap)), dim3(NT), 0, stream, s, n, out);
  return hipGetLastError();
}

hipError_t run_cache_reset(int32_t* valid, hipStream_t stream) {
  hipLaunchKernelGGL(k_cache_reset, dim3(1), dim3(1), 0, stream, valid);
  return hipGetLastError();
}

hipError_t run_debug_encode(const float* x, const uint16_t* u16, int64_t n, int which, uint8_t* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_debug_encode, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, stream, x, u16, n, which, out);
  return hipGetLastError();
}

}  // namespace fp4k
