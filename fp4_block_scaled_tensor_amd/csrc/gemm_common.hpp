// Shared pieces of the block-scaled FP4 GEMM kernels (gfx950).
//
// Model ("UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach (접근 방법),
// software GEMM model): 64-product groups; each group a float32 partial rounded to nearest
// even; groups added in K order with round-toward-zero; optional 1/1024 canonicalisation.
//
// Tiling: a workgroup of WM x WN waves owns a (WM*TM*32) x (WN*TN*32) output tile; each wave
// computes TM x TN MFMA tiles of 32x32. K advances by stages of 256 elements (4 groups,
// 128 payload bytes per row). Payload stages go straight from global memory into LDS with
// global_load_lds_dwordx4 (no staging registers), double-buffered; the scale bytes of a
// stage go through registers into a small LDS array. LDS payload rows are 128 bytes;
// 16-byte chunk j of row r sits at chunk position j ^ ((r >> 1) & 7): sixteen consecutive
// rows reading the same logical chunk then cover all 64 LDS banks (two rows per 256-byte
// bank line, eight distinct positions within each row parity).
//
// Workgroup order: 8 consecutive workgroup ids land on the 8 XCDs round-robin, so ids are
// remapped to give each XCD a contiguous run of tiles, ordered in groups of 8 M-tiles:
// consecutive workgroups on one XCD share the B tile and keep 8 A tiles hot in its L2.
#pragma once
#include "fp4_device.hpp"
#include "launch.hpp"
#include "quant_common.hpp"

namespace fp4k {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int KS = 256;        // K elements per stage
constexpr int SGR = KS / 64;   // groups per stage
constexpr int ROWB = KS / 2;   // payload bytes per row per stage

// Workgroup geometry: WM x WN waves, each TM x TN MFMA tiles of 32x32.
template <int WM_, int WN_, int TM_, int TN_>
struct Tiling {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
  static constexpr int NW = WM * WN;          // waves
  static constexpr int NT = NW * 64;          // threads
  static constexpr int BM = WM * TM * 32;     // output rows (A rows) per workgroup
  static constexpr int BN = WN * TN * 32;     // output cols (B rows) per workgroup
};

// wave index inside the workgroup, as a wave-uniform (scalar) value
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

#ifndef FP4_SWZ_SHIFT
#define FP4_SWZ_SHIFT 1
#endif
// chunk position of logical 16-byte chunk `chunk` in LDS row `row`
__device__ __forceinline__ int swz_pos(int row, int chunk) { return chunk ^ ((row >> FP4_SWZ_SHIFT) & 7); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * ROWB + (swz_pos(row, chunk) << 4); }

// LDS byte address of a pointer into a __shared__ array (a generic pointer to LDS keeps the
// LDS offset in its low 32 bits).
__device__ __forceinline__ uint32_t lds_offset(const void* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }

// One global_load_lds_dwordx4 for the wave: lane i copies the 16 bytes at sbase + voff(i)
// to LDS bytes [dst + 16 i, dst + 16 i + 16) (dst is wave-uniform and goes in M0, with the
// one-instruction gap the M0 write needs before the load). Written as inline assembly so
// that the compiler's wait-count insertion does not treat the copy as an LDS write that may
// alias later LDS reads of the other buffer: the kernels wait for these copies themselves
// (vmcnt(0) and a barrier before the buffer is read).
__device__ __forceinline__ void lds_dma16(const uint8_t* sbase, uint32_t voff, uint32_t dst) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 1\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(dst)
      : "memory", "m0");
}

// Direct global->LDS loads of one stage of a ROWS-row payload tile by NW waves. Each wave
// fills P = ROWS / (8 NW) contiguous 1024-byte LDS pieces; lane i of piece p writes LDS
// bytes [16i, 16i+16), i.e. row 8p + i/8 at chunk position i%8, so it loads the logical
// chunk stored there: chunk position ^ ((row >> 1) & 7) = (i%8) ^ ((p & 1) << 2 | i/16).
// Only two per-lane offsets exist (even and odd pieces); the piece's row base is
// wave-uniform. In a tile that reaches past the matrix, rows past it read a clamped
// (valid) row; their values only reach outputs that are not stored.
template <int ROWS, int NW>
struct StageLoader {
  static constexpr int P = ROWS / (8 * NW);
  static_assert(P >= 1 && P * 8 * NW == ROWS, "tile rows must be a multiple of 8 per wave");
  static_assert(FP4_SWZ_SHIFT == 1, "piece-parity offsets assume the row-pair swizzle");
  const uint8_t* base;     // q + row0 * K/2, wave-uniform
  uint32_t off_e, off_o;   // per-lane byte offsets inside an even / odd piece (row * K/2 + chunk * 16)
  int64_t ldq;
  int64_t last;            // last valid tile row (rows - 1 - row0), for clamping
  bool edge;               // tile reaches past the matrix

  __device__ __forceinline__ void init(const uint8_t* q, int64_t rows, int64_t K, int64_t row0) {
    ldq = K / 2;
    base = q + row0 * ldq;
    last = rows - 1 - row0;
    edge = row0 + ROWS > rows;
    const int l = threadIdx.x & 63;
    const uint32_t pos_e = (uint32_t)((l & 7) ^ (l >> 4));
    off_e = (uint32_t)((l >> 3) * ldq) + pos_e * 16;
    off_o = (uint32_t)((l >> 3) * ldq) + (pos_e ^ 4) * 16;
  }
  // stage st into lds when every row of the tile is inside the matrix and K is a multiple
  // of 256 (no clamping): scalar piece base + per-lane offset
  __device__ __forceinline__ void issue_interior(int64_t st, uint8_t* lds) const {
    const int w = wave_id();
    const uint8_t* b = base + st * ROWB;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int piece = w * P + j;
      const bool odd = (P % 2 == 0) ? (j & 1) : (piece & 1);
      lds_dma16(b + (int64_t)piece * 8 * ldq, odd ? off_o : off_e, lds_offset(lds + piece * 1024));
    }
  }
  // stage st into lds; only the last stage of a K that is not a multiple of 256 clamps chunks
  __device__ __forceinline__ void issue(int64_t st, uint8_t* lds) const {
    const int w = wave_id();
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));   // keep the edge-tile offsets inside their branch (not hoisted, not live)
    const uint32_t kb0 = (uint32_t)(st * ROWB);
    const bool full = (int64_t)kb0 + ROWB <= ldq;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int piece = w * P + j;
      const bool odd = (P % 2 == 0) ? (j & 1) : (piece & 1);
      const uint32_t dst = lds_offset(lds + piece * 1024);
      if (!(edge || !full)) {
        // scalar piece base + per-lane offset
        lds_dma16(base + ((int64_t)piece * 8 * ldq + kb0), odd ? off_o : off_e, dst);
      } else {
        const int64_t row = piece * 8 + (l >> 3);
        const int64_t r = row <= last ? row : last;
        uint32_t c = kb0 + (uint32_t)((((l & 7) ^ ((odd ? 4 : 0) | (l >> 4)))) * 16);
        if (!full && c + 16 > (uint32_t)ldq) c = (uint32_t)ldq - 16;
        lds_dma16(base, (uint32_t)(r * ldq) + c, dst);
      }
    }
  }
};

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

#ifndef FP4_GEMM_GM
#define FP4_GEMM_GM 8   // M tiles per group of the tile order
#endif

// Workgroup id -> (m tile, n tile), XCD-aware grouped order.
__device__ __forceinline__ void tile_coords(int64_t M, int64_t N, int BM, int BN, int64_t& m0, int64_t& n0) {
  const int64_t ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  const int64_t T = ntm * ntn;
  int64_t id = blockIdx.x;
  if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
  const int64_t GM = FP4_GEMM_GM;
  const int64_t gsize = GM * ntn;
  const int64_t gid = id / gsize;
  const int64_t first = gid * GM;
  const int64_t gm = (ntm - first) < GM ? (ntm - first) : GM;
  const int64_t r = id % gsize;
  m0 = (first + r % gm) * BM;
  n0 = (r / gm) * BN;
}

// Float additions are ordinary register operations: nothing orders them against the
// s_setreg that switches the rounding mode. An empty volatile asm that takes a value in and
// out of a register is ordered against the mode-switch asm (volatile asm statements keep
// their order), so routing operands and results through one pins the additions between
// the switches. It emits no instruction.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(v16f& x) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float v = x[r];
    pin(v);
    x[r] = v;
  }
}

// T0 + T1 rounded to nearest even, elementwise, called from round-toward-zero code: the
// mode is switched for the additions and restored afterwards.
__device__ __forceinline__ v16f add_rne_from_rtz(v16f T0, v16f T1) {
  mode_f32_rne();
  pin(T0);
  pin(T1);
  v16f G;
#pragma unroll
  for (int r = 0; r < 16; ++r) G[r] = T0[r] + T1[r];
  pin(G);
  mode_f32_rtz();
  pin(G);
  return G;
}

// Output row of register r of a 32x32 MFMA tile in lane l (column = l & 31).
__device__ __forceinline__ int tile_row(int r, int l) { return (r >> 2) * 8 + (l >> 5) * 4 + (r & 3); }

// Staging of a workgroup's 128 x 128 float32 output tile for the output quantizer, in the two
// 32 KB stage buffers of the K loop (free once the loop is done): rows 0-63 in st0, 64-127 in
// st1; element (r, c) sits at column c ^ ((r & 7) << 4) of its row, i.e. the row's 16-float
// blocks are permuted by the row, so that threads reading neighbouring rows' blocks spread
// over the LDS banks.
constexpr int QO_T = 128;
struct QoStage {
  float* st0;
  float* st1;
  int r0, c0;   // the wave's first row and column inside the workgroup tile
};
__device__ __forceinline__ float* qo_slot(float* st0, float* st1, int r, int c) {
  return (r < 64 ? st0 : st1) + (r & 63) * QO_T + (c ^ ((r & 7) << 4));
}

// Epilogue: nearest-even mode, optional canonicalisation, scale by alpha, store float32.
// (m0, n0) is the wave's first output row and column; tile (i, j) covers rows m0 + 32i and
// columns n0 + 32j. pre (a power of two) undoes a constant factor the K loop carried; it is
// exact and applied before the canonicalisation. epi: bits 0-7 Hadamard n; bits 8-15 / 16-23
// the log2 stripe height of A's / B's tile-local g (0: one g for the operand), in which case
// alpha = float32(g_a[row >> sa] * g_b[col >> sb]) per output. The float32 outputs are stored
// non-temporal: they stream past the L2, which keeps the operand tiles other workgroups reuse.
// With QOUT the values are also staged for the output quantizer (stage), and c may be null
// (no float32 output).
template <int TM, int TN, bool QOUT = false>
__device__ __forceinline__ void store_tiles(float* __restrict__ c, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                            v16f (&acc)[TM][TN], const float* ga, const float* gb, int canon,
                                            int epi, float pre = 1.0f, QoStage stage = QoStage{}) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) pin(acc[i][j]);   // accumulation done before the switch
  mode_f32_rne();
  const int hadamard_n = epi & 0xFF, sa = (epi >> 8) & 0xFF, sb = (epi >> 16) & 0xFF;
  const float hinv = hadamard_n ? 1.0f / (float)hadamard_n : 1.0f;
  const int l = threadIdx.x & 63;
  const bool store = !QOUT || c != nullptr;
  auto stage_value = [&](int rt, int ct, int r, float v) {
    if constexpr (QOUT)
      *qo_slot(stage.st0, stage.st1, stage.r0 + rt * 32 + tile_row(r, l), stage.c0 + ct * 32 + (l & 31)) = v;
  };
  if (sa == 0 && sb == 0) {
    float a = ga ? *ga : 1.0f;
    float b = gb ? *gb : 1.0f;
    asm volatile("" : "+v"(a), "+v"(b));        // keep the scale product after the mode switch
    float alpha = a * b;
    if (hadamard_n) alpha = alpha * hinv;
    auto value = [&](int rt, int ct, int r) {
      float v = acc[rt][ct][r] * pre;
      if (canon) v = __builtin_rintf(v * 1024.0f) * (1.0f / 1024.0f);
      return v * alpha;
    };
    if (m0 + TM * 32 <= M && n0 + TN * 32 <= N) {
      // the wave's outputs all lie inside C: one per-lane base, and every register's row
      // offset is a compile-time multiple of N (a scalar product)
      float* base = store ? c + (m0 + (l >> 5) * 4) * N + n0 + (l & 31) : nullptr;
#pragma unroll
      for (int rt = 0; rt < TM; ++rt)
#pragma unroll
        for (int ct = 0; ct < TN; ++ct)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t k = rt * 32 + (r >> 2) * 8 + (r & 3);   // tile_row(r, l) - 4 (l >> 5)
            const float v = value(rt, ct, r);
            if (store) __builtin_nontemporal_store(v, base + k * N + ct * 32);
            stage_value(rt, ct, r, v);
          }
    } else {
#pragma unroll
      for (int rt = 0; rt < TM; ++rt)
#pragma unroll
        for (int ct = 0; ct < TN; ++ct) {
          const int64_t col = n0 + ct * 32 + (l & 31);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t row = m0 + rt * 32 + tile_row(r, l);
            const float v = value(rt, ct, r);
            if (store && row < M && col < N) __builtin_nontemporal_store(v, &c[row * N + col]);
            stage_value(rt, ct, r, v);
          }
        }
    }
  } else {
    const float a0 = ga ? *ga : 1.0f, b0 = gb ? *gb : 1.0f;
#pragma unroll
    for (int rt = 0; rt < TM; ++rt)
#pragma unroll
      for (int ct = 0; ct < TN; ++ct) {
        const int64_t col = n0 + ct * 32 + (l & 31);
        float b = (sb && col < N) ? gb[col >> sb] : b0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + rt * 32 + tile_row(r, l);
          float a = (sa && row < M) ? ga[row >> sa] : a0;
          asm volatile("" : "+v"(a), "+v"(b));    // after the mode switch
          float alpha = a * b;
          if (hadamard_n) alpha = alpha * hinv;
          float v = acc[rt][ct][r] * pre;
          if (canon) v = __builtin_rintf(v * 1024.0f) * (1.0f / 1024.0f);
          v = v * alpha;
          if (store && row < M && col < N) __builtin_nontemporal_store(v, &c[row * N + col]);
          stage_value(rt, ct, r, v);
        }
      }
  }
}

// One block of the staged tile (row r, columns [c0, c0 + B)) quantized as the quantizer's ROW
// view would quantize the same float32 values: payload and scale byte stored, block maximum
// returned, health counted.
template <int FMT, int B, bool SR>
__device__ __forceinline__ float qo_block(const QoStage& st, int r, int c0, int64_t grow, int64_t gcol, int64_t N,
                                          const TensorScales& ts, const QuantOut& qo, Health& h) {
  float v[B];
#pragma unroll
  for (int k = 0; k < B / 16; ++k) {
    const float4* p = reinterpret_cast<const float4*>(qo_slot(st.st0, st.st1, r, c0 + 16 * k));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 t = p[j];
      v[16 * k + 4 * j] = t.x;
      v[16 * k + 4 * j + 1] = t.y;
      v[16 * k + 4 * j + 2] = t.z;
      v[16 * k + 4 * j + 3] = t.w;
    }
  }
  float amax_b = 0.0f;
#pragma unroll
  for (int j = 0; j < B; ++j) amax_b = mag_max(amax_b, fabsf(v[j]));
  uint32_t code;
  float mult;
  block_scale<FMT>(amax_b, ts, code, mult, h);
  uint32_t words[B / 8];
  payload<B, SR>(v, mult, (uint64_t)(grow * N + gcol), qo.seed, qo.offset, words);
  uint8_t* qp = qo.q + grow * (N / 2) + gcol / 2;
  if constexpr (B == 16) *reinterpret_cast<uint2*>(qp) = make_uint2(words[0], words[1]);
  else *reinterpret_cast<uint4*>(qp) = make_uint4(words[0], words[1], words[2], words[3]);
  qo.s[grow * (N / B) + gcol / B] = (uint8_t)code;
  return amax_b;
}

template <int FMT, int B>
__device__ __forceinline__ float qo_block_sr(const QoStage& st, int r, int c0, int64_t grow, int64_t gcol, int64_t N,
                                             const TensorScales& ts, const QuantOut& qo, Health& h) {
  return qo.sr ? qo_block<FMT, B, true>(st, r, c0, grow, gcol, N, ts, qo, h)
               : qo_block<FMT, B, false>(st, r, c0, grow, gcol, N, ts, qo, h);
}

// The output quantizer: all NTH threads of the workgroup, after every wave has staged its
// values with store_tiles<..., true>. The workgroup tile starts at (m0, n0) of C [M x N]; N is
// a multiple of the block. Writes q and s of the tile's blocks, g (workgroup 0), and folds the
// block maxima into amax_obs and the health counts into stats (one atomic each per workgroup).
template <int NTH>
__device__ __forceinline__ void quantize_out_tile(const QoStage& st, int64_t m0, int64_t n0, int64_t M, int64_t N,
                                                  const QuantOut& qo) {
  __syncthreads();
  TensorScales ts{1.0f, 1.0f, 1.0f};
  if (qo.fmt != FMT_E8M0) ts = tensor_scales(qo.amax, qo.T);
  if (qo.g && blockIdx.x == 0 && threadIdx.x == 0) *qo.g = qo.fmt == FMT_E8M0 ? 1.0f : ts.g;
  float obs = 0.0f;
  Health h;
  const int bpr = QO_T / qo.block;
  for (int id = threadIdx.x; id < QO_T * bpr; id += NTH) {
    const int r = id / bpr, c0 = (id - r * bpr) * qo.block;
    const int64_t grow = m0 + r, gcol = n0 + c0;
    if (grow >= M || gcol >= N) continue;
    float a;
    if (qo.fmt == FMT_E8M0) a = qo_block_sr<FMT_E8M0, 32>(st, r, c0, grow, gcol, N, ts, qo, h);
    else if (qo.fmt == FMT_UE5M3)
      a = qo.block == 16 ? qo_block_sr<FMT_UE5M3, 16>(st, r, c0, grow, gcol, N, ts, qo, h)
                         : qo_block_sr<FMT_UE5M3, 32>(st, r, c0, grow, gcol, N, ts, qo, h);
    else
      a = qo.block == 16 ? qo_block_sr<FMT_E4M3, 16>(st, r, c0, grow, gcol, N, ts, qo, h)
                         : qo_block_sr<FMT_E4M3, 32>(st, r, c0, grow, gcol, N, ts, qo, h);
    obs = mag_max(obs, a);
  }
  if (!qo.amax_obs && !qo.stats) return;
  uint32_t hc[3] = {h.sat, h.zero, h.nonfin};
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    obs = mag_max(obs, __shfl_xor(obs, o, 64));
#pragma unroll
    for (int k = 0; k < 3; ++k) hc[k] += __shfl_xor(hc[k], o, 64);
  }
  __shared__ float pobs[NTH / 64];
  __shared__ uint32_t ph[3][NTH / 64];
  if ((threadIdx.x & 63) == 0) {
    pobs[threadIdx.x >> 6] = obs;
#pragma unroll
    for (int k = 0; k < 3; ++k) ph[k][threadIdx.x >> 6] = hc[k];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = pobs[0];
    uint32_t t[3] = {ph[0][0], ph[1][0], ph[2][0]};
#pragma unroll
    for (int i = 1; i < NTH / 64; ++i) {
      m = mag_max(m, pobs[i]);
#pragma unroll
      for (int k = 0; k < 3; ++k) t[k] += ph[k][i];
    }
    if (qo.amax_obs) atomic_max_nonneg(qo.amax_obs, m);
    if (qo.stats)
#pragma unroll
      for (int k = 0; k < 3; ++k)
        if (t[k]) atomicAdd(qo.stats + k, t[k]);
  }
}

}  // namespace fp4k
