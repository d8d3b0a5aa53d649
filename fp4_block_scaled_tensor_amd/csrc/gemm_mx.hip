// MXFP4 GEMM (E2M1 payload, E8M0 scales per 32 along K) on the gfx950 scaled FP4 MFMA.
//
// Sources: "技術概要：MXFP4 による大規模言語モデルの事前学習", method (手法): native MXFP4 on
// MI355X for fprop, dgrad and wgrad. "UE5M3 FP4 Block Scaling for Stable Language Model
// Pretraining", approach (접근 방법): the 64-product group model.
//
// One 64-product group of a 32x32 output tile is exactly one
// v_mfma_scale_f32_32x32x64_f8f6f4 (lanes 0-31 hold K-block 0 of their row, lanes 32-63
// K-block 1, each with its own E8M0 scale byte). With C = 0 the instruction returns the
// exact two-block sum T0 + T1 whenever the combined block exponents of the two blocks,
// (ea0+eb0) - (ea1+eb1), differ by at most 10: the sum then has at most 24 significant
// bits, so it equals the model's nearest-even group partial. When a wave's rows or
// columns could exceed that gap in a group, the group is instead computed per tile as two
// MFMAs with the other K-block's payload zeroed (each an exact 32-block partial) and the
// two are added in float32 round-to-nearest-even. Group partials are accumulated with
// v_add_f32 under round-toward-zero (MODE register), in K order.
//
// Scales: per stage (4 groups) the thread that owns an operand row loads the row's 8 E8M0
// bytes and stages them as two words, one per K-half (byte g = group g, the byte the MFMA
// picks with op_sel g); each staging wave also stores the largest in-group exponent gap
// |e0 - e1| of each 32 of its rows. While the largest gaps of a wave's own A rows and B rows
// sum to at most 10, every group of the stage passes for that wave, which runs a
// branch-free stage whose additions are plain float adds (the K loop runs in
// round-toward-zero mode and contains no other rounding-sensitive operation). A stage that
// fails runs as a simple loop that tests each group, and the next stage goes back to the
// stage test (outlier channels fail only the stages that hold them).
//
// The per-group float32 add bounds this kernel: 16 v_add_f32 per lane per 32x32x64 MFMA,
// which take the vector ALU about twice as long as the matrix core takes for the MFMA, and
// the two pipes do not overlap. The stage loop is therefore kept free of other vector work:
// fragment addresses are a per-lane base plus immediate offsets (the interior kernel runs
// its passing stages in even/odd pairs, so that both LDS buffers are compile-time
// constants), and the direct-to-LDS loads use a scalar base plus a per-lane offset.
#include <type_traits>

#include "gemm_common.hpp"

namespace fp4k {

constexpr int SCB = SGR * 2;    // E8M0 scale bytes per row per stage (8)

__device__ __forceinline__ int iabs(int x) { return x < 0 ? -x : x; }

// Maximum over the wave, returned wave-uniform: xor swizzles within each 32-lane half
// (ds_swizzle bit mode: and 0x1F, xor m), then the two halves' lane 0 values.
__device__ __forceinline__ int wave_max_i(int d) {
  d = max(d, __builtin_amdgcn_ds_swizzle(d, (1 << 10) | 0x1F));
  d = max(d, __builtin_amdgcn_ds_swizzle(d, (2 << 10) | 0x1F));
  d = max(d, __builtin_amdgcn_ds_swizzle(d, (4 << 10) | 0x1F));
  d = max(d, __builtin_amdgcn_ds_swizzle(d, (8 << 10) | 0x1F));
  d = max(d, __builtin_amdgcn_ds_swizzle(d, (16 << 10) | 0x1F));
  return max(__builtin_amdgcn_readlane(d, 0), __builtin_amdgcn_readlane(d, 32));
}

// Scale bytes of one operand row, staged once per stage by one thread. load() fetches the
// stage's 8 E8M0 bytes (group g: bytes 2g and 2g+1, its two K-blocks, in one 2-byte
// load); split() turns them
// into h0 (K-block 0 of groups 0..3, byte g) and h1 (K-block 1) and the largest |e0 - e1|
// over the stage's groups. The two are separate so that nothing waits for the load before
// the stage's compute has been issued (a wait on it would also wait for the payload loads
// issued before it). Rows past the matrix and groups past K read as 127 (2^0).
struct ScaleStager {
  const uint8_t* p;   // the row, clamped to the last row of the matrix
  int64_t nblk;

  __device__ __forceinline__ void init(const uint8_t* s, int64_t row, int64_t rows, int64_t nb) {
    nblk = nb;
    p = s + (row < rows ? row : rows - 1) * nb;
  }
  // Unconditional: four 2-byte loads (the scale pointer is 2-byte aligned and K/32 is even)
  // at positions clamped into the row. Rows past the matrix and groups past K read real
  // scale bytes of another row or group: their values reach only outputs that are not
  // stored or groups that are not computed, and in the gap test they are real gaps (the
  // test stays conservative). Any condition on the load would let the compiler predicate
  // it and wait for it at once, and a wait on it also waits for the payload loads issued
  // before it.
  // (the four loads stay separate values until split(): combining them here would wait)
  __device__ __forceinline__ uint4 load(int64_t st) const {
    uint32_t h[SGR];
#pragma unroll
    for (int g = 0; g < SGR; ++g) {
      const int64_t i = st * SCB + 2 * g;
      h[g] = *reinterpret_cast<const uint16_t*>(p + (i < nblk ? i : nblk - 2));
    }
    return make_uint4(h[0], h[1], h[2], h[3]);
  }
  // interior form (K a multiple of 256, 8-byte aligned scales): the stage's 8 bytes in one
  // load, as two words (groups 0-1, groups 2-3)
  __device__ __forceinline__ uint4 load8(int64_t st) const {
    const uint2 v = *reinterpret_cast<const uint2*>(p + st * SCB);
    return make_uint4(v.x, v.y, 0u, 0u);
  }
  template <bool INTERIOR>
  __device__ __forceinline__ static void split(uint4 q, uint32_t& h0, uint32_t& h1, int& gap) {
    const uint32_t x = INTERIOR ? q.x : (q.x | (q.y << 16)), y = INTERIOR ? q.y : (q.z | (q.w << 16));
    h0 = __builtin_amdgcn_perm(y, x, 0x06040200u);
    h1 = __builtin_amdgcn_perm(y, x, 0x07050301u);
    gap = 0;
#pragma unroll
    for (int g = 0; g < SGR; ++g)
      gap = max(gap, iabs((int)((h0 >> (8 * g)) & 0xFFu) - (int)((h1 >> (8 * g)) & 0xFFu)));
  }
};

template <int G>
__device__ __forceinline__ v16f mfma_g(const v8i& a, const v8i& b, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, v16f{}, 4, 4, G, (int)sa, G, (int)sb);
}

__device__ __forceinline__ v16f mfma_sel(int g, const v8i& a, const v8i& b, uint32_t sa, uint32_t sb) {
  if (g == 0) return mfma_g<0>(a, b, sa, sb);
  if (g == 1) return mfma_g<1>(a, b, sa, sb);
  if (g == 2) return mfma_g<2>(a, b, sa, sb);
  return mfma_g<3>(a, b, sa, sb);
}

// LDS fragment addressing. Lane l reads row r = r0 + (l & 31) (r0 a multiple of 32) at
// logical chunk c = 2g + half of group g. With key = (r >> 1) & 7 = 2 k2 + k1 the stored
// chunk position is c ^ key = 2 (g ^ k2) + (half ^ k1), so the byte offset is
// r * 128 + 32 (g ^ k2) + 16 (half ^ k1) = L ^ (g << 5) with the per-lane base
// L = r * 128 + 32 k2 + 16 (half ^ k1). Tile t of the wave (rows + 32 t, same key) adds 4096 t.
__device__ __forceinline__ uint32_t frag_lane_base(int r0, int l) {
  const int r = r0 + (l & 31), key = (r >> 1) & 7, half = l >> 5;
  return (uint32_t)(r * ROWB + ((key >> 1) << 5) + ((half ^ (key & 1)) << 4));
}
__device__ __forceinline__ v8i frag(const uint8_t* lds, uint32_t L, int t, int g) {
  const uint4 v = *reinterpret_cast<const uint4*>(lds + (L ^ (uint32_t)(g << 5)) + t * 32 * ROWB);
  return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

template <int TM, int TN>
__device__ __forceinline__ void load_frags(const uint8_t* la, const uint8_t* lb, uint32_t La, uint32_t Lb, int g,
                                           v8i (&fa)[TM], v8i (&fb)[TN]) {
#pragma unroll
  for (int t = 0; t < TM; ++t) fa[t] = frag(la, La, t, g);
#pragma unroll
  for (int t = 0; t < TN; ++t) fb[t] = frag(lb, Lb, t, g);
}

__device__ __forceinline__ void add_tile(v16f& acc, const v16f& G) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = acc[r] + G[r];   // round toward zero (K-loop mode)
}

// Largest |e0 - e1| of group g over the wave's rows (TM row tiles from the A rows, TN from
// the B rows at offset bm), as a wave-uniform value. sw points at the stage's [K-half][row]
// scale words (K-half stride nr).
template <int TM, int TN>
__device__ __forceinline__ int group_gap_sum(const uint32_t* sw, int nr, int ra0, int rb0, int bm, int g) {
  int dga = 0, dgb = 0;
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const int r = ra0 + t * 32;
    dga = max(dga, iabs((int)((sw[r] >> (8 * g)) & 0xFFu) - (int)((sw[nr + r] >> (8 * g)) & 0xFFu)));
  }
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int r = bm + rb0 + t * 32;
    dgb = max(dgb, iabs((int)((sw[r] >> (8 * g)) & 0xFFu) - (int)((sw[nr + r] >> (8 * g)) & 0xFFu)));
  }
  return wave_max_i(dga) + wave_max_i(dgb);
}

// A full stage (4 groups) for a tile whose every group passed the gap test: one MFMA per
// group partial. All tile indices are compile-time constants.
template <int TM, int TN>
__device__ __forceinline__ void fast_stage(const uint8_t* la, const uint8_t* lb, uint32_t La, uint32_t Lb,
                                           const uint32_t (&sa)[TM], const uint32_t (&sb)[TN],
                                           v16f (&acc)[TM][TN]) {
#pragma unroll
  for (int g = 0; g < SGR; ++g) {
    v8i fa[TM], fb[TN];
    load_frags<TM, TN>(la, lb, La, Lb, g, fa, fb);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) add_tile(acc[i][j], mfma_sel(g, fa[i], fb[j], sa[i], sb[j]));
  }
}

// Groups [0, g_end) of a stage, one group at a time. With check set, each group is tested
// for the exponent gap and a failing group's partials are two MFMAs with the other
// K-block's payload zeroed, added in float32 nearest-even.
template <int TM, int TN>
__device__ __forceinline__ void plain_stage(const uint8_t* la, const uint8_t* lb, uint32_t La, uint32_t Lb,
                                            const uint32_t (&sa)[TM], const uint32_t (&sb)[TN], bool check,
                                            int g_end, const uint32_t* sw, int nr, int ra0, int rb0, int bm,
                                            int half, v16f (&acc)[TM][TN]) {
#pragma unroll
  for (int g = 0; g < SGR; ++g) {
    if (g >= g_end) break;
    const bool gf = !check || group_gap_sum<TM, TN>(sw, nr, ra0, rb0, bm, g) <= 10;
    if (gf) {
      v8i fa[TM], fb[TN];
      load_frags<TM, TN>(la, lb, La, Lb, g, fa, fb);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) add_tile(acc[i][j], mfma_sel(g, fa[i], fb[j], sa[i], sb[j]));
    } else {
      // one tile at a time, fragments read just in time: this path keeps few registers live
      const v8i z = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v8i fa = frag(la, La, i, g);
          const v8i fb = frag(lb, Lb, j, g);
          const v16f T0 = mfma_sel(g, half == 0 ? fa : z, fb, sa[i], sb[j]);
          const v16f T1 = mfma_sel(g, half == 1 ? fa : z, fb, sa[i], sb[j]);
          add_tile(acc[i][j], add_rne_from_rtz(T0, T1));   // nearest-even group partial, then toward zero
        }
      }
    }
  }
}

#ifndef FP4_MX_MINB
#define FP4_MX_MINB 4
#endif

// LDS of one workgroup: double-buffered payload tiles, scale words and gap maxima.
template <class TL>
struct MxSmem {
  static constexpr int NR = TL::BM + TL::BN;
  uint8_t a[2][TL::BM * ROWB];
  uint8_t b[2][TL::BN * ROWB];
  uint32_t sw[2][2][NR];      // [buf][K-half][A rows, then B rows]
  int gmax[2][NR / 32];       // [buf][32-row half of a staging wave] largest in-group exponent gap of its rows
};

// INTERIOR: every tile lies inside the matrix, K is a multiple of 256 and the scale rows are
// 8-byte aligned, so loads need no clamping.
// QOUT: the epilogue also quantizes C as the next GEMM's ROW-view operand (qo).
template <class TL, bool INTERIOR, bool QOUT>
__global__ __launch_bounds__(TL::NT, FP4_MX_MINB) void k_gemm_mx(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const uint8_t* __restrict__ qb,
    const uint8_t* __restrict__ sb, const float* __restrict__ ga, const float* __restrict__ gb, float* __restrict__ c,
    int64_t M, int64_t N, int64_t K, int canon, int epi, const QuantOut qo) {
  constexpr int TM = TL::TM, TN = TL::TN, BM = TL::BM, BN = TL::BN, NR = BM + BN;
  static_assert(TL::NT >= NR && BM % 64 == 0 && BN % 64 == 0, "one thread per staged scale row, whole waves");
  __shared__ __attribute__((aligned(1024))) MxSmem<TL> sm;
  const int l = threadIdx.x & 63, w = wave_id(), t = threadIdx.x;
  const int wm = w / TL::WN, wn = w % TL::WN;
  int64_t m0, n0;
  tile_coords(M, N, BM, BN, m0, n0);
  const int64_t nblk = K / 32;   // E8M0 scales per row
  // Stage and group counters (SI): 32-bit in the interior kernel, whose stage loop is
  // unrolled by two (their compares then stay on the scalar unit); 64-bit in the others.
  using SI = typename std::conditional<INTERIOR && !QOUT, int, int64_t>::type;
  const SI ngroups = (SI)(K / 64);
  const SI nstages = (SI)((K + KS - 1) / KS);
  const SI nfull = ngroups / SGR;   // stages with 4 groups
  const int half = l >> 5;
  const int ra0 = wm * (TM * 32) + (l & 31), rb0 = wn * (TN * 32) + (l & 31);
  const uint32_t La = frag_lane_base(wm * (TM * 32), l), Lb = frag_lane_base(wn * (TN * 32), l);

  StageLoader<BM, TL::NW> LA;
  StageLoader<BN, TL::NW> LB;
  LA.init(qa, M, K, m0);
  LB.init(qb, N, K, n0);
  // scale rows: whole waves (threads below NR), one row each; A rows first
  const bool stager = w < NR / 64;
  ScaleStager SS;
  if (t < BM) SS.init(sa, m0 + t, M, nblk);
  else SS.init(sb, n0 + t - BM, N, nblk);
  uint4 sraw = make_uint4(0, 0, 0, 0);   // the next stage's scale bytes, in flight during a stage
  auto load_scales = [&](SI st) {
    if (stager) sraw = INTERIOR ? SS.load8(st) : SS.load(st);
  };
  auto issue_stage = [&](SI st, int buf) {
    if (INTERIOR) {
      LA.issue_interior(st, sm.a[buf]);
      LB.issue_interior(st, sm.b[buf]);
    } else {
      LA.issue(st, sm.a[buf]);
      LB.issue(st, sm.b[buf]);
    }
    load_scales(st);
  };
  auto store_scales = [&](int buf) {
    if (stager) {
      uint32_t h0, h1;
      int gap;
      ScaleStager::split<INTERIOR>(sraw, h0, h1, gap);
      sm.sw[buf][0][t] = h0;
      sm.sw[buf][1][t] = h1;
      // maxima of the two 32-lane halves (32 rows each)
      int d = gap;
      d = max(d, __builtin_amdgcn_ds_swizzle(d, (1 << 10) | 0x1F));
      d = max(d, __builtin_amdgcn_ds_swizzle(d, (2 << 10) | 0x1F));
      d = max(d, __builtin_amdgcn_ds_swizzle(d, (4 << 10) | 0x1F));
      d = max(d, __builtin_amdgcn_ds_swizzle(d, (8 << 10) | 0x1F));
      d = max(d, __builtin_amdgcn_ds_swizzle(d, (16 << 10) | 0x1F));
      if ((l & 31) == 0) sm.gmax[buf][2 * w + (l >> 5)] = d;
    }
  };
  // every group of the stage in buffer buf passes the gap test (wave-uniform).
  // The test is per wave: it covers the 32-row staging maxima of this wave's TM*32 A rows and
  // TN*32 B rows, so a wave whose own rows pass runs the fast stage even when
  // another wave of the workgroup does not. Both stage forms issue the same loads, scale
  // stores and barrier, so waves may take different forms in the same stage.
  auto stage_passes = [&](int buf) {
    const int a0 = (wm * TM * 32) >> 5, b0 = (BM + wn * TN * 32) >> 5;   // 32-row maxima
    constexpr int SA = TM, SB = TN;
    int gA = 0, gB = 0;
#pragma unroll
    for (int i = 0; i < SA; ++i) gA = max(gA, sm.gmax[buf][a0 + i]);
#pragma unroll
    for (int i = 0; i < SB; ++i) gB = max(gB, sm.gmax[buf][b0 + i]);
    return __builtin_amdgcn_readfirstlane(gA) + __builtin_amdgcn_readfirstlane(gB) <= 10;
  };

  if (nstages > 0) issue_stage(0, 0);
  else load_scales(0);
  store_scales(0);
  wait_vm();
  __syncthreads();

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  mode_f32_rtz();
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) pin(acc[i][j]);   // additions after the switch

  // A full stage whose every group passes: one MFMA per group partial. Returns false, having
  // done nothing, when the stage fails the test. The stage's buffer (st & 1) is passed either
  // as a compile-time constant (an std::integral_constant), which turns every LDS address of
  // the stage into a per-lane base plus an immediate offset, or as a run-time int.
  auto fast_step = [&](auto bufc, SI st) -> bool {
    const int buf = (int)bufc;
    if (!stage_passes(buf)) return false;
    const bool more = st + 1 < nstages;
    if (more) issue_stage(st + 1, buf ^ 1);
    uint32_t s4a[TM], s4b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) s4a[i] = sm.sw[buf][half][ra0 + i * 32];
#pragma unroll
    for (int j = 0; j < TN; ++j) s4b[j] = sm.sw[buf][half][BM + rb0 + j * 32];
    fast_stage<TM, TN>(sm.a[buf], sm.b[buf], La, Lb, s4a, s4b, acc);
    if (more) {
      store_scales(buf ^ 1);
      wait_vm();
      __syncthreads();
    }
    return true;
  };

  SI st = 0;
  for (;;) {
    // full stages that pass
    if constexpr (INTERIOR && !QOUT) {
      // in pairs (even, odd) after re-aligning on an even stage, both buffers compile-time.
      // The edge and output-quantizing kernels keep one stage per iteration: the longer loop
      // body costs them more in register spills than it saves.
      constexpr std::integral_constant<int, 0> B0{};
      constexpr std::integral_constant<int, 1> B1{};
      if ((st & 1) && st < nfull && fast_step(B1, st)) ++st;
      if (!(st & 1)) {
        while (st < nfull) {
          if (!fast_step(B0, st)) break;
          ++st;
          if (st >= nfull || !fast_step(B1, st)) break;
          ++st;
        }
      }
    } else {
      for (; st < nfull; ++st) {
        if (!fast_step((int)(st & 1), st)) break;
      }
    }
    if (st >= nstages) break;
    // one stage that failed the test (or the partial last stage): each group tested on its
    // own; the stage after it goes back to the test above
    const int buf = (int)(st & 1);
    const bool more = st + 1 < nstages;
    if (more) issue_stage(st + 1, buf ^ 1);
    uint32_t s4a[TM], s4b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) s4a[i] = sm.sw[buf][half][ra0 + i * 32];
#pragma unroll
    for (int j = 0; j < TN; ++j) s4b[j] = sm.sw[buf][half][BM + rb0 + j * 32];
    const int g_end = (int)((ngroups - st * SGR) < SGR ? (ngroups - st * SGR) : (SI)SGR);
    plain_stage<TM, TN>(sm.a[buf], sm.b[buf], La, Lb, s4a, s4b, true, g_end, &sm.sw[buf][0][0], NR, ra0, rb0, BM,
                        half, acc);
    if (more) {
      store_scales(buf ^ 1);
      wait_vm();
      __syncthreads();
    }
    ++st;
  }
  if constexpr (QOUT) {
    static_assert(BM == QO_T && BN == QO_T, "the output quantizer stages 128 x 128 tiles");
    __syncthreads();   // every wave is done with the last stage's buffers
    const QoStage stg{reinterpret_cast<float*>(&sm.a[0][0]), reinterpret_cast<float*>(&sm.b[0][0]), wm * (TM * 32),
                      wn * (TN * 32)};
    store_tiles<TM, TN, true>(c, M, N, m0 + wm * (TM * 32), n0 + wn * (TN * 32), acc, ga, gb, canon, epi, 1.0f, stg);
    quantize_out_tile<TL::NT>(stg, m0, n0, M, N, qo);
  } else {
    store_tiles<TM, TN>(c, M, N, m0 + wm * (TM * 32), n0 + wn * (TN * 32), acc, ga, gb, canon, epi);
  }
}

#ifndef FP4_MX_TILING
#define FP4_MX_TILING 4, 2, 1, 2
#endif
using MxTiling = Tiling<FP4_MX_TILING>;
using MxTilingQ = Tiling<4, 2, 1, 2>;   // the epilogue quantizer stages 128 x 128 tiles

template <class TL, bool QOUT>
static hipError_t launch_mx(const GemmArgs& g) {
  const int64_t tiles = ((g.M + TL::BM - 1) / TL::BM) * ((g.N + TL::BN - 1) / TL::BN);
  const bool interior = g.M % TL::BM == 0 && g.N % TL::BN == 0 && g.K > 0 && g.K % KS == 0 &&
                        reinterpret_cast<uintptr_t>(g.a.s) % 8 == 0 && reinterpret_cast<uintptr_t>(g.b.s) % 8 == 0;
  auto kern = interior ? k_gemm_mx<TL, true, QOUT> : k_gemm_mx<TL, false, QOUT>;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(TL::NT), 0, g.stream, g.a.q, g.a.s, g.b.q, g.b.s, g.a.g,
                     g.b.g, g.c, g.M, g.N, g.K, g.canon, epilogue_word(g.hadamard_n, g.a.g_shift, g.b.g_shift),
                     g.qout ? *g.qout : QuantOut{});
  return hipGetLastError();
}

hipError_t run_gemm_mx(const GemmArgs& g) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  return g.qout ? launch_mx<MxTilingQ, true>(g) : launch_mx<MxTiling, false>(g);
}

}  // namespace fp4k
