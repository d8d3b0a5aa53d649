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
// columns could exceed that gap in a group, the group is instead computed as two MFMAs
// with the other K-block's payload zeroed (each an exact 32-block partial) and the two
// are added in float32 round-to-nearest-even. Group partials are then accumulated with
// v_add_f32 under round-toward-zero (MODE register), in K order.
#include "gemm_common.hpp"

namespace fp4k {

__device__ __forceinline__ int iabs(int x) { return x < 0 ? -x : x; }

__device__ __forceinline__ int wave_max_i(int d) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) d = max(d, __shfl_xor(d, o, 64));
  return d;
}

// Both E8M0 exponents (K-blocks 2g and 2g+1) of a row: low byte = block 2g.
__device__ __forceinline__ uint32_t scale_pair(const uint8_t* __restrict__ s, int64_t row, int64_t rows,
                                               int64_t nblk, int64_t g) {
  if (row >= rows) return 0x7F7Fu;
  return *reinterpret_cast<const uint16_t*>(s + row * nblk + 2 * g);
}

__global__ __launch_bounds__(GNT) void k_gemm_mx(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                 const uint8_t* __restrict__ qb, const uint8_t* __restrict__ sb,
                                                 const float* __restrict__ ga, const float* __restrict__ gb,
                                                 float* __restrict__ c, int64_t M, int64_t N, int64_t K, int canon,
                                                 int hadamard_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[2][GT * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t lB[2][GT * ROWB];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int64_t m0 = (int64_t)blockIdx.y * GT, n0 = (int64_t)blockIdx.x * GT;
  const int64_t nblk = K / 32;   // E8M0 scales per row
  const int64_t ngroups = K / 64;
  const int64_t nstages = (K + KS - 1) / KS;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  uint4 pa[4], pb[4];
  stage_load(qa, M, K, m0, 0, pa);
  stage_load(qb, N, K, n0, 0, pb);
  stage_store(lA[0], pa);
  stage_store(lB[0], pb);
  __syncthreads();

  // rows / cols of this lane in the wave's 2x2 tiles
  const int64_t arow[2] = {m0 + wm * 64 + (l & 31), m0 + wm * 64 + 32 + (l & 31)};
  const int64_t bcol[2] = {n0 + wn * 64 + (l & 31), n0 + wn * 64 + 32 + (l & 31)};
  const int half = l >> 5;

  mode_f32_rtz();
  for (int64_t st = 0; st < nstages; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) {
      stage_load(qa, M, K, m0, (st + 1) * KS, pa);
      stage_load(qb, N, K, n0, (st + 1) * KS, pb);
    }
    const int64_t g_end = (ngroups - st * 4) < 4 ? (ngroups - st * 4) : 4;
    for (int g = 0; g < g_end; ++g) {
      const int64_t gg = st * 4 + g;
      v8i fa[2], fb[2];
      uint32_t ea[2], eb[2];
      int da = 0, db = 0;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int rowa = wm * 64 + t * 32 + (l & 31);
        const int rowb = wn * 64 + t * 32 + (l & 31);
        const uint4 va = *reinterpret_cast<const uint4*>(lA[buf] + swz(rowa, g * 2 + half));
        const uint4 vb = *reinterpret_cast<const uint4*>(lB[buf] + swz(rowb, g * 2 + half));
        fa[t] = v8i{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
        fb[t] = v8i{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
        const uint32_t pa2 = scale_pair(sa, arow[t], M, nblk, gg);
        const uint32_t pb2 = scale_pair(sb, bcol[t], N, nblk, gg);
        ea[t] = half ? (pa2 >> 8) : (pa2 & 0xFFu);
        eb[t] = half ? (pb2 >> 8) : (pb2 & 0xFFu);
        da = max(da, iabs((int)(pa2 & 0xFFu) - (int)(pa2 >> 8)));
        db = max(db, iabs((int)(pb2 & 0xFFu) - (int)(pb2 >> 8)));
      }
      // Sufficient for every output of the wave: max|da| + max|db| <= 10. Cheap test first.
      bool fast = !__any(da > 5 || db > 5);
      if (!fast) fast = wave_max_i(da) + wave_max_i(db) <= 10;
      v16f G[2][2];
      if (fast) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            G[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], v16f{}, 4, 4, 0, (int)ea[i], 0,
                                                                       (int)eb[j]);
      } else {
        v8i fa0[2], fa1[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const v8i z = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          fa0[i] = half == 0 ? fa[i] : z;
          fa1[i] = half == 1 ? fa[i] : z;
        }
        v16f T0[2][2], T1[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            T0[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa0[i], fb[j], v16f{}, 4, 4, 0, (int)ea[i], 0,
                                                                        (int)eb[j]);
            T1[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa1[i], fb[j], v16f{}, 4, 4, 0, (int)ea[i], 0,
                                                                        (int)eb[j]);
          }
        mode_f32_rne();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) G[i][j][r] = add_in_mode(T0[i][j][r], T1[i][j][r]);
        mode_f32_rtz();
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = add_in_mode(acc[i][j][r], G[i][j][r]);
    }
    if (st + 1 < nstages) {
      stage_store(lA[buf ^ 1], pa);
      stage_store(lB[buf ^ 1], pb);
      __syncthreads();
    }
  }
  store_tiles(c, M, N, m0 + wm * 64, n0 + wn * 64, acc, ga, gb, canon, hadamard_n);
}

hipError_t run_gemm_mx(const GemmArgs& g) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  dim3 grid((unsigned)((g.N + GT - 1) / GT), (unsigned)((g.M + GT - 1) / GT));
  hipLaunchKernelGGL(k_gemm_mx, grid, dim3(GNT), 0, g.stream, g.a.q, g.a.s, g.b.q, g.b.s, g.a.g, g.b.g, g.c, g.M, g.N,
                     g.K, g.canon, g.hadamard_n);
  return hipGetLastError();
}

}  // namespace fp4k
