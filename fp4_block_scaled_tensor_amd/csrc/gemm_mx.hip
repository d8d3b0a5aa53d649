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
// The fast path's adds are plain float additions: the whole K loop runs in
// round-toward-zero mode and contains no other rounding-sensitive operation. The rare
// slow path switches to nearest-even around its own inline-asm additions.
#include "gemm_common.hpp"

namespace fp4k {

constexpr int SCB = SGR * 2;    // E8M0 scale bytes per row per stage (8)

__device__ __forceinline__ int iabs(int x) { return x < 0 ? -x : x; }

__device__ __forceinline__ int wave_max_i(int d) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) d = max(d, __shfl_xor(d, o, 64));
  return d;
}

// Load the 8 scale bytes (4 groups x 2 blocks) of one row for stage st into two dwords.
// Rows past the matrix get 127 (2^0); groups past K get 127 too.
__device__ __forceinline__ uint2 scale_row(const uint8_t* __restrict__ s, int64_t row, int64_t rows, int64_t nblk,
                                           int64_t st) {
  if (row >= rows) return make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
  const uint8_t* p = s + row * nblk + st * SCB;
  if ((nblk & 7) == 0 && (reinterpret_cast<uintptr_t>(s) & 7) == 0 && (st + 1) * SCB <= nblk)
    return *reinterpret_cast<const uint2*>(p);
  uint32_t w[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < SCB; ++i) {
    const uint32_t b = (st * SCB + i < nblk) ? p[i] : 0x7Fu;
    w[i >> 2] |= b << (8 * (i & 3));
  }
  return make_uint2(w[0], w[1]);
}

__global__ __launch_bounds__(GNT, 2) void k_gemm_mx(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                    const uint8_t* __restrict__ qb, const uint8_t* __restrict__ sb,
                                                    const float* __restrict__ ga, const float* __restrict__ gb,
                                                    float* __restrict__ c, int64_t M, int64_t N, int64_t K, int canon,
                                                    int hadamard_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lA[2][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lB[2][TILE_BYTES];
  __shared__ uint2 lS[2][2 * GT];   // [buf][A rows 0..127, B rows 0..127]: 8 scale bytes per row
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  int64_t m0, n0;
  tile_coords(M, N, m0, n0);
  const int64_t nblk = K / 32;   // E8M0 scales per row
  const int64_t ngroups = K / 64;
  const int64_t nstages = (K + KS - 1) / KS;
  const int half = l >> 5;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // scale row handled by this thread: threads 0..127 -> A rows, 128..255 -> B rows
  const bool srow_is_a = threadIdx.x < GT;
  const int srow = threadIdx.x & (GT - 1);
  uint2 sreg = srow_is_a ? scale_row(sa, m0 + srow, M, nblk, 0) : scale_row(sb, n0 + srow, N, nblk, 0);
  if (nstages > 0) {
    stage_issue(qa, M, K, m0, 0, lA[0]);
    stage_issue(qb, N, K, n0, 0, lB[0]);
  }
  lS[0][threadIdx.x] = sreg;
  wait_vm();
  __syncthreads();

  mode_f32_rtz();
  for (int64_t st = 0; st < nstages; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) {
      stage_issue(qa, M, K, m0, (st + 1) * KS, lA[buf ^ 1]);
      stage_issue(qb, N, K, n0, (st + 1) * KS, lB[buf ^ 1]);
      sreg = srow_is_a ? scale_row(sa, m0 + srow, M, nblk, st + 1) : scale_row(sb, n0 + srow, N, nblk, st + 1);
    }
    // this lane's rows / columns and their 8 stage scale bytes
    uint2 scA[2], scB[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      scA[t] = lS[buf][wm * 64 + t * 32 + (l & 31)];
      scB[t] = lS[buf][GT + wn * 64 + t * 32 + (l & 31)];
    }
    const int g_end = (int)((ngroups - st * SGR) < SGR ? (ngroups - st * SGR) : SGR);
    for (int g = 0; g < g_end; ++g) {
      v8i fa[2], fb[2];
      int ea[2], eb[2];
      int da = 0, db = 0;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint4 va = *reinterpret_cast<const uint4*>(lA[buf] + swz(wm * 64 + t * 32 + (l & 31), g * 2 + half));
        const uint4 vb = *reinterpret_cast<const uint4*>(lB[buf] + swz(wn * 64 + t * 32 + (l & 31), g * 2 + half));
        fa[t] = v8i{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
        fb[t] = v8i{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
        const uint32_t wa = (g < 2 ? scA[t].x : scA[t].y) >> (16 * (g & 1));
        const uint32_t wb = (g < 2 ? scB[t].x : scB[t].y) >> (16 * (g & 1));
        const int a0 = (int)(wa & 0xFFu), a1 = (int)((wa >> 8) & 0xFFu);
        const int b0 = (int)(wb & 0xFFu), b1 = (int)((wb >> 8) & 0xFFu);
        ea[t] = half ? a1 : a0;
        eb[t] = half ? b1 : b0;
        da = max(da, iabs(a0 - a1));
        db = max(db, iabs(b0 - b1));
      }
      // Sufficient for every output of the wave: max|da| + max|db| <= 10. Cheap test first.
      bool fast = !__any(da > 5 || db > 5);
      if (!fast) fast = wave_max_i(da) + wave_max_i(db) <= 10;
      if (fast) {
        v16f G[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            G[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], v16f{}, 4, 4, 0, ea[i], 0, eb[j]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = acc[i][j][r] + G[i][j][r];   // round toward zero
      } else {
        const v8i z = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const v8i fa0 = half == 0 ? fa[i] : z;
          const v8i fa1 = half == 1 ? fa[i] : z;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const v16f T0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa0, fb[j], v16f{}, 4, 4, 0, ea[i], 0, eb[j]);
            const v16f T1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa1, fb[j], v16f{}, 4, 4, 0, ea[i], 0, eb[j]);
            float Gs[16];
            mode_f32_rne();
#pragma unroll
            for (int r = 0; r < 16; ++r) Gs[r] = T0[r] + T1[r];
            mode_f32_rtz();
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = acc[i][j][r] + Gs[r];
          }
        }
      }
    }
    if (st + 1 < nstages) {
      lS[buf ^ 1][threadIdx.x] = sreg;
      wait_vm();
      __syncthreads();
    }
  }
  store_tiles(c, M, N, m0 + wm * 64, n0 + wn * 64, acc, ga, gb, canon, hadamard_n);
}

hipError_t run_gemm_mx(const GemmArgs& g) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const int64_t tiles = ((g.M + GT - 1) / GT) * ((g.N + GT - 1) / GT);
  hipLaunchKernelGGL(k_gemm_mx, dim3((unsigned)tiles), dim3(GNT), 0, g.stream, g.a.q, g.a.s, g.b.q, g.b.s, g.a.g,
                     g.b.g, g.c, g.M, g.N, g.K, g.canon, g.hadamard_n);
  return hipGetLastError();
}

}  // namespace fp4k
