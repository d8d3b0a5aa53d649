// Block-scaled FP4 GEMM with UE5M3 or E4M3 block scales (block 16 or 32) on gfx950.
//
// Sources: "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach (접근 방법):
// UE5M3 block-16 recipe, NVFP4-style E4M3 baseline, and the 64-product group model; limits
// section (한계): UE5M3 has no native hardware support, so it runs through an exact route.
//
// The gfx950 scaled MFMA carries only power-of-two scales per 32 elements, so it cannot
// apply a UE5M3/E4M3 scale per 16 elements. Every decoded operand value q*S (E2M1 times a
// 4-significant-bit scale) has at most 6 significant bits and lies within bf16 range, so
// it is exact in bf16; one v_mfma_f32_32x32x16_bf16 with C = 0 then returns the exact
// partial sum of a 16-wide K slice (all 16 products share one scale pair, so the sum has
// at most 21 significant bits). The slices are combined on the VALU:
//   block 16: G = ((T0 + T1) + T2) + T3, each add float32 nearest-even;
//   block 32: G = (T0 + T1) + (T2 + T3); the inner adds are exact (same scale pair), the
//             outer one nearest-even.
// Then acc = acc + G with round-toward-zero. Chaining the MFMA accumulator instead is not
// used: its C + sum rounding does not match nearest-even.
#include "gemm_common.hpp"

namespace fp4k {

// 8 E2M1 codes (one dword, element 0 in the low nibble) times scale value S -> 8 bf16.
__device__ __forceinline__ v8bf decode8(uint32_t codes, float S) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float2 q;
    typedef float v2f __attribute__((ext_vector_type(2)));
    v2f qq;
    if (j == 0) qq = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    else if (j == 1) qq = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    else if (j == 2) qq = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    else qq = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    q.x = qq.x * S;   // exact
    q.y = qq.y * S;
    o[j] = __builtin_amdgcn_perm(__float_as_uint(q.y), __float_as_uint(q.x), 0x07060302u);
  }
  return __builtin_bit_cast(v8bf, v4u{o[0], o[1], o[2], o[3]});
}

template <int FMT, int B>
__global__ __launch_bounds__(GNT) void k_gemm_dec16(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                    int la, const uint8_t* __restrict__ qb,
                                                    const uint8_t* __restrict__ sb, int lb,
                                                    const float* __restrict__ ga, const float* __restrict__ gb,
                                                    float* __restrict__ c, int64_t M, int64_t N, int64_t K, int canon,
                                                    int hadamard_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[2][GT * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t lB[2][GT * ROWB];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int64_t m0 = (int64_t)blockIdx.y * GT, n0 = (int64_t)blockIdx.x * GT;
  const int64_t bpr = K / B;        // blocks per row (1D layouts)
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

  uint4 pa[4], pb[4];
  stage_load(qa, M, K, m0, 0, pa);
  stage_load(qb, N, K, n0, 0, pb);
  stage_store(lA[0], pa);
  stage_store(lB[0], pb);
  __syncthreads();

  const int64_t arow[2] = {m0 + wm * 64 + (l & 31), m0 + wm * 64 + 32 + (l & 31)};
  const int64_t bcol[2] = {n0 + wn * 64 + (l & 31), n0 + wn * 64 + 32 + (l & 31)};
  // 2D layouts index scales by 16-element K-block and 16-row group
  const int64_t bpr_a = la == 0 ? bpr : K / 16;
  const int64_t bpr_b = lb == 0 ? bpr : K / 16;

  for (int64_t st = 0; st < nstages; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) {
      stage_load(qa, M, K, m0, (st + 1) * KS, pa);
      stage_load(qb, N, K, n0, (st + 1) * KS, pb);
    }
    const int64_t g_end = (ngroups - st * 4) < 4 ? (ngroups - st * 4) : 4;
    for (int g = 0; g < g_end; ++g) {
      const int64_t gg = st * 4 + g;
      // G: group partial per tile; H: second 32-block partial (block 32 only)
      v16f G[2][2], H[2][2];
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const int64_t kelem = gg * 64 + sub * 16;       // first K index of this 16-wide slice
        const int64_t blk = kelem / B;
        const int64_t blk16 = kelem / 16;
        v8bf fa[2], fb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int rowa = wm * 64 + t * 32 + (l & 31);
          const int rowb = wn * 64 + t * 32 + (l & 31);
          const int off = g * 32 + sub * 8 + half * 4;  // payload byte inside the stage row
          const uint32_t ca = *reinterpret_cast<const uint32_t*>(lA[buf] + swz(rowa, off >> 4) + (off & 15));
          const uint32_t cb = *reinterpret_cast<const uint32_t*>(lB[buf] + swz(rowb, off >> 4) + (off & 15));
          const uint32_t sca = arow[t] < M ? scale_at(sa, la, arow[t], la == 0 ? blk : blk16, M, bpr_a)
                                           : ScaleFmt<FMT>::ONE;
          const uint32_t scb = bcol[t] < N ? scale_at(sb, lb, bcol[t], lb == 0 ? blk : blk16, N, bpr_b)
                                           : ScaleFmt<FMT>::ONE;
          fa[t] = decode8(ca, dec_scale3<FMT>(sca));
          fb[t] = decode8(cb, dec_scale3<FMT>(scb));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const v16f T = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], v16f{}, 0, 0, 0);
            if constexpr (B == 16) {
              // ((T0 + T1) + T2) + T3, nearest-even
              if (sub == 0) G[i][j] = T;
              else
#pragma unroll
                for (int r = 0; r < 16; ++r) G[i][j][r] = add_in_mode(G[i][j][r], T[r]);
            } else {
              // (T0 + T1) + (T2 + T3): inner adds exact, outer nearest-even
              if (sub == 0) G[i][j] = T;
              else if (sub == 1)
#pragma unroll
                for (int r = 0; r < 16; ++r) G[i][j][r] = add_in_mode(G[i][j][r], T[r]);
              else if (sub == 2) H[i][j] = T;
              else
#pragma unroll
                for (int r = 0; r < 16; ++r) G[i][j][r] = add_in_mode(G[i][j][r], add_in_mode(H[i][j][r], T[r]));
            }
          }
      }
      mode_f32_rtz();
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = add_in_mode(acc[i][j][r], G[i][j][r]);
      mode_f32_rne();
    }
    if (st + 1 < nstages) {
      stage_store(lA[buf ^ 1], pa);
      stage_store(lB[buf ^ 1], pb);
      __syncthreads();
    }
  }
  store_tiles(c, M, N, m0 + wm * 64, n0 + wn * 64, acc, ga, gb, canon, hadamard_n);
}

template <int FMT, int B>
static hipError_t launch_dec16(const GemmArgs& g) {
  dim3 grid((unsigned)((g.N + GT - 1) / GT), (unsigned)((g.M + GT - 1) / GT));
  hipLaunchKernelGGL((k_gemm_dec16<FMT, B>), grid, dim3(GNT), 0, g.stream, g.a.q, g.a.s, g.a.layout, g.b.q, g.b.s,
                     g.b.layout, g.a.g, g.b.g, g.c, g.M, g.N, g.K, g.canon, g.hadamard_n);
  return hipGetLastError();
}

hipError_t run_gemm_dec16(const GemmArgs& g) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (g.fmt == FMT_UE5M3) return g.block == 16 ? launch_dec16<FMT_UE5M3, 16>(g) : launch_dec16<FMT_UE5M3, 32>(g);
  return g.block == 16 ? launch_dec16<FMT_E4M3, 16>(g) : launch_dec16<FMT_E4M3, 32>(g);
}

}  // namespace fp4k
