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
// The gap test runs once per stage (4 groups): the thread that stages a row's 8 scale
// bytes also stores the row's largest in-group exponent gap, and each wave checks its 64
// rows and 64 columns. A stage that passes runs a branch-free body of 4 groups whose
// additions are plain float adds (the K loop runs in round-toward-zero mode and contains
// no other rounding-sensitive operation).
#include "gemm_common.hpp"

namespace fp4k {

constexpr int SCB = SGR * 2;    // E8M0 scale bytes per row per stage (8)

__device__ __forceinline__ int iabs(int x) { return x < 0 ? -x : x; }

__device__ __forceinline__ int wave_max_i(int d) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) d = max(d, __shfl_xor(d, o, 64));
  return d;
}

// Scale bytes of one operand row, staged once per stage by one thread:
// .x/.y = the stage's 8 E8M0 bytes (group g: bytes 2g, 2g+1), .z = largest |e0 - e1| over
// the stage's groups. Rows past the matrix and groups past K read as 127 (2^0).
struct ScaleStager {
  const uint8_t* p;
  int64_t nblk;
  bool fast_load;

  __device__ __forceinline__ void init(const uint8_t* s, int64_t row, int64_t rows, int64_t nb) {
    nblk = nb;
    p = row < rows ? s + row * nb : nullptr;
    fast_load = (nb & 7) == 0 && (reinterpret_cast<uintptr_t>(s) & 7) == 0;
  }
  __device__ __forceinline__ uint4 load(int64_t st) const {
    uint32_t w0 = 0x7F7F7F7Fu, w1 = 0x7F7F7F7Fu;
    if (p) {
      if (fast_load && (st + 1) * SCB <= nblk) {
        const uint2 v = *reinterpret_cast<const uint2*>(p + st * SCB);
        w0 = v.x;
        w1 = v.y;
      } else {
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < SCB; ++i) {
          const uint32_t b = (st * SCB + i < nblk) ? p[st * SCB + i] : 0x7Fu;
          w[i >> 2] |= b << (8 * (i & 3));
        }
        w0 = w[0];
        w1 = w[1];
      }
    }
    int gap = 0;
#pragma unroll
    for (int g = 0; g < SGR; ++g) {
      const uint32_t h = (g < 2 ? w0 : w1) >> (16 * (g & 1));
      gap = max(gap, iabs((int)(h & 0xFFu) - (int)((h >> 8) & 0xFFu)));
    }
    return make_uint4(w0, w1, (uint32_t)gap, 0u);
  }
};

// The four scale bytes (groups 0..3) of this lane's K-half: bytes 0,2,4,6 of the staged
// pair (x, y) for lanes 0-31, bytes 1,3,5,7 for lanes 32-63; the MFMA picks group g's byte
// with op_sel g.
__device__ __forceinline__ uint32_t half_bytes(uint4 v, int half) {
  return __builtin_amdgcn_perm(v.y, v.x, half ? 0x07050301u : 0x06040200u);
}

template <int G>
__device__ __forceinline__ v16f mfma_g(const v8i& a, const v8i& b, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, v16f{}, 4, 4, G, (int)sa, G, (int)sb);
}

__device__ __forceinline__ void load_frags(const uint8_t* la, const uint8_t* lb, int ra0, int rb0, int half, int g,
                                           v8i (&fa)[2], v8i (&fb)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint4 va = *reinterpret_cast<const uint4*>(la + swz(ra0 + t * 32, g * 2 + half));
    const uint4 vb = *reinterpret_cast<const uint4*>(lb + swz(rb0 + t * 32, g * 2 + half));
    fa[t] = v8i{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
    fb[t] = v8i{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
  }
}

__device__ __forceinline__ void add_tile(v16f& acc, const v16f& G) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = acc[r] + G[r];   // round toward zero (K-loop mode)
}

// A full stage of 4 groups x 4 tiles, software-pipelined: the MFMA of unit u+1 is issued
// before the 16 additions of unit u (two partial buffers), and the fragments of group g+1
// are read from LDS while group g is computed.
__device__ __forceinline__ void fast_stage(const uint8_t* la, const uint8_t* lb, int ra0, int rb0, int half,
                                           const uint32_t (&sa)[2], const uint32_t (&sb)[2], v16f (&acc)[2][2]) {
  v8i fa[2][2], fb[2][2];
  load_frags(la, lb, ra0, rb0, half, 0, fa[0], fb[0]);
  v16f Gb[2];
  int pi = -1, pj = -1;
#pragma unroll
  for (int g = 0; g < SGR; ++g) {
    if (g + 1 < SGR) load_frags(la, lb, ra0, rb0, half, g + 1, fa[(g + 1) & 1], fb[(g + 1) & 1]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = t >> 1, j = t & 1;
      const int u = g * 4 + t;
      v16f& cur = Gb[u & 1];
      if (g == 0) cur = mfma_g<0>(fa[0][i], fb[0][j], sa[i], sb[j]);
      else if (g == 1) cur = mfma_g<1>(fa[1][i], fb[1][j], sa[i], sb[j]);
      else if (g == 2) cur = mfma_g<2>(fa[0][i], fb[0][j], sa[i], sb[j]);
      else cur = mfma_g<3>(fa[1][i], fb[1][j], sa[i], sb[j]);
      if (u > 0) add_tile(acc[pi][pj], Gb[(u - 1) & 1]);
      pi = i;
      pj = j;
    }
  }
  add_tile(acc[pi][pj], Gb[1]);
}

__global__ __launch_bounds__(GNT, 2) void k_gemm_mx(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                    const uint8_t* __restrict__ qb, const uint8_t* __restrict__ sb,
                                                    const float* __restrict__ ga, const float* __restrict__ gb,
                                                    float* __restrict__ c, int64_t M, int64_t N, int64_t K, int canon,
                                                    int hadamard_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lA[2][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lB[2][TILE_BYTES];
  __shared__ uint4 lS[2][2 * GT];   // [buf][A rows 0..127, B rows 0..127]
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  int64_t m0, n0;
  tile_coords(M, N, m0, n0);
  const int64_t nblk = K / 32;   // E8M0 scales per row
  const int64_t ngroups = K / 64;
  const int64_t nstages = (K + KS - 1) / KS;
  const int half = l >> 5;
  const int ra0 = wm * 64 + (l & 31), rb0 = wn * 64 + (l & 31);

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  StageLoader LA, LB;
  LA.init(qa, M, K, m0);
  LB.init(qb, N, K, n0);
  ScaleStager SS;
  if (threadIdx.x < GT) SS.init(sa, m0 + threadIdx.x, M, nblk);
  else SS.init(sb, n0 + threadIdx.x - GT, N, nblk);
  uint4 sreg = SS.load(0);
  if (nstages > 0) {
    LA.issue(0, lA[0]);
    LB.issue(0, lB[0]);
  }
  lS[0][threadIdx.x] = sreg;
  wait_vm();
  __syncthreads();

  mode_f32_rtz();
  for (int64_t st = 0; st < nstages; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) {
      LA.issue(st + 1, lA[buf ^ 1]);
      LB.issue(st + 1, lB[buf ^ 1]);
      sreg = SS.load(st + 1);
    }
    const uint4 sA0 = lS[buf][ra0], sA1 = lS[buf][ra0 + 32];
    const uint4 sB0 = lS[buf][GT + rb0], sB1 = lS[buf][GT + rb0 + 32];
    const uint32_t sa4[2] = {half_bytes(sA0, half), half_bytes(sA1, half)};
    const uint32_t sb4[2] = {half_bytes(sB0, half), half_bytes(sB1, half)};
    const int da = (int)max(sA0.z, sA1.z), db = (int)max(sB0.z, sB1.z);
    // sufficient for every output of the wave and every group of the stage: max|da| + max|db| <= 10
    bool fast = !__any(da > 5 || db > 5);
    if (!fast) fast = wave_max_i(da) + wave_max_i(db) <= 10;
    const int g_end = (int)((ngroups - st * SGR) < SGR ? (ngroups - st * SGR) : SGR);
    if (fast && g_end == SGR) {
      fast_stage(lA[buf], lB[buf], ra0, rb0, half, sa4, sb4, acc);
    } else {
      for (int g = 0; g < g_end; ++g) {
        v8i fa[2], fb[2];
        int ea[2], eb[2];
        int dga = 0, dgb = 0;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint4 va = *reinterpret_cast<const uint4*>(lA[buf] + swz(ra0 + t * 32, g * 2 + half));
          const uint4 vb = *reinterpret_cast<const uint4*>(lB[buf] + swz(rb0 + t * 32, g * 2 + half));
          fa[t] = v8i{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
          fb[t] = v8i{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
          const uint4 pa = t ? sA1 : sA0, pb = t ? sB1 : sB0;
          const uint32_t wa = (g < 2 ? pa.x : pa.y) >> (16 * (g & 1));
          const uint32_t wb = (g < 2 ? pb.x : pb.y) >> (16 * (g & 1));
          const int a0 = (int)(wa & 0xFFu), a1 = (int)((wa >> 8) & 0xFFu);
          const int b0 = (int)(wb & 0xFFu), b1 = (int)((wb >> 8) & 0xFFu);
          ea[t] = half ? a1 : a0;
          eb[t] = half ? b1 : b0;
          dga = max(dga, iabs(a0 - a1));
          dgb = max(dgb, iabs(b0 - b1));
        }
        const bool gfast = wave_max_i(dga) + wave_max_i(dgb) <= 10;
        if (gfast) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const v16f Gt = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], v16f{}, 4, 4, 0, ea[i], 0,
                                                                              eb[j]);
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[i][j][r] = acc[i][j][r] + Gt[r];
            }
        } else {
          const v8i z = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const v8i fa0 = half == 0 ? fa[i] : z;
            const v8i fa1 = half == 1 ? fa[i] : z;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const v16f T0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa0, fb[j], v16f{}, 4, 4, 0, ea[i], 0,
                                                                              eb[j]);
              const v16f T1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa1, fb[j], v16f{}, 4, 4, 0, ea[i], 0,
                                                                              eb[j]);
              float Gs[16];
              mode_f32_rne();
#pragma unroll
              for (int r = 0; r < 16; ++r) Gs[r] = T0[r] + T1[r];            // nearest-even group partial
              mode_f32_rtz();
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[i][j][r] = acc[i][j][r] + Gs[r];
            }
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
