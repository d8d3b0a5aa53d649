// Block-scaled FP4 GEMM with UE5M3 or E4M3 block scales (block 16 or 32) on gfx950.
//
// Sources: "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach (접근 방법):
// UE5M3 block-16 recipe, NVFP4-style E4M3 baseline, and the 64-product group model; limits
// section (한계): UE5M3 has no native hardware support, so it runs through an exact route.
//
// The gfx950 scaled MFMA carries only power-of-two scales per 32 elements, so it cannot
// apply a UE5M3/E4M3 scale per 16 elements. The operands are decoded exactly to fp16
// instead, shifted by 2^-3: with S = M 2^E (M in [1, 2), at most 4 significant bits),
// v_cvt_scalef32_pk_f16_fp4 gives q 2^(E-3) and one v_pk_mul_f16 multiplies by M. Every
// value q S 2^-3 has at most 6 significant bits and lies in [2^-21, 46080], inside fp16
// (subnormals included), so both steps are exact. One v_mfma_f32_32x32x16_f16 with C = 0
// then returns 2^-6 times the exact partial sum of a 16-wide K slice (all 16 products share
// one scale pair, so the sum has at most 21 significant bits). All sums below carry the same
// 2^-6 factor; a power-of-two factor commutes with every rounding of the model (no value
// comes near the float32 subnormal or overflow range), and the epilogue removes it. The
// slices are combined on the VALU:
//   block 16: G = ((T0 + T1) + T2) + T3, each add float32 nearest-even;
//   block 32: G = (T0 + T1) + (T2 + T3); the inner adds are exact (same scale pair), the
//             outer one nearest-even.
// Then acc = acc + G with round-toward-zero. Chaining the MFMA accumulator instead is not
// used: its C + sum rounding does not match nearest-even.
#include "gemm_common.hpp"

namespace fp4k {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// The decode factors of a scale code, straight from its bit fields: a normal code (exponent
// field e >= 1, mantissa m) has S = (1 + m/8) 2^(e - bias), giving 2^(e - bias - 3) as float
// (for the convert) and 1 + m/8 as a packed fp16 pair (for the multiply); a subnormal code
// has S = m q_s (q_s the subnormal quantum, 2^-17 for UE5M3, 2^-9 for E4M3), giving
// q_s 2^-3 and m itself (0..7, exact in fp16; code 0 decodes every value to zero).
struct DecScale {
  float p2;
  v2h m2;
};
template <int FMT>
__device__ __forceinline__ DecScale dec_factors_code(uint32_t c) {
  constexpr int SUB_EXP = FMT == FMT_UE5M3 ? 17 : 9;   // log2 of 1 / subnormal quantum
  const uint32_t e = c >> 3, m = c & 7u;
  DecScale d;
  uint32_t h;
  if (e != 0) {
    d.p2 = __uint_as_float((e + (uint32_t)(127 - ScaleFmt<FMT>::BIAS - 3)) << 23);
    h = 0x3C00u | (m << 7);                                  // fp16 1 + m/8
  } else {
    d.p2 = __uint_as_float((uint32_t)(127 - SUB_EXP - 3) << 23);
    const _Float16 mh = (_Float16)(float)m;                  // exact
    h = (uint32_t)__builtin_bit_cast(uint16_t, mh);
  }
  const uint32_t hh = h | (h << 16);
  d.m2 = __builtin_bit_cast(v2h, hh);
  return d;
}

// 8 E2M1 codes (one dword, element 0 in the low nibble) times S 2^-3 -> 8 fp16, exactly.
__device__ __forceinline__ v8h decode8(uint32_t codes, const DecScale& d) {
  v2h h[4];
  h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, d.p2, 0);
  h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, d.p2, 1);
  h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, d.p2, 2);
  h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, d.p2, 3);
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = h[j] * d.m2;   // v_pk_mul_f16, exact
  return v8h{h[0].x, h[0].y, h[1].x, h[1].y, h[2].x, h[2].y, h[3].x, h[3].y};
}

// The 16 scale codes (one per 16-wide K slice; block 32 repeats each code twice) of one
// operand row for stage st, in the operand's scale layout. Rows past the matrix and slices
// past K get the code of 1.0. With al (scale array 16-byte aligned, K % 256 == 0) a whole
// stage of a 1D or forward-2D row is one 16-byte load (block 32: one 8-byte load, each code
// doubled with v_perm); the transposed 2D layout, whose codes are strided, and a partial last
// stage read byte by byte.
template <int FMT, int B>
__device__ __forceinline__ uint4 scale_row16(const uint8_t* __restrict__ s, int layout, int64_t row, int64_t rows,
                                             int64_t K, int64_t st, bool al) {
  const uint32_t one = ScaleFmt<FMT>::ONE;
  if (row >= rows) {
    const uint32_t w = one * 0x01010101u;
    return make_uint4(w, w, w, w);
  }
  const int64_t k16 = K / 16;        // 16-wide slices per row
  if (al && layout != 2 && (st + 1) * 16 <= k16) {
    if (layout == 1 || B == 16) {
      const int64_t base = layout == 1 ? (row >> 4) * k16 : row * k16;
      return *reinterpret_cast<const uint4*>(s + base + st * 16);
    }
    const uint2 v = *reinterpret_cast<const uint2*>(s + row * (K / 32) + st * 8);
    return make_uint4(__builtin_amdgcn_perm(v.x, v.x, 0x01010000u), __builtin_amdgcn_perm(v.x, v.x, 0x03030202u),
                      __builtin_amdgcn_perm(v.y, v.y, 0x01010000u), __builtin_amdgcn_perm(v.y, v.y, 0x03030202u));
  }
  uint32_t w[4] = {0, 0, 0, 0};
  if (layout == 2) {
    // the transposed grid: slice i of the row's 16-row band is at i * (rows / 16) + row / 16
    // (32-bit offsets: the grid holds k16 * rows / 16 < 2^32 codes)
    const uint8_t* p = s + (row >> 4);
    const uint32_t stride = (uint32_t)(rows >> 4);
    uint32_t off = (uint32_t)(st * 16) * stride;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t b = st * 16 + i < k16 ? (uint32_t)p[off] : one;
      w[i >> 2] |= b << (8 * (i & 3));
      off += stride;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t slice = st * 16 + i;
    uint32_t b = one;
    if (slice < k16) {
      if (layout == 0) b = s[row * (K / B) + slice * 16 / B];
      else b = s[(row >> 4) * k16 + slice];
    }
    w[i >> 2] |= b << (8 * (i & 3));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// One code of a transposed-2D operand's stage, for a cooperative load: thread j of the
// operand's 128 staging threads takes slice j / 8 of the stage and 16-row band j % 8 of the
// tile (rows r0 .. r0 + 127; rows % 16 == 0 in this layout). Bands past the matrix and
// slices past K get the code of 1.0.
template <int FMT>
__device__ __forceinline__ uint32_t band_code(const uint8_t* __restrict__ s, int64_t rows, int64_t r0, int64_t K,
                                              int64_t st, int j) {
  const int64_t slice = st * 16 + (j >> 3), band = (r0 >> 4) + (j & 7);
  if (slice >= K / 16 || band >= (rows >> 4)) return ScaleFmt<FMT>::ONE;
  return s[(uint32_t)slice * (uint32_t)(rows >> 4) + (uint32_t)band];
}

// The decode-table entry of the scale code in byte `sub` of a word of codes:
// one 8-byte LDS read. The byte offset is made opaque so that the table's base address is
// added in the read's immediate offset rather than OR-ed into the address register, which
// would split the read in two.
__device__ __forceinline__ DecScale dec_entry(const uint2* table, uint32_t word, int sub) {
  uint32_t off = ((word >> (8 * sub)) & 0xFFu) << 3;
  asm("" : "+v"(off));
  const uint2 e = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(table) + off);
  DecScale d;
  d.p2 = __uint_as_float(e.x);
  d.m2 = __builtin_bit_cast(v2h, e.y);
  return d;
}

#ifndef FP4_DEC_UNROLL
#define FP4_DEC_UNROLL 1   // the group loop unrolled (interior stages always hold four groups)
#endif

using DecTiling = Tiling<2, 2, 2, 2>;   // 128x128 workgroup tile, 4 waves of 64x64

// INTERIOR: every tile lies inside the matrix and K is a multiple of 256 (no clamped loads;
// every stage holds four groups).
// QOUT: the epilogue also quantizes C as the next GEMM's ROW-view operand (qo).
template <int FMT, int B, bool INTERIOR, bool QOUT>
__global__ __launch_bounds__(DecTiling::NT, 2) void k_gemm_dec16(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                       int la, const uint8_t* __restrict__ qb,
                                                       const uint8_t* __restrict__ sb, int lb,
                                                       const float* __restrict__ ga, const float* __restrict__ gb,
                                                       float* __restrict__ c, int64_t M, int64_t N, int64_t K,
                                                       int canon, int epi, int align, const QuantOut qo) {
  using TL = DecTiling;
  constexpr int GT = TL::BM;        // == TL::BN
  __shared__ __attribute__((aligned(4096))) uint2 lDec[256];   // decode factors of every scale code (p2 bits, M pair)
  __shared__ __attribute__((aligned(1024))) uint8_t lA[2][TL::BM * ROWB];
  __shared__ __attribute__((aligned(1024))) uint8_t lB[2][TL::BN * ROWB];
  __shared__ uint4 lS[2][TL::BM + TL::BN];   // 16 slice-scale codes per row: A rows then B rows
  __shared__ uint4 lT[2][2][TL::BM / 16];     // transposed-2D operands: 16 codes per 16-row band
  static_assert(TL::NT == 256, "one decode-table entry per thread");
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  int64_t m0, n0;
  tile_coords(M, N, TL::BM, TL::BN, m0, n0);
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

  const bool srow_is_a = threadIdx.x < GT;
  const int srow = threadIdx.x & (GT - 1);
  const bool al_a = align & 1, al_b = align & 2;
  // scale staging: one row's 16 codes per thread, or for a transposed-2D operand one code per
  // thread (the operand's 128 threads cover its 8 bands x 16 slices)
  const int lay = srow_is_a ? la : lb;
  auto load_stage_scales = [&](int64_t st) -> uint4 {
    if (lay == 2)
      return make_uint4(srow_is_a ? band_code<FMT>(sa, M, m0, K, st, srow) : band_code<FMT>(sb, N, n0, K, st, srow), 0,
                        0, 0);
    return srow_is_a ? scale_row16<FMT, B>(sa, la, m0 + srow, M, K, st, al_a)
                     : scale_row16<FMT, B>(sb, lb, n0 + srow, N, K, st, al_b);
  };
  auto store_stage_scales = [&](int buf, const uint4& v) {
    if (lay == 2) reinterpret_cast<uint8_t*>(&lT[buf][srow_is_a ? 0 : 1][srow & 7])[srow >> 3] = (uint8_t)v.x;
    else lS[buf][threadIdx.x] = v;
  };
  {
    const DecScale d = dec_factors_code<FMT>(threadIdx.x);
    lDec[threadIdx.x] = make_uint2(__float_as_uint(d.p2), __builtin_bit_cast(uint32_t, d.m2));
  }
  uint4 sreg = load_stage_scales(0);
  StageLoader<TL::BM, TL::NW> LA;
  StageLoader<TL::BN, TL::NW> LB;
  LA.init(qa, M, K, m0);
  LB.init(qb, N, K, n0);
  if (nstages > 0) {
    if (INTERIOR) {
      LA.issue_interior(0, lA[0]);
      LB.issue_interior(0, lB[0]);
    } else {
      LA.issue(0, lA[0]);
      LB.issue(0, lB[0]);
    }
  }
  store_stage_scales(0, sreg);
  wait_vm();
  __syncthreads();

  for (int64_t st = 0; st < nstages; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) {
      if (INTERIOR) {
        LA.issue_interior(st + 1, lA[buf ^ 1]);
        LB.issue_interior(st + 1, lB[buf ^ 1]);
      } else {
        LA.issue(st + 1, lA[buf ^ 1]);
        LB.issue(st + 1, lB[buf ^ 1]);
      }
      sreg = load_stage_scales(st + 1);
    }
    // the stage's scale codes of this lane's rows: word g holds the codes of group g's four slices
    const uint32_t* scA[2];
    const uint32_t* scB[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int ra = wm * 64 + t * 32 + (l & 31), rb = wn * 64 + t * 32 + (l & 31);
      scA[t] = reinterpret_cast<const uint32_t*>(la == 2 ? &lT[buf][0][ra >> 4] : &lS[buf][ra]);
      scB[t] = reinterpret_cast<const uint32_t*>(lb == 2 ? &lT[buf][1][rb >> 4] : &lS[buf][GT + rb]);
    }
    const int g_end = INTERIOR ? SGR : (int)((ngroups - st * SGR) < SGR ? (ngroups - st * SGR) : SGR);
    uint32_t nwa[2], nwb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      nwa[t] = scA[t][0];
      nwb[t] = scB[t][0];
    }
#if FP4_DEC_UNROLL
#pragma unroll
#endif
    for (int g = 0; g < g_end; ++g) {
      uint32_t wa[2], wb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        wa[t] = nwa[t];
        wb[t] = nwb[t];
        nwa[t] = scA[t][(g + 1) & 3];
        nwb[t] = scB[t][(g + 1) & 3];
      }
      // decoded fp16 fragments (times 2^-3) of the group's four 16-wide slices
      v8h fa[4][2], fb[4][2];
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const int off = g * 32 + sub * 8 + half * 4;   // payload byte inside the stage row
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int rowa = wm * 64 + t * 32 + (l & 31);
          const int rowb = wn * 64 + t * 32 + (l & 31);
          const uint32_t ca = *reinterpret_cast<const uint32_t*>(lA[buf] + swz(rowa, off >> 4) + (off & 15));
          const uint32_t cb = *reinterpret_cast<const uint32_t*>(lB[buf] + swz(rowb, off >> 4) + (off & 15));
          fa[sub][t] = decode8(ca, dec_entry(lDec, wa[t], sub));
          fb[sub][t] = decode8(cb, dec_entry(lDec, wb[t], sub));
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // group partial of this tile, nearest-even (the loop's mode); the MFMA results
          // are pinned after the previous switch back to nearest-even
          v16f T[4];
#pragma unroll
          for (int sub = 0; sub < 4; ++sub)
            T[sub] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[sub][i], fb[sub][j], v16f{}, 0, 0, 0);
#pragma unroll
          for (int sub = 0; sub < 4; ++sub) pin(T[sub]);
          v16f G;
          if constexpr (B == 16) {
#pragma unroll
            for (int r = 0; r < 16; ++r) G[r] = ((T[0][r] + T[1][r]) + T[2][r]) + T[3][r];
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) G[r] = (T[0][r] + T[1][r]) + (T[2][r] + T[3][r]);   // inner adds exact
          }
          // cross-group accumulation, toward zero (pinned between the mode switches)
          pin(G);
          mode_f32_rtz();
          pin(G);
          pin(acc[i][j]);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = acc[i][j][r] + G[r];
          pin(acc[i][j]);
          mode_f32_rne();
          pin(acc[i][j]);
        }
    }
    if (st + 1 < nstages) {
      store_stage_scales(buf ^ 1, sreg);
      wait_vm();
      __syncthreads();
    }
  }
  if constexpr (QOUT) {
    static_assert(TL::BM == QO_T && TL::BN == QO_T, "the output quantizer stages 128 x 128 tiles");
    __syncthreads();   // every wave is done with the last stage's buffers
    const QoStage stg{reinterpret_cast<float*>(&lA[0][0]), reinterpret_cast<float*>(&lB[0][0]), wm * 64, wn * 64};
    store_tiles<2, 2, true>(c, M, N, m0 + wm * 64, n0 + wn * 64, acc, ga, gb, canon, epi, 64.0f, stg);
    quantize_out_tile<TL::NT>(stg, m0, n0, M, N, qo);
  } else {
    store_tiles<2, 2>(c, M, N, m0 + wm * 64, n0 + wn * 64, acc, ga, gb, canon, epi, 64.0f);   // undo 2^-3 x 2^-3
  }
}

template <int FMT, int B>
static hipError_t launch_dec16(const GemmArgs& g) {
  using TL = DecTiling;
  const int64_t tiles = ((g.M + TL::BM - 1) / TL::BM) * ((g.N + TL::BN - 1) / TL::BN);
  // per operand: scale array 16-byte aligned and K % 256 == 0 (whole-stage vector loads)
  const int align = (((reinterpret_cast<uintptr_t>(g.a.s) & 15) == 0 && g.K % 256 == 0) ? 1 : 0) |
                    (((reinterpret_cast<uintptr_t>(g.b.s) & 15) == 0 && g.K % 256 == 0) ? 2 : 0);
  const bool interior = g.M % TL::BM == 0 && g.N % TL::BN == 0 && g.K > 0 && g.K % KS == 0;
  auto kern = g.qout ? (interior ? k_gemm_dec16<FMT, B, true, true> : k_gemm_dec16<FMT, B, false, true>)
                     : (interior ? k_gemm_dec16<FMT, B, true, false> : k_gemm_dec16<FMT, B, false, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(TL::NT), 0, g.stream, g.a.q, g.a.s, g.a.layout, g.b.q, g.b.s,
                     g.b.layout, g.a.g, g.b.g, g.c, g.M, g.N, g.K, g.canon,
                     epilogue_word(g.hadamard_n, g.a.g_shift, g.b.g_shift), align, g.qout ? *g.qout : QuantOut{});
  return hipGetLastError();
}

hipError_t run_gemm_dec16(const GemmArgs& g) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (g.fmt == FMT_UE5M3) return g.block == 16 ? launch_dec16<FMT_UE5M3, 16>(g) : launch_dec16<FMT_UE5M3, 32>(g);
  return g.block == 16 ? launch_dec16<FMT_E4M3, 16>(g) : launch_dec16<FMT_E4M3, 32>(g);
}

}  // namespace fp4k
