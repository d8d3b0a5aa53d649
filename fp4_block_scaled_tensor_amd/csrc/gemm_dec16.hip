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
//
// Work per group: the model's additions (4 per output: three nearest-even slice adds and the
// toward-zero group add, 16 per MFMA) are fixed; the decode (8 vector instructions per 8
// values) is done once per workgroup. A workgroup owns a 128 x 128 output tile, 4 waves of
// 64 x 64. Each of its 256 threads owns one operand row (A rows 0-127, then B rows) and, one
// group ahead of the MFMAs, loads that row's 32 payload bytes and 4 slice scales of the next
// group from global memory into registers, decodes them (interleaved with the current
// group's MFMAs) and writes the 64 fp16 values to a double-buffered LDS tile (128 bytes per row; 16-byte chunk c of row r at position
// c ^ ((r >> 1) & 7): two rows share a 256-byte bank line, so sixteen consecutive rows cover
// all 64 banks for both the row-wise writes and the fragment reads). The waves read their MFMA fragments from that tile; one barrier per
// group hands the buffers over.
#include <algorithm>

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

// The 4 slice-scale codes of one operand row for group gi (byte i = 16-wide slice i; block 32
// repeats each code twice), in the operand's scale layout: 1D (row * K/B + block), forward
// 2D (16-row band * K/16 + slice) or transposed 2D (slice * rows/16 + band). With al (scale
// array 4-byte aligned) a 1D or forward-2D group is one 4-byte load (block 32: one 2-byte
// load, each code doubled with v_perm); the transposed layout, whose codes are strided,
// and unaligned arrays read byte by byte. row is clamped into the matrix.
template <int B>
__device__ __forceinline__ uint32_t group_codes(const uint8_t* __restrict__ s, int layout, int64_t row, int64_t rows,
                                                int64_t K, int64_t gi, bool al) {
  const int64_t k16 = K / 16;
  if (layout == 2) {
    // (32-bit offsets: the grid holds k16 * rows / 16 < 2^32 codes)
    const uint8_t* p = s + (row >> 4);
    const uint32_t stride = (uint32_t)(rows >> 4);
    uint32_t off = (uint32_t)(gi * 4) * stride, w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w |= (uint32_t)p[off] << (8 * i);
      off += stride;
    }
    return w;
  }
  if (layout == 0 && B == 32) {
    const int64_t off = row * (K / 32) + gi * 2;
    const uint32_t v = al ? (uint32_t)*reinterpret_cast<const uint16_t*>(s + off)
                          : ((uint32_t)s[off] | ((uint32_t)s[off + 1] << 8));
    return __builtin_amdgcn_perm(v, v, 0x01010000u);
  }
  const int64_t off = (layout == 1 ? (row >> 4) * k16 : row * k16) + gi * 4;
  if (al) return *reinterpret_cast<const uint32_t*>(s + off);
  return (uint32_t)s[off] | ((uint32_t)s[off + 1] << 8) | ((uint32_t)s[off + 2] << 16) | ((uint32_t)s[off + 3] << 24);
}

// One operand row's next group, in flight in registers: 32 payload bytes (8 words of 8 E2M1
// codes, K order) and the 4 slice-scale codes.
struct GroupRegs {
  uint4 p0, p1;
  uint32_t codes;
};

using DecTiling = Tiling<2, 2, 2, 2>;   // 128x128 workgroup tile, 4 waves of 64x64

// QOUT: the epilogue also quantizes C as the next GEMM's ROW-view operand (qo).
template <int FMT, int B, bool QOUT>
__global__ __launch_bounds__(DecTiling::NT, 2) void k_gemm_dec16(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                       int la, const uint8_t* __restrict__ qb,
                                                       const uint8_t* __restrict__ sb, int lb,
                                                       const float* __restrict__ ga, const float* __restrict__ gb,
                                                       float* __restrict__ c, int64_t M, int64_t N, int64_t K,
                                                       int canon, int epi, int align, const QuantOut qo) {
  using TL = DecTiling;
  constexpr int GT = TL::BM;                 // == TL::BN
  constexpr int DROW = 64 * 2;               // decoded bytes per operand row and group
  constexpr int DBUF = 2 * GT * DROW;        // one buffer: A rows then B rows (32 KB)
  __shared__ __attribute__((aligned(4096))) uint2 lDec[256];   // decode factors of every scale code (p2 bits, M pair)
  __shared__ __attribute__((aligned(1024))) uint8_t lD[2 * DBUF];
  static_assert(TL::NT == 2 * GT, "one operand row per thread");
  static_assert(TL::NT == 256, "one decode-table entry per thread");
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  int64_t m0, n0;
  tile_coords(M, N, TL::BM, TL::BN, m0, n0);
  const int64_t ngroups = K / 64;
  const int half = l >> 5;

  // the row this thread decodes (clamped into the matrix: rows past it feed only outputs
  // that are not stored)
  const bool is_a = threadIdx.x < GT;
  const int drow = threadIdx.x;              // row of the decoded tile (A rows, then B rows)
  const int64_t rows = is_a ? M : N;
  const int64_t grow0 = (is_a ? m0 : n0) + (drow & (GT - 1));
  const int64_t grow = grow0 < rows ? grow0 : rows - 1;
  const uint8_t* const qrow = (is_a ? qa : qb) + grow * (K / 2);
  const uint8_t* const srow = is_a ? sa : sb;
  const int lay = is_a ? la : lb;
  const bool al = is_a ? (align & 1) : (align & 2);
  auto load_group = [&](int64_t gi) {
    GroupRegs r;
    const uint4* p = reinterpret_cast<const uint4*>(qrow + gi * 32);
    r.p0 = p[0];
    r.p1 = p[1];
    r.codes = group_codes<B>(srow, lay, grow, rows, K, gi, al);
    return r;
  };
  const uint32_t wbase = (uint32_t)(drow * DROW);
  const uint32_t wkey = (uint32_t)((drow >> 1) & 7);
  // decoded chunk c of this thread's row goes to position c ^ ((drow >> 1) & 7); one call
  // decodes slice `sub` of a group (two words of codes)
  auto decode_sub = [&](const GroupRegs& r, int sub, int buf) {
    const uint32_t words[8] = {r.p0.x, r.p0.y, r.p0.z, r.p0.w, r.p1.x, r.p1.y, r.p1.z, r.p1.w};
    const DecScale d = dec_entry(lDec, r.codes, sub);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = 2 * sub + h;
      const v8h v = decode8(words[ch], d);
      *reinterpret_cast<v8h*>(lD + buf * DBUF + wbase + ((ch ^ wkey) << 4)) = v;
    }
  };
  // fragment reads: lane l reads row r0 + (l & 31) (r0 a multiple of 32, so r & 15 = l & 15),
  // logical chunk 2 sub + half at position (2 sub + half) ^ ((l >> 1) & 7)
  uint32_t ra[4], rb[4];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    const uint32_t pos = (uint32_t)((2 * sub + half) ^ ((l >> 1) & 7)) << 4;
    ra[sub] = (uint32_t)((wm * 64 + (l & 31)) * DROW) + pos;
    rb[sub] = (uint32_t)((GT + wn * 64 + (l & 31)) * DROW) + pos;
  }

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  {
    const DecScale d = dec_factors_code<FMT>(threadIdx.x);
    lDec[threadIdx.x] = make_uint2(__float_as_uint(d.p2), __builtin_bit_cast(uint32_t, d.m2));
  }
  GroupRegs nxt{};
  if (ngroups > 0) nxt = load_group(0);
  __syncthreads();   // decode table
  if (ngroups > 0) {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) decode_sub(nxt, sub, 0);
    if (ngroups > 1) nxt = load_group(1);
  }
  __syncthreads();

  // group partial G of tile (i, j) from its four slice sums, nearest-even (the loop's mode;
  // T is pinned after the previous switch back), then acc += G toward zero (pinned between
  // the mode switches)
  auto finish = [&](int i, int j, v16f (&T)[4]) {
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
    pin(G);
    mode_f32_rtz();
    pin(G);
    pin(acc[i][j]);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][j][r] = acc[i][j][r] + G[r];
    pin(acc[i][j]);
    mode_f32_rne();
    pin(acc[i][j]);
  };
  // one group: this group's MFMAs and additions from buffer gi & 1, with the next group's
  // decode into the other buffer (free since the last barrier) spread over the four tiles,
  // between each tile's MFMAs and its additions. Decoding again, in the last iteration, a
  // group already decoded only writes the buffer that no later read uses. The group after
  // the next is then loaded (clamped: the last iterations reload the final group).
  for (int64_t gi = 0; gi < ngroups; ++gi) {
    const int buf = (int)(gi & 1);
    const GroupRegs cur = nxt;
    const uint8_t* D = lD + buf * DBUF;
    v8h fa[4][2], fb[4][2];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        fa[sub][t] = *reinterpret_cast<const v8h*>(D + ra[sub] + t * 32 * DROW);
        fb[sub][t] = *reinterpret_cast<const v8h*>(D + rb[sub] + t * 32 * DROW);
      }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v16f T[4];
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
          T[sub] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[sub][i], fb[sub][j], v16f{}, 0, 0, 0);
        decode_sub(cur, 2 * i + j, buf ^ 1);
        finish(i, j, T);
      }
    nxt = load_group(gi + 2 < ngroups ? gi + 2 : ngroups - 1);
    __syncthreads();
  }
  if constexpr (QOUT) {
    static_assert(TL::BM == QO_T && TL::BN == QO_T, "the output quantizer stages 128 x 128 tiles");
    static_assert(DBUF >= 64 * QO_T * 4, "two 64-row float32 halves of the output tile");
    const QoStage stg{reinterpret_cast<float*>(lD), reinterpret_cast<float*>(lD + DBUF), wm * 64, wn * 64};
    store_tiles<2, 2, true>(c, M, N, m0 + wm * 64, n0 + wn * 64, acc, ga, gb, canon, epi, 64.0f, stg);
    quantize_out_tile<TL::NT>(stg, m0, n0, M, N, qo);
  } else {
    store_tiles<2, 2>(c, M, N, m0 + wm * 64, n0 + wn * 64, acc, ga, gb, canon, epi, 64.0f);   // undo 2^-3 x 2^-3
  }
}

// ---------------------------------------------------------------- decode once per operand
// The operand decoded once into fp16 [rows x K], K-contiguous: the same exact values
// q S 2^-3 the per-tile decode above produces. A GEMM whose two operands come with this copy
// reads it instead of decoding per workgroup (the per-tile decode costs more than a third
// of that kernel's time; the copy costs 2 bytes per element written once and read by the
// GEMM through L2). One thread per 8-element chunk of a row (a 4-byte payload word, its
// slice's scale code, 16 bytes out), so that a wave reads 256 and writes 1024 consecutive
// bytes of a row; workgroups of 256 chunks, rows strided over the grid's y.
template <int FMT>
__device__ __forceinline__ DecScale dec_factors_nb(uint32_t c) {
  // dec_factors_code without branches (lanes of one wave hold different codes)
  constexpr int SUB_EXP = FMT == FMT_UE5M3 ? 17 : 9;
  const uint32_t e = c >> 3, m = c & 7u;
  DecScale d;
  d.p2 = __uint_as_float(e != 0 ? (e + (uint32_t)(127 - ScaleFmt<FMT>::BIAS - 3)) << 23
                                : (uint32_t)(127 - SUB_EXP - 3) << 23);
  const uint32_t hs = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(float)m);   // exact
  const uint32_t h = e != 0 ? (0x3C00u | (m << 7)) : hs;
  d.m2 = __builtin_bit_cast(v2h, h | (h << 16));
  return d;
}

template <int FMT, int B>
__global__ __launch_bounds__(256) void k_decode_f16(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                    int layout, int64_t rows, int64_t K, bool al,
                                                    _Float16* __restrict__ out) {
  (void)al;
  const int64_t nc = K / 8;
  const int64_t kc = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (kc >= nc) return;
  const int64_t k16 = K / 16, slice = kc >> 1;
  for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
    const uint32_t word = *reinterpret_cast<const uint32_t*>(q + row * (K / 2) + kc * 4);
    uint32_t code;
    if (layout == 2) code = s[slice * (rows >> 4) + (row >> 4)];
    else if (layout == 1) code = s[(row >> 4) * k16 + slice];
    else code = s[row * (K / B) + (B == 16 ? slice : slice >> 1)];
    *reinterpret_cast<v8h*>(out + row * K + kc * 8) = decode8(word, dec_factors_nb<FMT>(code));
  }
}

template <int FMT, int B>
static hipError_t launch_decode_f16(const GemmOperand& a, int64_t K, void* out, hipStream_t stream) {
  const dim3 grid((unsigned)((K / 8 + 255) / 256), (unsigned)std::min<int64_t>(a.rows, 65535));
  hipLaunchKernelGGL((k_decode_f16<FMT, B>), grid, dim3(256), 0, stream, a.q, a.s, a.layout, a.rows, K, true,
                     reinterpret_cast<_Float16*>(out));
  return hipGetLastError();
}

hipError_t run_decode_f16(const GemmOperand& a, int fmt, int block, int64_t K, void* out, hipStream_t stream) {
  if (a.rows == 0 || K == 0) return hipSuccess;
  if (fmt == FMT_UE5M3)
    return block == 16 ? launch_decode_f16<FMT_UE5M3, 16>(a, K, out, stream)
                       : launch_decode_f16<FMT_UE5M3, 32>(a, K, out, stream);
  return block == 16 ? launch_decode_f16<FMT_E4M3, 16>(a, K, out, stream)
                     : launch_decode_f16<FMT_E4M3, 32>(a, K, out, stream);
}

// The GEMM over decoded fp16 operands: the group loop of k_gemm_dec16 without the decode.
// Each group's 128 fp16 rows of A and of B (128 bytes per row, one stage) go straight from
// global memory into a double-buffered LDS tile with global_load_lds (the same chunk swizzle:
// chunk c of row r at c ^ ((r >> 1) & 7)); the next group's copy is in flight during the
// current group's MFMAs and additions. Same MFMAs, additions, rounding modes and epilogue.
// This form (four waves of 64 x 64, two waves per SIMD) serves block 32; block 16 runs
// k_gemm_f16_w8 below.
#ifndef FP4_F16_TILING
#define FP4_F16_TILING 2, 2, 2, 2
#endif
using F16Tiling = Tiling<FP4_F16_TILING>;   // waves of 64 x 64 (TM = TN = 2)

template <int B, bool INTERIOR>
__global__ __launch_bounds__(F16Tiling::NT, 512 / F16Tiling::NT) void k_gemm_f16(const uint8_t* __restrict__ a16,
                                                     const uint8_t* __restrict__ b16,
                                                     const float* __restrict__ ga, const float* __restrict__ gb,
                                                     float* __restrict__ c, int64_t M, int64_t N, int64_t K,
                                                     int canon, int epi) {
  using TL = F16Tiling;
  static_assert(TL::TM == 2 && TL::TN == 2, "waves of 64 x 64");
  constexpr int DROW = 64 * 2;               // fp16 bytes per row and group (one stage)
  constexpr int DBUF = (TL::BM + TL::BN) * DROW;   // one buffer: A rows then B rows
  static_assert(DROW == ROWB, "one group of fp16 is one 128-byte stage row");
  __shared__ __attribute__((aligned(1024))) uint8_t lD[2 * DBUF];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / TL::WN, wn = w % TL::WN;
  int64_t m0, n0;
  tile_coords(M, N, TL::BM, TL::BN, m0, n0);
  const int64_t ngroups = K / 64;
  const int half = l >> 5;
  // the loaders see rows of 2K bytes: 4K "FP4 elements"
  StageLoader<TL::BM, TL::NW> LA;
  StageLoader<TL::BN, TL::NW> LB;
  LA.init(a16, M, 4 * K, m0);
  LB.init(b16, N, 4 * K, n0);
  auto issue = [&](int64_t gi, int buf) {
    if (INTERIOR) {
      LA.issue_interior(gi, lD + buf * DBUF);
      LB.issue_interior(gi, lD + buf * DBUF + TL::BM * DROW);
    } else {
      LA.issue(gi, lD + buf * DBUF);
      LB.issue(gi, lD + buf * DBUF + TL::BM * DROW);
    }
  };
  uint32_t ra[4], rb[4];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    const uint32_t pos = (uint32_t)((2 * sub + half) ^ ((l >> 1) & 7)) << 4;
    ra[sub] = (uint32_t)((wm * 64 + (l & 31)) * DROW) + pos;
    rb[sub] = (uint32_t)((TL::BM + wn * 64 + (l & 31)) * DROW) + pos;
  }
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (ngroups > 0) issue(0, 0);
  wait_vm();
  __syncthreads();
  for (int64_t gi = 0; gi < ngroups; ++gi) {
    const int buf = (int)(gi & 1);
    if (gi + 1 < ngroups) issue(gi + 1, buf ^ 1);
    const uint8_t* D = lD + buf * DBUF;
    v8h fa[4][2], fb[4][2];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        fa[sub][t] = *reinterpret_cast<const v8h*>(D + ra[sub] + t * 32 * DROW);
        fb[sub][t] = *reinterpret_cast<const v8h*>(D + rb[sub] + t * 32 * DROW);
      }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
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
    wait_vm();
    __syncthreads();
  }
  store_tiles<2, 2>(c, M, N, m0 + wm * 64, n0 + wn * 64, acc, ga, gb, canon, epi, 64.0f);   // undo 2^-3 x 2^-3
}

// Block 16 at four waves per SIMD: 128 x 128 workgroup tiles of 8 waves of 32 x 64 (two
// 32x32 output tiles per wave sharing each A fragment). Each 16-wide slice's fragments are
// read just before its MFMAs and each tile's group partial is accumulated slice by slice,
// ((T0 + T1) + T2) + T3 in K order with nearest-even adds, so that the kernel fits in 128
// VGPRs. Same staging, swizzle, rounding modes and epilogue as k_gemm_f16.
using F16TilingW8 = Tiling<4, 2, 1, 2>;

template <bool INTERIOR>
__global__ __launch_bounds__(F16TilingW8::NT, 4) void k_gemm_f16_w8(const uint8_t* __restrict__ a16,
                                                                const uint8_t* __restrict__ b16,
                                                                const float* __restrict__ ga,
                                                                const float* __restrict__ gb, float* __restrict__ c,
                                                                int64_t M, int64_t N, int64_t K, int canon, int epi) {
  using TL = F16TilingW8;
  constexpr int DROW = 64 * 2;
  constexpr int DBUF = (TL::BM + TL::BN) * DROW;
  __shared__ __attribute__((aligned(1024))) uint8_t lD[2 * DBUF];
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / TL::WN, wn = w % TL::WN;
  int64_t m0, n0;
  tile_coords(M, N, TL::BM, TL::BN, m0, n0);
  const int64_t ngroups = K / 64;
  const int half = l >> 5;
  StageLoader<TL::BM, TL::NW> LA;
  StageLoader<TL::BN, TL::NW> LB;
  LA.init(a16, M, 4 * K, m0);
  LB.init(b16, N, 4 * K, n0);
  auto issue = [&](int64_t gi, int buf) {
    if (INTERIOR) {
      LA.issue_interior(gi, lD + buf * DBUF);
      LB.issue_interior(gi, lD + buf * DBUF + TL::BM * DROW);
    } else {
      LA.issue(gi, lD + buf * DBUF);
      LB.issue(gi, lD + buf * DBUF + TL::BM * DROW);
    }
  };
  uint32_t ra[4], rb[4];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    const uint32_t pos = (uint32_t)((2 * sub + half) ^ ((l >> 1) & 7)) << 4;
    ra[sub] = (uint32_t)((wm * 32 + (l & 31)) * DROW) + pos;
    rb[sub] = (uint32_t)((TL::BM + wn * 64 + (l & 31)) * DROW) + pos;
  }
  v16f acc[1][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][j][r] = 0.0f;
  if (ngroups > 0) issue(0, 0);
  wait_vm();
  __syncthreads();
  for (int64_t gi = 0; gi < ngroups; ++gi) {
    const int buf = (int)(gi & 1);
    if (gi + 1 < ngroups) issue(gi + 1, buf ^ 1);
    const uint8_t* D = lD + buf * DBUF;
    v16f G[2];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const v8h fa = *reinterpret_cast<const v8h*>(D + ra[sub]);
      const v8h fb0 = *reinterpret_cast<const v8h*>(D + rb[sub]);
      const v8h fb1 = *reinterpret_cast<const v8h*>(D + rb[sub] + 32 * DROW);
      v16f T0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb0, v16f{}, 0, 0, 0);
      v16f T1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb1, v16f{}, 0, 0, 0);
      pin(T0);
      pin(T1);
      if (sub == 0) {
        G[0] = T0;
        G[1] = T1;
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          G[0][r] = G[0][r] + T0[r];   // nearest-even (the loop's mode), in K order
          G[1][r] = G[1][r] + T1[r];
        }
      }
    }
    pin(G[0]);
    pin(G[1]);
    mode_f32_rtz();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      pin(G[j]);
      pin(acc[0][j]);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[0][j][r] = acc[0][j][r] + G[j][r];
      pin(acc[0][j]);
    }
    mode_f32_rne();
#pragma unroll
    for (int j = 0; j < 2; ++j) pin(acc[0][j]);
    wait_vm();
    __syncthreads();
  }
  store_tiles<1, 2>(c, M, N, m0 + wm * 32, n0 + wn * 64, acc, ga, gb, canon, epi, 64.0f);   // undo 2^-3 x 2^-3
}

template <int B>
static hipError_t launch_f16(const GemmArgs& g) {
  if constexpr (B == 16) {
    using TW = F16TilingW8;
    const int64_t tw = ((g.M + TW::BM - 1) / TW::BM) * ((g.N + TW::BN - 1) / TW::BN);
    const bool inter = g.M % TW::BM == 0 && g.N % TW::BN == 0;
    auto kw = inter ? k_gemm_f16_w8<true> : k_gemm_f16_w8<false>;
    hipLaunchKernelGGL(kw, dim3((unsigned)tw), dim3(TW::NT), 0, g.stream, reinterpret_cast<const uint8_t*>(g.a16),
                       reinterpret_cast<const uint8_t*>(g.b16), g.a.g, g.b.g, g.c, g.M, g.N, g.K, g.canon,
                       epilogue_word(g.hadamard_n, g.a.g_shift, g.b.g_shift));
    return hipGetLastError();
  }
  using TL = F16Tiling;
  const int64_t tiles = ((g.M + TL::BM - 1) / TL::BM) * ((g.N + TL::BN - 1) / TL::BN);
  const bool interior = g.M % TL::BM == 0 && g.N % TL::BN == 0;
  auto kern = interior ? k_gemm_f16<B, true> : k_gemm_f16<B, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(TL::NT), 0, g.stream,
                     reinterpret_cast<const uint8_t*>(g.a16), reinterpret_cast<const uint8_t*>(g.b16), g.a.g, g.b.g,
                     g.c, g.M, g.N, g.K, g.canon, epilogue_word(g.hadamard_n, g.a.g_shift, g.b.g_shift));
  return hipGetLastError();
}

template <int FMT, int B>
static hipError_t launch_dec16(const GemmArgs& g) {
  using TL = DecTiling;
  const int64_t tiles = ((g.M + TL::BM - 1) / TL::BM) * ((g.N + TL::BN - 1) / TL::BN);
  // per operand: scale array aligned for the group's one-word load (4 bytes; block 32, 2 bytes)
  const uintptr_t am = B == 32 ? 1 : 3;
  const int align = ((reinterpret_cast<uintptr_t>(g.a.s) & am) == 0 ? 1 : 0) |
                    ((reinterpret_cast<uintptr_t>(g.b.s) & am) == 0 ? 2 : 0);
  auto kern = g.qout ? k_gemm_dec16<FMT, B, true> : k_gemm_dec16<FMT, B, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(TL::NT), 0, g.stream, g.a.q, g.a.s, g.a.layout, g.b.q, g.b.s,
                     g.b.layout, g.a.g, g.b.g, g.c, g.M, g.N, g.K, g.canon,
                     epilogue_word(g.hadamard_n, g.a.g_shift, g.b.g_shift), align, g.qout ? *g.qout : QuantOut{});
  return hipGetLastError();
}

hipError_t run_gemm_dec16(const GemmArgs& g) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (g.a16 && g.b16 && !g.qout) return g.block == 16 ? launch_f16<16>(g) : launch_f16<32>(g);
  if (g.fmt == FMT_UE5M3) return g.block == 16 ? launch_dec16<FMT_UE5M3, 16>(g) : launch_dec16<FMT_UE5M3, 32>(g);
  return g.block == 16 ? launch_dec16<FMT_E4M3, 16>(g) : launch_dec16<FMT_E4M3, 32>(g);
}

}  // namespace fp4k
