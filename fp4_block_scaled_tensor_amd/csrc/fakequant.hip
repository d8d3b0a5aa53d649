// Inference fake quantization and operand decode for gfx950 (HBM-bound).
//
// "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach (접근 방법),
// training and inference setup: held-out likelihoods are measured with FP4 fake
// quantization, the activation scale following a delayed (D = 50), current (D = 1) or
// frozen policy; the policies only decide which cached amax a call receives.
//
// Decoded value of an operand element: x_hat = E2M1(q) * S * g (g = 1 for E8M0). E2M1(q) comes
// from v_cvt_scalef32_pk_f32_fp4 with scale 1.0 (exact); E2M1(q) * S is exact in float32
// (at most 6 significant bits; an E8M0 scale is a power of two, 2^-127 included as a
// subnormal); the product with g is one float32 multiply, nearest-even. A bfloat16 output is
// rounded from that float32, nearest-even.
//
// Kernels:
//   k_fake_quant  x -> x_hat in one pass (ROW view, nearest-even): a 16-row x 512-column tile
//                 per workgroup, 64 lanes per 512-element row segment (1 KB of bf16), a block
//                 of B elements spans B/8 lanes whose maxima combine by DPP, codes are made and
//                 decoded in registers.
//   k_dequant     a quantized operand (1D, 2D or transposed-2D scales) -> x_hat, the same
//                 lane layout on 32-row x 512-column tiles (256 payload bytes per row).
//   k_mx_to_fp8   MXFP4 operand -> FP8 E4M3 with one E8M0 scale per 128-element chunk
//                 ("Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
//                 methodology: direct FP4 -> FP8 conversion, hierarchical scale alignment
//                 from block 32 to block 128, transpose fused): chunk code c = e_max -
//                 min(6, e_max) over the chunk's four block codes, element
//                 E4M3(E2M1(q) * 2^(e_b - c)) nearest-even with subnormals, sign kept. One
//                 lane per 32-element block, 4 lanes per 128-element chunk (e_max by DPP),
//                 codes by a per-block v_perm_b32 table; 128-row x 256-column tiles in the
//                 row-major form, 256-row x 128-column tiles in the transposed form, which
//                 goes through a 34 KB LDS byte tile.
// Raw buffer loads and stores with out-of-range offsets for lanes outside the matrix.
#include "quant_common.hpp"

namespace fp4k {

// Tile shapes (measured at 8192 x 4096 with inputs streamed from HBM: wider rows read and
// write longer contiguous segments; fake quant 16 x 512 against 64 x 128: 24.2 vs 26.9 us,
// decode 32 x 512 against 32 x 256: 19.9 vs 20.7 us).
#ifndef FP4_FQ_TILE
#define FP4_FQ_TILE 16, 512
#endif
#ifndef FP4_DQ_TILE
#define FP4_DQ_TILE 32, 512
#endif
constexpr int FQ_TILE[2] = {FP4_FQ_TILE}, DQ_TILE[2] = {FP4_DQ_TILE};
constexpr int FT = FQ_TILE[0];       // fake quant: rows per tile
constexpr int FF = FQ_TILE[1];       // fake quant: columns per tile
constexpr int FLR = FF / 8;          // lanes per tile row (8 elements each)
constexpr int FPP = NT / FLR;        // rows per pass
constexpr int FPASSES = FT / FPP;
constexpr int DT = DQ_TILE[0];       // decode: rows per tile
constexpr int DF = DQ_TILE[1];       // decode: columns per tile
constexpr int DLR = DF / 8;
constexpr int DPP = NT / DLR;
constexpr int DPASSES = DT / DPP;
static_assert(FLR <= NT && NT % FLR == 0 && FPASSES >= 1 && FPASSES * FPP == FT, "fake-quant tile");
static_assert(DLR <= NT && NT % DLR == 0 && DPASSES >= 1 && DPASSES * DPP == DT && DT % 16 == 0, "decode tile");

// nearest-even float32 -> bfloat16 bits (finite inputs; overflow rounds to infinity)
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// decoded float32 values of 8 codes (element 0 in the low nibble of w) for scale value sv
// and tensor decode scale g
template <int FMT, int J>
__device__ __forceinline__ void decode2(uint32_t w, float sv, float g, float* y) {
  const auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, J);
  float a = p[0] * sv, b = p[1] * sv;                // exact
  if constexpr (FMT != FMT_E8M0) {
    a = a * g;
    b = b * g;
  }
  y[2 * J] = a;
  y[2 * J + 1] = b;
}

template <int FMT>
__device__ __forceinline__ void decode8(uint32_t w, float sv, float g, float* y) {
  decode2<FMT, 0>(w, sv, g, y);
  decode2<FMT, 1>(w, sv, g, y);
  decode2<FMT, 2>(w, sv, g, y);
  decode2<FMT, 3>(w, sv, g, y);
}

// scale value of a code: UE5M3 / E4M3 by their decoders, E8M0 as 2^(c-127)
template <int FMT>
__device__ __forceinline__ float scale_value(uint32_t c) {
  if constexpr (FMT == FMT_E8M0) return e8m0_inv(254u - c);
  else return dec_scale3<FMT>(c);
}

// store 8 decoded values (float32: 32 bytes, bfloat16: 16 bytes) at byte offset off
template <bool BF16>
__device__ __forceinline__ void store8(rsrc_t r, uint32_t off, const float* y) {
  if constexpr (BF16) {
    const v4u w = {bf16_rne(y[0]) | (bf16_rne(y[1]) << 16), bf16_rne(y[2]) | (bf16_rne(y[3]) << 16),
                   bf16_rne(y[4]) | (bf16_rne(y[5]) << 16), bf16_rne(y[6]) | (bf16_rne(y[7]) << 16)};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, ST_NT);
  } else {
    const v4u a = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
    const v4u b = {__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]), __float_as_uint(y[7])};
    __builtin_amdgcn_raw_buffer_store_b128(a, r, off, 0, ST_NT);
    __builtin_amdgcn_raw_buffer_store_b128(b, r, off == OOB ? OOB : off + 16u, 0, ST_NT);
  }
}

template <int FMT, int B, bool F32, bool BF16>
__global__ __launch_bounds__(NT) void k_fake_quant(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                   int64_t ld, const float* __restrict__ d_amax, float T,
                                                   void* __restrict__ y, int64_t ldy) {
  constexpr int LB = B / 8;                     // lanes per block
  constexpr int ESZ = F32 ? 4 : 2, OSZ = BF16 ? 2 : 4;
  const int64_t nft = (cols + FF - 1) / FF;
  const int64_t t0 = (int64_t)(blockIdx.x / nft) * FT, f0 = (int64_t)(blockIdx.x % nft) * FF;
  TensorScales ts{1.0f, 1.0f, 1.0f};
  if constexpr (FMT != FMT_E8M0) ts = tensor_scales(d_amax, T);
  const int lc = threadIdx.x % FLR, lr = threadIdx.x / FLR;
  const int rl = (int)min(rows - t0, (int64_t)FT), cl = (int)min(cols - f0, (int64_t)FF);
  const bool cok = lc * 8 < cl;
  const rsrc_t rx = make_rsrc(reinterpret_cast<const char*>(x) + (t0 * ld + f0) * ESZ);
  const rsrc_t ry = make_rsrc(reinterpret_cast<char*>(y) + (t0 * ldy + f0) * OSZ);
  const uint32_t ld_b = (uint32_t)(ld * ESZ), ldy_b = (uint32_t)(ldy * OSZ);
  Chunk8<F32> c[FPASSES];
#pragma unroll
  for (int p = 0; p < FPASSES; ++p) {
    const int r = p * FPP + lr;
    c[p].load(rx, (cok && r < rl) ? (uint32_t)r * ld_b + (uint32_t)(lc * 8 * ESZ) : OOB);
  }
#pragma unroll
  for (int p = 0; p < FPASSES; ++p) {
    const int r = p * FPP + lr;
    float v[8];
    c[p].to_float(v);
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = mag_max(am, fabsf(v[j]));
    am = group_max<LB>(am);
    uint32_t code;
    float mult;
    block_scale<FMT>(am, ts, code, mult);
    uint32_t w;
    payload<8, false>(v, mult, 0, 0, 0, &w);
    float out[8];
    decode8<FMT>(w, scale_value<FMT>(code), ts.g, out);
    store8<BF16>(ry, (cok && r < rl) ? (uint32_t)r * ldy_b + (uint32_t)(lc * 8 * OSZ) : OOB, out);
  }
}

// scale code of element (r, k) of an operand: 1D [rows x K/B], 2D [rows/16 x K/16], or the
// transposed 2D grid [K/16 x rows/16] of the weight this operand is the transpose of
template <int LAYOUT, int B>
__device__ __forceinline__ int64_t scale_index(int64_t r, int64_t k, int64_t rows, int64_t K) {
  if constexpr (LAYOUT == 0) return r * (K / B) + k / B;
  else if constexpr (LAYOUT == 1) return (r / 16) * (K / 16) + k / 16;
  else return (k / 16) * (rows / 16) + r / 16;
}

template <int FMT, int B, int LAYOUT, bool BF16>
__global__ __launch_bounds__(NT) void k_dequant(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                const float* __restrict__ d_g, int64_t rows, int64_t K,
                                                void* __restrict__ y, int64_t ldy) {
  constexpr int OSZ = BF16 ? 2 : 4;
  const int64_t nft = (K + DF - 1) / DF;
  const int64_t t0 = (int64_t)(blockIdx.x / nft) * DT, f0 = (int64_t)(blockIdx.x % nft) * DF;
  const float g = (FMT == FMT_E8M0 || d_g == nullptr) ? 1.0f : *d_g;
  const int lc = threadIdx.x % DLR, lr = threadIdx.x / DLR;
  const int rl = (int)min(rows - t0, (int64_t)DT), cl = (int)min(K - f0, (int64_t)DF);
  const bool cok = lc * 8 < cl;
  const rsrc_t rq = make_rsrc(q + t0 * (K / 2) + f0 / 2);
  const rsrc_t ry = make_rsrc(reinterpret_cast<char*>(y) + (t0 * ldy + f0) * OSZ);
  const uint32_t qrow = (uint32_t)(K / 2), ldy_b = (uint32_t)(ldy * OSZ);
  uint32_t w[DPASSES];
  uint32_t sc[DPASSES];
#pragma unroll
  for (int p = 0; p < DPASSES; ++p) {
    const int r = p * DPP + lr;
    const bool ok = cok && r < rl;
    w[p] = __builtin_amdgcn_raw_buffer_load_b32(rq, ok ? (uint32_t)r * qrow + (uint32_t)(lc * 4) : OOB, 0, 0);
    sc[p] = ok ? s[scale_index<LAYOUT, B>(t0 + r, f0 + lc * 8, rows, K)] : 127u;
  }
#pragma unroll
  for (int p = 0; p < DPASSES; ++p) {
    const int r = p * DPP + lr;
    float out[8];
    decode8<FMT>(w[p], scale_value<FMT>(sc[p]), g, out);
    store8<BF16>(ry, (cok && r < rl) ? (uint32_t)r * ldy_b + (uint32_t)(lc * 8 * OSZ) : OOB, out);
  }
}

// ---------------------------------------------------------------- MXFP4 -> FP8
constexpr int XC = 128;   // FP8 scale chunk
// Conversion tile (measured at 8192 x 4096): the row-major form reads and writes longer row
// segments with two chunks per tile row (128 x 256); the transposed form keeps one chunk
// per row and 256 rows (its LDS byte tile's column writes conflict more as K grows, and
// its output rows are XT bytes long).
#ifndef FP4_XT_TR
#define FP4_XT_TR 128, 256   // transposed form: K, rows per tile
#endif
constexpr int XT_TR[2] = {FP4_XT_TR};
template <bool TRANSPOSE>
struct XTile {
  static constexpr int K = TRANSPOSE ? XT_TR[0] : 256;   // K per tile (a multiple of XC)
  static constexpr int T = TRANSPOSE ? XT_TR[1] : 128;   // rows per tile
  static constexpr int L = K / 32;                  // lanes per tile row (one 32-element block each)
  static constexpr int PP = NT / L;                 // rows per pass
  static constexpr int P = T / PP;                  // rows per thread
  static constexpr int RS = T + 16;                 // LDS byte-tile row stride (16-byte aligned, staggers banks)
};

// max over the 4 lanes of a quad (integers)
__device__ __forceinline__ int quad_max(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  return v;
}

// E4M3 code (sign in bit 7) of E2M1 value a times 2^k, k <= 6 (nearest-even; exact when the
// product is on E4M3's grid). Below 2^-20 every E2M1 value rounds to 0, so k is clamped.
__device__ __forceinline__ uint32_t e4m3_of(float a, int k) {
  k = k < -20 ? -20 : k;
  const float v = a * __uint_as_float((uint32_t)(k + 127) << 23);   // exact
  return enc_scale3<FMT_E4M3>(fabsf(v)) | ((__float_as_uint(v) >> 24) & 0x80u);
}

// 32 codes of one MXFP4 block (16 payload bytes) -> 32 E4M3 bytes (8 dwords).
// For k >= -5 every nonzero E2M1 magnitude times 2^k is a normal E4M3 number, whose code is
// the k = 0 code plus 8k (the exponent field moves by k): the block's 8-entry magnitude ->
// code table is two dwords, looked up 4 bytes at a time with v_perm_b32 (even and odd
// nibbles separately, then interleaved), and the E2M1 sign bit moves to bit 7. Smaller k
// (a block more than 11 binades below its chunk's largest) takes the per-element path.
__device__ __forceinline__ void block_to_fp8(const uint4& q, int k, uint32_t* out) {
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
  if (k >= -5) {
    const uint32_t add = (uint32_t)(k * 8);
    const uint32_t t_lo = 0x3C383000u + add * 0x01010100u;   // magnitudes 0, 0.5, 1, 1.5
    const uint32_t t_hi = 0x4C484440u + add * 0x01010101u;   // magnitudes 2, 3, 4, 6
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t w = qw[d];
      const uint32_t ev = __builtin_amdgcn_perm(t_hi, t_lo, w & 0x07070707u) | ((w & 0x08080808u) << 4);
      const uint32_t od = __builtin_amdgcn_perm(t_hi, t_lo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
      out[2 * d] = __builtin_amdgcn_perm(od, ev, 0x05010400u);       // elements 0..3
      out[2 * d + 1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);   // elements 4..7
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float v[8];
      decode8<FMT_E8M0>(qw[d], 1.0f, 1.0f, v);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        out[2 * d + h] = e4m3_of(v[4 * h], k) | (e4m3_of(v[4 * h + 1], k) << 8) | (e4m3_of(v[4 * h + 2], k) << 16) |
                         (e4m3_of(v[4 * h + 3], k) << 24);
    }
  }
}

template <bool TRANSPOSE>
__global__ __launch_bounds__(NT) void k_mx_to_fp8(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                  int64_t rows, int64_t K, uint8_t* __restrict__ y,
                                                  uint8_t* __restrict__ s8) {
  using X = XTile<TRANSPOSE>;
  constexpr int XK = X::K, XT = X::T, XL = X::L, XPP = X::PP, XP = X::P, XRS = X::RS;
  __shared__ __align__(16) uint8_t tile[TRANSPOSE ? XK : 1][TRANSPOSE ? XRS : 16];
  const int64_t nkt = (K + XK - 1) / XK;
  const int64_t r0 = (int64_t)(blockIdx.x / nkt) * XT, k0 = (int64_t)(blockIdx.x % nkt) * XK;
  const int b = threadIdx.x % XL, lr = threadIdx.x / XL;       // block within the tile row, row
  const int rl = (int)min(rows - r0, (int64_t)XT);
  const int kc = (int)min(K - k0, (int64_t)XK);                // K % 128 == 0: whole chunks
  const bool kok = b * 32 < kc;
  const rsrc_t rq = make_rsrc(q + r0 * (K / 2) + k0 / 2);
  const uint32_t qrow = (uint32_t)(K / 2);
  uint4 qv[XP];
  int eb[XP];
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    const int r = p * XPP + lr;
    const bool ok = kok && r < rl;
    const v4u t = __builtin_amdgcn_raw_buffer_load_b128(rq, ok ? (uint32_t)r * qrow + (uint32_t)(b * 16) : OOB, 0, 0);
    qv[p] = make_uint4(t[0], t[1], t[2], t[3]);
    eb[p] = ok ? (int)s[(r0 + r) * (K / 32) + k0 / 32 + b] : 0;
  }
  const rsrc_t ry = make_rsrc(TRANSPOSE ? y + k0 * rows + r0 : y + r0 * K + k0);
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    const int r = p * XPP + lr;
    const bool ok = kok && r < rl;
    const int emax = quad_max(eb[p]);                          // the chunk's four blocks: lanes 4j..4j+3
    const int c = emax - min(6, emax);
    if ((b & 3) == 0 && ok) s8[(r0 + r) * (K / XC) + k0 / XC + b / 4] = (uint8_t)c;
    uint32_t out[8];
    block_to_fp8(qv[p], eb[p] - c, out);
    if constexpr (!TRANSPOSE) {
      const uint32_t off = ok ? (uint32_t)r * (uint32_t)K + (uint32_t)(b * 32) : OOB;
      const v4u lo = {out[0], out[1], out[2], out[3]}, hi = {out[4], out[5], out[6], out[7]};
      __builtin_amdgcn_raw_buffer_store_b128(lo, ry, off, 0, ST_NT);
      __builtin_amdgcn_raw_buffer_store_b128(hi, ry, off == OOB ? OOB : off + 16u, 0, ST_NT);
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) tile[b * 32 + j][r] = (uint8_t)(out[j >> 2] >> (8 * (j & 3)));
    }
  }
  if constexpr (TRANSPOSE) {
    __syncthreads();
    // y_t rows k0 + kk, bytes [r0, r0 + XT) in 16-byte pieces
#pragma unroll
    for (int i = 0; i < XK * XT / 16 / NT; ++i) {
      const int piece = threadIdx.x + i * NT;
      const int kk = piece / (XT / 16), c16 = piece % (XT / 16);
      const uint4 w = *reinterpret_cast<const uint4*>(&tile[kk][c16 * 16]);
      const v4u wv = {w.x, w.y, w.z, w.w};
      __builtin_amdgcn_raw_buffer_store_b128(
          wv, ry, (kk < kc && c16 * 16 < rl) ? (uint32_t)kk * (uint32_t)rows + (uint32_t)(c16 * 16) : OOB, 0, ST_NT);
    }
  }
}

// ---------------------------------------------------------------- launchers
template <int FMT, int B, bool F32, bool BF16>
static hipError_t launch_fq(const FakeQuantArgs& a) {
  const int64_t tiles = ((a.rows + FT - 1) / FT) * ((a.cols + FF - 1) / FF);
  hipLaunchKernelGGL((k_fake_quant<FMT, B, F32, BF16>), dim3((unsigned)tiles), dim3(NT), 0, a.stream, a.x, a.rows,
                     a.cols, a.ld, a.d_amax, a.T, a.y, a.ldy);
  return hipGetLastError();
}

template <int FMT, int B>
static hipError_t fq_types(const FakeQuantArgs& a) {
  if (a.f32) return a.bf16_out ? launch_fq<FMT, B, true, true>(a) : launch_fq<FMT, B, true, false>(a);
  return a.bf16_out ? launch_fq<FMT, B, false, true>(a) : launch_fq<FMT, B, false, false>(a);
}

hipError_t run_fake_quant(const FakeQuantArgs& a) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  if (a.fmt == FMT_E8M0) return fq_types<FMT_E8M0, 32>(a);
  if (a.fmt == FMT_UE5M3) return a.block == 16 ? fq_types<FMT_UE5M3, 16>(a) : fq_types<FMT_UE5M3, 32>(a);
  return a.block == 16 ? fq_types<FMT_E4M3, 16>(a) : fq_types<FMT_E4M3, 32>(a);
}

template <int FMT, int B, int LAYOUT, bool BF16>
static hipError_t launch_dq(const DequantArgs& a) {
  const int64_t tiles = ((a.rows + DT - 1) / DT) * ((a.K + DF - 1) / DF);
  hipLaunchKernelGGL((k_dequant<FMT, B, LAYOUT, BF16>), dim3((unsigned)tiles), dim3(NT), 0, a.stream, a.q, a.s, a.g,
                     a.rows, a.K, a.y, a.ldy);
  return hipGetLastError();
}

template <int FMT, int B, int LAYOUT>
static hipError_t dq_out(const DequantArgs& a) {
  return a.bf16_out ? launch_dq<FMT, B, LAYOUT, true>(a) : launch_dq<FMT, B, LAYOUT, false>(a);
}

template <int FMT>
static hipError_t dq_layout(const DequantArgs& a) {
  if (a.layout == 1) return dq_out<FMT, 16, 1>(a);
  if (a.layout == 2) return dq_out<FMT, 16, 2>(a);
  return a.block == 16 ? dq_out<FMT, 16, 0>(a) : dq_out<FMT, 32, 0>(a);
}

hipError_t run_mx_to_fp8(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K, bool transpose, uint8_t* y,
                         uint8_t* s8, hipStream_t stream) {
  if (rows == 0 || K == 0) return hipSuccess;
  using XA = XTile<true>;
  using XB = XTile<false>;
  const int64_t tiles = transpose ? ((rows + XA::T - 1) / XA::T) * ((K + XA::K - 1) / XA::K)
                                  : ((rows + XB::T - 1) / XB::T) * ((K + XB::K - 1) / XB::K);
  if (transpose)
    hipLaunchKernelGGL(k_mx_to_fp8<true>, dim3((unsigned)tiles), dim3(NT), 0, stream, q, s, rows, K, y, s8);
  else
    hipLaunchKernelGGL(k_mx_to_fp8<false>, dim3((unsigned)tiles), dim3(NT), 0, stream, q, s, rows, K, y, s8);
  return hipGetLastError();
}

hipError_t run_dequantize(const DequantArgs& a) {
  if (a.rows == 0 || a.K == 0) return hipSuccess;
  if (a.fmt == FMT_E8M0) return dq_out<FMT_E8M0, 32, 0>(a);
  if (a.fmt == FMT_UE5M3) return dq_layout<FMT_UE5M3>(a);
  return dq_layout<FMT_E4M3>(a);
}

}  // namespace fp4k
