// Shared pieces of the block-scaled FP4 GEMM kernels (gfx950).
//
// Model ("UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach (접근 방법),
// software GEMM model): 64-product groups; each group a float32 partial rounded to nearest
// even; groups added in K order with round-toward-zero; optional 1/1024 canonicalisation.
//
// Tiling: a 256-thread workgroup owns a 128x128 output tile as 2x2 waves of 64x64; each
// wave computes 2x2 MFMA tiles of 32x32. K advances by stages of 256 elements (4 groups,
// 128 payload bytes per row), double-buffered through LDS with register prefetch. LDS
// rows are 128 bytes; 16-byte chunk j of row r is stored at chunk j ^ (r & 7) so that
// eight consecutive rows reading the same chunk hit distinct banks.
#pragma once
#include "fp4_device.hpp"
#include "launch.hpp"

namespace fp4k {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int GT = 128;        // output tile edge per workgroup
constexpr int KS = 256;        // K elements per stage
constexpr int ROWB = KS / 2;   // payload bytes per row per stage
constexpr int GNT = 256;       // threads per workgroup

__device__ __forceinline__ int swz(int row, int chunk) { return row * ROWB + ((chunk ^ (row & 7)) << 4); }

// Prefetch one stage of a 128-row payload tile into registers (4 x 16 bytes per thread).
__device__ __forceinline__ void stage_load(const uint8_t* __restrict__ q, int64_t rows, int64_t K, int64_t row0,
                                           int64_t k0, uint4* reg) {
  const int64_t ldq = K / 2, kb0 = k0 / 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = threadIdx.x + GNT * j;
    const int row = c >> 3, ch = c & 7;
    const int64_t gb = kb0 + ch * 16;
    if (row0 + row < rows && gb < ldq) reg[j] = *reinterpret_cast<const uint4*>(q + (row0 + row) * ldq + gb);
    else reg[j] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void stage_store(uint8_t* lds, const uint4* reg) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = threadIdx.x + GNT * j;
    *reinterpret_cast<uint4*>(lds + swz(c >> 3, c & 7)) = reg[j];
  }
}

// Scale code of (row, K-block blk) for a given layout. blocks_per_row = K / block.
__device__ __forceinline__ uint32_t scale_at(const uint8_t* __restrict__ s, int layout, int64_t row, int64_t blk,
                                             int64_t rows, int64_t blocks_per_row) {
  if (layout == 0) return s[row * blocks_per_row + blk];
  if (layout == 1) return s[(row >> 4) * blocks_per_row + blk];
  return s[blk * (rows >> 4) + (row >> 4)];
}

// Output element (row, col) of register r of a 32x32 MFMA tile in lane l.
__device__ __forceinline__ int tile_row(int r, int l) { return (r >> 2) * 8 + (l >> 5) * 4 + (r & 3); }

// Epilogue: nearest-even mode, optional canonicalisation, scale by alpha, store float32.
__device__ __forceinline__ void store_tiles(float* __restrict__ c, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                            v16f (&acc)[2][2], const float* ga, const float* gb, int canon,
                                            int hadamard_n) {
  mode_f32_rne();
  float a = ga ? *ga : 1.0f;
  float b = gb ? *gb : 1.0f;
  asm volatile("" : "+v"(a), "+v"(b));        // keep the scale product after the mode switch
  float alpha = a * b;
  if (hadamard_n) alpha = alpha * (1.0f / (float)hadamard_n);
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int64_t col = n0 + ct * 32 + (l & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + rt * 32 + tile_row(r, l);
        float v = acc[rt][ct][r];
        if (canon) v = __builtin_rintf(v * 1024.0f) * (1.0f / 1024.0f);
        v = v * alpha;
        if (row < M && col < N) c[row * N + col] = v;
      }
    }
}

}  // namespace fp4k
