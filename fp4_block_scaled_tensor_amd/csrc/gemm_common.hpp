// Shared pieces of the block-scaled FP4 GEMM kernels (gfx950).
//
// Model ("UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach (접근 방법),
// software GEMM model): 64-product groups; each group a float32 partial rounded to nearest
// even; groups added in K order with round-toward-zero; optional 1/1024 canonicalisation.
//
// Tiling: a 256-thread workgroup owns a 128x128 output tile as 2x2 waves of 64x64; each
// wave computes 2x2 MFMA tiles of 32x32. K advances by stages of 256 elements (4 groups,
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

namespace fp4k {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int GT = 128;        // output tile edge per workgroup
constexpr int KS = 256;        // K elements per stage
constexpr int SGR = KS / 64;   // groups per stage
constexpr int ROWB = KS / 2;   // payload bytes per row per stage
constexpr int GNT = 256;       // threads per workgroup
constexpr int TILE_BYTES = GT * ROWB;

#ifndef FP4_SWZ_SHIFT
#define FP4_SWZ_SHIFT 1
#endif
// chunk position of logical 16-byte chunk `chunk` in LDS row `row`
__device__ __forceinline__ int swz_pos(int row, int chunk) { return chunk ^ ((row >> FP4_SWZ_SHIFT) & 7); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * ROWB + (swz_pos(row, chunk) << 4); }

// Direct global->LDS loads of one stage of a 128-row payload tile. Each wave fills 4 x 1024
// contiguous LDS bytes; lane i of a 1024-byte piece writes LDS bytes [16i, 16i+16), i.e.
// row 8p + i/8 at chunk position i%8, so it loads the logical chunk stored there. Rows past
// the matrix read a clamped (valid) row; their values only reach outputs that are not
// stored. The per-lane byte offsets (row * K/2 + chunk * 16, below 2^31) are computed once.
struct StageLoader {
  const uint8_t* base;     // q + row0 * K/2, wave-uniform
  uint32_t roff[4];        // per-lane row offsets (row * K/2) of the 4 pieces this wave loads
  uint32_t coff[4];        // per-lane chunk offsets (logical chunk * 16) inside a stage row
  int64_t ldq;

  __device__ __forceinline__ void init(const uint8_t* q, int64_t rows, int64_t K, int64_t row0) {
    ldq = K / 2;
    base = q + row0 * ldq;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = (w * 4 + j) * 8 + (l >> 3);
      const int64_t r = (row0 + row) < rows ? row : (rows - 1 - row0);
      roff[j] = (uint32_t)(r * ldq);
      coff[j] = (uint32_t)(swz_pos(row, l & 7) * 16);   // swz_pos is an involution in `chunk`
    }
  }
  // stage st into lds; only the last stage of a K that is not a multiple of 256 clamps chunks
  __device__ __forceinline__ void issue(int64_t st, uint8_t* lds) const {
    const int w = threadIdx.x >> 6;
    const uint32_t kb0 = (uint32_t)(st * ROWB);
    const bool full = (int64_t)kb0 + ROWB <= ldq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t c = kb0 + coff[j];
      if (!full && c + 16 > (uint32_t)ldq) c = (uint32_t)ldq - 16;
      __builtin_amdgcn_global_load_lds(base + roff[j] + c, (lds_void*)(lds + (w * 4 + j) * 1024), 16, 0, 0);
    }
  }
};

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup id -> (m tile, n tile), XCD-aware grouped order.
__device__ __forceinline__ void tile_coords(int64_t M, int64_t N, int64_t& m0, int64_t& n0) {
  const int64_t ntm = (M + GT - 1) / GT, ntn = (N + GT - 1) / GT;
  const int64_t T = ntm * ntn;
  int64_t id = blockIdx.x;
  if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
  const int64_t GM = 8;
  const int64_t gsize = GM * ntn;
  const int64_t gid = id / gsize;
  const int64_t first = gid * GM;
  const int64_t gm = (ntm - first) < GM ? (ntm - first) : GM;
  const int64_t r = id % gsize;
  m0 = (first + r % gm) * GT;
  n0 = (r / gm) * GT;
}

// Output row of register r of a 32x32 MFMA tile in lane l (column = l & 31).
__device__ __forceinline__ int tile_row(int r, int l) { return (r >> 2) * 8 + (l >> 5) * 4 + (r & 3); }

// Epilogue: nearest-even mode, optional canonicalisation, scale by alpha, store float32.
__device__ __forceinline__ void store_tiles(float* __restrict__ c, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                            v16f (&acc)[2][2], const float* ga, const float* gb, int canon,
                                            int hadamard_n) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(acc[i][j][r]));   // accumulation done before the switch
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
