// Device helpers shared by the quantizer kernels (quant.hip, fakequant.hip) on gfx950.
#pragma once
#include <atomic>

#include "fp4_device.hpp"
#include "launch.hpp"

namespace fp4k {

constexpr int NT = 256;

// Maximum of two magnitudes with NaN propagation (IEEE 754-2019 maximum, v_maximum3_f32 on
// gfx950, abs folded into its operand modifiers): a NaN anywhere in a block or tensor makes
// its maximum NaN, as the float maximum of the oracle does, so the tensor amax, the stripe
// maxima and the block maxima of every kernel agree on NaN inputs (a maxNum-style max would
// return the other operand and hide the NaN).
__device__ __forceinline__ float mag_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = mag_max(v, __shfl_xor(v, o, 64));
  return v;
}

// The atomic is skipped when the word already holds at least v (a relaxed device-scope read:
// the word only grows, so a stale read can only cause an unneeded atomic). Same-address atomics
// from many workgroups serialise; most workgroups of a large grid now issue none.
__device__ __forceinline__ void atomic_max_nonneg(float* p, float v) {
  unsigned int* w = reinterpret_cast<unsigned int*>(p);
  const unsigned int cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__float_as_uint(v) > cur) atomicMax(w, __float_as_uint(v));
}

// Maximum of each unsigned 16-bit lane of two words (v_pk_max_u16).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b)));
}

// Workgroup max of a non-negative value folded into *out with one atomic (all NT threads call).
__device__ __forceinline__ void wg_max_to(float* out, float v) {
  __shared__ float part[NT / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = part[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) m = mag_max(m, part[i]);
    atomic_max_nonneg(out, m);
  }
}

// g of the operand (1 for E8M0), written once per launch.
template <int FMT>
__device__ __forceinline__ void write_g(float* d_g, const TensorScales& ts) {
  if (d_g && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *d_g = (FMT == FMT_E8M0) ? 1.0f : ts.g;
}

// Load 8 consecutive input elements (bf16 or fp32) as floats.
template <bool F32>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float* v) {
  if constexpr (F32) {
    const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + elem);
    const uint4 b = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + elem + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
  }
}

// Quantizer health counts ("UE5M3 FP4 Block Scaling for Stable Language Model Pretraining",
// key contributions: a stale cached amax is safe while the data grows by less than
// 61440 / T; these counts make that headroom visible per call). Per block:
//   sat     UE5M3/E4M3: the unrounded block scale amax_b * s_blk exceeds the format maximum
//           (the scale saturates); E8M0 has no tensor scale and counts none
//   zero    the block scale encodes to zero and the zero-scale rule replaces it by one
//           (E8M0: a zero block, which takes exponent 0)
//   nonfin  the block maximum is not finite (an Inf or NaN input)
struct Health {
  uint32_t sat = 0, zero = 0, nonfin = 0;
  __device__ __forceinline__ void add_if(bool c, const Health& o) {
    sat += c ? o.sat : 0u;
    zero += c ? o.zero : 0u;
    nonfin += c ? o.nonfin : 0u;
  }
};

// Scale code and payload multiplier of one block with maximum amax_b; adds the block to h.
template <int FMT>
__device__ __forceinline__ void block_scale(float amax_b, const TensorScales& ts, uint32_t& code, float& mult,
                                            Health& h) {
  h.nonfin += (amax_b <= 3.4028234663852886e38f) ? 0u : 1u;
  if constexpr (FMT == FMT_E8M0) {
    code = e8m0_code(amax_b);
    mult = e8m0_inv(code);
    h.zero += (amax_b == 0.0f) ? 1u : 0u;
  } else {
    const float v = amax_b * ts.s_blk;
    code = enc_scale3<FMT>(v);
    h.sat += (v > ScaleFmt<FMT>::MAXV) ? 1u : 0u;
    h.zero += (code == 0) ? 1u : 0u;
    if (code == 0) code = ScaleFmt<FMT>::ONE;          // zero-scale rule
    mult = ts.s_enc / dec_scale3<FMT>(code);           // correctly rounded division
  }
}
template <int FMT>
__device__ __forceinline__ void block_scale(float amax_b, const TensorScales& ts, uint32_t& code, float& mult) {
  Health unused;
  block_scale<FMT>(amax_b, ts, code, mult, unused);
}

// Adds the workgroup's counts to stats[0..2] (sat, zero, nonfin): a wave sum, a workgroup sum
// through LDS, then one atomic per non-zero count. Every thread of the workgroup calls it
// with the same stats pointer; nothing happens when it is null.
__device__ __forceinline__ void health_flush(uint32_t* stats, Health h) {
  if (!stats) return;
  __shared__ uint32_t part[3][NT / 64];
  uint32_t c[3] = {h.sat, h.zero, h.nonfin};
#pragma unroll
  for (int k = 0; k < 3; ++k) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c[k] += __shfl_xor(c[k], o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) part[k][threadIdx.x >> 6] = c[k];
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t += part[threadIdx.x][i];
    if (t) atomicAdd(stats + threadIdx.x, t);
  }
}

// Quantize n (multiple of 8) values with multiplier mult into n/8 dwords of codes.
// SR: logical index of v[0] is i0 (multiple of 8).
template <int N, bool SR>
__device__ __forceinline__ void payload(const float* v, float mult, uint64_t i0, uint64_t seed, uint64_t offset,
                                        uint32_t* words) {
#pragma unroll
  for (int w = 0; w < N / 8; ++w) {
    float r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = v[8 * w + j] * mult;
    if constexpr (SR) {
      uint32_t u[8];
      philox_u16x8((i0 >> 3) + w, seed, offset, u);
      words[w] = e2m1_sr_pack8(r, u);
    } else {
      words[w] = e2m1_pack8(r);
    }
  }
}

// max over groups of G neighbouring lanes (G = 1, 2 or 4; groups aligned to G)
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (G >= 2)
    v = mag_max(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));  // lane ^ 1
  if constexpr (G >= 4)
    v = mag_max(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));  // lane ^ 2
  static_assert(G == 1 || G == 2 || G == 4, "ROW blocks span 1, 2 or 4 lanes");
  return v;
}

// Output stores. Nontemporal (streaming) stores suit kernels whose waves write whole 128-byte
// lines: the written operand is read back by a later kernel, not from this kernel's caches,
// and the hint keeps the write stream from disturbing the read stream (8192 x 4096, inputs
// streamed from HBM: decode 19.9 -> 15.8 us, MXFP4 -> FP8 17.2 -> 13.9, tile-local 22.2 ->
// 19.6, fake quant 24.7 -> 23.8, ROW 18.0 -> 17.5). Kernels whose tiles write parts of lines
// that neighbouring tiles complete must let the L2 merge them and use ordinary stores (with
// the hint the fused ROW+COL pass went 31.5 -> 48.6 us and the 2D weight 43.7 -> 86.4).
constexpr int ST_NT = 2;     // cache-policy bits of a raw buffer store: nt
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ void out_u2(uint8_t* p, uint32_t a, uint32_t b) {
  if (NT) __builtin_nontemporal_store(u32x2_t{a, b}, reinterpret_cast<u32x2_t*>(p));
  else *reinterpret_cast<uint2*>(p) = make_uint2(a, b);
}
template <bool NT>
__device__ __forceinline__ void out_u4(uint8_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  if (NT) __builtin_nontemporal_store(u32x4_t{a, b, c, d}, reinterpret_cast<u32x4_t*>(p));
  else *reinterpret_cast<uint4*>(p) = make_uint4(a, b, c, d);
}
template <bool NT>
__device__ __forceinline__ void out_u8(uint8_t* p, uint8_t v) {
  if (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Raw buffer access: a per-tile resource (base, 0x7FFFFFF0 bytes) and 32-bit lane offsets.
// A lane whose element lies outside the matrix uses offset OOB instead: the hardware's range
// check then returns zeros for its load and drops its store, so every memory instruction is
// issued by every wave (no branches around them, exact wait counts).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
constexpr uint32_t OOB = 0x80000000u;
constexpr int RSRC_RANGE = 0x7FFFFFF0;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, RSRC_RANGE, 0x00020000);
}

// 8 consecutive input elements as loaded (one or two 16-byte words) and as floats
template <bool F32>
struct Chunk8 {
  uint4 w[F32 ? 2 : 1];
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
#pragma unroll
    for (int h = 0; h < (F32 ? 2 : 1); ++h) {
      const v4u t = __builtin_amdgcn_raw_buffer_load_b128(r, off == OOB ? OOB : off + 16u * h, 0, 0);
      w[h] = make_uint4(t[0], t[1], t[2], t[3]);
    }
  }
  __device__ __forceinline__ void to_float(float* v) const {
    if constexpr (F32) {
      v[0] = __uint_as_float(w[0].x); v[1] = __uint_as_float(w[0].y);
      v[2] = __uint_as_float(w[0].z); v[3] = __uint_as_float(w[0].w);
      v[4] = __uint_as_float(w[1].x); v[5] = __uint_as_float(w[1].y);
      v[6] = __uint_as_float(w[1].z); v[7] = __uint_as_float(w[1].w);
    } else {
      v[0] = bf16_lo(w[0].x); v[1] = bf16_hi(w[0].x); v[2] = bf16_lo(w[0].y); v[3] = bf16_hi(w[0].y);
      v[4] = bf16_lo(w[0].z); v[5] = bf16_hi(w[0].z); v[6] = bf16_lo(w[0].w); v[7] = bf16_hi(w[0].w);
    }
  }
};


}  // namespace fp4k
