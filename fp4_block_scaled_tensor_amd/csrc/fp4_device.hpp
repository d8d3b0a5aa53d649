// Device helpers for the block-scaled FP4 kernels on gfx950: scale-format encoders and
// decoders, E2M1 payload rounding, Philox-4x32-10, and the FP32 round-mode switch.
//
// Sources (page title, section):
//  - "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach (접근 방법):
//    E2M1 payload; unsigned E5M3 block scales (max 61,440); nearest-even for activations,
//    weights and block scales; stochastic rounding of dY only; zero block scale -> 1.
//  - "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs", methodology (방법론):
//    MXFP4 = E2M1 payload with a power-of-two scale per 32 elements.
// Bit layouts: UE5M3 eeeeemmm (bias 15, subnormals, exponent 31 unused);
// E4M3 0eeeemmm (bias 7, 0x7F is NaN and never produced); E8M0 2^(code-127).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4k {

enum : int { FMT_UE5M3 = 0, FMT_E4M3 = 1, FMT_E8M0 = 2 };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- block-scale formats with 3 mantissa bits (UE5M3: bias 15, E4M3: bias 7) ----
template <int FMT> struct ScaleFmt;
template <> struct ScaleFmt<FMT_UE5M3> {
  static constexpr int BIAS = 15;
  static constexpr uint32_t MAXCODE = 0xF7;      // 2^15 * 1.875 = 61440
  static constexpr float MAXV = 61440.0f;
  static constexpr uint32_t ONE = 0x78;          // 1.0
  static constexpr float SUB_SCALE = 131072.0f;  // 2^17: subnormal quantum 2^-17
  static constexpr float MIN_NORMAL = 6.103515625e-05f;  // 2^-14
};
template <> struct ScaleFmt<FMT_E4M3> {
  static constexpr int BIAS = 7;
  static constexpr uint32_t MAXCODE = 0x7E;      // 2^8 * 1.75 = 448
  static constexpr float MAXV = 448.0f;
  static constexpr uint32_t ONE = 0x38;
  static constexpr float SUB_SCALE = 512.0f;     // 2^9
  static constexpr float MIN_NORMAL = 0.015625f; // 2^-6
};

// Nearest-even, saturating code of v >= 0 (v may be +inf). Subnormal codes 0..7 continue
// into the first normal code 8, so below the normal range the code is simply
// rint(v / quantum); above it the 23-bit FP32 mantissa is rounded to 3 bits with
// ties-to-even and a carry that propagates into the exponent.
template <int FMT>
__device__ __forceinline__ uint32_t enc_scale3(float v) {
  using S = ScaleFmt<FMT>;
  if (!(v < S::MAXV)) return S::MAXCODE;
  if (v < S::MIN_NORMAL) return (uint32_t)__builtin_rintf(v * S::SUB_SCALE);
  const uint32_t b = __float_as_uint(v);
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  return (r >> 20) - ((uint32_t)(127 - S::BIAS) << 3);
}

template <int FMT>
__device__ __forceinline__ float dec_scale3(uint32_t c) {
  using S = ScaleFmt<FMT>;
  const uint32_t e = c >> 3, m = c & 7u;
  if (e == 0) return (float)m * (1.0f / S::SUB_SCALE);
  return __uint_as_float(((e - S::BIAS + 127u) << 23) | (m << 20));
}

// E8M0 block exponent for a block maximum a >= 0: floor(log2 a) - 2 clamped to [-127, 127],
// 0 for a == 0. Returns the code E + 127.
__device__ __forceinline__ uint32_t e8m0_code(float a) {
  const uint32_t b = __float_as_uint(a);
  if (b == 0) return 127;
  int fl;
  const uint32_t ex = b >> 23;
  if (ex != 0) fl = (int)ex - 127;
  else fl = (31 - __builtin_clz(b)) - 149;      // subnormal maximum
  int E = fl - 2;
  E = E < -127 ? -127 : (E > 127 ? 127 : E);
  return (uint32_t)(E + 127);
}

// 2^-E for the E8M0 code c = E + 127 (exact; 2^-127 is subnormal).
__device__ __forceinline__ float e8m0_inv(uint32_t c) {
  const int negE = 127 - (int)c;                 // -E in [-127, 127]
  if (negE >= -126) return __uint_as_float((uint32_t)(negE + 127) << 23);
  return __uint_as_float(1u << 22);              // 2^-127
}

// ---- E2M1 payload, nearest-even with saturation at 6 ----
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0 converts two floats to two E2M1 codes with
// nearest-even, saturation and the input sign kept (checked against a compare-based
// encoder on all 2^32 float32 inputs). src0 lands in the low nibble of the selected byte.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// 8 floats -> one dword of 8 codes (element 0 in the low nibble)
__device__ __forceinline__ uint32_t e2m1_pack8(const float* r) {
  uint32_t w = 0;
  w = e2m1_pack2<0>(w, r[0], r[1]);
  w = e2m1_pack2<1>(w, r[2], r[3]);
  w = e2m1_pack2<2>(w, r[4], r[5]);
  w = e2m1_pack2<3>(w, r[6], r[7]);
  return w;
}

// ---- stochastic E2M1 ----
// With lo <= |r| < hi the neighbouring codebook values, round up iff u16 < 65536 (|r| - lo) /
// (hi - lo); |r| >= 6 gives 6. Branch-free form: the codebook spacing around |r| is h = 1/2 below
// 2, 1 in [2, 4) and 2 from 4 on, so 2h = min(max(P, 1), 4) with P = 2^floor(log2 |r|) (the
// exponent bits of r alone: 0 for zero and subnormals). t = |r| / h is exact, floor(t) h = lo
// and frac(t) = (|r| - lo) / h. Then floor(t) + up = ceil(t - u16 / 2^16): t - u16 / 2^16 lies in
// (floor(t) - 1, floor(t) + 1) and exceeds floor(t) exactly when u16 < 2^16 frac(t). The fused
// multiply-add rounds once: for t >= 1 the difference is a multiple of t's quantum below 4,
// hence exact; for t < 1 only its sign matters, which rounding keeps.
// Returns twice the selected codebook value, (floor(t) + up) 2h, with the sign of r: the
// encoder below halves it exactly (its scale operand 2.0 divides) and maps it to its own code.
// |r| >= 6 gives 12 or more, which the encoder saturates to 6; so do infinities, and a NaN
// (whose 2h is 4) encodes as 6 with its sign, the same as min(|r|, 6) would give.
__device__ __forceinline__ float e2m1_sr_twice(float r, uint32_t u16) {
  const float h2 = __builtin_amdgcn_fmed3f(__uint_as_float(__float_as_uint(r) & 0x7F800000u), 1.0f, 4.0f);
  const float t = fabsf(r) * __uint_as_float(0x7F800000u - __float_as_uint(h2));   // |r| 2 / h2, exact
  const float v = __builtin_fmaf((float)u16, -1.0f / 65536.0f, t);
  return __builtin_copysignf(__builtin_ceilf(v) * h2, r);
}

// two values from e2m1_sr_twice -> two codes in byte SEL of old (src0 in the low nibble)
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_sr_pack2(uint32_t old, float a2, float b2) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a2, b2, 2.0f, SEL);
}

// 8 values with their 16-bit draws -> one dword of 8 stochastically rounded codes
__device__ __forceinline__ uint32_t e2m1_sr_pack8(const float* r, const uint32_t* u) {
  uint32_t w = 0;
  w = e2m1_sr_pack2<0>(w, e2m1_sr_twice(r[0], u[0]), e2m1_sr_twice(r[1], u[1]));
  w = e2m1_sr_pack2<1>(w, e2m1_sr_twice(r[2], u[2]), e2m1_sr_twice(r[3], u[3]));
  w = e2m1_sr_pack2<2>(w, e2m1_sr_twice(r[4], u[4]), e2m1_sr_twice(r[5], u[5]));
  w = e2m1_sr_pack2<3>(w, e2m1_sr_twice(r[6], u[6]), e2m1_sr_twice(r[7], u[7]));
  return w;
}

// ---- Philox-4x32-10 (Salmon et al., SC'11) ----
struct u4 { uint32_t x, y, z, w; };

// a ^ b ^ k in one v_bitop3_b32 (truth table 0x96); k must be wave-uniform (a scalar
// operand: the Philox key, derived from the seed argument)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

__device__ __forceinline__ u4 philox4x32_10(u4 c, uint32_t k0, uint32_t k1) {
  // the round keys are formed here on the scalar unit: hoisted out of the callers' loops, the
  // twenty of each key schedule would be spilled to vector lanes and read back with v_readlane
  asm volatile("" : "+s"(k0), "+s"(k1));
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c = u4{xor3(hi1, c.y, k0), lo1, xor3(hi0, c.w, k1), lo0};
  }
  return c;
}

// 16-bit draws for the 8 logical elements 8*blk8 .. 8*blk8+7 of an operand: element j
// takes word j>>1, low half for even j.
__device__ __forceinline__ void philox_u16x8(uint64_t blk8, uint64_t seed, uint64_t offset, uint32_t* u) {
  const u4 o = philox4x32_10(u4{(uint32_t)blk8, (uint32_t)(blk8 >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)},
                             (uint32_t)seed, (uint32_t)(seed >> 32));
  u[0] = o.x & 0xFFFFu; u[1] = o.x >> 16;
  u[2] = o.y & 0xFFFFu; u[3] = o.y >> 16;
  u[4] = o.z & 0xFFFFu; u[5] = o.z >> 16;
  u[6] = o.w & 0xFFFFu; u[7] = o.w >> 16;
}

// ---- tensor scales from the cached amax (float32, nearest-even) ----
struct TensorScales { float s_enc, s_blk, g; };

__device__ __forceinline__ TensorScales tensor_scales_from(float A, float T) {
  TensorScales ts{1.0f, 1.0f, 1.0f};
  if (A > 0.0f && A <= 3.4028234663852886e38f) {
    const float se = (6.0f * T) / A;
    if (se <= 3.4028234663852886e38f) {
      ts.s_enc = se;
      ts.s_blk = T / A;
      ts.g = 1.0f / se;
    }
  }
  return ts;
}

__device__ __forceinline__ TensorScales tensor_scales(const float* d_amax, float T) {
  return tensor_scales_from(d_amax ? *d_amax : 0.0f, T);
}

// ---- FP32 round-mode control (MODE register bits [1:0]; [3:2] = f64/f16 stay nearest) ----
// The switch is inline asm; sched_barrier(0) on both sides keeps the scheduler from moving
// any instruction (in particular the ordinary float additions whose rounding it selects)
// across it. The additions themselves stay ordinary C++ so that the compiler inserts the
// wait states an MFMA result needs before a VALU instruction reads it.
__device__ __forceinline__ void mode_f32_rtz() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 3\n\ts_nop 3" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void mode_f32_rne() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0\n\ts_nop 3" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace fp4k
