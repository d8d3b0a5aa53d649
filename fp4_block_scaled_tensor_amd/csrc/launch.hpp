// Internal launcher interface between the C ABI (capi.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fp4k {

// compute units of the current device (cached per device; 256 on MI355X)
inline int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

struct QuantArgs {
  const void* x;
  bool f32;
  int64_t rows, cols, ld;
  int fmt, block, view, stochastic, hadamard_n;
  float T;
  uint64_t seed, offset;
  const float* d_amax;
  uint8_t* q;
  uint8_t* s;
  uint8_t* qt;
  float* d_g;
  float* d_amax_obs;
  uint32_t* stats;    // optional health counts (FP4_STATS_WORDS words), overwritten
  hipStream_t stream;
};

// words of a health-count output: saturated, zero-scale, non-finite blocks
constexpr int FP4_STATS_WORDS = 3;

struct GemmOperand {
  const uint8_t* q;
  const uint8_t* s;
  const float* g;
  int layout;        // 0: 1D, 1: 2D forward view, 2: 2D transposed view
  int64_t rows;
  int g_shift;       // 0: g is one float; k > 0: g[row >> k] (tile-local scales, stripes of 2^k rows)
};

// Epilogue word passed to the GEMM kernels: bits 0-7 Hadamard n (0, 16, 32), bits 8-15 and
// 16-23 the A and B operands' g_shift.
inline int epilogue_word(int hadamard_n, int a_shift, int b_shift) {
  return hadamard_n | (a_shift << 8) | (b_shift << 16);
}

// Quantization of a GEMM's output as the next GEMM's ROW-view operand, in the epilogue
// ("Format-Aware Fusion for Fast FP4 Pretraining", abstract: the producer writes the
// consumer's layout): blocks of `block` along the output's columns, tensor scales from the
// cached amax, nearest-even or stochastic payload with the logical-index counter.
struct QuantOut {
  int fmt = 0, block = 16, sr = 0;
  float T = 448.0f;
  uint64_t seed = 0, offset = 0;
  const float* amax = nullptr;   // cached amax of the output operand (UE5M3 / E4M3)
  uint8_t* q = nullptr;          // [M x N/2]
  uint8_t* s = nullptr;          // [M x N/block]
  float* g = nullptr;            // optional: the operand's g
  float* amax_obs = nullptr;     // optional: max |C| (zeroed by the launcher)
  uint32_t* stats = nullptr;     // optional: health counts (zeroed by the launcher)
};

struct GemmArgs {
  GemmOperand a, b;
  int fmt, block;
  int64_t M, N, K;
  float* c;          // may be null when qout is set (no float32 output)
  int canon;
  int hadamard_n;
  const QuantOut* qout = nullptr;
  const void* a16 = nullptr;   // UE5M3/E4M3: both operands decoded to fp16 [rows x K] (run_decode_f16)
  const void* b16 = nullptr;
  hipStream_t stream;
};

hipError_t run_quantize(const QuantArgs& a);
// A UE5M3/E4M3 operand [rows x K] decoded to fp16 q S 2^-3 (exact), K-contiguous.
hipError_t run_decode_f16(const GemmOperand& a, int fmt, int block, int64_t K, void* out, hipStream_t stream);

// ROW and COL views of one tensor in one pass (same format and block; per-view amax, T,
// stochastic flag and counter offset; Hadamard on the COL view only).
struct RowColArgs {
  const void* x;
  bool f32;
  int64_t rows, cols, ld;
  int fmt, block;
  int hadamard_n;
  bool sr_r, sr_c;
  const float* amax_r;
  const float* amax_c;
  float T_r, T_c;
  uint64_t seed_r, offset_r, seed_c, offset_c;
  uint8_t *q, *s, *qt, *st;
  float *g_r, *g_c;
  float *obs_r, *obs_c;   // observed amax outputs (max-accumulated; cleared by the caller side)
  uint32_t *stats_r, *stats_c;   // optional health counts of each view, overwritten
  hipStream_t stream;
};
hipError_t run_quantize_rowcol(const RowColArgs& a);

// Quantize then decode (ROW view, nearest-even) into float32 or bfloat16.
struct FakeQuantArgs {
  const void* x;
  bool f32;
  int64_t rows, cols, ld;
  int fmt, block;
  const float* d_amax;
  float T;
  void* y;
  bool bf16_out;
  int64_t ldy;
  hipStream_t stream;
};
hipError_t run_fake_quant(const FakeQuantArgs& a);

// Decode a quantized operand [rows x K] (layout 0: 1D scales, 1: 2D, 2: transposed 2D).
struct DequantArgs {
  const uint8_t* q;
  const uint8_t* s;
  const float* g;
  int fmt, block, layout;
  int64_t rows, K;
  void* y;
  bool bf16_out;
  int64_t ldy;
  hipStream_t stream;
};
hipError_t run_dequantize(const DequantArgs& a);

// ROW-view quantization with one tensor scale per stripe of 2^stripe_log2 rows (current
// scaling from the stripe's own amax).
struct LocalQuantArgs {
  const void* x;
  bool f32;
  int64_t rows, cols, ld;
  int fmt, block, stripe_log2;
  bool stochastic;
  float T;
  uint64_t seed, offset;
  uint8_t* q;
  uint8_t* s;
  float* g;          // [ceil(rows / stripe)]
  float* amax;       // optional, [ceil(rows / stripe)]
  hipStream_t stream;
};
hipError_t run_quantize_local(const LocalQuantArgs& a);

// MXFP4 operand [rows x K] -> E4M3 [rows x K] or [K x rows] plus chunk scales [rows x K/128].
hipError_t run_mx_to_fp8(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K, bool transpose, uint8_t* y,
                         uint8_t* s8, hipStream_t stream);
hipError_t run_amax(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld, int hadamard_n, float* out,
                    hipStream_t stream);
hipError_t run_cache_update(float* amax, int32_t* valid, int32_t D, int64_t step, const float* obs, hipStream_t stream);
hipError_t run_cache_reset(int32_t* valid, hipStream_t stream);
hipError_t run_zero_stats(uint32_t* stats, hipStream_t stream);   // FP4_STATS_WORDS zeros (a kernel)
hipError_t run_scale_range(const uint8_t* s, int64_t n, int32_t* out, hipStream_t stream);   // out[0..1] = min, max
hipError_t run_debug_encode(const float* x, const uint16_t* u16, int64_t n, int which, uint8_t* out,
                            hipStream_t stream);
hipError_t run_gemm_mx(const GemmArgs& g);      // E8M0, block 32
hipError_t run_fill(float* p, float v, int64_t n, hipStream_t stream);   // p[0, n) = v (a kernel, no memset)
hipError_t run_gemm_dec16(const GemmArgs& g);   // UE5M3 / E4M3, block 16 or 32

}  // namespace fp4k
