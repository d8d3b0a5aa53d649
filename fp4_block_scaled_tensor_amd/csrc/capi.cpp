// C ABI of the block-scaled FP4 library: argument validation and dispatch. Every check
// runs before anything is enqueued; errors set a thread-local message.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fp4bs.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

fp4_status fail(fp4_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

fp4_status ok() {
  g_err[0] = '\0';
  return FP4_OK;
}

fp4_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP4_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

fp4_status check_fmt_block(int32_t fmt, int32_t block) {
  if (fmt != FP4_UE5M3 && fmt != FP4_E4M3 && fmt != FP4_E8M0) return fail(FP4_EINVAL, "unknown scale format %d", fmt);
  if (block != 16 && block != 32) return fail(FP4_EUNSUPPORTED, "block must be 16 or 32 (got %d)", block);
  if (fmt == FP4_E8M0 && block != 32) return fail(FP4_EUNSUPPORTED, "E8M0 (MXFP4) scales require block 32");
  return FP4_OK;
}

fp4_status check_cfg(const fp4_quant_cfg* c) {
  if (!c) return fail(FP4_EINVAL, "cfg is NULL");
  fp4_status st = check_fmt_block(c->fmt, c->block);
  if (st != FP4_OK) return st;
  if (c->view < FP4_VIEW_ROW || c->view > FP4_VIEW_TILE2D) return fail(FP4_EINVAL, "unknown view %d", c->view);
  if (c->stochastic != 0 && c->stochastic != 1) return fail(FP4_EINVAL, "stochastic must be 0 or 1");
  if (c->hadamard_n != 0 && c->hadamard_n != 16 && c->hadamard_n != 32)
    return fail(FP4_EINVAL, "hadamard_n must be 0, 16 or 32");
  if (c->hadamard_n != 0 && c->view != FP4_VIEW_COL)
    return fail(FP4_EUNSUPPORTED, "the Hadamard rotation applies to the COL (wgrad) view only");
  if (c->view == FP4_VIEW_TILE2D) {
    if (c->fmt == FP4_E8M0) return fail(FP4_EUNSUPPORTED, "TILE2D needs UE5M3 or E4M3 scales");
    if (c->block != 16) return fail(FP4_EUNSUPPORTED, "TILE2D uses 16x16 tiles (block 16)");
    if (c->stochastic) return fail(FP4_EUNSUPPORTED, "weights are rounded to nearest-even only");
  }
  if (c->fmt != FP4_E8M0 && !(c->T > 0.0f && c->T < 3.0e38f)) return fail(FP4_EINVAL, "T must be positive and finite");
  return FP4_OK;
}

fp4_status check_shape(int64_t rows, int64_t cols, const fp4_quant_cfg* c) {
  if (rows < 0 || cols < 0) return fail(FP4_EINVAL, "negative size");
  if (rows > (int64_t(1) << 40) || cols > (int64_t(1) << 40)) return fail(FP4_EINVAL, "size too large");
  const int B = c->block;
  if (c->view == FP4_VIEW_ROW && cols % B) return fail(FP4_EINVAL, "ROW view: cols %% block != 0");
  if (c->view == FP4_VIEW_COL) {
    if (rows % B) return fail(FP4_EINVAL, "COL view: rows (tokens) %% block != 0");
    if (c->hadamard_n && rows % c->hadamard_n) return fail(FP4_EINVAL, "COL view: rows %% hadamard_n != 0");
    if (cols % 8) return fail(FP4_EINVAL, "COL view: cols must be a multiple of 8");
  }
  if (c->view == FP4_VIEW_TILE2D && (rows % 16 || cols % 16))
    return fail(FP4_EINVAL, "TILE2D: rows and cols must be multiples of 16");
  return FP4_OK;
}

void sizes(int64_t rows, int64_t cols, const fp4_quant_cfg* c, size_t* q, size_t* s, size_t* qt) {
  const int64_t B = c->block;
  *q = (size_t)(rows * cols / 2);
  *qt = 0;
  if (c->view == FP4_VIEW_ROW) *s = (size_t)(rows * (cols / B));
  else if (c->view == FP4_VIEW_COL) *s = (size_t)(cols * (rows / B));
  else {
    *s = (size_t)((rows / 16) * (cols / 16));
    *qt = *q;
  }
}

fp4_status check_operand(const fp4_operand* o, const char* name) {
  if (!o) return fail(FP4_EINVAL, "%s is NULL", name);
  if (o->rows < 0 || o->k < 0) return fail(FP4_EINVAL, "%s: negative size", name);
  if (o->k % 64) return fail(FP4_EINVAL, "%s: K must be a multiple of 64 (got %lld)", name, (long long)o->k);
  fp4_status st = check_fmt_block(o->fmt, o->block);
  if (st != FP4_OK) return st;
  if (o->scale_layout < FP4_SCALES_1D || o->scale_layout > FP4_SCALES_2D_T)
    return fail(FP4_EINVAL, "%s: unknown scale layout", name);
  if (o->scale_layout != FP4_SCALES_1D) {
    if (o->fmt == FP4_E8M0 || o->block != 16) return fail(FP4_EUNSUPPORTED, "%s: 2D scales need UE5M3/E4M3 block 16", name);
    if (o->rows % 16) return fail(FP4_EINVAL, "%s: 2D-scaled operand rows must be a multiple of 16", name);
    if ((o->rows / 16) * (o->k / 16) >= (int64_t(1) << 32))
      return fail(FP4_EUNSUPPORTED, "%s: 2D scale grid of 2^32 codes or more", name);
  }
  if (o->rows > 0 && o->k > 0) {
    if (!o->q || !o->s) return fail(FP4_EINVAL, "%s: NULL payload or scales", name);
    if (!aligned(o->q, 16)) return fail(FP4_EALIGN, "%s: payload not 16-byte aligned", name);
    if (!aligned(o->s, 2)) return fail(FP4_EALIGN, "%s: scales not 2-byte aligned", name);
  }
  if (o->g && !aligned(o->g, 4)) return fail(FP4_EALIGN, "%s: g not 4-byte aligned", name);
  if (o->g_stripe != 0) {
    if (o->g_stripe != 16 && o->g_stripe != 32 && o->g_stripe != 64 && o->g_stripe != 128)
      return fail(FP4_EINVAL, "%s: g_stripe must be 0, 16, 32, 64 or 128", name);
    if (o->fmt == FP4_E8M0 || o->scale_layout != FP4_SCALES_1D)
      return fail(FP4_EUNSUPPORTED, "%s: tile-local g needs UE5M3/E4M3 with 1D scales", name);
    if (o->rows > 0 && !o->g) return fail(FP4_EINVAL, "%s: tile-local g needs the g array", name);
  }
  return FP4_OK;
}

int stripe_shift(int32_t stripe) {
  int k = 0;
  while (stripe > 1) {
    stripe >>= 1;
    ++k;
  }
  return k;
}

// The output operand of a *_q GEMM: a ROW view of C [M x N] (blocks along N).
fp4_status check_qout(const fp4_quant_cfg* cfg, const float* d_amax, uint8_t* q, uint8_t* s, float* d_g,
                      float* d_amax_obs, uint32_t* d_stats, fp4k::QuantOut& qo) {
  fp4_status st;
  if ((st = check_cfg(cfg)) != FP4_OK) return st;
  if (cfg->view != FP4_VIEW_ROW || cfg->hadamard_n != 0)
    return fail(FP4_EUNSUPPORTED, "the quantized GEMM output is a ROW view without rotation");
  if (!q || !s) return fail(FP4_EINVAL, "NULL q or s of the quantized output");
  if (!aligned(q, 16)) return fail(FP4_EALIGN, "output q must be 16-byte aligned");
  if (cfg->fmt != FP4_E8M0 && !d_amax) return fail(FP4_EINVAL, "UE5M3/E4M3 output needs the cached amax d_amax");
  if ((d_amax && !aligned(d_amax, 4)) || (d_g && !aligned(d_g, 4)) || (d_amax_obs && !aligned(d_amax_obs, 4)) ||
      (d_stats && !aligned(d_stats, 4)))
    return fail(FP4_EALIGN, "amax / g / stats pointers must be 4-byte aligned");
  qo.fmt = cfg->fmt;
  qo.block = cfg->block;
  qo.sr = cfg->stochastic;
  qo.T = cfg->T;
  qo.seed = cfg->seed;
  qo.offset = cfg->offset;
  qo.amax = d_amax;
  qo.q = q;
  qo.s = s;
  qo.g = d_g;
  qo.amax_obs = d_amax_obs;
  qo.stats = d_stats;
  return FP4_OK;
}

fp4_status gemm_common(const fp4_operand* a, const fp4_operand* b, float* c, int32_t canon, int32_t hadamard_n,
                       void* stream, const char* what, const fp4k::QuantOut* qout = nullptr,
                       const void* a16 = nullptr, const void* b16 = nullptr) {
  fp4_status st;
  if ((st = check_operand(a, "A")) != FP4_OK) return st;
  if ((st = check_operand(b, "B")) != FP4_OK) return st;
  if (a->k != b->k) return fail(FP4_EINVAL, "%s: operands have different K (%lld vs %lld)", what, (long long)a->k,
                                (long long)b->k);
  if (a->fmt != b->fmt || a->block != b->block) return fail(FP4_EUNSUPPORTED, "%s: operands differ in format/block", what);
  if (canon != 0 && canon != 1) return fail(FP4_EINVAL, "canon must be 0 or 1");
  if (a->rows > 0 && b->rows > 0) {
    if (!c && !qout) return fail(FP4_EINVAL, "%s: output is NULL", what);
    if (c && !aligned(c, 16)) return fail(FP4_EALIGN, "%s: output not 16-byte aligned", what);
  }
  if (qout) {
    if (b->rows % qout->block) return fail(FP4_EINVAL, "%s: N must be a multiple of the output block", what);
    if (a->k == 0) return fail(FP4_EUNSUPPORTED, "%s: K = 0 with a quantized output", what);
  }
  fp4k::GemmArgs g;
  g.a = fp4k::GemmOperand{a->q, a->s, a->g, a->scale_layout, a->rows, a->g_stripe ? stripe_shift(a->g_stripe) : 0};
  g.b = fp4k::GemmOperand{b->q, b->s, b->g, b->scale_layout, b->rows, b->g_stripe ? stripe_shift(b->g_stripe) : 0};
  g.fmt = a->fmt;
  g.block = a->block;
  g.M = a->rows;
  g.N = b->rows;
  g.K = a->k;
  g.c = c;
  g.canon = canon;
  g.hadamard_n = hadamard_n;
  g.qout = qout;
  g.a16 = a16;
  g.b16 = b16;
  g.stream = (hipStream_t)stream;
  if (qout) {
    hipError_t e = hipSuccess;
    if (qout->amax_obs) e = fp4k::run_fill(qout->amax_obs, 0.0f, 1, g.stream);
    if (e == hipSuccess && qout->stats) e = fp4k::run_zero_stats(qout->stats, g.stream);
    if (e != hipSuccess) return hip_status(e, what);
  }
  if (g.M == 0 || g.N == 0) return ok();
  // K = 0: every output is an empty sum, +0 after canonicalisation and the output scale
  const hipError_t e = g.K == 0 ? fp4k::run_fill(c, 0.0f, g.M * g.N, g.stream)
                                : (g.fmt == FP4_E8M0) ? fp4k::run_gemm_mx(g) : fp4k::run_gemm_dec16(g);
  return hip_status(e, what);
}

}  // namespace

extern "C" {

int32_t fp4_abi_version(void) { return FP4BS_ABI_VERSION; }

const char* fp4_last_error(void) { return g_err; }

fp4_status fp4_quantize_sizes(int64_t rows, int64_t cols, const fp4_quant_cfg* cfg, size_t* q_bytes, size_t* s_bytes,
                              size_t* qt_bytes) {
  fp4_status st;
  if ((st = check_cfg(cfg)) != FP4_OK) return st;
  if ((st = check_shape(rows, cols, cfg)) != FP4_OK) return st;
  if (!q_bytes || !s_bytes || !qt_bytes) return fail(FP4_EINVAL, "NULL size output");
  sizes(rows, cols, cfg, q_bytes, s_bytes, qt_bytes);
  return ok();
}

fp4_status fp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                        const fp4_quant_cfg* cfg, const float* d_amax, uint8_t* q, uint8_t* s, uint8_t* q_t,
                        float* d_g, float* d_amax_obs, uint32_t* d_stats, void* stream) {
  fp4_status st;
  if ((st = check_cfg(cfg)) != FP4_OK) return st;
  if ((st = check_shape(rows, cols, cfg)) != FP4_OK) return st;
  if (x_dtype != FP4_IN_BF16 && x_dtype != FP4_IN_FP32) return fail(FP4_EINVAL, "unknown input dtype %d", x_dtype);
  const int64_t esz = x_dtype == FP4_IN_FP32 ? 4 : 2;
  if (ld < cols) return fail(FP4_EINVAL, "ld (%lld) < cols (%lld)", (long long)ld, (long long)cols);
  const bool nonempty = rows > 0 && cols > 0;
  if (nonempty) {
    if (!x || !q || !s) return fail(FP4_EINVAL, "NULL x, q or s");
    if (cfg->view == FP4_VIEW_TILE2D && !q_t) return fail(FP4_EINVAL, "TILE2D requires q_t");
    if (!aligned(x, 16) || !aligned(q, 16) || (q_t && !aligned(q_t, 16)))
      return fail(FP4_EALIGN, "x, q and q_t must be 16-byte aligned");
    if ((ld * esz) % 16) return fail(FP4_EALIGN, "row stride must be a multiple of 16 bytes");
  }
  if (cfg->view != FP4_VIEW_TILE2D && q_t) return fail(FP4_EINVAL, "q_t is only written by TILE2D");
  if (cfg->fmt != FP4_E8M0 && !d_amax) return fail(FP4_EINVAL, "UE5M3/E4M3 need the cached amax d_amax");
  if ((d_amax && !aligned(d_amax, 4)) || (d_g && !aligned(d_g, 4)) || (d_amax_obs && !aligned(d_amax_obs, 4)))
    return fail(FP4_EALIGN, "amax / g pointers must be 4-byte aligned");
  if (d_stats && !aligned(d_stats, 4)) return fail(FP4_EALIGN, "d_stats must be 4-byte aligned");
  fp4k::QuantArgs a;
  a.x = x;
  a.f32 = x_dtype == FP4_IN_FP32;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.fmt = cfg->fmt;
  a.block = cfg->block;
  a.view = cfg->view;
  a.stochastic = cfg->stochastic;
  a.hadamard_n = cfg->hadamard_n;
  a.T = cfg->T;
  a.seed = cfg->seed;
  a.offset = cfg->offset;
  a.d_amax = d_amax;
  a.q = q;
  a.s = s;
  a.qt = q_t;
  a.d_g = d_g;
  a.d_amax_obs = d_amax_obs;
  a.stats = d_stats;
  a.stream = (hipStream_t)stream;
  return hip_status(fp4k::run_quantize(a), "fp4_quantize");
}

fp4_status fp4_quantize_rowcol(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                               const fp4_quant_cfg* cfg_row, const fp4_quant_cfg* cfg_col, const float* d_amax_row,
                               const float* d_amax_col, uint8_t* q, uint8_t* s, float* d_g, float* d_amax_obs_row,
                               uint8_t* q_t, uint8_t* s_t, float* d_g_t, float* d_amax_obs_col,
                               uint32_t* d_stats_row, uint32_t* d_stats_col, void* stream) {
  fp4_status st;
  if ((st = check_cfg(cfg_row)) != FP4_OK) return st;
  if ((st = check_cfg(cfg_col)) != FP4_OK) return st;
  if (cfg_row->view != FP4_VIEW_ROW || cfg_col->view != FP4_VIEW_COL)
    return fail(FP4_EINVAL, "rowcol: cfg_row must be a ROW view and cfg_col a COL view");
  if (cfg_row->fmt != cfg_col->fmt || cfg_row->block != cfg_col->block)
    return fail(FP4_EUNSUPPORTED, "rowcol: both views must use the same format and block");
  if ((st = check_shape(rows, cols, cfg_row)) != FP4_OK) return st;
  if ((st = check_shape(rows, cols, cfg_col)) != FP4_OK) return st;
  if (x_dtype != FP4_IN_BF16 && x_dtype != FP4_IN_FP32) return fail(FP4_EINVAL, "unknown input dtype %d", x_dtype);
  const int64_t esz = x_dtype == FP4_IN_FP32 ? 4 : 2;
  if (ld < cols) return fail(FP4_EINVAL, "ld (%lld) < cols (%lld)", (long long)ld, (long long)cols);
  if (rows > 0 && cols > 0) {
    if (!x || !q || !s || !q_t || !s_t) return fail(FP4_EINVAL, "NULL x, q, s, q_t or s_t");
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(q_t, 16))
      return fail(FP4_EALIGN, "x, q and q_t must be 16-byte aligned");
    if ((ld * esz) % 16) return fail(FP4_EALIGN, "row stride must be a multiple of 16 bytes");
  }
  // 32-bit lane offsets inside a tile (at most 128 token rows, 256 feature rows of x^T)
  if (ld * esz > (int64_t(1) << 24) || rows > (int64_t(1) << 24) || cols > (int64_t(1) << 25))
    return fail(FP4_EUNSUPPORTED, "rowcol: needs ld*elem_size <= 2^24 bytes, rows <= 2^24 and cols <= 2^25");
  if (cfg_row->fmt != FP4_E8M0 && (!d_amax_row || !d_amax_col))
    return fail(FP4_EINVAL, "UE5M3/E4M3 need the cached amax of both views");
  for (const float* p : {(const float*)d_amax_row, (const float*)d_amax_col, (const float*)d_g, (const float*)d_g_t,
                         (const float*)d_amax_obs_row, (const float*)d_amax_obs_col})
    if (p && !aligned(p, 4)) return fail(FP4_EALIGN, "amax / g pointers must be 4-byte aligned");
  if ((d_stats_row && !aligned(d_stats_row, 4)) || (d_stats_col && !aligned(d_stats_col, 4)))
    return fail(FP4_EALIGN, "stats pointers must be 4-byte aligned");
  fp4k::RowColArgs a;
  a.x = x;
  a.f32 = x_dtype == FP4_IN_FP32;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.fmt = cfg_row->fmt;
  a.block = cfg_row->block;
  a.hadamard_n = cfg_col->hadamard_n;
  a.sr_r = cfg_row->stochastic != 0;
  a.sr_c = cfg_col->stochastic != 0;
  a.amax_r = d_amax_row;
  a.amax_c = d_amax_col;
  a.T_r = cfg_row->T;
  a.T_c = cfg_col->T;
  a.seed_r = cfg_row->seed;
  a.offset_r = cfg_row->offset;
  a.seed_c = cfg_col->seed;
  a.offset_c = cfg_col->offset;
  a.q = q;
  a.s = s;
  a.qt = q_t;
  a.st = s_t;
  a.g_r = d_g;
  a.g_c = d_g_t;
  a.obs_r = d_amax_obs_row;
  a.obs_c = d_amax_obs_col;
  a.stats_r = d_stats_row;
  a.stats_c = d_stats_col;
  a.stream = (hipStream_t)stream;
  return hip_status(fp4k::run_quantize_rowcol(a), "fp4_quantize_rowcol");
}

fp4_status fp4_fake_quant(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                          const fp4_quant_cfg* cfg, const float* d_amax, void* y, int32_t y_dtype, int64_t ldy,
                          void* stream) {
  fp4_status st;
  if ((st = check_cfg(cfg)) != FP4_OK) return st;
  if (cfg->view != FP4_VIEW_ROW) return fail(FP4_EUNSUPPORTED, "fake_quant: ROW view only (blocks along cols)");
  if (cfg->stochastic) return fail(FP4_EUNSUPPORTED, "fake_quant: nearest-even only");
  if ((st = check_shape(rows, cols, cfg)) != FP4_OK) return st;
  if (x_dtype != FP4_IN_BF16 && x_dtype != FP4_IN_FP32) return fail(FP4_EINVAL, "unknown input dtype %d", x_dtype);
  if (y_dtype != FP4_IN_BF16 && y_dtype != FP4_IN_FP32) return fail(FP4_EINVAL, "unknown output dtype %d", y_dtype);
  const int64_t esz = x_dtype == FP4_IN_FP32 ? 4 : 2, osz = y_dtype == FP4_IN_FP32 ? 4 : 2;
  if (ld < cols || ldy < cols) return fail(FP4_EINVAL, "ld and ldy must be >= cols");
  if (rows > 0 && cols > 0) {
    if (!x || !y) return fail(FP4_EINVAL, "NULL x or y");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(FP4_EALIGN, "x and y must be 16-byte aligned");
    if ((ld * esz) % 16 || (ldy * osz) % 16) return fail(FP4_EALIGN, "row strides must be multiples of 16 bytes");
    if (ld * esz > (int64_t(1) << 24) || ldy * osz > (int64_t(1) << 24))
      return fail(FP4_EUNSUPPORTED, "fake_quant: row strides above 2^24 bytes");
  }
  if (cfg->fmt != FP4_E8M0 && !d_amax) return fail(FP4_EINVAL, "UE5M3/E4M3 need the cached amax d_amax");
  if (d_amax && !aligned(d_amax, 4)) return fail(FP4_EALIGN, "d_amax must be 4-byte aligned");
  fp4k::FakeQuantArgs a;
  a.x = x;
  a.f32 = x_dtype == FP4_IN_FP32;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.fmt = cfg->fmt;
  a.block = cfg->block;
  a.d_amax = d_amax;
  a.T = cfg->T;
  a.y = y;
  a.bf16_out = y_dtype == FP4_IN_BF16;
  a.ldy = ldy;
  a.stream = (hipStream_t)stream;
  return hip_status(fp4k::run_fake_quant(a), "fp4_fake_quant");
}

fp4_status fp4_dequantize(const fp4_operand* a, void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  fp4_status st;
  if ((st = check_operand(a, "operand")) != FP4_OK) return st;
  if (y_dtype != FP4_IN_BF16 && y_dtype != FP4_IN_FP32) return fail(FP4_EINVAL, "unknown output dtype %d", y_dtype);
  const int64_t osz = y_dtype == FP4_IN_FP32 ? 4 : 2;
  if (ldy < a->k) return fail(FP4_EINVAL, "ldy must be >= k");
  if (a->rows > 0 && a->k > 0) {
    if (!y) return fail(FP4_EINVAL, "NULL y");
    if (!aligned(y, 16)) return fail(FP4_EALIGN, "y must be 16-byte aligned");
    if ((ldy * osz) % 16) return fail(FP4_EALIGN, "ldy * element size must be a multiple of 16 bytes");
    if (ldy * osz > (int64_t(1) << 24) || a->k > (int64_t(1) << 25))
      return fail(FP4_EUNSUPPORTED, "dequantize: row stride above 2^24 bytes or k above 2^25");
  }
  fp4k::DequantArgs d;
  d.q = a->q;
  d.s = a->s;
  d.g = a->g;
  d.fmt = a->fmt;
  d.block = a->block;
  d.layout = a->scale_layout;
  d.rows = a->rows;
  d.K = a->k;
  d.y = y;
  d.bf16_out = y_dtype == FP4_IN_BF16;
  d.ldy = ldy;
  d.stream = (hipStream_t)stream;
  return hip_status(fp4k::run_dequantize(d), "fp4_dequantize");
}

fp4_status fp4_mxfp4_to_fp8(const fp4_operand* a, int32_t transpose, uint8_t* y, uint8_t* s8, void* stream) {
  fp4_status st;
  if ((st = check_operand(a, "operand")) != FP4_OK) return st;
  if (a->fmt != FP4_E8M0 || a->scale_layout != FP4_SCALES_1D)
    return fail(FP4_EUNSUPPORTED, "mxfp4_to_fp8: the operand must be MXFP4 (E8M0, block 32, 1D scales)");
  if (transpose != 0 && transpose != 1) return fail(FP4_EINVAL, "transpose must be 0 or 1");
  if (a->k % 128) return fail(FP4_EINVAL, "mxfp4_to_fp8: k must be a multiple of 128 (got %lld)", (long long)a->k);
  if (transpose && a->rows % 16) return fail(FP4_EINVAL, "mxfp4_to_fp8: transposed output needs rows % 16 == 0");
  if (a->k > (int64_t(1) << 23) || a->rows > (int64_t(1) << 23))
    return fail(FP4_EUNSUPPORTED, "mxfp4_to_fp8: rows and k must be <= 2^23");
  if (a->rows > 0 && a->k > 0) {
    if (!y || !s8) return fail(FP4_EINVAL, "NULL y or s8");
    if (!aligned(y, 16)) return fail(FP4_EALIGN, "y must be 16-byte aligned");
  }
  return hip_status(fp4k::run_mx_to_fp8(a->q, a->s, a->rows, a->k, transpose != 0, y, s8, (hipStream_t)stream),
                    "fp4_mxfp4_to_fp8");
}

fp4_status fp4_quantize_local(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                              const fp4_quant_cfg* cfg, int32_t stripe, uint8_t* q, uint8_t* s, float* d_g,
                              float* d_amax_obs, void* stream) {
  fp4_status st;
  if ((st = check_cfg(cfg)) != FP4_OK) return st;
  if (cfg->view != FP4_VIEW_ROW) return fail(FP4_EUNSUPPORTED, "quantize_local: ROW view only");
  if (cfg->fmt == FP4_E8M0) return fail(FP4_EUNSUPPORTED, "quantize_local: UE5M3 or E4M3 (E8M0 has no tensor scale)");
  if (stripe != 16 && stripe != 32 && stripe != 64 && stripe != 128)
    return fail(FP4_EINVAL, "quantize_local: stripe must be 16, 32, 64 or 128");
  if ((st = check_shape(rows, cols, cfg)) != FP4_OK) return st;
  if (x_dtype != FP4_IN_BF16 && x_dtype != FP4_IN_FP32) return fail(FP4_EINVAL, "unknown input dtype %d", x_dtype);
  const int64_t esz = x_dtype == FP4_IN_FP32 ? 4 : 2;
  if (ld < cols) return fail(FP4_EINVAL, "ld (%lld) < cols (%lld)", (long long)ld, (long long)cols);
  if (rows > 0 && cols > 0) {
    if (!x || !q || !s || !d_g) return fail(FP4_EINVAL, "NULL x, q, s or d_g");
    if (!aligned(x, 16) || !aligned(q, 16)) return fail(FP4_EALIGN, "x and q must be 16-byte aligned");
    if ((ld * esz) % 16) return fail(FP4_EALIGN, "row stride must be a multiple of 16 bytes");
  }
  if ((d_g && !aligned(d_g, 4)) || (d_amax_obs && !aligned(d_amax_obs, 4)))
    return fail(FP4_EALIGN, "g / amax pointers must be 4-byte aligned");
  fp4k::LocalQuantArgs a;
  a.x = x;
  a.f32 = x_dtype == FP4_IN_FP32;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.fmt = cfg->fmt;
  a.block = cfg->block;
  a.stripe_log2 = stripe_shift(stripe);
  a.stochastic = cfg->stochastic != 0;
  a.T = cfg->T;
  a.seed = cfg->seed;
  a.offset = cfg->offset;
  a.q = q;
  a.s = s;
  a.g = d_g;
  a.amax = d_amax_obs;
  a.stream = (hipStream_t)stream;
  return hip_status(fp4k::run_quantize_local(a), "fp4_quantize_local");
}

fp4_status fp4_tensor_amax(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld, int32_t hadamard_n,
                           float* d_amax_out, void* stream) {
  if (x_dtype != FP4_IN_BF16 && x_dtype != FP4_IN_FP32) return fail(FP4_EINVAL, "unknown input dtype %d", x_dtype);
  if (rows < 0 || cols < 0 || ld < cols) return fail(FP4_EINVAL, "bad sizes");
  if (hadamard_n != 0 && hadamard_n != 16 && hadamard_n != 32) return fail(FP4_EINVAL, "hadamard_n must be 0, 16, 32");
  if (hadamard_n && rows % hadamard_n) return fail(FP4_EINVAL, "rows %% hadamard_n != 0");
  if (cols % 8) return fail(FP4_EINVAL, "cols must be a multiple of 8");
  if (!d_amax_out || !aligned(d_amax_out, 4)) return fail(FP4_EINVAL, "d_amax_out must be a 4-byte aligned pointer");
  const int64_t esz = x_dtype == FP4_IN_FP32 ? 4 : 2;
  if (rows > 0 && cols > 0) {
    if (!x || !aligned(x, 16)) return fail(FP4_EALIGN, "x must be non-NULL and 16-byte aligned");
    if ((ld * esz) % 16) return fail(FP4_EALIGN, "row stride must be a multiple of 16 bytes");
  }
  return hip_status(fp4k::run_amax(x, x_dtype == FP4_IN_FP32, rows, cols, ld, hadamard_n, d_amax_out,
                                   (hipStream_t)stream),
                    "fp4_tensor_amax");
}

fp4_status amax_cache_update(const fp4_amax_cache* cache, int64_t step, const float* d_amax_obs, void* stream) {
  if (!cache || !cache->amax || !cache->valid || !d_amax_obs) return fail(FP4_EINVAL, "NULL cache field or amax");
  if (cache->D < 1) return fail(FP4_EINVAL, "cache period D must be >= 1");
  if (step < 0) return fail(FP4_EINVAL, "step must be >= 0");
  return hip_status(fp4k::run_cache_update(cache->amax, cache->valid, cache->D, step, d_amax_obs, (hipStream_t)stream),
                    "amax_cache_update");
}

fp4_status amax_cache_reset(const fp4_amax_cache* cache, void* stream) {
  if (!cache || !cache->valid) return fail(FP4_EINVAL, "NULL cache");
  return hip_status(fp4k::run_cache_reset(cache->valid, (hipStream_t)stream), "amax_cache_reset");
}

fp4_status fp4_scale_range(const fp4_operand* a, int32_t* d_range, void* stream) {
  fp4_status st;
  if ((st = check_operand(a, "operand")) != FP4_OK) return st;
  if (!d_range || !aligned(d_range, 4)) return fail(FP4_EINVAL, "d_range must be a 4-byte aligned device pointer");
  const int64_t n = a->scale_layout == FP4_SCALES_1D ? a->rows * (a->k / a->block) : (a->rows / 16) * (a->k / 16);
  return hip_status(fp4k::run_scale_range(a->s, n, d_range, (hipStream_t)stream), "fp4_scale_range");
}

fp4_status fp4_gemm_check_range(int32_t fmt, const int32_t* range_a, const int32_t* range_b) {
  if (!range_a || !range_b) return fail(FP4_EINVAL, "NULL range");
  if (fmt != FP4_UE5M3 && fmt != FP4_E4M3 && fmt != FP4_E8M0) return fail(FP4_EINVAL, "unknown scale format %d", fmt);
  for (const int32_t* r : {range_a, range_b})
    if (r[0] < 0 || r[1] > 255 || (r[0] > r[1] && !(r[0] == 255 && r[1] == 0)))
      return fail(FP4_EINVAL, "a range is [min code, max code] within [0, 255]");
  if (fmt != FP4_E8M0) return ok();   // UE5M3 / E4M3 partials always lie inside the normal range
  if ((range_a[0] == 255 && range_a[1] == 0) || (range_b[0] == 255 && range_b[1] == 0)) return ok();   // empty
  // E = code - 127; every combined exponent Ea + Eb must lie in [-124, 116]
  const int lo = range_a[0] + range_b[0] - 254, hi = range_a[1] + range_b[1] - 254;
  if (lo < -124 || hi > 116)
    return fail(FP4_ERANGE, "MXFP4 combined block exponents reach [%d, %d], outside the exact range [-124, 116]", lo,
                hi);
  return ok();
}

fp4_status fp4_gemm_fprop(const fp4_operand* x, const fp4_operand* w, float* y, int32_t canon, void* stream) {
  if (x && x->scale_layout != FP4_SCALES_1D) return fail(FP4_EUNSUPPORTED, "fprop: activation needs 1D scales");
  if (w && w->scale_layout == FP4_SCALES_2D_T)
    return fail(FP4_EUNSUPPORTED, "fprop: the weight's transposed (dgrad) view is not the forward operand");
  return gemm_common(x, w, y, canon, 0, stream, "fp4_gemm_fprop");
}

fp4_status fp4_gemm_dgrad(const fp4_operand* dy, const fp4_operand* wt, float* dx, int32_t canon, void* stream) {
  if (dy && dy->scale_layout != FP4_SCALES_1D) return fail(FP4_EUNSUPPORTED, "dgrad: dY needs 1D scales");
  if (wt && wt->scale_layout == FP4_SCALES_2D)
    return fail(FP4_EUNSUPPORTED, "dgrad: pass the weight's transposed payload with FP4_SCALES_2D_T");
  return gemm_common(dy, wt, dx, canon, 0, stream, "fp4_gemm_dgrad");
}

fp4_status fp4_gemm_fprop_q(const fp4_operand* x, const fp4_operand* w, float* y, int32_t canon,
                            const fp4_quant_cfg* out_cfg, const float* d_amax_out, uint8_t* q, uint8_t* s, float* d_g,
                            float* d_amax_obs, uint32_t* d_stats, void* stream) {
  if (x && x->scale_layout != FP4_SCALES_1D) return fail(FP4_EUNSUPPORTED, "fprop: activation needs 1D scales");
  if (w && w->scale_layout == FP4_SCALES_2D_T)
    return fail(FP4_EUNSUPPORTED, "fprop: the weight's transposed (dgrad) view is not the forward operand");
  fp4k::QuantOut qo;
  fp4_status st = check_qout(out_cfg, d_amax_out, q, s, d_g, d_amax_obs, d_stats, qo);
  if (st != FP4_OK) return st;
  return gemm_common(x, w, y, canon, 0, stream, "fp4_gemm_fprop_q", &qo);
}

fp4_status fp4_gemm_dgrad_q(const fp4_operand* dy, const fp4_operand* wt, float* dx, int32_t canon,
                            const fp4_quant_cfg* out_cfg, const float* d_amax_out, uint8_t* q, uint8_t* s, float* d_g,
                            float* d_amax_obs, uint32_t* d_stats, void* stream) {
  if (dy && dy->scale_layout != FP4_SCALES_1D) return fail(FP4_EUNSUPPORTED, "dgrad: dY needs 1D scales");
  if (wt && wt->scale_layout == FP4_SCALES_2D)
    return fail(FP4_EUNSUPPORTED, "dgrad: the weight's forward view is not the dgrad operand");
  fp4k::QuantOut qo;
  fp4_status st = check_qout(out_cfg, d_amax_out, q, s, d_g, d_amax_obs, d_stats, qo);
  if (st != FP4_OK) return st;
  return gemm_common(dy, wt, dx, canon, 0, stream, "fp4_gemm_dgrad_q", &qo);
}

fp4_status fp4_gemm_wgrad(const fp4_operand* dyt, const fp4_operand* xt, float* dw, int32_t hadamard_n, int32_t canon,
                          void* stream) {
  if (hadamard_n != 0 && hadamard_n != 16 && hadamard_n != 32) return fail(FP4_EINVAL, "hadamard_n must be 0, 16, 32");
  if ((dyt && dyt->scale_layout != FP4_SCALES_1D) || (xt && xt->scale_layout != FP4_SCALES_1D))
    return fail(FP4_EUNSUPPORTED, "wgrad: both operands need 1D scales along tokens");
  return gemm_common(dyt, xt, dw, canon, hadamard_n, stream, "fp4_gemm_wgrad");
}

fp4_status fp4_decode_f16(const fp4_operand* a, void* out, void* stream) {
  fp4_status st;
  if ((st = check_operand(a, "operand")) != FP4_OK) return st;
  if (a->fmt == FP4_E8M0) return fail(FP4_EUNSUPPORTED, "decode_f16: UE5M3 / E4M3 operands only (MXFP4 runs natively)");
  if (a->rows > 0 && a->k > 0) {
    if (!out) return fail(FP4_EINVAL, "NULL out");
    if (!aligned(out, 16)) return fail(FP4_EALIGN, "out must be 16-byte aligned");
  }
  fp4k::GemmOperand o{a->q, a->s, a->g, a->scale_layout, a->rows, 0};
  return hip_status(fp4k::run_decode_f16(o, a->fmt, a->block, a->k, out, (hipStream_t)stream), "fp4_decode_f16");
}

fp4_status fp4_gemm_f16(const fp4_operand* a, const void* a16, const fp4_operand* b, const void* b16, float* c,
                        int32_t hadamard_n, int32_t canon, void* stream) {
  if (hadamard_n != 0 && hadamard_n != 16 && hadamard_n != 32) return fail(FP4_EINVAL, "hadamard_n must be 0, 16, 32");
  if ((a && a->fmt == FP4_E8M0) || (b && b->fmt == FP4_E8M0))
    return fail(FP4_EUNSUPPORTED, "gemm_f16: UE5M3 / E4M3 operands only (MXFP4 runs natively)");
  if (a && b && a->rows > 0 && b->rows > 0 && a->k > 0) {
    if (!a16 || !b16) return fail(FP4_EINVAL, "gemm_f16: NULL decoded operand");
    if (!aligned(a16, 16) || !aligned(b16, 16)) return fail(FP4_EALIGN, "gemm_f16: decoded operands must be 16-byte aligned");
  }
  return gemm_common(a, b, c, canon, hadamard_n, stream, "fp4_gemm_f16", nullptr, a16, b16);
}

fp4_status fp4_debug_encode(const float* x, const uint16_t* u16, int64_t n, int32_t which, uint8_t* out, void* stream) {
  if (n < 0 || which < 0 || which > 4) return fail(FP4_EINVAL, "bad n or which");
  if (n > 0 && (!x || !out || (which == 4 && !u16))) return fail(FP4_EINVAL, "NULL input/output");
  return hip_status(fp4k::run_debug_encode(x, u16, n, which, out, (hipStream_t)stream), "fp4_debug_encode");
}

}  // extern "C"
