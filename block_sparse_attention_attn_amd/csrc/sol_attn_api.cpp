// C ABI of the Sol-Attn library: argument checking, dispatch, error reporting.
// Every check runs on the host before any HIP call, so a rejected call enqueues
// nothing and touches no output.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <string>
#include <utility>
#include <vector>

#include "../../include/sol_attn.h"
#include "launchers.h"

namespace {

thread_local std::string g_last_error;

sol_attn_status_t fail(sol_attn_status_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

sol_attn_status_t ok() {
  g_last_error.clear();
  return SOL_ATTN_OK;
}

sol_attn_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SOL_ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

sol_attn_status_t check_common(sol_attn_dtype_t dtype, int B, int H, int L, int d, int block) {
  if (dtype != SOL_ATTN_BF16 && dtype != SOL_ATTN_FP32)
    return fail(SOL_ATTN_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (B < 0 || H < 0 || L < 0) return fail(SOL_ATTN_ERR_SHAPE, "negative size B=%d H=%d L=%d", B, H, L);
  if (d <= 0 || block <= 0) return fail(SOL_ATTN_ERR_SHAPE, "d=%d and block=%d must be positive", d, block);
  if ((long long)B * H > 0x7fffffffLL) return fail(SOL_ATTN_ERR_SHAPE, "B*H too large");
  return SOL_ATTN_OK;
}

}  // namespace

extern "C" {

sol_attn_status_t sol_attn_pool(const void* q, const void* k, sol_attn_dtype_t dtype, int B, int H, int L, int d, int block,
                                double* q_pooled, double* k_pooled, void* stream) {
  sol_attn_status_t st = check_common(dtype, B, H, L, d, block);
  if (st != SOL_ATTN_OK) return st;
  const bool bf16 = dtype == SOL_ATTN_BF16;
  if (d > 512 || d % (bf16 ? 8 : 4) != 0)
    return fail(SOL_ATTN_ERR_UNSUPPORTED, "pool needs d <= 512 and d %% %d == 0 (d=%d)", bf16 ? 8 : 4, d);
  const long long BH = (long long)B * H;
  if (BH * L == 0) return ok();
  if (BH > 65535)
    return fail(SOL_ATTN_ERR_SHAPE, "pool grid too large (B*H must be <= 65535)");
  if (!q || !k || !q_pooled || !k_pooled) return fail(SOL_ATTN_ERR_NULL, "pool: NULL pointer");
  if (!aligned(q, 16) || !aligned(k, 16)) return fail(SOL_ATTN_ERR_ALIGN, "pool: q/k not 16-byte aligned");
  if (!aligned(q_pooled, 8) || !aligned(k_pooled, 8))
    return fail(SOL_ATTN_ERR_ALIGN, "pool: pooled outputs not 8-byte aligned");
  return hip_status(sol_attn::launch_pool(q, k, bf16, (int)BH, L, d, block, nullptr, q_pooled, k_pooled,
                                          static_cast<hipStream_t>(stream)),
                    "pool launch");
}

sol_attn_status_t sol_attn_select(const double* q_pooled, const double* k_pooled, int B, int H, int n_blocks, int d,
                                  int topk, int32_t* block_idx, double* scores_or_null, void* stream) {
  if (B < 0 || H < 0 || n_blocks < 0) return fail(SOL_ATTN_ERR_SHAPE, "negative size");
  if (d <= 0) return fail(SOL_ATTN_ERR_SHAPE, "d=%d must be positive", d);
  if (d > 512) return fail(SOL_ATTN_ERR_UNSUPPORTED, "select needs d <= 512 (d=%d)", d);
  if (n_blocks > 8192) return fail(SOL_ATTN_ERR_UNSUPPORTED, "select needs n_blocks <= 8192");
  const long long BH = (long long)B * H;
  if (BH * n_blocks == 0) return ok();
  if (topk < 1 || topk > n_blocks)
    return fail(SOL_ATTN_ERR_K, "topk=%d outside [1, n_blocks=%d]", topk, n_blocks);
  if (BH > 65535) return fail(SOL_ATTN_ERR_SHAPE, "select grid too large (B*H must be <= 65535)");
  if (!q_pooled || !k_pooled || !block_idx) return fail(SOL_ATTN_ERR_NULL, "select: NULL pointer");
  if (!aligned(q_pooled, 8) || !aligned(k_pooled, 8) || !aligned(block_idx, 4) ||
      (scores_or_null && !aligned(scores_or_null, 8)))
    return fail(SOL_ATTN_ERR_ALIGN, "select: misaligned pointer");
  return hip_status(sol_attn::launch_select(q_pooled, k_pooled, (int)BH, n_blocks, d, topk, block_idx,
                                            scores_or_null, static_cast<hipStream_t>(stream)),
                    "select launch");
}

sol_attn_status_t sol_attn_fwd(const void* q, const void* k, const void* v, sol_attn_dtype_t dtype, int B, int H, int L, int d,
                               int block, int topk, const int32_t* block_idx, const int32_t* qblock_order_or_null,
                               float softmax_scale, void* out, float* lse_or_null, void* stream) {
  sol_attn_status_t st = check_common(dtype, B, H, L, d, block);
  if (st != SOL_ATTN_OK) return st;
  if (std::isinf(softmax_scale) && softmax_scale > 0.f)
    return fail(SOL_ATTN_ERR_SHAPE, "fwd: softmax_scale must be finite");
  const bool bf16 = dtype == SOL_ATTN_BF16;
  if (bf16 && !(d == 128 && block == 128))
    return fail(SOL_ATTN_ERR_UNSUPPORTED, "bf16 fwd needs d == 128 and block == 128 (d=%d block=%d)", d, block);
  if (!bf16 && !((d == 64 || d == 128) && block <= 256))
    return fail(SOL_ATTN_ERR_UNSUPPORTED, "fp32 fwd needs d in {64,128} and block <= 256 (d=%d block=%d)", d,
                block);
  const long long BH = (long long)B * H;
  if (BH * L == 0) return ok();
  const int n_blocks = (int)(((long long)L + block - 1) / block);   // the last block may be short
  if (topk < 1 || topk > n_blocks) return fail(SOL_ATTN_ERR_K, "topk=%d outside [1, n_blocks=%d]", topk, n_blocks);
  if (!bf16 && BH > 65535) return fail(SOL_ATTN_ERR_SHAPE, "fp32 fwd grid too large (B*H must be <= 65535)");
  if (bf16 && (long long)L * d * 2 > 0x7fffffffLL)
    return fail(SOL_ATTN_ERR_UNSUPPORTED, "bf16 fwd needs L*d*2 < 2^31 bytes per head (L=%d)", L);
  if (!q || !k || !v || !block_idx || !out) return fail(SOL_ATTN_ERR_NULL, "fwd: NULL pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(SOL_ATTN_ERR_ALIGN, "fwd: q/k/v/out not 16-byte aligned");
  if (!aligned(block_idx, 4) || (lse_or_null && !aligned(lse_or_null, 4)) ||
      (qblock_order_or_null && !aligned(qblock_order_or_null, 4)))
    return fail(SOL_ATTN_ERR_ALIGN, "fwd: block_idx/qblock_order/lse not 4-byte aligned");
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return hip_status(sol_attn::launch_fwd_bf16(q, k, v, (int)BH, L, topk, block_idx, qblock_order_or_null,
                                                nullptr, scale, out, lse_or_null, s),
                      "fwd bf16 launch");
  return hip_status(sol_attn::launch_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                             static_cast<const float*>(v), (int)BH, L, d, block, topk,
                                             block_idx, qblock_order_or_null, scale, static_cast<float*>(out),
                                             lse_or_null, s),
                    "fwd fp32 launch");
}

sol_attn_status_t sol_attn_cube_permute(const void* src, void* dst, int B, int H, int T, int h, int w, int row_bytes, int bt,
                                        int by, int bx, int inverse, void* stream) {
  if (B < 0 || H < 0 || T < 0 || h < 0 || w < 0)
    return fail(SOL_ATTN_ERR_SHAPE, "cube_permute: negative size B=%d H=%d T=%d h=%d w=%d", B, H, T, h, w);
  if (row_bytes <= 0 || row_bytes % 4 != 0)
    return fail(SOL_ATTN_ERR_SHAPE, "cube_permute: row_bytes=%d must be a positive multiple of 4", row_bytes);
  if (bt < 1 || by < 1 || bx < 1 || T % bt || h % by || w % bx)
    return fail(SOL_ATTN_ERR_SHAPE, "cube_permute: box %dx%dx%d does not tile the %dx%dx%d grid", bt, by, bx, T, h,
                w);
  if (inverse != 0 && inverse != 1) return fail(SOL_ATTN_ERR_SHAPE, "cube_permute: inverse must be 0 or 1");
  const long long BH = (long long)B * H;
  const long long L = (long long)T * h * w;
  if (BH * L == 0) return ok();
  if (BH > 65535) return fail(SOL_ATTN_ERR_SHAPE, "cube_permute grid too large (B*H must be <= 65535)");
  if (L > 0x7fffffffLL || (long long)bt * by * bx * row_bytes > (1LL << 32))
    return fail(SOL_ATTN_ERR_SHAPE, "cube_permute: grid of %lld tokens or box of %lld bytes too large", L,
                (long long)bt * by * bx * row_bytes);
  if (!src || !dst) return fail(SOL_ATTN_ERR_NULL, "cube_permute: NULL pointer");
  if (!aligned(src, 4) || !aligned(dst, 4)) return fail(SOL_ATTN_ERR_ALIGN, "cube_permute: src/dst not 4-byte aligned");
  return hip_status(sol_attn::launch_cube_permute(src, dst, (int)BH, T, h, w, row_bytes, bt, by, bx, inverse == 1,
                                                  static_cast<hipStream_t>(stream)),
                    "cube_permute launch");
}

namespace {

// The latent grid and box of the cube-block calls; on success *L is T*h*w.
sol_attn_status_t check_cube(const char* call, int B, int H, int T, int h, int w, int bt, int by, int bx, long long* L) {
  if (B < 0 || H < 0 || T < 0 || h < 0 || w < 0)
    return fail(SOL_ATTN_ERR_SHAPE, "%s: negative size B=%d H=%d T=%d h=%d w=%d", call, B, H, T, h, w);
  if (bt < 1 || by < 1 || bx < 1 || T % bt || h % by || w % bx)
    return fail(SOL_ATTN_ERR_SHAPE, "%s: box %dx%dx%d does not tile the %dx%dx%d grid", call, bt, by, bx, T, h, w);
  *L = (long long)T * h * w;
  if (*L > 0x7fffffffLL) return fail(SOL_ATTN_ERR_SHAPE, "%s: grid of %lld tokens too large", call, *L);
  if ((long long)B * H > 0x7fffffffLL) return fail(SOL_ATTN_ERR_SHAPE, "%s: B*H too large", call);
  return SOL_ATTN_OK;
}

}  // namespace

sol_attn_status_t sol_attn_pool_cube(const void* q, const void* k, sol_attn_dtype_t dtype, int B, int H, int T, int h, int w, int d, int bt,
                                     int by, int bx, double* q_pooled, double* k_pooled, void* stream) {
  long long L = 0;
  sol_attn_status_t st = check_cube("pool_cube", B, H, T, h, w, bt, by, bx, &L);
  if (st != SOL_ATTN_OK) return st;
  const long long V = (long long)bt * by * bx;
  if (V > 0x7fffffffLL) return fail(SOL_ATTN_ERR_SHAPE, "pool_cube: box of %lld tokens too large", V);
  st = check_common(dtype, B, H, (int)L, d, (int)V);
  if (st != SOL_ATTN_OK) return st;
  const bool bf16 = dtype == SOL_ATTN_BF16;
  if (d > 512 || d % (bf16 ? 8 : 4) != 0)
    return fail(SOL_ATTN_ERR_UNSUPPORTED, "pool_cube needs d <= 512 and d %% %d == 0 (d=%d)", bf16 ? 8 : 4, d);
  const long long BH = (long long)B * H;
  if (BH * L == 0) return ok();
  if (BH > 65535) return fail(SOL_ATTN_ERR_SHAPE, "pool_cube grid too large (B*H must be <= 65535)");
  if (!q || !k || !q_pooled || !k_pooled) return fail(SOL_ATTN_ERR_NULL, "pool_cube: NULL pointer");
  if (!aligned(q, 16) || !aligned(k, 16)) return fail(SOL_ATTN_ERR_ALIGN, "pool_cube: q/k not 16-byte aligned");
  if (!aligned(q_pooled, 8) || !aligned(k_pooled, 8))
    return fail(SOL_ATTN_ERR_ALIGN, "pool_cube: pooled outputs not 8-byte aligned");
  const sol_attn::BoxGeom g = sol_attn::make_box_geom(h, w, bt, by, bx);
  return hip_status(sol_attn::launch_pool(q, k, bf16, (int)BH, (int)L, d, (int)V, &g, q_pooled, k_pooled,
                                          static_cast<hipStream_t>(stream)),
                    "pool_cube launch");
}

sol_attn_status_t sol_attn_fwd_cube(const void* q, const void* k, const void* v, int B, int H, int T, int h, int w, int bt, int by,
                                    int bx, int topk, const int32_t* block_idx, const int32_t* qblock_order_or_null,
                                    float softmax_scale, void* out, float* lse_or_null, void* stream) {
  long long L = 0;
  sol_attn_status_t st = check_cube("fwd_cube", B, H, T, h, w, bt, by, bx, &L);
  if (st != SOL_ATTN_OK) return st;
  if (std::isinf(softmax_scale) && softmax_scale > 0.f)
    return fail(SOL_ATTN_ERR_SHAPE, "fwd_cube: softmax_scale must be finite");
  if ((long long)bt * by * bx != 128)
    return fail(SOL_ATTN_ERR_UNSUPPORTED, "fwd_cube needs boxes of 128 tokens (box %dx%dx%d)", bt, by, bx);
  const long long BH = (long long)B * H;
  if (BH * L == 0) return ok();
  if (L * 128 * 2 > 0x7fffffffLL)
    return fail(SOL_ATTN_ERR_UNSUPPORTED, "fwd_cube needs T*h*w*256 < 2^31 bytes per head (%lld tokens)", L);
  const int n_blocks = (int)(L / 128);
  if (topk < 1 || topk > n_blocks) return fail(SOL_ATTN_ERR_K, "topk=%d outside [1, n_blocks=%d]", topk, n_blocks);
  if (!q || !k || !v || !block_idx || !out) return fail(SOL_ATTN_ERR_NULL, "fwd_cube: NULL pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(SOL_ATTN_ERR_ALIGN, "fwd_cube: q/k/v/out not 16-byte aligned");
  if (!aligned(block_idx, 4) || (lse_or_null && !aligned(lse_or_null, 4)) ||
      (qblock_order_or_null && !aligned(qblock_order_or_null, 4)))
    return fail(SOL_ATTN_ERR_ALIGN, "fwd_cube: block_idx/qblock_order/lse not 4-byte aligned");
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(128.0f);
  const sol_attn::BoxGeom g = sol_attn::make_box_geom(h, w, bt, by, bx);
  return hip_status(sol_attn::launch_fwd_bf16(q, k, v, (int)BH, (int)L, topk, block_idx, qblock_order_or_null, &g,
                                              scale, out, lse_or_null, static_cast<hipStream_t>(stream)),
                    "fwd_cube launch");
}

namespace {

sol_attn_status_t check_quant(const char* call, int B, int H, int L, int d, int format) {
  if (B < 0 || H < 0 || L < 0) return fail(SOL_ATTN_ERR_SHAPE, "%s: negative size B=%d H=%d L=%d", call, B, H, L);
  if (d <= 0) return fail(SOL_ATTN_ERR_SHAPE, "%s: d=%d must be positive", call, d);
  if (format != SOL_ATTN_INT8 && format != SOL_ATTN_FP8_E4M3)
    return fail(SOL_ATTN_ERR_UNSUPPORTED, "%s: unknown format %d", call, format);
  if (d % 8 != 0 || d > 512) return fail(SOL_ATTN_ERR_UNSUPPORTED, "%s needs d %% 8 == 0 and d <= 512 (d=%d)", call, d);
  return SOL_ATTN_OK;
}

}  // namespace

sol_attn_status_t sol_attn_quantize(const void* x, int B, int H, int L, int d, int format, void* codes, float* scales,
                                    void* stream) {
  sol_attn_status_t st = check_quant("quantize", B, H, L, d, format);
  if (st != SOL_ATTN_OK) return st;
  const long long rows = (long long)B * H * L;
  if (rows == 0) return ok();
  if (rows > 0x3fffffffLL * 16) return fail(SOL_ATTN_ERR_SHAPE, "quantize: too many rows");
  if (!x || !codes || !scales) return fail(SOL_ATTN_ERR_NULL, "quantize: NULL pointer");
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(scales, 4))
    return fail(SOL_ATTN_ERR_ALIGN, "quantize: x needs 16-byte, codes 8-byte, scales 4-byte alignment");
  return hip_status(sol_attn::launch_quantize(x, rows, d, format == SOL_ATTN_FP8_E4M3, codes, scales,
                                              static_cast<hipStream_t>(stream)),
                    "quantize launch");
}

sol_attn_status_t sol_attn_dequantize(const void* codes, const float* scales, int B, int H, int L, int d, int format, void* out,
                                      void* stream) {
  sol_attn_status_t st = check_quant("dequantize", B, H, L, d, format);
  if (st != SOL_ATTN_OK) return st;
  const long long rows = (long long)B * H * L;
  if (rows == 0) return ok();
  if (rows > 0x3fffffffLL * 16) return fail(SOL_ATTN_ERR_SHAPE, "dequantize: too many rows");
  if (!codes || !scales || !out) return fail(SOL_ATTN_ERR_NULL, "dequantize: NULL pointer");
  if (!aligned(out, 16) || !aligned(codes, 8) || !aligned(scales, 4))
    return fail(SOL_ATTN_ERR_ALIGN, "dequantize: out needs 16-byte, codes 8-byte, scales 4-byte alignment");
  return hip_status(sol_attn::launch_dequantize(codes, scales, rows, d, format == SOL_ATTN_FP8_E4M3, out,
                                                static_cast<hipStream_t>(stream)),
                    "dequantize launch");
}

sol_attn_status_t sol_attn_check_block_idx(const int32_t* block_idx, int B, int H, int n_blocks, int topk, int32_t* bad_rows,
                                           void* stream) {
  if (B < 0 || H < 0 || n_blocks < 0 || topk < 0)
    return fail(SOL_ATTN_ERR_SHAPE, "check_block_idx: negative size B=%d H=%d n_blocks=%d topk=%d", B, H, n_blocks,
                topk);
  if (!bad_rows) return fail(SOL_ATTN_ERR_NULL, "check_block_idx: NULL bad_rows");
  const long long rows = (long long)B * H * n_blocks;
  if (rows > 0 && topk > 0 && !block_idx) return fail(SOL_ATTN_ERR_NULL, "check_block_idx: NULL block_idx");
  if (!aligned(bad_rows, 4) || (block_idx && !aligned(block_idx, 4)))
    return fail(SOL_ATTN_ERR_ALIGN, "check_block_idx: pointers not 4-byte aligned");
  if (rows / 4 > 0x7fffffffLL) return fail(SOL_ATTN_ERR_SHAPE, "check_block_idx: too many rows");
  return hip_status(sol_attn::launch_check_block_idx(block_idx, topk > 0 ? rows : 0, n_blocks, topk, bad_rows,
                                                     static_cast<hipStream_t>(stream)),
                    "check_block_idx launch");
}

sol_attn_status_t sol_attn_probe_mfma(int workgroups, int iters, float* sink, void* stream) {
  if (workgroups < 1 || iters < 1) return fail(SOL_ATTN_ERR_SHAPE, "probe_mfma: workgroups and iters must be >= 1");
  if (!sink) return fail(SOL_ATTN_ERR_NULL, "probe_mfma: NULL sink");
  if (!aligned(sink, 4)) return fail(SOL_ATTN_ERR_ALIGN, "probe_mfma: sink not 4-byte aligned");
  return hip_status(sol_attn::launch_probe_mfma(workgroups, iters, sink, static_cast<hipStream_t>(stream)),
                    "probe_mfma launch");
}

sol_attn_status_t sol_attn_frame_order(int L, int block, int frame_tokens, int row_tokens, int32_t* order_host) {
  if (block <= 0 || L < 0 || frame_tokens <= 0 || row_tokens <= 0 || row_tokens > frame_tokens)
    return fail(SOL_ATTN_ERR_SHAPE, "frame_order: bad geometry L=%d block=%d frame=%d row=%d", L, block,
                frame_tokens, row_tokens);
  const int nb = (int)(((long long)L + block - 1) / block);
  if (nb > 0 && !order_host) return fail(SOL_ATTN_ERR_NULL, "frame_order: NULL output");
  std::vector<int32_t> idx(nb);
  for (int i = 0; i < nb; ++i) idx[i] = i;
  auto key = [&](int i) {
    const long long tok = (long long)i * block;
    const long long frame = tok / frame_tokens;
    const long long row = (tok % frame_tokens) / row_tokens;
    return std::make_pair(row, frame);
  };
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return key(a) < key(b); });
  for (int i = 0; i < nb; ++i) order_host[i] = idx[i];
  return ok();
}

sol_attn_status_t sol_attn_window_blocks(int n_blocks, int topk, int32_t* idx_host) {
  if (n_blocks < 0) return fail(SOL_ATTN_ERR_SHAPE, "window_blocks: n_blocks=%d < 0", n_blocks);
  if (n_blocks == 0) return ok();
  if (topk < 1 || topk > n_blocks)
    return fail(SOL_ATTN_ERR_K, "window_blocks: topk=%d outside [1, %d]", topk, n_blocks);
  if (!idx_host) return fail(SOL_ATTN_ERR_NULL, "window_blocks: NULL output");
  for (int i = 0; i < n_blocks; ++i) {
    const int start = std::min(std::max(i - (topk - 1) / 2, 0), n_blocks - topk);
    for (int t = 0; t < topk; ++t) idx_host[(size_t)i * topk + t] = start + t;
  }
  return ok();
}

const char* sol_attn_last_error(void) { return g_last_error.c_str(); }

int sol_attn_version(void) { return SOL_ATTN_VERSION; }

}  // extern "C"
