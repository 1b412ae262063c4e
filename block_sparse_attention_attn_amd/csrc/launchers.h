// Kernel launchers behind the C ABI (internal; argument checking happens in sol_attn_api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"

namespace sol_attn {

// 3-D cube blocks read in place: the T x h x w latent grid of a clip, stored
// frame-major (token n = (t*h + y)*w + x), cut into bt x by x bx boxes numbered time,
// row, column; the tokens of a box are taken frame-major, so row r of box c is token
// first_token(c) + row_offset(r).
// Box numbers reach the kernels once per tile, so their divisions go through FastDiv
// (multiply-high and shift) rather than a generic integer division.
struct BoxGeom {
  int w, hw;               // latent columns, tokens per latent frame
  int bt, by, bx;          // box extent in frames, rows, columns
  int nx, ny;              // boxes per latent row, per latent column
  FastDiv div_nx, div_nxy;   // by nx, by nx*ny
  __host__ __device__ int first_token(int c) const {
    const int q1 = (int)div_nx.div((uint32_t)c), tc = (int)div_nxy.div((uint32_t)c);
    const int xc = c - q1 * nx, yc = q1 - tc * ny;
    return tc * bt * hw + yc * by * w + xc * bx;
  }
  __host__ __device__ int row_offset(int r) const {
    const int xx = r % bx, yy = (r / bx) % by, tt = r / (bx * by);
    return tt * hw + yy * w + xx;
  }
};

inline BoxGeom make_box_geom(int h, int w, int bt, int by, int bx) {
  const int nx = w / bx, ny = h / by;
  return BoxGeom{w, h * w, bt, by, bx, nx, ny, FastDiv((uint32_t)nx), FastDiv((uint32_t)(nx * ny))};
}

// Block mean-pooling of q and k.  is_bf16 selects the element type.  cube == NULL: blocks
// of `block` consecutive tokens; else the boxes of *cube (block = box volume, L = T*h*w).
hipError_t launch_pool(const void* q, const void* k, bool is_bf16, int BH, int L, int d, int block,
                       const BoxGeom* cube, double* q_pooled, double* k_pooled, hipStream_t stream);

// Top-k key-block selection by pooled score.
hipError_t launch_select(const double* q_pooled, const double* k_pooled, int BH, int n_blocks, int d,
                         int topk, int32_t* block_idx, double* scores_or_null, hipStream_t stream);

// Sparse attention, bf16 matrix-core path (d == block == 128).  cube as for launch_pool
// (box volume 128).
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, int BH, int L, int topk,
                           const int32_t* block_idx, const int32_t* qblock_order, const BoxGeom* cube,
                           float scale, void* out, float* lse, hipStream_t stream);

// Sparse attention, fp32 path (d in {64,128}, block <= 256).
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, int BH, int L, int d,
                          int block, int topk, const int32_t* block_idx, const int32_t* qblock_order,
                          float scale, float* out, float* lse, hipStream_t stream);

// Token rows between frame-major and cube-major order (3-D cube blocks).
hipError_t launch_cube_permute(const void* src, void* dst, int BH, int T, int h, int w, int row_bytes, int bt,
                               int by, int bx, bool inverse, hipStream_t stream);

// 8-bit exchange formats: one float32 scale per row of d bf16 values.
hipError_t launch_quantize(const void* x, long long rows, int d, bool fp8, void* codes, float* scales,
                           hipStream_t stream);
hipError_t launch_dequantize(const void* codes, const float* scales, long long rows, int d, bool fp8, void* out,
                             hipStream_t stream);

// Count of block-index rows with an entry out of range or not strictly ascending.
hipError_t launch_check_block_idx(const int32_t* idx, long long rows, int n_blocks, int topk, int32_t* bad_rows,
                                  hipStream_t stream);

// Diagnostic matrix-core rate kernel (independent bf16 32x32x16 product chains).
hipError_t launch_probe_mfma(int workgroups, int iters, float* sink, hipStream_t stream);

}  // namespace sol_attn
