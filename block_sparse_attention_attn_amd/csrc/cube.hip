// Token reordering for 3-D cube blocks.
//
// A video latent is a T x h x w grid of tokens (Sol-H3-VAE model card, section
// "Usage"), stored frame-major: token n = (t*h + y)*w + x.  Cutting that sequence
// into runs of consecutive tokens makes a block a strip of 1.5 latent rows at
// 1344x768; a cube block is instead a bt x by x bx box of latents.  Block-sparse
// attention over cube blocks is block-sparse attention over consecutive blocks of
// the tokens taken in cube-major order (boxes numbered time, row, column; tokens
// frame-major inside a box), because pooling, scoring and softmax only see token
// sets.  This kernel moves token rows between the two orders, so the pool, select
// and attention kernels run unchanged on the reordered tensors.
//
// HBM-bound copy.  In both orders a box is bt*by runs of bx consecutive tokens
// (one latent row segment), so one workgroup moves one box of one (b, h) as bt*by
// contiguous runs of bx*row_bytes bytes.  The box's bytes are cut into units
// (16 bytes when the run length allows), each lane takes every 256th unit and
// issues a batch of loads before their stores, so several accesses per lane are in
// flight.  Bytes per token row: row_bytes read + row_bytes written.
#include "launchers.h"

namespace sol_attn {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;     // loads issued per lane before their stores
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename Unit>
__global__ __launch_bounds__(kThreads) void cube_permute_kernel(const unsigned char* __restrict__ src,
                                                                unsigned char* __restrict__ dst, int T, int h,
                                                                int w, int row_bytes, int bt, int by, int bx,
                                                                int inverse) {
  // blockIdx.x: box (numbered time, row, column), blockIdx.y: (b, h)
  const int nx = w / bx, ny = h / by;
  const int box = blockIdx.x;
  const int xc = box % nx, yc = (box / nx) % ny, tc = box / (nx * ny);
  const size_t head_bytes = (size_t)T * h * w * row_bytes;
  const unsigned char* s_head = src + (size_t)blockIdx.y * head_bytes;
  unsigned char* d_head = dst + (size_t)blockIdx.y * head_bytes;
  // first token of the box in frame-major order (n) and in cube-major order (p)
  const size_t n_box = ((size_t)tc * bt * h + (size_t)yc * by) * w + (size_t)xc * bx;
  const size_t p_box = (size_t)box * bt * by * bx;
  const int run_units = bx * row_bytes / (int)sizeof(Unit);
  const int total = bt * by * run_units;
  for (int g0 = threadIdx.x; g0 < total; g0 += kThreads * kBatch) {
    Unit v[kBatch];
    size_t dst_off[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int g = g0 + j * kThreads;
      if (g < total) {
        const int run = g / run_units, u = g - run * run_units;
        const int tt = run / by, yy = run - tt * by;
        const size_t n0 = n_box + ((size_t)tt * h + yy) * w;     // run start, frame-major
        const size_t p0 = p_box + (size_t)run * bx;              // run start, cube-major
        const size_t s_off = (inverse ? p0 : n0) * row_bytes + (size_t)u * sizeof(Unit);
        dst_off[j] = (inverse ? n0 : p0) * row_bytes + (size_t)u * sizeof(Unit);
        v[j] = __builtin_nontemporal_load(reinterpret_cast<const Unit*>(s_head + s_off));
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (g0 + j * kThreads < total)
        __builtin_nontemporal_store(v[j], reinterpret_cast<Unit*>(d_head + dst_off[j]));
  }
}

}  // namespace

hipError_t launch_cube_permute(const void* src, void* dst, int BH, int T, int h, int w, int row_bytes, int bt,
                               int by, int bx, bool inverse, hipStream_t stream) {
  const int n_boxes = (T / bt) * (h / by) * (w / bx);
  const dim3 grid(n_boxes, BH);
  const auto* s = static_cast<const unsigned char*>(src);
  auto* d = static_cast<unsigned char*>(dst);
  const bool vec = (bx * row_bytes) % 16 == 0 && (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 == 0;
  if (vec)
    cube_permute_kernel<u32x4><<<grid, kThreads, 0, stream>>>(s, d, T, h, w, row_bytes, bt, by, bx, inverse);
  else
    cube_permute_kernel<uint32_t><<<grid, kThreads, 0, stream>>>(s, d, T, h, w, row_bytes, bt, by, bx, inverse);
  return hipGetLastError();
}

}  // namespace sol_attn
