// Block mean-pooling of Q and K: the first half of Sol-Attn's selection step.
//
// Sol-Attn's preparation (the work done before the sparse attention proper) is
// named as separately optimised in "Videomodel MiniMax-H3 rendert sneller dan
// afspelen", section "Waar de snelheidswinst vandaan komt"; here it is the mean
// of every contiguous block of `block` tokens, for Q and for K.  When `block` does not
// divide L the last block holds the remaining tokens and their mean is taken.
//
// With cube blocks a block is a box of the frame-major latent grid and its rows are
// read where they lie (row r of box c at token first_token(c) + row_offset(r)); the
// summation order over the box's rows is the same as over a block of consecutive
// tokens holding them in that order.
//
// HBM-bound: every input byte is read once with 16-byte loads (one row of a
// block is covered by consecutive lanes, so a wave reads whole 256-byte rows),
// widened to float64 and summed in registers; per-thread partial sums are then
// combined through LDS in a fixed order.  Bytes per block: block*d*elem_size in,
// d*8 out.
#include "launchers.h"

namespace sol_attn {
namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool kBf16, bool kCube>
__global__ __launch_bounds__(kThreads) void pool_kernel(const void* __restrict__ q,
                                                        const void* __restrict__ k, int L, int d,
                                                        int block, int n_blocks, BoxGeom geom,
                                                        double* __restrict__ q_pooled,
                                                        double* __restrict__ k_pooled) {
  // blockIdx.x: block i, blockIdx.y: (b,h), blockIdx.z: 0 = Q, 1 = K
  constexpr int kElemPerChunk = kBf16 ? 8 : 4;      // 16 bytes
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const void* src = blockIdx.z == 0 ? q : k;
  double* dst = blockIdx.z == 0 ? q_pooled : k_pooled;

  const int chunks_per_row = d / kElemPerChunk;
  const int groups = kThreads / chunks_per_row;   // >= 1 (d <= 512 for bf16 needs 64 chunks)
  const int tid = threadIdx.x;
  const int c = tid % chunks_per_row;
  const int g = tid / chunks_per_row;

  double acc[kElemPerChunk];
#pragma unroll
  for (int e = 0; e < kElemPerChunk; ++e) acc[e] = 0.0;

  const size_t row0 = (size_t)bh * L + (size_t)(kCube ? geom.first_token(i) : i * block);
  const int rows = kCube ? block : min(block, L - i * block);   // fewer in a short last block
  if (g < groups) {
    const u32x4* base = reinterpret_cast<const u32x4*>(
        static_cast<const char*>(src) + (row0 * d) * (kBf16 ? 2 : 4));
    const int row_chunks = chunks_per_row;
#pragma unroll 4
    for (int r = g; r < rows; r += groups) {
      const int tok = kCube ? geom.row_offset(r) : r;
      const u32x4 x = __builtin_nontemporal_load(base + (size_t)tok * row_chunks + c);
      if constexpr (kBf16) {
        const uint32_t w[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[2 * t] += (double)__uint_as_float(w[t] << 16);
          acc[2 * t + 1] += (double)__uint_as_float(w[t] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] += (double)__uint_as_float(x[t]);
      }
    }
  }

  extern __shared__ double part[];   // [groups][d]
  if (g < groups) {
#pragma unroll
    for (int e = 0; e < kElemPerChunk; ++e) part[g * d + c * kElemPerChunk + e] = acc[e];
  }
  __syncthreads();
  const int ng = groups;
  for (int e = tid; e < d; e += kThreads) {
    double s = 0.0;
    for (int gg = 0; gg < ng; ++gg) s += part[gg * d + e];
    dst[((size_t)bh * n_blocks + i) * d + e] = s / (double)rows;
  }
}

}  // namespace

hipError_t launch_pool(const void* q, const void* k, bool is_bf16, int BH, int L, int d, int block,
                       const BoxGeom* cube, double* q_pooled, double* k_pooled, hipStream_t stream) {
  (void)hipGetLastError();   // report this launch only, not an earlier unrelated error
  const int n_blocks = (L + block - 1) / block;
  const int chunks_per_row = d / (is_bf16 ? 8 : 4);
  const int groups = kThreads / chunks_per_row;
  const size_t lds = (size_t)groups * d * sizeof(double);
  const BoxGeom geom = cube ? *cube : BoxGeom{};
  dim3 grid(n_blocks, BH, 2);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), lds, stream, q, k, L, d, block, n_blocks, geom, q_pooled,
                       k_pooled);
  };
  if (is_bf16)
    cube ? go(pool_kernel<true, true>) : go(pool_kernel<true, false>);
  else
    cube ? go(pool_kernel<false, true>) : go(pool_kernel<false, false>);
  return hipGetLastError();
}

}  // namespace sol_attn
