// Block-sparse exact softmax attention, float32 path.
//
// Each query row of block i attends with exact softmax over the tokens of its
// selected key blocks (the attention half of Sol-Attn, "Videomodel MiniMax-H3
// rendert sneller dan afspelen", section "Waar de snelheidswinst vandaan komt").
// This path serves float32 inputs with small head dims; it is plain VALU code:
// one thread per query row, the selected K/V block staged in LDS chunk by chunk
// and read by every thread as a broadcast, an online (running-max) softmax in
// float32 with accurate expf.  A short last block (block does not divide L) has only
// its remaining tokens, as queries and as keys.
#include "launchers.h"

namespace sol_attn {
namespace {

constexpr int kChunk = 32;   // key rows staged per step

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ v,
                                                      const int32_t* __restrict__ block_idx,
                                                      const int32_t* __restrict__ qblock_order, int L,
                                                      int block, int n_blocks, int topk,
                                                      float scale, float* __restrict__ out,
                                                      float* __restrict__ lse) {
  __shared__ float ks[kChunk][D];
  __shared__ float vs[kChunk][D];
  const int i = qblock_order ? min(max(qblock_order[blockIdx.x], 0), n_blocks - 1) : (int)blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const bool active = tid < min(block, L - i * block);
  const size_t head = (size_t)bh * L * D;
  const size_t qrow = head + ((size_t)i * block + (active ? tid : 0)) * D;

  float qv[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = q[qrow + e] * scale;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int32_t* sel = block_idx + ((size_t)bh * n_blocks + i) * topk;
  for (int t = 0; t < topk; ++t) {
    const int j = min(max(sel[t], 0), n_blocks - 1);
    const size_t kbase = head + (size_t)j * block * D;
    const int krows = min(block, L - j * block);
    for (int c0 = 0; c0 < krows; c0 += kChunk) {
      const int nc = min(kChunk, krows - c0);
      __syncthreads();
      for (int x = tid; x < nc * D; x += blockDim.x) {
        ks[x / D][x % D] = k[kbase + (size_t)c0 * D + x];
        vs[x / D][x % D] = v[kbase + (size_t)c0 * D + x];
      }
      __syncthreads();
      for (int r = 0; r < nc; ++r) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) s = fmaf(qv[e], ks[r][e], s);
        if (s > m) {
          const float c = expf(m - s);
          l *= c;
#pragma unroll
          for (int e = 0; e < D; ++e) o[e] *= c;
          m = s;
        }
        const float p = expf(s - m);
        l += p;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] = fmaf(p, vs[r][e], o[e]);
      }
    }
  }
  if (active) {
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < D; ++e) out[qrow + e] = o[e] * inv;
    if (lse) lse[(size_t)bh * L + (size_t)i * block + tid] = m + logf(l);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, int BH, int L, int d,
                          int block, int topk, const int32_t* block_idx, const int32_t* qblock_order,
                          float scale, float* out, float* lse, hipStream_t stream) {
  (void)hipGetLastError();   // report this launch only, not an earlier unrelated error
  const int n_blocks = (L + block - 1) / block;
  dim3 grid(n_blocks, BH);
  const int threads = ((block + 63) / 64) * 64;
  if (d == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(threads), 0, stream, q, k, v, block_idx, qblock_order, L,
                       block, n_blocks, topk, scale, out, lse);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(threads), 0, stream, q, k, v, block_idx, qblock_order, L,
                       block, n_blocks, topk, scale, out, lse);
  return hipGetLastError();
}

}  // namespace sol_attn
