// Top-k key-block selection by pooled score: the second half of Sol-Attn's
// selection step ("Videomodel MiniMax-H3 rendert sneller dan afspelen", section
// "Waar de snelheidswinst vandaan komt": the attention decides per query which
// parts matter, after a preparation step).
//
// Per (b,h) and query block i:  r_ij = sum_e Qbar_ie * Kbar_je  (float64),
// keep the `topk` largest r_ij with ties to the lower j, write them ascending.
//
// Work split: a workgroup owns R consecutive query blocks of one (b,h).
//   1. Qbar rows of the group -> LDS.
//   2. Each thread takes key blocks j = tid, tid+256, ...: streams Kbar_j once
//      and forms the R dot products (float64 FMA), storing an order-preserving
//      64-bit key of r_ij in LDS (and optionally r_ij/sqrt(d)).
//   3. One wave per row finds the k-th largest key T by a 64-step bitwise
//      search: at each step a candidate threshold is accepted if at least topk
//      keys are >= it; counts come from wave ballots + popcount (no shuffles).
//   4. Keys > T are taken, plus the first (topk - #(>T)) keys == T in ascending
//      j; positions come from two wave-wide exclusive scans over lanes that own
//      contiguous ranges of j, so the output is ascending without sorting.
#include "launchers.h"

namespace sol_attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxRows = 8;

// Order-preserving map float64 -> uint64 (larger r <=> larger key).  -0.0 is
// first turned into +0.0 (x + 0.0) so that the two zeros rank as equal.
__device__ __forceinline__ uint64_t order_key(double r) {
  const uint64_t u = (uint64_t)__double_as_longlong(r + 0.0);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ int wave_popcount(bool pred) {
  return __popcll(__ballot(pred));
}

// Exclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_excl_scan(int x, int lane) {
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  return incl - x;
}

__global__ __launch_bounds__(kThreads) void select_kernel(const double* __restrict__ q_pooled,
                                                          const double* __restrict__ k_pooled,
                                                          int n_blocks, int d, int topk, int rows,
                                                          int32_t* __restrict__ block_idx,
                                                          double* __restrict__ scores,
                                                          double sqrt_d) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  double* qs = reinterpret_cast<double*>(smem);                          // [rows][d]
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem + (size_t)rows * d * 8);  // [rows][n_blocks]

  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * rows;
  const int nrows = min(rows, n_blocks - i0);
  const int tid = threadIdx.x;
  const double* qbase = q_pooled + ((size_t)bh * n_blocks + i0) * d;
  const double* kbase = k_pooled + (size_t)bh * n_blocks * d;

  for (int t = tid; t < nrows * d; t += kThreads) qs[t] = qbase[t];
  __syncthreads();

  // --- scores
  for (int j = tid; j < n_blocks; j += kThreads) {
    double acc[kMaxRows];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) acc[r] = 0.0;
    const double* kr = kbase + (size_t)j * d;
    for (int e = 0; e < d; ++e) {
      const double kv = kr[e];
#pragma unroll
      for (int r = 0; r < kMaxRows; ++r)
        if (r < nrows) acc[r] = fma(qs[r * d + e], kv, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) {
      if (r < nrows) {
        keys[(size_t)r * n_blocks + j] = order_key(acc[r]);
        if (scores) scores[((size_t)bh * n_blocks + i0 + r) * n_blocks + j] = acc[r] / sqrt_d;
      }
    }
  }
  __syncthreads();

  // --- top-k per row, one wave per row
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int per_lane = (n_blocks + 63) / 64;      // lane owns j in [lane*per_lane, +per_lane)
  const int j_lo = lane * per_lane;
  const int j_hi = min(n_blocks, j_lo + per_lane);
  for (int r = wave; r < nrows; r += kWaves) {
    const uint64_t* rk = keys + (size_t)r * n_blocks;
    // k-th largest key value: the largest T with #(key >= T) >= topk
    uint64_t T = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = T | (1ull << bit);
      int cnt = 0;
      for (int t = 0; t < per_lane; ++t) {
        const int j = j_lo + t;
        const uint64_t x = rk[min(j, n_blocks - 1)];
        cnt += wave_popcount(j < j_hi && x >= cand);
      }
      if (cnt >= topk) T = cand;
    }
    int n_gt = 0, n_eq = 0;
    for (int j = j_lo; j < j_hi; ++j) {
      const uint64_t x = rk[j];
      n_gt += x > T;
      n_eq += x == T;
    }
    // total keys > T across the wave
    int tot_gt = n_gt;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tot_gt += __shfl_xor(tot_gt, off, 64);
    const int need_eq = topk - tot_gt;               // >= 1 by the choice of T
    int eq_before = wave_excl_scan(n_eq, lane);
    // selected count per lane
    int n_sel = n_gt + max(0, min(n_eq, need_eq - eq_before));
    int pos = wave_excl_scan(n_sel, lane);
    int32_t* out = block_idx + ((size_t)bh * n_blocks + i0 + r) * topk;
    for (int j = j_lo; j < j_hi; ++j) {
      const uint64_t x = rk[j];
      bool take = x > T;
      if (x == T) {
        take = eq_before < need_eq;
        ++eq_before;
      }
      if (take) out[pos++] = j;
    }
  }
}

}  // namespace

hipError_t launch_select(const double* q_pooled, const double* k_pooled, int BH, int n_blocks, int d,
                         int topk, int32_t* block_idx, double* scores_or_null, hipStream_t stream) {
  // rows per workgroup: as many as fit (<= 8) with the key rows in <= 128 KiB of LDS
  const size_t budget = 128 * 1024;
  int rows = kMaxRows;
  while (rows > 1 && (size_t)rows * (n_blocks + d) * 8 > budget) --rows;
  const size_t lds = (size_t)rows * (n_blocks + d) * 8;
  dim3 grid((n_blocks + rows - 1) / rows, BH);
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(select_kernel, grid, dim3(kThreads), lds, stream, q_pooled, k_pooled, n_blocks,
                     d, topk, rows, block_idx, scores_or_null, sqrt((double)d));
  return hipGetLastError();
}

}  // namespace sol_attn
