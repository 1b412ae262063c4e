// Validation of a block index list before it is handed to the sparse attention.
//
// sol_attn_fwd reads a row of block indices as the key blocks one query block attends
// to; it needs every entry in [0, n_blocks) and the entries of a row strictly
// ascending (distinct, in the order the selection emits them).  This kernel counts
// the rows that break either rule.  One wave per row: lanes read 64 consecutive
// entries (coalesced), compare each with its predecessor (the lane below, or the last
// entry of the previous 64), and a wave-wide vote marks the row.
#include "launchers.h"

namespace sol_attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__global__ void zero_word(int32_t* w) { *w = 0; }

__global__ __launch_bounds__(kThreads) void check_idx_kernel(const int32_t* __restrict__ idx, long long rows,
                                                             int n_blocks, int topk, int32_t* __restrict__ bad_rows) {
  const long long row = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;               // whole waves
  const int32_t* r = idx + row * topk;
  bool bad = false;
  int prev_last = -1;                    // last entry of the previous 64
  for (int t0 = 0; t0 < topk; t0 += 64) {
    const int t = t0 + lane;
    const int x = t < topk ? r[t] : 0;
    int below = __shfl_up(x, 1, 64);
    if (lane == 0) below = prev_last;
    if (t < topk) bad |= x < 0 || x >= n_blocks || x <= below;
    prev_last = __shfl(x, min(63, topk - 1 - t0), 64);
  }
  if (__ballot(bad) != 0 && lane == 0) atomicAdd(bad_rows, 1);
}

}  // namespace

hipError_t launch_check_block_idx(const int32_t* idx, long long rows, int n_blocks, int topk, int32_t* bad_rows,
                                  hipStream_t stream) {
  zero_word<<<1, 1, 0, stream>>>(bad_rows);
  if (rows > 0) {
    const dim3 grid((unsigned)((rows + kWaves - 1) / kWaves));
    check_idx_kernel<<<grid, kThreads, 0, stream>>>(idx, rows, n_blocks, topk, bad_rows);
  }
  return hipGetLastError();
}

}  // namespace sol_attn
