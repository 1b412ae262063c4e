// Top-k key-block selection by pooled score: the second half of Sol-Attn's
// selection step ("Videomodel MiniMax-H3 rendert sneller dan afspelen", section
// "Waar de snelheidswinst vandaan komt": the attention decides per query which
// parts matter, after a preparation step).
//
// Per (b,h) and query block i:  r_ij = sum_e Qbar_ie * Kbar_je  (float64),
// keep the `topk` largest r_ij with ties to the lower j, write them ascending.
//
// Two implementations share the top-k phase.  For d <= 128 and up to 1280 blocks
// the scores come from float64 matrix-core tiles (see select_mfma_kernel);
// otherwise from the general kernel below.
//
// General kernel: a workgroup (4 waves) owns R consecutive query blocks of one (b,h).
//   1. Qbar rows of the group -> LDS.
//   2. Kbar is streamed through LDS in chunks of 64 key blocks with coalesced
//      16-byte loads (rows padded by one double so that 64 lanes reading the
//      same column of 64 different rows hit distinct banks).  Lane l of a wave
//      owns key block j = chunk + l and forms the dot products of its rows
//      (float64 FMA; wave w takes rows w, w+4, ...), storing an order-preserving
//      64-bit key of r_ij in LDS (and optionally r_ij / sqrt(d)).
//   3. One wave per row finds a threshold T by a bitwise search from the top bit:
//      a candidate threshold is accepted if at least topk keys are >= it; counts
//      come from wave ballots + popcount.  Lane l owns keys j = 64*t + l.  The
//      search stops as soon as exactly topk keys are >= the candidate (those keys
//      are then the top k, with no tie at the boundary), which for real score gaps
//      happens after ~20-30 of the 64 bits; only an exact tie at the k-th place
//      runs all 64 steps, ending at the k-th largest key itself.
//   4. Keys > T are taken, plus the first (topk - #(>T)) keys == T in ascending
//      j.  With interleaved ownership, ascending j is (t, lane) order, so a key's
//      output position is a running count plus the popcount of the ballot bits
//      of lower lanes: the output comes out ascending without a sort or scan.
#include <atomic>

#include "launchers.h"

namespace sol_attn {
namespace {

// Allow a kernel the whole 160 KiB of dynamic LDS, once per device and kernel (the attribute
// is per function and device).  Later launches then make no call besides the launch itself,
// so a stream that is being captured into a graph records only kernel nodes.
__host__ hipError_t allow_full_lds(const void* kernel, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (err == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return err;
}

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxRows = 8;

// key blocks staged per pass: 64 (one per lane) for d <= 128, fewer for larger d
__host__ __device__ constexpr int chunk_for(int d) { return d <= 128 ? 64 : (d <= 256 ? 32 : 16); }

// Order-preserving map float64 -> uint64 (larger r <=> larger key).  -0.0 is
// first turned into +0.0 (x + 0.0) so that the two zeros rank as equal.
__device__ __forceinline__ uint64_t order_key(double r) {
  const uint64_t u = (uint64_t)__double_as_longlong(r + 0.0);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Top-k of rows of order keys held in LDS ([nrows][n_blocks]); one wave per row,
// lane owns key blocks j = 64*t + lane.  Writes `topk` ascending indices per row.
__device__ __forceinline__ void topk_rows(const uint64_t* keys, int n_blocks, int topk, int nrows, int wave,
                                          int lane, int32_t* __restrict__ out_rows) {
  const int per_lane = (n_blocks + 63) / 64;
  for (int r = wave; r < nrows; r += kWaves) {
    const uint64_t* rk = keys + (size_t)r * n_blocks;
    // threshold T with #(key >= T) >= topk whose keys > T plus the first keys == T in
    // ascending j are the top k: either #(key >= T) == topk, or T is the k-th largest
    // key (keys are >= 1)
    uint64_t T = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = T | (1ull << bit);
      int cnt = 0;
      for (int t = 0; t < per_lane; ++t) {
        const int j = 64 * t + lane;
        const bool ge = j < n_blocks && rk[min(j, n_blocks - 1)] >= cand;
        cnt += __popcll(__ballot(ge));
      }
      if (cnt >= topk) T = cand;
      if (cnt == topk) break;       // keys >= T are exactly the top k
    }
    int tot_gt = 0;
    for (int t = 0; t < per_lane; ++t) {
      const int j = 64 * t + lane;
      tot_gt += __popcll(__ballot(j < n_blocks && rk[min(j, n_blocks - 1)] > T));
    }
    const int need_eq = topk - tot_gt;     // keys == T still to take (0 if T is no key)
    int32_t* out = out_rows + (size_t)r * topk;
    int base = 0, eq_seen = 0;
    const uint64_t below = lanes_below(lane);
    for (int t = 0; t < per_lane; ++t) {
      const int j = 64 * t + lane;
      const uint64_t x = j < n_blocks ? rk[j] : 0;
      const bool gt = j < n_blocks && x > T;
      const bool eq = j < n_blocks && x == T;
      const uint64_t eq_mask = __ballot(eq);
      const bool take = gt || (eq && eq_seen + (int)__popcll(eq_mask & below) < need_eq);
      const uint64_t take_mask = __ballot(take);
      if (take) out[base + __popcll(take_mask & below)] = j;
      base += __popcll(take_mask);
      eq_seen += (int)__popcll(eq_mask);
    }
  }
}

// Same as topk_rows, with each lane's keys (at most MAXPL) cached in registers,
// so the 64 bisection steps touch no memory.
template <int MAXPL, int NW>
__device__ __forceinline__ void topk_rows_reg(const uint64_t* keys, int n_blocks, int topk, int nrows,
                                              int wave, int lane, int32_t* __restrict__ out_rows) {
  for (int r = wave; r < nrows; r += NW) {
    const uint64_t* rk = keys + (size_t)r * n_blocks;
    uint64_t x[MAXPL];
#pragma unroll
    for (int t = 0; t < MAXPL; ++t) {
      const int j = 64 * t + lane;
      x[t] = j < n_blocks ? rk[j] : 0;     // 0 ranks below every real key
    }
    uint64_t T = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = T | (1ull << bit);
      int cnt = 0;
#pragma unroll
      for (int t = 0; t < MAXPL; ++t) cnt += __popcll(__ballot(x[t] >= cand));
      if (cnt >= topk) T = cand;
      if (cnt == topk) break;       // keys >= T are exactly the top k
    }
    int tot_gt = 0;
#pragma unroll
    for (int t = 0; t < MAXPL; ++t) tot_gt += __popcll(__ballot(x[t] > T));
    const int need_eq = topk - tot_gt;
    int32_t* out = out_rows + (size_t)r * topk;
    int base = 0, eq_seen = 0;
    const uint64_t below = lanes_below(lane);
#pragma unroll
    for (int t = 0; t < MAXPL; ++t) {
      const int j = 64 * t + lane;
      const bool gt = x[t] > T;
      const bool eq = x[t] == T && j < n_blocks;
      const uint64_t eq_mask = __ballot(eq);
      const bool take = gt || (eq && eq_seen + (int)__popcll(eq_mask & below) < need_eq);
      const uint64_t take_mask = __ballot(take);
      if (take) out[base + __popcll(take_mask & below)] = j;
      base += __popcll(take_mask);
      eq_seen += (int)__popcll(eq_mask);
    }
  }
}

__global__ __launch_bounds__(kThreads) void select_kernel(const double* __restrict__ q_pooled,
                                                          const double* __restrict__ k_pooled,
                                                          int n_blocks, int d, int topk, int rows,
                                                          int32_t* __restrict__ block_idx,
                                                          double* __restrict__ scores,
                                                          double sqrt_d) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int dp = d + 1;                                                    // padded row length
  const int kchunk = chunk_for(d);
  double* qs = reinterpret_cast<double*>(smem);                            // [rows][d]
  double* ks = qs + (size_t)rows * d;                                      // [kchunk][d+1]
  uint64_t* keys = reinterpret_cast<uint64_t*>(ks + (size_t)kchunk * dp);  // [rows][n_blocks]

  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * rows;
  const int nrows = min(rows, n_blocks - i0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const double* qbase = q_pooled + ((size_t)bh * n_blocks + i0) * d;
  const double* kbase = k_pooled + (size_t)bh * n_blocks * d;

  for (int t = tid; t < nrows * d; t += kThreads) qs[t] = qbase[t];

  // --- scores, chunk by chunk of 64 key blocks
  for (int j0 = 0; j0 < n_blocks; j0 += kchunk) {
    const int nk = min(kchunk, n_blocks - j0);
    __syncthreads();   // previous chunk fully consumed (and Qbar visible on the first pass)
    // coalesced copy of Kbar[j0 .. j0+nk) (d doubles each) into the padded LDS rows
    const double* src = kbase + (size_t)j0 * d;
    for (int x = tid; x < nk * d; x += kThreads) {
      const int jj = x / d, e = x - jj * d;
      ks[jj * dp + e] = src[x];
    }
    __syncthreads();
    const int j = j0 + lane;
    if (lane < nk) {
      const double* kr = ks + lane * dp;
      for (int r = wave; r < nrows; r += kWaves) {
        const double* qr = qs + r * d;
        double acc = 0.0;
        for (int e = 0; e < d; ++e) acc = fma(qr[e], kr[e], acc);
        keys[(size_t)r * n_blocks + j] = order_key(acc);
        if (scores) scores[((size_t)bh * n_blocks + i0 + r) * n_blocks + j] = acc / sqrt_d;
      }
    }
  }
  __syncthreads();

  topk_rows(keys, n_blocks, topk, nrows, wave, lane, block_idx + ((size_t)bh * n_blocks + i0) * topk);
}

size_t select_lds_bytes(int rows, int n_blocks, int d) {
  return ((size_t)rows * d + (size_t)chunk_for(d) * (d + 1) + (size_t)rows * n_blocks) * 8;
}

// ---------------------------------------------------------------------------
// Matrix-core path (d <= 128, n_blocks <= 1280): scores of 16 query rows x 16 key
// blocks per v_mfma_f64_16x16x4_f64 chain.  For the 16x16x4 shape lane l supplies
// A[l%16][l/16] and B[l/16][l%16] and receives D[4*r + l/16][l%16] in its
// output register r = 0..3 (layout measured on gfx950).
// The contraction index is permuted, e = (l/16)*S + s for step s (S = ceil(d/4)),
// so every lane reads S contiguous doubles of its own Qbar row (kept in registers)
// and of its key block's Kbar row (coalesced 16-byte loads).  Each score is one
// fixed-order float64 FMA chain, so identical key blocks score identically.
constexpr int kMfmaRows = 16;
constexpr int kMaxMfmaBlocks = 1280;   // 16 rows of keys fill 160 KiB of LDS
constexpr int kMaxS = 32;          // d <= 128
typedef double f64x4 __attribute__((ext_vector_type(4)));

typedef double f64x2 __attribute__((ext_vector_type(2)));

// kS = d / 4 when that is 16 or 32 (d = 64, 128): every contraction index exists, so a
// lane's S doubles of Qbar and Kbar are read with unconditional 16-byte loads (rows
// clamped into range) and the next key tile is prefetched while the current one runs
// through the matrix cores.  kS = 0: any d <= 128, element-wise guarded loads.
// NW waves per workgroup: wave w scores key tiles w, w + NW, ... and then finds the
// top k of rows w, w + NW, ... of the 16.
template <int MAXPL, int kS, int NW>
__global__ __launch_bounds__(NW * 64) void select_mfma_kernel(const double* __restrict__ q_pooled,
                                                               const double* __restrict__ k_pooled,
                                                               int n_blocks, int d, int topk,
                                                               int32_t* __restrict__ block_idx,
                                                               double* __restrict__ scores,
                                                               double sqrt_d) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);       // [16][n_blocks]
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * kMfmaRows;
  const int nrows = min(kMfmaRows, n_blocks - i0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = kS > 0 ? kS : (d + 3) / 4;
  const int col = lane & 15, kk = lane >> 4;
  const int e0 = kk * S;
  const double* kbase = k_pooled + (size_t)bh * n_blocks * d;
  const double* qr = q_pooled + ((size_t)bh * n_blocks + min(i0 + col, n_blocks - 1)) * d + e0;

  // scores r_ij of one 16x16 tile (key blocks j0 .. j0+15) into the LDS key rows
  auto store_tile = [&](const f64x4& c, int j0) {
    const int j = j0 + col;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * r + kk;
      if (i < nrows && j < n_blocks) {
        keys[(size_t)i * n_blocks + j] = order_key(c[r]);
        if (scores) scores[((size_t)bh * n_blocks + i0 + i) * n_blocks + j] = c[r] / sqrt_d;
      }
    }
  };

  if constexpr (kS > 0) {
    constexpr int kV = kS / 2;                       // 16-byte vectors per lane and row
    f64x2 a[kV], b[kV], nb[kV];
#pragma unroll
    for (int t = 0; t < kV; ++t) {
      const f64x2 x = *reinterpret_cast<const f64x2*>(qr + 2 * t);
      a[t] = col < nrows ? x : f64x2{0.0, 0.0};
    }
    auto load_keys = [&](int j0, f64x2 (&dst)[kV]) {
      const double* kr = kbase + (size_t)min(j0 + col, n_blocks - 1) * d + e0;
#pragma unroll
      for (int t = 0; t < kV; ++t) dst[t] = *reinterpret_cast<const f64x2*>(kr + 2 * t);
    };
    int j0 = wave * 16;
    if (j0 < n_blocks) load_keys(j0, nb);
    for (; j0 < n_blocks; j0 += NW * 16) {
#pragma unroll
      for (int t = 0; t < kV; ++t) b[t] = nb[t];
      if (j0 + NW * 16 < n_blocks) load_keys(j0 + NW * 16, nb);
      f64x4 c = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int s = 0; s < kS; ++s) c = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s / 2][s % 2], b[s / 2][s % 2], c, 0, 0, 0);
      store_tile(c, j0);
    }
  } else {
    double a[kMaxS];
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) a[s] = (s < S && e0 + s < d && col < nrows) ? qr[s] : 0.0;
    for (int j0 = wave * 16; j0 < n_blocks; j0 += NW * 16) {
      const int j = j0 + col;
      const double* kr = kbase + (size_t)min(j, n_blocks - 1) * d + e0;
      f64x4 c = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int s = 0; s < kMaxS; ++s) {
        if (s < S) {
          const double bv = (e0 + s < d && j < n_blocks) ? kr[s] : 0.0;
          c = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], bv, c, 0, 0, 0);
        }
      }
      store_tile(c, j0);
    }
  }
  __syncthreads();
  topk_rows_reg<MAXPL, NW>(keys, n_blocks, topk, nrows, wave, lane, block_idx + ((size_t)bh * n_blocks + i0) * topk);
}

template <int kS>
hipError_t launch_select_mfma(const double* q_pooled, const double* k_pooled, int BH, int n_blocks, int d,
                              int topk, int32_t* block_idx, double* scores_or_null, hipStream_t stream) {
  const size_t lds = (size_t)kMfmaRows * n_blocks * 8;
  const int per_lane = (n_blocks + 63) / 64;
  // keys cached per lane in the top-k phase: the smallest instantiation that holds them.
  // Key rows of more than 80 KiB leave room for one workgroup per CU: it then runs 8
  // waves instead of 4 (2 per SIMD), which hides the latencies of both phases (2K:
  // 0.78 -> 0.65 ms); below that two 4-wave workgroups share a CU, which is faster.
  // (per_lane <= 8 means at most 64 KiB, never wide; per_lane > 16 always is)
  const bool wide = lds > 80 * 1024;
  auto kern = per_lane <= 4 ? select_mfma_kernel<4, kS, 4>
            : per_lane <= 8 ? select_mfma_kernel<8, kS, 4>
            : per_lane <= 16 ? (wide ? select_mfma_kernel<16, kS, 8> : select_mfma_kernel<16, kS, 4>)
            : select_mfma_kernel<(kMaxMfmaBlocks + 63) / 64, kS, 8>;
  const int threads = wide ? 8 * 64 : 4 * 64;
  // one flag word per instantiation that can be chosen here
  static std::atomic<uint64_t> done[5];
  const int which = per_lane <= 4 ? 0 : per_lane <= 8 ? 1 : per_lane <= 16 ? (wide ? 2 : 3) : 4;
  hipError_t err = allow_full_lds(reinterpret_cast<const void*>(kern), done[which]);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return err;
  }
  dim3 grid((n_blocks + kMfmaRows - 1) / kMfmaRows, BH);
  hipLaunchKernelGGL(kern, grid, dim3(threads), lds, stream, q_pooled, k_pooled, n_blocks, d, topk, block_idx,
                     scores_or_null, sqrt((double)d));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const double* q_pooled, const double* k_pooled, int BH, int n_blocks, int d,
                         int topk, int32_t* block_idx, double* scores_or_null, hipStream_t stream) {
  (void)hipGetLastError();   // report this launch only, not an earlier unrelated error
  const size_t budget = 160 * 1024;
  if (d <= 4 * kMaxS && n_blocks <= kMaxMfmaBlocks) {
    if (d == 128)
      return launch_select_mfma<32>(q_pooled, k_pooled, BH, n_blocks, d, topk, block_idx, scores_or_null, stream);
    if (d == 64)
      return launch_select_mfma<16>(q_pooled, k_pooled, BH, n_blocks, d, topk, block_idx, scores_or_null, stream);
    return launch_select_mfma<0>(q_pooled, k_pooled, BH, n_blocks, d, topk, block_idx, scores_or_null, stream);
  }
  // general path: rows per workgroup as many as fit (<= 8) in 160 KiB of LDS
  int rows = kMaxRows;
  while (rows > 1 && select_lds_bytes(rows, n_blocks, d) > budget) --rows;
  const size_t lds = select_lds_bytes(rows, n_blocks, d);
  if (lds > budget) return hipErrorInvalidValue;
  dim3 grid((n_blocks + rows - 1) / rows, BH);
  static std::atomic<uint64_t> done{0};
  hipError_t err = allow_full_lds(reinterpret_cast<const void*>(select_kernel), done);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return err;
  }
  hipLaunchKernelGGL(select_kernel, grid, dim3(kThreads), lds, stream, q_pooled, k_pooled, n_blocks,
                     d, topk, rows, block_idx, scores_or_null, sqrt((double)d));
  return hipGetLastError();
}

}  // namespace sol_attn
