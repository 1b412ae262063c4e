// 8-bit exchange formats for the tensors around the sparse attention.
//
// Between GPUs the Sol-H3 runtime sends Q, K and V as INT8 and the attention output
// as FP8, shrinking the exchanged data by about half ("Videomodel MiniMax-H3 rendert
// sneller dan afspelen", section "Waar de snelheidswinst vandaan komt").  Here every
// token row of one head (d values) gets one float32 scale, so a row costs d + 4 bytes
// instead of 2d (51.6 % at d = 128):
//   INT8  inv = 127 / amax, code = round-half-even(x * inv) clamped to [-127, 127]
//   FP8   inv = 448 / amax, code = x * inv rounded to nearest-even OCP E4M3 (|.| <= 448)
// with amax = max |x| over the row, stored scale = amax / 127 (or / 448), and a row of
// zeros giving scale 0 and zero codes.  Decoding is code * scale rounded to bf16.
// All of it is float32 with IEEE rounding, so the codes are reproducible bit for bit.
//
// HBM-bound.  16 lanes own a row: each loads 16-byte chunks (8 bf16), the row maximum
// is a 16-lane butterfly, and each lane writes its 8 codes as one 8-byte store (the
// 16 lanes of a row write its d codes contiguously).  A 16-lane group handles 4 rows
// (64 rows per workgroup, one wave covering 4 consecutive rows per access) and issues
// all their loads before the first reduction, so each lane has 4 accesses in flight.
// Bytes per row: quantise 2d in, d + 4 out; dequantise d + 4 in, 2d out.
#include "launchers.h"

namespace sol_attn {
namespace {

constexpr int kThreads = 256;
constexpr int kRowLanes = 16;
constexpr int kGroups = kThreads / kRowLanes;     // 16-lane groups per workgroup
constexpr int kRowsPerGroup = 4;
constexpr int kRowsPerBlock = kGroups * kRowsPerGroup;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));   // nearest-even
}

// 8 bytes of INT8 codes of 8 scaled values
__device__ __forceinline__ u32x2 int8_codes(const float (&v)[8]) {
  uint32_t w[2] = {0, 0};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = (int)fminf(fmaxf(__builtin_rintf(v[e]), -127.f), 127.f);
    w[e >> 2] |= (uint32_t)(c & 0xff) << (8 * (e & 3));
  }
  return u32x2{w[0], w[1]};
}

// 8 bytes of E4M3 codes of 8 scaled values (hardware conversion, nearest-even)
__device__ __forceinline__ u32x2 fp8_codes(const float (&v)[8]) {
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = fminf(fmaxf(v[4 * h + e], -448.f), 448.f);
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    x = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], x, true);
    w[h] = (uint32_t)x;
  }
  return u32x2{w[0], w[1]};
}

// Row r of the workgroup's 64 is (group, k) with r = 16 k + group: the 64 lanes of a
// wave then cover 4 consecutive rows in each access.
__device__ __forceinline__ long long group_row(int k) {
  return (long long)blockIdx.x * kRowsPerBlock + kGroups * k + threadIdx.x / kRowLanes;
}

// kChunks: 16-byte chunks per lane and row, ceil(d / 8 / 16)
template <bool kFp8, int kChunks>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint16_t* __restrict__ x, long long rows, int d,
                                                            uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x % kRowLanes;
  const int chunks = d / 8;
  u32x4 in[kRowsPerGroup][kChunks];
#pragma unroll
  for (int k = 0; k < kRowsPerGroup; ++k) {
    const long long row = group_row(k);
    const u32x4* src = reinterpret_cast<const u32x4*>(x + row * d);
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = lane + kRowLanes * j;
      in[k][j] = row < rows && c < chunks ? __builtin_nontemporal_load(src + c) : u32x4{0, 0, 0, 0};
    }
  }
  const float qmax = kFp8 ? 448.f : 127.f;
#pragma unroll
  for (int k = 0; k < kRowsPerGroup; ++k) {
    const long long row = group_row(k);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(in[k][j][t])), fabsf(bf16_hi(in[k][j][t]))));
#pragma unroll
    for (int m = kRowLanes / 2; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kRowLanes));
    if (row >= rows) continue;          // the 16 lanes of a row agree, so the butterfly above stays whole
    const float inv = amax > 0.f ? qmax / amax : 0.f;
    if (lane == 0) scales[row] = amax / qmax;
    u32x2* dst = reinterpret_cast<u32x2*>(codes + row * d);
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = lane + kRowLanes * j;
      if (c < chunks) {
        float v[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {     // a row of zeros codes +0 (also for -0.0 inputs)
          v[2 * t] = inv == 0.f ? 0.f : bf16_lo(in[k][j][t]) * inv;
          v[2 * t + 1] = inv == 0.f ? 0.f : bf16_hi(in[k][j][t]) * inv;
        }
        __builtin_nontemporal_store(kFp8 ? fp8_codes(v) : int8_codes(v), dst + c);
      }
    }
  }
}

template <bool kFp8, int kChunks>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint8_t* __restrict__ codes,
                                                              const float* __restrict__ scales, long long rows, int d,
                                                              uint16_t* __restrict__ out) {
  const int lane = threadIdx.x % kRowLanes;
  const int chunks = d / 8;
  u32x2 in[kRowsPerGroup][kChunks];
  float s[kRowsPerGroup];
#pragma unroll
  for (int k = 0; k < kRowsPerGroup; ++k) {
    const long long row = group_row(k);
    const u32x2* src = reinterpret_cast<const u32x2*>(codes + row * d);
    s[k] = row < rows ? scales[row] : 0.f;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = lane + kRowLanes * j;
      in[k][j] = row < rows && c < chunks ? __builtin_nontemporal_load(src + c) : u32x2{0, 0};
    }
  }
#pragma unroll
  for (int k = 0; k < kRowsPerGroup; ++k) {
    const long long row = group_row(k);
    if (row >= rows) continue;
    u32x4* dst = reinterpret_cast<u32x4*>(out + row * d);
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = lane + kRowLanes * j;
      if (c < chunks) {
        const u32x2 w = in[k][j];
        float v[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if constexpr (kFp8) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], true);
            v[4 * h] = lo[0];
            v[4 * h + 1] = lo[1];
            v[4 * h + 2] = hi[0];
            v[4 * h + 3] = hi[1];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * h + e] = (float)(int8_t)(w[h] >> (8 * e));
          }
        }
        u32x4 o;
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = pack_bf16(v[2 * t] * s[k], v[2 * t + 1] * s[k]);
        __builtin_nontemporal_store(o, dst + c);
      }
    }
  }
}

template <bool kFp8, int kChunks>
void quantize_as(const uint16_t* x, long long rows, int d, uint8_t* codes, float* scales, hipStream_t stream) {
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  quantize_kernel<kFp8, kChunks><<<grid, kThreads, 0, stream>>>(x, rows, d, codes, scales);
}

template <bool kFp8, int kChunks>
void dequantize_as(const uint8_t* codes, const float* scales, long long rows, int d, uint16_t* out,
                   hipStream_t stream) {
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  dequantize_kernel<kFp8, kChunks><<<grid, kThreads, 0, stream>>>(codes, scales, rows, d, out);
}

template <bool kFp8>
void quantize_d(const uint16_t* x, long long rows, int d, uint8_t* codes, float* scales, hipStream_t stream) {
  const int per_lane = (d / 8 + kRowLanes - 1) / kRowLanes;
  if (per_lane <= 1) quantize_as<kFp8, 1>(x, rows, d, codes, scales, stream);
  else if (per_lane == 2) quantize_as<kFp8, 2>(x, rows, d, codes, scales, stream);
  else quantize_as<kFp8, 4>(x, rows, d, codes, scales, stream);
}

template <bool kFp8>
void dequantize_d(const uint8_t* codes, const float* scales, long long rows, int d, uint16_t* out,
                  hipStream_t stream) {
  const int per_lane = (d / 8 + kRowLanes - 1) / kRowLanes;
  if (per_lane <= 1) dequantize_as<kFp8, 1>(codes, scales, rows, d, out, stream);
  else if (per_lane == 2) dequantize_as<kFp8, 2>(codes, scales, rows, d, out, stream);
  else dequantize_as<kFp8, 4>(codes, scales, rows, d, out, stream);
}

}  // namespace

hipError_t launch_quantize(const void* x, long long rows, int d, bool fp8, void* codes, float* scales,
                           hipStream_t stream) {
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* cs = static_cast<uint8_t*>(codes);
  if (fp8)
    quantize_d<true>(xs, rows, d, cs, scales, stream);
  else
    quantize_d<false>(xs, rows, d, cs, scales, stream);
  return hipGetLastError();
}

hipError_t launch_dequantize(const void* codes, const float* scales, long long rows, int d, bool fp8, void* out,
                             hipStream_t stream) {
  const auto* cs = static_cast<const uint8_t*>(codes);
  auto* o = static_cast<uint16_t*>(out);
  if (fp8)
    dequantize_d<true>(cs, scales, rows, d, o, stream);
  else
    dequantize_d<false>(cs, scales, rows, d, o, stream);
  return hipGetLastError();
}

}  // namespace sol_attn
