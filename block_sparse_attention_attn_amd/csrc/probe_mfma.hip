// Diagnostic: the bf16 matrix-core rate this chip sustains, as a practical ceiling to set
// the attention kernel's rate against (the nominal 2516.6 TFLOP/s assumes 2.4 GHz; under
// sustained matrix load the clock settles lower).  Every wave runs four independent
// chains of v_mfma_f32_32x32x16_bf16 on register operands, two waves per SIMD, with no
// memory traffic; the caller times the launch.  Flops per launch:
// grid * kWaves * iters * kChains * 32768.
#include "launchers.h"

namespace sol_attn {
namespace {

constexpr int kThreads = 256;
constexpr int kChains = 4;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(int iters, float* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (threadIdx.x + e));
    b[e] = (__bf16)(0.002f * (e - (int)threadIdx.x % 7));
  }
  f32x16 c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) c[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[k][r];
  if (s == 1234.5f) sink[blockIdx.x] = s;      // keeps the products; never true in practice
}

}  // namespace

hipError_t launch_probe_mfma(int workgroups, int iters, float* sink, hipStream_t stream) {
  mfma_rate_kernel<<<workgroups, kThreads, 0, stream>>>(iters, sink);
  return hipGetLastError();
}

}  // namespace sol_attn
