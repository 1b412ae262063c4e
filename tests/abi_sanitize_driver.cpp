// Host driver for tests/test_host_sanitizers.py: calls every C-ABI entry point with
// arguments its checks must reject (and a few valid host-only calls), built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code.  No call reaches the
// GPU: each returns from argument validation or is a host helper.
#include <cstdio>
#include <cstdint>
#include "sol_attn.h"
static int fails = 0;
#define EXPECT(call, code) do { int r_ = (call); if (r_ != (code)) { printf("FAIL %s -> %d (want %d): %s\n", #call, r_, (code), sol_attn_last_error()); ++fails; } } while (0)
int main() {
  void* F = reinterpret_cast<void*>(0x10000);
  void* M = reinterpret_cast<void*>(0x10002);
  int32_t* I = reinterpret_cast<int32_t*>(0x10000);
  double* D = reinterpret_cast<double*>(0x10000);
  EXPECT(sol_attn_fwd(F, F, F, (sol_attn_dtype_t)7, 1, 1, 256, 128, 128, 1, I, nullptr, 0.f, F, nullptr, nullptr), 4);
  EXPECT(sol_attn_fwd(F, F, F, (sol_attn_dtype_t)0, -1, 1, 256, 128, 128, 1, I, nullptr, 0.f, F, nullptr, nullptr), 2);
  EXPECT(sol_attn_fwd(F, F, F, (sol_attn_dtype_t)0, 1, 1, 256, 128, 128, 3, I, nullptr, 0.f, F, nullptr, nullptr), 3);
  EXPECT(sol_attn_fwd(nullptr, F, F, (sol_attn_dtype_t)0, 1, 1, 256, 128, 128, 1, I, nullptr, 0.f, F, nullptr, nullptr), 1);
  EXPECT(sol_attn_fwd(F, F, M, (sol_attn_dtype_t)0, 1, 1, 256, 128, 128, 1, I, nullptr, 0.f, F, nullptr, nullptr), 5);
  EXPECT(sol_attn_fwd(F, F, F, (sol_attn_dtype_t)0, 1, 1, 9000000, 128, 128, 1, I, nullptr, 0.f, F, nullptr, nullptr), 4);
  EXPECT(sol_attn_fwd(F, F, F, (sol_attn_dtype_t)0, 0, 1, 256, 128, 128, 99, I, nullptr, 0.f, F, nullptr, nullptr), 0);
  EXPECT(sol_attn_pool(F, F, (sol_attn_dtype_t)3, 1, 1, 256, 128, 128, D, D, nullptr), 4);
  EXPECT(sol_attn_pool(F, F, (sol_attn_dtype_t)0, 1, 1, 256, 12, 128, D, D, nullptr), 4);
  EXPECT(sol_attn_pool(F, nullptr, (sol_attn_dtype_t)0, 1, 1, 256, 128, 128, D, D, nullptr), 1);
  EXPECT(sol_attn_select(D, D, 1, 1, 8, 128, 0, I, nullptr, nullptr), 3);
  EXPECT(sol_attn_select(D, D, 1, 1, 8193, 128, 1, I, nullptr, nullptr), 4);
  EXPECT(sol_attn_select(D, D, 1, 1, 0, 128, 0, I, nullptr, nullptr), 0);
  EXPECT(sol_attn_cube_permute(F, F, 1, 1, 4, 16, 16, 256, 3, 8, 8, 0, nullptr), 2);
  EXPECT(sol_attn_cube_permute(F, F, 1, 1, 4, 16, 16, 6, 2, 8, 8, 0, nullptr), 2);
  EXPECT(sol_attn_pool_cube(F, F, (sol_attn_dtype_t)0, 1, 1, 4, 16, 16, 128, 2, 3, 8, D, D, nullptr), 2);
  EXPECT(sol_attn_fwd_cube(F, F, F, 1, 1, 4, 16, 16, 1, 4, 4, 2, I, nullptr, 0.f, F, nullptr, nullptr), 4);
  EXPECT(sol_attn_fwd_cube(F, F, F, 1, 1, 1024, 256, 256, 2, 8, 8, 2, I, nullptr, 0.f, F, nullptr, nullptr), 4);
  EXPECT(sol_attn_quantize(F, 1, 1, 8, 128, 7, F, reinterpret_cast<float*>(F), nullptr), 4);
  EXPECT(sol_attn_check_block_idx(I, -1, 1, 8, 2, I, nullptr), 2);
  EXPECT(sol_attn_probe_mfma(0, 1, reinterpret_cast<float*>(F), nullptr), 2);
  int32_t order[16];
  EXPECT(sol_attn_frame_order(1024, 64, 256, 16, order), 0);
  int32_t win[16 * 4];
  EXPECT(sol_attn_window_blocks(16, 4, win), 0);
  EXPECT(sol_attn_window_blocks(16, 17, win), 3);
  printf("checked, %d failures\n", fails);
  return fails != 0;
}
