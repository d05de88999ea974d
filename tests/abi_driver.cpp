// Host-side driver of the C ABI for the sanitizer build (ASan + UBSan on the
// host code only; the GPU code is built as usual).  It walks the argument
// checks of every entry point, the host-only split-KV planner over a sweep of
// shapes (including sizes near the int32 limits), the workspace-size queries
// and the status strings.  With no GPU visible it also checks that each entry
// point that reaches the device reports KLEIN_ERR_NO_DEVICE.  It never hands
// a real device a pointer: the "tensor" pointers below are fake, and every
// call that gets past the checks is made only when no device exists.
//
// Exit status 0 when every check holds; the sanitizers abort on any error.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../include/klein_attn.h"

static int g_fail = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

static void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(0x10000 + off); }
static const int32_t* fpos(uintptr_t off = 0) { return reinterpret_cast<const int32_t*>(fake(off)); }

int main() {
  const klein_status_t I = KLEIN_ERR_INVALID_ARG, U = KLEIN_ERR_UNSUPPORTED;
  void* F = fake();

  // ---- attention forward: nulls, sizes, head dims, alignment, dtype, grid
  CHECK(klein_rope4d_attn_fwd(nullptr, F, F, fpos(), F, 1, 8, 1, 128, KLEIN_DTYPE_BF16, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd(F, F, F, nullptr, F, 1, 8, 1, 128, KLEIN_DTYPE_BF16, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 0, 8, 1, 128, KLEIN_DTYPE_BF16, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1, 0, 1, 128, KLEIN_DTYPE_BF16, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1, 8, -3, 128, KLEIN_DTYPE_BF16, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1, 8, 1, 96, KLEIN_DTYPE_BF16, nullptr) == U);
  CHECK(klein_rope4d_attn_fwd(fake(2), F, F, fpos(), F, 1, 8, 1, 128, KLEIN_DTYPE_BF16, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(4), F, 1, 8, 1, 128, KLEIN_DTYPE_BF16, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1, 8, 1, 128, (klein_dtype_t)7, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1, 8, 1, 128, (klein_dtype_t)-1, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1, 8, 1, 128, KLEIN_DTYPE_SPAN_INT_, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1 << 20, 1 << 30, 1 << 10, 128,
                              KLEIN_DTYPE_BF16, nullptr) == U);
  CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1 << 20, 1 << 30, 1 << 10, 128,
                              KLEIN_DTYPE_FP8_E4M3, nullptr) == U);
  const float bad[][3] = {{0.f, 1.f, 1.f}, {1.f, -1.f, 1.f}, {1.f, 1.f, NAN}, {1.f, INFINITY, 1.f}};
  for (const auto& d : bad) {
    CHECK(klein_rope4d_attn_fwd_fp8(F, F, F, fpos(), F, 1, 8, 1, 128, d[0], d[1], d[2], nullptr) == I);
    CHECK(klein_rope4d_attn_fwd_ws(F, F, F, fpos(), F, 1, 8, 1, 128, KLEIN_DTYPE_FP8_E4M3, d[0],
                                   d[1], d[2], F, 1 << 20, nullptr) == I);
    CHECK(klein_rope4d_attn_fwd_noalloc(F, F, F, fpos(), F, 1, 8, 1, 128, KLEIN_DTYPE_FP8_E4M3,
                                        d[0], d[1], d[2], nullptr) == I);
    CHECK(klein_rope4d_attn_fwd_blocksparse(F, F, F, fpos(), F, 1, 8, 1, 128, KLEIN_DTYPE_FP8_E4M3,
                                            d[0], d[1], d[2], (const uint8_t*)F, nullptr) == I);
  }
  const float bad2[][2] = {{0.f, 1.f}, {1.f, -2.f}, {NAN, 1.f}, {1.f, INFINITY}};
  for (const auto& d : bad2)
    CHECK(klein_qkv_rope4d_proj_fp8(F, F, nullptr, fpos(), F, F, F, 1, 8, 128, 1, 64, d[0], d[1],
                                    nullptr) == I);

  // ---- workspace entry points
  CHECK(klein_rope4d_attn_fwd_ws(F, F, F, fpos(), F, 1, 4096, 1, 128, (klein_dtype_t)3, 1, 1, 1,
                                 F, 1 << 30, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd_ws(F, F, F, fpos(), F, 1, 4096, 1, 128, KLEIN_DTYPE_BF16, 1, 1, 1,
                                 fake(16), 1 << 30, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd_ws(F, F, F, fpos(), F, 1, 4096, 1, 80, KLEIN_DTYPE_BF16, 1, 1, 1, F,
                                 1 << 30, nullptr) == U);
  CHECK(klein_rope4d_attn_fwd_lse_ws(F, F, F, fpos(), F, nullptr, 1, 4096, 1, 128, F, 1 << 30,
                                     nullptr) == I);
  CHECK(klein_rope4d_attn_fwd_noalloc(F, F, F, fpos(), F, 1, 8, 1, 128, (klein_dtype_t)2, 1, 1, 1,
                                      nullptr) == I);
  CHECK(klein_rope4d_attn_fwd_noalloc(nullptr, F, F, fpos(), F, 1, 8, 1, 128, KLEIN_DTYPE_BF16, 1,
                                      1, 1, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd_noalloc(F, F, F, fpos(), F, 1, 8, 1, 32, KLEIN_DTYPE_BF16, 1, 1, 1,
                                      nullptr) == U);
  size_t n = 7;
  CHECK(klein_attn_workspace_size(1, 4096, 1, 128, KLEIN_DTYPE_BF16, nullptr) == I);
  CHECK(klein_attn_workspace_size(1, 4096, 1, 96, KLEIN_DTYPE_BF16, &n) == U);
  CHECK(klein_attn_workspace_size(1, 4096, 0, 128, KLEIN_DTYPE_BF16, &n) == I);
  CHECK(klein_attn_workspace_size(1, 4096, 1, 128, (klein_dtype_t)2, &n) == I);
  CHECK(n == 7);

  // ---- block-sparse
  CHECK(klein_rope4d_attn_fwd_blocksparse(F, F, F, fpos(), F, 1, 8, 1, 128, KLEIN_DTYPE_BF16, 1, 1,
                                          1, nullptr, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd_blocksparse(F, F, F, fpos(), F, 1, 64 * 4096 + 1, 1, 64,
                                          KLEIN_DTYPE_BF16, 1, 1, 1, (const uint8_t*)F, nullptr) == U);
  CHECK(klein_rope4d_attn_fwd_blocksparse_ws(F, F, F, fpos(), F, 1, 300, 1, 64, KLEIN_DTYPE_BF16,
                                             1, 1, 1, (const uint8_t*)F, F, 100, nullptr) == I);

  // ---- backward and its workspace
  size_t need = 0;
  CHECK(klein_attn_bwd_workspace_size(1, 100, 2, 64, &need) == KLEIN_OK);
  CHECK(need >= 4 * 100 * 2 * 64 + 4 * 2 * 100);
  CHECK(klein_attn_bwd_workspace_size(1, 100, 2, 96, &need) == U);
  CHECK(klein_attn_bwd_workspace_size(0, 100, 2, 64, &need) == I);
  CHECK(klein_attn_bwd_workspace_size(1, 100, 2, 64, nullptr) == I);
  CHECK(klein_rope4d_attn_bwd(F, F, F, fpos(), F, F, (const float*)F, F, F, F, 1, 100, 2, 64, F,
                              need - 1, nullptr) == I);
  CHECK(klein_rope4d_attn_bwd(F, F, F, fpos(), F, nullptr, (const float*)F, F, F, F, 1, 100, 2, 64,
                              F, need, nullptr) == I);
  CHECK(klein_rope4d_attn_bwd(F, F, F, fpos(), F, F, (const float*)F, F, F, F, 1, 100, 2, 64,
                              fake(16), need, nullptr) == I);
  CHECK(klein_rope4d_attn_fwd_lse(F, F, F, fpos(), F, (float*)fake(2), 1, 8, 1, 64, nullptr) == I);
  // a large backward workspace: the size arithmetic stays in 64 bits
  CHECK(klein_attn_bwd_workspace_size(64, 65536, 64, 128, &need) == KLEIN_OK);
  CHECK(need > (size_t)4 * 64 * 65536 * 64 * 128);

  // ---- QKV projection, pre-rotated attention, RoPE hook
  CHECK(klein_qkv_rope4d_proj(nullptr, F, nullptr, fpos(), F, F, F, 1, 8, 128, 2, 64, nullptr) == I);
  CHECK(klein_qkv_rope4d_proj(F, F, nullptr, fpos(), F, F, F, 1, 8, 96, 2, 64, nullptr) == U);
  CHECK(klein_qkv_rope4d_proj(F, F, fake(4), fpos(), F, F, F, 1, 8, 128, 2, 64, nullptr) == I);
  CHECK(klein_qkv_rope4d_proj(F, F, nullptr, fpos(), F, F, F, 1, 8, 65536 + 64, 2, 64, nullptr) == U);
  CHECK(klein_attn_fwd_prerotated(F, F, fake(8), F, 1, 8, 1, 64, nullptr) == I);
  CHECK(klein_attn_fwd_prerotated(F, F, F, F, 1, 8, 1, 80, nullptr) == U);
  CHECK(klein_rope4d_apply(F, fpos(), fake(4), 1, 8, 1, 64, nullptr) == I);
  CHECK(klein_rope4d_apply(F, fpos(), F, 1, 8, 1, 32, nullptr) == U);

  // ---- the split-KV planner (host only) over a sweep of shapes
  int plan[3];
  size_t part = 0;
  CHECK(klein_splitkv_plan(1, 8, 1, 128, 0, plan, &part) == I);
  CHECK(klein_splitkv_plan(1, 8, 1, 128, 256, nullptr, &part) == I);
  const int Ss[] = {1, 63, 2047, 2048, 4608, 8704, 16896, 33280, 66048, 1 << 20, 1 << 30};
  const int cus[] = {1, 80, 256, 304, 1024, 1 << 20};
  for (int B : {1, 2, 7})
    for (int H : {1, 3, 24, 1000})
      for (int S : Ss)
        for (int ncu : cus) {
          const klein_status_t st = klein_splitkv_plan(B, S, H, 128, ncu, plan, &part);
          CHECK(st == KLEIN_OK || st == U);
          if (st != KLEIN_OK) continue;
          const long long items = (long long)B * H * ((S + 255LL) / 256);
          CHECK(plan[0] >= 0 && plan[1] >= 0 && plan[2] >= 0);
          CHECK((long long)plan[0] + plan[1] == items);
          CHECK((plan[1] == 0) == (plan[2] == 0) && (plan[1] == 0) == (part == 0));
          CHECK(plan[2] <= 4LL * ncu);
        }

  // ---- status strings
  for (int s = 0; s < 5; ++s) CHECK(std::strlen(klein_status_string((klein_status_t)s)) > 0);
  CHECK(std::strcmp(klein_status_string((klein_status_t)99), "unknown status") == 0);
  CHECK(std::strcmp(klein_status_string((klein_status_t)-5), "unknown status") == 0);
  CHECK(std::strcmp(klein_status_string(KLEIN_STATUS_SPAN_INT_), "unknown status") == 0);
  CHECK(klein_version() >= 100);

  // ---- the buffer limit: no buffer is held, so no HIP call is made
  CHECK(klein_set_buffer_limit(0) == KLEIN_OK);
  CHECK(klein_set_buffer_limit(KLEIN_DEFAULT_BUFFER_LIMIT) == KLEIN_OK);

  // ---- without a GPU, every call that reaches the device reports NO_DEVICE
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
    const klein_status_t N = KLEIN_ERR_NO_DEVICE;
    size_t b = 0;
    CHECK(klein_attn_workspace_size(1, 4096, 2, 128, KLEIN_DTYPE_BF16, &b) == N);
    CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1, 300, 2, 128, KLEIN_DTYPE_BF16, nullptr) == N);
    CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1, 300, 2, 64, KLEIN_DTYPE_FP8_E4M3, nullptr) == N);
    CHECK(klein_set_buffer_limit(0) == KLEIN_OK);   // the per-tile kernels' path
    CHECK(klein_rope4d_attn_fwd(F, F, F, fpos(), F, 1, 300, 2, 128, KLEIN_DTYPE_BF16, nullptr) == N);
    CHECK(klein_rope4d_attn_fwd_fp8(F, F, F, fpos(), F, 1, 300, 2, 64, 1, 1, 1, nullptr) == N);
    CHECK(klein_set_buffer_limit(KLEIN_DEFAULT_BUFFER_LIMIT) == KLEIN_OK);
    CHECK(klein_rope4d_attn_fwd_ws(F, F, F, fpos(), F, 1, 4096, 2, 128, KLEIN_DTYPE_BF16, 1, 1, 1,
                                   F, 1 << 30, nullptr) == N);
    CHECK(klein_rope4d_attn_fwd_noalloc(F, F, F, fpos(), F, 1, 300, 2, 128, KLEIN_DTYPE_BF16, 1, 1,
                                        1, nullptr) == N);
    CHECK(klein_rope4d_attn_fwd_lse(F, F, F, fpos(), F, (float*)F, 1, 300, 2, 128, nullptr) == N);
    CHECK(klein_rope4d_attn_bwd(F, F, F, fpos(), F, F, (const float*)F, F, F, F, 1, 100, 2, 64, F,
                                1 << 30, nullptr) == N);
    CHECK(klein_rope4d_attn_fwd_blocksparse(F, F, F, fpos(), F, 1, 300, 1, 128, KLEIN_DTYPE_BF16, 1,
                                            1, 1, (const uint8_t*)F, nullptr) == N);
    CHECK(klein_qkv_rope4d_proj(F, F, nullptr, fpos(), F, F, F, 1, 8, 128, 2, 64, nullptr) == N);
    CHECK(klein_attn_fwd_prerotated(F, F, F, F, 1, 8, 1, 64, nullptr) == N);
    CHECK(klein_rope4d_apply(F, fpos(), F, 1, 8, 1, 64, nullptr) == N);
    std::printf("no device: device-reaching calls report NO_DEVICE\n");
  }
  std::printf("%s (%d failed checks)\n", g_fail ? "FAIL" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
