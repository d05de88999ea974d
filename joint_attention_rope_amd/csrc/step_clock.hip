// Measurement harness (not part of the library): where the cycles of the
// bf16 attention kernel's pipeline step go.
//
// This file compiles attn_fwd_bf16.hip with KLEIN_STEP_CLOCK defined, which
// makes every wave sum the shader-clock cycles (s_memtime) spent between
// marks in each step: the step start (key positions, tail mask), region A
// (the score MFMAs of the next tile with the softmax of this one), the
// rescale check, region B (the P.V MFMAs with the staging of later tiles),
// the buffer loads, and the barrier.  It is linked with the library's other
// objects (everything but attn_fwd_bf16.hip), so the public entry point
// klein_rope4d_attn_fwd_ws runs the instrumented kernel.  The marks add
// waits of their own; the harness reports the instrumented call's time so
// that the overhead can be read against the plain kernel's.
//
// Usage: step_clock [B S H D reps]   (default: the 2048x2048 CFG workload,
// B=2, S=16896, H=24, D=128).  Inputs are seeded N(0, 1) bf16; positions
// follow the workload's layout (512 text tokens on the l axis, then a
// square image grid).  Prints a markdown table: mean cycles per step for
// the waves 0-3 and 4-7 of the workgroups that run whole tiles (the two
// waves of a SIMD are w and w + 4), the loop's cycles per step, the clock
// (cycles over the fixed-rate 100 MHz timestamps) and the call time.
#define KLEIN_STEP_CLOCK 1
#include "attn_fwd_bf16.hip"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/klein_attn.h"

#define CHECK_HIP(x)                                                       \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));          \
      std::exit(1);                                                        \
    }                                                                      \
  } while (0)

static uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

int main(int argc, char** argv) {
  const int B = argc > 1 ? std::atoi(argv[1]) : 2;
  const int S = argc > 2 ? std::atoi(argv[2]) : 16896;
  const int H = argc > 3 ? std::atoi(argv[3]) : 24;
  const int D = argc > 4 ? std::atoi(argv[4]) : 128;
  const int reps = argc > 5 ? std::atoi(argv[5]) : 5;
  const size_t n = (size_t)B * S * H * D;

  // seeded N(0, 1) bf16 (Box-Muller on a 64-bit LCG)
  std::vector<uint16_t> host(n);
  uint64_t st = 20240611ull;
  auto uni = [&]() {
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return ((st >> 11) + 0.5) * (1.0 / 9007199254740992.0);
  };
  uint16_t* dev[3];
  for (int t = 0; t < 3; ++t) {
    for (size_t i = 0; i < n; ++i)
      host[i] = bf16_rne((float)(std::sqrt(-2.0 * std::log(uni())) * std::cos(6.283185307179586 * uni())));
    CHECK_HIP(hipMalloc(&dev[t], n * 2));
    CHECK_HIP(hipMemcpy(dev[t], host.data(), n * 2, hipMemcpyHostToDevice));
  }
  const int text = S >= 512 ? 512 : 0;
  const int grid = (int)std::lround(std::sqrt((double)(S - text)));
  std::vector<int32_t> pos((size_t)S * 4, 0);
  for (int s = 0; s < S; ++s) {
    if (s < text) {
      pos[4 * s + 3] = s;
    } else if (grid > 0) {
      const int i = s - text;
      pos[4 * s + 1] = (i / grid) % 4096;
      pos[4 * s + 2] = i % grid;
    }
  }
  int32_t* dpos;
  CHECK_HIP(hipMalloc(&dpos, pos.size() * 4));
  CHECK_HIP(hipMemcpy(dpos, pos.data(), pos.size() * 4, hipMemcpyHostToDevice));
  uint16_t* out;
  CHECK_HIP(hipMalloc(&out, n * 2));
  size_t wsb = 0;
  if (klein_attn_workspace_size(B, S, H, D, KLEIN_DTYPE_BF16, &wsb) != KLEIN_OK) return 1;
  void* ws = nullptr;
  CHECK_HIP(hipMalloc(&ws, wsb > 0 ? wsb : 256));
  int dev_id = 0, ncu = 0;
  CHECK_HIP(hipGetDevice(&dev_id));
  CHECK_HIP(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev_id));
  int plan[3];
  size_t part = 0;
  if (klein_splitkv_plan(B, S, H, D, ncu, plan, &part) != KLEIN_OK) return 1;
  const int whole = plan[0], wgs = plan[0] + plan[1] * plan[2];

  auto call = [&]() {
    const klein_status_t r = klein_rope4d_attn_fwd_ws(dev[0], dev[1], dev[2], dpos, out, B, S, H, D,
                                                      KLEIN_DTYPE_BF16, 1.f, 1.f, 1.f, ws, wsb,
                                                      nullptr);
    if (r != KLEIN_OK) {
      std::fprintf(stderr, "call failed: %s\n", klein_status_string(r));
      std::exit(1);
    }
  };
  unsigned long long* clk;
  const size_t nclk = (size_t)wgs * 8 * 10;
  CHECK_HIP(hipMalloc(&clk, nclk * 8));
  CHECK_HIP(hipMemset(clk, 0, nclk * 8));
  CHECK_HIP(hipMemcpyToSymbol(HIP_SYMBOL(klein::klein_step_clock_out), &clk, sizeof(clk)));
  for (int i = 0; i < 2; ++i) call();
  hipEvent_t e0, e1;
  CHECK_HIP(hipEventCreate(&e0));
  CHECK_HIP(hipEventCreate(&e1));
  CHECK_HIP(hipEventRecord(e0, nullptr));
  for (int i = 0; i < reps; ++i) call();
  CHECK_HIP(hipEventRecord(e1, nullptr));
  CHECK_HIP(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
  ms /= reps;
  std::vector<unsigned long long> c(nclk);
  CHECK_HIP(hipMemcpy(c.data(), clk, nclk * 8, hipMemcpyDeviceToHost));

  // workgroups that run whole tiles: sums per wave half
  double sum[2][7] = {}, realt = 0.0, cyc = 0.0;
  for (int wg = 0; wg < whole; ++wg)
    for (int w = 0; w < 8; ++w) {
      const unsigned long long* r = &c[((size_t)wg * 8 + w) * 10];
      for (int i = 0; i < 7; ++i) sum[w >= 4][i] += (double)r[i];
      cyc += (double)r[7];
      realt += (double)(r[9] - r[8]);
    }
  const char* names[6] = {"step start (key positions, tail mask)",
                          "region A: S(t+1) MFMAs with the softmax of S(t)",
                          "rescale check (and the rare rescale)",
                          "region B: O += V P MFMAs with the staging of K, V",
                          "buffer loads of later tiles", "barrier"};
  std::printf("| part of the step | waves 0-3: cycles per step | waves 4-7: cycles per step |\n");
  std::printf("|---|---|---|\n");
  double tot[2] = {0.0, 0.0};
  for (int i = 0; i < 6; ++i) {
    const double a = sum[0][i] / sum[0][6], b = sum[1][i] / sum[1][6];
    tot[0] += a;
    tot[1] += b;
    std::printf("| %s | %.0f | %.0f |\n", names[i], a, b);
  }
  std::printf("| the step | %.0f | %.0f |\n", tot[0], tot[1]);
  const double mhz = cyc / (realt * 1e-8) / 1e6 / 1.0;
  const double flops = 4.0 * B * H * (double)S * S * D;
  std::printf("\nB=%d S=%d H=%d D=%d: whole-tile workgroups %d of %d; steps per wave %.0f; "
              "MFMA cycles per step and SIMD (two waves x 32 MFMAs x 32 cycles) 2048; "
              "clock %.0f MHz (s_memtime over s_memrealtime); instrumented call %.4f ms "
              "(%.1f TFLOP/s)\n",
              B, S, H, D, whole, wgs, sum[0][6] / (4.0 * whole), mhz, ms, flops / (ms * 1e-3) / 1e12);
  return 0;
}
