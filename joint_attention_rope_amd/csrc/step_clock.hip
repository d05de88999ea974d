// Measurement harness (not part of the library): where the cycles of the
// bf16 and fp8 attention kernels' pipeline steps, and of the QKV
// projection, go; and the LDS rates those loops run against.
//
// This file compiles attn_fwd_bf16.hip, attn_fwd_fp8.hip and
// qkv_rope_proj.hip with KLEIN_STEP_CLOCK defined, which makes every wave
// sum the shader-clock cycles (s_memtime) spent between marks.  In the bf16
// attention kernel's step: the step start (key positions, tail mask), region
// A (the score MFMAs of the next tile with the softmax of this one), the
// rescale check, region B (the P.V MFMAs with the staging of later tiles),
// the buffer loads, and the barrier.  In the fp8 kernel's step: the softmax
// max with the rare rescale, region A, region B, the loads and the barrier.  In the projection's K step: each k-sub-step (8 MFMAs with the
// staging loads and stores placed among them) and the barrier.  The harness
// is linked with the library's other objects (everything but those two
// sources), so the public entry points klein_rope4d_attn_fwd_ws and
// klein_qkv_rope4d_proj(_fp8) run the instrumented kernels.  The marks add
// waits of their own; the harness reports the instrumented call's time so
// that the overhead can be read against the plain kernel's.
//
// Usage: step_clock [B S H D reps]        the attention (default: the
//                                         2048x2048 CFG workload, B=2,
//                                         S=16896, H=24, D=128)
//        step_clock fp8 [reps]            the FP8 attention on the 2048x2048
//                                         edit workload (B=1, S=33280:
//                                         512 text + image + reference)
//        step_clock qkv [B S H D reps]    the projection (C = H D), bf16
//                                         then fp8 operands
//        step_clock lds                   LDS rates of this GPU: bytes per
//                                         shader clock and CU for the access
//                                         forms the kernels use
// Inputs are seeded N(0, 1) (W scaled by 1/sqrt(C)); positions follow the
// workload's layout (512 text tokens on the l axis, then a square image
// grid).  The attention table gives mean cycles per step for the waves 0-3
// and 4-7 of the workgroups that run whole tiles (the two waves of a SIMD
// are w and w + 4), the loop's cycles per step, the clock (cycles over the
// fixed-rate 100 MHz timestamps) and the call time; the projection table
// the mean cycles per K step of the same two wave halves over all
// workgroups.
#define KLEIN_STEP_CLOCK 1
#include "attn_fwd_bf16.hip"
#include "attn_fwd_fp8.hip"
#include "qkv_rope_proj.hip"

#include <algorithm>
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

static std::vector<int32_t> workload_positions(int S) {
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
  return pos;
}

// E4M3 code of x (round to nearest even, saturating at 448)
static uint8_t e4m3_code(float x) {
  const double a = std::fmin(std::fabs((double)x), 448.0);
  int c;
  if (a < std::ldexp(1.0, -6)) {
    c = (int)std::nearbyint(std::ldexp(a, 9));           // subnormal: m 2^-9 (8 = 2^-6)
  } else {
    int E;
    const double f = std::frexp(a, &E);                   // a = f 2^E, f in [0.5, 1)
    int m = (int)std::nearbyint((2.0 * f - 1.0) * 8.0);   // a = (1 + m/8) 2^(E-1)
    int e = E - 1;
    if (m == 8) {
      m = 0;
      ++e;
    }
    c = ((e + 7) << 3) | m;
  }
  if (c > 126) c = 126;
  return (uint8_t)(c | (x < 0.f ? 0x80 : 0));
}

static int fp8_main(int argc, char** argv) {
  const int B = 1, H = 24, D = 128, text = 512, grid = 128;
  const int S = text + 2 * grid * grid;
  const int reps = argc > 2 ? std::atoi(argv[2]) : 5;
  const size_t n = (size_t)B * S * H * D;
  uint64_t st = 20240612ull;
  auto gauss = [&]() {
    auto uni = [&]() {
      st = st * 6364136223846793005ull + 1442695040888963407ull;
      return ((st >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    };
    return (float)(std::sqrt(-2.0 * std::log(uni())) * std::cos(6.283185307179586 * uni()));
  };
  // seeded N(0, 1) values as E4M3 codes with per-tensor descales max|x| / 448
  std::vector<float> f(n);
  std::vector<uint8_t> codes(n);
  uint8_t* dev[3];
  float descale[3];
  for (int t = 0; t < 3; ++t) {
    float mx = 0.f;
    for (auto& e : f) {
      e = gauss();
      mx = std::fmax(mx, std::fabs(e));
    }
    descale[t] = mx / 448.f;
    for (size_t i = 0; i < n; ++i) codes[i] = e4m3_code(f[i] / descale[t]);
    CHECK_HIP(hipMalloc(&dev[t], n));
    CHECK_HIP(hipMemcpy(dev[t], codes.data(), n, hipMemcpyHostToDevice));
  }
  // text on the l axis; the image at t = 0 and the reference at t = 1 share
  // the (h, w) grid
  std::vector<int32_t> pos((size_t)S * 4, 0);
  for (int s = 0; s < S; ++s) {
    if (s < text) {
      pos[4 * s + 3] = s;
    } else {
      const int i = (s - text) % (grid * grid);
      pos[4 * s + 0] = (s - text) / (grid * grid);
      pos[4 * s + 1] = i / grid;
      pos[4 * s + 2] = i % grid;
    }
  }
  int32_t* dpos;
  CHECK_HIP(hipMalloc(&dpos, pos.size() * 4));
  CHECK_HIP(hipMemcpy(dpos, pos.data(), pos.size() * 4, hipMemcpyHostToDevice));
  uint16_t* out;
  CHECK_HIP(hipMalloc(&out, n * 2));
  size_t wsb = 0;
  if (klein_attn_workspace_size(B, S, H, D, KLEIN_DTYPE_FP8_E4M3, &wsb) != KLEIN_OK) return 1;
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
                                                      KLEIN_DTYPE_FP8_E4M3, descale[0], descale[1],
                                                      descale[2], ws, wsb, nullptr);
    if (r != KLEIN_OK) {
      std::fprintf(stderr, "call failed: %s\n", klein_status_string(r));
      std::exit(1);
    }
  };
  unsigned long long* clk;
  const size_t nclk = (size_t)wgs * 8 * 10;
  CHECK_HIP(hipMalloc(&clk, nclk * 8));
  CHECK_HIP(hipMemset(clk, 0, nclk * 8));
  CHECK_HIP(hipMemcpyToSymbol(HIP_SYMBOL(klein::klein_fp8_clock_out), &clk, sizeof(clk)));
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
  double sum[2][7] = {}, realt = 0.0, cyc = 0.0;
  for (int wg = 0; wg < whole; ++wg)
    for (int w = 0; w < 8; ++w) {
      const unsigned long long* r = &c[((size_t)wg * 8 + w) * 10];
      for (int i = 0; i < 7; ++i) sum[w >= 4][i] += (double)r[i];
      cyc += (double)r[7];
      realt += (double)(r[9] - r[8]);
    }
  const char* names[5] = {"step start and softmax max (with the rare rescale)",
                          "region A: Y(t+1) MFMAs with the P8 codes of Y(t)",
                          "region B: O += V P8 and row-sum MFMAs with the staging of K'', V",
                          "buffer loads of later tiles", "barrier"};
  std::printf("| part of the step | waves 0-3: cycles per step | waves 4-7: cycles per step |\n");
  std::printf("|---|---|---|\n");
  double tot[2] = {0.0, 0.0};
  for (int i = 0; i < 5; ++i) {
    const double a = sum[0][i] / sum[0][6], b = sum[1][i] / sum[1][6];
    tot[0] += a;
    tot[1] += b;
    std::printf("| %s | %.0f | %.0f |\n", names[i], a, b);
  }
  std::printf("| the step | %.0f | %.0f |\n", tot[0], tot[1]);
  const double mhz = cyc / (realt * 1e-8) / 1e6;
  const double flops = 4.0 * B * H * (double)S * S * D;
  std::printf("\nB=%d S=%d H=%d D=%d fp8: whole-tile workgroups %d of %d; steps per wave %.0f; "
              "MFMA cycles per step and SIMD (two waves x 8 MFMAs x 64 cycles, plus two row-sum "
              "MFMAs of 32 cycles) 1,088; clock %.0f MHz (s_memtime over s_memrealtime); instrumented call %.4f "
              "ms (%.1f TFLOP/s)\n",
              B, S, H, D, whole, wgs, sum[0][6] / (4.0 * whole), mhz, ms, flops / (ms * 1e-3) / 1e12);
  return 0;
}

static int qkv_main(int argc, char** argv) {
  const int B = argc > 2 ? std::atoi(argv[2]) : 2;
  const int S = argc > 3 ? std::atoi(argv[3]) : 16896;
  const int H = argc > 4 ? std::atoi(argv[4]) : 24;
  const int D = argc > 5 ? std::atoi(argv[5]) : 128;
  const int reps = argc > 6 ? std::atoi(argv[6]) : 10;
  const int C = H * D, M = B * S, N = 3 * H * D;
  uint64_t st = 404ull;
  auto gauss = [&]() {
    auto uni = [&]() {
      st = st * 6364136223846793005ull + 1442695040888963407ull;
      return ((st >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    };
    return (float)(std::sqrt(-2.0 * std::log(uni())) * std::cos(6.283185307179586 * uni()));
  };
  std::vector<float> xf((size_t)M * C), wf((size_t)N * C);
  for (auto& e : xf) e = gauss();
  for (auto& e : wf) e = gauss() / std::sqrt((float)C);
  std::vector<uint16_t> xb(xf.size()), wb(wf.size()), bias(N, 0);
  for (size_t i = 0; i < xf.size(); ++i) xb[i] = bf16_rne(xf[i]);
  for (size_t i = 0; i < wf.size(); ++i) wb[i] = bf16_rne(wf[i]);
  float xmax = 0.f, wmax = 0.f;
  for (float e : xf) xmax = std::fmax(xmax, std::fabs(e));
  for (float e : wf) wmax = std::fmax(wmax, std::fabs(e));
  const float sx = xmax / 448.f, sw = wmax / 448.f;
  std::vector<uint8_t> x8(xf.size()), w8(wf.size());
  for (size_t i = 0; i < xf.size(); ++i) x8[i] = e4m3_code(xf[i] / sx);
  for (size_t i = 0; i < wf.size(); ++i) w8[i] = e4m3_code(wf[i] / sw);
  const std::vector<int32_t> pos = workload_positions(S);
  void *dx, *dw, *dx8, *dw8, *db, *dq, *dk, *dv;
  int32_t* dpos;
  CHECK_HIP(hipMalloc(&dx, xb.size() * 2));
  CHECK_HIP(hipMalloc(&dw, wb.size() * 2));
  CHECK_HIP(hipMalloc(&dx8, x8.size()));
  CHECK_HIP(hipMalloc(&dw8, w8.size()));
  CHECK_HIP(hipMalloc(&db, bias.size() * 2));
  CHECK_HIP(hipMalloc(&dpos, pos.size() * 4));
  CHECK_HIP(hipMalloc(&dq, (size_t)M * C * 2));
  CHECK_HIP(hipMalloc(&dk, (size_t)M * C * 2));
  CHECK_HIP(hipMalloc(&dv, (size_t)M * C * 2));
  CHECK_HIP(hipMemcpy(dx, xb.data(), xb.size() * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dw, wb.data(), wb.size() * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dx8, x8.data(), x8.size(), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dw8, w8.data(), w8.size(), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(db, bias.data(), bias.size() * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dpos, pos.data(), pos.size() * 4, hipMemcpyHostToDevice));
  const long long wgs = klein::qkv_rope_proj_grid(B, S, H, D);
  const size_t nclk = (size_t)wgs * 8 * 10;
  unsigned long long* clk;
  CHECK_HIP(hipMalloc(&clk, nclk * 8));
  CHECK_HIP(hipMemcpyToSymbol(HIP_SYMBOL(klein::klein_qkv_clock_out), &clk, sizeof(clk)));
  for (int fp8 = 0; fp8 < 2; ++fp8) {
    auto call = [&]() {
      const klein_status_t r =
          fp8 ? klein_qkv_rope4d_proj_fp8(dx8, dw8, db, dpos, dq, dk, dv, B, S, C, H, D, sx, sw, nullptr)
              : klein_qkv_rope4d_proj(dx, dw, db, dpos, dq, dk, dv, B, S, C, H, D, nullptr);
      if (r != KLEIN_OK) {
        std::fprintf(stderr, "call failed: %s\n", klein_status_string(r));
        std::exit(1);
      }
    };
    CHECK_HIP(hipMemset(clk, 0, nclk * 8));
    for (int i = 0; i < 10; ++i) call();
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
    const int ksub = fp8 ? 2 : 4;
    double sum[2][5] = {}, steps[2] = {0.0, 0.0}, loop[2] = {0.0, 0.0}, pro[2] = {0.0, 0.0},
           epi[2] = {0.0, 0.0};
    for (long long wg = 0; wg < wgs; ++wg)
      for (int w = 0; w < 8; ++w) {
        const unsigned long long* r = &c[((size_t)wg * 8 + w) * 10];
        for (int i = 0; i < 5; ++i) sum[w >= 4][i] += (double)r[i];
        steps[w >= 4] += (double)r[5];
        loop[w >= 4] += (double)r[6];
        pro[w >= 4] += (double)r[7];
        epi[w >= 4] += (double)r[8];
      }
    std::printf("\n%s operands: M=%d N=%d K=%d, %lld tiles; cycles per K step of one wave\n\n",
                fp8 ? "FP8 (E4M3)" : "bf16", M, N, C, wgs);
    std::printf("| part of the K step | waves 0-3 | waves 4-7 |\n|---|---|---|\n");
    double tot[2] = {0.0, 0.0};
    for (int i = 0; i < 5; ++i) {
      if (i >= ksub && i < 4) continue;
      const double a = sum[0][i] / steps[0], b = sum[1][i] / steps[1];
      tot[0] += a;
      tot[1] += b;
      if (i < 4)
        std::printf("| k-sub-step %d: 8 MFMAs with their staging slots | %.0f | %.0f |\n", i, a, b);
      else
        std::printf("| barrier | %.0f | %.0f |\n", a, b);
    }
    std::printf("| the K step | %.0f | %.0f |\n", tot[0], tot[1]);
    const double nw = 4.0 * (double)wgs;
    std::printf("\nPer tile and wave, cycles: before its K loop (kernel entry, or the end of the "
                "wave's previous tile) %.0f / %.0f, "
                "K loop %.0f / %.0f, epilogue (bias, RoPE, stores) %.0f / %.0f "
                "(waves 0-3 / 4-7)\n",
                pro[0] / nw, pro[1] / nw, loop[0] / nw, loop[1] / nw, epi[0] / nw, epi[1] / nw);
    const double flops = 2.0 * M * (double)N * C;
    std::printf("\nMFMA cycles per K step and SIMD: 2048; instrumented call %.4f ms (%.1f TFLOP/s)\n",
                ms, flops / (ms * 1e-3) / 1e12);
  }
  return 0;
}

// ---- LDS rates: one workgroup of 512 threads per CU, each thread with a
// fixed address, 8 accesses per iteration at constant offsets (16 or 8
// bytes a lane, 16 consecutive lanes on consecutive slots: no bank
// conflicts), s_memtime around the loop per wave.
typedef unsigned lds_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned lds_u32x2 __attribute__((ext_vector_type(2)));
typedef short lds_s16x4 __attribute__((ext_vector_type(4)));
template <int MODE>
__global__ __launch_bounds__(512) void lds_rate_kernel(unsigned long long* out, unsigned* sink,
                                                       int iters) {
  __shared__ __attribute__((aligned(16))) unsigned lds[16384];     // 64 KB
  const int tid = threadIdx.x;
  for (int i = tid; i < 16384; i += 512) lds[i] = i * 2654435761u;
  __syncthreads();
  lds_u32x4 acc = {0, 0, 0, 0};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (MODE == 0) {                 // ds_read_b128: 16 bytes at 16 tid + 8 KB u
        acc ^= *reinterpret_cast<const lds_u32x4*>(&lds[4 * tid + 2048 * u]);
      } else if (MODE == 1) {          // ds_write_b128
        *reinterpret_cast<lds_u32x4*>(&lds[4 * tid + 2048 * u]) = acc;
        acc.x += 1u;
      } else {                         // ds_read_b64_tr_b16: 8 bytes at 8 tid + 4 KB u
        const lds_s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) lds_s16x4*)(reinterpret_cast<short*>(
                &lds[2 * tid + 1024 * u])));
        const lds_u32x2 w = __builtin_bit_cast(lds_u32x2, v);
        acc.x ^= w.x;
        acc.y ^= w.y;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if ((tid & 63) == 0) out[blockIdx.x * 8 + (tid >> 6)] = t1 - t0;
  sink[blockIdx.x * 512 + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

static int lds_main() {
  int ncu = 0;
  CHECK_HIP(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0));
  const int iters = 4096;
  unsigned long long* d_out = nullptr;
  unsigned* d_sink = nullptr;
  CHECK_HIP(hipMalloc(&d_out, (size_t)ncu * 8 * sizeof(unsigned long long)));
  CHECK_HIP(hipMalloc(&d_sink, (size_t)ncu * 512 * sizeof(unsigned)));
  const char* names[3] = {"ds_read_b128 (16 bytes a lane)", "ds_write_b128 (16 bytes a lane)",
                          "ds_read_b64_tr_b16 (8 bytes a lane)"};
  const int bytes[3] = {16, 16, 8};
  std::printf("LDS rates, one 512-thread workgroup per CU on %d CUs, %d x 8 accesses per thread\n\n",
              ncu, iters);
  std::printf("| access | bytes per shader clock and CU, mean over workgroups | slowest workgroup |\n");
  std::printf("|---|---|---|\n");
  for (int mode = 0; mode < 3; ++mode) {
    for (int rep = 0; rep < 2; ++rep) {
      if (mode == 0) hipLaunchKernelGGL(lds_rate_kernel<0>, dim3(ncu), dim3(512), 0, 0, d_out, d_sink, iters);
      if (mode == 1) hipLaunchKernelGGL(lds_rate_kernel<1>, dim3(ncu), dim3(512), 0, 0, d_out, d_sink, iters);
      if (mode == 2) hipLaunchKernelGGL(lds_rate_kernel<2>, dim3(ncu), dim3(512), 0, 0, d_out, d_sink, iters);
      CHECK_HIP(hipGetLastError());
      CHECK_HIP(hipDeviceSynchronize());
    }
    std::vector<unsigned long long> h((size_t)ncu * 8);
    CHECK_HIP(hipMemcpy(h.data(), d_out, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
    double sum = 0, mx = 0;
    for (int b = 0; b < ncu; ++b) {
      unsigned long long m = 0;
      for (int w = 0; w < 8; ++w) m = std::max(m, h[(size_t)b * 8 + w]);
      sum += (double)m;
      mx = std::max(mx, (double)m);
    }
    const double wg_bytes = 512.0 * 8 * iters * bytes[mode];
    std::printf("| %s | %.1f | %.1f |\n", names[mode], wg_bytes / (sum / ncu), wg_bytes / mx);
  }
  CHECK_HIP(hipFree(d_out));
  CHECK_HIP(hipFree(d_sink));
  return 0;
}

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "lds") == 0) return lds_main();
  if (argc > 1 && std::strcmp(argv[1], "qkv") == 0) return qkv_main(argc, argv);
  if (argc > 1 && std::strcmp(argv[1], "fp8") == 0) return fp8_main(argc, argv);
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
  const std::vector<int32_t> pos = workload_positions(S);
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
