// Test hook kernel: y = RoPE-4D(x) in bf16, through rope_chunk, the very
// routine the attention kernels apply to Q and K.  One thread per 16-byte
// chunk (8 channels of one axis block of one token and head).
#include "klein_device.hpp"
#include "klein_launch.hpp"

namespace klein {

template <int D>
__global__ __launch_bounds__(256) void rope4d_apply_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ y, long long nchunks, int S, int H, RopeFreqs fr) {
  constexpr int CPR = D / 8, DA = D / 4;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    const int lc = (int)(c % CPR);
    const long long row = c / CPR;                  // ((b * S) + s) * H + h
    const int s = (int)((row / H) % S);
    const int a = (8 * lc) / DA, j0 = ((8 * lc) % DA) / 2;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + 8 * c);
    *reinterpret_cast<u32x4_t*>(y + 8 * c) =
        rope_chunk(v, pos[4 * s + a], &fr.hi[j0], &fr.lo[j0], 1.0f);
  }
}

hipError_t launch_rope4d_apply(const LaunchArgs& a) {
  const long long nchunks = (long long)a.B * a.S * a.H * (a.D / 8);
  long long blocks = (nchunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (a.D == 128)
    hipLaunchKernelGGL(rope4d_apply_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, a.stream,
                       (const uint16_t*)a.q, a.pos, (uint16_t*)a.out, nchunks, a.S, a.H, a.freqs);
  else
    hipLaunchKernelGGL(rope4d_apply_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, a.stream,
                       (const uint16_t*)a.q, a.pos, (uint16_t*)a.out, nchunks, a.S, a.H, a.freqs);
  return hipGetLastError();
}

// y = fp16(R(pos) x * scale): k rotated once before an attention kernel that
// copies its tiles (the values the kernel would form from its cos/sin table,
// which holds the same angles).
template <int D>
__global__ __launch_bounds__(256) void rope4d_fp16_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ y, long long nchunks, int S, int H, RopeFreqs fr, float scale) {
  constexpr int CPR = D / 8, DA = D / 4;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    const int lc = (int)(c % CPR);
    const long long row = c / CPR;                  // ((b * S) + s) * H + h
    const int s = (int)((row / H) % S);
    const int a = (8 * lc) / DA, j0 = ((8 * lc) % DA) / 2;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + 8 * c);
    *reinterpret_cast<u32x4_t*>(y + 8 * c) =
        rope_chunk<true>(v, pos[4 * s + a], &fr.hi[j0], &fr.lo[j0], scale);
  }
}

hipError_t launch_rope4d_fp16(const void* x, const int32_t* pos, void* y, int B, int S, int H,
                              int D, const RopeFreqs& fr, float scale, hipStream_t stream) {
  const long long nchunks = (long long)B * S * H * (D / 8);
  long long blocks = (nchunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (D == 128)
    hipLaunchKernelGGL(rope4d_fp16_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)x, pos, (uint16_t*)y, nchunks, S, H, fr, scale);
  else
    hipLaunchKernelGGL(rope4d_fp16_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)x, pos, (uint16_t*)y, nchunks, S, H, fr, scale);
  return hipGetLastError();
}

}  // namespace klein
