// Elementwise passes around the attention kernels: the test hook
// y = RoPE-4D(x) in bf16 (through rope_chunk, the very routine the attention
// kernels apply to Q and K; one thread per 16-byte chunk, 8 channels of one
// axis block of one token and head), the keys rotated once into fp16, and the
// values regrouped into key-major tiles for the bf16 attention kernel.
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

// V regrouped for the bf16 attention kernel: for every (b, h) and 64-key tile
// t, a block of D rows (one per channel) of the tile's 64 keys in order, bf16
// (vt[((b H + h) ntile + t) D 64 + d 64 + key - 64 t]), zero for keys past S.
// The kernel then reads each operand of O^T += V^T P^T (8 keys of one
// channel) with one 16-byte LDS read.  One thread per 8 keys x 8 channels:
// eight 16-byte row loads, a 16-bit transpose in registers, eight 16-byte
// stores (8 threads, one per key group, write a row's 128 bytes).
template <int D>
__global__ __launch_bounds__(256) void v_tiles_kernel(const uint16_t* __restrict__ v,
                                                      uint16_t* __restrict__ vt, long long nitems,
                                                      int S, int H, int ntile) {
  constexpr int DG = D / 8;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x; c < nitems; c += stride) {
    const int kg = (int)(c & 7);
    const int dg = (int)((c >> 3) % DG);
    const long long tile = (c >> 3) / DG;            // (b H + h) ntile + t
    const int t = (int)(tile % ntile);
    const long long bh = tile / ntile;
    const int h = (int)(bh % H);
    const long long b = bh / H;
    const int key0 = 64 * t + 8 * kg;
    u32x4_t x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = key0 + i;
      x[i] = key < S ? *reinterpret_cast<const u32x4_t*>(
                           v + ((b * S + key) * H + h) * D + 8 * dg)
                     : (u32x4_t){0u, 0u, 0u, 0u};
    }
    uint16_t* dst = vt + (tile * D + 8 * dg) * 64 + 8 * kg;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
      // channel 8 dg + ch of keys key0 .. key0 + 7, two keys a word
      const int w = ch >> 1, hi = ch & 1;
      u32x4_t y;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = x[2 * p][w], bw = x[2 * p + 1][w];
        y[p] = hi ? (a >> 16) | (bw & 0xffff0000u) : (a & 0xffffu) | (bw << 16);
      }
      *reinterpret_cast<u32x4_t*>(dst + ch * 64) = y;
    }
  }
}

long long v_tiles_bytes(int B, int S, int H, int D) {
  const long long ntile = (S + 63) / 64;
  return (long long)B * H * ntile * 64 * D * 2;
}

hipError_t launch_v_tiles(const void* v, void* vt, int B, int S, int H, int D,
                          hipStream_t stream) {
  const int ntile = (S + 63) / 64;
  const long long nitems = (long long)B * H * ntile * 8 * (D / 8);
  long long blocks = (nitems + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (D == 128)
    hipLaunchKernelGGL(v_tiles_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)v, (uint16_t*)vt, nitems, S, H, ntile);
  else
    hipLaunchKernelGGL(v_tiles_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)v, (uint16_t*)vt, nitems, S, H, ntile);
  return hipGetLastError();
}

}  // namespace klein
