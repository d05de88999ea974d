// QKV projection with the RoPE-4D rotation in its epilogue, for gfx950.
//
//   y = x W^T (+ bias)          x [M = B S][C] bf16, W [N = 3 H D][C] bf16
//   q' = R(y[:, 0:HD]) -> fp16, k' = R(y[:, HD:2HD]) -> fp16, v = y[:, 2HD:] -> bf16
//
// or, with FP8 operands, x and W as E4M3 codes with per-tensor descales and
// y = (x_code W_code^T) dx dw (+ bias) on v_mfma_f32_32x32x64_f8f6f4 (twice
// the bf16 rate); the epilogue and the outputs are the same.  A K step is 128
// bytes of each operand row either way (64 bf16 or 128 fp8 elements), so the
// staging and the LDS layout below are shared.
//
// computed as C^T = W x^T so that output features run down the MFMA rows:
// accumulator registers 4c .. 4c+3 of a lane then hold four consecutive
// channels d of one token (its MFMA column), and the interleaved RoPE pairs
// (d, d+1) are register pairs of one lane.  The rotation, the bias and the
// conversions happen in registers before the only store; the angle of each
// pair is formed once per output element, like the attention kernels' Q.
//
// One workgroup of 8 waves computes 256 features x 256 tokens, K in steps of
// 128 bytes; each wave owns 128 features x 64 tokens (4 x 2 MFMA tiles of
// 32 x 32; bf16: 0.75 16-byte LDS operand reads per MFMA, fp8: 1.5 per MFMA
// of twice the length).  W and x tiles
// are double-buffered in LDS (rows padded to 144 bytes, so the 16 rows one
// 16-lane read phase touches fall on distinct banks) and staged through
// registers one K step ahead, the stores interleaved with the MFMAs; one
// barrier per K step.  Rows past N or M read
// as zeros through the buffer descriptors and are not stored.
#include "klein_device.hpp"
#include "klein_launch.hpp"

namespace klein {

template <int D, bool FP8>
__global__ __launch_bounds__(512) void qkv_rope_proj_kernel(
    const void* __restrict__ xv, const void* __restrict__ wv,
    const uint16_t* __restrict__ bias, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ qo, uint16_t* __restrict__ ko, uint16_t* __restrict__ vo,
    int M, int N, int C, int S, int H, int ntile_n, RopeFreqs fr, float yscale) {
  constexpr int TN = 256, TM = 256;
  constexpr int ES = FP8 ? 1 : 2;              // bytes per operand element
  constexpr int KB = 128;                      // bytes of a row per K step
  constexpr int ROW = 72;                      // LDS row stride (16-bit units: 144 bytes)
  constexpr int DA = D / 4;
  constexpr int CPR = KB / 16;                 // 16-byte chunks per tile row
  constexpr int KSUB = FP8 ? 2 : 4;            // MFMA k-steps per K step
  constexpr int NLD = (TN + TM) * CPR / 512;   // chunks per thread per K step
  static_assert(NLD == 8, "staging split");

  __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][TN * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t b_lds[2][TM * ROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lr = lane & 31;
  const int wn = wave & 1, wm = wave >> 1;     // 2 x 4 waves: 128 features x 64 tokens
  const int tn = blockIdx.x % ntile_n, tmi = blockIdx.x / ntile_n;
  const int n0 = tn * TN, m0 = tmi * TM;
  const int HD = H * D;

  // ---- staging: chunk c = tid + 512 i; the first TN*CPR chunks are W rows,
  // the rest x rows
  const int rowb = C * ES;
  const int nrows_a = min(TN, N - n0), nrows_b = min(TM, M - m0);
  const __amdgpu_buffer_rsrc_t ra =
      uniform_rsrc(static_cast<const uint8_t*>(wv) + (size_t)n0 * rowb, nrows_a * rowb);
  const __amdgpu_buffer_rsrc_t rb =
      uniform_rsrc(static_cast<const uint8_t*>(xv) + (size_t)m0 * rowb, nrows_b * rowb);
  u32x4_t stg[NLD];
  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = tid + 512 * i;
      const bool isa = c < TN * CPR;
      const int cc = isa ? c : c - TN * CPR;
      const int row = cc / CPR, ch = cc % CPR;
      const int off = row * rowb + kt * KB + 16 * ch;
      stg[i] = __builtin_bit_cast(u32x4_t, isa ? __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0)
                                               : __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = tid + 512 * i;
      const bool isa = c < TN * CPR;
      const int cc = isa ? c : c - TN * CPR;
      const int row = cc / CPR, ch = cc % CPR;
      uint16_t* dst = isa ? &a_lds[buf][row * ROW + 8 * ch] : &b_lds[buf][row * ROW + 8 * ch];
      *reinterpret_cast<u32x4_t*>(dst) = stg[i];
    }
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = (f32x16_t){};

  const int nk = C * ES / KB;
  load(0);
  store(0);
  __syncthreads();
  // K step kt: the loads of step kt+1 go out first (past the last step they
  // read in-range rows or the descriptors' zeros, and are never used); the
  // operands of sub-step ks+1 are read during the MFMAs of ks; the stores of
  // step kt+1 into the other buffer ride along the last two sub-steps (that
  // buffer was last read before the previous barrier).
  // a lane's operand of k-step ks: 16 bytes (bf16) or 32 bytes (fp8) of its
  // row, the second half-wave taking the next 16 or 32
  typedef uint32_t opnd_t __attribute__((ext_vector_type(FP8 ? 8 : 4)));
  opnd_t av[2][4], bv[2][2];
  auto read_op = [&](const uint16_t* rowp, int ks) {
    const uint16_t* p = rowp + (FP8 ? 32 * ks + 16 * g : 16 * ks + 8 * g);
    if constexpr (FP8) {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(p);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(p + 8);
      return (opnd_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return *reinterpret_cast<const opnd_t*>(p);
    }
  };
  auto read_ops = [&](int buf, int ks, int slot) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      av[slot][nb] = read_op(&a_lds[buf][(128 * wn + 32 * nb + lr) * ROW], ks);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      bv[slot][mb] = read_op(&b_lds[buf][(64 * wm + 32 * mb + lr) * ROW], ks);
  };
  auto mfma = [&](const opnd_t& a, const opnd_t& b, const f32x16_t& c) {
    if constexpr (FP8)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          __builtin_bit_cast(i32x8_t, a), __builtin_bit_cast(i32x8_t, b), c, 0, 0, 0, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                     __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  };
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    load(kt + 1);
    read_ops(buf, 0, 0);
#pragma unroll
    for (int ks = 0; ks < KSUB; ++ks) {
      if (ks + 1 < KSUB) read_ops(buf, ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int nb = i >> 1, mb = i & 1;
        acc[nb][mb] = mfma(av[ks & 1][nb], bv[ks & 1][mb], acc[nb][mb]);
        // the 8 stores ride along the second half of the k-steps (on the
        // last step they fill a buffer no one reads)
        constexpr int PER = 2 * NLD / KSUB;        // stores per k-step there
        if (ks >= KSUB / 2) {
          const int j = PER * (ks - KSUB / 2) + i * PER / 8;
          if ((i * PER) % 8 < PER) {
            const int c = tid + 512 * j;
            const bool isa = c < TN * CPR;
            const int cc = isa ? c : c - TN * CPR;
            const int row = cc / CPR, ch = cc % CPR;
            uint16_t* dst = isa ? &a_lds[buf ^ 1][row * ROW + 8 * ch]
                                : &b_lds[buf ^ 1][row * ROW + 8 * ch];
            *reinterpret_cast<u32x4_t*>(dst) = stg[j];
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }

  // ---- epilogue: lane column = token m, registers 4c..4c+3 = features
  // n0 + 128 wn + 32 nb + 8 c + 4 g + 0..3
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + 64 * wm + 32 * mb + lr;
    if (m >= M) continue;
    const int s = m % S;
    const int32_t* pm = pos + 4 * s;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int n = n0 + 128 * wn + 32 * nb + 8 * c4 + 4 * g;    // multiple of 4
        if (n >= N) continue;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[e] = acc[nb][mb][4 * c4 + e] * yscale + (bias ? bf16_lo((uint32_t)bias[n + e]) : 0.f);
        const int which = n / HD, hd = n % HD, d = hd % D;
        uint2 outw;
        if (which < 2) {
          const int a = d / DA, j0 = (d % DA) / 2;
          const float fp = (float)pm[a];
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const int j = j0 + pr;
            const float rev = rope_rev(fp, fr.hi[j], fr.lo[j]);
            const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
            const f32x2_t r = rope_rot(y[2 * pr], y[2 * pr + 1], cs, sn);
            y[2 * pr] = r[0];
            y[2 * pr + 1] = r[1];
          }
          outw.x = pack_f16x2(y[0], y[1]);
          outw.y = pack_f16x2(y[2], y[3]);
          uint16_t* dst = (which == 0 ? qo : ko) + (size_t)m * HD + hd;
          *reinterpret_cast<uint2*>(dst) = outw;
        } else {
          outw.x = pack_bf16x2(y[0], y[1]);
          outw.y = pack_bf16x2(y[2], y[3]);
          *reinterpret_cast<uint2*>(vo + (size_t)m * HD + hd) = outw;
        }
      }
  }
}

template <bool FP8>
static hipError_t launch_qkv(const QkvArgs& a) {
  const int M = a.B * a.S, N = 3 * a.H * a.D;
  const int ntn = (N + 255) / 256, ntm = (M + 255) / 256;
  const dim3 grid((unsigned)(ntn * ntm));
  const float ys = FP8 ? a.x_descale * a.w_descale : 1.0f;
  if (a.D == 128)
    hipLaunchKernelGGL((qkv_rope_proj_kernel<128, FP8>), grid, dim3(512), 0, a.stream, a.x, a.w,
                       a.bias, a.pos, a.q, a.k, a.v, M, N, a.C, a.S, a.H, ntn, a.freqs, ys);
  else
    hipLaunchKernelGGL((qkv_rope_proj_kernel<64, FP8>), grid, dim3(512), 0, a.stream, a.x, a.w,
                       a.bias, a.pos, a.q, a.k, a.v, M, N, a.C, a.S, a.H, ntn, a.freqs, ys);
  return hipGetLastError();
}

hipError_t launch_qkv_rope_proj(const QkvArgs& a) {
  return a.fp8 ? launch_qkv<true>(a) : launch_qkv<false>(a);
}

long long qkv_rope_proj_grid(int B, int S, int H, int D) {
  const long long M = (long long)B * S, N = 3LL * H * D;
  return ((N + 255) / 256) * ((M + 255) / 256);
}

}  // namespace klein
