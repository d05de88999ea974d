// RoPE-4D joint self-attention forward, FP8 E4M3 in / bf16 out, for gfx950.
//
// Inputs are OCP E4M3FN codes with per-tensor descales: value = code * dX.
// One workgroup of 8 waves owns one (batch, head, tile of 256 queries); each
// wave owns 32 queries and streams all keys in tiles of 64.  Every key is
// rotated and re-quantised on its way to LDS, and scores are fp8 MFMAs:
//
//   Q'' = e4m3(R(q_code) / sqrt 2)      (registers, once)
//   K'' = e4m3(R(k_code) / sqrt 2)      (LDS, per tile)
//   V   = v_code                        (LDS as V^T, per tile, bytes transposed)
//
// R is RoPE-4D on the decoded codes; a rotated pair component can grow by at
// most sqrt 2, so |R(code)| / sqrt 2 <= 448 and re-quantisation never leaves
// the E4M3 range.  The descales factor out: <q', k'> = 2 dq dk <Q'', K''>.
//
//   S^T  = K'' Q''^T                    v_mfma_f32_32x32x64_f8f6f4, fp32 acc
//   s    = S * 2 dq dk log2(e)/sqrt(D)  exp2 domain, fused into the exponent
//   p    = 2^(s - m), m the running row max, rescaled only when it grows by
//          more than TAU = 8, so p <= 2^8
//   P8   = e4m3(p * 448 / 2^8)          within range by construction
//   O^T += V^T P8^T                     fp8 MFMA, fp32 acc (64 keys per MFMA)
//   out  = O * dv * 2^8 / 448 / l,      l = sum of p (fp32)
//
// The score MFMA orientation, the permuted key order inside a 32-key block and
// the lane-pair row reductions are those of the bf16 kernel.  Unlike the bf16
// kernel this one is limited by VALU work (one fp8 MFMA covers 64 keys), so
// all eight waves run the same sequence -- stage tile t+1, S(t), softmax(t),
// O += P(t) V(t) -- with K'' and V^T double-buffered in LDS and one barrier
// per tile; the two waves sharing a SIMD interleave freely.
#include "klein_device.hpp"
#include "klein_launch.hpp"

namespace klein {

namespace {

constexpr float kInvSqrt2 = 0.70710678118654752f;
constexpr float kP8Scale = 448.0f / 256.0f;      // p <= 2^TAU = 256 maps to <= 448

__device__ __forceinline__ int key_to_row8(int kk) {
  const int g = kk >> 4, i = kk & 15;
  return ((i >> 2) << 3) + (g << 2) + (i & 3);
}

// Decode 16 E4M3 codes, rotate the 8 interleaved pairs (pairs j0 .. j0+7 of
// one axis block) at position p, scale by 1/sqrt 2 and re-encode (RNE).
__device__ __forceinline__ u32x4_t rope_requant16(u32x4_t x, int p, const float* whi,
                                                  const float* wlo) {
  const float fp = (float)p;
  u32x4_t y;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const auto v0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[w], false);   // bytes 0, 1
    const auto v1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[w], true);    // bytes 2, 3
    float c[2], s[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int jj = 2 * w + half;
      const float rev = __builtin_amdgcn_fractf(fp * whi[jj]) + fp * wlo[jj];
      s[half] = __builtin_amdgcn_sinf(rev) * kInvSqrt2;
      c[half] = __builtin_amdgcn_cosf(rev) * kInvSqrt2;
    }
    int outw = __builtin_amdgcn_cvt_pk_fp8_f32(v0[0] * c[0] - v0[1] * s[0],
                                               v0[0] * s[0] + v0[1] * c[0], 0, false);
    outw = __builtin_amdgcn_cvt_pk_fp8_f32(v1[0] * c[1] - v1[1] * s[1],
                                           v1[0] * s[1] + v1[1] * c[1], outw, true);
    y[w] = (uint32_t)outw;
  }
  return y;
}

// 4 x 4 byte transpose: in[i] holds bytes (d0..d3) of key i; out[j] holds
// byte j of keys 0..3.
__device__ __forceinline__ void transpose4x4(const uint32_t in[4], uint32_t out[4]) {
  const uint32_t a_lo = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);  // k0d0 k1d0 k0d1 k1d1
  const uint32_t a_hi = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);  // k0d2 k1d2 k0d3 k1d3
  const uint32_t b_lo = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t b_hi = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);
}

}  // namespace

template <int D>
__global__ __launch_bounds__(512) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const int32_t* __restrict__ pos, uint16_t* __restrict__ out, int S, int H, int nqt,
    RopeFreqs fr, float s_scale, float o_scale) {
  constexpr int BM = 256;              // queries per workgroup (8 waves x 32)
  constexpr int BN = 64;               // keys per tile
  constexpr int CPK = D / 16;          // 16-byte chunks per K row
  constexpr int KS = D / 64;           // fp8 MFMA k-steps of Q K^T
  constexpr int MB = D / 32;           // 32-row blocks of O^T
  constexpr int KROW = D + 16;         // LDS row stride of K'' (bytes), padded
  constexpr int VROW = BN + 16;        // LDS row stride of V^T (bytes), padded
  constexpr int DA = D / 4;            // channels per RoPE axis
  constexpr float TAU = 8.0f;
  constexpr int KTHREADS = BN * CPK;   // threads that stage K (one chunk each)
  constexpr int VTHREADS = (BN / 4) * (D / 4);   // threads that stage V (4 keys x 4 d)
  static_assert(KTHREADS <= 512 && VTHREADS <= 512, "staging split");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][BN * KROW];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[2][D * VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lr = lane & 31;

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = work % nqt;
  const int bh = work / nqt;
  const int h = bh % H, b = bh / H;
  const size_t rs = (size_t)H * D;                       // token stride (bytes)
  const size_t base = (size_t)b * S * rs + (size_t)h * D;
  const uint8_t* qb = q + base;
  const uint8_t* kbase = k + base;
  const uint8_t* vbase = v + base;
  const int rowb = (int)rs;

  // ---- Q'': this lane's query, dims 64 ks + 32 g + [0, 32) per k-step
  const int qrow = qt * BM + wave * 32 + lr;
  const int qload = qrow < S ? qrow : S - 1;
  i32x8_t qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      const int d0 = 64 * ks + 32 * g + 16 * hc;
      const int a = d0 / DA, j0 = (d0 % DA) / 2;
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qb + (size_t)qload * rs + d0);
      const u32x4_t y = rope_requant16(x, pos[4 * qload + a], &fr.hi[j0], &fr.lo[j0]);
#pragma unroll
      for (int w = 0; w < 4; ++w) qreg[ks][4 * hc + w] = (int)y[w];
    }
  }

  // ---- staging assignment
  const bool kst = tid < KTHREADS;
  const int kkey = tid / CPK, kc = tid % CPK;           // K: key, 16-byte chunk
  const int ka = (16 * kc) / DA, kj0 = ((16 * kc) % DA) / 2;
  float whi[8], wlo[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int j = kj0 + jj < D / 8 ? kj0 + jj : D / 8 - 1;
    whi[jj] = fr.hi[j];
    wlo[jj] = fr.lo[j];
  }
  const bool vst = tid < VTHREADS;
  const int vkq = tid % (BN / 4), vdq = tid / (BN / 4);  // V: keys 4 vkq.., d 4 vdq..
  const int voff_k = kkey * rowb + 16 * kc;
  const int voff_p = (kkey * 4 + ka) * 4;
  int voff_v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff_v[i] = (4 * vkq + i) * rowb + 4 * vdq;

  const int nkt = (S + BN - 1) / BN;
  u32x4_t kx = {0u, 0u, 0u, 0u};
  int kp = 0;
  uint32_t vx[4] = {0u, 0u, 0u, 0u};

  auto tile_rows = [&](int kt) {
    const int n = S - kt * BN;
    return n < 0 ? 0 : (n > BN ? BN : n);
  };
  // global -> registers (rows past S read as zero through the descriptors)
  auto load_tile = [&](int kt) {
    const int n = tile_rows(kt);
    if (kst) {
      const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(kbase + (size_t)kt * BN * rs, n * rowb);
      const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(pos + (size_t)kt * BN * 4, n * 16);
      kx = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, voff_k, 0, 0));
      kp = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, voff_p, 0, 0);
    }
    if (vst) {
      const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(vbase + (size_t)kt * BN * rs, n * rowb);
#pragma unroll
      for (int i = 0; i < 4; ++i) vx[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff_v[i], 0, 0);
    }
  };
  // registers -> LDS: K'' at its permuted row, V transposed to V^T
  auto stage_tile = [&](int buf) {
    if (kst) {
      const int row = (kkey & ~31) + key_to_row8(kkey & 31);
      *reinterpret_cast<u32x4_t*>(&k_lds[buf][row * KROW + 16 * kc]) =
          rope_requant16(kx, kp, whi, wlo);
    }
    if (vst) {
      uint32_t t4[4];
      transpose4x4(vx, t4);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint32_t*>(&v_lds[buf][(4 * vdq + j) * VROW + 4 * vkq]) = t4[j];
    }
  };

  f32x16_t o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = (f32x16_t){};
  float m_run = kNegInf, l_run = 0.f;

  load_tile(0);
  stage_tile(0);
  load_tile(1);
  __syncthreads();

  for (int t = 0; t < nkt; ++t) {
    const int buf = t & 1;
    // ---- S^T = K'' Q''^T: two 32-key blocks, KS k-steps of 64 dims
    f32x16_t sc[2];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
      sc[kbk] = (f32x16_t){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint8_t* src = &k_lds[buf][(32 * kbk + lr) * KROW + 64 * ks + 32 * g];
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(src);
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(src + 16);
        const i32x8_t a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sc[kbk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qreg[ks], sc[kbk], 0, 0,
                                                                  0, 0, 0, 0);
      }
    }
    // ---- stage tile t+1 into the other buffer while the MFMAs run
    stage_tile(buf ^ 1);

    // ---- softmax step on raw scores (scaled into the exp2 domain)
    if (t * BN + BN > S) {
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (t * BN + 32 * kbk + 16 * g + i >= S) sc[kbk][i] = kNegInf;
    }
    float m8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      m8[i] = __builtin_fmaxf(__builtin_fmaxf(sc[0][i], sc[0][i + 8]),
                              __builtin_fmaxf(sc[1][i], sc[1][i + 8]));
#pragma unroll
    for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) m8[i] = __builtin_fmaxf(m8[i], m8[i + w]);
    const float mx = pair_max(m8[0]) * s_scale;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU)) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
    }
    // p = 2^(raw * s_scale - m); P8 packed in key order 16g + i, 32 + 16g + i
    float ls4[4] = {0.f, 0.f, 0.f, 0.f};
    i32x8_t pb;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][4 * w + e], s_scale, -m_run));
          ls4[e] += pv[e];
        }
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0] * kP8Scale, pv[1] * kP8Scale, 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2] * kP8Scale, pv[3] * kP8Scale, word, true);
        pb[4 * kbk + w] = word;
      }
    l_run += (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);

    // ---- O^T += V^T P8^T: one 64-key MFMA per 32-row block of D
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint8_t* src = &v_lds[buf][(32 * mb + lr) * VROW + 16 * g];
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(src);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(src + 32);
      const i32x8_t a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      o[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, o[mb], 0, 0, 0, 0, 0, 0);
    }
    load_tile(t + 2);
    __syncthreads();
  }

  // ---- epilogue: O * dv * 2^8/448 / l -> bf16
  const float inv = o_scale / pair_sum(l_run);
  if (qrow < S) {
    uint16_t* orow = out + (size_t)b * S * rs + (size_t)h * D + (size_t)qrow * rs;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * mb + 8 * i4 + 4 * g;
        uint2 w;
        w.x = pack_bf16x2(o[mb][4 * i4] * inv, o[mb][4 * i4 + 1] * inv);
        w.y = pack_bf16x2(o[mb][4 * i4 + 2] * inv, o[mb][4 * i4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
  }
}

template <int D>
static hipError_t launch_fp8(const LaunchArgs& a) {
  const int nqt = (a.S + 255) / 256;
  const long long n = (long long)a.B * a.H * nqt;
  // scores: <q', k'> = 2 dq dk <Q'', K''>, times log2(e)/sqrt(D)
  const float s_scale = 2.0f * a.descale[0] * a.descale[1] * a.qscale_log2;
  const float o_scale = a.descale[2] / (448.0f / 256.0f);
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D>), dim3((unsigned)n), dim3(512), 0, a.stream,
                     (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, a.pos,
                     (uint16_t*)a.out, a.S, a.H, nqt, a.freqs, s_scale, o_scale);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_fp8(const LaunchArgs& a) {
  if (a.D == 128) return launch_fp8<128>(a);
  return launch_fp8<64>(a);
}

long long attn_fwd_fp8_grid(int B, int S, int H) {
  return (long long)B * H * ((S + 255) / 256);
}

}  // namespace klein
