// RoPE-4D joint self-attention forward, bf16 in / bf16 out, for gfx950.
//
// One workgroup owns one (batch, head, tile of BM = 256 queries) and streams
// every key of the sequence (no mask: all tokens attend to all tokens) in tiles
// of BN = 64 keys.  It runs 8 waves, 32 queries each, two waves per SIMD:
// group A = waves 0-3 and group B = waves 4-7, so each SIMD holds one wave of
// each group.  The groups ping-pong: while one group issues its MFMAs, the
// other does its VALU work on the same SIMDs, and a workgroup barrier ends
// each phase:
//
//   phase X_t:  A: O^T += V(t-1)^T P(t-1)^T ; S(t) = K'(t) Q'^T      [MFMA]
//               B: P(t-1) = softmax step of S(t-1); stage V(t), half of K(t+1)
//   phase Y_t:  A: P(t) = softmax step of S(t); stage the other half of K(t+1)
//               B: O^T += V(t-1)^T P(t-1)^T ; S(t) = K'(t) Q'^T      [MFMA]
//
// "Staging" moves a tile from registers (loaded from HBM a phase earlier) to
// LDS: K is rotated by RoPE-4D on the way, V is transposed to V^T.  K and V^T
// are double-buffered in LDS (tile t in buffer t & 1).
//
// Precision: the rotated Q' (times log2(e)/sqrt(D)) and K' are rounded to
// fp16, not bf16, and S^T = K' Q'^T runs on v_mfma_f32_32x32x16_f16 (same
// rate as bf16).  With bf16 the rounding of Q' and K' alone reaches a relative
// L2 error of ~5e-3 on key channels with x8 outliers; fp16's three extra
// mantissa bits cut it about 2x.  The price is range: elementwise |k| must
// stay below ~46000 and |q| below ~360000 (fp16 max 65504 after the
// rotation's sqrt 2 and the softmax scale).  P and V stay bf16 for O^T += V^T P^T.
//
// MFMA orientation: S^T = K' Q'^T puts keys on the MFMA rows and queries on
// its columns, so a lane holds 16 keys of one query and the row max / row sum
// need one exchange with the lane 32 apart.  O^T += V^T P^T
// (v_mfma_f32_32x32x16_bf16) uses P straight from the S^T accumulators (as
// bf16) as the B operand.  Keys of a tile sit in LDS in a permuted row order so that
// accumulator register i of a lane in half g holds key 16g + i of its 32-key
// block; P's registers 8j..8j+7 then pair with the 8 contiguous keys
// 16g + 8j .. 16g + 8j + 7 of a V^T row, one 16-byte LDS read.
//
// Softmax runs in the exp2 domain (Q carries log2(e)/sqrt(D)).  O and l are
// rescaled only when a row's running max grows by more than TAU = 8, so
// p = 2^(s - m) <= 2^8 in between; the final O / l is the same either way.
//
// LDS bank spreading: K rows are padded by 16 bytes (the 16 lanes of one
// 16-byte read phase hit 16 consecutive rows); V^T rows (64 keys, 128 bytes)
// are unpadded and their 8-key chunks are XOR-swizzled by (d ^ (d >> 3)) & 7,
// which keeps both the MFMA operand reads and the transposing stores spread.
#include "klein_device.hpp"
#include "klein_launch.hpp"

namespace klein {

// LDS row of key kk (0..31) of a 32-key block: the MFMA output row r holds
// key 16*((r/4)&1) + 4*(r/8) + (r%4); this is the inverse map.
__device__ __forceinline__ int key_to_row(int kk) {
  const int g = kk >> 4, i = kk & 15;
  return ((i >> 2) << 3) + (g << 2) + (i & 3);
}

template <int D>
__global__ __launch_bounds__(512) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ out, int S, int H, int nqt, RopeFreqs fr, float qscale) {
  constexpr int BM = 256;              // queries per workgroup (8 waves x 32)
  constexpr int BN = 64;               // keys per tile
  constexpr int CPR = D / 8;           // 16-byte chunks per token row
  constexpr int KPV = BN * CPR / 256;  // keys per thread when a group stages V
  constexpr int KPK = 32 * CPR / 256;  // keys per thread when a group stages half of K
  constexpr int KS = D / 16;           // MFMA k-steps of Q K^T
  constexpr int MB = D / 32;           // 32-row blocks of O^T
  constexpr int KROW = D + 8;          // LDS row stride of K (bf16), padded
  constexpr int VROW = BN;             // LDS row stride of V^T (bf16), swizzled
  constexpr int DA = D / 4;            // channels per RoPE axis
  constexpr float TAU = 8.0f;
  static_assert(KPV >= 2 && KPV % 2 == 0 && KPK >= 1, "tile/thread split");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BN * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lr = lane & 31;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);   // 0 = A, 1 = B (wave-uniform)
  const int gt = tid & 255;            // thread index inside the group

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = work % nqt;
  const int bh = work / nqt;
  const int h = bh % H, b = bh / H;
  const size_t rs = (size_t)H * D;                       // token stride
  const size_t base = (size_t)b * S * rs + (size_t)h * D;
  const uint16_t* qb = q + base;
  const uint16_t* kb = k + base;
  const uint16_t* vb = v + base;

  // ---- this lane's query: rotate, scale by log2(e)/sqrt(D), keep in VGPRs.
  // Rows past S load row S-1 (in bounds) and are never stored.
  const int qrow = qt * BM + wave * 32 + lr;
  const int qload = qrow < S ? qrow : S - 1;
  f16x8_t qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int d0 = 16 * ks + 8 * g;
    const int a = d0 / DA, j0 = (d0 % DA) / 2;
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qb + (size_t)qload * rs + d0);
    qreg[ks] = __builtin_bit_cast(
        f16x8_t, rope_chunk<true>(x, pos[4 * qload + a], &fr.hi[j0], &fr.lo[j0], qscale));
  }

  // ---- staging assignment (per group of 256 threads): chunk lc of a row
  const int lc = gt % CPR;
  const int vk0 = (gt / CPR) * KPV;    // V: keys vk0 .. vk0+KPV-1 of the tile
  const int kk0 = (gt / CPR) * KPK;    // K: keys kk0 .. kk0+KPK-1 of a half tile
  const int la = (8 * lc) / DA, lj0 = ((8 * lc) % DA) / 2;
  float whi[4], wlo[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) { whi[jj] = fr.hi[lj0 + jj]; wlo[jj] = fr.lo[lj0 + jj]; }

  const int nkt = (S + BN - 1) / BN;
  u32x4_t kx[KPK], vx[KPV];
  int kp[KPK];

  // Global -> registers through buffer loads.  Each tile gets a descriptor
  // whose base is the tile's first row and whose size covers only the rows
  // that exist, so the hardware returns zeros for rows past S (no clamping and
  // no per-load address arithmetic: the per-thread byte offsets below are
  // fixed for the whole loop).
  const int rowb = (int)(rs * 2);                          // bytes per token row
  int voff_k[KPK], voff_p[KPK], voff_v[KPV];
#pragma unroll
  for (int it = 0; it < KPK; ++it) {
    voff_k[it] = (32 * grp + kk0 + it) * rowb + 16 * lc;
    voff_p[it] = ((32 * grp + kk0 + it) * 4 + la) * 4;
  }
#pragma unroll
  for (int it = 0; it < KPV; ++it) voff_v[it] = (vk0 + it) * rowb + 16 * lc;
  auto tile_rows = [&](int kt) {
    const int n = S - kt * BN;
    return n < 0 ? 0 : (n > BN ? BN : n);
  };
  auto load_k_half = [&](int kt, int half) {
    const int n = tile_rows(kt);
    const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(kb + (size_t)kt * BN * rs, n * rowb);
    const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(pos + (size_t)kt * BN * 4, n * 16);
    (void)half;   // the offsets already select this group's half
#pragma unroll
    for (int it = 0; it < KPK; ++it) {
      kx[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, voff_k[it], 0, 0));
      kp[it] = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, voff_p[it], 0, 0);
    }
  };
  auto load_v = [&](int kt) {
    const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(vb + (size_t)kt * BN * rs, tile_rows(kt) * rowb);
#pragma unroll
    for (int it = 0; it < KPV; ++it)
      vx[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v[it], 0, 0));
  };
  // Registers -> LDS: K rotated, at its permuted row; V transposed to V^T.
  auto stage_k_half = [&](int buf, int half) {
#pragma unroll
    for (int it = 0; it < KPK; ++it) {
      const int key = kk0 + it;                         // 0..31 within the half
      const int row = 32 * half + key_to_row(key);
      *reinterpret_cast<u32x4_t*>(&k_lds[buf][row * KROW + 8 * lc]) =
          rope_chunk<true>(kx[it], kp[it], whi, wlo, 1.0f);
    }
  };
  auto stage_v = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * lc + e;
      uint16_t* vrow = &v_lds[buf][d * VROW];
      const int sw = (d ^ (d >> 3)) & 7;
#pragma unroll
      for (int it = 0; it < KPV; it += 2) {
        const int key = vk0 + it;
        const uint32_t w0 = vx[it][e >> 1], w1 = vx[it + 1][e >> 1];
        const uint32_t pk = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                    : ((w0 & 0xffffu) | (w1 << 16));
        *reinterpret_cast<uint32_t*>(&vrow[(((key >> 3) ^ sw) << 3) + (key & 7)]) = pk;
      }
    }
  };

  f32x16_t o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = (f32x16_t){};
  f32x16_t sc[2];
  uint32_t pw[2][8];
  float m_run = kNegInf, l_run = 0.f;

  // S^T = K'(tile in buf) Q'^T, two 32-key blocks
  auto gemm1 = [&](int buf) {
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) sc[kbk] = (f32x16_t){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) {
        const f16x8_t a = *reinterpret_cast<const f16x8_t*>(
            &k_lds[buf][(32 * kbk + lr) * KROW + 16 * ks + 8 * g]);
        sc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qreg[ks], sc[kbk], 0, 0, 0);
      }
  };
  // O^T += V^T(tile in buf) P^T
  auto gemm2 = [&](int buf) {
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_t pv = {pw[kbk][4 * j], pw[kbk][4 * j + 1], pw[kbk][4 * j + 2], pw[kbk][4 * j + 3]};
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int d = 32 * mb + lr;
          const int kc = 4 * kbk + 2 * g + j;
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
              &v_lds[buf][d * VROW + ((kc ^ ((d ^ (d >> 3)) & 7)) << 3)]);
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[mb], 0, 0, 0);
        }
      }
  };
  // P(t) from S(t): mask keys past S, lazy rescale, exp2, row sum, pack to bf16
  auto softmax = [&](int t) {
    if (t * BN + BN > S) {
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (t * BN + 32 * kbk + 16 * g + i >= S) sc[kbk][i] = kNegInf;
    }
    // row max as a balanced tree (the VALU wave has no partner to hide
    // the latency of a serial chain)
    float m8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      m8[i] = __builtin_fmaxf(__builtin_fmaxf(sc[0][i], sc[0][i + 8]),
                              __builtin_fmaxf(sc[1][i], sc[1][i + 8]));
#pragma unroll
    for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) m8[i] = __builtin_fmaxf(m8[i], m8[i + w]);
    const float mx = pair_max(m8[0]);
    if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU)) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
    }
    // p = 2^(s - m); four independent partial row sums
    float ls4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(sc[kbk][2 * w] - m_run);
        const float p1 = __builtin_amdgcn_exp2f(sc[kbk][2 * w + 1] - m_run);
        ls4[(2 * w) & 3] += p0;
        ls4[(2 * w + 1) & 3] += p1;
        pw[kbk][w] = pack_bf16x2(p0, p1);
      }
    const float ls = (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
    l_run += ls;
  };

  // ---- prologue: K(0) into LDS (half per group); each group pre-loads what
  // its first VALU phase stages (A: K(1) half 0; B: V(0), K(1) half 1)
  load_k_half(0, grp);
  stage_k_half(0, grp);
  load_k_half(1, grp);
  if (grp == 1) load_v(0);
  __syncthreads();

  // Each group runs its own copy of the loop, so values one group keeps
  // across phases never occupy registers in the other.  Both copies execute
  // exactly two barriers per iteration, in step.  MFMA phases hold only LDS
  // reads and MFMAs; a group issues the global loads for its next VALU phase
  // at the end of its current one, so they fly during its MFMA phase.
  if (grp == 0) {
    for (int t = 0; t <= nkt; ++t) {
      // X_t: MFMA phase
      if (t >= 1) gemm2((t - 1) & 1);
      if (t < nkt) gemm1(t & 1);
      __syncthreads();
      // Y_t: VALU phase
      if (t < nkt) {
        softmax(t);
        stage_k_half((t + 1) & 1, 0);                // K(t+1) half 0
        load_k_half(t + 2, 0);                       // staged in Y_{t+1}
      }
      __syncthreads();
    }
  } else {
    for (int t = 0; t <= nkt; ++t) {
      // X_t: VALU phase
      if (t >= 1) softmax(t - 1);
      if (t < nkt) {
        stage_v(t & 1);                              // V(t)
        stage_k_half((t + 1) & 1, 1);                // K(t+1) half 1
        load_v(t + 1);                               // staged in X_{t+1}
        load_k_half(t + 2, 1);
      }
      __syncthreads();
      // Y_t: MFMA phase
      if (t >= 1) gemm2((t - 1) & 1);
      if (t < nkt) gemm1(t & 1);
      __syncthreads();
    }
  }

  // ---- epilogue: O / l, bf16, store (lane holds channels 32mb + 8(i/4) + 4g + i%4)
  const float inv = 1.0f / pair_sum(l_run);
  if (qrow < S) {
    uint16_t* orow = out + base + (size_t)qrow * rs;
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
static hipError_t launch_bf16(const LaunchArgs& a) {
  constexpr int BM = 256;
  const int nqt = (a.S + BM - 1) / BM;
  const long long n = (long long)a.B * a.H * nqt;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D>), dim3((unsigned)n), dim3(512), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     a.pos, (uint16_t*)a.out, a.S, a.H, nqt, a.freqs, a.qscale_log2);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_bf16(const LaunchArgs& a) {
  if (a.D == 128) return launch_bf16<128>(a);
  return launch_bf16<64>(a);
}

long long attn_fwd_bf16_grid(int B, int S, int H) {
  const int BM = 256;
  return (long long)B * H * ((S + BM - 1) / BM);
}

}  // namespace klein
