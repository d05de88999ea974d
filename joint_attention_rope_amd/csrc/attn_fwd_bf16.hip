// RoPE-4D joint self-attention forward, bf16 in / bf16 out, for gfx950.
//
// One workgroup owns one (batch, head, tile of BM = 32*NW queries); each of its
// NW waves owns 32 of those queries and streams every key of the sequence
// (no mask: all tokens attend to all tokens).  Per key tile of BN = 64 tokens:
//
//   1. the tile of K and V is read from HBM with 16-byte loads (issued one tile
//      ahead, so the loads fly while the previous tile is computed);
//   2. K is rotated by RoPE-4D in registers as it is written to LDS; V is
//      transposed in registers and written to LDS as V^T;
//   3. S^T = K' Q'^T on v_mfma_f32_32x32x16_bf16: keys are the MFMA rows,
//      queries the columns, so one lane holds 16 keys of one query and the
//      row max / row sum need a single exchange with the lane 32 apart;
//   4. online softmax in the exp2 domain (Q carries log2(e)/sqrt(D));
//   5. O^T += V^T P^T on the same MFMA, with P taken straight from the S^T
//      accumulators (converted to bf16) as the B operand.
//
// Keys of the tile are stored in LDS in a permuted row order so that the
// accumulator register i of a lane in half g (lanes 32g..32g+31) holds key
// 16g + i of the 32-key block; P's registers 8j..8j+7 then pair with the 8
// contiguous keys 16g + 8j .. 16g + 8j + 7 of a V^T row, one 16-byte LDS read.
//
// LDS bank spreading: K rows are padded by 16 bytes (the 16 lanes of one
// 16-byte read phase hit 16 consecutive rows); V^T rows (64 keys, 128 bytes)
// are unpadded and their 8-key chunks are XOR-swizzled by
// (d ^ (d >> 3)) & 7, which keeps both the MFMA operand reads (16
// consecutive d) and the transposing stores spread over the banks.
#include "klein_device.hpp"
#include "klein_launch.hpp"

namespace klein {

// LDS row of key kk (0..31) of a 32-key block: the MFMA output row r holds
// key 16*((r/4)&1) + 4*(r/8) + (r%4); this is the inverse map.
__device__ __forceinline__ int key_to_row(int kk) {
  const int g = kk >> 4, i = kk & 15;
  return ((i >> 2) << 3) + (g << 2) + (i & 3);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ out, int S, int H, int nqt, RopeFreqs fr, float qscale) {
  constexpr int BM = 32 * NW;          // queries per workgroup
  constexpr int BN = 64;               // keys per tile
  constexpr int NT = 64 * NW;          // threads
  constexpr int CPR = D / 8;           // 16-byte chunks per token row
  constexpr int KPT = BN * CPR / NT;   // keys per thread in the tile loads
  constexpr int KS = D / 16;           // MFMA k-steps of Q K^T
  constexpr int MB = D / 32;           // 32-row blocks of O^T
  constexpr int KROW = D + 8;          // LDS row stride of K (bf16), padded
  constexpr int VROW = BN;             // LDS row stride of V^T (bf16), swizzled
  constexpr int DA = D / 4;            // channels per RoPE axis
  static_assert(KPT >= 1 && (BN * CPR) % NT == 0, "tile/thread mismatch");
  static_assert(NT % CPR == 0, "thread row split");
  static_assert(KPT == 1 || KPT % 2 == 0, "V^T store packs key pairs");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BN * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lr = lane & 31;

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = work % nqt;
  const int bh = work / nqt;
  const int h = bh % H, b = bh / H;
  const size_t rs = (size_t)H * D;                       // token stride
  const size_t base = (size_t)b * S * rs + (size_t)h * D;
  const uint16_t* qb = q + base;
  const uint16_t* kb = k + base;
  const uint16_t* vb = v + base;

  // ---- this lane's query: rotate, scale by log2(e)/sqrt(D), keep in VGPRs
  const int qrow = qt * BM + wave * 32 + lr;
  const bool qvalid = qrow < S;
  bf16x8_t qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int d0 = 16 * ks + 8 * g;
    const int a = d0 / DA, j0 = (d0 % DA) / 2;
    u32x4_t x = {0u, 0u, 0u, 0u};
    int p = 0;
    if (qvalid) {
      x = *reinterpret_cast<const u32x4_t*>(qb + (size_t)qrow * rs + d0);
      p = pos[4 * qrow + a];
    }
    qreg[ks] = __builtin_bit_cast(bf16x8_t, rope_chunk(x, p, &fr.hi[j0], &fr.lo[j0], qscale));
  }

  // ---- tile-load assignment: chunk lc of keys lk .. lk+KPT-1
  const int lc = tid % CPR;
  const int lk = (tid / CPR) * KPT;
  const int la = (8 * lc) / DA, lj0 = ((8 * lc) % DA) / 2;
  float whi[4], wlo[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) { whi[jj] = fr.hi[lj0 + jj]; wlo[jj] = fr.lo[lj0 + jj]; }

  f32x16_t o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = (f32x16_t){};
  float m_run = kNegInf, l_run = 0.f;

  const int nkt = (S + BN - 1) / BN;
  u32x4_t kx[KPT], vx[KPT];
  int kp[KPT];

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int it = 0; it < KPT; ++it) {
      const int key = kt * BN + lk + it;
      if (key < S) {
        kx[it] = *reinterpret_cast<const u32x4_t*>(kb + (size_t)key * rs + 8 * lc);
        vx[it] = *reinterpret_cast<const u32x4_t*>(vb + (size_t)key * rs + 8 * lc);
        kp[it] = pos[4 * key + la];
      } else {
        kx[it] = (u32x4_t){0u, 0u, 0u, 0u};
        vx[it] = (u32x4_t){0u, 0u, 0u, 0u};
        kp[it] = 0;
      }
    }
  };

  load_tile(0);
  for (int kt = 0; kt < nkt; ++kt) {
    // ---- K: rotate and store at the permuted row; V: transpose to V^T
#pragma unroll
    for (int it = 0; it < KPT; ++it) {
      const int key = lk + it;
      const int row = (key & ~31) + key_to_row(key & 31);
      *reinterpret_cast<u32x4_t*>(&k_lds[row * KROW + 8 * lc]) =
          rope_chunk(kx[it], kp[it], whi, wlo, 1.0f);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * lc + e;
      uint16_t* vrow = &v_lds[d * VROW];
      const int sw = (d ^ (d >> 3)) & 7;
      if constexpr (KPT == 1) {
        const uint32_t w = vx[0][e >> 1];
        vrow[(((lk >> 3) ^ sw) << 3) + (lk & 7)] = (uint16_t)((e & 1) ? (w >> 16) : w);
      } else {
#pragma unroll
        for (int it = 0; it < KPT; it += 2) {
          const int key = lk + it;
          const uint32_t w0 = vx[it][e >> 1], w1 = vx[it + 1][e >> 1];
          const uint32_t pk = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                      : ((w0 & 0xffffu) | (w1 << 16));
          *reinterpret_cast<uint32_t*>(&vrow[(((key >> 3) ^ sw) << 3) + (key & 7)]) = pk;
        }
      }
    }
    __syncthreads();
    if (kt + 1 < nkt) load_tile(kt + 1);

    // ---- S^T = K' Q'^T  (two 32-key blocks)
    f32x16_t s[2];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
      s[kbk] = (f32x16_t){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            &k_lds[(32 * kbk + lr) * KROW + 16 * ks + 8 * g]);
        s[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s[kbk], 0, 0, 0);
      }
    }
    // ---- keys beyond S in the last tile do not exist
    if (kt * BN + BN > S) {
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * BN + 32 * kbk + 16 * g + i >= S) s[kbk][i] = kNegInf;
    }
    // ---- online softmax (exp2 domain)
    float mx = kNegInf;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, s[kbk][i]);
    mx = pair_max(mx);
    const float m_new = __builtin_fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
    uint32_t pw[2][8];
    float ls = 0.f;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(s[kbk][2 * w] - m_new);
        const float p1 = __builtin_amdgcn_exp2f(s[kbk][2 * w + 1] - m_new);
        ls += p0 + p1;
        pw[kbk][w] = pack_bf16x2(p0, p1);
      }
    l_run += ls;
    // ---- O^T += V^T P^T
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
              &v_lds[d * VROW + ((kc ^ ((d ^ (d >> 3)) & 7)) << 3)]);
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[mb], 0, 0, 0);
        }
      }
    __syncthreads();
  }

  // ---- epilogue: O / l, bf16, store (lane holds channels 32mb + 8(i/4) + 4g + i%4)
  const float inv = 1.0f / pair_sum(l_run);
  if (qvalid) {
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

template <int D, int NW>
static hipError_t launch_bf16(const LaunchArgs& a) {
  constexpr int BM = 32 * NW;
  const int nqt = (a.S + BM - 1) / BM;
  const long long n = (long long)a.B * a.H * nqt;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW>), dim3((unsigned)n), dim3(64 * NW), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     a.pos, (uint16_t*)a.out, a.S, a.H, nqt, a.freqs, a.qscale_log2);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_bf16(const LaunchArgs& a) {
  if (a.D == 128) return launch_bf16<128, 8>(a);
  return launch_bf16<64, 8>(a);
}

long long attn_fwd_bf16_grid(int B, int S, int H) {
  const int BM = 32 * 8;
  return (long long)B * H * ((S + BM - 1) / BM);
}

}  // namespace klein
