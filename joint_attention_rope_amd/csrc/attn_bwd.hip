// Backward of the RoPE-4D joint self-attention, bf16 in / bf16 gradients, for
// gfx950.  Per batch entry and head, with q'_i = R_i q_i, k'_j = R_j k_j,
// s_ij = <q'_i, k'_j> / sqrt(D), p = softmax_j(s), o = p v, and dout = dL/do:
//
//   dv_j = sum_i p_ij dout_i                 dp_ij = <dout_i, v_j>
//   ds_ij = p_ij (dp_ij - delta_i),          delta_i = <dout_i, o_i>
//   dq_i = R_i^T (1/sqrt(D)) sum_j ds_ij k'_j,  dk_j = R_j^T (1/sqrt(D)) sum_i ds_ij q'_i
//
// with p recomputed from the scores and the forward's log-sum-exp lse_i
// (p_ij = exp(s_ij - lse_i)).  Three kernels, no atomics:
//
//   prep:  q'' = fp16(R q * log2(e)/sqrt(D)) and k' = fp16(R k), exactly the
//          values the forward kernel forms on chip (so the recomputed scores
//          match the ones lse was taken over), delta_i, and the squared row
//          norms of dout and v;
//   scale: per (batch, head), the power of two 2^e that puts the largest
//          possible |ds| near 2^14 (below);
//   dk/dv: one workgroup per 256 keys (8 waves x 32 keys, two per SIMD; the
//          keys on the MFMA columns), streaming all queries in tiles of 32
//          (64 for D = 64);
//   dq:    one workgroup per 256 queries (8 waves x 32 queries, two per SIMD),
//          streaming all keys in tiles of 64.
//
// Range of ds.  ds enters its MFMAs as fp16, whose normal range (2^-14 ..
// 65504) is far narrower than fp32's: with small gradients (|dout| ~ 1e-4
// and below, common in fine-tuning) most ds would fall into fp16's subnormals
// or to zero, with large ones they would overflow.  So both gradient kernels
// work with 2^e p and 2^e ds instead: e is added to the score MFMA's initial
// value (-lse2 + e), so exp2 already returns 2^e p, and the epilogues
// multiply the accumulated gradients by 2^-e, exactly.  Since sum_j p_ij = 1,
// |delta_i| <= max_j |dp_ij|, and |ds_ij| <= 2 max_i |dout_i| max_j |v_j|
// (Cauchy-Schwarz); e puts that bound just under 2^14, a quarter of fp16's
// largest value.  The same e serves the whole (batch, head), because dk and
// dv sum over all its queries.
//
// Each MFMA keeps the fast operand layout of the forward kernel: the tile
// that streams through LDS is the A operand, read row-wise (rows of a
// 32-row block stored in the permuted order of key_to_row, so that
// accumulator register i of lane half g belongs to row 16g + i) or
// transposed with ds_read_b64_tr_b16; the per-lane operand (this wave's keys
// or queries) sits in registers.  The products whose k dimension is the
// streamed rows take P or dS straight from the score accumulators as the B
// operand, the k order matching the transposed reads.  The gradients leave
// through the rotation's transpose (rotation by -p) in registers: in the
// accumulators a lane holds the interleaved channel pairs (d, d+1) of one
// token in adjacent registers.
#include <cmath>
#include <type_traits>

#include "klein_device.hpp"
#include "klein_launch.hpp"

namespace klein {

// one channel pair of an output gradient, rotated back: R(-phi) (x, y)
__device__ __forceinline__ void rotate_back(float& x, float& y, int p, float whi, float wlo) {
  const float fp = (float)p;
  const float rev = rope_rev(fp, whi, wlo);
  const float s = __builtin_amdgcn_sinf(rev), c = __builtin_amdgcn_cosf(rev);
  const float a = x, b = y;
  x = a * c + b * s;
  y = b * c - a * s;
}

// ---------------------------------------------------------------- prep
// One thread per 16-byte chunk (8 channels) of a token row of one head.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
    uint16_t* __restrict__ qr, uint16_t* __restrict__ kr, float* __restrict__ delta,
    float* __restrict__ norm2, int S, int H, long long nchunks, RopeFreqs fr, float qscale) {
  constexpr int CPR = D / 8, DA = D / 4;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nchunks) return;            // whole rows (CPR aligned lanes) leave together
  const long long row = idx / CPR;       // (b S + s) H + h
  const int c = (int)(idx % CPR);
  const int h = (int)(row % H);
  const long long bs = row / H;
  const int s = (int)(bs % S), b = (int)(bs / S);
  const size_t off = (size_t)idx * 8;
  const int a = (8 * c) / DA, j0 = ((8 * c) % DA) / 2;
  const int p = pos[4 * s + a];
  *reinterpret_cast<u32x4_t*>(qr + off) =
      rope_chunk<true>(*reinterpret_cast<const u32x4_t*>(q + off), p, &fr.hi[j0], &fr.lo[j0], qscale);
  *reinterpret_cast<u32x4_t*>(kr + off) =
      rope_chunk<true>(*reinterpret_cast<const u32x4_t*>(k + off), p, &fr.hi[j0], &fr.lo[j0], 1.0f);
  const u32x4_t ov = *reinterpret_cast<const u32x4_t*>(o + off);
  const u32x4_t dv = *reinterpret_cast<const u32x4_t*>(dout + off);
  const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(v + off);
  float sum = 0.f, dd = 0.f, vn = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    sum += bf16_lo(ov[w]) * bf16_lo(dv[w]) + bf16_hi(ov[w]) * bf16_hi(dv[w]);
    dd += bf16_lo(dv[w]) * bf16_lo(dv[w]) + bf16_hi(dv[w]) * bf16_hi(dv[w]);
    vn += bf16_lo(vv[w]) * bf16_lo(vv[w]) + bf16_hi(vv[w]) * bf16_hi(vv[w]);
  }
#pragma unroll
  for (int m = 1; m < CPR; m <<= 1) {
    sum += __shfl_xor(sum, m);
    dd += __shfl_xor(dd, m);
    vn += __shfl_xor(vn, m);
  }
  if (c == 0) {
    const size_t r = ((size_t)b * H + h) * S + s;
    delta[r] = sum;
    norm2[r] = dd;                                   // |dout_i|^2 [B][H][S], then
    norm2[nchunks / CPR + r] = vn;                   // |v_i|^2 [B][H][S]
  }
}

// ---------------------------------------------------------------- scale
// One workgroup per (batch, head): e = 14 - ceil(log2(2 max|dout_i| max|v_j|))
// (see "Range of ds" above), clamped to [-100, 100]; as a float, in
// escale[bh].  A zero bound (dout or v all zero, so ds = 0) gives e = 14.
__global__ __launch_bounds__(256) void attn_bwd_scale_kernel(const float* __restrict__ norm2,
                                                             float* __restrict__ escale, int S,
                                                             long long rows) {
  __shared__ float red[2][4];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* nd = norm2 + (size_t)bh * S;
  const float* nv = nd + rows;
  float md = 0.f, mv = 0.f;
  for (int i = tid; i < S; i += 256) {
    md = __builtin_fmaxf(md, nd[i]);
    mv = __builtin_fmaxf(mv, nv[i]);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    md = __builtin_fmaxf(md, __shfl_xor(md, m));
    mv = __builtin_fmaxf(mv, __shfl_xor(mv, m));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = md;
    red[1][tid >> 6] = mv;
  }
  __syncthreads();
  if (tid == 0) {
    md = __builtin_fmaxf(__builtin_fmaxf(red[0][0], red[0][1]), __builtin_fmaxf(red[0][2], red[0][3]));
    mv = __builtin_fmaxf(__builtin_fmaxf(red[1][0], red[1][1]), __builtin_fmaxf(red[1][2], red[1][3]));
    // 2 sqrt(md) sqrt(mv), 1/256 larger for the rounding of the norms
    const float bound = 2.f * __builtin_sqrtf(md) * __builtin_sqrtf(mv) * (1.f + 1.f / 256.f);
    int e = 14;
    if (!(bound < __builtin_huge_valf())) {
      e = -100;
    } else if (bound > 0.f) {
      int ex = 0;
      (void)__builtin_frexpf(bound, &ex);             // bound < 2^ex
      e = 14 - ex;
      e = e < -100 ? -100 : (e > 100 ? 100 : e);
    }
    escale[bh] = (float)e;
  }
}

// Per-lane base (16-bit elements) of the transposing reads of a 64-row tile
// stored in key_to_row order within each 32-row block: lane L of a 16-lane
// group points at row t = L/4 of its 4-row group (natural row 16g + t, stored
// at 4g + t), channels 16 (group % 2) + 4 (L % 4); natural row + 4 is stored
// 8 rows further, natural row + 8 16 rows further.  Two reads (+0, +8 rows)
// hand lane i channel c0 + i of natural rows 16g + 8j + [0, 8) of the block.
__device__ __forceinline__ int tr_base(int lane, int row_stride) {
  return (4 * (lane >> 5) + ((lane & 15) >> 2)) * row_stride + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x8_t read_tr8(const uint16_t* p, int row_stride) {
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p + 8 * row_stride));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------- dk, dv
template <int D>
__global__ __launch_bounds__(512) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ escale, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int S, int H, int nkb, RopeFreqs fr) {
  constexpr int BK = 256;              // keys per workgroup (8 waves x 32)
  constexpr int NBLK = D == 128 ? 1 : 2;   // 32-query blocks per step (one staging chunk a thread)
  constexpr int BQ = 32 * NBLK;        // queries per step
  constexpr int NT = 512;
  constexpr int KS = D / 16, MB = D / 32, DA = D / 4;
  // Each tile sits in LDS twice: rows padded by 16 bytes for the row-wise
  // 16-byte reads (16 lanes of a phase on 16 consecutive rows hit disjoint
  // banks), and by 64 bytes for the transposing reads (the 4 rows x 64 bytes
  // of a phase on disjoint banks); no one stride serves both.
  constexpr int ROW = D + 8;           // row-read copy stride (16-bit elements)
  constexpr int TROW = D + 32;         // transposed-read copy stride
  constexpr int CPR = D / 8;
  constexpr int NCH = BQ * CPR / NT;   // 16-byte chunks per thread per tile, each tensor
  static_assert(NCH >= 1 && BQ * CPR % NT == 0, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t q_lds[2][BQ * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t o_lds[2][BQ * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t qt_lds[2][BQ * TROW];
  __shared__ __attribute__((aligned(16))) uint16_t ot_lds[2][BQ * TROW];
  // -lse2 (-inf past S) and -delta of the tile's queries: the MFMA initial
  // values as they are
  __shared__ __attribute__((aligned(16))) float st_lds[2][2 * BQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lr = lane & 31;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int kb = work % nkb, bh = work / nkb;
  const int h = bh % H, b = bh / H;
  const size_t rs = (size_t)H * D;
  const size_t base = (size_t)b * S * rs + (size_t)h * D;
  const int rowb = (int)(rs * 2);
  const int key = kb * BK + wave * 32 + lr;
  const bool kval = key < S;

  // this lane's key as the B operand of S = q'' k'^T and dP = dout v^T
  f16x8_t kreg[KS];
  bf16x8_t vreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const size_t e = base + (size_t)key * rs + 16 * ks + 8 * g;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    kreg[ks] = __builtin_bit_cast(f16x8_t, kval ? *reinterpret_cast<const u32x4_t*>(kr + e) : z);
    vreg[ks] = __builtin_bit_cast(bf16x8_t, kval ? *reinterpret_cast<const u32x4_t*>(v + e) : z);
  }
  f32x16_t dva[MB], dka[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) dva[mb] = dka[mb] = (f32x16_t){};

  const float* lse_bh = lse + (size_t)bh * S;
  const float* dl_bh = delta + (size_t)bh * S;
  const float e2 = escale[bh];                   // P and dS carry 2^e2
  u32x4_t sq[NCH], so[NCH];
  float sl = 0.f, sd = 0.f;
  auto load = [&](int qt) {
    const int q0 = qt * BQ;
    const int n = S - q0 < BQ ? S - q0 : BQ;
    const __amdgpu_buffer_rsrc_t rq = uniform_rsrc(qr + base + (size_t)q0 * rs, n * rowb);
    const __amdgpu_buffer_rsrc_t ro = uniform_rsrc(dout + base + (size_t)q0 * rs, n * rowb);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int j = tid + NT * i, row = j / CPR, ch = j % CPR;
      const int off = row * rowb + 16 * ch;
      sq[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      so[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
    }
    if (tid < BQ) {
      // through wave-uniform descriptors: no per-lane 64-bit addresses to keep
      const __amdgpu_buffer_rsrc_t rl = uniform_rsrc(lse_bh + q0, n * 4);
      const __amdgpu_buffer_rsrc_t rd = uniform_rsrc(dl_bh + q0, n * 4);
      const float l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * tid, 0, 0));
      const float d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, 4 * tid, 0, 0));
      sl = tid < n ? e2 - l * kLog2e : kNegInf;
      sd = tid < n ? -d : 0.f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int j = tid + NT * i, row = j / CPR, ch = j % CPR;
      const int lrow = (row & ~31) + key_to_row(row & 31);
      *reinterpret_cast<u32x4_t*>(&q_lds[buf][lrow * ROW + 8 * ch]) = sq[i];
      *reinterpret_cast<u32x4_t*>(&o_lds[buf][lrow * ROW + 8 * ch]) = so[i];
      *reinterpret_cast<u32x4_t*>(&qt_lds[buf][lrow * TROW + 8 * ch]) = sq[i];
      *reinterpret_cast<u32x4_t*>(&ot_lds[buf][lrow * TROW + 8 * ch]) = so[i];
    }
    if (tid < BQ) {
      st_lds[buf][tid] = sl;
      st_lds[buf][BQ + tid] = sd;
    }
  };

  const int trb = tr_base(lane, TROW);
  const int nqt = (S + BQ - 1) / BQ;
  load(0);
  store(0);
  __syncthreads();
  for (int qt = 0; qt < nqt; ++qt) {
    const int buf = qt & 1;
    if (qt + 1 < nqt) load(qt + 1);
    f32x16_t sc[NBLK], dp[NBLK];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      // initial values -lse2 and -delta of rows 32 blk + 16 g + i
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(&st_lds[buf][32 * blk + 16 * g + 4 * i4]);
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&st_lds[buf][BQ + 32 * blk + 16 * g + 4 * i4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[blk][4 * i4 + e] = l4[e];
          dp[blk][4 * i4 + e] = d4[e];
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = (32 * blk + lr) * ROW + 16 * ks + 8 * g;
        const f16x8_t aq = *reinterpret_cast<const f16x8_t*>(&q_lds[buf][off]);
        sc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aq, kreg[ks], sc[blk], 0, 0, 0);
        const bf16x8_t ao = *reinterpret_cast<const bf16x8_t*>(&o_lds[buf][off]);
        dp[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vreg[ks], dp[blk], 0, 0, 0);
      }
    }
    // P = 2^(s2 - lse2 + e2) (bf16, for dV) and dS = P (dP - delta) (fp16,
    // for dK), both carrying 2^e2
    uint32_t pw[NBLK][8], sw[NBLK][8];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(sc[blk][2 * w]);
        const float p1 = __builtin_amdgcn_exp2f(sc[blk][2 * w + 1]);
        pw[blk][w] = pack_bf16x2(p0, p1);
        sw[blk][w] = pack_f16x2(p0 * dp[blk][2 * w], p1 * dp[blk][2 * w + 1]);
      }
    // dV^T += dout^T P, dK'^T += q''^T dS: k = the 64 queries of the tile, in
    // steps (blk, j) of 16: k slot (g, e) is query 32 blk + 16 g + 8 j + e
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8_t pb = __builtin_bit_cast(
            bf16x8_t, (u32x4_t){pw[blk][4 * j], pw[blk][4 * j + 1], pw[blk][4 * j + 2], pw[blk][4 * j + 3]});
        const f16x8_t sb = __builtin_bit_cast(
            f16x8_t, (u32x4_t){sw[blk][4 * j], sw[blk][4 * j + 1], sw[blk][4 * j + 2], sw[blk][4 * j + 3]});
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int off = trb + (32 * blk + 16 * j) * TROW + 32 * mb;
          const bf16x8_t ot = __builtin_bit_cast(bf16x8_t, read_tr8(&ot_lds[buf][off], TROW));
          dva[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ot, pb, dva[mb], 0, 0, 0);
          const f16x8_t qt8 = __builtin_bit_cast(f16x8_t, read_tr8(&qt_lds[buf][off], TROW));
          dka[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qt8, sb, dka[mb], 0, 0, 0);
        }
      }
    if (qt + 1 < nqt) store(buf ^ 1);   // that buffer was last read before the previous barrier
    __syncthreads();
  }

  // ---- epilogue: lane = key, register i of block mb = channel 32 mb + 8 (i/4) + 4 g + i%4
  if (!kval) return;
  const size_t row = base + (size_t)key * rs;
  // q'' carries log2(e)/sqrt(D) (dk' needs 1/sqrt(D)); dS and P carry 2^e2
  const float vscale = __builtin_ldexpf(1.0f, -(int)e2);
  const float kscale = vscale / kLog2e;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * mb + 8 * i4 + 4 * g;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = dka[mb][4 * i4 + e] * kscale;
      const int a = d / DA, jp = (d % DA) / 2;
      const int p = pos[4 * key + a];
      rotate_back(y[0], y[1], p, fr.hi[jp], fr.lo[jp]);
      rotate_back(y[2], y[3], p, fr.hi[jp + 1], fr.lo[jp + 1]);
      uint2 w;
      w.x = pack_bf16x2(y[0], y[1]);
      w.y = pack_bf16x2(y[2], y[3]);
      *reinterpret_cast<uint2*>(dk + row + d) = w;
      w.x = pack_bf16x2(dva[mb][4 * i4] * vscale, dva[mb][4 * i4 + 1] * vscale);
      w.y = pack_bf16x2(dva[mb][4 * i4 + 2] * vscale, dva[mb][4 * i4 + 3] * vscale);
      *reinterpret_cast<uint2*>(dv + row + d) = w;
    }
}

// ---------------------------------------------------------------- dq
template <int D>
__global__ __launch_bounds__(512) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ escale, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ dq, int S, int H, int nqb, RopeFreqs fr, float dqscale) {
  constexpr int BQ = 256;              // queries per workgroup (8 waves x 32)
  constexpr int BK = 64;               // keys per step
  constexpr int NT = 512;
  constexpr int KS = D / 16, MB = D / 32, DA = D / 4;
  constexpr int ROW = D + 8;           // row-read copy stride (as in the dk/dv kernel)
  constexpr int TROW = D + 32;         // transposed-read copy stride (k' only)
  constexpr int CPR = D / 8;
  constexpr int NCH = BK * CPR / NT;
  static_assert(NCH >= 1 && BK * CPR % NT == 0, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BK * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][BK * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t kt_lds[2][BK * TROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lr = lane & 31;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = work % nqb, bh = work / nqb;
  const int h = bh % H, b = bh / H;
  const size_t rs = (size_t)H * D;
  const size_t base = (size_t)b * S * rs + (size_t)h * D;
  const int rowb = (int)(rs * 2);
  const int query = qb * BQ + wave * 32 + lr;
  const bool qval = query < S;

  // this lane's query as the B operand of S^T = k' q''^T and dP^T = v dout^T
  f16x8_t qreg[KS];
  bf16x8_t oreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const size_t e = base + (size_t)query * rs + 16 * ks + 8 * g;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    qreg[ks] = __builtin_bit_cast(f16x8_t, qval ? *reinterpret_cast<const u32x4_t*>(qr + e) : z);
    oreg[ks] = __builtin_bit_cast(bf16x8_t, qval ? *reinterpret_cast<const u32x4_t*>(dout + e) : z);
  }
  const float e2 = escale[bh];                   // dS carries 2^e2
  const float nlse2 = qval ? e2 - lse[(size_t)bh * S + query] * kLog2e : 0.f;
  const float ndl = qval ? -delta[(size_t)bh * S + query] : 0.f;
  f32x16_t dqa[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) dqa[mb] = (f32x16_t){};

  u32x4_t sk[NCH], sv[NCH];
  auto load = [&](int kt) {
    const int k0 = kt * BK;
    const int n = S - k0 < BK ? S - k0 : BK;
    const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(kr + base + (size_t)k0 * rs, n * rowb);
    const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(v + base + (size_t)k0 * rs, n * rowb);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int j = tid + NT * i, row = j / CPR, ch = j % CPR;
      const int off = row * rowb + 16 * ch;
      sk[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      sv[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int j = tid + NT * i, row = j / CPR, ch = j % CPR;
      const int lrow = (row & ~31) + key_to_row(row & 31);
      *reinterpret_cast<u32x4_t*>(&k_lds[buf][lrow * ROW + 8 * ch]) = sk[i];
      *reinterpret_cast<u32x4_t*>(&v_lds[buf][lrow * ROW + 8 * ch]) = sv[i];
      *reinterpret_cast<u32x4_t*>(&kt_lds[buf][lrow * TROW + 8 * ch]) = sk[i];
    }
  };

  const int trb = tr_base(lane, TROW);
  const int nkt = (S + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();
  // one key tile; the last one (LAST) masks keys past S and prefetches
  // nothing, so the others form one branch-free block that the compiler can
  // interleave (MFMAs of one 32-key block with the exponentials of the other)
  auto step = [&](int kt, auto last) {
    constexpr bool LAST = decltype(last)::value;
    const int buf = kt & 1;
    if constexpr (!LAST) load(kt + 1);
    f32x16_t sc[2], dp[2];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[kbk][i] = nlse2;
        dp[kbk][i] = ndl;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = (32 * kbk + lr) * ROW + 16 * ks + 8 * g;
        const f16x8_t ak = *reinterpret_cast<const f16x8_t*>(&k_lds[buf][off]);
        sc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, qreg[ks], sc[kbk], 0, 0, 0);
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&v_lds[buf][off]);
        dp[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, oreg[ks], dp[kbk], 0, 0, 0);
      }
    }
    // keys past S (last tile only): p = 0 (their k' rows read as zeros, but
    // 2^(-lse2) alone could overflow)
    if constexpr (LAST) {
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * BK + 32 * kbk + 16 * g + i >= S) sc[kbk][i] = kNegInf;
    }
    uint32_t sw[2][8];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(sc[kbk][2 * w]);
        const float p1 = __builtin_amdgcn_exp2f(sc[kbk][2 * w + 1]);
        sw[kbk][w] = pack_f16x2(p0 * dp[kbk][2 * w], p1 * dp[kbk][2 * w + 1]);
      }
    // dQ'^T += k'^T dS^T: k = the 64 keys of the tile, slot (g, e) of step
    // (kbk, j) is key 32 kbk + 16 g + 8 j + e
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f16x8_t sb = __builtin_bit_cast(
            f16x8_t, (u32x4_t){sw[kbk][4 * j], sw[kbk][4 * j + 1], sw[kbk][4 * j + 2], sw[kbk][4 * j + 3]});
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int off = trb + (32 * kbk + 16 * j) * TROW + 32 * mb;
          const f16x8_t kt8 = __builtin_bit_cast(f16x8_t, read_tr8(&kt_lds[buf][off], TROW));
          dqa[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kt8, sb, dqa[mb], 0, 0, 0);
        }
      }
    if constexpr (!LAST) {
      store(buf ^ 1);
      __syncthreads();
    }
  };
  for (int kt = 0; kt + 1 < nkt; ++kt) step(kt, std::false_type{});
  step(nkt - 1, std::true_type{});

  if (!qval) return;
  const size_t row = base + (size_t)query * rs;
  const float qscale = __builtin_ldexpf(dqscale, -(int)e2);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * mb + 8 * i4 + 4 * g;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = dqa[mb][4 * i4 + e] * qscale;
      const int a = d / DA, jp = (d % DA) / 2;
      const int p = pos[4 * query + a];
      rotate_back(y[0], y[1], p, fr.hi[jp], fr.lo[jp]);
      rotate_back(y[2], y[3], p, fr.hi[jp + 1], fr.lo[jp + 1]);
      uint2 w;
      w.x = pack_bf16x2(y[0], y[1]);
      w.y = pack_bf16x2(y[2], y[3]);
      *reinterpret_cast<uint2*>(dq + row + d) = w;
    }
}

template <int D>
static hipError_t launch_bwd(const BwdArgs& a) {
  const long long nchunks = (long long)a.B * a.S * a.H * (D / 8);
  hipLaunchKernelGGL(attn_bwd_prep_kernel<D>, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0,
                     a.stream, a.q, a.k, a.v, a.pos, a.out, a.dout, a.qr, a.kr, a.delta, a.norm2,
                     a.S, a.H, nchunks, a.freqs, a.qscale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_scale_kernel, dim3((unsigned)(a.B * a.H)), dim3(256), 0, a.stream,
                     a.norm2, a.escale, a.S, (long long)a.B * a.H * a.S);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dK/dV and dQ read the same inputs and write disjoint outputs.  Given a
  // second stream, dQ runs on it beside dK/dV, so that the workgroups of
  // each fill the compute units the other's last, partial round leaves idle.
  const bool two = a.side != nullptr && a.fork != nullptr && a.join != nullptr;
  hipStream_t sq = a.stream;
  if (two) {
    e = hipEventRecord(a.fork, a.stream);
    if (e != hipSuccess) return e;
    e = hipStreamWaitEvent(a.side, a.fork, 0);
    if (e != hipSuccess) return e;
    sq = a.side;
  }
  const int nb = (a.S + 255) / 256;
  const dim3 grid((unsigned)(a.B * a.H * nb));
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, grid, dim3(512), 0, a.stream, a.qr, a.kr, a.v,
                     a.dout, a.lse, a.delta, a.escale, a.pos, a.dk, a.dv, a.S, a.H, nb, a.freqs);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (a.S + 255) / 256;
  hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3((unsigned)(a.B * a.H * nqb)), dim3(512), 0, sq,
                     a.qr, a.kr, a.v, a.dout, a.lse, a.delta, a.escale, a.pos, a.dq, a.S, a.H, nqb,
                     a.freqs, (float)(1.0 / std::sqrt((double)D)));
  e = hipGetLastError();
  if (e != hipSuccess || !two) return e;
  e = hipEventRecord(a.join, a.side);
  if (e != hipSuccess) return e;
  return hipStreamWaitEvent(a.stream, a.join, 0);
}

hipError_t launch_attn_bwd(const BwdArgs& a) {
  return a.D == 128 ? launch_bwd<128>(a) : launch_bwd<64>(a);
}

BwdWorkspace attn_bwd_workspace(int B, int S, int H, int D) {
  const auto up = [](long long x) { return (x + 255) / 256 * 256; };
  const long long n = (long long)B * S * H * D, rows = (long long)B * H * S;
  BwdWorkspace w{};
  w.kr = up(n * 2);                       // qr at 0, then kr: fp16 [B][S][H][D] each
  w.delta = 2 * w.kr;                     // fp32 [B][H][S]
  w.norm2 = w.delta + up(rows * 4);       // fp32 [2][B][H][S]
  w.escale = w.norm2 + up(rows * 8);      // fp32 [B][H]
  w.total = w.escale + up((long long)B * H * 4);
  return w;
}

}  // namespace klein
