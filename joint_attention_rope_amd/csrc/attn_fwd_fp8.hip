// RoPE-4D joint self-attention forward, FP8 E4M3 in / bf16 out, for gfx950.
//
// Inputs are OCP E4M3FN codes with per-tensor descales: value = code * dX.
// One workgroup of 8 waves (two per SIMD) owns one (batch, head, tile of 256
// queries); each wave owns 32 queries and streams all keys in tiles of 64.
// Every key is rotated and re-quantised on its way to LDS, and both products
// are fp8 MFMAs (v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation):
//
//   Q'' = e4m3(R(q_code) * c)            registers, once; c = G / 2^n
//   K'' = e4m3(R(k_code) / 2)            LDS, per tile
//   Y^T = 2^(n+3) K'' Q''^T + 118 - 8m   the 2^(n+3) is the MFMA's E8M0
//                                        operand scale, 118 - 8m the chain's
//                                        initial value: Y = 8 (s - m) + 118
//   P8  = code rne(clamp(Y, 0, 255))     an E4M3 code read as an integer
//                                        (v_cvt_pk_u8_f32); m is the running
//                                        row max, raised only when a row's
//                                        code would pass 126 (448), and then
//                                        to code 110
//   O^T += V^T P8^T                      V row-major in LDS, read transposed
//   l  += ones^T P8^T                    row sums of P8, on the MFMA as well
//   out = O * dv / l
//
// with G = 2 dq dk log2(e) / sqrt(D): the exp2-domain score of query i and
// key j is dq dk log2(e)/sqrt(D) <R q_i, R k_j> = G <R q_i, K''_j>, and n is
// picked so that c lies in (1/(2 sqrt 2), 1/sqrt 2].  A rotated pair
// component grows by at most sqrt 2, so |R(code)| c <= 448, |R(code)| / 2 <=
// 317, and neither re-quantisation leaves the E4M3 range.  Halving K (a power
// of two) keeps the channels the rotation leaves alone -- the t and l axis
// blocks of image tokens, at position 0 -- exact codes, which is worth a
// fifth of the fp8 path's error against the oracle.
//
// Softmax without an exponential: an E4M3 code c of a normal number is
// 8 (e + 7) + f for the value 2^e (1 + f/8), so c / 8 - 7 is log2 of the
// value within the binade's linear interpolation (at most 0.086 off, i.e. at
// most 6.2 % too large).  The code nearest to 8 x + 118 therefore encodes
// about 2^(x + 7.75), with x = s - m the exp2-domain score against the
// running max: one full-rate conversion per score replaces a quarter-rate
// v_exp_f32 and half an fp8 conversion.  O and l take the very same P8, so
// the common factor cancels and only the interpolation's variation within a
// binade remains (rel-L2 on the 2048^2 edit workload 4.1e-2 -> 4.5e-2, by a
// CPU model of these roundings).
// Range: the first max (tile 0's exact row max) sits at code 118 (224): P8
// stays a normal number down to x = -13.75, within a binade of what an
// exact exponential scaled to 448 keeps.  A raise puts the new max at code
// 110, leaving two binades of headroom (12.75 binades of normals below it):
// rescales then come about once in 45 wave-tiles on N(0, 1) scores of the
// 2048^2 edit workload (once in 20 with the raised max at 118, once in 800
// with the max at 94 and four binades of headroom, which cut keys off at
// x = -11.7).  Below code 8 the codes are subnormals (value c 2^-9, no longer
// 2^(c/8 - 7)), and codes below 0.5 round to 0 (a masked key's -inf as
// well).  A key that far below the row max carries a weight of at most
// 2^-12.7 of it, which matters only when thousands of such keys face one
// dominant key.
//
// Schedule (per wave; K'' and V double-buffered in LDS, one barrier a tile):
//   softmax max of S(t); rare rescale of O and l
//   region A:  Y(t+1) MFMAs      interleaved with  the P8 codes of Y(t)
//   region B:  O^T += V(t)^T P8  interleaved with  staging K''(t+2) and
//              and l += 1^T P8                      V(t+1) into LDS
//   buffer loads of K(t+3), V(t+2); barrier
//
// Rotation of keys: cos and sin (times 1/2) of every (position, pair)
// with position in [0, 1024) come from an LDS table built once per workgroup;
// a wave that holds any other position computes them directly instead.
//
// MFMA operands: the score MFMA puts keys on rows and queries on columns, and
// keys sit in LDS in a permuted row order so that accumulator register i of a
// lane in half g holds key 16g + i of its 32-key block.  The P8 bytes of a
// lane then cover keys 16g + [0,16) and 32 + 16g + [0,16); the V^T operand
// holds the same keys of one channel, gathered by ds_read_b64_tr_b8 reads: in
// a group of 16 lanes, lane i receives byte i % 8 of the 8-byte words that
// lanes 2e + i/8 (e = 0..7) address, so pointing lane 2e + h at
// V[key0 + e][c0 + 8h .. + 7] hands lane i channel c0 + i of keys key0 ..
// key0 + 7.
#include <cmath>

#include "klein_device.hpp"
#include "klein_launch.hpp"

namespace klein {

// Per-region cycle counts of the pipeline step, for a measurement build
// only: defined by the step_clock.hip harness, never by the library.  Each
// wave sums, over its steps, the shader-clock cycles (s_memtime) between
// marks after the softmax max (with the rare rescale), after region A, after
// region B, after the buffer loads and after the barrier, and lane 0 writes
// them, with the step count, the cycles of the whole loop and its
// fixed-rate timestamps (s_memrealtime), to klein_fp8_clock_out[8 wg +
// wave][0..9].
#ifdef KLEIN_STEP_CLOCK
__device__ unsigned long long* klein_fp8_clock_out;
#define KLEIN_FP8_CLOCK_START                                                \
  unsigned long long fclk_sum[6] = {0, 0, 0, 0, 0, 0};                       \
  const unsigned long long fclk_real0 = __builtin_amdgcn_s_memrealtime();    \
  unsigned long long fclk_prev = __builtin_amdgcn_s_memtime();               \
  const unsigned long long fclk_start = fclk_prev;
#define KLEIN_FP8_CLOCK_MARK(i)                                              \
  do {                                                                       \
    const unsigned long long fclk_now = __builtin_amdgcn_s_memtime();        \
    fclk_sum[i] += fclk_now - fclk_prev;                                     \
    fclk_prev = fclk_now;                                                    \
  } while (0)
#define KLEIN_FP8_CLOCK_STORE(nsteps)                                        \
  if (klein_fp8_clock_out != nullptr && lane == 0) {                         \
    unsigned long long* co = klein_fp8_clock_out + ((size_t)blockIdx.x * 8 + wave) * 10; \
    for (int i = 0; i < 6; ++i) co[i] = fclk_sum[i];                         \
    co[6] = (unsigned long long)(nsteps);                                    \
    co[7] = fclk_prev - fclk_start;                                          \
    co[8] = fclk_real0;                                                      \
    co[9] = __builtin_amdgcn_s_memrealtime();                                \
  }
#else
#define KLEIN_FP8_CLOCK_START
#define KLEIN_FP8_CLOCK_MARK(i) do {} while (0)
#define KLEIN_FP8_CLOCK_STORE(nsteps)
#endif

// Race check build: KLEIN_SYNC_CHECK is defined only for the library's
// synchronised copy (libklein_attn_sync.so), never for the library itself.
// At every stage boundary of the pipeline step each wave then waits for all
// of its outstanding memory operations (s_waitcnt 0) and for the whole
// workgroup, so no LDS hand-off between waves can overlap the next stage.
// The arithmetic is unchanged, so both builds must give the same bits; a
// difference means the fast build reads LDS data before it is written or
// overwrites it before it is read.
#ifdef KLEIN_SYNC_CHECK
#define KLEIN_SYNC_POINT()                                                   \
  do {                                                                       \
    __builtin_amdgcn_s_waitcnt(0);                                           \
    __syncthreads();                                                         \
  } while (0)
#else
#define KLEIN_SYNC_POINT() do {} while (0)
#endif

namespace {

constexpr float kHalf = 0.5f;
constexpr int kFp8TabN = 1024;       // positions covered by the cos/sin table

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef short s2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int key_to_row8(int kk) {
  const int g = kk >> 4, i = kk & 15;
  return ((i >> 2) << 3) + (g << 2) + (i & 3);
}

// (cos, sin) * scale of the angle pos * w (w in revolutions, split hi + lo)
__device__ __forceinline__ float2 rope_cs(int p, float whi, float wlo, float scale) {
  const float fp = (float)p;
  const float rev = rope_rev(fp, whi, wlo);
  return make_float2(__builtin_amdgcn_cosf(rev) * scale, __builtin_amdgcn_sinf(rev) * scale);
}

// Rotate pair (x, y) held as E4M3 bytes 2h, 2h+1 of `word` by (c, s) and
// write it, re-encoded (RNE), into half h of `acc`.
template <bool HI>
__device__ __forceinline__ int rope_pair_fp8(uint32_t word, float2 cs, int acc) {
  const auto xy = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
  return __builtin_amdgcn_cvt_pk_fp8_f32(xy[0] * cs.x - xy[1] * cs.y, xy[0] * cs.y + xy[1] * cs.x,
                                         acc, HI);
}

// The same in packed fp16 (decode, two packed FMA-type ops, encode): E4M3
// values are exact in fp16, and (c, s) carry fp16's 11-bit mantissa, far
// finer than the 4 significant bits the result is rounded to.
template <bool HI>
__device__ __forceinline__ int rope_pair_fp8_h(uint32_t word, h2_t cs, int acc) {
  const h2_t xy = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)word, 1.0f, HI);
  const h2_t xx = {xy[0], xy[0]}, yy = {xy[1], xy[1]};
  const h2_t t = yy * (h2_t){cs[1], cs[0]};                    // (y s, y c)
  const h2_t r = __builtin_elementwise_fma(xx, cs, (h2_t){-t[0], t[1]});
  const s2_t out = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(__builtin_bit_cast(s2_t, acc), r,
                                                            1.0f, HI);
  return __builtin_bit_cast(int, out);
}

}  // namespace

// SPARSE: block-sparse variant (one mask byte per batch, head, query tile of
// 256 and key tile of 64; only kept key tiles stream through the pipeline, in
// ascending order, so with every tile kept the result equals the dense one).
// KPRE: the key codes arrive rotated (K'' = e4m3(R k / 2), written once per
// call by rope4d_fp8_kernel with the very arithmetic of the in-kernel path),
// and K tiles are copied to LDS as they are: no table, positions or rotation.
// SPLIT: the split-KV schedule (SplitArgs): whole items first, then the key
// chunks of the remaining items, merged through the workspace.
template <int D, bool SPARSE, bool KPRE, bool SPLIT>
__global__ __launch_bounds__(512) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const int32_t* __restrict__ pos, uint16_t* __restrict__ out, int S, int H, int nqt,
    RopeFreqs fr, float q_mul, int sc_a, int sc_b, float o_scale,
    const uint8_t* __restrict__ bmask, SplitArgs sp) {
  constexpr int BM = 256;              // queries per workgroup (8 waves x 32)
  constexpr int BN = 64;               // keys per tile
  constexpr int NT = 512;              // threads
  constexpr int CPK = D / 16;          // 16-byte chunks per token row
  constexpr int NCH = BN * CPK;        // chunks per K (or V) tile
  constexpr int KS = D / 64;           // k-steps of the score MFMA
  constexpr int MB = D / 32;           // 32-row blocks of O^T
  constexpr int KROW = D + 16;         // LDS row stride of K'' (bytes)
  constexpr int VROW = D + 32;         // LDS row stride of V (bytes)
  constexpr int DA = D / 4;            // channels per RoPE axis
  constexpr int NJ = D / 8;            // rotation pairs per axis
  constexpr int TROW = NJ + 2;         // cos/sin table row stride (half2)
  constexpr int TSLOT = 10;            // per-thread fallback slot stride
  constexpr int TAB = kFp8TabN * TROW;    // start of the fallback slots
  constexpr float YM = 118.0f;         // code of a score equal to the first running max
  constexpr float YR = 110.0f;         // code of the running max after a raise
  constexpr float YMAX = 126.0f;       // largest finite E4M3 code (448)
  static_assert(NCH == NT || 2 * NCH == NT, "one K and one V chunk per thread (D 128) "
                                            "or one of either (D 64)");
  static_assert(!(SPARSE && SPLIT), "one schedule at a time");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][BN * KROW];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[2][BN * VROW];
  // fp16 (cos, sin) / 2: table rows for positions [0, kFp8TabN), then 8
  // per-thread slots.  Row and slot strides of 2 (mod 4) dwords spread 32
  // rows over all banks and keep pairs of entries 8-byte aligned.
  __shared__ __attribute__((aligned(16))) h2_t cs_tab[TAB + TSLOT * NT];
  __shared__ uint16_t klist[SPARSE ? kSparseMaxTiles + kSparsePad : 1];
  __shared__ int klist_n;
  // A operand of the row-sum MFMA: E4M3 ones (words 0-3) or zeros (4-7)
  __shared__ __attribute__((aligned(16))) uint32_t ones_lds[8];
  if (threadIdx.x < 8) ones_lds[threadIdx.x] = threadIdx.x < 4 ? 0x38383838u : 0u;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lr = lane & 31;
  const int nkt = (S + BN - 1) / BN;
  const size_t rs = (size_t)H * D;                       // token stride (bytes)
  const int rowb = (int)rs;

  // ---- this workgroup's work: an item (b, h, query tile) and its key tiles
  // [k0, k1): all of them, or with SPLIT past the whole items, chunk `chunk`
  int work, k0 = 0, k1 = nkt, chunk = 0;
  if (SPLIT && (int)blockIdx.x >= sp.n_dp) {
    const int s = xcd_remap(blockIdx.x - sp.n_dp, sp.n_sk);
    chunk = s / sp.n_rem;
    work = sp.n_dp + s % sp.n_rem;
    k0 = split_chunk_begin(chunk, nkt, sp.n_chunk);
    k1 = split_chunk_begin(chunk + 1, nkt, sp.n_chunk);
  } else {
    work = xcd_remap(blockIdx.x, SPLIT ? sp.n_dp : gridDim.x);
  }

  // ---- cos/sin table: entry p * TROW + j = (cos, sin)(p w_j) / 2
  if constexpr (!KPRE) {
    for (int e = tid; e < kFp8TabN * NJ; e += NT) {
      const int j = e % NJ, p = e / NJ;
      const float2 c = rope_cs(p, fr.hi[j], fr.lo[j], kHalf);
      cs_tab[p * TROW + j] = (h2_t){(_Float16)c.x, (_Float16)c.y};
    }
  }

  const int qt = work % nqt;
  const int bh = work / nqt;
  const int h = bh % H, b = bh / H;
  const size_t base = (size_t)b * S * rs + (size_t)h * D;
  const uint8_t* qb = q + base;
  // keys, values and key positions from the segment's first tile on; Sk
  // keys remain from there
  const uint8_t* kbase = k + base + (size_t)k0 * BN * rs;
  const uint8_t* vbase = v + base + (size_t)k0 * BN * rs;
  const int32_t* kposb = pos + (size_t)k0 * BN * 4;
  const int Sk = S - k0 * BN;

  // ---- Q'': this lane's query, dims 64 ks + 32 g + [0, 32) per k-step.
  // Rows past S load row S-1 (in bounds) and are never stored.
  const int qrow = qt * BM + wave * 32 + lr;
  const int qload = qrow < S ? qrow : S - 1;
  i32x8_t qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      const int d0 = 64 * ks + 32 * g + 16 * hc;
      const int a = d0 / DA, j0 = (d0 % DA) / 2;
      const int p = pos[4 * qload + a];
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qb + (size_t)qload * rs + d0);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        int word = rope_pair_fp8<false>(x[w], rope_cs(p, fr.hi[j0 + 2 * w], fr.lo[j0 + 2 * w], q_mul), 0);
        word = rope_pair_fp8<true>(x[w], rope_cs(p, fr.hi[j0 + 2 * w + 1], fr.lo[j0 + 2 * w + 1], q_mul), word);
        qreg[ks][4 * hc + w] = word;
      }
    }
  }

  // ---- staging assignment.  D = 128: every thread stages chunk tid of the K
  // tile and chunk tid of the V tile.  D = 64: threads [0, 256) stage K,
  // threads [256, 512) stage V.
  const bool kst = NCH == NT || tid < NCH;
  const bool vst = NCH == NT || tid >= NCH;
  const int vid = NCH == NT ? tid : tid - NCH;
  const int kkey = tid / CPK, kc = tid % CPK;            // K: key, chunk
  const int ka = (16 * kc) / DA, kj0 = ((16 * kc) % DA) / 2;
  const int vkey = vid / CPK, vc = vid % CPK;            // V: key, chunk
  const int voff_k = kkey * rowb + 16 * kc;
  const int voff_p = (kkey * 4 + ka) * 4;
  const int voff_v = vkey * rowb + 16 * vc;
  const int krow = (kkey & ~31) + key_to_row8(kkey & 31);

  // tile index of pipeline position t (the kept list when SPARSE)
  auto tl = [&](int t) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)klist[t]);
    else return t;
  };
  u32x4_t kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
  // positions of this thread's K chunk, loaded one step ahead of the K data:
  // slot kt & 1 holds tile kt's
  int kpos0 = 0, kpos1 = 0;

  auto tile_rows = [&](int kt) {
    const int n = Sk - kt * BN;
    return n < 0 ? 0 : (n > BN ? BN : n);
  };
  // global -> registers (rows past S read as zero through the descriptors)
  auto load_k = [&](int kt) {
    if (kst) {
      const int n = tile_rows(kt);
      const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(kbase + (size_t)kt * BN * rs, n * rowb);
      kx = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, voff_k, 0, 0));
    }
  };
  auto load_pos = [&](int kt, int& slot) {
    if constexpr (KPRE) return;
    if (kst) {
      const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(kposb + (size_t)kt * BN * 4, tile_rows(kt) * 16);
      slot = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, voff_p, 0, 0);
    }
  };
  auto load_v = [&](int kt) {
    if (vst) {
      const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(vbase + (size_t)kt * BN * rs, tile_rows(kt) * rowb);
      vx = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, 0, 0));
    }
  };
  auto stage_v = [&](int buf) {
    if (vst) *reinterpret_cast<u32x4_t*>(&v_lds[buf][vkey * VROW + 16 * vc]) = vx;
  };
  // (cos, sin) / 2 of the 8 pairs of this thread's K chunk, as an index
  // into cs_tab: the table row of its position, or (position outside the
  // table) its own 8 slots past the table, filled here.  The branch is
  // divergent and skipped by waves whose positions all lie in the table.
  auto key_cs_index = [&](int kp) {
    if constexpr (KPRE) return 0;
    const bool oob = kst && (unsigned)kp >= (unsigned)kFp8TabN;
    if (oob) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        int j = kj0 + jj;
        asm volatile("" : "+v"(j));      // keep the loads in this rare path
        const float2 c = rope_cs(kp, fr.hi[j], fr.lo[j], kHalf);
        cs_tab[TAB + TSLOT * tid + jj] = (h2_t){(_Float16)c.x, (_Float16)c.y};
      }
    }
    return oob ? TAB + TSLOT * tid : (kst ? kp : 0) * TROW + kj0;
  };
  // one rotated pair of the K chunk; the 16-byte LDS store after the last
  u32x4_t ky;
  auto rope_item = [&](int kdst, int jj, h2_t cs) {
    if constexpr (KPRE) {              // a rotated chunk: one copy
      if (jj == 0 && kst) *reinterpret_cast<u32x4_t*>(&k_lds[kdst][krow * KROW + 16 * kc]) = kx;
      return;
    }
    const int w = jj >> 1;
    ky[w] = (uint32_t)((jj & 1) ? rope_pair_fp8_h<true>(kx[w], cs, (int)ky[w])
                                : rope_pair_fp8_h<false>(kx[w], cs, (int)ky[w]));
    if (jj == 7 && kst) *reinterpret_cast<u32x4_t*>(&k_lds[kdst][krow * KROW + 16 * kc]) = ky;
  };
  auto stage_k = [&](int buf, int kp) {
    const int ci = key_cs_index(kp);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) rope_item(buf, jj, KPRE ? h2_t{} : cs_tab[ci + jj]);
  };
  // lane base of the transposing V reads: lane L of group G = L / 16 reads
  // row 16 (G / 2) + (L % 16) / 2, channels 16 (G % 2) + 8 (L % 2) .. + 7
  const int vtr_base = (16 * (lane >> 5) + ((lane & 15) >> 1)) * VROW +
                       16 * ((lane >> 4) & 1) + 8 * (lane & 1);

  f32x16_t o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = (f32x16_t){};
  float m8 = 0.f;                      // running row max, in code units (8 m)
  // Row sums of P8 on a 16x16x128 MFMA that reads the P8 operand of the
  // 32x32x64 one as it is.  Lane 16b + n of that operand holds 32 keys of
  // query 16 (b & 1) + n, so an A operand whose lane 16b + r is all ones
  // exactly when bit 2 of r equals bit 0 of b makes output row r, column n
  // the row sum of query 16 ((r >> 2) & 1) + n -- and output lane L, which
  // holds rows 4 (L / 16) + [0, 4) of column L % 16, gets the sum of its own
  // query L % 32 in all 4 registers.
  f32x4_t lacc = {};
  const int ones_off = ((lane >> 2) & 1) == ((lane >> 4) & 1) ? 0 : 4;

  auto read_k = [&](int kbuf, int kbk, int ks) {
    const uint8_t* src = &k_lds[kbuf][(32 * kbk + lr) * KROW + 64 * ks + 32 * g];
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(src);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(src + 16);
    return (i32x8_t){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto score_mfma = [&](i32x8_t a, int ks, f32x16_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qreg[ks], c, 0, 0, 0, sc_a, 0, sc_b);
  };
  // largest of the 32 values a lane holds (rowmax32: of its row, both lanes)
  auto lanemax32 = [&](const f32x16_t* sc) {
    float m[12];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      const int a = 3 * i, b2 = 3 * i + 1, c = 3 * i + 2;
      m[i] = __builtin_fmaxf(sc[a >> 4][a & 15],
                             __builtin_fmaxf(sc[b2 >> 4][b2 & 15], sc[c >> 4][c & 15]));
    }
    m[10] = sc[1][14];
    m[11] = sc[1][15];
    float n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) n[i] = __builtin_fmaxf(m[3 * i], __builtin_fmaxf(m[3 * i + 1], m[3 * i + 2]));
    return __builtin_fmaxf(n[0], __builtin_fmaxf(n[1], __builtin_fmaxf(n[2], n[3])));
  };
  auto rowmax32 = [&](const f32x16_t* sc) { return pair_max(lanemax32(sc)); };
  f32x16_t cinit;
  auto set_cinit = [&]() {
#pragma unroll
    for (int i = 0; i < 16; ++i) cinit[i] = YM - m8;
  };
  auto mask_tail = [&](int t, f32x16_t* sc) {
    if (t * BN + BN > Sk) {
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (t * BN + 32 * kbk + 16 * g + i >= Sk) sc[kbk][i] = kNegInf;
    }
  };
  auto softmax_max = [&](int t, f32x16_t* sc) {
    mask_tail(t, sc);
    // a row passes YMAX exactly when one of its two lanes does, so the test
    // needs no exchange; the rare rescale takes the row max
    const float lm = lanemax32(sc);
    if (__builtin_amdgcn_ballot_w64(lm > YMAX)) {
      const float mx = pair_max(lm);            // code of the row's largest score
      const float delta = __builtin_fmaxf(mx - YR, 0.f);
      const float alpha = __builtin_amdgcn_exp2f(-0.125f * delta);
      m8 += delta;
      lacc *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) sc[kbk] -= delta;
      set_cinit();
    }
  };

  // Region A: S(t+1) (2 KS MFMAs, K'' operands read two ahead) with the
  // softmax of S(t) in 8 slices of 4 scores (one P8 word each).  The row
  // sums are taken in region B, from P8 itself.
  constexpr int NA = 2 * KS;
  auto region_a = [&](int kbuf, const f32x16_t* cur, f32x16_t* nxt, i32x8_t& pb) {
    i32x8_t kop[NA];
    nxt[0] = cinit;
    nxt[1] = cinit;
    kop[0] = read_k(kbuf, 0 / KS, 0 % KS);
    if (NA > 1) kop[1 % NA] = read_k(kbuf, 1 / KS, 1 % KS);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (i + 2 < NA) kop[i + 2] = read_k(kbuf, (i + 2) / KS, (i + 2) % KS);
      const int kbk = i / KS, ks = i % KS;
      nxt[kbk] = score_mfma(kop[i], ks, nxt[kbk]);
#pragma unroll
      for (int sl = i * 8 / NA; sl < (i + 1) * 8 / NA; ++sl) {
        const int kb2 = sl >> 2, w = sl & 3;
        // four codes, each rounded to nearest even and clamped to [0, 255]
        // into its byte of the word
        uint32_t word = __builtin_amdgcn_cvt_pk_u8_f32(cur[kb2][4 * w], 0u, 0u);
#pragma unroll
        for (int e = 1; e < 4; ++e)
          word = __builtin_amdgcn_cvt_pk_u8_f32(cur[kb2][4 * w + e], (unsigned)e, word);
        pb[4 * kb2 + w] = (int)word;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Pin the score MFMAs here: their results are only read in the next
    // step, and without a use here they would be sunk to it, away from the
    // softmax work they are meant to overlap.
    asm volatile("" : "+v"(nxt[0]), "+v"(nxt[1]));
  };

  // Region B: O^T += V(t)^T P8^T (MB MFMAs, V^T operands read two ahead) and
  // the row sums (one more MFMA) with the staging of K''(t+2) (8 rotated
  // pairs) and V(t+1) spread over them.
  auto read_v = [&](int vbuf, int mb) {
    typedef int i32x2v_t __attribute__((ext_vector_type(2)));
    i32x2v_t r[4];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
        r[2 * qq + rr] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2v_t*)(&v_lds[vbuf][vtr_base + (32 * qq + 8 * rr) * VROW + 32 * mb]));
    return (i32x8_t){r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
  };
  constexpr int NIT = 9;               // 8 rotated pairs, then the V chunk
  auto region_b = [&](int vbuf, int kdst, int vdst, const i32x8_t& pb, int ci) {
    i32x8_t vop[MB];
    h2_t kcs[8];
    vop[0] = read_v(vbuf, 0);
    vop[1] = read_v(vbuf, 1);
    if constexpr (!KPRE) {
      kcs[0] = cs_tab[ci];
      kcs[1] = cs_tab[ci + 1];
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (i + 2 < MB) vop[i + 2] = read_v(vbuf, i + 2);
      o[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[i], pb, o[i], 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int item = i * NIT / MB; item < (i + 1) * NIT / MB; ++item) {
        if (!KPRE && item + 2 < 8) kcs[item + 2] = cs_tab[ci + item + 2];
        if (item < 8) rope_item(kdst, item, kcs[item]);
        else stage_v(vdst);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const u32x4_t on = *reinterpret_cast<const u32x4_t*>(ones_lds + ones_off);
    const i32x8_t ones = {(int)on[0], (int)on[1], (int)on[2], (int)on[3],
                          (int)on[0], (int)on[1], (int)on[2], (int)on[3]};
    lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pb, lacc, 0, 0, 0, 0, 0, 0);
  };

  int nsteps = k1 - k0;
  if constexpr (SPARSE) {
    if (wave == 0) {
      const int n = build_kept_list(bmask + ((size_t)bh * nqt + qt) * nkt, nkt, klist, lane);
      if (lane == 0) klist_n = n;
    }
    __syncthreads();
    nsteps = __builtin_amdgcn_readfirstlane(klist_n);
    if (nsteps == 0) {                 // nothing kept: the rows are zero
      if (qrow < S) {
        uint16_t* orow = out + (size_t)b * S * rs + (size_t)h * D + (size_t)qrow * rs;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<uint2*>(orow + 32 * mb + 8 * i4 + 4 * g) = make_uint2(0u, 0u);
      }
      return;
    }
  }

  // ---- prologue: table, K''(0), K''(1), V(0) in LDS; S(0) in registers;
  // K(2), V(1) in flight (pipeline positions; tl() maps them to tiles)
  load_k(tl(0));
  load_pos(tl(0), kpos0);
  load_v(tl(0));
  __syncthreads();                     // table complete
  stage_k(0, kpos0);
  stage_v(0);
  load_k(tl(1));
  load_pos(tl(1), kpos1);
  stage_k(1, kpos1);
  load_k(tl(2));
  load_pos(tl(2), kpos0);
  load_pos(tl(3), kpos1);
  load_v(tl(1));
  __syncthreads();
  f32x16_t sa[2], sb[2];
#pragma unroll
  for (int kbk = 0; kbk < 2; ++kbk) {
    sa[kbk] = (f32x16_t){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sa[kbk] = score_mfma(read_k(0, kbk, ks), ks, sa[kbk]);
  }
  __syncthreads();                     // K'' buffer 0 is refilled in iteration 0
  // m starts at tile 0's exact row max, so scores are relative from the start
  mask_tail(tl(0), sa);
  m8 = rowmax32(sa);
#pragma unroll
  for (int kbk = 0; kbk < 2; ++kbk) sa[kbk] -= m8 - YM;
  set_cinit();

  i32x8_t pb = {};
  // one pipeline step; `cur` holds S(t), `nxt` receives S(t+1), `kps` holds
  // the positions of K(t+2) and receives those of K(t+4).  The only branches
  // (rare rescale, rare rotation fallback) come first, so that regions A and
  // B form one block whose interleaving the compiler keeps.
  KLEIN_FP8_CLOCK_START
  auto step = [&](int t, f32x16_t* cur, f32x16_t* nxt, int& kps) {
    const int ci = key_cs_index(kps);
    softmax_max(tl(t), cur);
    KLEIN_SYNC_POINT();
    KLEIN_FP8_CLOCK_MARK(0);
    region_a((t + 1) & 1, cur, nxt, pb);
    KLEIN_SYNC_POINT();
    KLEIN_FP8_CLOCK_MARK(1);
    // K''(t+2) into buffer t&1 (it held K''(t)); V(t+1) into buffer (t+1)&1
    region_b(t & 1, t & 1, (t + 1) & 1, pb, ci);
    KLEIN_SYNC_POINT();
    KLEIN_FP8_CLOCK_MARK(2);
    load_k(tl(t + 3));
    load_pos(tl(t + 4), kps);
    load_v(tl(t + 2));
    KLEIN_SYNC_POINT();
    KLEIN_FP8_CLOCK_MARK(3);
    __syncthreads();
    KLEIN_FP8_CLOCK_MARK(4);
  };
  int t = 0;
  for (; t + 1 < nsteps; t += 2) {
    step(t, sa, sb, kpos0);
    step(t + 1, sb, sa, kpos1);
  }
  if (t < nsteps) step(t, sa, sb, kpos0);
  KLEIN_FP8_CLOCK_STORE(nsteps)

  // ---- epilogue: O * dv / l -> bf16; a chunk of a split item stores its
  // partial instead (the merge kernel writes those rows)
  const float lsum = lacc[0];
  if constexpr (SPLIT)
    if (k0 != 0 || k1 != nkt) {
      split_store<MB>(o, 0.125f * m8, lsum, sp, work - sp.n_dp, chunk);
      return;
    }
  if (qrow < S) {
    const float inv = o_scale / lsum;
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

// Score scale split: G = 2 dq dk log2(e) / sqrt(D) = c * 2^n with c in
// (1/(2 sqrt 2), 1/sqrt 2]; 2^(n+3) (the 8 turns exp2-domain scores into
// E4M3 code units) goes to the MFMA as two E8M0 operand scales (each in
// [2^-127, 2^127]).  |n + 3| > 254 is clamped (descale products that far out
// underflow or overflow fp32 scores anyway).
struct Fp8Scales {
  float q_mul;
  int sc_a, sc_b;
};
static Fp8Scales fp8_scales(const LaunchArgs& a) {
  const double G = (double)a.descale[0] * (double)a.descale[1] *
                   1.4426950408889634 * 2.0 / std::sqrt((double)a.D);
  const int n = (int)std::ceil(std::log2(G * 1.4142135623730951));
  int e = n + 3;
  if (e > 254) e = 254;
  if (e < -254) e = -254;
  const int na = e / 2, nb = e - na;
  return {(float)std::ldexp(G, -n), 127 + na, 127 + nb};
}

// K'' = e4m3(R k / 2) for the whole key tensor, one thread per 16-byte chunk
// (16 codes = 8 pairs of one axis block): the same table values, (cos, sin)/2
// in fp16, and the same packed-fp16 rotation as the kernel's staging of K.
template <int D>
__global__ __launch_bounds__(256) void rope4d_fp8_kernel(const uint8_t* __restrict__ k,
                                                         const int32_t* __restrict__ pos,
                                                         uint8_t* __restrict__ kr, long long nchunks,
                                                         int S, int H, RopeFreqs fr) {
  constexpr int CPK = D / 16, DA = D / 4;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    const int kc = (int)(c % CPK);
    const int s = (int)((c / CPK / H) % S);
    const int a = (16 * kc) / DA, j0 = ((16 * kc) % DA) / 2;
    const int p = pos[4 * s + a];
    const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(k + 16 * c);
    u32x4_t ky = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const float2 cf = rope_cs(p, fr.hi[j0 + jj], fr.lo[j0 + jj], kHalf);
      const h2_t cs = {(_Float16)cf.x, (_Float16)cf.y};
      const int w = jj >> 1;
      ky[w] = (uint32_t)((jj & 1) ? rope_pair_fp8_h<true>(kx[w], cs, (int)ky[w])
                                  : rope_pair_fp8_h<false>(kx[w], cs, (int)ky[w]));
    }
    *reinterpret_cast<u32x4_t*>(kr + 16 * c) = ky;
  }
}

template <int D, bool SPARSE, bool KPRE = false, bool SPLIT = false>
static hipError_t launch_fp8(const LaunchArgs& a) {
  const int nqt = (a.S + 255) / 256;
  const long long n = SPLIT ? (long long)a.split.n_dp + a.split.n_sk : (long long)a.B * a.H * nqt;
  const Fp8Scales s = fp8_scales(a);
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, SPARSE, KPRE, SPLIT>), dim3((unsigned)n), dim3(512), 0,
                     a.stream, (const uint8_t*)a.q, (const uint8_t*)(KPRE ? a.krot : a.k),
                     (const uint8_t*)a.v,
                     a.pos, (uint16_t*)a.out, a.S, a.H, nqt, a.freqs, s.q_mul, s.sc_a, s.sc_b,
                     a.descale[2], a.bmask, a.split);
  return hipGetLastError();
}

// the key codes rotated once into the workspace (a.krot)
template <int D>
static hipError_t rotate_keys_fp8(const LaunchArgs& a) {
  const long long nchunks = (long long)a.B * a.S * a.H * (D / 16);
  long long blocks = (nchunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(rope4d_fp8_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, a.stream,
                     (const uint8_t*)a.k, a.pos, (uint8_t*)a.krot, nchunks, a.S, a.H, a.freqs);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fp8_sparse(const LaunchArgs& a) {
  if (!a.krot) return launch_fp8<D, true>(a);
  const hipError_t e = rotate_keys_fp8<D>(a);
  return e != hipSuccess ? e : launch_fp8<D, true, true>(a);
}

template <int D>
static hipError_t launch_fp8_dense(const LaunchArgs& a) {
  if (a.krot) {
    // key codes rotated once into the workspace, then the kernel without K rotation
    hipError_t e = rotate_keys_fp8<D>(a);
    if (e != hipSuccess) return e;
    if (a.split.n_sk == 0) return launch_fp8<D, false, true>(a);
    e = launch_fp8<D, false, true, true>(a);
    return e != hipSuccess ? e : launch_split_merge(a, a.descale[2], nullptr);
  }
  if (a.split.n_sk > 0) {
    const hipError_t e = launch_fp8<D, false, false, true>(a);
    return e != hipSuccess ? e : launch_split_merge(a, a.descale[2], nullptr);
  }
  return launch_fp8<D, false>(a);
}

hipError_t launch_attn_fwd_fp8(const LaunchArgs& a) {
  if (a.bmask) return a.D == 128 ? launch_fp8_sparse<128>(a) : launch_fp8_sparse<64>(a);
  return a.D == 128 ? launch_fp8_dense<128>(a) : launch_fp8_dense<64>(a);
}

long long attn_fwd_fp8_grid(int B, int S, int H) {
  return (long long)B * H * ((S + 255) / 256);
}

}  // namespace klein
