// RoPE-4D joint self-attention forward, bf16 in / bf16 out, for gfx950.
//
// One workgroup owns one (batch, head, tile of BM = 256 queries) and streams
// every key of the sequence (no mask: all tokens attend to all tokens) in tiles
// of BN = 64 keys.  Its 8 waves (two per SIMD) own 32 queries each and run the
// same software pipeline; K' and V^T are double-buffered in LDS and one
// workgroup barrier per tile separates producers from consumers:
//
//   iteration t (S(t) already in registers):
//     region A:  S(t+1) = K'(t+1) Q'^T  (16 MFMAs)       interleaved with
//                P(t) = 2^(S(t) - m), row sums, bf16 pack   (VALU)
//     rare rescale of O, l and P(t) when P(t) came out too large
//     region B:  O^T += V(t)^T P(t)^T  (16 MFMAs)        interleaved with
//                staging K'(t+2) (RoPE-4D) and V(t+1)^T into LDS; before
//                its last two MFMAs (operands already in registers) the
//                buffer loads of K(t+3), V(t+2) from HBM, the barrier, and
//                the reads of region A's first K'(t+2) operands, which the
//                two MFMAs then cover
//
// Each wave overlaps its own MFMAs with its own VALU work, and both waves of
// a SIMD issue VALU: measured on this chip, one wave alone issues VALU at
// about half the rate two waves reach together, and the softmax / RoPE VALU
// work per tile is as large as the MFMA work.
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
// bf16) as the B operand.  Keys of a tile sit in LDS in a permuted row order
// so that accumulator register i of a lane in half g holds key 16g + i of its
// 32-key block; P's registers 8j..8j+7 then pair with the 8 contiguous keys
// 16g + 8j .. 16g + 8j + 7 of a V^T row, one 16-byte LDS read.
//
// Softmax runs in the exp2 domain (Q carries log2(e)/sqrt(D)).  The score
// MFMA chains start from -m (the running row max) rather than zero, so the
// accumulators hold s - m directly.  No row max is taken per tile: m moves
// (and O and l are rescaled) only when a tile's p = 2^(s - m), summed over the
// 32 keys a lane holds, exceeds 2^16, so p <= 2^16 in between (or on overflow
// to inf); the tile's P is then recomputed from its scores.  The final O / l
// is the same either way.
//
// V^T operands, two ways.  When v arrives regrouped into key-major tiles (a
// pass before the kernel writes, per 64-key tile, one row of 64 keys per
// channel), the tile is staged with plain 16-byte copies and each operand (8
// keys of one channel) is one 16-byte LDS read.  Otherwise V stays row-major
// in LDS ([key][d], plain 16-byte copies too) and the operand is read with
// ds_read_b64_tr_b16: inside a 16-lane group, lane i receives element i % 4
// of the 8-byte words addressed by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.
// Pointing lane L at V[key0 + L/4][d0 + 4 (L % 4) .. + 3] hands lane i keys
// key0 .. key0+3 of channel d0 + i; two such reads give the 8 keys of one
// MFMA operand.  The transposing reads move half the bytes per clock of plain
// 16-byte reads, and the LDS is nearly a second bound of this loop.
//
// LDS bank spreading: K rows are padded by 16 bytes (the 16 lanes of one
// 16-byte read phase hit 16 consecutive rows); row-major V rows by 64 bytes,
// so the 4 rows x 64 bytes a 32-lane transposing read phase touches fall on
// disjoint banks; key-major V rows (128 bytes) by 16 bytes, so 16 lanes on
// consecutive channels hit all 64 banks once.  Every operand address is a
// per-lane base plus a constant.
#include "klein_device.hpp"
#include "klein_launch.hpp"

namespace klein {

// Per-region cycle counts of the pipeline step, for a measurement build
// only: defined by the step_clock.hip harness, never by the library.  Each
// wave sums, over its steps, the shader-clock cycles (s_memtime) between
// marks at the step start, after region A, after the rescale check, after
// region B, after the buffer loads and after the barrier, and lane 0
// writes them, with the step count, the cycles of the whole loop and its
// fixed-rate timestamps (s_memrealtime), to klein_step_clock_out[8 wg +
// wave][0..9].
#ifdef KLEIN_STEP_CLOCK
__device__ unsigned long long* klein_step_clock_out;
#define KLEIN_CLOCK_START                                                    \
  unsigned long long clk_sum[6] = {0, 0, 0, 0, 0, 0};                        \
  const unsigned long long clk_real0 = __builtin_amdgcn_s_memrealtime();     \
  unsigned long long clk_prev = __builtin_amdgcn_s_memtime();                \
  const unsigned long long clk_start = clk_prev;
#define KLEIN_CLOCK_MARK(i)                                                  \
  do {                                                                       \
    const unsigned long long clk_now = __builtin_amdgcn_s_memtime();         \
    clk_sum[i] += clk_now - clk_prev;                                        \
    clk_prev = clk_now;                                                      \
  } while (0)
#define KLEIN_CLOCK_STORE(nsteps)                                            \
  if (klein_step_clock_out != nullptr && lane == 0) {                        \
    unsigned long long* co = klein_step_clock_out + ((size_t)blockIdx.x * 8 + wave) * 10; \
    for (int i = 0; i < 6; ++i) co[i] = clk_sum[i];                          \
    co[6] = (unsigned long long)(nsteps);                                    \
    co[7] = clk_prev - clk_start;                                            \
    co[8] = clk_real0;                                                       \
    co[9] = __builtin_amdgcn_s_memrealtime();                                \
  }
#else
#define KLEIN_CLOCK_START
#define KLEIN_CLOCK_MARK(i) do {} while (0)
#define KLEIN_CLOCK_STORE(nsteps)
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

constexpr int kTabN = 256;        // positions covered by the cos/sin table

// SPARSE: block-sparse variant; bmask holds one byte per (batch, head, query
// tile of 256, key tile of 64), nonzero = compute, and only the kept key
// tiles of a query tile stream through the pipeline (in ascending order, so
// with every tile kept the result is bit-identical to the dense kernel).
// ROT: where the rotation happens.  kRotInKernel: Q once per workgroup and
// every K tile on its way to LDS (cos/sin from an LDS table).  kRotKPre: k
// arrives rotated, as fp16 (one elementwise pass over K before the call, so
// each key is rotated once instead of once per query tile); Q is rotated in
// the kernel.  kRotBothPre: q and k both arrive rotated as fp16 (the
// projection's RoPE epilogue emits them so); Q is only scaled.  With k
// pre-rotated, K tiles are copied to LDS as they are, with no table,
// positions or rotation.
// SPLIT: the split-KV schedule (SplitArgs): whole items first, then the key
// chunks of the remaining items, merged through the workspace.
// VT: v arrives regrouped into key-major tiles (per (b, h) and 64-key tile, D
// rows of 64 keys, zero past S; launch_v_tiles), so each V^T operand is one
// 16-byte LDS read instead of two transposing 8-byte reads.
template <int D, bool SPARSE, int ROT, bool SPLIT, bool VT>
__global__ __launch_bounds__(512) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ out, int S, int H, int nqt, RopeFreqs fr, float qscale,
    const uint8_t* __restrict__ bmask, SplitArgs sp, float* __restrict__ lse) {
  constexpr int BM = 256;              // queries per workgroup (8 waves x 32)
  constexpr int BN = 64;               // keys per tile
  constexpr int NT = 512;              // threads
  constexpr int CPR = D / 8;           // 16-byte chunks per token row
  constexpr int KPT = BN * CPR / NT;   // keys per thread when staging a tile
  constexpr int KS = D / 16;           // MFMA k-steps of Q K^T
  constexpr int MB = D / 32;           // 32-row blocks of O^T
  constexpr int KROW = D + 8;          // LDS row stride of K' (16-bit), padded
  constexpr int VROW = D + 32;         // LDS row stride of V (bf16), padded
  constexpr int VTROW = BN + 8;        // LDS row stride of a key-major V tile (bf16), padded
  constexpr int DA = D / 4;            // channels per RoPE axis
  constexpr float kSumLimit = 65536.0f;   // 2^16: the rescale trigger
  constexpr int NJ = D / 8;            // rotation pairs per axis
  constexpr int TROW = NJ + 1;         // cos/sin table row stride (float2)
  constexpr int TSLOT = 4 * KPT + 1;   // per-thread fallback slot stride
  constexpr int TAB = kTabN * TROW;    // start of the fallback slots
  static_assert(KPT >= 1 && (BN * CPR) % NT == 0, "tile/thread split");
  static_assert(KPT == 1 || KPT % 2 == 0, "V^T store packs key pairs");
  static_assert(!(SPARSE && SPLIT), "one schedule at a time");
  static_assert(!VT || (!SPARSE && D * VTROW <= BN * VROW), "key-major V tiles: dense, fit");
  constexpr bool QPRE = ROT == kRotBothPre;     // q arrives rotated (fp16)
  constexpr bool KPRE = ROT != kRotInKernel;    // k arrives rotated (fp16)

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BN * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][BN * VROW];
  // (cos, sin) of every pair at positions [0, kTabN), then per-thread slots
  // for keys at other positions; odd strides spread rows over the banks
  __shared__ __attribute__((aligned(16))) float2 cs_tab[TAB + TSLOT * NT];
  __shared__ uint16_t klist[SPARSE ? kSparseMaxTiles + kSparsePad : 1];
  __shared__ int klist_n;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lr = lane & 31;
  const int nkt = (S + BN - 1) / BN;
  const size_t rs = (size_t)H * D;                       // token stride

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

  // ---- cos/sin table (the very values rope_chunk computes)
  if constexpr (!KPRE) {
    for (int e = tid; e < kTabN * NJ; e += NT) {
      const int j = e % NJ, p = e / NJ;
      const float rev = rope_rev((float)p, fr.hi[j], fr.lo[j]);
      cs_tab[p * TROW + j] = make_float2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
    }
  }

  const int qt = work % nqt;
  const int bh = work / nqt;
  const int h = bh % H, b = bh / H;
  const size_t base = (size_t)b * S * rs + (size_t)h * D;
  const uint16_t* qb = q + base;
  // keys, values and key positions from the segment's first tile on; Sk
  // keys remain from there
  const uint16_t* kb = k + base + (size_t)k0 * BN * rs;
  const uint16_t* vb = VT ? v + ((size_t)bh * nkt + k0) * (D * BN) : v + base + (size_t)k0 * BN * rs;
  const int32_t* kposb = pos + (size_t)k0 * BN * 4;
  const int Sk = S - k0 * BN;

  // ---- this lane's query: rotate, scale by log2(e)/sqrt(D), fp16 in VGPRs.
  // Rows past S load row S-1 (in bounds) and are never stored.
  const int qrow = qt * BM + wave * 32 + lr;
  const int qload = qrow < S ? qrow : S - 1;
  f16x8_t qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int d0 = 16 * ks + 8 * g;
    const int a = d0 / DA, j0 = (d0 % DA) / 2;
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qb + (size_t)qload * rs + d0);
    if constexpr (QPRE) {
      typedef float f32x8v_t __attribute__((ext_vector_type(8)));
      const f32x8v_t xf = __builtin_convertvector(__builtin_bit_cast(f16x8_t, x), f32x8v_t);
      qreg[ks] = __builtin_convertvector(xf * qscale, f16x8_t);
    } else {
      qreg[ks] = __builtin_bit_cast(
          f16x8_t, rope_chunk<true>(x, pos[4 * qload + a], &fr.hi[j0], &fr.lo[j0], qscale));
    }
  }

  // ---- staging assignment: chunk lc of keys lk .. lk+KPT-1 of a K or V tile
  // (CPR lanes per key row, whole rows per load)
  const int lc = tid % CPR;
  const int lk = (tid / CPR) * KPT;
  const int la = (8 * lc) / DA, lj0 = ((8 * lc) % DA) / 2;

  // Global -> registers through buffer loads.  Each tile gets a descriptor
  // whose base is the tile's first row and whose size covers only the rows
  // that exist, so the hardware returns zeros for rows past S (no clamping and
  // no per-load address arithmetic: the per-thread byte offsets are fixed).
  const int rowb = (int)(rs * 2);                          // bytes per token row
  // byte offsets of key lk (key lk + it adds it * rowb, a scalar offset)
  const int voff = lk * rowb + 16 * lc;
  const int voff_p = (lk * 4 + la) * 4;
  // tile index of pipeline position t (the kept list when SPARSE)
  auto tl = [&](int t) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)klist[t]);
    else return t;
  };
  u32x4_t kx[KPT], vx[KPT];
  // positions of this thread's K keys, loaded one step ahead of the K data:
  // ring slot kt & 1 holds tile kt's
  int kpos0[KPT], kpos1[KPT];
  auto tile_rows = [&](int kt) {
    const int n = Sk - kt * BN;
    return n < 0 ? 0 : (n > BN ? BN : n);
  };
  auto load_k = [&](int kt) {
    const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(kb + (size_t)kt * BN * rs, tile_rows(kt) * rowb);
#pragma unroll
    for (int it = 0; it < KPT; ++it)
      kx[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, voff, it * rowb, 0));
  };
  auto load_pos = [&](int kt, int* slot) {
    if constexpr (KPRE) return;
    const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(kposb + (size_t)kt * BN * 4, tile_rows(kt) * 16);
#pragma unroll
    for (int it = 0; it < KPT; ++it)
      slot[it] = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, voff_p, it * 16, 0);
  };
  // (cos, sin) of the 4 pairs of K chunk `it`, as an index into cs_tab: the
  // table row of its position, or (position outside the table) the thread's
  // own slots, filled here in a divergent branch that waves whose positions
  // all lie in the table skip.
  auto key_cs_index = [&](const int* kp, int it) {
    if constexpr (KPRE) return 0;
    const bool oob = (unsigned)kp[it] >= (unsigned)kTabN;
    if (oob) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        int j = lj0 + jj;
        asm volatile("" : "+v"(j));      // keep the loads in this rare path
        const float rev = rope_rev((float)kp[it], fr.hi[j], fr.lo[j]);
        cs_tab[TAB + TSLOT * tid + 4 * it + jj] =
            make_float2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
      }
    }
    return oob ? TAB + TSLOT * tid + 4 * it : kp[it] * TROW + lj0;
  };
  // one rotated pair (x, y) -> (x c - y s, x s + y c), fp16
  auto rot_pair = [&](uint32_t xw, float2 cs) {
    const f32x2_t r = rope_rot(bf16_lo(xw), bf16_hi(xw), cs.x, cs.y);
    return pack_f16x2(r[0], r[1]);
  };
  auto load_v = [&](int kt) {
    if constexpr (VT) {
      // the whole key-major tile (its padding is zero), 16-byte chunk tid + NT it;
      // an empty descriptor past the segment's last tile
      const __amdgpu_buffer_rsrc_t rv =
          uniform_rsrc(vb + (size_t)kt * D * BN, tile_rows(kt) > 0 ? D * BN * 2 : 0);
#pragma unroll
      for (int it = 0; it < KPT; ++it)
        vx[it] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, 16 * (tid + NT * it), 0, 0));
    } else {
      const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(vb + (size_t)kt * BN * rs, tile_rows(kt) * rowb);
#pragma unroll
      for (int it = 0; it < KPT; ++it)
        vx[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, it * rowb, 0));
    }
  };
  // Registers -> LDS: K rotated (fp16), at its permuted row; V transposed.
  auto stage_k = [&](int buf, const int* kp) {
#pragma unroll
    for (int it = 0; it < KPT; ++it) {
      const int key = lk + it;
      const int row = (key & ~31) + key_to_row(key & 31);
      u32x4_t y;
      if constexpr (KPRE) {
        y = kx[it];
      } else {
        const int ci = key_cs_index(kp, it);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) y[jj] = rot_pair(kx[it][jj], cs_tab[ci + jj]);
      }
      *reinterpret_cast<u32x4_t*>(&k_lds[buf][row * KROW + 8 * lc]) = y;
    }
  };
  auto stage_v_chunk = [&](int buf, int it) {
    if constexpr (VT) {
      const int c = tid + NT * it;     // channel c / 8, keys 8 (c % 8) .. + 7
      *reinterpret_cast<u32x4_t*>(&v_lds[buf][(c >> 3) * VTROW + 8 * (c & 7)]) = vx[it];
    } else {
      *reinterpret_cast<u32x4_t*>(&v_lds[buf][(lk + it) * VROW + 8 * lc]) = vx[it];
    }
  };
  auto stage_v = [&](int buf) {
#pragma unroll
    for (int it = 0; it < KPT; ++it) stage_v_chunk(buf, it);
  };
  // this lane's base element of the transposing V reads (see the header):
  // lane L = lane % 16 of group G = lane / 16 reads row 16 (G / 2) + L / 4,
  // channels 16 (G % 2) + 4 (L % 4) .. + 3, of the 4-key group addressed
  const int vtr_base = (16 * (lane >> 5) + ((lane & 15) >> 2)) * VROW +
                       16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16_t o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = (f32x16_t){};
  float m_run = 0.f, l_run = 0.f;

  // S^T = K'(tile in buf) Q'^T, two 32-key blocks, each a chain of KS MFMAs
  // (used on its own only in the prologue)
  auto qk = [&](int buf, f32x16_t* s) {
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
      s[kbk] = (f32x16_t){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const f16x8_t a = *reinterpret_cast<const f16x8_t*>(
            &k_lds[buf][(32 * kbk + lr) * KROW + 16 * ks + 8 * g]);
        s[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qreg[ks], s[kbk], 0, 0, 0);
      }
    }
  };
  // Scores are kept relative to the running max: the S MFMA chains start
  // from C = cinit = -m_run instead of zero, so S' = S - m needs no VALU
  // subtraction.  Row max of the 32 values a lane holds, as a max3 tree.
  auto rowmax32 = [&](const f32x16_t* sc) {
    float m[12];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      const int a = 3 * i, b = 3 * i + 1, c = 3 * i + 2;
      m[i] = __builtin_fmaxf(sc[a >> 4][a & 15],
                             __builtin_fmaxf(sc[b >> 4][b & 15], sc[c >> 4][c & 15]));
    }
    m[10] = sc[1][14];
    m[11] = sc[1][15];
    float n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) n[i] = __builtin_fmaxf(m[3 * i], __builtin_fmaxf(m[3 * i + 1], m[3 * i + 2]));
    return pair_max(__builtin_fmaxf(n[0], __builtin_fmaxf(n[1], __builtin_fmaxf(n[2], n[3]))));
  };
  f32x16_t cinit;
  auto set_cinit = [&]() {
#pragma unroll
    for (int i = 0; i < 16; ++i) cinit[i] = -m_run;
  };
  // keys past S (last tile only) take -inf before the exponent
  auto mask_tail = [&](int t, f32x16_t* sc) {
    if (t * BN + BN > Sk) {
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (t * BN + 32 * kbk + 16 * g + i >= Sk) sc[kbk][i] = kNegInf;
    }
  };
  const bf16x2_t kOnesBf16x2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  // The rare rescale, once a tile's P (from S(t) = cur) came out too large:
  // m_run moves up to the tile's row max where that is higher, O and l take
  // 2^-delta, S(t) and S(t+1) (already formed against the old m) shift by
  // -delta, and P(t) and this lane's sum of it are recomputed.
  auto rescale = [&](f32x16_t* cur, f32x16_t* nxt, uint32_t (*pw)[8]) {
    const float delta = __builtin_fmaxf(rowmax32(cur), 0.f);
    const float alpha = __builtin_amdgcn_exp2f(-delta);
    m_run += delta;
    l_run *= alpha;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
      cur[kbk] -= delta;
      nxt[kbk] -= delta;
    }
    set_cinit();
    float ls = 0.f;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const uint32_t pk = pack_bf16x2(__builtin_amdgcn_exp2f(cur[kbk][2 * w]),
                                        __builtin_amdgcn_exp2f(cur[kbk][2 * w + 1]));
        pw[kbk][w] = pk;
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), kOnesBf16x2, ls, false);
      }
    return ls;
  };

  // Region A: S(t+1) = K'(t+1) Q'^T (2 KS MFMAs, operands read two MFMAs
  // ahead) with one slice of the softmax of S(t) after each MFMA; the
  // sched_barrier fences keep the compiler from regrouping the slices.
  // Returns this lane's sum of P(t).
  constexpr int NA = 2 * KS;                 // MFMAs in region A
  constexpr int SA = 16;                     // softmax slices (2 scores each)
  // the K' operand of region A's MFMA i (the first two are read ahead of the
  // region, right after the barrier that completes the buffer)
  auto read_k_op = [&](int kbuf, int i) {
    const int kbk = i / KS, ks = i % KS;
    return *reinterpret_cast<const f16x8_t*>(&k_lds[kbuf][(32 * kbk + lr) * KROW + 16 * ks + 8 * g]);
  };
  auto region_a = [&](int kbuf, const f32x16_t* cur, f32x16_t* nxt, uint32_t (*pw)[8],
                      const f16x8_t* pre) {
    f16x8_t ka[NA];
    auto read_k = [&](int i) {
      const int kbk = i / KS, ks = i % KS;
      ka[i] = *reinterpret_cast<const f16x8_t*>(
          &k_lds[kbuf][(32 * kbk + lr) * KROW + 16 * ks + 8 * g]);
    };
    nxt[0] = cinit;
    nxt[1] = cinit;
    ka[0] = pre[0];
    ka[1] = pre[1];
    float ls4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (i + 2 < NA) read_k(i + 2);
      const int kbk = i / KS, ks = i % KS;
      nxt[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[i], qreg[ks], nxt[kbk], 0, 0, 0);
#pragma unroll
      for (int sl = i * SA / NA; sl < (i + 1) * SA / NA; ++sl) {
        const int kb2 = sl >> 3, w = sl & 7;
        const float p0 = __builtin_amdgcn_exp2f(cur[kb2][2 * w]);
        const float p1 = __builtin_amdgcn_exp2f(cur[kb2][2 * w + 1]);
        const uint32_t pk = pack_bf16x2(p0, p1);
        pw[kb2][w] = pk;
        // row sum of the bf16 P that the MFMA consumes: one dot2 per pair
        ls4[w & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk),
                                                     kOnesBf16x2, ls4[w & 3], false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
  };

  // Region B: O^T += V(t)^T P(t)^T (4 MB MFMAs) with the staging of K'(t+2)
  // (RoPE-4D, one pair per slice) and V(t+1) spread over the MFMAs; then the
  // loads of K(t+3), V(t+2).
  constexpr int NB = 4 * MB;                 // MFMAs in region B
  constexpr int NROT = KPRE ? KPT : 4 * KPT;   // RoPE pairs (or K chunks) to stage
  constexpr int NVW = KPT;                   // V chunks to stage
  constexpr int NIT = NROT + NVW;
  // `mid` runs before the last two MFMAs (the loads of later tiles, the
  // barrier, the reads ahead of the next region A); the staging items all
  // sit in the MFMA slots before it
  constexpr int NBS = NB - 2;
  auto region_b = [&](int vbuf, int kdst, int vdst, const uint32_t (*pw)[8], const int* ci,
                      auto&& mid) {
    float2 kcs[NROT];
    auto read_cs = [&](int item) {
      if constexpr (!KPRE)
        if (item < NROT) kcs[item] = cs_tab[ci[item / 4] + item % 4];
    };
    read_cs(0);
    read_cs(1);
    bf16x8_t va[NB];
    auto read_v = [&](int i) {
      const int mb = i / 4, kbk = (i >> 1) & 1, j = i & 1;
      // keys 32 kbk + 16 g + 8 j + [0, 4) and + [4, 8), channel 32 mb + lr
      if constexpr (VT) {
        va[i] = *reinterpret_cast<const bf16x8_t*>(
            &v_lds[vbuf][(32 * mb + lr) * VTROW + 32 * kbk + 16 * g + 8 * j]);
        return;
      }
      const uint16_t* src = &v_lds[vbuf][vtr_base + (32 * kbk + 8 * j) * VROW + 32 * mb];
      typedef short s16x4_t __attribute__((ext_vector_type(4)));
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(src));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(src + 4 * VROW));
      const s16x8_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      va[i] = __builtin_bit_cast(bf16x8_t, both);
    };
    read_v(0);
    read_v(1);
    u32x4_t ky;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i == NBS) mid();
      if (i + 2 < NB) read_v(i + 2);
      const int mb = i / 4, kbk = (i >> 1) & 1, j = i & 1;
      const u32x4_t pvw = {pw[kbk][4 * j], pw[kbk][4 * j + 1], pw[kbk][4 * j + 2],
                           pw[kbk][4 * j + 3]};
      o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], __builtin_bit_cast(bf16x8_t, pvw),
                                                      o[mb], 0, 0, 0);
#pragma unroll
      for (int item = i * NIT / NBS; item < (i < NBS ? (i + 1) * NIT / NBS : 0); ++item) {
        read_cs(item + 2);
        if (KPRE && item < NROT) {
          // one pre-rotated K chunk, copied
          const int key = lk + item;
          const int row = (key & ~31) + key_to_row(key & 31);
          *reinterpret_cast<u32x4_t*>(&k_lds[kdst][row * KROW + 8 * lc]) = kx[item];
        } else if (item < NROT) {
          // one RoPE pair of K chunk c
          const int c = item / 4, jj = item % 4;
          ky[jj] = rot_pair(kx[c][jj], kcs[item]);
          if (jj == 3) {        // chunk complete: one 16-byte store
            const int key = lk + c;
            const int row = (key & ~31) + key_to_row(key & 31);
            *reinterpret_cast<u32x4_t*>(&k_lds[kdst][row * KROW + 8 * lc]) = ky;
          }
        } else {
          stage_v_chunk(vdst, item - NROT);    // one V chunk
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
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
        uint16_t* orow = out + base + (size_t)qrow * rs;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<uint2*>(orow + 32 * mb + 8 * i4 + 4 * g) = make_uint2(0u, 0u);
      }
      return;
    }
  }

  // ---- prologue: K'(0), K'(1), V(0)^T in LDS; S(0) in registers; K(2), V(1)
  // in flight (pipeline positions; tl() maps them to tiles)
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
  uint32_t pw[2][8];
  qk(0, sa);
  __syncthreads();        // K buffer 0 is refilled in iteration 0
  // m_run starts at tile 0's exact row max (keys past S masked), so scores
  // are relative from the first tile on and no row can underflow
  const int kt0 = tl(0);
  if (kt0 * BN + BN > Sk) {
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kt0 * BN + 32 * kbk + 16 * g + i >= Sk) sa[kbk][i] = kNegInf;
  }
  m_run = rowmax32(sa);
#pragma unroll
  for (int kbk = 0; kbk < 2; ++kbk) sa[kbk] -= m_run;
  set_cinit();

  // one pipeline step; `cur` holds S(t), `nxt` receives S(t+1)
  // `kps` holds the positions of K(t+2) and receives those of K(t+4).  The
  // rare branches (rotation fallback, rescale) sit between the regions.
  KLEIN_CLOCK_START
  f16x8_t kpre[2] = {read_k_op(1, 0), read_k_op(1, 1)};
  auto step = [&](int t, f32x16_t* cur, f32x16_t* nxt, int* kps) {
    int ci[KPT];
#pragma unroll
    for (int it = 0; it < KPT; ++it) ci[it] = key_cs_index(kps, it);
    mask_tail(tl(t), cur);
    KLEIN_SYNC_POINT();
    KLEIN_CLOCK_MARK(0);
    float lt = region_a((t + 1) & 1, cur, nxt, pw, kpre);
    KLEIN_SYNC_POINT();
    KLEIN_CLOCK_MARK(1);
    if (__builtin_amdgcn_ballot_w64(lt > kSumLimit)) lt = rescale(cur, nxt, pw);
    l_run += lt;
    KLEIN_SYNC_POINT();
    KLEIN_CLOCK_MARK(2);
    // K(t+2) into buffer t&1 (it held K(t), consumed last step); V(t+1) into
    // buffer (t+1)&1 (it held V(t-1), consumed last step).  The barrier comes
    // before region B's last two MFMAs, whose V operands are already in
    // registers, and the next region A's first K(t+2) operands are read
    // while they run.
    region_b(t & 1, t & 1, (t + 1) & 1, pw, ci, [&]() {
      KLEIN_SYNC_POINT();
      KLEIN_CLOCK_MARK(3);
      load_k(tl(t + 3));
      load_pos(tl(t + 4), kps);
      load_v(tl(t + 2));
      KLEIN_CLOCK_MARK(4);
      __syncthreads();
      KLEIN_CLOCK_MARK(5);
      kpre[0] = read_k_op(t & 1, 0);
      kpre[1] = read_k_op(t & 1, 1);
    });
    KLEIN_SYNC_POINT();
    KLEIN_CLOCK_MARK(3);
  };
  int t = 0;
  for (; t + 1 < nsteps; t += 2) {
    step(t, sa, sb, kpos0);
    step(t + 1, sb, sa, kpos1);
  }
  if (t < nsteps) step(t, sa, sb, kpos0);
  KLEIN_CLOCK_STORE(nsteps)

  // ---- epilogue: O / l, bf16, store (lane holds channels 32mb + 8(i/4) + 4g + i%4);
  // a chunk of a split item stores its partial instead (the merge kernel
  // writes those rows)
  const float lsum = pair_sum(l_run);
  if constexpr (SPLIT)
    if (k0 != 0 || k1 != nkt) {
      split_store<MB>(o, m_run, lsum, sp, work - sp.n_dp, chunk);
      return;
    }
  if (qrow < S) {
    const float inv = 1.0f / lsum;
    // the softmax log-sum-exp (natural log of sum_j exp(s_ij)) for a backward
    // pass: the scores are kept in log2 units relative to m_run
    if (lse != nullptr && g == 0)
      lse[((size_t)b * H + h) * S + qrow] = (m_run + __builtin_amdgcn_logf(lsum)) * kLn2;
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

template <int D, bool SPARSE, int ROT = kRotInKernel, bool SPLIT = false, bool VT = false>
static hipError_t launch_bf16(const LaunchArgs& a) {
  constexpr int BM = 256;
  const int nqt = (a.S + BM - 1) / BM;
  const long long n = SPLIT ? (long long)a.split.n_dp + a.split.n_sk : (long long)a.B * a.H * nqt;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, SPARSE, ROT, SPLIT, VT>), dim3((unsigned)n),
                     dim3(512), 0, a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)(ROT == kRotKPre ? a.krot : a.k),
                     (const uint16_t*)(VT ? a.vt : a.v),
                     a.pos, (uint16_t*)a.out, a.S, a.H, nqt, a.freqs, a.qscale_log2, a.bmask,
                     a.split, a.lse);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bf16_dense(const LaunchArgs& a) {
  if (a.krot) {
    // k rotated once into the workspace, then the kernel without K rotation
    hipError_t e = launch_rope4d_fp16(a.k, a.pos, a.krot, a.B, a.S, a.H, D, a.freqs, 1.0f, a.stream);
    if (e != hipSuccess) return e;
    if (a.vt) {
      // and v regrouped into key-major tiles
      e = launch_v_tiles(a.v, a.vt, a.B, a.S, a.H, D, a.stream);
      if (e != hipSuccess) return e;
      if (a.split.n_sk == 0) return launch_bf16<D, false, kRotKPre, false, true>(a);
      e = launch_bf16<D, false, kRotKPre, true, true>(a);
      return e != hipSuccess ? e : launch_split_merge(a, 1.0f, a.lse);
    }
    if (a.split.n_sk == 0) return launch_bf16<D, false, kRotKPre>(a);
    e = launch_bf16<D, false, kRotKPre, true>(a);
    return e != hipSuccess ? e : launch_split_merge(a, 1.0f, a.lse);
  }
  if (a.split.n_sk > 0) {
    const hipError_t e = launch_bf16<D, false, kRotInKernel, true>(a);
    return e != hipSuccess ? e : launch_split_merge(a, 1.0f, a.lse);
  }
  return launch_bf16<D, false>(a);
}

template <int D>
static hipError_t launch_bf16_sparse(const LaunchArgs& a) {
  if (!a.krot) return launch_bf16<D, true>(a);
  // k rotated once into the workspace, then the block-sparse kernel without K rotation
  const hipError_t e = launch_rope4d_fp16(a.k, a.pos, a.krot, a.B, a.S, a.H, D, a.freqs, 1.0f,
                                          a.stream);
  return e != hipSuccess ? e : launch_bf16<D, true, kRotKPre>(a);
}

hipError_t launch_attn_fwd_bf16(const LaunchArgs& a) {
  if (a.bmask) return a.D == 128 ? launch_bf16_sparse<128>(a) : launch_bf16_sparse<64>(a);
  return a.D == 128 ? launch_bf16_dense<128>(a) : launch_bf16_dense<64>(a);
}

hipError_t launch_attn_fwd_prerotated(const LaunchArgs& a) {
  return a.D == 128 ? launch_bf16<128, false, kRotBothPre>(a) : launch_bf16<64, false, kRotBothPre>(a);
}

long long attn_fwd_bf16_grid(int B, int S, int H) {
  const int BM = 256;
  return (long long)B * H * ((S + BM - 1) / BM);
}

}  // namespace klein
