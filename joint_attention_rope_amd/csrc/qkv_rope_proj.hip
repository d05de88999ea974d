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
// conversions happen in registers (the angle of each pair is formed once per
// output element, like the attention kernels' Q); the rounded outputs then
// pass through LDS so that the only stores write whole cache lines.
//
// One workgroup of 8 waves computes 256 features x 256 tokens, K in steps of
// 128 bytes; each wave owns 128 features x 64 tokens (4 x 2 MFMA tiles of
// 32 x 32; bf16: 0.75 16-byte LDS operand reads per MFMA, fp8: 1.5 per MFMA
// of twice the length).  W and x tiles
// are double-buffered in LDS (rows padded to 144 bytes, so the 16 rows one
// 16-lane read phase touches fall on distinct banks) and staged through
// registers, two K steps ahead (bf16) or one (fp8), with the loads and the
// stores spread between the MFMAs; one barrier per K step, which bf16 places
// before the step's last sub-step so that the reads of the next buffer
// overlap MFMAs.  Rows past N or M read as zeros through the buffer
// descriptors and are not stored.
//
// The grid is persistent: one workgroup per compute unit, each looping over
// its share of the tiles.  The last K steps of a tile load the next tile's
// first steps (into the LDS buffer its epilogue leaves alone, and for bf16
// its second step into the staging registers), and its epilogue loads the
// next tile's positions and bias into a second LDS copy, so a tile after the
// first starts with its first K step in place.
#include <type_traits>

#include "klein_device.hpp"
#include "klein_launch.hpp"

namespace klein {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Per-part cycle counts of the K step, for a measurement build only: defined
// by the step_clock.hip harness, never by the library.  Each wave sums, over
// the K steps of all its tiles, the shader-clock cycles (s_memtime) of each
// k-sub-step (with the staging slots in it) and of the barrier, and lane 0
// writes them, with the K-step count and the cycles of the K loops, of what
// precedes each (kernel entry or the previous tile's end) and of the
// epilogues, to klein_qkv_clock_out[10 (8 wg + wave) + 0..8].
#ifdef KLEIN_STEP_CLOCK
__device__ unsigned long long* klein_qkv_clock_out;
#define KLEIN_QKV_CLOCK_ENTRY                                                \
  unsigned long long qclk_sum[5] = {0, 0, 0, 0, 0};                          \
  unsigned long long qclk_pro = 0, qclk_loop = 0, qclk_epi = 0, qclk_nk = 0; \
  unsigned long long qclk_prev = __builtin_amdgcn_s_memtime();               \
  unsigned long long qclk_start = qclk_prev, qclk_tile_end = qclk_prev;
#define KLEIN_QKV_CLOCK_START                                                \
  qclk_prev = __builtin_amdgcn_s_memtime();                                  \
  qclk_start = qclk_prev;                                                    \
  qclk_pro += qclk_start - qclk_tile_end;
#define KLEIN_QKV_CLOCK_MARK(i)                                              \
  do {                                                                       \
    const unsigned long long qclk_now = __builtin_amdgcn_s_memtime();        \
    qclk_sum[i] += qclk_now - qclk_prev;                                     \
    qclk_prev = qclk_now;                                                    \
  } while (0)
#define KLEIN_QKV_CLOCK_TILE_END(nk)                                         \
  do {                                                                       \
    const unsigned long long qclk_now = __builtin_amdgcn_s_memtime();        \
    qclk_loop += qclk_prev - qclk_start;                                     \
    qclk_epi += qclk_now - qclk_prev;                                        \
    qclk_nk += (unsigned long long)(nk);                                     \
    qclk_tile_end = qclk_now;                                                \
  } while (0)
#define KLEIN_QKV_CLOCK_STORE                                                \
  if (klein_qkv_clock_out != nullptr && lane == 0) {                         \
    unsigned long long* co = klein_qkv_clock_out + ((size_t)blockIdx.x * 8 + wave) * 10; \
    for (int i = 0; i < 5; ++i) co[i] = qclk_sum[i];                         \
    co[5] = qclk_nk;                                                         \
    co[6] = qclk_loop;                                                       \
    co[7] = qclk_pro;                                                        \
    co[8] = qclk_epi;                                                        \
  }
#else
#define KLEIN_QKV_CLOCK_ENTRY
#define KLEIN_QKV_CLOCK_START
#define KLEIN_QKV_CLOCK_MARK(i) do {} while (0)
#define KLEIN_QKV_CLOCK_TILE_END(nk) do {} while (0)
#define KLEIN_QKV_CLOCK_STORE
#endif

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
  // What the epilogue reads besides the accumulators: the tile's token
  // positions and bias as fp32 (two copies: the next tile's are loaded while
  // this tile's epilogue runs), and the RoPE frequencies (hi[16], lo[16]),
  // which a lane reads with one LDS read instead of selecting between kernel
  // arguments.
  __shared__ __attribute__((aligned(16))) float ep_pos[2][TM][4];
  __shared__ __attribute__((aligned(16))) float ep_bias[2][TN];
  __shared__ __attribute__((aligned(16))) float ep_fr[32];

  KLEIN_QKV_CLOCK_ENTRY
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lr = lane & 31;
  const int wn = wave & 1, wm = wave >> 1;     // 2 x 4 waves: 128 features x 64 tokens
  // Tile order: each XCD (own L2) takes a contiguous range of the tile list
  // (xcd_remap), and the list runs through groups of kGroupM token tiles,
  // token tile fastest: the 32 workgroups an XCD runs at once then cover
  // 8 token tiles x 4 feature tiles, so 12 operand panels (8 of x, 4 of W,
  // 1.5 MB each at C = 3072) are shared in its L2 instead of 1 of x and 32
  // of W.
  constexpr int kGroupM = 8;
  const int ntile_m = (M + TM - 1) / TM;
  const int ntiles = ntile_m * ntile_n;
  const int gsz = kGroupM * ntile_n;
  const int HD = H * D;
  const int rowb = C * ES;
  const int nk = C * ES / KB;
  // Persistent: workgroup b computes the tiles of the virtual workgroups
  // b, b + G, b + 2G, ... (G = gridDim.x, a multiple of 8, so virtual
  // workgroup v runs on XCD v mod 8 as xcd_remap assumes); (n0, m0) of the
  // tile of virtual workgroup v:
  auto tile_origin = [&](int v, int& n0o, int& m0o) {
    const int L = xcd_remap(v, ntiles);
    const int m_first = (L / gsz) * kGroupM;
    const int gm = min(ntile_m - m_first, kGroupM);
    m0o = (m_first + (L % gsz) % gm) * TM;
    n0o = ((L % gsz) / gm) * TN;
  };
  auto rsrc_w = [&](int n0o) {
    return uniform_rsrc(static_cast<const uint8_t*>(wv) + (size_t)n0o * rowb,
                        min(TN, N - n0o) * rowb);
  };
  auto rsrc_x = [&](int m0o) {
    return uniform_rsrc(static_cast<const uint8_t*>(xv) + (size_t)m0o * rowb,
                        min(TM, M - m0o) * rowb);
  };
  int v = blockIdx.x, n0, m0;
  tile_origin(v, n0, m0);
  __amdgpu_buffer_rsrc_t ra = rsrc_w(n0), rb = rsrc_x(m0);
  // the next tile (the same one again after the last: its loads are then
  // valid and unused)
  int n0n = n0, m0n = m0;
  __amdgpu_buffer_rsrc_t ran = ra, rbn = rb;
  auto next_tile = [&]() {
    if (v + (int)gridDim.x < ntiles) {
      tile_origin(v + gridDim.x, n0n, m0n);
      ran = rsrc_w(n0n);
      rbn = rsrc_x(m0n);
    } else {
      n0n = n0; m0n = m0; ran = ra; rbn = rb;
    }
  };
  next_tile();

  // ---- staging: chunk c = tid + 512 i; the first TN*CPR chunks are W rows,
  // the rest x rows.  Step s of this tile, s >= nk reading step s - nk of the
  // next tile (so the last steps' loads bring the next tile's first steps).
  u32x4_t stg[NLD];
  // The staging addresses derive from tid_t, a copy of tid that each tile
  // makes opaque again, so that the compiler recomputes them per tile instead
  // of keeping them in registers through the epilogue.
  int tid_t = tid;
  // chunk i of a thread: W rows for i < 4, x rows after (TN * CPR = 4 * 512)
  static_assert(TN * CPR == 4 * 512, "staging split");
  auto load_one = [&](int s, int i) {
    const int cc = tid_t + 512 * (i & 3);
    const int row = cc / CPR, ch = cc % CPR;
    const bool nx = s >= nk;
    const int off = row * rowb + (nx ? s - nk : s) * KB + 16 * ch;
    stg[i] = __builtin_bit_cast(
        u32x4_t, i < 4 ? __builtin_amdgcn_raw_buffer_load_b128(nx ? ran : ra, off, 0, 0)
                       : __builtin_amdgcn_raw_buffer_load_b128(nx ? rbn : rb, off, 0, 0));
  };
  auto store_one = [&](int buf, int i) {
    const int cc = tid_t + 512 * (i & 3);
    const int row = cc / CPR, ch = cc % CPR;
    uint16_t* dst = i < 4 ? &a_lds[buf][row * ROW + 8 * ch] : &b_lds[buf][row * ROW + 8 * ch];
    *reinterpret_cast<u32x4_t*>(dst) = stg[i];
  };

  f32x16_t acc[4][2];
  // the epilogue inputs of the tile at (n0o, m0o): thread tid < TM loads a
  // token's positions, TM <= tid < TM + TN / 4 four bias words
  int4 ep_p = make_int4(0, 0, 0, 0);
  uint2 ep_b = make_uint2(0, 0);
  auto ep_load = [&](int n0o, int m0o) {
    if (tid < TM) {
      // rows past M take the last token's positions; they are not stored
      ep_p = *reinterpret_cast<const int4*>(pos + 4 * (min(m0o + tid, M - 1) % S));
    } else if (tid < TM + TN / 4) {
      const int n = n0o + 4 * (tid - TM);     // N is a multiple of 4
      ep_b = make_uint2(0, 0);
      if (bias != nullptr && n < N) ep_b = *reinterpret_cast<const uint2*>(bias + n);
    }
  };
  auto ep_store = [&](int eb) {
    if (tid < TM)
      *reinterpret_cast<f32x4_t*>(ep_pos[eb][tid]) =
          (f32x4_t){(float)ep_p.x, (float)ep_p.y, (float)ep_p.z, (float)ep_p.w};
    else if (tid < TM + TN / 4)
      *reinterpret_cast<f32x4_t*>(&ep_bias[eb][4 * (tid - TM)]) =
          (f32x4_t){bf16_lo(ep_b.x), bf16_hi(ep_b.x), bf16_lo(ep_b.y), bf16_hi(ep_b.y)};
  };
  ep_load(n0, m0);
  if (tid >= TM + TN / 4 && tid < TM + TN / 4 + 32) {
    const int i = tid - TM - TN / 4;
    ep_fr[i] = i < 16 ? fr.hi[i] : fr.lo[i - 16];
  }
#pragma unroll
  for (int i = 0; i < NLD; ++i) load_one(0, i);
  ep_store(0);
#pragma unroll
  for (int i = 0; i < NLD; ++i) store_one(0, i);
  if constexpr (!FP8) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) load_one(1, i);
  }
  __syncthreads();
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
  // The operands of sub-step ks+1 are read during the MFMAs of ks.  Loads
  // past the last step read in-range rows or the descriptors' zeros and are
  // never used.
  //
  // bf16: staging slot j of K step kt stores chunk j of step kt+1 (loaded a
  // step earlier) into the other buffer (last read before the previous
  // barrier) and reloads its registers with chunk j of step kt+2.  The slots
  // spread a step's loads and stores over it: issued together at the top,
  // the 64 KB of loads of all 8 waves fill the vector memory queue and hold
  // the waves at issue for 500-1000 cycles of a ~3,500-cycle step.
  //
  // fp8 (operands twice as wide: a register set held across the whole step
  // would spill): one load of step kt+1 after each MFMA of the first
  // sub-step, one store of it after each MFMA of the second.
  // gb: K steps of the earlier tiles; step kt of this tile uses LDS buffer
  // (gb + kt) & 1, which at the tile's start holds its first step.
  int gb = 0;
  for (int tile = 0;; ++tile) {
  const int eb = tile & 1;
  __asm__ volatile("" : "+v"(tid_t));
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = (f32x16_t){};
  KLEIN_QKV_CLOCK_START
  if constexpr (FP8) {
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = (gb + kt) & 1;
      read_ops(buf, 0, 0);
#pragma unroll
      for (int ks = 0; ks < KSUB; ++ks) {
        if (ks + 1 < KSUB) read_ops(buf, ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int nb = i >> 1, mb = i & 1;
          acc[nb][mb] = mfma(av[ks & 1][nb], bv[ks & 1][mb], acc[nb][mb]);
          static_assert(!FP8 || KSUB == 2, "one k-step of loads, one of stores");
          if (ks == 0) load_one(kt + 1, i);
          else store_one(buf ^ 1, i);
          __builtin_amdgcn_sched_barrier(0);
        }
        KLEIN_QKV_CLOCK_MARK(ks);
      }
      __syncthreads();
      KLEIN_QKV_CLOCK_MARK(4);
    }
  } else {
    // bf16: the 8 staging slots of step kt sit in its first three
    // sub-steps (3, 3, 2); the barrier comes before the last sub-step, whose
    // operands are already in registers, and the operands of the next
    // step's first sub-step are read while its MFMAs run
    static_assert(KSUB == 4 && NLD == 8, "slot layout");
    read_ops(gb & 1, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = (gb + kt) & 1;
#pragma unroll
      for (int ks = 0; ks < KSUB; ++ks) {
        if (ks == KSUB - 1) {
          __syncthreads();
          KLEIN_QKV_CLOCK_MARK(4);
          read_ops(buf ^ 1, 0, 0);
        } else {
          read_ops(buf, ks + 1, (ks + 1) & 1);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int nb = i >> 1, mb = i & 1;
          acc[nb][mb] = mfma(av[ks & 1][nb], bv[ks & 1][mb], acc[nb][mb]);
          // slots after MFMAs 0, 3, 6 of sub-steps 0 and 1, 0 and 4 of sub-step 2
          const bool slot = ks < 2 ? (i % 3 == 0) : (ks == 2 && i % 4 == 0);
          if (slot) {
            const int j = ks < 2 ? 3 * ks + i / 3 : 6 + i / 4;
            store_one(buf ^ 1, j);
            load_one(kt + 2, j);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        KLEIN_QKV_CLOCK_MARK(ks);
      }
    }
  }

  // ---- epilogue: lane column = token m0 + tl, tl = 64 wm + 32 mb + lr;
  // registers 4c..4c+3 = features n0 + 128 wn + 32 nb + 8 c + 4 g + 0..3.
  // H D is a multiple of 64, so a 32-feature block nb lies in one of q, k, v
  // and in one head: the output, the head offset and the RoPE axis are
  // wave-uniform per block, and only the pair index follows the lane half g.
  // Stores go through a descriptor over the tile's rows of the output, which
  // drops rows past M: the row is always part of the lane offset (the range
  // check may leave the scalar offset out), the scalar offset only moves
  // within a row.  (readfirstlane: the compiler cannot see that wn is
  // wave-uniform.)
  ep_load(n0n, m0n);     // the next tile's epilogue inputs, stored after this epilogue
  int lane_e = lane;
  __asm__ volatile("" : "+v"(lane_e));
  {
  // the epilogue's lane indices from an opaque copy, so that its addresses
  // are formed here rather than kept in registers through the K loop
  const int lane = lane_e, g = lane_e >> 5, lr = lane_e & 31;
  const int nrows_b = min(TM, M - m0);
  const int nw = __builtin_amdgcn_readfirstlane(n0 + 128 * wn);
  // frequencies of the pairs jb + 2 g + 0..1, jb = (8 c4 mod D/4) / 2
  f32x2_t fhi[4], flo[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) {
    const int jb = (8 * c4 % DA) / 2;
    fhi[c4] = *reinterpret_cast<const f32x2_t*>(&ep_fr[jb + 2 * g]);
    flo[c4] = *reinterpret_cast<const f32x2_t*>(&ep_fr[16 + jb + 2 * g]);
  }
  // the 4 outputs of (nb, c4, mb), rounded: bias, then the rotation for q
  // and k (channel db + 8 c4 + 4 g + 0..3 of a head, db the block's first)
  // (`rot` is a compile-time flag, so that the caller's loops over the
  // outputs hold no branch and their LDS reads can be issued together)
  auto emit = [&](int nb, int c4, int mb, auto rot, int db) -> u32x2_t {
    const f32x4_t bs = *reinterpret_cast<const f32x4_t*>(&ep_bias[eb][128 * wn + 32 * nb + 8 * c4 + 4 * g]);
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = acc[nb][mb][4 * c4 + e] * yscale + bs[e];
    if constexpr (!decltype(rot)::value) {
      return (u32x2_t){pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    } else {
      // one axis a for both lane halves (D/4 divides 32)
      const float fp = ep_pos[eb][64 * wm + 32 * mb + lr][(db + 8 * c4) / DA];
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const float rev = rope_rev(fp, fhi[c4][pr], flo[c4][pr]);
        const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
        const f32x2_t r = rope_rot(y[2 * pr], y[2 * pr + 1], cs, sn);
        y[2 * pr] = r[0];
        y[2 * pr + 1] = r[1];
      }
      return (u32x2_t){pack_f16x2(y[0], y[1]), pack_f16x2(y[2], y[3])};
    }
  };
  if (HD % 128 == 0) {
    // The wave's 128 features are one contiguous segment of one output's
    // rows.  Each 32-token half goes through the wave's own slice of the LDS
    // buffer the last K step no longer reads (32 rows of 256 bytes, padded
    // to 272), and leaves in 8-byte stores of which 16 lanes cover one
    // 128-byte half of a row: each store writes 4 whole cache lines instead
    // of 16-byte pieces of 32 rows.  Within one wave, LDS accesses take
    // effect in program order.  (Not 16-byte stores: the compiler then reused
    // a store's first data register in the very next instruction, and on
    // this GPU some lanes stored the new value.)
    if (nw < N) {
      const int which = nw / HD, hdw = nw - which * HD;
      const uint16_t* const obase = which == 0 ? qo : which == 1 ? ko : vo;
      const __amdgpu_buffer_rsrc_t ro = uniform_rsrc(obase + (size_t)m0 * HD, nrows_b * HD * 2);
      constexpr int XR = 136;                    // LDS row stride, 16-bit units
      const int lbuf = (gb + nk - 1) & 1;
      uint16_t* const xl = (wave < 4 ? a_lds[lbuf] : b_lds[lbuf]) + (wave & 3) * (32 * XR);
      static_assert(4 * 32 * XR <= TN * ROW, "transpose slices");
      const int rr = lane >> 4, cc = lane & 15;  // row 4 i + rr, 8-byte chunk cc of a half
      // one straight-line copy of the output loop for q and k (rotated), one for v
      auto out_half = [&](int mb, auto rot) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const u32x2_t o = emit(nb, c4, mb, rot, (hdw + 32 * nb) % D);
            *reinterpret_cast<u32x2_t*>(xl + lr * XR + 32 * nb + 8 * c4 + 4 * g) = o;
          }
      };
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (which < 2)
          out_half(mb, std::true_type{});
        else
          out_half(mb, std::false_type{});
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x2_t part =
                *reinterpret_cast<const u32x2_t*>(xl + (4 * i + rr) * XR + 64 * h + 4 * cc);
            // the row in the lane offset, which the descriptor's range check
            // sees; the column (inside the row) in the scalar offset
            const int vo = ((64 * wm + 32 * mb + 4 * i + rr) * HD + 64 * h + 4 * cc) * 2;
            __builtin_amdgcn_raw_buffer_store_b64(part, ro, vo, hdw * 2, 0);
          }
      }
    }
  } else {
    int voff[2];                                // byte offset of (token, 4 g)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) voff[mb] = ((64 * wm + 32 * mb + lr) * HD + 4 * g) * 2;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int nbase = nw + 32 * nb;
      if (nbase >= N) continue;
      const int which = nbase / HD, hdb = nbase - which * HD;
      const uint16_t* const obase = which == 0 ? qo : which == 1 ? ko : vo;
      const __amdgpu_buffer_rsrc_t ro = uniform_rsrc(obase + (size_t)m0 * HD, nrows_b * HD * 2);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          __builtin_amdgcn_raw_buffer_store_b64(
              which < 2 ? emit(nb, c4, mb, std::true_type{}, hdb % D)
                        : emit(nb, c4, mb, std::false_type{}, hdb % D),
              ro, voff[mb], (hdb + 8 * c4) * 2, 0);
    }
  }
  }
  KLEIN_QKV_CLOCK_TILE_END(nk);
  v += gridDim.x;
  if (v >= ntiles) break;
  ep_store(eb ^ 1);
  gb += nk;
  n0 = n0n; m0 = m0n; ra = ran; rb = rbn;
  next_tile();
  // this epilogue's LDS reads (its slices of buffer (gb - 1) & 1, the inputs
  // copy eb) end before the next tile stores into them
  __syncthreads();
  }
  KLEIN_QKV_CLOCK_STORE
}

template <bool FP8>
static hipError_t launch_qkv(const QkvArgs& a) {
  const int M = a.B * a.S, N = 3 * a.H * a.D;
  const int ntn = (N + 255) / 256, ntm = (M + 255) / 256;
  // persistent: one workgroup per compute unit (it needs most of a CU's LDS),
  // a multiple of 8 so that each keeps to one XCD's share of the tile list
  const long long ntiles = (long long)ntn * ntm;
  long long nwg = a.ncu > 0 ? a.ncu : ntiles;
  if (nwg >= 8) nwg -= nwg % 8;
  if (nwg > ntiles) nwg = ntiles;
  const dim3 grid((unsigned)nwg);
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
