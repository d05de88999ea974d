// Device-side building blocks shared by the gfx950 kernels of this library:
// vector types, bf16 packing, the RoPE-4D chunk rotation and the XCD-aware
// workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace klein {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// RoPE-4D frequencies in revolutions per unit of position, w_j = omega_j/(2 pi),
// omega_j = 10000^(-2j/(D/4)), j < D/8.  Each w_j is split as hi + lo with hi
// holding at most 12 significant bits, so pos * hi is exact in fp32 for
// |pos| < 4096 and its fractional part loses nothing; lo carries the rest.
struct RopeFreqs {
  float hi[16];
  float lo[16];
};

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.44269504088896341f;

// Fourth word of a raw buffer descriptor on gfx9-family GPUs (32-bit data
// format, no swizzle): loads past the descriptor's size return zero.
constexpr int kBufferWord3 = 0x00020000;

// Raw buffer descriptor over [base, base + bytes).  Every operand is forced
// into scalar registers (all callers pass wave-uniform values), so loads
// through it never need a per-lane descriptor loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), 0, n, kBufferWord3);
}

// bf16 halves of a packed word (element 2j in the low half: little endian)
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// two floats -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// two floats -> packed f16x2, round to nearest even
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2_t r = __builtin_convertvector((f32x2_t){a, b}, f16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// Angle of RoPE pair j at integer position p, in revolutions (v_sin_f32 and
// v_cos_f32 take revolutions): fract(p * hi) + p * lo, one explicit fma, so
// that every kernel forms bit-identical angles whatever the compiler contracts.
__device__ __forceinline__ float rope_rev(float fp, float whi, float wlo) {
  return __builtin_fmaf(fp, wlo, __builtin_amdgcn_fractf(fp * whi));
}

// One pair (x, y) -> (x c - y s, x s + y c), with explicit fmas (same bits in
// every kernel that rotates).
__device__ __forceinline__ f32x2_t rope_rot(float x, float y, float c, float s) {
  return (f32x2_t){__builtin_fmaf(x, c, -(y * s)), __builtin_fmaf(x, s, y * c)};
}

// Rotate one 16-byte chunk of bf16: 8 consecutive channels = 4 interleaved
// pairs of a single axis block, pairs j0 .. j0+3, at integer position p on
// that axis.  Each pair (x, y) -> (x cos - y sin, x sin + y cos), then
// * scale, rounded to bf16 (F16 = false) or to fp16 (F16 = true).
// v_sin_f32 / v_cos_f32 take their argument in revolutions.
template <bool F16 = false>
__device__ __forceinline__ u32x4_t rope_chunk(u32x4_t x, int p, const float* whi,
                                              const float* wlo, float scale) {
  const float fp = (float)p;
  u32x4_t y;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float rev = rope_rev(fp, whi[jj], wlo[jj]);
    const float s = __builtin_amdgcn_sinf(rev);
    const float c = __builtin_amdgcn_cosf(rev);
    const f32x2_t r = rope_rot(bf16_lo(x[jj]), bf16_hi(x[jj]), c, s);
    const float u = r[0] * scale, w = r[1] * scale;
    y[jj] = F16 ? pack_f16x2(u, w) : pack_bf16x2(u, w);
  }
  return y;
}

// LDS row of element kk (0..31) of a 32-row block such that, after a 32x32
// MFMA whose A operand rows are read in LDS row order, accumulator register i
// of lane half g holds element 16g + i: the MFMA output row r holds element
// 16*((r/4)&1) + 4*(r/8) + (r%4), and this is the inverse map.
__device__ __forceinline__ int key_to_row(int kk) {
  const int g = kk >> 4, i = kk & 15;
  return ((i >> 2) << 3) + (g << 2) + (i & 3);
}

// Workgroups are handed to the 8 XCDs round robin (block i -> XCD i % 8), and
// each XCD has its own L2.  Remap so that XCD x runs a contiguous range of the
// logical work list; consecutive logical items share a (batch, head) and so
// stream the same K/V through that XCD's L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = n >> 3, extra = n & 7;
  return xcd * per + (xcd < extra ? xcd : extra) + slot;
}

// Block-sparse attention: the kept key tiles of one query tile, listed in
// ascending order by one wave (ballot + mbcnt compaction, so the order and
// the result are deterministic).  kSparsePad sentinel entries (tile index
// nkt, whose rows lie past S and read as zeros) follow the list, so a
// pipeline that prefetches a few tiles ahead needs no bounds checks.
constexpr int kSparseMaxTiles = 4096;
constexpr int kSparsePad = 8;

__device__ __forceinline__ int build_kept_list(const uint8_t* mrow, int nkt, uint16_t* list,
                                               int lane) {
  int n = 0;
  for (int c = 0; c < nkt; c += 64) {
    const int kt = c + lane;
    const bool keep = kt < nkt && mrow[kt] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
    if (keep) {
      const int r = (int)__builtin_amdgcn_mbcnt_hi(
          (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      list[n + r] = (uint16_t)kt;
    }
    n += __builtin_popcountll(bal);
  }
  if (lane < kSparsePad) list[n + lane] = (uint16_t)nkt;
  return n;
}

// Split-KV schedule of the attention kernels (split variant).  The work list
// holds B*H*ceil(S/256) items (one query tile each, all key tiles).  The
// first n_dp items (whole rounds of the GPU) run one per workgroup.  Each of
// the n_rem items that would fill only part of a last round is cut into
// n_chunk chunks of key tiles at the same boundaries for every item, one
// workgroup per (chunk, item); consecutive workgroups take the same chunk of
// consecutive items, so the workgroups of one XCD stream the same keys and
// values through its L2, as in the dense schedule.  A chunk stores its
// unnormalised O, running max m and row sum l in the workspace slot
// chunk * n_rem + item, and a second kernel on the same stream merges each
// item's slots in chunk order into the output rows (the kernel boundary
// orders the stores before the loads; the merge order is fixed, so the
// result is deterministic).
struct SplitArgs {
  float* part;     // n_chunk * n_rem slots of split_slot_floats(D) floats
  int n_dp;        // items run whole, by workgroups [0, n_dp)
  int n_sk;        // split workgroups, [n_dp, n_dp + n_sk): n_chunk * n_rem
  int n_rem;       // items split
  int n_chunk;     // chunks per split item
};

// slot of a 256-query tile: O as [wave][32-row block][4][lane] float4 (the
// accumulator registers of each lane, in order), then (m, l) as [wave][lane]
// float2
__host__ __device__ constexpr long long split_slot_floats(int D) { return 256LL * D + 1024; }

// first key tile of chunk c of nkt tiles cut into n (c = n gives nkt)
__host__ __device__ inline int split_chunk_begin(int c, int nkt, int n) {
  return (int)((long long)c * nkt / n);
}

// Store this workgroup's partial (o, m, l: l already summed over the lane
// pair) of chunk `chunk` of split item r.
template <int MB>
__device__ __forceinline__ void split_store(const f32x16_t* o, float m, float l,
                                            const SplitArgs& sp, int r, int chunk) {
  constexpr int D = 32 * MB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* my = sp.part + (size_t)(chunk * sp.n_rem + r) * split_slot_floats(D);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      *reinterpret_cast<f32x4_t*>(my + 4 * (((wave * MB + mb) * 4 + i4) * 64 + lane)) =
          (f32x4_t){o[mb][4 * i4], o[mb][4 * i4 + 1], o[mb][4 * i4 + 2], o[mb][4 * i4 + 3]};
  *reinterpret_cast<f32x2_t*>(my + 256 * D + 2 * (wave * 64 + lane)) = (f32x2_t){m, l};
}

// Reduce a per-lane value with the lane 32 apart (lanes l and l^32 hold the
// two halves of one query's keys in the 32x32 MFMA accumulator layout).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace klein
