// Split-KV schedule of the attention kernels: how a work list that does not
// fill whole rounds of the GPU is cut, the workspace it needs, and the kernel
// that merges the chunks' partial results into the output rows.
#include "klein_launch.hpp"

namespace klein {

// A chunk keeps at least this many 64-key tiles; below 32 key tiles
// (S < 2048) a call is short enough that whole items are kept.
constexpr int kSplitMinChunk = 8;
constexpr int kSplitMinKeyTiles = 32;
// Fixed cost of one workgroup (table, Q tile, pipeline fill, partial store,
// its share of the merge), in units of one 64-key tile step, for choosing the
// chunk count (fitted to timings on MI355X).
constexpr int kSplitOverheadSteps = 6;
// A last round that runs whole items on only part of the GPU runs each of them
// faster (the chip is power-limited, and its clock rises when fewer compute
// units are busy), so a split must promise at least this gain.
constexpr double kSplitMinGain = 0.85;
// The split workgroups never exceed this many rounds' worth of the GPU, which
// bounds the workspace.
constexpr int kSplitMaxRounds = 4;

SplitPlan plan_split(int B, int S, int H, int D, int n_cu) {
  SplitPlan p{};
  const long long nqt = (S + 255) / 256, nkt = (S + 63) / 64;
  const long long items = (long long)B * H * nqt;
  if (n_cu < 1 || nkt < kSplitMinKeyTiles) return p;
  const long long rem = items % n_cu;
  if (rem == 0) return p;
  // cost of the tail in tile steps: whole items (c = 1) take nkt; c chunks per
  // item take ceil(c rem / n_cu) rounds of nkt / c steps plus the overhead
  double best = (double)nkt;
  long long best_c = 1;
  for (long long c = 2; c * kSplitMinChunk <= nkt && c * rem <= (long long)kSplitMaxRounds * n_cu;
       ++c) {
    const long long rounds = (c * rem + n_cu - 1) / n_cu;
    const double cost = (double)rounds * ((double)nkt / c + kSplitOverheadSteps);
    if (cost < best) { best = cost; best_c = c; }
  }
  if (best_c == 1 || best > kSplitMinGain * (double)nkt) return p;
  p.n_dp = (int)(items - rem);
  p.n_rem = (int)rem;
  p.n_chunk = (int)best_c;
  p.n_sk = (int)(best_c * rem);
  p.bytes = (long long)p.n_sk * split_slot_floats(D) * 4;
  return p;
}

// One workgroup of 256 threads per (split item, 32-query slice = one wave of
// the attention workgroup).  The slice's O entries in a slot are the MB * 4
// float4 accumulator quads of each of its 64 lanes; entry e = 256 i + tid is
// quad (mb, i4) = (e / 256, (e / 64) % 4) of lane e % 64, i.e. query row
// 32 slice + lane % 32, channels 32 mb + 8 i4 + 4 (lane / 32) + [0, 4).
// out = (sum_c 2^(m_c - M) O_c) * o_scale / (sum_c 2^(m_c - M) l_c), chunks
// in order, M = max_c m_c: the merge of softmax partials taken relative to
// different running maxima.
template <int D>
__global__ __launch_bounds__(256) void split_merge_kernel(const float* __restrict__ part,
                                                          uint16_t* __restrict__ out, int S, int H,
                                                          int nqt, SplitArgs sp, float o_scale,
                                                          float* __restrict__ lse) {
  constexpr int MB = D / 32;
  constexpr long long SLOT = split_slot_floats(D);
  const int tid = threadIdx.x;
  const int r = blockIdx.x >> 3, w = blockIdx.x & 7;
  const int item = sp.n_dp + r;
  const int qt = item % nqt, bh = item / nqt, h = bh % H, b = bh / H;
  const size_t rs = (size_t)H * D;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int e = 256 * i + tid;
    const int lane = e & 63, i4 = (e >> 6) & 3, mb = e >> 8;
    const int row = qt * 256 + 32 * w + (lane & 31);
    const int d = 32 * mb + 8 * i4 + 4 * (lane >> 5);
    const long long o_off = 4LL * (w * MB * 256 + e);
    const long long ml_off = 256LL * D + 2 * (w * 64 + lane);
    float M = kNegInf;
    for (int c = 0; c < sp.n_chunk; ++c)
      M = __builtin_fmaxf(M, part[(size_t)(c * sp.n_rem + r) * SLOT + ml_off]);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    for (int c = 0; c < sp.n_chunk; ++c) {
      const float* s = part + (size_t)(c * sp.n_rem + r) * SLOT;
      const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(s + ml_off);
      const float f = __builtin_amdgcn_exp2f(ml[0] - M);
      L += f * ml[1];
      acc += f * *reinterpret_cast<const f32x4_t*>(s + o_off);
    }
    if (row < S) {
      const float inv = o_scale / L;
      // the log-sum-exp of the row (natural log), once per row (mb = i4 = 0, first lane half)
      if (lse != nullptr && e < 32) lse[((size_t)b * H + h) * S + row] = (M + __builtin_amdgcn_logf(L)) * kLn2;
      uint2 v;
      v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
      *reinterpret_cast<uint2*>(out + (size_t)b * S * rs + (size_t)h * D + (size_t)row * rs + d) = v;
    }
  }
}

hipError_t launch_split_merge(const LaunchArgs& a, float o_scale, float* lse) {
  const int nqt = (a.S + 255) / 256;
  const dim3 grid((unsigned)a.split.n_rem * 8);
  if (a.D == 128)
    hipLaunchKernelGGL(split_merge_kernel<128>, grid, dim3(256), 0, a.stream, a.split.part,
                       (uint16_t*)a.out, a.S, a.H, nqt, a.split, o_scale, lse);
  else
    hipLaunchKernelGGL(split_merge_kernel<64>, grid, dim3(256), 0, a.stream, a.split.part,
                       (uint16_t*)a.out, a.S, a.H, nqt, a.split, o_scale, lse);
  return hipGetLastError();
}

}  // namespace klein
