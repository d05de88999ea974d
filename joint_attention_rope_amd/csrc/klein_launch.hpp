// Host-side launch descriptors shared by the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "klein_device.hpp"

namespace klein {

struct LaunchArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* pos;
  void* out;
  int B, S, H, D;
  float qscale_log2;   // log2(e) / sqrt(D), folded into Q after the rotation
  float descale[3];    // fp8 per-tensor descales of q, k, v (1 for bf16)
  RopeFreqs freqs;
  hipStream_t stream;
  // block-sparse mask [B][H][ceil(S/256)][ceil(S/64)] (nonzero = compute), or
  // null for dense attention
  const uint8_t* bmask = nullptr;
  // split-KV schedule (n_sk > 0) over the caller's workspace, or none
  SplitArgs split{};
  // bf16 dense/split paths: also write the softmax log-sum-exp, fp32
  // [B][H][S], natural log (null: not written)
  float* lse = nullptr;
  // bf16 dense/split paths: workspace for k rotated once (fp16 [B][S][H][D])
  // before the attention kernel, or null (rotate every K tile in the kernel)
  void* krot = nullptr;
  // bf16 dense/split paths with krot: workspace for v regrouped into
  // key-major 64-key tiles (v_tiles_bytes), or null (the kernel reads the
  // V^T operands transposed out of row-major V tiles)
  void* vt = nullptr;
};

// where the attention kernels rotate (see attn_fwd_bf16.hip)
constexpr int kRotInKernel = 0;
constexpr int kRotKPre = 1;
constexpr int kRotBothPre = 2;

// y = fp16(R(pos) x * scale) for bf16 x [B][S][H][D] (the kernels' rotation routine)
hipError_t launch_rope4d_fp16(const void* x, const int32_t* pos, void* y, int B, int S, int H,
                              int D, const RopeFreqs& fr, float scale, hipStream_t stream);

// v [B][S][H][D] bf16 -> per (b, h) and 64-key tile, D rows of 64 keys
// (zero past S), for the bf16 attention kernel's V^T operands
long long v_tiles_bytes(int B, int S, int H, int D);
hipError_t launch_v_tiles(const void* v, void* vt, int B, int S, int H, int D,
                          hipStream_t stream);

// Split-KV cut of a dense call for a GPU of n_cu compute units (n_sk == 0:
// whole items only, no workspace).  The workspace holds the partial slots.
struct SplitPlan {
  int n_dp, n_sk, n_rem, n_chunk;
  long long bytes;
};
SplitPlan plan_split(int B, int S, int H, int D, int n_cu);
// merges the split items' slots into their output rows (after the attention
// kernel, on the same stream); o_scale multiplies O / l (v's descale for fp8)
hipError_t launch_split_merge(const LaunchArgs& a, float o_scale, float* lse);

hipError_t launch_attn_fwd_bf16(const LaunchArgs& a);
hipError_t launch_attn_fwd_prerotated(const LaunchArgs& a);
long long attn_fwd_bf16_grid(int B, int S, int H);
hipError_t launch_attn_fwd_fp8(const LaunchArgs& a);
long long attn_fwd_fp8_grid(int B, int S, int H);
hipError_t launch_rope4d_apply(const LaunchArgs& a);

// Attention backward (bf16): q, k, v, out, dout [B][S][H][D] bf16, lse fp32
// [B][H][S] (natural log) -> dq, dk, dv bf16; qr, kr (fp16 [B][S][H][D]),
// delta (fp32 [B][H][S]), the squared row norms of dout and v (fp32
// [2][B][H][S]) and the per-head exponent of the ds scale (fp32 [B][H]) in
// the caller's workspace.
struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;
  const uint16_t* dout;
  const int32_t* pos;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* qr;
  uint16_t* kr;
  float* delta;
  float* norm2;
  float* escale;
  int B, S, H, D;
  float qscale_log2;
  RopeFreqs freqs;
  hipStream_t stream;
  // a second stream for the dq kernel, forked from and joined back into
  // `stream` with these two events (all null: everything on `stream`)
  hipStream_t side;
  hipEvent_t fork, join;
};
hipError_t launch_attn_bwd(const BwdArgs& a);
// byte offsets of the backward's workspace parts (qr at 0) and its size
struct BwdWorkspace {
  long long kr, delta, norm2, escale, total;
};
BwdWorkspace attn_bwd_workspace(int B, int S, int H, int D);

// Scratch of the no-allocation entry point (noalloc.hip): the device address,
// on the current GPU, of a static array of kNoallocScratchBytes, looked up
// once per GPU.  Calls that use it at the same time on one GPU race.
constexpr long long kNoallocScratchBytes = 320LL << 20;
hipError_t noalloc_scratch(void** ptr);

// QKV projection with the RoPE-4D epilogue: x [B S][C] bf16, w [3 H D][C]
// bf16 (or both E4M3 codes with descales, fp8), bias [3 H D] bf16 or null
// -> q', k' fp16 and v bf16, [B][S][H][D].
struct QkvArgs {
  const void* x;
  const void* w;
  bool fp8;
  float x_descale, w_descale;
  const uint16_t* bias;
  const int32_t* pos;
  uint16_t* q;
  uint16_t* k;
  uint16_t* v;
  int B, S, C, H, D;
  RopeFreqs freqs;
  int ncu;                 // compute units of the device (the persistent grid)
  hipStream_t stream;
};
hipError_t launch_qkv_rope_proj(const QkvArgs& a);
long long qkv_rope_proj_grid(int B, int S, int H, int D);

}  // namespace klein
