// C ABI of the RoPE-4D joint-attention library: argument checks, RoPE
// frequency tables, kernel dispatch, status mapping.  Declarations and the
// contract of every entry point live in include/klein_attn.h.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/klein_attn.h"
#include "klein_launch.hpp"

namespace {

using klein::LaunchArgs;

constexpr double kTheta = 10000.0;
constexpr double kPi = 3.14159265358979323846;

// w_j = theta^(-2j/(D/4)) / (2 pi) revolutions per position unit, split into a
// 12-significant-bit head and an fp32 tail (see RopeFreqs).
klein::RopeFreqs make_freqs(int D) {
  klein::RopeFreqs f{};
  const int da = D / 4;
  for (int j = 0; j < 16; ++j) {
    if (j >= da / 2) { f.hi[j] = 0.f; f.lo[j] = 0.f; continue; }
    const double w = std::pow(kTheta, -2.0 * j / da) / (2.0 * kPi);
    int e = 0;
    const double m = std::frexp(w, &e);                 // w = m * 2^e, m in [0.5, 1)
    const double hi = std::ldexp(std::nearbyint(std::ldexp(m, 12)), e - 12);
    f.hi[j] = (float)hi;                                 // exact: <= 12 bits
    f.lo[j] = (float)(w - hi);
  }
  return f;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The kernels form byte offsets within a tile's rows in 32-bit integers (up
// to 256 rows of H D 16-bit elements), so H D stays below 2^22, and index
// pos_thwl as 4 s + axis in 32 bits, so S stays below 2^29.
constexpr long long kMaxHeadWidth = (1LL << 22) - 1;
constexpr long long kMaxTokens = (1LL << 29) - 1;
bool shape_ok(int S, int H, int D) {
  return (long long)H * D <= kMaxHeadWidth && (long long)S <= kMaxTokens;
}

klein_status_t check_common(const void* q, const void* k, const void* v, const int32_t* pos,
                            const void* out, int B, int S, int H, int D) {
  if (!q || !k || !v || !pos || !out) return KLEIN_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || H < 1) return KLEIN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return KLEIN_ERR_UNSUPPORTED;
  if (!shape_ok(S, H, D)) return KLEIN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(pos))
    return KLEIN_ERR_INVALID_ARG;
  return KLEIN_OK;
}

klein_status_t map_hip(hipError_t e) {
  if (e == hipSuccess) return KLEIN_OK;
  if (e == hipErrorNoDevice || e == hipErrorInvalidDevice) return KLEIN_ERR_NO_DEVICE;
  if (e == hipErrorNotSupported) return KLEIN_ERR_UNSUPPORTED;
  return KLEIN_ERR_LAUNCH;
}

LaunchArgs make_args(const void* q, const void* k, const void* v, const int32_t* pos, void* out,
                     int B, int S, int H, int D, klein_stream_t stream) {
  LaunchArgs a{};
  a.q = q; a.k = k; a.v = v; a.pos = pos; a.out = out;
  a.B = B; a.S = S; a.H = H; a.D = D;
  a.qscale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  a.descale[0] = a.descale[1] = a.descale[2] = 1.0f;
  a.freqs = make_freqs(D);
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return a;
}

constexpr long long kMaxGrid = 2147483647LL;

// Sequences from which the bf16 workspace schedule also regroups v into
// key-major tiles.  The pass costs a read and a write of V per call; the
// kernel saves LDS time per key tile and query tile, so the gain grows with S.
// Measured (same process, MI355X): +1.9 % at S = 16,896 (B = 2, H = 24),
// -1.3 % at S = 8,704 and -1.7 % at S = 4,608 (B = 1, H = 24).
constexpr int kVTilesMinS = 12288;

// Workspace of klein_rope4d_attn_fwd_ws: k rotated once (fp16 for bf16
// inputs, e4m3 codes for fp8, [B][S][H][D]), for bf16 with `vt` and S of at
// least kVTilesMinS v in key-major tiles (klein::v_tiles_bytes), and the
// split-KV partials.
struct WsLayout {
  long long krot_bytes;
  long long vt_bytes;         // at offset krot_bytes
  klein::SplitPlan plan;      // partials at offset krot_bytes + vt_bytes
  long long total;
};
WsLayout ws_layout(int B, int S, int H, int D, klein_dtype_t dtype, int ncu, bool vt = true) {
  WsLayout w{};
  const int elem = dtype == KLEIN_DTYPE_BF16 ? 2 : 1;      // fp16 or e4m3 rotated keys
  w.krot_bytes = ((long long)B * S * H * D * elem + 255) / 256 * 256;
  w.vt_bytes = vt && dtype == KLEIN_DTYPE_BF16 && S >= kVTilesMinS
                   ? klein::v_tiles_bytes(B, S, H, D) : 0;
  w.plan = klein::plan_split(B, S, H, D, ncu);
  w.total = w.krot_bytes + w.vt_bytes + w.plan.bytes;
  return w;
}

// Compute units of the current device, cached per device (the split-KV plan
// depends on them).  0 on error, with the HIP error in *err.
int current_cu_count(hipError_t* err) {
  static std::atomic<int> cache[64];
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  *err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (*err != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// The checks of the split-KV entry points that need no device.
klein_status_t check_ws_call(const void* q, const void* k, const void* v,
                             const int32_t* pos_thwl, const void* out, int B, int S, int H,
                             int D, klein_dtype_t dtype, float q_descale, float k_descale,
                             float v_descale) {
  if (dtype != KLEIN_DTYPE_BF16 && dtype != KLEIN_DTYPE_FP8_E4M3) return KLEIN_ERR_INVALID_ARG;
  klein_status_t st = check_common(q, k, v, pos_thwl, out, B, S, H, D);
  if (st != KLEIN_OK) return st;
  if (dtype == KLEIN_DTYPE_FP8_E4M3)
    for (float s : {q_descale, k_descale, v_descale})
      if (!(std::isfinite(s) && s > 0.f)) return KLEIN_ERR_INVALID_ARG;
  if (klein::attn_fwd_bf16_grid(B, S, H) > kMaxGrid) return KLEIN_ERR_UNSUPPORTED;
  return KLEIN_OK;
}

klein_status_t attn_ws(const void* q, const void* k, const void* v,
                       const int32_t* pos_thwl, void* out, float* lse, int B, int S, int H,
                       int D, klein_dtype_t dtype, float q_descale, float k_descale,
                       float v_descale, void* workspace, size_t workspace_bytes,
                       klein_stream_t stream, bool vt = true) {
  klein_status_t st = check_ws_call(q, k, v, pos_thwl, out, B, S, H, D, dtype, q_descale,
                                    k_descale, v_descale);
  if (st != KLEIN_OK) return st;
  const bool fp8 = dtype == KLEIN_DTYPE_FP8_E4M3;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return KLEIN_ERR_INVALID_ARG;
  try {
    hipError_t e;
    const int ncu = current_cu_count(&e);
    if (e != hipSuccess) return map_hip(e);
    const WsLayout w = ws_layout(B, S, H, D, dtype, ncu, vt);
    const klein::SplitPlan& plan = w.plan;
    if (w.total > 0 && (!workspace || workspace_bytes < (size_t)w.total))
      return KLEIN_ERR_INVALID_ARG;
    LaunchArgs a = make_args(q, k, v, pos_thwl, out, B, S, H, D, stream);
    a.lse = lse;
    if (w.krot_bytes > 0) a.krot = workspace;
    if (w.vt_bytes > 0) a.vt = static_cast<char*>(workspace) + w.krot_bytes;
    if (plan.n_sk > 0) {
      a.split.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.krot_bytes +
                                              w.vt_bytes);
      a.split.n_dp = plan.n_dp;
      a.split.n_sk = plan.n_sk;
      a.split.n_rem = plan.n_rem;
      a.split.n_chunk = plan.n_chunk;
    }
    if (!fp8) return map_hip(klein::launch_attn_fwd_bf16(a));
    a.descale[0] = q_descale; a.descale[1] = k_descale; a.descale[2] = v_descale;
    return map_hip(klein::launch_attn_fwd_fp8(a));
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

// The buffer klein_rope4d_attn_fwd and klein_rope4d_attn_fwd_fp8 keep per
// device for the split-KV schedule (rotated keys, then the split partials).
// It is created on the first call that needs it and replaced by a larger one
// when a call needs more, never beyond the limit.  Every call that uses it
// holds the device's mutex from the look-up to the last launch, makes its
// stream wait for `done` (the event recorded after the previous user's
// kernels, on whatever stream they ran) and records `done` again, so uses
// of the buffer are ordered across streams and threads; a replaced buffer is
// freed only once `done` has completed.
constexpr int kMaxDevices = 64;
constexpr size_t kBufferGrain = size_t(32) << 20;

struct DeviceBuffer {
  std::mutex mu;
  void* ptr = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;
  bool used = false;          // `done` has been recorded
};
DeviceBuffer g_buffers[kMaxDevices];

// Per device, the backward's second stream (non-blocking, default priority)
// and its fork/join events, created on first use and kept until the process
// ends.  The lock covers one call's records and waits.
struct BwdSide {
  std::mutex mu;
  bool tried = false;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
BwdSide g_bwd_side[kMaxDevices];

// Creates the device's side stream and events once; on failure the backward
// runs on the caller's stream alone (same kernels, one after the other).
void bwd_side_init(BwdSide& s) {
  if (s.tried) return;
  s.tried = true;
  if (hipStreamCreateWithFlags(&s.side, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    s.side = nullptr;
    s.fork = s.join = nullptr;
  }
}
std::atomic<size_t> g_buffer_limit{KLEIN_DEFAULT_BUFFER_LIMIT};

// Frees b's buffer after its last use has completed.  Caller holds b.mu and
// has b's device current.
hipError_t release_buffer(DeviceBuffer& b) {
  if (!b.ptr) return hipSuccess;
  hipError_t e = b.used ? hipEventSynchronize(b.done) : hipSuccess;
  if (e != hipSuccess) return e;
  e = hipFree(b.ptr);
  b.ptr = nullptr;
  b.bytes = 0;
  return e;
}

// The split-KV call on the device's buffer.  *ran is false (and nothing is
// launched) when the call should run the kernels that need no memory: the
// stream is being captured into a graph (a graph must not hold the address of
// a buffer that a later call may free), the shape needs more than the limit,
// or the allocation failed for lack of memory.
klein_status_t attn_on_buffer(const void* q, const void* k, const void* v, const int32_t* pos,
                              void* out, int B, int S, int H, int D, klein_dtype_t dtype,
                              float q_descale, float k_descale, float v_descale,
                              klein_stream_t stream, bool* ran) {
  *ran = false;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(hs, &cap);
  if (e != hipSuccess) return map_hip(e);
  if (cap != hipStreamCaptureStatusNone) return KLEIN_OK;
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return map_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return KLEIN_OK;
  const int ncu = current_cu_count(&e);
  if (e != hipSuccess) return map_hip(e);
  const size_t need = (size_t)ws_layout(B, S, H, D, dtype, ncu).total;
  const size_t limit = g_buffer_limit.load();
  if (need > limit) return KLEIN_OK;
  DeviceBuffer& b = g_buffers[dev];
  std::lock_guard<std::mutex> lock(b.mu);
  if (b.bytes < need) {
    e = release_buffer(b);
    if (e != hipSuccess) return map_hip(e);
    const size_t want = std::max(need, std::min((need + kBufferGrain - 1) / kBufferGrain *
                                                 kBufferGrain, limit));
    e = hipMalloc(&b.ptr, want);
    if (e == hipErrorOutOfMemory) {
      (void)hipGetLastError();
      b.ptr = nullptr;
      return KLEIN_OK;
    }
    if (e != hipSuccess) {
      b.ptr = nullptr;
      return map_hip(e);
    }
    b.bytes = want;
  }
  if (!b.done) {
    e = hipEventCreateWithFlags(&b.done, hipEventDisableTiming);
    if (e != hipSuccess) {
      b.done = nullptr;
      return map_hip(e);
    }
  }
  if (b.used) {
    e = hipStreamWaitEvent(hs, b.done, 0);
    if (e != hipSuccess) return map_hip(e);
  }
  const klein_status_t st = attn_ws(q, k, v, pos, out, nullptr, B, S, H, D, dtype, q_descale,
                                    k_descale, v_descale, b.ptr, b.bytes, stream);
  if (st != KLEIN_OK) return st;
  e = hipEventRecord(b.done, hs);
  if (e != hipSuccess) return map_hip(e);
  b.used = true;
  *ran = true;
  return KLEIN_OK;
}

}  // namespace

extern "C" {

klein_status_t klein_set_buffer_limit(size_t max_bytes) {
  g_buffer_limit.store(max_bytes);
  klein_status_t st = KLEIN_OK;
  int cur = -1;
  for (int d = 0; d < kMaxDevices; ++d) {
    DeviceBuffer& b = g_buffers[d];
    std::lock_guard<std::mutex> lock(b.mu);
    if (!b.ptr || b.bytes <= max_bytes) continue;
    if (cur < 0 && hipGetDevice(&cur) != hipSuccess) return KLEIN_ERR_NO_DEVICE;
    hipError_t e = hipSetDevice(d);
    if (e == hipSuccess) e = release_buffer(b);
    if (e != hipSuccess && st == KLEIN_OK) st = map_hip(e);
  }
  if (cur >= 0) {
    const hipError_t e = hipSetDevice(cur);
    if (e != hipSuccess && st == KLEIN_OK) st = map_hip(e);
  }
  return st;
}

klein_status_t klein_rope4d_attn_fwd(const void* q, const void* k, const void* v,
                                     const int32_t* pos_thwl, void* out, int B, int S, int H,
                                     int D, klein_dtype_t dtype, klein_stream_t stream) {
  if (dtype == KLEIN_DTYPE_FP8_E4M3)
    return klein_rope4d_attn_fwd_fp8(q, k, v, pos_thwl, out, B, S, H, D, 1.f, 1.f, 1.f, stream);
  if (dtype != KLEIN_DTYPE_BF16) return KLEIN_ERR_INVALID_ARG;
  klein_status_t st = check_common(q, k, v, pos_thwl, out, B, S, H, D);
  if (st != KLEIN_OK) return st;
  if (klein::attn_fwd_bf16_grid(B, S, H) > kMaxGrid) return KLEIN_ERR_UNSUPPORTED;
  try {
    bool ran = false;
    st = attn_on_buffer(q, k, v, pos_thwl, out, B, S, H, D, KLEIN_DTYPE_BF16, 1.f, 1.f, 1.f,
                        stream, &ran);
    if (st != KLEIN_OK || ran) return st;
    return map_hip(klein::launch_attn_fwd_bf16(make_args(q, k, v, pos_thwl, out, B, S, H, D, stream)));
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

klein_status_t klein_rope4d_attn_fwd_fp8(const void* q, const void* k, const void* v,
                                         const int32_t* pos_thwl, void* out, int B, int S, int H,
                                         int D, float q_descale, float k_descale, float v_descale,
                                         klein_stream_t stream) {
  klein_status_t st = check_common(q, k, v, pos_thwl, out, B, S, H, D);
  if (st != KLEIN_OK) return st;
  for (float s : {q_descale, k_descale, v_descale})
    if (!(std::isfinite(s) && s > 0.f)) return KLEIN_ERR_INVALID_ARG;
  if (klein::attn_fwd_fp8_grid(B, S, H) > kMaxGrid) return KLEIN_ERR_UNSUPPORTED;
  try {
    bool ran = false;
    st = attn_on_buffer(q, k, v, pos_thwl, out, B, S, H, D, KLEIN_DTYPE_FP8_E4M3, q_descale,
                        k_descale, v_descale, stream, &ran);
    if (st != KLEIN_OK || ran) return st;
    LaunchArgs a = make_args(q, k, v, pos_thwl, out, B, S, H, D, stream);
    a.descale[0] = q_descale; a.descale[1] = k_descale; a.descale[2] = v_descale;
    return map_hip(klein::launch_attn_fwd_fp8(a));
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

klein_status_t klein_rope4d_attn_fwd_lse(const void* q, const void* k, const void* v,
                                         const int32_t* pos_thwl, void* out, float* lse, int B,
                                         int S, int H, int D, klein_stream_t stream) {
  klein_status_t st = check_common(q, k, v, pos_thwl, out, B, S, H, D);
  if (st != KLEIN_OK) return st;
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u)) return KLEIN_ERR_INVALID_ARG;
  if (klein::attn_fwd_bf16_grid(B, S, H) > kMaxGrid) return KLEIN_ERR_UNSUPPORTED;
  try {
    LaunchArgs a = make_args(q, k, v, pos_thwl, out, B, S, H, D, stream);
    a.lse = lse;
    return map_hip(klein::launch_attn_fwd_bf16(a));
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

klein_status_t klein_attn_bwd_workspace_size(int B, int S, int H, int D, size_t* bytes) {
  if (!bytes) return KLEIN_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || H < 1) return KLEIN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return KLEIN_ERR_UNSUPPORTED;
  if (!shape_ok(S, H, D)) return KLEIN_ERR_UNSUPPORTED;
  *bytes = (size_t)klein::attn_bwd_workspace(B, S, H, D).total;
  return KLEIN_OK;
}

klein_status_t klein_rope4d_attn_bwd(const void* q, const void* k, const void* v,
                                     const int32_t* pos_thwl, const void* out, const void* dout,
                                     const float* lse, void* dq, void* dk, void* dv, int B, int S,
                                     int H, int D, void* workspace, size_t workspace_bytes,
                                     klein_stream_t stream) {
  klein_status_t st = check_common(q, k, v, pos_thwl, out, B, S, H, D);
  if (st != KLEIN_OK) return st;
  for (const void* p : {dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!p || !aligned16(p)) return KLEIN_ERR_INVALID_ARG;
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u)) return KLEIN_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return KLEIN_ERR_INVALID_ARG;
  const klein::BwdWorkspace wl = klein::attn_bwd_workspace(B, S, H, D);
  if (workspace_bytes < (size_t)wl.total) return KLEIN_ERR_INVALID_ARG;
  const long long nb = (S + 127) / 128;
  if ((long long)B * H * nb > kMaxGrid || (long long)B * S * H * D / 8 / 256 > kMaxGrid)
    return KLEIN_ERR_UNSUPPORTED;
  try {
    char* ws = static_cast<char*>(workspace);
    klein::BwdArgs a{};
    a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
    a.out = (const uint16_t*)out; a.dout = (const uint16_t*)dout; a.pos = pos_thwl; a.lse = lse;
    a.dq = (uint16_t*)dq; a.dk = (uint16_t*)dk; a.dv = (uint16_t*)dv;
    a.qr = reinterpret_cast<uint16_t*>(ws);
    a.kr = reinterpret_cast<uint16_t*>(ws + wl.kr);
    a.delta = reinterpret_cast<float*>(ws + wl.delta);
    a.norm2 = reinterpret_cast<float*>(ws + wl.norm2);
    a.escale = reinterpret_cast<float*>(ws + wl.escale);
    a.B = B; a.S = S; a.H = H; a.D = D;
    a.qscale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
    a.freqs = make_freqs(D);
    a.stream = reinterpret_cast<hipStream_t>(stream);
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return map_hip(e);
    if (dev < 0 || dev >= kMaxDevices) return map_hip(klein::launch_attn_bwd(a));
    BwdSide& side = g_bwd_side[dev];
    std::lock_guard<std::mutex> lock(side.mu);
    bwd_side_init(side);
    a.side = side.side;
    a.fork = side.fork;
    a.join = side.join;
    return map_hip(klein::launch_attn_bwd(a));
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

klein_status_t klein_attn_workspace_size(int B, int S, int H, int D, klein_dtype_t dtype,
                                         size_t* bytes) {
  if (!bytes) return KLEIN_ERR_INVALID_ARG;
  if (dtype != KLEIN_DTYPE_BF16 && dtype != KLEIN_DTYPE_FP8_E4M3) return KLEIN_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || H < 1) return KLEIN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return KLEIN_ERR_UNSUPPORTED;
  if (!shape_ok(S, H, D)) return KLEIN_ERR_UNSUPPORTED;
  if (klein::attn_fwd_bf16_grid(B, S, H) > kMaxGrid) return KLEIN_ERR_UNSUPPORTED;
  try {
    hipError_t e;
    const int ncu = current_cu_count(&e);
    if (e != hipSuccess) return map_hip(e);
    *bytes = (size_t)ws_layout(B, S, H, D, dtype, ncu).total;
    return KLEIN_OK;
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

klein_status_t klein_splitkv_plan(int B, int S, int H, int D, int n_cu, int* plan,
                                  size_t* partial_bytes) {
  if (!plan || !partial_bytes) return KLEIN_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || H < 1 || n_cu < 1) return KLEIN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return KLEIN_ERR_UNSUPPORTED;
  if (!shape_ok(S, H, D)) return KLEIN_ERR_UNSUPPORTED;
  if (klein::attn_fwd_bf16_grid(B, S, H) > kMaxGrid) return KLEIN_ERR_UNSUPPORTED;
  const klein::SplitPlan p = klein::plan_split(B, S, H, D, n_cu);
  plan[0] = p.n_sk > 0 ? p.n_dp : (int)klein::attn_fwd_bf16_grid(B, S, H);
  plan[1] = p.n_sk > 0 ? p.n_rem : 0;
  plan[2] = p.n_sk > 0 ? p.n_chunk : 0;
  *partial_bytes = (size_t)p.bytes;
  return KLEIN_OK;
}

klein_status_t klein_rope4d_attn_fwd_ws(const void* q, const void* k, const void* v,
                                        const int32_t* pos_thwl, void* out, int B, int S, int H,
                                        int D, klein_dtype_t dtype, float q_descale,
                                        float k_descale, float v_descale, void* workspace,
                                        size_t workspace_bytes, klein_stream_t stream) {
  return attn_ws(q, k, v, pos_thwl, out, nullptr, B, S, H, D, dtype, q_descale, k_descale,
                 v_descale, workspace, workspace_bytes, stream);
}

klein_status_t klein_rope4d_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                             const int32_t* pos_thwl, void* out, int B, int S,
                                             int H, int D, klein_dtype_t dtype, float q_descale,
                                             float k_descale, float v_descale,
                                             klein_stream_t stream) {
  static_assert(KLEIN_NOALLOC_SCRATCH_BYTES == klein::kNoallocScratchBytes,
                "the header states the scratch size");
  const klein_status_t st = check_ws_call(q, k, v, pos_thwl, out, B, S, H, D, dtype, q_descale,
                                          k_descale, v_descale);
  if (st != KLEIN_OK) return st;
  try {
    hipError_t e;
    const int ncu = current_cu_count(&e);
    if (e != hipSuccess) return map_hip(e);
    // v in key-major tiles where the scratch holds them too
    const bool vt = ws_layout(B, S, H, D, dtype, ncu, true).total <= klein::kNoallocScratchBytes;
    if (!vt && ws_layout(B, S, H, D, dtype, ncu, false).total > klein::kNoallocScratchBytes)
      return KLEIN_ERR_UNSUPPORTED;
    void* scratch = nullptr;
    e = klein::noalloc_scratch(&scratch);
    if (e != hipSuccess) return map_hip(e);
    return attn_ws(q, k, v, pos_thwl, out, nullptr, B, S, H, D, dtype, q_descale, k_descale,
                   v_descale, scratch, (size_t)klein::kNoallocScratchBytes, stream, vt);
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

klein_status_t klein_rope4d_attn_fwd_lse_ws(const void* q, const void* k, const void* v,
                                            const int32_t* pos_thwl, void* out, float* lse,
                                            int B, int S, int H, int D, void* workspace,
                                            size_t workspace_bytes, klein_stream_t stream) {
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u)) return KLEIN_ERR_INVALID_ARG;
  return attn_ws(q, k, v, pos_thwl, out, lse, B, S, H, D, KLEIN_DTYPE_BF16, 1.f, 1.f, 1.f,
                 workspace, workspace_bytes, stream);
}

static klein_status_t blocksparse(const void* q, const void* k, const void* v,
                                  const int32_t* pos_thwl, void* out, int B, int S, int H, int D,
                                  klein_dtype_t dtype, float q_descale, float k_descale,
                                  float v_descale, const uint8_t* block_mask, void* workspace,
                                  size_t workspace_bytes, bool use_ws, klein_stream_t stream) {
  if (dtype != KLEIN_DTYPE_BF16 && dtype != KLEIN_DTYPE_FP8_E4M3) return KLEIN_ERR_INVALID_ARG;
  klein_status_t st = check_common(q, k, v, pos_thwl, out, B, S, H, D);
  if (st != KLEIN_OK) return st;
  if (!block_mask) return KLEIN_ERR_INVALID_ARG;
  if ((S + KLEIN_SPARSE_KBLOCK - 1) / KLEIN_SPARSE_KBLOCK > klein::kSparseMaxTiles)
    return KLEIN_ERR_UNSUPPORTED;
  const bool fp8 = dtype == KLEIN_DTYPE_FP8_E4M3;
  if (fp8)
    for (float s : {q_descale, k_descale, v_descale})
      if (!(std::isfinite(s) && s > 0.f)) return KLEIN_ERR_INVALID_ARG;
  if ((fp8 ? klein::attn_fwd_fp8_grid(B, S, H) : klein::attn_fwd_bf16_grid(B, S, H)) > kMaxGrid)
    return KLEIN_ERR_UNSUPPORTED;
  if (use_ws) {
    const long long need = ((long long)B * S * H * D * (fp8 ? 1 : 2) + 255) / 256 * 256;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
        workspace_bytes < (size_t)need)
      return KLEIN_ERR_INVALID_ARG;
  }
  try {
    LaunchArgs a = make_args(q, k, v, pos_thwl, out, B, S, H, D, stream);
    a.bmask = block_mask;
    if (use_ws) a.krot = workspace;
    if (!fp8) return map_hip(klein::launch_attn_fwd_bf16(a));
    a.descale[0] = q_descale; a.descale[1] = k_descale; a.descale[2] = v_descale;
    return map_hip(klein::launch_attn_fwd_fp8(a));
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

klein_status_t klein_rope4d_attn_fwd_blocksparse(const void* q, const void* k, const void* v,
                                                 const int32_t* pos_thwl, void* out, int B,
                                                 int S, int H, int D, klein_dtype_t dtype,
                                                 float q_descale, float k_descale,
                                                 float v_descale, const uint8_t* block_mask,
                                                 klein_stream_t stream) {
  return blocksparse(q, k, v, pos_thwl, out, B, S, H, D, dtype, q_descale, k_descale, v_descale,
                     block_mask, nullptr, 0, false, stream);
}

klein_status_t klein_rope4d_attn_fwd_blocksparse_ws(const void* q, const void* k, const void* v,
                                                    const int32_t* pos_thwl, void* out, int B,
                                                    int S, int H, int D, klein_dtype_t dtype,
                                                    float q_descale, float k_descale,
                                                    float v_descale, const uint8_t* block_mask,
                                                    void* workspace, size_t workspace_bytes,
                                                    klein_stream_t stream) {
  return blocksparse(q, k, v, pos_thwl, out, B, S, H, D, dtype, q_descale, k_descale, v_descale,
                     block_mask, workspace, workspace_bytes, true, stream);
}

klein_status_t klein_attn_fwd_prerotated(const void* q, const void* k, const void* v, void* out,
                                        int B, int S, int H, int D, klein_stream_t stream) {
  if (!q || !k || !v || !out) return KLEIN_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || H < 1) return KLEIN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return KLEIN_ERR_UNSUPPORTED;
  if (!shape_ok(S, H, D)) return KLEIN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return KLEIN_ERR_INVALID_ARG;
  if (klein::attn_fwd_bf16_grid(B, S, H) > kMaxGrid) return KLEIN_ERR_UNSUPPORTED;
  try {
    return map_hip(klein::launch_attn_fwd_prerotated(
        make_args(q, k, v, nullptr, out, B, S, H, D, stream)));
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

static klein_status_t qkv_proj(const void* x, const void* w, const void* bias,
                               const int32_t* pos_thwl, void* q_out, void* k_out, void* v_out,
                               int B, int S, int C, int H, int D, bool fp8, float x_descale,
                               float w_descale, klein_stream_t stream) {
  if (!x || !w || !pos_thwl || !q_out || !k_out || !v_out) return KLEIN_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || C < 1 || H < 1) return KLEIN_ERR_INVALID_ARG;
  if (fp8 && !(std::isfinite(x_descale) && x_descale > 0.f && std::isfinite(w_descale) &&
               w_descale > 0.f))
    return KLEIN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return KLEIN_ERR_UNSUPPORTED;
  if (!shape_ok(S, H, D)) return KLEIN_ERR_UNSUPPORTED;
  if (C % (fp8 ? 128 : 64) != 0 || C > 65536) return KLEIN_ERR_UNSUPPORTED;
  for (const void* p : {x, w, (const void*)q_out, (const void*)k_out, (const void*)v_out,
                        (const void*)pos_thwl})
    if (!aligned16(p)) return KLEIN_ERR_INVALID_ARG;
  if (bias && (reinterpret_cast<uintptr_t>(bias) & 7u)) return KLEIN_ERR_INVALID_ARG;
  if (klein::qkv_rope_proj_grid(B, S, H, D) > kMaxGrid) return KLEIN_ERR_UNSUPPORTED;
  if ((long long)B * S * H * D * 3 >= (1LL << 40)) return KLEIN_ERR_UNSUPPORTED;
  if ((long long)B * S >= (1LL << 31)) return KLEIN_ERR_UNSUPPORTED;   // M = B S in 32 bits
  try {
    klein::QkvArgs a{};
    a.x = x; a.w = w; a.bias = (const uint16_t*)bias;
    a.fp8 = fp8; a.x_descale = x_descale; a.w_descale = w_descale;
    a.pos = pos_thwl;
    a.q = (uint16_t*)q_out; a.k = (uint16_t*)k_out; a.v = (uint16_t*)v_out;
    a.B = B; a.S = S; a.C = C; a.H = H; a.D = D;
    a.freqs = make_freqs(D);
    hipError_t e = hipSuccess;
    a.ncu = current_cu_count(&e);
    if (e != hipSuccess) return map_hip(e);
    a.stream = reinterpret_cast<hipStream_t>(stream);
    return map_hip(klein::launch_qkv_rope_proj(a));
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

klein_status_t klein_qkv_rope4d_proj(const void* x, const void* w, const void* bias,
                                     const int32_t* pos_thwl, void* q_out, void* k_out,
                                     void* v_out, int B, int S, int C, int H, int D,
                                     klein_stream_t stream) {
  return qkv_proj(x, w, bias, pos_thwl, q_out, k_out, v_out, B, S, C, H, D, false, 1.f, 1.f,
                  stream);
}

klein_status_t klein_qkv_rope4d_proj_fp8(const void* x, const void* w, const void* bias,
                                         const int32_t* pos_thwl, void* q_out, void* k_out,
                                         void* v_out, int B, int S, int C, int H, int D,
                                         float x_descale, float w_descale,
                                         klein_stream_t stream) {
  return qkv_proj(x, w, bias, pos_thwl, q_out, k_out, v_out, B, S, C, H, D, true, x_descale,
                  w_descale, stream);
}

klein_status_t klein_rope4d_apply(const void* x, const int32_t* pos_thwl, void* y, int B, int S,
                                  int H, int D, klein_stream_t stream) {
  if (!x || !pos_thwl || !y) return KLEIN_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || H < 1) return KLEIN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return KLEIN_ERR_UNSUPPORTED;
  if (!shape_ok(S, H, D)) return KLEIN_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y) || !aligned16(pos_thwl)) return KLEIN_ERR_INVALID_ARG;
  try {
    return map_hip(klein::launch_rope4d_apply(make_args(x, x, x, pos_thwl, y, B, S, H, D, stream)));
  } catch (...) {
    return KLEIN_ERR_LAUNCH;
  }
}

const char* klein_status_string(klein_status_t status) {
  switch (status) {
    case KLEIN_OK: return "ok";
    case KLEIN_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, size < 1, bad dtype or descale)";
    case KLEIN_ERR_UNSUPPORTED: return "unsupported (head dim must be 64 or 128, H*D below 2^22 and S below 2^29; grid or block mask too large; or, for klein_rope4d_attn_fwd_noalloc, the call needs more than its fixed scratch)";
    case KLEIN_ERR_NO_DEVICE: return "no usable GPU";
    case KLEIN_ERR_LAUNCH: return "kernel launch failed";
    case KLEIN_STATUS_SPAN_INT_: break;
  }
  return "unknown status";
}

int klein_version(void) { return 131; }

}  // extern "C"
