/*
 * klein_attn.h -- C ABI of the MI355X (gfx950) RoPE-4D joint-attention library.
 *
 * What the library computes
 * -------------------------
 * The joint blocks of FLUX.3 Image Klein run self-attention over one sequence
 * that concatenates text, noisy-image-latent and reference-image tokens, with
 * every token attending to every other token, and encode position with a
 * rotary embedding over four axes: time step t, height h, width w and sequence
 * length l ("Flux.3 Image Klein arrives in Diffusers with a modular
 * architecture", bytechap.com, section "How it works").  The prompt padding is
 * attended and one prompt is handled per call ("FLUX.3 Image Klein open
 * weights ...", kimiseek.app, section "Limitations and unconfirmed points"),
 * so there is no mask; reference and output share (h, w) coordinates (same
 * page, section "Adoption and evaluation proposals"), so positions are given
 * per token.  For every batch entry b and head h:
 *
 *   q'_i = R(pos_i) q_i,   k'_j = R(pos_j) k_j
 *   out_i = sum_j softmax_j(<q'_i, k'_j> / sqrt(D)) v_j      (i, j in [0, S))
 *
 * R is RoPE-4D: D is split into four blocks of D/4 channels in the order
 * t, h, w, l; inside axis block a the interleaved channel pair (2j, 2j+1),
 * j < D/8, is rotated by the angle pos_a * 10000^(-2j/(D/4)), a pair (x, y)
 * becoming (x cos - y sin, x sin + y cos).  V is not rotated.  (The pages
 * name the axes but print no formula; this is the plainest reading and the
 * one the CPU oracle of this repository implements.)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers to tensors are DEVICE pointers, owned by the caller, 16-byte
 *    aligned.  The library keeps no per-call state.  It holds device memory
 *    of its own in two places only: the buffer per GPU that
 *    klein_rope4d_attn_fwd and klein_rope4d_attn_fwd_fp8 create on first use
 *    (see there; klein_set_buffer_limit bounds it), and the static scratch
 *    array of klein_rope4d_attn_fwd_noalloc.  No other entry point
 *    allocates.
 *  - q, k, v, out are contiguous [B][S][H][D] (D fastest, then heads, then
 *    tokens, then batch).  out is always bfloat16.
 *  - pos_thwl is contiguous int32 [S][4] in the order (t, h, w, l) and is
 *    shared by every batch entry.  Angles are formed in fp32; accuracy is
 *    stated for |pos| < 4096 on every axis (larger values are accepted, with
 *    angle error growing like |pos| * 2^-24 revolutions).
 *  - D must be 64 or 128; B, S, H >= 1; B*H*ceil(S/256) < 2^31; H*D < 2^22
 *    and S < 2^29 (every entry point; larger shapes return UNSUPPORTED).
 *  - bf16 path: the rotated Q (times log2(e)/sqrt(D)) and K are held on chip
 *    as fp16 for the score products (three more mantissa bits than bf16), so
 *    elementwise |k| must stay below ~46000 and |q| below ~360000; larger
 *    magnitudes overflow fp16.  P and V are bf16; accumulation is fp32.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL means the null
 *    stream).  The status reports argument and launch errors only, never
 *    results of device work.  Argument checks run before any HIP call, so an
 *    invalid call touches no device.  No C++ exception crosses this ABI.
 *  - Calls are thread-safe; concurrent calls on different streams are fine,
 *    except for klein_rope4d_attn_fwd_noalloc (see there).
 */
#ifndef KLEIN_ATTN_H
#define KLEIN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums carry one more enumerator, at INT_MIN, that is no value of the
 * type: it makes each type span every int, so that any int a caller passes
 * (and the library rejects) is a valid value of the type in C++ too. */
typedef enum {
  KLEIN_DTYPE_BF16 = 0,      /* q, k, v are bfloat16 */
  KLEIN_DTYPE_FP8_E4M3 = 1,  /* q, k, v are OCP FP8 E4M3FN codes, descale 1 */
  KLEIN_DTYPE_SPAN_INT_ = -0x7fffffff - 1
} klein_dtype_t;

typedef enum {
  KLEIN_OK = 0,
  KLEIN_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, size < 1, bad dtype, bad descale */
  KLEIN_ERR_UNSUPPORTED = 2,  /* D not in {64, 128}, H*D >= 2^22, S >= 2^29, or grid too large */
  KLEIN_ERR_NO_DEVICE = 3,    /* the HIP runtime found no usable GPU */
  KLEIN_ERR_LAUNCH = 4,       /* the kernel launch itself failed */
  KLEIN_STATUS_SPAN_INT_ = -0x7fffffff - 1
} klein_status_t;

/* Opaque stream handle: a hipStream_t passed as a pointer. */
typedef void* klein_stream_t;

/*
 * RoPE-4D joint self-attention forward (the definition above).
 *   q, k, v : [B][S][H][D] bfloat16 (dtype BF16) or E4M3FN codes (FP8_E4M3,
 *             all descales 1; use klein_rope4d_attn_fwd_fp8 for scales)
 *   pos_thwl: [S][4] int32 (t, h, w, l)
 *   out     : [B][S][H][D] bfloat16, written completely; must not alias inputs
 * Softmax scale is fixed at 1/sqrt(D).  Accumulation is fp32.
 *
 * Schedule and memory.  The call runs the schedule of klein_rope4d_attn_fwd_ws
 * (keys rotated once, the last round's query tiles split over key chunks)
 * in a buffer the library owns: one per GPU, created by the first call on
 * that GPU, replaced by a larger one when a call needs more (its size is
 * what klein_attn_workspace_size reports, rounded up to 32 MiB), and kept
 * until klein_set_buffer_limit lowers the limit below it or the process
 * ends.  Calls that share the buffer are ordered on the GPU: each call's
 * stream waits for the previous call's kernels, whatever stream they ran on,
 * so concurrent calls on different streams of one GPU run one after the
 * other (each fills the GPU).  The call instead runs kernels that need no
 * memory (each workgroup rotates the key tiles it loads; the last round may
 * leave compute units idle) when
 *   - the stream is being captured into a HIP graph (a graph must not hold
 *     the address of a buffer a later call may free),
 *   - the shape needs more than the limit (default 2 GiB), or
 *   - the buffer cannot be allocated for lack of memory (the error is
 *     cleared).
 * The two schedules give the same bits for every query tile that no split
 * touches; split tiles are merged from fp32 partials and agree to rounding.
 * Growing the buffer waits on the host for the previous call's kernels.
 */
klein_status_t klein_rope4d_attn_fwd(const void* q, const void* k, const void* v,
                                     const int32_t* pos_thwl, void* out,
                                     int B, int S, int H, int D,
                                     klein_dtype_t dtype, klein_stream_t stream);

/*
 * Limit, in bytes, of the buffer klein_rope4d_attn_fwd and
 * klein_rope4d_attn_fwd_fp8 keep per GPU (default KLEIN_DEFAULT_BUFFER_LIMIT).
 * Shapes whose schedule needs more run the kernels that need no memory; a
 * limit of 0 makes those calls allocate nothing.  A buffer larger than the
 * new limit is freed at once, after the host has waited for the kernels
 * already queued on it (the call then makes HIP calls on each GPU that holds
 * one and restores the current device).  Thread-safe.
 * Returns KLEIN_OK, or the error of a HIP call that failed (the limit is set
 * in any case).
 */
#define KLEIN_DEFAULT_BUFFER_LIMIT ((size_t)2 << 30)
klein_status_t klein_set_buffer_limit(size_t max_bytes);

/*
 * FP8 variant with per-tensor scales: the value of an element is
 * decode_e4m3(code) * descale, for q, k and v separately (the FP8 attention
 * the Blackwell write-up benchmarks -- "How FLUX 3 Image Klein was made 3-4x
 * faster on NVIDIA Blackwell", section "Method 2", attention table -- read as
 * per-tensor scaled E4M3).  Descales must be finite and > 0.  out is
 * bfloat16.  Precision on chip: the rotated Q/K are re-quantised to E4M3; the
 * scores are fp32 sums, taken relative to a running row max; the
 * probabilities fed to the P.V product are E4M3 codes rounded straight from
 * the scores, code = rne(8 (s - m) + 118) with s, m in log2 units, which
 * reads a code as the log2 of its value: within a binade this is a linear
 * interpolation of 2^x, up to 6.2 % high, and the same codes give the row
 * sums, so only the variation of that bias is left in out.  The row max is
 * raised lazily, only when a row's code would pass 126 (448), and then to
 * code 110: a key is kept as a normal E4M3 number down to 13.75 binades
 * (9.5 nats) below its row's first max (12.75 below a raised one), as a
 * subnormal about one binade further, and as 0 below that.  On N(0, 1) inputs of
 * the 2048^2 edit workload the result is within 4.5e-2 relative L2 of exact
 * attention of the decoded inputs (bound 6e-2).  Schedule and memory as
 * klein_rope4d_attn_fwd.
 */
klein_status_t klein_rope4d_attn_fwd_fp8(const void* q, const void* k, const void* v,
                                         const int32_t* pos_thwl, void* out,
                                         int B, int S, int H, int D,
                                         float q_descale, float k_descale,
                                         float v_descale, klein_stream_t stream);

/*
 * The same attention (bf16, or FP8 E4M3 with per-tensor descales as in
 * klein_rope4d_attn_fwd_fp8; dtype BF16 ignores the descales), scheduled so
 * that every compute unit of the GPU stays busy to the end of the call.  The
 * dense entry points give each workgroup one tile of 256 queries against all
 * keys; when the B*H*ceil(S/256) tiles do not fill whole rounds of the GPU,
 * the last round leaves compute units idle.  Here the whole rounds run the
 * same way and each remaining tile's keys are cut into chunks at the same
 * boundaries for every tile, one workgroup per chunk, so that all compute
 * units share the tail; the chunks' partial results (unnormalised output,
 * running max, row sum) go to `workspace`, and a second kernel on the same
 * stream merges them in key order into the output rows.  Rows of tiles that
 * run whole are bit-identical to the dense entry points'; rows of split tiles
 * differ by the rounding of the probabilities against each chunk's own
 * running max and the fp32 merge, within the same error bounds.  The result
 * is deterministic (fixed merge order).
 * The keys are also rotated once, into `workspace` (fp16 for bf16 inputs,
 * E4M3 codes of R k / 2 for fp8), before the attention kernel; the dense
 * entry points rotate every key tile once per tile of 256 queries.  The
 * values equal those the dense kernels form.  For bf16 with S >= 12,288 the
 * values are also regrouped once into key-major tiles (per head and 64-key
 * tile, one row of 64 keys per channel), which the kernel reads with plain
 * 16-byte LDS reads instead of transposing ones; this moves data only, so
 * the output bits do not change (shorter sequences gain less than the pass
 * costs).
 *   workspace      : DEVICE pointer, 256-byte aligned, caller-owned, at least
 *                    the size klein_attn_workspace_size reports for the same
 *                    shape on the current device (may be NULL when that is 0).
 *                    Its contents on entry do not matter.  Two calls that
 *                    use one workspace at the same time on different streams
 *                    race.
 *   workspace_bytes: its size; smaller than required is INVALID_ARG.
 */
klein_status_t klein_rope4d_attn_fwd_ws(const void* q, const void* k, const void* v,
                                        const int32_t* pos_thwl, void* out,
                                        int B, int S, int H, int D, klein_dtype_t dtype,
                                        float q_descale, float k_descale, float v_descale,
                                        void* workspace, size_t workspace_bytes,
                                        klein_stream_t stream);

/*
 * Workspace bytes klein_rope4d_attn_fwd_ws needs for this shape on the
 * current HIP device: the rotated keys (B*S*H*D*2 bytes for bf16, B*S*H*D
 * for fp8, rounded up to a multiple of 256), for bf16 with S >= 12,288 the
 * key-major value tiles (B*H*ceil(S/64)*64*D*2 bytes), then the split
 * partials (0 when the tiles fill whole rounds, or the sequence is shorter
 * than 2048 keys, and nothing is split; at most 4 * (number of compute
 * units) * (256 * D + 1024) * 4 bytes, 138 MB for D = 128 on 256 compute
 * units).  Writes *bytes; INVALID_ARG for a null `bytes`, sizes < 1 or a bad
 * dtype, UNSUPPORTED for D not in {64, 128}, NO_DEVICE without a usable GPU.
 */
klein_status_t klein_attn_workspace_size(int B, int S, int H, int D, klein_dtype_t dtype,
                                         size_t* bytes);

/*
 * The split-KV plan that klein_rope4d_attn_fwd_ws follows for this shape on a
 * GPU with n_cu compute units.  Host-only: touches no device, so it also
 * serves to inspect the schedule for other GPUs.  With
 *   items = B * H * ceil(S / 256)      (one workgroup each: 256 queries)
 *   nkt   = ceil(S / 64)               (64-key tiles per item)
 *   rem   = items mod n_cu             (items of the last, partial round)
 * nothing is cut when nkt < 32 or rem == 0.  Otherwise each chunk count
 * c = 2, 3, ... with 8 c <= nkt and c * rem <= 4 * n_cu is priced at
 *   cost(c) = ceil(c * rem / n_cu) * (nkt / c + 6)   tile steps
 * against cost(1) = nkt for whole items; the cheapest c (the smallest on a
 * tie) is taken if its cost is at most 0.85 * nkt, else nothing is cut.
 * On return:
 *   plan[0] = items run whole (first, in whole rounds when anything is cut)
 *   plan[1] = items cut into key chunks (rem, or 0)
 *   plan[2] = chunks per cut item (c, or 0)
 *   *partial_bytes = c * rem * (256 * D + 1024) * 4, the fp32 partials'
 *                    share of the workspace (0 when nothing is cut)
 * INVALID_ARG for null outputs or sizes < 1 (n_cu included), UNSUPPORTED
 * for D not in {64, 128} or a grid past 2^31 - 1 workgroups.
 */
klein_status_t klein_splitkv_plan(int B, int S, int H, int D, int n_cu, int* plan,
                                  size_t* partial_bytes);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the call
 * klein_rope4d_attn_fwd_ws makes (same arguments, same kernels, same
 * result bit for bit), with its workspace replaced by a scratch array that
 * the library holds in static device memory, one per GPU.  The call itself
 * allocates nothing and calls no allocating routine.
 *   Scratch: KLEIN_NOALLOC_SCRATCH_BYTES (320 MiB) per GPU, taken when the
 *   process first calls this function on that GPU and held until the
 *   process ends.  Where the bf16 workspace layout (keys, key-major value
 *   tiles, partials) does not fit, the call keeps the values row-major and
 *   reads them with transposing LDS reads (same output bits, a few percent
 *   slower).  A call that does not fit even so returns UNSUPPORTED before
 *   any device work (e.g. B = 4, S = 16,896, H = 24, D = 128, bf16 needs
 *   517 MB with the values row-major; the 2048^2 shapes with B = 2 bf16
 *   (311 MB, values row-major) or B = 1 fp8 fit).
 *   Every call on one GPU uses that GPU's single array: two calls that run
 *   at the same time on one GPU (different streams, threads or processes
 *   sharing a context) race, and their results are undefined; calls in
 *   stream order are fine.  The array keeps the last call's contents; no
 *   part of it needs to start at zero (every byte a call reads, it has
 *   written before, in stream order).
 * Other arguments and errors as klein_rope4d_attn_fwd_ws (dtype BF16
 * ignores the descales); NO_DEVICE without a usable GPU.
 */
#define KLEIN_NOALLOC_SCRATCH_BYTES (320LL * 1024 * 1024)
klein_status_t klein_rope4d_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                             const int32_t* pos_thwl, void* out,
                                             int B, int S, int H, int D, klein_dtype_t dtype,
                                             float q_descale, float k_descale,
                                             float v_descale, klein_stream_t stream);

/*
 * Training forward: klein_rope4d_attn_fwd for bfloat16 inputs that also
 * writes the softmax statistic the backward needs,
 *   lse[b][h][i] = log sum_j exp(<q'_i, k'_j> / sqrt(D))   (natural log),
 * lse: DEVICE pointer, fp32 [B][H][S], 4-byte aligned, caller-owned.
 * Training is the use the pages give for it: LoRA and DreamBooth-style
 * training of the model ("Flux.3 Image Klein arrives in Diffusers with a
 * modular architecture", sections "What happened" and "Key details").
 */
klein_status_t klein_rope4d_attn_fwd_lse(const void* q, const void* k, const void* v,
                                         const int32_t* pos_thwl, void* out, float* lse,
                                         int B, int S, int H, int D, klein_stream_t stream);

/*
 * klein_rope4d_attn_fwd_lse on the schedule of klein_rope4d_attn_fwd_ws (keys
 * rotated once into the workspace, the last round's query tiles split over
 * key chunks and merged, lse written by the kernel for whole tiles and by the
 * merge for split ones).  Workspace as klein_rope4d_attn_fwd_ws with dtype
 * BF16; lse as klein_rope4d_attn_fwd_lse.  Tiles that run whole give the
 * same out and lse bits as klein_rope4d_attn_fwd_lse.
 */
klein_status_t klein_rope4d_attn_fwd_lse_ws(const void* q, const void* k, const void* v,
                                            const int32_t* pos_thwl, void* out, float* lse,
                                            int B, int S, int H, int D, void* workspace,
                                            size_t workspace_bytes, klein_stream_t stream);

/*
 * Backward of the bf16 attention: given the forward's inputs, its output
 * `out` and lse (klein_rope4d_attn_fwd_lse), and dout = dL/dout, writes the
 * gradients of L with respect to the unrotated q, k and v:
 *   dv_j = sum_i p_ij dout_i,  ds_ij = p_ij (<dout_i, v_j> - <dout_i, out_i>),
 *   dq_i = R(pos_i)^T sum_j ds_ij k'_j / sqrt(D),
 *   dk_j = R(pos_j)^T sum_i ds_ij q'_i / sqrt(D)
 * with p_ij = exp(<q'_i, k'_j> / sqrt(D) - lse_i).  R^T turns each channel
 * pair back by the same angle.
 *   q, k, v, out, dout: [B][S][H][D] bfloat16; lse: fp32 [B][H][S];
 *   dq, dk, dv: [B][S][H][D] bfloat16, written completely, must not alias
 *   the inputs.  Accumulation is fp32; the recomputed scores use the same
 *   fp16 rotated operands as the forward, P is rounded to bf16 and ds to
 *   fp16 as MFMA operands.  Both carry a power-of-two factor 2^e per (b, h),
 *   removed exactly at the end, with e chosen from the largest row norms of
 *   dout and v so that |2^e ds| stays below 2^14: ds keeps fp16's full
 *   precision whether dout is tiny (fine-tuning gradients of 1e-6 and
 *   below) or large, instead of falling into fp16's subnormals or
 *   overflowing.
 *   workspace: DEVICE pointer, 256-byte aligned, caller-owned, at least
 *   klein_attn_bwd_workspace_size bytes (the rotated q and k in fp16,
 *   <dout_i, out_i>, the squared row norms of dout and v, and the per-head
 *   exponents, in fp32); contents on entry do not matter.
 * Two calls sharing one workspace on different streams race.  A smaller
 * workspace is INVALID_ARG.
 * Ordering: the call is ordered on `stream` as one unit.  Inside, the dq
 * kernel runs on a second stream the library creates once per device
 * (non-blocking, default priority), forked from `stream` and joined back
 * into it with events, so it overlaps the dk/dv kernel; under graph capture
 * of `stream` that stream joins the capture.
 */
klein_status_t klein_rope4d_attn_bwd(const void* q, const void* k, const void* v,
                                     const int32_t* pos_thwl, const void* out, const void* dout,
                                     const float* lse, void* dq, void* dk, void* dv,
                                     int B, int S, int H, int D, void* workspace,
                                     size_t workspace_bytes, klein_stream_t stream);

/*
 * Workspace bytes klein_rope4d_attn_bwd needs: 2 * (2 B S H D) + 4 B H S +
 * 8 B H S + 4 B H, each part rounded up to a multiple of 256 bytes.
 * INVALID_ARG for a null `bytes` or sizes < 1, UNSUPPORTED for D not in
 * {64, 128}.
 */
klein_status_t klein_attn_bwd_workspace_size(int B, int S, int H, int D, size_t* bytes);

/*
 * Block-sparse variant: the same attention with each query attending only to
 * the keys of the kept blocks of its query block.  This is how this library
 * reads the sparsified attention of the Blackwell write-up ("How FLUX 3 Image
 * Klein was made 3-4x faster on NVIDIA Blackwell", section "Method 2": weakly
 * related query/key combinations are left out, the early denoising steps
 * stay dense).  The page gives no rule for choosing the combinations, so the
 * caller passes them:
 *   block_mask: DEVICE pointer, uint8 [B][H][ceil(S/KLEIN_SPARSE_QBLOCK)]
 *               [ceil(S/KLEIN_SPARSE_KBLOCK)], contiguous; nonzero = compute
 *               the block of queries [i*QBLOCK, (i+1)*QBLOCK) against keys
 *               [j*KBLOCK, (j+1)*KBLOCK).
 * For query i in query block I: out_i = sum over keys j in kept blocks (I, J)
 * of softmax_j(<q'_i, k'_j> / sqrt(D)) v_j, the softmax taken over those keys
 * only; a query block with no kept block gets out = 0.  Work and time scale
 * with the kept blocks; with every block kept the result is bit-identical to
 * the dense entry points.  dtype BF16 ignores the descales; FP8_E4M3 uses
 * them as klein_rope4d_attn_fwd_fp8 does (finite, > 0).
 * ceil(S/KLEIN_SPARSE_KBLOCK) must not exceed 4096 (else UNSUPPORTED);
 * a null mask is INVALID_ARG.
 */
#define KLEIN_SPARSE_QBLOCK 256
#define KLEIN_SPARSE_KBLOCK 64
klein_status_t klein_rope4d_attn_fwd_blocksparse(const void* q, const void* k, const void* v,
                                                 const int32_t* pos_thwl, void* out,
                                                 int B, int S, int H, int D,
                                                 klein_dtype_t dtype, float q_descale,
                                                 float k_descale, float v_descale,
                                                 const uint8_t* block_mask,
                                                 klein_stream_t stream);

/*
 * The block-sparse variant with the keys rotated once into a caller-owned
 * workspace first (as klein_rope4d_attn_fwd_ws does) instead of once per
 * query tile; the result equals klein_rope4d_attn_fwd_blocksparse's bit for
 * bit.  Nothing is split.
 *   workspace      : DEVICE pointer, 256-byte aligned, caller-owned, at least
 *                    B*S*H*D*2 bytes for bf16 (B*S*H*D for fp8), rounded up
 *                    to a multiple of 256 (klein_attn_workspace_size for the
 *                    same shape is always enough); contents on entry do not
 *                    matter; calls that share one at the same time race.
 *   workspace_bytes: its size; smaller than required, or a null or
 *                    misaligned workspace, is INVALID_ARG.
 * Other arguments and errors as klein_rope4d_attn_fwd_blocksparse.
 */
klein_status_t klein_rope4d_attn_fwd_blocksparse_ws(const void* q, const void* k, const void* v,
                                                    const int32_t* pos_thwl, void* out,
                                                    int B, int S, int H, int D,
                                                    klein_dtype_t dtype, float q_descale,
                                                    float k_descale, float v_descale,
                                                    const uint8_t* block_mask, void* workspace,
                                                    size_t workspace_bytes,
                                                    klein_stream_t stream);

/*
 * QKV projection with the RoPE-4D rotation fused into its epilogue -- the
 * step that feeds the attention in each joint block ("Flux.3 Image Klein
 * arrives in Diffusers with a modular architecture", section "How it works";
 * the fused QKV GEMMs of "How FLUX 3 Image Klein was made 3-4x faster on
 * NVIDIA Blackwell", section "Method 1"):
 *   y = x W^T (+ bias);  q = y[:, 0:HD], k = y[:, HD:2HD], v = y[:, 2HD:3HD]
 *   q_out = R(pos) q, k_out = R(pos) k  (fp16),  v_out = v  (bfloat16)
 *   x       : [B][S][C] bfloat16 (C % 64 == 0, C <= 65536, B*S < 2^31, else
 *             UNSUPPORTED)
 *   w       : [3*H*D][C] bfloat16 (a linear layer's [out, in] layout)
 *   bias    : [3*H*D] bfloat16, 8-byte aligned, or NULL
 *   pos_thwl: [S][4] int32, shared by all batch entries
 *   q_out, k_out: [B][S][H][D] fp16 (IEEE binary16), rotated; v_out: [B][S][H][D]
 *   bfloat16.  Accumulation is fp32; the outputs are rounded once.  The fp16
 *   q/k outputs hold |value| < 65504; klein_attn_fwd_prerotated takes them.
 * Device pointers, 16-byte aligned (bias 8), caller-owned; nothing allocated.
 */
klein_status_t klein_qkv_rope4d_proj(const void* x, const void* w, const void* bias,
                                     const int32_t* pos_thwl, void* q_out, void* k_out,
                                     void* v_out, int B, int S, int C, int H, int D,
                                     klein_stream_t stream);

/*
 * The same projection with FP8 operands (the quantised GEMMs of "How FLUX 3
 * Image Klein was made 3-4x faster on NVIDIA Blackwell", section "Method 1",
 * in the E4M3 format this library's FP8 attention takes):
 *   x : [B][S][C] E4M3FN codes, value = decode(code) * x_descale
 *   w : [3*H*D][C] E4M3FN codes, value = decode(code) * w_descale
 *   y = (sum_c x_code w_code) * x_descale * w_descale (+ bias), fp32
 *   accumulation; bias bfloat16 as above; outputs, rotation and rounding as
 *   klein_qkv_rope4d_proj (fp16 q', k', bfloat16 v).
 * C must be a multiple of 128 (UNSUPPORTED otherwise) and at most 65536;
 * descales finite and > 0 (else INVALID_ARG).  Device pointers, 16-byte
 * aligned (bias 8), caller-owned; nothing allocated.
 */
klein_status_t klein_qkv_rope4d_proj_fp8(const void* x, const void* w, const void* bias,
                                         const int32_t* pos_thwl, void* q_out, void* k_out,
                                         void* v_out, int B, int S, int C, int H, int D,
                                         float x_descale, float w_descale,
                                         klein_stream_t stream);

/*
 * Joint attention of queries and keys that are already rotated (as
 * klein_qkv_rope4d_proj emits them): out_i = sum_j softmax_j(<q_i, k_j> /
 * sqrt(D)) v_j over all j, no mask -- the definition above with the rotation
 * done upstream, so no positions are needed and the kernel's K tiles are
 * plain copies.
 *   q, k: [B][S][H][D] fp16 (|k| < ~46000, |q| < ~360000 as for the bf16 path)
 *   v, out: [B][S][H][D] bfloat16.  D in {64, 128}.
 */
klein_status_t klein_attn_fwd_prerotated(const void* q, const void* k, const void* v, void* out,
                                        int B, int S, int H, int D, klein_stream_t stream);

/*
 * Test hook: y = R(pos) x for bfloat16 x, y [B][S][H][D] (same layout rules),
 * computed with the very device routine the attention kernels use for Q and
 * K, rounded to bfloat16.  x and y may be the same buffer.
 */
klein_status_t klein_rope4d_apply(const void* x, const int32_t* pos_thwl, void* y,
                                  int B, int S, int H, int D,
                                  klein_stream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* klein_status_string(klein_status_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int klein_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KLEIN_ATTN_H */
