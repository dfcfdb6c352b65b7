/*
 * kda.h -- C ABI of the MI355X (gfx950) chunked forward of Kimi Delta Attention (KDA).
 *
 * What one call computes.  For every sequence b and value head h (query/key head
 * hq = h / (n_v / n_qk)), starting from S = initial_state[b, h] (a d_v x d_k fp32 matrix whose
 * rows are value channels), every token t of the sequence does
 *     S <- S * Diag(exp(g_t))                 decay of the key columns
 *     S <- S + beta_t * (v_t - S k_t) k_t^T    delta-rule write
 *     o_t = scale * S q_t                      read after the write
 * and final_state[b, h] = S at the end.  This is the recurrence that the FlashKDA README
 * (section 功能说明) evaluates chunk by chunk; the state decay is the natural-base exp(g) of the
 * vLLM PR #43195 summary (section 功能与动机).  The library evaluates it in 64-token chunks
 * with 16-token sub-blocks, log2-space gates and bf16 MFMA, exactly up to rounding.
 *
 * Interface model: the FlashKDA README (sections 参数说明, 返回值说明, 约束说明) -- q, k, v,
 * g, beta, scale, initial_state, layout, cu_seqlens in; out and a new final_state back.  g is
 * the activated natural-log decay for kda_chunk_fwd; kda_chunk_fwd_raw_gate takes the raw gate
 * with A_log, dt_bias and lower_bound and activates it in the kernel.  The Ascend scheduling
 * metadata of that interface has no counterpart here (the plan follows from the shape).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device, 16-byte aligned and
 *     contiguous in the stated layout.  The caller owns all buffers and the stream; the library
 *     allocates no device memory and keeps no state between calls (it is reentrant; concurrent
 *     calls need distinct workspaces).  The one exception is kda_chunk_fwd_noalloc, whose
 *     workspace is a device array the library holds per GPU (see there).
 *   - Work is enqueued on `stream`; the call returns right after enqueueing.  The host never
 *     reads device data.
 *   - Arguments are validated on the host, from shapes and pointers only, before any launch.
 *     A failed check returns an error and launches nothing.
 *   - Not checked (preconditions, as in the FlashKDA README, section 约束说明): cu_seqlens
 *     starts at 0, is strictly increasing and ends at seq_len (TND); with BNSD/BSND each valid
 *     length lies in [1, seq_len]; -5 <= g <= 0; all tensors live on one device.  The decayed
 *     keys (at most |k|), the decayed queries times scale (at most |q| scale), the values
 *     transformed inside a chunk (about |v|), the innovation v - S k of the state update and
 *     the state itself (initial, carried from chunk to chunk and, in the two-level scan, the
 *     segment entry state) are held in fp16 or as fp16 hi/lo pairs (limit 65504; larger
 *     magnitudes overflow to inf).  Tested range: L2-normalised
 *     keys with v and the initial state scaled by up to 2048 (|v| up to about 1e4), every output
 *     and final state within the tolerance in units of that scale, one- and two-level scans,
 *     head dims 128 and 64.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Physical layouts (FlashKDA README, section 参数说明).  B = batch, N = heads, S = stored
 * length, T = packed tokens, D = d_k = d_v (128, or 64):
 *   BNSD: q,k [B,n_qk,S,D]  v,g,out [B,n_v,S,D]  beta [B,n_v,S]
 *   BSND: q,k [B,S,n_qk,D]  v,g,out [B,S,n_v,D]  beta [B,S,n_v]
 *   TND:  q,k [T,n_qk,D]    v,g,out [T,n_v,D]    beta [T,n_v]   (packed; cu_seqlens required) */
typedef enum {
    KDA_LAYOUT_BNSD = 0,
    KDA_LAYOUT_BSND = 1,
    KDA_LAYOUT_TND = 2
} kda_layout;

/* Fused prologue options (FlashKDA README, section 功能说明: q/k row L2 normalise and the beta
 * sigmoid are fused into the operator).  KDA_QK_L2NORM replaces each q and k row x by
 * x / sqrt(sum(x^2) + 1e-6); KDA_BETA_SIGMOID reads beta as a logit and applies 1/(1+e^-x).
 * KDA_SCALAR_GATE selects the scalar-gate (GDN) form: g holds one value per (token, value head),
 * laid out like beta, and exp(g_t) decays every key channel alike (the GDN kernels of the vLLM
 * PR #42076 and #45000 summaries, sections 关键源码片段, apply the gate after the key product,
 * which only a channel-independent gate allows). */
enum {
    KDA_QK_L2NORM = 1u << 0,
    KDA_BETA_SIGMOID = 1u << 1,
    KDA_SCALAR_GATE = 1u << 2,
    KDA_RAW_GATE = 1u << 3     /* kda_chunk_fwd_raw_gate only: g is the raw bf16 gate */
};

/* Raw-gate activation (FlashKDA README, sections 参数说明 and 快速开始: a raw bf16 gate shaped
 * like v with A_log [n_v] fp32, "the log time scale of each value head", dt_bias [n_v, d_k] fp32,
 * "the gate bias", and lower_bound in [-5, 0], "the gate's lower bound"; section 约束说明 bounds
 * lower_bound).  The README prints no formula; this library reads it as
 *     g[t, j] = lower_bound * sigmoid(exp(A_log[h]) * (g_raw[t, j] + dt_bias[h, j]))
 * for value head h and key channel j, so every activated gate lies in [lower_bound, 0] (the
 * form -5 * sigmoid(x) of the 8K-prefill workload's own gate), and then runs the recurrence
 * above on it. */
typedef struct {
    const float* a_log;     /* device pointer, fp32 [n_v], 4-byte aligned                   */
    const float* dt_bias;   /* device pointer, fp32 [n_v, d_k], 16-byte aligned             */
    float lower_bound;      /* in [-5, 0]; KDA_ERR_INVALID_ARG otherwise (NaN included)      */
} kda_raw_gate;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,  /* a NULL or misaligned pointer, bad enum, negative size, alias */
    KDA_ERR_UNSUPPORTED = 2,  /* a valid request the library does not implement: head dim, or
                                 sizes past its limits (n_v * d_k >= 2^24; more than 2^31 - 1
                                 workgroups in a kernel; tensors of 2^60 elements or more) */
    KDA_ERR_WORKSPACE = 3,    /* workspace pointer NULL or workspace_bytes too small */
    KDA_ERR_HIP = 4           /* a HIP launch or event call failed (hipGetLastError) */
} kda_status;

typedef struct {
    int32_t layout;    /* a kda_layout value                                                 */
    int32_t batch;     /* B for BNSD/BSND; number of packed sequences for TND                 */
    int32_t seq_len;   /* S (stored length) for BNSD/BSND; T (total packed tokens) for TND    */
    int32_t n_qk;      /* query/key heads, 1 <= n_qk <= n_v                                   */
    int32_t n_v;       /* value heads, n_v % n_qk == 0 (GQA groups of n_v / n_qk)            */
    int32_t d_k;       /* head dim of q/k: 128 (FlashKDA README, 约束说明) or 64; equal to d_v  */
    int32_t d_v;       /* head dim of v and out: equal to d_k                                 */
    float scale;       /* output scale, typically d_k ** -0.5; must be finite                 */
    uint32_t flags;    /* KDA_QK_L2NORM | KDA_BETA_SIGMOID | KDA_SCALAR_GATE | KDA_RAW_GATE   */
} kda_shape;

/* Bytes of device workspace kda_chunk_fwd needs for `shape` (FlashKDA README, section 功能说明:
 * the per-chunk intermediates of the chunk equations, W, U, the q-side operand, the decayed
 * keys and the intra-chunk output, live here between the kernels of one call, with the
 * two-level scan's segment matrices and partial outputs).  Depends only on the shape.  Returns KDA_ERR_INVALID_ARG / KDA_ERR_UNSUPPORTED for shapes kda_chunk_fwd rejects. */
kda_status kda_chunk_fwd_workspace(const kda_shape* shape, size_t* bytes);

/* The chunked forward (prefill) of KDA.  Semantics: see the top of this file.
 *   q, k           bf16 in `layout`; raw rows when KDA_QK_L2NORM is set
 *   v              bf16 in `layout`
 *   g              fp32, same shape as v: activated natural-log decay per token and key channel;
 *                  with KDA_SCALAR_GATE, beta's shape: one decay per token and value head
 *   beta           bf16 (logits when KDA_BETA_SIGMOID is set)
 *   initial_state  fp32 [batch, n_v, d_v, d_k] or NULL (zero state); never written
 *   cu_seqlens     int32 [batch + 1] prefix sum: required for TND; for BNSD/BSND optional, then
 *                  batch row b holds cu_seqlens[b+1]-cu_seqlens[b] valid tokens at its start
 *   out            bf16, same shape and layout as v.  Rows past a row's valid length are
 *                  written with zeros (the FlashKDA README leaves them undefined)
 *   final_state    fp32 [batch, n_v, d_v, d_k] or NULL (not produced); must not overlap
 *                  initial_state
 *   workspace      device buffer of at least kda_chunk_fwd_workspace() bytes, 256-byte aligned
 * Buffers the call writes (out, final_state, the first kda_chunk_fwd_workspace() bytes of the
 * workspace) must not overlap each other or any input; overlap is KDA_ERR_INVALID_ARG.
 * Returns KDA_OK once the kernels are enqueued on `stream`. */
kda_status kda_chunk_fwd(const kda_shape* shape,
                         const void* q, const void* k, const void* v,
                         const float* g, const void* beta,
                         const float* initial_state, const int32_t* cu_seqlens,
                         void* out, float* final_state,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* kda_chunk_fwd with the gate activation fused (FlashKDA README, sections 功能说明 and 参数说明:
 * the operator activates the raw gate itself).  shape->flags must include KDA_RAW_GATE (and
 * not KDA_SCALAR_GATE: KDA_ERR_UNSUPPORTED); g_raw is bf16 with v's shape and layout; gate holds
 * A_log, dt_bias (device pointers, read only, not overlapping anything the call writes) and
 * lower_bound (see kda_raw_gate).  Every other argument, the workspace size and the errors are
 * those of kda_chunk_fwd; KDA_ERR_INVALID_ARG also for a NULL gate or parameter pointer, a
 * lower_bound outside [-5, 0], or the KDA_RAW_GATE flag missing (kda_chunk_fwd rejects the flag). */
kda_status kda_chunk_fwd_raw_gate(const kda_shape* shape,
                                  const void* q, const void* k, const void* v,
                                  const void* g_raw, const void* beta, const kda_raw_gate* gate,
                                  const float* initial_state, const int32_t* cu_seqlens,
                                  void* out, float* final_state,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Allocation-free variant of kda_chunk_fwd, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and kernels, with the workspace taken from a device array of
 * KDA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on, until the process
 * ends, instead of a caller buffer.  The caller still passes every input and output.
 * Limit: shapes whose kda_chunk_fwd_workspace() exceeds KDA_NOALLOC_SCRATCH_BYTES return
 * KDA_ERR_WORKSPACE and launch nothing (64 MiB holds, e.g., the 8K-token prefill with three
 * 128-dim heads).  The first call on a device looks up the array's device address
 * (hipGetSymbolAddress; a failure is KDA_ERR_HIP); no call allocates or frees device memory.
 * Every call on one GPU uses the same array: calls that overlap in time on one GPU (two
 * streams, two host threads) race and must be serialised by the caller.  Nothing in the array
 * needs to be cleared between calls. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_chunk_fwd_noalloc(const kda_shape* shape,
                                 const void* q, const void* k, const void* v,
                                 const float* g, const void* beta,
                                 const float* initial_state, const int32_t* cu_seqlens,
                                 void* out, float* final_state, hipStream_t stream);

/* Number of stages of one kda_chunk_fwd call and the name of each, one kernel per stage: the
 * intra-chunk kernel; then, when few (sequence, head) chains would leave the GPU idle through a
 * long sequential scan, the two-level scan's segment pass (every segment walked at once from a
 * zero state and from the identity), combine (segment entry states) and completion (outputs of
 * segments after the first) kernels; otherwise the one-level scan with outputs.  Stages the
 * plan does not enqueue are empty. */
int32_t kda_num_stages(void);
const char* kda_stage_name(int32_t stage);

/* The plan kda_chunk_fwd follows for `shape`, from the shape alone (nothing is launched):
 *   stage_mask  bit s set when stage s enqueues a kernel (the others are empty);
 *   segments    segments per sequence of the two-level scan, 1 for the one-level scan.
 * Either output pointer may be NULL.  Returns the status kda_chunk_fwd_workspace returns for
 * the same shape, and leaves the outputs untouched unless it is KDA_OK. */
kda_status kda_chunk_fwd_plan(const kda_shape* shape, uint32_t* stage_mask, int32_t* segments);

/* Profiling variant of kda_chunk_fwd: identical work.  For each stage s, the kernel's own
 * dispatch records stage_events[2s] when the kernel starts and stage_events[2s+1] when it ends
 * (hipExtLaunchKernel; no marker packet between the kernels), so hipEventElapsedTime of the pair
 * is the kernel's duration.  A stage with no kernel records its two events back to back on
 * `stream`.  n_stage_events must be at least 2 * kda_num_stages(); the caller creates the events.
 * Returns KDA_ERR_INVALID_ARG for a NULL array or too few events, launching nothing. */
kda_status kda_chunk_fwd_timed(const kda_shape* shape,
                               const void* q, const void* k, const void* v,
                               const float* g, const void* beta,
                               const float* initial_state, const int32_t* cu_seqlens,
                               void* out, float* final_state,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream,
                               hipEvent_t* stage_events, int32_t n_stage_events);

/* The kernels kda_chunk_fwd launches for `shape`, in launch order, as one NUL-terminated string:
 * each kernel's name with its template arguments (as in "kda_intra_kernel<0,128,2>"), separated
 * by ';'.  The choice follows from the shape alone (head dim, how many (sequence, head) chains
 * and chunk records it has, the gate form); nothing is launched.  `names` is caller memory of
 * `capacity` bytes.  Returns the status kda_chunk_fwd_workspace returns for the shape, or
 * KDA_ERR_INVALID_ARG when `names` is NULL or `capacity` is too small (then nothing is written).
 * (What the kernels compute: the FlashKDA README, section 功能说明; see the top of this file.) */
kda_status kda_chunk_fwd_plan_kernels(const kda_shape* shape, char* names, size_t capacity);

/* Every kernel variant compiled into the library: kda_num_kernel_variants() of them, named as
 * kda_chunk_fwd_plan_kernels names them; kda_kernel_variant(i) returns a static string for
 * 0 <= i < kda_num_kernel_variants() and NULL otherwise.  Each variant is one specialisation of
 * the same chunk method (FlashKDA README, section 功能说明) for a head dim, a gate form or a
 * launch shape. */
int32_t kda_num_kernel_variants(void);
const char* kda_kernel_variant(int32_t i);

/* Profiling variant of kda_chunk_fwd_raw_gate, with the stage events of kda_chunk_fwd_timed. */
kda_status kda_chunk_fwd_raw_gate_timed(const kda_shape* shape,
                                        const void* q, const void* k, const void* v,
                                        const void* g_raw, const void* beta,
                                        const kda_raw_gate* gate,
                                        const float* initial_state, const int32_t* cu_seqlens,
                                        void* out, float* final_state,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream,
                                        hipEvent_t* stage_events, int32_t n_stage_events);

/* Static string naming a status code ("KDA_OK", ...); "unknown kda_status" otherwise.  The codes
 * report the argument checks of the FlashKDA README, section 约束说明 (supported head dims,
 * layouts, head counts, cu_seqlens), made on the host before anything is launched. */
const char* kda_status_str(kda_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
