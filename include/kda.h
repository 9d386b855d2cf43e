/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention operator.
 *
 * The operator is the per-head KDA recurrence with its readout,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                      (read after the update)
 *
 * with alpha_t = exp(log_alpha_t) (one decay per key channel) and beta_t a
 * scalar write strength.  The state equation is the one stated in
 * "Kimi K3 核心算子拆解" (devpress.csdn.net) section 2.2 and in
 * "把注意力换成一块「会遗忘的内存」" (jokeuncle.github.io) section "第四步";
 * the readout after the update in "Kimi K3 技术报告解读" (marsggbo.github.io)
 * section 3.2.  Two entry points share these semantics: a chunkwise-parallel
 * prefill over whole sequences and a one-token decode step that updates the
 * state in place ("把注意力换成一块「会遗忘的内存」", section "层的实现":
 * chunked path for training / prefill, recurrent path for decode).
 *
 * Common contract
 *   - Head dimension: dk == dv == 128 (any other value -> KDA_ERR_BAD_SHAPE).
 *   - q, k, v are in `in_dtype` (KDA_BF16 or KDA_F32); log_alpha, beta, the
 *     states and o are float32.  log_alpha must lie in [-5, 0] (the lower-
 *     bounded decay of "Kimi K3 技术报告解读" section 3.5); beta is used as
 *     given (no clamping).  q and k are used as given (the caller normalises);
 *     there is no query scale.  Values outside the log_alpha contract give
 *     unspecified (possibly non-finite) results but never out-of-bounds
 *     memory accesses.
 *   - All tensor pointers are DEVICE pointers owned by the caller, which
 *     allocates every buffer (including the workspace).  The library
 *     allocates no memory, keeps no mutable global state (apart from the
 *     scratch array of kda_chunk_fwd_noalloc and the per-device second
 *     stream of kda_chunk_bwd), never synchronises the host, and enqueues
 *     its kernels on `stream` (0 = the null stream), which must belong to
 *     the current device (the one every pointer refers to); kda_chunk_bwd
 *     and the sequence-parallel path of kda_chunk_fwd also run one pass on
 *     that second stream, ordered against `stream` by events (see
 *     kda_chunk_bwd).
 *   - Every argument is validated before anything is enqueued; on error the
 *     call returns a non-zero kda_status and has no effect.  Faults raised by
 *     the device asynchronously surface at the caller's next synchronisation.
 *   - Tensor pointers must be 16-byte aligned (beta and cu_seqlens 4-byte).
 *   - Results are deterministic: no atomics; the same inputs and launch give
 *     the same bits.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 4

/* Largest head count any entry point accepts: the kernels address a chunk's
 * token rows (up to 32 rows of H * 128 fp32 values) with 32-bit byte
 * offsets, which stay below 2^31 for H <= 65536.  Larger H ->
 * KDA_ERR_TOO_LARGE (the workspace queries return 0). */
#define KDA_MAX_HEADS 65536

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1,   /* a required pointer is NULL */
    KDA_ERR_BAD_SHAPE = 2,      /* dk/dv not 128, negative sizes, H < 1 */
    KDA_ERR_BAD_DTYPE = 3,      /* in_dtype is not KDA_BF16 / KDA_F32 */
    KDA_ERR_MISALIGNED = 4,     /* pointer alignment contract violated */
    KDA_ERR_ALIASING = 5,       /* an output overlaps an input illegally */
    KDA_ERR_WORKSPACE = 6,      /* workspace missing or too small */
    KDA_ERR_TOO_LARGE = 7,      /* sizes beyond the launch limits (or H > KDA_MAX_HEADS) */
    KDA_ERR_HIP = 8             /* the kernel launch itself failed */
} kda_status;

typedef enum kda_dtype {
    KDA_BF16 = 0,
    KDA_F32 = 1
} kda_dtype;

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* kda_status_str(int status);

/*
 * Workspace size in bytes for kda_chunk_fwd with these sizes (0 when none
 * is used).  `varlen` != 0 when cu_seqlens will be passed.
 *   varlen: a longest-first order of the sequences (n_seqs int32); the
 *       workspace is then required.
 *   equal lengths: when n_seqs * H is small (at most 64 (sequence, head)
 *       pairs) and T is long, the sequence-parallel path cuts every
 *       sequence into P = min(256 / (n_seqs * H), T / 2048) segments, if
 *       that is at least 3 (every segment a whole number of 32-token chunks
 *       but the last; the first and the last 1.6 to 2.1 times as long as
 *       the others), and needs (3 * P - 4) * n_seqs * H * 64 KiB (the
 *       transition and local
 *       final state of each of the P - 2 middle segments, the incoming state
 *       of each of the P - 1 later segments and the first segment's final
 *       state).  That workspace is optional: without it (NULL or smaller),
 *       the sequential path runs instead, with the same result up to
 *       rounding.
 * Returns 0 for invalid sizes as well; kda_chunk_fwd then reports the real
 * error.
 */
size_t kda_chunk_fwd_workspace_bytes(int32_t n_seqs, int64_t T, int32_t H,
                                     int32_t dk, int32_t dv, int varlen);

/*
 * Chunkwise prefill: runs the recurrence over whole sequences and returns
 * every o_t and, optionally, each sequence's final state.  With equal-length
 * sequences and few (sequence, head) pairs, the sequence-parallel path
 * (when its workspace is given) runs the first segment of each sequence
 * from S0 (writing its o) beside the middle segments, which run as
 * independent chains from zero and from the identity (their local final
 * states and d_k x d_k transitions); a merge through the transitions gives
 * the incoming state of every later segment, from which the middle segments
 * run again and the last one runs once, writing their o; "Kimi K3 技术报告解读"
 * section 7.3 describes this within-GPU split.  The chunkwise
 * evaluation (cumulative in-chunk log-decay, k+ = k e^{g}, k- = k e^{-g},
 * the strictly lower-triangular A_tj = beta_t k+_t . k-_j solved by forward
 * substitution, O = Q+ S + Tril(Q+ K-^T) U and the state hand-off
 * S <- Diag(e^{g_C}) S + K_end^T U) is the derivation of
 * "尝试对Kimi KDA的数学推导&算子实现分析" (hjcheng0602.cn), eqs. (8)-(66); it
 * gives the recurrence's result up to rounding.
 *
 * Layout (row-major, last index fastest):
 *   cu_seqlens == NULL: n_seqs sequences of T tokens each;
 *       q, k, log_alpha [n_seqs, T, H, dk]; v, o [n_seqs, T, H, dv];
 *       beta [n_seqs, T, H].
 *   cu_seqlens != NULL: n_seqs sequences packed along one token axis of
 *       length T (the total); q, k, log_alpha [T, H, dk]; v, o [T, H, dv];
 *       beta [T, H]; cu_seqlens int32 [n_seqs + 1] (device) with
 *       cu_seqlens[0] = 0, non-decreasing, cu_seqlens[n_seqs] = T.  The
 *       device clamps each range into [0, T] (a malformed table gives wrong
 *       rows, never an out-of-bounds access).
 *   S0  : [n_seqs, H, dk, dv] float32 initial states, or NULL for zeros.
 *   S_T : [n_seqs, H, dk, dv] float32 final states, or NULL to skip.  S_T
 *         may be the same pointer as S0 (in-place carry); any other overlap
 *         with an input is rejected.
 *   o   : must not overlap any input or S_T.
 *   workspace: kda_chunk_fwd_workspace_bytes(...) bytes of device memory,
 *         16-byte aligned, overlapping no other argument (required for
 *         packed batches when that size is not 0, optional otherwise; see
 *         above); contents need no initialisation and are clobbered.
 * Numerics: fp32 accumulation throughout.  With KDA_F32 inputs every
 * product runs on fp32 matrix cores.  With KDA_BF16 inputs the products run
 * on 16-bit matrix cores, with operands whose single rounding would exceed
 * the 2e-3 budget split into hi + lo bf16 pairs; which operands are split
 * depends on the kernel the call selects:
 *   - n_seqs * H >= 256 (sequence, head) pairs: one workgroup per pair, every
 *     product on bf16 (fp32's exponent range); the state is split in
 *     K+ S and Q+ S.
 *   - fewer pairs: two workgroups per pair (64 value columns each); the
 *     scaled state enters K+ S rounded once to bf16, and Q+ S runs on fp16
 *     matrix cores with q e^{g} and the (unscaled) state rounded once to
 *     fp16, which is more precise (11-bit significands) but has fp16's
 *     range: every element of q and every state entry must stay below 65504
 *     in magnitude (larger ones give inf in o), and state entries below
 *     about 6e-5 lose relative precision in that product (fp16 subnormals),
 *     which matters only when the whole output is that small.  q normalised
 *     by the caller meets the first condition; for the state it means |v|
 *     and |S0| of ordinary size (the tests cover value scales from 1e-4 to
 *     3e4 within 2e-3).
 *   The two plans round differently, so the same sequence can give results
 *   that differ in the last bits depending on how many (sequence, head)
 *   pairs share the call; both stay within 2e-3 of the exact recurrence.
 *   On the sequence-parallel path the first and the last segment of every
 *   sequence run on the two-workgroup plan and the middle segments on the
 *   one-workgroup plan.
 * The chunk form carries per-channel factors of up to e^{+-80}: in a key
 * channel whose decay sits at the bound (log_alpha = -5 for 16 tokens) the
 * state enters the products scaled by e^{-80}, so its entries below about
 * 1e-3 become bf16 subnormals there; the terms they feed are below 5e-6 in
 * absolute value whatever the scale of the rest of the state.
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v, int in_dtype,
                  const float* log_alpha, const float* beta, const float* S0,
                  const int32_t* cu_seqlens, int32_t n_seqs, int64_t T,
                  int32_t H, int32_t dk, int32_t dv, float* o, float* S_T,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, the same kernels and results.
 * The workspace comes from a scratch array of KDA_NOALLOC_SCRATCH_BYTES in
 * the library's device memory (one per GPU, held until the process ends;
 * its address is looked up on a device's first call).  That size covers
 * every case kda_chunk_fwd_workspace_bytes can report (a longest-first
 * order of up to 4096 sequences, or the sequence-parallel path's at most
 * 3 * 256 - 4 segment states); a larger need returns KDA_ERR_TOO_LARGE.  The call
 * allocates nothing.  All calls on one GPU share its scratch array and it
 * keeps the last call's contents: calls that may overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (48u * 1024u * 1024u)
int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, int in_dtype,
                          const float* log_alpha, const float* beta, const float* S0,
                          const int32_t* cu_seqlens, int32_t n_seqs, int64_t T,
                          int32_t H, int32_t dk, int32_t dv, float* o, float* S_T,
                          hipStream_t stream);

/*
 * One decode step for B independent requests, updating their states in
 * place: per (request, head) the state is decayed, corrected by the rank-1
 * erase computed from the decayed state, written, and read after the update
 * (the three-step method of "Kimi K3 核心算子拆解" section 2.3).  The state
 * is streamed once: the readout uses
 *     o = (Diag(alpha) S)^T q + beta (q . k) (v - x),  x = k^T Diag(alpha) S,
 * which equals S_t^T q_t for the updated state.
 *
 * Layout: q, k, log_alpha [B, H, dk]; v [B, H, dv]; beta [B, H];
 *         S [B, H, dk, dv] float32, read and overwritten in place;
 *         o [B, H, dv] float32 (must not overlap any input or S).
 */
int kda_decode_step(const void* q, const void* k, const void* v, int in_dtype,
                    const float* log_alpha, const float* beta, float* S,
                    int32_t B, int32_t H, int32_t dk, int32_t dv, float* o,
                    hipStream_t stream);

/*
 * Multi-token recurrent decode with on-chip replay.  For each (request,
 * head) the state S is loaded once; the first n_replay[b] of the Tr replay
 * tokens are applied (state only, no outputs); then the T tokens are applied
 * one by one, each emitting o_t = S_t^T q_t (read after its update); finally
 * the state is written back either after the replay (commit == 0) or after
 * all tokens (commit != 0).  Each token is the same step as kda_decode_step.
 *   - decode of up to 64 tokens per request: Tr = 0, commit = 1 (the fused
 *     recurrent path of "把注意力换成一块「会遗忘的内存」", section
 *     "层的实现:低秩门控与两条执行路径");
 *   - speculative decoding: the replay tokens are the previous step's drafts
 *     with n_replay the accepted counts, the T tokens are the new drafts and
 *     commit = 0, so the state holds exactly the accepted tokens and only the
 *     drafts' inputs are kept between steps ("Kimi K3 技术报告解读"
 *     section 9).
 *
 * Layout: q, k, log_alpha [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H];
 *         rq, rk, rlog_alpha [B, Tr, H, dk]; rv [B, Tr, H, dv];
 *         rbeta [B, Tr, H] (all may be NULL when Tr == 0);
 *         n_replay int32 [B] on the device, each clamped into [0, Tr], or
 *         NULL for all Tr;
 *         S [B, H, dk, dv] float32, read and overwritten in place;
 *         o [B, T, H, dv] float32 (must not overlap any input or S).
 * Sizes: 0 <= T <= 64, 0 <= Tr <= 64.  Replay and new tokens share in_dtype.
 * Numerics: fp32 throughout.  With T + Tr <= 2 the kernel is the one of
 * kda_decode_step (T = 1, Tr = 0 gives its bits exactly); with T + Tr >= 3
 * a form with two workgroups per compute unit runs, whose sums over key
 * rows are formed in a different order, so results agree with the other
 * form to fp32 rounding, not bitwise.  Both are deterministic.
 */
int kda_recurrent_fwd(const void* q, const void* k, const void* v, int in_dtype,
                      const float* log_alpha, const float* beta, const void* rq,
                      const void* rk, const void* rv, const float* rlog_alpha,
                      const float* rbeta, const int32_t* n_replay, float* S, int32_t B,
                      int32_t T, int32_t Tr, int32_t H, int32_t dk, int32_t dv, int commit,
                      float* o, hipStream_t stream);

/*
 * Layer prologue: from the projected (pre-convolution) q, k, v and the gate
 * pre-activations to the recurrence's inputs.  Per token t, head h, channel c:
 *   y = sum_{j<4} w[j] x_{t-3+j}  (causal depthwise convolution of width 4;
 *       x_{t<0} from the conv cache, or zeros when it is NULL)
 *   q = l2norm(silu(y_q)), k = l2norm(silu(y_k)), v = silu(y_v),
 *   log_alpha = -5 sigmoid(a), beta = sigmoid(b),
 * silu(z) = z sigmoid(z), l2norm over the head's dk channels with eps 1e-6
 * ("Kimi K3 四个核心模块的公式与真实张量流" section 1.2; "Kimi K3 核心算子拆解"
 * section 2.6; "Kimi K3 技术报告解读" section 3.3).  The cache then holds each
 * sequence's last three raw inputs (older entries shift in for sequences
 * shorter than three tokens).
 *
 * Layout: q_raw, k_raw, q, k, a [rows, H, dk]; v_raw, v [rows, H, dk];
 *   b, beta [rows, H]; log_alpha [rows, H, dk] float32, with rows = n_seqs * T
 *   (equal lengths, cu_seqlens NULL) or T (packed, cu_seqlens [n_seqs + 1]
 *   as in kda_chunk_fwd).  q_raw, k_raw, v_raw and q, k, v are in_dtype;
 *   a, b float32.  conv_w float32 [3, H, dk, 4] (q, k, v; tap 0 applies to
 *   t-3).  conv_cache float32 [n_seqs, 3, 3, H, dk] (tensor, tap t-3..t-1)
 *   read and updated in place, or NULL.  Outputs must not overlap inputs
 *   (the convolution reads neighbouring tokens).  dk = dv = 128.
 */
int kda_prologue(const void* q_raw, const void* k_raw, const void* v_raw, int in_dtype,
                 const float* conv_w, float* conv_cache, const float* a, const float* b,
                 const int32_t* cu_seqlens, int32_t n_seqs, int64_t T, int32_t H, int32_t dk,
                 void* q, void* k, void* v, float* log_alpha, float* beta,
                 hipStream_t stream);

/*
 * Layer epilogue: out = o / sqrt(mean_c o_c^2 + 1e-6) * w * sigmoid(g) over
 * each (row, head)'s 128 channels: RMSNorm with a per-channel weight and the
 * sigmoid output gate ("把注意力换成一块「会遗忘的内存」" section
 * "层的实现:低秩门控与两条执行路径"; "Kimi K3 四个核心模块的公式与真实张量流"
 * section 1.4).  o, g, out float32 [rows, H, dv]; w float32 [dv].  out may
 * be o itself; no other overlap.
 */
int kda_epilogue(const float* o, const float* g, const float* w, int64_t rows, int32_t H,
                 int32_t dv, float* out, hipStream_t stream);

/*
 * Workspace size in bytes for kda_chunk_bwd (always required).  It holds,
 * per 32-token chunk and head, the state at the chunk's start and the state
 * gradient at its end (2 * 64 KiB) and the chunk's matrices (three 32 x 32,
 * three 128 x 32 and one 128-vector of fp32: 61952 bytes), and per token and
 * head three fp32 value rows (1536 bytes), for:
 *   packed batches (varlen != 0): every chunk, slots = T / 32 + n_seqs
 *     chunk slots and T tokens;
 *   equal lengths (varlen == 0): one window of every sequence.  The backward
 *     runs each sequence in windows of W chunks, the last window first
 *     (W = KDA_BWD_WINDOW / 32, or all chunks when T is no longer): n_seqs * W
 *     slots and n_seqs * 32 W tokens, plus the state at the start of every
 *     window after the first and one state gradient per (sequence, head)
 *     carried between windows (n_seqs * H * 64 KiB each).
 * 0 for invalid sizes.
 */
#define KDA_BWD_WINDOW 2048
size_t kda_chunk_bwd_workspace_bytes(int32_t n_seqs, int64_t T, int32_t H,
                                     int32_t dk, int32_t dv, int varlen);

/*
 * Workspace size in bytes for kda_chunk_bwd on an equal-length batch with
 * windows of window_tokens tokens, rounded up to 32 times a power of two (a
 * window at least as long as T: one window, the largest and fastest
 * layout).  kda_chunk_bwd uses the longest window whose layout fits in the
 * workspace it is given: one window if it fits, else the longest
 * power-of-two number of chunks.  At most 65536 windows per sequence: a
 * window so short that more would be needed gives 0 here (and such a
 * workspace KDA_ERR_WORKSPACE).  0 for invalid sizes.
 */
size_t kda_chunk_bwd_workspace_bytes_window(int32_t n_seqs, int64_t T, int32_t H,
                                            int32_t dk, int32_t dv, int64_t window_tokens);

/*
 * Backward pass of kda_chunk_fwd: the gradients of a scalar loss L with
 * respect to every input, given grad_o = dL/do and grad_S_T = dL/dS_T.
 * Needed for training ("尝试对Kimi KDA的数学推导&算子实现分析" lists the
 * chunk backward kernel beside the forward); the pages give no formula, so
 * it is the reverse-mode derivative of the same chunk form (eqs. (51)-(66)
 * of that page), evaluated chunk by chunk: a forward pass storing each
 * chunk's incoming state, the chunk matrices, one backward walk per
 * (sequence, head) carrying dL/dS, and the per-chunk gradients.
 *
 * Inputs q, k, v, log_alpha, beta, S0, cu_seqlens, n_seqs, T, H, dk, dv and
 * in_dtype exactly as for the kda_chunk_fwd call being differentiated.
 *   grad_o   : float32 like o.
 *   grad_S_T : float32 [n_seqs, H, dk, dv], or NULL for zero.
 * Outputs (float32, overwritten, all token rows of every sequence):
 *   grad_q, grad_k, grad_log_alpha like q; grad_v like v; grad_beta like
 *   beta; grad_S0 [n_seqs, H, dk, dv] or NULL to skip (it may be the same
 *   pointer as grad_S_T; any other overlap between an output, an input or
 *   the workspace is rejected).
 *   workspace: kda_chunk_bwd_workspace_bytes(...) bytes or more (equal
 *   lengths: any size kda_chunk_bwd_workspace_bytes_window reports),
 *   16-byte aligned, contents clobbered.
 * Equal-length batches run window by window (see the workspace queries):
 * the forward pass first walks the windows to store the state at each
 * window's start, then each window, last first, recomputes its chunk
 * states and runs the backward passes over it.  Every window after the
 * first costs one more launch of the forward chain over the window before
 * it.  Every window length evaluates the same chunk arithmetic in the same
 * order (the carried state and state gradient pass through memory in fp32
 * unchanged), so the gradients do not depend on it.
 * Numerics: fp32 accumulation throughout.  With KDA_F32 inputs every
 * product runs on fp32 matrix cores; with KDA_BF16 inputs the products of
 * the state-gradient walk and of the per-chunk gradients use split (hi + lo)
 * bf16 operands, and the states come from the same kernel as kda_chunk_fwd
 * (its split-bf16 rounding).  Deterministic: no atomics.
 * Streams: the chunk-matrix pass reads only the inputs, so it runs beside
 * the forward pass on a second stream of the current device (created by the
 * library on the first call, default priority, never destroyed).  Events
 * order it: each such pass starts after everything enqueued on `stream`
 * before it (for the first, before the call), and the walk that reads it
 * waits for it, so all of the call's work is complete before anything
 * enqueued on `stream` after the call runs.  Under HIP graph capture of
 * `stream` the second stream joins the capture the same way.  If the
 * second stream cannot be created every pass runs on `stream`.  Calls on
 * one device serialise their enqueueing on a lock; their work on the
 * second stream runs in call order.  A call that fails with KDA_ERR_HIP
 * after work reached the second stream still makes `stream` wait for that
 * work before it returns, so the buffers may be released in stream order
 * as after a successful call (their contents are then unspecified).
 */
int kda_chunk_bwd(const void* q, const void* k, const void* v, int in_dtype,
                  const float* log_alpha, const float* beta, const float* S0,
                  const int32_t* cu_seqlens, int32_t n_seqs, int64_t T,
                  int32_t H, int32_t dk, int32_t dv, const float* grad_o,
                  const float* grad_S_T, float* grad_q, float* grad_k,
                  float* grad_v, float* grad_log_alpha, float* grad_beta,
                  float* grad_S0, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
