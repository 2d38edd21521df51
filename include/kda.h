/*
 * kda.h -- C ABI of libkda: the Kimi Delta Attention (KDA) forward pass on
 * AMD Instinct MI355X (gfx950), hand-written HIP.
 *
 * Pages cited (by title):
 *   [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer (KDA equations).
 *   [K3-memory]     "Kimi K3 Changed the Memory Math for Agentic AI Forever"
 *                   (hubwiz.com translation, "Kimi K3 混合线性注意力").
 *   [Kimi-Linear]   "Kimi Linear 最多砍掉 75% KV Cache：全注意力真要退场了吗？"
 *                   (ai.concitech.org).
 *
 * What the library computes.  For every sequence and head it keeps one state
 * S in R^{d_k x d_v} ([K3-explainer] §二.1) and applies, token by token,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 *
 * the KDA update of [K3-explainer] §四 (per-channel decay alpha_t in
 * [0,1]^{d_k}, scalar write strength beta_t) with the read of §二.1.  There is
 * no 1/sqrt(d_k) scale and no normalisation of q or k inside the library.
 *
 * Conventions shared by every entry point:
 *   - Gates are passed as natural logs: alpha_t[c] = exp(log_alpha[t,h,c]).
 *   - States are fp32 and stored transposed, M = S^T, shape [.., H, d_v, d_k]
 *     (row = value channel, contiguous along the key channel): the
 *     [batch, heads, value_dim, key_dim] layout [K3-memory] §3 reports.
 *   - q, k, v and out share one element type: KDA_DTYPE_F32 or KDA_DTYPE_BF16.
 *     log_alpha, beta and states are always fp32.
 *   - Every pointer is a device pointer to a dense row-major (contiguous)
 *     array, 16-byte aligned (beta and cu_seqlens: 4-byte aligned, they are
 *     read one element at a time).  The caller owns all memory; the library
 *     allocates nothing and keeps no state between calls.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *     stream).  They return as soon as the work is queued.  Arguments are
 *     validated on the host before any HIP call, so errors are reported
 *     without touching the device.  Calls on different streams may run
 *     concurrently if their outputs do not overlap.
 *   - Debug mode: with the environment variable KDA_DEBUG set (to anything
 *     but "0"; read at every call) each call also copies packed-sequence
 *     offsets to the host and rejects malformed ones (KDA_ERR_SHAPE) before
 *     launching, then waits for its stream and reports a failure of its
 *     kernels as KDA_ERR_LAUNCH, with a line on stderr naming the entry point.
 *     Calls are then synchronous; results are unchanged.
 *   - Supported now: d_k == d_v in {64, 128}, and for kda_chunk_fwd
 *     num_heads * d_k <= 8388607 (64 tokens of one tensor must span less
 *     than 2^31 bytes).  Other valid sizes return KDA_ERR_UNSUPPORTED.
 *
 * Gates: every alpha in [0, 1] is accepted, i.e. any log_alpha <= 0
 * including -inf (alpha = 0), by the prefill and decode entry points.  The
 * chunked prefill factorises each chunk's products with e^{+-(decay within a
 * 16-token block)}; a (sequence, head) in which some block decays by more than
 * 2^-100 in some channel (or has a -inf gate) is recomputed by a second
 * launch on the same stream, those chunks token by token in fp32 (exact, but
 * slower for such sequences).  NaN inputs propagate; they are not trapped.
 * kda_chunk_bwd accepts the same domain: a (sequence, head) in which some
 * 16-token block (counted from the sequence start) decays by more than 2^-100
 * in some channel, or has a -inf gate, has all its gradients recomputed token
 * by token in fp32 by a launch after the chunked ones (exact, much slower for
 * such sequences: it steps each 16-token block again once per token).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 7

/* Element type of q, k, v and out. */
enum kda_dtype { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 };

/* Status codes (0 = success, negative = error). */
enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = -2,       /* a size is negative or the sizes disagree */
    KDA_ERR_UNSUPPORTED = -3, /* valid request this build does not implement */
    KDA_ERR_ALIGN = -4,       /* a pointer is not aligned as documented above */
    KDA_ERR_ALIAS = -5,       /* an output overlaps an input it must not */
    KDA_ERR_DEVICE = -6,      /* the current device is not a gfx950 GPU */
    KDA_ERR_LAUNCH = -7,      /* the kernel launch failed (hipGetLastError) */
    KDA_ERR_SCRATCH = -8      /* needs more than KDA_SCRATCH_BYTES of fixed scratch */
};

/*
 * kda_chunk_fwd -- prefill: the KDA recurrence over whole sequences, computed
 * chunkwise: sequential from chunk to chunk, parallel inside a chunk
 * ([K3-explainer] §六.1), through the WY/UT representation of the chunk's
 * rank-one updates ([K3-explainer] §六.2).  The result equals the token-by-
 * token recurrence up to floating-point rounding; the chunk length (32) only
 * affects speed.
 *
 * Layout (dense, cu_seqlens == NULL): B = batch sequences of T = seq_len
 *   q, k       [B, T, H, d_k]   dtype
 *   v, out     [B, T, H, d_v]   dtype
 *   log_alpha  [B, T, H, d_k]   fp32
 *   beta       [B, T, H]        fp32
 *   initial_state, final_state  [B, H, d_v, d_k] fp32
 * Layout (packed, cu_seqlens != NULL): batch must be 1, T = total tokens, and
 *   N = num_seqs sequences are packed along T; sequence n covers tokens
 *   [cu_seqlens[n], cu_seqlens[n+1]).  cu_seqlens is a DEVICE int32 array of
 *   N + 1 entries with cu_seqlens[0] == 0, non-decreasing, cu_seqlens[N] == T.
 *   States are [N, H, d_v, d_k].  The host cannot read cu_seqlens without a
 *   sync, so its contents are not validated; the kernel clamps every offset to
 *   [0, T] (malformed offsets give wrong results, never out-of-bounds access).
 *
 * initial_state == NULL means zero initial states.  final_state == NULL means
 * the final states are not written.  final_state may be the same pointer as
 * initial_state (in-place update); any other overlap between outputs and
 * inputs returns KDA_ERR_ALIAS.  Empty sequences (and T == 0) are allowed:
 * their final state is their initial state.
 *
 * Returns KDA_OK or a kda_status error code.
 */
int kda_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                  const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                  void *out, float *final_state, int32_t batch, int32_t seq_len,
                  int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v, int32_t num_seqs,
                  int32_t dtype, hipStream_t stream);

/*
 * kda_chunk_fwd_snapshots -- kda_chunk_fwd that also keeps the recurrent state
 * at regular points of each sequence: restartable checkpoints and the state
 * blocks a prefix cache stores, since a KDA state depends on its whole prefix
 * and cannot be assembled from pieces the way paged KV blocks can
 * ([K3-memory] §5: one state snapshot every 20,000 tokens of a 1M-token run).
 *
 * Every argument shared with kda_chunk_fwd has the same meaning, layout and
 * rules.  In addition, for each sequence n (dense: each batch row) of length
 * L_n, the state after its first j * snapshot_every tokens, for
 * j = 1 .. floor(L_n / snapshot_every), is written (fp32, stored transposed
 * like every state) to entry base_n + j - 1 of
 *   snapshots  [num_snapshots, H, d_v, d_k] fp32,
 * where base_n = sum over m < n of floor(L_m / snapshot_every): the snapshots
 * of all sequences in sequence order, each sequence's in token order.  When
 * snapshot_every divides L_n, the last one equals that sequence's final state.
 *
 *   snapshot_every  > 0 (else KDA_ERR_SHAPE); this build supports multiples of
 *                   32 only (else KDA_ERR_UNSUPPORTED).
 *   num_snapshots   entries the buffer holds (>= 0).  Dense: must be at least
 *                   batch * floor(seq_len / snapshot_every) (else
 *                   KDA_ERR_SHAPE).  Packed: the host cannot read cu_seqlens,
 *                   so the count is not checked; entries at or beyond
 *                   num_snapshots are not written.
 *   snapshots       caller-owned device buffer, 16-byte aligned; may be NULL
 *                   only when num_snapshots == 0.  It must not overlap any
 *                   input, out or final_state (KDA_ERR_ALIAS).  Entries no
 *                   sequence reaches are left untouched.
 *
 * Returns KDA_OK or a kda_status error code.
 */
int kda_chunk_fwd_snapshots(const void *q, const void *k, const void *v, const float *log_alpha,
                            const float *beta, const float *initial_state,
                            const int32_t *cu_seqlens, void *out, float *final_state,
                            float *snapshots, int32_t snapshot_every, int32_t num_snapshots,
                            int32_t batch, int32_t seq_len, int32_t num_heads,
                            int32_t head_dim_k, int32_t head_dim_v, int32_t num_seqs,
                            int32_t dtype, hipStream_t stream);

/*
 * kda_chunk_fwd_scalar_gate -- kda_chunk_fwd with one gate per (token, head)
 * applied to every key channel: the Gated DeltaNet update that KDA refines
 * ([K3-explainer] §四: a scalar forget gate per head, where KDA has one per
 * channel),  S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T.
 * It is kda_chunk_fwd with log_alpha[t, h, c] = log_alpha[t, h] for every c.
 *
 * Every argument has the meaning, rules and layout of kda_chunk_fwd except
 *   log_alpha  [B, T, H] fp32 (dense) or [1, T, H] (packed), 4-byte aligned,
 * and the same gate domain (any log_alpha <= 0, -inf included).
 * Returns KDA_OK or a kda_status error code.
 */
int kda_chunk_fwd_scalar_gate(const void *q, const void *k, const void *v,
                              const float *log_alpha, const float *beta,
                              const float *initial_state, const int32_t *cu_seqlens, void *out,
                              float *final_state, int32_t batch, int32_t seq_len,
                              int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                              int32_t num_seqs, int32_t dtype, hipStream_t stream);

/*
 * kda_chunk_fwd_segmented -- kda_chunk_fwd of ONE long sequence (batch 1, no
 * cu_seqlens) split into segments that run side by side, for the long-context
 * prefill ([Kimi-Linear] Fig. 7: batch 1 up to 1M tokens) where a few heads
 * leave most of the GPU idle while one chain of chunks runs in order.
 *
 * A run of chunks maps its entering state affinely, S_out = P S_in + R, with P
 * the product of the chunks' transitions ([K3-explainer] §六.2: a chunk's
 * rank-one updates collapse into one transition matrix, P = D - K W^T).  The
 * call (1) computes every segment's R (the segment from S = 0) and P (from
 * S = I with zero values) in one launch each, all segments and heads in
 * parallel, (2) folds the maps in segment order to get each segment's true
 * entering state, and (3) reruns every segment from that state, writing out.
 * The result is kda_chunk_fwd's up to rounding order, at about three times
 * its arithmetic and reads.
 *
 * Arguments as kda_chunk_fwd with batch = 1 and cu_seqlens = NULL, plus
 *   num_segments     >= 1 (else KDA_ERR_SHAPE): the requested split.  Segments
 *                    hold L = 32 * ceil(ceil(seq_len / num_segments) / 32)
 *                    tokens (the last one the rest), so ceil(seq_len / L) of
 *                    them run; when that is 1 the call is kda_chunk_fwd and
 *                    the workspace is not touched.  It is kda_chunk_fwd too
 *                    (workspace untouched; its size is still checked) when the
 *                    plain prefill's own workgroups, one per head and d_v
 *                    slice (d_k / 64 slices for bf16, d_k / 16 for fp32),
 *                    already fill a third of the device's compute units: the
 *                    segmented call does about three times the work and
 *                    cannot win there.
 *   workspace        caller-owned device scratch, 256-byte aligned (else
 *                    KDA_ERR_ALIGN), of at least
 *                    kda_chunk_fwd_segmented_workspace_size(seq_len,
 *                    num_heads, head_dim_k, num_segments) bytes (else
 *                    KDA_ERR_SHAPE); NULL (KDA_ERR_NULL) only where it is not
 *                    touched.  It must not overlap any argument array
 *                    (KDA_ERR_ALIAS); its contents on return are unspecified.
 *   workspace_bytes  its size in bytes.
 * Calls that share a workspace must not run concurrently.
 * Returns KDA_OK or a kda_status error code.
 */
int kda_chunk_fwd_segmented(const void *q, const void *k, const void *v, const float *log_alpha,
                            const float *beta, const float *initial_state, void *out,
                            float *final_state, int32_t seq_len, int32_t num_heads,
                            int32_t head_dim_k, int32_t head_dim_v, int32_t num_segments,
                            int32_t dtype, void *workspace, int64_t workspace_bytes,
                            hipStream_t stream);

/*
 * Bytes of workspace kda_chunk_fwd_segmented needs for these sizes: the
 * segment offsets (padded to 256 bytes) and four fp32 arrays of
 * n_seg * num_heads * head_dim^2 (two maps, entering and leaving states).
 * -1 for seq_len < 0, num_heads < 0, num_segments < 1 or head_dim not 64/128.
 * Host only; touches no device.
 */
int64_t kda_chunk_fwd_segmented_workspace_size(int32_t seq_len, int32_t num_heads,
                                               int32_t head_dim, int32_t num_segments);

/*
 * kda_chunk_fwd_segmented_noalloc -- kda_chunk_fwd_segmented for callers that
 * cannot allocate device memory (code under stream capture, tight serving
 * loops, hosts that forbid allocation): its workspace is a fixed buffer of
 * KDA_SCRATCH_BYTES inside the library, one per GPU, reserved when the
 * library's code is loaded on that GPU and held until the process ends.  The
 * call allocates nothing and frees nothing.
 *
 * Arguments, rules and result are those of kda_chunk_fwd_segmented without
 * the workspace.  Requests whose workspace
 * (kda_chunk_fwd_segmented_workspace_size) exceeds KDA_SCRATCH_BYTES return
 * KDA_ERR_SCRATCH before any device work; with one segment the call is
 * kda_chunk_fwd and the scratch is not touched.  Every call on one GPU uses
 * that GPU's one buffer: calls that may overlap in time on the same GPU (other
 * streams, other host threads) race and give undefined results; serialise them.
 * Returns KDA_OK or a kda_status error code.
 */
#define KDA_SCRATCH_BYTES (64u << 20) /* 64 MiB: e.g. 4 segments x 32 heads at d = 128 */
int kda_chunk_fwd_segmented_noalloc(const void *q, const void *k, const void *v,
                                    const float *log_alpha, const float *beta,
                                    const float *initial_state, void *out, float *final_state,
                                    int32_t seq_len, int32_t num_heads, int32_t head_dim_k,
                                    int32_t head_dim_v, int32_t num_segments, int32_t dtype,
                                    hipStream_t stream);

/*
 * kda_chunk_bwd -- gradients of kda_chunk_fwd: given dL/d out and dL/d
 * final_state, the gradients with respect to q, k, v, log_alpha, beta and
 * initial_state, for training.  The pages give training as the reason for the
 * chunkwise form ([Kimi-Linear], the section on KDA's per-channel forgetting:
 * training runs as matrix products instead of a token-serial RNN) but state
 * no gradient; this is the exact derivative of the recurrence of kda_chunk_fwd
 * (up to rounding), per chunk of 16 tokens, in three launches on `stream`:
 * (1) a forward pass writes every chunk's entering state to the workspace (bf16
 * at d 64 or 128 and fp32 at d 64: the prefill kernel in a states-only mode,
 * 32 tokens per step; fp32 at d 128: 16-token steps at the start of launch 2);
 * (2) two workgroups per (sequence, head), one per half of the value columns
 * (four at d 128 when four per pair fit on the device's compute units; one
 * where launch 2 also computes the states), carry dL/dS backwards over the
 * chunks, which needs no forward state, and write the gradient at every
 * chunk's end to the workspace; (3) one workgroup per (chunk, head) forms all
 * other gradients of its chunk from those two states.
 *
 * Inputs: q, k, v, log_alpha, beta, initial_state, cu_seqlens, batch, seq_len,
 * num_heads, head_dim_k, head_dim_v, num_seqs and dtype exactly as given to
 * kda_chunk_fwd (same layouts and rules; initial_state may be NULL = zeros), and
 *   d_out          [B, T, H, d_v] dtype: dL/d out.
 *   d_final_state  [N, H, d_v, d_k] fp32 (stored transposed like every
 *                  state), or NULL for zero.
 * Outputs (caller-owned, written completely for every token of every sequence):
 *   dq, dk         [B, T, H, d_k] dtype;  dv [B, T, H, d_v] dtype;
 *   dlog_alpha     [B, T, H, d_k] fp32;   dbeta [B, T, H] fp32 (4-byte aligned);
 *   d_initial_state [N, H, d_v, d_k] fp32, or NULL (not written).
 * workspace: caller-owned device scratch, 16-byte aligned, of at least
 * kda_chunk_bwd_workspace_size(B * T, N, H, d_k) bytes (else KDA_ERR_SHAPE;
 * NULL: KDA_ERR_NULL), holding each 16-token chunk's entering state and the
 * gradient at its end (both in the input dtype) and the flag words; contents on return are
 * unspecified.  No output may overlap an input, another output or
 * the workspace (KDA_ERR_ALIAS).  Supported: d_k == d_v in {64, 128}, fp32 or
 * bf16 (bf16 inputs: bf16 matrix products with fp32 accumulation; fp32 inputs:
 * fp32 throughout).  Gates: any log_alpha <= 0, -inf included, as stated at
 * the top of this file; a first launch marks the (sequence, head) pairs
 * outside the chunked range in the workspace's flag words and a last one
 * recomputes them.  Returns KDA_OK or a kda_status error code.
 */
int kda_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                  const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                  const void *d_out, const float *d_final_state, void *dq, void *dk, void *dv,
                  float *dlog_alpha, float *dbeta, float *d_initial_state, int32_t batch,
                  int32_t seq_len, int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                  int32_t num_seqs, int32_t dtype, void *workspace, int64_t workspace_bytes,
                  hipStream_t stream);

/*
 * Bytes of workspace kda_chunk_bwd needs for total_tokens = B * T tokens in
 * num_seqs sequences: 2 * (total_tokens / 16 + num_seqs + 1) * num_heads *
 * head_dim^2 * 4 (two regions of one state per 16-token slot and head) +
 * 16 * num_seqs * num_heads * 4 (the out-of-range flag words).  -1 for
 * negative sizes or head_dim not 64/128.  Host only.
 */
int64_t kda_chunk_bwd_workspace_size(int32_t total_tokens, int32_t num_seqs, int32_t num_heads,
                                     int32_t head_dim);

/*
 * kda_decode_step -- one new token per session against a stored state: the
 * fixed-size read and in-place update that decoding performs instead of
 * appending to a cache ([K3-memory] §2; [Kimi-Linear], the decode discussion).
 * In predict/correct form ([K3-explainer] §三, §四), per session b and head h:
 *     S' = Diag(alpha) S,  e = v - S'^T k,  S <- S' + beta k e^T,  o = S^T q.
 *
 * Layout:
 *   q, k       [B, H, d_k]   dtype
 *   v, out     [B, H, d_v]   dtype
 *   log_alpha  [B, H, d_k]   fp32
 *   beta       [B, H]        fp32
 *   state      [B, H, d_v, d_k] fp32, read and updated in place.
 * out must not overlap any input or the state (KDA_ERR_ALIAS).  B == 0 is a
 * no-op.  Returns KDA_OK or a kda_status error code.
 */
int kda_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                    const float *beta, float *state, void *out, int32_t batch,
                    int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v, int32_t dtype,
                    hipStream_t stream);

/*
 * kda_decode_step_scalar_gate -- kda_decode_step with one gate per (session,
 * head) applied to every key channel (the Gated DeltaNet update, as for
 * kda_chunk_fwd_scalar_gate).  Arguments as kda_decode_step except
 *   log_alpha  [B, H] fp32, 4-byte aligned.
 * Returns KDA_OK or a kda_status error code.
 */
int kda_decode_step_scalar_gate(const void *q, const void *k, const void *v,
                                const float *log_alpha, const float *beta, float *state,
                                void *out, int32_t batch, int32_t num_heads, int32_t head_dim_k,
                                int32_t head_dim_v, int32_t dtype, hipStream_t stream);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char *kda_status_string(int status);

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
