// kda_internal.h -- host-side launch functions shared by the library's
// translation units (not part of the public ABI; see include/kda.h).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kda {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;

// Queue one decode step for `units` = B * H (session, head) pairs whose
// arguments were already validated.  Returns 0, or -1 if the launch failed.
int launch_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                       const float *beta, float *state, void *out, int64_t units, int head_dim,
                       int dtype, int scalar_gate, hipStream_t stream);

// Queue the chunked prefill.  Dense when cu_seqlens == NULL (num_seqs = batch
// sequences of seq_len tokens each); packed otherwise (batch == 1).  With
// snapshots != NULL the state after every snapshot_every tokens (a positive
// multiple of 32) of each sequence is also written, at most num_snapshots
// entries.  scalar_gate != 0: log_alpha holds one gate per (token, head),
// [T, H], applied to every key channel (the Gated DeltaNet gate); otherwise
// [T, H, d_k].  out == NULL (channel gates only): final states only.
// init_identity != 0 (then v, out, snapshots and initial_state are NULL and
// the gates are per channel): every sequence starts from S = I with zero
// values, so its final state is its state transition (stored transposed).
// Arguments are already validated.  Returns 0, or -1 if the launch failed or
// the combination is not one of these.
int launch_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                     const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                     void *out, float *final_state, float *snapshots, int32_t snapshot_every,
                     int32_t num_snapshots, int32_t num_seqs, int32_t seq_len,
                     int32_t total_tokens, int32_t num_heads, int head_dim, int dtype,
                     int scalar_gate, int init_identity, hipStream_t stream);

// The state entering every 16-token block of every sequence, written to
// `states` as the chunked backward's checkpoints (slot tbeg / 16 + n + j for
// block j of sequence n, [slot][H][d_v][d_k]; chunk_bwd_workspace_floats(...)
// floats), computed by the prefill kernel without outputs.  Sequences as for
// launch_chunk_fwd.  bf16 at head_dim 64 or 128, fp32 at 64.  far_flags, if
// not NULL, receives the 16 flag words of every (sequence, head) that
// launch_bwd_far_detect would write (word 0 nonzero where a 16-token block
// decays beyond 2^-100 in some channel or has a -inf / NaN gate, the others
// 0).  Returns 0, or -1 if the launch failed or the configuration is not one
// of these.
int launch_chunk_states(const void *q, const void *k, const void *v, const float *log_alpha,
                        const float *beta, const float *initial_state,
                        const int32_t *cu_seqlens, float *states, int32_t num_seqs,
                        int32_t seq_len, int32_t total_tokens, int32_t num_heads, int head_dim,
                        int dtype, unsigned *far_flags, hipStream_t stream);

// Workgroups the prefill kernel runs per (sequence, head): one per d_v slice.
int chunk_fwd_slices(int head_dim, int dtype);

// What a prefill launch produces (see chunk_fwd_kernel): outputs, final
// states and snapshots; final states only; the state transition (identity
// start, zero values); the backward's per-16-token checkpoints.
constexpr int kModeOut = 0, kModeState = 1, kModeMap = 2, kModeStates = 3;

// The prefill for fp32 inputs at head_dim 128 as the token recurrence itself
// (kda_seq.hip): same arguments and results as launch_chunk_fwd for the modes
// kModeOut (scalar_gate allowed), kModeState and kModeMap.  Returns 0, or -1
// if the launch failed or the combination is not one of these.
int launch_chunk_seq(const void *q, const void *k, const void *v, const float *log_alpha,
                     const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                     void *out, float *final_state, float *snapshots, int32_t snapshot_every,
                     int32_t num_snapshots, int32_t num_seqs, int32_t seq_len,
                     int32_t total_tokens, int32_t num_heads, int scalar_gate, int mode,
                     hipStream_t stream);

// Tokens per chunk of the prefill; snapshot intervals are multiples of it.
constexpr int kChunkTokens = 32;

// Segmented prefill of one sequence.  cu[g] = min(g * seg_len, total) for
// g = 0 .. nseg (the segment boundaries as packed-sequence offsets).
int launch_segment_bounds(int32_t *cu, int nseg, int seg_len, int total, hipStream_t stream);

// Entering states of the segments, [nseg, H, D, D] in the stored orientation
// M = S^T: m_in[0] = m0 (zero when m0 == NULL), m_in[g + 1] = m_in[g] X[g] + Y[g]
// (X[g], Y[g]: the final states of segment g from S = I with zero values and
// from S = 0).  head_dim is 64 or 128.  Returns 0, or -1 if the launch failed.
int launch_segment_fold(const float *m0, const float *X, const float *Y, float *m_in, int nseg,
                        int H, int head_dim, hipStream_t stream);

// The backward's fallback for (sequence, head) units whose gates leave the
// chunked backward's range (a 16-token block decaying beyond 2^-100 in some
// channel, -inf or NaN gates).  launch_bwd_far_detect writes
// bwd_far_flag_words(N, H) flag words (nonzero: the unit is out of range);
// launch_bwd_seq, run after the chunked backward on the same stream,
// recomputes every gradient of the flagged units token by token in fp32 and
// leaves the others alone; ckpt holds (total_tokens / 16 + N + 1) * H * d^2
// fp32 values (the chunked backward's first workspace region).
int64_t bwd_far_flag_words(int64_t num_seqs, int64_t num_heads);
int launch_bwd_far_detect(const float *log_alpha, const int32_t *cu_seqlens, int32_t num_seqs,
                          int32_t seq_len, int32_t total_tokens, int32_t num_heads, int head_dim,
                          unsigned *flags, hipStream_t stream);
int launch_bwd_seq(const void *q, const void *k, const void *v, const float *log_alpha,
                   const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                   const void *d_out, const float *d_final_state, void *dq, void *dk, void *dv,
                   float *dlog_alpha, float *dbeta, float *d_initial_state, float *ckpt,
                   const unsigned *flags, int32_t num_seqs, int32_t seq_len,
                   int32_t total_tokens, int32_t num_heads, int head_dim, int dtype,
                   hipStream_t stream);

// The chunked backward's dL/dS chain for bf16 inputs (bf16 checkpoints): one
// workgroup per (sequence, head, half of the value columns), preparation waves
// one chunk ahead of the scan waves.  Writes the gradient at every 16-token
// chunk's end to dckpt (the backward workspace's second region, bf16
// [slot][H][d_v][d_k]) and d_initial_state (if not NULL).  Returns 0, or -1 if
// the launch failed.
int launch_bwd_chain(const void *q, const void *k, const float *log_alpha, const float *beta,
                     const int32_t *cu_seqlens, const void *d_out, const float *d_final_state,
                     float *d_initial_state, float *dckpt, int32_t num_seqs, int32_t seq_len,
                     int32_t total_tokens, int32_t num_heads, int head_dim, hipStream_t stream);

// Chunked backward: gradients of the prefill's outputs and final states with
// respect to q, k, v, log_alpha, beta and the initial states.  Sequences as
// for launch_chunk_fwd (dense when cu_seqlens == NULL).  d_final_state,
// initial_state and d_initial_state may be NULL (zero / not written).  The
// workspace holds chunk_bwd_workspace_floats(...) fp32 values (the entering
// state of every 16-token chunk).  Arguments are already validated.  Returns
// 0, or -1 if the launch failed.
int64_t chunk_bwd_workspace_floats(int64_t total_tokens, int64_t num_seqs, int64_t num_heads,
                                   int head_dim);
int launch_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                     const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                     const void *d_out, const float *d_final_state, void *dq, void *dk, void *dv,
                     float *dlog_alpha, float *dbeta, float *d_initial_state, float *workspace,
                     int32_t num_seqs, int32_t seq_len, int32_t total_tokens, int32_t num_heads,
                     int head_dim, int dtype, hipStream_t stream);

}  // namespace kda
