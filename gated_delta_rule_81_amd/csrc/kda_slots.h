// kda_slots.h -- the backward's workspace slots, for the kernels that write
// them and the one that finds its chunk from its slot (host and device code,
// so that the host can check the layout).
//
// Each workspace region holds one d x d state per slot and head.  Chunk j (16
// tokens) of sequence n, whose first token is t0, owns slot t0 / 16 + n + j:
// the + n keeps a sequence's last, partial chunk from sharing its slot with
// the next sequence's first, so a region of total_tokens tokens packed in
// num_seqs sequences needs total_tokens / 16 + num_seqs + 1 slots.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kSlotTokens = 16;  // tokens per slot (the backward's chunk)

// The slot of chunk 0 of sequence n, whose first token is t0.
__host__ __device__ __forceinline__ int64_t first_slot(int64_t t0, int n) {
    return t0 / kSlotTokens + n;
}

// Slots in one region for total_tokens tokens in num_seqs sequences.
__host__ __device__ __forceinline__ int64_t region_slots(int64_t total_tokens, int64_t num_seqs) {
    return total_tokens / kSlotTokens + num_seqs + 1;
}

// First token of sequence m: the packed offset clamped into [0, total_tokens],
// or m * seq_len for equal-length sequences (no offsets).
__host__ __device__ __forceinline__ int64_t seq_first_token(const int32_t *cu_seqlens, int seq_len,
                                                            int total_tokens, int m) {
    if (!cu_seqlens) return (int64_t)m * seq_len;
    const int a = cu_seqlens[m];
    return a < 0 ? 0 : (a > total_tokens ? total_tokens : a);
}

// The sequence whose chunks own `slot`: the last m in [0, num_seqs) whose
// first slot is at or before it (a bisection, which ends for any offsets);
// *chunk receives slot - first_slot of that sequence, which lies outside
// [0, its chunk count) for a slot that no chunk owns.
__host__ __device__ __forceinline__ int slot_sequence(const int32_t *cu_seqlens, int num_seqs,
                                                      int seq_len, int total_tokens, int64_t slot,
                                                      int *chunk) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first_slot(seq_first_token(cu_seqlens, seq_len, total_tokens, mid), mid) <= slot)
            lo = mid;
        else
            hi = mid - 1;
    }
    *chunk = (int)(slot - first_slot(seq_first_token(cu_seqlens, seq_len, total_tokens, lo), lo));
    return lo;
}

}  // namespace kda
