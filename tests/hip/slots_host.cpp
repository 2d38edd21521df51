// Host build of the backward's workspace-slot arithmetic (kda_slots.h, the
// functions the kernels call), exported with C linkage for the CPU tests.
#include "kda_slots.h"

extern "C" {
long long kda_test_first_slot(long long t0, int n) { return kda::first_slot(t0, n); }
long long kda_test_region_slots(long long total_tokens, long long num_seqs) {
    return kda::region_slots(total_tokens, num_seqs);
}
int kda_test_slot_sequence(const int *cu_seqlens, int num_seqs, int seq_len, int total_tokens,
                           long long slot, int *chunk) {
    return kda::slot_sequence(cu_seqlens, num_seqs, seq_len, total_tokens, slot, chunk);
}
}
