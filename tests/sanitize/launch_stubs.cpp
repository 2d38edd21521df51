// launch_stubs.cpp -- stand-ins for the library's kernel launchers, so that
// the host validation of kda_api.cpp can be built and run without the GPU
// code.  Reaching one means a call got past every host and device check on a
// host without a GPU, which abi_driver.cpp never expects: abort loudly.
#include <stdio.h>
#include <stdlib.h>

#include "kda_internal.h"

namespace {
[[noreturn]] void reached(const char *name) {
    fprintf(stderr, "launch stub reached: %s\n", name);
    abort();
}
}  // namespace

namespace kda {
int launch_decode_step(const void *, const void *, const void *, const float *, const float *,
                       float *, void *, int64_t, int, int, int, hipStream_t) {
    reached("launch_decode_step");
}
int launch_chunk_fwd(const void *, const void *, const void *, const float *, const float *,
                     const float *, const int32_t *, void *, float *, float *, int32_t, int32_t,
                     int32_t, int32_t, int32_t, int32_t, int, int, int, int, hipStream_t) {
    reached("launch_chunk_fwd");
}
int chunk_fwd_slices(int, int) { reached("chunk_fwd_slices"); }
int launch_segment_bounds(int32_t *, int, int, int, hipStream_t) {
    reached("launch_segment_bounds");
}
int launch_segment_fold(const float *, const float *, const float *, float *, int, int, int,
                        hipStream_t) {
    reached("launch_segment_fold");
}
int64_t chunk_bwd_workspace_floats(int64_t total_tokens, int64_t num_seqs, int64_t num_heads,
                                   int head_dim) {
    // two regions of one fp32 state per 16-token slot and head, then 16 flag
    // words per (sequence, head) (the library's rule)
    return 2 * (total_tokens / 16 + num_seqs + 1) * num_heads * head_dim * head_dim +
           16 * num_seqs * num_heads;
}
int launch_chunk_bwd(const void *, const void *, const void *, const float *, const float *,
                     const float *, const int32_t *, const void *, const float *, void *, void *,
                     void *, float *, float *, float *, float *, int32_t, int32_t, int32_t,
                     int32_t, int, int, hipStream_t) {
    reached("launch_chunk_bwd");
}
}  // namespace kda
