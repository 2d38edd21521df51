// kda_api.cpp -- the C ABI declared in include/kda.h: argument validation on
// the host, then one kernel launch on the caller's stream.
//
// Validation order: NULL pointers, sizes, supported configurations,
// alignment, aliasing (all pure host checks, no HIP call), then the device
// architecture (cached per device), then the launch.  Nothing here allocates:
// workspaces are the caller's, or (kda_chunk_fwd_segmented_noalloc) a fixed
// buffer compiled into the library.
#include "kda.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <vector>

#include "kda_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

bool aligned16(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned4(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

struct Range {
    const void *p;
    uint64_t bytes;
};

bool overlap(const Range &a, const Range &b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Compute units of the current device (cached per device; 0 if unknown).
std::atomic<int> g_device_cus[kMaxDevices];
int device_cus() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = g_device_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        g_device_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KDA_ERR_DEVICE;
    if (dev >= kMaxDevices) return KDA_ERR_DEVICE;
    int st = g_device_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KDA_ERR_DEVICE;
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_device_ok[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? KDA_OK : KDA_ERR_DEVICE;
}

// Debug mode (environment variable KDA_DEBUG set to a value other than "0",
// read at every call): packed-sequence offsets are copied to the host and
// checked before the launch, and every call waits for its stream and reports
// any failure of its kernels as KDA_ERR_LAUNCH, with a line on stderr naming
// the entry point.  Off by default: calls stay asynchronous.
bool debug_mode() {
    const char *e = getenv("KDA_DEBUG");
    return e && e[0] && strcmp(e, "0") != 0;
}

// Debug mode: cu_seqlens must hold num_seqs + 1 offsets starting at 0,
// non-decreasing and ending at total.  Returns KDA_OK or KDA_ERR_SHAPE.
int debug_check_offsets(const int32_t *cu_seqlens, int64_t num_seqs, int64_t total,
                        hipStream_t stream, const char *where) {
    if (!cu_seqlens) return KDA_OK;
    std::vector<int32_t> cu((size_t)num_seqs + 1);
    if (hipStreamSynchronize(stream) != hipSuccess ||
        hipMemcpy(cu.data(), cu_seqlens, cu.size() * 4, hipMemcpyDeviceToHost) != hipSuccess) {
        fprintf(stderr, "[kda debug] %s: cannot read cu_seqlens\n", where);
        return KDA_ERR_LAUNCH;
    }
    bool ok = cu[0] == 0 && cu[(size_t)num_seqs] == total;
    for (size_t i = 0; ok && i < (size_t)num_seqs; ++i) ok = cu[i] <= cu[i + 1];
    if (!ok) {
        fprintf(stderr, "[kda debug] %s: cu_seqlens is not 0 = c0 <= c1 <= ... <= cN = %lld\n",
                where, (long long)total);
        return KDA_ERR_SHAPE;
    }
    return KDA_OK;
}

// The status of a call whose launches returned `rc` (0 = queued): in debug
// mode also wait for the stream and check what its kernels did.
int launch_status(int rc, hipStream_t stream, const char *where) {
    if (rc != 0) {
        if (debug_mode()) fprintf(stderr, "[kda debug] %s: launch failed\n", where);
        return KDA_ERR_LAUNCH;
    }
    if (debug_mode()) {
        const hipError_t e = hipStreamSynchronize(stream);
        const hipError_t l = hipGetLastError();
        if (e != hipSuccess || l != hipSuccess) {
            fprintf(stderr, "[kda debug] %s: %s\n", where,
                    hipGetErrorString(e != hipSuccess ? e : l));
            return KDA_ERR_LAUNCH;
        }
    }
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_status_string(int status) {
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is negative or the sizes disagree";
    case KDA_ERR_UNSUPPORTED: return "configuration not supported by this build";
    case KDA_ERR_ALIGN: return "a pointer is not aligned as the ABI requires";
    case KDA_ERR_ALIAS: return "an output overlaps an input";
    case KDA_ERR_DEVICE: return "the current device is not a gfx950 GPU";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
    case KDA_ERR_SCRATCH: return "the request needs more than the library's fixed scratch buffer";
    default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// Shared by the prefill entry points: kda_chunk_fwd (no snapshots, gates per
// channel), kda_chunk_fwd_snapshots and kda_chunk_fwd_scalar_gate (log_alpha
// [T, H]: one gate per token and head).
int chunk_fwd_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                   const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                   void *out, float *final_state, float *snapshots, int32_t snapshot_every,
                   int32_t num_snapshots, int32_t batch, int32_t seq_len, int32_t num_heads,
                   int32_t head_dim_k, int32_t head_dim_v, int32_t num_seqs, int32_t dtype,
                   bool scalar_gate, hipStream_t stream, bool check_only = false) {
    // sizes
    if (batch < 0 || seq_len < 0 || num_heads < 0 || head_dim_k <= 0 || head_dim_v <= 0)
        return KDA_ERR_SHAPE;
    if (num_snapshots < 0) return KDA_ERR_SHAPE;
    const bool snap = snapshots != nullptr || num_snapshots > 0;
    if (snap && snapshot_every <= 0) return KDA_ERR_SHAPE;
    if (dtype != kda::kDtypeF32 && dtype != kda::kDtypeBf16) return KDA_ERR_UNSUPPORTED;
    const bool packed = cu_seqlens != nullptr;
    if (packed && (batch != 1 || num_seqs < 0)) return KDA_ERR_SHAPE;
    const int64_t tokens = (int64_t)batch * seq_len;
    if (tokens > INT32_MAX) return KDA_ERR_SHAPE;
    const int64_t nseq = packed ? num_seqs : batch;
    // dense: every sequence has seq_len tokens, so the count is known here
    if (snap && !packed && (int64_t)batch * (seq_len / snapshot_every) > num_snapshots)
        return KDA_ERR_SHAPE;
    const uint64_t esz = dtype == kda::kDtypeBf16 ? 2 : 4;
    const uint64_t th = (uint64_t)tokens * num_heads;
    // pointers required whenever the array they describe is not empty
    const bool have_tokens = th > 0;
    if (have_tokens && (!q || !k || !v || !log_alpha || !beta || !out)) return KDA_ERR_NULL;
    if (num_snapshots > 0 && num_heads > 0 && !snapshots) return KDA_ERR_NULL;
    // supported configurations
    if (head_dim_k != head_dim_v) return KDA_ERR_UNSUPPORTED;
    const int d = head_dim_k;
    if (d != 64 && d != 128) return KDA_ERR_UNSUPPORTED;
    if (snap && snapshot_every % kda::kChunkTokens != 0) return KDA_ERR_UNSUPPORTED;
    // the kernel addresses 64 tokens of one tensor with 32-bit byte offsets
    if ((int64_t)num_heads * d * 4 * 64 > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    // alignment
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) ||
        !(scalar_gate ? aligned4(log_alpha) : aligned16(log_alpha)) || !aligned4(beta) ||
        !aligned16(initial_state) || !aligned16(out) || !aligned16(final_state) ||
        !aligned4(cu_seqlens) || !aligned16(snapshots))
        return KDA_ERR_ALIGN;
    // aliasing
    const uint64_t state_bytes = (uint64_t)nseq * num_heads * d * d * 4;
    const Range rq{q, th * d * esz}, rk{k, th * d * esz}, rv{v, th * d * esz},
        rg{log_alpha, th * (scalar_gate ? 1 : d) * 4}, rb{beta, th * 4},
        rs0{initial_state, state_bytes},
        rcu{cu_seqlens, packed ? (uint64_t)(nseq + 1) * 4 : 0}, ro{out, th * d * esz},
        rs1{final_state, state_bytes},
        rsn{snapshots, (uint64_t)num_snapshots * num_heads * d * d * 4};
    const Range inputs[] = {rq, rk, rv, rg, rb, rs0, rcu};
    for (const Range &r : inputs)
        if (overlap(ro, r) || overlap(rsn, r)) return KDA_ERR_ALIAS;
    if (overlap(ro, rs1) || overlap(rsn, ro) || overlap(rsn, rs1)) return KDA_ERR_ALIAS;
    for (int i = 0; i < 7; ++i) {
        if (i == 5 && final_state && (const void *)final_state == (const void *)initial_state)
            continue;  // in-place state update is allowed
        if (overlap(rs1, inputs[i])) return KDA_ERR_ALIAS;
    }
    if (check_only) return KDA_OK;
    if (nseq == 0 || num_heads == 0) return KDA_OK;
    int st = check_device();
    if (st != KDA_OK) return st;
    const char *where = snap ? "kda_chunk_fwd_snapshots"
                             : (scalar_gate ? "kda_chunk_fwd_scalar_gate" : "kda_chunk_fwd");
    if (debug_mode() && (st = debug_check_offsets(cu_seqlens, nseq, tokens, stream, where)) != KDA_OK)
        return st;
    const int rc = kda::launch_chunk_fwd(q, k, v, log_alpha, beta, initial_state, cu_seqlens, out,
                                         final_state, num_snapshots > 0 ? snapshots : nullptr,
                                         snapshot_every, num_snapshots, (int32_t)nseq, seq_len,
                                         (int32_t)tokens, num_heads, d, dtype, scalar_gate ? 1 : 0,
                                         0, stream);
    return launch_status(rc, stream, where);
}

// Shared by kda_decode_step and kda_decode_step_scalar_gate (log_alpha [B, H]).
int decode_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                const float *beta, float *state, void *out, int32_t batch, int32_t num_heads,
                int32_t head_dim_k, int32_t head_dim_v, int32_t dtype, bool scalar_gate,
                hipStream_t stream) {
    if (batch < 0 || num_heads < 0 || head_dim_k <= 0 || head_dim_v <= 0) return KDA_ERR_SHAPE;
    if (dtype != kda::kDtypeF32 && dtype != kda::kDtypeBf16) return KDA_ERR_UNSUPPORTED;
    const uint64_t units = (uint64_t)batch * num_heads;
    if (units > 0 && (!q || !k || !v || !log_alpha || !beta || !state || !out))
        return KDA_ERR_NULL;
    if (head_dim_k != head_dim_v) return KDA_ERR_UNSUPPORTED;
    const int d = head_dim_k;
    if (d != 64 && d != 128) return KDA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) ||
        !(scalar_gate ? aligned4(log_alpha) : aligned16(log_alpha)) || !aligned4(beta) ||
        !aligned16(state) || !aligned16(out))
        return KDA_ERR_ALIGN;
    const uint64_t esz = dtype == kda::kDtypeBf16 ? 2 : 4;
    const Range ro{out, units * d * esz};
    const Range others[] = {{q, units * d * esz}, {k, units * d * esz}, {v, units * d * esz},
                            {log_alpha, units * (scalar_gate ? 1 : d) * 4}, {beta, units * 4},
                            {state, units * d * d * 4}};
    for (const Range &r : others)
        if (overlap(ro, r)) return KDA_ERR_ALIAS;
    for (int i = 0; i < 5; ++i)
        if (overlap(others[5], others[i])) return KDA_ERR_ALIAS;
    if (units == 0) return KDA_OK;
    const int st = check_device();
    if (st != KDA_OK) return st;
    const int rc = kda::launch_decode_step(q, k, v, log_alpha, beta, state, out, (int64_t)units,
                                           d, dtype, scalar_gate ? 1 : 0, stream);
    return launch_status(rc, stream,
                         scalar_gate ? "kda_decode_step_scalar_gate" : "kda_decode_step");
}

// Segment plan of the segmented prefill: segments of seg_len tokens (a
// multiple of the chunk length, at least one chunk), nseg of them (0 for T = 0).
struct SegPlan {
    int seg_len, nseg;
};
SegPlan seg_plan(int32_t seq_len, int32_t num_segments) {
    if (seq_len <= 0) return {kda::kChunkTokens, 0};
    int64_t L = ((int64_t)seq_len + num_segments - 1) / num_segments;
    L = (L + kda::kChunkTokens - 1) / kda::kChunkTokens * kda::kChunkTokens;
    return {(int)L, (int)(((int64_t)seq_len + L - 1) / L)};
}
// Workspace: segment offsets (padded to 256 bytes), then four [nseg, H, D, D]
// fp32 arrays: the segments' maps Y (from S = 0) and X (from S = I, zero
// values), their entering states and their final states.
uint64_t seg_cu_bytes(int nseg) { return ((uint64_t)(nseg + 1) * 4 + 255) / 256 * 256; }
uint64_t seg_state_bytes(int nseg, int H, int d) { return (uint64_t)nseg * H * d * d * 4; }

}  // namespace

extern "C" {

int64_t kda_chunk_fwd_segmented_workspace_size(int32_t seq_len, int32_t num_heads,
                                               int32_t head_dim, int32_t num_segments) {
    if (seq_len < 0 || num_heads < 0 || num_segments < 1 || (head_dim != 64 && head_dim != 128))
        return -1;
    const SegPlan sp = seg_plan(seq_len, num_segments);
    return (int64_t)(seg_cu_bytes(sp.nseg) + 4 * seg_state_bytes(sp.nseg, num_heads, head_dim));
}

int kda_chunk_fwd_segmented(const void *q, const void *k, const void *v, const float *log_alpha,
                            const float *beta, const float *initial_state, void *out,
                            float *final_state, int32_t seq_len, int32_t num_heads,
                            int32_t head_dim_k, int32_t head_dim_v, int32_t num_segments,
                            int32_t dtype, void *workspace, int64_t workspace_bytes,
                            hipStream_t stream) {
    if (num_segments < 1 || workspace_bytes < 0) return KDA_ERR_SHAPE;
    // every kda_chunk_fwd rule for one dense sequence
    int st = chunk_fwd_impl(q, k, v, log_alpha, beta, initial_state, nullptr, out, final_state,
                            nullptr, 0, 0, 1, seq_len, num_heads, head_dim_k, head_dim_v, 0,
                            dtype, false, stream, true);
    if (st != KDA_OK) return st;
    const SegPlan sp = seg_plan(seq_len, num_segments);
    if (sp.nseg <= 1 || num_heads == 0)  // nothing to split: the plain prefill
        return chunk_fwd_impl(q, k, v, log_alpha, beta, initial_state, nullptr, out,
                              final_state, nullptr, 0, 0, 1, seq_len, num_heads, head_dim_k,
                              head_dim_v, 0, dtype, false, stream);
    const int d = head_dim_k;
    const uint64_t cu_b = seg_cu_bytes(sp.nseg), sb = seg_state_bytes(sp.nseg, num_heads, d);
    const uint64_t need = cu_b + 4 * sb;
    if (!workspace) return KDA_ERR_NULL;
    if ((uint64_t)workspace_bytes < need) return KDA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return KDA_ERR_ALIGN;
    const uint64_t esz = dtype == kda::kDtypeBf16 ? 2 : 4;
    const uint64_t th = (uint64_t)seq_len * num_heads, hs = (uint64_t)num_heads * d * d * 4;
    const Range rw{workspace, need};
    const Range others[] = {{q, th * d * esz}, {k, th * d * esz}, {v, th * d * esz},
                            {log_alpha, th * d * 4}, {beta, th * 4}, {initial_state, hs},
                            {out, th * d * esz}, {final_state, hs}};
    for (const Range &r : others)
        if (overlap(rw, r)) return KDA_ERR_ALIAS;
    st = check_device();
    if (st != KDA_OK) return st;
    // The segmented call does about three times the chunk work in exchange for
    // parallelism along the sequence, so it can only win while the plain
    // launch leaves at least two thirds of the compute units idle.
    const int cus = device_cus();
    if (cus > 0 && 3 * (int64_t)num_heads * kda::chunk_fwd_slices(d, dtype) > cus)
        return chunk_fwd_impl(q, k, v, log_alpha, beta, initial_state, nullptr, out,
                              final_state, nullptr, 0, 0, 1, seq_len, num_heads, head_dim_k,
                              head_dim_v, 0, dtype, false, stream);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    int32_t *cu = reinterpret_cast<int32_t *>(ws);
    float *Y = reinterpret_cast<float *>(ws + cu_b);
    float *X = reinterpret_cast<float *>(ws + cu_b + sb);
    float *Min = reinterpret_cast<float *>(ws + cu_b + 2 * sb);
    float *Fin = reinterpret_cast<float *>(ws + cu_b + 3 * sb);
    const int T = seq_len, n = sp.nseg;
    int rc = kda::launch_segment_bounds(cu, n, sp.seg_len, T, stream);
    // each segment's map from a zero state (Y) and, with zero values, from the
    // identity (X), no outputs
    if (rc == 0)
        rc = kda::launch_chunk_fwd(q, k, v, log_alpha, beta, nullptr, cu, nullptr, Y, nullptr, 0,
                                   0, n, T, T, num_heads, d, dtype, 0, 0, stream);
    if (rc == 0)
        rc = kda::launch_chunk_fwd(q, k, nullptr, log_alpha, beta, nullptr, cu, nullptr, X,
                                   nullptr, 0, 0, n, T, T, num_heads, d, dtype, 0, 1, stream);
    // the entering state of every segment, then the segments from their true
    // entering states
    if (rc == 0) rc = kda::launch_segment_fold(initial_state, X, Y, Min, n, num_heads, d, stream);
    if (rc == 0)
        rc = kda::launch_chunk_fwd(q, k, v, log_alpha, beta, Min, cu, out, Fin, nullptr, 0, 0, n,
                                   T, T, num_heads, d, dtype, 0, 0, stream);
    if (rc == 0 && final_state &&
        hipMemcpyAsync(final_state, Fin + (uint64_t)(n - 1) * num_heads * d * d, hs,
                       hipMemcpyDeviceToDevice, stream) != hipSuccess)
        rc = -1;
    return launch_status(rc, stream, "kda_chunk_fwd_segmented");
}

}  // extern "C"

// The fixed scratch of kda_chunk_fwd_segmented_noalloc: one copy per GPU, in
// the code object's device memory, reserved when the library's code is
// loaded on that GPU and held until the process ends.  In host code `scratch`
// names only a host-side stand-in; its device address comes from
// hipGetSymbolAddress, once per device, with that device current, and only
// that address is ever handed to kernels or copies.
static __device__ __align__(256) unsigned char scratch[KDA_SCRATCH_BYTES];

namespace {

std::atomic<void *> g_scratch[kMaxDevices];  // per device: the address of `scratch`

// Device address of the current device's scratch, or NULL if it cannot be had.
void *scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

int kda_chunk_fwd_segmented_noalloc(const void *q, const void *k, const void *v,
                                    const float *log_alpha, const float *beta,
                                    const float *initial_state, void *out, float *final_state,
                                    int32_t seq_len, int32_t num_heads, int32_t head_dim_k,
                                    int32_t head_dim_v, int32_t num_segments, int32_t dtype,
                                    hipStream_t stream) {
    if (num_segments < 1) return KDA_ERR_SHAPE;
    int st = chunk_fwd_impl(q, k, v, log_alpha, beta, initial_state, nullptr, out, final_state,
                            nullptr, 0, 0, 1, seq_len, num_heads, head_dim_k, head_dim_v, 0,
                            dtype, false, stream, true);
    if (st != KDA_OK) return st;
    const SegPlan sp = seg_plan(seq_len, num_segments);
    if (sp.nseg <= 1 || num_heads == 0)  // the plain prefill: no scratch
        return kda_chunk_fwd_segmented(q, k, v, log_alpha, beta, initial_state, out,
                                       final_state, seq_len, num_heads, head_dim_k, head_dim_v,
                                       num_segments, dtype, nullptr, 0, stream);
    const int64_t need =
        kda_chunk_fwd_segmented_workspace_size(seq_len, num_heads, head_dim_k, num_segments);
    if (need < 0 || need > (int64_t)KDA_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
    st = check_device();
    if (st != KDA_OK) return st;
    void *ws = scratch_for_current_device();
    if (!ws) return KDA_ERR_LAUNCH;
    return kda_chunk_fwd_segmented(q, k, v, log_alpha, beta, initial_state, out, final_state,
                                   seq_len, num_heads, head_dim_k, head_dim_v, num_segments,
                                   dtype, ws, (int64_t)KDA_SCRATCH_BYTES, stream);
}

int64_t kda_chunk_bwd_workspace_size(int32_t total_tokens, int32_t num_seqs, int32_t num_heads,
                                     int32_t head_dim) {
    if (total_tokens < 0 || num_seqs < 0 || num_heads < 0 || (head_dim != 64 && head_dim != 128))
        return -1;
    return kda::chunk_bwd_workspace_floats(total_tokens, num_seqs, num_heads, head_dim) * 4;
}

int kda_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                  const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                  const void *d_out, const float *d_final_state, void *dq, void *dk, void *dv,
                  float *dlog_alpha, float *dbeta, float *d_initial_state, int32_t batch,
                  int32_t seq_len, int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                  int32_t num_seqs, int32_t dtype, void *workspace, int64_t workspace_bytes,
                  hipStream_t stream) {
    if (batch < 0 || seq_len < 0 || num_heads < 0 || head_dim_k <= 0 || head_dim_v <= 0 ||
        workspace_bytes < 0)
        return KDA_ERR_SHAPE;
    if (dtype != kda::kDtypeF32 && dtype != kda::kDtypeBf16) return KDA_ERR_UNSUPPORTED;
    const bool packed = cu_seqlens != nullptr;
    if (packed && (batch != 1 || num_seqs < 0)) return KDA_ERR_SHAPE;
    const int64_t tokens = (int64_t)batch * seq_len;
    if (tokens > INT32_MAX) return KDA_ERR_SHAPE;
    const int64_t nseq = packed ? num_seqs : batch;
    const uint64_t th = (uint64_t)tokens * num_heads;
    if (th > 0 && (!q || !k || !v || !log_alpha || !beta || !d_out || !dq || !dk || !dv ||
                   !dlog_alpha || !dbeta))
        return KDA_ERR_NULL;
    if (head_dim_k != head_dim_v) return KDA_ERR_UNSUPPORTED;
    const int d = head_dim_k;
    if (d != 64 && d != 128) return KDA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) ||
        !aligned4(beta) || !aligned16(initial_state) || !aligned4(cu_seqlens) ||
        !aligned16(d_out) || !aligned16(d_final_state) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv) || !aligned16(dlog_alpha) || !aligned4(dbeta) ||
        !aligned16(d_initial_state) || !aligned16(workspace))
        return KDA_ERR_ALIGN;
    const uint64_t need =
        (uint64_t)kda::chunk_bwd_workspace_floats(tokens, nseq, num_heads, d) * 4;
    const bool work = nseq > 0 && num_heads > 0;
    if (work && !workspace) return KDA_ERR_NULL;
    if (work && (uint64_t)workspace_bytes < need) return KDA_ERR_SHAPE;
    const uint64_t esz = dtype == kda::kDtypeBf16 ? 2 : 4;
    const uint64_t sb = (uint64_t)nseq * num_heads * d * d * 4;
    const Range inputs[] = {{q, th * d * esz}, {k, th * d * esz}, {v, th * d * esz},
                            {log_alpha, th * d * 4}, {beta, th * 4}, {initial_state, sb},
                            {cu_seqlens, packed ? (uint64_t)(nseq + 1) * 4 : 0},
                            {d_out, th * d * esz}, {d_final_state, sb}};
    const Range outputs[] = {{dq, th * d * esz}, {dk, th * d * esz}, {dv, th * d * esz},
                             {dlog_alpha, th * d * 4}, {dbeta, th * 4}, {d_initial_state, sb},
                             {workspace, work ? need : 0}};
    for (int i = 0; i < 7; ++i) {
        for (const Range &r : inputs)
            if (overlap(outputs[i], r)) return KDA_ERR_ALIAS;
        for (int j = i + 1; j < 7; ++j)
            if (overlap(outputs[i], outputs[j])) return KDA_ERR_ALIAS;
    }
    if (!work) return KDA_OK;
    int st = check_device();
    if (st != KDA_OK) return st;
    if (debug_mode() &&
        (st = debug_check_offsets(cu_seqlens, nseq, tokens, stream, "kda_chunk_bwd")) != KDA_OK)
        return st;
    const int rc = kda::launch_chunk_bwd(q, k, v, log_alpha, beta, initial_state, cu_seqlens,
                                         d_out, d_final_state, dq, dk, dv, dlog_alpha, dbeta,
                                         d_initial_state, static_cast<float *>(workspace),
                                         (int32_t)nseq, seq_len, (int32_t)tokens, num_heads, d,
                                         dtype, stream);
    return launch_status(rc, stream, "kda_chunk_bwd");
}

int kda_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                  const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                  void *out, float *final_state, int32_t batch, int32_t seq_len,
                  int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v, int32_t num_seqs,
                  int32_t dtype, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, initial_state, cu_seqlens, out, final_state,
                          nullptr, 0, 0, batch, seq_len, num_heads, head_dim_k, head_dim_v,
                          num_seqs, dtype, false, stream);
}

int kda_chunk_fwd_scalar_gate(const void *q, const void *k, const void *v,
                              const float *log_alpha, const float *beta,
                              const float *initial_state, const int32_t *cu_seqlens, void *out,
                              float *final_state, int32_t batch, int32_t seq_len,
                              int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                              int32_t num_seqs, int32_t dtype, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, initial_state, cu_seqlens, out, final_state,
                          nullptr, 0, 0, batch, seq_len, num_heads, head_dim_k, head_dim_v,
                          num_seqs, dtype, true, stream);
}

int kda_chunk_fwd_snapshots(const void *q, const void *k, const void *v, const float *log_alpha,
                            const float *beta, const float *initial_state,
                            const int32_t *cu_seqlens, void *out, float *final_state,
                            float *snapshots, int32_t snapshot_every, int32_t num_snapshots,
                            int32_t batch, int32_t seq_len, int32_t num_heads,
                            int32_t head_dim_k, int32_t head_dim_v, int32_t num_seqs,
                            int32_t dtype, hipStream_t stream) {
    if (snapshot_every <= 0) return KDA_ERR_SHAPE;
    return chunk_fwd_impl(q, k, v, log_alpha, beta, initial_state, cu_seqlens, out, final_state,
                          snapshots, snapshot_every, num_snapshots, batch, seq_len, num_heads,
                          head_dim_k, head_dim_v, num_seqs, dtype, false, stream);
}

int kda_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                    const float *beta, float *state, void *out, int32_t batch, int32_t num_heads,
                    int32_t head_dim_k, int32_t head_dim_v, int32_t dtype, hipStream_t stream) {
    return decode_impl(q, k, v, log_alpha, beta, state, out, batch, num_heads, head_dim_k,
                       head_dim_v, dtype, false, stream);
}

int kda_decode_step_scalar_gate(const void *q, const void *k, const void *v,
                                const float *log_alpha, const float *beta, float *state,
                                void *out, int32_t batch, int32_t num_heads, int32_t head_dim_k,
                                int32_t head_dim_v, int32_t dtype, hipStream_t stream) {
    return decode_impl(q, k, v, log_alpha, beta, state, out, batch, num_heads, head_dim_k,
                       head_dim_v, dtype, true, stream);
}

}  // extern "C"
