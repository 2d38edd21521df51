// kda_seq.hip -- the KDA prefill as the token recurrence itself, for fp32
// inputs at d_k = d_v = 128 (the chunked prefill kernel's fp32 operand sets do
// not fit one CU's LDS at that size).
//
// Pages cited (by title):
//   [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer.
//
// Per token, exactly the update of [K3-explainer] §三/§四 in predict/correct
// form, in fp32 with an fp32 state:
//   S' = Diag(alpha_t) S,  p = S'^T k_t,  delta = beta_t (v_t - p),
//   S = S' + k_t delta^T,  o_t = S^T q_t.
// One workgroup per (sequence, head, 64 value columns): wave w owns value
// columns v0 + 16 w .. + 15 of the state for all d_k key rows, lane (l16, l4)
// holding column l16 and key rows 16 t + 4 l4 + e (t < D / 16, e < 4) in
// registers.  Every 32 tokens the workgroup stages the rows of k, q,
// alpha = e^{log_alpha} (computed once per element here), the v slice and beta
// in LDS, double buffered so the next rows load while this block's tokens are
// stepped; each wave then steps the tokens on its own, the sums over key rows
// (p and o) reduced across the four lane groups.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_lanes.h"
#include "kda_slots.h"

namespace kda {

namespace {

constexpr int kSeqT = 32;  // tokens staged per block

template <int D, int DVS, bool SG>
struct SeqCfg {
    static constexpr int W = DVS / 16;        // waves
    static constexpr int THREADS = 64 * W;
    static constexpr int NRT = D / 16;        // 16-row key tiles held per lane
    static constexpr int LDR = D + 4;         // floats per staged k / q / alpha row
    static constexpr int LDV = DVS + 4;       // floats per staged v row
    // one staged block: k, q, alpha rows, v slice, beta
    static constexpr int oK = 0, oQ = oK + kSeqT * LDR, oA = oQ + kSeqT * LDR,
                         oV = oA + (SG ? kSeqT : kSeqT * LDR), oB = oV + kSeqT * LDV,
                         BLOCK = oB + kSeqT;  // floats
    static constexpr int BYTES = 2 * BLOCK * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(D % 16 == 0 && DVS % 16 == 0 && D % DVS == 0, "tile shapes");
};

template <int D, int DVS, bool SG, int MODE>
__global__ __launch_bounds__(64 * (DVS / 16)) void chunk_seq_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ initial_state, const int32_t *__restrict__ cu_seqlens,
    float *__restrict__ out, float *__restrict__ final_state, float *__restrict__ snapshots,
    int snap_every, int snap_cap, int num_seqs, int seq_len, int total_tokens, int H,
    int units) {
    typedef SeqCfg<D, DVS, SG> G;
    constexpr int NS = D / DVS;
    __shared__ __attribute__((aligned(16))) float smem[G::BYTES / 4];

    const int unit = blockIdx.x;
    if (unit >= units) return;
    const int slice = unit % NS, nh = unit / NS;
    const int h = nh % H, n = nh / H;
    const int v0 = slice * DVS;
    int64_t tbeg, tend;
    if (cu_seqlens) {
        int a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > total_tokens ? total_tokens : a);
        b = b < a ? a : (b > total_tokens ? total_tokens : b);
        tbeg = a;
        tend = b;
    } else {
        tbeg = (int64_t)n * seq_len;
        tend = tbeg + seq_len;
    }
    const int nblk = (int)((tend - tbeg + kSeqT - 1) / kSeqT);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, l4 = lane >> 4;
    const int vcol = v0 + 16 * wave + l16;

    // Snapshots as in the chunked prefill: the state after the first
    // j * snap_every tokens of sequence n goes to entry snap_base + j - 1.
    int snap_base = 0;
    if (snapshots) {
        if (cu_seqlens) {
            int cnt = 0;
            for (int m = lane; m < n; m += 64) {
                int a = cu_seqlens[m], b = cu_seqlens[m + 1];
                a = a < 0 ? 0 : (a > total_tokens ? total_tokens : a);
                b = b < a ? a : (b > total_tokens ? total_tokens : b);
                cnt += (b - a) / snap_every;
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
            snap_base = cnt;
        } else {
            snap_base = n * (seq_len / snap_every);
        }
    }

    const int64_t sbase = ((int64_t)n * H + h) * D * D;  // M = S^T: [d_v][d_k]
    f32x4 Sm[G::NRT];
#pragma unroll
    for (int t = 0; t < G::NRT; ++t) {
        if constexpr (MODE == kModeMap) {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = vcol == 16 * t + 4 * l4 + e ? 1.f : 0.f;
            Sm[t] = x;
        } else {
            Sm[t] = initial_state ? *reinterpret_cast<const f32x4 *>(
                                        initial_state + sbase + (int64_t)vcol * D + 16 * t +
                                        4 * l4)
                                  : zero4();
        }
    }

    // Block b's rows, loaded into registers (16-byte pieces, rows past the
    // sequence end as an inert token: zero k, q, v, beta and alpha = 1, never
    // stepped) and then stored to buffer b & 1, alpha = e^{log_alpha} formed
    // on the way; the next block's loads are in flight while this block is
    // stepped.
    constexpr int Q4 = D / 4, V4 = DVS / 4;  // 16-byte pieces per k / q / v row
    constexpr int PK = kSeqT * Q4 / G::THREADS, PV = kSeqT * V4 / G::THREADS;
    static_assert(PK * G::THREADS == kSeqT * Q4 && PV * G::THREADS == kSeqT * V4, "piece map");
    struct Rows {
        f32x4 k[PK], q[PK], g[PK], v[PV];
        float b, g1;
    };
    auto load = [&](int b, Rows &R) {
        const int64_t t0 = tbeg + (int64_t)b * kSeqT;
        const int nv = (int)((tend - t0) < kSeqT ? (tend - t0) : kSeqT);
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int p = i * G::THREADS + tid, r = p / Q4, c = 4 * (p % Q4);
            R.k[i] = R.q[i] = R.g[i] = zero4();
            if (r < nv) {
                const int64_t base = ((t0 + r) * H + h) * (int64_t)D + c;
                R.k[i] = *reinterpret_cast<const f32x4 *>(k + base);
                R.q[i] = *reinterpret_cast<const f32x4 *>(q + base);
                if constexpr (!SG) R.g[i] = *reinterpret_cast<const f32x4 *>(log_alpha + base);
            }
        }
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int p = i * G::THREADS + tid, r = p / V4, c = 4 * (p % V4);
            R.v[i] = zero4();
            if (r < nv && MODE != kModeMap)
                R.v[i] = *reinterpret_cast<const f32x4 *>(v + ((t0 + r) * H + h) * (int64_t)D +
                                                          v0 + c);
        }
        R.b = 0.f;
        R.g1 = 0.f;
        if (tid < nv) {
            const int64_t row = (t0 + tid) * H + h;
            R.b = beta[row];
            if constexpr (SG) R.g1 = log_alpha[row];
        }
    };
    auto store = [&](int b, const Rows &R) {
        float *S = smem + (b & 1) * G::BLOCK;
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int p = i * G::THREADS + tid, r = p / Q4, c = 4 * (p % Q4);
            *reinterpret_cast<f32x4 *>(S + G::oK + r * G::LDR + c) = R.k[i];
            *reinterpret_cast<f32x4 *>(S + G::oQ + r * G::LDR + c) = R.q[i];
            if constexpr (!SG) {
                f32x4 a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = fast_exp2(R.g[i][e] * kLog2e);
                *reinterpret_cast<f32x4 *>(S + G::oA + r * G::LDR + c) = a;
            }
        }
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int p = i * G::THREADS + tid, r = p / V4, c = 4 * (p % V4);
            *reinterpret_cast<f32x4 *>(S + G::oV + r * G::LDV + c) = R.v[i];
        }
        if (tid < kSeqT) {
            S[G::oB + tid] = R.b;
            if constexpr (SG) S[G::oA + tid] = fast_exp2(R.g1 * kLog2e);
        }
    };

    Rows R;
    if (nblk > 0) {
        load(0, R);
        store(0, R);
    }
    __syncthreads();
    for (int b = 0; b < nblk; ++b) {
        if (b + 1 < nblk) load(b + 1, R);
        const float *S = smem + (b & 1) * G::BLOCK;
        const int64_t t0 = tbeg + (int64_t)b * kSeqT;
        const int nv = (int)((tend - t0) < kSeqT ? (tend - t0) : kSeqT);
        for (int j = 0; j < nv; ++j) {
            const float *kr = S + G::oK + j * G::LDR + 4 * l4;
            const float *qr = S + G::oQ + j * G::LDR + 4 * l4;
            float p = 0.f;
#pragma unroll
            for (int t = 0; t < G::NRT; ++t) {
                const f32x4 kk = *reinterpret_cast<const f32x4 *>(kr + 16 * t);
                f32x4 aa;
                if constexpr (SG) {
                    const float a = S[G::oA + j];
                    aa = f32x4{a, a, a, a};
                } else {
                    aa = *reinterpret_cast<const f32x4 *>(S + G::oA + j * G::LDR + 16 * t + 4 * l4);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Sm[t][e] *= aa[e];
                    p += Sm[t][e] * kk[e];
                }
            }
            p = rows4_sum(p);
            const float dl = S[G::oB + j] * (S[G::oV + j * G::LDV + 16 * wave + l16] - p);
            float o = 0.f;
#pragma unroll
            for (int t = 0; t < G::NRT; ++t) {
                const f32x4 kk = *reinterpret_cast<const f32x4 *>(kr + 16 * t);
                const f32x4 qq = *reinterpret_cast<const f32x4 *>(qr + 16 * t);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Sm[t][e] += kk[e] * dl;
                    o += Sm[t][e] * qq[e];
                }
            }
            if constexpr (MODE == kModeOut) {
                o = rows4_sum(o);
                if (l4 == 0) out[((t0 + j) * H + h) * (int64_t)D + vcol] = o;
            }
        }
        // a snapshot after every snap_every tokens (a multiple of the block)
        const int64_t done = (int64_t)(b + 1) * kSeqT;
        if (snapshots && done % snap_every == 0 && done <= tend - tbeg) {
            const int64_t idx = snap_base + done / snap_every - 1;
            if (idx < snap_cap) {
                float *dst = snapshots + (idx * H + h) * D * D + (int64_t)vcol * D + 4 * l4;
#pragma unroll
                for (int t = 0; t < G::NRT; ++t) *reinterpret_cast<f32x4 *>(dst + 16 * t) = Sm[t];
            }
        }
        if (b + 1 < nblk) store(b + 1, R);  // the other buffer: its last readers left it
        __syncthreads();
    }
    if (final_state) {
#pragma unroll
        for (int t = 0; t < G::NRT; ++t)
            *reinterpret_cast<f32x4 *>(final_state + sbase + (int64_t)vcol * D + 16 * t +
                                       4 * l4) = Sm[t];
    }
}

template <bool SG, int MODE>
int launch_seq(const void *q, const void *k, const void *v, const float *log_alpha,
               const float *beta, const float *initial_state, const int32_t *cu_seqlens,
               void *out, float *final_state, float *snapshots, int snap_every, int snap_cap,
               int num_seqs, int seq_len, int total_tokens, int H, hipStream_t stream) {
    constexpr int D = 128, DVS = 64;
    const int64_t units64 = (int64_t)num_seqs * H * (D / DVS);
    if (units64 == 0) return 0;
    if (units64 > INT32_MAX) return -1;
    hipLaunchKernelGGL((chunk_seq_kernel<D, DVS, SG, MODE>), dim3((unsigned)units64),
                       dim3(SeqCfg<D, DVS, SG>::THREADS), 0, stream,
                       static_cast<const float *>(q), static_cast<const float *>(k),
                       static_cast<const float *>(v), log_alpha, beta, initial_state,
                       cu_seqlens, static_cast<float *>(out), final_state, snapshots,
                       snap_every, snap_cap, num_seqs, seq_len, total_tokens, H, (int)units64);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_chunk_seq(const void *q, const void *k, const void *v, const float *log_alpha,
                     const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                     void *out, float *final_state, float *snapshots, int32_t snapshot_every,
                     int32_t num_snapshots, int32_t num_seqs, int32_t seq_len,
                     int32_t total_tokens, int32_t num_heads, int scalar_gate, int mode,
                     hipStream_t stream) {
#define KDA_SEQ_ARGS                                                                           \
    q, k, v, log_alpha, beta, initial_state, cu_seqlens, out, final_state, snapshots,          \
        snapshot_every, num_snapshots, num_seqs, seq_len, total_tokens, num_heads, stream
    if (scalar_gate) return mode == kModeOut ? launch_seq<true, kModeOut>(KDA_SEQ_ARGS) : -1;
    switch (mode) {
    case kModeOut: return launch_seq<false, kModeOut>(KDA_SEQ_ARGS);
    case kModeState: return launch_seq<false, kModeState>(KDA_SEQ_ARGS);
    case kModeMap: return launch_seq<false, kModeMap>(KDA_SEQ_ARGS);
    default: return -1;
    }
#undef KDA_SEQ_ARGS
}

// ---------------------------------------------------------------------------
// The backward of the token recurrence, for (sequence, head) units whose gates
// leave the chunked backward's range (a 16-token block decaying beyond
// 2^-100 in some channel, or a -inf / NaN gate): the chunked kernels hold
// e^{+-(decay within 16 tokens)}, which overflows there.  A detect pass marks
// such units before the chunked backward runs; after it, bwd_seq_kernel
// recomputes every gradient of the marked units exactly in fp32 (the other
// units return at once), using the chunked backward's workspace (free by then)
// for its state checkpoints.
//
// Reverse-mode derivative of one step ([K3-explainer] §三/§四 forward:
// S' = Diag(a) S_prev, p = S'^T k, delta = b (v - p), S = S' + k delta^T,
// o = S^T q), with G = dL/dS + q do^T the gradient reaching S:
//   d_delta = G^T k,  dS' = G - b k d_delta^T,  dv = b d_delta,
//   db = sum_v d_delta (v - p),  dk = G delta - b S' d_delta,
//   dq = S do,  d log a = a (.) rowsum(dS' (.) S_prev),  dS_prev = Diag(a) dS'.

namespace {

constexpr int kDetectParts = 16;  // detect workgroups per unit
constexpr float kFarLn = 69.31471805599453f;  // 100 ln 2

// Unit u's flag word p (p < kDetectParts) is nonzero if one of the unit's
// 16-token blocks b = p, p + kDetectParts, ... (from the sequence start) has a
// channel whose log_alpha sum is below -kFarLn (or NaN).
template <int D>
__global__ __launch_bounds__(256) void bwd_far_detect_kernel(
    const float *__restrict__ log_alpha, const int32_t *__restrict__ cu_seqlens, int seq_len,
    int total_tokens, int H, unsigned *__restrict__ flags) {
    const int unit = blockIdx.x / kDetectParts, part = blockIdx.x % kDetectParts;
    const int n = unit / H, h = unit % H;
    int64_t tbeg, tend;
    if (cu_seqlens) {
        int a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > total_tokens ? total_tokens : a);
        b = b < a ? a : (b > total_tokens ? total_tokens : b);
        tbeg = a;
        tend = b;
    } else {
        tbeg = (int64_t)n * seq_len;
        tend = tbeg + seq_len;
    }
    const int nblk = (int)((tend - tbeg + 15) / 16);
    const int tid = threadIdx.x;
    // thread (c, half): channel c, every other 16-token block of this part
    const int c = tid % D, half = tid / D;  // D = 128: two threads per channel
    constexpr int SPLIT = 256 / D;
    bool far = false;
    for (int b = part + kDetectParts * half; b < nblk; b += kDetectParts * SPLIT) {
        const int64_t t0 = tbeg + 16 * (int64_t)b;
        const int nv = (int)((tend - t0) < 16 ? (tend - t0) : 16);
        float s = 0.f;
        for (int j = 0; j < nv; ++j) s += log_alpha[((t0 + j) * H + h) * (int64_t)D + c];
        far = far || !(s >= -kFarLn);
    }
    const int any = __syncthreads_or(far ? 1 : 0);
    if (tid == 0) flags[unit * kDetectParts + part] = any ? 1u : 0u;
}

// Sum over the 16 lanes of a row (lanes 16 r .. 16 r + 15); lane 15 of each
// row receives the total.
__device__ __forceinline__ float row_total(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
    return x;
}

template <int D>
struct BwdSeqCfg {
    static constexpr int W = D / 16;  // waves: wave w owns value columns 16 w .. 16 w + 15
    static constexpr int THREADS = 64 * W;
    static constexpr int NT = D / 16;
    static constexpr int LR = D + 4;  // floats per staged row
    // one 16-token block of rows: k, q, alpha, v, d_out, beta
    static constexpr int oK = 0, oQ = oK + 16 * LR, oA = oQ + 16 * LR, oV = oA + 16 * LR,
                         oO = oV + 16 * LR, oB = oO + 16 * LR, BLOCK = oB + 16;
    // per-key partial sums of one token, per wave: dq, dk, d(alpha) rows and db
    static constexpr int PART = 3 * D + 4, oP = BLOCK, FLOATS = oP + 2 * W * PART;
    static_assert(FLOATS * 4 <= 160 * 1024, "LDS budget");
};

template <typename T, int D>
__global__ __launch_bounds__(64 * (D / 16)) void bwd_seq_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ initial_state, const int32_t *__restrict__ cu_seqlens,
    const T *__restrict__ d_out, const float *__restrict__ d_final, T *__restrict__ dq,
    T *__restrict__ dk, T *__restrict__ dv, float *__restrict__ dlog_alpha,
    float *__restrict__ dbeta, float *__restrict__ d_initial, float *__restrict__ ckpt,
    const unsigned *__restrict__ flags, int seq_len, int total_tokens, int H) {
    typedef BwdSeqCfg<D> G;
    constexpr int NT = G::NT, LR = G::LR;
    __shared__ __attribute__((aligned(16))) float sm[G::FLOATS];
    const int unit = blockIdx.x, n = unit / H, h = unit % H;
    unsigned mk = 0;
#pragma unroll
    for (int p = 0; p < kDetectParts; ++p) mk |= flags[unit * kDetectParts + p];
    if (mk == 0) return;  // the chunked backward's results stand

    int64_t tbeg, tend;
    if (cu_seqlens) {
        int a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > total_tokens ? total_tokens : a);
        b = b < a ? a : (b > total_tokens ? total_tokens : b);
        tbeg = a;
        tend = b;
    } else {
        tbeg = (int64_t)n * seq_len;
        tend = tbeg + seq_len;
    }
    const int nblk = (int)((tend - tbeg + 15) / 16);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, l4 = lane >> 4;
    const int vcol = 16 * w + l16;
    const int64_t DD = (int64_t)D * D, sbase = ((int64_t)n * H + h) * DD;
    // this unit's checkpoint slot j: the state entering 16-token block j, fp32
    auto slot = [&](int j) { return ckpt + ((first_slot(tbeg, n) + j) * H + h) * DD; };

    // stage block b's rows as fp32 (alpha = e^{log_alpha}); rows past the end
    // are never stepped
    auto stage = [&](int b, bool with_grad) {
        const int64_t t0 = tbeg + 16 * (int64_t)b;
        const int nv = (int)((tend - t0) < 16 ? (tend - t0) : 16);
        for (int i = tid; i < 16 * D; i += G::THREADS) {
            const int r = i / D, c = i % D;
            float kk = 0.f, qq = 0.f, aa = 1.f, vv = 0.f, oo = 0.f;
            if (r < nv) {
                const int64_t e = ((t0 + r) * H + h) * (int64_t)D + c;
                kk = to_f32(k[e]);
                vv = to_f32(v[e]);
                aa = fast_exp2(log_alpha[e] * kLog2e);
                if (with_grad) {
                    qq = to_f32(q[e]);
                    oo = to_f32(d_out[e]);
                }
            }
            sm[G::oK + r * LR + c] = kk;
            sm[G::oQ + r * LR + c] = qq;
            sm[G::oA + r * LR + c] = aa;
            sm[G::oV + r * LR + c] = vv;
            sm[G::oO + r * LR + c] = oo;
        }
        if (tid < 16) sm[G::oB + tid] = tid < nv ? beta[(t0 + tid) * H + h] : 0.f;
    };
    // one forward step with staged row j: S <- Diag(a) S + k (b (v - (Diag(a) S)^T k))^T
    auto fwd_step = [&](f32x4 (&S)[NT], int j) {
        float p = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(sm + G::oA + j * LR + 16 * t + 4 * l4);
            const f32x4 kk = *reinterpret_cast<const f32x4 *>(sm + G::oK + j * LR + 16 * t + 4 * l4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S[t][e] *= a[e];
                p += S[t][e] * kk[e];
            }
        }
        p = rows4_sum(p);
        const float dl = sm[G::oB + j] * (sm[G::oV + j * LR + vcol] - p);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 kk = *reinterpret_cast<const f32x4 *>(sm + G::oK + j * LR + 16 * t + 4 * l4);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[t][e] += kk[e] * dl;
        }
    };

    // pass 1: the state entering every 16-token block, into the checkpoints
    f32x4 S[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        S[t] = initial_state ? *reinterpret_cast<const f32x4 *>(initial_state + sbase +
                                                                (int64_t)vcol * D + 16 * t + 4 * l4)
                             : zero4();
    for (int b = 0; b < nblk; ++b) {
        float *dst = slot(b) + (int64_t)vcol * D + 4 * l4;
#pragma unroll
        for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4 *>(dst + 16 * t) = S[t];
        __syncthreads();  // the previous block's rows are no longer read
        stage(b, false);
        __syncthreads();
        const int nv = (int)((tend - tbeg - 16 * (int64_t)b) < 16 ? (tend - tbeg - 16 * b) : 16);
        for (int j = 0; j < nv; ++j) fwd_step(S, j);
    }

    // pass 2: dL/dS backwards over the tokens
    f32x4 dS[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        dS[t] = d_final ? *reinterpret_cast<const f32x4 *>(d_final + sbase + (int64_t)vcol * D +
                                                           16 * t + 4 * l4)
                        : zero4();
    int buf = 0;
    for (int b = nblk - 1; b >= 0; --b) {
        __syncthreads();
        stage(b, true);
        f32x4 Sb[NT];
        const float *src = slot(b) + (int64_t)vcol * D + 4 * l4;
#pragma unroll
        for (int t = 0; t < NT; ++t) Sb[t] = *reinterpret_cast<const f32x4 *>(src + 16 * t);
        __syncthreads();
        const int64_t t0 = tbeg + 16 * (int64_t)b;
        const int nv = (int)((tend - t0) < 16 ? (tend - t0) : 16);
        for (int j = nv - 1; j >= 0; --j) {
            // S_prev: the state entering token j of the block, recomputed
#pragma unroll
            for (int t = 0; t < NT; ++t) S[t] = Sb[t];
            for (int i = 0; i < j; ++i) fwd_step(S, i);
            const float bt = sm[G::oB + j];
            // forward quantities of token j
            float p = 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(sm + G::oA + j * LR + 16 * t + 4 * l4);
                const f32x4 kk = *reinterpret_cast<const f32x4 *>(sm + G::oK + j * LR + 16 * t + 4 * l4);
#pragma unroll
                for (int e = 0; e < 4; ++e) p += a[e] * S[t][e] * kk[e];
            }
            p = rows4_sum(p);
            const float vv = sm[G::oV + j * LR + vcol], dlt = bt * (vv - p);
            const float dov = sm[G::oO + j * LR + vcol];
            // d_delta = G^T k with G = dS + q do^T
            float dd = 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const f32x4 kk = *reinterpret_cast<const f32x4 *>(sm + G::oK + j * LR + 16 * t + 4 * l4);
                const f32x4 qq = *reinterpret_cast<const f32x4 *>(sm + G::oQ + j * LR + 16 * t + 4 * l4);
#pragma unroll
                for (int e = 0; e < 4; ++e) dd += (dS[t][e] + qq[e] * dov) * kk[e];
            }
            dd = rows4_sum(dd);
            // per-key partials of this lane's column, summed over the row's 16
            // columns; lane 15 of each row writes its 4 NT key rows
            float *P = sm + G::oP + (buf * G::W + w) * G::PART;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(sm + G::oA + j * LR + 16 * t + 4 * l4);
                const f32x4 kk = *reinterpret_cast<const f32x4 *>(sm + G::oK + j * LR + 16 * t + 4 * l4);
                const f32x4 qq = *reinterpret_cast<const f32x4 *>(sm + G::oQ + j * LR + 16 * t + 4 * l4);
                f32x4 xq, xk, xa;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float sp = a[e] * S[t][e];          // S'
                    const float g = dS[t][e] + qq[e] * dov;   // G
                    const float dsp = g - bt * kk[e] * dd;    // dS'
                    xq[e] = row_total((sp + kk[e] * dlt) * dov);   // dq: S_t do
                    xk[e] = row_total(g * dlt - bt * sp * dd);     // dk
                    xa[e] = row_total(dsp * S[t][e]);              // d alpha
                    dS[t][e] = a[e] * dsp;                         // dL/dS_prev
                }
                if (l16 == 15) {
                    *reinterpret_cast<f32x4 *>(P + 16 * t + 4 * l4) = xq;
                    *reinterpret_cast<f32x4 *>(P + D + 16 * t + 4 * l4) = xk;
                    *reinterpret_cast<f32x4 *>(P + 2 * D + 16 * t + 4 * l4) = xa;
                }
            }
            {
                const float xb = row_total(l4 == 0 ? dd * (vv - p) : 0.f);  // db
                if (l4 == 0 && l16 == 15) P[3 * D] = xb;
            }
            const int64_t tok = t0 + j, row = tok * H + h;
            if (l4 == 0) dv[row * D + vcol] = from_f32<T>(bt * dd);
            __syncthreads();
            // sums over the waves (fixed order): dq, dk, dlog_alpha, dbeta
            for (int i = tid; i < 3 * D + 1; i += G::THREADS) {
                const float *Pb = sm + G::oP + buf * G::W * G::PART;
                float s = 0.f;
                for (int ww = 0; ww < G::W; ++ww) s += Pb[ww * G::PART + i];
                if (i < D) dq[row * D + i] = from_f32<T>(s);
                else if (i < 2 * D) dk[row * D + i - D] = from_f32<T>(s);
                else if (i < 3 * D) dlog_alpha[row * D + i - 2 * D] = s * sm[G::oA + j * LR + i - 2 * D];
                else dbeta[row] = s;
            }
            buf ^= 1;  // the next token's partials go to the other buffer
        }
    }
    if (d_initial) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            *reinterpret_cast<f32x4 *>(d_initial + sbase + (int64_t)vcol * D + 16 * t + 4 * l4) =
                dS[t];
    }
}

template <typename T, int D>
int launch_bwd_seq_t(const void *q, const void *k, const void *v, const float *log_alpha,
                     const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                     const void *d_out, const float *d_final, void *dq, void *dk, void *dv,
                     float *dlog_alpha, float *dbeta, float *d_initial, float *ckpt,
                     const unsigned *flags, int num_seqs, int seq_len, int total_tokens, int H,
                     hipStream_t stream) {
    const int64_t units = (int64_t)num_seqs * H;
    hipLaunchKernelGGL((bwd_seq_kernel<T, D>), dim3((unsigned)units),
                       dim3(BwdSeqCfg<D>::THREADS), 0, stream, static_cast<const T *>(q),
                       static_cast<const T *>(k), static_cast<const T *>(v), log_alpha, beta,
                       initial_state, cu_seqlens, static_cast<const T *>(d_out), d_final,
                       static_cast<T *>(dq), static_cast<T *>(dk), static_cast<T *>(dv),
                       dlog_alpha, dbeta, d_initial, ckpt, flags, seq_len, total_tokens, H);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int64_t bwd_far_flag_words(int64_t num_seqs, int64_t num_heads) {
    return num_seqs * num_heads * kDetectParts;
}

int launch_bwd_far_detect(const float *log_alpha, const int32_t *cu_seqlens, int32_t num_seqs,
                          int32_t seq_len, int32_t total_tokens, int32_t num_heads, int head_dim,
                          unsigned *flags, hipStream_t stream) {
    const int64_t grid = (int64_t)num_seqs * num_heads * kDetectParts;
    if (grid == 0) return 0;
    if (grid > INT32_MAX) return -1;
    if (head_dim == 128)
        hipLaunchKernelGGL((bwd_far_detect_kernel<128>), dim3((unsigned)grid), dim3(256), 0, stream,
                           log_alpha, cu_seqlens, seq_len, total_tokens, num_heads, flags);
    else
        hipLaunchKernelGGL((bwd_far_detect_kernel<64>), dim3((unsigned)grid), dim3(256), 0, stream,
                           log_alpha, cu_seqlens, seq_len, total_tokens, num_heads, flags);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_bwd_seq(const void *q, const void *k, const void *v, const float *log_alpha,
                   const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                   const void *d_out, const float *d_final_state, void *dq, void *dk, void *dv,
                   float *dlog_alpha, float *dbeta, float *d_initial_state, float *ckpt,
                   const unsigned *flags, int32_t num_seqs, int32_t seq_len,
                   int32_t total_tokens, int32_t num_heads, int head_dim, int dtype,
                   hipStream_t stream) {
    if ((int64_t)num_seqs * num_heads == 0) return 0;
#define KDA_BWD_SEQ_ARGS                                                                       \
    q, k, v, log_alpha, beta, initial_state, cu_seqlens, d_out, d_final_state, dq, dk, dv,     \
        dlog_alpha, dbeta, d_initial_state, ckpt, flags, num_seqs, seq_len, total_tokens,      \
        num_heads, stream
    if (dtype == kDtypeBf16)
        return head_dim == 128 ? launch_bwd_seq_t<bf16, 128>(KDA_BWD_SEQ_ARGS)
                               : launch_bwd_seq_t<bf16, 64>(KDA_BWD_SEQ_ARGS);
    return head_dim == 128 ? launch_bwd_seq_t<float, 128>(KDA_BWD_SEQ_ARGS)
                           : launch_bwd_seq_t<float, 64>(KDA_BWD_SEQ_ARGS);
#undef KDA_BWD_SEQ_ARGS
}

}  // namespace kda
