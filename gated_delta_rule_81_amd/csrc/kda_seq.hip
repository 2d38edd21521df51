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
            p += __shfl_xor(p, 16, 64);
            p += __shfl_xor(p, 32, 64);
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
                o += __shfl_xor(o, 16, 64);
                o += __shfl_xor(o, 32, 64);
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

}  // namespace kda
