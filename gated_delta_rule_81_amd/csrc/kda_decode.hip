// kda_decode.hip -- single-token KDA decode: stream every state row once,
// update it in place, read the output.
//
// Pages cited (by title):
//   [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer.
//   [K3-memory]     "Kimi K3 Changed the Memory Math for Agentic AI Forever".
//
// Per session b and head h the state is M = S^T, [d_v][d_k] fp32 ([K3-memory]
// §3 layout).  Row v of M is column v of S, i.e. the value channel v of every
// key channel, and the predict/correct step of [K3-explainer] §三/§四 touches
// each row independently:
//     m'  = alpha (.) m                (Diag(alpha) S: decay along key channels)
//     p   = <m', k>                    (v_hat[v] = (S'^T k)[v])
//     d   = beta * (v[v] - p)          (beta * error)
//     m   = m' + d k                   (S' + beta k e^T, column v)
//     o_v = <m, q> = <m', q> + d <k, q>
// so one pass reads and writes every state byte exactly once: the kernel is a
// pure HBM stream (about 0.86 flop per byte) and is written for bandwidth:
// 16-byte coalesced loads and stores, all of a workgroup's state rows in flight
// before any arithmetic, no LDS round trip for the state.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// One workgroup (4 waves) per (session, head).  A state row of D floats is
// held by D/4 lanes, four consecutive key channels each.
// SG: one gate per (session, head) applied to every key channel (the Gated
// DeltaNet gate); otherwise one per key channel.
template <typename T, int D, bool SG>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    float *__restrict__ state, T *__restrict__ out) {
    constexpr int kLanesPerRow = D / 4;
    constexpr int kRowsPerStep = 64 / kLanesPerRow;  // rows one wave touches per instruction
    constexpr int kRowsPerWave = D / 4;              // D rows over 4 waves
    constexpr int kSteps = kRowsPerWave / kRowsPerStep;
    static_assert(kSteps * kRowsPerStep * 4 == D, "row tiling");

    __shared__ float s_val[D];
    __shared__ float s_out[D];

    const int64_t unit = blockIdx.x;  // b * H + h
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int c4 = lane % kLanesPerRow;   // this lane's key channels: 4*c4 .. 4*c4+3
    const int sub = lane / kLanesPerRow;  // which of the wave's rows this lane is on

    float *S = state + unit * (int64_t)(D * D);
    const int row0 = wave * kRowsPerWave + sub;

    // Issue every state load of this lane first: the whole 64 KB (D=128) of
    // the unit is in flight before the first arithmetic instruction.
    f32x4 m[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i)
        m[i] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(S + (int64_t)(row0 + i * kRowsPerStep) * D) + c4);

    const int64_t vec = unit * D;
    float kf[4], qf[4], af[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kf[j] = to_f32(k[vec + 4 * c4 + j]);
        qf[j] = to_f32(q[vec + 4 * c4 + j]);
    }
    if constexpr (SG) {
        const float a = fast_exp2(log_alpha[unit] * kLog2e);
        af[0] = af[1] = af[2] = af[3] = a;
    } else {
        const float4 g4 = *reinterpret_cast<const float4 *>(log_alpha + vec + 4 * c4);
        af[0] = fast_exp2(g4.x * kLog2e);
        af[1] = fast_exp2(g4.y * kLog2e);
        af[2] = fast_exp2(g4.z * kLog2e);
        af[3] = fast_exp2(g4.w * kLog2e);
    }
    const float b = beta[unit];
    if (tid < D) s_val[tid] = to_f32(v[vec + tid]);

    float kq = kf[0] * qf[0] + kf[1] * qf[1] + kf[2] * qf[2] + kf[3] * qf[3];
    kq = group_sum<kLanesPerRow>(kq);
    __syncthreads();

#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int row = row0 + i * kRowsPerStep;
        const float mp[4] = {m[i][0] * af[0], m[i][1] * af[1], m[i][2] * af[2], m[i][3] * af[3]};
        float p = mp[0] * kf[0] + mp[1] * kf[1] + mp[2] * kf[2] + mp[3] * kf[3];
        float r = mp[0] * qf[0] + mp[1] * qf[1] + mp[2] * qf[2] + mp[3] * qf[3];
        p = group_sum<kLanesPerRow>(p);
        r = group_sum<kLanesPerRow>(r);
        const float d = b * (s_val[row] - p);
        const f32x4 mn = {mp[0] + d * kf[0], mp[1] + d * kf[1], mp[2] + d * kf[2],
                          mp[3] + d * kf[3]};
        __builtin_nontemporal_store(mn, reinterpret_cast<f32x4 *>(S + (int64_t)row * D) + c4);
        if (c4 == 0) s_out[row] = r + d * kq;
    }
    __syncthreads();
    if (tid < D) out[vec + tid] = from_f32<T>(s_out[tid]);
}

template <typename T, int D, bool SG>
static int launch_decode(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, float *state, void *out, int64_t units,
                         hipStream_t stream) {
    hipLaunchKernelGGL((decode_step_kernel<T, D, SG>), dim3((unsigned)units), dim3(256), 0,
                       stream, static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), log_alpha, beta, state, static_cast<T *>(out));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <bool SG>
static int launch_decode_dtype(const void *q, const void *k, const void *v,
                               const float *log_alpha, const float *beta, float *state, void *out,
                               int64_t units, int head_dim, int dtype, hipStream_t stream) {
    if (dtype == kDtypeBf16) {
        return head_dim == 128 ? launch_decode<bf16, 128, SG>(q, k, v, log_alpha, beta, state,
                                                              out, units, stream)
                               : launch_decode<bf16, 64, SG>(q, k, v, log_alpha, beta, state,
                                                             out, units, stream);
    }
    return head_dim == 128
               ? launch_decode<float, 128, SG>(q, k, v, log_alpha, beta, state, out, units, stream)
               : launch_decode<float, 64, SG>(q, k, v, log_alpha, beta, state, out, units, stream);
}

int launch_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                       const float *beta, float *state, void *out, int64_t units, int head_dim,
                       int dtype, int scalar_gate, hipStream_t stream) {
    if (units == 0) return 0;
    return scalar_gate ? launch_decode_dtype<true>(q, k, v, log_alpha, beta, state, out, units,
                                                   head_dim, dtype, stream)
                       : launch_decode_dtype<false>(q, k, v, log_alpha, beta, state, out, units,
                                                    head_dim, dtype, stream);
}

}  // namespace kda
