// kda_segment.hip -- the pieces of the segmented prefill of one long sequence
// that the chunk kernel does not cover: segment boundaries and the fold of the
// segments' affine state maps.
//
// Pages cited (by title):
//   [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer (§六.2: a chunk's
//                   rank-one updates collapse to one transition, P = D - K W^T).
//
// A segment of chunks maps its entering state affinely, S_out = P S_in + R
// (the composition of the chunks' transitions).  With R and P^T known for every
// segment (the chunk kernel run from S = 0, and from S = I with zero values),
// the entering states follow by a short sequential fold over the segments.  In
// the stored orientation M = S^T ([d_v][d_k], [K3-memory] §3) the fold is
//     M_{g+1} = M_g X_g + Y_g,   X_g = P_g^T,  Y_g = R_g^T,
// and X_g, Y_g are exactly what the chunk kernel writes as "final states".
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

// cu[g] = min(g * seg_len, total) for g = 0 .. nseg.
__global__ void segment_bounds_kernel(int32_t *cu, int nseg, int seg_len, int total) {
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g <= nseg) {
        const int64_t t = (int64_t)g * seg_len;
        cu[g] = (int32_t)(t < total ? t : total);
    }
}

// One workgroup per head: M <- M X_g + Y_g for g = 0 .. nseg - 1, writing the
// entering state M_g of every segment to m_in[g].  Thread (ti, tj) of a 16 x 16
// grid owns the BR x BR block of rows BR ti.., columns BR tj.. (BR = D / 16);
// M (transposed) and X_g are staged in LDS.  fp32 throughout.
template <int D>
__global__ __launch_bounds__(256) void segment_fold_kernel(const float *__restrict__ m0,
                                                           const float *__restrict__ X,
                                                           const float *__restrict__ Y,
                                                           float *__restrict__ m_in, int nseg,
                                                           int H) {
    constexpr int BR = D / 16, LD = D + 4;
    static_assert(BR % 4 == 0, "fold tiling");
    __shared__ __attribute__((aligned(16))) float sMt[D * LD];  // sMt[k][i] = M[i][k]
    __shared__ __attribute__((aligned(16))) float sX[D * LD];   // sX[k][j] = X[k][j]
    const int h = blockIdx.x, tid = threadIdx.x;
    const int r0 = BR * (tid / 16), c0 = BR * (tid % 16);
    const int64_t hs = (int64_t)D * D;

    float m[BR][BR];
#pragma unroll
    for (int i = 0; i < BR; ++i)
#pragma unroll
        for (int j = 0; j < BR; ++j)
            m[i][j] = m0 ? m0[h * hs + (int64_t)(r0 + i) * D + c0 + j] : 0.f;
    for (int g = 0; g < nseg; ++g) {
        const int64_t base = ((int64_t)g * H + h) * hs;
#pragma unroll
        for (int i = 0; i < BR; ++i) {
#pragma unroll
            for (int j = 0; j < BR; j += 4)
                *reinterpret_cast<f32x4 *>(m_in + base + (int64_t)(r0 + i) * D + c0 + j) =
                    f32x4{m[i][j], m[i][j + 1], m[i][j + 2], m[i][j + 3]};
#pragma unroll
            for (int j = 0; j < BR; ++j) sMt[(c0 + j) * LD + r0 + i] = m[i][j];
        }
        for (int e = 4 * tid; e < D * D; e += 4 * 256) {
            const int k = e / D, j = e % D;
            *reinterpret_cast<f32x4 *>(sX + k * LD + j) =
                *reinterpret_cast<const f32x4 *>(X + base + e);
        }
        __syncthreads();
        float acc[BR][BR];
#pragma unroll
        for (int i = 0; i < BR; ++i)
#pragma unroll
            for (int j = 0; j < BR; j += 4) {
                const f32x4 y =
                    *reinterpret_cast<const f32x4 *>(Y + base + (int64_t)(r0 + i) * D + c0 + j);
                acc[i][j] = y[0]; acc[i][j + 1] = y[1]; acc[i][j + 2] = y[2]; acc[i][j + 3] = y[3];
            }
        for (int kk = 0; kk < D; ++kk) {
            float a[BR], b[BR];
#pragma unroll
            for (int i = 0; i < BR; i += 4) {
                const f32x4 av = *reinterpret_cast<const f32x4 *>(sMt + kk * LD + r0 + i);
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(sX + kk * LD + c0 + i);
                a[i] = av[0]; a[i + 1] = av[1]; a[i + 2] = av[2]; a[i + 3] = av[3];
                b[i] = bv[0]; b[i + 1] = bv[1]; b[i + 2] = bv[2]; b[i + 3] = bv[3];
            }
#pragma unroll
            for (int i = 0; i < BR; ++i)
#pragma unroll
                for (int j = 0; j < BR; ++j) acc[i][j] += a[i] * b[j];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < BR; ++i)
#pragma unroll
            for (int j = 0; j < BR; ++j) m[i][j] = acc[i][j];
    }
}

}  // namespace

int launch_segment_bounds(int32_t *cu, int nseg, int seg_len, int total, hipStream_t stream) {
    hipLaunchKernelGGL(segment_bounds_kernel, dim3((nseg + 1 + 255) / 256), dim3(256), 0, stream,
                       cu, nseg, seg_len, total);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_segment_fold(const float *m0, const float *X, const float *Y, float *m_in, int nseg,
                        int H, int head_dim, hipStream_t stream) {
    if (head_dim == 128)
        hipLaunchKernelGGL(segment_fold_kernel<128>, dim3(H), dim3(256), 0, stream, m0, X, Y,
                           m_in, nseg, H);
    else
        hipLaunchKernelGGL(segment_fold_kernel<64>, dim3(H), dim3(256), 0, stream, m0, X, Y, m_in,
                           nseg, H);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kda
