// mfma_chain.hip -- test-only probe: the result of one bf16 MFMA shape fed
// straight in as the accumulator of the other, back to back, on gfx950.
//
// The backward kernels keep each product in its own accumulator because a
// 16x16x32 result chained into a 16x16x16 product once gave wrong values in
// two of four accumulator components (no cause established).  This probe runs
// both chain orders, dependent and back to back, plus the separate-
// accumulator form, on one 16 x 16 tile, so that the test can compare every
// element with a CPU sum of the same bf16 products.
//
//   out[0]: C = A2 B2 + A1 B1, the 16x16x32 product first, chained into 16x16x16
//   out[1]: C = A1 B1 + A2 B2, the 16x16x16 product first, chained into 16x16x32
//   out[2]: the two products in separate accumulators, summed on the VALU
//   out[3]: as out[0] with 16 more wait cycles between the two products
// A1 [16 x 16], B1 [16 x 16] (16x16x16 operands), A2 [16 x 32], B2 [32 x 16]
// (16x16x32 operands), all bf16 row-major; out [4][16][16] fp32 row-major.
// Lane layout (both shapes): lane l supplies row l % 16 of A and column
// l % 16 of B; 16x16x16 takes k = 4 (l / 16) + e (e < 4), 16x16x32 takes
// k = 8 (l / 16) + e (e < 8); the accumulator holds rows 4 (l / 16) + e of
// column l % 16.
#include <hip/hip_runtime.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void mfma_chain_kernel(const __bf16 *a1, const __bf16 *b1,
                                                        const __bf16 *a2, const __bf16 *b2,
                                                        float *out) {
    const int l = threadIdx.x, r = l & 15, g = l >> 4;
    __bf16 x1[4], y1[4];
    bf16x8 x2, y2;
    for (int e = 0; e < 4; ++e) {
        x1[e] = a1[r * 16 + 4 * g + e];
        y1[e] = b1[(4 * g + e) * 16 + r];
    }
    for (int e = 0; e < 8; ++e) {
        x2[e] = a2[r * 32 + 8 * g + e];
        y2[e] = b2[(8 * g + e) * 16 + r];
    }
    i16x4 p1 = __builtin_bit_cast(i16x4, x1), q1 = __builtin_bit_cast(i16x4, y1);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    // each form in its own scheduling region, its operands opaque to the
    // compiler so that no product is shared or moved between forms: the two
    // products of a chain stay back to back
    auto fence = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" : "+v"(x2), "+v"(y2), "+v"(p1), "+v"(q1));
        __builtin_amdgcn_sched_barrier(0);
    };
    // 16x16x32 first, its result straight into the 16x16x16 accumulator
    f32x4 c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x2, y2, z, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p1, q1, c0, 0, 0, 0);
    fence();
    // the same chain with extra independent cycles between the two products
    f32x4 c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x2, y2, z, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p1, q1, c3, 0, 0, 0);
    fence();
    // 16x16x16 first, into the 16x16x32 accumulator
    f32x4 c1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p1, q1, z, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x2, y2, c1, 0, 0, 0);
    fence();
    // separate accumulators
    const f32x4 s1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p1, q1, z, 0, 0, 0);
    fence();
    const f32x4 s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x2, y2, z, 0, 0, 0);
    for (int e = 0; e < 4; ++e) {
        const int row = 4 * g + e;
        out[0 * 256 + row * 16 + r] = c0[e];
        out[1 * 256 + row * 16 + r] = c1[e];
        out[2 * 256 + row * 16 + r] = s1[e] + s2[e];
        out[3 * 256 + row * 16 + r] = c3[e];
    }
}

extern "C" int mfma_chain(const void *a1, const void *b1, const void *a2, const void *b2,
                          float *out, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_chain_kernel, dim3(1), dim3(64), 0, stream,
                       static_cast<const __bf16 *>(a1), static_cast<const __bf16 *>(b1),
                       static_cast<const __bf16 *>(a2), static_cast<const __bf16 *>(b2), out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
