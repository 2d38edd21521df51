// kda_device.h -- device-side building blocks for the KDA kernels on gfx950.
//
// Element types, bf16 conversion, the 16x16 MFMA tile contract used by every
// matrix product in the chunk kernel, and DPP lane shifts.  gfx950 only.
//
// MFMA tile contract (CDNA 64-wide waves, 16x16 output tiles):
//   * Operands are read from LDS arrays stored "outer-major, k contiguous":
//     the A operand as A[row][k] and the B operand transposed, Bt[col][k].
//     Lane l reads outer index (l % 16) and a run of k starting at
//     KRUN * (l / 16) (+ KSTEP * step), so both operands use the same
//     lane -> k mapping and the contraction is independent of how the
//     hardware orders k inside one instruction.
//   * The 16x16 fp32 accumulator holds, in lane l, column (l % 16) and rows
//     4 * (l / 16) + e for e = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// 2^x on the transcendental unit (v_exp_f32); inputs here are <= ~+90.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Eight consecutive elements of type T <-> eight floats (16/32-byte accesses).
// Native clang vectors only: HIP's float4/uint4 are union-based classes that
// the optimiser cannot always keep in registers.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
    typedef u32x4 raw;  // 16 bytes
    __device__ static void to_float(const raw &r, float (&f)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(r[i] << 16);
            f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
        }
    }
    __device__ static raw zero() { return raw{0u, 0u, 0u, 0u}; }
};
template <> struct Vec8<float> {
    typedef f32x8 raw;  // 32 bytes
    __device__ static void to_float(const raw &r, float (&f)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = r[i];
    }
    __device__ static raw zero() { return raw{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}; }
};

template <typename T>
__device__ __forceinline__ typename Vec8<T>::raw load8(const T *p) {
    return *reinterpret_cast<const typename Vec8<T>::raw *>(p);
}

// Store eight floats as eight consecutive T (p must be 16-byte aligned).
__device__ __forceinline__ void store8(bf16 *p, const float (&f)[8]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<bf16>(f[i]);
    *reinterpret_cast<bf16x8 *>(p) = v;
}
__device__ __forceinline__ void store8(float *p, const float (&f)[8]) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}

// Store two floats as two consecutive T.
__device__ __forceinline__ void store2(bf16 *p, float a, float b) {
    bf16x2 v;
    v[0] = static_cast<bf16>(a);
    v[1] = static_cast<bf16>(b);
    *reinterpret_cast<bf16x2 *>(p) = v;
}
__device__ __forceinline__ void store2(float *p, float a, float b) {
    *reinterpret_cast<f32x2 *>(p) = f32x2{a, b};
}

// Store four floats as four consecutive T.
__device__ __forceinline__ void store4(bf16 *p, float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = static_cast<bf16>(a); v[1] = static_cast<bf16>(b);
    v[2] = static_cast<bf16>(c); v[3] = static_cast<bf16>(d);
    *reinterpret_cast<bf16x4 *>(p) = v;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{a, b, c, d};
}

// ---------------------------------------------------------------------------
// 16x16 MFMA with operands of type T read from LDS (see the contract above).
template <typename T> struct Mma;

// bf16: v_mfma_f32_16x16x32_bf16, eight k per lane per step.
template <> struct Mma<bf16> {
    static constexpr int KSTEP = 32;
    typedef bf16x8 Frag;
    __device__ static Frag load(const bf16 *base, int ld, int lane) {
        return *reinterpret_cast<const bf16x8 *>(base + (lane & 15) * ld + 8 * (lane >> 4));
    }
    // Same fragment with every element multiplied by scale[k] (k along the run).
    __device__ static Frag load_scaled(const bf16 *base, int ld, const float *scale, int lane) {
        const Frag raw = load(base, ld, lane);
        const float *s = scale + 8 * (lane >> 4);
        Frag out;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            out[i] = static_cast<bf16>(static_cast<float>(raw[i]) * s[i]);
        return out;
    }
    __device__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

// fp32: v_mfma_f32_16x16x4_f32, one k per lane per step.
template <> struct Mma<float> {
    static constexpr int KSTEP = 4;
    typedef float Frag;
    __device__ static Frag load(const float *base, int ld, int lane) {
        return base[(lane & 15) * ld + (lane >> 4)];
    }
    __device__ static Frag load_scaled(const float *base, int ld, const float *scale, int lane) {
        return load(base, ld, lane) * scale[lane >> 4];
    }
    __device__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// acc += A[16 x K] * B[K x 16] with A stored A[row][k] (leading dim lda) and
// B stored transposed Bt[col][k] (leading dim ldb); K a multiple of KSTEP.
template <typename T, int K>
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const T *A, int lda, const T *Bt, int ldb,
                                          int lane) {
    typedef Mma<T> M;
#pragma unroll
    for (int k = 0; k < K; k += M::KSTEP)
        acc = M::mma(M::load(A + k, lda, lane), M::load(Bt + k, ldb, lane), acc);
    return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// DPP: value of lane (l - n) within the same 16-lane row; lanes without a
// source (l % 16 < n) receive 0.
template <int N>
__device__ __forceinline__ float dpp_row_shr(float x) {
    static_assert(N >= 1 && N <= 15, "row_shr range");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf,
                                                      true));
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64);
// every lane of the group receives the sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Keep the compiler from moving LDS accesses across this point (one wave's
// own LDS traffic is processed in program order by the hardware).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace kda
