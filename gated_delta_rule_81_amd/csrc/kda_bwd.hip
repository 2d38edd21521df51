// kda_bwd.hip -- chunked backward of the KDA forward pass (gradients of the
// outputs and the final state with respect to q, k, v, log_alpha, beta and
// the initial state), fp32 arithmetic on the matrix cores.
//
// Pages cited (by title):
//   [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer (§四: the KDA
//                   update; §六.2: a chunk's updates as matrix products).
//   [Kimi-Linear]   "Kimi Linear 最多砍掉 75% KV Cache：全注意力真要退场了吗？"
//                   (ai.concitech.org), the section on KDA's per-channel
//                   forgetting: the chunkwise kernel exists so that training
//                   runs as matrix products.
//
// The pages give no gradient; this is the reverse-mode derivative of the
// chunk form of the forward, per chunk of C = 16 tokens with entering state
// S0 (d_k x d_v) and Gamma = the within-chunk prefix of log_alpha:
//   K+ = K e^G, K- = K e^-G, Q+ = Q e^G, Ke = K e^(G_last - G), gam = e^G_last,
//   A = StrictTril(diag(b) K+ K-^T), M = Tril(Q+ K-^T), T = (I + A)^-1,
//   X = V - K+ S0,  Delta = T diag(b) X,
//   O = Q+ S0 + M Delta,  S_C = diag(gam) S0 + Ke^T Delta.
// Given dO and dS_C:
//   dDelta = M^T dO + Ke dS_C,  lam = T^T dDelta,  dX = dV = diag(b) lam,
//   dA = -StrictTril(lam Delta^T),  P = diag(b) dA,  dM = Tril(dO Delta^T),
//   db = rowsum(X * lam) + rowsum(dA * K+K-^T),
//   dQ+ = dO S0^T + dM K-,  dK+ = -dX S0^T + P K-,  dK- = dM^T Q+ + P^T K+,
//   dKe = Delta dS_C^T,  dS0 = diag(gam) dS_C + Q+^T dO - K+^T dX,
//   dG_last = gam * rowsum(S0 * dS_C) + colsum(dKe * Ke),
//   dQ = dQ+ e^G,  dK = dK+ e^G + dK- e^-G + dKe e^(G_last - G),
//   dlog_alpha[t] = sum_{i >= t} (dO S0^T * Q+ - dX S0^T * K+)[i]
//                 + sum_{j < t} (dKe * Ke)[j] + gam * rowsum(S0 * dS_C)
//                 + sum_{i >= t > j} (dM[i][j] Q+[i] + P[i][j] K+[i]) K-[j],
// i.e. every factor e^{G_a - G_b} (a > b) of the chunk form that alpha_t
// enters (b < t <= a), weighted by its gradient.  This equals the suffix sum
// of dG = dQ+ Q+ + dK+ K+ - dK- K- - dKe Ke (+ dG_last on the last row) but
// adds no pair that cancels, so it keeps its relative precision for strongly
// decaying gates.
// A ragged last chunk is padded with zero rows (and zero gates), which add
// nothing.  16-token chunks keep e^(+-G) within fp32 where no 16-token block
// decays beyond 2^-100 in a channel; (sequence, head) pairs with such a block
// (or a -inf gate) are redone token by token afterwards (bwd_seq_kernel).
//
// The dS recursion, dS_prev = diag(gam) dS_C + Q+^T dO - K+^T dX, with dX =
// diag(b) T^T (M^T dO + Ke dS_C), involves no forward state, so the work is
// split over launches on one stream:
//   1. every chunk's entering state S0 into the workspace (the prefill kernel's
//      states mode; for fp32 at d = 128 the chain kernel's pass 1 instead);
//   2. the chain kernel, two workgroups per (sequence, head), one per half of
//      the value columns (kBwdChainHalf; four, kBwdChainQuarter, at d = 128
//      when four per pair still fit on the device's CUs; kBwdChain, one
//      workgroup per head, where pass 1 runs in it): the dS recursion over the
//      chunks in reverse, dS_C of every chunk into the workspace's second
//      region;
//   3. the gradient kernel (kBwdGrad), one workgroup per (16-token slot, head):
//      every other gradient of its chunk from its S0 and dS_C.
// D / 16 waves per workgroup.  States are held in registers in two
// orientations: wave w owns value columns 16w.. of S (for products that
// contract over d_k) and key columns 16w.. of M = S^T (for products that
// contract over d_v), so no product needs a cross-wave reduction.  Chunk
// operands are staged in LDS as fp32.
#include <atomic>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_lanes.h"
#include "kda_slots.h"

namespace kda {

namespace {

constexpr int kBC = 16;  // tokens per chunk of the backward
static_assert(kBC == kSlotTokens, "one workspace slot per chunk");

template <int D, bool GRAD>
struct BwdCfg {
    static constexpr int W = D / 16;  // waves; also 16-wide tiles along d
    static constexpr int THREADS = 64 * W;
    static constexpr int LD = D + 4;   // row stride of [16][D] arrays (floats)
    static constexpr int LS = 20;      // row stride of 16 x 16 arrays (16-byte rows)
    static constexpr int ROW = kBC * LD;
    static constexpr int SQ = kBC * LS;
    // lambda (gradient kernel only) takes V's rows: each lane reads its V
    // entries (for X) before it writes the same entries of lambda
    static constexpr int oQp = 0, oKp = ROW, oKm = 2 * ROW, oKe = 3 * ROW, oG = 4 * ROW,
                         oV = 5 * ROW, oDO = 6 * ROW, oDl = 7 * ROW, oLm = oV;
    // P shares A's space (A is dead once T is formed) and dM shares M's (M is
    // last read before the barrier that precedes dM)
    static constexpr int oBr = 8 * ROW, oA = oBr + SQ, oM = oA + SQ, oT = oM + SQ,
                         oTt = oT + SQ, oP = oA, oDM = oM;
    static constexpr int oGam = oTt + SQ, oBeta = oGam + D, oDB = oBeta + kBC;
    static constexpr int oX = oDB + (W + 1) * kBC;
    // the chain kernel: transposed Q+ and K+ ([D][16], row stride LDT), then
    // the split chain's partial K_end dS tiles (one f32x4 per lane and wave)
    static constexpr int LDT = kBC + 4, oQT = oX, oKT = oQT + (GRAD ? 0 : D * LDT),
                         oXC = oKT + (GRAD ? 0 : D * LDT), XEND = oXC + (GRAD ? 0 : W * 64 * 4);
    // A transposed (column m of A as a row), read by the triangular solve
    static constexpr int oAt = XEND, FLOATS_ALL = oAt + SQ;
};

__device__ __forceinline__ f32x4 mf(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The products below follow one lane contract (v_mfma_f32_16x16x4f32): lane
// l supplies row i = l % 16 of A and column j = l % 16 of B for contraction
// indices chosen by g = l / 16, and holds output rows 4g + e (e = 0..3) of
// column l % 16.  The contraction index of step e within a 16-block is
// 4g + e, identical on both operands.

// A row-major in LDS (A[i][kk]), B from registers: B[t][e] = B[kk = 16t+4g+e][j].
template <int NT>
__device__ __forceinline__ f32x4 mm_lds_reg(f32x4 acc, const float *A, int lda,
                                            const f32x4 (&B)[NT], int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(A + r * lda + 16 * t + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mf(a[e], B[t][e], acc);
    }
    return acc;
}

// A row-major 16 x 16 in LDS, B a register tile: B[e] = B[kk = 4g+e][j].
__device__ __forceinline__ f32x4 mm_lds_tile(f32x4 acc, const float *A, int lda, const f32x4 &B,
                                             int lane) {
    const int r = lane & 15, g = lane >> 4;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(A + r * lda + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mf(a[e], B[e], acc);
    return acc;
}

// A row-major in LDS, B given by rows of Bt (Bt[j][kk]), contraction K.
template <int K>
__device__ __forceinline__ f32x4 mm_lds_ldst(f32x4 acc, const float *A, int lda, const float *Bt,
                                             int ldb, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < K / 16; ++kb) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(A + r * lda + 16 * kb + 4 * g);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(Bt + r * ldb + 16 * kb + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mf(a[e], b[e], acc);
    }
    return acc;
}

// A given transposed (A[i][kk] = At[kk][i]), B row-major (Bm[kk][j]), contraction 16.
__device__ __forceinline__ f32x4 mm_ldst_lds(f32x4 acc, const float *At, int lda, const float *Bm,
                                             int ldb, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        acc = mf(At[(4 * g + e) * lda + r], Bm[(4 * g + e) * ldb + r], acc);
    return acc;
}

// A row-major 16 x 16 in LDS, B row-major (Bm[kk][j]), contraction 16.
__device__ __forceinline__ f32x4 mm_lds_lds(f32x4 acc, const float *A, int lda, const float *Bm,
                                            int ldb, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(A + r * lda + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mf(a[e], Bm[(4 * g + e) * ldb + r], acc);
    return acc;
}

// A given transposed (A[i][kk] = At[kk][i]), B a register tile, contraction 16.
__device__ __forceinline__ f32x4 mm_ldst_tile(f32x4 acc, const float *At, int lda,
                                              const f32x4 &B, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mf(At[(4 * g + e) * lda + r], B[e], acc);
    return acc;
}

// The same products with bf16 operands (fp32 accumulation) for bf16 inputs:
// v_mfma_f32_16x16x32_bf16 for the d-long contractions (lane group g takes
// k = 32b + 4g + e and 32b + 16 + 4g + e, e = 0..3, on both operands, so two
// 16-row register tiles form one B fragment) and v_mfma_f32_16x16x16_bf16 for
// the 16-long ones (lane group g takes k = 4g + e, the f32 path's order).
__device__ __forceinline__ bf16x8 pack8(const f32x4 &a, const f32x4 &b) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = static_cast<bf16>(a[e]);
        r[4 + e] = static_cast<bf16>(b[e]);
    }
    return r;
}
__device__ __forceinline__ i16x4 pack4(float a, float b, float c, float d) {
    bf16x4 r;
    r[0] = static_cast<bf16>(a);
    r[1] = static_cast<bf16>(b);
    r[2] = static_cast<bf16>(c);
    r[3] = static_cast<bf16>(d);
    return __builtin_bit_cast(i16x4, r);
}
__device__ __forceinline__ f32x4 mf32(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mf16(const i16x4 &a, const i16x4 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// fp32 A rows from LDS (packed to bf16 here) times B tiles of four bf16 as
// loaded (tile t: k = 16 t + 4 g + e), contraction 16 NT
template <int NT>
__device__ __forceinline__ f32x4 mm_lds_raw(f32x4 acc, const float *A, int lda,
                                            const u32x2 (&B)[NT], int lane) {
    static_assert(NT % 2 == 0, "bf16 products take tiles in pairs");
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int b = 0; b < NT / 2; ++b) {
        const float *a0 = A + r * lda + 32 * b + 4 * g;
        acc = mf32(pack8(*reinterpret_cast<const f32x4 *>(a0),
                         *reinterpret_cast<const f32x4 *>(a0 + 16)),
                   __builtin_bit_cast(bf16x8, u32x4{B[2 * b][0], B[2 * b][1], B[2 * b + 1][0],
                                                    B[2 * b + 1][1]}),
                   acc);
    }
    return acc;
}

template <bool BF>
struct Prod;

template <>
struct Prod<false> {
    template <int NT>
    __device__ static f32x4 lds_reg(f32x4 acc, const float *A, int lda, const f32x4 (&B)[NT],
                                    int lane) {
        return mm_lds_reg(acc, A, lda, B, lane);
    }
    __device__ static f32x4 lds_tile(f32x4 acc, const float *A, int lda, const f32x4 &B,
                                     int lane) {
        return mm_lds_tile(acc, A, lda, B, lane);
    }
    template <int K>
    __device__ static f32x4 lds_ldst(f32x4 acc, const float *A, int lda, const float *Bt, int ldb,
                                     int lane) {
        return mm_lds_ldst<K>(acc, A, lda, Bt, ldb, lane);
    }
    __device__ static f32x4 ldst_lds(f32x4 acc, const float *At, int lda, const float *Bm, int ldb,
                                     int lane) {
        return mm_ldst_lds(acc, At, lda, Bm, ldb, lane);
    }
    __device__ static f32x4 lds_lds(f32x4 acc, const float *A, int lda, const float *Bm, int ldb,
                                    int lane) {
        return mm_lds_lds(acc, A, lda, Bm, ldb, lane);
    }
    __device__ static f32x4 ldst_tile(f32x4 acc, const float *At, int lda, const f32x4 &B,
                                      int lane) {
        return mm_ldst_tile(acc, At, lda, B, lane);
    }
};

template <>
struct Prod<true> {
    template <int NT>
    __device__ static f32x4 lds_reg(f32x4 acc, const float *A, int lda, const f32x4 (&B)[NT],
                                    int lane) {
        static_assert(NT % 2 == 0, "bf16 products take register tiles in pairs");
        const int r = lane & 15, g = lane >> 4;
#pragma unroll
        for (int b = 0; b < NT / 2; ++b) {
            const float *a0 = A + r * lda + 32 * b + 4 * g;
            acc = mf32(pack8(*reinterpret_cast<const f32x4 *>(a0),
                             *reinterpret_cast<const f32x4 *>(a0 + 16)),
                       pack8(B[2 * b], B[2 * b + 1]), acc);
        }
        return acc;
    }
    __device__ static f32x4 lds_tile(f32x4 acc, const float *A, int lda, const f32x4 &B,
                                     int lane) {
        const int r = lane & 15, g = lane >> 4;
        const f32x4 a = *reinterpret_cast<const f32x4 *>(A + r * lda + 4 * g);
        return mf16(pack4(a[0], a[1], a[2], a[3]), pack4(B[0], B[1], B[2], B[3]), acc);
    }
    template <int K>
    __device__ static f32x4 lds_ldst(f32x4 acc, const float *A, int lda, const float *Bt, int ldb,
                                     int lane) {
        const int r = lane & 15, g = lane >> 4;
#pragma unroll
        for (int b = 0; b < K / 32; ++b) {
            const float *a0 = A + r * lda + 32 * b + 4 * g;
            const float *b0 = Bt + r * ldb + 32 * b + 4 * g;
            acc = mf32(pack8(*reinterpret_cast<const f32x4 *>(a0),
                             *reinterpret_cast<const f32x4 *>(a0 + 16)),
                       pack8(*reinterpret_cast<const f32x4 *>(b0),
                             *reinterpret_cast<const f32x4 *>(b0 + 16)),
                       acc);
        }
        return acc;
    }
    __device__ static f32x4 ldst_lds(f32x4 acc, const float *At, int lda, const float *Bm, int ldb,
                                     int lane) {
        const int r = lane & 15, g = lane >> 4;
        const float *a0 = At + 4 * g * lda + r, *b0 = Bm + 4 * g * ldb + r;
        return mf16(pack4(a0[0], a0[lda], a0[2 * lda], a0[3 * lda]),
                    pack4(b0[0], b0[ldb], b0[2 * ldb], b0[3 * ldb]), acc);
    }
    __device__ static f32x4 lds_lds(f32x4 acc, const float *A, int lda, const float *Bm, int ldb,
                                    int lane) {
        const int r = lane & 15, g = lane >> 4;
        const f32x4 a = *reinterpret_cast<const f32x4 *>(A + r * lda + 4 * g);
        const float *b0 = Bm + 4 * g * ldb + r;
        return mf16(pack4(a[0], a[1], a[2], a[3]),
                    pack4(b0[0], b0[ldb], b0[2 * ldb], b0[3 * ldb]), acc);
    }
    __device__ static f32x4 ldst_tile(f32x4 acc, const float *At, int lda, const f32x4 &B,
                                      int lane) {
        const int r = lane & 15, g = lane >> 4;
        const float *a0 = At + 4 * g * lda + r;
        return mf16(pack4(a0[0], a0[lda], a0[2 * lda], a0[3 * lda]),
                    pack4(B[0], B[1], B[2], B[3]), acc);
    }
};

// Every lane of a group of 4 receives x from lane SRC of its group (DPP
// quad_perm, all lanes active).
template <int SRC>
__device__ __forceinline__ float quad_bcast(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), SRC * 0x55, 0xf, 0xf, false));
}

// The workspace's checkpoints (chunk-entering states in the first region,
// chunk-end gradients in the second) are kept in the input dtype: bf16 for
// bf16 inputs, whose matrix products read them as bf16 operands anyway (only
// the fp32 row sums behind dG_last see the rounding).  `base` points at a
// slot of a region; offsets count elements.
template <typename T>
__device__ __forceinline__ void ckpt_store(float *base, int64_t off, const f32x4 &x) {
    if constexpr (sizeof(T) == 2) {
        bf16x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = static_cast<bf16>(x[e]);
        *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(base) + off) = h;
    } else {
        *reinterpret_cast<f32x4 *>(base + off) = x;
    }
}
// (offsets of any integer type: an unsigned one lets the compiler address a
// uniform base plus a 32-bit lane offset)
template <typename T, typename I>
__device__ __forceinline__ f32x4 ckpt_load4(const float *base, I off) {
    if constexpr (sizeof(T) == 2) {
        const bf16x4 h =
            *reinterpret_cast<const bf16x4 *>(reinterpret_cast<const bf16 *>(base) + off);
        return f32x4{static_cast<float>(h[0]), static_cast<float>(h[1]),
                     static_cast<float>(h[2]), static_cast<float>(h[3])};
    } else {
        return *reinterpret_cast<const f32x4 *>(base + off);
    }
}
template <typename T, typename I>
__device__ __forceinline__ float ckpt_load1(const float *base, I off) {
    if constexpr (sizeof(T) == 2)
        return static_cast<float>(reinterpret_cast<const bf16 *>(base)[off]);
    else
        return base[off];
}

// base advanced by off elements of T (bf16 or fp32 checkpoints)
template <typename T>
__device__ __forceinline__ const float *ckpt_at(const float *base, int64_t off) {
    return sizeof(T) == 2
               ? reinterpret_cast<const float *>(reinterpret_cast<const bf16 *>(base) + off)
               : base + off;
}

// acc + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs (v_dot2c_f32_bf16,
// fp32 accumulation).  Written as an instruction: the compiler's builtin for it
// has been seen to take the first pair's registers for every pair of a vector.
// The compiler does not see a dot instruction inside inline assembly, so the
// block carries its own wait states: another VALU instruction that reads a dot
// product's result needs three after it (without them the row sums read stale
// values whenever the scheduler puts their consumer right behind the block).
__device__ __forceinline__ float dot2_bf16(unsigned a, unsigned b, float acc) {
    asm volatile("v_dot2c_f32_bf16 %0, %1, %2\n\ts_nop 3" : "+v"(acc) : "v"(a), "v"(b));
    return acc;
}

// Keeps the scheduler from hoisting the LDS reads of later products above
// this point (which would hold their operands in registers early).
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }

// Sum over the 16 lanes of a row group (lanes with equal l / 16).
__device__ __forceinline__ float row16_sum(float x) { return row16_total(x); }

// One thread's raw inputs of a chunk row piece: four elements as stored.
template <typename T> struct RawIn;
template <> struct RawIn<bf16> {
    typedef u32x2 W;
    W q, k, v, o;
    f32x4 g;
    float b;
    __device__ static W ld(const bf16 *p) {
        return __builtin_nontemporal_load(reinterpret_cast<const W *>(p));
    }
    __device__ static W zero() { return W{0u, 0u}; }
    __device__ static f32x4 f32(const W &w) {
        return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                     __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
    }
};
template <> struct RawIn<float> {
    typedef f32x4 W;
    W q, k, v, o;
    f32x4 g;
    float b;
    __device__ static W ld(const float *p) {
        return __builtin_nontemporal_load(reinterpret_cast<const W *>(p));
    }
    __device__ static W zero() { return zero4(); }
    __device__ static f32x4 f32(const W &w) { return w; }
};

// BMODE (compile time): kBwdChain runs one workgroup per (sequence, head)
// over the chunks in reverse and carries only dL/dS across them, writing the
// gradient at every chunk's end to `dckpt` (and the initial-state gradient);
// kBwdChainHalf does the same with two workgroups per (sequence, head), each
// owning half of the value columns (the columns of dL/dS evolve independently):
// its wave w holds 16 value columns for half of the key tiles, so the one
// product that contracts over d_k (K_end dS) sums two waves' halves in LDS;
// kBwdChainQuarter likewise with four workgroups and quarters;
// kBwdGrad runs one workgroup per (16-token slot, head) and forms every
// other gradient of its chunk from the chunk's entering state (`ckpt`) and
// end gradient (`dckpt`), independently of all other chunks.
constexpr int kBwdChain = 1, kBwdGrad = 2, kBwdChainHalf = 3, kBwdChainQuarter = 4;

// The gradient kernel's LDS (76 KiB at d = 128) lets two workgroups share a
// CU; its registers are held to that too (4 waves per SIMD at d = 128).
template <int D, int BMODE>
constexpr int bwd_min_waves_per_simd() {
    return BMODE == kBwdGrad ? 2 * (D / 16) / 4 : 1;
}

template <typename T, int D, int BMODE>
__global__ __launch_bounds__(64 * (D / 16), (bwd_min_waves_per_simd<D, BMODE>())) void chunk_bwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ initial_state, const int32_t *__restrict__ cu_seqlens,
    const T *__restrict__ d_out, const float *__restrict__ d_final, T *__restrict__ dq,
    T *__restrict__ dk, T *__restrict__ dv, float *__restrict__ dlog_alpha,
    float *__restrict__ dbeta, float *__restrict__ d_initial, float *__restrict__ ckpt,
    float *__restrict__ dckpt, int num_seqs, int seq_len, int total_tokens, int H,
    int states_ready) {
    typedef BwdCfg<D, BMODE == kBwdGrad> G;
    typedef Prod<sizeof(T) == 2> PR;  // bf16 inputs: bf16 products, fp32 accumulation
    constexpr int NT = D / 16, LD = G::LD, LS = G::LS;
    __shared__ __attribute__((aligned(16))) float sm[G::FLOATS_ALL];
    float *sQp = sm + G::oQp, *sKp = sm + G::oKp, *sKm = sm + G::oKm, *sKe = sm + G::oKe;
    float *sG = sm + G::oG, *sV = sm + G::oV, *sDO = sm + G::oDO, *sDl = sm + G::oDl;
    float *sLm = sm + G::oLm, *sBr = sm + G::oBr;
    float *sM = sm + G::oM, *sT = sm + G::oT, *sTt = sm + G::oTt, *sP = sm + G::oP;
    float *sDM = sm + G::oDM, *sGam = sm + G::oGam, *sBeta = sm + G::oBeta, *sDB = sm + G::oDB;
    float *sAt = sm + G::oAt;
    float *sQT = sm + G::oQT, *sKT = sm + G::oKT;  // chain kernel only
    // the split chain: workgroups per (sequence, head) and key tiles per wave
    constexpr int PARTS = BMODE == kBwdChainHalf ? 2 : BMODE == kBwdChainQuarter ? 4 : 1;
    constexpr int NTW = NT / PARTS, VG = G::W / PARTS;  // VG: value groups per workgroup
    static_assert(PARTS == 1 || sizeof(T) == 4 || NTW % 2 == 0, "bf16 products take tile pairs");

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g4 = lane >> 4;
    const int h = blockIdx.x % H;
    const int kh = w / VG;  // the split chain: this wave's part of the key tiles
    const int vpart = (int)((blockIdx.x / H) % PARTS);  // and its workgroup's value part
    int n, cfix = 0;
    if constexpr (BMODE == kBwdGrad) {
        // the slot's sequence and chunk
        n = slot_sequence(cu_seqlens, num_seqs, seq_len, total_tokens, blockIdx.x / H, &cfix);
    } else {
        n = (int)(blockIdx.x / H / PARTS);
        if (cu_seqlens && num_seqs <= 64) {
            // packed: the chains of the longest sequences go first (workgroups
            // are dispatched in index order); lane m ranks sequence m by its
            // clamped length, ties by index
            const int lane = tid & 63;
            int len = -1;
            if (lane < num_seqs) {
                int a = cu_seqlens[lane], b = cu_seqlens[lane + 1];
                a = a < 0 ? 0 : (a > total_tokens ? total_tokens : a);
                b = b < a ? a : (b > total_tokens ? total_tokens : b);
                len = b - a;
            }
            int rank = 0;
            for (int m = 0; m < num_seqs; ++m) {
                const int lm = __builtin_amdgcn_readlane(len, m);
                rank += (lm > len || (lm == len && m < lane)) ? 1 : 0;
            }
            const unsigned long long hit = __ballot(lane < num_seqs && rank == n);
            n = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
        }
    }
    int64_t tbeg, tend;
    if (cu_seqlens) {
        int a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > total_tokens ? total_tokens : a);
        b = b < a ? a : (b > total_tokens ? total_tokens : b);
        tbeg = a, tend = b;
    } else {
        tbeg = (int64_t)n * seq_len, tend = tbeg + seq_len;
    }
    const int nch = (int)((tend - tbeg + kBC - 1) / kBC);
    // a slot between two sequences' chunks has no work
    if (BMODE == kBwdGrad && (cfix < 0 || cfix >= nch)) return;
    const int64_t DD = (int64_t)D * D;
    // chunk c of this sequence keeps its entering state in slot tbeg / 16 + n + c
    // this sequence's first checkpoint slot, counted in elements of T
    float *ck = sizeof(T) == 2
                    ? reinterpret_cast<float *>(reinterpret_cast<bf16 *>(ckpt) +
                                                (first_slot(tbeg, n) * H + h) * DD)
                    : ckpt + (first_slot(tbeg, n) * H + h) * DD;
    float *dck = sizeof(T) == 2  // same slots, end gradients
                     ? reinterpret_cast<float *>(reinterpret_cast<bf16 *>(dckpt) +
                                                 (first_slot(tbeg, n) * H + h) * DD)
                     : dckpt + (first_slot(tbeg, n) * H + h) * DD;
    const int64_t ck_stride = (int64_t)H * DD;
    const unsigned HD = (unsigned)H * D;  // elements between two tokens' rows
    const int64_t sbase = ((int64_t)n * H + h) * DD;
    // S orientation: this lane's value column (the split chain: value group
    // w % VG of value part vpart)
    const int vcol = D / PARTS * vpart + 16 * (w % VG) + r;
    const int kcol = 16 * w + r;  // M orientation: this lane's key column

    // Stage chunk c: raw rows as fp32, the prefix G, K+, K-, Q+, Ke, gam, the
    // 16 x 16 matrices K+K-^T, A, M and T = (I + A)^-1 (and T^T).
    // Thread tid's raw inputs of chunk c: four consecutive channels of one row
    // (16 x D = 4 x THREADS), kept as stored (bf16 bits or fp32) so that the
    // loads can be in flight while other work runs; converted when staged.
    // The forward pass (with_grad false) needs neither q nor d_out, the dL/dS
    // chain no v.
    auto raw_load = [&](int c, bool with_grad, bool with_v) -> RawIn<T> {
        const int64_t t0 = tbeg + (int64_t)c * kBC;
        const int nval = (int)((tend - t0) < kBC ? (tend - t0) : kBC);
        const int tok = tid / (D / 4), ch = 4 * (tid % (D / 4));
        const bool ok = tok < nval;
        const int64_t rb = (t0 * H + h) * (int64_t)D;  // the chunk's first row
        const unsigned li = (unsigned)tok * HD + ch;
        RawIn<T> R;
        R.q = with_grad && ok ? RawIn<T>::ld(q + rb + li) : RawIn<T>::zero();
        R.k = ok ? RawIn<T>::ld(k + rb + li) : RawIn<T>::zero();
        R.v = with_v && ok ? RawIn<T>::ld(v + rb + li) : RawIn<T>::zero();
        R.g = ok ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(log_alpha + rb + li))
                 : zero4();
        R.o = with_grad && ok ? RawIn<T>::ld(d_out + rb + li) : RawIn<T>::zero();
        R.b = tid < kBC && tid < nval
                  ? __builtin_nontemporal_load((beta + t0 * H + h) + (unsigned)tid * H)
                  : 0.f;
        return R;
    };
    // `early` runs in every wave once the scaled rows are staged, before the
    // 16 x 16 work; `late` after its share of that work, before the closing
    // barrier (the waves without such work run both while wave 0 solves)
    auto prep = [&](int c, bool with_grad, const RawIn<T> &R, auto &&early, auto &&late) -> int {
        const int64_t t0 = tbeg + (int64_t)c * kBC;
        const int nval = (int)((tend - t0) < kBC ? (tend - t0) : kBC);
        {
            const int tok = tid / (D / 4), ch = 4 * (tid % (D / 4));
            if (with_grad) *reinterpret_cast<f32x4 *>(sQp + tok * LD + ch) = RawIn<T>::f32(R.q);
            *reinterpret_cast<f32x4 *>(sKp + tok * LD + ch) = RawIn<T>::f32(R.k);
            *reinterpret_cast<f32x4 *>(sV + tok * LD + ch) = RawIn<T>::f32(R.v);
            *reinterpret_cast<f32x4 *>(sG + tok * LD + ch) = R.g;
            if (with_grad) *reinterpret_cast<f32x4 *>(sDO + tok * LD + ch) = RawIn<T>::f32(R.o);
            if (tid < kBC) sBeta[tid] = R.b;
        }
        __syncthreads();
        if (tid < D) {  // per channel prefix over the 16 rows
            const int ch = tid;
            float gv[kBC];
#pragma unroll
            for (int tok = 0; tok < kBC; ++tok) gv[tok] = sG[tok * LD + ch];
            float acc = 0.f;
#pragma unroll
            for (int tok = 0; tok < kBC; ++tok) {
                acc += gv[tok];
                sG[tok * LD + ch] = acc;
            }
            sGam[ch] = __expf(acc);
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kBC * D / G::THREADS; ++it) {  // the scaled rows, all threads
            const int idx = tid + it * G::THREADS;
            const int tok = idx / D, ch = idx % D;
            const float gm = sG[tok * LD + ch], eg = __expf(gm);
            const float gl = sG[(kBC - 1) * LD + ch];
            const float kr = sKp[tok * LD + ch];
            sKp[tok * LD + ch] = kr * eg;
            sKm[tok * LD + ch] = kr * __expf(-gm);  // (no division)
            sKe[tok * LD + ch] = kr * __expf(gl - gm);
            if (with_grad) sQp[tok * LD + ch] *= eg;
            if (BMODE != kBwdGrad && with_grad) {  // A operands of the dS products
                sKT[ch * G::LDT + tok] = kr * eg;
                sQT[ch * G::LDT + tok] = sQp[tok * LD + ch];
            }
        }
        __syncthreads();
        early();
        if (w == 0) {
            const f32x4 b = PR::template lds_ldst<D>(zero4(), sKp, LD, sKm, LD, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * g4 + e;
                sBr[i * LS + r] = b[e];
            }
            // A^T: lane (r, g) holds rows 4g .. 4g + 3 of column r of A
            *reinterpret_cast<f32x4 *>(sAt + r * LS + 4 * g4) =
                f32x4{4 * g4 > r ? sBeta[4 * g4] * b[0] : 0.f,
                      4 * g4 + 1 > r ? sBeta[4 * g4 + 1] * b[1] : 0.f,
                      4 * g4 + 2 > r ? sBeta[4 * g4 + 2] * b[2] : 0.f,
                      4 * g4 + 3 > r ? sBeta[4 * g4 + 3] * b[3] : 0.f};
            // A^T is this wave's own LDS writes: a wave fence, no workgroup barrier
            wave_lds_fence();
            // T = (I + A)^{-1} by right-looking substitution: lane 4 j + q holds
            // rows 4 q .. 4 q + 3 of column j; at step m the pivot T[m][j] comes
            // from quad lane m / 4 and every row below it takes -A[row][m] x
            {
                const int j = lane >> 2, q = lane & 3;
                float t[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = (4 * q + e == j) ? 1.f : 0.f;
                constexpr int LA = 4;  // columns of A read ahead of their step
                f32x4 col[kBC - 1];
#pragma unroll
                for (int m = 0; m < LA; ++m)
                    col[m] = *reinterpret_cast<const f32x4 *>(sAt + m * LS + 4 * q);
#pragma unroll
                for (int m = 0; m < kBC - 1; ++m) {
                    if (m + LA < kBC - 1)
                        col[m + LA] = *reinterpret_cast<const f32x4 *>(sAt + (m + LA) * LS + 4 * q);
                    float x;
                    switch (m >> 2) {
                        case 0: x = quad_bcast<0>(t[m & 3]); break;
                        case 1: x = quad_bcast<1>(t[m & 3]); break;
                        case 2: x = quad_bcast<2>(t[m & 3]); break;
                        default: x = quad_bcast<3>(t[m & 3]); break;
                    }
                    // A[row][m] = 0 for row <= m: settled rows are unchanged
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[e] -= col[m][e] * x;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) sT[(4 * q + e) * LS + j] = t[e];
                *reinterpret_cast<f32x4 *>(sTt + j * LS + 4 * q) = f32x4{t[0], t[1], t[2], t[3]};
            }
        } else if (w == 1 && with_grad) {
            const f32x4 m = PR::template lds_ldst<D>(zero4(), sQp, LD, sKm, LD, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * g4 + e;
                sM[i * LS + r] = r <= i ? m[e] : 0.f;
            }
        }
        late();
        __syncthreads();
        return nval;
    };

    // ------------------------------------------------------------ pass 1
    // (skipped when an earlier launch on the stream, the prefill kernel's
    // states mode, has already written every chunk's entering state)
    f32x4 Ss[NT];  // S0 of the chunk: [k = 16t + 4g + e][v = vcol]
#pragma unroll
    for (int t = 0; t < NT; ++t)
        Ss[t] = initial_state ? *reinterpret_cast<const f32x4 *>(
                                    initial_state + sbase + (int64_t)vcol * D + 16 * t + 4 * g4)
                              : zero4();
    for (int c = 0; BMODE == kBwdChain && !states_ready && c < nch; ++c) {
        prep(c, false, raw_load(c, false, true), [] {}, [] {});
#pragma unroll
        for (int t = 0; t < NT; ++t)
            ckpt_store<T>(ck, c * ck_stride + (int64_t)vcol * D + 16 * t + 4 * g4, Ss[t]);
        const f32x4 pk = PR::lds_reg(zero4(), sKp, LD, Ss, lane);
        f32x4 xb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tok = 4 * g4 + e;
            xb[e] = sBeta[tok] * (sV[tok * LD + vcol] - pk[e]);
        }
        const f32x4 dl = PR::lds_tile(zero4(), sT, LS, xb, lane);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 u = PR::ldst_tile(zero4(), sKe + 16 * t, LD, dl, lane);
            const f32x4 gm = *reinterpret_cast<const f32x4 *>(sGam + 16 * t + 4 * g4);
#pragma unroll
            for (int e = 0; e < 4; ++e) Ss[t][e] = gm[e] * Ss[t][e] + u[e];
            sched_fence();
        }
        __syncthreads();
    }

    // ------------------------------------------------------------ pass 2
    // dL/dS at the chunk end, S orientation (value column vcol; key tiles
    // kh * NTW + t)
    f32x4 dSs[NTW];
    constexpr bool GRAD = BMODE == kBwdGrad, CHAIN = !GRAD;
#pragma unroll
    for (int t = 0; t < NTW; ++t)
        dSs[t] = CHAIN && d_final
                     ? *reinterpret_cast<const f32x4 *>(d_final + sbase + (int64_t)vcol * D +
                                                        16 * (kh * NTW + t) + 4 * g4)
                     : zero4();
    // the chain prefetches chunk c - 1's rows while it works on chunk c
    RawIn<T> nxt;
    if (CHAIN && nch > 0) nxt = raw_load(nch - 1, true, false);
    for (int c = GRAD ? cfix : nch - 1; c >= (GRAD ? cfix : 0); --c) {
        if constexpr (CHAIN) {
            // the chain's dO rows and beta alternate between two buffers by chunk
            // parity (the second ones in the gradient kernel's dDelta and dbeta
            // space): they are the only staged arrays read after prep's closing
            // barrier, so the next chunk's staging cannot overwrite what a slower
            // wave still reads, and no barrier closes the chunk
            sDO = (c & 1) ? sm + G::oDl : sm + G::oDO;
            sBeta = (c & 1) ? sm + G::oDB : sm + G::oBeta;
        }
        RawIn<T> cur;
        if constexpr (CHAIN) {
            cur = nxt;
            if (c > 0) nxt = raw_load(c - 1, true, false);
        } else {
            cur = raw_load(c, true, true);
        }
        if constexpr (CHAIN) {
            // the chunk's end gradient for the gradient kernel
#pragma unroll
            for (int t = 0; t < NTW; ++t)
                ckpt_store<T>(dck, c * ck_stride + (int64_t)vcol * D + 16 * (kh * NTW + t) + 4 * g4,
                              dSs[t]);
        }
        const int64_t s0 = c * ck_stride;  // element offset of S0 in the checkpoints
        // the gradient kernel: the chunk's entering state and end gradient in
        // the S orientation
        const float *ckc = ckpt_at<T>(ck, s0), *dckc = ckpt_at<T>(dck, s0);
        // bf16 checkpoints: key tiles t and t + 1 as one 16-byte load per lane
        // (the even lane rows, g4 = 2 i, read keys 16 t + 8 i .. + 7 of tile t,
        // the odd rows keys 16 (t + 1) + 8 i .. + 7 of tile t + 1), issued
        // before the staging's 16 x 16 work so that their latency runs beside
        // wave 0's triangular solve; then one permlane16 swap per word pair
        // gives each lane its four keys of both tiles, kept as loaded (the B
        // operands of their products)
        constexpr bool RAW = GRAD && sizeof(T) == 2;
        u32x4 cw[NT / 2], dcw[NT / 2];
        auto issue = [&] {
            if constexpr (RAW) {
                const bf16 *cb = reinterpret_cast<const bf16 *>(ckc);
                const bf16 *db = reinterpret_cast<const bf16 *>(dckc);
#pragma unroll
                for (int p = 0; p < NT / 2; ++p) {
                    const unsigned off =
                        (unsigned)(vcol * D + 16 * (2 * p + (g4 & 1)) + 8 * (g4 >> 1));
                    cw[p] = *reinterpret_cast<const u32x4 *>(cb + off);
                    dcw[p] = *reinterpret_cast<const u32x4 *>(db + off);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // the split chain's K_end dS partial (K_end is staged before the 16 x 16
        // work), published for the partner waves before prep's closing barrier
        f32x4 *sx = reinterpret_cast<f32x4 *>(sm + G::oXC);
        f32x4 dde = zero4();
        const int nval = prep(c, true, cur, issue, [&] {
            if constexpr (PARTS > 1) {
                dde = PR::lds_reg(zero4(), sKe + 16 * NTW * kh, LD, dSs, lane);
                sx[w * 64 + lane] = dde;
            }
        });
        const int64_t t0 = tbeg + (int64_t)c * kBC;
        u32x2 Sr[NT], dSr[NT];
        if constexpr (RAW) {
            auto split = [&](const u32x4 &x, int t, u32x2 (&out)[NT]) {
                const auto p0 = __builtin_amdgcn_permlane16_swap(x[0], x[2], false, false);
                const auto p1 = __builtin_amdgcn_permlane16_swap(x[1], x[3], false, false);
                out[t] = u32x2{p0[0], p1[0]};
                out[t + 1] = u32x2{p0[1], p1[1]};
            };
#pragma unroll
            for (int p = 0; p < NT / 2; ++p) {
                split(cw[p], 2 * p, Sr);
                split(dcw[p], 2 * p, dSr);
            }
        }
#pragma unroll
        for (int t = 0; t < NT && GRAD && !RAW; ++t) {
            Ss[t] = ckpt_load4<T>(ckc, (unsigned)(vcol * D + 16 * t + 4 * g4));
            dSs[t] = ckpt_load4<T>(dckc, (unsigned)(vcol * D + 16 * t + 4 * g4));
        }
        // value-column products (this wave's 16 columns of X, Delta, lam, dX)
        f32x4 x = zero4(), dl = zero4();
        if constexpr (GRAD) {
            f32x4 pk;
            if constexpr (RAW) pk = mm_lds_raw(zero4(), sKp, LD, Sr, lane);
            else pk = PR::lds_reg(zero4(), sKp, LD, Ss, lane);
            f32x4 xb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tok = 4 * g4 + e;
                x[e] = sV[tok * LD + vcol] - pk[e];
                xb[e] = sBeta[tok] * x[e];
            }
            dl = PR::lds_tile(zero4(), sT, LS, xb, lane);
            sched_fence();
        }
        // each product in its own accumulator: with bf16 operands the two are
        // different MFMA shapes (16x16x16 and 16x16x32), and the compiler puts
        // too few wait states between one's result and the other's accumulator
        // input on gfx950 (half the accumulator rows then read stale values;
        // tests/hip/mfma_chain.hip); the library never chains the shapes
        const f32x4 ddm = PR::ldst_lds(zero4(), sM, LS, sDO + (vcol - r), LD, lane);
        if constexpr (RAW) dde = mm_lds_raw(zero4(), sKe, LD, dSr, lane);
        else if constexpr (PARTS == 1) dde = PR::lds_reg(zero4(), sKe, LD, dSs, lane);
        f32x4 ddl;
        if constexpr (PARTS > 1) {
            // the partials of the waves with the same value columns (one per
            // part of the key tiles, written before prep's closing barrier),
            // summed in one order in all of them
            f32x4 o = sx[(w % VG) * 64 + lane];
#pragma unroll
            for (int j = 1; j < PARTS; ++j) {
                const f32x4 p = sx[(w % VG + VG * j) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] += p[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ddl[e] = ddm[e] + o[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) ddl[e] = ddm[e] + dde[e];
        }
        sched_fence();
        const f32x4 lam = PR::lds_tile(zero4(), sTt, LS, ddl, lane);
        f32x4 dxr;  // dX in the accumulator layout: the B operand of K+^T dX
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tok = 4 * g4 + e;
            const float dx = sBeta[tok] * lam[e];
            dxr[e] = dx;
            if constexpr (GRAD) {
                sDl[tok * LD + vcol] = dl[e];
                sLm[tok * LD + vcol] = lam[e];
                if (tok < nval) (dv + (t0 * H + h) * D)[(unsigned)tok * HD + vcol] = from_f32<T>(dx);
                const float pb = row16_sum(x[e] * lam[e]);
                if (r == 0) sDB[w * kBC + tok] = pb;
            }
        }
        // (the chain's dS products below read only prep's LDS rows and registers)
        if constexpr (GRAD) __syncthreads();
        if constexpr (GRAD) {
        // (T and T^T are dead from here: their space takes P^T and dM^T)
        float *sPt = sT, *sDMt = sTt;
        if (w == 0) {  // dA, P = diag(b) dA and the K+K-^T part of db
            const f32x4 ld = PR::template lds_ldst<D>(zero4(), sLm, LD, sDl, LD, lane);
            f32x4 pc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * g4 + e;
                const float da = r < i ? -ld[e] : 0.f;
                pc[e] = sBeta[i] * da;
                sP[i * LS + r] = pc[e];
                const float pb = row16_sum(da * sBr[i * LS + r]);
                if (r == 0) sDB[G::W * kBC + i] = pb;
            }
            *reinterpret_cast<f32x4 *>(sPt + r * LS + 4 * g4) = pc;
        } else if (w == 1) {  // dM = Tril(dO Delta^T)
            const f32x4 od = PR::template lds_ldst<D>(zero4(), sDO, LD, sDl, LD, lane);
            f32x4 mc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * g4 + e;
                mc[e] = r <= i ? od[e] : 0.f;
                sDM[i * LS + r] = mc[e];
            }
            *reinterpret_cast<f32x4 *>(sDMt + r * LS + 4 * g4) = mc;
        }
        __syncthreads();
        if (tid < nval) {
            float s = 0.f;
#pragma unroll
            for (int ww = 0; ww <= G::W; ++ww) s += sDB[ww * kBC + tid];
            (dbeta + t0 * H + h)[(unsigned)tid * H] = s;
        }
        // key-column products (this wave's 16 key columns) that contract over
        // d_v, with S0 and dS_C in the M orientation ([v = 16j + 4g + e][k =
        // kcol]) read from the checkpoints 32 rows of v at a time (registers for
        // two workgroups per CU): dO S0^T, lam S0^T, dKe = Delta dS_C^T and
        // rowsum(S0 * dS_C)
        f32x4 dqs = zero4(), xs = zero4(), dke = zero4();
        float s1 = 0.f;
#pragma unroll
        for (int hv = 0; hv < NT / 2; ++hv) {
            constexpr int NH = 2;  // tiles per step (a bf16 product's pair)
            if constexpr (sizeof(T) == 2) {
                // bf16 checkpoints: the eight values of a B fragment as loaded
                // (packed in pairs, no round trip through fp32), the row sum
                // of S0 * dS_C by two-term bf16 dot products
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const short *cs = reinterpret_cast<const short *>(ckc);
                const short *ds = reinterpret_cast<const short *>(dckc);
                s16x8 sv, dv8;
#pragma unroll
                for (int t = 0; t < NH; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const unsigned off =
                            (unsigned)((16 * (NH * hv + t) + 4 * g4 + e) * D + kcol);
                        sv[4 * t + e] = __builtin_nontemporal_load(cs + off);
                        dv8[4 * t + e] = __builtin_nontemporal_load(ds + off);
                    }
                const bf16x8 sb = __builtin_bit_cast(bf16x8, sv);
                const bf16x8 db = __builtin_bit_cast(bf16x8, dv8);
                auto arow = [&](const float *A) {
                    const float *a0 = A + r * LD + 32 * hv + 4 * g4;
                    return pack8(*reinterpret_cast<const f32x4 *>(a0),
                                 *reinterpret_cast<const f32x4 *>(a0 + 16));
                };
                dqs = mf32(arow(sDO), sb, dqs);
                xs = mf32(arow(sLm), sb, xs);
                dke = mf32(arow(sDl), db, dke);
                const u32x4 sw = __builtin_bit_cast(u32x4, sv), dw = __builtin_bit_cast(u32x4, dv8);
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) s1 = dot2_bf16(sw[pp], dw[pp], s1);
                // (the next step's loads stay below: registers for two
                // workgroups per CU)
                __builtin_amdgcn_sched_barrier(0);
            } else {
                f32x4 Sm[NH], dSm[NH];
#pragma unroll
                for (int t = 0; t < NH; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const unsigned off =
                            (unsigned)((16 * (NH * hv + t) + 4 * g4 + e) * D + kcol);
                        Sm[t][e] = ckpt_load1<T>(ckc, off);
                        dSm[t][e] = ckpt_load1<T>(dckc, off);
                    }
                dqs = PR::lds_reg(dqs, sDO + 16 * NH * hv, LD, Sm, lane);
                xs = PR::lds_reg(xs, sLm + 16 * NH * hv, LD, Sm, lane);
                dke = PR::lds_reg(dke, sDl + 16 * NH * hv, LD, dSm, lane);
#pragma unroll
                for (int t = 0; t < NH; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s1 += Sm[t][e] * dSm[t][e];
            }
            sched_fence();
        }
        // (separate accumulators for the two MFMA shapes, as for ddl above)
        const f32x4 dqm = PR::lds_lds(zero4(), sDM, LS, sKm + 16 * w, LD, lane);
        f32x4 dqp;
#pragma unroll
        for (int e = 0; e < 4; ++e) dqp[e] = dqs[e] + dqm[e];
        // dX S0^T = diag(b) (lam S0^T)
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[e] *= sBeta[4 * g4 + e];
        const f32x4 pkm = PR::lds_lds(zero4(), sP, LS, sKm + 16 * w, LD, lane);
        const f32x4 dkm = PR::ldst_lds(PR::ldst_lds(zero4(), sDM, LS, sQp + 16 * w, LD, lane), sP,
                                      LS, sKp + 16 * w, LD, lane);
        sched_fence();
        s1 = rows4_sum(s1);
        const float gamk = sGam[kcol];
        const float gl = sG[(kBC - 1) * LD + kcol];
        // dlog_alpha[t] = d/d log alpha_t of every factor e^{G_a - G_b} (a > b) of
        // the chunk form with b < t <= a, summed as such: the pairs (i >= t > j)
        // of M and A, the rows i >= t of Q+ S0 and K+ S0, the rows j < t of Ke
        // and gam (a = 16, b = 0), which all carry alpha_t's decay.  (The suffix
        // sum of dG = dQ+ Q+ + dK+ K+ - dK- K- - dKe Ke is the same sum with
        // every pair inside the suffix added and taken away again; the pairs on
        // the diagonal weigh 1 however small alpha_t is, so that form loses all
        // relative precision where the gates decay strongly.)
        float suf[4], pre[4], qpv[4], kpv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tok = 4 * g4 + e;
            const float gm = sG[tok * LD + kcol], eg = __expf(gm);
            qpv[e] = sQp[tok * LD + kcol];
            kpv[e] = sKp[tok * LD + kcol];
            const float dkp = pkm[e] - xs[e];
            const float qv = dqp[e] * eg;
            const float kv = dkp * eg + dkm[e] * __expf(-gm) + dke[e] * __expf(gl - gm);
            suf[e] = dqs[e] * qpv[e] - xs[e] * kpv[e];
            pre[e] = dke[e] * sKe[tok * LD + kcol];
            if (tok < nval) {
                const unsigned gi = (unsigned)tok * HD + kcol;
                (dq + (t0 * H + h) * D)[gi] = from_f32<T>(qv);
                (dk + (t0 * H + h) * D)[gi] = from_f32<T>(kv);
            }
        }
        if (g4 == 3) suf[3] += gamk * s1;  // gam: every row of the chunk
        // suffix sums of suf and exclusive prefix sums of pre over the 16 rows:
        // within the lane, then over the lane groups above / below
        suf[2] += suf[3];
        suf[1] += suf[2];
        suf[0] += suf[1];
        float ex[4];
        ex[0] = 0.f;
        ex[1] = pre[0];
        ex[2] = pre[0] + pre[1];
        ex[3] = ex[2] + pre[2];
        const float ptot = ex[3] + pre[3];
        float above = 0.f, below = 0.f, ts[4], tp[4];
        rows4_gather(suf[0], ts);
        rows4_gather(ptot, tp);
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            if (gg > g4) above += ts[gg];
            if (gg < g4) below += tp[gg];
        }
        // the pairs: R_t = sum_{i >= t} Z_i(t) with Z_i(t) = sum_{j < t} (Q+_i
        // dM[i][j] + K+_i P[i][j]) K-_j; this lane holds rows i = 4 g4 + e, and
        // a row leaves the sum (its Z and weights set to zero) at t = i + 1
        // (qpv and kpv serve as the weights: their last use above is done)
        float z[4] = {0.f, 0.f, 0.f, 0.f}, *qw = qpv, *kw = kpv;
        float part[kBC];  // this lane's share of R_t
        part[0] = 0.f;
#pragma unroll
        for (int t = 1; t < kBC; ++t) {
            const float km = sKm[(t - 1) * LD + kcol];
            const f32x4 mc = *reinterpret_cast<const f32x4 *>(sDMt + (t - 1) * LS + 4 * g4);
            const f32x4 pc = *reinterpret_cast<const f32x4 *>(sPt + (t - 1) * LS + 4 * g4);
            {
                const int eo = (t - 1) & 3;  // row t - 1 leaves (lane group (t - 1) / 4)
                const bool out = g4 == ((t - 1) >> 2);
                z[eo] = out ? 0.f : z[eo];
                qw[eo] = out ? 0.f : qw[eo];
                kw[eo] = out ? 0.f : kw[eo];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] += (qw[e] * mc[e] + kw[e] * pc[e]) * km;
            part[t] = (z[0] + z[1]) + (z[2] + z[3]);
        }
        // R_t summed over the four lane groups, t = 4 g4 + e left in lane group
        // g4 (a reduce-scatter by permlane swaps: upper with lower 32 lanes
        // for t and t + 8, then odd with even rows for t and t + 4)
        float h8[8], rt[4];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[t]),
                                                            __float_as_uint(part[t + 8]), false,
                                                            false);
            h8[t] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(h8[t]),
                                                            __float_as_uint(h8[t + 4]), false,
                                                            false);
            rt[t] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tok = 4 * g4 + e;
            if (tok < nval)
                (dlog_alpha + (t0 * H + h) * D)[(unsigned)tok * HD + kcol] =
                    (suf[e] + above) + (ex[e] + below) + rt[e];
        }
        }  // GRAD
        // state gradient before the chunk: Q+^T dO and K+^T dX per key tile, A from
        // the transposed rows, B (this wave's value columns) from registers
        f32x4 dor;
#pragma unroll
        for (int e = 0; e < 4 && CHAIN; ++e) dor[e] = sDO[(4 * g4 + e) * LD + vcol];
#pragma unroll
        for (int t = 0; t < NTW && CHAIN; ++t) {
            const int tg = kh * NTW + t;
            const f32x4 u = PR::lds_tile(zero4(), sQT + 16 * tg * G::LDT, G::LDT, dor, lane);
            const f32x4 y = PR::lds_tile(zero4(), sKT + 16 * tg * G::LDT, G::LDT, dxr, lane);
            const f32x4 gm = *reinterpret_cast<const f32x4 *>(sGam + 16 * tg + 4 * g4);
#pragma unroll
            for (int e = 0; e < 4; ++e) dSs[t][e] = gm[e] * dSs[t][e] + u[e] - y[e];
            sched_fence();
        }
    }
    if (CHAIN && d_initial) {
#pragma unroll
        for (int t = 0; t < NTW; ++t)
            *reinterpret_cast<f32x4 *>(d_initial + sbase + (int64_t)vcol * D +
                                       16 * (kh * NTW + t) + 4 * g4) = dSs[t];
    }
}

// Compute units of the current device (0 if the query fails), cached per device.
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < 64 && (n = cached[dev].load(std::memory_order_relaxed)) > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <typename T, int D>
int launch_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
               const float *beta, const float *initial_state, const int32_t *cu_seqlens,
               const void *d_out, const float *d_final, void *dq, void *dk, void *dv,
               float *dlog_alpha, float *dbeta, float *d_initial, float *ckpt, int num_seqs,
               int seq_len, int total_tokens, int H, hipStream_t stream) {
    const int64_t units = (int64_t)num_seqs * H;
    if (units == 0) return 0;
    const int64_t slots = region_slots(total_tokens, num_seqs);
    if (units > (int64_t)1 << 30 || slots * H > (int64_t)1 << 30) return -1;
    // Units whose gates leave the chunked kernels' range are marked (flag words
    // after the two regions) and redone token by token at the end.
    unsigned *far_flags =
        reinterpret_cast<unsigned *>(ckpt + 2 * slots * H * (int64_t)D * D);
    // The chunk-entering states from the prefill kernel (32-token chunks, all
    // CUs' worth of parallelism per head as in the forward), which also marks
    // the units, where it supports the configuration; otherwise a detect pass
    // marks them and the chain kernel recomputes the states first.
    int ready = 0;
    if ((sizeof(T) == 2 || D == 64) && (int64_t)H * D * 4 * 64 <= INT32_MAX) {
        if (launch_chunk_states(q, k, v, log_alpha, beta, initial_state, cu_seqlens, ckpt,
                                num_seqs, seq_len, total_tokens, H, D,
                                sizeof(T) == 2 ? kDtypeBf16 : kDtypeF32, far_flags,
                                stream) != 0)
            return -1;
        ready = 1;
    } else if (launch_bwd_far_detect(log_alpha, cu_seqlens, num_seqs, seq_len, total_tokens, H,
                                     D, far_flags, stream) != 0) {
        return -1;
    }
    float *dckpt = ckpt + slots * H * D * D;  // second region: chunk-end gradients
#define KDA_BWD_KERNEL_ARGS                                                                    \
    static_cast<const T *>(q), static_cast<const T *>(k), static_cast<const T *>(v), log_alpha, \
        beta, initial_state, cu_seqlens, static_cast<const T *>(d_out), d_final,              \
        static_cast<T *>(dq), static_cast<T *>(dk), static_cast<T *>(dv), dlog_alpha, dbeta,   \
        d_initial, ckpt, dckpt, num_seqs, seq_len, total_tokens, H, ready
    // the chain: two workgroups per (sequence, head), one per value half, when
    // the states are ready (the pass that computes them runs on whole heads);
    // four at d = 128 when four per pair still fit on the device's CUs
    if (sizeof(T) == 2 && ready) {
        // bf16: the pipelined chain (preparation one chunk ahead of the scan)
        if (launch_bwd_chain(q, k, log_alpha, beta, cu_seqlens, d_out, d_final, d_initial, dckpt,
                             num_seqs, seq_len, total_tokens, H, D, stream) != 0)
            return -1;
    } else if (D == 128 && ready && 4 * units <= device_cus())
        hipLaunchKernelGGL((chunk_bwd_kernel<T, D, D == 128 ? kBwdChainQuarter : kBwdChainHalf>),
                           dim3((unsigned)(4 * units)), dim3(BwdCfg<D, false>::THREADS), 0, stream,
                           KDA_BWD_KERNEL_ARGS);
    else if (ready)
        hipLaunchKernelGGL((chunk_bwd_kernel<T, D, kBwdChainHalf>), dim3((unsigned)(2 * units)),
                           dim3(BwdCfg<D, false>::THREADS), 0, stream, KDA_BWD_KERNEL_ARGS);
    else
        hipLaunchKernelGGL((chunk_bwd_kernel<T, D, kBwdChain>), dim3((unsigned)units),
                           dim3(BwdCfg<D, false>::THREADS), 0, stream, KDA_BWD_KERNEL_ARGS);
    if (hipGetLastError() != hipSuccess) return -1;
    hipLaunchKernelGGL((chunk_bwd_kernel<T, D, kBwdGrad>), dim3((unsigned)(slots * H)),
                       dim3(BwdCfg<D, false>::THREADS), 0, stream, KDA_BWD_KERNEL_ARGS);
#undef KDA_BWD_KERNEL_ARGS
    if (hipGetLastError() != hipSuccess) return -1;
    return launch_bwd_seq(q, k, v, log_alpha, beta, initial_state, cu_seqlens, d_out, d_final,
                          dq, dk, dv, dlog_alpha, dbeta, d_initial, ckpt, far_flags, num_seqs,
                          seq_len, total_tokens, H, D, sizeof(T) == 2 ? kDtypeBf16 : kDtypeF32,
                          stream);
}

}  // namespace

int64_t chunk_bwd_workspace_floats(int64_t total_tokens, int64_t num_seqs, int64_t num_heads,
                                   int head_dim) {
    // two regions of one state per slot and head (entering states, end
    // gradients), then the out-of-range flag words of every (sequence, head)
    return 2 * region_slots(total_tokens, num_seqs) * num_heads * head_dim * head_dim +
           bwd_far_flag_words(num_seqs, num_heads);
}

int launch_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                     const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                     const void *d_out, const float *d_final_state, void *dq, void *dk, void *dv,
                     float *dlog_alpha, float *dbeta, float *d_initial_state, float *workspace,
                     int32_t num_seqs, int32_t seq_len, int32_t total_tokens, int32_t num_heads,
                     int head_dim, int dtype, hipStream_t stream) {
#define KDA_BWD_ARGS                                                                           \
    q, k, v, log_alpha, beta, initial_state, cu_seqlens, d_out, d_final_state, dq, dk, dv,     \
        dlog_alpha, dbeta, d_initial_state, workspace, num_seqs, seq_len, total_tokens,        \
        num_heads, stream
    if (dtype == kDtypeBf16)
        return head_dim == 128 ? launch_bwd<bf16, 128>(KDA_BWD_ARGS)
                               : launch_bwd<bf16, 64>(KDA_BWD_ARGS);
    return head_dim == 128 ? launch_bwd<float, 128>(KDA_BWD_ARGS)
                           : launch_bwd<float, 64>(KDA_BWD_ARGS);
#undef KDA_BWD_ARGS
}

}  // namespace kda
