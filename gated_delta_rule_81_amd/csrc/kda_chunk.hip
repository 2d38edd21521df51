// kda_chunk.hip -- chunked KDA prefill: one persistent workgroup per
// (sequence, head, d_v slice) walks the sequence chunk by chunk.
//
// Pages cited (by title):
//   [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer.
//   [K3-memory]     "Kimi K3 Changed the Memory Math for Agentic AI Forever".
//
// The recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t ([K3-explainer] §四, §二.1) is evaluated per chunk of C = 32
// tokens: state recurrence between chunks, dense products inside a chunk
// ([K3-explainer] §六.1), with the chunk's rank-one erase/write products
// gathered into a few matrices ([K3-explainer] §六.2, WY representation).
// The concrete form used here (a UT-transform variant; the page gives only
// the idea) is, for a chunk with entering state S and per-channel cumulative
// log-decay Gamma_r = sum_{s<=r} log a_s (reset each chunk):
//
//   K+ = K (.) e^Gamma,  Q+ = Q (.) e^Gamma,  K- = K (.) e^-Gamma
//   A       = StrictTril(diag(b) K+ K-^T),  T = (I + A)^{-1},  T' = T diag(b)
//   X       = V - K+ S                        (prediction error against S)
//   Delta   = T' X                            (the chunk's corrected writes)
//   O       = Q+ S + Tril(Q+ K-^T) Delta
//   S_next  = Diag(e^{Gamma_last}) S + (K (.) e^{Gamma_last - Gamma})^T Delta
//
// The chunk transition S -> S_next is the page's "P = D - K W^T" form
// ([K3-explainer] §六.2) with D = Diag(e^{Gamma_last}).
//
// Range of the factors.  The products inside a chunk only need
// e^{Gamma_i - Gamma_j} for j <= i, which is <= 1, but e^{-Gamma} alone grows
// with the decay accumulated since its reference point.  The chunk is two
// 16-token blocks; block 0 is referenced to the chunk start and block 1 to
// its own start rho = Gamma_15:
//   * K+, Q+ (chunk-relative, <= |k|, |q|) feed [K+; Q+] S and the block
//     (1,0) tiles; K- of block 0 (chunk-relative) feeds tiles (0,0), (1,0);
//   * the diagonal tile (1,1) uses K+, Q+, K- of block 1 relative to rho.
// Every factor is then bounded by e^{decay over 16 tokens}.  Gates may be
// anything in [0, 1]: a (sequence, head, slice) unit in which some 16-token
// block decays beyond 2^-100 in some channel (or has alpha = 0) is marked by
// this fast kernel and recomputed by a second launch of the same kernel
// (FAR), which takes exactly those chunks token by token in fp32 on the scan
// side; see chunk_fwd_kernel.
// K_end = K (.) e^{Gamma_last - Gamma} is applied as (K e^{rho - Gamma}),
// stored in LDS, times the per-channel f = e^{Gamma_last - rho} in fp32 on the
// scan side: both factors stay in fp32 range.
//
// Work split inside a workgroup.  D/16 preparation waves and DVS/16 scan
// waves run in lockstep, two workgroup barriers per chunk: while the
// preparation waves build chunk n+1's operands, each scan wave advances its
// 16 value columns of the state over chunk n.  Prepared operands are double
// buffered in LDS.
//   preparation, phase 1: cumulative log-decay (DPP lane scan), e^{+-Gamma}
//                (v_exp_f32), operand tiles in LDS, next chunk's loads;
//                phase 2: A and Tril(Q+ K-^T) (6 MFMA tiles), the diagonal
//                blocks T_00, T_11 of (I + A)^{-1} by substitution.
//   scan, phase 1: [K+; Q+] S, X, Delta by block substitution
//                (Delta_0 = T_00 b_0 X_0, Delta_1 = T_11 (b_1 X_1 - A_10 Delta_0)),
//                O (stored);
//         phase 2: S <- gamma S + f (K e^{rho - Gamma})^T Delta.
// A scan wave keeps its state columns (all d_k rows) in fp32 MFMA
// accumulators and feeds them straight back as the B operand of the next
// chunk's products: the contraction index is permuted so that the
// accumulator layout is the operand layout (see `phys`), and the operand
// tiles in LDS are stored in that permuted order.  X, Delta and O stay in
// registers the same way.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kC = kChunkTokens;  // chunk length
constexpr int kBS = 16;  // block / tile size
// The factorised products of a chunk hold e^{+-(decay within a 16-token
// block)} in fp32 / bf16 operands.  A chunk in which some channel decays by
// more than 2^-kFarLog2 over one block (or whose gates are -inf or NaN) is
// taken token by token on the scan side instead (the exact recurrence in
// fp32).
constexpr float kFarLog2 = 100.f;

// Physical position of contraction index i (a key channel or a token) in
// the LDS operand tiles.  For bf16 the 16x16x32 MFMA reads, in lane group
// g = lane / 16, 8 consecutive physical entries; they hold the logical
// indices {4g .. 4g+3, 16 + 4g .. 16 + 4g + 3} of each group of 32, which are
// exactly the rows that lane holds of two stacked 16x16 accumulator tiles.
// fp32 (16x16x4 MFMA, one index per lane per step) keeps the natural order.
template <typename T>
__device__ __forceinline__ int phys(int i) {
    if constexpr (sizeof(T) == 2) {
        const int j = i & 31;
        return (i & ~31) + 8 * ((j & 15) >> 2) + 4 * (j >> 4) + (j & 3);
    } else {
        return i;
    }
}

template <typename T, int D, int DVS, bool SG>
struct Cfg {
    static constexpr int SZ = (int)sizeof(T);
    static constexpr int kPad = 16 / SZ;
    static constexpr int PW = D / 16;        // preparation waves
    static constexpr int SWV = DVS / 16;     // scan waves (one per 16 value columns)
    static constexpr int THREADS = 64 * (PW + SWV);
    static constexpr int LDK = D + kPad;     // [token][channel] tiles
    static constexpr int LDT = kC + kPad;    // [*][token] tiles
    static constexpr int LDV = DVS + kPad;   // V slice rows
    static constexpr int LDAT = kBS + 4;     // fp32 transposed diagonal blocks of A
    static constexpr int LDTT = kBS + kPad;  // 16x16 operand blocks of the substitution
    static constexpr int NRT = D / 16;       // d_k row tiles of the state
    static constexpr int KB = sizeof(T) == 2 ? 32 : 16;  // contraction block per operand fragment
    static constexpr int VE = 16 / SZ;       // elements per 16-byte V access
    static constexpr int VTH = kC * DVS / VE;  // preparation threads that move the V slice
    static constexpr int RW = 4 * SZ / 4;    // words per 4-channel run of k / q
    // whole-row loads: 16 bytes per lane, a row of k / q (RBK bytes), log_alpha
    // (RBG; none with a scalar gate, which is loaded like beta) or the V slice
    // (RBV) covered by RBX / 16 consecutive lanes
    static constexpr int RBK = D * SZ, RBG = SG ? 0 : D * 4, RBV = DVS * SZ;
    static constexpr int IK = RBK / 16 / 2 / PW;  // k (and q) load instructions per wave
    static constexpr int IG = RBG / 16 / 2 / PW;  // log_alpha load instructions per wave
    static constexpr int NIV = RBV / 16 / 2;      // V load instructions (waves 0 .. NIV-1)
    static constexpr int IO = RBV / 16 / 2 / SWV; // O store instructions per scan wave
    static constexpr int LSK = RBK + 16, LSG = RBG + 16, LSV = RBV + 16;  // staging row bytes
    static constexpr int NGA = IG > 0 ? IG : 1;   // register slots for the gate pieces

    // one buffer set of prepared operands (byte offsets inside the set)
    static constexpr int B_TK = kC * LDK * SZ;
    static constexpr int B_TT = kC * LDT * SZ;
    // T3: T'_00 = T_00 diag(b_0), A_10, T_11 (16x16 each, row-major)
    static constexpr int B_T16 = kBS * LDTT * SZ;
    static constexpr int sKP = 0, sQP = B_TK, sKET = 2 * B_TK, sMQ = sKET + D * LDT * SZ,
                         sT3 = sMQ + B_TT, sV = sT3 + 3 * B_T16, sGam = sV + kC * LDV * SZ,
                         sF1 = sGam + D * 4, sBeta = sF1 + D * 4, SET = sBeta + kC * 4;
    // Out-of-range words, one per (preparation wave, lane group): word j sits
    // in the (never read) padding of K+'s row j / 4.
    __host__ __device__ static constexpr int flag_offset(int j) {
        return sKP + (j >> 2) * LDK * SZ + D * SZ + 4 * (j & 3);
    }
    static_assert(kPad * SZ >= 16 && 4 * PW <= 4 * kC, "flag words in the row padding");
    // the fast kernel's sticky word (some chunk of the unit was out of range),
    // in the padding of K+'s first row (the fix-up kernel's words use it)
    static constexpr int sMark = sKP + D * SZ;

    // preparation scratch
    static constexpr int oKD = 2 * SET, oQD = oKD + kBS * LDK * SZ, oKM = oQD + kBS * LDK * SZ,
                         oAt = oKM + B_TK;
    // staging of the next chunk's raw rows (k, q, log_alpha, V slice, beta)
    static constexpr int oRK = oAt + 2 * kBS * LDAT * 4, oRQ = oRK + kC * LSK,
                         oRG = oRQ + kC * LSK, oRV = oRG + (SG ? kC * 4 : kC * LSG),
                         oRB = oRV + kC * LSV;
    // O staging (all scan waves), stored as whole rows in the next phase
    static constexpr int oO = oRB + kC * 4, BYTES = oO + kC * LSV;

    static_assert(D == 64 || D == 128, "head dim");
    static_assert(DVS % 16 == 0 && D % DVS == 0, "d_v slice");
    static_assert(VTH <= PW * 64 && VTH >= kC, "V slice map");
    static_assert(D % KB == 0, "state contraction blocks");
    static_assert(IK >= 1 && (IG >= 1 || SG) && IO >= 1 && NIV <= PW &&
                      IK * PW * 2 * 16 == RBK && IG * PW * 2 * 16 == RBG &&
                      IO * SWV * 2 * 16 == RBV, "whole-row load maps");
    static_assert(SET % 16 == 0 && oKM % 16 == 0 && oAt % 16 == 0 && oO % 16 == 0 &&
                      oRK % 16 == 0 && oRG % 16 == 0 && oRV % 16 == 0, "16-byte alignment");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// --------------------------------------------------------------- raw loads
// Buffer descriptors for one chunk: the base points at the chunk's first
// token and the size covers exactly its nvalid tokens, so every load of a row
// at or beyond nvalid returns zeros (an inert token: k = q = v = 0, a = 1,
// b = 0) without a branch.
struct ChunkSrc {
    __amdgpu_buffer_rsrc_t k, q, g, v, b;
};

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// ZV: zero values (v is not read; its descriptor covers no bytes, so every V
// load returns zeros).
template <bool ZV, typename T>
__device__ __forceinline__ ChunkSrc chunk_src(const T *q, const T *k, const T *v,
                                              const float *log_alpha, const float *beta,
                                              int64_t tok0, int nvalid, int H, int D,
                                              bool scalar_gate) {
    const int64_t e0 = tok0 * H * D;
    const int elems = nvalid * H * D;  // the host keeps 64 * H * D * 4 < 2^31
    ChunkSrc s;
    s.k = __builtin_amdgcn_make_buffer_rsrc((void *)(k + e0), 0, elems * (int)sizeof(T),
                                            kRsrcWord3);
    s.q = __builtin_amdgcn_make_buffer_rsrc((void *)(q + e0), 0, elems * (int)sizeof(T),
                                            kRsrcWord3);
    if constexpr (ZV)
        s.v = __builtin_amdgcn_make_buffer_rsrc((void *)k, 0, 0, kRsrcWord3);
    else
        s.v = __builtin_amdgcn_make_buffer_rsrc((void *)(v + e0), 0, elems * (int)sizeof(T),
                                                kRsrcWord3);
    s.g = scalar_gate ? __builtin_amdgcn_make_buffer_rsrc((void *)(log_alpha + tok0 * H), 0,
                                                          nvalid * H * 4, kRsrcWord3)
                      : __builtin_amdgcn_make_buffer_rsrc((void *)(log_alpha + e0), 0, elems * 4,
                                                          kRsrcWord3);
    s.b = __builtin_amdgcn_make_buffer_rsrc((void *)(beta + tok0 * H), 0, nvalid * H * 4,
                                            kRsrcWord3);
    return s;
}

template <int NW> struct Raw { unsigned w[NW]; };

template <int NW>
__device__ __forceinline__ Raw<NW> buf_load(__amdgpu_buffer_rsrc_t r, int off) {
    Raw<NW> x;
    if constexpr (NW == 1) {
        x.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    } else if constexpr (NW == 2) {
        const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        x.w[0] = a[0];
        x.w[1] = a[1];
    } else {
        static_assert(NW == 4, "access width");
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) x.w[i] = a[i];
    }
    return x;
}

// N elements of T held in raw words -> floats.
template <typename T, int N, int NW>
__device__ __forceinline__ void unpack(const Raw<NW> &x, float *f) {
    if constexpr (sizeof(T) == 2) {
        static_assert(2 * NW == N, "bf16 words");
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            f[2 * i] = __uint_as_float(x.w[i] << 16);
            f[2 * i + 1] = __uint_as_float(x.w[i] & 0xffff0000u);
        }
    } else {
        static_assert(NW == N, "fp32 words");
#pragma unroll
        for (int i = 0; i < N; ++i) f[i] = __uint_as_float(x.w[i]);
    }
}

// Four consecutive elements of T (8-byte aligned for bf16, 16 for fp32) as floats.
__device__ __forceinline__ void load4(const bf16 *p, float (&f)[4]) {
    const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
    f[0] = __uint_as_float(w[0] << 16);
    f[1] = __uint_as_float(w[0] & 0xffff0000u);
    f[2] = __uint_as_float(w[1] << 16);
    f[3] = __uint_as_float(w[1] & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float *p, float (&f)[4]) {
    const f32x4 w = *reinterpret_cast<const f32x4 *>(p);
    f[0] = w[0]; f[1] = w[1]; f[2] = w[2]; f[3] = w[3];
}

// Two floats as one packed word of T pairs (bf16) or two words (fp32).
__device__ __forceinline__ unsigned pack2(float a, float b) {
    bf16x2 h;
    h[0] = static_cast<bf16>(a);
    h[1] = static_cast<bf16>(b);
    return __builtin_bit_cast(unsigned, h);
}

// Eight floats -> eight consecutive T in LDS (16-byte aligned).
__device__ __forceinline__ void st8(bf16 *p, const float (&f)[8]) {
    *reinterpret_cast<u32x4 *>(p) =
        u32x4{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
}
__device__ __forceinline__ void st8(float *p, const float (&f)[8]) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}

// Four floats -> four consecutive T in LDS (8-byte aligned for bf16, 16 for fp32).
__device__ __forceinline__ void st4(bf16 *p, const float (&f)[4]) {
    *reinterpret_cast<u32x2 *>(p) = u32x2{pack2(f[0], f[1]), pack2(f[2], f[3])};
}
__device__ __forceinline__ void st4(float *p, const float (&f)[4]) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{f[0], f[1], f[2], f[3]};
}

// One chunk's raw inputs in flight for one preparation thread, loaded as
// whole rows (16 bytes per lane, consecutive lanes along a row): IK pieces
// each of k and q, IG of log_alpha, one of the V slice (last NIV waves), one
// beta (last wave).  Waves 0 and 1 run the triangular solves, so the extra
// pieces go to the other waves.
template <typename T, int D, int DVS, bool SG>
struct ChunkRegs {
    typedef Cfg<T, D, DVS, SG> G;
    Raw<4> k[G::IK], q[G::IK], g[G::NGA], v;
    float beta, gs;  // gs: the scalar gate (scalar-gate variant only)
};

// Where a preparation thread's pieces come from (byte offsets relative to a
// chunk's first token; loop-invariant) and where they go in the staging area.
template <typename T, int D, int DVS, bool SG>
struct ChunkOffsets {
    typedef Cfg<T, D, DVS, SG> G;
    int gk[G::IK], sk[G::IK], gg[G::NGA], sg[G::NGA], gv, sv, gb;
    __device__ ChunkOffsets(int wave, int lane, int h, int H, int v0) {
        constexpr int LK = G::RBK / 16, LG = G::RBG / 16 > 0 ? G::RBG / 16 : 1,
                      LV = G::RBV / 16;
#pragma unroll
        for (int i = 0; i < G::IK; ++i) {
            const int p = (wave * G::IK + i) * 64 + lane, row = p / LK, b = 16 * (p % LK);
            gk[i] = (row * H + h) * G::RBK + b;
            sk[i] = row * G::LSK + b;
        }
#pragma unroll
        for (int i = 0; i < G::IG; ++i) {
            const int p = (wave * G::IG + i) * 64 + lane, row = p / LG, b = 16 * (p % LG);
            gg[i] = (row * H + h) * G::RBG + b;
            sg[i] = row * G::LSG + b;
        }
        const int p = (wave - (G::PW - G::NIV)) * 64 + lane, row = p / LV, b = 16 * (p % LV);
        gv = ((row * H + h) * D + v0) * (int)sizeof(T) + b;
        sv = row * G::LSV + b;
        gb = (lane * H + h) * 4;
    }
};

// WQ: with the q rows (the states-only mode reads none).
template <bool WQ, typename T, int D, int DVS, bool SG>
__device__ __forceinline__ void load_chunk(ChunkRegs<T, D, DVS, SG> &R, const ChunkSrc &s,
                                           const ChunkOffsets<T, D, DVS, SG> &o, int wave,
                                           int lane) {
    typedef Cfg<T, D, DVS, SG> G;
#pragma unroll
    for (int i = 0; i < G::IK; ++i) {
        R.k[i] = buf_load<4>(s.k, o.gk[i]);
        if constexpr (WQ) R.q[i] = buf_load<4>(s.q, o.gk[i]);
    }
#pragma unroll
    for (int i = 0; i < G::IG; ++i) R.g[i] = buf_load<4>(s.g, o.gg[i]);
    if (wave >= G::PW - G::NIV) R.v = buf_load<4>(s.v, o.gv);
    if (wave == G::PW - 1 && lane < kC) {
        R.beta = __uint_as_float(buf_load<1>(s.b, o.gb).w[0]);
        if constexpr (SG) R.gs = __uint_as_float(buf_load<1>(s.g, o.gb).w[0]);
    }
}

// The pieces into the staging area (waits for the loads to land).
template <bool WQ, typename T, int D, int DVS, bool SG>
__device__ __forceinline__ void stage_chunk(const ChunkRegs<T, D, DVS, SG> &R, unsigned char *smem,
                                            const ChunkOffsets<T, D, DVS, SG> &o, int wave,
                                            int lane) {
    typedef Cfg<T, D, DVS, SG> G;
    auto st16 = [](unsigned char *p, const Raw<4> &x) {
        *reinterpret_cast<u32x4 *>(p) = u32x4{x.w[0], x.w[1], x.w[2], x.w[3]};
    };
#pragma unroll
    for (int i = 0; i < G::IK; ++i) {
        st16(smem + G::oRK + o.sk[i], R.k[i]);
        if constexpr (WQ) st16(smem + G::oRQ + o.sk[i], R.q[i]);
    }
#pragma unroll
    for (int i = 0; i < G::IG; ++i) st16(smem + G::oRG + o.sg[i], R.g[i]);
    if (wave >= G::PW - G::NIV) st16(smem + G::oRV + o.sv, R.v);
    if (wave == G::PW - 1 && lane < kC) {
        reinterpret_cast<float *>(smem + G::oRB)[lane] = R.beta;
        if constexpr (SG) reinterpret_cast<float *>(smem + G::oRG)[lane] = R.gs;
    }
}

// DPP helpers (all lanes active).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf,
                                                      false));
}
// every lane of a group of 4 receives x from lane SRC of its group
template <int SRC>
__device__ __forceinline__ float quad_bcast(float x) { return dpp<SRC * 0x55, 0xf>(x); }

// ------------------------------------------------------------ scan products
// A-operand fragment of contraction block kb for the 16 rows starting at
// `row0` (leading dimension ld, physical order), and the MFMA with a B operand
// taken from accumulator tiles (bf16: two stacked 16x16 tiles; fp32: one).
template <typename T> struct ScanMma;
template <> struct ScanMma<bf16> {
    typedef bf16x8 Frag;
    __device__ static Frag a(const bf16 *row0, int ld, int kb, int lane) {
        return *reinterpret_cast<const bf16x8 *>(row0 + (lane & 15) * ld + 32 * kb +
                                                 8 * (lane >> 4));
    }
    __device__ static Frag b(const f32x4 &lo, const f32x4 &hi) {
        Frag f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = static_cast<bf16>(lo[e]);
            f[4 + e] = static_cast<bf16>(hi[e]);
        }
        return f;
    }
    __device__ static f32x4 mma(f32x4 acc, const Frag &a, const Frag &b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
};
template <> struct ScanMma<float> {
    typedef f32x4 Frag;
    __device__ static Frag a(const float *row0, int ld, int kb, int lane) {
        return *reinterpret_cast<const f32x4 *>(row0 + (lane & 15) * ld + 16 * kb +
                                                4 * (lane >> 4));
    }
    __device__ static Frag b(const f32x4 &t, const f32x4 &) { return t; }
    __device__ static f32x4 mma(f32x4 acc, const Frag &a, const Frag &b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
        return acc;
    }
};

// acc += A B for 16x16 blocks over a contraction of 16: A row-major in LDS
// (leading dimension ld, lane reads 4 consecutive k), B an accumulator tile
// (its rows are the contraction index).
template <typename T>
__device__ __forceinline__ f32x4 mm16(f32x4 acc, const T *A, int ld, const f32x4 &B, int lane);
template <>
__device__ __forceinline__ f32x4 mm16<bf16>(f32x4 acc, const bf16 *A, int ld, const f32x4 &B,
                                            int lane) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(A + (lane & 15) * ld + 4 * (lane >> 4));
    bf16x4 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) b[e] = static_cast<bf16>(B[e]);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                      __builtin_bit_cast(i16x4, b), acc, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mm16<float>(f32x4 acc, const float *A, int ld, const f32x4 &B,
                                             int lane) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(A + (lane & 15) * ld + 4 * (lane >> 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], B[e], acc, 0, 0, 0);
    return acc;
}

// MODE (compile time, so the output path's code is untouched by it):
//   kModeOut    the prefill: outputs, final states, snapshots;
//   kModeState  no outputs (out is not used): final states only;
//   kModeMap    no outputs, zero values (v is not used) and every workgroup
//               starting from S = I: the final state is the sequence's state
//               transition (transposed like every state);
//   kModeStates no outputs: the state entering every 16-token block of each
//               sequence (the checkpoints of the chunked backward) goes to
//               `snapshots`, slot tbeg / 16 + n + j for block j of sequence n,
//               [slot][H][d_v][d_k] in the input dtype (bf16 for bf16 inputs).
//               A 32-token chunk's second block enters
//               with e^{Gamma_15} S + (K e^{Gamma_15 - Gamma})_{0..15}^T Delta_0,
//               the block-0 half of the chunk's own transition.
// LPT (compile time, packed input with at most 64 sequences): workgroups take
// the sequences longest first (see below); otherwise in sequence order.
// FAR (compile time): false = the fast kernel: every chunk through the
// factorised products; a (sequence, head, slice) unit with a chunk out of
// their range (a 16-token block decaying beyond 2^-kFarLog2 in some channel,
// or a -inf / NaN gate) is marked instead of finished: its final state is
// left unwritten and the first element of its output slice (of its final
// state when there are no outputs) is set to NaN.  true = the fix-up kernel,
// launched right after on the same stream: units without the mark return at
// once; marked units are recomputed from their initial state, out-of-range
// chunks token by token (exact recurrence in fp32).  The states mode of the
// backward uses the fast kernel without marks.
template <typename T, int D, int DVS, bool SG, int MODE, bool LPT, bool FAR>
__global__ __launch_bounds__(64 * (D / 16 + DVS / 16)) void chunk_fwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ initial_state, const int32_t *__restrict__ cu_seqlens,
    T *__restrict__ out, float *__restrict__ final_state, float *__restrict__ snapshots,
    int snap_every, int snap_cap, int num_seqs, int seq_len, int total_tokens,
    int H, int units, int units_per_xcd, unsigned *__restrict__ far_flags) {
    typedef Cfg<T, D, DVS, SG> G;
    typedef Mma<T> M;
    typedef ScanMma<T> SM;
    constexpr int NS = D / DVS;

    __shared__ __attribute__((aligned(16))) unsigned char smem[G::BYTES];

    // XCD-aware unit order: workgroups are dealt to the 8 XCDs round-robin,
    // so give each XCD a contiguous run of units; the NS slices of one
    // (sequence, head) then share that XCD's L2 for their common inputs.
    const int bid = blockIdx.x;
    int unit = (bid & 7) * units_per_xcd + (bid >> 3);
    if constexpr (LPT) {
        // Packed sequences of unequal length: longest first, so the longest
        // chains start at once and shorter ones fill in behind them.  The k-th
        // workgroup dispatched to XCD x takes position u of the longest-first
        // order; the NS slices of a head stay together on one XCD and heads go
        // round-robin over the XCDs.  (The grid is padded to 8 NS units.)
        const int lane = threadIdx.x & 63, k = bid >> 3;
        const int u = NS * (8 * (k / NS) + (bid & 7)) + k % NS;
        int len = -1;  // lane m: the clamped length of sequence m
        if (lane < num_seqs) {
            int a = cu_seqlens[lane], b = cu_seqlens[lane + 1];
            a = a < 0 ? 0 : (a > total_tokens ? total_tokens : a);
            b = b < a ? a : (b > total_tokens ? total_tokens : b);
            len = b - a;
        }
        int rank = 0;  // longer sequences, then equal ones with a smaller index
        for (int m = 0; m < num_seqs; ++m) {
            const int lm = __builtin_amdgcn_readlane(len, m);
            rank += (lm > len || (lm == len && m < lane)) ? 1 : 0;
        }
        const int p = u / (H * NS);
        const unsigned long long hit = __ballot(lane < num_seqs && rank == p);
        const int m = hit ? __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1) : num_seqs;
        unit = m * H * NS + u % (H * NS);
    }
    if (unit >= units) return;
    const int slice = unit % NS;
    const int nh = unit / NS;
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
    const int nchunks = (int)((tend - tbeg + kC - 1) / kC);
    // the fast kernel marks far units (states mode: for the backward's flags)
    constexpr bool MARK = !FAR;
    // the states-only mode forms no outputs: no q rows, Q+ or Mqk tiles
    constexpr bool WQ = MODE != kModeStates;
    if constexpr (FAR) {
        // the fix-up pass: only units the fast kernel marked (the same
        // element for every thread, so the whole workgroup returns together)
        if (nchunks == 0) return;
        const float mk = out ? to_f32(out[(tbeg * H + h) * (int64_t)D + v0])
                             : final_state[((int64_t)n * H + h) * D * D + (int64_t)v0 * D];
        if (!__builtin_isnan(mk)) return;
    }

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a scalar: the role branches below contain barriers and
    // must be uniform branches, never exec-masked ones
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, l4 = lane >> 4;

    // The sticky out-of-range words start cleared in both buffer sets.
    if (tid < 2) *reinterpret_cast<unsigned *>(smem + tid * G::SET + G::sMark) = 0u;
    // The upper-right 16x16 block of Mqk is never written: zero it once in
    // both buffer sets.
    for (int i = tid; i < 2 * kBS * kBS; i += G::THREADS) {
        unsigned char *set = smem + (i / (kBS * kBS)) * G::SET;
        const int r = (i / kBS) % kBS, c = phys<T>(kBS + i % kBS);
        reinterpret_cast<T *>(set + G::sMQ)[r * G::LDT + c] = from_f32<T>(0.f);
    }

    // The two wave groups run separate loops with the same number of
    // workgroup barriers (one before the loop, three per chunk), so each
    // group keeps only its own loop-carried registers.
    if (wave < G::PW) {
        T *sKD = reinterpret_cast<T *>(smem + G::oKD);
        T *sQD = reinterpret_cast<T *>(smem + G::oQD);
        T *sKM = reinterpret_cast<T *>(smem + G::oKM);
        float *sAt = reinterpret_cast<float *>(smem + G::oAt);
        // thread map: token rows r (block 0) and r + 16 (block 1), r = lane % 16,
        // so the 16 lanes of a DPP row are the 16 tokens of each block; logical
        // channels c .. c + 3 (physical pc .. pc + 3), c = 4 (4 wave + lane / 16)
        const int r = lane & 15;
        const int c = 4 * (4 * wave + (lane >> 4));
        const int pc = phys<T>(c);
        const ChunkOffsets<T, D, DVS, SG> offs(wave, lane, h, H, v0);
        auto src = [&](int ci) {
            const int64_t t0 = tbeg + (int64_t)ci * kC;
            return chunk_src<MODE == kModeMap>(q, k, v, log_alpha, beta, t0,
                             (int)((tend - t0) < kC ? (tend - t0) : kC), H, D, SG);
        };
        // Two register sets: the loads of chunk n + 2 go out at the start of
        // tick n and are staged at the end of tick n + 1, so a load has about
        // two ticks to land (global loads under this kernel's traffic take
        // about as long as one tick).
        ChunkRegs<T, D, DVS, SG> RA, RB;
        if (nchunks > 0) {
            load_chunk<WQ>(RA, src(0), offs, wave, lane);
            stage_chunk<WQ>(RA, smem, offs, wave, lane);
        }
        __syncthreads();
        if (nchunks > 1) load_chunk<WQ>(RB, src(1), offs, wave, lane);

        // one tick: Rl receives chunk tick + 2, Rs (chunk tick + 1) is staged
        auto prep_tick = [&](int tick, ChunkRegs<T, D, DVS, SG> &Rl,
                             ChunkRegs<T, D, DVS, SG> &Rs) {
            const bool on = tick < nchunks;  // prepares chunk `tick`
            unsigned char *PS = smem + (tick & 1) * G::SET;
            T *pKP = reinterpret_cast<T *>(PS + G::sKP);
            T *pQP = reinterpret_cast<T *>(PS + G::sQP);
            T *pKET = reinterpret_cast<T *>(PS + G::sKET);
            T *pMQ = reinterpret_cast<T *>(PS + G::sMQ);
            T *pT3 = reinterpret_cast<T *>(PS + G::sT3);
            T *pV = reinterpret_cast<T *>(PS + G::sV);
            float *pGam = reinterpret_cast<float *>(PS + G::sGam);
            float *pF1 = reinterpret_cast<float *>(PS + G::sF1);
            float *pBeta = reinterpret_cast<float *>(PS + G::sBeta);

            // ------------------------------------------------------ phase 1
            if (on) {
                // the loads of chunk tick + 2 go out first (staged next tick)
                if (tick + 2 < nchunks) load_chunk<WQ>(Rl, src(tick + 2), offs, wave, lane);
                // this chunk's rows r and r + 16 from the staging area
                Raw<G::RW> rk[2], rq[2];
                float d0[4], d1[4], erho[4];  // gates of rows r, r + 16 (channels c .. c + 3)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int row = r + kBS * j;
                    if constexpr (G::RW == 2) {
                        const u32x2 a = *reinterpret_cast<const u32x2 *>(
                            smem + G::oRK + row * G::LSK + c * G::SZ);
                        rk[j].w[0] = a[0]; rk[j].w[1] = a[1];
                        if constexpr (WQ) {
                            const u32x2 b = *reinterpret_cast<const u32x2 *>(
                                smem + G::oRQ + row * G::LSK + c * G::SZ);
                            rq[j].w[0] = b[0]; rq[j].w[1] = b[1];
                        }
                    } else {
                        const u32x4 a = *reinterpret_cast<const u32x4 *>(
                            smem + G::oRK + row * G::LSK + c * G::SZ);
#pragma unroll
                        for (int i = 0; i < 4; ++i) rk[j].w[i] = a[i];
                        if constexpr (WQ) {
                            const u32x4 b = *reinterpret_cast<const u32x4 *>(
                                smem + G::oRQ + row * G::LSK + c * G::SZ);
#pragma unroll
                            for (int i = 0; i < 4; ++i) rq[j].w[i] = b[i];
                        }
                    }
                    if constexpr (!SG) {
                        const f32x4 gg = *reinterpret_cast<const f32x4 *>(
                            smem + G::oRG + row * G::LSG + c * 4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) (j ? d1 : d0)[i] = gg[i];
                    }
                }
                // block-relative inclusive prefix of the log2-gates (block 0's is
                // chunk-relative); rho = Gamma_15 = block 0's total (lane 15)
                if constexpr (SG) {
                    // one gate per token: a single prefix serves all four channels
                    const float *gsv = reinterpret_cast<const float *>(smem + G::oRG);
                    float x = gsv[r] * kLog2e, y = gsv[r + kBS] * kLog2e;
                    x += dpp_row_shr<1>(x);
                    y += dpp_row_shr<1>(y);
                    x += dpp_row_shr<2>(x);
                    y += dpp_row_shr<2>(y);
                    x += dpp_row_shr<4>(x);
                    y += dpp_row_shr<4>(y);
                    x += dpp_row_shr<8>(x);
                    y += dpp_row_shr<8>(y);
                    const float er = fast_exp2(dpp<0x15f, 0xf>(x));  // row_newbcast:15
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        d0[e] = x;
                        d1[e] = y;
                        erho[e] = er;
                    }
                } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x = d0[e] * kLog2e, y = d1[e] * kLog2e;
                    x += dpp_row_shr<1>(x);
                    y += dpp_row_shr<1>(y);
                    x += dpp_row_shr<2>(x);
                    y += dpp_row_shr<2>(y);
                    x += dpp_row_shr<4>(x);
                    y += dpp_row_shr<4>(y);
                    x += dpp_row_shr<8>(x);
                    y += dpp_row_shr<8>(y);
                    d0[e] = x;
                    d1[e] = y;
                    erho[e] = fast_exp2(dpp<0x15f, 0xf>(x));  // row_newbcast:15
                }
                }
                float kf[4], qf[4];
                float kt0[4], kt1[4], ep1[4];
                {
                    // block 0: chunk-relative K+, Q+, K- and K e^{rho - Gamma}
                    float kp[4], qp[4], km[4];
                    unpack<T, 4>(rk[0], kf);
                    if constexpr (WQ) unpack<T, 4>(rq[0], qf);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float ep = fast_exp2(d0[e]), em = fast_exp2(-d0[e]);
                        kp[e] = kf[e] * ep;
                        if constexpr (WQ) qp[e] = qf[e] * ep;
                        km[e] = kf[e] * em;
                        kt0[e] = km[e] * erho[e];
                    }
                    st4(pKP + r * G::LDK + pc, kp);
                    if constexpr (WQ) st4(pQP + r * G::LDK + pc, qp);
                    st4(sKM + r * G::LDK + pc, km);
                }
                {
                    // block 1: K+, Q+, K- relative to rho, chunk-relative K+, Q+
                    float kd[4], qd[4], kp[4], qp[4];
                    unpack<T, 4>(rk[1], kf);
                    if constexpr (WQ) unpack<T, 4>(rq[1], qf);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ep1[e] = fast_exp2(d1[e]);
                        const float em = fast_exp2(-d1[e]);
                        kd[e] = kf[e] * ep1[e];
                        if constexpr (WQ) qd[e] = qf[e] * ep1[e];
                        kp[e] = kd[e] * erho[e];
                        if constexpr (WQ) qp[e] = qd[e] * erho[e];
                        kt1[e] = kf[e] * em;  // K- of block 1 = K e^{rho - Gamma}
                    }
                    st4(pKP + (kBS + r) * G::LDK + pc, kp);
                    if constexpr (WQ) st4(pQP + (kBS + r) * G::LDK + pc, qp);
                    st4(sKM + (kBS + r) * G::LDK + pc, kt1);
                    st4(sKD + r * G::LDK + pc, kd);
                    if constexpr (WQ) st4(sQD + r * G::LDK + pc, qd);
                }
                if (r == kBS - 1) {
                    // row 15 holds both blocks' total decay: a block that decays
                    // beyond 2^-kFarLog2 in one of these channels (or a -inf or
                    // NaN gate) makes the scan take this chunk token by token
                    bool far = false;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        far = far || !(d0[e] >= -kFarLog2) || !(d1[e] >= -kFarLog2);
                    if constexpr (FAR)  // this chunk, read by the scan next tick
                        *reinterpret_cast<unsigned *>(
                            PS + G::flag_offset(4 * wave + (lane >> 4))) = far ? 1u : 0u;
                    else if constexpr (MARK)  // sticky: some chunk of this unit
                        if (far) *reinterpret_cast<unsigned *>(PS + G::sMark) = 1u;
                    // row 31: f = e^{Gamma_last - rho}, gamma = e^{Gamma_last}
                    *reinterpret_cast<f32x4 *>(pF1 + c) = f32x4{ep1[0], ep1[1], ep1[2], ep1[3]};
                    *reinterpret_cast<f32x4 *>(pGam + c) =
                        f32x4{erho[0] * ep1[0], erho[1] * ep1[1], erho[2] * ep1[2],
                              erho[3] * ep1[3]};
                    // e^{rho} for the mid-chunk state (states mode: the O staging
                    // area is free, one D-float slot per buffer set)
                    if constexpr (MODE == kModeStates)
                        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(smem + G::oO) +
                                                   (tick & 1) * D + c) =
                            f32x4{erho[0], erho[1], erho[2], erho[3]};
                }
                // (K e^{rho - Gamma})^T, channel rows, token pairs (r, r + 1) of
                // both blocks: the even lane stores channels c, c + 1, the odd
                // lane channels c + 2, c + 3
                {
                    const bool odd = r & 1;
                    const int tr = r & ~1;
                    T *dst = pKET + (c + (odd ? 2 : 0)) * G::LDT;
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        const float *kt = b ? kt1 : kt0;
                        const int tcol = phys<T>(kBS * b + tr);
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const float own = odd ? kt[e + 2] : kt[e];
                            const float send = odd ? kt[e] : kt[e + 2];
                            const float recv = dpp<0xb1, 0xf>(send);  // quad_perm [1,0,3,2]
                            const float lo = odd ? recv : own, hi = odd ? own : recv;
                            if constexpr (sizeof(T) == 2)
                                *reinterpret_cast<unsigned *>(dst + e * G::LDT + tcol) =
                                    pack2(lo, hi);
                            else
                                *reinterpret_cast<f32x2 *>(dst + e * G::LDT + tcol) =
                                    f32x2{lo, hi};
                        }
                    }
                }
                // V slice and beta copies last: their LDS round trips stay off
                // the path of the elementwise work
                if (tid < G::VTH) {
                    const int vr = tid / (DVS / G::VE), vc = G::VE * (tid % (DVS / G::VE));
                    *reinterpret_cast<u32x4 *>(pV + vr * G::LDV + vc) =
                        *reinterpret_cast<const u32x4 *>(smem + G::oRV + vr * G::LSV +
                                                         vc * G::SZ);
                }
                if (tid < kC) pBeta[tid] = reinterpret_cast<const float *>(smem + G::oRB)[tid];
            }
            __syncthreads();

            // ------------------------------------------------------ phase 2
            // tiles 0-5 = A_00 (then T_00), A_11 (then T_11), A_10, Mqk_00,
            // Mqk_11, Mqk_10; wave w takes tiles w and w + PW (products over
            // physical channels, both operands in the same order)
            // the waves without a diagonal tile hold back briefly, so the LDS
            // reads of the two diagonal tiles (the head of the substitution
            // chain, the longest path of this phase) are served first
            if (wave >= 2) __builtin_amdgcn_s_sleep(2);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tile = wave + u * G::PW;
                if (!on || tile >= (WQ ? 6 : 3)) continue;  // (no Mqk without outputs)
                const bool isA = tile < 3;
                const int t = isA ? tile : tile - 3;  // 0: (0,0), 1: (1,1), 2: (1,0)
                const int I = t == 0 ? 0 : 1, J = t == 1 ? 1 : 0;
                const T *left = t == 0 ? (isA ? pKP : pQP)
                                       : (t == 1 ? (isA ? sKD : sQD)
                                                 : (isA ? pKP : pQP) + kBS * G::LDK);
                const f32x4 acc = tile_mma<T, D>(zero4(), left, G::LDK, sKM + kBS * J * G::LDK,
                                                 G::LDK, lane);
                if (!isA) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int rr = 4 * l4 + e;
                        const float val = (I == J && l16 > rr) ? 0.f : acc[e];
                        pMQ[(kBS * I + rr) * G::LDT + phys<T>(kBS * J + l16)] = from_f32<T>(val);
                    }
                } else if (I != J) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int rr = 4 * l4 + e;  // A_10 = diag(b_1) (K+ K-^T)_10
                        pT3[G::B_T16 / G::SZ + rr * G::LDTT + l16] =
                            from_f32<T>(acc[e] * pBeta[kBS + rr]);
                    }
                } else {
                    // diagonal block: strictly lower part, stored transposed
                    // (row c of At = column c of A_II), then inverted here
                    float a[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int rr = 4 * l4 + e;
                        a[e] = l16 < rr ? acc[e] * pBeta[kBS * I + rr] : 0.f;
                    }
                    float *At = sAt + I * kBS * G::LDAT;
                    store4(At + l16 * G::LDAT + 4 * l4, a[0], a[1], a[2], a[3]);
                    wave_lds_fence();
                    // lane 4 j + g holds rows 4 g .. 4 g + 3 of column j of
                    // (I + A_II)^{-1}; forward substitution, one column of A per
                    // step, the pivot broadcast inside the lane quad
                    const int j = lane >> 2, g = lane & 3;
                    float s[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[e] = (4 * g + e == j) ? 1.f : 0.f;
                    constexpr int LA = 4;  // columns of A read ahead of their step
                    f32x4 col[kBS - 1];
#pragma unroll
                    for (int i = 0; i < LA; ++i)
                        col[i] = *reinterpret_cast<const f32x4 *>(At + i * G::LDAT + 4 * g);
#pragma unroll
                    for (int i = 0; i < kBS - 1; ++i) {
                        if (i + LA < kBS - 1)
                            col[i + LA] = *reinterpret_cast<const f32x4 *>(
                                At + (i + LA) * G::LDAT + 4 * g);
                        float x;
                        switch (i >> 2) {  // pivot T[i][j] from quad lane i / 4
                            case 0: x = quad_bcast<0>(s[i & 3]); break;
                            case 1: x = quad_bcast<1>(s[i & 3]); break;
                            case 2: x = quad_bcast<2>(s[i & 3]); break;
                            default: x = quad_bcast<3>(s[i & 3]); break;
                        }
                        // A[rr][i] = 0 for rr <= i, so settled rows are unchanged
#pragma unroll
                        for (int e = 0; e < 4; ++e) s[e] -= col[i][e] * x;
                    }
                    // T'_00 = T_00 diag(b_0) (block 0 of T3) or T_11 (block 2)
                    const float bj = I == 0 ? pBeta[j] : 1.f;
                    T *dstT = pT3 + (2 * I) * (G::B_T16 / G::SZ);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dstT[(4 * g + e) * G::LDTT + j] = from_f32<T>(s[e] * bj);
                }
            }
            // the next chunk's rows, loaded during phase 1, into the staging area
            if (tick + 1 < nchunks) stage_chunk<WQ>(Rs, smem, offs, wave, lane);
            __syncthreads();
        };
        for (int tick = 0; nchunks > 0 && tick <= nchunks; tick += 2) {
            prep_tick(tick, RA, RB);
            if (tick + 1 <= nchunks) prep_tick(tick + 1, RB, RA);
        }
        return;
    }

    // ------------------------------------------------------------------ scan
    // wave PW + ct owns value columns v0 + 16 ct .. + 15 of the state for all
    // d_k rows: NRT fp32 accumulator tiles (lane: value column 16 ct + l16,
    // key rows 16 t + 4 l4 + e)
    const int ct = wave - G::PW;
    T *sO = reinterpret_cast<T *>(smem + G::oO);  // [kC][LSV bytes], all scan waves
    const int64_t sbase = ((int64_t)n * H + h) * D * D;  // M = S^T: [d_v][d_k]
    // State snapshots: the state after the first j * snap_every tokens of this
    // sequence goes to entry snap_base + j - 1 of [snap_cap, H, d_v, d_k], where
    // snap_base counts the snapshots of the sequences before it (their lengths
    // clamped exactly as their own workgroups clamp them).
    int snap_base = 0;
    if (MODE != kModeStates && snapshots) {
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
    const int vcol = v0 + 16 * ct + l16;
    f32x4 Sm[G::NRT];
#pragma unroll
    for (int t = 0; t < G::NRT; ++t)
        Sm[t] = MODE == kModeMap
                    ? f32x4{vcol == 16 * t + 4 * l4 ? 1.f : 0.f, vcol == 16 * t + 4 * l4 + 1 ? 1.f : 0.f,
                            vcol == 16 * t + 4 * l4 + 2 ? 1.f : 0.f,
                            vcol == 16 * t + 4 * l4 + 3 ? 1.f : 0.f}
                : initial_state ? *reinterpret_cast<const f32x4 *>(initial_state + sbase +
                                                                  (int64_t)vcol * D + 16 * t +
                                                                  4 * l4)
                                : zero4();
    __syncthreads();

    bool far_next = false;  // the chunk scanned in the next tick is out of range
    for (int tick = 0; nchunks > 0 && tick <= nchunks; ++tick) {
        const bool on = tick > 0;  // scans chunk `tick - 1`
        const unsigned char *SS = smem + ((tick & 1) ^ 1) * G::SET;
        const T *cKP = reinterpret_cast<const T *>(SS + G::sKP);
        const T *cQP = reinterpret_cast<const T *>(SS + G::sQP);
        const T *cKET = reinterpret_cast<const T *>(SS + G::sKET);
        const T *cMQ = reinterpret_cast<const T *>(SS + G::sMQ);
        const T *cT3 = reinterpret_cast<const T *>(SS + G::sT3);
        const T *cV = reinterpret_cast<const T *>(SS + G::sV);
        const float *cBeta = reinterpret_cast<const float *>(SS + G::sBeta);
        const float *cGam = reinterpret_cast<const float *>(SS + G::sGam);
        const float *cF1 = reinterpret_cast<const float *>(SS + G::sF1);
        f32x4 Dl[2];  // Delta row tiles (tokens 0-15, 16-31), kept for phase 2
        const int64_t tok0 = tbeg + (int64_t)(tick - 1) * kC;
        const int nvalid = (int)((tend - tok0) < kC ? (tend - tok0) : kC);
        // chunks the preparation flagged as beyond the factorised range are
        // taken token by token (uniform over the workgroup; the flag was read
        // in the previous tick, right after the preparation wrote it)
        const bool far = FAR && on && far_next;

        // ---------------------------------------------------------- phase 1
        if (on && far) {
            // The recurrence itself, token by token, in fp32: S' = Diag(a) S,
            // p = S'^T k, delta = b (v - p), S = S' + k delta^T, o = S^T q
            // ([K3-explainer] §三/§四).  Lane (l16, l4) holds value column vcol
            // and key rows 16 t + 4 l4 + e of S; each token's k, q and gates
            // come straight from global memory.
            const int m2 = 2 * (tick - 1);
            const bool mid = m2 + 1 < (int)((tend - tbeg + kBS - 1) / kBS);
            const int64_t soff = ((tbeg / kBS + n + m2) * H + h) * (int64_t)D * D +
                                 (int64_t)vcol * D + 4 * l4;
            auto put_state = [&](int64_t e0) {
#pragma unroll
                for (int t = 0; t < G::NRT; ++t) {
                    if constexpr (sizeof(T) == 2)
                        *reinterpret_cast<u32x2 *>(reinterpret_cast<bf16 *>(snapshots) + e0 +
                                                   16 * t) =
                            u32x2{pack2(Sm[t][0], Sm[t][1]), pack2(Sm[t][2], Sm[t][3])};
                    else
                        *reinterpret_cast<f32x4 *>(snapshots + e0 + 16 * t) = Sm[t];
                }
            };
            if constexpr (MODE == kModeStates) put_state(soff);
            for (int j = 0; j < nvalid; ++j) {
                const int64_t row = (tok0 + j) * H + h;
                const T *kr = k + row * D + 4 * l4;
                const T *qr = q + row * D + 4 * l4;
                float p = 0.f;
#pragma unroll
                for (int t = 0; t < G::NRT; ++t) {
                    float kf[4], af[4];
                    load4(kr + 16 * t, kf);
                    if constexpr (SG) {
                        const float a = fast_exp2(log_alpha[row] * kLog2e);
#pragma unroll
                        for (int e = 0; e < 4; ++e) af[e] = a;
                    } else {
                        const f32x4 g = *reinterpret_cast<const f32x4 *>(
                            log_alpha + row * D + 16 * t + 4 * l4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) af[e] = fast_exp2(g[e] * kLog2e);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Sm[t][e] *= af[e];
                        p += Sm[t][e] * kf[e];
                    }
                }
                p += __shfl_xor(p, 16, 64);
                p += __shfl_xor(p, 32, 64);
                const float vv = MODE == kModeMap ? 0.f : to_f32(v[row * D + vcol]);
                const float dl = beta[row] * (vv - p);
                float o = 0.f;
#pragma unroll
                for (int t = 0; t < G::NRT; ++t) {
                    float kf[4], qf[4];
                    load4(kr + 16 * t, kf);
                    load4(qr + 16 * t, qf);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Sm[t][e] += kf[e] * dl;
                        o += Sm[t][e] * qf[e];
                    }
                }
                if constexpr (MODE == kModeOut) {
                    o += __shfl_xor(o, 16, 64);
                    o += __shfl_xor(o, 32, 64);
                    if (l4 == 0) sO[j * (G::LSV / G::SZ) + 16 * ct + l16] = from_f32<T>(o);
                }
                if constexpr (MODE == kModeStates)
                    if (j == kBS - 1 && mid) put_state(soff + (int64_t)H * D * D);
            }
        } else if (on) {
            // the state as B operands, one per contraction block
            typename SM::Frag Sb[D / G::KB];
#pragma unroll
            for (int kb = 0; kb < D / G::KB; ++kb) {
                if constexpr (sizeof(T) == 2)
                    Sb[kb] = SM::b(Sm[2 * kb], Sm[2 * kb + 1]);
                else
                    Sb[kb] = SM::b(Sm[kb], Sm[kb]);
            }
            f32x4 PK[2], PQ[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                PK[rt] = zero4();
                PQ[rt] = zero4();
#pragma unroll
                for (int kb = 0; kb < D / G::KB; ++kb) {
                    PK[rt] = SM::mma(PK[rt], SM::a(cKP + kBS * rt * G::LDK, G::LDK, kb, lane),
                                     Sb[kb]);
                    PQ[rt] = SM::mma(PQ[rt], SM::a(cQP + kBS * rt * G::LDK, G::LDK, kb, lane),
                                     Sb[kb]);
                }
            }
            // X = V - K+ S (accumulator layout: token rows 16 rt + 4 l4 + e)
            f32x4 X[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    X[rt][e] = to_f32(cV[(kBS * rt + 4 * l4 + e) * G::LDV + 16 * ct + l16]) -
                               PK[rt][e];
            // Delta solves (I + A) Delta = diag(b) X block by block:
            // Delta_0 = T_00 b_0 X_0, Delta_1 = T_11 (b_1 X_1 - A_10 Delta_0)
            constexpr int T16 = G::B_T16 / G::SZ;
            Dl[0] = mm16<T>(zero4(), cT3, G::LDTT, X[0], lane);
            {
                const f32x4 ad = mm16<T>(zero4(), cT3 + T16, G::LDTT, Dl[0], lane);
                const f32x4 b1 = *reinterpret_cast<const f32x4 *>(cBeta + kBS + 4 * l4);
                f32x4 r1;
#pragma unroll
                for (int e = 0; e < 4; ++e) r1[e] = b1[e] * X[1][e] - ad[e];
                Dl[1] = mm16<T>(zero4(), cT3 + 2 * T16, G::LDTT, r1, lane);
            }
            // O = Q+ S + Mqk Delta (Mqk lower triangular); only with outputs
            const typename SM::Frag Db0 = SM::b(Dl[0], Dl[1]);
            const typename SM::Frag Db1 = SM::b(Dl[1], Dl[1]);
#pragma unroll
            for (int rt = 0; rt < 2 && MODE == kModeOut; ++rt) {
                PQ[rt] = SM::mma(PQ[rt], SM::a(cMQ + kBS * rt * G::LDT, G::LDT, 0, lane), Db0);
                if (sizeof(T) == 4 && rt == 1)
                    PQ[rt] = SM::mma(PQ[rt], SM::a(cMQ + kBS * rt * G::LDT, G::LDT, 1, lane), Db1);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sO[(kBS * rt + 4 * l4 + e) * (G::LSV / G::SZ) + 16 * ct + l16] =
                        from_f32<T>(PQ[rt][e]);
            }
        }
        __syncthreads();

        // ---------------------------------------------------------- phase 2
        if (FAR && tick < nchunks) {
            // chunk `tick`, just prepared, is scanned next tick: the
            // preparation's out-of-range words for it (lane j < 4 PW reads word j)
            const unsigned fw =
                lane < 4 * G::PW ? *reinterpret_cast<const unsigned *>(
                                       smem + (tick & 1) * G::SET + G::flag_offset(lane))
                                 : 0u;
            far_next = __ballot(fw != 0u) != 0ull;
        }
        if (on) {
            // the chunk's O rows (32 x DVS), whole rows in 16-byte pieces
            constexpr int LV = G::RBV / 16;
#pragma unroll
            for (int i = 0; i < G::IO && MODE == kModeOut; ++i) {
                const int p = (ct * G::IO + i) * 64 + lane, orow = p / LV, b = 16 * (p % LV);
                if (orow < nvalid)
                    *reinterpret_cast<u32x4 *>(reinterpret_cast<unsigned char *>(
                                                   out + ((tok0 + orow) * H + h) * (int64_t)D +
                                                   v0) + b) =
                        *reinterpret_cast<const u32x4 *>(
                            reinterpret_cast<const unsigned char *>(sO) + orow * G::LSV + b);
            }
            // S <- Diag(gamma) S + Diag(f1) (K e^{rho - Gamma})^T Delta
            // (far chunks: already stepped token by token in phase 1)
            const typename SM::Frag Db0 = SM::b(Dl[0], Dl[1]);
            const typename SM::Frag Db1 = SM::b(Dl[1], Dl[1]);
            if (!far) {
            if constexpr (MODE == kModeStates) {
                // the chunk's entering state (block 2 m) and, if the sequence has
                // a block 2 m + 1, the state after block 0:
                // e^{rho} S + (K e^{rho - Gamma})_{block 0}^T Delta_0.
                // (K e^{rho - Gamma})^T Delta is taken as its block-0 and block-1
                // halves, the second accumulated onto the first (one product
                // shape): the first half is also the mid-chunk state's product.
                // The mid test sits outside the tile loop, so that the tiles'
                // operand reads can run ahead of their products.
                const int m2 = 2 * (tick - 1);
                const int nblk = (int)((tend - tbeg + kBS - 1) / kBS);
                const bool mid = m2 + 1 < nblk;
                const float *cRho =
                    reinterpret_cast<const float *>(smem + G::oO) + ((tick - 1) & 1) * D;
                // element offset of this lane's four rows; the states are kept in
                // the input dtype (bf16 for bf16 inputs)
                const int64_t off = ((tbeg / kBS + n + m2) * H + h) * (int64_t)D * D +
                                    (int64_t)vcol * D + 4 * l4;
                const int64_t blk = (int64_t)H * D * D;
                auto put = [&](int64_t e0, const f32x4 &x) {
                    if constexpr (sizeof(T) == 2)
                        *reinterpret_cast<u32x2 *>(reinterpret_cast<bf16 *>(snapshots) + e0) =
                            u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])};
                    else
                        *reinterpret_cast<f32x4 *>(snapshots + e0) = x;
                };
                auto halves = [&](int t, f32x4 &h0, f32x4 &hf) {
                    if constexpr (sizeof(T) == 2) {
                        // block 0 holds elements 0-3 of each lane's fragment
                        // (tokens 4 g .. 4 g + 3), block 1 elements 4-7
                        const bf16x8 af = SM::a(cKET + 16 * t * G::LDT, G::LDT, 0, lane);
                        const bf16x4 lo{af[0], af[1], af[2], af[3]}, hi{af[4], af[5], af[6], af[7]};
                        const bf16x4 d0{static_cast<bf16>(Dl[0][0]), static_cast<bf16>(Dl[0][1]),
                                        static_cast<bf16>(Dl[0][2]), static_cast<bf16>(Dl[0][3])};
                        const bf16x4 d1{static_cast<bf16>(Dl[1][0]), static_cast<bf16>(Dl[1][1]),
                                        static_cast<bf16>(Dl[1][2]), static_cast<bf16>(Dl[1][3])};
                        h0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                            __builtin_bit_cast(i16x4, lo), __builtin_bit_cast(i16x4, d0), zero4(),
                            0, 0, 0);
                        hf = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                            __builtin_bit_cast(i16x4, hi), __builtin_bit_cast(i16x4, d1), h0, 0,
                            0, 0);
                    } else {
                        h0 = SM::mma(zero4(), SM::a(cKET + 16 * t * G::LDT, G::LDT, 0, lane), Db0);
                        hf = SM::mma(h0, SM::a(cKET + 16 * t * G::LDT, G::LDT, 1, lane), Db1);
                    }
                };
                // bf16: tiles t and t + 1 stored together, 16 bytes per lane.  A
                // lane holds keys 16 t + 4 l4 .. + 3 of each tile; one permlane16
                // swap per packed word gives the even rows (l4 = 2 j) keys 16 t +
                // 8 j .. + 7 of tile t and the odd rows keys 16 (t + 1) + 8 j .. + 7
                // of tile t + 1
                auto put2 = [&](int64_t e0, int t, const f32x4 &x0, const f32x4 &x1) {
                    const unsigned a0 = pack2(x0[0], x0[1]), a1 = pack2(x0[2], x0[3]);
                    const unsigned b0 = pack2(x1[0], x1[1]), b1 = pack2(x1[2], x1[3]);
                    const auto p0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
                    const auto p1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
                    const int64_t k0 = 16 * (t + (l4 & 1)) + 8 * (l4 >> 1);
                    *reinterpret_cast<u32x4 *>(reinterpret_cast<bf16 *>(snapshots) + e0 - 4 * l4 +
                                               k0) = u32x4{p0[0], p1[0], p0[1], p1[1]};
                };
                auto step = [&](int t, bool with_mid) {
                    // tiles t and t + 1 (bf16) or tile t (fp32)
                    constexpr int NP = sizeof(T) == 2 ? 2 : 1;
                    f32x4 h0[NP], hf[NP], sm[NP];
#pragma unroll
                    for (int u = 0; u < NP; ++u) {
                        halves(t + u, h0[u], hf[u]);
                        if (with_mid) {
                            const f32x4 rh =
                                *reinterpret_cast<const f32x4 *>(cRho + 16 * (t + u) + 4 * l4);
#pragma unroll
                            for (int e = 0; e < 4; ++e) sm[u][e] = rh[e] * Sm[t + u][e] + h0[u][e];
                        }
                    }
                    if constexpr (NP == 2) {
                        put2(off, t, Sm[t], Sm[t + 1]);
                        if (with_mid) put2(off + blk, t, sm[0], sm[1]);
                    } else {
                        put(off + 16 * t, Sm[t]);
                        if (with_mid) put(off + blk + 16 * t, sm[0]);
                    }
#pragma unroll
                    for (int u = 0; u < NP; ++u) {
                        const f32x4 gm = *reinterpret_cast<const f32x4 *>(cGam + 16 * (t + u) + 4 * l4);
                        const f32x4 f1 = *reinterpret_cast<const f32x4 *>(cF1 + 16 * (t + u) + 4 * l4);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            Sm[t + u][e] = gm[e] * Sm[t + u][e] + f1[e] * hf[u][e];
                    }
                };
                constexpr int TS = sizeof(T) == 2 ? 2 : 1;  // tiles per step
                static_assert(G::NRT % TS == 0, "tile pairs");
                if (mid) {
#pragma unroll
                    for (int t = 0; t < G::NRT; t += TS) step(t, true);
                } else {
#pragma unroll
                    for (int t = 0; t < G::NRT; t += TS) step(t, false);
                }
            } else {
#pragma unroll
            for (int t = 0; t < G::NRT; ++t) {
                f32x4 acc = SM::mma(zero4(), SM::a(cKET + 16 * t * G::LDT, G::LDT, 0, lane), Db0);
                if (sizeof(T) == 4)
                    acc = SM::mma(acc, SM::a(cKET + 16 * t * G::LDT, G::LDT, 1, lane), Db1);
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(cGam + 16 * t + 4 * l4);
                const f32x4 f1 = *reinterpret_cast<const f32x4 *>(cF1 + 16 * t + 4 * l4);
#pragma unroll
                for (int e = 0; e < 4; ++e) Sm[t][e] = gm[e] * Sm[t][e] + f1[e] * acc[e];
            }
            }
            }
            // a snapshot after every snap_every tokens (a multiple of the chunk
            // length, so only full chunks end on one)
            const int64_t done = (int64_t)tick * kC;
            if (MODE != kModeStates && snapshots && done % snap_every == 0 &&
                done <= tend - tbeg) {
                const int64_t idx = snap_base + done / snap_every - 1;
                if (idx < snap_cap) {
                    float *dst = snapshots + (idx * H + h) * D * D + (int64_t)vcol * D + 4 * l4;
#pragma unroll
                    for (int t = 0; t < G::NRT; ++t)
                        *reinterpret_cast<f32x4 *>(dst + 16 * t) = Sm[t];
                }
            }
        }
        __syncthreads();
    }

    bool marked = false;
    if constexpr (MARK) {
        // the preparation's sticky out-of-range words of both buffer sets
        // (their last writes came before the loop's last barrier)
        marked = __builtin_amdgcn_readfirstlane(
                     *reinterpret_cast<const unsigned *>(smem + G::sMark) |
                     *reinterpret_cast<const unsigned *>(smem + G::SET + G::sMark)) != 0u;
        if constexpr (MODE == kModeStates) {
            // the (sequence, head)'s 16 flag words: word 0 the mark, the rest 0
            if (far_flags && v0 == 0 && ct == 0 && lane < 16)
                far_flags[((int64_t)n * H + h) * 16 + lane] = (lane == 0 && marked) ? 1u : 0u;
        } else if (marked && ct == 0 && lane == 0) {
            if (out)
                out[(tbeg * H + h) * (int64_t)D + v0] = from_f32<T>(__builtin_nanf(""));
            else
                final_state[sbase + (int64_t)v0 * D] = __builtin_nanf("");
        }
    }
    if (final_state && !marked) {
#pragma unroll
        for (int t = 0; t < G::NRT; ++t)
            *reinterpret_cast<f32x4 *>(final_state + sbase + (int64_t)vcol * D + 16 * t +
                                       4 * l4) = Sm[t];
    }
}

template <typename T, int D, int DVS, bool SG, int MODE>
int launch(const void *q, const void *k, const void *v, const float *log_alpha, const float *beta,
           const float *initial_state, const int32_t *cu_seqlens, void *out, float *final_state,
           float *snapshots, int snap_every, int snap_cap, int num_seqs, int seq_len,
           int total_tokens, int H, unsigned *far_flags, hipStream_t stream) {
    const int64_t units64 = (int64_t)num_seqs * H * (D / DVS);
    if (units64 == 0) return 0;
    if (units64 > (int64_t)1 << 30) return -1;
    const int units = (int)units64;
    // a multiple of the slices per head, so that the longest-first order of
    // packed sequences maps the grid onto every unit
    const int per_xcd = (units + 8 * (D / DVS) - 1) / (8 * (D / DVS)) * (D / DVS);
#define KDA_KERNEL_ARGS                                                                        \
    static_cast<const T *>(q), static_cast<const T *>(k), static_cast<const T *>(v), log_alpha,  \
        beta, initial_state, cu_seqlens, static_cast<T *>(out), final_state, snapshots,        \
        snap_every, snap_cap, num_seqs, seq_len, total_tokens, H, units, per_xcd, far_flags
    // the fast kernel, then (except for the backward's states mode) the fix-up
    // pass over the units it marked
    constexpr bool FIXUP = MODE != kModeStates;
    if (cu_seqlens && num_seqs <= 64) {  // packed: longest sequences first
        hipLaunchKernelGGL((chunk_fwd_kernel<T, D, DVS, SG, MODE, true, false>),
                           dim3(8 * per_xcd), dim3(Cfg<T, D, DVS, SG>::THREADS), 0, stream,
                           KDA_KERNEL_ARGS);
        if (FIXUP)
            hipLaunchKernelGGL((chunk_fwd_kernel<T, D, DVS, SG, MODE, true, FIXUP>),
                               dim3(8 * per_xcd), dim3(Cfg<T, D, DVS, SG>::THREADS), 0, stream,
                               KDA_KERNEL_ARGS);
    } else {
        hipLaunchKernelGGL((chunk_fwd_kernel<T, D, DVS, SG, MODE, false, false>),
                           dim3(8 * per_xcd), dim3(Cfg<T, D, DVS, SG>::THREADS), 0, stream,
                           KDA_KERNEL_ARGS);
        if (FIXUP)
            hipLaunchKernelGGL((chunk_fwd_kernel<T, D, DVS, SG, MODE, false, FIXUP>),
                               dim3(8 * per_xcd), dim3(Cfg<T, D, DVS, SG>::THREADS), 0, stream,
                               KDA_KERNEL_ARGS);
    }
#undef KDA_KERNEL_ARGS
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <bool SG, int MODE>
int launch_dtype(const void *q, const void *k, const void *v, const float *log_alpha,
                 const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                 void *out, float *final_state, float *snapshots, int snapshot_every,
                 int num_snapshots, int num_seqs, int seq_len, int total_tokens, int num_heads,
                 int head_dim, int dtype, hipStream_t stream, unsigned *far_flags = nullptr) {
#define KDA_LAUNCH_ARGS                                                                        \
    q, k, v, log_alpha, beta, initial_state, cu_seqlens, out, final_state, snapshots,          \
        snapshot_every, num_snapshots, num_seqs, seq_len, total_tokens, num_heads, far_flags,  \
        stream
    if (dtype == kDtypeBf16)
        return head_dim == 128 ? launch<bf16, 128, 64, SG, MODE>(KDA_LAUNCH_ARGS)
                               : launch<bf16, 64, 64, SG, MODE>(KDA_LAUNCH_ARGS);
    if (head_dim == 128)  // fp32 operand sets at d = 128 exceed the LDS: the token recurrence
        return MODE == kModeStates
                   ? -1
                   : launch_chunk_seq(q, k, v, log_alpha, beta, initial_state, cu_seqlens, out,
                                      final_state, snapshots, snapshot_every, num_snapshots,
                                      num_seqs, seq_len, total_tokens, num_heads, SG ? 1 : 0,
                                      MODE, stream);
    return launch<float, 64, 16, SG, MODE>(KDA_LAUNCH_ARGS);
#undef KDA_LAUNCH_ARGS
}

}  // namespace

int chunk_fwd_slices(int head_dim, int dtype) {
    // bf16: 64 value columns per workgroup; fp32: 16 (d = 64), and at d = 128
    // the token recurrence's 64
    if (dtype == kDtypeBf16 || head_dim == 128) return head_dim / 64;
    return head_dim / 16;
}

int launch_chunk_states(const void *q, const void *k, const void *v, const float *log_alpha,
                        const float *beta, const float *initial_state,
                        const int32_t *cu_seqlens, float *states, int32_t num_seqs,
                        int32_t seq_len, int32_t total_tokens, int32_t num_heads, int head_dim,
                        int dtype, unsigned *far_flags, hipStream_t stream) {
    if (dtype != kDtypeBf16 && head_dim != 64) return -1;
    return launch_dtype<false, kModeStates>(q, k, v, log_alpha, beta, initial_state, cu_seqlens,
                                            nullptr, nullptr, states, kC, 0, num_seqs, seq_len,
                                            total_tokens, num_heads, head_dim, dtype, stream,
                                            far_flags);
}

int launch_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                     const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                     void *out, float *final_state, float *snapshots, int32_t snapshot_every,
                     int32_t num_snapshots, int32_t num_seqs, int32_t seq_len,
                     int32_t total_tokens, int32_t num_heads, int head_dim, int dtype,
                     int scalar_gate, int init_identity, hipStream_t stream) {
    if (!snapshots) snapshot_every = kC, num_snapshots = 0;
#define KDA_CHUNK_ARGS                                                                         \
    q, k, v, log_alpha, beta, initial_state, cu_seqlens, out, final_state, snapshots,          \
        snapshot_every, num_snapshots, num_seqs, seq_len, total_tokens, num_heads, head_dim,   \
        dtype, stream
    if (init_identity) {  // the transition map: no values, no outputs, no snapshots
        if (v || out || snapshots || initial_state || scalar_gate) return -1;
        return launch_dtype<false, kModeMap>(KDA_CHUNK_ARGS);
    }
    // without outputs (the state-only pass of the segmented prefill): the
    // channel-gate kernels only
    if (!out) return scalar_gate ? -1 : launch_dtype<false, kModeState>(KDA_CHUNK_ARGS);
    return scalar_gate ? launch_dtype<true, kModeOut>(KDA_CHUNK_ARGS)
                       : launch_dtype<false, kModeOut>(KDA_CHUNK_ARGS);
#undef KDA_CHUNK_ARGS
}

}  // namespace kda
