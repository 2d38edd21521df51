// kda_chunk.hip -- chunked KDA prefill: one persistent workgroup per
// (sequence, head, d_v slice) walks the sequence chunk by chunk.
//
// Pages cited (by title):
//   [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer.
//   [K3-memory]     "Kimi K3 Changed the Memory Math for Agentic AI Forever".
//
// The recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t ([K3-explainer] §四, §二.1) is evaluated per chunk of C = 64
// tokens: state recurrence between chunks, dense products inside a chunk
// ([K3-explainer] §六.1), with the chunk's rank-one erase/write products
// gathered into a few matrices ([K3-explainer] §六.2, WY representation).
// The concrete form used here (a UT-transform variant; the page gives only
// the idea) is, for a chunk with entering state S and per-channel cumulative
// log-decay Gamma_r = sum_{s<=r} log a_s (reset each chunk):
//
//   K+ = K (.) e^Gamma,  Q+ = Q (.) e^Gamma,  K- = K (.) e^-Gamma
//   A       = StrictTril(diag(b) K+ K-^T),  T = (I + A)^{-1}
//   X       = V - K+ S                        (prediction error against S)
//   Delta   = T diag(b) X                     (the chunk's corrected writes)
//   O       = Q+ S + Tril(Q+ K-^T) Delta
//   S_next  = Diag(e^{Gamma_last}) S + (K (.) e^{Gamma_last - Gamma})^T Delta
//
// The chunk transition S -> S_next is the page's "P = D - K W^T" form
// ([K3-explainer] §六.2) with D = Diag(e^{Gamma_last}).
//
// Range of the factors.  e^Gamma <= 1 but e^-Gamma grows with the decay
// accumulated inside the chunk.  A chunk whose |Gamma| (log2 units) reaches
// 120 anywhere is recomputed as four 16-token windows, each a chunk of its own
// (rows outside the window are zero); inside 16 tokens the factors stay in
// range as long as 16 consecutive log-gates sum to more than -80 per channel.
//
// Work split inside a workgroup (8 waves, 512 threads), per chunk:
//   prep   : cumulative log-decay per 16-token block (DPP lane scan) plus
//            block offsets, e^{+-Gamma} (v_exp_f32), operand tiles in LDS;
//   A, Mqk : 20 MFMA tiles of 16x16 (lower triangle only);
//   T      : diagonal 16x16 blocks by right-looking substitution on one wave
//            while waves 4-7 compute [K+; Q+] S; then the off-diagonal blocks
//            in three dependency levels (MFMA);
//   scan   : Delta = T' X, O = Q+ S + Mqk Delta, and S <- gamma S + Kend^T
//            Delta with the fp32 master state held in MFMA accumulators
//            across chunks; a bf16 (or fp32) shadow copy of S in LDS feeds the
//            next chunk's products.
// Inputs for chunk n+1 are loaded into registers while chunk n is computed.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kC = 64;              // chunk length
constexpr int kBS = 16;             // tile / sub-block size
constexpr int kNB = kC / kBS;       // sub-blocks per chunk
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr float kMaxLog2Decay = 120.f;  // |Gamma| bound of the single-pass chunk

// (I, J) of the lower-triangular 16x16 tiles, J <= I, row-major order.
__device__ __forceinline__ void tile_ij(int t, int &I, int &J) {
    I = (t >= 1) + (t >= 3) + (t >= 6);
    J = t - I * (I + 1) / 2;
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// K_end^T is stored [key channel][token] with the token index XOR-swizzled by
// a multiple of 16 per channel group: the prep's transposed stores (8 channel
// groups x 8 token pairs per wave) and the MFMA reads (16 channels x 4 runs of
// 8 tokens) then both spread over all 64 LDS banks.  Runs of 8 tokens stay
// contiguous and inside [0, 64).
__device__ __forceinline__ int kend_col(int c, int t) { return t ^ (8 * ((c >> 3) & 6)); }

template <typename T, int D, int DVS>
struct Cfg {
    static constexpr int SZ = (int)sizeof(T);
    static constexpr int kPad = 16 / SZ;
    static constexpr int LDK = D + kPad;     // [C][D] tiles
    static constexpr int LDC = kC + kPad;    // [*][C] tiles
    static constexpr int LDA = kC + 4;       // fp32 A
    static constexpr int LDAT = kBS + 4;     // fp32 transposed diagonal blocks of A
    static constexpr int LDV = DVS + kPad;   // V slice
    static constexpr int LDD = kBS + kPad;   // diagonal T blocks
    static constexpr int TDB = kBS * LDD + kPad;  // stride between diagonal blocks
    static constexpr int LDX = kBS + 4;      // fp32 scratch
    static constexpr int NCT = DVS / 16;     // d_v column tiles
    static constexpr int NRT = D / 16;       // d_k row tiles of the state
    static constexpr int RPT = D / 64;       // prep: rows per thread
    static constexpr int RGB = kBS / RPT;    // prep: row groups per 16-row block
    static constexpr int VTH = kC * DVS / 8; // threads that move the V and O slices

    static constexpr int TILE = kC * LDK * SZ;
    static constexpr int XB = DVS * LDC * SZ;       // X (and Delta) transposed
    static constexpr int SCRB = 3 * kBS * LDX * 4;  // fp32 T-level scratch
    static constexpr int LDO = DVS + kPad;          // O staging rows (padded)
    static constexpr int OB = kC * LDO * SZ;        // O staging
    static constexpr int RKM = cmax(TILE, XB + cmax(SCRB, OB));
    static constexpr int AB = kC * LDA * 4;

    // byte offsets; K- region later holds X, scratch and O, the A region Delta
    static constexpr int oKP = 0, oQP = TILE, oKM = 2 * TILE;
    static constexpr int oX = oKM, oScr = oKM + XB, oO = oKM + XB;
    static constexpr int oA = oKM + RKM, oDL = oA;
    static constexpr int oAt = oA + AB;
    static constexpr int oKendT = oAt + kNB * kBS * LDAT * 4;
    static constexpr int oMqk = oKendT + D * LDC * SZ;
    static constexpr int oTr = oMqk + kC * LDC * SZ;
    static constexpr int oTt = oTr + kC * LDC * SZ;
    static constexpr int oTd = oTt + kC * LDC * SZ;
    static constexpr int oS = oTd + kNB * TDB * SZ;
    static constexpr int oV = oS + DVS * LDK * SZ;
    static constexpr int oBeta = oV + kC * LDV * SZ;
    static constexpr int oTot = oBeta + kC * 4;
    static constexpr int oGam = oTot + kNB * D * 4;
    static constexpr int oFlag = oGam + D * 4;
    static constexpr int BYTES = oFlag + kWaves * 4;

    static_assert(D == 64 || D == 128, "head dim");
    static_assert(DVS % 16 == 0 && D % DVS == 0, "d_v slice");
    static_assert(VTH <= kThreads && VTH >= kC, "V slice map");
    static_assert(2 * (64 / RGB) * 8 == D, "prep: two waves cover the channels of a block");
    static_assert(XB <= AB, "Delta fits in the A region");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(TILE % 16 == 0 && RKM % 16 == 0 && XB % 16 == 0 && oS % 16 == 0 &&
                      oV % 16 == 0 && oTd % 16 == 0 && oMqk % 16 == 0 && oKendT % 16 == 0,
                  "16-byte alignment");
};

// Registers holding one chunk's raw inputs (loaded one chunk ahead).
template <typename T, int D, int DVS>
struct ChunkRegs {
    typedef Cfg<T, D, DVS> G;
    typename Vec8<T>::raw k[G::RPT], q[G::RPT];
    f32x4 g[G::RPT][2];
    typename Vec8<T>::raw v;
    float beta;
};

// Buffer descriptors for one chunk: the base points at the chunk's first
// token and the size covers exactly its nvalid tokens, so every load of a row
// at or beyond nvalid returns zeros (an inert token) without a branch.
struct ChunkSrc {
    __amdgpu_buffer_rsrc_t k, q, g, v, b;
};

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

template <typename T>
__device__ __forceinline__ ChunkSrc chunk_src(const T *q, const T *k, const T *v,
                                              const float *log_alpha, const float *beta,
                                              int64_t tok0, int nvalid, int H, int D) {
    const int64_t e0 = tok0 * H * D;
    const int bytes = nvalid * H * D;  // elements; callers keep H * D * 64 * 4 < 2^31
    ChunkSrc s;
    s.k = __builtin_amdgcn_make_buffer_rsrc((void *)(k + e0), 0, bytes * (int)sizeof(T), kRsrcWord3);
    s.q = __builtin_amdgcn_make_buffer_rsrc((void *)(q + e0), 0, bytes * (int)sizeof(T), kRsrcWord3);
    s.v = __builtin_amdgcn_make_buffer_rsrc((void *)(v + e0), 0, bytes * (int)sizeof(T), kRsrcWord3);
    s.g = __builtin_amdgcn_make_buffer_rsrc((void *)(log_alpha + e0), 0, bytes * 4, kRsrcWord3);
    s.b = __builtin_amdgcn_make_buffer_rsrc((void *)(beta + tok0 * H), 0, nvalid * H * 4,
                                            kRsrcWord3);
    return s;
}

template <typename T> __device__ __forceinline__ typename Vec8<T>::raw buf8(__amdgpu_buffer_rsrc_t r, int off);
template <> __device__ __forceinline__ u32x4 buf8<bf16>(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
template <> __device__ __forceinline__ f32x8 buf8<float>(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
    return f32x8{__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]),
                 __uint_as_float(a[3]), __uint_as_float(b[0]), __uint_as_float(b[1]),
                 __uint_as_float(b[2]), __uint_as_float(b[3])};
}
__device__ __forceinline__ f32x4 buf4f(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return f32x4{__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]),
                 __uint_as_float(a[3])};
}

// Byte offsets (relative to a chunk's first token) of this thread's loads;
// loop-invariant, so the chunk loop only rebuilds the scalar descriptors.
template <typename T, int D, int DVS>
struct ChunkOffsets {
    typedef Cfg<T, D, DVS> G;
    int kq[G::RPT], g[G::RPT], v, b;
    __device__ ChunkOffsets(int tid, int h, int H, int v0) {
        const int lane = tid & 63, wave = tid >> 6;
        const int I = wave >> 1, cb = (wave & 1) * (D / 2);
        const int rg = lane % G::RGB, cg = lane / G::RGB;
        const int c0 = cb + 8 * cg;
#pragma unroll
        for (int j = 0; j < G::RPT; ++j) {
            const int r = kBS * I + G::RPT * rg + j;
            kq[j] = ((r * H + h) * D + c0) * (int)sizeof(T);
            g[j] = ((r * H + h) * D + c0) * 4;
        }
        const int vr = tid / (DVS / 8), vc = 8 * (tid % (DVS / 8));
        v = ((vr * H + h) * D + v0 + vc) * (int)sizeof(T);
        b = (tid * H + h) * 4;
    }
};

// The next chunk's registers are loaded in three parts, issued in different
// phases so the vector memory unit drains them in the background.
template <typename T, int D, int DVS>
__device__ __forceinline__ void load_kq(ChunkRegs<T, D, DVS> &R, const ChunkSrc &s,
                                        const ChunkOffsets<T, D, DVS> &o) {
#pragma unroll
    for (int j = 0; j < Cfg<T, D, DVS>::RPT; ++j) {
        R.k[j] = buf8<T>(s.k, o.kq[j]);
        R.q[j] = buf8<T>(s.q, o.kq[j]);
    }
}
template <typename T, int D, int DVS>
__device__ __forceinline__ void load_g(ChunkRegs<T, D, DVS> &R, const ChunkSrc &s,
                                       const ChunkOffsets<T, D, DVS> &o) {
#pragma unroll
    for (int j = 0; j < Cfg<T, D, DVS>::RPT; ++j) {
        R.g[j][0] = buf4f(s.g, o.g[j]);
        R.g[j][1] = buf4f(s.g, o.g[j] + 16);
    }
}
template <typename T, int D, int DVS>
__device__ __forceinline__ void load_vb(ChunkRegs<T, D, DVS> &R, const ChunkSrc &s,
                                        const ChunkOffsets<T, D, DVS> &o, int tid) {
    R.v = tid < Cfg<T, D, DVS>::VTH ? buf8<T>(s.v, o.v) : Vec8<T>::zero();
    R.beta = tid < kC ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(s.b, o.b, 0, 0)) : 0.f;
}

template <typename T, int D, int DVS>
__global__ __launch_bounds__(kThreads) void chunk_fwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ initial_state, const int32_t *__restrict__ cu_seqlens,
    T *__restrict__ out, float *__restrict__ final_state, int num_seqs, int seq_len,
    int total_tokens, int H, int units, int units_per_xcd) {
    typedef Cfg<T, D, DVS> G;
    typedef Mma<T> M;
    constexpr int KS = M::KSTEP;
    constexpr int NS = D / DVS;

    __shared__ __attribute__((aligned(16))) unsigned char smem[G::BYTES];
    T *sKP = reinterpret_cast<T *>(smem + G::oKP);
    T *sQP = reinterpret_cast<T *>(smem + G::oQP);
    T *sKM = reinterpret_cast<T *>(smem + G::oKM);
    T *sX = reinterpret_cast<T *>(smem + G::oX);
    float *sScr = reinterpret_cast<float *>(smem + G::oScr);
    T *sO = reinterpret_cast<T *>(smem + G::oO);
    float *sA = reinterpret_cast<float *>(smem + G::oA);
    T *sDL = reinterpret_cast<T *>(smem + G::oDL);
    float *sAt = reinterpret_cast<float *>(smem + G::oAt);
    T *sKendT = reinterpret_cast<T *>(smem + G::oKendT);
    T *sMqk = reinterpret_cast<T *>(smem + G::oMqk);
    T *sTr = reinterpret_cast<T *>(smem + G::oTr);
    T *sTt = reinterpret_cast<T *>(smem + G::oTt);
    T *sTd = reinterpret_cast<T *>(smem + G::oTd);
    T *sS = reinterpret_cast<T *>(smem + G::oS);
    T *sV = reinterpret_cast<T *>(smem + G::oV);
    float *sBeta = reinterpret_cast<float *>(smem + G::oBeta);
    float *sTot = reinterpret_cast<float *>(smem + G::oTot);
    float *sGam = reinterpret_cast<float *>(smem + G::oGam);
    int *sFlag = reinterpret_cast<int *>(smem + G::oFlag);

    // XCD-aware unit order: workgroups are dealt to the 8 XCDs round-robin,
    // so give each XCD a contiguous run of units; the NS slices of one
    // (sequence, head) then share that XCD's L2 for their common inputs.
    const int bid = blockIdx.x;
    const int unit = (bid & 7) * units_per_xcd + (bid >> 3);
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

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, l4 = lane >> 4;

    // Upper off-diagonal blocks of Mqk and T' are never written: zero once.
    for (int i = tid; i < kC * kC; i += kThreads) {
        const int r = i / kC, c = i % kC;
        if (c / kBS > r / kBS) {
            sMqk[r * G::LDC + c] = from_f32<T>(0.f);
            sTr[r * G::LDC + c] = from_f32<T>(0.f);
        }
    }

    // fp32 master state: wave w owns state rows (key channels) 16w..16w+15
    // for all DVS value columns, in MFMA accumulator layout.
    const bool owns_state = wave < G::NRT;
    const int64_t sbase = ((int64_t)n * H + h) * D * D;  // M = S^T: [d_v][d_k]
    f32x4 Sm[G::NCT];
#pragma unroll
    for (int ct = 0; ct < G::NCT; ++ct) {
        Sm[ct] = zero4();
        if (owns_state && initial_state)
            Sm[ct] = *reinterpret_cast<const f32x4 *>(
                initial_state + sbase + (int64_t)(v0 + 16 * ct + l16) * D + 16 * wave + 4 * l4);
        if (owns_state)
            store4(sS + (16 * ct + l16) * G::LDK + 16 * wave + 4 * l4, Sm[ct][0], Sm[ct][1],
                   Sm[ct][2], Sm[ct][3]);
    }

    // prep thread map: block I = wave / 2, channels c0..c0+7, rows r_j.
    const int pI = wave >> 1;
    const int prg = lane % G::RGB, pcg = lane / G::RGB;
    const int pc0 = (wave & 1) * (D / 2) + 8 * pcg;

    const ChunkOffsets<T, D, DVS> offs(tid, h, H, v0);
    ChunkRegs<T, D, DVS> R;
    if (nchunks > 0) {
        const ChunkSrc s0 = chunk_src(q, k, v, log_alpha, beta, tbeg,
                                      (int)((tend - tbeg) < kC ? (tend - tbeg) : kC), H, D);
        load_kq(R, s0, offs);
        load_g(R, s0, offs);
        load_vb(R, s0, offs, tid);
    }

    for (int ch = 0; ch < nchunks; ++ch) {
        const int64_t tok0 = tbeg + (int64_t)ch * kC;
        const int nvalid = (int)((tend - tok0) < kC ? (tend - tok0) : kC);
        const int64_t ntok0 = tok0 + kC;
        const int nnext = ch + 1 < nchunks ? (int)((tend - ntok0) < kC ? (tend - ntok0) : kC) : 0;
        const ChunkSrc nsrc = chunk_src(q, k, v, log_alpha, beta, ntok0, nnext, H, D);

        int npass = 1;  // 4 when the chunk is redone as 16-token windows
        for (int pass = 0; pass < npass; ++pass) {
            // A windowed pass keeps the rows of one 16-token block; the rows of
            // a thread all lie in block pI, so masking is per thread.
            const int lo = npass == 1 ? 0 : kBS * pass;
            const int hi = npass == 1 ? kC : lo + kBS;
            const bool keep = npass == 1 || pI == pass;

            // -------------------------------------------------------- prep
            float P[G::RPT][8];
            {
                float gl[G::RPT][8];
#pragma unroll
                for (int j = 0; j < G::RPT; ++j) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        gl[j][e] = keep ? R.g[j][0][e] * kLog2e : 0.f;
                        gl[j][4 + e] = keep ? R.g[j][1][e] * kLog2e : 0.f;
                    }
                }
                // inclusive prefix over this thread's rows, then over the lanes
                // of the 16-row block (consecutive lanes of one DPP row).
                float btot[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float run = 0.f;
#pragma unroll
                    for (int j = 0; j < G::RPT; ++j) {
                        run += gl[j][e];
                        P[j][e] = run;
                    }
                    float x = run;
                    float y = dpp_row_shr<1>(x);
                    if (prg >= 1) x += y;
                    y = dpp_row_shr<2>(x);
                    if (prg >= 2) x += y;
                    y = dpp_row_shr<4>(x);
                    if (prg >= 4) x += y;
                    if (G::RGB == 16) {
                        y = dpp_row_shr<8>(x);
                        if (prg >= 8) x += y;
                    }
                    const float excl = x - run;
#pragma unroll
                    for (int j = 0; j < G::RPT; ++j) P[j][e] += excl;
                    btot[e] = __shfl(x, lane | (G::RGB - 1), 64);
                }
                if (prg == G::RGB - 1) {
                    store4(sTot + pI * D + pc0, btot[0], btot[1], btot[2], btot[3]);
                    store4(sTot + pI * D + pc0 + 4, btot[4], btot[5], btot[6], btot[7]);
                }
            }
            float vf[8];
            Vec8<T>::to_float(R.v, vf);
            {
                const int vr = tid / (DVS / 8);
                if (vr < lo || vr >= hi) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) vf[e] = 0.f;
                }
            }
            const float beta_r = (tid >= lo && tid < hi) ? R.beta : 0.f;
            __syncthreads();

            {
                float Gb[8], Gend[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    Gb[e] = 0.f;
                    Gend[e] = 0.f;
                }
#pragma unroll
                for (int J = 0; J < kNB; ++J) {
                    const f32x4 t0 = *reinterpret_cast<const f32x4 *>(sTot + J * D + pc0);
                    const f32x4 t1 = *reinterpret_cast<const f32x4 *>(sTot + J * D + pc0 + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (J < pI) {
                            Gb[e] += t0[e];
                            Gb[4 + e] += t1[e];
                        }
                        Gend[e] += t0[e];
                        Gend[4 + e] += t1[e];
                    }
                }
                float fend[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) fend[e] = fast_exp2(Gend[e]);
                float mx = 0.f;
                float ke[G::RPT][8];
#pragma unroll
                for (int j = 0; j < G::RPT; ++j) {
                    float kf[8], qf[8], kp[8], qp[8], km[8];
                    Vec8<T>::to_float(R.k[j], kf);
                    Vec8<T>::to_float(R.q[j], qf);
                    if (!keep) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            kf[e] = 0.f;
                            qf[e] = 0.f;
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float gam = Gb[e] + P[j][e];
                        mx = fmaxf(mx, fabsf(gam));
                        const float ep = fast_exp2(gam);
                        const float em = fast_exp2(-gam);
                        kp[e] = kf[e] * ep;
                        qp[e] = qf[e] * ep;
                        km[e] = kf[e] * em;
                        ke[j][e] = km[e] * fend[e];
                    }
                    const int r = kBS * pI + G::RPT * prg + j;
                    store8(sKP + r * G::LDK + pc0, kp);
                    store8(sQP + r * G::LDK + pc0, qp);
                    store8(sKM + r * G::LDK + pc0, km);
                }
                // NaN compares false: a non-finite gate also takes the windowed path
                const bool bad = !(mx < kMaxLog2Decay);
                const unsigned long long any = __ballot(bad);
                if (lane == 0) sFlag[wave] = any != 0ull;
                // K_end^T: key-channel rows, token columns (RPT consecutive tokens)
                const int r0 = kBS * pI + G::RPT * prg;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if constexpr (G::RPT == 2) {
                        store2(sKendT + (pc0 + e) * G::LDC + kend_col(pc0 + e, r0), ke[0][e],
                               ke[1][e]);
                    } else {
                        sKendT[(pc0 + e) * G::LDC + kend_col(pc0 + e, r0)] =
                            from_f32<T>(ke[0][e]);
                    }
                }
                if (tid < D) {
                    // gamma = e^{Gamma_last} for key channel tid
                    float s = 0.f;
#pragma unroll
                    for (int J = 0; J < kNB; ++J) s += sTot[J * D + tid];
                    sGam[tid] = fast_exp2(s);
                }
            }
            if (tid < G::VTH) {
                const int vr = tid / (DVS / 8), vc = 8 * (tid % (DVS / 8));
                store8(sV + vr * G::LDV + vc, vf);
            }
            if (tid < kC) sBeta[tid] = beta_r;
            __syncthreads();

            {
                bool unsafe = false;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) unsafe |= sFlag[w] != 0;
                if (npass == 1 && unsafe) {
                    npass = kNB;  // redo this chunk as four 16-token windows
                    pass = -1;
                    continue;
                }
            }
            // Prefetch the next chunk's inputs once this chunk's last pass has
            // consumed the registers; they arrive while the chunk is computed.
            const bool prefetch = pass == npass - 1 && nnext > 0;
            if (prefetch) load_kq(R, nsrc, offs);

            // -------------------------------------------------------- A, Mqk
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                const int t = wave + kWaves * s;
                if (t >= 20) continue;
                const bool isA = t < 10;
                int I, J;
                tile_ij(isA ? t : t - 10, I, J);
                const T *left = (isA ? sKP : sQP) + kBS * I * G::LDK;
                const T *right = sKM + kBS * J * G::LDK;
                f32x4 acc = tile_mma<T, D>(zero4(), left, G::LDK, right, G::LDK, lane);
                if (isA) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * l4 + e;
                        float val = acc[e] * sBeta[kBS * I + r];
                        if (I == J && l16 >= r) val = 0.f;
                        acc[e] = val;
                        sA[(kBS * I + r) * G::LDA + kBS * J + l16] = val;
                    }
                    if (I == J)  // transposed copy of the diagonal block
                        store4(sAt + (I * kBS + l16) * G::LDAT + 4 * l4, acc[0], acc[1], acc[2],
                               acc[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * l4 + e;
                        const float val = (I == J && l16 > r) ? 0.f : acc[e];
                        sMqk[(kBS * I + r) * G::LDC + kBS * J + l16] = from_f32<T>(val);
                    }
                }
            }
            __syncthreads();

            if (prefetch) load_g(R, nsrc, offs);

            // ------------------------------------- T diagonal || [K+; Q+] S
            f32x4 PQ[G::NCT];
#pragma unroll
            for (int ct = 0; ct < G::NCT; ++ct) PQ[ct] = zero4();
            if (wave == 0) {
                // lane 16*I + j: column j of (I + A_II)^{-1}, right-looking
                const int I = l4, j = l16;
                const float *At = sAt + I * kBS * G::LDAT;
                float s[kBS];
#pragma unroll
                for (int r = 0; r < kBS; ++r) s[r] = (r == j) ? 1.f : 0.f;
                // column i of A_II (all 16 lanes of a group read the same row
                // of the transposed block: an LDS broadcast); one column of
                // lookahead, no more, to bound register use.
                f32x4 cur[kBS / 4], nxt[kBS / 4];
#pragma unroll
                for (int c4 = 0; c4 < kBS / 4; ++c4)
                    cur[c4] = *reinterpret_cast<const f32x4 *>(At + 4 * c4);
#pragma unroll
                for (int i = 0; i < kBS - 1; ++i) {
                    if (i + 1 < kBS - 1) {
#pragma unroll
                        for (int c4 = 0; c4 < kBS / 4; ++c4)
                            nxt[c4] = *reinterpret_cast<const f32x4 *>(At + (i + 1) * G::LDAT +
                                                                       4 * c4);
                    }
                    const float xi = s[i];
#pragma unroll
                    for (int r = i + 1; r < kBS; ++r) s[r] -= cur[r >> 2][r & 3] * xi;
#pragma unroll
                    for (int c4 = 0; c4 < kBS / 4; ++c4) cur[c4] = nxt[c4];
                    __builtin_amdgcn_sched_barrier(0);
                }
                const float bj = sBeta[kBS * I + j];
#pragma unroll
                for (int r = 0; r < kBS; ++r) {
                    sTd[I * G::TDB + r * G::LDD + j] = from_f32<T>(s[r]);
                    sTr[(kBS * I + r) * G::LDC + kBS * I + j] = from_f32<T>(s[r] * bj);
                }
#pragma unroll
                for (int r = 0; r < kBS; r += 4)
                    store4(sTt + (kBS * I + j) * G::LDC + kBS * I + r, s[r], s[r + 1], s[r + 2],
                           s[r + 3]);
            } else if (wave >= 4) {
                // rows 16i..16i+15 of K+ S (-> X = V - K+ S) and of Q+ S
                const int i = wave - 4;
                f32x4 PK[G::NCT];
#pragma unroll
                for (int ct = 0; ct < G::NCT; ++ct) PK[ct] = zero4();
#pragma unroll
                for (int kk = 0; kk < D; kk += KS) {
                    const typename M::Frag ak = M::load(sKP + kBS * i * G::LDK + kk, G::LDK, lane);
                    const typename M::Frag aq = M::load(sQP + kBS * i * G::LDK + kk, G::LDK, lane);
#pragma unroll
                    for (int ct = 0; ct < G::NCT; ++ct) {
                        const typename M::Frag b =
                            M::load(sS + 16 * ct * G::LDK + kk, G::LDK, lane);
                        PK[ct] = M::mma(ak, b, PK[ct]);
                        PQ[ct] = M::mma(aq, b, PQ[ct]);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < G::NCT; ++ct) {
                    float x[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = kBS * i + 4 * l4 + e;
                        x[e] = to_f32(sV[r * G::LDV + 16 * ct + l16]) - PK[ct][e];
                    }
                    store4(sX + (16 * ct + l16) * G::LDC + kBS * i + 4 * l4, x[0], x[1], x[2],
                           x[3]);
                }
            }
            __syncthreads();

            if (prefetch) load_vb(R, nsrc, offs, tid);

            // Off-diagonal blocks: T_IJ = -T_II sum_{J<=K<I} A_IK T_KJ, level by level.
#pragma unroll
            for (int lvl = 1; lvl < kNB; ++lvl) {
                if (wave < kNB - lvl) {
                    const int J = wave, I = wave + lvl;
                    f32x4 acc = zero4();
                    f32x4 Y = zero4();
                    if constexpr (sizeof(T) == 2) {
                        for (int K = J; K < I; ++K) {
                            const f32x4 a4 = *reinterpret_cast<const f32x4 *>(
                                sA + (kBS * I + l16) * G::LDA + kBS * K + 4 * l4);
                            bf16x4 ab;
                            ab[0] = static_cast<bf16>(a4[0]);
                            ab[1] = static_cast<bf16>(a4[1]);
                            ab[2] = static_cast<bf16>(a4[2]);
                            ab[3] = static_cast<bf16>(a4[3]);
                            const bf16x4 bb = *reinterpret_cast<const bf16x4 *>(
                                sTt + (kBS * J + l16) * G::LDC + kBS * K + 4 * l4);
                            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                                __builtin_bit_cast(i16x4, ab), __builtin_bit_cast(i16x4, bb), acc,
                                0, 0, 0);
                        }
                        const bf16x4 ta = *reinterpret_cast<const bf16x4 *>(
                            sTd + I * G::TDB + l16 * G::LDD + 4 * l4);
                        bf16x4 xb;
                        xb[0] = static_cast<bf16>(-acc[0]);
                        xb[1] = static_cast<bf16>(-acc[1]);
                        xb[2] = static_cast<bf16>(-acc[2]);
                        xb[3] = static_cast<bf16>(-acc[3]);
                        Y = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                            __builtin_bit_cast(i16x4, ta), __builtin_bit_cast(i16x4, xb), Y, 0, 0,
                            0);
                    } else {
                        for (int K = J; K < I; ++K) {
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const float a =
                                    sA[(kBS * I + l16) * G::LDA + kBS * K + 4 * s + l4];
                                const float b = to_f32(
                                    sTt[(kBS * J + l16) * G::LDC + kBS * K + 4 * s + l4]);
                                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
                            }
                        }
                        float *scr = sScr + wave * kBS * G::LDX;
                        store4(scr + l16 * G::LDX + 4 * l4, -acc[0], -acc[1], -acc[2], -acc[3]);
                        wave_lds_fence();
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const float a = to_f32(sTd[I * G::TDB + l16 * G::LDD + 4 * s + l4]);
                            const float b = scr[l16 * G::LDX + 4 * s + l4];
                            Y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, Y, 0, 0, 0);
                        }
                    }
                    // lane holds T_IJ[4*l4 + e][l16]
                    store4(sTt + (kBS * J + l16) * G::LDC + kBS * I + 4 * l4, Y[0], Y[1], Y[2],
                           Y[3]);
                    const float bj = sBeta[kBS * J + l16];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sTr[(kBS * I + 4 * l4 + e) * G::LDC + kBS * J + l16] =
                            from_f32<T>(Y[e] * bj);
                }
                __syncthreads();
            }

            // ------------------------------------------------------- scan
            // Delta = T' X (waves 0-3, lower-triangular k range), stored transposed.
            if (wave < 4) {
                const int rt = wave;
                const int nks = (kBS * (rt + 1) + KS - 1) / KS;
                f32x4 acc[G::NCT];
#pragma unroll
                for (int ct = 0; ct < G::NCT; ++ct) acc[ct] = zero4();
#pragma unroll
                for (int ks = 0; ks < kC / KS; ++ks) {
                    if (ks < nks) {
                        const typename M::Frag a =
                            M::load(sTr + kBS * rt * G::LDC + ks * KS, G::LDC, lane);
#pragma unroll
                        for (int ct = 0; ct < G::NCT; ++ct)
                            acc[ct] = M::mma(
                                a, M::load(sX + 16 * ct * G::LDC + ks * KS, G::LDC, lane),
                                acc[ct]);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < G::NCT; ++ct)
                    store4(sDL + (16 * ct + l16) * G::LDC + kBS * rt + 4 * l4, acc[ct][0],
                           acc[ct][1], acc[ct][2], acc[ct][3]);
            }
            __syncthreads();

            // O = Q+ S + Mqk Delta (waves 4-7), staged for a coalesced store.
            if (wave >= 4) {
                const int rt = wave - 4;
                const int nks = (kBS * (rt + 1) + KS - 1) / KS;
#pragma unroll
                for (int ks = 0; ks < kC / KS; ++ks) {
                    if (ks < nks) {
                        const typename M::Frag a =
                            M::load(sMqk + kBS * rt * G::LDC + ks * KS, G::LDC, lane);
#pragma unroll
                        for (int ct = 0; ct < G::NCT; ++ct)
                            PQ[ct] = M::mma(
                                a, M::load(sDL + 16 * ct * G::LDC + ks * KS, G::LDC, lane),
                                PQ[ct]);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < G::NCT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sO[(kBS * rt + 4 * l4 + e) * G::LDO + 16 * ct + l16] =
                            from_f32<T>(PQ[ct][e]);
            }
            // S <- Diag(gamma) S + Kend^T Delta on the owning waves.
            if (owns_state) {
                float gm[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) gm[e] = sGam[16 * wave + 4 * l4 + e];
#pragma unroll
                for (int ct = 0; ct < G::NCT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) Sm[ct][e] *= gm[e];
#pragma unroll
                for (int kk = 0; kk < kC; kk += KS) {
                    const int c = 16 * wave + l16;
                    const int t0 = kk + (KS == 32 ? 8 * l4 : l4);
                    const typename M::Frag a = *reinterpret_cast<const typename M::Frag *>(
                        sKendT + c * G::LDC + kend_col(c, t0));
#pragma unroll
                    for (int ct = 0; ct < G::NCT; ++ct)
                        Sm[ct] = M::mma(a, M::load(sDL + 16 * ct * G::LDC + kk, G::LDC, lane),
                                        Sm[ct]);
                }
#pragma unroll
                for (int ct = 0; ct < G::NCT; ++ct)
                    store4(sS + (16 * ct + l16) * G::LDK + 16 * wave + 4 * l4, Sm[ct][0],
                           Sm[ct][1], Sm[ct][2], Sm[ct][3]);
            }
            __syncthreads();

            // Output rows of this pass.
            if (tid < G::VTH) {
                const int orow = tid / (DVS / 8), ocol = 8 * (tid % (DVS / 8));
                if (orow >= lo && orow < hi && orow < nvalid) {
                    float of[8];
                    Vec8<T>::to_float(load8(sO + orow * G::LDO + ocol), of);
                    store8(out + ((tok0 + orow) * H + h) * (int64_t)D + v0 + ocol, of);
                }
            }
        }
    }

    if (final_state && owns_state) {
#pragma unroll
        for (int ct = 0; ct < G::NCT; ++ct)
            *reinterpret_cast<f32x4 *>(final_state + sbase + (int64_t)(v0 + 16 * ct + l16) * D +
                                       16 * wave + 4 * l4) = Sm[ct];
    }
}

template <typename T, int D, int DVS>
int launch(const void *q, const void *k, const void *v, const float *log_alpha, const float *beta,
           const float *initial_state, const int32_t *cu_seqlens, void *out, float *final_state,
           int num_seqs, int seq_len, int total_tokens, int H, hipStream_t stream) {
    const int64_t units64 = (int64_t)num_seqs * H * (D / DVS);
    if (units64 == 0) return 0;
    if (units64 > (int64_t)1 << 30) return -1;
    const int units = (int)units64;
    const int per_xcd = (units + 7) / 8;
    hipLaunchKernelGGL((chunk_fwd_kernel<T, D, DVS>), dim3(8 * per_xcd), dim3(kThreads), 0,
                       stream, static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), log_alpha, beta, initial_state, cu_seqlens,
                       static_cast<T *>(out), final_state, num_seqs, seq_len, total_tokens, H,
                       units, per_xcd);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                     const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                     void *out, float *final_state, int32_t num_seqs, int32_t seq_len,
                     int32_t total_tokens, int32_t num_heads, int head_dim, int dtype,
                     hipStream_t stream) {
    if (dtype == kDtypeBf16) {
        if (head_dim == 128)
            return launch<bf16, 128, 64>(q, k, v, log_alpha, beta, initial_state, cu_seqlens, out,
                                         final_state, num_seqs, seq_len, total_tokens, num_heads,
                                         stream);
        return launch<bf16, 64, 64>(q, k, v, log_alpha, beta, initial_state, cu_seqlens, out,
                                    final_state, num_seqs, seq_len, total_tokens, num_heads,
                                    stream);
    }
    return launch<float, 64, 16>(q, k, v, log_alpha, beta, initial_state, cu_seqlens, out,
                                 final_state, num_seqs, seq_len, total_tokens, num_heads, stream);
}

}  // namespace kda
