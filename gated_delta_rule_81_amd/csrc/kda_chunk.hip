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
//   A[r,i]  = b_r sum_c k_r[c] k_i[c] exp(Gamma_r[c] - Gamma_i[c])   (i < r)
//   T       = (I + A)^{-1}                       (unit lower triangular)
//   X       = V - (K (.) e^Gamma) S              (prediction error vs. S)
//   Delta   = T diag(b) X                        (the chunk's corrected writes)
//   O       = (Q (.) e^Gamma) S + Mqk Delta,  Mqk[r,i] = sum_c q_r k_i e^{G_r-G_i} (i <= r)
//   S_next  = Diag(e^{Gamma_last}) S + (K (.) e^{Gamma_last - Gamma})^T Delta
//
// The chunk transition S -> S_next is the page's "P = D - K W^T" form
// ([K3-explainer] §六.2) with D = Diag(e^{Gamma_last}).
//
// Overflow control.  exp(Gamma_r - Gamma_i) is split into a left factor
// (<= 1) and a right factor around a reference at the start of each 16-token
// block: left = exp(Gamma_r - Gamma_{b-1}) for r in block I (b = 16 I);
// right = exp(Gamma_{b-1} - Gamma_i) for i in block I (>= 1, bounded by 15
// tokens of decay).  Off-diagonal blocks (J < I) rescale the left factor by
// exp(Gamma_{16I-1} - Gamma_{16J-1}) <= 1.  Every factor stays in fp32 range
// as long as 15 consecutive gates sum to more than -87 per channel.
//
// Work split inside a workgroup (8 waves, 512 threads), per chunk:
//   prep   : cumulative log-decay per 16-token block (DPP lane scan), the
//            decay factors (v_exp_f32), and the scaled bf16/fp32 operand
//            tiles in LDS;
//   A, Mqk : 20 MFMA tiles of 16x16 (lower triangle only);
//   T      : 16x16 diagonal blocks by forward substitution (one wave), then
//            off-diagonal blocks in three dependency levels (MFMA);
//   scan   : [K+; Q+] S (MFMA), X, Delta = T' X, O, and the state update
//            S <- gamma S + Kend^T Delta with the fp32 master state held in
//            MFMA accumulators across chunks; a bf16 (or fp32) shadow copy of
//            S in LDS feeds the next chunk's products.
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

// (I, J) of the lower-triangular 16x16 tiles, J <= I, row-major order.
__device__ __forceinline__ void tile_ij(int t, int &I, int &J) {
    I = (t >= 1) + (t >= 3) + (t >= 6);
    J = t - I * (I + 1) / 2;
}
// Index of the off-diagonal pair (I, J), J < I, in 0..5.
__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

template <typename T, int D, int DVS>
struct Cfg {
    static constexpr int kPad = 16 / (int)sizeof(T);
    static constexpr int LDK = D + kPad;     // [C][D] tiles
    static constexpr int LDC = kC + kPad;    // [*][C] tiles
    static constexpr int LDA = kC + 4;       // fp32 A
    static constexpr int LDV = DVS + kPad;   // V slice
    static constexpr int LDD = kBS + kPad;   // diagonal T blocks
    static constexpr int LDX = kBS + 4;      // fp32 scratch
    static constexpr int NCT = DVS / 16;     // d_v column tiles
    static constexpr int NRT = D / 16;       // d_k row tiles of the state
    static constexpr int RPT = D / 64;       // prep: rows per thread
    static constexpr int RGB = kBS / RPT;    // prep: row groups per 16-row block
    static constexpr int VTH = kC * DVS / 8; // threads that load the V slice

    static constexpr int TILE = kC * LDK * (int)sizeof(T);
    static constexpr int R1 = 3 * TILE > 2 * TILE + kC * LDA * 4 ? 3 * TILE
                                                                 : 2 * TILE + kC * LDA * 4;
    // byte offsets
    static constexpr int oKL = 0, oQL = TILE, oKE = 2 * TILE;   // prep -> A/Mqk
    static constexpr int oKP = 0, oQP = TILE, oA = 2 * TILE;    // -> T, scan
    static constexpr int oX = oA, oDL = oKP, oO = oQP;          // scan
    static constexpr int oKendT = R1;
    static constexpr int oMqk = oKendT + D * LDC * (int)sizeof(T);
    static constexpr int oTr = oMqk + kC * LDC * (int)sizeof(T);
    static constexpr int oTt = oTr + kC * LDC * (int)sizeof(T);
    static constexpr int oTd = oTt + kC * LDC * (int)sizeof(T);
    static constexpr int oScr = oTd + kNB * kBS * LDD * (int)sizeof(T);
    static constexpr int oS = oScr + 3 * kBS * LDX * 4;
    static constexpr int oV = oS + DVS * LDK * (int)sizeof(T);
    static constexpr int oBeta = oV + kC * LDV * (int)sizeof(T);
    static constexpr int oTot = oBeta + kC * 4;
    static constexpr int oDp = oTot + kNB * D * 4;
    static constexpr int oGam = oDp + 6 * D * 4;
    static constexpr int BYTES = oGam + D * 4;

    static_assert(D == 64 || D == 128, "head dim");
    static_assert(DVS % 16 == 0 && D % DVS == 0, "d_v slice");
    static_assert(VTH <= kThreads, "V slice load");
    static_assert(2 * (64 / RGB) * 8 == D, "prep: two waves cover the channels of a block");
    static_assert(DVS * LDC * (int)sizeof(T) <= kC * LDA * 4, "X fits in the A area");
    static_assert(kC * DVS * (int)sizeof(T) <= TILE, "O staging fits in a tile");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(oS % 16 == 0 && oV % 16 == 0 && oTd % 16 == 0 && oMqk % 16 == 0, "align");
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

template <typename T, int D, int DVS>
__device__ __forceinline__ void load_chunk(ChunkRegs<T, D, DVS> &R, const T *__restrict__ q,
                                           const T *__restrict__ k, const T *__restrict__ v,
                                           const float *__restrict__ log_alpha,
                                           const float *__restrict__ beta, int64_t tok0,
                                           int nvalid, int h, int H, int v0, int tid) {
    typedef Cfg<T, D, DVS> G;
    const int lane = tid & 63, wave = tid >> 6;
    const int I = wave >> 1, cb = (wave & 1) * (D / 2);
    const int rg = lane % G::RGB, cg = lane / G::RGB;
    const int c0 = cb + 8 * cg;
#pragma unroll
    for (int j = 0; j < G::RPT; ++j) {
        const int r = kBS * I + G::RPT * rg + j;
        if (r < nvalid) {
            const int64_t off = ((tok0 + r) * H + h) * (int64_t)D + c0;
            R.k[j] = load8(k + off);
            R.q[j] = load8(q + off);
            R.g[j][0] = *reinterpret_cast<const f32x4 *>(log_alpha + off);
            R.g[j][1] = *reinterpret_cast<const f32x4 *>(log_alpha + off + 4);
        } else {
            R.k[j] = Vec8<T>::zero();
            R.q[j] = Vec8<T>::zero();
            R.g[j][0] = zero4();
            R.g[j][1] = zero4();
        }
    }
    R.v = Vec8<T>::zero();
    if (tid < G::VTH) {
        const int vr = tid / (DVS / 8), vc = 8 * (tid % (DVS / 8));
        if (vr < nvalid) R.v = load8(v + ((tok0 + vr) * H + h) * (int64_t)D + v0 + vc);
    }
    R.beta = (tid < kC && tid < nvalid) ? beta[(tok0 + tid) * H + h] : 0.f;
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
    T *sKL = reinterpret_cast<T *>(smem + G::oKL);
    T *sQL = reinterpret_cast<T *>(smem + G::oQL);
    T *sKE = reinterpret_cast<T *>(smem + G::oKE);
    T *sKP = reinterpret_cast<T *>(smem + G::oKP);
    T *sQP = reinterpret_cast<T *>(smem + G::oQP);
    float *sA = reinterpret_cast<float *>(smem + G::oA);
    T *sX = reinterpret_cast<T *>(smem + G::oX);
    T *sDL = reinterpret_cast<T *>(smem + G::oDL);
    T *sO = reinterpret_cast<T *>(smem + G::oO);
    T *sKendT = reinterpret_cast<T *>(smem + G::oKendT);
    T *sMqk = reinterpret_cast<T *>(smem + G::oMqk);
    T *sTr = reinterpret_cast<T *>(smem + G::oTr);
    T *sTt = reinterpret_cast<T *>(smem + G::oTt);
    T *sTd = reinterpret_cast<T *>(smem + G::oTd);
    float *sScr = reinterpret_cast<float *>(smem + G::oScr);
    T *sS = reinterpret_cast<T *>(smem + G::oS);
    T *sV = reinterpret_cast<T *>(smem + G::oV);
    float *sBeta = reinterpret_cast<float *>(smem + G::oBeta);
    float *sTot = reinterpret_cast<float *>(smem + G::oTot);
    float *sDp = reinterpret_cast<float *>(smem + G::oDp);
    float *sGam = reinterpret_cast<float *>(smem + G::oGam);

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
        if (owns_state && initial_state) {
            Sm[ct] = *reinterpret_cast<const f32x4 *>(
                initial_state + sbase + (int64_t)(v0 + 16 * ct + l16) * D + 16 * wave + 4 * l4);
        }
        if (owns_state)
            store4(sS + (16 * ct + l16) * G::LDK + 16 * wave + 4 * l4, Sm[ct][0], Sm[ct][1],
                   Sm[ct][2], Sm[ct][3]);
    }

    // prep thread map: block I = wave / 2, channels c0..c0+7, rows r_j.
    const int pI = wave >> 1;
    const int prg = lane % G::RGB, pcg = lane / G::RGB;
    const int pc0 = (wave & 1) * (D / 2) + 8 * pcg;

    ChunkRegs<T, D, DVS> R;
    if (nchunks > 0)
        load_chunk<T, D, DVS>(R, q, k, v, log_alpha, beta, tbeg,
                              (int)((tend - tbeg) < kC ? (tend - tbeg) : kC), h, H, v0, tid);

    for (int ch = 0; ch < nchunks; ++ch) {
        const int64_t tok0 = tbeg + (int64_t)ch * kC;
        const int nvalid = (int)((tend - tok0) < kC ? (tend - tok0) : kC);

        // ------------------------------------------------------------ prep
        float kf[G::RPT][8], qf[G::RPT][8], P[G::RPT][8];
        float btot[8];
        {
            float gl[G::RPT][8];
#pragma unroll
            for (int j = 0; j < G::RPT; ++j) {
                Vec8<T>::to_float(R.k[j], kf[j]);
                Vec8<T>::to_float(R.q[j], qf[j]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gl[j][e] = R.g[j][0][e] * kLog2e;
                    gl[j][4 + e] = R.g[j][1][e] * kLog2e;
                }
            }
            // inclusive prefix over this thread's rows, then over the lanes of
            // the block (lanes prg = 0..RGB-1 are consecutive in a DPP row).
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float run = 0.f;
#pragma unroll
                for (int j = 0; j < G::RPT; ++j) {
                    run += gl[j][e];
                    P[j][e] = run;
                }
                float x = run;
                {
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
                }
                const float excl = x - run;
#pragma unroll
                for (int j = 0; j < G::RPT; ++j) P[j][e] += excl;
                btot[e] = __shfl(x, lane | (G::RGB - 1), 64);
            }
        }
        float vf[8];
        Vec8<T>::to_float(R.v, vf);
        const float beta_r = R.beta;
        if (prg == G::RGB - 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sTot[pI * D + pc0 + e] = btot[e];
        }

        // Output of the previous chunk: copy the staged tile to global memory
        // (the staging area is reused by the operand tiles below).
        if (ch > 0 && tid < G::VTH) {
            const int64_t ptok = tok0 - kC;  // previous chunk was full
            const int orow = tid / (DVS / 8), ocol = 8 * (tid % (DVS / 8));
            float of[8];
            Vec8<T>::to_float(load8(sO + orow * DVS + ocol), of);
            store8(out + ((ptok + orow) * H + h) * (int64_t)D + v0 + ocol, of);
        }
        __syncthreads();

        float eGb[8];
        {
            float Gb[8], Gend[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = 0.f, pre = 0.f;
#pragma unroll
                for (int J = 0; J < kNB; ++J) {
                    const float t = sTot[J * D + pc0 + e];
                    if (J < pI) pre += t;
                    acc += t;
                }
                Gb[e] = pre;
                Gend[e] = acc;
            }
            float KLv[G::RPT][8], QLv[G::RPT][8], KEv[G::RPT][8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float fend = fast_exp2(Gend[e] - Gb[e]);  // decay from block start to chunk end
                eGb[e] = fast_exp2(Gb[e]);                     // decay from chunk start to block start
#pragma unroll
                for (int j = 0; j < G::RPT; ++j) {
                    const float L = fast_exp2(P[j][e]);
                    const float E = fast_exp2(-P[j][e]);
                    KLv[j][e] = kf[j][e] * L;
                    QLv[j][e] = qf[j][e] * L;
                    KEv[j][e] = kf[j][e] * E;
                    // K_end^T: key channel row, chunk-token column
                    const int r = kBS * pI + G::RPT * prg + j;
                    sKendT[(pc0 + e) * G::LDC + r] = from_f32<T>(KEv[j][e] * fend);
                }
            }
#pragma unroll
            for (int j = 0; j < G::RPT; ++j) {
                const int r = kBS * pI + G::RPT * prg + j;
                store8(sKL + r * G::LDK + pc0, KLv[j]);
                store8(sQL + r * G::LDK + pc0, QLv[j]);
                store8(sKE + r * G::LDK + pc0, KEv[j]);
            }
        }
        if (tid < G::VTH) {
            const int vr = tid / (DVS / 8), vc = 8 * (tid % (DVS / 8));
            store8(sV + vr * G::LDV + vc, vf);
        }
        if (tid < kC) sBeta[tid] = beta_r;
        // Off-diagonal rescale vectors exp(Gamma_{16I-1} - Gamma_{16J-1}) and
        // the chunk decay gamma = exp(Gamma_last).
        for (int i = tid; i < 6 * D; i += kThreads) {
            const int p = i / D, c = i % D;
            const int I = (p >= 1) + (p >= 3) + 1;
            const int J = p - (I - 1) * I / 2;
            float s = 0.f;
            for (int K = J; K < I; ++K) s += sTot[K * D + c];
            sDp[i] = fast_exp2(s);
        }
        if (tid < D) {
            float s = 0.f;
#pragma unroll
            for (int K = 0; K < kNB; ++K) s += sTot[K * D + tid];
            sGam[tid] = fast_exp2(s);
        }
        __syncthreads();

        // ------------------------------------------------------------ A, Mqk
        f32x4 Areg[3];
        int Aij[3];
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            Areg[s] = zero4();
            Aij[s] = -1;
            const int t = wave + kWaves * s;
            if (t >= 20) continue;
            const bool isA = t < 10;
            int I, J;
            tile_ij(isA ? t : t - 10, I, J);
            const T *left = (isA ? sKL : sQL) + kBS * I * G::LDK;
            const T *right = sKE + kBS * J * G::LDK;
            f32x4 acc = zero4();
            if (J < I) {
                const float *sc = sDp + pair_index(I, J) * D;
#pragma unroll
                for (int kk = 0; kk < D; kk += KS)
                    acc = M::mma(M::load_scaled(left + kk, G::LDK, sc + kk, lane),
                                 M::load(right + kk, G::LDK, lane), acc);
            } else {
                acc = tile_mma<T, D>(acc, left, G::LDK, right, G::LDK, lane);
            }
            if (isA) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * l4 + e;
                    float val = acc[e] * sBeta[kBS * I + r];
                    if (I == J && l16 >= r) val = 0.f;
                    acc[e] = val;
                }
                Areg[s] = acc;
                Aij[s] = I * kNB + J;
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

        // A to LDS (fp32), K+ = K e^Gamma and Q+ = Q e^Gamma over the old tiles.
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            if (Aij[s] < 0) continue;
            const int I = Aij[s] / kNB, J = Aij[s] % kNB;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sA[(kBS * I + 4 * l4 + e) * G::LDA + kBS * J + l16] = Areg[s][e];
        }
        // In place over K L and Q L: rows of block I scaled by exp(Gamma_{16I-1}).
#pragma unroll
        for (int j = 0; j < G::RPT; ++j) {
            const int r = kBS * pI + G::RPT * prg + j;
            float kp[8], qp[8];
            Vec8<T>::to_float(load8(sKP + r * G::LDK + pc0), kp);
            Vec8<T>::to_float(load8(sQP + r * G::LDK + pc0), qp);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kp[e] *= eGb[e];
                qp[e] *= eGb[e];
            }
            store8(sKP + r * G::LDK + pc0, kp);
            store8(sQP + r * G::LDK + pc0, qp);
        }
        // Prefetch the next chunk's inputs; they arrive while this chunk runs.
        if (ch + 1 < nchunks) {
            const int64_t nt0 = tok0 + kC;
            load_chunk<T, D, DVS>(R, q, k, v, log_alpha, beta, nt0,
                                  (int)((tend - nt0) < kC ? (tend - nt0) : kC), h, H, v0, tid);
        }
        __syncthreads();

        // ------------------------------------------------------------ T
        // Diagonal blocks: lane 16*I + j solves column j of (I + A_II)^{-1}.
        if (wave == 0) {
            const int I = l4, j = l16;
            float x[kBS];
#pragma unroll
            for (int r = 0; r < kBS; ++r) {
                const float *arow = sA + (kBS * I + r) * G::LDA + kBS * I;
                float s = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) s -= arow[i] * x[i];
                x[r] = s;
            }
            const float bj = sBeta[kBS * I + j];
#pragma unroll
            for (int r = 0; r < kBS; ++r) {
                sTd[(I * kBS + r) * G::LDD + j] = from_f32<T>(x[r]);
                sTr[(kBS * I + r) * G::LDC + kBS * I + j] = from_f32<T>(x[r] * bj);
            }
#pragma unroll
            for (int r = 0; r < kBS; r += 4)
                store4(sTt + (kBS * I + j) * G::LDC + kBS * I + r, x[r], x[r + 1], x[r + 2],
                       x[r + 3]);
        }
        __syncthreads();
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
                        ab[0] = static_cast<bf16>(a4[0]); ab[1] = static_cast<bf16>(a4[1]);
                        ab[2] = static_cast<bf16>(a4[2]); ab[3] = static_cast<bf16>(a4[3]);
                        const bf16x4 bb = *reinterpret_cast<const bf16x4 *>(
                            sTt + (kBS * J + l16) * G::LDC + kBS * K + 4 * l4);
                        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                            __builtin_bit_cast(i16x4, ab), __builtin_bit_cast(i16x4, bb), acc, 0,
                            0, 0);
                    }
                    const bf16x4 ta = *reinterpret_cast<const bf16x4 *>(
                        sTd + (I * kBS + l16) * G::LDD + 4 * l4);
                    bf16x4 xb;
                    xb[0] = static_cast<bf16>(-acc[0]); xb[1] = static_cast<bf16>(-acc[1]);
                    xb[2] = static_cast<bf16>(-acc[2]); xb[3] = static_cast<bf16>(-acc[3]);
                    Y = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        __builtin_bit_cast(i16x4, ta), __builtin_bit_cast(i16x4, xb), Y, 0, 0,
                        0);
                } else {
                    for (int K = J; K < I; ++K) {
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const float a = sA[(kBS * I + l16) * G::LDA + kBS * K + 4 * s + l4];
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
                        const float a = to_f32(sTd[(I * kBS + l16) * G::LDD + 4 * s + l4]);
                        const float b = scr[l16 * G::LDX + 4 * s + l4];
                        Y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, Y, 0, 0, 0);
                    }
                }
                // lane holds T_IJ[4*l4 + e][l16]
                store4(sTt + (kBS * J + l16) * G::LDC + kBS * I + 4 * l4, Y[0], Y[1], Y[2], Y[3]);
                const float bj = sBeta[kBS * J + l16];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sTr[(kBS * I + 4 * l4 + e) * G::LDC + kBS * J + l16] = from_f32<T>(Y[e] * bj);
            }
            __syncthreads();
        }

        // ------------------------------------------------------------ scan
        // [K+; Q+] S: waves 0-3 predict (K+ S), waves 4-7 read (Q+ S).
        f32x4 Pacc[G::NCT];
        {
            const int rt = wave & 3;
            const T *src = (wave < 4 ? sKP : sQP) + kBS * rt * G::LDK;
#pragma unroll
            for (int ct = 0; ct < G::NCT; ++ct) Pacc[ct] = zero4();
#pragma unroll
            for (int kk = 0; kk < D; kk += KS) {
                const typename M::Frag a = M::load(src + kk, G::LDK, lane);
#pragma unroll
                for (int ct = 0; ct < G::NCT; ++ct)
                    Pacc[ct] = M::mma(a, M::load(sS + 16 * ct * G::LDK + kk, G::LDK, lane),
                                      Pacc[ct]);
            }
            if (wave < 4) {
                // X = V - K+ S, stored transposed (value column, token).
#pragma unroll
                for (int ct = 0; ct < G::NCT; ++ct) {
                    float x[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = kBS * rt + 4 * l4 + e;
                        x[e] = to_f32(sV[r * G::LDV + 16 * ct + l16]) - Pacc[ct][e];
                    }
                    store4(sX + (16 * ct + l16) * G::LDC + kBS * rt + 4 * l4, x[0], x[1], x[2],
                           x[3]);
                }
            }
        }
        __syncthreads();

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
                    const typename M::Frag a = M::load(sTr + kBS * rt * G::LDC + ks * KS, G::LDC, lane);
#pragma unroll
                    for (int ct = 0; ct < G::NCT; ++ct)
                        acc[ct] = M::mma(a, M::load(sX + 16 * ct * G::LDC + ks * KS, G::LDC, lane),
                                         acc[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < G::NCT; ++ct)
                store4(sDL + (16 * ct + l16) * G::LDC + kBS * rt + 4 * l4, acc[ct][0], acc[ct][1],
                       acc[ct][2], acc[ct][3]);
        }
        __syncthreads();

        // O = Q+ S + Mqk Delta (waves 4-7), staged for a coalesced store.
        if (wave >= 4) {
            const int rt = wave - 4;
            const int nks = (kBS * (rt + 1) + KS - 1) / KS;
#pragma unroll
            for (int ks = 0; ks < kC / KS; ++ks) {
                if (ks < nks) {
                    const typename M::Frag a = M::load(sMqk + kBS * rt * G::LDC + ks * KS, G::LDC, lane);
#pragma unroll
                    for (int ct = 0; ct < G::NCT; ++ct)
                        Pacc[ct] = M::mma(a, M::load(sDL + 16 * ct * G::LDC + ks * KS, G::LDC, lane),
                                          Pacc[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < G::NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sO[(kBS * rt + 4 * l4 + e) * DVS + 16 * ct + l16] = from_f32<T>(Pacc[ct][e]);
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
                const typename M::Frag a = M::load(sKendT + 16 * wave * G::LDC + kk, G::LDC, lane);
#pragma unroll
                for (int ct = 0; ct < G::NCT; ++ct)
                    Sm[ct] = M::mma(a, M::load(sDL + 16 * ct * G::LDC + kk, G::LDC, lane), Sm[ct]);
            }
#pragma unroll
            for (int ct = 0; ct < G::NCT; ++ct)
                store4(sS + (16 * ct + l16) * G::LDK + 16 * wave + 4 * l4, Sm[ct][0], Sm[ct][1],
                       Sm[ct][2], Sm[ct][3]);
        }
        __syncthreads();

        // The last chunk's output (possibly partial) is stored here; earlier
        // chunks are stored at the top of the next iteration.
        if (ch + 1 == nchunks && tid < G::VTH) {
            const int orow = tid / (DVS / 8), ocol = 8 * (tid % (DVS / 8));
            if (orow < nvalid) {
                float of[8];
                Vec8<T>::to_float(load8(sO + orow * DVS + ocol), of);
                store8(out + ((tok0 + orow) * H + h) * (int64_t)D + v0 + ocol, of);
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
    return launch<float, 64, 32>(q, k, v, log_alpha, beta, initial_state, cu_seqlens, out,
                                 final_state, num_seqs, seq_len, total_tokens, num_heads, stream);
}

}  // namespace kda
