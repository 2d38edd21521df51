// kda_bwd_chain.hip -- the backward's dL/dS chain for bf16 inputs, pipelined.
//
// Pages cited (by title):
//   [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer (§四: the KDA
//                   update; §六.2: a chunk's updates as matrix products).
//
// The chunk form of the forward (per 16-token chunk with entering state S0,
// Gamma = the within-chunk prefix of log_alpha, K+ = K e^G, K- = K e^-G,
// Q+ = Q e^G, Ke = K e^(G_last - G), gam = e^G_last, A = StrictTril(diag(b)
// K+ K-^T), M = Tril(Q+ K-^T), T = (I + A)^-1) carries dL/dS backwards over
// the chunks with
//   dS_prev = diag(gam) dS + Q+^T dO - K+^T dX,
//   dX = diag(b) T^T (M^T dO + Ke dS),
// which needs no forward state.  Everything in it except the products with dS
// is fixed by the chunk's inputs, so it is split the way the prefill splits
// its chunk recurrence: preparation waves form, one chunk ahead, the operands
// of a chunk (Ke, K+^T, Q+^T, dO^T, T^T, gam, b and M^T dO) in one of two LDS
// operand sets, while the scan waves carry dS through the previous chunk from
// the other set:
//   ddl = M^T dO + Ke dS        (dS in registers, Ke from the set)
//   lam = T^T ddl,  dX = b lam  (register tiles feed the next product)
//   dS  = diag(gam) dS + Q+^T dO - K+^T dX.
// Two barriers per chunk, which wait for LDS operations only.  The chunk's
// input rows reach the preparation through LDS: six preparation waves stage
// them two chunks ahead with direct-to-LDS loads (no registers, and no load
// issue on the waves with the triangular solve), waiting for their own loads
// before the barrier that precedes the rows' first read.  One workgroup per
// (sequence, head, half of the value columns); the scan waves hold 16 value columns each, all d_k rows, as
// fp32 registers.  Before a chunk is processed its dS (the gradient at the
// chunk's end) is written to the checkpoint slot the gradient kernel reads;
// after the first chunk dS is the initial state's gradient.  bf16 matrix
// products with fp32 accumulation throughout (v_mfma_f32_16x16x32_bf16 for the
// d_k contractions, 16x16x16 for the 16-token ones; never one shape's result
// as the other's accumulator).
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_lanes.h"
#include "kda_slots.h"

namespace kda {

namespace {

constexpr int kCC = 16;  // tokens per chunk
static_assert(kCC == kSlotTokens, "one workspace slot per chunk");

template <int D>
struct ChainCfg {
    static constexpr int DV = D / 2;     // value columns per workgroup
    static constexpr int PW = D / 16;    // preparation waves: (channel, 4 tokens) per thread
    static constexpr int SW = DV / 16;   // scan waves: 16 value columns each
    static constexpr int THREADS = 64 * (PW + SW);
    static constexpr int NT = D / 16;    // 16-row key tiles of a scan lane's state
    static_assert(NT % 2 == 0, "key tiles are stored in pairs");
    static constexpr int LR = D + 8;     // bf16 row stride of [16][D] arrays
    static constexpr int LT = 24;        // bf16 row stride of [x][16 tokens] arrays
    // one operand set (byte offsets)
    static constexpr int oKe = 0;                       // Ke [16][LR]
    static constexpr int oKpT = oKe + 16 * LR * 2;      // K+^T [D][LT]
    static constexpr int oQpT = oKpT + D * LT * 2;      // Q+^T [D][LT]
    static constexpr int oDOT = oQpT + D * LT * 2;      // dO^T [DV][LT] (this half)
    static constexpr int oTt = oDOT + DV * LT * 2;      // T^T [16][LT]
    static constexpr int oDM = oTt + 16 * LT * 2;       // M^T dO, [SW][64 lanes] f32x4
    static constexpr int oGam = oDM + SW * 64 * 16;     // gam [D] fp32
    static constexpr int oBeta = oGam + D * 4;          // b [16] fp32
    static constexpr int SET = oBeta + 16 * 4;
    // the preparation's own rows (one copy): K+, K-, Q+ [16][LR] bf16, A^T fp32
    static constexpr int oKp = 2 * SET, oKm = oKp + 16 * LR * 2, oQp = oKm + 16 * LR * 2;
    static constexpr int LA = 20;                       // fp32 row stride of A^T
    static constexpr int oAt = oQp + 16 * LR * 2;
    // two staging buffers of a chunk's rows as stored (k, q bf16 [16][D]; log_alpha
    // fp32 [16][D]; this half's d_out bf16 [16][DV]; beta [16]), filled by the scan
    // waves' direct-to-LDS loads two chunks ahead of their preparation
    // 16-byte pieces per lane: one instruction moves 1 KiB, stored BLK bytes
    // apart (the pad puts the rows four tokens apart on other LDS banks)
    static constexpr int NK = 16 * D * 2 / 1024, NG = 16 * D * 4 / 1024, NO = 16 * DV * 2 / 1024;
    static constexpr int BLK = 1024 + 32;
    static constexpr int sK = 0, sQ = sK + NK * BLK, sG = sQ + NK * BLK, sO = sG + NG * BLK,
                         sB = sO + NO * BLK, STG = sB + 16 * 4;
    static constexpr int oStg = oAt + 16 * LA * 4;
    static constexpr int BYTES = oStg + 2 * STG;
    static constexpr int NSTG = 2 * NK + NG + NO;  // instructions per chunk (beta apart)
    static_assert(STG % 16 == 0 && NO >= 1, "staging layout");
    static_assert(SET % 16 == 0 && oAt % 16 == 0 && oStg % 16 == 0, "16-byte aligned arrays");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// 8 bf16 of a row with k contiguous: k = 32 b + 4 g + e and 32 b + 16 + 4 g + e
// (the 16x16x32 operand of lane group g)
__device__ __forceinline__ bf16x8 row8(const bf16 *row, int b, int g) {
    const u32x2 lo = *reinterpret_cast<const u32x2 *>(row + 32 * b + 4 * g);
    const u32x2 hi = *reinterpret_cast<const u32x2 *>(row + 32 * b + 16 + 4 * g);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
// 4 bf16 of a row: k = 4 g + e (the 16x16x16 operand of lane group g)
__device__ __forceinline__ i16x4 row4(const bf16 *row, int g) {
    return __builtin_bit_cast(i16x4, *reinterpret_cast<const u32x2 *>(row + 4 * g));
}
// two floats as bf16 in one word (the first in the low half)
__device__ __forceinline__ unsigned pack2(float a, float b) {
    return __builtin_bit_cast(unsigned, bf16x2{static_cast<bf16>(a), static_cast<bf16>(b)});
}
__device__ __forceinline__ i16x4 pk4(const f32x4 &x) {
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = static_cast<bf16>(x[e]);
    return __builtin_bit_cast(i16x4, r);
}
__device__ __forceinline__ bf16x8 pk8(const f32x4 &a, const f32x4 &b) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = static_cast<bf16>(a[e]);
        r[4 + e] = static_cast<bf16>(b[e]);
    }
    return r;
}
__device__ __forceinline__ f32x4 mma32(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const i16x4 &a, const i16x4 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// keeps the scheduler from moving LDS accesses across this point
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }
// a workgroup barrier that no instruction is scheduled across and that
// waits for the wave's LDS operations only: the staging waves' direct-to-LDS
// loads stay in flight across it (their issuer waits for them a tick later,
// before the barrier that precedes their first read)
__device__ __forceinline__ void phase_sync() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
template <int SRC>
__device__ __forceinline__ float quad_from(float x) {  // lane SRC of each group of 4
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), SRC * 0x55, 0xf, 0xf, false));
}

template <int D>
__global__ __launch_bounds__(ChainCfg<D>::THREADS) void bwd_chain_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const float *__restrict__ log_alpha,
    const float *__restrict__ beta, const int32_t *__restrict__ cu_seqlens,
    const bf16 *__restrict__ d_out, const float *__restrict__ d_final,
    float *__restrict__ d_initial, bf16 *__restrict__ dckpt, int num_seqs, int seq_len,
    int total_tokens, int H, int units, int units_per_xcd) {
    typedef ChainCfg<D> G;
    constexpr int NT = G::NT, LR = G::LR, LT = G::LT;
    __shared__ __attribute__((aligned(16))) unsigned char sm[G::BYTES];

    // workgroup -> (unit, value half): the units of an XCD are contiguous and
    // both halves of a unit run on the same XCD (shared chunk inputs in L2)
    const int bid = blockIdx.x, kx = bid >> 3;
    const int unit = (bid & 7) * units_per_xcd + (kx >> 1), half = kx & 1;
    if (unit >= units) return;
    const int h = unit % H;
    int n = unit / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // role branches: uniform
    const int r = lane & 15, g4 = lane >> 4;
    if (cu_seqlens && num_seqs <= 64) {
        // packed: the chains of the longest sequences first (position n takes
        // the sequence of rank n by clamped length, ties by index)
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
    int64_t tbeg, tend;
    if (cu_seqlens) {
        int a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > total_tokens ? total_tokens : a);
        b = b < a ? a : (b > total_tokens ? total_tokens : b);
        tbeg = a, tend = b;
    } else {
        tbeg = (int64_t)n * seq_len, tend = tbeg + seq_len;
    }
    const int nch = (int)((tend - tbeg + kCC - 1) / kCC);
    const int64_t DD = (int64_t)D * D;
    const unsigned HD = (unsigned)H * D;
    const int64_t sbase = ((int64_t)n * H + h) * DD;
    // chunk c's end gradient goes to slot tbeg / 16 + n + c ([slot][H][d_v][d_k])
    bf16 *dck = dckpt + (first_slot(tbeg, n) * H + h) * DD;
    const int64_t ck_stride = (int64_t)H * DD;
    auto set_at = [&](int s) { return sm + s * G::SET; };
    auto stage_at = [&](int s) { return sm + G::oStg + s * G::STG; };
    // Preparation wave 2 + sw's share of chunk c's rows (the waves without 16 x
    // 16 work), into staging buffer b: piece i of NSTG (k, q, log_alpha, then
    // this half's d_out, 1 KiB each, 16 bytes per lane in row order) for i = sw,
    // sw + NSW, ...; the last of them also takes beta.  Rows past the chunk's end
    // read its first row instead (in bounds; the preparation zeroes them).
    constexpr int NSW = G::PW - 2;
    auto stage_rows = [&](int c, int b, int sw) {
        const int64_t t0 = tbeg + (int64_t)c * kCC;
        const int nv = (int)((tend - t0) < kCC ? (tend - t0) : kCC);
        const int64_t row0 = (t0 * H + h) * (int64_t)D;
        unsigned char *B = stage_at(b);
#pragma unroll
        for (int i0 = 0; i0 < G::NSTG; i0 += NSW) {
            const int i = i0 + sw;
            if (i >= G::NSTG) break;
            const void *src;
            unsigned char *dst;
            if (i < 2 * G::NK) {  // k, q: D / 8 lanes per row
                const int j = i % G::NK, lr = j * (1024 / (2 * D)) + lane / (D / 8);
                const int row = lr < nv ? lr : 0;
                const bf16 *base = i < G::NK ? k : q;
                src = base + row0 + (int64_t)row * HD + 8 * (lane % (D / 8));
                dst = B + (i < G::NK ? G::sK : G::sQ) + j * G::BLK;
            } else if (i < 2 * G::NK + G::NG) {  // log_alpha: D / 4 lanes per row
                const int j = i - 2 * G::NK, lr = j * (1024 / (4 * D)) + lane / (D / 4);
                const int row = lr < nv ? lr : 0;
                src = log_alpha + row0 + (int64_t)row * HD + 4 * (lane % (D / 4));
                dst = B + G::sG + j * G::BLK;
            } else {  // this half's d_out: DV / 8 lanes per row
                const int j = i - 2 * G::NK - G::NG, lr = j * (1024 / (2 * G::DV)) + lane / (G::DV / 8);
                const int row = lr < nv ? lr : 0;
                src = d_out + row0 + (int64_t)row * HD + half * G::DV + 8 * (lane % (G::DV / 8));
                dst = B + G::sO + j * G::BLK;
            }
            __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
        }
        if (sw == NSW - 1 && lane < kCC) {
            const int row = lane < nv ? lane : 0;
            __builtin_amdgcn_global_load_lds(beta + (t0 + row) * H + h, B + G::sB, 4, 0, 0);
        }
    };

    if (wave < G::PW) {
        // ======================================================== preparation
        // thread (channel ch, token quarter tq) for the elementwise work;
        // (value column dv, token quarter dq) for the dO rows of this half
        const int ch = 16 * wave + r, tq = g4;
        const int dv = tid % G::DV, dq = tid / G::DV;
        const bool has_o = tid < 4 * G::DV;
        float rg[4], rb = 0.f;
        bf16 rk[4], rq[4], ro[4];
        // chunk c's rows from staging buffer b (rows past its end as zeros)
        auto rows = [&](int c, int b) {
            const int64_t t0 = tbeg + (int64_t)c * kCC;
            const int nv = (int)((tend - t0) < kCC ? (tend - t0) : kCC);
            const unsigned char *B = stage_at(b);
            // byte offset of row i in a tensor of rows of RB bytes (1 KiB blocks)
            auto at = [](int i, int RB) { return (i / (1024 / RB)) * G::BLK + (i % (1024 / RB)) * RB; };
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 4 * tq + j;
                const bool ok = i < nv;
                rg[j] = ok ? reinterpret_cast<const float *>(B + G::sG + at(i, 4 * D))[ch] : 0.f;
                rk[j] = ok ? reinterpret_cast<const bf16 *>(B + G::sK + at(i, 2 * D))[ch]
                           : static_cast<bf16>(0.f);
                rq[j] = ok ? reinterpret_cast<const bf16 *>(B + G::sQ + at(i, 2 * D))[ch]
                           : static_cast<bf16>(0.f);
                const int io = 4 * dq + j;
                ro[j] = has_o && io < nv
                            ? reinterpret_cast<const bf16 *>(B + G::sO + at(io, 2 * G::DV))[dv]
                            : static_cast<bf16>(0.f);
            }
            rb = tid < kCC && tid < nv ? reinterpret_cast<const float *>(B + G::sB)[tid] : 0.f;
        };
        // the rows of the first two chunks prepared (ticks 0 and 1)
        if (wave >= 2) {
            if (nch > 0) stage_rows(nch - 1, 0, wave - 2);
            if (nch > 1) stage_rows(nch - 2, 1, wave - 2);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        if (nch > 0) rows(nch - 1, 0);
        for (int tick = 0; tick <= nch && nch > 0; ++tick) {
            const int c = nch - 1 - tick;  // the chunk prepared in this tick
            unsigned char *S = set_at(tick & 1);
            if (c >= 0) {
                // ---- phase 1: prefix, exponentials, the operand rows (in
                // registers since the previous tick; waves 0 and 1, which have
                // the 16 x 16 work in phase 2, read theirs here, where the
                // preparation waits for the scan)
                if (wave < 2 && tick > 0) rows(c, tick & 1);
                float pre[4], acc = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc += rg[j];
                    pre[j] = acc;
                }
                float sq[4];  // the four token quarters' sums of this channel
                rows4_gather(acc, sq);
                const float s0 = sq[0], s1 = sq[1], s2 = sq[2], s3 = sq[3];
                const float off = tq == 0 ? 0.f : tq == 1 ? s0 : tq == 2 ? s0 + s1 : (s0 + s1) + s2;
                const float glast = ((s0 + s1) + s2) + s3;
                bf16 kp[4], qp[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 4 * tq + j;
                    const float gi = off + pre[j];
                    const float eg = __expf(gi), kv = static_cast<float>(rk[j]);
                    kp[j] = static_cast<bf16>(kv * eg);
                    qp[j] = static_cast<bf16>(static_cast<float>(rq[j]) * eg);
                    reinterpret_cast<bf16 *>(sm + G::oKp)[i * LR + ch] = kp[j];
                    reinterpret_cast<bf16 *>(sm + G::oKm)[i * LR + ch] =
                        static_cast<bf16>(kv * __expf(-gi));
                    reinterpret_cast<bf16 *>(sm + G::oQp)[i * LR + ch] = qp[j];
                    reinterpret_cast<bf16 *>(S + G::oKe)[i * LR + ch] =
                        static_cast<bf16>(kv * __expf(glast - gi));
                }
                *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(S + G::oKpT) + ch * LT +
                                            4 * tq) = bf16x4{kp[0], kp[1], kp[2], kp[3]};
                *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(S + G::oQpT) + ch * LT +
                                            4 * tq) = bf16x4{qp[0], qp[1], qp[2], qp[3]};
                if (tq == 0) reinterpret_cast<float *>(S + G::oGam)[ch] = __expf(glast);
                if (has_o)
                    *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(S + G::oDOT) + dv * LT +
                                                4 * dq) = bf16x4{ro[0], ro[1], ro[2], ro[3]};
                if (tid < kCC) reinterpret_cast<float *>(S + G::oBeta)[tid] = rb;
            }
            // the staged rows of the next chunk (issued last tick) have landed
            // before barrier A: every preparation wave reads them after it
            if (wave >= 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            phase_sync();  // A
            if (c >= 0) {
                // ---- phase 2: the 16 x 16 work on waves 0 and 1; the other
                // waves read the next chunk's rows from its staging buffer into
                // registers and stage the rows of the chunk prepared two ticks
                // on (c - 2) into the buffer this chunk's rows came from (read
                // before barrier A)
                if (wave >= 2) {
                    if (c > 0) rows(c - 1, (tick + 1) & 1);
                    if (c >= 2) stage_rows(c - 2, tick & 1, wave - 2);
                }
                const bf16 *kpr = reinterpret_cast<const bf16 *>(sm + G::oKp) + r * LR;
                const bf16 *kmr = reinterpret_cast<const bf16 *>(sm + G::oKm) + r * LR;
                const bf16 *qpr = reinterpret_cast<const bf16 *>(sm + G::oQp) + r * LR;
                if (wave == 0) {
                    // A = diag(b) StrictTril(K+ K-^T): lane (column r, rows 4 g4 + e)
                    f32x4 a = zero4();
#pragma unroll
                    for (int b = 0; b < D / 32; ++b) a = mma32(row8(kpr, b, g4), row8(kmr, b, g4), a);
                    const f32x4 bt = *reinterpret_cast<const f32x4 *>(
                        reinterpret_cast<const float *>(S + G::oBeta) + 4 * g4);
                    float *at = reinterpret_cast<float *>(sm + G::oAt);
                    f32x4 av;
#pragma unroll
                    for (int e = 0; e < 4; ++e) av[e] = 4 * g4 + e > r ? bt[e] * a[e] : 0.f;
                    *reinterpret_cast<f32x4 *>(at + r * G::LA + 4 * g4) = av;  // A^T row r
                    wave_lds_fence();
                    // T = (I + A)^-1 by right-looking substitution: lane 4 j + qd holds
                    // rows 4 qd .. 4 qd + 3 of column j; at step m the pivot T[m][j]
                    // comes from quad lane m / 4, and every row below m takes
                    // -A[row][m] times it
                    const int j = lane >> 2, qd = lane & 3;
                    // all 15 columns in registers first: the substitution's
                    // steps then wait on no LDS read
                    f32x4 cols[kCC - 1];
#pragma unroll
                    for (int m = 0; m < kCC - 1; ++m)
                        cols[m] = *reinterpret_cast<const f32x4 *>(at + m * G::LA + 4 * qd);
                    sched_fence();
                    float t[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[e] = (4 * qd + e == j) ? 1.f : 0.f;
#pragma unroll
                    for (int m = 0; m < kCC - 1; ++m) {
                        const f32x4 col = cols[m];
                        float x;
                        switch (m >> 2) {
                            case 0: x = quad_from<0>(t[m & 3]); break;
                            case 1: x = quad_from<1>(t[m & 3]); break;
                            case 2: x = quad_from<2>(t[m & 3]); break;
                            default: x = quad_from<3>(t[m & 3]); break;
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) t[e] -= col[e] * x;
                    }
                    // T^T row j, columns 4 qd .. 4 qd + 3
                    *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(S + G::oTt) + j * LT +
                                                4 * qd) =
                        bf16x4{static_cast<bf16>(t[0]), static_cast<bf16>(t[1]),
                               static_cast<bf16>(t[2]), static_cast<bf16>(t[3])};
                } else if (wave == 1) {
                    // M = Tril(Q+ K-^T): lane (column r, rows i = 4 g4 + e), which is
                    // M^T as the A operand (row r, k = i); then M^T dO per 16 columns
                    f32x4 m = zero4();
#pragma unroll
                    for (int b = 0; b < D / 32; ++b) m = mma32(row8(qpr, b, g4), row8(kmr, b, g4), m);
                    f32x4 mv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) mv[e] = r <= 4 * g4 + e ? m[e] : 0.f;
                    const i16x4 mt = pk4(mv);
                    const bf16 *dot = reinterpret_cast<const bf16 *>(S + G::oDOT);
                    i16x4 dr[G::SW];  // the dO^T rows first, then the products
#pragma unroll
                    for (int u = 0; u < G::SW; ++u) dr[u] = row4(dot + (16 * u + r) * LT, g4);
                    f32x4 d[G::SW];
#pragma unroll
                    for (int u = 0; u < G::SW; ++u) d[u] = mma16(mt, dr[u], zero4());
#pragma unroll
                    for (int u = 0; u < G::SW; ++u)
                        *reinterpret_cast<f32x4 *>(S + G::oDM + (u * 64 + lane) * 16) = d[u];
                }
            }
            phase_sync();  // B
        }
    } else {
        // ======================================================== scan
        const int sw = wave - G::PW;
        const int vl = 16 * sw + r;             // value column within this half
        const int vg = half * G::DV + vl;       // value column of the head
        f32x4 dS[NT];  // dL/dS: key rows 16 t + 4 g4 + e, value column vg
#pragma unroll
        for (int t = 0; t < NT; ++t)
            dS[t] = d_final ? *reinterpret_cast<const f32x4 *>(d_final + sbase + (int64_t)vg * D +
                                                               16 * t + 4 * g4)
                            : zero4();
        __syncthreads();  // the staging of the first two chunks
        for (int tick = 0; tick <= nch && nch > 0; ++tick) {
            const int c = nch - tick;  // the chunk carried in this tick
            const unsigned char *S = set_at((tick + 1) & 1);
            f32x4 u[NT];
            i16x4 dxp;
            if (tick > 0) {
                // ddl = M^T dO + Ke dS (the dependent chain first; the stores and
                // Q+^T dO below fill its matrix-core latency)
                f32x4 ddl = *reinterpret_cast<const f32x4 *>(S + G::oDM + (sw * 64 + lane) * 16);
                const bf16 *ke = reinterpret_cast<const bf16 *>(S + G::oKe) + r * LR;
#pragma unroll
                for (int b = 0; b < D / 32; ++b) ddl = mma32(row8(ke, b, g4), pk8(dS[2 * b], dS[2 * b + 1]), ddl);
                // lam = T^T ddl, dX = b lam
                const f32x4 lam = mma16(row4(reinterpret_cast<const bf16 *>(S + G::oTt) + r * LT, g4),
                                        pk4(ddl), zero4());
                const f32x4 bt = *reinterpret_cast<const f32x4 *>(
                    reinterpret_cast<const float *>(S + G::oBeta) + 4 * g4);
                f32x4 dx;
#pragma unroll
                for (int e = 0; e < 4; ++e) dx[e] = bt[e] * lam[e];
                dxp = pk4(dx);
                // the chunk's end gradient for the gradient kernel, key tiles t and
                // t + 1 together, 16 bytes per lane: one permlane16 swap per packed
                // word gives the even rows (g4 = 2 j) keys 16 t + 8 j .. + 7 of tile
                // t and the odd rows keys 16 (t + 1) + 8 j .. + 7 of tile t + 1
                bf16 *dst = dck + c * ck_stride + (int64_t)vg * D;
#pragma unroll
                for (int t = 0; t < NT; t += 2) {
                    const unsigned a0 = pack2(dS[t][0], dS[t][1]), a1 = pack2(dS[t][2], dS[t][3]);
                    const unsigned b0 = pack2(dS[t + 1][0], dS[t + 1][1]);
                    const unsigned b1 = pack2(dS[t + 1][2], dS[t + 1][3]);
                    const auto p0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
                    const auto p1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
                    *reinterpret_cast<u32x4 *>(dst + 16 * (t + (g4 & 1)) + 8 * (g4 >> 1)) =
                        u32x4{p0[0], p1[0], p0[1], p1[1]};
                }
                // Q+^T dO (no dS in it)
                const i16x4 dof = row4(reinterpret_cast<const bf16 *>(S + G::oDOT) + vl * LT, g4);
                const bf16 *qpt = reinterpret_cast<const bf16 *>(S + G::oQpT);
#pragma unroll
                for (int t = 0; t < NT; ++t) u[t] = mma16(row4(qpt + (16 * t + r) * LT, g4), dof, zero4());
            }
            phase_sync();  // A
            if (tick > 0) {
                // dS <- diag(gam) dS + Q+^T dO - K+^T dX
                const bf16 *kpt = reinterpret_cast<const bf16 *>(S + G::oKpT);
                const float *gam = reinterpret_cast<const float *>(S + G::oGam);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const f32x4 y = mma16(row4(kpt + (16 * t + r) * LT, g4), dxp, zero4());
                    const f32x4 gm = *reinterpret_cast<const f32x4 *>(gam + 16 * t + 4 * g4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dS[t][e] = gm[e] * dS[t][e] + u[t][e] - y[e];
                }
            }
            phase_sync();  // B
        }
        if (d_initial) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                *reinterpret_cast<f32x4 *>(d_initial + sbase + (int64_t)vg * D + 16 * t + 4 * g4) =
                    dS[t];
        }
    }
}

}  // namespace

int launch_bwd_chain(const void *q, const void *k, const float *log_alpha, const float *beta,
                     const int32_t *cu_seqlens, const void *d_out, const float *d_final_state,
                     float *d_initial_state, float *dckpt, int32_t num_seqs, int32_t seq_len,
                     int32_t total_tokens, int32_t num_heads, int head_dim, hipStream_t stream) {
    const int64_t units64 = (int64_t)num_seqs * num_heads;
    if (units64 == 0) return 0;
    if (units64 > (int64_t)1 << 29) return -1;
    const int units = (int)units64, per_xcd = (units + 7) / 8;
    const dim3 grid((unsigned)(16 * per_xcd));
#define KDA_CHAIN_ARGS                                                                         \
    static_cast<const bf16 *>(q), static_cast<const bf16 *>(k), log_alpha, beta, cu_seqlens,    \
        static_cast<const bf16 *>(d_out), d_final_state, d_initial_state,                      \
        reinterpret_cast<bf16 *>(dckpt), num_seqs, seq_len, total_tokens, num_heads, units,    \
        per_xcd
    if (head_dim == 128)
        hipLaunchKernelGGL((bwd_chain_kernel<128>), grid, dim3(ChainCfg<128>::THREADS), 0, stream,
                           KDA_CHAIN_ARGS);
    else
        hipLaunchKernelGGL((bwd_chain_kernel<64>), grid, dim3(ChainCfg<64>::THREADS), 0, stream,
                           KDA_CHAIN_ARGS);
#undef KDA_CHAIN_ARGS
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kda
