// Exact attention backward, bf16 in/out, fp32 accumulation, gfx950.
//
// The pages report training results of the fused method ("Attention Is
// Memory-Bound, and Nobody Noticed for Five Years", the results paragraph:
// faster GPT-2 training, memory linear in sequence length); its gradient is
// the chain rule applied to the forward definition (grasp.study lesson on
// standard self-attention, section "The Computational Steps of Standard
// Self-Attention").  With P the softmax probabilities and dO the upstream
// gradient:
//
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij = dO_i . O_i,
//   dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Like the forward, nothing N x N reaches memory: P is recomputed tile by
// tile from Q, K and the forward's log-sum-exp (P_ij = exp(s_ij - lse_i)).
// Three launches on one stream, no atomics (the result is deterministic):
//   1. stats: -lse_i / scale and -D_i, D_i = dO_i . O_i (fp32, into the
//      caller's workspace, rows padded to a multiple of 32 with zeros); the
//      dK/dV kernel loads them straight into its S and dP accumulators as the
//      MFMAs' starting values, so S' = S - lse/scale and dP' = dP - D come out
//      of the matrix cores and P = exp2(scale log2(e) S'), dS = P dP';
//   2. dK/dV: a workgroup owns 128 keys (four waves of 32), keeps their K
//      rows in VGPRs and their V rows in LDS, and streams 32-query tiles of
//      Q, dO (with the tile's statistics) through LDS;
//   3. dQ:   a workgroup owns 128 queries, keeps their Q and dO rows in VGPRs
//      and streams 64-key tiles of K, V through LDS (the forward's shape).
//
// Orientation.  In the dK/dV kernel the products are S = Q K^T and
// dP = dO V^T on the 32x32x16 bf16 MFMA, so a lane owns one key column and
// its P and dS values are directly the B operands of dV^T += dO^T P and
// dK^T += Q^T dS.  The dQ kernel uses S^T = K Q^T, dP^T = V dO^T and
// dQ^T += K^T dS^T, so a lane owns one query.  The transposed A operands
// (dO^T, Q^T, K^T) come from LDS transpose reads (ds_read_b64_tr_b16).
#include "common.h"
#include "launch.h"

#include <atomic>
#include <mutex>

namespace attn {
namespace bwd_bf16 {

struct Params {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;   // forward log-sum-exp (natural log), [BH, N]
    float *stats;       // workspace [BH][2][Npad]: -lse / scale, then -D; zero past N
    int Npad;           // N rounded up to a multiple of 32
    uint16_t *dq, *dk, *dv;
    int N;
    int nblk;           // blocks per slice (keys for dK/dV, queries for dQ)
    float scale;
    float scale_log2;   // scale * log2(e)
    int paired;         // causal: each workgroup runs blocks i and nblk-1-i
    int xcds;           // L2 domains of the device (block remap)
};

// Tiles read both row-wise (ds_read_b128 of one 16-byte chunk of 16
// consecutive rows per quarter-wave) and transposed (ds_read_b64_tr_b16 of 4
// consecutive rows x 32 columns per half-wave) use this XOR swizzle of the
// 16-byte chunk index, which keeps both access patterns free of bank
// conflicts: it differs on 16 consecutive rows (same parity rows, for the
// 128-byte rows of d=64), and four consecutive rows land in different
// aligned groups of four chunks.
template <int D>
__device__ __forceinline__ int swz(int row) {
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
// LDS element offset of 16-byte chunk `chunk` of tile row `row`.
template <int D>
__device__ __forceinline__ int at(int row, int chunk) {
    return row * D + 8 * (chunk ^ swz<D>(row));
}
// Tile byte offset that LDS chunk c (row-major chunk order) takes its 16
// bytes from, for the HBM -> LDS loads.
template <int D>
__device__ __forceinline__ uint32_t src_off(int c) {
    const int row = c / (D / 8), pc = c % (D / 8);
    return (uint32_t)(row * D + 8 * (pc ^ swz<D>(row))) * 2u;
}
// A operand [32 rows x 16 columns] for contraction step st from rows
// rbase.. of a tile: lane l reads row rbase + l%32, columns 16*st + 8*(l/32).
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const uint16_t *tile, int rbase, int st, int lane) {
    const int r = rbase + (lane & 31);
    return *reinterpret_cast<const bf16x8 *>(tile + at<D>(r, 2 * st + (lane >> 5)));
}
// Transposed A operand [32 columns x 16 rows] for row step st (rows
// 16*st ..) and column block t (columns 32*t ..): lane l receives column
// 32*t + l%32 at rows {16*st + 4*(l/32) + 0..3, 16*st + 8 + 4*(l/32) + 0..3},
// the row order of a 32x32 accumulator's lane halves.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t *tile, int st, int t, int lane) {
    const int tg = lane >> 4, ti = lane & 15;
    const int dd = 32 * t + 16 * (tg & 1) + 4 * (ti & 3);
    i16x4 h[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = 16 * st + 8 * r + 4 * (tg >> 1) + (ti >> 2);
        h[r] = lds_read_tr16(tile + row * D + 8 * ((dd >> 3) ^ swz<D>(row)) + (dd & 7));
    }
    return __builtin_bit_cast(bf16x8, h);
}

// Store a [D x 32] accumulator pair (rows = columns of the output row,
// lane = output row) as one bf16 row per lane, multiplied by `mul`.
template <int D>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[D / 32], float mul, __amdgpu_buffer_rsrc_t r,
                                           int row, int hf) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[t][4 * g] * mul, acc[t][4 * g + 1] * mul);
            w[1] = pack_bf16x2(acc[t][4 * g + 2] * mul, acc[t][4 * g + 3] * mul);
            buf_store8(w, r, (uint32_t)(row * D + 32 * t + 8 * g + 4 * hf) * 2u);
        }
    }
}

// ---------------------------------------------------------------------------
// 1. Row statistics: -lse_i / scale and -D_i, D_i = dO_i . O_i, 16 lanes per
//    row, over the padded rows of every slice (zeros past N).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void stats_kernel(const uint16_t *__restrict__ o, const uint16_t *__restrict__ dout,
                                                    const float *__restrict__ lse, float *__restrict__ stats, int N,
                                                    int Npad, long long prow_total, float scale) {
    constexpr int PER = D / 16;  // elements per lane
    const long long prow = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);  // padded row
    const int l16 = threadIdx.x & 15;
    const long long bh = prow / Npad;
    const int r = (int)(prow - bh * Npad);
    const bool live = prow < prow_total && r < N;
    const long long row = bh * N + r;
    float acc = 0.f;
    if (live) {
        const uint16_t *po = o + row * D + l16 * PER;
        const uint16_t *pd = dout + row * D + l16 * PER;
        uint32_t wo[PER / 2], wd[PER / 2];
        if (PER == 8) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(po), b = *reinterpret_cast<const u32x4 *>(pd);
#pragma unroll
            for (int i = 0; i < PER / 2; ++i) { wo[i] = a[i]; wd[i] = b[i]; }
        } else {
            const u32x2 a = *reinterpret_cast<const u32x2 *>(po), b = *reinterpret_cast<const u32x2 *>(pd);
#pragma unroll
            for (int i = 0; i < PER / 2; ++i) { wo[i] = a[i]; wd[i] = b[i]; }
        }
#pragma unroll
        for (int i = 0; i < PER / 2; ++i) {
            acc = fmaf(bf16_lo(wo[i]), bf16_lo(wd[i]), acc);
            acc = fmaf(bf16_hi(wo[i]), bf16_hi(wd[i]), acc);
        }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (prow < prow_total && l16 == 0) {
        float *st = stats + bh * 2 * Npad;
        st[r] = live ? -lse[row] / scale : 0.f;
        st[Npad + r] = -acc;
    }
}

// ---------------------------------------------------------------------------
// 2. dK, dV.  WAVES waves x 32 keys; BQ-query tiles of Q and dO stream
//    through double-buffered LDS.  K stays in VGPRs (B operand of S = Q K^T);
//    the workgroup's V rows sit in LDS (B operand of dP = dO V^T), which
//    leaves the register room for the 128 accumulator registers of dK and dV
//    without spilling.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int WAVES, int BQ, int OCC>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void dkdv_kernel(Params p) {
    constexpr int BK = 32 * WAVES, NQB = BQ / 32;  // keys per workgroup, 32-query blocks per tile
    constexpr int QT = BQ * D;                       // elements per Q or dO tile
    constexpr int LPW = QT / 512 / WAVES;            // wave-loads per wave per tile
    static_assert(LPW >= 1 && (QT / 512) % WAVES == 0, "tile loads must split evenly");
    constexpr int VLW = BK * D / 512 / WAVES;        // wave-loads per wave of the V rows
    static_assert(VLW >= 1 && (BK * D / 512) % WAVES == 0, "V loads must split evenly");
    constexpr int SLW = 2 * BQ / 64;                 // 4-byte wave-loads of one tile's statistics
    static_assert(SLW >= 1 && SLW <= WAVES, "statistics loads: one per wave at most");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * QT];
    __shared__ __attribute__((aligned(1024))) uint16_t vsm[BK * D];  // V rows of the workgroup's keys
    __shared__ __attribute__((aligned(16))) float sstat[2][2 * BQ];  // [buf][-lse/scale of BQ rows, then -D]
    uint16_t *const Qbuf = smem;             // [2][QT]
    uint16_t *const Obuf = smem + 2 * QT;    // [2][QT] (dO)

    // Causal, paired: the workgroup runs key blocks item and nblk-1-item one
    // after the other (low key blocks see the most queries), so every
    // workgroup gets the same number of tiles.  Unpaired: one block, in
    // ascending order, which is longest first.
    const bool paired = CAUSAL && p.paired != 0;
    const int logical = xcd_remap(blockIdx.x, gridDim.x, p.xcds);
    const int per = paired ? (p.nblk + 1) / 2 : p.nblk;  // workgroups per slice
    const int bh = logical / per;
    const int item = logical - bh * per;
    const int npass = (paired && p.nblk - 1 - item != item) ? 2 : 1;
    for (int pass = 0; pass < npass; ++pass) {
        const int kb = (paired && pass == 1) ? p.nblk - 1 - item : item;
        // readfirstlane: the wave index is uniform, so the edge-tile test below
        // is a scalar branch that interior tiles skip.
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int l32 = lane & 31, hf = lane >> 5;
        const int N = p.N;

        const size_t slice = (size_t)bh * N * D;
        const uint32_t slice_bytes = (uint32_t)N * D * 2u;
        const auto rq = make_rsrc(p.q + slice, slice_bytes);
        const auto rk = make_rsrc(p.k + slice, slice_bytes);
        const auto rv = make_rsrc(p.v + slice, slice_bytes);
        const auto rdo = make_rsrc(p.dout + slice, slice_bytes);
        const auto rdk = make_rsrc(p.dk + slice, slice_bytes);
        const auto rdv = make_rsrc(p.dv + slice, slice_bytes);
        // Statistics of this slice: [2][Npad] floats.  With 32-query tiles one
        // wave loads both halves of a tile's block (rows stay below Npad);
        // with 64-query tiles wave w loads statistic w, each through a
        // resource of its own half, so rows past Npad read as zero.
        const float *st = p.stats + (size_t)bh * 2 * p.Npad;
        const auto rst = SLW == 1 ? make_rsrc(st, (uint32_t)p.Npad * 8u)
                                  : make_rsrc(st + (wave % SLW) * p.Npad, (uint32_t)p.Npad * 4u);

        const int k0 = kb * BK + wave * 32;  // first key of this wave
        const int key = k0 + l32;            // this lane's key

        // Resident K: lane holds key `key`, columns 16*st + 8*hf .. +7.  Keys
        // >= N read as zero.
        bf16x8 kf[D / 16];
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
            kf[st] = __builtin_bit_cast(bf16x8, buf_load16(rk, (uint32_t)(key * D + 16 * st + 8 * hf) * 2u));

        // All direct-to-LDS loads are issued from inline assembly, so that the
        // compiler does not drain them before every LDS read of the current
        // tile; each wave waits for its own with wait_vmem before the barrier
        // that ends the tile.  V rows of the block first (in the tiles' row
        // layout; rows >= N read as zero); the first tile's barrier covers them.
        if (pass > 0) __syncthreads();  // every wave is done with the previous block's V
        {
            const uint32_t vbase = __builtin_amdgcn_readfirstlane((uint32_t)(kb * BK * D) * 2u);
#pragma unroll
            for (int n = 0; n < VLW; ++n)
                load16_lds_async_so(rv, src_off<D>((wave + WAVES * n) * 64 + lane), vbase,
                                    vsm + (wave + WAVES * n) * 512);
        }

        const int nqt = (N + BQ - 1) / BQ;
        const int t0 = CAUSAL ? (kb * BK) / BQ : 0;  // first query tile that sees any key of the block

        // Q and dO tiles; the statistics of the tile's BQ query rows come with
        // them, 4 bytes per lane, as a [2][BQ] block (-lse/scale, then -D).
        uint32_t ld_off[LPW];
#pragma unroll
        for (int n = 0; n < LPW; ++n) ld_off[n] = src_off<D>((wave + WAVES * n) * 64 + lane);
        auto load_tile = [&](int i, int buf) __attribute__((always_inline)) {
            if (wave < SLW) {
                const uint32_t st_off = SLW == 1 ? (uint32_t)(hf * p.Npad + l32) * 4u : (uint32_t)lane * 4u;
                load4_lds_async_so(rst, st_off, __builtin_amdgcn_readfirstlane((uint32_t)(i * BQ) * 4u),
                                   &sstat[buf][64 * wave]);
            }
            const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(i * BQ * D) * 2u);
#pragma unroll
            for (int n = 0; n < LPW; ++n) {
                load16_lds_async_so(rq, ld_off[n], base, Qbuf + buf * QT + (wave + WAVES * n) * 512);
                load16_lds_async_so(rdo, ld_off[n], base, Obuf + buf * QT + (wave + WAVES * n) * 512);
            }
        };

        const float c = p.scale_log2;
        f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
            dk[t] = f32x16{};
            dv[t] = f32x16{};
        }

        if (t0 < nqt) load_tile(t0, 0);
        wait_vmem();
        __syncthreads();
        // Every tile from t0 on is computed by every wave: a causal wave whose
        // keys all lie past the tile's last query gets P = 0 from the edge
        // test (three such tiles at most, for the block's upper waves), which
        // keeps the loop free of a per-wave skip and its register copies.
        for (int i = t0; i < nqt; ++i) {
            const int buf = (i - t0) & 1;
            const uint16_t *Qs = Qbuf + buf * QT, *Os = Obuf + buf * QT;
            // Accumulator starting values: -lse/scale and -D of this lane's
            // query rows 32*qb + 8*g + 4*hf + 0..3, four rows per 16-byte LDS
            // read (rows past N hold the padding zeros).
            const float *Ss = sstat[buf];
            f32x16 s[NQB], dp[NQB];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                f32x4 a[4], b[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    a[g] = *reinterpret_cast<const f32x4 *>(Ss + 32 * qb + 8 * g + 4 * hf);
                    b[g] = *reinterpret_cast<const f32x4 *>(Ss + BQ + 32 * qb + 8 * g + 4 * hf);
                }
                s[qb] = __builtin_bit_cast(f32x16, a);
                dp[qb] = __builtin_bit_cast(f32x16, b);
            }
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    s[qb] = mfma32(row_operand<D>(Qs, 32 * qb, st, lane), kf[st], s[qb]);
                    dp[qb] = mfma32(row_operand<D>(Os, 32 * qb, st, lane), row_operand<D>(vsm, 32 * wave, st, lane),
                                    dp[qb]);
                }
            }
            // The next tile's loads are issued once S and dP are done: a
            // vector-memory wait before that point (a register reload) would
            // otherwise wait for them too.
            if (i + 1 < nqt) load_tile(i + 1, buf ^ 1);
            // P = exp2(c S'), dS = P dP'; pairs past the sequence end or above
            // the causal diagonal get P = 0, in a block of its own that interior
            // tiles branch around.
            const bool edge = (i * BQ + BQ > N) || (CAUSAL && i * BQ < k0 + 31);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[qb][r] = fast_exp2(s[qb][r] * c);
            if (edge) {
                // Query row of element r of block qb: g0 + cr with g0 = i*BQ +
                // 4*hf and cr = 32*qb + 8*(r/4) + r%4 a constant, so the tests
                // row >= N and key > row compare cr against two per-lane values
                // (kept opaque so that the per-element offsets are not hoisted
                // out of the loop into registers).
                const int g0 = i * BQ + 4 * hf;
                int lim = N - g0, rel = key - g0;
                asm volatile("" : "+v"(lim), "+v"(rel));
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int cr = 32 * qb + 8 * (r >> 2) + (r & 3);
                        if (cr >= lim || (CAUSAL && rel > cr)) s[qb][r] = 0.f;
                    }
            }
            bf16x8 pb[2 * NQB], db[2 * NQB];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pr = s[qb][r];
                    pb[2 * qb + (r >> 3)][r & 7] = (__bf16)pr;
                    db[2 * qb + (r >> 3)][r & 7] = (__bf16)(pr * dp[qb][r]);
                }
            // dV^T += dO^T P, dK^T += Q^T dS (scale applied at the end).
#pragma unroll
            for (int st = 0; st < BQ / 16; ++st) {
#pragma unroll
                for (int t = 0; t < D / 32; ++t) {
                    dv[t] = mfma32(tr_operand<D>(Os, st, t, lane), pb[st], dv[t]);
                    dk[t] = mfma32(tr_operand<D>(Qs, st, t, lane), db[st], dk[t]);
                }
            }
            wait_vmem();
            __syncthreads();
        }

        if (key < N) {
            store_rows<D>(dk, p.scale, rdk, key, hf);
            store_rows<D>(dv, 1.f, rdv, key, hf);
        }
    }
}

// ---------------------------------------------------------------------------
// 3. dQ.  Four waves x 32 queries; 64-key tiles of K and V stream through
//    double-buffered LDS.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_kernel(Params p) {
    constexpr int WAVES = 4, BR = 32 * WAVES, BC = 64;
    constexpr int KT = BC * D;
    constexpr int LPW = KT / 512 / WAVES;
    static_assert(LPW >= 1 && (KT / 512) % WAVES == 0, "tile loads must split evenly");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * KT];
    uint16_t *const Kbuf = smem;           // [2][KT]
    uint16_t *const Vbuf = smem + 2 * KT;  // [2][KT]

    // Causal: paired (query blocks nblk-1-item, then item) or one block,
    // longest first, as in the forward.
    const bool paired = CAUSAL && p.paired != 0;
    const int logical = xcd_remap(blockIdx.x, gridDim.x, p.xcds);
    const int per = paired ? (p.nblk + 1) / 2 : p.nblk;  // workgroups per slice
    const int bh = logical / per;
    const int item = logical - bh * per;
    const int npass = (paired && p.nblk - 1 - item != item) ? 2 : 1;
    for (int pass = 0; pass < npass; ++pass) {
        const int qb = (CAUSAL && (!paired || pass == 0)) ? p.nblk - 1 - item : item;
        const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int l32 = lane & 31, hf = lane >> 5;
        const int N = p.N;

        const size_t slice = (size_t)bh * N * D;
        const uint32_t slice_bytes = (uint32_t)N * D * 2u;
        const auto rq = make_rsrc(p.q + slice, slice_bytes);
        const auto rk = make_rsrc(p.k + slice, slice_bytes);
        const auto rv = make_rsrc(p.v + slice, slice_bytes);
        const auto rdo = make_rsrc(p.dout + slice, slice_bytes);
        const auto rdq = make_rsrc(p.dq + slice, slice_bytes);

        const int r0 = qb * BR;
        const int q0 = r0 + wave * 32;
        const int qrow = q0 + l32;

        // Resident Q and dO (B operands of S^T = K Q^T and dP^T = V dO^T).
        bf16x8 qf[D / 16], of[D / 16];
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const uint32_t off = (uint32_t)(qrow * D + 16 * st + 8 * hf) * 2u;
            qf[st] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
            of[st] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
        }
        const bool live = qrow < N;
        const float *stq = p.stats + (size_t)bh * 2 * p.Npad;
        const float nlse2 = live ? stq[qrow] * p.scale_log2 : 0.f;  // -lse * log2(e)
        const float ndlt = live ? stq[p.Npad + qrow] : 0.f;           // -D

        // Key tiles of the block: interior tiles [0, nint) need no mask; the
        // edge tiles [nint, ntiles) (the ragged end, and for causal blocks the
        // tiles that reach past the block's first query) run a copy of the loop
        // body with the mask.  Every wave computes every tile (a causal wave
        // whose queries all precede a tile's keys gets P = 0 there).
        int ntiles = (N + BC - 1) / BC;
        int nint = N / BC;
        if (CAUSAL) {
            ntiles = min(ntiles, (r0 + BR - 1) / BC + 1);
            nint = min(nint, (r0 + 1) / BC);
        }

        // Direct-to-LDS tile loads from inline assembly, as in the dK/dV kernel.
        uint32_t ld_off[LPW];
#pragma unroll
        for (int n = 0; n < LPW; ++n) ld_off[n] = src_off<D>((wave + WAVES * n) * 64 + lane);
        auto load_tile = [&](int j, int buf) __attribute__((always_inline)) {
            const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(j * BC * D) * 2u);
#pragma unroll
            for (int n = 0; n < LPW; ++n) {
                load16_lds_async_so(rk, ld_off[n], base, Kbuf + buf * KT + (wave + WAVES * n) * 512);
                load16_lds_async_so(rv, ld_off[n], base, Vbuf + buf * KT + (wave + WAVES * n) * 512);
            }
        };

        const float c = p.scale_log2;
        const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;  // last key this lane's query sees
        f32x16 dq[D / 32];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) dq[t] = f32x16{};

        auto tile = [&](int j, int buf, bool masked) __attribute__((always_inline)) {
            if (j + 1 < ntiles) load_tile(j + 1, buf ^ 1);
            const uint16_t *Ks = Kbuf + buf * KT, *Vs = Vbuf + buf * KT;
            // The tile's two 32-key blocks one after the other (scores, dS,
            // then their share of the dQ product), which halves the live
            // score registers.
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
                for (int st = 0; st < D / 16; ++st) {
                    s = mfma32(row_operand<D>(Ks, 32 * b, st, lane), qf[st], s);
                    dp = mfma32(row_operand<D>(Vs, 32 * b, st, lane), of[st], dp);
                }
                // dS = P (dP - D) as the bf16 B operand of the dQ product;
                // masked tiles zero P for keys past `lim`.  Key of element r:
                // j*BC + 32*b + 8*(r/4) + 4*hf + r%4.
                bf16x8 db[2];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pr = fast_exp2(fmaf(s[r], c, nlse2));
                    if (masked) {
                        const int kk = j * BC + 32 * b + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if (kk > lim) pr = 0.f;
                    }
                    db[r >> 3][r & 7] = (__bf16)(pr * (dp[r] + ndlt));
                }
                // dQ^T += K^T dS^T over the block's keys (scale applied at the end).
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int t = 0; t < D / 32; ++t)
                        dq[t] = mfma32(tr_operand<D>(Ks, 2 * b + h, t, lane), db[h], dq[t]);
                }
            }
            wait_vmem();
            __syncthreads();
        };

        if (pass > 0) __syncthreads();  // every wave is done with the previous block's tiles
        load_tile(0, 0);
        wait_vmem();
        __syncthreads();
        // Interior tiles two at a time: the LDS buffer of each copy is a
        // constant, so the operand addresses become fixed registers plus
        // immediate offsets instead of being recomputed every tile (41 vector
        // instructions per tile; the same in the dK/dV kernel spills).
        int j = 0;
        for (; j + 1 < nint; j += 2) {
            tile(j, 0, false);
            tile(j + 1, 1, false);
        }
        for (; j < nint; ++j) tile(j, j & 1, false);
        for (; j < ntiles; ++j) tile(j, j & 1, true);
        if (live) store_rows<D>(dq, p.scale, rdq, qrow, hf);
    }
}

template <int D, bool CAUSAL, int WAVES, int BQ, int OCC>
hipError_t launch_dkdv(Params p, const BwdArgs &a, hipStream_t s) {
    p.nblk = (a.N + 32 * WAVES - 1) / (32 * WAVES);
    p.paired = CAUSAL && pair_causal_blocks((long long)a.BH * p.nblk, 2);
    const unsigned blocks = (unsigned)a.BH * (unsigned)(p.paired ? (p.nblk + 1) / 2 : p.nblk);
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL, WAVES, BQ, OCC>), dim3(blocks), dim3(64 * WAVES), 0, s, p);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs &a, hipStream_t s) {
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<const uint16_t *>(a.o);
    p.dout = static_cast<const uint16_t *>(a.dout);
    p.lse = a.lse;
    p.stats = a.stats;
    p.Npad = (a.N + 31) / 32 * 32;
    p.dq = static_cast<uint16_t *>(a.dq);
    p.dk = static_cast<uint16_t *>(a.dk);
    p.dv = static_cast<uint16_t *>(a.dv);
    p.N = a.N;
    p.scale = a.scale;
    p.scale_log2 = a.scale * kLog2e;
    p.xcds = device_shape().xcds;
    const long long prows = (long long)a.BH * p.Npad;
    hipLaunchKernelGGL((stats_kernel<D>), dim3((unsigned)((prows + 15) / 16)), dim3(256), 0, s, p.o, p.dout,
                       p.lse, p.stats, a.N, p.Npad, prows, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Two waves per SIMD: d=128 with 32-query tiles (the 256-register budget
    // spills a few values, still 20-30 % faster than one wave per SIMD),
    // d=64 with 64-query tiles.
    if constexpr (D == 128) e = launch_dkdv<D, CAUSAL, 4, 32, 2>(p, a, s);
    else e = launch_dkdv<D, CAUSAL, 4, 64, 2>(p, a, s);
    if (e != hipSuccess) return e;
    p.nblk = (a.N + 127) / 128;
    p.paired = CAUSAL && pair_causal_blocks((long long)a.BH * p.nblk, 2);
    const unsigned blocks = (unsigned)a.BH * (unsigned)(p.paired ? (p.nblk + 1) / 2 : p.nblk);
    hipLaunchKernelGGL((dq_kernel<D, CAUSAL>), dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace bwd_bf16

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s) {
    using namespace bwd_bf16;
    if (a.d == 128) return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
    return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

// ---------------------------------------------------------------------------
// Statistics without a workspace argument: a static device array, one copy per
// GPU, that every attn_bwd_noalloc call on that GPU reuses.  In host code the
// name `scratch` is only a stand-in for the symbol; the device address of the
// current GPU's copy comes from hipGetSymbolAddress, looked up once per device
// with that device current, and only that address is handed to kernels.  The
// statistics kernel writes every entry the other two kernels read (zeros for
// padding rows), so nothing needs clearing between calls.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_for_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

size_t bwd_scratch_bytes() { return kScratchBytes; }

hipError_t launch_bwd_bf16_noalloc(BwdArgs a, hipStream_t s) {
    void *p = nullptr;
    const hipError_t e = scratch_for_current_device(&p);
    if (e != hipSuccess) return e;
    a.stats = static_cast<float *>(p);
    return launch_bwd_bf16(a, s);
}

}  // namespace attn
