// Fused exact attention forward with 8-bit floating-point Q, K, V (OCP e4m3
// or e5m2, chosen per tensor), bf16 output, fp32 accumulation, gfx950.
//
// The function is the one of the bf16 kernel ("The Attention Bottleneck --
// and How FlashAttention Fixed It", section "The fix: tiling and fusion, never
// touch HBM"), on inputs stored as 8-bit floats with one fp32 dequantisation
// factor per tensor: the real query matrix is q_descale * Q8, and so on.  The
// low-precision variant is the one "Attention Is Memory-Bound, and Nobody
// Noticed for Five Years" reports for the FlashAttention-3 generation (results
// paragraph).  Both products run on the 32x32x64 fp8 MFMA, which issues
// twice the multiply-adds per cycle of the bf16 one:
//  * S^T = K Q^T: a lane holds one query and 32 consecutive head dims of each
//    64-wide contraction step in its 32 bytes; K rows come from LDS with two
//    ds_read_b128.  The scores are fp32, scaled by scale * q_descale *
//    k_descale * log2(e) inside the exponent.
//  * The online softmax is that of the bf16 kernel (lazy reference maximum,
//    moved only when a row exceeds it by 2^8), so every probability is at
//    most 2^8 and fits e4m3 (largest finite value 448).  Probabilities are
//    rounded to e4m3 (nearest even) two at a time with v_cvt_pk_fp8_f32 and
//    become the B operand of O^T = V^T P^T without leaving the lane; the row
//    sum adds the fp32 probabilities.
//  * The V^T operand comes from ds_read_b64_tr_b8: in each 16-lane group, lane
//    j receives byte j%8 of the 8-byte vectors addressed by lanes j/8 + 2i
//    (i = 0..7), so eight lanes addressing eight key rows deliver eight keys
//    of one head dim to every lane.  The key order of the four reads matches
//    the order in which the score accumulator holds its keys.
//  * O = v_descale * acc / l, stored as bf16; lse as in the bf16 kernel.
// The input formats are template arguments (the matrix instruction takes each
// operand's format as an immediate); both formats are bytes, so loads,
// layouts and transposes are the same for either.
// Tiles are 128 keys, double-buffered in LDS (32 KiB per K or V tile pair at
// d = 128); causal skipping, the pairing of long and short causal query blocks
// and the XCD remap follow the bf16 kernel.
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace attn {
namespace fwd_fp8 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Operand format codes of v_mfma_*_f8f6f4: 0 = fp8 (OCP e4m3), 1 = bf8 (OCP
// e5m2).  The probabilities (B operand of the second product) are always e4m3.
enum Fp8Format { kE4M3 = 0, kE5M2 = 1 };

// v_mfma_f32_32x32x64_f8f6f4, A in format FA, B in format FB, no block
// scales: C(32x32) += A(32x64) * B(64x32).  Lane l supplies row (l % 32) of A
// and column (l % 32) of B as 32 bytes; A and B use the same assignment of
// (lane half, byte) to the contraction index, so any consistent packing of
// both operands contracts correctly.  The result layout is that of the bf16
// 32x32 MFMA.
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2 *)(p));
}

__device__ __forceinline__ u32x4 lds_read16(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Four floats -> four e4m3 bytes (round to nearest even), a in the low byte.
// The two conversions overwrite both 16-bit halves of `dst`, the register
// the packed word is stored in (its old contents are dead), so no zeroed or
// copied destination has to be materialised.
__device__ __forceinline__ int pack_e4m3x4(float a, float b, float c, float d, int dst) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, dst, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

struct Params {
    const uint8_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int N;
    int nqb;           // query blocks per slice
    float scale_log2;  // scale * q_descale * k_descale * log2(e)
    float v_descale;
    int paired;        // causal: each workgroup runs blocks nqb-1-i and i
    int xcds;          // L2 domains of the device (block remap)
};

template <int D, int WAVES, int BC_>
struct Tile {
    static constexpr int BR = 32 * WAVES;  // query rows per workgroup
    static constexpr int BC = BC_;         // keys per tile
    static constexpr int NB = BC / 32;     // 32-key blocks per tile
    static constexpr int NG = BC / 64;     // 64-key groups (P*V contraction steps) per tile
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TILE = BC * D;  // bytes per K or V tile
    static constexpr int LOADS = TILE / 1024;  // wave-loads (1 KiB) per tile
    static constexpr int LOADS_PER_WAVE = (LOADS + WAVES - 1) / WAVES;
    static_assert(BC % 64 == 0 && TILE % 1024 == 0, "tiles are whole 64-key groups and wave-loads");
    static constexpr int LDS_BYTES = 4 * TILE;  // K[2], V[2]
};

// LDS layout of a tile: key rows of D bytes, 16-byte chunks XOR-swizzled per
// row.  LDS chunk c holds source chunk (c % CH) ^ swz(row) of row c / CH, so
// the HBM -> LDS copy (lane l -> chunk 64*load + l) stays row-coalesced.
// K rows are read as 16 consecutive keys x one chunk per quarter-wave and V
// rows as 8 keys x two chunks per half-wave; each swizzle spreads its access
// pattern over distinct 16-byte bank groups (rows of 128 B / 64 B alias onto
// the same banks without it).
template <int D>
struct Layout {
    static constexpr int CH = D / 16;  // chunks per key row
    __device__ static __forceinline__ int k_swz(int row) { return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3); }
    __device__ static __forceinline__ int v_swz(int row) {
        return D == 128 ? 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1)) : 2 * ((row >> 3) & 1);
    }
    __device__ static __forceinline__ uint32_t k_src(int c) {
        const int row = c / CH, pc = c % CH;
        return (uint32_t)(row * D + 16 * (pc ^ k_swz(row)));
    }
    __device__ static __forceinline__ uint32_t v_src(int c) {
        const int row = c / CH, pc = c % CH;
        return (uint32_t)(row * D + 16 * (pc ^ v_swz(row)));
    }
    // K operand of key block blk, contraction step st (head dims 64*st ..
    // 64*st + 63): lane l reads key 32*blk + l%32, dims 64*st + 32*(l/32) +
    // 16*part .. +15.
    __device__ static __forceinline__ int k_read(int st, int blk, int part, int lane) {
        const int key = 32 * blk + (lane & 31);
        const int chunk = 4 * st + 2 * (lane >> 5) + part;
        return key * D + 16 * (chunk ^ k_swz(key));
    }
    // Transpose read R (0..3) of the V^T operand of head-dim block t for the
    // 64-key group at key offset 0: 16-lane group g serves dims 32*t +
    // 16*(g%2) + 0..15 of lane half g/2; lane pair (2i, 2i+1) of the group
    // addresses key 32*(R/2) + 16*(R%2) + 8*(i/4) + 4*(g/2) + i%4, the even
    // lane its first 8 dims, the odd lane the next 8.
    __device__ static __forceinline__ int v_read(int R, int t, int lane) {
        const int g = lane >> 4, j = lane & 15, i = j >> 1, e = j & 1;
        const int key = 32 * (R >> 1) + 16 * (R & 1) + 8 * (i >> 2) + 4 * (g >> 1) + (i & 3);
        const int chunk = 2 * t + (g & 1);
        return key * D + 16 * (chunk ^ v_swz(key)) + 8 * e;
    }
};

constexpr float kLazyThreshold = 8.0f;  // log2 units; probabilities stay <= 2^8 < 448

template <int D, bool CAUSAL, int WAVES, int BC, int FQ, int FK, int FV>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kernel(Params p) {
    using T = Tile<D, WAVES, BC>;
    using L = Layout<D>;
    constexpr int BR = T::BR, NB = T::NB, NG = T::NG;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];
    uint8_t *const Kbuf = smem;                // [2][TILE]
    uint8_t *const Vbuf = smem + 2 * T::TILE;  // [2][TILE]

    // Causal: paired (blocks nqb-1-item, then item) or one block, longest
    // first, as in the bf16 kernel.
    const bool paired = CAUSAL && p.paired != 0;
    const int logical = xcd_remap(blockIdx.x, gridDim.x, p.xcds);
    const int per = paired ? (p.nqb + 1) / 2 : p.nqb;  // workgroups per slice
    const int bh = logical / per;
    const int item = logical - bh * per;
    const int npass = (paired && p.nqb - 1 - item != item) ? 2 : 1;
    for (int pass = 0; pass < npass; ++pass) {
        const int qb = (CAUSAL && (!paired || pass == 0)) ? p.nqb - 1 - item : item;

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = tid >> 6;
        const int l32 = lane & 31;
        const int hf = lane >> 5;
        const int N = p.N;

        const size_t slice = (size_t)bh * N * D;
        const uint32_t in_bytes = (uint32_t)N * D;
        const auto rq = make_rsrc(p.q + slice, in_bytes);
        const auto rk = make_rsrc(p.k + slice, in_bytes);
        const auto rv = make_rsrc(p.v + slice, in_bytes);
        const auto ro = make_rsrc(p.o + slice, in_bytes * 2u);

        const int r0 = qb * BR;
        const int q0 = r0 + wave * 32;
        const int qrow = q0 + l32;

        // Q fragment (B operand of S^T = K Q^T): query qrow, head dims 64*st +
        // 32*hf .. +31 for each contraction step st.  Rows >= N read as zero.
        i32x8 qf[D / 64];
#pragma unroll
        for (int st = 0; st < D / 64; ++st) {
            const uint32_t off = (uint32_t)(qrow * D + 64 * st + 32 * hf);
            const u32x4 a = buf_load16(rq, off), b = buf_load16(rq, off + 16u);
            const u32x4 w[2] = {a, b};
            qf[st] = __builtin_bit_cast(i32x8, w);
        }

        int ntiles = (N + BC - 1) / BC;
        int nfull = N / BC;
        if (CAUSAL) {
            ntiles = min(ntiles, (r0 + BR - 1) / BC + 1);
            nfull = min(nfull, (r0 + 1) / BC);
        }

        // ---- HBM -> LDS, 16 bytes per lane; wave-load n of this wave fills LDS
        // chunks [64*(wave + WAVES*n), +64).  Past-the-end rows read as zero.
        uint32_t k_off[T::LOADS_PER_WAVE], v_off[T::LOADS_PER_WAVE];
#pragma unroll
        for (int n = 0; n < T::LOADS_PER_WAVE; ++n) {
            const int c = (wave + WAVES * n) * 64 + lane;
            k_off[n] = L::k_src(c);
            v_off[n] = L::v_src(c);
        }
        auto load_k = [&](int tile, int buf) __attribute__((always_inline)) {
            const uint32_t base = (uint32_t)(tile * BC * D);
#pragma unroll
            for (int n = 0; n < T::LOADS_PER_WAVE; ++n)
                if (T::LOADS % WAVES == 0 || wave + WAVES * n < T::LOADS)
                    buf_load16_lds(rk, base + k_off[n], Kbuf + buf * T::TILE + (wave + WAVES * n) * 1024);
        };
        auto load_v = [&](int tile, int buf) __attribute__((always_inline)) {
            const uint32_t base = (uint32_t)(tile * BC * D);
#pragma unroll
            for (int n = 0; n < T::LOADS_PER_WAVE; ++n)
                if (T::LOADS % WAVES == 0 || wave + WAVES * n < T::LOADS)
                    buf_load16_lds(rv, base + v_off[n], Vbuf + buf * T::TILE + (wave + WAVES * n) * 1024);
        };

        auto scores = [&](int buf, f32x16 (&s)[NB]) __attribute__((always_inline)) {
            const uint8_t *Ks = Kbuf + buf * T::TILE;
#pragma unroll
            for (int b = 0; b < NB; ++b) s[b] = f32x16{};
#pragma unroll
            for (int st = 0; st < D / 64; ++st) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const u32x4 w[2] = {lds_read16(Ks + L::k_read(st, b, 0, lane)),
                                        lds_read16(Ks + L::k_read(st, b, 1, lane))};
                    s[b] = mfma_f8<FK, FQ>(__builtin_bit_cast(i32x8, w), qf[st], s[b]);
                }
            }
        };
        auto active = [&](int j) __attribute__((always_inline)) { return !CAUSAL || j * BC <= q0 + 31; };

        const float c = p.scale_log2;
        float m_run = -INFINITY;
        float l_run = 0.f;
        f32x16 acc[D / 32];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

        // Online softmax of score tile j.  pf[g] is the e4m3 B operand of the P*V
        // product for 64-key group g: byte 16*(b%2) + r holds accumulator element
        // r of key block b = 2g + b%2.
        auto softmax = [&](int j, f32x16 (&s)[NB], i32x8 (&pf)[NG], bool masked) __attribute__((always_inline)) {
            if (masked) {
                const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = j * BC + 32 * b + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if (kk > lim) s[b][r] = -INFINITY;
                    }
                }
            }
            float mx = s[0][0];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = (b == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[b][r]);
            mx = pair_max(mx) * c;
            if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyThreshold) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = fast_exp2(m_run - m_safe);
                m_run = m_safe;
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
            }
            float rs0, rs1;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    const float p0 = fast_exp2(fmaf(s[b][r], c, -m_run));
                    const float p1 = fast_exp2(fmaf(s[b][r + 1], c, -m_run));
                    const float p2 = fast_exp2(fmaf(s[b][r + 2], c, -m_run));
                    const float p3 = fast_exp2(fmaf(s[b][r + 3], c, -m_run));
                    if (b == 0 && r == 0) {
                        rs0 = p0 + p2;
                        rs1 = p1 + p3;
                    } else {
                        rs0 += p0 + p2;
                        rs1 += p1 + p3;
                    }
                    const int slot = 4 * (b & 1) + (r >> 2);
                    pf[b >> 1][slot] = pack_e4m3x4(p0, p1, p2, p3, pf[b >> 1][slot]);
                }
            }
            l_run += rs0 + rs1;
        };
        // O^T += V_tile^T P^T, one 64-key contraction per head-dim block.
        auto pv = [&](int buf, const i32x8 (&pf)[NG]) __attribute__((always_inline)) {
            const uint8_t *Vs = Vbuf + buf * T::TILE;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
#pragma unroll
                for (int t = 0; t < D / 32; ++t) {
                    const uint8_t *Vg = Vs + 64 * g * D;
                    const i32x2 w[4] = {lds_read_tr8(Vg + L::v_read(0, t, lane)),
                                        lds_read_tr8(Vg + L::v_read(1, t, lane)),
                                        lds_read_tr8(Vg + L::v_read(2, t, lane)),
                                        lds_read_tr8(Vg + L::v_read(3, t, lane))};
                    acc[t] = mfma_f8<FV, kE4M3>(__builtin_bit_cast(i32x8, w), pf[g], acc[t]);
                }
            }
        };

        i32x8 pf[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) pf[g] = i32x8{};
        // Double-buffered tiles: tile j+1 streams into LDS while tile j is used.
        load_k(0, 0);
        load_v(0, 0);
        wait_vmem();
        __syncthreads();
        // Causal: tiles below nfull are visited by every wave and need no
        // mask, so they run in a loop without the per-tile tests; the rest
        // (the diagonal, a ragged last tile) run checked.
        auto step = [&](int j, auto checked) __attribute__((always_inline)) {
            constexpr bool CHECKED = decltype(checked)::value;
            const int buf = j & 1;
            if (!CHECKED || j + 1 < ntiles) {
                load_k(j + 1, buf ^ 1);
                load_v(j + 1, buf ^ 1);
            }
            if (!CHECKED || active(j)) {
                f32x16 s[NB];
                scores(buf, s);
                softmax(j, s, pf, CHECKED && j >= nfull);
                pv(buf, pf);
            }
            wait_vmem();
            __syncthreads();
        };
        // (Causal only: on the dense 8k shape the split loop measured 2 %
        // slower than one checked loop, on causal 32k 4.7 % faster.)
        int j = 0;
        if constexpr (CAUSAL)
            for (; j + 1 < nfull; ++j) step(j, std::false_type{});
        for (; j < ntiles; ++j) step(j, std::true_type{});

        const float l_tot = pair_sum(l_run);
        const float inv = p.v_descale / l_tot;
        if (qrow < N) {
#pragma unroll
            for (int t = 0; t < D / 32; ++t) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv);
                    w[1] = pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv);
                    buf_store8(w, ro, (uint32_t)(qrow * D + 32 * t + 8 * g + 4 * hf) * 2u);
                }
            }
            if (hf == 0 && p.lse) p.lse[(size_t)bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
        }
    }
}

template <int D, bool CAUSAL, int WAVES, int BC, int FQ, int FK, int FV>
hipError_t launch(const Fp8Args &a, hipStream_t s) {
    using T = Tile<D, WAVES, BC>;
    Params p;
    p.q = static_cast<const uint8_t *>(a.f.q);
    p.k = static_cast<const uint8_t *>(a.f.k);
    p.v = static_cast<const uint8_t *>(a.f.v);
    p.o = static_cast<uint16_t *>(a.f.o);
    p.lse = a.f.lse;
    p.N = a.f.N;
    p.nqb = (a.f.N + T::BR - 1) / T::BR;
    p.scale_log2 = a.f.scale * a.q_descale * a.k_descale * kLog2e;
    p.v_descale = a.v_descale;
    p.paired = CAUSAL && pair_causal_blocks((long long)a.f.BH * p.nqb, WAVES == 8 ? 1 : 2);
    p.xcds = device_shape().xcds;
    const unsigned blocks = (unsigned)a.f.BH * (unsigned)(p.paired ? (p.nqb + 1) / 2 : p.nqb);
    hipLaunchKernelGGL((kernel<D, CAUSAL, WAVES, BC, FQ, FK, FV>), dim3(blocks), dim3(T::THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace fwd_fp8

#ifndef ATTN_FWD_FP8_NO_DEFAULT_LAUNCHER
// 128-key tiles.  8 waves (256 query rows) per workgroup for dense grids of
// at least four such workgroups per CU, else 4 waves (128 rows, two
// workgroups per CU); causal sequences always take 4 waves, whose shorter
// blocks waste less work on the diagonal.
template <int D, bool CAUSAL, int FQ, int FK, int FV>
static hipError_t launch_fp8_d(const Fp8Args &a, hipStream_t s) {
    using namespace fwd_fp8;
    const long long blocks8 = (long long)a.f.BH * ((a.f.N + 255) / 256);
    const bool wide = !CAUSAL && blocks8 >= 4 * 256;
    return wide ? launch<D, CAUSAL, 8, 128, FQ, FK, FV>(a, s) : launch<D, CAUSAL, 4, 128, FQ, FK, FV>(a, s);
}

template <int FQ, int FK, int FV>
static hipError_t launch_fp8_f(const Fp8Args &a, hipStream_t s) {
    if (a.f.d == 128)
        return a.f.causal ? launch_fp8_d<128, true, FQ, FK, FV>(a, s) : launch_fp8_d<128, false, FQ, FK, FV>(a, s);
    return a.f.causal ? launch_fp8_d<64, true, FQ, FK, FV>(a, s) : launch_fp8_d<64, false, FQ, FK, FV>(a, s);
}

// Formats: 0 = e4m3, 1 = e5m2 (validated by the caller).
hipError_t launch_fwd_fp8(const Fp8Args &a, hipStream_t s) {
    switch (a.q_format * 4 + a.k_format * 2 + a.v_format) {
    case 0: return launch_fp8_f<0, 0, 0>(a, s);
    case 1: return launch_fp8_f<0, 0, 1>(a, s);
    case 2: return launch_fp8_f<0, 1, 0>(a, s);
    case 3: return launch_fp8_f<0, 1, 1>(a, s);
    case 4: return launch_fp8_f<1, 0, 0>(a, s);
    case 5: return launch_fp8_f<1, 0, 1>(a, s);
    case 6: return launch_fp8_f<1, 1, 0>(a, s);
    default: return launch_fp8_f<1, 1, 1>(a, s);
    }
}
#endif

}  // namespace attn
