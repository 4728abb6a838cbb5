// Fused exact attention forward with a general mask and an additive bias,
// bf16 in/out, fp32 accumulation, gfx950.
//
// The pages warn that custom attention biases and unusual masks are where a
// computation falls off the fused fast path ("Attention Is Memory-Bound, and
// Nobody Noticed for Five Years", the paragraph on what the result means in
// practice).  This kernel keeps them on it: the scores of one tile are
//     s_ij = scale * q_i . k_j + bias_ij,
// restricted to the keys a causal and/or sliding-window mask allows, and go
// through the same online softmax as the bf16 kernel; S and P stay on chip.
//  * Mask: key j is allowed for query i iff (not causal or j <= i) and
//    (window_left < 0 or j >= i - window_left) and (window_right < 0 or
//    j <= i + window_right).  Tiles outside the workgroup's allowed key range
//    are never loaded; each wave skips tiles outside its own range; only
//    tiles that cut a row's range run the per-element mask.
//  * Bias: fp32, element (b, h, i, j) at bias + b*sb + h*sh + i*si + j (any
//    stride may be 0 to broadcast); -inf removes a key.  Each lane reads the
//    runs of four keys its score accumulator holds straight from HBM into
//    registers, as one 16-byte read when the bias and its strides keep every
//    run 16-byte aligned (BIAS = 2), else as four 4-byte reads (BIAS = 1);
//    the reads of a tile are issued before its score MFMAs and consumed
//    after them.
//  * With a bias the scores are formed in natural-log units (one fma of the
//    dot product with scale and the bias); without one the raw dot products
//    are kept and the scale folds into the exponent as in the bf16 kernel.
//    The running maximum is in log2 units.  Rows that
//    have seen no finite score keep the maximum at -inf and contribute
//    nothing; a row with no allowed finite score at all ends with o = 0 and
//    lse = -inf.
// The tile layout, operand orientation (S^T = K Q^T, O^T = V^T P^T) and lazy
// rescale are those of the bf16 kernel; workgroups are 4 waves x 32 queries
// with 64-key tiles, double-buffered.
#define ATTN_FWD_BF16_NO_DEFAULT_LAUNCHER
#include "attn_fwd_bf16.hip"

namespace attn {
namespace fwd_masked {

using fwd_bf16::Layout;
using fwd_bf16::Tile;

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    const float *bias;
    long long sb, sh, si;  // bias strides in elements
    int N, H;
    int nqb;
    int wl, wr;  // window sides, < 0 = unbounded
    float scale;
    int xcds;    // L2 domains of the device (block remap)
};

constexpr int WAVES = 4, BC = 64;
constexpr float kLazy = 8.0f;

template <int D, bool CAUSAL, int BIAS, bool WINDOW>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kernel(Params p) {
    using T = Tile<D, WAVES, BC>;
    using L = Layout<D>;
    constexpr int BR = T::BR, NB = T::NB;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[T::LDS_ELEMS];
    uint16_t *const Kbuf = smem;
    uint16_t *const Vbuf = smem + 2 * T::TILE;

    const int logical = xcd_remap(blockIdx.x, gridDim.x, p.xcds);
    const int bh = logical / p.nqb;
    int qb = logical - bh * p.nqb;
    if (CAUSAL) qb = p.nqb - 1 - qb;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave-uniform by construction; readfirstlane lets the compiler see it,
    // so per-wave tile decisions (active, full) become scalar branches.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int N = p.N;

    const size_t slice = (size_t)bh * N * D;
    const uint32_t slice_bytes = (uint32_t)N * D * 2u;
    const auto rq = make_rsrc(p.q + slice, slice_bytes);
    const auto rk = make_rsrc(p.k + slice, slice_bytes);
    const auto rv = make_rsrc(p.v + slice, slice_bytes);
    const auto ro = make_rsrc(p.o + slice, slice_bytes);

    const int r0 = qb * BR;
    const int q0 = r0 + wave * 32;
    const int qrow = q0 + l32;
    const int rlast = min(r0 + BR - 1, N - 1);  // last real row of the workgroup

    // Key range of the workgroup and of this wave (inclusive).
    int klo = 0, khi = N - 1, wlo = 0, whi = N - 1;
    if (CAUSAL) {
        khi = min(khi, rlast);
        whi = min(whi, q0 + 31);
    }
    if (WINDOW) {
        if (p.wl >= 0) {
            klo = max(klo, r0 - p.wl);
            wlo = max(wlo, q0 - p.wl);
        }
        if (p.wr >= 0) {
            khi = min(khi, rlast + p.wr);
            whi = min(whi, q0 + 31 + p.wr);
        }
    }
    const int jlo = klo / BC, jhi = khi / BC;  // tiles jlo .. jhi
    auto active = [&](int j) __attribute__((always_inline)) {
        return j * BC <= whi && j * BC + BC - 1 >= wlo;
    };
    // Every key of tile j allowed for every row of this wave (and < N).
    auto full = [&](int j) __attribute__((always_inline)) {
        const int a = j * BC, b = j * BC + BC - 1;
        bool f = b <= N - 1;
        if (CAUSAL) f = f && b <= q0;
        if (WINDOW) {
            if (p.wl >= 0) f = f && a >= q0 + 31 - p.wl;
            if (p.wr >= 0) f = f && b <= q0 + p.wr;
        }
        return f;
    };

    bf16x8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(qrow * D + 16 * s + 8 * hf) * 2u));

    // Bias rows of this wave: a resource over rows q0 .. min(q0 + 31, N - 1).
    // A wave of the last block may start at or past row N (it holds padding
    // rows only); its resource is empty, so every bias load returns zero and
    // none of them touches memory beyond the bias tensor.
    const float *bbase = p.bias;
    uint32_t bbytes = 0;
    if constexpr (BIAS) {
        if (q0 < N) {
            const int b_idx = bh / p.H, h_idx = bh - b_idx * p.H;
            bbase = p.bias + (long long)b_idx * p.sb + (long long)h_idx * p.sh + (long long)q0 * p.si;
            const int rows = min(31, N - 1 - q0);
            bbytes = (uint32_t)(((long long)rows * p.si + N) * 4);
        }
    }
    const auto rb = make_rsrc(bbase, bbytes);

    uint32_t k_off[T::LOADS_PER_WAVE], v_off[T::LOADS_PER_WAVE];
#pragma unroll
    for (int n = 0; n < T::LOADS_PER_WAVE; ++n) {
        const int c = (wave + WAVES * n) * 64 + lane;
        k_off[n] = L::k_src(c);
        v_off[n] = L::v_src(c);
    }
    // K/V tile copies go straight to LDS from inline assembly: the compiler
    // does not see them, so it does not drain them (and, loads completing in
    // order, the bias reads issued after them) before every LDS read.  Each
    // wave waits for its own copies before the barrier that ends the tile.
    auto load_kv = [&](int tile, int buf) __attribute__((always_inline)) {
        const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(tile * BC * D) * 2u);
#pragma unroll
        for (int n = 0; n < T::LOADS_PER_WAVE; ++n) {
            load16_lds_async_so(rk, k_off[n], base, Kbuf + buf * T::TILE + (wave + WAVES * n) * 512);
            load16_lds_async_so(rv, v_off[n], base, Vbuf + buf * T::TILE + (wave + WAVES * n) * 512);
        }
    };
    // Bias of tile j: 4 keys per 16-byte read, in accumulator order.
    constexpr int BIAS_LOADS = BIAS == 2 ? NB * 4 : BIAS == 1 ? NB * 16 : 0;  // vector loads per tile
    auto load_bias = [&](int j, f32x4 (&bz)[NB][4]) __attribute__((always_inline)) {
        if constexpr (BIAS) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int kk = j * BC + 32 * b + 8 * g + 4 * hf;
                    const uint32_t off = (uint32_t)(l32 * p.si + kk) * 4u;
                    if constexpr (BIAS == 2) {
                        bz[b][g] = __builtin_bit_cast(f32x4, buf_load16(rb, off));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            bz[b][g][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, off + 4u * e, 0, 0));
                    }
                }
        }
    };

    const float sc = p.scale;
    const float cu = BIAS != 0 ? kLog2e : sc * kLog2e;
    float m_run = -INFINITY;  // running reference maximum, log2 units
    float l_run = 0.f;
    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

    // S^T = K_tile Q^T.
    auto scores = [&](int buf, f32x16 (&s)[NB]) __attribute__((always_inline)) {
        const uint16_t *Ks = Kbuf + buf * T::TILE;
#pragma unroll
        for (int b = 0; b < NB; ++b) s[b] = f32x16{};
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                s[b] = mfma32(*reinterpret_cast<const bf16x8 *>(Ks + L::k_read(st, b, lane)), qf[st], s[b]);
    };
    // Bias, mask and online softmax of score tile j, then O^T += V^T P^T with
    // V from LDS buffer buf.
    auto softmax_pv = [&](int j, int buf, f32x16 (&s)[NB], const f32x4 (&bz)[NB][4]) __attribute__((always_inline)) {
        // Natural-log scores with bias and mask.
        const bool masked = !full(j);
        int lo = 0, hi = N - 1;
        if (CAUSAL) hi = min(hi, qrow);
        if (WINDOW) {
            if (p.wl >= 0) lo = max(lo, qrow - p.wl);
            if (p.wr >= 0) hi = min(hi, qrow + p.wr);
        }
        // u = the score in units where exp2(u * cu - m) is the probability:
        // without a bias the raw dot product (cu = scale * log2 e, one FMA per
        // probability as in the bf16 kernel), with one scale * dot + bias in
        // natural-log units (cu = log2 e).
        if constexpr (BIAS != 0) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[b][r] = fmaf(s[b][r], sc, bz[b][r >> 2][r & 3]);
        }
        // A separate block (not folded into the loop above) so that unmasked
        // tiles branch around it.
        if (masked) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kk = j * BC + 32 * b + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (kk < lo || kk > hi) s[b][r] = -INFINITY;
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = (b == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[b][r]);
        mx = pair_max(mx) * cu;  // cu > 0: scaling commutes with max
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
        }
        const float m_sub = m_run == -INFINITY ? 0.f : m_run;  // no finite score yet: every p is 0
        bf16x8 pb[2 * NB];
        // The row sum adds the probabilities as rounded for P*V.
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            u32x4 w[2];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(s[b][r], cu, -m_sub));
                const float p1 = fast_exp2(fmaf(s[b][r + 1], cu, -m_sub));
                w[r >> 3][(r & 7) >> 1] = pack_sum_bf16x2(p0, p1, (r & 2) ? rs1 : rs0);
            }
            pb[2 * b] = __builtin_bit_cast(bf16x8, w[0]);
            pb[2 * b + 1] = __builtin_bit_cast(bf16x8, w[1]);
        }
        l_run += rs0 + rs1;
        // O^T += V_tile^T P^T.
        const uint16_t *Vs = Vbuf + buf * T::TILE;
#pragma unroll
        for (int st = 0; st < BC / 16; ++st)
#pragma unroll
            for (int t = 0; t < D / 32; ++t) {
                const i16x4 w[2] = {lds_read_tr16(Vs + L::v_read(st, t, 0, lane)),
                                    lds_read_tr16(Vs + L::v_read(st, t, 1, lane))};
                acc[t] = mfma32(__builtin_bit_cast(bf16x8, w), pb[st], acc[t]);
            }
    };
    auto tile_step = [&](int j, int buf, const f32x4 (&bz)[NB][4]) __attribute__((always_inline)) {
        f32x16 s[NB];
        scores(buf, s);
        softmax_pv(j, buf, s, bz);
    };

    // The bias of tile j + 1 is read while tile j is computed (issued after
    // tile j + 1's K/V copies, so the end-of-tile wait can leave it in flight):
    // the bias is the kernel's only HBM stream without reuse, and a read issued
    // at the top of its own tile would stall the tile for a full memory round
    // trip.  Two register sets alternate, the loop unrolled by two.  The last
    // tile also copies and reads "tile jhi + 1" (unused; reads past the K/V
    // slice or the bias rows return zero): with no branch around the loads
    // the compiler's count of outstanding loads stays exact, where a
    // conditional prefetch makes it wait for the newest loads as well.
    f32x4 bzA[NB][4], bzB[NB][4];
    if constexpr (BIAS == 0) {
        // Without a bias, K runs one tile ahead of V as in the bf16 kernel:
        // during step j the LDS holds K(j+1) and V(j), and K(j+2) and V(j+1)
        // are in flight, so the score products of tile j+1 are issued before
        // the softmax of tile j.  (With a bias the second score buffer does
        // not fit beside the bias registers.)
        auto load_k = [&](int tile, int buf) __attribute__((always_inline)) {
            const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(tile * BC * D) * 2u);
#pragma unroll
            for (int n = 0; n < T::LOADS_PER_WAVE; ++n)
                load16_lds_async_so(rk, k_off[n], base, Kbuf + buf * T::TILE + (wave + WAVES * n) * 512);
        };
        auto load_v = [&](int tile, int buf) __attribute__((always_inline)) {
            const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(tile * BC * D) * 2u);
#pragma unroll
            for (int n = 0; n < T::LOADS_PER_WAVE; ++n)
                load16_lds_async_so(rv, v_off[n], base, Vbuf + buf * T::TILE + (wave + WAVES * n) * 512);
        };
        if (jlo <= jhi) {
            load_k(jlo, 0);
            load_v(jlo, 0);
            if (jlo + 1 <= jhi) load_k(jlo + 1, 1);
            wait_vmem();
            __syncthreads();
            f32x16 sa[NB], sb[NB];
            if (active(jlo)) scores(0, sa);
            __syncthreads();  // K buffer 0 is refilled (tile jlo + 2) in the first step
            auto step = [&](int j, f32x16 (&cur)[NB], f32x16 (&nxt)[NB]) __attribute__((always_inline)) {
                const int buf = (j - jlo) & 1;
                if (j + 2 <= jhi) load_k(j + 2, buf);
                if (j + 1 <= jhi) {
                    load_v(j + 1, buf ^ 1);
                    if (active(j + 1)) scores(buf ^ 1, nxt);
                }
                if (active(j)) softmax_pv(j, buf, cur, bzA);
                wait_vmem();
                __syncthreads();
            };
            int j = jlo;
            for (; j + 1 <= jhi; j += 2) {
                step(j, sa, sb);
                step(j + 1, sb, sa);
            }
            if (j <= jhi) step(j, sa, sb);
        }
    }
    auto iter = [&](int j, const f32x4 (&cur)[NB][4], f32x4 (&nxt)[NB][4]) __attribute__((always_inline)) {
        const int buf = (j - jlo) & 1;
        load_kv(j + 1, buf ^ 1);
        load_bias(j + 1, nxt);
        if (active(j)) tile_step(j, buf, cur);
        wait_vmcnt<BIAS_LOADS>();  // this wave's copies of tile j + 1 have landed
        __syncthreads();
    };
    if (BIAS != 0 && jlo <= jhi) {
        load_kv(jlo, 0);
        load_bias(jlo, bzA);
        wait_vmem();
        __syncthreads();
        int j = jlo;
        for (; j + 1 <= jhi; j += 2) {
            iter(j, bzA, bzB);
            iter(j + 1, bzB, bzA);
        }
        if (j <= jhi) iter(j, bzA, bzB);
    }

    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
        if (hf == 0 && p.lse)
            p.lse[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

template <int D, bool CAUSAL, int BIAS, bool WINDOW>
hipError_t launch(const MaskedArgs &a, hipStream_t s) {
    Params p;
    p.q = static_cast<const uint16_t *>(a.f.q);
    p.k = static_cast<const uint16_t *>(a.f.k);
    p.v = static_cast<const uint16_t *>(a.f.v);
    p.o = static_cast<uint16_t *>(a.f.o);
    p.lse = a.f.lse;
    p.bias = a.bias;
    p.sb = a.bias_stride_b;
    p.sh = a.bias_stride_h;
    p.si = a.bias_stride_i;
    p.N = a.f.N;
    p.H = a.H;
    p.nqb = (a.f.N + 32 * WAVES - 1) / (32 * WAVES);
    p.wl = a.window_left;
    p.wr = a.window_right;
    p.scale = a.f.scale;
    p.xcds = device_shape().xcds;
    const unsigned blocks = (unsigned)a.f.BH * (unsigned)p.nqb;
    hipLaunchKernelGGL((kernel<D, CAUSAL, BIAS, WINDOW>), dim3(blocks), dim3(64 * WAVES), 0, s, p);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_c(const MaskedArgs &a, hipStream_t s) {
    const bool window = a.window_left >= 0 || a.window_right >= 0;
    if (a.bias) {
        const bool vec = ((uintptr_t)a.bias & 15) == 0 && ((a.bias_stride_b | a.bias_stride_h | a.bias_stride_i) & 3) == 0;
        if (vec) return window ? launch<D, CAUSAL, 2, true>(a, s) : launch<D, CAUSAL, 2, false>(a, s);
        return window ? launch<D, CAUSAL, 1, true>(a, s) : launch<D, CAUSAL, 1, false>(a, s);
    }
    return window ? launch<D, CAUSAL, 0, true>(a, s) : launch<D, CAUSAL, 0, false>(a, s);
}

}  // namespace fwd_masked

hipError_t launch_fwd_masked(const MaskedArgs &a, hipStream_t s) {
    using namespace fwd_masked;
    if (a.f.d == 128) return a.f.causal ? launch_c<128, true>(a, s) : launch_c<128, false>(a, s);
    return a.f.causal ? launch_c<64, true>(a, s) : launch_c<64, false>(a, s);
}

}  // namespace attn
