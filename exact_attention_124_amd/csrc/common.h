// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Raw buffer resource over `bytes` bytes at `base`.  Loads past the end return
// zero and stores past the end are dropped, which handles ragged tails without
// branches.  `bytes` must be below 2^32.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16(u32x4 x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(u32x2 x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(x, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(uint32_t x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(x, r, off, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: C(32x32) += A(32x16) * B(16x32).
// Lane l supplies row (l % 32) of A and column (l % 32) of B, each as 8 values
// along the contraction; the two lane halves (l / 32) carry the two halves of
// the 16-long contraction.  Result: lane l holds column (l % 32) and rows
// 8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_permlane32_swap exchanges the two 32-lane halves of a wave; with the same
// register as both operands, every lane ends up holding {x[l], x[l ^ 32]} in
// its two results.  Max and sum over that pair are symmetric, so they do not
// depend on which result carries which half.
__device__ __forceinline__ float pair_max(float x) {
    const uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte load from a buffer straight into LDS (no VGPR staging).  Lane l's
// 16 bytes land at lds_wave_base + 16*l; the base must be wave-uniform.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_wave_base, 16, off,
                                             0, 0, 0);
}

// The same with the tile's byte offset in the scalar soffset operand, so that
// a loop over tiles needs no per-lane address arithmetic (voff stays fixed).
__device__ __forceinline__ void buf_load16_lds_so(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                  void *lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_wave_base, 16, voff,
                                             soff, 0, 0);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives element
// (j % 4) of the 4-element vectors addressed by lanes j/4, j/4+4, j/4+8 and
// j/4+12 of its group (a 16x4 -> 4x16 transpose of 16-bit elements).
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Wait until at most N_ vector-memory operations of this wave are outstanding.
// Loads complete in issue order, so this means every load older than the
// newest N_ has landed.
template <int N_>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N_ >= 0 && N_ < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt((N_ & 15) | (((N_ >> 4) & 3) << 14) | 0x0F70);
}

// buf_load16_lds issued from inline assembly, for kernels that keep several
// tiles in flight.  The compiler counts its own direct-to-LDS loads as writes
// to all of LDS that every barrier (a release fence) and every LDS read must
// wait for, which would drain all of them at each tile; hidden from it, the
// caller tracks completion with wait_vmcnt.  M0, which holds the LDS
// destination, is saved and restored around the load.
__device__ __forceinline__ void load16_lds_async(__amdgpu_buffer_rsrc_t r, uint32_t voff, const void *lds) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(base), "v"(voff), "s"(r)
        : "memory");
}

// The same with a scalar byte offset (soffset) added to voff, and a 4-byte
// variant (lane l's 4 bytes land at lds + 4*l), for loops whose per-tile
// offset is wave-uniform.
__device__ __forceinline__ void load16_lds_async_so(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                    const void *lds) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(base), "v"(voff), "s"(r), "s"(soff)
        : "memory");
}
__device__ __forceinline__ void load4_lds_async_so(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                   const void *lds) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(base), "v"(voff), "s"(r), "s"(soff)
        : "memory");
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats -> two bf16 (round to nearest even) packed low/high in one word.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Two probabilities rounded to bf16 (nearest even) and packed low/high, the
// word the P*V product consumes; their sum as rounded is added to `acc` with
// one v_dot2c_f32_bf16 against (1, 1).  Normalising O by the sum of the
// rounded probabilities makes it a weighted mean of V rows whose weights add
// up to one: the rounding of a dominant probability then cancels between the
// numerator and the denominator instead of moving O by up to 2^-8 |v|.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_sum_bf16x2(float lo, float hi, float &acc) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(v, one, acc, false);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Causal launches may give each workgroup two blocks, n-1-i and i, so that all
// workgroups carry the same number of tiles.  That halves the grid, so it is
// done only when the unpaired grid fills the chip at least twice over
// (workgroups resident per CU given by the caller).  Beyond eight rounds the
// longest-first order already keeps the tail short and the second prologue
// per workgroup costs more than pairing saves (measured +0.2 to +1.7 % at
// sixteen rounds, -10 to -17 % at four).  Unpaired grids run one block per
// workgroup, longest first.
// Compute units and L2 domains (XCDs) of the current device, read once per
// device.  gfx950 groups 32 CUs per XCD; a partitioned device (fewer CUs)
// reports fewer XCDs.  The dispatcher hands workgroup i to XCD i % xcds.
struct DeviceShape {
    int cus;
    int xcds;
};
inline DeviceShape device_shape() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];  // cus + 1, 0 = not read yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
    int cus = dev >= 0 ? cache[dev].load(std::memory_order_relaxed) - 1 : -1;
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        if (dev >= 0) cache[dev].store(cus + 1, std::memory_order_relaxed);
    }
    const int xcds = (cus % 32 == 0 && cus >= 32) ? cus / 32 : 1;
    return DeviceShape{cus, xcds};
}
inline bool pair_causal_blocks(long long workgroups, int resident_per_cu) {
    const long long round = (long long)device_shape().cus * resident_per_cu;
    return workgroups >= 2 * round && workgroups <= 8 * round;
}

// Block index remap so that consecutive logical blocks land on the same XCD.
// The dispatcher hands workgroup i to XCD (i % xcds); this inverts that so the
// blocks of one attention head share one XCD's L2.  A bijection of
// [0, nblocks) for any xcds >= 1 (so a wrong count costs locality only).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks, int xcds) {
    const int xcd = bid % xcds;
    const int local = bid / xcds;
    const int per = nblocks / xcds;
    const int rem = nblocks - per * xcds;
    const int start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    return start + local;
}

}  // namespace attn
