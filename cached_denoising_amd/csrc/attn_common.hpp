// Device helpers shared by the block-attention kernels: MFMA fragments, bf16
// packing, exact e4m3 widening, LDS transpose reads, direct-to-LDS loads,
// wait counters and the index helpers both kernels use.
#pragma once

#include "common.hpp"

namespace dllm {
namespace attn {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazy = 8.0f;          // log2 headroom before the running max moves
constexpr float kMinit = -1.0e30f;     // finite start of the running max

union Frag {
    uint4 u;
    bf16x8_t v;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    // one v_cvt_pk_bf16_f32: round to nearest even
    const bf16x2_t p = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, p);
}

// 8 e4m3 codes (two words) -> 8 bf16 (exact)
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    return r;
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 8 bytes addressed by lane 4r + i/4, for r = 0..3
__device__ __forceinline__ uint2 lds_tr16(const unsigned char *p) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
    const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u8 *)p);
    return __builtin_bit_cast(uint2, r);
#else
    (void)p;
    return make_uint2(0, 0);
#endif
}

// ds_read_b64_tr_b8: within each 16-lane group, lane i receives byte i%8 of
// the 8 bytes addressed by lane 2r + i/8, for r = 0..7
__device__ __forceinline__ uint2 lds_tr8(const unsigned char *p) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __attribute__((address_space(3))) v2i32_t lds_v2i32;
    const v2i32_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32 *)(lds_u8 *)p);
    return __builtin_bit_cast(uint2, r);
#else
    (void)p;
    return make_uint2(0, 0);
#endif
}

// Direct-to-LDS loads (global_load_lds): lane i of the wave reads sbase +
// voff_i and writes LDS byte lds + size * i, sbase and lds wave-uniform (the
// scalar-base form: one 32-bit offset per lane, no 64-bit address).  The LDS
// address is an integer, as lds_addr gives it once for a buffer: a generic
// pointer converted to the LDS address space carries a null check (a scalar
// compare and select) at every use.  They are issued from inline assembly, so
// the compiler's wait-count pass does not see an LDS write in flight: seen,
// it makes every later LDS read of the kernel wait for all outstanding loads
// (vmcnt 0), which empties the load pipeline at each tile.  The kernels wait
// for these loads themselves (vm_wait) before the data is read.  NT marks the
// load non-temporal: right when the rows are read once, wrong when other
// workgroups re-read them through L2.  M0 holds the LDS address; the s_nop is
// the wait state an M0 write needs before an LDS-DMA instruction.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
#if defined(__HIP_DEVICE_COMPILE__)
    return (uint32_t)(uintptr_t)(lds_u8 *)(const_cast<void *>(p));
#else
    return (uint32_t)(uintptr_t)p;
#endif
}

template <bool NT>
__device__ __forceinline__ void lds_dma16(const void *sbase, uint32_t voff, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    if (NT)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                     : : "v"(voff), "s"(sbase), "s"(m0) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     : : "v"(voff), "s"(sbase), "s"(m0) : "memory", "m0");
#else
    (void)sbase;
    (void)voff;
    (void)lds;
#endif
}

__device__ __forceinline__ void lds_dma4(const void *sbase, uint32_t voff, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 : : "v"(voff), "s"(sbase), "s"(m0) : "memory", "m0");
#else
    (void)sbase;
    (void)voff;
    (void)lds;
#endif
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// XOR swizzle of the 16-byte chunks of V row rho in LDS: the rows a 16-lane
// transposed read touches land on distinct banks (bf16: 4 rows, 32-byte
// windows; e4m3: 8 rows, 16-byte windows, two rows per 256 bytes)
template <int KVDT>
__device__ __forceinline__ int vswz(int rho) {
    return KVDT == DLLM_E4M3 ? ((rho >> 1) & 3) : 2 * (rho & 3);
}

// key index of tile-local key k (or -1): NULL map means identity over [0, n_keys)
__device__ __forceinline__ int key_at(const int32_t *kmap, int n_keys, int L, int j) {
    if (j >= n_keys) return -1;
    const int k = kmap ? kmap[j] : j;
    return (k >= 0 && k < L) ? k : -1;
}

// First dim of k-chunk c (8 dims) held by lane group g in the first product.
// Any assignment works as long as Q and K agree; this one makes the four lane
// groups of one key row read 64 contiguous bytes per load instruction.  e4m3
// rows load two chunks (16 codes) at once, bf16 rows one chunk (8 values).
template <int KVDT>
__device__ __forceinline__ int chunk_dim(int c, int g) {
    if (KVDT == DLLM_E4M3) return ((c >> 1) * 4 + g) * 16 + (c & 1) * 8;
    return (c * 4 + g) * 8;
}

// IEEE maximum (NaN-propagating).  For scores, which are finite or -inf, it
// equals fmaxf; on gfx950 it becomes v_maximum3_f32 chains, without the
// canonicalising moves that fmaxf's NaN rule adds before every input.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max and sum over the four 16-lane groups (lanes l, l^16, l^32, l^48), the
// result in every lane: two gfx950 lane swaps (v_permlane32_swap, then
// v_permlane16_swap) on the VALU instead of cross-lane LDS permutes.  With
// both operands equal, a swap leaves the lane's own value in one register
// and its partner's in the other.
__device__ __forceinline__ float group4_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Logical block order that keeps the row groups of one (sequence, KV head,
// split) on one XCD: workgroups are dealt to the 8 XCDs round robin.
__device__ __forceinline__ int xcd_remap(int pid, int nblk) {
    if ((nblk & 7) != 0) return pid;
    const int per = nblk >> 3;
    return (pid & 7) * per + (pid >> 3);
}

constexpr int kLdsBytes = 160 * 1024;  // LDS of one gfx950 CU

}  // namespace attn
}  // namespace dllm
