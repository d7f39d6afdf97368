// mfma_util.hpp -- device building blocks of the gfx950 MFMA kernels: bf16
// fragment types and conversions, v_mfma_f32_32x32x16_bf16, the swizzled LDS
// tile layout, wavefront scans on DPP, and asynchronous HBM -> LDS copies with
// their waits.  gfx950 only.
#pragma once
#include "ssd_device.hpp"

namespace ssd {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // register-friendly 16-byte piece
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kXcds = 8;     // MI355X accelerator complex dies; workgroups alternate over them
constexpr int kT = 64;       // steps per block
constexpr int kPRow = 40;    // padded row (elements) of a shared 32x32 bf16 score tile (16-byte aligned)

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }
__device__ __forceinline__ i16x4 lds_tr4(const u16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}
__device__ __forceinline__ bf16x8 join8(i16x4 lo, i16x4 hi) {
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x8 join8(u32x2 lo, u32x2 hi) {
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}
// two floats rounded (to nearest even) into one packed bf16 pair: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}
// registers 8h .. 8h+7 of an accumulator as a bf16 operand
__device__ __forceinline__ bf16x8 acc_half(const f32x16& v, int h) {
    return as_bf16x8(u32x4{pack2(v[8 * h + 0], v[8 * h + 1]), pack2(v[8 * h + 2], v[8 * h + 3]),
                           pack2(v[8 * h + 4], v[8 * h + 5]), pack2(v[8 * h + 6], v[8 * h + 7])});
}
// the remainders v - hi of the eight values acc_half(v, h) rounded, themselves
// rounded to bf16: hi + lo carries v to about 16 significant bits
__device__ __forceinline__ bf16x8 acc_half_lo(const f32x16& v, int h, const bf16x8& hi) {
    const u32x4 u = as_u32x4(hi);
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        o[k] = pack2(v[8 * h + 2 * k] - __uint_as_float(u[k] << 16),
                     v[8 * h + 2 * k + 1] - __uint_as_float(u[k] & 0xffff0000u));
    return as_bf16x8(o);
}
// bf16x8 scaled elementwise in fp32 and rounded back
// v * 2^k, exact (one v_ldexp_f32 per element; no factor is formed, so a k
// beyond fp32's exponent range is fine while the products stay in it)
__device__ __forceinline__ void scale_pow2(f32x16& v, int k) {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = __builtin_amdgcn_ldexpf(v[e], k);
}

__device__ __forceinline__ bf16x8 scale8(bf16x8 v, const float (&s)[8]) {
    const u32x4 u = as_u32x4(v);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = pack2(s[2 * e] * __uint_as_float(u[e] << 16), s[2 * e + 1] * __uint_as_float(u[e] & 0xffff0000u));
    return as_bf16x8(o);
}

// Swizzle of a row-major LDS tile with PR 16-byte pieces per row: piece q of
// row r is stored at q ^ swzbits<PR>(r).  swzbits is a bijection of the row's
// low bits chosen for the two access patterns of these tiles with 64 banks of
// 4 bytes: 16 consecutive rows read at one column land on distinct 16-byte
// slots of the 256-byte bank window, and the 8 rows of one transposing read
// (64 bytes each) fill the window's four 64-byte quarters two rows apiece.
template <int PR>
__device__ __forceinline__ int swzbits(int r) {
    static_assert(PR == 4 || PR == 8 || PR == 16, "pieces per row");
    if constexpr (PR == 16) return (((r >> 1) & 3) << 2) | (((r >> 3) & 1) << 1) | (r & 1);
    else if constexpr (PR == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return (r >> 2) & 3;
}
// Element offset of (row, col) in such a tile (col a multiple of 4 for 8-byte
// accesses, of 8 for 16-byte ones).
template <int PR>
__device__ __forceinline__ int swz(int row, int col) {
    return row * (PR * 8) + ((((col >> 3) ^ swzbits<PR>(row)) << 3) | (col & 7));
}

// Inclusive prefix sum of v over the 64 lanes: shifts of 1, 2, 4, 8 within each
// row of 16 lanes (DPP row_shr, zero shifted in), then the row totals.  The
// same four DPP steps run on w in between (two independent chains, so each
// fills the other's DPP wait states) and leave in lane 16r + 15 the sum of w
// over row r.
__device__ __forceinline__ float wave_scan64_rowsum(float v, float& w, int lane) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
    w += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(w), 0x111, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
    w += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(w), 0x112, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
    w += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(w), 0x114, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
    w += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(w), 0x118, 0xf, 0xf, true));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
    if (lane >= 16) v += r0;
    if (lane >= 32) v += r1;
    if (lane >= 48) v += r2;
    return v;
}

// ---- asynchronous HBM -> LDS copies and their synchronisation -----------------
// (M0 is named as clobbered so the compiler re-initialises it before any use
// of its own; clang warns that reserved registers are not preserved.)
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}
// 16 (or 4) bytes per lane from base + off (base wave-uniform, off a 32-bit
// byte offset per lane); lane L writes LDS byte lds + 16 L (4 L).  `lds` must
// be wave-uniform (it is moved into M0).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
// no vector-memory operation of this wave outstanding
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// at most K vector-memory operations of this wave outstanding (loads complete
// in issue order, so every operation but the last K issued has completed)
template <int K>
__device__ __forceinline__ void vm_wait_le() {
    static_assert(K >= 0 && K < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(K) : "memory");
}
// workgroup barrier ordering LDS only (no wait on HBM traffic)
__device__ __forceinline__ void sync_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace ssd
