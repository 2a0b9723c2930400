// attn_gfx950.h -- device helpers shared by the gfx950 attention kernels
// (attn_fwd_kernel.hip, attn_decode.hip): operand types, LDS addressing,
// lane-half reductions, buffer loads (to registers and straight to LDS),
// wait counts and the per-pair operand masks of the window.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// 32-bit LDS address <-> LDS pointer.
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(const lds_u8_t *)p; }
__device__ __forceinline__ const lds_u8_t *lds_ptr(uint32_t a) { return (const lds_u8_t *)(uintptr_t)a; }

// v_permlane32_swap exchanges lanes 0..31 of one register with lanes 32..63
// of another.  Swapping x with itself leaves {x[l], x[l ^ 32]} in the two
// results of every lane l, so their max / sum is the reduction over the two
// lane halves, identical in both halves.
__device__ __forceinline__ float max_halves(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + lo + hi of a packed pair of bf16 values (v_dot2_f32_bf16 against
// (1, 1)).  The row sums l add up the bf16-rounded P that the PV MFMAs use.
__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), bf16x2_t{(__bf16)1.0f, (__bf16)1.0f},
                                           acc, false);
}

// Buffer resource over [base, base + bytes); loads beyond it return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float4 bload16f(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

template <typename T>
__device__ __forceinline__ T &lds_at(uint8_t *base, int off) { return *reinterpret_cast<T *>(base + off); }

// Buffer load of 16 bytes per lane straight into LDS: lane i writes
// lds_base + 16 i (lds_base wave-uniform, passed in M0).  Out-of-range lanes
// write zeros.  Issued through inline assembly so that the compiler does not
// treat these asynchronous LDS writes as pending on every later LDS read and
// barrier; the kernel waits for them itself (wait_vmcnt) before the barrier
// that publishes the tile.  M0 is an input operand of the statement (the
// "{m0}" constraint): the compiler writes it and knows it is in use.
// The compiler checks no hazards on the scalar operands of an inline
// statement, so the statement starts with five wait states itself: a VALU
// write of an SGPR (the descriptor words often come from v_readfirstlane)
// needs 5 before a VMEM instruction reads it, an SALU write of M0 needs 1
// before an LDS DMA.  With fewer, a load can take a descriptor word's
// previous value, another buffer's base address, and read out of bounds.
//
// Debug build (ATTN_SERIAL_LOADS=1): every such load is waited for right
// after it is issued, so no load is ever in flight while the kernel goes on.
// The arithmetic and its order are unchanged: the outputs must be bitwise
// those of the pipelined build.  A read of a slot whose load the pipelined
// kernel had not waited for, or a load overwriting a slot another wave still
// reads, would make them differ.
// The wait is part of the same statement as the load, so nothing the
// compiler schedules can fall between them.
#ifndef ATTN_SERIAL_LOADS
#define ATTN_SERIAL_LOADS 0
#endif
#if ATTN_SERIAL_LOADS
#define ATTN_LDS_LOAD_TAIL "\n\ts_waitcnt vmcnt(0)"
#else
#define ATTN_LDS_LOAD_TAIL ""
#endif

// The same kind of buffer resource as four 32-bit words (base, stride 0,
// size, flags), for the inline assembly below, which takes it as a scalar
// operand.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t make_desc(const void *base, uint32_t bytes)
{
    const uint64_t p = (uint64_t)(uintptr_t)base;
    u32x4_t d;
    d.x = (uint32_t)p;
    d.y = (uint32_t)(p >> 32) & 0xffffu;
    d.z = bytes;
    d.w = 0x00020000u;
    return d;
}

__device__ __forceinline__ void dma16(u32x4_t r, uint32_t voff, const uint8_t *lds_base)
{
    // Both scalar operands pass through readfirstlane: free when the value
    // already lives in SGPRs, one v_readfirstlane per word when register
    // allocation moved it to a VGPR (the asm operands must be SGPRs).
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)lds_base);
    u32x4_t rs;
    rs.x = __builtin_amdgcn_readfirstlane(r.x);
    rs.y = __builtin_amdgcn_readfirstlane(r.y);
    rs.z = __builtin_amdgcn_readfirstlane(r.z);
    rs.w = __builtin_amdgcn_readfirstlane(r.w);
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ATTN_LDS_LOAD_TAIL
                 :
                 : "v"(voff), "s"(rs), "{m0}"(m0)
                 : "memory");
}

// The same with the LDS destination as a 32-bit LDS byte address (no
// generic-pointer conversion, hence no null check in scalar code).
__device__ __forceinline__ void dma16(u32x4_t r, uint32_t voff, uint32_t lds_base)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    u32x4_t rs;
    rs.x = __builtin_amdgcn_readfirstlane(r.x);
    rs.y = __builtin_amdgcn_readfirstlane(r.y);
    rs.z = __builtin_amdgcn_readfirstlane(r.z);
    rs.w = __builtin_amdgcn_readfirstlane(r.w);
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ATTN_LDS_LOAD_TAIL
                 :
                 : "v"(voff), "s"(rs), "{m0}"(m0)
                 : "memory");
}

// s_waitcnt on the vector-memory counter only: at most n loads of this wave
// still in flight (loads retire in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Zero the pairs of an 8-pair K operand chunk whose bit in keep_bits is clear
// (element e of the chunk belongs to pair e of the 8 in both lane halves).
__device__ __forceinline__ bf16x8_t mask_pairs(bf16x8_t x, uint32_t keep_bits)
{
    uint4 u = __builtin_bit_cast(uint4, x);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t m = ((keep_bits >> (2 * i)) & 1u ? 0x0000ffffu : 0u) |
                           ((keep_bits >> (2 * i + 1)) & 1u ? 0xffff0000u : 0u);
        w[i] &= m;
    }
    return __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}

struct WordMask {
    uint32_t m[4];
};
// The same masks for keep bits that are wave-uniform, built in scalar
// registers: s_bitreplicate_b64_b32 writes each bit of its 32-bit source
// twice into a 64-bit result, so four rounds spread each of the 8 keep bits
// over 16 bits, and word i of the result masks pairs 2i and 2i+1.  (No memory
// access: a scalar load here would share its wait counter with the LDS operand
// reads in flight, and its wait would drain them.)
__device__ __forceinline__ uint64_t bit_replicate(uint32_t x)
{
    uint64_t r;
    asm("s_bitreplicate_b64_b32 %0, %1" : "=s"(r) : "s"(x));
    return r;
}
__device__ __forceinline__ WordMask pair_mask(uint64_t keep, int kc)
{
    const uint32_t b = (uint32_t)(keep >> (8 * kc)) & 0xffu;
    const uint64_t r3 = bit_replicate((uint32_t)bit_replicate((uint32_t)bit_replicate(b)));   // each bit x8
    const uint64_t lo = bit_replicate((uint32_t)r3), hi = bit_replicate((uint32_t)(r3 >> 32));   // x16
    return WordMask{{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)}};
}
__device__ __forceinline__ bf16x8_t apply_mask(bf16x8_t x, const WordMask &m)
{
    const uint4 u = __builtin_bit_cast(uint4, x);
    return __builtin_bit_cast(bf16x8_t, make_uint4(u.x & m.m[0], u.y & m.m[1], u.z & m.m[2], u.w & m.m[3]));
}

}  // namespace
}  // namespace attn
