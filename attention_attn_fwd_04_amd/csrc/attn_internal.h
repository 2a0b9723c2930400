// attn_internal.h -- declarations shared by the host API (attn_api.cpp) and
// the gfx950 kernels.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Largest head dimension built; the per-pair window table in the kernel
// arguments is sized for it.
constexpr int kMaxPairs = 64;

// RoPE cos/sin table, built once per (device, D, theta) on the host in fp64
// and stored rounded to fp16 (nearest even).  Position p and pair group g
// (pairs 8g .. 8g+7) own two 16-byte quarters: the eight cosines, then the
// eight sines.  Quarter i of (p, g) starts at half index
// ((p * 2 + i) * (D / 16) + g) * 8, so the threads of one row that each
// rotate one pair group read one contiguous run per quarter.
struct RopeTable {
    const uint16_t *cs = nullptr;
    int capacity = 0;  // number of positions held
};

struct FwdArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    uint16_t *o;
    const uint16_t *rope_cs;  // fp16 cos/sin table; null when RoPE is off
    int rope_k;               // with RoPE: 1 rotates the keys in the kernel, 0 takes them rotated
    float *lse;               // [B, Hq, S] natural-log LSE of each row's scores; null: not written
    int B, Hq, Hkv, S, D;
    int causal;
    int use_window;
    float scale_log2e;  // scale * log2(e): scores enter exp2 directly
    int32_t window[kMaxPairs];
    // Persistent schedule (null: one work-group per query tile): sched_bins + 1
    // bin offsets, then the tasks qt | hq << 12 | b << 22, built and checked on
    // the host; causal calls only.
    const uint32_t *sched;
    int sched_bins;
};

struct RopeArgs {
    const uint16_t *q;
    const uint16_t *k;
    uint16_t *q_out;
    uint16_t *k_out;
    const uint16_t *rope_cs;
    int B, Hq, Hkv, S, D;
};

// Launchers (attn_fwd_kernel.hip, rope_pass.hip).  Return hipSuccess or the
// launch error.  The decode and backward launchers are declared in
// attn_ext_args.h.
hipError_t launch_attn_fwd(const FwdArgs &a, hipStream_t stream);
hipError_t launch_rope_pass(const RopeArgs &a, hipStream_t stream);

// ---------------------------------------------------------------------------
// Device helpers used by both the fused kernel and the separate RoPE pass, so
// that both produce the same rotated bf16 bits (for K; the fused kernel's
// query is scaled before its one rounding).
// ---------------------------------------------------------------------------
#if defined(__HIPCC__)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest even) and pack them, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Rotate eight NeoX pairs held as two 16-byte groups: lo = dims 8g..8g+7 and
// hi = dims D/2+8g..D/2+8g+7 of one row, with cq / sq the eight fp16 cosines
// and sines of that (position, group).  x' = x cos - y sin,
// y' = y cos + x sin in fp32 (fp16 -> fp32 is exact), evaluated with explicit
// fused multiply-adds so every caller rounds identically.
__device__ __forceinline__ float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// One 32-bit word of each half: two pairs.
__device__ __forceinline__ void rope_rotate_word(uint32_t &l, uint32_t &h, const uint32_t cw, const uint32_t sw)
{
    const float x0 = bf16_lo(l), x1 = bf16_hi(l);
    const float y0 = bf16_lo(h), y1 = bf16_hi(h);
    const float c0 = half_lo(cw), c1 = half_hi(cw);
    const float s0 = half_lo(sw), s1 = half_hi(sw);
    const float xr0 = __builtin_fmaf(x0, c0, -(y0 * s0));
    const float xr1 = __builtin_fmaf(x1, c1, -(y1 * s1));
    const float yr0 = __builtin_fmaf(y0, c0, x0 * s0);
    const float yr1 = __builtin_fmaf(y1, c1, x1 * s1);
    l = pack_bf16x2(xr0, xr1);
    h = pack_bf16x2(yr0, yr1);
}

// The same rotation with the results multiplied by k before the bf16
// rounding (one rounding of k x', k y').
__device__ __forceinline__ void rope_rotate_word_scaled(uint32_t &l, uint32_t &h, const uint32_t cw, const uint32_t sw,
                                                        const float k)
{
    const float x0 = bf16_lo(l), x1 = bf16_hi(l);
    const float y0 = bf16_lo(h), y1 = bf16_hi(h);
    const float c0 = half_lo(cw), c1 = half_hi(cw);
    const float s0 = half_lo(sw), s1 = half_hi(sw);
    l = pack_bf16x2(__builtin_fmaf(x0, c0, -(y0 * s0)) * k, __builtin_fmaf(x1, c1, -(y1 * s1)) * k);
    h = pack_bf16x2(__builtin_fmaf(y0, c0, x0 * s0) * k, __builtin_fmaf(y1, c1, x1 * s1) * k);
}

__device__ __forceinline__ void rope_rotate8_scaled(uint4 &lo, uint4 &hi, const uint4 cq, const uint4 sq, const float k)
{
    rope_rotate_word_scaled(lo.x, hi.x, cq.x, sq.x, k);
    rope_rotate_word_scaled(lo.y, hi.y, cq.y, sq.y, k);
    rope_rotate_word_scaled(lo.z, hi.z, cq.z, sq.z, k);
    rope_rotate_word_scaled(lo.w, hi.w, cq.w, sq.w, k);
}

// bf16 words times k, rounded once.
__device__ __forceinline__ uint4 scale_bf16x8(const uint4 u, const float k)
{
    return make_uint4(pack_bf16x2(bf16_lo(u.x) * k, bf16_hi(u.x) * k), pack_bf16x2(bf16_lo(u.y) * k, bf16_hi(u.y) * k),
                      pack_bf16x2(bf16_lo(u.z) * k, bf16_hi(u.z) * k), pack_bf16x2(bf16_lo(u.w) * k, bf16_hi(u.w) * k));
}

__device__ __forceinline__ void rope_rotate8(uint4 &lo, uint4 &hi, const uint4 cq, const uint4 sq)
{
    rope_rotate_word(lo.x, hi.x, cq.x, sq.x);
    rope_rotate_word(lo.y, hi.y, cq.y, sq.y);
    rope_rotate_word(lo.z, hi.z, cq.z, sq.z);
    rope_rotate_word(lo.w, hi.w, cq.w, sq.w);
}
#endif

}  // namespace attn
