// attn_internal.h -- declarations shared by the host API (attn_api.cpp) and
// the gfx950 kernels (attn_fwd_kernel.hip, rope_pass.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Largest head dimension built; the per-pair window table in the kernel
// arguments is sized for it.
constexpr int kMaxPairs = 64;

// RoPE cos/sin table, fp32, built once per (device, D, theta) on the host in
// fp64: for position p and pair group g (pairs 8g .. 8g+7) sixteen floats,
// cos of the eight angles then sin of the eight angles.  A thread that
// rotates one 8-pair group of one row reads these 64 contiguous bytes.
// Index: ((p * (D / 16)) + g) * 16 + {0..7: cos, 8..15: sin}.
struct RopeTable {
    const float *cs = nullptr;
    int capacity = 0;  // number of positions held
};

struct FwdArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    uint16_t *o;
    const float *rope_cs;  // null when RoPE is off
    int B, Hq, Hkv, S, D;
    int causal;
    int use_window;
    float scale_log2e;  // scale * log2(e): scores enter exp2 directly
    int32_t window[kMaxPairs];
};

struct RopeArgs {
    const uint16_t *q;
    const uint16_t *k;
    uint16_t *q_out;
    uint16_t *k_out;
    const float *rope_cs;
    int B, Hq, Hkv, S, D;
};

// Launchers (attn_fwd_kernel.hip, rope_pass.hip).  Return hipSuccess or the
// launch error.
hipError_t launch_attn_fwd(const FwdArgs &a, hipStream_t stream);
hipError_t launch_rope_pass(const RopeArgs &a, hipStream_t stream);

// ---------------------------------------------------------------------------
// Device helpers used by both the fused kernel and the separate RoPE pass, so
// that both produce the same rotated bf16 bits.
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
// hi = dims D/2+8g..D/2+8g+7 of one row, with cs the 16 table floats of that
// (position, group).  x' = x cos - y sin, y' = y cos + x sin, evaluated with
// explicit fused multiply-adds so every caller rounds identically.
__device__ __forceinline__ void rope_rotate8(uint4 &lo, uint4 &hi, const float *cs)
{
    uint32_t l[4] = {lo.x, lo.y, lo.z, lo.w};
    uint32_t h[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float x0 = bf16_lo(l[w]), x1 = bf16_hi(l[w]);
        float y0 = bf16_lo(h[w]), y1 = bf16_hi(h[w]);
        float c0 = cs[2 * w], c1 = cs[2 * w + 1];
        float s0 = cs[8 + 2 * w], s1 = cs[8 + 2 * w + 1];
        float xr0 = __builtin_fmaf(x0, c0, -(y0 * s0));
        float xr1 = __builtin_fmaf(x1, c1, -(y1 * s1));
        float yr0 = __builtin_fmaf(y0, c0, x0 * s0);
        float yr1 = __builtin_fmaf(y1, c1, x1 * s1);
        l[w] = pack_bf16x2(xr0, xr1);
        h[w] = pack_bf16x2(yr0, yr1);
    }
    lo = make_uint4(l[0], l[1], l[2], l[3]);
    hi = make_uint4(h[0], h[1], h[2], h[3]);
}
#endif

}  // namespace attn
