// rope_pass.hip -- the separate RoPE pre-rotation pass ("AttnFuse", section 1
// and Figure 1(a): rotate Q and K in their own kernel, then run plain
// attention on the rotated copies).
//
// Memory-bound elementwise work: each thread rotates one 8-pair group of one
// row (reads 2 x 16 bytes of the row and the two 16-byte cos/sin quarters of its
// position, writes 2 x 16 bytes), using the same rotation routine and table
// as the fused kernel so both produce identical bf16 bits.  Rows of Q and of
// K are numbered together, Q rows first (without a query, only the keys are
// rotated); a row is (b, s, h) in BSHD order, so
// consecutive threads walk contiguous memory and the heads of one position
// share one cos/sin line in cache.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void rope_pass_kernel(const RopeArgs a, long long n_q_units,
                                                             long long n_units)
{
    constexpr int PG = D / 16;
    const long long u = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (u >= n_units) return;
    const bool is_q = u < n_q_units;
    const long long uu = is_q ? u : u - n_q_units;
    const int H = is_q ? a.Hq : a.Hkv;
    const long long row = uu / PG;                 // (b * S + s) * H + h
    const int pg = (int)(uu - row * PG);
    const int s = (int)((row / H) % a.S);
    const uint16_t *src = (is_q ? a.q : a.k) + row * D;
    uint16_t *dst = (is_q ? a.q_out : a.k_out) + row * D;

    uint4 lo = *reinterpret_cast<const uint4 *>(src + 8 * pg);
    uint4 hi = *reinterpret_cast<const uint4 *>(src + D / 2 + 8 * pg);
    const uint4 cq = *reinterpret_cast<const uint4 *>(a.rope_cs + (((size_t)s * 2 + 0) * PG + pg) * 8);
    const uint4 sq = *reinterpret_cast<const uint4 *>(a.rope_cs + (((size_t)s * 2 + 1) * PG + pg) * 8);
    rope_rotate8(lo, hi, cq, sq);
    *reinterpret_cast<uint4 *>(dst + 8 * pg) = lo;
    *reinterpret_cast<uint4 *>(dst + D / 2 + 8 * pg) = hi;
}

template <int D>
hipError_t launch_d(const RopeArgs &a, hipStream_t stream)
{
    constexpr int PG = D / 16;
    const long long rows_q = a.q != nullptr ? (long long)a.B * a.S * a.Hq : 0;   // q NULL: keys only
    const long long rows_k = (long long)a.B * a.S * a.Hkv;
    const long long n_q_units = rows_q * PG;
    const long long n_units = (rows_q + rows_k) * PG;
    if (n_units == 0) return hipSuccess;
    const long long blocks = (n_units + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rope_pass_kernel<D>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a,
                       n_q_units, n_units);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_pass(const RopeArgs &a, hipStream_t stream)
{
    if (a.D == 128) return launch_d<128>(a, stream);
    if (a.D == 64) return launch_d<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
