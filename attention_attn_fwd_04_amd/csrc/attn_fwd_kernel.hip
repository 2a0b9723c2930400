// attn_fwd_kernel.hip -- fused causal attention forward with RoPE at load,
// written for gfx950 (MI355X): bf16 MFMA 32x32x16 with fp32 accumulation,
// wave64, LDS staging.
//
// The computation ("Flash Attention: Causal Prefill D=128", "Online softmax:
// what must remain invariant"; "AttnFuse", section 2 and section 4.1):
//   for each query tile, walk the key tiles it may see;
//     S = Q' K'^T (Q', K' rotated by RoPE), masked on the tiles that cross
//     the causal diagonal or the end of the sequence;
//     online softmax in base 2 with c = scale * log2 e; O += P V;
//   O / l at the end.
//
// gfx950 design:
//  * Everything is computed transposed: S^T = K' Q'^T and O^T = V^T P^T.
//    In the 32x32 MFMA result each lane owns one query column, so the row
//    max / row sum are reductions inside the lane plus one
//    v_permlane32_swap, and the rescale multiplies whole registers.  The
//    S^T accumulator converted to bf16 is already the B operand of the PV
//    MFMA (its key order is matched on the V side), so P never leaves
//    registers.
//  * The V^T A operand is read straight from a row-major V tile with
//    ds_read_b64_tr_b16 (gfx950's LDS transpose read): a 16-lane group reads
//    4 keys x 16 dims and each lane receives 4 keys of one dim.  V is
//    therefore staged as a plain copy.
//  * One MFMA k-step covers 8 complete RoPE pairs: k-index (g, e) of chunk
//    kc maps to dimension 8 kc + (D/2) g + e.  Any consistent permutation of
//    the contraction axis leaves Q'K'^T unchanged; this one keeps the two
//    halves of a NeoX pair in the same MFMA, which the per-pair window uses.
//  * A work-group of 8 waves (two per SIMD) owns 256 query rows, 32 per
//    wave.  Each K/V tile staged in LDS is rotated once for 256 rows; while
//    one wave of a SIMD runs its softmax the other can issue MFMAs.
//  * K is rotated in registers while it is staged into LDS (each thread
//    loads both halves of its pairs, so no half swap is needed).
//  * All global loads are buffer loads: rows past the sequence end read as
//    zero, so staging has no lane-divergent branches and the loads of tile
//    j+1 stay in flight while tile j is computed.
//  * LDS tiles are XOR-swizzled in 16-byte chunks so the MFMA operand reads
//    and the transpose reads are free of bank conflicts without padding.
//  * The softmax rescale is lazy: the reference max only moves (and O, l are
//    rescaled) when a row's max grows by more than 8 in log2 units, so P is
//    at most 2^8 and the common tile skips the 64 multiplies of O.
//  * Key tiles are visited from 0 upwards; the masked tiles are the last
//    ones.  Query tiles are issued longest first, and the block index is
//    remapped so one head's tiles run on one XCD (shared L2 for its K/V).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;  // 256 query rows per work-group
constexpr int kBN = 64;                     // keys per iteration (two 32-key blocks)
constexpr float kRescaleLog2 = 8.0f;        // lazy-rescale threshold (P <= 2^8)

template <int D>
struct Geo {
    static constexpr int KCH = D / 16;      // MFMA k-steps over D (8 pairs each)
    static constexpr int PG = D / 16;       // 8-pair groups per row
    static constexpr int DB = D / 32;       // 32-row blocks of O^T
    static constexpr int CH = D / 8;        // 16-byte chunks per row
    static constexpr int ROWB = D * 2;      // bytes per row (unpadded)
    static constexpr int K_BYTES = kBN * ROWB;
    static constexpr int V_BYTES = kBN * ROWB;
    static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
    static constexpr int Q_BYTES = kBM * ROWB;
    static constexpr int LDS_BYTES = (2 * BUF_BYTES > Q_BYTES) ? 2 * BUF_BYTES : Q_BYTES;
    static constexpr int K_UNITS = kBN * PG;          // (key, pair group)
    static constexpr int V_UNITS = kBN * CH;          // (key, 16-byte chunk)
    static constexpr int V_PER_THREAD = (V_UNITS + kThreads - 1) / kThreads;
    static_assert(K_UNITS <= kThreads, "at most one K unit per thread");
    static_assert(V_UNITS % kThreads == 0 || V_UNITS < kThreads, "V units split evenly");

    // Swizzled byte offset of 16-byte chunk c of row r in a K or Q tile:
    // 16 consecutive rows read at one logical chunk land in 16 distinct
    // 4-bank groups.
    static __device__ __forceinline__ int k_off(int r, int c)
    {
        if constexpr (D == 128) return r * ROWB + ((c ^ (r & 15)) << 4);
        else return r * ROWB + ((c ^ ((r >> 1) & 7)) << 4);
    }
    // Swizzled byte offset of chunk c of row r in a V tile: the 4 rows x 4
    // chunks read by one half-wave of ds_read_b64_tr_b16 cover all banks.
    static __device__ __forceinline__ int v_off(int r, int c)
    {
        if constexpr (D == 128) return r * ROWB + ((c ^ ((r & 3) << 2)) << 4);
        else return r * ROWB + ((c ^ (((r >> 1) & 1) << 2)) << 4);
    }
};

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

// ---------------------------------------------------------------------------
// Per-pair distance window on one 32-key x 32-query block and one MFMA
// k-step kc, which holds the 8 complete pairs r = 8 kc .. 8 kc + 7 ("ATFlash
// -- Per-RoPE-Wavelength Attention Windows", "The idea": pair r contributes
// to score (n, m) only when n - m <= w[r]; w is non-decreasing in r).  The
// block's distances lie in [dlo, dhi] (dhi clipped to rows that are stored;
// causally masked cells are discarded later, so dlo is clamped at 0).
//  - every pair below dlo: the chunk is skipped (never multiplied);
//  - every pair at or above dhi: the usual MFMA;
//  - otherwise one MFMA over the pairs kept in the whole block (the others
//    zeroed in the K operand), plus, for each pair whose limit falls inside
//    [dlo, dhi), an MFMA of that pair alone added only where n - m <= w[r].
// All decisions depend on block coordinates only: wave-uniform branches.
// ---------------------------------------------------------------------------
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

__device__ __forceinline__ void window_chunk(const FwdArgs &a, bf16x8_t ka, bf16x8_t qop, f32x16_t &acc,
                                             int kc, int nq0, int mk0, int l32, int g)
{
    const int dlo = max(0, nq0 - (mk0 + 31));
    const int dhi = min(nq0 + 31, a.S - 1) - mk0;
    const int r0 = 8 * kc;
    if (a.window[r0 + 7] < dlo) return;  // all 8 pairs pruned in this block
    if (a.window[r0] >= dhi) {           // all 8 pairs kept in this block
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop, acc, 0, 0, 0);
        return;
    }
    uint32_t keep = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (a.window[r0 + j] >= dhi) keep |= 1u << j;
    if (keep) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mask_pairs(ka, keep), qop, acc, 0, 0, 0);
    const int n = nq0 + l32;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int w = a.window[r0 + j];
        if (w < dlo || w >= dhi) continue;  // pruned or kept in the whole block
        f32x16_t part;
#pragma unroll
        for (int i = 0; i < 16; ++i) part[i] = 0.f;
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mask_pairs(ka, 1u << j), qop, part, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = mk0 + 8 * (i >> 2) + 4 * g + (i & 3);
            acc[i] += (n - m <= w) ? part[i] : 0.0f;
        }
    }
}

template <int D, bool ROPE, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(const FwdArgs a)
{
    using G = Geo<D>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave index read through readfirstlane: the compiler then knows every
    // quantity derived from it (row ranges, tile skips, window decisions) is
    // wave-uniform and branches on scalars instead of masking lanes.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // ---- work decode: XCD-contiguous, longest query tile first ----------
    const int n_qt = (a.S + kBM - 1) / kBM;
    const int n_work = n_qt * a.Hq * a.B;
    int work = blockIdx.x;
    if ((n_work & 7) == 0)
        work = (blockIdx.x & 7) * (n_work >> 3) + (blockIdx.x >> 3);
    const int bh = work / n_qt;
    const int qt = n_qt - 1 - (work - bh * n_qt);
    const int b = bh / a.Hq;
    const int hq = bh - b * a.Hq;
    const int hk = hq / (a.Hq / a.Hkv);
    const int n0 = qt * kBM;
    const int S = a.S;

    // Buffer resources per head: row m of head h starts at m * row_bytes;
    // everything at or past row S reads as zero.
    const uint32_t q_rowb = (uint32_t)a.Hq * D * 2;
    const uint32_t kv_rowb = (uint32_t)a.Hkv * D * 2;
    const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(a.q + ((size_t)b * S * a.Hq + hq) * D, (uint32_t)S * q_rowb);
    const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(a.k + ((size_t)b * S * a.Hkv + hk) * D, (uint32_t)S * kv_rowb);
    const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(a.v + ((size_t)b * S * a.Hkv + hk) * D, (uint32_t)S * kv_rowb);
    const __amdgpu_buffer_rsrc_t cs_rs = make_rsrc(a.rope_cs, ROPE ? (uint32_t)S * G::PG * 64u : 0u);
    uint16_t *og = a.o + ((size_t)b * S * a.Hq + hq) * D;

    // ---- Q tile: load, rotate, stage through LDS into B-operand registers --
    for (int u = tid; u < kBM * G::PG; u += kThreads) {
        const int row = u / G::PG, pg = u - row * G::PG;
        const uint32_t n = (uint32_t)(n0 + row);
        uint4 lo = bload16(q_rs, n * q_rowb + 16u * pg);
        uint4 hi = bload16(q_rs, n * q_rowb + (uint32_t)D + 16u * pg);
        if constexpr (ROPE) {
            float cs[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 t = bload16f(cs_rs, (n * G::PG + pg) * 64u + 16u * i);
                cs[4 * i] = t.x; cs[4 * i + 1] = t.y; cs[4 * i + 2] = t.z; cs[4 * i + 3] = t.w;
            }
            rope_rotate8(lo, hi, cs);
        }
        lds_at<uint4>(smem, G::k_off(row, pg)) = lo;
        lds_at<uint4>(smem, G::k_off(row, G::PG + pg)) = hi;
    }
    __syncthreads();
    bf16x8_t qreg[G::KCH];
#pragma unroll
    for (int kc = 0; kc < G::KCH; ++kc)
        qreg[kc] = lds_at<bf16x8_t>(smem, G::k_off(wave * kRowsPerWave + l32, kc + G::PG * g));
    __syncthreads();

    // ---- key range ----------------------------------------------------------
    const int kv_end = CAUSAL ? min(S, n0 + kBM) : S;
    const int n_tiles = (kv_end + kBN - 1) / kBN;
    const int nw0 = n0 + wave * kRowsPerWave;            // first query of this wave
    const bool wave_active = nw0 < S;
    const int wave_kv_end = CAUSAL ? min(S, nw0 + kRowsPerWave) : S;
    const float c = a.scale_log2e;

    // ---- staging ---------------------------------------------------------
    const bool k_thread = tid < G::K_UNITS;
    const int k_key = tid / G::PG, k_pg = tid - (tid / G::PG) * G::PG;
    uint4 k_lo = make_uint4(0, 0, 0, 0), k_hi = k_lo;
    float k_cs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) k_cs[i] = 0.f;
    uint4 v_r[G::V_PER_THREAD];

    // Smallest query-key distance in the work-group's tile starting at key m0:
    // a pair group whose widest window is below it is pruned everywhere in
    // the tile, so its K columns are neither loaded nor rotated.
    auto group_pruned = [&](int m0, int pg) {
        const int dmin = max(0, n0 - (m0 + kBN - 1));
        return WINDOW && a.window[8 * pg + 7] < dmin;
    };

    auto stage_load = [&](int m0) {
        if (k_thread && !group_pruned(m0, k_pg)) {
            const uint32_t m = (uint32_t)(m0 + k_key);
            k_lo = bload16(k_rs, m * kv_rowb + 16u * k_pg);
            k_hi = bload16(k_rs, m * kv_rowb + (uint32_t)D + 16u * k_pg);
            if constexpr (ROPE) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 t = bload16f(cs_rs, (m * G::PG + k_pg) * 64u + 16u * i);
                    k_cs[4 * i] = t.x; k_cs[4 * i + 1] = t.y; k_cs[4 * i + 2] = t.z; k_cs[4 * i + 3] = t.w;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < G::V_PER_THREAD; ++i) {
            const int u = tid + i * kThreads;
            if (u < G::V_UNITS) {
                const uint32_t m = (uint32_t)(m0 + u / G::CH);
                v_r[i] = bload16(v_rs, m * kv_rowb + 16u * (u % G::CH));
            }
        }
    };

    auto stage_store = [&](int buf, int m0) {
        uint8_t *ks = smem + buf * G::BUF_BYTES;
        uint8_t *vs = ks + G::K_BYTES;
        if (k_thread && !group_pruned(m0, k_pg)) {  // pruned groups are never read
            uint4 lo = k_lo, hi = k_hi;
            if constexpr (ROPE) rope_rotate8(lo, hi, k_cs);
            lds_at<uint4>(ks, G::k_off(k_key, k_pg)) = lo;
            lds_at<uint4>(ks, G::k_off(k_key, G::PG + k_pg)) = hi;
        }
#pragma unroll
        for (int i = 0; i < G::V_PER_THREAD; ++i) {
            const int u = tid + i * kThreads;
            if (u < G::V_UNITS) lds_at<uint4>(vs, G::v_off(u / G::CH, u % G::CH)) = v_r[i];
        }
    };

    // ---- state ------------------------------------------------------------
    f32x16_t acc_o[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[db][i] = 0.f;
    float m_ref = -__builtin_inff(), l_run = 0.f;

    // Transpose-read addressing for the PV A operand: within each 16-lane
    // group, source lane s reads key (s / 4) of a 4-key group at dims
    // D0 + 4 (s % 4) .. +3, with D0 = 32 db + 16 ((lane / 16) % 2).  Lane i
    // of the group then holds dim D0 + i of the 4 keys.
    const int tr_key = (lane & 15) >> 2;
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    if (n_tiles > 0) {
        stage_load(0);
        stage_store(0, 0);
    }
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const int m0 = j * kBN;
        if (j + 1 < n_tiles) stage_load(m0 + kBN);
        uint8_t *ks = smem + (j & 1) * G::BUF_BYTES;
        uint8_t *vs = ks + G::K_BYTES;

        if (wave_active && m0 < wave_kv_end) {
            // S^T = K' Q'^T for two 32-key blocks x one 32-query block.
            f32x16_t acc_s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc_s[kb][i] = 0.f;
#pragma unroll
            for (int kc = 0; kc < G::KCH; ++kc) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8_t ka = lds_at<bf16x8_t>(ks, G::k_off(kb * 32 + l32, kc + G::PG * g));
                    if constexpr (WINDOW)
                        window_chunk(a, ka, qreg[kc], acc_s[kb], kc, nw0, m0 + kb * 32, l32, g);
                    else
                        acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[kc], acc_s[kb], 0, 0, 0);
                }
            }

            // Mask: tiles crossing the diagonal or the sequence end.
            const bool need_mask = (CAUSAL && m0 + kBN - 1 > nw0) || (m0 + kBN > S);
            if (need_mask) {
                const int n = nw0 + l32;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int m = m0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                        const bool masked = (CAUSAL && m > n) || m >= S;
                        acc_s[kb][i] = masked ? -__builtin_inff() : acc_s[kb][i];
                    }
            }

            // Online softmax, one query per lane (and its mirror lane).
            float mx = acc_s[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc_s[kb][i]);
            mx = max_halves(mx);
            // Lazy rescale: move the reference max only when some row's max
            // grew by more than 2^8 in probability; the decision is per wave.
            const bool grow = (mx - m_ref) * c > kRescaleLog2;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float m_new = fmaxf(m_ref, mx);
                const float alpha = fast_exp2((m_ref - m_new) * c);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < G::DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
                m_ref = m_new;
            }
            const float mc = m_ref * c;
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(__builtin_fmaf(acc_s[kb][i], c, -mc));
                    acc_s[kb][i] = p;
                    rs += p;
                }
            l_run += rs;

            // O^T += V^T P^T over four 16-key chunks.
#pragma unroll
            for (int ch = 0; ch < kBN / 16; ++ch) {
                const int kb = ch >> 1, h8 = (ch & 1) * 8;
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(acc_s[kb][h8 + 2 * e], acc_s[kb][h8 + 2 * e + 1]);
                const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
                for (int db = 0; db < G::DB; ++db) {
                    const int dim = 32 * db + tr_dim;
                    const int key0 = 16 * ch + 4 * g + tr_key;
                    const int off0 = G::v_off(key0, dim >> 3) + ((dim & 4) << 1);
                    const int off1 = G::v_off(key0 + 8, dim >> 3) + ((dim & 4) << 1);
                    const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vs + off0));
                    const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vs + off1));
                    const uint2 u0 = __builtin_bit_cast(uint2, t0), u1 = __builtin_bit_cast(uint2, t1);
                    const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y));
                    acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf, acc_o[db], 0, 0, 0);
                }
            }
        }

        if (j + 1 < n_tiles) stage_store((j + 1) & 1, m0 + kBN);
        __syncthreads();
    }

    // ---- epilogue: O / l, bf16, store --------------------------------------
    if (!wave_active) return;
    const float inv = 1.0f / sum_halves(l_run);
    const int n = nw0 + l32;
    if (n >= S) return;
    uint16_t *orow = og + (size_t)n * a.Hq * D;
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint2 w;
            w.x = pack_bf16x2(acc_o[db][4 * r] * inv, acc_o[db][4 * r + 1] * inv);
            w.y = pack_bf16x2(acc_o[db][4 * r + 2] * inv, acc_o[db][4 * r + 3] * inv);
            *reinterpret_cast<uint2 *>(orow + db * 32 + 8 * r + 4 * g) = w;
        }
}

template <int D, bool ROPE, bool CAUSAL, bool WINDOW>
hipError_t launch_t(const FwdArgs &a, hipStream_t stream)
{
    const int n_qt = (a.S + kBM - 1) / kBM;
    const long long n_work = (long long)n_qt * a.Hq * a.B;
    if (n_work <= 0) return hipSuccess;
    hipLaunchKernelGGL((attn_fwd_kernel<D, ROPE, CAUSAL, WINDOW>), dim3((unsigned)n_work), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs &a, hipStream_t stream)
{
    const bool rope = a.rope_cs != nullptr;
    if (a.use_window) {
        // The window is defined on the causal triangle only (checked by the host API).
        if (!a.causal) return hipErrorInvalidValue;
        return rope ? launch_t<D, true, true, true>(a, stream) : launch_t<D, false, true, true>(a, stream);
    }
    if (rope)
        return a.causal ? launch_t<D, true, true, false>(a, stream) : launch_t<D, true, false, false>(a, stream);
    return a.causal ? launch_t<D, false, true, false>(a, stream) : launch_t<D, false, false, false>(a, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs &a, hipStream_t stream)
{
    if (a.D == 128) return launch_d<128>(a, stream);
    if (a.D == 64) return launch_d<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
