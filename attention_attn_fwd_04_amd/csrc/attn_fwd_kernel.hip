// attn_fwd_kernel.hip -- fused causal attention forward with RoPE at load,
// written for gfx950 (MI355X): bf16 MFMA 32x32x16 with fp32 accumulation,
// wave64, LDS staging.
//
// The computation ("Flash Attention: Causal Prefill D=128", "Online softmax:
// what must remain invariant"; "AttnFuse", section 2 and section 4.1):
//   for each query tile, walk the key tiles it may see;
//     S = Q' K'^T (Q', K' rotated by RoPE), masked on the tiles that cross
//     the causal diagonal or the end of the sequence;
//     m_new = max(m, rowmax S); alpha = exp2((m - m_new) c); P = exp2(S c - m_new c)
//     l = alpha l + rowsum P; O = alpha O + P V
//   O / l at the end, with c = scale * log2 e.
//
// gfx950 design (see the repository's design notes for the reasoning):
//  * Everything is computed transposed: S^T = K' Q'^T and O^T = V^T P^T.
//    In the 32x32 MFMA result each lane then owns one query column, so the
//    row max / row sum of the softmax are reductions inside the lane plus one
//    v_permlane32_swap, and the alpha rescale multiplies whole registers.
//    The S^T accumulator converted to bf16 is already the B operand of the
//    PV MFMA (keys permuted consistently on the V side), so P never leaves
//    registers.
//  * One MFMA k-step covers 8 complete RoPE pairs: k-index (g, e) of chunk
//    kc maps to dimension 8 kc + (D/2) g + e.  Any consistent permutation of
//    the contraction axis leaves Q'K'^T unchanged; this one keeps the two
//    halves of a NeoX pair in the same MFMA, which the per-pair window uses.
//  * A work-group of 4 waves owns 256 query rows (64 per wave, as two
//    32-row MFMA blocks), so each K/V tile staged in LDS feeds 64 rows per
//    wave read and is rotated once for 256 rows.
//  * K is rotated in registers while it is staged into LDS (each thread loads
//    both halves of its pairs, so no half swap is needed); V is transposed
//    while it is staged so the PV A operand is one 16-byte LDS read.
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

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 64;             // two 32-query MFMA blocks
constexpr int kQB = kRowsPerWave / 32;
constexpr int kBM = kWaves * kRowsPerWave;   // 256 query rows per work-group
constexpr int kBN = 64;                      // keys per iteration (two 32-key blocks)

template <int D>
struct Geo {
    static constexpr int KCH = D / 16;       // MFMA k-steps over D (8 pairs each)
    static constexpr int PG = D / 16;        // 8-pair groups per row
    static constexpr int DB = D / 32;        // 32-row blocks of O^T
    static constexpr int KP = D + 8;         // K / Q tile pitch in bf16 (16-byte pad)
    static constexpr int VP = kBN + 8;       // V^T tile pitch in bf16
    static constexpr int K_ELEMS = kBN * KP;
    static constexpr int V_ELEMS = D * VP;
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int Q_ELEMS = kBM * KP;
    static constexpr int LDS_ELEMS = (2 * BUF_ELEMS > Q_ELEMS) ? 2 * BUF_ELEMS : Q_ELEMS;
    static constexpr int K_UNITS = kBN * PG;                 // (key, pair group) units
    static constexpr int K_PER_THREAD = K_UNITS / kThreads;  // 2 (D=128) or 1 (D=64)
    static constexpr int V_UNITS = (kBN / 4) * (D / 8);      // (4 keys, 8 dims) units
    static_assert(K_UNITS % kThreads == 0, "K staging must split evenly");
    static_assert(V_UNITS <= kThreads, "one V unit per thread at most");
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

__device__ __forceinline__ uint4 load16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// Position of 4-key group q4 (keys 4 q4 .. 4 q4 + 3 of a 16-key chunk) in the
// V^T row, so that the PV A operand of lane half g is the 8 contiguous
// positions 8g .. 8g+7 holding keys {4g .. 4g+3, 8+4g .. 8+4g+3}: the key
// order of the S^T accumulator registers 8c' .. 8c'+7.
__device__ __forceinline__ int vt_group_pos(int q4) { return ((q4 & 1) << 3) | ((q4 & 2) << 1); }

// Per-pair distance window on one 32-key x 32-query block and one MFMA
// k-step kc, which holds the 8 complete pairs r = 8 kc .. 8 kc + 7 ("ATFlash
// -- Per-RoPE-Wavelength Attention Windows", "The idea": pair r contributes
// to score (n, m) only when n - m <= w[r]; w is non-decreasing in r).  The
// block's distances lie in [dlo, dhi]; causally masked cells (n < m) are
// discarded later, so the lower end is clamped at 0.
//  - every pair below dlo: the chunk is skipped (never multiplied);
//  - every pair at or above dhi: the usual MFMA;
//  - otherwise one MFMA over the pairs kept in the whole block (the others
//    zeroed in the K operand), plus, for each pair whose limit falls inside
//    [dlo, dhi), an MFMA of that pair alone added only where n - m <= w[r].
// The decisions depend only on block coordinates, so they are wave-uniform.
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

__device__ __forceinline__ void window_chunk(const FwdArgs &a, bf16x8_t ka, bf16x8_t qb_op, f32x16_t &acc,
                                             int kc, int nq0, int mk0, int l32, int g)
{
    const int dlo = max(0, nq0 - (mk0 + 31));
    const int dhi = min(nq0 + 31, a.S - 1) - mk0;  // rows past the sequence end are never stored
    const int r0 = 8 * kc;
    if (a.window[r0 + 7] < dlo) return;  // all 8 pairs pruned in this block
    if (a.window[r0] >= dhi) {           // all 8 pairs kept in this block
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb_op, acc, 0, 0, 0);
        return;
    }
    uint32_t keep = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (a.window[r0 + j] >= dhi) keep |= 1u << j;
    if (keep) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mask_pairs(ka, keep), qb_op, acc, 0, 0, 0);
    const int n = nq0 + l32;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int w = a.window[r0 + j];
        if (w < dlo || w >= dhi) continue;  // pruned or kept in the whole block
        f32x16_t part;
#pragma unroll
        for (int i = 0; i < 16; ++i) part[i] = 0.f;
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mask_pairs(ka, 1u << j), qb_op, part, 0, 0, 0);
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
    __shared__ __attribute__((aligned(16))) uint16_t smem[G::LDS_ELEMS];

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

    const size_t q_row = (size_t)a.Hq * D;
    const size_t kv_row = (size_t)a.Hkv * D;
    const uint16_t *qg = a.q + ((size_t)b * S * a.Hq + hq) * D;
    const uint16_t *kg = a.k + ((size_t)b * S * a.Hkv + hk) * D;
    const uint16_t *vg = a.v + ((size_t)b * S * a.Hkv + hk) * D;
    uint16_t *og = a.o + ((size_t)b * S * a.Hq + hq) * D;

    // ---- Q tile: load, rotate, stage through LDS into B-operand registers --
    for (int u = tid; u < kBM * G::PG; u += kThreads) {
        const int row = u / G::PG, pg = u - row * G::PG;
        const int n = n0 + row;
        uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
        if (n < S) {
            lo = load16(qg + (size_t)n * q_row + 8 * pg);
            hi = load16(qg + (size_t)n * q_row + D / 2 + 8 * pg);
            if constexpr (ROPE) {
                const float4 *cp = reinterpret_cast<const float4 *>(a.rope_cs + ((size_t)n * G::PG + pg) * 16);
                float cs[16];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float4 t = cp[i];
                    cs[4 * i] = t.x; cs[4 * i + 1] = t.y; cs[4 * i + 2] = t.z; cs[4 * i + 3] = t.w;
                }
                rope_rotate8(lo, hi, cs);
            }
        }
        *reinterpret_cast<uint4 *>(&smem[row * G::KP + 8 * pg]) = lo;
        *reinterpret_cast<uint4 *>(&smem[row * G::KP + D / 2 + 8 * pg]) = hi;
    }
    __syncthreads();
    bf16x8_t qreg[kQB][G::KCH];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int kc = 0; kc < G::KCH; ++kc)
            qreg[qb][kc] = *reinterpret_cast<const bf16x8_t *>(
                &smem[(wave * kRowsPerWave + qb * 32 + l32) * G::KP + 8 * kc + (D / 2) * g]);
    __syncthreads();

    // ---- key range ----------------------------------------------------------
    const int kv_end = CAUSAL ? min(S, n0 + kBM) : S;
    const int n_tiles = (kv_end + kBN - 1) / kBN;
    const int nw0 = n0 + wave * kRowsPerWave;          // first query of this wave
    const bool wave_active = nw0 < S;
    const int wave_kv_end = CAUSAL ? min(S, nw0 + kRowsPerWave) : S;
    const float c = a.scale_log2e;

    // ---- staging registers --------------------------------------------------
    uint4 k_lo[G::K_PER_THREAD], k_hi[G::K_PER_THREAD];
    float k_cs[G::K_PER_THREAD][16];
    uint4 v_r[4];
    const bool v_thread = tid < G::V_UNITS;
    const int v_kg = tid / (D / 8), v_dc = tid - v_kg * (D / 8);

    // Smallest query-key distance in the work-group's tile starting at key m0:
    // a pair group whose widest window is below it is pruned everywhere in
    // the tile, so its K columns are neither loaded nor rotated.
    auto group_pruned = [&](int m0, int pg) {
        const int dmin = max(0, n0 - (m0 + kBN - 1));
        return WINDOW && a.window[8 * pg + 7] < dmin;
    };

    auto stage_load = [&](int m0) {
#pragma unroll
        for (int i = 0; i < G::K_PER_THREAD; ++i) {
            const int u = tid + i * kThreads;
            const int key = u / G::PG, pg = u - key * G::PG;
            const int m = m0 + key;
            if (m < S && !group_pruned(m0, pg)) {
                k_lo[i] = load16(kg + (size_t)m * kv_row + 8 * pg);
                k_hi[i] = load16(kg + (size_t)m * kv_row + D / 2 + 8 * pg);
                if constexpr (ROPE) {
                    const float4 *cp = reinterpret_cast<const float4 *>(a.rope_cs + ((size_t)m * G::PG + pg) * 16);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float4 t = cp[j];
                        k_cs[i][4 * j] = t.x; k_cs[i][4 * j + 1] = t.y;
                        k_cs[i][4 * j + 2] = t.z; k_cs[i][4 * j + 3] = t.w;
                    }
                }
            } else {
                k_lo[i] = make_uint4(0, 0, 0, 0);
                k_hi[i] = k_lo[i];
                if constexpr (ROPE) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) k_cs[i][j] = 0.f;
                }
            }
        }
        if (v_thread) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = m0 + 4 * v_kg + j;
                v_r[j] = (m < S) ? load16(vg + (size_t)m * kv_row + 8 * v_dc) : make_uint4(0, 0, 0, 0);
            }
        }
    };

    auto stage_store = [&](int buf, int m0) {
        uint16_t *ks = smem + buf * G::BUF_ELEMS;
        uint16_t *vt = ks + G::K_ELEMS;
#pragma unroll
        for (int i = 0; i < G::K_PER_THREAD; ++i) {
            const int u = tid + i * kThreads;
            const int key = u / G::PG, pg = u - key * G::PG;
            if (group_pruned(m0, pg)) continue;  // never read by any MFMA of this tile
            uint4 lo = k_lo[i], hi = k_hi[i];
            if constexpr (ROPE) rope_rotate8(lo, hi, k_cs[i]);
            *reinterpret_cast<uint4 *>(&ks[key * G::KP + 8 * pg]) = lo;
            *reinterpret_cast<uint4 *>(&ks[key * G::KP + D / 2 + 8 * pg]) = hi;
        }
        if (v_thread) {
            // 4 keys x 8 dims -> for each dim, 4 consecutive keys (8 bytes).
            const uint32_t w0[4] = {v_r[0].x, v_r[0].y, v_r[0].z, v_r[0].w};
            const uint32_t w1[4] = {v_r[1].x, v_r[1].y, v_r[1].z, v_r[1].w};
            const uint32_t w2[4] = {v_r[2].x, v_r[2].y, v_r[2].z, v_r[2].w};
            const uint32_t w3[4] = {v_r[3].x, v_r[3].y, v_r[3].z, v_r[3].w};
            const int pos = 16 * (v_kg >> 2) + vt_group_pos(v_kg & 3);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint2 even, odd;
                even.x = (w0[w] & 0xffffu) | (w1[w] << 16);
                even.y = (w2[w] & 0xffffu) | (w3[w] << 16);
                odd.x = (w0[w] >> 16) | (w1[w] & 0xffff0000u);
                odd.y = (w2[w] >> 16) | (w3[w] & 0xffff0000u);
                const int d = 8 * v_dc + 2 * w;
                *reinterpret_cast<uint2 *>(&vt[d * G::VP + pos]) = even;
                *reinterpret_cast<uint2 *>(&vt[(d + 1) * G::VP + pos]) = odd;
            }
        }
    };

    // ---- state ------------------------------------------------------------
    f32x16_t acc_o[G::DB][kQB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc_o[db][qb][i] = 0.f;
    float m_run[kQB], l_run[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) { m_run[qb] = -__builtin_inff(); l_run[qb] = 0.f; }

    if (n_tiles > 0) {
        stage_load(0);
        stage_store(0, 0);
    }
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const int m0 = j * kBN;
        if (j + 1 < n_tiles) stage_load(m0 + kBN);
        const uint16_t *ks = smem + (j & 1) * G::BUF_ELEMS;
        const uint16_t *vt = ks + G::K_ELEMS;

        if (wave_active && m0 < wave_kv_end) {
            // S^T = K' Q'^T for two 32-key blocks x two 32-query blocks.
            f32x16_t acc_s[2][kQB];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc_s[kb][qb][i] = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int kc = 0; kc < G::KCH; ++kc) {
                    const bf16x8_t ka = *reinterpret_cast<const bf16x8_t *>(
                        &ks[(kb * 32 + l32) * G::KP + 8 * kc + (D / 2) * g]);
#pragma unroll
                    for (int qb = 0; qb < kQB; ++qb) {
                        if constexpr (WINDOW) {
                            window_chunk(a, ka, qreg[qb][kc], acc_s[kb][qb], kc,
                                         nw0 + qb * 32, m0 + kb * 32, l32, g);
                        } else {
                            acc_s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][kc], acc_s[kb][qb], 0, 0, 0);
                        }
                    }
                }
            }

            // Mask: tiles crossing the diagonal or the sequence end.
            const bool need_mask = (CAUSAL && m0 + kBN - 1 > nw0) || (m0 + kBN > S);
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    const int n = nw0 + qb * 32 + l32;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int m = m0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                            const bool masked = (CAUSAL && m > n) || m >= S;
                            if (masked) acc_s[kb][qb][i] = -__builtin_inff();
                        }
                }
            }

            // Online softmax, one query per lane (and its mirror lane).
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                float mx = acc_s[0][qb][0];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc_s[kb][qb][i]);
                mx = max_halves(mx);
                const float m_new = fmaxf(m_run[qb], mx);
                const float alpha = fast_exp2((m_run[qb] - m_new) * c);
                const float mc = m_new * c;
                float rs = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float p = fast_exp2(__builtin_fmaf(acc_s[kb][qb][i], c, -mc));
                        acc_s[kb][qb][i] = p;
                        rs += p;
                    }
                l_run[qb] = __builtin_fmaf(l_run[qb], alpha, rs);
                m_run[qb] = m_new;
#pragma unroll
                for (int db = 0; db < G::DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc_o[db][qb][i] *= alpha;
            }

            // O^T += V^T P^T over four 16-key chunks.
#pragma unroll
            for (int ch = 0; ch < kBN / 16; ++ch) {
                const int kb = ch >> 1, h8 = (ch & 1) * 8;
                bf16x8_t pf[kQB];
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = pack_bf16x2(acc_s[kb][qb][h8 + 2 * e], acc_s[kb][qb][h8 + 2 * e + 1]);
                    pf[qb] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
                }
#pragma unroll
                for (int db = 0; db < G::DB; ++db) {
                    const bf16x8_t va = *reinterpret_cast<const bf16x8_t *>(
                        &vt[(db * 32 + l32) * G::VP + 16 * ch + 8 * g]);
#pragma unroll
                    for (int qb = 0; qb < kQB; ++qb)
                        acc_o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[qb], acc_o[db][qb], 0, 0, 0);
                }
            }
        }

        if (j + 1 < n_tiles) stage_store((j + 1) & 1, m0 + kBN);
        __syncthreads();
    }

    // ---- epilogue: O / l, bf16, store --------------------------------------
    if (!wave_active) return;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const float l = sum_halves(l_run[qb]);
        const float inv = 1.0f / l;
        const int n = nw0 + qb * 32 + l32;
        if (n >= S) continue;
        uint16_t *orow = og + (size_t)n * q_row;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint2 w;
                w.x = pack_bf16x2(acc_o[db][qb][4 * r] * inv, acc_o[db][qb][4 * r + 1] * inv);
                w.y = pack_bf16x2(acc_o[db][qb][4 * r + 2] * inv, acc_o[db][qb][4 * r + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + db * 32 + 8 * r + 4 * g) = w;
            }
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
