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
    static constexpr int ROWB = D * 2;      // bytes per K / V row in LDS (unpadded)
    static constexpr int TILE_B = kBN * ROWB;             // one K or V tile
    static constexpr int NI = TILE_B / 1024;              // 1 KB direct-load instructions per tile
    static constexpr int NI_W = NI / kWaves;               // ... per wave
    static constexpr int RPI = 1024 / ROWB;               // rows per direct-load instruction
    static constexpr int KRING = 0, VRING = 3 * TILE_B;   // 3-slot rings for K and V
    static constexpr int RING_BYTES = 6 * TILE_B;
    static constexpr int QP_B = ROWB + 16;                // padded Q staging rows
    static constexpr int Q_BYTES = kBM * QP_B;
    static constexpr int LDS_BYTES = (RING_BYTES > Q_BYTES) ? RING_BYTES : Q_BYTES;
    static constexpr int K_UNITS = kBN * PG;              // (key, pair group) rotation units
    static_assert(NI % kWaves == 0, "direct-load instructions split over the waves");

    // K tiles are stored as rows of ROWB bytes whose 16-byte chunks are
    // XOR-permuted per row: 16 lanes reading one logical chunk of 16
    // consecutive rows hit 16 distinct 4-bank groups.
    static __device__ __forceinline__ int kx(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static __device__ __forceinline__ int k_off(int r, int c) { return r * ROWB + ((c ^ kx(r)) << 4); }
    // V tiles: the 4 rows x 64 bytes half a wave of ds_read_b64_tr_b16 reads
    // land on distinct banks.
    static __device__ __forceinline__ int vx(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
    static __device__ __forceinline__ int v_off(int r, int c) { return r * ROWB + ((c ^ vx(r)) << 4); }
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

// Buffer load of 16 bytes per lane straight into LDS: lane i writes
// lds_base + 16 i (lds_base wave-uniform, passed in M0).  Out-of-range lanes
// write zeros.  Issued through inline assembly so that the compiler does not
// treat these asynchronous LDS writes as pending on every later LDS read and
// barrier; the kernel waits for them itself (wait_vmcnt) before the barrier
// that publishes the tile.  One wait state separates the M0 write from its use.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, const uint8_t *lds_base)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)lds_base;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(m0)
                 : "memory", "m0");
}

// s_waitcnt on the vector-memory counter only: at most n loads of this wave
// still in flight (loads retire in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

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
    const __amdgpu_buffer_rsrc_t cs_rs = make_rsrc(a.rope_cs, ROPE ? (uint32_t)S * G::PG * 32u : 0u);
    uint16_t *og = a.o + ((size_t)b * S * a.Hq + hq) * D;

    // ---- Q tile: load, rotate, stage through LDS into B-operand registers --
    for (int u = tid; u < kBM * G::PG; u += kThreads) {
        const int row = u / G::PG, pg = u - row * G::PG;
        const uint32_t n = (uint32_t)(n0 + row);
        uint4 lo = bload16(q_rs, n * q_rowb + 16u * pg);
        uint4 hi = bload16(q_rs, n * q_rowb + (uint32_t)D + 16u * pg);
        if constexpr (ROPE) {
            const uint4 cq = bload16(cs_rs, ((n * 2u + 0) * G::PG + pg) * 16u);
            const uint4 sq = bload16(cs_rs, ((n * 2u + 1) * G::PG + pg) * 16u);
            rope_rotate8(lo, hi, cq, sq);
        }
        lds_at<uint4>(smem, row * G::QP_B + 16 * pg) = lo;
        lds_at<uint4>(smem, row * G::QP_B + 16 * (G::PG + pg)) = hi;
    }
    __syncthreads();
    bf16x8_t qreg[G::KCH];
#pragma unroll
    for (int kc = 0; kc < G::KCH; ++kc)
        qreg[kc] = lds_at<bf16x8_t>(smem, (wave * kRowsPerWave + l32) * G::QP_B + 16 * (kc + G::PG * g));
    __syncthreads();

    // ---- key range ----------------------------------------------------------
    const int kv_end = CAUSAL ? min(S, n0 + kBM) : S;
    const int T = (kv_end + kBN - 1) / kBN;              // key tiles of the work-group
    const int nw0 = n0 + wave * kRowsPerWave;            // first query of this wave
    const bool wave_active = nw0 < S;
    const int wave_kv_end = CAUSAL ? min(S, nw0 + kRowsPerWave) : S;
    const int wave_tiles = wave_active ? (wave_kv_end + kBN - 1) / kBN : 0;
    const float c = a.scale_log2e;

    // ---- ping-pong schedule ----------------------------------------------------
    // The 8 waves form two groups, A = waves 0..3 and B = waves 4..7, one wave
    // of each on every SIMD.  Each wave alternates a matrix phase (PV of the
    // previous tile, then the scores of the current tile: 32 MFMAs) and a
    // vector phase (mask, online softmax and P packing of the current tile,
    // and, with RoPE, rotating its share of the next K tile into LDS).  Two
    // barriers per period keep the groups half a period apart, so on every
    // SIMD one wave's vector phase runs under the other wave's MFMAs:
    //
    //   period j:      [Y(j-1) .. X(j)]           [X(j) .. Y(j)]
    //   group A:   PV(j-1), QK(j)              softmax(j)
    //   group B:   softmax(j-1)                PV(j-1), QK(j)
    //
    // During period j only K(j) and V(j-1) are read.  K and V tiles live in
    // 3-slot rings (tile t in slot t % 3).  V(j+1) and, without RoPE, K(j+2)
    // are fetched with buffer loads straight into LDS during period j (each
    // wave issues 1 KB per tile) and each wave waits for its own copies just
    // before barrier Y(j+1); with RoPE, K(j+1) is loaded into registers,
    // rotated and written during period j.
    const int grp = wave >> 2;
    auto kslot = [&](int t) __attribute__((always_inline)) { return smem + G::KRING + (t % 3) * G::TILE_B; };
    auto vslot = [&](int t) __attribute__((always_inline)) { return smem + G::VRING + (t % 3) * G::TILE_B; };

    // Direct loads of this wave's share of a K or V tile: instructions
    // wave + 8 i, each 1 KB = RPI rows; lane l writes chunk slot l % CH of row
    // l / CH, i.e. the global chunk (slot ^ swizzle(row)).
    const int dl_row = lane / G::CH, dl_slot = lane % G::CH;
    auto dload_k = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < G::NI_W; ++i) {
            const int ins = wave + kWaves * i;
            const int r = ins * G::RPI + dl_row;
            const uint32_t off = (uint32_t)(t * kBN + r) * kv_rowb + 16u * (uint32_t)(dl_slot ^ G::kx(r));
            dma16(k_rs, off, kslot(t) + ins * 1024);
        }
    };
    auto dload_v = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < G::NI_W; ++i) {
            const int ins = wave + kWaves * i;
            const int r = ins * G::RPI + dl_row;
            const uint32_t off = (uint32_t)(t * kBN + r) * kv_rowb + 16u * (uint32_t)(dl_slot ^ (G::vx(r) >> 0));
            dma16(v_rs, off, vslot(t) + ins * 1024);
        }
    };

    // RoPE path: each group rotates half of the K tile (thread tg of the group
    // owns unit tg + 256 grp: one key's 8-pair group).
    const int tg = tid & 255;
    const int k_unit = tg + 256 * grp;
    const int k_key = k_unit / G::PG, k_pg = k_unit % G::PG;
    uint4 k_lo = make_uint4(0, 0, 0, 0), k_hi = k_lo, k_cq = k_lo, k_sq = k_lo;

    // Smallest query-key distance in the work-group's tile starting at key m0:
    // a pair group whose widest window is below it is pruned everywhere in
    // the tile, so its K columns are neither loaded nor rotated.
    auto group_pruned = [&](int m0, int pg) __attribute__((always_inline)) {
        const int dmin = max(0, n0 - (m0 + kBN - 1));
        return WINDOW && a.window[8 * pg + 7] < dmin;
    };
    auto rload_k = [&](int m0, int unit, int key, int pg) __attribute__((always_inline)) {
        if (unit < G::K_UNITS && !group_pruned(m0, pg)) {
            const uint32_t m = (uint32_t)(m0 + key);
            k_lo = bload16(k_rs, m * kv_rowb + 16u * pg);
            k_hi = bload16(k_rs, m * kv_rowb + (uint32_t)D + 16u * pg);
            k_cq = bload16(cs_rs, ((m * 2u + 0) * G::PG + pg) * 16u);
            k_sq = bload16(cs_rs, ((m * 2u + 1) * G::PG + pg) * 16u);
        }
    };
    auto rstore_k = [&](uint8_t *ks, int m0, int unit, int key, int pg) __attribute__((always_inline)) {
        if (unit < G::K_UNITS && !group_pruned(m0, pg)) {  // pruned groups are never read
            uint4 lo = k_lo, hi = k_hi;
            rope_rotate8(lo, hi, k_cq, k_sq);
            lds_at<uint4>(ks, G::k_off(key, pg)) = lo;
            lds_at<uint4>(ks, G::k_off(key, G::PG + pg)) = hi;
        }
    };

    // ---- state ------------------------------------------------------------
    f32x16_t acc_o[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[db][i] = 0.f;
    float m_ref = -__builtin_inff(), l_run = 0.f;
    f32x16_t acc_s[2];
    bf16x8_t pf[kBN / 16];

    // Per-lane LDS byte offsets of the MFMA operands; the tile base and the
    // key-block / chunk terms are compile-time constants.
    // K operand of k-step kc: row l32 (+32 for the second key block), logical
    // chunk kc + PG g.
    int k_addr[G::KCH];
#pragma unroll
    for (int kc = 0; kc < G::KCH; ++kc) k_addr[kc] = G::k_off(l32, kc + G::PG * g);
    // PV A operand through ds_read_b64_tr_b16: within each 16-lane group,
    // source lane s reads key (s / 4) of a 4-key group at dims D0 + 4 (s % 4)
    // .. +3, D0 = 32 db + 16 ((lane / 16) % 2); lane i of the group then holds
    // dim D0 + i of those 4 keys.  Key rows 16 ch + 4 g + s / 4 (+8).
    const int tr_key = (lane & 15) >> 2;
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    int v_addr[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
        v_addr[db] = G::v_off(4 * g + tr_key, (32 * db + tr_dim) >> 3) + 2 * (tr_dim & 4);

    // S^T = K' Q'^T for the 64-key tile at m0 (two 32-key blocks).
    auto qk = [&](const uint8_t *ks, int m0) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc_s[kb][i] = 0.f;
#pragma unroll
        for (int kc = 0; kc < G::KCH; ++kc) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8_t ka = lds_at<bf16x8_t>(const_cast<uint8_t *>(ks), k_addr[kc] + kb * 32 * G::ROWB);
                if constexpr (WINDOW)
                    window_chunk(a, ka, qreg[kc], acc_s[kb], kc, nw0, m0 + kb * 32, l32, g);
                else
                    acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[kc], acc_s[kb], 0, 0, 0);
            }
        }
        if constexpr (!WINDOW) {
            // Keep the K operand reads PF steps ahead of the MFMAs that use
            // them, so the LDS latency is hidden inside this wave.
            constexpr int NM = 2 * G::KCH, PF = 4;
            __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
            for (int i = 0; i < NM - PF; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
        }
    };

    // Mask, online-softmax update and bf16 packing of P for the tile at m0.
    auto softmax = [&](int m0) __attribute__((always_inline)) {
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
#pragma unroll
        for (int ch = 0; ch < kBN / 16; ++ch) {
            const int kb = ch >> 1, h8 = (ch & 1) * 8;
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(acc_s[kb][h8 + 2 * e], acc_s[kb][h8 + 2 * e + 1]);
            pf[ch] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }
    };

    // O^T += V^T P^T over four 16-key chunks of the V tile in vs.
    auto pv = [&](const uint8_t *vs) __attribute__((always_inline)) {
#pragma unroll
        for (int ch = 0; ch < kBN / 16; ++ch) {
#pragma unroll
            for (int db = 0; db < G::DB; ++db) {
                const int off0 = v_addr[db] + 16 * ch * G::ROWB;
                const int off1 = off0 + 8 * G::ROWB;
                const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vs + off0));
                const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vs + off1));
                const uint2 u0 = __builtin_bit_cast(uint2, t0), u1 = __builtin_bit_cast(uint2, t1);
                const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y));
                acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[ch], acc_o[db], 0, 0, 0);
            }
        }
        // Two transpose reads feed each MFMA; keep them PF MFMAs ahead.
        constexpr int NM = (kBN / 16) * G::DB, PF = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
        for (int i = 0; i < NM - PF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
    };

    // Matrix phase of period j: PV(j-1), QK(j).
    auto matrix_phase = [&](int j) __attribute__((always_inline)) {
        if (j >= 1 && j - 1 < wave_tiles) pv(vslot(j - 1));
        if (j < wave_tiles) qk(kslot(j), j * kBN);
    };
    // Loads issued at the start of a wave's matrix phase in period j: direct
    // copies of V(j+1) and (no RoPE) K(j+2); with RoPE, the registers for the
    // group's share of K(j+1) (A) or K(j+2) (B), stored in its next vector phase.
    auto issue_loads = [&](int j) __attribute__((always_inline)) {
        if constexpr (ROPE) {
            const int t = j + 1 + grp;
            if (t < T) rload_k(t * kBN, k_unit, k_key, k_pg);
        }
        if (j + 1 < T) dload_v(j + 1);
        if constexpr (!ROPE) {
            if (j + 2 < T) dload_k(j + 2);
        }
    };
    // Before barrier Y(j): every load issued in period j-1 has landed.  The
    // loads still allowed in flight are the ones issued in period j (loads
    // retire in issue order).
    auto wait_before_y = [&](int j) __attribute__((always_inline)) {
        if constexpr (ROPE && WINDOW) {
            wait_vmcnt<0>();  // pruned pair groups make the per-wave load count data dependent
        } else if constexpr (ROPE) {
            constexpr int RL = 4;  // K lo/hi and the cos/sin quarters of one unit
            const bool rl = (j + 1 + grp < T) && (G::K_UNITS > 256 * grp);
            if (j + 1 < T) {
                if (rl) wait_vmcnt<RL + G::NI_W>();
                else wait_vmcnt<G::NI_W>();
            } else {
                if (rl) wait_vmcnt<RL>();
                else wait_vmcnt<0>();
            }
        } else {
            if (j + 2 < T) wait_vmcnt<2 * G::NI_W>();
            else if (j + 1 < T) wait_vmcnt<G::NI_W>();
            else wait_vmcnt<0>();
        }
    };
    auto vector_phase = [&](int ts, int tk) __attribute__((always_inline)) {
        if (ts >= 0 && ts < wave_tiles) softmax(ts * kBN);
        if constexpr (ROPE) {
            if (tk < T) rstore_k(kslot(tk), tk * kBN, k_unit, k_key, k_pg);
        }
    };

    // Prologue: K(0) (and, without RoPE, K(1)) and V(0) in LDS before Y(-1).
    if (T > 0) {
        if constexpr (ROPE) {
            rload_k(0, tid, tid / G::PG, tid % G::PG);
            rstore_k(kslot(0), 0, tid, tid / G::PG, tid % G::PG);
        } else {
            dload_k(0);
            if (T > 1) dload_k(1);
        }
        dload_v(0);
    }
    wait_vmcnt<0>();
    if constexpr (ROPE) {
        if (grp == 1 && 1 < T) rload_k(kBN, k_unit, k_key, k_pg);  // B's share of K(1)
    }
    __syncthreads();  // Y(-1)

    if (grp == 0) {
        for (int j = 0; j <= T; ++j) {
            issue_loads(j);
            matrix_phase(j);
            __syncthreads();  // X(j)
            vector_phase(j, j + 1);
            wait_before_y(j);
            __syncthreads();  // Y(j)
        }
    } else {
        for (int j = 0; j <= T; ++j) {
            vector_phase(j - 1, j + 1);
            __syncthreads();  // X(j)
            issue_loads(j);
            matrix_phase(j);
            wait_before_y(j);
            __syncthreads();  // Y(j)
        }
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
