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
//    wave, and walks the key tiles in lock step, one barrier per tile.  Each
//    wave software-pipelines its own work: the scores of tile i are computed
//    by MFMAs while the same wave's VALU turns tile i-1's scores into P, and
//    the PV MFMAs of tile i-1 run while the VALU rotates part of tile i+1.
//    On gfx950 VALU work overlaps MFMAs well inside one wave's instruction
//    stream (a few VALU operations and one or two exp per 32x32x16 MFMA come
//    for free), and poorly when one wave only issues MFMAs while the other
//    wave on the SIMD only issues VALU.
//  * K, V (and with RoPE the cos/sin rows of each key tile) stream into LDS
//    rings through buffer loads that write LDS directly (no registers).  With
//    RoPE each K tile is then rotated in place, once for all 256 rows, each
//    thread rotating one (key, 8-pair group) unit.
//  * All global loads are buffer loads: rows past the sequence end read as
//    zero, so staging has no lane-divergent branches.
//  * LDS tiles are XOR-swizzled in 16-byte chunks so the MFMA operand reads,
//    the transpose reads and the rotation's reads and writes are free of bank
//    conflicts without padding.
//  * Scores leave the MFMAs in the exp2 domain, already shifted: Q' is kept
//    multiplied by c = scale log2 e, and each QK accumulator chain starts
//    from -m_ref, so P = exp2(accumulator) needs no multiply-add.
//  * The softmax rescale is lazy: P is computed against the running reference
//    m_ref (set from the wave's first tile); only when a lane's partial row
//    sum of P exceeds 2^14 (or is not finite) is the tile's max taken, m_ref
//    raised, O and l rescaled, and P recomputed.  So every P is at most
//    2^14, the common tile needs no max pass, and the 64 multiplies of O are
//    rare.
//  * Key tiles are visited from 0 upwards; the masked tiles are the last
//    ones.  Query tiles are issued longest first within bands of heads, and
//    the block index is remapped so a band's tiles run on one XCD (shared
//    L2 for its K/V).
//  * The same per-tile code also runs persistently ("Flash Attention: Causal
//    Prefill D=128", "Step 4"): one work-group per compute unit walks the
//    query tiles of its bin in a task list that the host built (cost-balanced
//    bins, heads grouped per XCD) and checked.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_gfx950.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;  // 256 query rows per work-group
constexpr int kBN = 64;                     // keys per iteration (two 32-key blocks)
constexpr float kLazyMaxSum = 16384.0f;     // lazy rescale: partial row sums of P stay <= 2^14
constexpr int kBandTiles = 64;              // query tiles per band of heads in the work order

// CS: the tiles carry a cos/sin ring (keys rotated in LDS).
template <int D, bool CS>
struct Geo {
    static constexpr int KCH = D / 16;      // MFMA k-steps over D (8 pairs each)
    static constexpr int PG = D / 16;       // 8-pair groups per row
    static constexpr int DB = D / 32;       // 32-row blocks of O^T
    static constexpr int CH = D / 8;        // 16-byte chunks per row
    static constexpr int ROWB = D * 2;      // bytes per K / V / cos-sin row in LDS (unpadded)
    static constexpr int TILE_B = kBN * ROWB;             // one K, V or cos/sin tile
    static constexpr int NI = TILE_B / 1024;              // 1 KB direct-load instructions per tile
    static constexpr int NI_W = NI / kWaves;               // ... per wave
    static constexpr int RPI = 1024 / ROWB;               // rows per direct-load instruction
    // Rings: K tile t in slot t % 4, V and cos/sin tiles in slot t % 3.
    static constexpr int KSLOTS = 4, VSLOTS = 3, CSLOTS = 3;
    static constexpr int KRING = 0;
    static constexpr int VRING = KSLOTS * TILE_B;
    static constexpr int CRING = VRING + VSLOTS * TILE_B;
    static constexpr int RING_BYTES = CRING + (CS ? CSLOTS * TILE_B : 0);
    static constexpr int QP_B = ROWB + 16;                // padded Q staging rows
    static constexpr int Q_BYTES = kBM * QP_B;
    static constexpr int LDS_BYTES = (RING_BYTES > Q_BYTES) ? RING_BYTES : Q_BYTES;
    static constexpr int K_UNITS = kBN * PG;              // (key, pair group) rotation units
    static_assert(NI % kWaves == 0, "direct-load instructions split over the waves");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS per work-group");

    // K (and cos/sin) tiles are stored as rows of ROWB bytes whose 16-byte
    // chunks are XOR-permuted per row: 16 lanes reading one logical chunk of
    // 16 consecutive rows hit 16 distinct 4-bank groups.
    static constexpr __host__ __device__ int kx(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static constexpr __host__ __device__ int k_off(int r, int c) { return r * ROWB + ((c ^ kx(r)) << 4); }
    // V tiles: the 4 rows x 64 bytes half a wave of ds_read_b64_tr_b16 reads
    // land on distinct banks.
    static constexpr __host__ __device__ int vx(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
    static constexpr __host__ __device__ int v_off(int r, int c) { return r * ROWB + ((c ^ vx(r)) << 4); }
    // The kernel forms the operand offsets of every chunk / block from one per
    // lane by an XOR below bit 10, applied after adding a 1 KiB aligned slot
    // base (which leaves those bits as they are): the identities hold for
    // every row of a tile.
    static constexpr bool offsets_by_xor() {
        for (int r = 0; r < kBN; ++r)
            for (int g = 0; g < 2; ++g) {
                for (int kc = 0; kc < KCH; ++kc)
                    if (k_off(r, kc + PG * g) != (k_off(r, PG * g) ^ (kc << 4)) || (kc << 4) >= 1024) return false;
                for (int t = 0; t < 4; ++t)
                    for (int db = 0; db < DB; ++db)
                        if (v_off(r, 4 * db + t) != (v_off(r, t) ^ (db << 6)) || (db << 6) >= 1024) return false;
            }
        return TILE_B % 1024 == 0 && KSLOTS * TILE_B % 1024 == 0;
    }
    static_assert(offsets_by_xor(), "operand offsets by XOR from one base");
};

// PERSIST false: one work-group per query tile (work decoded from the block
// index).  PERSIST true: one work-group per compute unit, running the query
// tiles of its bin in a host-built task list, one after the other.
// ROPE: the query is rotated at load.  ROPE_K: each key tile is rotated in
// LDS as well (fused RoPE); without it the keys arrive rotated (a separate
// pass rotated them) and the cos/sin stream and its ring are not used.
template <int D, bool ROPE, bool ROPE_K, bool CAUSAL, bool WINDOW, bool PERSIST>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(const FwdArgs a)
{
    static_assert(ROPE || !ROPE_K, "keys are rotated in the kernel only with the query");
    using G = Geo<D, ROPE_K>;
    // (1 KiB aligned: so are the ring slots, whose bases then leave the low 10
    // bits of an operand address, where the chunk XOR acts, unchanged)
    __shared__ __attribute__((aligned(1024))) uint8_t smem[G::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave index read through readfirstlane: the compiler then knows every
    // quantity derived from it (row ranges, tile skips, window decisions) is
    // wave-uniform and branches on scalars instead of masking lanes.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // One query tile (b, hq, qt): everything below runs per tile.
    auto tile = [&](const int b, const int hq, const int qt) __attribute__((always_inline)) {
        const int hk = __builtin_amdgcn_readfirstlane(hq / (a.Hq / a.Hkv));
        const int n0 = qt * kBM;
        const int S = a.S;

        // Buffer resources per head: row m of head h starts at m * row_bytes;
        // everything at or past row S reads as zero.
        const uint32_t q_rowb = (uint32_t)a.Hq * D * 2;
        const uint32_t kv_rowb = (uint32_t)a.Hkv * D * 2;
        const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(a.q + ((size_t)b * S * a.Hq + hq) * D, (uint32_t)S * q_rowb);
        const __amdgpu_buffer_rsrc_t cs_rs = make_rsrc(a.rope_cs, ROPE ? (uint32_t)S * G::ROWB : 0u);
        // K, V and the cos/sin table for the direct-to-LDS loads.
        const u32x4_t k_rs = make_desc(a.k + ((size_t)b * S * a.Hkv + hk) * D, (uint32_t)S * kv_rowb);
        const u32x4_t v_rs = make_desc(a.v + ((size_t)b * S * a.Hkv + hk) * D, (uint32_t)S * kv_rowb);
        const u32x4_t cs_desc = make_desc(a.rope_cs, ROPE_K ? (uint32_t)S * G::ROWB : 0u);
        uint16_t *og = a.o + ((size_t)b * S * a.Hq + hq) * D;

        // ---- Q tile: load, rotate, stage through LDS into B-operand registers --
        static_assert((kBM * G::PG) % kThreads == 0, "whole Q staging rounds");
#pragma unroll
        for (int it = 0; it < kBM * G::PG / kThreads; ++it) {
            const int u = tid + it * kThreads;
            const int row = u / G::PG, pg = u - row * G::PG;
            const uint32_t n = (uint32_t)(n0 + row);
            uint4 lo = bload16(q_rs, n * q_rowb + 16u * pg);
            uint4 hi = bload16(q_rs, n * q_rowb + (uint32_t)D + 16u * pg);
            // Q' is kept multiplied by c = scale log2 e (rounded to bf16 once,
            // after the rotation): the MFMAs then deliver scores in the exp2
            // domain and P needs no multiply-add.
            if constexpr (ROPE) {
                const uint4 cq = bload16(cs_rs, n * G::ROWB + 16u * pg);
                const uint4 sq = bload16(cs_rs, n * G::ROWB + 16u * (G::PG + pg));
                rope_rotate8_scaled(lo, hi, cq, sq, a.scale_log2e);
            } else {
                lo = scale_bf16x8(lo, a.scale_log2e);
                hi = scale_bf16x8(hi, a.scale_log2e);
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
        // Per-pair window table, read in place in the kernel-argument segment (the
        // kernel's only argument, at offset 0) so that runtime-indexed reads are
        // scalar loads rather than reads of a private copy of the arguments.
        typedef __attribute__((address_space(4))) const int32_t kconst_i32;
        kconst_i32 *wtab = (kconst_i32 *)((__attribute__((address_space(4))) const char *)
                                              __builtin_amdgcn_kernarg_segment_ptr() + __builtin_offsetof(FwdArgs, window));

        // ---- schedule -----------------------------------------------------------
        // Iteration i (all waves, i = 0 .. T) does, for this wave's rows:
        //   block 1:  S(i) = K'(i) Q'^T (MFMA)  ||  rotate this thread's unit of K(i+1)
        //   block 2:  O^T += V(i-1)^T P(i-1)^T  ||  P(i) = 2^(S(i) c - m c) (VALU)
        // then one barrier.  Loads go straight into LDS: in iteration i, K(i+3)
        // and its cos/sin rows (slot (i+3) % 4, % 3) and V(i+1) (slot (i+1) % 3).
        // Each wave waits for its own loads of iteration i-1 before the barrier
        // that ends iteration i, so K(t) is raw in LDS from the end of iteration
        // t-2, rotated in t-1, read in t; V(t) is visible from iteration t+1 on.
        auto kslot = [&](int t) __attribute__((always_inline)) { return smem + G::KRING + (t & 3) * G::TILE_B; };
        auto vslot = [&](int t) __attribute__((always_inline)) { return smem + G::VRING + (t % 3) * G::TILE_B; };
        auto cslot = [&](int t) __attribute__((always_inline)) { return smem + G::CRING + (t % 3) * G::TILE_B; };
        // The same slots as 32-bit LDS addresses, for the direct loads.
        const uint32_t smem32 = lds_addr(smem);
        auto kslot32 = [&](int t) __attribute__((always_inline)) { return smem32 + (uint32_t)(G::KRING + (t & 3) * G::TILE_B); };
        auto vslot32 = [&](int t) __attribute__((always_inline)) { return smem32 + (uint32_t)(G::VRING + (t % 3) * G::TILE_B); };
        auto cslot32 = [&](int t) __attribute__((always_inline)) { return smem32 + (uint32_t)(G::CRING + (t % 3) * G::TILE_B); };

        // Direct loads of this wave's share of a tile: instructions wave + 8 i,
        // each 1 KB = RPI rows; lane l writes chunk slot l % CH of row l / CH, i.e.
        // the global chunk (slot ^ swizzle(row)).  Rows are keys (K, V) or
        // positions (the cos/sin table, whose rows have the K row geometry).
        // A load's byte offset is the lane's part (row within the tile, swizzled
        // chunk), computed once here, plus the tile's row offset, a wave-uniform
        // product added per load: one vector add instead of a 32-bit multiply.
        const int dl_row = lane / G::CH, dl_slot = lane % G::CH;
        uint32_t lane_v[G::NI_W], lane_k[G::NI_W], lane_c[G::NI_W];
#pragma unroll
        for (int j = 0; j < G::NI_W; ++j) {
            const int r = (wave + kWaves * j) * G::RPI + dl_row;
            lane_v[j] = (uint32_t)r * kv_rowb + 16u * (uint32_t)(dl_slot ^ G::vx(r));
            lane_k[j] = (uint32_t)r * kv_rowb + 16u * (uint32_t)(dl_slot ^ G::kx(r));
            lane_c[j] = (uint32_t)r * (uint32_t)G::ROWB + 16u * (uint32_t)(dl_slot ^ G::kx(r));
        }
        auto dload = [&](u32x4_t rs, uint32_t rowb, uint32_t dst, int t, const uint32_t (&lane_off)[G::NI_W])
            __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < G::NI_W; ++j)
                dma16(rs, (uint32_t)(t * kBN) * rowb + lane_off[j], dst + (uint32_t)((wave + kWaves * j) * 1024));
        };
        auto dload_k = [&](int t) __attribute__((always_inline)) {
            dload(k_rs, kv_rowb, kslot32(t), t, lane_k);
            if constexpr (ROPE_K) dload(cs_desc, (uint32_t)G::ROWB, cslot32(t), t, lane_c);
        };
        auto dload_v = [&](int t) __attribute__((always_inline)) { dload(v_rs, kv_rowb, vslot32(t), t, lane_v); };
        // Loads of iteration i, one 1 KB instruction per step: V(i+1), K(i+3)
        // and, with RoPE, the cos/sin rows of K(i+3).  They are issued in every
        // iteration: tiles past the end read as zeros into slots that are free
        // and never read again, which keeps the wait counts constant.
        constexpr int NDMA = G::NI_W * (ROPE_K ? 3 : 2);
        auto dma_step = [&](int i, int j) __attribute__((always_inline)) {
            const int which = j / G::NI_W, jj = j % G::NI_W;
            const uint32_t dst = (uint32_t)((wave + kWaves * jj) * 1024);
            if (which == 0)
                dma16(v_rs, (uint32_t)((i + 1) * kBN) * kv_rowb + lane_v[jj], vslot32(i + 1) + dst);
            else if (which == 1)
                dma16(k_rs, (uint32_t)((i + 3) * kBN) * kv_rowb + lane_k[jj], kslot32(i + 3) + dst);
            else
                dma16(cs_desc, (uint32_t)((i + 3) * kBN) * (uint32_t)G::ROWB + lane_c[jj], cslot32(i + 3) + dst);
        };

        // RoPE: lane l of wave w rotates unit (key l, pair group w) of
        // each K tile in place.  A pair group whose widest window is below the
        // smallest query-key distance in the work-group's tile is pruned
        // everywhere in it and is never read, so it is not rotated.
        static_assert(kBN == 64, "one rotation pair group per wave");
        const int r_key = lane, r_pg = wave;
        const int w_rot = WINDOW ? wtab[8 * r_pg + 7] : 0;   // widest window of the pair group
        auto rotate_k = [&](int t) __attribute__((always_inline)) {
            if constexpr (ROPE_K) {
                if (wave * 64 < G::K_UNITS) {   // K_UNITS is a multiple of 64: wave-uniform
                    if constexpr (WINDOW) {
                        const int dmin = max(0, n0 - (t * kBN + kBN - 1));
                        if (w_rot < dmin) return;
                    }
                    uint8_t *ks = kslot(t);
                    const uint8_t *cs = cslot(t);
                    const int o_lo = G::k_off(r_key, r_pg), o_hi = G::k_off(r_key, G::PG + r_pg);
                    uint4 lo = lds_at<uint4>(ks, o_lo), hi = lds_at<uint4>(ks, o_hi);
                    const uint4 cq = lds_at<uint4>(const_cast<uint8_t *>(cs), o_lo);
                    const uint4 sq = lds_at<uint4>(const_cast<uint8_t *>(cs), o_hi);
                    rope_rotate8(lo, hi, cq, sq);
                    lds_at<uint4>(ks, o_lo) = lo;
                    lds_at<uint4>(ks, o_hi) = hi;
                }
            }
        };

        // ---- state ------------------------------------------------------------
        f32x16_t acc_o[G::DB];
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc_o[db][i] = 0.f;
        // Softmax reference in the exp2 domain: every QK MFMA chain starts from
        // -m_ref in all 16 accumulator entries, so the accumulator holds
        // s c - m_ref and P is exp2 of it directly.  m_ref is set from the first
        // tile's max.
        float m_ref = 0.f, l_run = 0.f;
        f32x16_t sc[2];                        // scores of one tile (S^T, two 32-key blocks)
        bf16x8_t pf_a[kBN / 16], pf_b[kBN / 16];   // P of two consecutive tiles as PV B operands

        // Per-lane LDS byte offsets of the MFMA operands within a tile.
        // K operand of k-step kc: row l32 (+32 for the second key block), logical
        // chunk kc + PG g.
        // The chunk index enters k_off only through an XOR on bits disjoint from
        // the row's, and kc < PG: k_off(l32, kc + PG g) == k_addr0 ^ (kc << 4).
        // One base per lane instead of KCH offsets kept through the loop.
        const int k_addr0 = G::k_off(l32, G::PG * g);
        // PV A operand through ds_read_b64_tr_b16: within each 16-lane group,
        // source lane s reads key (s / 4) of a 4-key group at dims D0 + 4 (s % 4)
        // .. +3, D0 = 32 db + 16 ((lane / 16) % 2); lane i of the group then holds
        // dim D0 + i of those 4 keys.  Key rows 16 ch + 4 g + s / 4 (+8).
        const int tr_key = (lane & 15) >> 2;
        const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        // Likewise v_off(r, 4 db + t) == v_off(r, t) ^ (db << 6) for t < 4:
        // V operand offset of block db = v_addr0 ^ (db << 6).
        const int v_addr0 = G::v_off(4 * g + tr_key, tr_dim >> 3) + 2 * (tr_dim & 4);

        // Causal / sequence-end mask of tile t, needed only on the tiles that
        // cross the wave's first row or the end of the sequence.
        auto need_mask = [&](int t) __attribute__((always_inline)) {
            const int m0 = t * kBN;
            return (CAUSAL && m0 + kBN - 1 > nw0) || (m0 + kBN > S);
        };
        auto mask_tile = [&](f32x16_t (&s)[2], int t) __attribute__((always_inline)) {
            const int m0 = t * kBN;
            const int n = nw0 + l32;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = m0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                    const bool masked = (CAUSAL && m > n) || m >= S;
                    s[kb][i] = masked ? -__builtin_inff() : s[kb][i];
                }
        };

        // P = 2^(s c - m_ref) of one (masked) tile (s the accumulator: already
        // shifted), packed into pf; returns the lane's partial row sum (of the
        // fp32 P, before the bf16 rounding for the PV operand).
        auto exp_tile = [&](const f32x16_t (&s)[2], bf16x8_t (&pf)[kBN / 16]) __attribute__((always_inline)) {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int ch = 0; ch < kBN / 16; ++ch) {
                const int kb = ch >> 1, h8 = (ch & 1) * 8;
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] = fast_exp2(s[kb][h8 + e]);
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
                    r0 += p[2 * e];
                    r1 += p[2 * e + 1];
                }
                pf[ch] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
            }
            return r0 + r1;
        };
        auto tile_max = [&](const f32x16_t (&s)[2]) __attribute__((always_inline)) {
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
            return max_halves(mx);
        };
        // Exact path: move m_ref up by the tile's excess d over it, rescale O and
        // l by 2^-d, redo P.
        auto rescale_exp_tile = [&](f32x16_t (&s)[2], bf16x8_t (&pf)[kBN / 16]) __attribute__((always_inline)) {
            const float d = fmaxf(tile_max(s), 0.f);
            const float alpha = fast_exp2(-d);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
            m_ref += d;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] -= d;
            return exp_tile(s, pf);
        };
        // The wave's first tile (m_ref = 0, O = l = 0): m_ref becomes the tile's
        // row max (0 for padding rows past S, which see no key).
        auto first_exp_tile = [&](f32x16_t (&s)[2], bf16x8_t (&pf)[kBN / 16]) __attribute__((always_inline)) {
            const float mx = tile_max(s);
            m_ref = (mx == -__builtin_inff()) ? 0.f : mx;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] -= m_ref;
            return exp_tile(s, pf);
        };

        // ---- per-pair window ("ATFlash -- Per-RoPE-Wavelength Attention Windows",
        // "The idea": pair r contributes to score (n, m) only when n - m <= w[r]) --
        // Lane r holds w[r] (pairs past D/2: never pruned).  Comparing it with a
        // block's distance bounds and taking the ballot gives, in scalar
        // registers, the pairs pruned on the whole block, the pairs kept on the
        // whole block and, in between, the pairs whose limit falls inside it.
        const int w_lane = (WINDOW && lane < D / 2) ? wtab[lane] : INT_MAX;
        // The partial pairs of one 32-key block: each by an MFMA of that pair
        // alone, counted only where n - m <= w[r].  Wave-uniform branches.
        auto window_partial = [&](f32x16_t &acc, uint64_t bits, uint32_t kbase_blk, int m0) __attribute__((always_inline)) {
            const int n = nw0 + l32;
            while (bits) {
                const int r = __builtin_ctzll(bits);
                bits &= bits - 1;
                const int kc = r >> 3, j = r & 7;
                const int w = __builtin_amdgcn_readlane(w_lane, r);
                const bf16x8_t ka = mask_pairs(*(const lds_bf16x8_t *)lds_ptr(kbase_blk + (uint32_t)G::k_off(l32, kc + G::PG * g)),
                                               1u << j);
                f32x16_t one{};
#pragma unroll
                for (int c2 = 0; c2 < G::KCH; ++c2)   // the Q operand register of chunk kc
                    if (kc == c2) one = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[c2], f32x16_t{}, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int m = m0 + 8 * (e >> 2) + 4 * g + (e & 3);
                    acc[e] += (n - m <= w) ? one[e] : 0.0f;
                }
            }
        };

        // ---- the softmax chain of one tile -------------------------------------
        // Step e (0 .. 17): the exps of pair e (scores 2e, 2e+1 in P order:
        // chunk e / 4, word e % 4; pairs 0-7 are key block 0), the bf16 packing
        // of pair e-1, the fp32 row-sum adds of pair e-2, so that no instruction
        // waits on the one just before it.  The steps are spread over MFMA
        // segments of block 2, or of both blocks; the empty volatile asm
        // statements pin each step before the next fence (without them the
        // arithmetic is sunk below the last MFMA).
        constexpr int NSTEP = 18;
        float xr[4];
        uint32_t xw[16];
        float xpe[16][2];
        auto exp_step = [&](int e) __attribute__((always_inline)) {
            if (e < 16) {
                const int ch = e >> 2, kb = ch >> 1, h = (ch & 1) * 8 + 2 * (e & 3);
                xpe[e][0] = fast_exp2(sc[kb][h]);
                xpe[e][1] = fast_exp2(sc[kb][h + 1]);
                asm volatile("" : "+v"(xpe[e][0]), "+v"(xpe[e][1]));
            }
            if (e >= 1 && e <= 16) {
                xw[e - 1] = pack_bf16x2(xpe[e - 1][0], xpe[e - 1][1]);
                asm volatile("" : "+v"(xw[e - 1]));
            }
            if (e >= 2) {
                xr[(e - 2) & 1] += xpe[e - 2][0];
                xr[2 + ((e - 2) & 1)] += xpe[e - 2][1];
                asm volatile("" : "+v"(xr[(e - 2) & 1]), "+v"(xr[2 + ((e - 2) & 1)]));
            }
        };

        // ---- the two steady-state blocks, hand-interleaved ---------------------
        // Each block is a sequence of segments, one per MFMA, fenced with
        // sched_barrier(0) so that the issue order is the one written here: the
        // LDS reads of the MFMA PF segments ahead, the MFMA, then this segment's
        // share of the VALU work.  The compiler still inserts the waits.
        constexpr int NM1 = 2 * G::KCH;                 // QK MFMAs per tile
        constexpr int NM2 = (kBN / 16) * G::DB;         // PV MFMAs per tile
        constexpr int PF = 3;

        // Block 1: S(i) = K'(i) Q'^T; with ROT, rotation of this thread's unit of
        // K(i+1) spread over the MFMAs (one 32-bit word of each half at a time).
        // The unit's LDS reads go out after the first K operand reads (LDS
        // requests complete in order: issued first, they would hold up the
        // first MFMA) and are first used a few MFMAs later.
        // EXPS: the tile's scores need no mask, and the chain of key block 0
        // runs first (after both chains' first MFMAs, so that the -m_ref seed
        // is dead after two), finishing at MFMA KCH; the first KCH - 2 softmax
        // steps (block 2's E1), on block 0's scores, then go one each with MFMAs
        // KCH + 2 .. 2 KCH - 1.  The
        // sums are those of the alternating order (each chain adds its chunks
        // in the same order), so the outputs do not depend on EXPS.
        auto block1 = [&](auto rot_c, auto exps_c, int i) __attribute__((always_inline)) {
            constexpr bool ROT = decltype(rot_c)::value;
            constexpr bool EXPS = decltype(exps_c)::value;
            // MFMA k: key block kb_of(k), chunk kc_of(k)
            auto kb_of = [&](int k) __attribute__((always_inline)) {
                return EXPS ? (k == 1 || k > G::KCH ? 1 : 0) : (k & 1);
            };
            auto kc_of = [&](int k) __attribute__((always_inline)) {
                return EXPS ? (k <= 1 ? 0 : k <= G::KCH ? k - 1 : k - G::KCH) : (k >> 1);
            };
            f32x16_t minit;   // -m_ref: the start of both QK chains
#pragma unroll
            for (int e = 0; e < 16; ++e) minit[e] = -m_ref;
            const uint32_t kbase = lds_addr(kslot(i));
            uint32_t kp[G::KCH];
#pragma unroll
            for (int kc = 0; kc < G::KCH; ++kc) {
                kp[kc] = (kbase + (uint32_t)k_addr0) ^ (uint32_t)(kc << 4);
                asm("" : "+v"(kp[kc]));
            }
            bf16x8_t kop[NM1];
            auto kread = [&](int k) __attribute__((always_inline)) {
                kop[k] = *(const lds_bf16x8_t *)(lds_ptr(kp[kc_of(k)]) + kb_of(k) * 32 * G::ROWB);
            };
            if constexpr (EXPS) {
#pragma unroll
                for (int q = 0; q < 4; ++q) xr[q] = 0.f;
            }
            uint4 rlo, rhi, rcq, rsq;
            uint8_t *rks = kslot(i + 1);
            const int o_lo = G::k_off(r_key, r_pg), o_hi = G::k_off(r_key, G::PG + r_pg);
#pragma unroll
            for (int k = 0; k < PF; ++k) kread(k);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NM1; ++k) {
                if (k + PF < NM1) kread(k + PF);
                if constexpr (ROT) {
                    if (k == 0) {
                        const uint8_t *rcs = cslot(i + 1);
                        rlo = lds_at<uint4>(rks, o_lo);
                        rhi = lds_at<uint4>(rks, o_hi);
                        rcq = lds_at<uint4>(const_cast<uint8_t *>(rcs), o_lo);
                        rsq = lds_at<uint4>(const_cast<uint8_t *>(rcs), o_hi);
                    }
                }
                {
                    constexpr int EVERY_DMA = (NM1 - 2) / NDMA;
                    if (k % EVERY_DMA == 1 && k / EVERY_DMA < NDMA) dma_step(i, k / EVERY_DMA);
                }
                const int kc = kc_of(k), kb = kb_of(k);
                if (kc == 0) {
                    sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[k], qreg[kc], minit, 0, 0, 0);
                } else {
                    sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[k], qreg[kc], sc[kb], 0, 0, 0);
                }
                if constexpr (EXPS) {
                    if (k >= G::KCH + 2) exp_step(k - (G::KCH + 2));
                }
                if constexpr (ROT) {
                    constexpr int R0 = NM1 / 4 + 1, RS = (NM1 - 1 - R0) / 3;   // words at R0 + RS r
                    if (k >= R0 && (k - R0) % RS == 0 && (k - R0) / RS < 4) {
                        const int wr = (k - R0) / RS;
                        uint32_t &l = (wr == 0) ? rlo.x : (wr == 1) ? rlo.y : (wr == 2) ? rlo.z : rlo.w;
                        uint32_t &h = (wr == 0) ? rhi.x : (wr == 1) ? rhi.y : (wr == 2) ? rhi.z : rhi.w;
                        uint32_t cw = (wr == 0) ? rcq.x : (wr == 1) ? rcq.y : (wr == 2) ? rcq.z : rcq.w;
                        uint32_t sw = (wr == 0) ? rsq.x : (wr == 1) ? rsq.y : (wr == 2) ? rsq.z : rsq.w;
                        rope_rotate_word(l, h, cw, sw);
                        asm volatile("" : "+v"(l), "+v"(h));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (ROT) {
                lds_at<uint4>(rks, o_lo) = rlo;
                lds_at<uint4>(rks, o_hi) = rhi;
            }
        };

        // Block 1 with a window.  Per 32-key block, wprune / wkeep mark the pairs
        // pruned / kept on the whole block.  The 8-pair chunks of a tile then fall
        // into: chunks below NS, pruned on both blocks (no MFMA); chunks NS and
        // NS + 1, computed over each block's kept pairs (masked operand); chunks
        // from NS + 2 on, kept on both blocks (plain MFMA).  NS < 0: every chunk
        // masked.  NS is a template constant, so each variant is a fixed sequence
        // of MFMAs with this iteration's loads and rotation spread over it.
        auto block1w = [&](auto rot_c, auto ns_c, int i, const uint64_t (&wprune)[2], const uint64_t (&wkeep)[2])
            __attribute__((always_inline)) {
            constexpr bool ROT = decltype(rot_c)::value;
            constexpr int NS = decltype(ns_c)::value;
            constexpr bool GEN = NS < 0;
            constexpr int C0 = GEN ? 0 : NS;                  // first chunk computed
            constexpr int NM = 2 * (G::KCH - C0);             // MFMAs of this variant
            static_assert(NM >= 4, "rotation words spread over the MFMAs");
            f32x16_t minit;   // -m_ref: the start of both QK chains
#pragma unroll
            for (int e = 0; e < 16; ++e) minit[e] = -m_ref;
            const uint32_t kbase = lds_addr(kslot(i));
            uint32_t kp[G::KCH];
#pragma unroll
            for (int kc = 0; kc < G::KCH; ++kc) {
                kp[kc] = (kbase + (uint32_t)k_addr0) ^ (uint32_t)(kc << 4);
                asm("" : "+v"(kp[kc]));
            }
            bf16x8_t kop[NM];
            auto kread = [&](int k) __attribute__((always_inline)) {
                kop[k] = *(const lds_bf16x8_t *)(lds_ptr(kp[C0 + (k >> 1)]) + (k & 1) * 32 * G::ROWB);
            };
            uint4 rlo, rhi, rcq, rsq;
            uint8_t *rks = kslot(i + 1);
            const int o_lo = G::k_off(r_key, r_pg), o_hi = G::k_off(r_key, G::PG + r_pg);
            WordMask msk[2][2];   // chunks NS, NS + 1 of each block
            if constexpr (!GEN) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 2; ++j) msk[kb][j] = pair_mask(wkeep[kb], NS + j);
            }
#pragma unroll
            for (int k = 0; k < PF && k < NM; ++k) kread(k);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NM; ++k) {
                if (k + PF < NM) kread(k + PF);
                if constexpr (ROT) {
                    if (k == 0) {   // after the first operand reads, as in block 1
                        const uint8_t *rcs = cslot(i + 1);
                        rlo = lds_at<uint4>(rks, o_lo);
                        rhi = lds_at<uint4>(rks, o_hi);
                        rcq = lds_at<uint4>(const_cast<uint8_t *>(rcs), o_lo);
                        rsq = lds_at<uint4>(const_cast<uint8_t *>(rcs), o_hi);
                    }
                }
#pragma unroll
                for (int j = 0; j < NDMA; ++j)
                    if (j * NM / NDMA == k) dma_step(i, j);
                const int kc = C0 + (k >> 1), kb = k & 1;
                bf16x8_t op = kop[k];
                if constexpr (GEN) op = apply_mask(op, pair_mask(wkeep[kb], kc));
                else if (kc < NS + 2) op = apply_mask(op, msk[kb][kc - NS]);
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qreg[kc], kc == C0 ? minit : sc[kb], 0, 0, 0);
                if constexpr (ROT) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if ((r + 1) * NM / 4 - 1 == k) {
                            uint32_t &l = (r == 0) ? rlo.x : (r == 1) ? rlo.y : (r == 2) ? rlo.z : rlo.w;
                            uint32_t &h = (r == 0) ? rhi.x : (r == 1) ? rhi.y : (r == 2) ? rhi.z : rhi.w;
                            const uint32_t cw = (r == 0) ? rcq.x : (r == 1) ? rcq.y : (r == 2) ? rcq.z : rcq.w;
                            const uint32_t sw = (r == 0) ? rsq.x : (r == 1) ? rsq.y : (r == 2) ? rsq.z : rsq.w;
                            rope_rotate_word(l, h, cw, sw);
                            asm volatile("" : "+v"(l), "+v"(h));
                        }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (ROT) {
                lds_at<uint4>(rks, o_lo) = rlo;
                lds_at<uint4>(rks, o_hi) = rhi;
            }
        };

        // Block 2: O^T += V(i-1)^T P(i-1)^T from pp; with EXP, P(i) = 2^(S(i) c
        // - m_ref) into pn: softmax steps E1 .. 17 spread over the MFMAs (E1 > 0:
        // block 1 took the first ones).  Returns the lane's partial row sum of
        // P(i) (fp32, before rounding).
        auto block2 = [&](auto exp_c, auto e1_c, int i, const bf16x8_t (&pp)[kBN / 16], bf16x8_t (&pn)[kBN / 16])
            __attribute__((always_inline)) {
            constexpr bool EXP = decltype(exp_c)::value;
            constexpr int E1 = decltype(e1_c)::value;
            const uint32_t vbase = lds_addr(vslot(i - 1));
            uint32_t vp[G::DB];
#pragma unroll
            for (int db = 0; db < G::DB; ++db) {
                vp[db] = (vbase + (uint32_t)v_addr0) ^ (uint32_t)(db << 6);
                asm("" : "+v"(vp[db]));
            }
            i16x4_t vt0[NM2], vt1[NM2];
            auto vread = [&](int k) __attribute__((always_inline)) {
                const int ch = k / G::DB, db = k % G::DB;
                const lds_u8_t *p0 = lds_ptr(vp[db]) + 16 * ch * G::ROWB;
                vt0[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
                vt1[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p0 + 8 * G::ROWB));
            };
            if constexpr (EXP && E1 == 0) {
#pragma unroll
                for (int q = 0; q < 4; ++q) xr[q] = 0.f;
            }
#pragma unroll
            for (int k = 0; k < PF; ++k) vread(k);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NM2; ++k) {
                if (k + PF < NM2) vread(k + PF);
                const int ch = k / G::DB, db = k % G::DB;
                const uint2 u0 = __builtin_bit_cast(uint2, vt0[k]), u1 = __builtin_bit_cast(uint2, vt1[k]);
                const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y));
                acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pp[ch], acc_o[db], 0, 0, 0);
                if constexpr (EXP && E1 == 0) {
                    constexpr int PER = 16 / NM2;   // exp steps per MFMA; the last MFMA also drains the chain
#pragma unroll
                    for (int q = 0; q < PER; ++q) exp_step(k * PER + q);
                    if (k == NM2 - 1) {
                        exp_step(16);
                        exp_step(17);
                    }
                } else if constexpr (EXP) {
                    // steps E1 + [k n / NM2, (k + 1) n / NM2), n = NSTEP - E1
                    constexpr int NREM = NSTEP - E1;
#pragma unroll
                    for (int e = E1 + k * NREM / NM2; e < E1 + (k + 1) * NREM / NM2; ++e) exp_step(e);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (EXP) {
#pragma unroll
                for (int ch = 0; ch < kBN / 16; ++ch)
                    pn[ch] = __builtin_bit_cast(bf16x8_t, make_uint4(xw[4 * ch], xw[4 * ch + 1], xw[4 * ch + 2], xw[4 * ch + 3]));
            }
            return (xr[0] + xr[1]) + (xr[2] + xr[3]);
        };

        // ---- iterations ---------------------------------------------------------
        // Iteration i issues its loads first and ends with the wait for the loads
        // of iteration i-1 and the barrier; every wave runs all T + 1 iterations.
        auto issue = [&](int i) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NDMA; ++j) dma_step(i, j);
        };
        auto finish = [&](int i) __attribute__((always_inline)) {
            wait_vmcnt<NDMA>();   // loads of iteration i-1 have landed; those of iteration i may fly
            __syncthreads();
        };
        // D = 64 has 256 rotation units: only waves 0..3 rotate (wave-uniform).
        // With a window, a pair group pruned on the whole work-group tile is
        // never read, so it is not rotated.
        auto rot_on = [&](int i) __attribute__((always_inline)) {
            return ROPE_K && i + 1 < T && wave * 64 < G::K_UNITS &&
                   !(WINDOW && w_rot < max(0, n0 - ((i + 1) * kBN + kBN - 1)));
        };
        // S(i) into sc, with K(i+1) rotated alongside.
        // Block 1 with S(i); also issues the loads of iteration i.
        // With a window: the distances of this wave's 32 queries to the two
        // 32-key blocks of tile t lie in [dlo, dhi] (dlo clamped at 0: causally
        // masked cells are discarded later; dhi clipped to stored rows).
        struct WinMasks { uint64_t prune[2], keep[2]; };
        auto win_masks = [&](int t) __attribute__((always_inline)) {
            WinMasks m;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int mk0 = t * kBN + kb * 32;
                const int dlo = max(0, nw0 - (mk0 + 31)), dhi = min(nw0 + 31, S - 1) - mk0;
                m.prune[kb] = __builtin_amdgcn_ballot_w64(w_lane < dlo);
                m.keep[kb] = ~__builtin_amdgcn_ballot_w64(w_lane < dhi);
            }
            return m;
        };
        // The variant NS of a tile: the even number of leading chunks pruned on
        // both blocks, valid if every chunk from NS + 2 on is kept on both (else
        // -1, the generic one).
        auto win_variant = [&](const WinMasks &m) __attribute__((always_inline)) {
            const uint64_t pr = m.prune[0] & m.prune[1], kp = m.keep[0] & m.keep[1];
            const int lead = (~pr == 0) ? 64 : __builtin_ctzll(~pr);
            int ns = min((lead >> 3) & ~1, G::KCH - 2);
            const int top = 8 * (ns + 2);
            if (top < 64 && (kp | ((1ull << top) - 1)) != ~0ull) ns = -1;
            return ns;
        };
        // S(i) with a window: the variant chosen at run time, then the partial
        // pairs.  VARIANTS false: the generic variant only.
        auto scores_w = [&](auto variants_c, int i, const WinMasks &m) __attribute__((always_inline)) {
            const int ns = decltype(variants_c)::value ? win_variant(m) : -1;
            const bool rot = rot_on(i);
            auto run = [&](auto ns_c) __attribute__((always_inline)) {
                if (rot) block1w(std::true_type{}, ns_c, i, m.prune, m.keep);
                else block1w(std::false_type{}, ns_c, i, m.prune, m.keep);
            };
            if constexpr (decltype(variants_c)::value) {
                static_assert(G::KCH == 4 || G::KCH == 8, "variant list");
                // (the partial pairs are added after the variant's MFMAs)
                if (ns == 0) run(std::integral_constant<int, 0>{});
                else if (ns == 2) run(std::integral_constant<int, 2>{});
                else if (G::KCH == 8 && ns == 4) run(std::integral_constant<int, (G::KCH == 8 ? 4 : -1)>{});
                else if (G::KCH == 8 && ns == 6) run(std::integral_constant<int, (G::KCH == 8 ? 6 : -1)>{});
                else run(std::integral_constant<int, -1>{});
            } else {
                run(std::integral_constant<int, -1>{});
            }
            // The pairs whose limit falls inside a block's distance range.
            const uint32_t kbase = lds_addr(kslot(i));
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (const uint64_t part = ~(m.prune[kb] | m.keep[kb]))
                    window_partial(sc[kb], part, kbase + (uint32_t)(kb * 32 * G::ROWB), i * kBN + kb * 32);
            if (need_mask(i)) mask_tile(sc, i);
        };
        auto scores = [&](int i) __attribute__((always_inline)) {
            if (rot_on(i)) block1(std::true_type{}, std::false_type{}, i);
            else block1(std::false_type{}, std::false_type{}, i);
            if (need_mask(i)) mask_tile(sc, i);
        };
        auto accept = [&](float rs, bf16x8_t (&pn)[kBN / 16]) __attribute__((always_inline)) {
            if (__builtin_amdgcn_ballot_w64(!(rs <= kLazyMaxSum)) != 0) rs = rescale_exp_tile(sc, pn);
            l_run += rs;
        };
        using E0 = std::integral_constant<int, 0>;
        // Steady state, 1 <= i < wave_tiles: S(i) || rotation; PV(i-1) from pp || P(i) into pn.
        auto steady = [&](int i, const bf16x8_t (&pp)[kBN / 16], bf16x8_t (&pn)[kBN / 16]) __attribute__((always_inline)) {
            scores(i);   // issues the loads of iteration i between its MFMAs
            accept(block2(std::true_type{}, E0{}, i, pp, pn), pn);
            finish(i);
        };
        // The same for a tile that needs no mask, with the first softmax steps
        // (key block 0) under the MFMAs of block 1: only a wave's last tile can
        // need the causal or sequence-end mask (for t <= wave_tiles - 2, 64 t + 63
        // <= nw0 and 64 t + 64 < S).
        auto steady_split = [&](int i, const bf16x8_t (&pp)[kBN / 16], bf16x8_t (&pn)[kBN / 16]) __attribute__((always_inline)) {
            if (rot_on(i)) block1(std::true_type{}, std::true_type{}, i);
            else block1(std::false_type{}, std::true_type{}, i);
            accept(block2(std::true_type{}, std::integral_constant<int, G::KCH - 2>{}, i, pp, pn), pn);
            finish(i);
        };
        // The same with a window (the masks of tile i taken at its start).
        auto steady_w = [&](int i, const bf16x8_t (&pp)[kBN / 16], bf16x8_t (&pn)[kBN / 16]) __attribute__((always_inline)) {
            scores_w(std::true_type{}, i, win_masks(i));
            accept(block2(std::true_type{}, E0{}, i, pp, pn), pn);
            finish(i);
        };
        // i = wave_tiles: the last PV; later iterations only load and rotate.
        auto last_pv = [&](int i, const bf16x8_t (&pp)[kBN / 16], bf16x8_t (&scratch_pf)[kBN / 16]) __attribute__((always_inline)) {
            issue(i);
            if (rot_on(i)) rotate_k(i + 1);
            block2(std::false_type{}, E0{}, i, pp, scratch_pf);
            finish(i);
        };
        auto idle = [&](int i) __attribute__((always_inline)) {
            issue(i);
            if (rot_on(i)) rotate_k(i + 1);
            finish(i);
        };

        // Prologue: K(0..2) (with cos/sin) and V(0) in LDS, K(0) rotated.
        dload_k(0);
        if (1 < T) dload_k(1);
        if (2 < T) dload_k(2);
        dload_v(0);
        wait_vmcnt<0>();
        __syncthreads();
        if constexpr (ROPE_K) {
            rotate_k(0);
            __syncthreads();
        }

        int i = 0;
        if (wave_tiles > 0) {
            // iteration 0: S(0), P(0) into pf_a
            if constexpr (WINDOW) scores_w(std::false_type{}, 0, win_masks(0));
            else scores(0);
            l_run = first_exp_tile(sc, pf_a);
            finish(0);
            if constexpr (WINDOW) {
                // One iteration per trip (the window variants make the body
                // large): P moves from pf_b back to pf_a.
                for (i = 1; i < wave_tiles; ++i) {
                    steady_w(i, pf_a, pf_b);
#pragma unroll
                    for (int ch = 0; ch < kBN / 16; ++ch) pf_a[ch] = pf_b[ch];
                }
                last_pv(i, pf_a, pf_b);
            } else if constexpr (ROPE_K) {
                // P(j) is in pf_a for even j, in pf_b for odd j.  (Block 1
                // carries the key rotation here: all the exps stay in block 2.)
                for (i = 1; i + 1 < wave_tiles; i += 2) {
                    steady(i, pf_a, pf_b);
                    steady(i + 1, pf_b, pf_a);
                }
                if (i < wave_tiles) {
                    steady(i, pf_a, pf_b);
                    ++i;
                    last_pv(i, pf_b, pf_a);
                } else {
                    last_pv(i, pf_a, pf_b);
                }
            } else {
                // P(j) is in pf_a for even j, in pf_b for odd j; the last tile
                // takes the masked path.
                for (i = 1; i + 2 < wave_tiles; i += 2) {
                    steady_split(i, pf_a, pf_b);
                    steady_split(i + 1, pf_b, pf_a);
                }
                if (i + 1 < wave_tiles) {   // one more unmasked tile (once per wave: P copied back)
                    steady_split(i, pf_a, pf_b);
#pragma unroll
                    for (int ch = 0; ch < kBN / 16; ++ch) pf_a[ch] = pf_b[ch];
                    ++i;
                }
                if (i < wave_tiles) {
                    steady(i, pf_a, pf_b);
                    ++i;
                    last_pv(i, pf_b, pf_a);
                } else {
                    last_pv(i, pf_a, pf_b);
                }
            }
            ++i;
        }
        for (; i <= T; ++i) idle(i);
        wait_vmcnt<0>();   // no load may still be writing LDS when the work-group ends

        // ---- epilogue: O / l, bf16, store --------------------------------------
        if (!wave_active) return;
        const float l_row = sum_halves(l_run);
        const float inv = 1.0f / l_row;
        const int n = nw0 + l32;
        if (n >= S) return;
        // Optional log-sum-exp of the row's scaled scores, L = m + log l in the
        // natural-log domain ("AttnFuse", section 4.4: the one value per row the
        // forward pass keeps for a backward pass): sum_m 2^(s c) = 2^m_ref l.
        if (a.lse != nullptr && g == 0)
            a.lse[((size_t)b * a.Hq + hq) * S + n] =
                (m_ref + __builtin_amdgcn_logf(l_row)) * 0.693147180559945309f;
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
    };

    if constexpr (PERSIST) {
        // Task list: sched[0 .. bins] are the bin offsets, sched[bins + 1 + j]
        // task j = qt | hq << 12 | b << 22.  The host checked that the offsets
        // rise from 0 to the task count and that every (b, hq, qt) of the call
        // appears exactly once.  A barrier separates consecutive tiles: every
        // wave has waited for its own direct loads at the end of a tile, so
        // after it no load of the previous tile can still write LDS when the
        // next tile stages its Q.
        const uint32_t *off = a.sched;
        const uint32_t *task = a.sched + a.sched_bins + 1;
        const int j0 = (int)off[blockIdx.x], j1 = (int)off[blockIdx.x + 1];
        for (int j = j0; j < j1; ++j) {
            if (j > j0) __syncthreads();
            const uint32_t t = __builtin_amdgcn_readfirstlane(task[j]);
            tile((int)(t >> 22), (int)((t >> 12) & 1023u), (int)(t & 4095u));
        }
    } else {
        // ---- work decode: XCD-contiguous, longest query tile first ----------
        // Work-groups are dealt to the 8 XCDs round robin; remapped, each XCD
        // takes a contiguous range of work.  Within it the heads go in bands of
        // kb heads (about 64 query tiles per band: one head at S = 16k, two at
        // 8k, eight at 2k), and a band runs its tiles longest first across its
        // heads.  Few heads in flight per XCD keep their K and V in its L2; a
        // band of several heads at short S keeps the short tiles of one head
        // from running alone at its end.
        const int n_qt = (a.S + kBM - 1) / kBM;
        const int n_bh = a.Hq * a.B;
        const int n_work = n_qt * n_bh;
        int work = blockIdx.x;
        if ((n_work & 7) == 0)
            work = (blockIdx.x & 7) * (n_work >> 3) + (blockIdx.x >> 3);
        const int kb = max(1, kBandTiles / n_qt);
        const int band = work / (kb * n_qt);
        const int in_band = work - band * kb * n_qt;
        const int band_heads = min(kb, n_bh - band * kb);
        const int rank = in_band / band_heads;
        // (readfirstlane: the divisions run on the vector unit; their results are
        // wave-uniform, and everything derived from them can then live in scalar
        // registers, the load descriptors included.)
        const int bh = __builtin_amdgcn_readfirstlane(band * kb + (in_band - rank * band_heads));
        const int qt = __builtin_amdgcn_readfirstlane(n_qt - 1 - rank);
        const int b = __builtin_amdgcn_readfirstlane(bh / a.Hq);
        const int hq = bh - b * a.Hq;
        tile(b, hq, qt);
    }
}

template <int D, bool ROPE, bool ROPE_K, bool CAUSAL, bool WINDOW>
hipError_t launch_t(const FwdArgs &a, hipStream_t stream)
{
    const int n_qt = (a.S + kBM - 1) / kBM;
    const long long n_work = (long long)n_qt * a.Hq * a.B;
    if (n_work <= 0) return hipSuccess;
    if (a.sched != nullptr) {
        // Persistent: one work-group per bin of the task list (causal, no
        // window: without the mask every query tile costs the same).
        if constexpr (CAUSAL && !WINDOW)
            hipLaunchKernelGGL((attn_fwd_kernel<D, ROPE, ROPE_K, CAUSAL, WINDOW, true>), dim3((unsigned)a.sched_bins),
                               dim3(kThreads), 0, stream, a);
        else
            return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((attn_fwd_kernel<D, ROPE, ROPE_K, CAUSAL, WINDOW, false>), dim3((unsigned)n_work), dim3(kThreads),
                           0, stream, a);
    }
    return hipGetLastError();
}

template <int D, bool ROPE, bool ROPE_K>
hipError_t launch_c(const FwdArgs &a, hipStream_t stream)
{
    if (a.use_window) {
        // The window is defined on the causal triangle only (checked by the host API).
        if (!a.causal) return hipErrorInvalidValue;
        return launch_t<D, ROPE, ROPE_K, true, true>(a, stream);
    }
    return a.causal ? launch_t<D, ROPE, ROPE_K, true, false>(a, stream)
                    : launch_t<D, ROPE, ROPE_K, false, false>(a, stream);
}

template <int D>
hipError_t launch_d(const FwdArgs &a, hipStream_t stream)
{
    if (a.rope_cs == nullptr) return launch_c<D, false, false>(a, stream);
    return a.rope_k ? launch_c<D, true, true>(a, stream) : launch_c<D, true, false>(a, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs &a, hipStream_t stream)
{
    if (a.D == 128) return launch_d<128>(a, stream);
    if (a.D == 64) return launch_d<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
