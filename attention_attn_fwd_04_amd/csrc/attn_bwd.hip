// attn_bwd.hip -- attention backward for gfx950 (MI355X).
//
// The computation ("AttnFuse: A Composable DSL for Compiling Attentions to
// Fused GPU Kernels", section 4.4 "Backward Pass", the FlashAttention-2
// decomposition): a preprocessing kernel computes the row-reduced gradient
// Delta = rowsum(dO o O); one kernel accumulates dK and dV per key tile,
// another dQ per query tile, each writing its own output tile (no atomics).
// The forward pass keeps one value per row, L = m + log l (attn_fwd_lse),
// from which P = exp(S - L) is rebuilt tile by tile:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - Delta),
//   dQ' = scale dS K',  dK' = scale dS^T Q',
// and, with RoPE, dQ = R(n)^T dQ', dK = R(m)^T dK' (the rotation is
// orthogonal), applied in the kernels' epilogues.
//
// gfx950 design (correctness first; the forward kernel's software
// pipelining is not repeated here):
//  * The preprocessing kernel also stages the operands: Q as
//    bf16(scale log2e R(n) q), rounded once exactly as the forward kernel
//    stages it, and K as bf16(R(m) k), bitwise the forward's K'.  Scores
//    then come out of the MFMAs in the exp2 domain.
//  * Work-groups of 8 waves own 256 rows (32 per wave): queries in the dQ
//    kernel, keys in the dK/dV kernel.  The other side streams through LDS
//    in 32-row tiles (direct-to-LDS buffer loads, two slots, the next tile
//    loading while the current one is used), one barrier per tile; each
//    streamed tile feeds all 8 waves.
//  * All products are 32x32x16 bf16 MFMAs with fp32 accumulation.  The
//    operands that stay (Q and dO for dQ; K' and V for dK, dV) sit in
//    B-operand registers; the streamed tile gives A operands, as 16-byte
//    row reads or, for the transposed products, ds_read_b64_tr_b16 reads.
//    The score and dP accumulators hold exactly the B operands the next
//    products need (P, dS), as in the forward kernel.  Each score chain
//    starts from -L log2 e, so P = exp2(accumulator).
//  * With grouped heads the dK/dV kernel walks the group's query heads in
//    turn, accumulating into the same registers.  When its grid is short
//    (under four rounds of resident work-groups), each (key tile, KV head)
//    is split into one work-group per query head instead, four times as
//    many shorter work-groups, which balance better over the CUs (measured
//    faster on the grouped-head workload).  The splits write fp32 partial
//    sums, and a reduction kernel adds them in a fixed order (no atomics).
//  * Both gradient kernels fit 256 registers per lane, so two waves share
//    each SIMD: one wave's LDS waits and softmax arithmetic overlap the
//    other's MFMAs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_gfx950.h"
#include "attn_internal.h"
#include "attn_ext_args.h"

namespace attn {
namespace {

constexpr int kBwdWaves = 8;
constexpr int kBwdThreads = kBwdWaves * 64;
constexpr int kBwdBM = kBwdWaves * 32;   // rows per work-group
constexpr int kBwdBN = 32;               // rows per streamed tile
constexpr float kLog2e = 1.44269504088896340736f;

template <int D>
struct BGeo {
    static constexpr int KCH = D / 16;
    static constexpr int PG = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int CH = D / 8;
    static constexpr int ROWB = 2 * D;
    static constexpr int TILE_B = kBwdBN * ROWB;
    static constexpr int NI = TILE_B / 1024;
    static constexpr int NI_W = NI >= kBwdWaves ? NI / kBwdWaves : 1;
    static constexpr int RPI = 1024 / ROWB;
    static_assert(NI % kBwdWaves == 0 || kBwdWaves % NI == 0, "direct loads split over the waves");
    // 16-byte chunks XOR-permuted per row.  The streamed tiles are read both
    // as rows (ds_read_b128: 16 lanes, 16 consecutive rows, one logical
    // chunk) and transposed (ds_read_b64_tr_b16: 32 lanes, 4 consecutive rows
    // x 4 consecutive chunks), so the permutation must spread both over the
    // 16 four-bank groups of a 256-byte bank cycle: it is injective over 16
    // rows and its top two bits differ among any 4 aligned rows (for D = 64,
    // two rows share a bank cycle, so the same holds per row parity).
    static __device__ __forceinline__ int kx(int r)
    {
        return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    }
    static __device__ __forceinline__ int off(int r, int c) { return r * ROWB + ((c ^ kx(r)) << 4); }
    // Byte address of dim d of row r in that layout.
    static __device__ __forceinline__ int dim_off(int r, int d) { return off(r, d >> 3) + 2 * (d & 7); }
};

// A operands of one streamed tile.  Row reads: lane (l32, g) gets row l32,
// dims 8 kc + (D/2) g .. +7 (the pair-aligned order of the prefill kernel).
// Transposed reads (ds_read_b64_tr_b16): within each 16-lane group, source
// lane s reads row s / 4 of a 4-row group at dims D0 + 4 (s % 4) .. +3,
// D0 = 32 db + 16 ((lane / 16) % 2); lane i of the group then holds dim
// D0 + i of those 4 rows.  With the rows 16 ch + 4 g + (0..3) and the same
// + 8, the 8 values of a lane follow the row order of the MFMA C layout,
// which is the order of the P / dS operands built from an accumulator.
// The per-lane byte offsets are recomputed from the lane index in every
// tile (refresh() hides the index from loop-invariant code motion): 16
// registers held across the loop would cost the kernels their second wave
// per SIMD.
template <int D>
struct TileReader {
    using G = BGeo<D>;
    int lane_;
    __device__ __forceinline__ void init(int lane) { lane_ = lane; }
    __device__ __forceinline__ void refresh() { asm volatile("" : "+v"(lane_)); }
    // Chunk kc + PG g of row l32 sits at l32 ROWB + ((kc + PG g) ^ kx(l32)) 16.
    // kc and PG g occupy disjoint bits, so that is the lane's chunk-0 address
    // XOR kc 16: one XOR per read once the lane part is known (tile bases are
    // multiples of 256 bytes, so the XOR never reaches them).
    __device__ __forceinline__ bf16x8_t row(uint32_t base, int kc) const
    {
        const int l32 = lane_ & 31, g = lane_ >> 5;
        const uint32_t lane_off = (uint32_t)(l32 * G::ROWB + (((G::PG * g) ^ G::kx(l32)) << 4));
        return *(const lds_bf16x8_t *)lds_ptr((base + lane_off) ^ (uint32_t)(kc << 4));
    }
    // rows 16 ch + ...: the chunk permutation repeats every 16 rows.  Chunk
    // 4 db + c0 (c0 < 4) XOR kx(r) = (c0 XOR kx(r)) XOR 4 db: the lane's db = 0
    // address XOR db 64.
    __device__ __forceinline__ bf16x8_t tr(uint32_t base, int ch, int db) const
    {
        const int g = lane_ >> 5;
        const int tr_row = (lane_ & 15) >> 2;
        const int tr_dim = 16 * ((lane_ >> 4) & 1) + 4 * (lane_ & 3);
        const uint32_t a0 = (base + (uint32_t)G::dim_off(4 * g + tr_row, tr_dim)) ^ (uint32_t)(db << 6);
        const uint32_t a1 = (base + (uint32_t)G::dim_off(4 * g + tr_row + 8, tr_dim)) ^ (uint32_t)(db << 6);
        const lds_u8_t *p0 = lds_ptr(a0) + 16 * ch * G::ROWB;
        const lds_u8_t *p1 = lds_ptr(a1) + 16 * ch * G::ROWB;
        const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
        const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p1);
        const uint2 u0 = __builtin_bit_cast(uint2, t0), u1 = __builtin_bit_cast(uint2, t1);
        return __builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y));
    }
};

// Instruction order of one block of MFMAs fed from LDS: the first group of
// reads, then alternately two MFMAs and the reads of the next two (the
// scheduler otherwise issues each read right before its MFMA and waits on
// it).  n_mfma MFMAs, reads_per_mfma LDS reads each.
template <int n_mfma, int reads_per_mfma>
__device__ __forceinline__ void interleave_reads_mfma()
{
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * reads_per_mfma, 0);   // DS reads
#pragma unroll
    for (int j = 0; j < n_mfma / 2 - 1; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * reads_per_mfma, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

// Direct loads of one 32-row tile (rows row0 .. row0 + 31 of a tensor whose
// rows are row_b bytes apart, D bf16 values each) into LDS at lds_dst in the
// permuted-chunk layout; wave w issues instructions w, w + 4, ...  Rows past
// the descriptor's range read as zeros.
template <int D>
__device__ __forceinline__ void stream_tile(u32x4_t rs, uint32_t row_b, int row0, uint32_t lds_dst, int wave, int lane)
{
    using G = BGeo<D>;
    const int dl_row = lane / G::CH, dl_slot = lane % G::CH;
#pragma unroll
    for (int i = 0; i < G::NI_W; ++i) {
        const int ins = wave + kBwdWaves * i;
        if (ins >= G::NI) break;   // D = 64: fewer load instructions than waves (wave-uniform)
        const int r = ins * G::RPI + dl_row;
        dma16(rs, (uint32_t)(row0 + r) * row_b + 16u * (uint32_t)(dl_slot ^ G::kx(r)), lds_dst + (uint32_t)(ins * 1024));
    }
}

// Work order of the gradient kernels: one work-group per (row tile, head),
// the tiles with the most streamed work first, over all heads, so the long
// ones do not start last.  When the heads split evenly over the 8 XCDs
// (work-groups are dealt to them round robin), XCD x takes heads
// x * H/8 .. and runs them longest tile first.  Returns the tile rank
// (0 = most work) and the (batch, head) index, both wave-uniform.
__device__ __forceinline__ void decode_work(int n_bh, int &rank, int &bh)
{
    const int w = blockIdx.x;
    int r, h;
    if ((n_bh & 7) == 0) {
        const int hpx = n_bh >> 3, j = w >> 3;
        r = j / hpx;
        h = (w & 7) * hpx + (j - r * hpx);
    } else {
        r = w / n_bh;
        h = w - r * n_bh;
    }
    rank = __builtin_amdgcn_readfirstlane(r);
    bh = __builtin_amdgcn_readfirstlane(h);
}

// Inverse RoPE of one lane's column of a transposed accumulator (rows = dims
// 32 db + 8 r + 4 g + j; the pair (d, d + D/2) is (acc[db], acc[db + DB/2])):
// x = x' c + y' s, y = y' c - x' s with the cosines / sines of position p
// (cos of pair d at table index p D + d, sin at p D + D/2 + d).
template <int D>
__device__ __forceinline__ void unrotate_acc(f32x16_t (&acc)[D / 32], const uint16_t *cs, int p, int g)
{
    constexpr int DB = D / 32;
#pragma unroll
    for (int db = 0; db < DB / 2; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d0 = 32 * db + 8 * r + 4 * g;
            const uint2 cw = *reinterpret_cast<const uint2 *>(cs + (size_t)p * D + d0);
            const uint2 sw = *reinterpret_cast<const uint2 *>(cs + (size_t)p * D + D / 2 + d0);
            const float cv[4] = {half_lo(cw.x), half_hi(cw.x), half_lo(cw.y), half_hi(cw.y)};
            const float sv[4] = {half_lo(sw.x), half_hi(sw.x), half_lo(sw.y), half_hi(sw.y)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x = acc[db][4 * r + j], y = acc[db + DB / 2][4 * r + j];
                acc[db][4 * r + j] = __builtin_fmaf(x, cv[j], y * sv[j]);
                acc[db + DB / 2][4 * r + j] = __builtin_fmaf(y, cv[j], -(x * sv[j]));
            }
        }
}

// Stores one lane's column of a transposed accumulator, times k, as bf16.
template <int D>
__device__ __forceinline__ void store_acc(uint16_t *row, const f32x16_t (&acc)[D / 32], float k, int g)
{
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint2 w;
            w.x = pack_bf16x2(acc[db][4 * r] * k, acc[db][4 * r + 1] * k);
            w.y = pack_bf16x2(acc[db][4 * r + 2] * k, acc[db][4 * r + 3] * k);
            *reinterpret_cast<uint2 *>(row + db * 32 + 8 * r + 4 * g) = w;
        }
}

// The same column as fp32, times k (partial sums of a split dK/dV).
template <int D>
__device__ __forceinline__ void store_acc_f32(float *row, const f32x16_t (&acc)[D / 32], float k, int g)
{
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<float4 *>(row + db * 32 + 8 * r + 4 * g) =
                make_float4(acc[db][4 * r] * k, acc[db][4 * r + 1] * k, acc[db][4 * r + 2] * k, acc[db][4 * r + 3] * k);
}

// ---- preprocessing --------------------------------------------------------
// One thread per (row, 8-pair group), rows in [B, S, H] order as in the RoPE
// pass: query rows first (stage bf16(c R(n) q) and add the group's share of
// Delta = rowsum(dO o O), reduced over the row's D/16 threads), then, with
// RoPE, key rows (stage bf16(R(m) k)).
template <int D, bool ROPE>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdArgs a, long long n_q_units, long long n_units)
{
    constexpr int PG = D / 16;
    const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
    if (u >= n_units) return;   // whole rows: n_units and n_q_units are multiples of PG
    const bool is_q = u < n_q_units;
    const long long uu = is_q ? u : u - n_q_units;
    const int H = is_q ? a.Hq : a.Hkv;
    const long long row = uu / PG;   // (b S + s) H + h
    const int pg = (int)(uu - row * PG);
    const int s = (int)((row / H) % a.S);
    const uint16_t *src = (is_q ? a.q : a.k) + row * D;
    uint16_t *dst = (is_q ? a.qs : a.kr) + row * D;

    uint4 lo = *reinterpret_cast<const uint4 *>(src + 8 * pg);
    uint4 hi = *reinterpret_cast<const uint4 *>(src + D / 2 + 8 * pg);
    const float k = is_q ? a.scale_log2e : 1.0f;
    if constexpr (ROPE) {
        const uint4 cq = *reinterpret_cast<const uint4 *>(a.rope_cs + (((size_t)s * 2 + 0) * PG + pg) * 8);
        const uint4 sq = *reinterpret_cast<const uint4 *>(a.rope_cs + (((size_t)s * 2 + 1) * PG + pg) * 8);
        if (is_q)
            rope_rotate8_scaled(lo, hi, cq, sq, k);
        else
            rope_rotate8(lo, hi, cq, sq);
    } else {
        lo = scale_bf16x8(lo, k);
        hi = scale_bf16x8(hi, k);
    }
    *reinterpret_cast<uint4 *>(dst + 8 * pg) = lo;
    *reinterpret_cast<uint4 *>(dst + D / 2 + 8 * pg) = hi;

    float part = 0.f;
    if (is_q) {
        const uint16_t *orow = a.o + row * D, *drow = a.dout + row * D;
        const uint4 x[2] = {*reinterpret_cast<const uint4 *>(orow + 8 * pg),
                            *reinterpret_cast<const uint4 *>(orow + D / 2 + 8 * pg)};
        const uint4 y[2] = {*reinterpret_cast<const uint4 *>(drow + 8 * pg),
                            *reinterpret_cast<const uint4 *>(drow + D / 2 + 8 * pg)};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t xs[4] = {x[h].x, x[h].y, x[h].z, x[h].w}, ys[4] = {y[h].x, y[h].y, y[h].z, y[h].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                part = __builtin_fmaf(bf16_lo(xs[e]), bf16_lo(ys[e]), part);
                part = __builtin_fmaf(bf16_hi(xs[e]), bf16_hi(ys[e]), part);
            }
        }
    }
    // The PG threads of a row are consecutive lanes of one wave, all active.
#pragma unroll
    for (int w = PG / 2; w >= 1; w >>= 1) part += __shfl_xor(part, w, PG);
    if (is_q && pg == 0) {
        const int h = (int)(row % a.Hq);
        const int b = (int)(row / ((long long)a.Hq * a.S));
        a.delta[((size_t)b * a.Hq + h) * a.S + s] = part;
    }
}

// ---- dQ: per 128-query tile and head, keys streamed -----------------------
template <int D, bool CAUSAL, bool ROPE>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(const BwdArgs a)
{
    using G = BGeo<D>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * G::TILE_B];   // K' and V, two slots each
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    int rank, bh;
    decode_work(a.B * a.Hq, rank, bh);
    const int qt = (a.S + kBwdBM - 1) / kBwdBM - 1 - rank;   // the last query tile streams the most keys
    const int b = __builtin_amdgcn_readfirstlane(bh / a.Hq);
    const int hq = bh - b * a.Hq;
    const int S = a.S, hk = __builtin_amdgcn_readfirstlane(hq / (a.Hq / a.Hkv));
    const int n0 = qt * kBwdBM, nw0 = n0 + wave * 32, n = nw0 + l32;

    // Resident B operands: the staged query (c R(n) q) and dO of the lane's
    // query (buffer loads: zero past S).
    const uint32_t q_rowb = (uint32_t)a.Hq * D * 2;
    const size_t qoff = (((size_t)b * S + n) * a.Hq + hq) * D;
    bf16x8_t qreg[G::KCH], doreg[G::KCH];
    {
        const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(a.qs + ((size_t)b * S * a.Hq + hq) * D, (uint32_t)S * q_rowb);
        const __amdgpu_buffer_rsrc_t d_rs = make_rsrc(a.dout + ((size_t)b * S * a.Hq + hq) * D, (uint32_t)S * q_rowb);
#pragma unroll
        for (int kc = 0; kc < G::KCH; ++kc) {
            const uint32_t off = (uint32_t)n * q_rowb + 2u * (uint32_t)(8 * kc + (D / 2) * g);
            qreg[kc] = __builtin_bit_cast(bf16x8_t, bload16(q_rs, off));
            doreg[kc] = __builtin_bit_cast(bf16x8_t, bload16(d_rs, off));
        }
    }
    const size_t rowid = ((size_t)b * a.Hq + hq) * S + n;
    const float L2 = n < S ? a.lse[rowid] * kLog2e : 0.f;
    const float dlt = n < S ? a.delta[rowid] : 0.f;
    wait_vmcnt<0>();

    const uint32_t kv_rowb = (uint32_t)a.Hkv * D * 2;
    const u32x4_t k_rs = make_desc(a.kop + ((size_t)b * S * a.Hkv + hk) * D, (uint32_t)S * kv_rowb);
    const u32x4_t v_rs = make_desc(a.v + ((size_t)b * S * a.Hkv + hk) * D, (uint32_t)S * kv_rowb);
    const uint32_t smem32 = lds_addr(smem);
    auto kslot = [&](int t) { return smem32 + (uint32_t)((t & 1) * 2 * G::TILE_B); };
    auto vslot = [&](int t) { return smem32 + (uint32_t)((t & 1) * 2 * G::TILE_B + G::TILE_B); };
    auto load = [&](int t) {
        stream_tile<D>(k_rs, kv_rowb, t * kBwdBN, kslot(t), wave, lane);
        stream_tile<D>(v_rs, kv_rowb, t * kBwdBN, vslot(t), wave, lane);
    };
    TileReader<D> rd;
    rd.init(lane);

    const int kv_end = CAUSAL ? min(S, n0 + kBwdBM) : S;
    const int T = (kv_end + kBwdBN - 1) / kBwdBN;
    const int wave_end = CAUSAL ? min(S, nw0 + 32) : S;
    f32x16_t acc[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

    load(0);
    for (int t = 0; t < T; ++t) {
        wait_vmcnt<0>();
        __syncthreads();   // tile t visible to all waves; every wave is done with slot (t + 1) & 1
        if (t + 1 < T) load(t + 1);
        const int m0 = t * kBwdBN;
        if (m0 >= wave_end) continue;   // wave-uniform: all keys after this wave's queries
        const uint32_t kb = kslot(t), vb = vslot(t);
        rd.refresh();
        // S^T (exp2 domain, minus L log2 e) and dP^T = V dO^T: rows keys, columns queries
        f32x16_t s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s[i] = -L2;
            dp[i] = 0.f;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kc = 0; kc < G::KCH; ++kc) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.row(kb, kc), qreg[kc], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.row(vb, kc), doreg[kc], dp, 0, 0, 0);
        }
        interleave_reads_mfma<2 * G::KCH, 1>();
        __builtin_amdgcn_sched_barrier(0);
        // dS^T = P^T o (dP^T - Delta) with masked P set to zero: on the key
        // tiles that cross this wave's first query or the end of the sequence
        // (a wave-uniform test) the masked scores become -inf, so their P is
        // exp2(-inf) = 0; the other tiles keep every entry.
        if ((CAUSAL && m0 + kBwdBN - 1 > nw0) || m0 + kBwdBN > S) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + 8 * (i >> 2) + 4 * g + (i & 3);
                s[i] = ((CAUSAL && m > n) || m >= S) ? -__builtin_inff() : s[i];
            }
        }
        bf16x8_t dsop[2];
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            uint32_t w4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v2[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i = 8 * ch + 2 * e + h;
                    const float p = fast_exp2(s[i]);
                    v2[h] = p * (dp[i] - dlt);
                }
                w4[e] = pack_bf16x2(v2[0], v2[1]);
            }
            dsop[ch] = __builtin_bit_cast(bf16x8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
        }
        // dQ'^T += K'^T dS^T
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.tr(kb, ch, db), dsop[ch], acc[db], 0, 0, 0);
        interleave_reads_mfma<2 * G::DB, 2>();
        __builtin_amdgcn_sched_barrier(0);
    }
    if (n >= S) return;
    if constexpr (ROPE) unrotate_acc<D>(acc, a.rope_cs, n, g);
    store_acc<D>(a.dq + qoff, acc, a.scale, g);
}

// ---- dK, dV: per 128-key tile and KV head, queries streamed ----------------
template <int D, bool CAUSAL, bool ROPE>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dkdv_kernel(const BwdArgs a)
{
    using G = BGeo<D>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * G::TILE_B];   // Q and dO, two slots each
    __shared__ __attribute__((aligned(16))) float rowv[2][2][kBwdBN];      // -L log2 e and Delta, two slots
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    int rank, bhs;
    decode_work(a.B * a.Hkv * a.split, rank, bhs);
    const int kt = CAUSAL ? rank : (a.S + kBwdBM - 1) / kBwdBM - 1 - rank;   // the first key tile streams the most queries
    const int bh = __builtin_amdgcn_readfirstlane(bhs / a.split);
    const int sp = bhs - bh * a.split;   // which share of the group's query heads
    const int b = __builtin_amdgcn_readfirstlane(bh / a.Hkv);
    const int hk = bh - b * a.Hkv;
    const int S = a.S, grp = a.Hq / a.Hkv / a.split;   // query heads walked by this work-group
    const int hq0 = hk * (a.Hq / a.Hkv) + sp * grp;
    const int m0 = kt * kBwdBM, mw0 = m0 + wave * 32, m = mw0 + l32;

    // Resident B operands: K' and V of the lane's key (buffer loads: zero
    // past S).
    const uint32_t kv_rowb = (uint32_t)a.Hkv * D * 2;
    const size_t koff = (((size_t)b * S + m) * a.Hkv + hk) * D;
    bf16x8_t kreg[G::KCH], vreg[G::KCH];
    {
        const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(a.kop + ((size_t)b * S * a.Hkv + hk) * D, (uint32_t)S * kv_rowb);
        const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(a.v + ((size_t)b * S * a.Hkv + hk) * D, (uint32_t)S * kv_rowb);
#pragma unroll
        for (int kc = 0; kc < G::KCH; ++kc) {
            const uint32_t off = (uint32_t)m * kv_rowb + 2u * (uint32_t)(8 * kc + (D / 2) * g);
            kreg[kc] = __builtin_bit_cast(bf16x8_t, bload16(k_rs, off));
            vreg[kc] = __builtin_bit_cast(bf16x8_t, bload16(v_rs, off));
        }
    }

    const uint32_t q_rowb = (uint32_t)a.Hq * D * 2;
    const uint32_t smem32 = lds_addr(smem);
    auto qslot = [&](int u) { return smem32 + (uint32_t)((u & 1) * 2 * G::TILE_B); };
    auto dslot = [&](int u) { return smem32 + (uint32_t)((u & 1) * 2 * G::TILE_B + G::TILE_B); };
    // Streamed tiles u = 0 .. U-1: query head hq0 + u / nt, query tile
    // t0 + u % nt (causal: from the first tile that reaches this key tile).
    const int t0 = CAUSAL ? m0 / kBwdBN : 0;
    const int nt = (S + kBwdBN - 1) / kBwdBN - t0;
    const int U = grp * nt;
    // L log2 e and Delta of a tile's 32 queries: fetched into registers one
    // tile ahead by lanes 0..31 of wave 0, written to LDS after the barrier
    // that frees their slot.
    float pre_l = 0.f, pre_d = 0.f;
    auto rows_fetch = [&](int u) {
        if (wave == 0 && lane < kBwdBN) {
            const int hq = hq0 + u / nt, nq = (t0 + u % nt) * kBwdBN + lane;
            const size_t rowid = ((size_t)b * a.Hq + hq) * S + nq;
            pre_l = nq < S ? -(a.lse[rowid] * kLog2e) : 0.f;   // the start of the S chain
            pre_d = nq < S ? a.delta[rowid] : 0.f;
        }
    };
    auto rows_store = [&](int u) {
        if (wave == 0 && lane < kBwdBN) {
            rowv[u & 1][0][lane] = pre_l;
            rowv[u & 1][1][lane] = pre_d;
        }
    };
    auto load = [&](int u) {
        const int hq = hq0 + u / nt, t = t0 + u % nt;
        const u32x4_t q_rs = make_desc(a.qs + ((size_t)b * S * a.Hq + hq) * D, (uint32_t)S * q_rowb);
        const u32x4_t d_rs = make_desc(a.dout + ((size_t)b * S * a.Hq + hq) * D, (uint32_t)S * q_rowb);
        stream_tile<D>(q_rs, q_rowb, t * kBwdBN, qslot(u), wave, lane);
        stream_tile<D>(d_rs, q_rowb, t * kBwdBN, dslot(u), wave, lane);
    };
    TileReader<D> rd;
    rd.init(lane);

    f32x16_t dk[G::DB], dv[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            dk[db][i] = 0.f;
            dv[db][i] = 0.f;
        }

    rows_fetch(0);
    wait_vmcnt<0>();   // register loads done before the first direct load
    rows_store(0);
    load(0);
    for (int u = 0; u < U; ++u) {
        if (u + 1 < U) rows_fetch(u + 1);
        wait_vmcnt<0>();
        __syncthreads();   // tile u and its row values visible; slot (u + 1) & 1 free
        if (u + 1 < U) {
            rows_store(u + 1);
            load(u + 1);
        }
        const int n0 = (t0 + u % nt) * kBwdBN;
        if (CAUSAL && n0 + kBwdBN - 1 < mw0) continue;   // wave-uniform: all queries before this wave's keys
        const uint32_t qb = qslot(u), dbs = dslot(u);
        rd.refresh();
        const float *lrow = rowv[u & 1][0], *drow = rowv[u & 1][1];
        // S = Q K'^T (exp2 domain, minus L log2 e) and dP = dO V^T: rows queries, columns keys
        f32x16_t s, dp;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 l4 = *reinterpret_cast<const float4 *>(lrow + 8 * q4 + 4 * g);
            s[4 * q4 + 0] = l4.x;
            s[4 * q4 + 1] = l4.y;
            s[4 * q4 + 2] = l4.z;
            s[4 * q4 + 3] = l4.w;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) dp[i] = 0.f;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kc = 0; kc < G::KCH; ++kc) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.row(qb, kc), kreg[kc], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.row(dbs, kc), vreg[kc], dp, 0, 0, 0);
        }
        interleave_reads_mfma<2 * G::KCH, 1>();
        __builtin_amdgcn_sched_barrier(0);
        // P and dS = P o (dP - Delta), masked entries zero: on the query
        // tiles that cross this wave's last key or the end of the sequence (a
        // wave-uniform test) the masked scores become -inf, so their P is
        // exp2(-inf) = 0; the other tiles keep every entry.
        if ((CAUSAL && n0 < mw0 + 31) || n0 + kBwdBN > S || mw0 + 32 > S) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int nq = n0 + 8 * (i >> 2) + 4 * g + (i & 3);
                s[i] = ((CAUSAL && nq < m) || nq >= S || m >= S) ? -__builtin_inff() : s[i];
            }
        }
        bf16x8_t pop[2], dsop[2];
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            const float4 d0 = *reinterpret_cast<const float4 *>(drow + 16 * ch + 4 * g);
            const float4 d1 = *reinterpret_cast<const float4 *>(drow + 16 * ch + 8 + 4 * g);
            const float dl[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            uint32_t wp[4], wd[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float pv[2], dsv[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int j = 2 * e + h, i = 8 * ch + j;
                    const float p = fast_exp2(s[i]);
                    pv[h] = p;
                    dsv[h] = p * (dp[i] - dl[j]);
                }
                wp[e] = pack_bf16x2(pv[0], pv[1]);
                wd[e] = pack_bf16x2(dsv[0], dsv[1]);
            }
            pop[ch] = __builtin_bit_cast(bf16x8_t, make_uint4(wp[0], wp[1], wp[2], wp[3]));
            dsop[ch] = __builtin_bit_cast(bf16x8_t, make_uint4(wd[0], wd[1], wd[2], wd[3]));
        }
        // dV^T += dO^T P, dK'^T += Q^T dS
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int db = 0; db < G::DB; ++db) {
                dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.tr(dbs, ch, db), pop[ch], dv[db], 0, 0, 0);
                dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.tr(qb, ch, db), dsop[ch], dk[db], 0, 0, 0);
            }
        interleave_reads_mfma<4 * G::DB, 2>();
        __builtin_amdgcn_sched_barrier(0);
    }
    if (m >= S) return;
    if constexpr (ROPE) unrotate_acc<D>(dk, a.rope_cs, m, g);
    // The streamed queries carry c = scale log2 e: dK' = scale dS^T Q' = (scale / c) dS^T (c Q').
    const float kscale = a.scale / a.scale_log2e;
    if (a.split == 1) {
        store_acc<D>(a.dv + koff, dv, 1.0f, g);
        store_acc<D>(a.dk + koff, dk, kscale, g);
    } else {
        const size_t poff = (size_t)sp * a.B * S * a.Hkv * D + koff;
        store_acc_f32<D>(a.part_dv + poff, dv, 1.0f, g);
        store_acc_f32<D>(a.part_dk + poff, dk, kscale, g);
    }
}

// ---- sum of the split dK/dV partials: one thread per 4 values ---------------
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const BwdArgs a, long long n4)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const size_t stride = (size_t)a.B * a.S * a.Hkv * a.D;
    float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
    for (int s = 0; s < a.split; ++s) {
        const float4 pk = reinterpret_cast<const float4 *>(a.part_dk + s * stride)[i];
        const float4 pv = reinterpret_cast<const float4 *>(a.part_dv + s * stride)[i];
        sk.x += pk.x; sk.y += pk.y; sk.z += pk.z; sk.w += pk.w;
        sv.x += pv.x; sv.y += pv.y; sv.z += pv.z; sv.w += pv.w;
    }
    reinterpret_cast<uint2 *>(a.dk)[i] = make_uint2(pack_bf16x2(sk.x, sk.y), pack_bf16x2(sk.z, sk.w));
    reinterpret_cast<uint2 *>(a.dv)[i] = make_uint2(pack_bf16x2(sv.x, sv.y), pack_bf16x2(sv.z, sv.w));
}

template <int D, bool CAUSAL, bool ROPE>
hipError_t launch_bwd_d(const BwdArgs &a, hipStream_t stream)
{
    constexpr int PG = D / 16;
    const long long n_q_units = (long long)a.B * a.S * a.Hq * PG;
    const long long n_units = n_q_units + (ROPE ? (long long)a.B * a.S * a.Hkv * PG : 0);
    const long long blocks = (n_units + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_prep_kernel<D, ROPE>), dim3((unsigned)blocks), dim3(256), 0, stream, a, n_q_units,
                       n_units);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long tiles = (a.S + kBwdBM - 1) / kBwdBM;
    const long long n_dkdv = tiles * a.Hkv * a.B * a.split, n_dq = tiles * a.Hq * a.B;
    if (n_dq > 0x7fffffffLL || n_dkdv > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, ROPE>), dim3((unsigned)n_dkdv), dim3(kBwdThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.split > 1) {
        const long long n4 = (long long)a.B * a.S * a.Hkv * D / 4;
        hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, a, n4);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, ROPE>), dim3((unsigned)n_dq), dim3(kBwdThreads), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_c(const BwdArgs &a, hipStream_t stream)
{
    const bool rope = a.rope_cs != nullptr;
    if (a.causal) return rope ? launch_bwd_d<D, true, true>(a, stream) : launch_bwd_d<D, true, false>(a, stream);
    return rope ? launch_bwd_d<D, false, true>(a, stream) : launch_bwd_d<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_attn_bwd(const BwdArgs &a, hipStream_t stream)
{
    if (a.B == 0 || a.S == 0) return hipSuccess;
    if (a.D == 128) return launch_bwd_c<128>(a, stream);
    if (a.D == 64) return launch_bwd_c<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
