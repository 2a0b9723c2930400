// attn_decode.hip -- split-KV decode for gfx950 (MI355X): one new query per
// sequence against its KV cache.
//
// The computation ("AttnFuse: A Composable DSL for Compiling Attentions to
// Fused GPU Kernels", section 4.2 "Flash Decoding"): phase 1 splits the
// cache's keys into chunks; each chunk yields a partial (m, l, acc) triple
// from the online-softmax loop; phase 2 merges the partials of a query head
// through their log-sum-exp.  The query heads that share a KV head are packed
// into one MFMA (the page pads them to 16 by cyclic replication; here to the
// 32 columns of a 32x32 MFMA), so K and V are read once per KV head.
//
// gfx950 design:
//  * Decode reads every K and V byte once and does little arithmetic per
//    byte: it is bound by HBM bandwidth.  What matters is keeping enough
//    bytes in flight: a work-group of 4 waves, each wave its own split and
//    its own 2-slot LDS ring of 32-key K and V tiles (direct-to-LDS buffer
//    loads, so the data never passes through registers), one tile in flight
//    while the previous one is computed.  No wave reads another wave's LDS,
//    so the kernel has no barriers.
//  * Scores S^T = K Q'^T and O^T += V^T P^T use the same 32x32x16 bf16 MFMA
//    layouts as the prefill kernel: the column of a lane is one (replicated)
//    query head, the K operand is a 16-byte LDS read, the V^T operand two
//    ds_read_b64_tr_b16 reads, P goes from the score accumulator to the PV
//    operand in registers.  The online softmax is exact per tile (decode's
//    arithmetic is far from the bound).
//  * The cache holds keys as they were stored (rotated when appended, e.g. by
//    attn_rope_apply); with RoPE the query is rotated at position L-1 with
//    the same fp16 cos/sin values and routine as the other kernels (its one
//    row travels in the kernel arguments).
//  * With a per-pair window ("ATFlash -- Per-RoPE-Wavelength Attention
//    Windows", "The idea") the query's pairs are masked per tile: pairs
//    pruned on the whole tile drop out of the MFMA (and their K columns are
//    not fetched), pairs whose limit falls inside the tile are added back
//    one MFMA each where n - m <= w[r].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <type_traits>

#include "attn_ext_args.h"
#include "attn_gfx950.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kDecWaves = 4;     // waves (splits) per work-group
constexpr int kDecBN = 32;       // keys per tile: one 32x32 MFMA block
constexpr int kDecSlots = 2;     // LDS ring depth per wave

template <int D>
struct DGeo {
    static constexpr int KCH = D / 16;               // MFMA k-steps (8 pairs each)
    static constexpr int PG = D / 16;                // 8-pair groups per row
    static constexpr int DB = D / 32;                // 32-dim blocks of O^T
    static constexpr int CH = D / 8;                 // 16-byte chunks per row
    static constexpr int ROWB = 2 * D;               // bytes per row
    static constexpr int TILE_B = kDecBN * ROWB;     // one K or V tile
    static constexpr int NI = TILE_B / 1024;         // 1 KB direct loads per tile
    static constexpr int RPI = 1024 / ROWB;          // rows per direct load
    static constexpr int WAVE_B = kDecSlots * 2 * TILE_B;
    static constexpr int LDS_B = kDecWaves * WAVE_B;
    static_assert(LDS_B <= 160 * 1024, "gfx950 LDS per work-group");
    // The prefill kernel's swizzles: conflict-free K operand and V transpose reads.
    static __device__ __forceinline__ int kx(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static __device__ __forceinline__ int k_off(int r, int c) { return r * ROWB + ((c ^ kx(r)) << 4); }
    static __device__ __forceinline__ int vx(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
    static __device__ __forceinline__ int v_off(int r, int c) { return r * ROWB + ((c ^ vx(r)) << 4); }
};

template <int D, bool ROPE, bool WINDOW>
__global__ __launch_bounds__(kDecWaves * 64, 1) void decode_split_kernel(const DecodeArgs a)
{
    using G = DGeo<D>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS_B];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int split = blockIdx.x * kDecWaves + wave;
    const int hk = blockIdx.y, b = blockIdx.z;
    const int L = a.L, grp = a.Hq / a.Hkv;
    if (split >= a.n_split) return;
    const int m_begin = split * a.keys_per_split;
    const int m_end = min(L, m_begin + a.keys_per_split);
    const int T = m_end > m_begin ? (m_end - m_begin + kDecBN - 1) / kDecBN : 0;
    const float c = a.scale_log2e;
    const int pos = L - 1;   // the query's position

    // ---- Q'^T as the B operand: column l32 is query head (l32 % grp) of this
    // KV head; k-step kc holds pairs 8kc..8kc+7 (lane half 0: their first
    // halves, half 1: their second halves), as in the prefill kernel.
    const int hq = hk * grp + (l32 % grp);
    const uint16_t *qrow = a.q + ((size_t)b * a.Hq + hq) * D;   // lane-dependent: plain global loads
    // The cos/sin row of position L-1 sits in the kernel arguments (scalar
    // loads from the argument segment).
    typedef __attribute__((address_space(4))) const u32x4_t kconst_u4;
    kconst_u4 *cs_row = (kconst_u4 *)((__attribute__((address_space(4))) const char *)
                                          __builtin_amdgcn_kernarg_segment_ptr() + __builtin_offsetof(DecodeArgs, rope_row));
    auto cs_words = [&](int i) __attribute__((always_inline)) {
        const u32x4_t w = cs_row[i];
        return make_uint4(w.x, w.y, w.z, w.w);
    };
    bf16x8_t qreg[G::KCH];
#pragma unroll
    for (int kc = 0; kc < G::KCH; ++kc) {
        uint4 lo = *reinterpret_cast<const uint4 *>(qrow + 8 * kc);
        uint4 hi = *reinterpret_cast<const uint4 *>(qrow + D / 2 + 8 * kc);
        if constexpr (ROPE) {
            const uint4 cq = cs_words(kc);
            const uint4 sq = cs_words(G::PG + kc);
            rope_rotate8(lo, hi, cq, sq);
        }
        qreg[kc] = __builtin_bit_cast(bf16x8_t, g == 0 ? lo : hi);
    }
    // The query loads are complete before the first direct load is issued
    // (the compiler's own wait counts do not see the direct loads).
    wait_vmcnt<0>();

    // ---- K / V tiles: direct loads into this wave's ring ------------------
    const size_t kv_head = ((size_t)b * L * a.Hkv + hk) * D;
    const uint32_t kv_rowb = (uint32_t)a.Hkv * D * 2;
    const u32x4_t k_rs = make_desc(a.k + kv_head, (uint32_t)L * kv_rowb);
    const u32x4_t v_rs = make_desc(a.v + kv_head, (uint32_t)L * kv_rowb);
    uint8_t *ring = smem + wave * G::WAVE_B;
    auto kslot = [&](int t) { return ring + (t & 1) * (2 * G::TILE_B); };
    auto vslot = [&](int t) { return ring + (t & 1) * (2 * G::TILE_B) + G::TILE_B; };
    const int dl_row = lane / G::CH, dl_slot = lane % G::CH;
    // Window: lane r holds w[r] (pairs past D/2: never pruned).
    typedef __attribute__((address_space(4))) const int32_t kconst_i32;
    kconst_i32 *wtab = (kconst_i32 *)((__attribute__((address_space(4))) const char *)
                                          __builtin_amdgcn_kernarg_segment_ptr() + __builtin_offsetof(DecodeArgs, window));
    const int w_lane = (WINDOW && lane < D / 2) ? wtab[lane] : INT_MAX;

    // With a window, the K columns of an 8-pair group pruned on the whole
    // tile are not fetched ("ATFlash", the out-of-window prefix never enters
    // on-chip memory): their lanes get an offset past the buffer, which
    // loads zeros without a memory access.
    auto load_tile = [&](int t) __attribute__((always_inline)) {
        const int m0 = m_begin + t * kDecBN;
        uint64_t gpr = 0;   // pairs pruned on the whole tile
        if constexpr (WINDOW) gpr = __builtin_amdgcn_ballot_w64(w_lane < max(0, pos - (m0 + kDecBN - 1)));
#pragma unroll
        for (int ins = 0; ins < G::NI; ++ins) {
            const int r = ins * G::RPI + dl_row;
            const uint32_t row = (uint32_t)(m0 + r) * kv_rowb;
            const int kc = dl_slot ^ G::kx(r);   // chunk of the row: pair group kc % PG
            uint32_t koff = row + 16u * (uint32_t)kc;
            if constexpr (WINDOW)
                if (((gpr >> (8 * (kc % G::PG))) & 0xffu) == 0xffu) koff = 0x80000000u;
            dma16(k_rs, koff, kslot(t) + ins * 1024);
            dma16(v_rs, row + 16u * (uint32_t)(dl_slot ^ G::vx(r)), vslot(t) + ins * 1024);
        }
    };

    int k_addr[G::KCH];
#pragma unroll
    for (int kc = 0; kc < G::KCH; ++kc) k_addr[kc] = G::k_off(l32, kc + G::PG * g);
    const int tr_key = (lane & 15) >> 2;
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    int v_addr[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
        v_addr[db] = G::v_off(4 * g + tr_key, (32 * db + tr_dim) >> 3) + 2 * (tr_dim & 4);

    f32x16_t acc_o[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[db][i] = 0.f;
    float m_run = -__builtin_inff(), l_run = 0.f;

    if (T > 0) load_tile(0);
    if (T > 1) load_tile(1);
    for (int t = 0; t < T; ++t) {
        if (t + 1 < T) wait_vmcnt<2 * G::NI>();   // tile t has landed; tile t+1 may fly
        else wait_vmcnt<0>();
        const int m0 = m_begin + t * kDecBN;
        const uint32_t kbase = lds_addr(kslot(t));

        // S^T = K Q'^T over the tile's 32 keys.
        f32x16_t s;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
        uint64_t wprune = 0, wkeep = ~0ull;
        if constexpr (WINDOW) {
            // distances pos - m of the tile's keys lie in [dlo, dhi]
            const int dlo = max(0, pos - (m0 + kDecBN - 1)), dhi = pos - m0;
            wprune = __builtin_amdgcn_ballot_w64(w_lane < dlo);
            wkeep = ~__builtin_amdgcn_ballot_w64(w_lane < dhi);
        }
#pragma unroll
        for (int kc = 0; kc < G::KCH; ++kc) {
            bf16x8_t kop = *(const lds_bf16x8_t *)lds_ptr(kbase + (uint32_t)k_addr[kc]);
            if constexpr (WINDOW) {
                if (((wprune >> (8 * kc)) & 0xffu) == 0xffu) continue;   // pruned on the whole tile
                kop = apply_mask(kop, pair_mask(wkeep, kc));
            }
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[kc], s, 0, 0, 0);
        }
        if constexpr (WINDOW) {
            // Pairs whose limit falls inside the tile: one MFMA each, counted
            // where pos - m <= w[r].
            uint64_t part = ~(wprune | wkeep);
            while (part) {
                const int r = __builtin_ctzll(part);
                part &= part - 1;
                const int kc = r >> 3, j = r & 7;
                const int w = __builtin_amdgcn_readlane(w_lane, r);
                const bf16x8_t ka = mask_pairs(*(const lds_bf16x8_t *)lds_ptr(kbase + (uint32_t)k_addr[kc]), 1u << j);
                f32x16_t one{};
#pragma unroll
                for (int c2 = 0; c2 < G::KCH; ++c2)
                    if (kc == c2) one = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[c2], f32x16_t{}, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int m = m0 + 8 * (e >> 2) + 4 * g + (e & 3);
                    s[e] += (pos - m <= w) ? one[e] : 0.0f;
                }
            }
        }
        // keys past the split (and past L) do not exist
        if (m0 + kDecBN > m_end) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + 8 * (e >> 2) + 4 * g + (e & 3);
                s[e] = (m < m_end) ? s[e] : -__builtin_inff();
            }
        }

        // Online softmax for the lane's column (exact: new max every tile).
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == m_run) ? 1.0f : fast_exp2((m_run - m_new) * c);
        m_run = m_new;
        const float nmc = -m_new * c;
        // P in bf16 for the PV MFMAs; the row sum adds the fp32 P (two
        // independent chains) as the prefill kernel does.
        bf16x8_t pf[2];
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            uint32_t w4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(__builtin_fmaf(s[8 * ch + 2 * e], c, nmc));
                const float p1 = fast_exp2(__builtin_fmaf(s[8 * ch + 2 * e + 1], c, nmc));
                w4[e] = pack_bf16x2(p0, p1);
                rs0 += p0;
                rs1 += p1;
            }
            pf[ch] = __builtin_bit_cast(bf16x8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
        }
        l_run = l_run * alpha + (rs0 + rs1);

        // O^T = alpha O^T + V^T P^T.
        const uint32_t vbase = lds_addr(vslot(t));
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int db = 0; db < G::DB; ++db) {
                const lds_u8_t *p0 = lds_ptr(vbase + (uint32_t)v_addr[db]) + 16 * ch * G::ROWB;
                const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
                const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p0 + 8 * G::ROWB));
                const uint2 u0 = __builtin_bit_cast(uint2, t0), u1 = __builtin_bit_cast(uint2, t1);
                const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y));
                acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[ch], acc_o[db], 0, 0, 0);
            }

        // The slot of tile t is free once its LDS reads have returned.
        if (t + 2 < T) {
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): every LDS read of this wave done
            load_tile(t + 2);
        }
    }
    wait_vmcnt<0>();

    // ---- partial result of this split: columns 0 .. grp-1 are the heads ---
    const float l_tot = sum_halves(l_run);
    if (l32 >= grp) return;
    const size_t pidx = ((size_t)b * a.Hq + hq) * a.n_split + split;
    float *po = a.part_o + pidx * D;
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<float4 *>(po + 32 * db + 8 * r + 4 * g) =
                make_float4(acc_o[db][4 * r], acc_o[db][4 * r + 1], acc_o[db][4 * r + 2], acc_o[db][4 * r + 3]);
    if (g == 0) *reinterpret_cast<float2 *>(a.part_ml + pidx * 2) = make_float2(m_run, l_tot);
}

// Phase 2: merge the splits of one (b, hq) through their log-sum-exp: the
// max M of the split maxima, the weights 2^((m_s - M) c) of the splits, the
// weighted sums of l and of the partial outputs.
constexpr int kCombThreads = 256;
constexpr int kCombDims = 32;   // output dims per combine work-group

// Max or sum of x over the work-group: within each wave by lane shuffles,
// then over the waves through LDS (one barrier).
__device__ __forceinline__ float wg_reduce(float x, float *red, bool is_max)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float y = __shfl_xor(x, off, 64);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    const int tid = threadIdx.x;
    if ((tid & 63) == 0) red[tid >> 6] = x;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kCombThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    __syncthreads();   // red is reused by the next reduction
    return r;
}

// One work-group per (sequence, query head, 32-dim slice of the output): the
// split weights 2^((m_s - M) c) and l = sum_s w_s l_s are formed in every
// slice's work-group (a few KB of partials), then 8 groups of 32 threads
// each sum a strided share of the splits for the slice's dims, all their
// loads in flight at once.
template <int D>
__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(const DecodeArgs a)
{
    constexpr int NG = kCombThreads / kCombDims;
    __shared__ float red[kCombThreads / 64];
    __shared__ float wsh[kMaxDecodeSplits];
    __shared__ float accs[NG][kCombDims];
    const int bh = blockIdx.x, d0 = blockIdx.y * kCombDims, tid = threadIdx.x;
    const int ns = a.n_split;
    const float c = a.scale_log2e;
    const float *ml = a.part_ml + (size_t)bh * ns * 2;
    const float *po = a.part_o + (size_t)bh * ns * D;

    float mloc = -__builtin_inff();
    for (int s = tid; s < ns; s += kCombThreads) mloc = fmaxf(mloc, ml[2 * s]);
    const float M = wg_reduce(mloc, red, true);
    float lloc = 0.f;
    for (int s = tid; s < ns; s += kCombThreads) {
        const float ms = ml[2 * s];
        const float w = (ms == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f((ms - M) * c);   // empty split: 0
        wsh[s] = w;
        lloc += w * ml[2 * s + 1];
    }
    const float lsum = wg_reduce(lloc, red, false);   // its barriers also publish wsh

    const int j = tid / kCombDims, d = tid % kCombDims;
    const float *pd = po + d0 + d;
    float acc0 = 0.f, acc1 = 0.f;
    int s = j;
#pragma unroll 8
    for (; s + NG < ns; s += 2 * NG) {
        acc0 += wsh[s] * pd[(size_t)s * D];
        acc1 += wsh[s + NG] * pd[(size_t)(s + NG) * D];
    }
    if (s < ns) acc0 += wsh[s] * pd[(size_t)s * D];
    accs[j][d] = acc0 + acc1;
    __syncthreads();
    if (tid < kCombDims) {
        float t = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < NG; ++g2) t += accs[g2][tid];
        a.o[(size_t)bh * D + d0 + tid] = (uint16_t)(pack_bf16x2(t / lsum, 0.f) & 0xffffu);
        if (a.lse != nullptr && tid == 0 && blockIdx.y == 0)
            a.lse[bh] = (M * c + __builtin_amdgcn_logf(lsum)) * 0.693147180559945309f;
    }
}

template <int D, bool ROPE, bool WINDOW>
hipError_t launch_split(const DecodeArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.n_split + kDecWaves - 1) / kDecWaves), (unsigned)a.Hkv, (unsigned)a.B);
    hipLaunchKernelGGL((decode_split_kernel<D, ROPE, WINDOW>), grid, dim3(kDecWaves * 64), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t stream)
{
    const bool rope = a.use_rope != 0;
    hipError_t e;
    if (rope) e = a.use_window ? launch_split<D, true, true>(a, stream) : launch_split<D, true, false>(a, stream);
    else e = a.use_window ? launch_split<D, false, true>(a, stream) : launch_split<D, false, false>(a, stream);
    if (e != hipSuccess) return e;
    static_assert(D % kCombDims == 0, "combine slices");
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(a.B * a.Hq), (unsigned)(D / kCombDims)), dim3(kCombThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    return a.D == 128 ? launch_d<128>(a, stream) : launch_d<64>(a, stream);
}

// ---- static scratch of the split partials ----------------------------------
// For callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid hipMalloc): attn_decode_noalloc keeps the partial
// outputs and (m, l) pairs here instead of in a caller workspace.  Every GPU
// that loads the library holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not the device memory: its
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is handed to kernels.
namespace {
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];
std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;
}  // namespace

hipError_t decode_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return e != hipSuccess ? e : hipErrorInvalidSymbol;
        }
        it = g_scratch_ptr.emplace(dev, p).first;
    }
    *ptr = it->second;
    return hipSuccess;
}

}  // namespace attn
