// attn_api.cpp -- host side of the C ABI declared in include/attn.h:
// argument validation, the per-device RoPE cos/sin table cache, dispatch to
// the gfx950 kernels, and the host-only window helpers.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "attn_internal.h"
#include "attn_ext_args.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Fault injection for tests of the error path: with ATTN_INJECT_LAUNCH_ERROR=1
// in the environment (read once per process), every entry point that would
// launch a kernel returns ATTN_ELAUNCH at that point instead, after all its
// checks and set-up, without launching anything.
bool inject_launch_error()
{
    static const bool on = [] {
        const char *e = std::getenv("ATTN_INJECT_LAUNCH_ERROR");
        return e != nullptr && e[0] == '1' && e[1] == '\0';
    }();
    return on;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int check_shapes(int B, int Hq, int Hkv, int S, int D)
{
    if (B < 0 || S < 0 || Hq < 1 || Hkv < 1) return ATTN_EINVAL;
    if (Hq % Hkv != 0) return ATTN_EINVAL;
    if (D != 64 && D != 128) return (D > 0 && D % 2 == 0) ? ATTN_EUNSUPPORTED : ATTN_EINVAL;
    // Element offsets must fit the kernels' 32-bit block indexing and size_t.
    const long long rows = (long long)B * S * (long long)(Hq > Hkv ? Hq : Hkv);
    if (rows > (1LL << 40)) return ATTN_EINVAL;
    const long long q_tiles = ((long long)S + 255) / 256;
    if (q_tiles * Hq * (long long)B > 0x7fffffffLL) return ATTN_EINVAL;
    // The kernels address one head's rows (and the cos/sin table) through
    // 32-bit buffer offsets.
    const long long head_span = (long long)S * (Hq > Hkv ? Hq : Hkv) * D * 2;
    if (head_span > 0x7fffffffLL || (long long)S * D * 2 > 0x7fffffffLL) return ATTN_EUNSUPPORTED;
    return ATTN_OK;
}

int check_theta(float rope_theta)
{
    if (rope_theta == 0.0f) return ATTN_OK;
    if (!std::isfinite(rope_theta) || !(rope_theta > 1.0f)) return ATTN_EINVAL;
    return ATTN_OK;
}

// ---- device check ---------------------------------------------------------
std::mutex g_mu;
std::map<int, bool> g_dev_ok;

int current_device_ok(int *dev_out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ENODEVICE;
    *dev_out = dev;
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_dev_ok.find(dev);
    if (it == g_dev_ok.end()) {
        hipDeviceProp_t prop;
        bool ok = false;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
            ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        it = g_dev_ok.emplace(dev, ok).first;
    }
    return it->second ? ATTN_OK : ATTN_ENODEVICE;
}

// ---- RoPE cos/sin tables ---------------------------------------------------
// Built in fp64 on the host and stored rounded to fp16 (layout documented on
// attn::RopeTable).  One table per (device, D, theta), grown on demand;
// replaced tables are kept until attn_release because work already enqueued
// may still read them.
struct TableKey {
    int dev, D;
    uint32_t theta_bits;
    bool operator<(const TableKey &o) const
    {
        return std::tie(dev, D, theta_bits) < std::tie(o.dev, o.D, o.theta_bits);
    }
};
std::map<TableKey, attn::RopeTable> g_tables;
std::vector<std::pair<int, void *>> g_retired;

// Round a value in [-1, 1] from fp64 to the nearest fp16 (ties to even),
// returning its bit pattern.  One rounding step: the value is scaled by the
// fp16 quantum of its binade (2^-24 in the subnormal range) and rounded there.
uint16_t fp16_bits_rne(double x)
{
    if (x == 0.0) return std::signbit(x) ? 0x8000u : 0u;
    int e;
    std::frexp(x, &e);                  // |x| = m * 2^e, 0.5 <= m < 1
    int qexp = e - 11;                  // 11 significant bits
    if (qexp < -24) qexp = -24;         // subnormal quantum
    const double q = std::ldexp(1.0, qexp);
    const double r = std::nearbyint(x / q) * q;  // exact scaling, RNE rounding
    const float f = (float)r;           // exactly representable in fp16 and fp32
    uint32_t u;
    std::memcpy(&u, &f, sizeof u);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const int fe = (int)((u >> 23) & 0xff) - 127;
    const uint32_t mant = u & 0x7fffffu;
    if (fe >= -14) return (uint16_t)(sign | ((uint32_t)(fe + 15) << 10) | (mant >> 13));
    // subnormal fp16: value = mant' * 2^-24
    const uint32_t full = (mant | 0x800000u) >> (-14 - fe);
    return (uint16_t)(sign | (full >> 13));
}

// One position's row of the cos/sin table (D halves): quarter 0 holds the
// cosines, quarter 1 the sines, pair r = 8 grp + e at half grp * 8 + e of its
// quarter (see attn::RopeTable).  The angle is p * theta^(-2r/D) in fp64.
void rope_inv_freq(float theta, int D, double *inv_freq)
{
    const double th = (double)theta;
    for (int r = 0; r < D / 2; ++r) inv_freq[r] = std::pow(th, -2.0 * (double)r / (double)D);
}
void rope_row(const double *inv_freq, int D, int p, uint16_t *row)
{
    const int PG = D / 16;
    for (int r = 0; r < D / 2; ++r) {
        const double ang = (double)p * inv_freq[r];
        const int grp = r / 8, e = r % 8;
        row[(0 * PG + grp) * 8 + e] = fp16_bits_rne(std::cos(ang));
        row[(1 * PG + grp) * 8 + e] = fp16_bits_rne(std::sin(ang));
    }
}

int get_table(int dev, int D, float theta, int S, const uint16_t **out)
{
    uint32_t bits;
    std::memcpy(&bits, &theta, sizeof bits);
    std::lock_guard<std::mutex> lk(g_mu);
    attn::RopeTable &t = g_tables[TableKey{dev, D, bits}];
    if (t.cs != nullptr && t.capacity >= S) {
        *out = t.cs;
        return ATTN_OK;
    }
    const int cap = ((S + 1023) / 1024) * 1024;
    std::vector<uint16_t> host((size_t)cap * D);
    double inv_freq[attn::kMaxPairs];
    rope_inv_freq(theta, D, inv_freq);
    for (int p = 0; p < cap; ++p) rope_row(inv_freq, D, p, host.data() + (size_t)p * D);
    void *dptr = nullptr;
    if (hipMalloc(&dptr, host.size() * sizeof(uint16_t)) != hipSuccess) {
        (void)hipGetLastError();
        return ATTN_ENOMEM;
    }
    if (hipMemcpy(dptr, host.data(), host.size() * sizeof(uint16_t), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(dptr);
        return ATTN_ELAUNCH;
    }
    if (t.cs != nullptr) g_retired.emplace_back(dev, const_cast<uint16_t *>(t.cs));
    t.cs = static_cast<const uint16_t *>(dptr);
    t.capacity = cap;
    *out = t.cs;
    return ATTN_OK;
}

// ---- persistent schedule ("Croqtile", "Step 4") ------------------------------
// Task j = qt | hq << 12 | b << 22 for the 256-row query tile qt of head hq
// of batch b.  The list holds bins + 1 bin offsets, then the tasks bin by bin.
constexpr int kSchedTileRows = 256, kSchedKeyTile = 64;

bool sched_fits(int B, int Hq, int S)
{
    return (S + kSchedTileRows - 1) / kSchedTileRows <= 4096 && Hq <= 1024 && B <= 1024;
}

// Cost of causal query tile qt: the 64-key tiles it visits plus 2 for its Q
// load and epilogue (the pages' 2(bm + 1) + c, in this kernel's tile units).
long long tile_cost(int qt, int S)
{
    const long long keys = std::min<long long>(S, (long long)(qt + 1) * kSchedTileRows);
    return (keys + kSchedKeyTile - 1) / kSchedKeyTile + 2;
}

// Heads per band of the task list: about 64 query tiles per band (one head
// at S = 16k, two at 8k, eight at 2k), as in attn_fwd's own work order.
int sched_band_heads(int n_qt) { return std::max(1, 64 / n_qt); }

// Bins are the work-groups of the launch; work-group g runs on XCD g % 8.
// When the head count and the bin count are multiples of 8, XCD x takes the
// heads [x n_bh / 8, (x + 1) n_bh / 8) (their K and V then stay in its L2);
// otherwise one group spans all bins.  Within a group the heads go in bands;
// band by band, the band's tasks go longest first to the bin with the least
// work so far (lowest index on ties).  A bin runs its tasks in the order they
// were dealt: band by band, so all bins of an XCD work on the same few heads
// at a time, and within a band longest first.
std::vector<uint32_t> build_schedule(int B, int Hq, int S, int bins)
{
    const int n_qt = (S + kSchedTileRows - 1) / kSchedTileRows;
    const long long n_bh = (long long)B * Hq;
    const long long n_tasks = n_bh * n_qt;
    if (bins > n_tasks) bins = (int)n_tasks;
    const int n_groups = (n_bh % 8 == 0 && bins % 8 == 0) ? 8 : 1;
    const int kb = sched_band_heads(n_qt);
    std::vector<std::vector<uint32_t>> bin_tasks(bins);
    std::vector<long long> load(bins, 0);
    for (int x = 0; x < n_groups; ++x) {
        const long long h0 = x * n_bh / n_groups, h1 = (x + 1) * n_bh / n_groups;
        for (long long hb = h0; hb < h1; hb += kb) {
            std::vector<std::pair<long long, uint32_t>> ts;
            for (long long bh = hb; bh < std::min(h1, hb + kb); ++bh) {
                const uint32_t b = (uint32_t)(bh / Hq), hq = (uint32_t)(bh % Hq);
                for (int qt = n_qt - 1; qt >= 0; --qt)
                    ts.emplace_back(tile_cost(qt, S), (uint32_t)qt | hq << 12 | b << 22);
            }
            std::stable_sort(ts.begin(), ts.end(),
                             [](const std::pair<long long, uint32_t> &u, const std::pair<long long, uint32_t> &v) {
                                 return u.first > v.first;
                             });
            for (const auto &t : ts) {
                int best = x;
                for (int g = x; g < bins; g += n_groups)
                    if (load[g] < load[best]) best = g;
                bin_tasks[best].push_back(t.second);
                load[best] += t.first;
            }
        }
    }
    std::vector<uint32_t> out;
    out.reserve((size_t)bins + 1 + (size_t)n_tasks);
    out.push_back(0);
    for (int g = 0; g < bins; ++g) out.push_back(out.back() + (uint32_t)bin_tasks[g].size());
    for (int g = 0; g < bins; ++g) out.insert(out.end(), bin_tasks[g].begin(), bin_tasks[g].end());
    return out;
}

// Every index the kernel derives from the list stays in range: offsets rise
// from 0 to the task count, and each (b, hq, qt) of the call is there once.
bool check_schedule(const std::vector<uint32_t> &l, int B, int Hq, int S, int bins)
{
    const int n_qt = (S + kSchedTileRows - 1) / kSchedTileRows;
    const long long n_tasks = (long long)B * Hq * n_qt;
    if (bins < 1 || (long long)l.size() != bins + 1 + n_tasks || l[0] != 0 || (long long)l[bins] != n_tasks)
        return false;
    for (int g = 0; g < bins; ++g)
        if (l[g + 1] < l[g]) return false;
    std::vector<uint8_t> seen((size_t)n_tasks, 0);
    for (long long j = 0; j < n_tasks; ++j) {
        const uint32_t t = l[(size_t)(bins + 1 + j)];
        const uint32_t qt = t & 4095u, hq = (t >> 12) & 1023u, b = t >> 22;
        if ((int)qt >= n_qt || (int)hq >= Hq || (int)b >= B) return false;
        uint8_t &f = seen[((size_t)b * Hq + hq) * n_qt + qt];
        if (f) return false;
        f = 1;
    }
    return true;
}

struct SchedKey {
    int dev, B, Hq, S;
    bool operator<(const SchedKey &o) const { return std::tie(dev, B, Hq, S) < std::tie(o.dev, o.B, o.Hq, o.S); }
};
struct SchedList {
    const uint32_t *d = nullptr;
    int bins = 0;
};
std::map<SchedKey, SchedList> g_sched;

// The device copy of the task list for (dev, B, Hq, S) over one bin per
// compute unit, built on first use.
int get_schedule(int dev, int B, int Hq, int S, const uint32_t **out, int *bins_out)
{
    std::lock_guard<std::mutex> lk(g_mu);
    SchedList &e = g_sched[SchedKey{dev, B, Hq, S}];
    if (e.d == nullptr) {
        int n_cu = 0;
        if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1) {
            (void)hipGetLastError();
            return ATTN_ENODEVICE;
        }
        const std::vector<uint32_t> l = build_schedule(B, Hq, S, n_cu);
        const int bins = (int)(l.size() - 1 - (size_t)B * Hq * ((S + kSchedTileRows - 1) / kSchedTileRows));
        if (!check_schedule(l, B, Hq, S, bins)) return ATTN_EINVAL;
        void *dptr = nullptr;
        if (hipMalloc(&dptr, l.size() * sizeof(uint32_t)) != hipSuccess) {
            (void)hipGetLastError();
            return ATTN_ENOMEM;
        }
        if (hipMemcpy(dptr, l.data(), l.size() * sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipFree(dptr);
            return ATTN_ELAUNCH;
        }
        e.d = static_cast<const uint32_t *>(dptr);
        e.bins = bins;
    }
    *out = e.d;
    *bins_out = e.bins;
    return ATTN_OK;
}

int check_window(const int32_t *w, int D, int causal)
{
    if (w == nullptr) return ATTN_OK;
    if (!causal) return ATTN_EINVAL;
    if (D / 2 > attn::kMaxPairs) return ATTN_EUNSUPPORTED;
    for (int r = 0; r + 1 < D / 2; ++r)
        if (w[r + 1] < w[r]) return ATTN_EINVAL;
    return ATTN_OK;
}

int fwd_common(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int S,
               int D, float rope_theta, int causal, float scale, const int32_t *window_table, void *stream,
               bool persistent = false, bool k_rotated = false)
{
    int st = attn_check_args(q, k, v, o, B, Hq, Hkv, S, D, rope_theta, causal, scale, window_table);
    if (st != ATTN_OK) return st;
    if (k_rotated && rope_theta == 0.0f) return ATTN_EINVAL;   // the query is rotated: theta > 1
    if (persistent && (window_table != nullptr || !sched_fits(B, Hq, S))) return ATTN_EUNSUPPORTED;
    int dev = -1;
    st = current_device_ok(&dev);
    if (st != ATTN_OK) return st;
    if (B == 0 || S == 0) return ATTN_OK;

    attn::FwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = static_cast<uint16_t *>(o);
    a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S; a.D = D;
    a.causal = causal;
    a.scale_log2e = (float)((double)scale * 1.4426950408889634073599246810019);
    if (window_table) {
        a.use_window = 1;
        for (int r = 0; r < D / 2; ++r) a.window[r] = window_table[r];
    }
    if (rope_theta != 0.0f) {
        st = get_table(dev, D, rope_theta, S, &a.rope_cs);
        if (st != ATTN_OK) return st;
        a.rope_k = k_rotated ? 0 : 1;
    }
    if (persistent && causal) {
        st = get_schedule(dev, B, Hq, S, &a.sched, &a.sched_bins);
        if (st != ATTN_OK) return st;
    }
    if (inject_launch_error() || attn::launch_attn_fwd(a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return ATTN_ELAUNCH;
    return ATTN_OK;
}

// Split count of attn_decode: num_splits > 0 as asked (at most one split per
// 32 keys and at most kMaxDecodeSplits), otherwise enough splits for about
// 1024 waves over the whole batch (one resident round at four waves per CU),
// each split at least 64 keys.  Keys per split are a multiple of 32,
// and every split is non-empty.
void decode_plan(int B, int Hkv, int L, int num_splits, int *n_split, int *keys_per_split)
{
    const int max_split = (L + 31) / 32;
    int n = num_splits;
    if (n <= 0) {
        const long long groups = (long long)B * Hkv;
        long long want = (1024 + groups - 1) / (groups > 0 ? groups : 1);
        const int cap = (L + 63) / 64;
        if (want > cap) want = cap;
        n = (int)(want < 1 ? 1 : want);
    }
    if (n > max_split) n = max_split;
    if (n > attn::kMaxDecodeSplits) n = attn::kMaxDecodeSplits;
    if (n < 1) n = 1;
    int kps = (L + n - 1) / n;
    kps = (kps + 31) / 32 * 32;
    *keys_per_split = kps;
    *n_split = (L + kps - 1) / kps;
}

// Work-groups of attn_bwd's dK/dV kernel per (256-key tile, KV head): the
// group's query heads are split over separate work-groups (fp32 partial sums,
// then a reduction) when the unsplit grid would be under four rounds of
// resident work-groups (1 per CU on 256 CUs); the finer work-groups balance
// better over the CUs.
int bwd_split(int B, int Hq, int Hkv, int S)
{
    const int grp = Hq / Hkv;
    if (grp <= 1) return 1;
    const long long grid = ((long long)S + 255) / 256 * Hkv * (long long)B;
    return grid < 4 * 256 ? grp : 1;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

extern "C" {

const char *attn_strerror(int status)
{
    switch (status) {
    case ATTN_OK: return "success";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported configuration (head dimension must be 64 or 128)";
    case ATTN_EALIGN: return "pointer not aligned (tensors: 16 bytes, lse: 4 bytes)";
    case ATTN_ENOMEM: return "device allocation failed";
    case ATTN_ELAUNCH: return "HIP runtime error while launching or copying";
    case ATTN_ENODEVICE: return "no gfx950 HIP device is current";
    case ATTN_ESCRATCH: return "the call needs more memory than the library's static scratch holds";
    default: return "unknown status";
    }
}

int attn_check_args(const void *q, const void *k, const void *v, const void *o, int B, int Hq, int Hkv,
                    int S, int D, float rope_theta, int causal, float scale, const int32_t *window_table)
{
    int st = check_shapes(B, Hq, Hkv, S, D);
    if (st != ATTN_OK) return st;
    const bool empty = (B == 0 || S == 0);  // nothing is read or written: pointers may be NULL
    if (!empty && (!q || !k || !v || !o)) return ATTN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_EALIGN;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return ATTN_EINVAL;
    st = check_theta(rope_theta);
    if (st != ATTN_OK) return st;
    const size_t nq = (size_t)B * S * Hq * D * 2, nkv = (size_t)B * S * Hkv * D * 2;
    if (!empty && (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv)))
        return ATTN_EINVAL;
    return check_window(window_table, D, causal);
}


int attn_fwd(const void *q, const void *k, const void *v, void *o, int B, int Hq, int Hkv, int S, int D,
             float rope_theta, int causal, float scale, const int32_t *window_table, void *stream)
{
    return fwd_common(q, k, v, o, nullptr, B, Hq, Hkv, S, D, rope_theta, causal, scale, window_table, stream);
}

int attn_fwd_lse(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int S,
                 int D, float rope_theta, int causal, float scale, const int32_t *window_table, void *stream)
{
    const bool empty = (B <= 0 || S <= 0);
    if (!empty) {
        if (lse == nullptr) return ATTN_EINVAL;
        if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_EALIGN;
        if (B > 0 && Hq > 0 && S > 0 && D > 0) {
            const size_t nl = (size_t)B * Hq * S * 4, nq = (size_t)B * S * Hq * D * 2;
            const size_t nkv = (Hkv > 0) ? (size_t)B * S * Hkv * D * 2 : 0;
            if (overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv) ||
                overlaps(lse, nl, o, nq))
                return ATTN_EINVAL;
        }
    }
    return fwd_common(q, k, v, o, lse, B, Hq, Hkv, S, D, rope_theta, causal, scale, window_table, stream);
}

int attn_fwd_persistent(const void *q, const void *k, const void *v, void *o, int B, int Hq, int Hkv, int S, int D,
                        float rope_theta, int causal, float scale, const int32_t *window_table, void *stream)
{
    return fwd_common(q, k, v, o, nullptr, B, Hq, Hkv, S, D, rope_theta, causal, scale, window_table, stream, true);
}

int attn_fwd_rotated_k(const void *q, const void *k_rot, const void *v, void *o, int B, int Hq, int Hkv, int S,
                       int D, float rope_theta, int causal, float scale, const int32_t *window_table, void *stream)
{
    return fwd_common(q, k_rot, v, o, nullptr, B, Hq, Hkv, S, D, rope_theta, causal, scale, window_table, stream,
                      false, true);
}

long long attn_persistent_schedule(int B, int Hq, int S, int bins, uint32_t *out, long long cap)
{
    if (B < 1 || Hq < 1 || S < 1 || bins < 1 || out == nullptr) return ATTN_EINVAL;
    if (!sched_fits(B, Hq, S)) return ATTN_EUNSUPPORTED;
    const long long n_tasks = (long long)B * Hq * ((S + kSchedTileRows - 1) / kSchedTileRows);
    const long long used = std::min<long long>(bins, n_tasks) + 1 + n_tasks;
    if (cap < used) return ATTN_EINVAL;
    const std::vector<uint32_t> l = build_schedule(B, Hq, S, bins);
    std::memcpy(out, l.data(), l.size() * sizeof(uint32_t));
    return (long long)l.size();
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int L, int D, int num_splits)
{
    if (B <= 0 || L <= 0 || Hq < 1 || Hkv < 1 || D <= 0 || num_splits < 0) return 0;
    int n_split = 1, kps = 32;
    decode_plan(B, Hkv, L, num_splits, &n_split, &kps);
    // partial outputs, then the (m, l) pairs; 256-byte aligned sections
    const size_t po = ((size_t)B * Hq * n_split * D * 4 + 255) / 256 * 256;
    const size_t ml = (size_t)B * Hq * n_split * 2 * 4;
    return po + ml;
}

}  // extern "C"

namespace {

// attn_decode with the partials in `workspace` (caller-owned: size and
// overlap checked here), or with noalloc in the library's static scratch.
int decode_common(const void *q, const void *k, const void *v, void *o, float *lse, void *workspace,
                  size_t workspace_bytes, int B, int Hq, int Hkv, int L, int D, float rope_theta, float scale,
                  const int32_t *window_table, int num_splits, void *stream, bool noalloc)
{
    int st = check_shapes(B, Hq, Hkv, L, D);
    if (st != ATTN_OK) return st;
    if (Hq / Hkv > 32) return ATTN_EUNSUPPORTED;   // query heads per KV head: one MFMA's 32 columns
    if (num_splits < 0) return ATTN_EINVAL;
    const bool empty = (B == 0 || L == 0);
    if (!empty && (!q || !k || !v || !o || (!noalloc && !workspace))) return ATTN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (!noalloc && !aligned16(workspace)))
        return ATTN_EALIGN;
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_EALIGN;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return ATTN_EINVAL;
    st = check_theta(rope_theta);
    if (st != ATTN_OK) return st;
    st = check_window(window_table, D, 1);
    if (st != ATTN_OK) return st;
    if (empty) return ATTN_OK;
    const size_t nws = attn_decode_workspace_bytes(B, Hq, Hkv, L, D, num_splits);
    if (noalloc) {
        if (nws > attn::kDecodeScratchBytes) return ATTN_ESCRATCH;
    } else if (workspace_bytes < nws) {
        return ATTN_EINVAL;
    }
    const size_t nq = (size_t)B * Hq * D * 2, nkv = (size_t)B * L * Hkv * D * 2;
    const size_t nl = (size_t)B * Hq * 4;
    if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv))
        return ATTN_EINVAL;
    if (!noalloc && (overlaps(workspace, nws, q, nq) || overlaps(workspace, nws, k, nkv) ||
                     overlaps(workspace, nws, v, nkv) || overlaps(workspace, nws, o, nq)))
        return ATTN_EINVAL;
    if (lse && (overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv) ||
                overlaps(lse, nl, o, nq) || (!noalloc && overlaps(lse, nl, workspace, nws))))
        return ATTN_EINVAL;
    int dev = -1;
    st = current_device_ok(&dev);
    if (st != ATTN_OK) return st;
    if (noalloc && attn::decode_scratch(&workspace) != hipSuccess) return ATTN_ELAUNCH;

    attn::DecodeArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = static_cast<uint16_t *>(o);
    a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.L = L; a.D = D;
    decode_plan(B, Hkv, L, num_splits, &a.n_split, &a.keys_per_split);
    const size_t po = ((size_t)B * Hq * a.n_split * D * 4 + 255) / 256 * 256;
    a.part_o = static_cast<float *>(workspace);
    a.part_ml = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + po);
    a.scale_log2e = (float)((double)scale * 1.4426950408889634073599246810019);
    if (window_table) {
        a.use_window = 1;
        for (int r = 0; r < D / 2; ++r) a.window[r] = window_table[r];
    }
    if (rope_theta != 0.0f) {
        // the query's row of the cos/sin table (position L-1), by value
        a.use_rope = 1;
        double inv_freq[attn::kMaxPairs];
        rope_inv_freq(rope_theta, D, inv_freq);
        rope_row(inv_freq, D, L - 1, a.rope_row);
    }
    if (inject_launch_error() || attn::launch_decode(a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return ATTN_ELAUNCH;
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode(const void *q, const void *k, const void *v, void *o, float *lse, void *workspace,
                size_t workspace_bytes, int B, int Hq, int Hkv, int L, int D, float rope_theta, float scale,
                const int32_t *window_table, int num_splits, void *stream)
{
    return decode_common(q, k, v, o, lse, workspace, workspace_bytes, B, Hq, Hkv, L, D, rope_theta, scale,
                         window_table, num_splits, stream, false);
}

int attn_decode_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv,
                        int L, int D, float rope_theta, float scale, const int32_t *window_table, int num_splits,
                        void *stream)
{
    return decode_common(q, k, v, o, lse, nullptr, 0, B, Hq, Hkv, L, D, rope_theta, scale, window_table,
                         num_splits, stream, true);
}

size_t attn_decode_scratch_bytes(void) { return attn::kDecodeScratchBytes; }


// Workspace of attn_bwd: the staged queries, the staged keys, Delta, then
// (split dK/dV only) the fp32 partial dK and dV, each section 256-byte
// aligned.
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D)
{
    if (B <= 0 || S <= 0 || Hq < 1 || Hkv < 1 || D <= 0 || Hq % Hkv != 0) return 0;
    size_t n = align256((size_t)B * S * Hq * D * 2) + align256((size_t)B * S * Hkv * D * 2) +
               align256((size_t)B * Hq * S * 4);
    const int split = bwd_split(B, Hq, Hkv, S);
    if (split > 1) n += 2 * align256((size_t)split * B * S * Hkv * D * 4);
    return n;
}

int attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
             void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int S,
             int D, float rope_theta, int causal, float scale, const int32_t *window_table, void *stream)
{
    int st = check_shapes(B, Hq, Hkv, S, D);
    if (st != ATTN_OK) return st;
    if (window_table != nullptr) return ATTN_EUNSUPPORTED;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return ATTN_EINVAL;
    st = check_theta(rope_theta);
    if (st != ATTN_OK) return st;
    const bool empty = (B == 0 || S == 0);
    if (!empty && (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)) return ATTN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
        return ATTN_EALIGN;
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_EALIGN;
    if (empty) return ATTN_OK;
    const size_t nws = attn_bwd_workspace_bytes(B, Hq, Hkv, S, D);
    if (workspace_bytes < nws) return ATTN_EINVAL;
    const size_t nq = (size_t)B * S * Hq * D * 2, nkv = (size_t)B * S * Hkv * D * 2, nl = (size_t)B * Hq * S * 4;
    // Every written buffer is disjoint from every other buffer.
    const void *ins[6] = {q, k, v, o, dout, lse};
    const size_t in_n[6] = {nq, nkv, nkv, nq, nq, nl};
    void *outs[4] = {dq, dk, dv, workspace};
    const size_t out_n[4] = {nq, nkv, nkv, nws};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return ATTN_EINVAL;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return ATTN_EINVAL;
    }
    int dev = -1;
    st = current_device_ok(&dev);
    if (st != ATTN_OK) return st;

    attn::BwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = static_cast<const uint16_t *>(o);
    a.dout = static_cast<const uint16_t *>(dout);
    a.lse = lse;
    a.dq = static_cast<uint16_t *>(dq);
    a.dk = static_cast<uint16_t *>(dk);
    a.dv = static_cast<uint16_t *>(dv);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const size_t qs_b = align256(nq), kr_b = align256(nkv), dl_b = align256((size_t)B * Hq * S * 4);
    a.qs = reinterpret_cast<uint16_t *>(ws);
    a.kr = reinterpret_cast<uint16_t *>(ws + qs_b);
    a.delta = reinterpret_cast<float *>(ws + qs_b + kr_b);
    a.split = bwd_split(B, Hq, Hkv, S);
    if (a.split > 1) {
        const size_t part_b = align256((size_t)a.split * B * S * Hkv * D * 4);
        a.part_dk = reinterpret_cast<float *>(ws + qs_b + kr_b + dl_b);
        a.part_dv = reinterpret_cast<float *>(ws + qs_b + kr_b + dl_b + part_b);
    }
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S; a.D = D;
    a.causal = causal;
    a.scale = scale;
    a.scale_log2e = (float)((double)scale * 1.4426950408889634073599246810019);
    if (rope_theta != 0.0f) {
        st = get_table(dev, D, rope_theta, S, &a.rope_cs);
        if (st != ATTN_OK) return st;
        a.kop = a.kr;
    } else {
        a.kop = a.k;
    }
    if (inject_launch_error() || attn::launch_attn_bwd(a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return ATTN_ELAUNCH;
    return ATTN_OK;
}

int attn_rope_apply(const void *q, const void *k, void *q_out, void *k_out, int B, int Hq, int Hkv, int S,
                    int D, float rope_theta, void *stream)
{
    int st = check_shapes(B, Hq, Hkv, S, D);
    if (st != ATTN_OK) return st;
    const bool empty = (B == 0 || S == 0);
    // q and q_out both NULL: rotate the keys only.
    if ((q == nullptr) != (q_out == nullptr)) return ATTN_EINVAL;
    const bool with_q = q != nullptr;
    if (!empty && (!k || !k_out)) return ATTN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(q_out) || !aligned16(k_out)) return ATTN_EALIGN;
    if (rope_theta == 0.0f || check_theta(rope_theta) != ATTN_OK) return ATTN_EINVAL;
    const size_t nq = with_q ? (size_t)B * S * Hq * D * 2 : 0, nk = (size_t)B * S * Hkv * D * 2;
    if (!empty && (overlaps(k_out, nk, k, nk) ||
                   (with_q && (overlaps(q_out, nq, q, nq) || overlaps(q_out, nq, k, nk) ||
                               overlaps(k_out, nk, q, nq) || overlaps(q_out, nq, k_out, nk)))))
        return ATTN_EINVAL;
    int dev = -1;
    st = current_device_ok(&dev);
    if (st != ATTN_OK) return st;
    if (B == 0 || S == 0) return ATTN_OK;
    attn::RopeArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.q_out = static_cast<uint16_t *>(q_out);
    a.k_out = static_cast<uint16_t *>(k_out);
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S; a.D = D;
    st = get_table(dev, D, rope_theta, S, &a.rope_cs);
    if (st != ATTN_OK) return st;
    if (inject_launch_error() || attn::launch_rope_pass(a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return ATTN_ELAUNCH;
    return ATTN_OK;
}

int attn_window_table(double rope_theta, int D, double k_turns, int32_t *out_host)
{
    if (!out_host || D <= 0 || (D % 2) != 0) return ATTN_EINVAL;
    if (!std::isfinite(rope_theta) || !(rope_theta > 1.0) || !std::isfinite(k_turns) || !(k_turns > 0.0))
        return ATTN_EINVAL;
    // Pair r turns by theta^(-2r/D) per position, so one full turn takes the
    // wavelength 2*pi*theta^(2r/D) positions; the window keeps k_turns of them.
    const double pi = 3.14159265358979323846264338327950288;
    for (int r = 0; r < D / 2; ++r) {
        const double wavelength = 2.0 * pi * std::pow(rope_theta, 2.0 * (double)r / (double)D);
        const double w = std::floor(k_turns * wavelength);
        out_host[r] = (w >= 2147483647.0) ? 2147483647 : (int32_t)w;
    }
    return ATTN_OK;
}

int attn_pruned_terms(const int32_t *w_host, int D, int S, long long *per_head_out)
{
    if (!w_host || !per_head_out || D <= 0 || (D % 2) != 0 || S < 0) return ATTN_EINVAL;
    // Distance d = n - m occurs S - d times in the causal triangle; pair r is
    // removed at every distance above w[r], i.e. from d0 = w[r] + 1 to S - 1:
    // (S - d0) + ... + 1 cells.
    long long total = 0;
    for (int r = 0; r < D / 2; ++r) {
        long long d0 = (long long)w_host[r] + 1;
        if (d0 < 0) d0 = 0;
        if (d0 >= S) continue;
        const long long len = (long long)S - d0;
        total += len * (len + 1) / 2;
    }
    *per_head_out = total;
    return ATTN_OK;
}

void attn_release(void)
{
    std::lock_guard<std::mutex> lk(g_mu);
    int cur = -1;
    (void)hipGetDevice(&cur);
    auto free_on = [](int dev, void *p) {
        if (hipSetDevice(dev) == hipSuccess) (void)hipFree(p);
    };
    for (auto &kv : g_tables)
        if (kv.second.cs) free_on(kv.first.dev, const_cast<uint16_t *>(kv.second.cs));
    for (auto &r : g_retired) free_on(r.first, r.second);
    for (auto &kv : g_sched)
        if (kv.second.d) free_on(kv.first.dev, const_cast<uint32_t *>(kv.second.d));
    g_tables.clear();
    g_retired.clear();
    g_sched.clear();
    if (cur >= 0) (void)hipSetDevice(cur);
}

}  // extern "C"
