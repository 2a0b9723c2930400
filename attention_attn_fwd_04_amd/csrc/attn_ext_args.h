// attn_ext_args.h -- kernel arguments and launchers of the split-KV decode
// (attn_decode.hip) and of the attention backward (attn_bwd.hip), shared
// with the host API (attn_api.cpp).  Kept apart from attn_internal.h so that
// the prefill kernel's sources do not change with them.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {

// Most splits of one decode: the merge keeps one weight per split in LDS.
constexpr int kMaxDecodeSplits = 1024;

struct DecodeArgs {
    const uint16_t *q;        // [B, Hq, D]
    const uint16_t *k;        // [B, L, Hkv, D] cache
    const uint16_t *v;
    uint16_t *o;              // [B, Hq, D]
    float *lse;               // [B, Hq] or null
    float *part_o;            // [B, Hq, n_split, D] partial (unnormalised) outputs
    float *part_ml;           // [B, Hq, n_split, 2] partial (m, l)
    int B, Hq, Hkv, L, D;
    int n_split, keys_per_split;
    int use_window;
    int use_rope;
    float scale_log2e;
    int32_t window[kMaxPairs];
    // With RoPE: the fp16 cosines, then sines, of the query's position L-1,
    // in the cos/sin table's row layout (pair group g: cos of pairs 8g..8g+7
    // at halves 8g.., their sines at D/2 + 8g..), the same bits the table
    // holds.  Passed by value, so decode reads no table.
    alignas(16) uint16_t rope_row[2 * kMaxPairs];
};

// Static device scratch of the split partials for the entry point that
// allocates nothing (attn_decode.hip): its size, and its address on the
// current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void **ptr);

struct BwdArgs {
    const uint16_t *q;        // [B, S, Hq, D]
    const uint16_t *k;        // [B, S, Hkv, D]
    const uint16_t *v;
    const uint16_t *o;        // forward output [B, S, Hq, D]
    const uint16_t *dout;     // dL/dO [B, S, Hq, D]
    const float *lse;         // [B, Hq, S] natural-log LSE of the forward's rows
    uint16_t *dq;             // [B, S, Hq, D]
    uint16_t *dk;             // [B, S, Hkv, D]
    uint16_t *dv;
    uint16_t *qs;             // workspace [B, S, Hq, D]: bf16(scale log2e R(n) q)
    uint16_t *kr;             // workspace [B, S, Hkv, D]: bf16(R(m) k); unused without RoPE
    const uint16_t *kop;      // the K operand: kr with RoPE, k without
    float *delta;             // workspace [B, Hq, S]: rowsum(dO o O)
    float *part_dk;           // workspace [split, B, S, Hkv, D] fp32 partial dK, dV when split > 1
    float *part_dv;
    int split;                // dK/dV work-groups per (key tile, KV head), each over Hq/Hkv/split query heads
    const uint16_t *rope_cs;  // fp16 cos/sin table; null when RoPE is off
    int B, Hq, Hkv, S, D;
    int causal;
    float scale;
    float scale_log2e;
};

// Launchers.  Return hipSuccess or the launch error.
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_attn_bwd(const BwdArgs &a, hipStream_t stream);

}  // namespace attn
