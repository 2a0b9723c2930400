/*
 * attn.h -- C ABI of the MI355X (gfx950) fused causal RoPE attention forward.
 *
 * The library computes, for every batch b, query head hq and query row n,
 *
 *   O[b,n,hq,:] = sum_m softmax_m( scale * <R(n) q[b,n,hq,:], R(m) k[b,m,hk,:]> ) v[b,m,hk,:]
 *
 * with hk = hq / (Hq / Hkv) (grouped-query heads), m ranging over 0..n under
 * the causal mask (over 0..S-1 otherwise), and R(p) the rotary position
 * embedding in the NeoX convention: dimension pair r = (r, r + D/2) turned by
 * the angle p * rope_theta^(-2r/D) ("AttnFuse: A Composable DSL for Compiling
 * Attentions to Fused GPU Kernels", section 2 "Rotary Position Embeddings"
 * and section 4.1 "Fused RoPE").  The softmax is evaluated tile by tile with
 * the online recurrence (running max m, denominator l, rescale
 * alpha = exp2((m_old - m_new) * scale * log2 e), O += P V, one division by l
 * at the end), so no S x S score matrix is ever written to memory ("Flash
 * Attention: Causal Prefill D=128", "Online softmax: what must remain
 * invariant").
 *
 * Conventions shared by every entry point:
 *  - Tensors are bf16, contiguous [B, S, H, D] ("BSHD"); q and o have Hq
 *    heads, k and v have Hkv heads.  Device pointers are owned by the caller
 *    (PyTorch allocates them); the library never frees them.  Every tensor
 *    pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously; no entry point synchronises the
 *    stream.  Kernel faults surface at the caller's next synchronisation.
 *  - All arguments are validated on the host before anything is enqueued;
 *    on error nothing is launched and a negative attn_status is returned.
 *  - Calls on one device from several host threads are safe; the library's
 *    shared host state is its cache of RoPE cos/sin tables and of persistent
 *    task lists, guarded by a mutex.  The one exception is
 *    attn_decode_noalloc, whose calls share a static device buffer: calls of
 *    it that overlap on one device race.
 */
#ifndef ATTN_MI355X_ATTN_H
#define ATTN_MI355X_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_EINVAL = -1,       /* bad argument (NULL, negative size, Hq % Hkv, scale, ...) */
    ATTN_EUNSUPPORTED = -2, /* valid but not built: D not in {64, 128} */
    ATTN_EALIGN = -3,       /* a tensor pointer is not 16-byte aligned (lse: 4-byte) */
    ATTN_ENOMEM = -4,       /* device allocation of the cos/sin table failed */
    ATTN_ELAUNCH = -5,      /* the HIP runtime refused the launch or a copy (also returned,
                               without launching, when the environment of the process sets
                               ATTN_INJECT_LAUNCH_ERROR=1: a test hook for the error path) */
    ATTN_ENODEVICE = -6,    /* no HIP device / the current device is not gfx950 */
    ATTN_ESCRATCH = -7      /* attn_decode_noalloc: the partials exceed the static scratch */
} attn_status;

/*
 * Fused causal attention forward with RoPE applied to the Q and K tiles as
 * they are staged on chip.
 *
 *  q [B,S,Hq,D], k/v [B,S,Hkv,D], o [B,S,Hq,D]: bf16 device pointers.  o must
 *      not overlap q, k or v.
 *  B >= 0, S >= 0 (either being 0 is a no-op), Hq >= 1, Hkv >= 1,
 *      Hq % Hkv == 0, D in {64, 128}.
 *  rope_theta: > 1 rotates Q and K (positions 0..S-1); 0 disables RoPE (the
 *      inputs are used as given).  Other values are rejected.
 *  causal: 1 keeps keys m <= n, 0 keeps all keys.
 *  scale: finite and > 0; multiplies q.k (natural-log softmax domain; the
 *      kernel folds log2 e into it itself).
 *  window_table: NULL, or a HOST array of D/2 int32 per-pair distance limits
 *      w[r], non-decreasing in r.  Pair r then contributes to score (n, m)
 *      only when n - m <= w[r] ("ATFlash -- Per-RoPE-Wavelength Attention
 *      Windows", "The idea").  Requires causal == 1 and D/2 <= 64.  With
 *      rope_theta == 0 the pairs are those of inputs rotated beforehand
 *      (attn_rope_apply).  The table is copied by value into the kernel
 *      arguments; the caller may free it when the call returns.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o,
             int B, int Hq, int Hkv, int S, int D,
             float rope_theta, int causal, float scale,
             const int32_t *window_table, void *stream);

/*
 * attn_fwd that also writes, for every query row, the natural-log
 * log-sum-exp of its (masked, windowed) scaled scores,
 *
 *   lse[b, hq, n] = log sum_m exp(scale * <R(n) q, R(m) k>),
 *
 * i.e. L = m + log l of the online softmax: the one value per row that a
 * forward pass keeps so that a backward pass can rebuild the softmax
 * probabilities tile by tile, and that partial results over disjoint key
 * ranges need to be merged ("AttnFuse", section 4.4 "Backward Pass" and
 * section 4.2 "Flash Decoding").
 *
 *  lse: fp32 device pointer to [B, Hq, S] (row-major, caller-owned, 4-byte
 *       aligned, not overlapping q, k, v or o); NULL is rejected unless B or
 *       S is 0.  All other arguments and errors are those of attn_fwd, and o
 *       is bitwise the same as attn_fwd's.  l is the fp32 sum of the
 *       probabilities (P V takes their bf16 roundings).
 */
int attn_fwd_lse(const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int Hq, int Hkv, int S, int D,
                 float rope_theta, int causal, float scale,
                 const int32_t *window_table, void *stream);

/*
 * attn_fwd on a persistent, cost-balanced schedule of the causal query tiles
 * ("Croqtile", "Step 4": persistent blocks fed from a task list built on the
 * host, each task costed by its position on the diagonal, tasks dealt to the
 * lightest bin, in an order that keeps K/V reuse).  One work-group per
 * compute unit runs the 256-row query tiles of its bin one after another.  A
 * tile's cost is the number of 64-key tiles it visits plus 2 (its Q load and
 * epilogue).  When B*Hq and the bin count are multiples of 8, the heads are
 * split evenly over the 8 XCDs (work-group g runs on XCD g % 8); otherwise
 * one group spans all bins.  Within a group the heads go in bands of about
 * 64 query tiles; band by band, tiles go longest first to the lightest bin,
 * and each bin runs its tiles in that order.  The list for
 * (device, B, Hq, S) is built and checked (every query tile exactly once) on
 * the first call, copied to device memory and kept until attn_release.
 *
 *  Arguments, layout and errors as attn_fwd, and o is bitwise the same as
 *  attn_fwd's.  causal == 0 runs attn_fwd's schedule (every tile then costs
 *  the same).  ATTN_EUNSUPPORTED: a window_table, or S > 1048576, Hq > 1024
 *  or B > 1024 (the task encoding).  ATTN_ENOMEM: the list's device copy
 *  could not be allocated.
 */
int attn_fwd_persistent(const void *q, const void *k, const void *v, void *o,
                        int B, int Hq, int Hkv, int S, int D,
                        float rope_theta, int causal, float scale,
                        const int32_t *window_table, void *stream);

/*
 * attn_fwd with RoPE for keys that are already rotated: the query is rotated
 * at load as in attn_fwd, the keys k_rot [B,S,Hkv,D] are taken as R(m) k
 * (attn_rope_apply with q = q_out = NULL writes them), so the key tiles are
 * neither rotated nor accompanied by cos/sin tiles in the kernel.  This is
 * "AttnFuse" section 5.3's fuse-or-pre-rotate choice made per operand: the
 * query's rotation costs one pass over Q per work-group wherever it is done,
 * while the keys' rotation inside the kernel is repeated for every query
 * tile that reads them (the O(N^2 D / BM) term of the crossover), against one
 * O(N D) pass outside it.  With keys from that pass, o is bitwise attn_fwd's.
 *
 *  rope_theta must be > 1 (the query's rotation); other arguments, layout and
 *  errors as attn_fwd.
 */
int attn_fwd_rotated_k(const void *q, const void *k_rot, const void *v, void *o,
                       int B, int Hq, int Hkv, int S, int D,
                       float rope_theta, int causal, float scale,
                       const int32_t *window_table, void *stream);

/*
 * The task list attn_fwd_persistent uses for (B, Hq, S) over `bins` bins
 * (min(bins, task count) are used), written to the HOST array out:
 * out[0 .. bins'] the bin offsets, then the tasks qt | hq << 12 | b << 22 bin
 * by bin, qt being the 256-row query tile.  Returns the number of uint32
 * written, bins' + 1 + B*Hq*ceil(S/256); ATTN_EINVAL for a bad argument or
 * cap below that, ATTN_EUNSUPPORTED beyond the limits of attn_fwd_persistent.
 * Host only: no device is touched (for tests and inspection).
 */
long long attn_persistent_schedule(int B, int Hq, int S, int bins, uint32_t *out, long long cap);

/*
 * Split-KV decode: one new query per sequence against its KV cache
 * ("AttnFuse", section 4.2 "Flash Decoding": phase 1 computes, per chunk of
 * the cache, a partial (m, l, acc) triple with the online-softmax loop;
 * phase 2 merges the partials through their log-sum-exp).  For every batch b
 * and query head hq,
 *
 *   o[b,hq,:] = sum_{m < L} softmax_m( scale * <R(L-1) q[b,hq,:], k[b,m,hk,:]> ) v[b,m,hk,:]
 *
 * with hk = hq / (Hq / Hkv).  The query is the token at position L-1 and is
 * rotated there when rope_theta > 1 (rope_theta = 0: used as given); the
 * cache holds keys as they were stored, i.e. already rotated when appended
 * (attn_rope_apply produces them).  All L keys are visible.
 *
 *  q [B,Hq,D], o [B,Hq,D]; k/v [B,L,Hkv,D] (BSHD cache): bf16 device
 *      pointers, 16-byte aligned; o must not overlap the inputs.
 *  lse: NULL, or a 4-byte aligned fp32 device array [B,Hq] that receives the
 *      natural-log log-sum-exp of each head's scaled scores.
 *  workspace: caller-owned device memory of at least
 *      attn_decode_workspace_bytes(B, Hq, Hkv, L, D, num_splits) bytes,
 *      16-byte aligned, for the partial results; its contents on entry do
 *      not matter.
 *  Hq / Hkv <= 32 (query heads sharing a KV head go into one MFMA's
 *      columns); D in {64, 128}; B >= 0, L >= 0 (either 0: no-op).
 *  window_table: NULL or a HOST array of D/2 non-decreasing int32 limits:
 *      pair r counts for key m only when (L-1) - m <= w[r] (as in attn_fwd).
 *  num_splits: 0 lets the library choose (about 1024 waves over the batch,
 *      at least 64 keys per split); k > 0 asks for k splits (at most one per
 *      32 keys, at most 1024).  Errors as for attn_fwd.
 *  The query's cos/sin row travels by value in the kernel arguments: decode
 *  reads and allocates no table.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int L, int D, int num_splits);
int attn_decode(const void *q, const void *k, const void *v, void *o, float *lse,
                void *workspace, size_t workspace_bytes,
                int B, int Hq, int Hkv, int L, int D,
                float rope_theta, float scale, const int32_t *window_table,
                int num_splits, void *stream);

/*
 * attn_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * runs the same kernels with the same arguments (and returns the same o and
 * lse bit for bit) but keeps the split partials in a static device buffer
 * of the library instead of a caller workspace, and calls no allocating
 * routine.  The caller still owns q, k, v, o and lse.
 *
 *  Limit: the partials take attn_decode_workspace_bytes(B, Hq, Hkv, L, D,
 *      num_splits) bytes, about B * Hq * splits * (4 D + 8); they must fit in
 *      attn_decode_scratch_bytes() (32 MiB).  Larger calls return
 *      ATTN_ESCRATCH and launch nothing.  For example the Llama-3-70B head
 *      shape (Hq 64, Hkv 8, D 128) with the default split plan needs 4.1 MiB
 *      at B = 1 and at B = 8.
 *  Sharing: each device holds one such buffer (it lives until the process
 *      ends), shared by every call on that device and left holding the last
 *      call's partials.  Calls that overlap on one device (concurrent streams
 *      or host threads) race on it; calls ordered on one stream do not.  The
 *      kernels write every partial they read, so nothing needs clearing.
 *  Other arguments and errors as attn_decode.
 */
int attn_decode_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                        int B, int Hq, int Hkv, int L, int D,
                        float rope_theta, float scale, const int32_t *window_table,
                        int num_splits, void *stream);
size_t attn_decode_scratch_bytes(void);

/*
 * Attention backward: the gradients of the attn_fwd loss with respect to q,
 * k and v, given dout = dL/do ("AttnFuse", section 4.4 "Backward Pass": a
 * preprocessing kernel for the row-reduced Delta = rowsum(dout o o), one
 * kernel per key tile for dK and dV, one per query tile for dQ, each writing
 * its own tile, with the softmax probabilities rebuilt from the saved
 * per-row lse).  With S(n,m) = scale <R(n) q_n, R(m) k_m> and
 * P = softmax over the visible m:
 *
 *   dv_m = sum_n P(n,m) dout_n
 *   dS(n,m) = P(n,m) (<dout_n, v_m> - Delta_n)
 *   dq_n = scale R(n)^T sum_m dS(n,m) R(m) k_m
 *   dk_m = scale R(m)^T sum_n dS(n,m) R(n) q_n
 *
 * summed over the query heads of a group for dk and dv.
 *
 *  q, k, v, o, dout: bf16 [B,S,H,D] as for attn_fwd; o is the forward's
 *      output and lse [B,Hq,S] (fp32, 4-byte aligned) the one attn_fwd_lse
 *      wrote for the same inputs and arguments.
 *  dq [B,S,Hq,D], dk, dv [B,S,Hkv,D]: bf16 outputs, overwritten (not
 *      accumulated into); they must not overlap each other, the inputs or the
 *      workspace.
 *  workspace: caller-owned device memory of at least
 *      attn_bwd_workspace_bytes(B, Hq, Hkv, S, D) bytes, 16-byte aligned
 *      (staged operands and Delta); contents on entry do not matter.
 *  window_table must be NULL (the backward of the per-pair window is not
 *      built: ATTN_EUNSUPPORTED).  Other arguments, size limits and errors as
 *      for attn_fwd (the gradient grids have at most one work-group per 256
 *      rows and query head, within attn_fwd's bound).
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D);
int attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
             const float *lse, void *dq, void *dk, void *dv,
             void *workspace, size_t workspace_bytes,
             int B, int Hq, int Hkv, int S, int D,
             float rope_theta, int causal, float scale,
             const int32_t *window_table, void *stream);

/*
 * The separate RoPE pass ("AttnFuse", section 1 and Figure 1(a): rotate Q
 * and K in their own kernel, then run plain attention): writes the rotated
 * q_out [B,S,Hq,D] and k_out [B,S,Hkv,D] (bf16, rounded to nearest even from
 * the same fp32 arithmetic the fused kernel uses: the rotated keys are the
 * fused kernel's bit for bit; the fused kernel rounds the rotated query once
 * after scaling it by scale * log2 e, attn_fwd(rope_theta = 0) on q_out
 * rounds it a second time, so the two paths agree to that rounding).
 * q_out/k_out are caller-owned workspaces that must not overlap the inputs.
 * q and q_out may both be NULL: then only the keys are rotated (for
 * attn_fwd_rotated_k).  rope_theta must be > 1.
 */
int attn_rope_apply(const void *q, const void *k, void *q_out, void *k_out,
                    int B, int Hq, int Hkv, int S, int D, float rope_theta,
                    void *stream);

/*
 * Host-only: the per-pair window table w[r] = floor(k_turns * 2*pi *
 * rope_theta^(2r/D)), r = 0..D/2-1, evaluated in fp64 (pair r's wavelength
 * times the number of full turns; "ATFlash", "The idea").  Values beyond
 * INT32_MAX saturate.  out_host holds D/2 int32.  rope_theta > 1, k_turns > 0,
 * D even and positive.
 */
int attn_window_table(double rope_theta, int D, double k_turns, int32_t *out_host);

/*
 * Host-only: the number of (query, key, pair) terms the window removes from
 * one head's causal triangle 0 <= m <= n < S, i.e. sum over r of the cells
 * with n - m > w[r].  Exact int64 closed form.  w_host holds D/2 int32.
 */
int attn_pruned_terms(const int32_t *w_host, int D, int S, long long *per_head_out);

/*
 * Host-only validation of an attn_fwd argument list, without touching the
 * device (pointers are checked for NULL and alignment only).  Returns the
 * status attn_fwd would return before launching.
 */
int attn_check_args(const void *q, const void *k, const void *v, const void *o,
                    int B, int Hq, int Hkv, int S, int D, float rope_theta,
                    int causal, float scale, const int32_t *window_table);

/* A static English description of a status code. */
const char *attn_strerror(int status);

/* Frees the cached cos/sin tables on every device.  Not to be called while
 * work that uses them may still be running. */
void attn_release(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_ATTN_H */
