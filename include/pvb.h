/*
 * pvb.h -- packed, padding-free, block-causal varlen attention for MI355X (gfx950).
 *
 * A flat token axis of length T carries several independent sequences back to
 * back.  cu_seqlens (int32, B+1 entries, cu[0] = 0, cu[B] = T) cuts it into
 * slices [cu[b], cu[b+1]); attention is causal inside each slice only, so the
 * whole computation is block-diagonal causal attention and no [T, T] mask is
 * ever built ("Packing与 FlashAttention Varlen", section 1 and section 3).
 *
 * Conventions for every entry point
 *   - Return value: pvb_status; PVB_OK (0) on success.
 *   - Host planners run synchronously on the calling thread, validate every
 *     argument before writing anything, and leave outputs untouched on error.
 *   - Device entry points validate their scalar arguments on the host, enqueue
 *     their kernels on `stream` and never synchronise.  Problems that only the
 *     device can see (a bad device-resident cu_seqlens, lengths that overflow)
 *     are reported through a caller-provided device status word (int32, written
 *     by the call: 0 or a pvb_status code); the kernels then write no outputs.
 *   - Every buffer is allocated and owned by the caller.  The library keeps no
 *     allocations and no mutable global state; calls are reentrant.  Pointers
 *     named d_* are device pointers, h_* host pointers.
 *   - A device entry point only launches kernels on `stream` (no allocation,
 *     memset, copy or synchronisation), so it can be recorded into a HIP graph.
 *     Called without the optional host mirror of cu_seqlens, it plans its work
 *     on the device from the device cu_seqlens, so a recorded call stays valid
 *     when the boundaries (and the data) change in place between replays, as
 *     long as T, B and the other scalar arguments do not.
 *   - Tensors Q, K, V, O, dO, dQ, dK, dV are contiguous [T, H, d] (token-major,
 *     then head, then feature): element (t, h, c) at offset (t*H + h)*d + c.
 *     LSE and the backward's D are fp32 [H, T].
 *   - d in {64, 128}.  Causal self-attention takes one cu_seqlens for queries
 *     and keys; the *_cross_* entry points take separate query and key
 *     boundaries and a local window.  H query heads = H key/value heads, or
 *     grouped key/value heads through the *_gqa and *_cross_* entry points.
 *     The softmax scale is an argument (1/sqrt(d) is the usual value).
 */
#ifndef PVB_H
#define PVB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pvb_status {
  PVB_OK = 0,
  PVB_E_INVALID_ARG = 1,    /* null pointer, negative size, bad enum, capacity <= 0 */
  PVB_E_OVERSIZED = 2,      /* a sample longer than the capacity (never split)     */
  PVB_E_OVERFLOW = 3,       /* a count or offset would not fit int32              */
  PVB_E_BAD_CU_SEQLENS = 4, /* cu[0] != 0, decreasing, or cu[B] != T             */
  PVB_E_WORKSPACE = 5,      /* workspace missing or smaller than required         */
  PVB_E_UNSUPPORTED = 6,    /* head_dim other than 64/128, or a size beyond limits */
  PVB_E_HIP = 7,            /* a HIP runtime call failed (launch error)           */
  PVB_E_NO_TARGETS = 8      /* a mean loss over zero eligible targets              */
} pvb_status;

/* The largest count a caller may pass to a device entry point (token counts T
 * and capacity, segment counts B and n_seg, the vocabulary V): 2^31 - 65536, so
 * that no kernel's stride loop over such a count steps past INT32_MAX.  A larger
 * count returns PVB_E_OVERFLOW before anything is enqueued.
 * A launch also holds fewer than 2^32 work-items (the dispatch's grid size is
 * a 32-bit count): an attention call whose work list would need 2^24 or more
 * workgroups of 256 (about (T / 128 + min(B, T)) * H of them), a gated delta
 * forward with B * H >= 2^22 or backward with B * H >= 2^21 (its group walks
 * launch four and eight workgroups per slice and head), or a loss over
 * C >= 2^24 cells returns PVB_E_UNSUPPORTED, again before anything is enqueued. */
#define PVB_MAX_COUNT (2147483647 - 65535)

typedef enum pvb_dtype { PVB_BF16 = 0, PVB_F32 = 1 } pvb_dtype;

/* Precision of the probability operands (P, dS) fed to the matrix cores.
 * PVB_PREC_BF16: one bf16 rounding.  PVB_PREC_SPLIT: each value is split as
 * hi = bf16(x), lo = bf16(x - hi) and both parts are multiplied (two MFMAs),
 * giving about 16 significant bits.  Scores, softmax and accumulation are fp32
 * in both modes.
 * Accuracy against an fp64 reference (measured on MI355X over packs of up to
 * 1500-token segments, d = 64 and 128, up to 4 query heads per key/value head,
 * logit spreads -- the standard deviation of scale * q.k -- from 0.5 to 3):
 *   PVB_PREC_BF16: max-abs errors of dQ and dK of about 0.2-0.4% of their
 *     largest magnitude, and of O about 0.3% of max|V|.  An absolute bar of
 *     2e-2 on O, dQ, dK, dV therefore holds while the gradients stay below
 *     about 5 in magnitude: in the measured packs, logit spreads up to 1.0
 *     with unit-scale V and dO (the pages' workloads sit at 0.25-1.0).  Beyond
 *     that use PVB_PREC_SPLIT with fp32 O.
 *   PVB_PREC_SPLIT with an fp32 O: errors below 2e-4 up to spread 3 (largest
 *     |dQ| 17).  The backward forms D = rowsum(dO * O) from the O it is given,
 *     so a bf16 O brings back errors of the PVB_PREC_BF16 size in dQ and dK. */
typedef enum pvb_precision { PVB_PREC_BF16 = 0, PVB_PREC_SPLIT = 1 } pvb_precision;

/* ------------------------------------------------------------------ host planners */

/* Order-preserving next-fit ("Pack sequences without joining their contexts",
 * "Fill only the current row"; the sequential strategy of "Packing与
 * FlashAttention Varlen", section 2).  Items are read in order; an item that
 * does not fit in the room left in the current row starts a new row; rows are
 * never revisited and items are never split.  A zero-length item is placed in
 * the current row at its fill level.
 *   lengths  [n]  item lengths, 0 <= lengths[i] <= capacity   (host)
 *   row_of   [n]  out: row of item i                          (host)
 *   start_of [n]  out: offset of item i inside its row        (host)
 *   n_rows        out: number of rows (0 when n == 0)          (host)
 * Errors: PVB_E_INVALID_ARG (null pointer with n > 0, n < 0, capacity <= 0,
 * negative length), PVB_E_OVERSIZED (a length > capacity), PVB_E_OVERFLOW
 * (n > 2^31, so ordinals would not fit int32). */
pvb_status pvb_pack_plan_nextfit(const int32_t* lengths, int64_t n, int32_t capacity,
                                 int32_t* row_of, int32_t* start_of, int64_t* n_rows);

/* Best-fit-decreasing (the default packing strategy named in "Packing与
 * FlashAttention Varlen", section 2).  Items are taken by decreasing length,
 * ties by lower index; each goes to the open bin with the least room left that
 * still fits it (room >= length), ties to the lowest bin number, else to a new
 * bin.  Bins are numbered in creation order and keep insertion order.
 *   lengths     [n]    item lengths, 0 <= lengths[i] <= capacity   (host)
 *   bin_of      [n]    out: bin of item i                          (host)
 *   start_of    [n]    out: offset of item i inside its bin        (host)
 *   n_bins             out: number of bins                          (host)
 *   order       [n]    out: item ids bin by bin, insertion order    (host)
 *   bin_offsets [n+1]  out: bin j's items are order[bin_offsets[j] .. bin_offsets[j+1]);
 *                      entries past n_bins are left untouched       (host)
 * Errors as pvb_pack_plan_nextfit. */
pvb_status pvb_pack_plan_bfd(const int32_t* lengths, int64_t n, int32_t capacity,
                             int32_t* bin_of, int32_t* start_of, int64_t* n_bins,
                             int32_t* order, int64_t* bin_offsets);

/* ------------------------------------------------------------ device packed row */

/* Packed-row metadata by a device prefix scan ("Packing与 FlashAttention
 * Varlen", sections 1-3: cu_seqlens = running sum of lengths, local
 * position_ids restart at 0 in every sample; "Pack sequences without joining
 * their contexts", "Fill only the current row": occurrence segment ids,
 * padding cells with segment -1 and position 0).
 *   d_lengths   [n_seg]     segment lengths (>= 0)                        (device)
 *   n_seg                   number of segments, >= 0
 *   capacity                cells in the row C (>= sum of lengths; = T for a flat pack)
 *   segment_base            id of segment 0 (occurrence ordinal offset)
 *   d_cu        [n_seg+1]   out: cu[0] = 0, cu[b+1] = cu[b] + L_b           (device)
 *   d_pos       [capacity]  out: t - cu[s(t)] for real cells, 0 for padding (device)
 *   d_seg       [capacity]  out: segment_base + s(t), -1 for padding        (device)
 *                           where s(t) = max{ b : cu[b] <= t } (a zero-length
 *                           segment owns no cell but consumes an id)
 *   d_max_seqlen [1]        out, nullable: max length                       (device)
 *   Optional token gather (all four null, or d_tokens/d_tok_off and at least
 *   one output non-null): segment b is a document whose L_b + 1 tokens start at
 *   d_tokens[d_tok_off[b]]; cell cu[b] + j gets input tok[j] and target
 *   tok[j+1] (next-token pairs never cross documents: "Form pairs inside each
 *   source range"); padding cells get -1 and valid 0.
 *   d_tokens    [*]         int32 token ids                                 (device)
 *   d_tok_off   [n_seg]     int64 first-token offsets                       (device)
 *   d_inputs, d_targets [capacity]  out, nullable                          (device)
 *   d_valid     [capacity]  out, nullable: 1 real / 0 padding (uint8)       (device)
 *   d_status    [1]         out: device status word (required)              (device)
 * Device-detected errors (status word): PVB_E_INVALID_ARG (negative length),
 * PVB_E_OVERFLOW (cu would exceed int32), PVB_E_OVERSIZED (sum > capacity);
 * then only d_cu may have been written. */
pvb_status pvb_build_packed_row(const int32_t* d_lengths, int32_t n_seg, int32_t capacity,
                                int32_t segment_base, int32_t* d_cu, int32_t* d_pos,
                                int32_t* d_seg, int32_t* d_max_seqlen,
                                const int32_t* d_tokens, const int64_t* d_tok_off,
                                int32_t* d_inputs, int32_t* d_targets, uint8_t* d_valid,
                                int32_t* d_status, void* stream);

/* The reverse direction: segment boundaries compiled back from a flat
 * position stream ("Packing与 FlashAttention Varlen", section 3: the tokens
 * whose sample-local position restarts are the segment starts; appending the
 * token count gives cu_seqlens, and the largest difference is max_seqlen).
 * PVB_SENTINEL_ZERO takes position == 0 as a start; PVB_SENTINEL_MIN takes
 * position == the smallest position in the stream (the general path of
 * section 3, for encodings whose first position is not 0).  When the model's
 * positions are rotary coordinates that repeat inside a sample, pass the
 * separate text-position plane that restarts per sample (section 6) -- for a
 * [P, T] position tensor, the pointer to that plane's row.  Zero-length
 * segments cannot be represented in a position stream and do not appear.
 *   d_pos        int32 [T] positions                                   (device)
 *   T            tokens, >= 0
 *   sentinel     PVB_SENTINEL_ZERO or PVB_SENTINEL_MIN
 *   d_cu         out int32 [cu_capacity]: cu[0..n_seg], cu[0] = 0, cu[n_seg] = T
 *                                                                      (device)
 *   cu_capacity  entries d_cu can hold (T + 1 always suffices), >= 1
 *   d_n_seg      out int32 [1]: number of segments n_seg                (device)
 *   d_max_seqlen out int32 [1], nullable: largest segment length (0 if T = 0)
 *                                                                      (device)
 *   d_status     out: device status word (required)                     (device)
 * Device-detected errors (status word; then d_cu, d_n_seg and d_max_seqlen
 * are not written): PVB_E_BAD_CU_SEQLENS (T > 0 and the first token does not
 * start a segment, so cu[0] could not be 0), PVB_E_OVERSIZED (n_seg + 1 >
 * cu_capacity).  Host-detected: PVB_E_INVALID_ARG, PVB_E_OVERFLOW
 * (T > PVB_MAX_COUNT). */
typedef enum pvb_sentinel { PVB_SENTINEL_ZERO = 0, PVB_SENTINEL_MIN = 1 } pvb_sentinel;
pvb_status pvb_boundaries_from_positions(const int32_t* d_pos, int32_t T, int32_t sentinel,
                                         int32_t* d_cu, int32_t cu_capacity,
                                         int32_t* d_n_seg, int32_t* d_max_seqlen,
                                         int32_t* d_status, void* stream);

/* ---------------------------------------------------------------- attention */

/* Bytes of device workspace pvb_varlen_attn_fwd (bwd = 0) or
 * pvb_varlen_attn_bwd (bwd = 1) needs for these sizes.  Returns 0 for
 * invalid sizes. */
size_t pvb_varlen_attn_workspace_bytes(int32_t T, int32_t H, int32_t d, int32_t n_seg,
                                       int32_t bwd, int32_t grad_dtype);

/* Forward block-causal attention over the packed stream.  For every segment b
 * and head h, query i (cu[b] <= i < cu[b+1]) attends to keys j with
 * cu[b] <= j <= i:  O_i = sum_j softmax_j(scale * q_i.k_j) v_j and
 * LSE_i = ln sum_j exp(scale * q_i.k_j) ("Packing与 FlashAttention Varlen",
 * section 1: independent attentions written back in flat order; section 5:
 * per-slice base and extent, causal inside the slice, O at Q's offsets).
 * Zero-length segments are allowed (repeated cu values) and do no work.
 *   d_q, d_k, d_v  bf16 [T, H, d]                                  (device)
 *   d_cu           int32 [n_seg+1]                                 (device)
 *   h_cu           int32 [n_seg+1] host mirror, nullable: when given it is
 *                  validated on the host and a bad one returns
 *                  PVB_E_BAD_CU_SEQLENS before anything is enqueued; for a
 *                  small pack (at most 256 segments, 448 tiles of 128 rows,
 *                  32768 tokens per segment) the forward then lists its work
 *                  on the host and passes it with the launch, and does not
 *                  read d_cu (which must hold the same values)  (host)
 *   d_o            out [T, H, d], bf16 or fp32 per o_dtype          (device)
 *   d_lse          out fp32 [H, T] natural-log LSE                   (device)
 *   workspace      >= pvb_varlen_attn_workspace_bytes(..., 0, ...) bytes  (device)
 *   d_status       out: device status word (required)               (device)
 * Device-detected error: PVB_E_BAD_CU_SEQLENS in the status word; then O and
 * LSE are not written. */
pvb_status pvb_varlen_attn_fwd(const void* d_q, const void* d_k, const void* d_v,
                               const int32_t* d_cu, const int32_t* h_cu, int32_t n_seg,
                               int32_t T, int32_t H, int32_t d, float softmax_scale,
                               void* d_o, int32_t o_dtype, float* d_lse, int32_t precision,
                               void* workspace, size_t workspace_bytes, int32_t* d_status,
                               void* stream);

/* Backward of pvb_varlen_attn_fwd for the loss sum(O * dO): the textbook
 * softmax-attention gradient restricted to the same slices (the same ranges
 * drive forward and backward: "Pack sequences without joining their
 * contexts", "Extend the existing storage and decoder").
 *   D_i = sum_c dO_ic O_ic;  P_ij = exp(scale q_i.k_j - LSE_i);
 *   dV_j = sum_i P_ij dO_i;  dS_ij = P_ij (dO_i.v_j - D_i);
 *   dQ_i = scale sum_j dS_ij k_j;  dK_j = scale sum_i dS_ij q_i.
 *   d_q, d_k, d_v, d_do  bf16 [T, H, d]                            (device)
 *   d_o                  forward output, bf16 or fp32 per o_dtype   (device)
 *   d_lse                fp32 [H, T] from the forward               (device)
 *   d_dq, d_dk, d_dv     out [T, H, d], bf16 or fp32 per grad_dtype (device)
 *   other arguments as in pvb_varlen_attn_fwd.
 * Cross-segment derivatives are exactly zero. */
pvb_status pvb_varlen_attn_bwd(const void* d_q, const void* d_k, const void* d_v,
                               const void* d_o, int32_t o_dtype, const void* d_do,
                               const float* d_lse, const int32_t* d_cu, const int32_t* h_cu,
                               int32_t n_seg, int32_t T, int32_t H, int32_t d,
                               float softmax_scale, void* d_dq, void* d_dk, void* d_dv,
                               int32_t grad_dtype, int32_t precision, void* workspace,
                               size_t workspace_bytes, int32_t* d_status, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid allocation): pvb_varlen_attn_bwd_gqa
 * without a workspace argument.  Its scratch (the work list and the per-row
 * {LSE, D} records) is a fixed device array inside the library of
 * PVB_STATIC_SCRATCH_BYTES (64 MiB), held by every GPU the library runs on
 * until the process ends; the call itself allocates nothing.  It serves sizes
 * whose workspace, pvb_varlen_attn_workspace_bytes(T, H, d, n_seg, 1, ...),
 * fits that array (8 bytes per token and head plus 8 per 128-row tile:
 * T = 131072 at H = 32 fits, T = 262144 at H = 32 does not); larger ones
 * return PVB_E_WORKSPACE before anything is enqueued.  All calls on one
 * GPU share the array, so calls that overlap on that GPU (other streams,
 * other threads) race and give wrong gradients: serialise them.  Arguments,
 * outputs and other errors as pvb_varlen_attn_bwd_gqa; the results are the
 * same bit for bit.  PVB_E_HIP when the array's device address cannot be
 * obtained on the current device. */
#define PVB_STATIC_SCRATCH_BYTES (64u << 20)
pvb_status pvb_varlen_attn_bwd_noalloc(const void* d_q, const void* d_k, const void* d_v,
                                       const void* d_o, int32_t o_dtype, const void* d_do,
                                       const float* d_lse, const int32_t* d_cu, const int32_t* h_cu,
                                       int32_t n_seg, int32_t T, int32_t H, int32_t H_kv, int32_t d,
                                       float softmax_scale, void* d_dq, void* d_dk, void* d_dv,
                                       int32_t grad_dtype, int32_t precision, int32_t* d_status,
                                       void* stream);

/* ---------------------------------------------------------------- packed loss */

/* Token-weighted negative log-likelihood over packed cells and its logit
 * gradient ("Pack sequences without joining their contexts", "Keep the same
 * nine-target objective").  Cell c is eligible when targets[c] >= 0 and, if a
 * mask is given, mask[c] != 0 (so PAD_CELL = -1 and the ignore label -100 are
 * never supervised).  With N eligible cells:
 *   row_nll[c] = logsumexp(logits[c, :]) - logits[c, targets[c]]  (eligible),
 *                0 (excluded);
 *   loss[0] = sum of row_nll (float64, fixed summation order), loss[1] = loss[0] / N;
 *   grad[c, v] = (softmax(logits[c, :])_v - 1[v = targets[c]]) / N  (eligible),
 *                0 (excluded).
 * Excluded cells are skipped before any arithmetic: NaN or Inf logits there
 * change nothing.  Targets must already be sample-local (for next-token
 * training: shifted inside each sample, the last cell of a sample ignored,
 * "Packing与 FlashAttention Varlen", section 2).
 *   d_logits     [C, V] bf16 or fp32 per logits_dtype (row-major)      (device)
 *   C, V         cells (>= 0) and vocabulary size (> 0)
 *   d_targets    int32 [C]                                             (device)
 *   d_mask       uint8 [C], nullable: loss eligibility                 (device)
 *   d_row_nll    out fp32 [C] (required when C > 0)                    (device)
 *   d_loss       out float64 [2]: sum, mean                            (device)
 *   d_count      out int32 [1]: N                                      (device)
 *   d_grad       out [C, V] per grad_dtype, nullable (no gradient)     (device)
 *   d_status     out: device status word (required)                   (device)
 * Device-detected errors (status word; then d_row_nll, d_loss and d_grad are
 * not written): PVB_E_NO_TARGETS (N = 0), PVB_E_INVALID_ARG (an eligible
 * target >= V).  Host-detected: PVB_E_INVALID_ARG, PVB_E_OVERFLOW
 * (V > PVB_MAX_COUNT), PVB_E_UNSUPPORTED (C >= 2^24: one workgroup of 256
 * work-items per cell, and a launch holds fewer than 2^32 work-items). */
pvb_status pvb_packed_nll(const void* d_logits, int32_t logits_dtype, int64_t C, int32_t V,
                          const int32_t* d_targets, const uint8_t* d_mask, float* d_row_nll,
                          double* d_loss, int32_t* d_count, void* d_grad, int32_t grad_dtype,
                          int32_t* d_status, void* stream);

/* Grouped key/value heads ("Packing与 FlashAttention Varlen", section 5: the
 * key view carries h_k heads beside the query view's h).  As
 * pvb_varlen_attn_fwd / pvb_varlen_attn_bwd, with K and V (and dK, dV)
 * [T, H_kv, d], H a multiple of H_kv: query head h reads key/value head
 * h / (H / H_kv), and dK, dV of a key/value head sum the contributions of its
 * H / H_kv query heads (each written once; no atomics).  Q, O, dO, dQ stay
 * [T, H, d] and LSE [H, T]; the workspace size is that of the H-head call.
 * H_kv = H is exactly the plain call.  Extra error: PVB_E_INVALID_ARG when
 * H_kv <= 0 or H is not a multiple of H_kv. */
pvb_status pvb_varlen_attn_fwd_gqa(const void* d_q, const void* d_k, const void* d_v,
                                   const int32_t* d_cu, const int32_t* h_cu, int32_t n_seg,
                                   int32_t T, int32_t H, int32_t H_kv, int32_t d, float softmax_scale,
                                   void* d_o, int32_t o_dtype, float* d_lse, int32_t precision,
                                   void* workspace, size_t workspace_bytes, int32_t* d_status,
                                   void* stream);
pvb_status pvb_varlen_attn_bwd_gqa(const void* d_q, const void* d_k, const void* d_v,
                                   const void* d_o, int32_t o_dtype, const void* d_do,
                                   const float* d_lse, const int32_t* d_cu, const int32_t* h_cu,
                                   int32_t n_seg, int32_t T, int32_t H, int32_t H_kv, int32_t d,
                                   float softmax_scale, void* d_dq, void* d_dk, void* d_dv,
                                   int32_t grad_dtype, int32_t precision, void* workspace,
                                   size_t workspace_bytes, int32_t* d_status, void* stream);

/* ------------------------------------------------- cross attention, local windows */

/* Separate query and key boundaries with a local window ("Packing与
 * FlashAttention Varlen", section 5: cu_seqlens_q / cu_seqlens_k, the key
 * extent L_k of a slice, the causal clamp moved by L_k - L_q and widened by
 * window_right, and the per-row key range of a sliding window).  Segment b
 * pairs queries [cu_q[b], cu_q[b+1]) with keys [cu_k[b], cu_k[b+1]); with
 * L_q, L_k its extents and delta = L_k - L_q, local query row r may use local
 * keys j with
 *   max(0, r + delta - window_left) <= j <= min(L_k - 1, r + delta + window_right),
 * a negative window_left (window_right) leaving that side unbounded.
 * (window_left, window_right) = (-1, 0) is causal attention aligned to the
 * bottom right of the slice (the last query sees every key); (-1, -1) is full
 * bidirectional attention inside the slice; (w, 0) is a causal window of
 * w + 1 keys.  With cu_k = cu_q and (-1, 0) it is exactly the causal
 * self-attention call.  A query row with no key (possible when L_k < L_q or
 * with a window) gets O = 0 and LSE = -inf, and contributes no gradient.
 *   Q, O, dO, dQ  [T_q, H, d];  K, V, dK, dV  [T_k, H_kv, d];  LSE fp32 [H, T_q]
 *   d_cu_q, h_cu_q  query boundaries, device and host mirror, int32 [n_seg+1]
 *   d_cu_k, h_cu_k  key boundaries, device and host mirror, int32 [n_seg+1]
 *   window_left, window_right   >= -1
 *   workspace  >= pvb_varlen_cross_attn_workspace_bytes(...) bytes   (device)
 * Both host mirrors are required here and are validated on the host
 * (PVB_E_BAD_CU_SEQLENS); the device copies must hold the same values.  The
 * kernels still clip every key range to [0, T_k), so a device copy that
 * differs gives wrong values but no access outside the buffers.  Other
 * arguments, dtypes and errors as in the *_gqa calls; a window below -1 is
 * PVB_E_INVALID_ARG. */
size_t pvb_varlen_cross_attn_workspace_bytes(int32_t T_q, int32_t T_k, int32_t H, int32_t d,
                                             int32_t n_seg, int32_t bwd, int32_t grad_dtype);
pvb_status pvb_varlen_cross_attn_fwd(const void* d_q, const void* d_k, const void* d_v,
                                     const int32_t* d_cu_q, const int32_t* h_cu_q,
                                     const int32_t* d_cu_k, const int32_t* h_cu_k, int32_t n_seg,
                                     int32_t T_q, int32_t T_k, int32_t H, int32_t H_kv, int32_t d,
                                     int32_t window_left, int32_t window_right, float softmax_scale,
                                     void* d_o, int32_t o_dtype, float* d_lse, int32_t precision,
                                     void* workspace, size_t workspace_bytes, int32_t* d_status,
                                     void* stream);
pvb_status pvb_varlen_cross_attn_bwd(const void* d_q, const void* d_k, const void* d_v,
                                     const void* d_o, int32_t o_dtype, const void* d_do,
                                     const float* d_lse, const int32_t* d_cu_q, const int32_t* h_cu_q,
                                     const int32_t* d_cu_k, const int32_t* h_cu_k, int32_t n_seg,
                                     int32_t T_q, int32_t T_k, int32_t H, int32_t H_kv, int32_t d,
                                     int32_t window_left, int32_t window_right, float softmax_scale,
                                     void* d_dq, void* d_dk, void* d_dv, int32_t grad_dtype,
                                     int32_t precision, void* workspace, size_t workspace_bytes,
                                     int32_t* d_status, void* stream);

/* ------------------------------------------- linear attention: gated delta rule */

/* Gated delta rule over the packed stream with its recurrent state reset at
 * every boundary ("Packing与 FlashAttention Varlen", section 6: the
 * linear-attention layers take the same cumulative boundaries, which keep
 * one sample's recurrent state out of the next).  The recurrence is the
 * published gated delta rule: for slice b and head h, with a [d, d] state S
 * (key dims x value dims) starting at h0[b, h] (zero when d_h0 is null), for
 * each token t of the slice in order:
 *   S <- exp(g_t) S;  u_t = beta_t (v_t - S^T k_t);  S <- S + k_t u_t^T;
 *   o_t = scale S^T q_t;
 * and ht[b, h] = the slice's final S.  Zero-length slices give ht = h0.
 *   d_q, d_k, d_v  bf16 [T, H, d] (normalise q and k beforehand if wanted)  (device)
 *   d_g            fp32 [T, H] log gates, expected <= 0                      (device)
 *   d_beta         fp32 [T, H] write strengths                               (device)
 *   d_cu, h_cu     as in pvb_varlen_attn_fwd (h_cu nullable)
 *   d_h0           fp32 [n_seg, H, d, d] initial states, nullable            (device)
 *   d_o            out [T, H, d], bf16 or fp32 per o_dtype                   (device)
 *   d_ht           out fp32 [n_seg, H, d, d] final states, nullable          (device)
 *   workspace      >= pvb_gated_delta_fwd_workspace_bytes(T, H, n_seg) bytes
 *                  (device), or null with workspace_bytes = 0: 12 KB per
 *                  64-token chunk slot and head (T/64 + n_seg + 1 slots) and
 *                  192 KB per 1024-token group slot and head (T/1024 + n_seg
 *                  + 1 slots); about 0.62 GB at T = 32768, H = 32
 *   d_status       out: device status word (required)                       (device)
 * d = 128 (else PVB_E_UNSUPPORTED).  The slices are computed in chunks of 64
 * tokens (UT transform) in fp32 with matrix-core products whose fp32 operands
 * are split into two bf16 parts.  With a workspace, the chain of chunks is cut
 * into groups of 16 chunks (1024 tokens): T = (I + A)^-1 of every chunk first,
 * then each group's map of its starting state (S_out = A_g S_in + Z_g, a
 * product of the chunks' affine maps) for all groups at once, then each
 * slice's group starting states in order, then every group's chunks from its
 * starting state; a slice of n chunks then takes about 16 + n/16 + 16 serial
 * steps instead of n.  Without one (null, 0), each (slice, head) walks its
 * chunks in one chain, solving each chunk's triangle in place.  Both give the
 * same results up to rounding.  A workspace smaller than required (or null
 * with workspace_bytes > 0): PVB_E_WORKSPACE.  Device-detected error:
 * PVB_E_BAD_CU_SEQLENS (then O and ht are not written). */
size_t pvb_gated_delta_fwd_workspace_bytes(int32_t T, int32_t H, int32_t n_seg);
pvb_status pvb_gated_delta_fwd(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                               const float* d_beta, const int32_t* d_cu, const int32_t* h_cu,
                               int32_t n_seg, int32_t T, int32_t H, int32_t d, float scale,
                               const float* d_h0, void* d_o, int32_t o_dtype, float* d_ht,
                               void* workspace, size_t workspace_bytes, int32_t* d_status, void* stream);
/* The same with grouped query/key heads: q and k are [T, H_k, d], v, g, beta,
 * O and the states carry H value heads, H a multiple of H_k, and value head h
 * reads query/key head h / (H / H_k) (the published Gated DeltaNet layers use
 * fewer query/key heads than value heads; the pages give no layout).  H_k = H
 * is exactly pvb_gated_delta_fwd.  Extra error: PVB_E_INVALID_ARG when
 * H_k <= 0 or H is not a multiple of H_k. */
pvb_status pvb_gated_delta_fwd_gqa(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                                   const float* d_beta, const int32_t* d_cu, const int32_t* h_cu,
                                   int32_t n_seg, int32_t T, int32_t H, int32_t H_k, int32_t d,
                                   float scale, const float* d_h0, void* d_o, int32_t o_dtype,
                                   float* d_ht, void* workspace, size_t workspace_bytes, int32_t* d_status,
                                   void* stream);

/* Backward of pvb_gated_delta_fwd_gqa: the gradients of
 *   sum_t o_t . dO_t + sum_b <ht[b], dht[b]>
 * with respect to q, k, v, g, beta and the initial states, slice by slice
 * (nothing crosses a boundary; "Packing与 FlashAttention Varlen", section 6).
 * Exact in exact arithmetic: reverse-mode differentiation of the recurrence of
 * pvb_gated_delta_fwd, evaluated on 64-token chunks.  The call enqueues on
 * the stream (after clearing dq and dk when query/key heads are shared):
 * T = (I + A)^-1 of every chunk; then, side by side,
 * the forward's recomputation (each chunk's starting state and solved update)
 * and the chain that carries the gradient of the state from each slice's last
 * chunk to its first (with dv and dh0); then one pass over all chunks at once
 * for dq, dk, dg and dbeta.  Products keep about 16 significant bits (two
 * bf16 parts per fp32 operand); the rest is fp32.
 *   d_q, d_k, d_v, d_g, d_beta, d_cu, h_cu, n_seg, T, H, H_k, d, scale, d_h0
 *                  as in pvb_gated_delta_fwd_gqa (d_h0 nullable)
 *   d_dout         bf16 [T, H, d] gradient of O                         (device)
 *   d_dht          fp32 [n_seg, H, d, d] gradient of the final states, nullable
 *                  (zero)                                              (device)
 *   d_dq, d_dk     out fp32 [T, H_k, d]; a query/key head shared by several
 *                  value heads gets the sum (then the call clears them first
 *                  and adds with atomics, so their summation order varies)
 *   d_dv           out [T, H, d], bf16 or fp32 per grad_dtype
 *   d_dg, d_dbeta  out fp32 [T, H]
 *   d_dh0          out fp32 [n_seg, H, d, d], nullable
 *   workspace      >= pvb_gated_delta_bwd_workspace_bytes(T, H, n_seg) bytes
 *                  (216 KB per 64-token chunk slot and head, T/64 + n_seg + 1
 *                  slots, and 320 KB per 1024-token group slot and head,
 *                  T/1024 + n_seg + 1 slots: about 4.5 GB at T = 32768,
 *                  H = 32)                                              (device)
 * d = 128.  Device-detected error: PVB_E_BAD_CU_SEQLENS (then no gradient is
 * written). */
size_t pvb_gated_delta_bwd_workspace_bytes(int32_t T, int32_t H, int32_t n_seg);
pvb_status pvb_gated_delta_bwd(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                               const float* d_beta, const int32_t* d_cu, const int32_t* h_cu,
                               int32_t n_seg, int32_t T, int32_t H, int32_t H_k, int32_t d, float scale,
                               const float* d_h0, const void* d_dout, const float* d_dht, float* d_dq,
                               float* d_dk, void* d_dv, float* d_dg, float* d_dbeta, float* d_dh0,
                               int32_t grad_dtype, void* workspace, size_t workspace_bytes,
                               int32_t* d_status, void* stream);

/* Training pair: the forward of pvb_gated_delta_fwd_gqa (same arguments and
 * the same O and ht up to rounding; "Packing与 FlashAttention Varlen",
 * section 6, as above) that
 * also leaves in the backward's workspace what pvb_gated_delta_bwd recomputes
 * (T and T^T of every chunk, every chunk's starting state and solved update,
 * the 1024-token groups' maps), and the backward that reads them instead.
 *   workspace      >= pvb_gated_delta_bwd_workspace_bytes(T, H, n_seg) bytes
 *                  (device), written by pvb_gated_delta_fwd_train
 * pvb_gated_delta_bwd_after_fwd takes pvb_gated_delta_bwd's arguments; its
 * workspace must hold what pvb_gated_delta_fwd_train left for the same q, k,
 * v, g, beta, cu_seqlens, H, H_k and h0, untouched since (the call does not
 * check this: other contents give wrong gradients, never an out-of-bounds
 * access, as every index comes from cu_seqlens).  The forward always uses the
 * grouped evaluation; the results equal pvb_gated_delta_fwd_gqa's with a
 * workspace and pvb_gated_delta_bwd's up to rounding.  Errors as those two
 * calls, with PVB_E_WORKSPACE for a workspace under the backward's size. */
pvb_status pvb_gated_delta_fwd_train(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                                     const float* d_beta, const int32_t* d_cu, const int32_t* h_cu,
                                     int32_t n_seg, int32_t T, int32_t H, int32_t H_k, int32_t d,
                                     float scale, const float* d_h0, void* d_o, int32_t o_dtype,
                                     float* d_ht, void* workspace, size_t workspace_bytes, int32_t* d_status,
                                     void* stream);
pvb_status pvb_gated_delta_bwd_after_fwd(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                                         const float* d_beta, const int32_t* d_cu, const int32_t* h_cu,
                                         int32_t n_seg, int32_t T, int32_t H, int32_t H_k, int32_t d,
                                         float scale, const float* d_h0, const void* d_dout,
                                         const float* d_dht, float* d_dq, float* d_dk, void* d_dv,
                                         float* d_dg, float* d_dbeta, float* d_dh0, int32_t grad_dtype,
                                         void* workspace, size_t workspace_bytes, int32_t* d_status,
                                         void* stream);

/* Human-readable name of a status code (static string). */
const char* pvb_status_string(int32_t status);

/* Library version string (static). */
const char* pvb_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PVB_H */
