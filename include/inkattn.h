/*
 * inkattn.h -- C ABI of the MI355X (gfx950) learned-relative grouped-query
 * attention forward with per-query sinks.
 *
 * The operation is the forward of Inkling2FlexAttention (page
 * "nemo_automodel.components.models.inkling2.flex_attention", section API:
 * the class, its `scale` attribute and its `forward` parameters), with the
 * zero-valued virtual sink of Inkling2Attention.forward (page
 * "nemo_automodel.components.models.inkling2.attention", v0.4) and the
 * sliding-window semantics of the page
 * "nemo_automodel.components.attention.flex_attention" (sliding-window mask mod
 * and forward's `sliding_window` parameter).  For query i of batch row b and
 * query head h (K/V head g = h / (Hq/Hkv)), with gi = query_offset + i:
 *
 *   key j is allowed  <=>  valid[b,i] and key_valid[b,j] and j <= gi
 *                          and gi - positions[b,i] == j - key_positions[b,j]
 *                          and (window <= 0 or positions[b,i] - key_positions[b,j] < window)
 *   z_j   = head_dim^-0.5 * <q[b,i,h,:], k[b,j,g,:]> + bias_j
 *   bias_j = profiles[b,h,i,r] with r = positions[b,i] - key_positions[b,j]
 *            when 0 <= r < E, and 0 otherwise
 *   s     = sink[b,i,h]  (one more logit in the denominator, zero value)
 *   out[b,i,h,:] = sum_j e^{z_j} v[b,j,g,:] / (e^s + sum_j e^{z_j})
 *   lse[b,i,h]   = ln(e^s + sum_j e^{z_j})            (natural log)
 *   a row with no allowed key: out = 0, lse = s.
 *
 * No sequence-by-sequence score or bias tensor is formed.  The two tokens
 * of an allowed pair always satisfy r = gi - j (same document start column).
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer to C-contiguous memory owned by
 *    the caller; the library allocates nothing and keeps no global mutable
 *    state, so calls are reentrant (the one exception is attn_fwd_noalloc,
 *    whose per-GPU scratch is shared by its calls).  Inputs are never written.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  A successful return means the work was enqueued.
 *  - Every argument check runs on the host before any launch; on failure
 *    nothing is enqueued and a nonzero INKATTN_* status is returned, with a
 *    description in attn_last_error().  Launch failures return
 *    INKATTN_ERR_LAUNCH with the HIP error text in attn_last_error().
 *  - Sizes: B >= 0, Sq >= 0, Sk >= 0, Hq >= 1, Hkv >= 1 with Hq % Hkv == 0,
 *    D in {64, 128}, E >= 1, B*Sq*Hq*D and B*Hq*Sq*E below 2^40 elements,
 *    Sq, Sk and query_offset + Sq below 2^30; one batch row of k / v
 *    (Sk*Hkv*D*2 bytes) and one (batch row, head) block of profiles (Sq*E
 *    entries) below 4 GiB each.
 *  - Preconditions not checked (they would need a device read): positions and
 *    key_positions hold values in [0, 2^30); inputs at tokens that are not
 *    valid hold finite values.
 *  - Values of v: the probabilities multiply v in fp16 (exact for bf16 values
 *    within +-65504).  A value at a real key outside that range, or not
 *    finite, cannot be represented: the forward then writes NaN at (at least)
 *    every output element it would enter, never a clamped result, and
 *    attn_check_values reports INKATTN_ERR_RANGE for the workspace.
 */
#ifndef INKATTN_H
#define INKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Data type of the `profiles` tensor (the projection's fp32 or bf16 output). */
enum inkattn_dtype { INKATTN_F32 = 0, INKATTN_BF16 = 1 };

/* Status codes. */
enum inkattn_status {
    INKATTN_OK = 0,
    INKATTN_ERR_NULL = 1,        /* a required pointer is NULL                 */
    INKATTN_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes         */
    INKATTN_ERR_UNSUPPORTED = 3, /* head_dim / dtype outside what is built     */
    INKATTN_ERR_ALIGN = 4,       /* a pointer is not aligned as required       */
    INKATTN_ERR_WORKSPACE = 5,   /* workspace missing or too small             */
    INKATTN_ERR_LAUNCH = 6,      /* a HIP launch reported an error             */
    INKATTN_ERR_RANGE = 7        /* a value outside the supported range        */
};

/*
 * Bytes of device workspace attn_fwd needs for these sizes: what the
 * scheduler pre-pass writes (per-tile mask summaries, 16 bytes per 32-token
 * query block and per 64-key tile, then one int32 document start column per
 * key, padded to whole 64-key tiles; each part rounded up to 256 bytes),
 * followed by an fp16 copy of the values in whole 64-key tiles,
 * B*Hkv*ceil(Sk/64)*64*D*2 bytes, and one flag byte per staged tile (rounded
 * up to 256 bytes; see attn_check_values).  Never fails; returns 0 for
 * non-positive B.
 */
size_t attn_fwd_workspace_size(int B, int Sq, int Sk, int Hkv, int D);

/*
 * attn_fwd -- the fused forward (scheduler pre-pass + attention kernel).
 *
 *   q          [B, Sq, Hq, D]  bf16, 16-byte aligned
 *   k, v       [B, Sk, Hkv, D] bf16, 16-byte aligned
 *   profiles   [B, Hq, Sq, E]  fp32 or bf16 (profiles_dtype), element-aligned
 *   sink       [B, Sq, Hq]     fp32 (may hold -inf: no sink)
 *   valid      [B, Sq]         uint8 (0 / nonzero), true for real tokens
 *   key_valid  [B, Sk]         uint8, or NULL: then `valid` (requires Sk == Sq
 *                              and query_offset == 0)
 *   positions  [B, Sq]         int32 logical positions restarting at 0 at each
 *                              document start, or NULL: gi (one document)
 *   key_positions [B, Sk]      int32, or NULL: `positions` when Sk == Sq and
 *                              query_offset == 0, else the key column j
 *   window     keys a query may see counting itself (distance r < window);
 *              <= 0: no window
 *   query_offset  global column of the first local query (0 without context
 *              parallelism); keys are always global columns 0..Sk-1
 *   out        [B, Sq, Hq, D]  fp32, 16-byte aligned, written
 *   lse        [B, Sq, Hq]     fp32, written
 *   workspace  device buffer of at least attn_fwd_workspace_size(B, Sq, Sk,
 *              Hkv, D) bytes, 16-byte aligned; contents on entry are ignored
 */
int attn_fwd(const void* q, const void* k, const void* v,
             const void* profiles, int profiles_dtype,
             const float* sink, const uint8_t* valid, const uint8_t* key_valid,
             const int32_t* positions, const int32_t* key_positions,
             int64_t window, int64_t query_offset,
             int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
             float* out, float* lse,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace attn_bwd needs: the pre-pass summaries as for
 * attn_fwd, then per query 8 bytes and per (query, head) row 8 bytes of row
 * statistics and a bf16 copy of dout (B*Sq*Hq*D*2); each part rounded up to
 * 256 bytes.  Never fails; returns 0 for non-positive B.
 */
size_t attn_bwd_workspace_size(int B, int Sq, int Sk, int Hq, int Hkv, int D);

/*
 * attn_bwd -- gradients of attn_fwd.  The page
 * "nemo_automodel.components.models.inkling2.flex_attention" (module summary;
 * class Inkling2FlexAttention) makes the per-query sinks differentiable and
 * passes gradients to the captured profiles and through the returned
 * log-sum-exp.  For a loss L with dout = dL/dout and dlse = dL/dlse, per row
 * (b, i, h) with P_j = e^{z_j - lse} over the allowed keys j:
 *
 *   Delta  = <dout[b,i,h,:], out[b,i,h,:]>
 *   dz_j   = P_j (<dout[b,i,h,:], v[b,j,g,:]> - Delta + dlse[b,i,h])
 *   dq[b,i,h,:]  = head_dim^-0.5 sum_j dz_j k[b,j,g,:]
 *   dk[b,j,g,:] += head_dim^-0.5 dz_j q[b,i,h,:]     (summed over rows and
 *   dv[b,j,g,:] += P_j dout[b,i,h,:]                   the G heads of g)
 *   dprofiles[b,h,i,r] = dz_j for the allowed key j at distance r < E, else 0
 *   dsink[b,i,h] = e^{sink - lse} (dlse - Delta)      (0 where lse = -inf)
 *
 * Arguments q ... E as for attn_fwd (same masks, window, offset); the same
 * tensors the forward saw must be passed.
 *   out, lse   the forward's outputs for these inputs (fp32, [B,Sq,Hq,D] and
 *              [B,Sq,Hq]); out 16-byte aligned
 *   dout       [B, Sq, Hq, D] fp32, 16-byte aligned (rounded to bf16 for the
 *              matrix products)
 *   dlse       [B, Sq, Hq] fp32, or NULL (zero)
 *   dq         [B, Sq, Hq, D] fp32, 16-byte aligned, written
 *   dk, dv     [B, Sk, Hkv, D] fp32, 16-byte aligned, written
 *   dprofiles  [B, Hq, Sq, E] in profiles_dtype, written in full (zeros
 *              included)
 *   dsink      [B, Sq, Hq] fp32, written
 *   workspace  at least attn_bwd_workspace_size(B, Sq, Sk, Hq, Hkv, D) bytes,
 *              16-byte aligned; contents on entry are ignored
 * Inputs at tokens that are not valid never reach an output; as for the
 * forward, q, k and v there must hold finite values (dout there may hold
 * anything: it is ignored).  The products run in
 * bf16 MFMA with fp32 accumulation: P and dz are rounded to bf16 for dv / dq /
 * dk, dout for dz and dv.
 */
int attn_bwd(const void* q, const void* k, const void* v,
             const void* profiles, int profiles_dtype,
             const float* sink, const uint8_t* valid, const uint8_t* key_valid,
             const int32_t* positions, const int32_t* key_positions,
             int64_t window, int64_t query_offset,
             int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
             const float* out, const float* lse, const float* dout, const float* dlse,
             float* dq, float* dk, float* dv, void* dprofiles, float* dsink,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_plan -- the scheduler pre-pass alone: writes the per-tile mask
 * summaries (document start columns and real-token counts of every 32-token
 * query block and 64-key tile) into `workspace`.  The summaries depend only on
 * valid / key_valid / positions / key_positions / query_offset (the masks are
 * rebuilt from each forward's token validity, as on the flex_attention page,
 * class description), not on the window or any tensor values, so one plan
 * serves every attention layer of a forward that shares them.  Arguments as
 * for attn_fwd.
 */
int attn_plan(const uint8_t* valid, const uint8_t* key_valid,
              const int32_t* positions, const int32_t* key_positions,
              int64_t query_offset, int B, int Sq, int Sk,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_stage_values -- converts v [B, Sk, Hkv, D] (bf16) into the fp16 copy
 * the attention kernel stages from, in `workspace` after the summaries: per
 * (batch row, K/V head, 64-key tile) the tile's values transposed, D rows of
 * 64 keys, the keys of each row in the order the kernel's PV product consumes
 * them (a layout private to this library).  Values of keys whose key_valid
 * is 0, and of the padding past Sk, are written as 0.  The probabilities
 * multiply the values in fp16 MFMA (fp16 keeps 11 significant bits where bf16
 * keeps 8; a bf16 value inside the fp16 range converts exactly).  A real value
 * outside +-65504 or not finite is written as NaN and sets its tile's flag
 * byte (every tile's byte is rewritten on every call; attn_check_values reads
 * them).  key_valid defaults as in attn_fwd.  One call per layer (the values
 * differ per layer).
 */
int attn_stage_values(const void* v, const uint8_t* valid, const uint8_t* key_valid, int64_t query_offset,
                      int B, int Sq, int Sk, int Hkv, int D, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * attn_fwd_planned -- the attention kernel alone, reading the summaries that
 * attn_plan wrote into `workspace` for the same mask arguments (enqueued
 * earlier on `stream`, or completed).  A workspace planned for other mask
 * arguments gives undefined results, and reading the fp16 values that
 * attn_stage_values wrote there for this v (v itself is not read).
 * attn_fwd == attn_plan + attn_stage_values + attn_fwd_planned.
 */
int attn_fwd_planned(const void* q, const void* k, const void* v,
                     const void* profiles, int profiles_dtype,
                     const float* sink, const uint8_t* valid, const uint8_t* key_valid,
                     const int32_t* positions, const int32_t* key_positions,
                     int64_t window, int64_t query_offset,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
                     float* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_fwd_relproj -- attn_fwd with the profile rows formed in the kernel
 * from relative features instead of read from a profiles tensor, so that no
 * [B, Hq, Sq, E] tensor exists.  The page
 * "nemo_automodel.components.models.inkling2.attention" (v0.4, class
 * Inkling2Attention) names the pieces -- the fused projection qkvr that also
 * yields relative features, their width d_rel, relative_table and
 * rel_extent -- and the page "nemo_automodel.components.models.inkling2.
 * flex_attention" (forward parameter profiles) calls the profiles relative
 * logits of shape [batch, heads, sequence, relative_extent]; neither prints a
 * formula.  The reading built here:
 *
 *   profiles[b,h,i,r] = sum_c rfeat[b,i,h,c] * table[t,r,c]   (0 <= r < E)
 *
 * with t = h for a table of one slice per head (table_heads == Hq) and t = 0
 * for a shared one (table_heads == 1); bf16 products accumulated in fp32 and
 * used unrounded (the fp32 boundary).  Everything else as attn_fwd.
 *
 *   rfeat   [B, Sq, Hq, d_rel] bf16, 16-byte aligned
 *   table   [table_heads, E, d_rel] bf16, 16-byte aligned
 *   d_rel   16 or 32 (INKATTN_ERR_UNSUPPORTED otherwise)
 *   workspace as for attn_fwd (attn_fwd_workspace_size bytes)
 */
int attn_fwd_relproj(const void* q, const void* k, const void* v,
                     const void* rfeat, const void* table, int table_heads, int d_rel,
                     const float* sink, const uint8_t* valid, const uint8_t* key_valid,
                     const int32_t* positions, const int32_t* key_positions,
                     int64_t window, int64_t query_offset,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
                     float* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_fwd_noalloc -- attn_fwd for callers that cannot allocate device
 * memory: code under stream capture, tight serving loops, harnesses that
 * forbid allocation.  The same forward (the same kernels, the same results
 * bit for bit), with no workspace argument: its workspace is a scratch array
 * of INKATTN_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU
 * it runs on, from the first call there until the process ends.  The call
 * allocates nothing; the caller still passes every input and `out` / `lse`.
 * Sizes whose workspace (attn_fwd_workspace_size) exceeds the scratch are
 * rejected with INKATTN_ERR_WORKSPACE before any launch.  The scratch of the
 * current device is used (`stream` must belong to it).  Every call on a GPU
 * shares that GPU's scratch and leaves its contents behind: calls that
 * overlap on one GPU (on different streams or from different host threads)
 * race and must be serialised by the caller; calls in order on one stream are
 * safe.  (The value flags of attn_check_values stay in the scratch, which no
 * entry point reads back: a caller that wants that check calls attn_fwd with
 * a workspace of its own.)
 */
#define INKATTN_NOALLOC_SCRATCH_BYTES (72u << 20)
int attn_fwd_noalloc(const void* q, const void* k, const void* v,
                     const void* profiles, int profiles_dtype,
                     const float* sink, const uint8_t* valid, const uint8_t* key_valid,
                     const int32_t* positions, const int32_t* key_positions,
                     int64_t window, int64_t query_offset,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
                     float* out, float* lse, void* stream);

/*
 * attn_debug_counts -- number of allowed keys per query row, n_allowed[B, Sq]
 * (int32), evaluated with the same device mask predicate as attn_fwd.  Same
 * argument meanings as attn_fwd; used to check the mask exactly.
 */
int attn_debug_counts(const uint8_t* valid, const uint8_t* key_valid,
                      const int32_t* positions, const int32_t* key_positions,
                      int64_t window, int64_t query_offset, int B, int Sq, int Sk,
                      int32_t* n_allowed, void* stream);

/*
 * attn_debug_mask -- the whole visibility matrix mask[B, Sq, Sk] (uint8, 1 =
 * key j allowed for query i), from the same device predicate attn_fwd
 * applies on masked tiles (the masks are rebuilt from each forward's token
 * validity and positions: page "nemo_automodel.components.models.inkling2.
 * flex_attention", class description).  Meant for small shapes: B*Sq*Sk must
 * not exceed 2^32 (INKATTN_ERR_SHAPE otherwise).  Same argument meanings as
 * attn_fwd; `mask` is a caller-owned device buffer of B*Sq*Sk bytes.
 */
int attn_debug_mask(const uint8_t* valid, const uint8_t* key_valid,
                    const int32_t* positions, const int32_t* key_positions,
                    int64_t window, int64_t query_offset, int B, int Sq, int Sk,
                    uint8_t* mask, void* stream);

/*
 * attn_check_values -- reads back the flag bytes the last value staging
 * (attn_fwd, attn_stage_values or flex_attn_fwd) wrote into `workspace` for
 * these sizes, after waiting for `stream` (this call synchronises the
 * stream).  Returns INKATTN_OK when every real value of v fitted fp16, or
 * INKATTN_ERR_RANGE naming the first (batch row, K/V head, key tile) that
 * held a value outside +-65504 or not finite; the forward's output is then
 * NaN where that value enters it.  For flex_attn_fwd's workspace pass its
 * (B, Sq, Sk, Hkv, D): the flags sit at the same place.
 */
int attn_check_values(const void* workspace, size_t workspace_bytes, int B, int Sq, int Sk, int Hkv, int D,
                      void* stream);

/*
 * attn_debug_tiles -- the class attn_fwd gives each (query block, key tile):
 * tile_class[B, ceil(Sq/32), ceil(Sk/64)] (uint8): 0 = skipped, 1 = masked
 * element by element, 2 = full (no mask applied).  Uses the same pre-pass
 * and the same classification code as attn_fwd; `workspace` as for attn_fwd.
 */
int attn_debug_tiles(const uint8_t* valid, const uint8_t* key_valid,
                     const int32_t* positions, const int32_t* key_positions,
                     int64_t window, int64_t query_offset, int B, int Sq, int Sk,
                     uint8_t* tile_class, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * flex_attn_workspace_size / flex_attn_fwd -- the generic flex-attention
 * forward without the relative term: FlexAttention.forward on the page
 * "nemo_automodel.components.attention.flex_attention" (section API: forward's
 * q / k / v layouts, scale, sink_weights, sliding_window and enable_gqa;
 * attn_mask_type "causal" / "block_causal" and fixed_block_size of the class;
 * the block-causal and fixed-block mask mods).  For query i and key j of batch
 * row b, query head h, K/V head g = h / (Hq/Hkv):
 *
 *   key j is allowed  <=>  j <= i
 *                          and (tokens == NULL or i and j lie in the same
 *                               EOS-delimited block: a block ends with a token
 *                               equal to eos_id, which belongs to it)
 *                          and (fixed_block_size <= 0 or
 *                               i / fixed_block_size == j / fixed_block_size)
 *                          and (sliding_window <= 0 or i - j < sliding_window)
 *   z_j = scale * <q[b,h,i,:], k[b,g,j,:]>, where scale is the given one
 *         (> 0) only when sink_weights is NULL, head_dim^-0.5 otherwise
 *   s   = sink_weights[h] (a per-head logit in the denominator with a zero
 *         value), or no sink when sink_weights is NULL
 *   out[b,h,i,:] = sum_j e^{z_j} v[b,g,j,:] / (e^s + sum_j e^{z_j})   rounded to bf16
 *   lse[b,h,i]   = ln(e^s + sum_j e^{z_j})   (natural log; -inf for an empty row
 *                  without sink)
 *
 *   q    [B, Hq, Sq, D]  bf16, 16-byte aligned (head-major, as on the page)
 *   k, v [B, Hkv, Sk, D] bf16, 16-byte aligned
 *   sink_weights [Hq] fp32 or NULL
 *   tokens [B, Sq] int32 or NULL (NULL: "causal"; else "block_causal" by eos_id)
 *   out  [B, Hq, Sq, D]  bf16 (the dtype of q), 16-byte aligned, written
 *   lse  [B, Hq, Sq]     fp32, written when not NULL
 *   Block masks (tokens or fixed_block_size > 0) need Sq == Sk.  Queries are
 *   aligned with the first keys (query i is key column i).  The workspace
 *   holds the per-token positions and validity this entry derives, then the
 *   same pre-pass and value copy as attn_fwd.  Errors as for attn_fwd.
 */
size_t flex_attn_workspace_size(int B, int Sq, int Sk, int Hkv, int D);
int flex_attn_fwd(const void* q, const void* k, const void* v, const float* sink_weights,
                  const int32_t* tokens, int32_t eos_id, int64_t fixed_block_size, int64_t sliding_window,
                  float scale, int B, int Sq, int Sk, int Hq, int Hkv, int D, void* out, float* lse,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* attn_status_string(int status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* attn_last_error(void);

/* Query-block and key-tile sizes the kernels use (32 and 64). */
int attn_query_block(void);
int attn_key_tile(void);

#ifdef __cplusplus
}
#endif

#endif /* INKATTN_H */
