/*
 * rat.h -- C ABI of the RAT+ inference hot path on AMD MI355X (gfx950).
 *
 * The method ("RAT+: Train Dense, Infer Sparse -- Recurrence Augmented
 * Attention for Dilated Inference", abstract; zhichai.net deep dive
 * "RAT+ 深度拆解", sections 一, 2.1, 2.2 and 六):
 *
 *   1. a per-channel, input-gated recurrence over keys and values that runs
 *      over the whole sequence (deep dive, section 2.1):
 *          h_t = g_t * h_{t-1} + (1 - g_t) * x_t,   h_{-1} = 0,
 *      the same gate for keys and values, computed in fp32;
 *   2. causal softmax attention dilated by D (abstract; deep dive, section
 *      一): query t attends to the recurrent states at the anchors
 *      j = D-1 (mod D), j < t, to its own position t, and optionally to a
 *      local window of the W positions before t (abstract: the window is an
 *      option).  D = 1 and W = 0 is dense causal attention (deep
 *      dive, section 2.2).  D and W are chosen per head at inference time
 *      (abstract; deep dive, sections 六 and 7.1: head-wise hybrids).
 *   3. the KV cache keeps only the anchors, floor(T_cap / D) rows per head,
 *      which is the D-fold cache cut of the abstract, plus a ring of the
 *      last W states for the window.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller (any allocator),
 *    contiguous in the stated layout and 16-byte aligned.  The library never
 *    allocates device memory, never synchronises and keeps no global mutable
 *    state.  All GPU work is enqueued on `stream` (a hipStream_t; NULL is
 *    the default stream) and completes asynchronously.
 *  - Per-head tables D[H], W[H] are HOST int32 arrays, the same for every
 *    batch row; 1 <= D[h], 0 <= W[h]; H <= RAT_MAX_HEADS.
 *  - dtype is RAT_DTYPE_BF16 or RAT_DTYPE_F32: the storage type (ST) of
 *    q, k, v, g, the states hk/hv, the caches and o.  Recurrent state
 *    (state_k/state_v) and lse are always fp32.  hd (head dim) is 64 or 128.
 *  - Layouts: activations [B, H, T, hd]; state [B, H, hd];
 *    anchor cache Kc/Vc [B, R, hd] with head h's rows at
 *    off[h] = sum_{h'<h} floor(T_cap / D[h']) (R = off[H]); anchor row a of
 *    head h holds position a*D[h] + D[h] - 1;
 *    window ring k_ring/v_ring [B, sum(W), hd] with head h's W[h] slots at
 *    roff[h] = sum_{h'<h} W[h']; position p lives in slot p mod W[h].
 *  - Every function validates all arguments on the host before enqueuing
 *    anything; a call that fails validation writes nothing.  Return values:
 *    RAT_OK (0) or a negative RAT_ERR_* code; no C++ exception crosses the
 *    ABI.  RAT_ERR_HIP means a launch was rejected by the HIP runtime.
 *  - Thread-safe and reentrant.  Calls that share a workspace or write the
 *    same outputs must be ordered by the caller (same stream).
 */
#ifndef RAT_H_
#define RAT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RAT_OK 0
#define RAT_ERR_INVALID_ARG (-1)
#define RAT_ERR_UNSUPPORTED (-2)
#define RAT_ERR_CAPACITY (-3)
#define RAT_ERR_WORKSPACE (-4)
#define RAT_ERR_HIP (-5)

#define RAT_DTYPE_BF16 0
#define RAT_DTYPE_F32 1

#define RAT_MAX_HEADS 128

/* Library version string (static storage). */
const char* rat_version(void);

/* Static, human-readable message for a status code. */
const char* rat_status_string(int status);

/*
 * Rows per batch row of the anchor-only cache for capacity T_cap (abstract:
 * the cache shrinks by D).  R = sum_h floor(T_cap / D[h]).  If offsets_out
 * is not NULL it receives H+1 values: off[h] and off[H] = R.
 * Pure host function.  Returns R >= 0, or RAT_ERR_INVALID_ARG.
 */
int64_t rat_anchor_rows(int H, int64_t T_cap, const int32_t* D,
                        int64_t* offsets_out);

/*
 * Slots per batch row of the window ring: sum_h W[h]; offsets_out (nullable)
 * receives H+1 values roff[h], roff[H] = total.  Pure host function.
 * Returns the total >= 0, or RAT_ERR_INVALID_ARG.
 */
int64_t rat_ring_rows(int H, const int32_t* W, int64_t* offsets_out);

/*
 * Bytes of device workspace rat_scan_prefill needs for (B, H, T, hd).
 * The workspace carries the scan's chunk-to-chunk carries.  It must be
 * zero-filled once before its first use; every call leaves it ready for the
 * next call (after a call that returned an error, or a launch that was
 * aborted, zero-fill it again).  One workspace must not be used by two calls
 * that can run at the same time.  The first 32 KB are a header (uint32
 * word 0: launch epoch; word 2: error word; then completion counters), the
 * rest holds the tagged chunk aggregates.  The error word is != 0 after a
 * call in which a chunk gave up waiting for a predecessor's aggregate (the
 * results of that call are invalid).  It is sticky: no later call clears
 * it, so a non-zero word means some call since the workspace was last
 * zero-filled failed; a caller that finds it set discards those results and
 * zero-fills the whole workspace before its next use.  The scan kernel is persistent: its
 * grid never exceeds what the device holds at once, and with the device to
 * itself every workgroup is resident immediately; if other streams keep CUs
 * busy past the (bounded) wait, the call reports it here instead of
 * hanging.  Pure host function; returns bytes (> 0) or a negative code.
 */
int64_t rat_scan_workspace_bytes(int B, int H, int64_t T, int hd);

/*
 * Prefill recurrence with fused anchor compaction (deep dive, section 2.1:
 * full-sequence recurrence computed by an associative scan in prefill;
 * abstract: anchor-only KV cache).
 *
 * Reads  k, v, g          [B, H, T, hd] ST (g in [0, 1])
 * Writes hk, hv           [B, H, T, hd] ST: h_t of keys / values (both
 *                         NULL = cache-only mode: only the outputs below)
 *        Kc, Vc           [B, R(T_cap), hd] ST: rows a < floor(T / D[h]) of
 *                         each head (other rows untouched)
 *        k_ring, v_ring   [B, sum W, hd] ST: slots of positions
 *                         max(0, T - W[h]) .. T-1 (NULL allowed iff all W = 0)
 *        state_k, state_v [B, H, hd] fp32: h_{T-1} (zeros when T = 0)
 * Requires 0 <= T <= T_cap.  Starts from the zero state at position 0.
 * workspace: see rat_scan_workspace_bytes (RAT_ERR_WORKSPACE if too small).
 */
int rat_scan_prefill(int dtype, int B, int H, int64_t T, int hd,
                     const int32_t* D, const int32_t* W, int64_t T_cap,
                     const void* k, const void* v, const void* g, void* hk,
                     void* hv, void* Kc, void* Vc, void* k_ring, void* v_ring,
                     float* state_k, float* state_v, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Prefill dilated attention (abstract; deep dive, sections 一, 2.2, 六).
 * For each (b, h, t): keys S(t) = {t} U {j < t : j = D-1 mod D}
 *                                 U {max(0, t-W) .. t-1},
 *   o_t = sum_{j in S(t)} softmax_j(scale * q_t . hk_j) hv_j,
 *   lse_t = log sum_{j in S(t)} exp(scale * q_t . hk_j)   (natural log).
 * Anchors j < max(0, t-W) are read from the compact cache Kc/Vc (as written
 * by rat_scan_prefill with the same D, T_cap); window and own positions are
 * read from hk/hv.
 * Reads  q, hk, hv [B, H, T, hd] ST; Kc, Vc [B, R(T_cap), hd] ST.
 * Writes o [B, H, T, hd] ST; lse [B, H, T] fp32 (nullable).
 * scale <= 0 selects 1/sqrt(hd).  Requires 0 <= T <= T_cap.
 */
int rat_dilated_attn_prefill(int dtype, int B, int H, int64_t T, int hd,
                             const int32_t* D, const int32_t* W, float scale,
                             int64_t T_cap, const void* q, const void* hk,
                             const void* hv, const void* Kc, const void* Vc,
                             void* o, float* lse, void* stream);

/*
 * Chunked prefill: the recurrence of a chunk of T positions that follows
 * t0 positions already processed (deep dive, section 2.1: the recurrent
 * state is carried along the whole sequence; abstract: anchor-only cache).
 * Position t of the chunk is absolute position t0 + t; the result equals
 * rat_scan_prefill over the t0 + T positions, restricted to the chunk.
 *
 * Reads  k, v, g                [B, H, T, hd] ST: the chunk
 *        state_k_in, state_v_in [B, H, hd] fp32: h_{t0-1} (the state after
 *                               the previous chunk, or zeros when t0 = 0);
 *                               must not alias state_k / state_v
 *        k_ring_in, v_ring_in   [B, sum W, hd] ST: the ring after the
 *                               previous chunk (nullable when all W = 0 or
 *                               t0 = 0).  When it is not k_ring/v_ring, the
 *                               slots of positions max(0, t0+T-W) .. t0-1
 *                               are copied from it into k_ring/v_ring first.
 * Writes hk, hv           [B, H, T, hd] ST: h of the chunk's positions (both
 *                         NULL = cache-only mode)
 *        Kc, Vc           rows a with t0 <= a*D + D-1 < t0 + T (other rows,
 *                         from earlier chunks, untouched)
 *        k_ring, v_ring   slots of positions max(0, t0+T-W) .. t0+T-1
 *        state_k, state_v h_{t0+T-1} (the input state when T = 0)
 * Requires t0 >= 0, T >= 0, t0 + T <= T_cap (else RAT_ERR_CAPACITY).
 * Updating the ring in place (k_ring_in == k_ring) is valid for the scan,
 * but it overwrites window positions before t0 that the chunk's attention
 * reads: keep the previous ring in a second buffer for
 * rat_dilated_attn_prefill_continue (two rings used alternately).
 * workspace: rat_scan_workspace_bytes(B, H, T, hd), as for rat_scan_prefill.
 */
int rat_scan_prefill_continue(int dtype, int B, int H, int64_t T, int hd,
                              const int32_t* D, const int32_t* W, int64_t T_cap,
                              int64_t t0, const void* k, const void* v,
                              const void* g, const float* state_k_in,
                              const float* state_v_in, void* hk, void* hv,
                              void* Kc, void* Vc, const void* k_ring_in,
                              const void* v_ring_in, void* k_ring,
                              void* v_ring, float* state_k, float* state_v,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Chunked prefill attention: queries of a chunk at absolute positions
 * t0 .. t0+T-1 over the key sets of rat_dilated_attn_prefill (abstract;
 * deep dive, sections 一, 2.2).  Anchors come from Kc/Vc (all chunks so far,
 * after rat_scan_prefill_continue of this chunk); window positions >= t0
 * and the own position from hk/hv of the chunk [B, H, T, hd]; window
 * positions < t0 from k_ring_prev/v_ring_prev [B, sum W, hd], the ring as
 * it was after the previous chunk (required when t0 > 0 and some W > 0,
 * else nullable).  Writes o [B, H, T, hd] ST, lse [B, H, T] fp32
 * (nullable).  Requires t0 + T <= T_cap (else RAT_ERR_CAPACITY).
 */
int rat_dilated_attn_prefill_continue(int dtype, int B, int H, int64_t T,
                                      int hd, const int32_t* D,
                                      const int32_t* W, float scale,
                                      int64_t T_cap, int64_t t0,
                                      const void* q, const void* hk,
                                      const void* hv, const void* Kc,
                                      const void* Vc,
                                      const void* k_ring_prev,
                                      const void* v_ring_prev, void* o,
                                      float* lse, void* stream);

/*
 * Bytes of device workspace rat_decode_step needs for any pos < T_cap with
 * num_splits (0 = automatic choice).  0 means no workspace is needed
 * (the single-split path).  Pure host function; negative on error.
 */
int64_t rat_decode_workspace_bytes(int B, int H, int hd, int64_t T_cap,
                                   const int32_t* D, const int32_t* W,
                                   int num_splits);

/*
 * One decode step at position pos for every batch row (the single-state
 * update of the full-sequence recurrence, then dilated attention over the
 * anchor-only cache; abstract: the cache is D times smaller).
 *   s <- g*s + (1-g)*x  (fp32, x in {k, v});  hat = ST(s);
 *   o = attention of q over anchors a < floor(max(0, pos-W)/D) from Kc/Vc,
 *       the window positions max(0,pos-W) .. pos-1 from the ring, and hat.
 * Then, after every read: state_k/state_v <- s; ring slot pos mod W <- hat
 * (if W > 0); anchor row pos / D <- hat (if pos mod D = D-1).
 * Reads  q, k, v, g [B, H, hd] ST.  Updates state_k, state_v [B, H, hd] fp32,
 * Kc, Vc, k_ring, v_ring (layouts above).  Writes o [B, H, hd] ST.
 * The cache must hold positions 0 .. pos-1 (rat_scan_prefill of T = pos,
 * or earlier decode steps).  Requires 0 <= pos < T_cap, else
 * RAT_ERR_CAPACITY.  num_splits: split-K factor (0 = automatic).
 * workspace: rat_decode_workspace_bytes bytes (NULL if that is 0).
 */
int rat_decode_step(int dtype, int B, int H, int hd, const int32_t* D,
                    const int32_t* W, float scale, int64_t pos, int64_t T_cap,
                    const void* q, const void* k, const void* v, const void* g,
                    float* state_k, float* state_v, void* Kc, void* Vc,
                    void* k_ring, void* v_ring, void* o, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * rat_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, semantics and results as
 * rat_decode_step (same kernels, same split choice).  The split-K partials
 * go to a device array of RAT_NOALLOC_SCRATCH_BYTES that the library holds
 * on every device it runs on, from its first use there until the process
 * ends; the call itself allocates nothing.  A call whose partials would not
 * fit, B*H*splits*(hd+2)*4 > RAT_NOALLOC_SCRATCH_BYTES, returns
 * RAT_ERR_WORKSPACE and launches nothing.  All calls on one device share
 * that array: two calls that can run at the same time on one device (other
 * streams, other threads) race and must not overlap.  The array needs no
 * clearing (every partial is written before it is read).
 */
#define RAT_NOALLOC_SCRATCH_BYTES (16u << 20)
int rat_decode_step_noalloc(int dtype, int B, int H, int hd, const int32_t* D,
                            const int32_t* W, float scale, int64_t pos,
                            int64_t T_cap, const void* q, const void* k,
                            const void* v, const void* g, float* state_k,
                            float* state_v, void* Kc, void* Vc, void* k_ring,
                            void* v_ring, void* o, int num_splits,
                            void* stream);

/*
 * Decode combined with top-k block selection (RAT+ abstract, v1: RAT+
 * sparsified to top-k block attention; deep dive, section 四: dilation and
 * top-k block selection combine, the anchors covering the whole past and the
 * selected blocks adding density).  The pages fix neither block size nor
 * scoring; this library's reading: blocks are the aligned runs of
 * RAT_TOPK_BLOCK positions; a block is eligible at position pos when it lies
 * wholly before max(0, pos - W); its score is q . (mean stored key state of
 * the block); the k_blocks highest are selected (equal scores: the lower
 * block first).
 *
 * rat_topk_cache_build: the history cache of a prefill or of one chunk of a
 * chunked prefill.  hk, hv [B, H, T, hd] ST hold the stored states of
 * positions t0 .. t0+T-1 (t0 = 0 for a whole prefill); they are copied into
 * rows t0 .. t0+T-1 of hk_hist, hv_hist [B, H, T_cap, hd] ST, and the mean
 * of every block that ends in t0 .. t0+T-1 is written to block_means
 * [B, H, T_cap / RAT_TOPK_BLOCK, hd] fp32 (other rows untouched; the rows of
 * such a block before t0 are read from the history, so the chunks must be
 * built in order).  Requires t0 >= 0 and t0 + T <= T_cap (else
 * RAT_ERR_CAPACITY) and B, H <= 65535.  block_means may be NULL when no
 * block ends in the call's rows.
 */
#define RAT_TOPK_BLOCK 64
#define RAT_TOPK_MAX_K 64
int rat_topk_cache_build(int dtype, int B, int H, int64_t T, int hd,
                         int64_t T_cap, int64_t t0, const void* hk,
                         const void* hv, void* hk_hist, void* hv_hist,
                         float* block_means, void* stream);

/*
 * rat_decode_step_topk: one decode step at position pos, as rat_decode_step
 * (same state update, anchors from Kc/Vc, window from the ring, own
 * position), with the k_blocks selected blocks' positions added to the key
 * set; an anchor position inside a selected block is counted once.  Reads
 * hk_hist/hv_hist rows < pos and block_means rows of the eligible blocks.
 * Then, after every read, also writes history row pos <- hat and, when pos
 * ends a block (pos mod RAT_TOPK_BLOCK = RAT_TOPK_BLOCK-1), that block's
 * mean.  sel_out (nullable): [B, H, k_blocks] int32, the selected blocks of
 * each (b, h) best first, -1 past the number selected.  One workgroup per
 * (b, h), no workspace.  Requires 0 <= pos < T_cap (else RAT_ERR_CAPACITY);
 * k_blocks <= RAT_TOPK_MAX_K and T_cap / RAT_TOPK_BLOCK <= 8192 (else
 * RAT_ERR_UNSUPPORTED).
 */
int rat_decode_step_topk(int dtype, int B, int H, int hd, const int32_t* D,
                         const int32_t* W, float scale, int64_t pos,
                         int64_t T_cap, int k_blocks, const void* q,
                         const void* k, const void* v, const void* g,
                         float* state_k, float* state_v, void* Kc, void* Vc,
                         void* k_ring, void* v_ring, void* hk_hist,
                         void* hv_hist, float* block_means, void* o,
                         int32_t* sel_out, void* stream);

/*
 * Bytes of device workspace rat_prefill_backward needs for (B, H, T, hd, D,
 * W).  Zero-fill it once before its first use; afterwards it is ready for
 * every later call of this size or smaller (it starts with the reverse
 * scan's tree workspace, laid out as the forward scan's, whose header sits
 * at offset 0 for every size).  Pure host function; returns bytes (> 0) or
 * a negative code.
 */
int64_t rat_prefill_backward_workspace_bytes(int B, int H, int64_t T, int hd,
                                             const int32_t* D, const int32_t* W);

/*
 * Backward of the prefill (scan + dilated attention) for a loss L with
 * dL/do = dO: the gradient the training path needs (deep dive, sections 2.2
 * and 2.3: dense pretraining with active recurrence learning and a short
 * adaptation to a dilation; section 2.1: the recurrence).
 *   attention, per query t over its key set S(t): P = softmax(scale q.hk),
 *     delta_t = dO_t . o_t, dS = P (dO_t . hv - delta_t);
 *     dq_t = scale sum_j dS_j hk_j;  dh^k_j += scale dS_j q_t;
 *     dh^v_j += P_j dO_t;
 *   recurrence in reverse: lambda_t = dh_t + g_{t+1} lambda_{t+1}
 *     (lambda_T = 0); dk = (1-g) lambda^k, dv = (1-g) lambda^v,
 *     dg = lambda^k (h^k_{t-1} - k) + lambda^v (h^v_{t-1} - v), h_{-1} = 0.
 * The storage rounding of the states is taken as the identity; h_{t-1} in
 * dg is the stored state.
 * Reads  q, k, v, g, dO       [B, H, T, hd] ST (the prefill's inputs)
 *        hk, hv, o            [B, H, T, hd] ST (rat_scan_prefill's states and
 *                             rat_dilated_attn_prefill's output, same D, W,
 *                             scale)
 *        lse                  [B, H, T] fp32 (rat_dilated_attn_prefill's lse)
 * Writes dq, dk, dv, dg       [B, H, T, hd] ST
 * workspace: rat_prefill_backward_workspace_bytes bytes, zero-filled once
 * (the reverse scan's chunk tree, then fp32 intermediates).  The reverse
 * recurrence is one persistent pass whose chunks wait on the maps of the
 * chunks after them; as in rat_scan_prefill every wait is bounded, and a
 * wait that runs out sets uint32 word 2 of the workspace (sticky until the
 * workspace is zero-filled again) instead of hanging: a caller that finds it
 * set discards the gradients.  One workspace must not be used by two calls
 * at once.  scale <= 0 selects 1/sqrt(hd).
 */
int rat_prefill_backward(int dtype, int B, int H, int64_t T, int hd,
                         const int32_t* D, const int32_t* W, float scale,
                         const void* q, const void* k, const void* v,
                         const void* g, const void* hk, const void* hv,
                         const void* o, const float* lse, const void* dO,
                         void* dq, void* dk, void* dv, void* dg,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Bytes of device workspace rat_layer_prefill needs.  Zero-fill it once
 * before its first use (it starts with a scan workspace, at offset 0 for
 * every size, so its error word is uint32 word 2 of the buffer); afterwards
 * it is ready for every later call, of this size or smaller.  Pure host
 * function; bytes (> 0) or a negative code.
 */
int64_t rat_layer_workspace_bytes(int dtype, int B, int H, int64_t T, int hd);

/*
 * One RAT+ layer over a prefill: the steps on either side of the hot path
 * (abstract: RAT+ augments the attention of a transformer layer; deep dive,
 * section 2.1: the input-dependent forget gate) around rat_scan_prefill and
 * rat_dilated_attn_prefill:
 *   q = x W_q, k = x W_k, v = x W_v (per head h: columns h*hd .. h*hd+hd-1);
 *   g = sigmoid(x W_g + b_g)   (the bias and sigmoid fused into the scan);
 *   recurrence, anchor cache, ring, state and dilated attention as in the
 *   two prefill entry points (same D, W, scale, T_cap);
 *   out = o W_o with o [B, T, H*hd] (heads concatenated).
 * Reads  x [B, T, dm] ST; w_q, w_k, w_v, w_g [dm, H*hd] ST (row-major);
 *        b_g [H*hd] fp32; w_o [H*hd, dm] ST.
 * Writes out [B, T, dm] ST; lse [B, H, T] fp32 (nullable); Kc, Vc, k_ring,
 *        v_ring, state_k, state_v as rat_scan_prefill.
 * The projections run on the library's own MFMA GEMM (bf16 or fp32 in and
 * out, fp32 accumulation) on the same stream; like every other entry point
 * this one allocates nothing and keeps no state.  bf16 requires dm % 8 == 0
 * and B*T <= 65535*256 (else RAT_ERR_UNSUPPORTED).
 * workspace: rat_layer_workspace_bytes bytes (a scan workspace, then q, k,
 * v, the gate pre-activation, the states and o).
 */
int rat_layer_prefill(int dtype, int B, int H, int64_t T, int hd, int dm,
                      const int32_t* D, const int32_t* W, float scale,
                      int64_t T_cap, const void* x, const void* w_q,
                      const void* w_k, const void* w_v, const void* w_g,
                      const float* b_g, const void* w_o, void* out, float* lse,
                      void* Kc, void* Vc, void* k_ring, void* v_ring,
                      float* state_k, float* state_v, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace rat_stack_prefill needs: one layer workspace
 * (reused by every layer) and the activations between layers [B, T, dm].
 * Zero-fill it once (the scan workspace inside it is reused across calls);
 * negative status on invalid sizes.
 */
int64_t rat_stack_workspace_bytes(int dtype, int B, int H, int64_t T, int hd, int dm);

/*
 * A stack of nlayers RAT+ layers over a prefill, each with its own D and W
 * per head: the layer-wise hybrid of the deep dive, section 六 (some layers
 * dense, D = 1, others dilated), and the RAT+ abstract's hybrid layer
 * compositions.  Layer l is rat_layer_prefill on the previous layer's output
 * (layer 0 on x): x_{l+1} = out_l, stored in the storage type between
 * layers.  The pages give no residual path or normalisation around a layer,
 * so none is applied.
 * D, W: host int32 [nlayers][H].  w_q, w_k, w_v, w_g, b_g, w_o: host arrays
 * of nlayers device pointers with the shapes of rat_layer_prefill.  Kc, Vc,
 * k_ring, v_ring, state_k, state_v: host arrays of nlayers device pointers,
 * each layer's cache as rat_layer_prefill (sized by that layer's D and W).
 * Writes out [B, T, dm] and every layer's cache.  Every layer's arguments
 * are checked before the first launch, so a failed call writes nothing.
 * workspace: rat_stack_workspace_bytes bytes.  No lse is produced.
 */
int rat_stack_prefill(int dtype, int nlayers, int B, int H, int64_t T, int hd, int dm,
                      const int32_t* D, const int32_t* W, float scale, int64_t T_cap,
                      const void* x, const void* const* w_q, const void* const* w_k,
                      const void* const* w_v, const void* const* w_g,
                      const float* const* b_g, const void* const* w_o, void* out,
                      void* const* Kc, void* const* Vc, void* const* k_ring,
                      void* const* v_ring, float* const* state_k, float* const* state_v,
                      void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RAT_H_ */
