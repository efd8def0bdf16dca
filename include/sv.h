/*
 * sv.h -- SparseVILA decoupled visual sparsity: the data-parallel hot path on
 * AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * Method (arXiv 2510.17777, "SparseVILA: Decoupling Visual Sparsity for
 * Efficient VLM Inference"): prefill prunes visual tokens by query-agnostic
 * salience computed from the vision encoder's self-attention; decode keeps
 * the retained visual KV cache and, per query, activates only the top-k most
 * relevant visual tokens for attention.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or writes its inputs; outputs and the
 *    caller-provided workspace are the only memory it writes.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Nothing synchronises (except sv_workspace_status); results
 *    are valid once the stream has executed the enqueued work.  Device-side
 *    faults surface at the caller's next synchronisation.
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    non-OK status means nothing was launched (except SV_EHIP, which reports
 *    a failed launch); sv_last_error() then returns a thread-local message.
 *  - Element strides are in ELEMENTS, not bytes.  Within a token row the
 *    layout is [H][D] with D contiguous (head stride D).
 *  - Outputs that are indices are int32; scores, salience and attention
 *    outputs are fp32.  No C++ exception crosses this boundary.
 *  - NaN or Inf inputs give unspecified (but memory-safe) results.
 *  - Concurrent calls on different streams are safe if their workspaces and
 *    outputs do not overlap.
 */
#ifndef SV_H_
#define SV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_EINVAL = 1,        /* bad shape, count, pointer or stride           */
  SV_EUNSUPPORTED = 2,  /* valid request outside the compiled kernels     */
  SV_EWORKSPACE = 3,    /* workspace_bytes below the *_workspace() size   */
  SV_EHIP = 4           /* a HIP runtime call or kernel launch failed     */
} sv_status;

typedef enum {
  SV_F32 = 0,           /* IEEE binary32                                  */
  SV_BF16 = 1           /* bfloat16 (upper half of binary32)              */
} sv_dtype;

/* Library version, major*10000 + minor*100 + patch. */
int sv_version(void);

/* Message describing the last non-OK status returned on this thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char* sv_last_error(void);

/* ------------------------------------------------------------------------
 * Bounded in-kernel waits
 *
 * sv_retrieve (rows of more than 2048 tokens) and sv_retrieve_attend run
 * work items that wait on other workgroups of the same launch (a select on
 * the scan items, the attention items on the select).  The hardware
 * dispatches each XCD's share of a 1-D grid in increasing workgroup order
 * and every item waits only on items of lower index, so every wait ends;
 * each is still bounded, by a number of polls.  A wait that reaches the
 * bound gives up: the item carries on with what it read (memory-safe, but
 * the launch's indices and outputs are then invalid) and ORs a bit into the
 * workspace's STATUS WORD, the first 32-bit word of the workspace (the
 * workspaces of these two calls begin with a 256-byte status line that the
 * kernels never clear):
 *     1 scores never complete (select)      2 indices never complete (attention)
 *     4 scan items never all counted        8 candidate items never all counted
 *    16 threshold never published           (4, 8, 16: rows over 2048 tokens)
 * After a give-up the workspace's other control words may be left non-zero:
 * zero the whole workspace before its next use.
 *
 * sv_workspace_status: enqueues a copy of the status word on `stream`, WAITS
 * for the stream (the only call of this library that synchronises) and
 * returns SV_OK if the word is zero, SV_EHIP (with the bits in
 * sv_last_error()) if a wait has given up since the workspace was zeroed.
 * workspace == NULL reads the static scratch of the current device instead
 * (sv_retrieve_attend_noalloc, which zeroes it at every call: the status of
 * the last such call on the device).
 * Errors: SV_EHIP (copy or sync failed).
 *
 * sv_set_wait_limit: sets the bound, in polls, for launches enqueued after
 * it in this process (0 restores the default, 2^24 polls, seconds of
 * polling) and returns the previous bound.  A small bound makes waits give
 * up early; this is meant for testing the failure path, where every kernel
 * still runs to completion.
 * ---------------------------------------------------------------------- */
sv_status sv_workspace_status(const void* workspace, void* stream);

uint32_t sv_set_wait_limit(uint32_t polls);

/* ------------------------------------------------------------------------
 * Query-aware retrieval (decode stage)
 *
 * SparseVILA velog summary, Sec. 3.2 "Query-Aware Token Selection": the
 * current text query is the Query, the cached vision tokens are the Keys,
 * and the aggregated attention strength ranks the tokens; high scorers are
 * activated, the rest stay cached but deactivated.  xllm-io review,
 * core formulas: Selected = TopK(Query . KV_Cache, k).
 *
 * Computes, per sequence b,
 *     s[b,t] = sum_{tau<Tq} sum_{h<Hq} q[b,tau,h,:] . K[b,t,h/G,:]   (G = Hq/Hkv)
 * (raw logits, no 1/sqrt(D)), then the k largest s[b,.] with ties broken
 * toward the lower token index, written in ascending index order.
 *
 *  q          [B][Tq][Hq][D], contiguous, dtype `dtype`.  Tq = 1 scores the
 *             current decode token; Tq > 1 scores a whole question.
 *  k_vis      retained visual keys: element (b,t,g,d) at
 *             k_vis[b*k_bstride + t*k_tstride + g*D + d].  Read only.
 *  N          visual tokens per sequence (N >= 1).
 *  k          tokens to select, 0 <= k <= N.
 *  idx_out    [B][k] int32, ascending, distinct, each in [0, N).
 *  scores_out optional [B][N] fp32 scores s (NULL to skip).
 *  workspace  at least sv_retrieve_workspace(B, N, k) bytes, 256-byte
 *             aligned, ZERO-FILLED before its first use.  It holds the status
 *             line (see sv_workspace_status), the scores and one completion
 *             counter per sequence and, for rows
 *             of more than 2048 tokens, the histograms, counters and
 *             candidate lists of the parallel select; every call returns
 *             the counters and histograms to zero, so the same workspace can
 *             be reused for calls of the same B and N (and a call can be
 *             captured in a HIP graph) without clearing it again.
 * Rows of more than 2048 tokens with Hq/Hkv <= 8 and k > 0 are selected by
 * many workgroups (each pass over a row split into 2048-score chunks);
 * other rows by the last scan workgroup of each sequence.
 * Supported: dtype SV_BF16 or SV_F32; D in {64, 128}; Hkv*D <= 8192 (bf16)
 * or <= 4096 (fp32); Hq % Hkv == 0; Hq/Hkv <= 64; B <= 65535.
 * Errors: SV_EINVAL (k > N, k < 0, N < 1, B < 1, Tq < 1, Hq % Hkv != 0,
 * NULL q/k_vis/idx_out/workspace, strides smaller than a row),
 * SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP.
 * ---------------------------------------------------------------------- */
size_t sv_retrieve_workspace(int B, int N, int k);

sv_status sv_retrieve(const void* q, int B, int Tq, int Hq,
                      const void* k_vis, int64_t k_bstride, int64_t k_tstride,
                      int N, int Hkv, int D, sv_dtype dtype, int k,
                      int32_t* idx_out, float* scores_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Sparse decode attention over the retrieved visual entries plus the text
 * entries (decode stage)
 *
 * SparseVILA velog summary, Sec. 3.2 (only the query-relevant subset of the
 * visual cache is activated; the cache itself is kept) and Sec. 4.5
 * (decoding attention over the reduced effective KV cache).
 *
 * For each sequence b and query head h (KV head g = h / G):
 *     E = { visual idx[b][0..k) } U { text rows 0..txt_len[b]-1 }
 *     z_j = scale * q[b,h,:] . K_j[g,:]
 *     out[b,h,:] = sum_j softmax(z)_j V_j[g,:]
 * Visual indices outside [0, N) are skipped; txt_len[b] is clamped to
 * [0, Tmax].  If E is empty for some b, out[b,:,:] = 0.
 *
 *  q          [B][Hq][D], contiguous, dtype `dtype` (the current token's
 *             post-RoPE queries).
 *  k_vis,v_vis visual cache, element (b,t,g,d) at
 *             ptr[b*vis_bstride + t*vis_tstride + g*D + d].  Read only.
 *  idx        [B][k] int32 visual token indices (any order; distinct), or
 *             NULL: the visual entries are rows 0..k-1 of the visual cache (a
 *             packed cache such as sv_pack_selected writes; no index list is
 *             read).
 *  k_txt,v_txt text cache, element (b,t,g,d) at
 *             ptr[b*txt_bstride + t*txt_tstride + g*D + d], t < Tmax.
 *             May be NULL only if Tmax == 0.
 *  txt_len    [B] int32 device array, text rows attended per sequence.
 *  scale      softmax scale; <= 0 selects 1/sqrt(D).
 *  out        [B][Hq][D] fp32.
 *  workspace  at least sv_sparse_decode_attn_workspace(B, Hq, Hkv, D, k, Tmax)
 *             bytes, 256-byte aligned, ZERO-FILLED before its first use.  It
 *             holds the split partials and one completion counter per
 *             (sequence, KV head); every call returns the counters to zero,
 *             so the workspace can be reused without clearing.
 * Supported: dtype SV_BF16 or SV_F32; D in {64, 128}; Hq/Hkv in 1..8.
 * Errors: SV_EINVAL (k < 0, k + Tmax == 0, k > N, Hq % Hkv != 0, NULL
 * required pointer (q, out, workspace; the caches when k > 0; the text
 * arrays when Tmax > 0), B < 1), SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP.
 * ---------------------------------------------------------------------- */
size_t sv_sparse_decode_attn_workspace(int B, int Hq, int Hkv, int D, int k, int Tmax);

sv_status sv_sparse_decode_attn(const void* q, int B, int Hq,
                                const void* k_vis, const void* v_vis,
                                int64_t vis_bstride, int64_t vis_tstride, int N,
                                int Hkv, int D, const int32_t* idx, int k,
                                const void* k_txt, const void* v_txt,
                                int64_t txt_bstride, int64_t txt_tstride,
                                const int32_t* txt_len, int Tmax,
                                sv_dtype dtype, float scale, float* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Retrieval + sparse decode attention of one layer in one launch
 *
 * The same computation as sv_retrieve (Tq = 1) followed by
 * sv_sparse_decode_attn on its indices (SparseVILA velog summary, Sec. 3.2:
 * the current query selects the top-k visual tokens, and only those plus the
 * text entries are attended; Sec. 4.5: decode attention over the reduced
 * cache), as one kernel: the select of a sequence overlaps the attention
 * over its text entries and the other sequences' work.
 *
 *  q          [B][Hq][D], contiguous (Tq = 1: one decode token).
 *  k_vis,v_vis visual cache, element (b,t,g,d) at
 *             ptr[b*vis_bstride + t*vis_tstride + g*D + d], t < N.
 *  k          visual tokens to select and attend, 1 <= k <= N.
 *  k_txt,v_txt,txt_len,Tmax,scale  as for sv_sparse_decode_attn.
 *  idx_out    [B][k] int32: the selected indices, ascending (as sv_retrieve).
 *  scores_out optional [B][N] fp32 scores (NULL: kept in the workspace).
 *  out        [B][Hq][D] fp32 attention output.
 *  workspace  at least sv_retrieve_attend_workspace(B, Hq, Hkv, D, N, k, Tmax)
 *             bytes, 256-byte aligned, ZERO-FILLED before its first use.  It
 *             holds the status line (see sv_workspace_status), the scores,
 *             the split partials and a control block (completion counters,
 *             per-sequence ready flags); every call
 *             leaves it ready for the next call with the same B, N, Hq, Hkv,
 *             D, k and Tmax, so it can be reused as is and the call captured
 *             in a HIP graph.  For other sizes, zero it again (or use
 *             another).  Two calls that share a workspace must not run
 *             concurrently.
 * Supported: dtype SV_BF16 or SV_F32; D in {64, 128}; Hq/Hkv in 1..8;
 * Hkv*D <= 8192 (bf16) or <= 4096 (fp32); B <= 65535.
 * Errors: SV_EINVAL (k < 1, k > N, Hq % Hkv != 0, NULL required pointer,
 * bad strides or alignment), SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP.
 * ---------------------------------------------------------------------- */
size_t sv_retrieve_attend_workspace(int B, int Hq, int Hkv, int D, int N, int k, int Tmax);

sv_status sv_retrieve_attend(const void* q, int B, int Hq,
                             const void* k_vis, const void* v_vis,
                             int64_t vis_bstride, int64_t vis_tstride, int N,
                             int Hkv, int D, int k,
                             const void* k_txt, const void* v_txt,
                             int64_t txt_bstride, int64_t txt_tstride,
                             const int32_t* txt_len, int Tmax,
                             sv_dtype dtype, float scale,
                             int32_t* idx_out, float* scores_out, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * sv_retrieve_attend without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).
 *
 * Computes exactly what sv_retrieve_attend computes (same kernel, same
 * arguments and errors, minus the workspace).  Its workspace is a static
 * device array of SV_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * every device it runs on until the process ends; the call zeroes the part
 * it needs on `stream` (a fill kernel, no memset node) before the layer's
 * kernel.  Nothing is allocated.  All calls on one device share that array:
 * two calls that overlap on one device (different streams, or host threads)
 * race and both give undefined results; serialise them.
 * Errors: as sv_retrieve_attend, and SV_EWORKSPACE when
 * sv_retrieve_attend_workspace(...) of the sizes exceeds
 * SV_NOALLOC_SCRATCH_BYTES (16 MiB: enough for 8 x 131072 visual tokens of
 * 32 x 128 heads with k = 4096 and 256 text rows).
 * ---------------------------------------------------------------------- */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)

sv_status sv_retrieve_attend_noalloc(const void* q, int B, int Hq,
                                     const void* k_vis, const void* v_vis,
                                     int64_t vis_bstride, int64_t vis_tstride, int N,
                                     int Hkv, int D, int k,
                                     const void* k_txt, const void* v_txt,
                                     int64_t txt_bstride, int64_t txt_tstride,
                                     const int32_t* txt_len, int Tmax,
                                     sv_dtype dtype, float scale,
                                     int32_t* idx_out, float* scores_out, float* out,
                                     void* stream);

/* ------------------------------------------------------------------------
 * Dense packing of the selected visual entries (decode stage, once per
 * question)
 *
 * SparseVILA velog summary, Sec. 3.2, decode side: the selected KV entries
 * are gathered into contiguous memory, so that decode reads them with
 * regular, coalesced accesses; Sec. 3.3, kernel table, decoding-attention
 * row: decode attends that packed, reduced cache.  Typical use: sv_retrieve
 * with Tq = the question's tokens, then sv_pack_selected, then every decode
 * step of the answer calls sv_sparse_decode_attn on the packed rows
 * (N = k, idx = 0..k-1) plus the text entries.
 *
 * For each sequence b and j < k, with t = idx[b][j]:
 *     k_pack[b][j][:][:] = K[b][t][:][:],  v_pack[b][j][:][:] = V[b][t][:][:]
 * for 0 <= t < N; a zero row for any other t.  Every KV head of the token is
 * copied; values are moved, never converted (bit-exact).
 *
 *  k_vis,v_vis visual cache, element (b,t,g,d) at
 *             ptr[b*vis_bstride + t*vis_tstride + g*D + d], t < N.  Read only.
 *  idx        [B][k] int32 (any order; repeats allowed).
 *  k_pack,v_pack  [B][k][Hkv][D] contiguous, dtype `dtype`; must not overlap
 *             the caches.
 * No workspace.  k == 0 enqueues nothing and returns SV_OK.
 * Supported: dtype SV_BF16 or SV_F32; Hkv*D a multiple of 8 (bf16) or 4
 * (fp32), at most 2^24; 16-byte aligned pointers.
 * Errors: SV_EINVAL (B < 1, N < 1, Hkv < 1, D < 1, k < 0, NULL pointer,
 * strides smaller than a row or not multiples of 16 bytes, misalignment),
 * SV_EUNSUPPORTED, SV_EHIP.
 * ---------------------------------------------------------------------- */
sv_status sv_pack_selected(const void* k_vis, const void* v_vis, int64_t vis_bstride,
                           int64_t vis_tstride, int N, int Hkv, int D, sv_dtype dtype,
                           const int32_t* idx, int B, int k, void* k_pack, void* v_pack,
                           void* stream);

/* ------------------------------------------------------------------------
 * Query-agnostic salience and per-frame pruning (prefill stage)
 *
 * SparseVILA velog summary, Sec. 3.1: salience is read off the vision
 * encoder's self-attention; for encoders without a summary token (SigLIP,
 * QwenVL) it is the intra-visual attention averaged over all tokens, and the
 * lowest-salience tokens are pruned before the cache is stored.  The same
 * section's kernel streams the softmax normalisation and the salience
 * accumulation without materialising the attention matrix.  xllm-io review,
 * core formulas: Salience(t_i) = (1/N) sum_j Attention(., .), read as the
 * attention token i receives (column mean).
 *
 * For each frame f (an independent attention of N tokens) and head h:
 *     A_h = row_softmax(scale * Q_h K_h^T)                 (never stored)
 *     sal[f,j] = (1/H) sum_h (1/N) sum_i A_h[i,j]           (sums to 1)
 * then the `keep` largest sal[f,.] (ties toward the lower index) in
 * ascending order.
 *
 *  vis_q,vis_k [F][H][N][D] contiguous bf16 (one encoder layer's Q and K).
 *  scale       softmax scale; <= 0 selects 1/sqrt(D).
 *  keep        tokens kept per frame, 0 <= keep <= N.
 *  salience_out optional [F][N] fp32 (NULL to skip).
 *  idx_out     [F][keep] int32 ascending (may be NULL if keep == 0).
 *  workspace   at least sv_salience_prune_workspace(F, H, N) bytes,
 *              256-byte aligned.
 * Kernels: frames of N <= 768 tokens with D <= 96 keep one frame-head's
 * keys on chip (one fused pass); longer frames (QwenVL-style encoders,
 * 10^4 - 10^5 tokens) or wider heads take two streaming passes (row
 * log-sum-exp, then column sums), the attention map never stored either way.
 * Supported: dtype SV_BF16; D a multiple of 8 with 8 <= D <= 128; N >= 1;
 * F*H*ceil(N/256) <= 2^31-1.
 * Errors: SV_EINVAL, SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP.
 * ---------------------------------------------------------------------- */
size_t sv_salience_prune_workspace(int F, int H, int N);

sv_status sv_salience_prune(const void* vis_q, const void* vis_k, int F, int H,
                            int N, int D, sv_dtype dtype, float scale, int keep,
                            float* salience_out, int32_t* idx_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Summary-token salience and per-frame pruning (prefill stage)
 *
 * SparseVILA velog summary, Sec. 3.1, salience table: for an encoder with
 * one summary token (CLIP) a token's importance is the attention through
 * which it feeds that global token; with several summary tokens (RADIO) it
 * is that attention averaged over them.  The summary tokens are the first S
 * tokens of each frame (CLIP's CLS token: S = 1).
 *
 * For each frame f and head h:
 *     A_h = row_softmax(scale * Q_h[0:S] K_h^T)            (S x N, never stored)
 *     sal[f,j] = (1/H) sum_h (1/S) sum_{s<S} A_h[s,j]       (sums to 1)
 * over every token j, summary tokens included; then the `keep` largest
 * sal[f,.] (ties toward the lower index) in ascending order.
 *
 *  vis_q,vis_k [F][H][N][D] contiguous bf16 (one encoder layer's Q and K;
 *             only rows 0..S-1 of Q are read).
 *  scale       softmax scale; <= 0 selects 1/sqrt(D).
 *  S           summary tokens, 1 <= S <= N.
 *  keep        tokens kept per frame, 0 <= keep <= N.
 *  salience_out optional [F][N] fp32 (NULL: kept in the workspace).
 *  idx_out     [F][keep] int32 ascending (may be NULL if keep == 0).
 *  workspace   at least sv_summary_salience_prune_workspace(F, H, N) bytes,
 *              256-byte aligned; no zero-fill needed.
 * Supported: dtype SV_BF16; D a multiple of 8, at most 128; S <= 16,
 * N <= 4096, S*N <= 12288; F <= 65535.
 * Errors: SV_EINVAL (NULL pointer, S or keep out of range, bad sizes,
 * misalignment), SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP.
 * ---------------------------------------------------------------------- */
size_t sv_summary_salience_prune_workspace(int F, int H, int N);

sv_status sv_summary_salience_prune(const void* vis_q, const void* vis_k, int F, int H, int N,
                                    int D, sv_dtype dtype, float scale, int S, int keep,
                                    float* salience_out, int32_t* idx_out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Prefill attention of a question chunk with the query-aware retrieval
 * fused into it (once per question)
 *
 * SparseVILA velog summary, Sec. 3.2 (query-aware token selection, its
 * implementation note): the question's retrieval salience is computed
 * alongside its ordinary (FlashAttention) prefill attention; Sec. 3.3,
 * kernel table (retrieval-salience row).  The logits of every question token
 * against every visual key feed both: the causal softmax attention of the
 * question, and (raw, summed over the question's tokens and the query heads
 * of each KV head) the retrieval score.  One pass over the caches does both.
 *
 * For each sequence b, question token tau < Tq (text position
 * p = txt_len[b] - Tq + tau) and query head h (KV head g = h / G):
 *     E = { all N visual tokens } U { text rows 0..p }      (none if p < 0)
 *     out[b,tau,h,:] = sum_{j in E} softmax_j(scale * q[b,tau,h,:] . K_j[g,:]) V_j[g,:]
 *     s[b,t] = sum_{tau<Tq} sum_{h<Hq} q[b,tau,h,:] . K_vis[b,t,g,:]
 * (s exactly as sv_retrieve with the same Tq), then the k largest s[b,.]
 * (ties toward the lower index) in ascending order.
 *
 *  q          [B][Tq][Hq][D], contiguous, bf16 (post-RoPE question tokens).
 *  k_vis,v_vis visual cache, element (b,t,g,d) at
 *             ptr[b*vis_bstride + t*vis_tstride + g*D + d], t < N.  Read only.
 *  k_txt,v_txt text cache, element (b,t,g,d) at
 *             ptr[b*txt_bstride + t*txt_tstride + g*D + d], t < Tmax; the
 *             first txt_len[b] rows are valid and the LAST Tq of them are
 *             the question's own K/V (appended by the caller).  May be NULL
 *             only if Tmax == 0.
 *  txt_len    [B] int32 device array (clamped to [0, Tmax]).
 *  scale      softmax scale; <= 0 selects 1/sqrt(D).
 *  k          tokens to select, 0 <= k <= N (0: no selection).
 *  out        [B][Tq][Hq][D] fp32.
 *  idx_out    [B][k] int32, ascending (may be NULL if k == 0).
 *  scores_out optional [B][N] fp32 retrieval scores (NULL: workspace).
 *  workspace  at least sv_prefill_attend_retrieve_workspace(...) bytes,
 *             256-byte aligned, ZERO-FILLED before its first use.  It holds
 *             one completion counter per sequence (the last workgroup of a
 *             sequence runs its retrieval), the split partials and the
 *             partial scores; every call returns the counters to zero, so
 *             the workspace can be reused without clearing.  Two calls that
 *             share a workspace must not run concurrently.
 * Supported: dtype SV_BF16; D in {64, 128}; Hq % Hkv == 0;
 * Tq * Hq / Hkv <= 2^20; (N + 32) * vis_tstride and (Tmax + 32) * txt_tstride
 * elements below 2^30 (one sequence's cache under 2 GiB).
 * Errors: SV_EINVAL (bad sizes or k, NULL required pointer, strides smaller
 * than a row or not multiples of 8 elements, misalignment),
 * SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP.
 * ---------------------------------------------------------------------- */
size_t sv_prefill_attend_retrieve_workspace(int B, int Tq, int Hq, int Hkv, int D, int N,
                                            int Tmax);

sv_status sv_prefill_attend_retrieve(const void* q, int B, int Tq, int Hq,
                                     const void* k_vis, const void* v_vis,
                                     int64_t vis_bstride, int64_t vis_tstride, int N,
                                     int Hkv, int D,
                                     const void* k_txt, const void* v_txt,
                                     int64_t txt_bstride, int64_t txt_tstride,
                                     const int32_t* txt_len, int Tmax,
                                     sv_dtype dtype, float scale, int k,
                                     float* out, int32_t* idx_out, float* scores_out,
                                     void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SV_H_ */
