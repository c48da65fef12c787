/*
 * rva.h -- C ABI of the ragged verify + acceptance library (librva.so, gfx950 / MI355X).
 *
 * One speculative-decoding step, verify side, as five calls (and a measurement variant) that each only enqueue HIP
 * kernels on the caller's stream:
 *
 *   rva_schedule_windows   stage 1  confidence head + temperature scaling, prefix
 *                                   survival, per-request verify window
 *   rva_pack_ragged        stage 2  ragged packing of the window rows + tier rounding
 *   rva_schedule_and_pack  stages 1 + 2 in one launch (same outputs)
 *   rva_verify_attention   stage 3  varlen GQA attention over the paged KV cache (+ append)
 *   rva_verify_attention_noalloc  stage 3 with a library-owned scratch (no workspace)
 *   rva_accept_and_commit  stage 4  speculative-sampling acceptance, draw, commit
 *                          (+ stage 5 TV labels when `labels` is given)
 *   rva_confidence_labels  stage 5  TV-distance confidence labels on their own
 *   rva_accept_capped      stage 4 in cap-accept mode (whole block verified, commit capped
 *                          at the window, uncapped acceptance reported)
 *   rva_sts_fit            calibration: per-position temperatures of the confidence head
 *                          fitted to acceptance traces (input of stage 1)
 *   rva_calibration_ece    calibration: expected calibration error of the survival
 *   rva_markov_sample      drafter side: Markov sequential head, per-position logits and
 *                          draws in order (produces the draft tokens and logits of stage 4)
 *
 * Sources, cited by page title and section:
 *   [SGL]   "DFlash 到 DSpark in SGLang：解码提速 4.3×，以及 DeepSeek-V4 支持"
 *           (yichizhang.dev, AI-Infra-Visualized).
 *   [CSDN]  devpress.csdn.net (awstech) article on DSpark in SGLang, sections 2-5.
 *   [NOTES] "DSpark：投机解码与生产级 Serving 学习笔记" (sorenprojections.com).
 *
 * Conventions shared by every call
 *   - Ownership: the caller allocates every buffer and owns it; the library allocates
 *     nothing and keeps no state between calls (the thread-local error text aside, and the
 *     static scratch that rva_verify_attention_noalloc uses in place of a workspace).
 *   - Pointers: all array arguments are DEVICE pointers unless the parameter name ends
 *     in `_host`.  Scalars are passed by value.
 *   - Asynchrony: a call validates its scalar arguments on the host, enqueues kernels on
 *     `stream` and returns.  No call synchronises or reads device memory back, so the
 *     packed total and the tier stay on the device (kernels are sized by host-known
 *     bounds and exit early).
 *   - Errors: the return value reports argument errors (nothing is enqueued) and launch
 *     failures; rva_last_error() gives a message for the calling thread.  Errors found in
 *     device data (a window out of range, a token id >= V, ...) are OR-ed as
 *     RVA_DEV_* bits into the optional `device_status` word (caller zeroes it); the
 *     kernels then clamp or skip so that every access stays in bounds, and the affected
 *     outputs are unspecified.
 *   - Windows count packed verify rows ANCHOR INCLUDED: a block has `gamma` positions,
 *     position 0 is the anchor (last committed token) and positions 1..gamma-1 are
 *     drafts, so a window w is in [1, gamma] and verifies w-1 drafts.
 *   - Overlapping calls on one stream are ordered by the stream; two calls that write the
 *     same buffers on different streams race.
 */
#ifndef RVA_H
#define RVA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RVA_VERSION 100 /* 1.0.0 */

typedef enum {
  RVA_OK = 0,
  RVA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, inconsistent sizes, bad enum        */
  RVA_ERR_UNSUPPORTED = 2,        /* valid but not implemented (e.g. D not in {64,128}) */
  RVA_ERR_WORKSPACE_TOO_SMALL = 3,
  RVA_ERR_HIP = 4                 /* a HIP launch or runtime call failed                */
} rva_status;

typedef enum { RVA_F32 = 0, RVA_BF16 = 1 } rva_dtype;
typedef enum { RVA_MODE_COMPACT = 0, RVA_MODE_STATIC = 1 } rva_mode;

/* device_status bits */
#define RVA_DEV_BAD_WINDOW   0x01 /* window outside [1, gamma] / [1, max_window]        */
#define RVA_DEV_BAD_TOKEN    0x02 /* draft token id outside [0, V)                      */
#define RVA_DEV_BAD_CONF     0x04 /* confidence NaN or outside [0, 1]                   */
#define RVA_DEV_BAD_COST     0x08 /* a step cost T(B, K) that is not > 0                */
#define RVA_DEV_BAD_CONTEXT  0x10 /* context_lens[b] < 0 or L + w beyond the page table */
#define RVA_DEV_BAD_PAGE     0x20 /* block_table entry outside [0, num_pages)           */
#define RVA_DEV_BAD_ROWS     0x40 /* packed rows beyond max_rows                        */

/*
 * Stage 1 -- rva_schedule_windows
 *
 * [SGL] "DSpark：sequential head 加验证预算", [NOTES] section 07: the confidence head is a
 * linear layer + sigmoid on the drafter hidden state, one score per draft position, and
 * a per-position temperature (Sequential Temperature Scaling) calibrates it.
 * [NOTES] section 07: prefix survival a_j = prod_{i<=j} c_i.
 * [NOTES] section 08 and [CSDN] section 4: windows maximise expected accepted tokens per
 * unit of step time against the additive cost T(bs, K) = bias + alpha(bs) + theta(bs+K).
 *
 *   c[b,k]  = conf_in[b,k]                            if conf_in != NULL
 *           = sigmoid((hidden[b,k,:].head_w + head_b) / T_k)   otherwise
 *             (T_k = sts_T[k], or 1 when sts_T == NULL; float64 math, rounded to float32)
 *   a[b,0]  = c[b,0];  a[b,j] = fl32(a[b,j-1] * c[b,j])      (left to right, float32)
 *   rank all (b, j) by a descending, then b ascending, then j ascending;
 *   E_K = B + (float64 sum of the K largest a);  T_K = (bias + alpha[B]) + theta[B+K]
 *   K*  = argmax_{0<=K<=B(gamma-1)} E_K / T_K (smallest K on a tie); RVA_MODE_STATIC: K* = B(gamma-1)
 *   windows[b] = 1 + number of request b's candidates among the first K*
 *
 * Arguments
 *   B, gamma        requests, block length (anchor included); 2 <= gamma <= 64,
 *                   1 <= B, B*(gamma-1) <= 4096.
 *   mode            RVA_MODE_COMPACT (scheduled windows) or RVA_MODE_STATIC (all gamma).
 *   hidden          [B, gamma-1, H] of hidden_dtype, row-major; NULL iff conf_in given.
 *   head_w          [H] float32 (device); head_b by value.
 *   conf_in         [B, gamma-1] float32 in [0,1], or NULL.  sts_T must be NULL with it.
 *   sts_T           [gamma-1] float32 temperatures (> 0) or NULL.
 *   bias_ms         float32 scalar; alpha_ms [alpha_len] with alpha_len > B;
 *                   theta_ms [theta_len] with theta_len > B*gamma (device, float32).
 *   conf_out, surv_out  [B, gamma-1] float32 outputs (c and a).  Above 1024 candidates the
 *                   call is two launches and surv_out carries the candidates' ranks (as bits)
 *                   from the first to the second, which then writes a: like every output, it
 *                   holds its result once the call's work on `stream` is done.
 *   windows         [B] int32 output; K_out [1] int32; ratio_out [1] float64 (E over T at K*).
 *   device_status   optional int32 word (RVA_DEV_BAD_CONF, RVA_DEV_BAD_COST).
 */
rva_status rva_schedule_windows(int B, int gamma, int mode,
                                const void* hidden, int hidden_dtype, int H,
                                const float* head_w, float head_b,
                                const float* conf_in, const float* sts_T,
                                float bias_ms, const float* alpha_ms, int alpha_len,
                                const float* theta_ms, int theta_len,
                                float* conf_out, float* surv_out,
                                int32_t* windows, int32_t* K_out, double* ratio_out,
                                int32_t* device_status, hipStream_t stream);

/*
 * Stage 2 -- rva_pack_ragged
 *
 * [SGL] "Ragged verify under full CUDA graphs", [CSDN] section 3: the scheduled rows are
 * packed end to end into one [total_tokens, hidden] buffer with cu_seqlens-style
 * offsets, and the total is rounded up to the nearest captured tier.
 *
 *   cu_seqlens[0] = 0, cu_seqlens[b+1] = cu_seqlens[b] + windows[b];  M = cu_seqlens[B]
 *   tier = smallest tiers_host[t] >= M;  total_tier = {M, tier}
 *   dst[cu[b] + i] = src[b, i] for i < windows[b];  dst rows [M, tier) = 0
 *   row_req[r] = owning request or -1;  row_pos[r] = context_lens[b] + i or -1
 *   (row_req/row_pos are written for every r < max_rows; dst rows >= tier are untouched)
 *
 * Arguments
 *   windows [B], context_lens [B] int32 (device).
 *   tiers_host      HOST array of n_tiers ascending int32, 1 <= n_tiers <= 512,
 *                   tiers_host[n_tiers-1] >= B*gamma.
 *   src             [B, gamma, row_bytes] bytes or NULL (metadata only); dst
 *                   [max_rows, row_bytes] (NULL iff src NULL); max_rows >= tiers_host[n_tiers-1].
 *   cu_seqlens [B+1], row_req [max_rows], row_pos [max_rows], total_tier [2] int32 outputs.
 *   device_status   optional (RVA_DEV_BAD_WINDOW: the window is clamped into [1, gamma]).
 */
rva_status rva_pack_ragged(int B, int gamma, const int32_t* windows,
                           const int32_t* context_lens,
                           const int32_t* tiers_host, int n_tiers,
                           const void* src, size_t row_bytes, void* dst, int max_rows,
                           int32_t* cu_seqlens, int32_t* row_req, int32_t* row_pos,
                           int32_t* total_tier, int32_t* device_status, hipStream_t stream);

/*
 * Stages 1 + 2 in one call -- rva_schedule_and_pack
 *
 * [SGL] "Zero-overhead scheduling 与 kernel", [CSDN] section 4: the scheduling decision is on
 * the step's critical path, so it should cost as little as possible.  Exactly
 * rva_schedule_windows followed by rva_pack_ragged with the windows it wrote (same
 * arguments, same outputs bit for bit, same device-status bits), enqueued as ONE kernel
 * launch when B*(gamma-1) <= 1024 (plus the head kernel when hidden states are given):
 * every workgroup of the pack grid runs the scheduling pass itself, so the windows never
 * make a round trip through memory between the stages.  Larger batches take the two
 * kernels.  Validation is that of both calls (pack's gamma is this call's gamma).
 */
rva_status rva_schedule_and_pack(int B, int gamma, int mode, const void* hidden, int hidden_dtype, int H,
                                 const float* head_w, float head_b, const float* conf_in,
                                 const float* sts_T, float bias_ms, const float* alpha_ms, int alpha_len,
                                 const float* theta_ms, int theta_len, float* conf_out, float* surv_out,
                                 int32_t* windows, int32_t* K_out, double* ratio_out,
                                 const int32_t* context_lens, const int32_t* tiers_host, int n_tiers,
                                 const void* src, size_t row_bytes, void* dst, int max_rows,
                                 int32_t* cu_seqlens, int32_t* row_req, int32_t* row_pos,
                                 int32_t* total_tier, int32_t* device_status, hipStream_t stream);

/*
 * Stage 3 -- rva_verify_attention
 *
 * [SGL] "Ragged verify under full CUDA graphs", [CSDN] section 3: each packed token attends
 * only to its own request's KV (varlen, cu_seqlens).  Window row i of request b (packed
 * row r = cu[b] + i), query head h, kv head g = h / (Hq / Hkv):
 *   keys/values: cache positions 0 .. L_b-1 (L_b = context_lens[b]) through the page
 *   table, then the window's own rows 0 .. i from k_new / v_new (causal);
 *   out[r, h] = softmax(q[r,h] . K^T * softmax_scale) V, float32 accumulation.
 * Output rows [M, tier) are zeroed.  The window's K/V rows are appended to the cache at
 * positions L_b .. L_b + w_b - 1 (context_lens itself is not changed here).
 *
 * Cache layout (the pages only say "paged, page table on the device"; this layout is the
 * library's choice):
 *   k_cache [num_pages, Hkv, page_size, D]             element (page, g, slot, d)
 *   v_cache [num_pages, Hkv, page_size / VB, D, VB]    element (page, g, slot / VB, d, slot % VB)
 *     V is stored transposed in column blocks of VB slots, VB = 32 when page_size is a
 *     multiple of 32, else VB = page_size (the whole page is one block).  A block of 32
 *     keys of one d is 64 contiguous bf16 bytes, so the P.V product reads V in full
 *     128-byte lines for a 64-slot page instead of half lines.
 *   position p of request b -> page block_table[b * max_pages + p / page_size], slot p % page_size.
 *   Pages the append writes into must not be shared with another request.
 *
 * Arguments
 *   B               1 <= B <= 65535.
 *   max_window      upper bound of every window (gamma); max_window * (Hq/Hkv) <= 4096
 *                   (otherwise RVA_ERR_UNSUPPORTED).  Above 64 (query columns per kv
 *                   head) the call takes the generic path.
 *   max_rows        rows of q / k_new / v_new / out (>= the largest tier).
 *   Hq, Hkv, D      Hq % Hkv == 0; D in {64, 128}.
 *   page_size       >= 1 (the bf16 MFMA path needs a power of two >= 32; others take the
 *                   generic path).
 *   kv_dtype        RVA_BF16 or RVA_F32: dtype of q, k_new, v_new, caches and out.
 *   q [max_rows, Hq, D], k_new / v_new [max_rows, Hkv, D], out [max_rows, Hq, D].
 *   block_table [B, max_pages], context_lens [B], cu_seqlens [B+1], total_tier [2] int32.
 *   workspace       device scratch of at least rva_verify_attention_workspace_size(...)
 *                   bytes (may be NULL when that size is 0); contents need no init.
 *   device_status   optional (BAD_WINDOW, BAD_CONTEXT, BAD_PAGE, BAD_ROWS: the request is
 *                   skipped).
 */
rva_status rva_verify_attention(int B, int max_window, int max_rows, int Hq, int Hkv, int D,
                                int page_size, int num_pages, int max_pages, int kv_dtype,
                                const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int32_t* block_table,
                                const int32_t* context_lens, const int32_t* cu_seqlens,
                                const int32_t* total_tier, float softmax_scale, void* out,
                                int32_t* device_status, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

size_t rva_verify_attention_workspace_size(int B, int max_window, int Hq, int Hkv, int D,
                                           int page_size, int max_pages, int kv_dtype);

/*
 * Stage 3 without a workspace -- rva_verify_attention_noalloc
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Identical to rva_verify_attention
 * (same arguments minus the workspace, same kernels, bit-identical results), except that
 * the stream-K partials and merge records go to a library-owned static scratch of
 * 24 MiB per device instead of a caller workspace.  Nothing is allocated by the call.
 *   - The scratch is a file-scope device array, zero at load and held by each device the
 *     library runs on until the process ends; its device address is looked up once per
 *     device (on the first call with that device current).
 *   - Every call on one device shares that device's scratch and leaves the last call's
 *     contents in it; calls that overlap on one device (two streams, or two host threads)
 *     RACE and must be serialised by the caller.  Calls on different devices are
 *     independent.
 *   - A shape whose scratch need (rva_verify_attention_workspace_size) exceeds 24 MiB
 *     returns RVA_ERR_WORKSPACE_TOO_SMALL and enqueues nothing: use rva_verify_attention
 *     then.  Shapes whose path needs no scratch (fp32 KV, non-power-of-two pages) always
 *     fit.
 */
rva_status rva_verify_attention_noalloc(int B, int max_window, int max_rows, int Hq, int Hkv,
                                        int D, int page_size, int num_pages, int max_pages,
                                        int kv_dtype, const void* q, const void* k_new,
                                        const void* v_new, void* k_cache, void* v_cache,
                                        const int32_t* block_table, const int32_t* context_lens,
                                        const int32_t* cu_seqlens, const int32_t* total_tier,
                                        float softmax_scale, void* out, int32_t* device_status,
                                        hipStream_t stream);

/*
 * Stages 4 (+5) -- rva_accept_and_commit
 *
 * [NOTES] section 02: acceptance compares target and draft distributions so that the
 * target's output distribution is kept, and only a contiguous prefix survives;
 * [SGL] "Background": each verify forward also yields one target (bonus) token.  The
 * standard speculative-sampling rule at temperature 1 is used.  With w = cu[b+1]-cu[b]:
 *   draft k (1 <= k < w): x = draft_tokens[b, k-1];
 *     r = p_t(x) / p_d(x),  p_t = softmax(target_logits[cu[b] + k - 1]),
 *                           p_d = softmax(draft_logits[b, k-1]);
 *     accept iff u_accept[b, k-1] < min(1, r); stop at the first rejection.
 *   n = number of accepted drafts; y is drawn with u_resample[b] by inverse CDF in
 *   ascending token order from  max(0, p_t - p_d) of the rejecting pair (renormalised;
 *   p_t if that is identically 0), or from p_t of row cu[b] + w - 1 when n = w - 1.
 *   Commit: committed[b, 0..n-1] = x_1..x_n, committed[b, n] = y, the rest -1;
 *   accept_len[b] = n; context_lens[b] += n + 1 (the anchor and accepted drafts keep their
 *   appended KV; y is the next anchor).
 *   [NOTES] section 07: labels[b, k-1] = 1 - 0.5 * ||p_d - p_t||_1 for the same row pair,
 *   k < w (NaN for k >= w).  p_t_at_draft / p_d_at_draft: p_t(x), p_d(x) for k < w (NaN
 *   otherwise).
 *   Precision: the accept test evaluates p_t(x) and p_d(x) in float64 at the drafted token,
 *   over normalisers summed from float32 exponentials in float64 (relative error ~1e-7);
 *   the draw of y -- an index that must agree with a float64 definition -- uses float64
 *   exponentials, float64 normalisers and float64 running sums throughout; the labels sum
 *   float32 terms in float64 (absolute error well below 1e-5).
 *
 * Arguments
 *   B, gamma, V     V >= 1; 2 <= gamma <= 64; B * gamma <= 65535 and
 *                   max_rows + B * (gamma-1) <= 65535.
 *   logit_dtype     RVA_BF16 or RVA_F32.  Logit buffers must be 16-byte aligned.
 *   target_logits   [max_rows, V] packed rows; draft_logits [B, gamma-1, V].
 *   draft_tokens    [B, gamma-1] int32; u_accept [B, gamma-1] and u_resample [B] float32
 *                   uniforms in [0, 1).
 *   cu_seqlens      [B+1] int32 (windows are its differences).
 *   accept_len [B], committed [B, gamma] int32 outputs; context_lens [B] int32 in/out.
 *   p_t_at_draft, p_d_at_draft, labels   optional [B, gamma-1] float32 outputs (NULL to
 *                   skip; labels == NULL skips the TV pass entirely).
 *   workspace       at least rva_accept_workspace_size(B, gamma, V, max_rows) bytes.
 *   device_status   optional (BAD_WINDOW, BAD_TOKEN).
 */
rva_status rva_accept_and_commit(int B, int gamma, int V, int logit_dtype, int max_rows,
                                 const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_tokens, const float* u_accept,
                                 const float* u_resample, const int32_t* cu_seqlens,
                                 int32_t* accept_len, int32_t* committed,
                                 int32_t* context_lens, float* p_t_at_draft,
                                 float* p_d_at_draft, float* labels, int32_t* device_status,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t rva_accept_workspace_size(int B, int gamma, int V, int max_rows);

/*
 * Stage 4 in cap-accept mode -- rva_accept_capped
 *
 * [SGL] "Confidence scheduler 与 verify 模式" and [CSDN] section 5: the verify ran on the
 * whole drafted block (as in static mode), but only positions inside the scheduler's window
 * may be committed.  The commit is therefore the one compact mode makes for that window,
 * and the acceptance the whole block would have reached -- the ceiling the trimming gave
 * up -- is reported beside it (a measurement arm, not the production path).
 *
 * With w = cu[b+1]-cu[b] verified rows (normally gamma) and cap = cap_windows[b] in [1, w]:
 *   n_full = drafts accepted over the whole block (the rule of rva_accept_and_commit over
 *            all w-1 drafts)  -> accept_len_full[b];
 *   n = min(n_full, cap - 1) -> accept_len[b];
 *   y = the residual draw of the rejecting pair when n_full < cap - 1, else the bonus draw
 *       from p_t of row cu[b] + cap - 1;
 *   committed[b] = x_1..x_n, y, then -1;  context_lens[b] += n + 1.
 * p_t_at_draft / p_d_at_draft / labels cover every draft of the verified block (k < w).
 * The utilisation of the acceptance ceiling is sum(accept_len) / sum(accept_len_full).
 *
 * Arguments: as rva_accept_and_commit, plus
 *   cap_windows     [B] int32 (device) windows of the commit cap, anchor included;
 *                   outside [1, w] sets RVA_DEV_BAD_WINDOW and is clamped.
 *   accept_len_full [B] int32 output.
 * The workspace is the one of rva_accept_and_commit (rva_accept_workspace_size).
 */
rva_status rva_accept_capped(int B, int gamma, int V, int logit_dtype, int max_rows,
                             const void* target_logits, const void* draft_logits,
                             const int32_t* draft_tokens, const float* u_accept,
                             const float* u_resample, const int32_t* cu_seqlens,
                             const int32_t* cap_windows, int32_t* accept_len,
                             int32_t* accept_len_full, int32_t* committed,
                             int32_t* context_lens, float* p_t_at_draft, float* p_d_at_draft,
                             float* labels, int32_t* device_status, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Stage 5 on its own -- rva_confidence_labels
 *
 * [NOTES] section 07: training label of the confidence head,
 *   labels[b, k-1] = 1 - 0.5 * || softmax(draft_logits[b,k-1]) - softmax(target_logits[cu[b]+k-1]) ||_1
 * for 1 <= k < w_b; NaN otherwise.  Same argument meanings and workspace as
 * rva_accept_and_commit (workspace >= rva_accept_workspace_size(B, gamma, V, max_rows)).
 */
rva_status rva_confidence_labels(int B, int gamma, int V, int logit_dtype, int max_rows,
                                 const void* target_logits, const void* draft_logits,
                                 const int32_t* cu_seqlens, float* labels,
                                 int32_t* device_status, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Calibration -- rva_sts_fit (Sequential Temperature Scaling)
 *
 * [NOTES] section 07 ("为什么还要做 Sequential Temperature Scaling？"): the head's scores
 * are over-confident, so a temperature per draft position is fitted that makes the
 * predicted prefix survival match the measured one; [SGL] "DSpark：sequential head 加验证
 * 预算": STS calibrates the block's survival to the real acceptance rate.  The fitted
 * temperatures are the `sts_T` argument of rva_schedule_windows.
 *
 * A trace holds N samples (one request at one step).  Sample i: head logits z[i, k] for
 * the G1 = gamma-1 draft positions (the logit before the sigmoid), the accepted drafts
 * accept_len[i] of a full-block verification, and the positions actually verified,
 * observed_len[i] (NULL: all G1; a compact run observes only w_i - 1).  Position k
 * (0-based) is observed iff k < observed_len[i]; its outcome is [accept_len[i] > k].
 * Predicted survival: a[i, k] = exp(sum_{j <= k} log sigmoid(z[i, j] / T_j)), float64.
 * Fit, in position order with the earlier temperatures fixed: T_k in [T_lo, T_hi]
 * minimises the Bernoulli negative log-likelihood of position k's observed outcomes
 * (global minimum located by iterated 64-point grid refinement in ln T, six rounds; final
 * spacing ~1e-8 relative).  A position with no observed sample gets T_k = 1.
 *
 *   N               samples, 1 .. 2^26; G1 = gamma - 1 in [1, 63].
 *   z               [N, G1] float32; accept_len [N] int32; observed_len [N] int32 or NULL.
 *   T_lo, T_hi      bracket, 0 < T_lo < T_hi (float32; the search runs in float64).
 *   T_out           [G1] float32 output; nll_out [G1] float64 output or NULL (the
 *                   minimised negative log-likelihood of each position).
 *   workspace       rva_sts_fit_workspace_size(N) bytes, 256-byte aligned; its contents on
 *                   entry do not matter.
 * Launches 1 + 6 * G1 kernels (one per refinement round; the last workgroup of a round
 * makes its selection); nothing is read back to the host.
 */
rva_status rva_sts_fit(int N, int G1, const float* z, const int32_t* accept_len,
                       const int32_t* observed_len, float T_lo, float T_hi, float* T_out,
                       double* nll_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);
size_t rva_sts_fit_workspace_size(int N);

/*
 * Calibration -- rva_calibration_ece (expected calibration error)
 *
 * [CSDN] section 5: per-request confidence and calibration metrics such as ECE for
 * analysis after the fact.  The predicted survival a[i, k] (as in rva_sts_fit, with
 * temperatures T, or T_k = 1 when T is NULL) of every observed (i, k) is put in one of
 * n_bins equal bins of [0, 1]: bin = min(floor(a * n_bins), n_bins - 1).  Per bin: count,
 * mean a, mean outcome; ECE = sum over bins of count/total * |mean a - mean outcome|.
 *
 *   N, G1, z, accept_len, observed_len   as rva_sts_fit.
 *   T               [G1] float32 or NULL.
 *   n_bins          1 .. 64, with G1 * n_bins <= 3840.
 *   ece_out         [G1 + 1] float64 output: [0] pooled over every observed position,
 *                   [1 + k] position k alone (0 when it has no observed sample).
 *   bin_counts      [G1, n_bins] int32 output or NULL.
 *   workspace       rva_calibration_ece_workspace_size(N, G1, n_bins) bytes, 256-aligned.
 */
rva_status rva_calibration_ece(int N, int G1, const float* z, const int32_t* accept_len,
                               const int32_t* observed_len, const float* T, int n_bins,
                               double* ece_out, int32_t* bin_counts, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
size_t rva_calibration_ece_workspace_size(int N, int G1, int n_bins);

/*
 * Drafter side -- rva_markov_sample (Markov sequential head)
 *
 * [NOTES] "05 · Core Innovation A", 5.1-5.3: the parallel backbone gives base logits U_k
 * for every draft position in one pass; the sequential head adds a bias that depends on
 * the previous token, B(x_{k-1}, v), a rank-r product W1 W2 (r = 256 by default), and the
 * positions are sampled in order ("09 · End-to-End Cycle").  Output: the draft tokens and
 * the final draft logits that rva_accept_and_commit consumes as the draft distribution.
 *
 * For each request b and k = 1 .. G1 (x_0 = anchor[b]):
 *   l_k(v) = U[b, k-1, v] + (w1_scale[x] * w2_scale[v]) * sum_j w1[x, j] * w2[v, j],
 *            x = x_{k-1}; the int8 dot is exact, the rest is float64 with one rounded
 *            multiply and one rounded add; stored in logit_dtype (bf16: via float32, RNE);
 *   x_k = the smallest v whose cumulative exp(l_k - max) in ascending token order exceeds
 *         u[b, k-1] * (total), computed from the STORED logits in float64.
 *
 *   B in [1, 4096]; G1 = gamma - 1 in [1, 63]; V >= 1; r in {64, 128, 256}.
 *   logit_dtype     RVA_BF16 or RVA_F32 for base_logits and draft_logits.
 *   base_logits     [B, G1, V]; draft_logits [B, G1, V] output (must not alias).
 *   anchor          [B] int32; u [B, G1] float32 in [0, 1).
 *   w1, w2          [V, r] int8 (16-byte aligned): embedding rows of the previous token and
 *                   projection rows of the next; w1_scale, w2_scale [V] float32.
 *   draft_tokens    [B, G1] int32 output; p_at [B, G1] float32 output (probability of
 *                   each drawn token) or NULL.
 *   workspace       rva_markov_workspace_size(B, V) bytes, 256-byte aligned.
 *   device_status   optional: RVA_DEV_BAD_TOKEN for an anchor outside [0, V) (token 0 is
 *                   used in its place).
 * Launches 2 * G1 kernels (a tile-parallel logits pass with int8 MFMA and a per-request
 * draw, per position).
 */
rva_status rva_markov_sample(int B, int G1, int V, int r, int logit_dtype,
                             const void* base_logits, const int32_t* anchor, const float* u,
                             const int8_t* w1, const float* w1_scale, const int8_t* w2,
                             const float* w2_scale, void* draft_logits, int32_t* draft_tokens,
                             float* p_at, int32_t* device_status, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);
size_t rva_markov_workspace_size(int B, int V);

/* Message for the last error returned on the calling thread ("" if none). */
const char* rva_last_error(void);
/* RVA_VERSION of the built library. */
int rva_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RVA_H */
