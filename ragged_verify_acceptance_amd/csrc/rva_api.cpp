// extern "C" entry points of librva: host-side argument validation, workspace sizing, the
// thread-local error text, and dispatch to the HIP launchers.  Nothing here touches device
// memory or synchronises; a call that fails validation enqueues nothing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "rva_common.h"

namespace {

thread_local std::string g_last_error;

rva_status fail(rva_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

rva_status ok() {
  g_last_error.clear();
  return RVA_OK;
}

rva_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RVA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, ...) \
  do {                     \
    if (!(cond)) return fail(RVA_ERR_INVALID_ARGUMENT, __VA_ARGS__); \
  } while (0)

}  // namespace

extern "C" {

const char* rva_last_error(void) { return g_last_error.c_str(); }

int rva_version(void) { return RVA_VERSION; }

}  // extern "C"

namespace {

rva_status check_schedule(int B, int gamma, int mode, const void* hidden, int hidden_dtype, int H,
                          const float* head_w, const float* conf_in, const float* sts_T,
                          const float* alpha_ms, int alpha_len, const float* theta_ms, int theta_len,
                          float* conf_out, float* surv_out, int32_t* windows, int32_t* K_out,
                          double* ratio_out) {
  REQUIRE(B >= 1, "B must be >= 1 (got %d)", B);
  REQUIRE(gamma >= 2 && gamma <= 64, "gamma must be in [2, 64] (got %d)", gamma);
  REQUIRE((long long)B * (gamma - 1) <= 4096, "B*(gamma-1) must be <= 4096 (got %lld)",
          (long long)B * (gamma - 1));
  REQUIRE(mode == RVA_MODE_COMPACT || mode == RVA_MODE_STATIC, "unknown mode %d", mode);
  REQUIRE((hidden == nullptr) != (conf_in == nullptr),
          "exactly one of hidden and conf_in must be given");
  if (hidden) {
    REQUIRE(hidden_dtype == RVA_BF16 || hidden_dtype == RVA_F32, "unknown hidden_dtype %d", hidden_dtype);
    REQUIRE(H >= 1, "H must be >= 1 (got %d)", H);
    REQUIRE(head_w != nullptr, "head_w is NULL");
  } else {
    REQUIRE(sts_T == nullptr, "sts_T applies to the head's logits; it must be NULL with conf_in");
  }
  REQUIRE(alpha_ms && theta_ms, "alpha_ms and theta_ms are required");
  REQUIRE(alpha_len > B, "alpha_len must be > B (got %d, B = %d)", alpha_len, B);
  REQUIRE((long long)theta_len > (long long)B * gamma, "theta_len must be > B*gamma (got %d)", theta_len);
  REQUIRE(conf_out && surv_out && windows && K_out && ratio_out, "an output pointer is NULL");
  return RVA_OK;
}

rva_status check_pack(int B, int gamma, const int32_t* windows, const int32_t* context_lens,
                      const int32_t* tiers_host, int n_tiers, const void* src, size_t row_bytes,
                      void* dst, int max_rows, int32_t* cu_seqlens, int32_t* row_req, int32_t* row_pos,
                      int32_t* total_tier, rva::TierTable* tt) {
  REQUIRE(B >= 1 && B <= 4096, "B must be in [1, 4096] (got %d)", B);
  REQUIRE(gamma >= 1 && gamma <= 4096, "gamma must be in [1, 4096] (got %d)", gamma);
  REQUIRE(windows && context_lens, "windows and context_lens are required");
  REQUIRE(tiers_host != nullptr, "tiers_host is NULL");
  REQUIRE(n_tiers >= 1 && n_tiers <= 512, "n_tiers must be in [1, 512] (got %d)", n_tiers);
  tt->n = n_tiers;
  for (int i = 0; i < n_tiers; ++i) {
    REQUIRE(tiers_host[i] >= 1, "tiers must be positive");
    REQUIRE(i == 0 || tiers_host[i] > tiers_host[i - 1], "tiers must be strictly ascending");
    tt->t[i] = tiers_host[i];
  }
  REQUIRE((long long)tiers_host[n_tiers - 1] >= (long long)B * gamma,
          "largest tier %d is below B*gamma = %lld", tiers_host[n_tiers - 1], (long long)B * gamma);
  REQUIRE(max_rows >= tiers_host[n_tiers - 1], "max_rows %d is below the largest tier %d", max_rows,
          tiers_host[n_tiers - 1]);
  REQUIRE((src == nullptr) == (dst == nullptr), "src and dst must both be given or both NULL");
  REQUIRE(src == nullptr || row_bytes >= 1, "row_bytes must be >= 1");
  REQUIRE(cu_seqlens && row_req && row_pos && total_tier, "an output pointer is NULL");
  return RVA_OK;
}

}  // namespace

extern "C" {

rva_status rva_schedule_windows(int B, int gamma, int mode, const void* hidden, int hidden_dtype,
                                int H, const float* head_w, float head_b, const float* conf_in,
                                const float* sts_T, float bias_ms, const float* alpha_ms,
                                int alpha_len, const float* theta_ms, int theta_len,
                                float* conf_out, float* surv_out, int32_t* windows,
                                int32_t* K_out, double* ratio_out, int32_t* device_status,
                                hipStream_t stream) {
  rva_status st = check_schedule(B, gamma, mode, hidden, hidden_dtype, H, head_w, conf_in, sts_T, alpha_ms,
                                 alpha_len, theta_ms, theta_len, conf_out, surv_out, windows, K_out, ratio_out);
  if (st != RVA_OK) return st;
  return hip_result(rva::launch_schedule(B, gamma, mode, hidden, hidden_dtype, H, head_w, head_b,
                                         conf_in, sts_T, bias_ms, alpha_ms, theta_ms, conf_out,
                                         surv_out, windows, K_out, ratio_out, device_status, stream),
                    "rva_schedule_windows launch");
}

rva_status rva_pack_ragged(int B, int gamma, const int32_t* windows, const int32_t* context_lens,
                           const int32_t* tiers_host, int n_tiers, const void* src,
                           size_t row_bytes, void* dst, int max_rows, int32_t* cu_seqlens,
                           int32_t* row_req, int32_t* row_pos, int32_t* total_tier,
                           int32_t* device_status, hipStream_t stream) {
  rva::TierTable tt;
  rva_status st = check_pack(B, gamma, windows, context_lens, tiers_host, n_tiers, src, row_bytes, dst, max_rows,
                             cu_seqlens, row_req, row_pos, total_tier, &tt);
  if (st != RVA_OK) return st;
  return hip_result(rva::launch_pack(B, gamma, windows, context_lens, tt, src, row_bytes, dst,
                                     max_rows, cu_seqlens, row_req, row_pos, total_tier,
                                     device_status, stream),
                    "rva_pack_ragged launch");
}

rva_status rva_schedule_and_pack(int B, int gamma, int mode, const void* hidden, int hidden_dtype, int H,
                                 const float* head_w, float head_b, const float* conf_in, const float* sts_T,
                                 float bias_ms, const float* alpha_ms, int alpha_len, const float* theta_ms,
                                 int theta_len, float* conf_out, float* surv_out, int32_t* windows,
                                 int32_t* K_out, double* ratio_out, const int32_t* context_lens,
                                 const int32_t* tiers_host, int n_tiers, const void* src, size_t row_bytes,
                                 void* dst, int max_rows, int32_t* cu_seqlens, int32_t* row_req,
                                 int32_t* row_pos, int32_t* total_tier, int32_t* device_status,
                                 hipStream_t stream) {
  rva_status st = check_schedule(B, gamma, mode, hidden, hidden_dtype, H, head_w, conf_in, sts_T, alpha_ms,
                                 alpha_len, theta_ms, theta_len, conf_out, surv_out, windows, K_out, ratio_out);
  if (st != RVA_OK) return st;
  rva::TierTable tt;
  st = check_pack(B, gamma, windows, context_lens, tiers_host, n_tiers, src, row_bytes, dst, max_rows, cu_seqlens,
                  row_req, row_pos, total_tier, &tt);
  if (st != RVA_OK) return st;
  return hip_result(rva::launch_schedule_pack(B, gamma, mode, hidden, hidden_dtype, H, head_w, head_b, conf_in,
                                              sts_T, bias_ms, alpha_ms, theta_ms, conf_out, surv_out, windows,
                                              K_out, ratio_out, context_lens, tt, src, row_bytes, dst, max_rows,
                                              cu_seqlens, row_req, row_pos, total_tier, device_status, stream),
                    "rva_schedule_and_pack launch");
}

size_t rva_verify_attention_workspace_size(int B, int max_window, int Hq, int Hkv, int D,
                                           int page_size, int max_pages, int kv_dtype) {
  if (B < 1 || max_window < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || page_size < 1 || max_pages < 1)
    return 0;
  return rva::attention_workspace_bytes(B, max_window, Hq, Hkv, D, page_size, max_pages, kv_dtype);
}

namespace {

// Shared by both attention entry points.  lib_scratch: the workspace is the library's
// static scratch (looked up after the arguments are validated).
rva_status attention_call(const char* name, int B, int max_window, int max_rows, int Hq,
                          int Hkv, int D, int page_size, int num_pages, int max_pages,
                          int kv_dtype, const void* q, const void* k_new, const void* v_new,
                          void* k_cache, void* v_cache, const int32_t* block_table,
                          const int32_t* context_lens, const int32_t* cu_seqlens,
                          const int32_t* total_tier, float softmax_scale, void* out,
                          int32_t* device_status, void* workspace, size_t workspace_bytes,
                          bool lib_scratch, hipStream_t stream) {
  REQUIRE(B >= 1 && B <= 65535, "B must be in [1, 65535] (got %d)", B);
  REQUIRE(max_window >= 1, "max_window must be >= 1");
  REQUIRE(max_rows >= 1, "max_rows must be >= 1");
  REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  REQUIRE(Hkv <= 65535, "Hkv must be <= 65535");
  if (D != 64 && D != 128) return fail(RVA_ERR_UNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  REQUIRE(kv_dtype == RVA_BF16 || kv_dtype == RVA_F32, "unknown kv_dtype %d", kv_dtype);
  if ((long long)max_window * (Hq / Hkv) > 4096)
    return fail(RVA_ERR_UNSUPPORTED, "max_window * Hq/Hkv must be <= 4096 (got %lld)",
                (long long)max_window * (Hq / Hkv));
  REQUIRE(page_size >= 1 && num_pages >= 1 && max_pages >= 1, "page_size, num_pages, max_pages must be >= 1");
  REQUIRE((long long)page_size * max_pages <= (1LL << 30), "page_size * max_pages too large");
  REQUIRE(q && k_new && v_new && k_cache && v_cache && block_table && context_lens && cu_seqlens &&
              total_tier && out,
          "a required pointer is NULL");
  const size_t esz = kv_dtype == RVA_BF16 ? 2 : 4;
  REQUIRE(aligned(q, 16) && aligned(k_new, 16) && aligned(v_new, 16) && aligned(k_cache, 16) &&
              aligned(v_cache, 16) && aligned(out, 16),
          "q, k_new, v_new, caches and out must be 16-byte aligned");
  (void)esz;
  const size_t need = rva::attention_workspace_bytes(B, max_window, Hq, Hkv, D, page_size, max_pages, kv_dtype);
  if (lib_scratch) {
    rva_status s = hip_result(rva::attention_scratch(&workspace, &workspace_bytes), name);
    if (s != RVA_OK) return s;
    if (need > workspace_bytes)
      return fail(RVA_ERR_WORKSPACE_TOO_SMALL,
                  "%s: this shape needs %zu bytes of scratch; the library's static scratch holds "
                  "%zu (use rva_verify_attention with a workspace)",
                  name, need, workspace_bytes);
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(RVA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes (got %zu)", name, need,
                workspace_bytes);
  REQUIRE(workspace == nullptr || aligned(workspace, 16), "workspace must be 16-byte aligned");
  rva::AttnArgs a;
  a.B = B;
  a.max_window = max_window;
  a.max_rows = max_rows;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.page_size = page_size;
  a.log2_page = -1;
  for (int lp = 0; lp < 31; ++lp)
    if ((1 << lp) == page_size) a.log2_page = lp;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.cu = cu_seqlens;
  a.total_tier = total_tier;
  a.scale = softmax_scale;
  a.out = out;
  a.status = device_status;
  a.ws = workspace;
  return hip_result(rva::launch_attention(a, kv_dtype, stream), name);
}

}  // namespace

rva_status rva_verify_attention(int B, int max_window, int max_rows, int Hq, int Hkv, int D,
                                int page_size, int num_pages, int max_pages, int kv_dtype,
                                const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int32_t* block_table,
                                const int32_t* context_lens, const int32_t* cu_seqlens,
                                const int32_t* total_tier, float softmax_scale, void* out,
                                int32_t* device_status, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return attention_call("rva_verify_attention", B, max_window, max_rows, Hq, Hkv, D, page_size,
                        num_pages, max_pages, kv_dtype, q, k_new, v_new, k_cache, v_cache,
                        block_table, context_lens, cu_seqlens, total_tier, softmax_scale, out,
                        device_status, workspace, workspace_bytes, false, stream);
}

rva_status rva_verify_attention_noalloc(int B, int max_window, int max_rows, int Hq, int Hkv,
                                        int D, int page_size, int num_pages, int max_pages,
                                        int kv_dtype, const void* q, const void* k_new,
                                        const void* v_new, void* k_cache, void* v_cache,
                                        const int32_t* block_table, const int32_t* context_lens,
                                        const int32_t* cu_seqlens, const int32_t* total_tier,
                                        float softmax_scale, void* out, int32_t* device_status,
                                        hipStream_t stream) {
  return attention_call("rva_verify_attention_noalloc", B, max_window, max_rows, Hq, Hkv, D,
                        page_size, num_pages, max_pages, kv_dtype, q, k_new, v_new, k_cache,
                        v_cache, block_table, context_lens, cu_seqlens, total_tier, softmax_scale,
                        out, device_status, nullptr, 0, true, stream);
}

size_t rva_accept_workspace_size(int B, int gamma, int V, int max_rows) {
  if (B < 1 || gamma < 2 || V < 1 || max_rows < 1) return 0;
  return rva::accept_workspace_bytes(B, gamma, V, max_rows);
}

namespace {

rva_status accept_common(const char* name, int B, int gamma, int V, int logit_dtype, int max_rows,
                         const void* target_logits, const void* draft_logits,
                         const int32_t* cu_seqlens, void* workspace, size_t workspace_bytes) {
  REQUIRE(B >= 1, "B must be >= 1 (got %d)", B);
  REQUIRE(gamma >= 2 && gamma <= 64, "gamma must be in [2, 64] (got %d)", gamma);
  REQUIRE(V >= 1, "V must be >= 1 (got %d)", V);
  REQUIRE(max_rows >= 1, "max_rows must be >= 1");
  REQUIRE(logit_dtype == RVA_BF16 || logit_dtype == RVA_F32, "unknown logit_dtype %d", logit_dtype);
  REQUIRE((long long)max_rows + (long long)B * (gamma - 1) <= 65535,
          "max_rows + B*(gamma-1) must be <= 65535");
  REQUIRE((long long)B * gamma <= 65535, "B*gamma must be <= 65535");
  REQUIRE(target_logits && draft_logits && cu_seqlens, "logits and cu_seqlens are required");
  REQUIRE(aligned(target_logits, 16) && aligned(draft_logits, 16), "logits must be 16-byte aligned");
  const size_t need = rva::accept_workspace_bytes(B, gamma, V, max_rows);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(RVA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes (got %zu)", name, need,
                workspace_bytes);
  REQUIRE(aligned(workspace, 256), "workspace must be 256-byte aligned");
  return RVA_OK;
}

}  // namespace

rva_status rva_accept_and_commit(int B, int gamma, int V, int logit_dtype, int max_rows,
                                 const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_tokens, const float* u_accept,
                                 const float* u_resample, const int32_t* cu_seqlens,
                                 int32_t* accept_len, int32_t* committed, int32_t* context_lens,
                                 float* p_t_at_draft, float* p_d_at_draft, float* labels,
                                 int32_t* device_status, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  rva_status s = accept_common("rva_accept_and_commit", B, gamma, V, logit_dtype, max_rows,
                               target_logits, draft_logits, cu_seqlens, workspace, workspace_bytes);
  if (s != RVA_OK) return s;
  REQUIRE(draft_tokens && u_accept && u_resample, "draft_tokens, u_accept and u_resample are required");
  REQUIRE(accept_len && committed && context_lens, "accept_len, committed and context_lens are required");
  rva::AcceptArgs a{};
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.max_rows = max_rows;
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = draft_tokens;
  a.u_acc = u_accept;
  a.u_res = u_resample;
  a.cu = cu_seqlens;
  a.accept_len = accept_len;
  a.committed = committed;
  a.context_lens = context_lens;
  a.pt_at = p_t_at_draft;
  a.pd_at = p_d_at_draft;
  a.labels = labels;
  a.status = device_status;
  a.ws = workspace;
  return hip_result(rva::launch_accept(a, logit_dtype, true, stream), "rva_accept_and_commit launch");
}

rva_status rva_accept_capped(int B, int gamma, int V, int logit_dtype, int max_rows,
                             const void* target_logits, const void* draft_logits,
                             const int32_t* draft_tokens, const float* u_accept,
                             const float* u_resample, const int32_t* cu_seqlens,
                             const int32_t* cap_windows, int32_t* accept_len,
                             int32_t* accept_len_full, int32_t* committed, int32_t* context_lens,
                             float* p_t_at_draft, float* p_d_at_draft, float* labels,
                             int32_t* device_status, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  rva_status s = accept_common("rva_accept_capped", B, gamma, V, logit_dtype, max_rows,
                               target_logits, draft_logits, cu_seqlens, workspace, workspace_bytes);
  if (s != RVA_OK) return s;
  REQUIRE(draft_tokens && u_accept && u_resample, "draft_tokens, u_accept and u_resample are required");
  REQUIRE(cap_windows != nullptr, "cap_windows is required");
  REQUIRE(accept_len && accept_len_full && committed && context_lens,
          "accept_len, accept_len_full, committed and context_lens are required");
  rva::AcceptArgs a{};
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.max_rows = max_rows;
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = draft_tokens;
  a.u_acc = u_accept;
  a.u_res = u_resample;
  a.cu = cu_seqlens;
  a.accept_len = accept_len;
  a.committed = committed;
  a.context_lens = context_lens;
  a.pt_at = p_t_at_draft;
  a.pd_at = p_d_at_draft;
  a.labels = labels;
  a.status = device_status;
  a.ws = workspace;
  a.cap = cap_windows;
  a.accept_len_full = accept_len_full;
  return hip_result(rva::launch_accept(a, logit_dtype, true, stream), "rva_accept_capped launch");
}

rva_status rva_confidence_labels(int B, int gamma, int V, int logit_dtype, int max_rows,
                                 const void* target_logits, const void* draft_logits,
                                 const int32_t* cu_seqlens, float* labels, int32_t* device_status,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  rva_status s = accept_common("rva_confidence_labels", B, gamma, V, logit_dtype, max_rows,
                               target_logits, draft_logits, cu_seqlens, workspace, workspace_bytes);
  if (s != RVA_OK) return s;
  REQUIRE(labels != nullptr, "labels is NULL");
  rva::AcceptArgs a{};
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.max_rows = max_rows;
  a.target = target_logits;
  a.draft = draft_logits;
  a.cu = cu_seqlens;
  a.labels = labels;
  a.status = device_status;
  a.ws = workspace;
  return hip_result(rva::launch_accept(a, logit_dtype, false, stream), "rva_confidence_labels launch");
}

size_t rva_sts_fit_workspace_size(int N) {
  if (N < 1 || N > (1 << 26)) return 0;
  return rva::sts_workspace_bytes(N);
}

rva_status rva_sts_fit(int N, int G1, const float* z, const int32_t* accept_len,
                       const int32_t* observed_len, float T_lo, float T_hi, float* T_out,
                       double* nll_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  REQUIRE(N >= 1 && N <= (1 << 26), "N must be in [1, 2^26] (got %d)", N);
  REQUIRE(G1 >= 1 && G1 <= 63, "G1 must be in [1, 63] (got %d)", G1);
  REQUIRE(z && accept_len && T_out, "z, accept_len and T_out are required");
  REQUIRE(T_lo > 0.f && T_hi > T_lo && std::isfinite(T_hi), "need 0 < T_lo < T_hi (got %g, %g)",
          double(T_lo), double(T_hi));
  const size_t need = rva::sts_workspace_bytes(N);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(RVA_ERR_WORKSPACE_TOO_SMALL, "rva_sts_fit: workspace needs %zu bytes (got %zu)", need,
                workspace_bytes);
  REQUIRE(aligned(workspace, 256), "workspace must be 256-byte aligned");
  rva::StsArgs a{};
  a.N = N;
  a.G1 = G1;
  a.z = z;
  a.accept_len = accept_len;
  a.observed_len = observed_len;
  a.T_lo = T_lo;
  a.T_hi = T_hi;
  a.T_out = T_out;
  a.nll_out = nll_out;
  a.ws = workspace;
  return hip_result(rva::launch_sts_fit(a, stream), "rva_sts_fit launch");
}

size_t rva_calibration_ece_workspace_size(int N, int G1, int n_bins) {
  if (N < 1 || N > (1 << 26) || G1 < 1 || G1 > 63 || n_bins < 1 || n_bins > 64 || G1 * n_bins > 3840)
    return 0;
  return rva::ece_workspace_bytes(N, G1, n_bins);
}

rva_status rva_calibration_ece(int N, int G1, const float* z, const int32_t* accept_len,
                               const int32_t* observed_len, const float* T, int n_bins,
                               double* ece_out, int32_t* bin_counts, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  REQUIRE(N >= 1 && N <= (1 << 26), "N must be in [1, 2^26] (got %d)", N);
  REQUIRE(G1 >= 1 && G1 <= 63, "G1 must be in [1, 63] (got %d)", G1);
  REQUIRE(n_bins >= 1 && n_bins <= 64 && G1 * n_bins <= 3840,
          "n_bins must be in [1, 64] with G1*n_bins <= 3840 (got %d)", n_bins);
  REQUIRE(z && accept_len && ece_out, "z, accept_len and ece_out are required");
  const size_t need = rva::ece_workspace_bytes(N, G1, n_bins);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(RVA_ERR_WORKSPACE_TOO_SMALL, "rva_calibration_ece: workspace needs %zu bytes (got %zu)",
                need, workspace_bytes);
  REQUIRE(aligned(workspace, 256), "workspace must be 256-byte aligned");
  rva::EceArgs a{};
  a.N = N;
  a.G1 = G1;
  a.n_bins = n_bins;
  a.z = z;
  a.accept_len = accept_len;
  a.observed_len = observed_len;
  a.T = T;
  a.ece_out = ece_out;
  a.bin_counts = bin_counts;
  a.ws = workspace;
  return hip_result(rva::launch_ece(a, stream), "rva_calibration_ece launch");
}

size_t rva_markov_workspace_size(int B, int V) {
  if (B < 1 || B > 4096 || V < 1) return 0;
  return rva::markov_workspace_bytes(B, V);
}

rva_status rva_markov_sample(int B, int G1, int V, int r, int logit_dtype, const void* base_logits,
                             const int32_t* anchor, const float* u, const int8_t* w1,
                             const float* w1_scale, const int8_t* w2, const float* w2_scale,
                             void* draft_logits, int32_t* draft_tokens, float* p_at,
                             int32_t* device_status, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  REQUIRE(B >= 1 && B <= 4096, "B must be in [1, 4096] (got %d)", B);
  REQUIRE(G1 >= 1 && G1 <= 63, "G1 must be in [1, 63] (got %d)", G1);
  REQUIRE(V >= 1 && (long long)V * r <= (1LL << 40), "V must be >= 1 (got %d)", V);
  REQUIRE((long long)B * G1 * V <= (1LL << 40), "B*G1*V too large");
  REQUIRE(r == 64 || r == 128 || r == 256, "r must be 64, 128 or 256 (got %d)", r);
  REQUIRE(logit_dtype == RVA_BF16 || logit_dtype == RVA_F32, "unknown logit_dtype %d", logit_dtype);
  REQUIRE(base_logits && anchor && u && w1 && w1_scale && w2 && w2_scale && draft_logits && draft_tokens,
          "an input or output pointer is NULL");
  REQUIRE(aligned(w1, 16) && aligned(w2, 16), "w1 and w2 must be 16-byte aligned");
  REQUIRE(base_logits != draft_logits, "draft_logits must not alias base_logits");
  const size_t need = rva::markov_workspace_bytes(B, V);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(RVA_ERR_WORKSPACE_TOO_SMALL, "rva_markov_sample: workspace needs %zu bytes (got %zu)",
                need, workspace_bytes);
  REQUIRE(aligned(workspace, 256), "workspace must be 256-byte aligned");
  rva::MarkovArgs a{};
  a.B = B;
  a.G1 = G1;
  a.V = V;
  a.r = r;
  a.base = base_logits;
  a.anchor = anchor;
  a.u = u;
  a.w1 = w1;
  a.s1 = w1_scale;
  a.w2 = w2;
  a.s2 = w2_scale;
  a.out = draft_logits;
  a.tokens = draft_tokens;
  a.p_at = p_at;
  a.status = device_status;
  a.ws = workspace;
  a.vec_ok = V % 8 == 0 && aligned(base_logits, 16) && aligned(draft_logits, 16) && aligned(w2_scale, 16);
  return hip_result(rva::launch_markov(a, logit_dtype, stream), "rva_markov_sample launch");
}

}  // extern "C"
