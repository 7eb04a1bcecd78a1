// The library's C ABI (include/jt.h): host-side argument validation and
// dispatch to the kernels' launchers.  Nothing here touches device memory;
// a call that fails validation has enqueued nothing.
#include "jt_host.h"

#include <limits.h>

#include <cmath>

namespace {

constexpr int kMaxNodes = 1024;
constexpr int kMaxDepth = 64;
constexpr int kMaxWidth = 16;
constexpr size_t kMaxSelectLds = 160 * 1024;  // gfx950 LDS per workgroup

inline jt_status launched(hipError_t e) { return e == hipSuccess ? JT_OK : JT_ERR_LAUNCH; }

inline bool valid_dtype(jt_dtype dt) { return dt == JT_F32 || dt == JT_BF16; }

}  // namespace

extern "C" {

const char* jt_status_string(jt_status s) {
  switch (s) {
    case JT_OK: return "ok";
    case JT_ERR_INVALID_ARG: return "invalid argument";
    case JT_ERR_UNSUPPORTED: return "unsupported configuration";
    case JT_ERR_WORKSPACE: return "workspace missing or too small";
    case JT_ERR_LAUNCH: return "kernel launch failed";
    case JT_ERR_SCRATCH: return "inputs need more than the no-allocation entry point's scratch";
    default: break;
  }
  return "unknown status";
}

int jt_version(void) { return 200; }

size_t jt_build_tree_workspace(int batch, int depth_n, int vocab, int width_w, int budget_b) {
  (void)budget_b;
  if (batch <= 0 || depth_n < 1 || vocab < 1 || width_w < 1) return 0;
  return jt::build_tree_workspace_bytes(batch, depth_n, vocab, width_w);
}

jt_status jt_build_tree(const void* draft_logits, jt_dtype dt, int batch, int depth_n, int vocab,
                        int width_w, int budget_b, const int32_t* root_token, int32_t* parent,
                        int32_t* token, int32_t* depth, double* score, int32_t* n_nodes,
                        int32_t* err, void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || depth_n < 1 || vocab < 1 || width_w < 1 || budget_b < 0 || !valid_dtype(dt))
    return JT_ERR_INVALID_ARG;
  if (width_w > vocab) return JT_ERR_INVALID_ARG;
  if (depth_n > kMaxDepth || width_w > kMaxWidth || budget_b + 1 > kMaxNodes ||
      vocab > jt::build_tree_max_vocab())
    return JT_ERR_UNSUPPORTED;
  if (jt::build_tree_lds_bytes(depth_n, width_w, budget_b) > kMaxSelectLds)
    return JT_ERR_UNSUPPORTED;
  if (batch == 0) return JT_OK;
  if (!draft_logits || !root_token || !parent || !token || !depth || !n_nodes)
    return JT_ERR_INVALID_ARG;
  const size_t need = jt::build_tree_workspace_bytes(batch, depth_n, vocab, width_w);
  if (need > 0 && (!workspace || workspace_bytes < need)) return JT_ERR_WORKSPACE;
  return launched(jt::build_tree_launch(draft_logits, dt, batch, depth_n, vocab, width_w,
                                        budget_b, root_token, parent, token, depth, score,
                                        n_nodes, err, workspace,
                                        static_cast<hipStream_t>(stream)));
}

jt_status jt_build_tree_variant(const void* draft_logits, jt_dtype dt, int batch, int depth_n,
                                int vocab, int width_w, int budget_b, jt_expand expand_mode,
                                double entropy_weight, const int32_t* root_token,
                                int32_t* parent, int32_t* token, int32_t* depth, double* score,
                                int32_t* n_nodes, int32_t* err, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (batch < 0 || depth_n < 1 || vocab < 1 || width_w < 1 || budget_b < 0 || !valid_dtype(dt))
    return JT_ERR_INVALID_ARG;
  if (width_w > vocab) return JT_ERR_INVALID_ARG;
  if (expand_mode != JT_EXPAND_CANDIDATE && expand_mode != JT_EXPAND_NODE_BLOCK)
    return JT_ERR_INVALID_ARG;
  if (!(entropy_weight >= 0.0 && entropy_weight <= 1.0)) return JT_ERR_INVALID_ARG;
  if (depth_n > kMaxDepth || width_w > kMaxWidth || budget_b + 1 > kMaxNodes ||
      vocab > jt::build_tree_max_vocab())
    return JT_ERR_UNSUPPORTED;
  if (batch == 0) return JT_OK;
  if (!draft_logits || !root_token || !parent || !token || !depth || !n_nodes)
    return JT_ERR_INVALID_ARG;
  const size_t need = jt::build_tree_workspace_bytes(batch, depth_n, vocab, width_w);
  if (need > 0 && (!workspace || workspace_bytes < need)) return JT_ERR_WORKSPACE;
  return launched(jt::build_tree_variant_launch(
      draft_logits, dt, batch, depth_n, vocab, width_w, budget_b, static_cast<int>(expand_mode),
      entropy_weight, root_token, parent, token, depth, score, n_nodes, err, workspace,
      static_cast<hipStream_t>(stream)));
}

jt_status jt_tree_meta(const int32_t* parent, const int32_t* n_nodes, int batch, int max_nodes,
                       uint32_t* anc_mask, int32_t* err, void* stream) {
  if (batch < 0 || max_nodes < 1) return JT_ERR_INVALID_ARG;
  if (max_nodes > kMaxNodes) return JT_ERR_UNSUPPORTED;
  if (batch == 0) return JT_OK;
  if (!parent || !n_nodes || !anc_mask) return JT_ERR_INVALID_ARG;
  return launched(jt::tree_meta_launch(parent, n_nodes, batch, max_nodes, anc_mask, err,
                                       static_cast<hipStream_t>(stream)));
}

static jt_status check_attention_shape(int batch, int max_nodes, int hq, int hkv, int head_dim,
                                       int max_pages, int page_size, jt_dtype dt) {
  if (batch < 0 || max_nodes < 1 || hq < 1 || hkv < 1 || head_dim < 1 || max_pages < 1 ||
      page_size < 1 || !valid_dtype(dt))
    return JT_ERR_INVALID_ARG;
  if (hq % hkv != 0) return JT_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return JT_ERR_UNSUPPORTED;
  if (page_size != 16) return JT_ERR_UNSUPPORTED;
  if (hq / hkv > 16 || max_nodes > kMaxNodes) return JT_ERR_UNSUPPORTED;
  if (static_cast<long long>(max_pages) * page_size > INT_MAX / 2) return JT_ERR_UNSUPPORTED;
  return JT_OK;
}

size_t jt_tree_attention_workspace(int batch, int max_nodes, int num_q_heads, int num_kv_heads,
                                   int head_dim, int max_pages_per_seq, int page_size,
                                   jt_dtype dt) {
  if (check_attention_shape(batch, max_nodes, num_q_heads, num_kv_heads, head_dim,
                            max_pages_per_seq, page_size, dt) != JT_OK)
    return 0;
  jt::AttnShape s{batch, max_nodes, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq,
                  1, page_size, dt};
  return jt::tree_attention_workspace_bytes(s);
}

jt_status jt_tree_attention(const void* q, const void* k_pool, const void* v_pool, jt_dtype dt,
                            int batch, int max_nodes, int num_q_heads, int num_kv_heads,
                            int head_dim, const int32_t* n_nodes, const int32_t* prefix_len,
                            const int32_t* page_table, int max_pages_per_seq, int num_pages,
                            int page_size, const uint32_t* anc_mask, float scale, void* out,
                            float* lse, int32_t* err, void* workspace, size_t workspace_bytes,
                            void* stream) {
  const jt_status st = check_attention_shape(batch, max_nodes, num_q_heads, num_kv_heads,
                                             head_dim, max_pages_per_seq, page_size, dt);
  if (st != JT_OK) return st;
  if (num_pages < 1 || !(scale > 0.0f) || !std::isfinite(scale)) return JT_ERR_INVALID_ARG;
  if (static_cast<long long>(num_pages) * num_kv_heads * page_size * head_dim > (1LL << 40))
    return JT_ERR_UNSUPPORTED;
  if (batch == 0) return JT_OK;
  if (!q || !k_pool || !v_pool || !n_nodes || !prefix_len || !page_table || !anc_mask || !out)
    return JT_ERR_INVALID_ARG;
  jt::AttnShape s{batch, max_nodes, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq,
                  num_pages, page_size, dt};
  const size_t need = jt::tree_attention_workspace_bytes(s);
  if (need > 0 && (!workspace || workspace_bytes < need)) return JT_ERR_WORKSPACE;
  return launched(jt::tree_attention_launch(s, q, k_pool, v_pool, n_nodes, prefix_len,
                                            page_table, anc_mask, scale, out, lse, err, workspace,
                                            static_cast<hipStream_t>(stream)));
}

size_t jt_accept_workspace(int batch, int max_nodes, int vocab) {
  if (batch <= 0 || max_nodes < 1 || vocab < 1) return 0;
  return jt::accept_workspace_bytes(batch, max_nodes, vocab);
}

namespace {

jt_status accept_common(const void* target_logits, jt_dtype dt, int batch, int max_nodes,
                        int vocab, int depth_n, const int32_t* parent, const int32_t* token,
                        const int32_t* depth, const int32_t* n_nodes, int32_t* accept_len,
                        int32_t* accept_nodes, int32_t* bonus_token, int32_t* err,
                        void* workspace, size_t workspace_bytes, void* stream, int mode,
                        double margin) {
  if (batch < 0 || max_nodes < 1 || vocab < 1 || depth_n < 1 || !valid_dtype(dt))
    return JT_ERR_INVALID_ARG;
  if (mode == 1 && !(margin <= 0.0 && std::isfinite(margin))) return JT_ERR_INVALID_ARG;
  if (max_nodes > kMaxNodes || depth_n > kMaxDepth) return JT_ERR_UNSUPPORTED;
  if (batch == 0) return JT_OK;
  if (!target_logits || !parent || !token || !depth || !n_nodes || !accept_len ||
      !accept_nodes || !bonus_token)
    return JT_ERR_INVALID_ARG;
  const size_t need = jt::accept_workspace_bytes(batch, max_nodes, vocab);
  if (need > 0 && (!workspace || workspace_bytes < need)) return JT_ERR_WORKSPACE;
  return launched(jt::accept_launch(target_logits, dt, batch, max_nodes, vocab, depth_n, parent,
                                    token, depth, n_nodes, accept_len, accept_nodes, bonus_token,
                                    err, workspace, static_cast<hipStream_t>(stream), mode,
                                    margin));
}

}  // namespace

jt_status jt_accept(const void* target_logits, jt_dtype dt, int batch, int max_nodes, int vocab,
                    int depth_n, const int32_t* parent, const int32_t* token,
                    const int32_t* depth, const int32_t* n_nodes, int32_t* accept_len,
                    int32_t* accept_nodes, int32_t* bonus_token, int32_t* err, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return accept_common(target_logits, dt, batch, max_nodes, vocab, depth_n, parent, token,
                       depth, n_nodes, accept_len, accept_nodes, bonus_token, err, workspace,
                       workspace_bytes, stream, 0, 0.0);
}

jt_status jt_accept_noalloc(const void* target_logits, jt_dtype dt, int batch, int max_nodes,
                            int vocab, int depth_n, const int32_t* parent, const int32_t* token,
                            const int32_t* depth, const int32_t* n_nodes, int32_t* accept_len,
                            int32_t* accept_nodes, int32_t* bonus_token, int32_t* err,
                            void* stream) {
  if (batch < 0 || max_nodes < 1 || vocab < 1 || depth_n < 1 || !valid_dtype(dt))
    return JT_ERR_INVALID_ARG;
  if (max_nodes > kMaxNodes || depth_n > kMaxDepth) return JT_ERR_UNSUPPORTED;
  if (batch == 0) return JT_OK;
  if (!target_logits || !parent || !token || !depth || !n_nodes || !accept_len ||
      !accept_nodes || !bonus_token)
    return JT_ERR_INVALID_ARG;
  const size_t need = jt::accept_workspace_bytes(batch, max_nodes, vocab);
  if (need > jt::kAcceptScratchBytes) return JT_ERR_SCRATCH;
  void* scratch = nullptr;
  if (jt::accept_scratch_address(&scratch) != hipSuccess) return JT_ERR_LAUNCH;
  return launched(jt::accept_launch(target_logits, dt, batch, max_nodes, vocab, depth_n, parent,
                                    token, depth, n_nodes, accept_len, accept_nodes, bonus_token,
                                    err, scratch, static_cast<hipStream_t>(stream), 0, 0.0));
}

jt_status jt_accept_margin(const void* target_logits, jt_dtype dt, int batch, int max_nodes,
                           int vocab, int depth_n, const int32_t* parent, const int32_t* token,
                           const int32_t* depth, const int32_t* n_nodes, double theta,
                           double temperature, int32_t* accept_len, int32_t* accept_nodes,
                           int32_t* bonus_token, int32_t* err, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!(theta > 0.0 && theta <= 1.0)) return JT_ERR_INVALID_ARG;
  if (!(temperature > 0.0) || !std::isfinite(temperature)) return JT_ERR_INVALID_ARG;
  // p(x) / p(top1) >= theta with p = softmax(L / T)  <=>  L[x] - max L >= T ln(theta)
  const double logit_margin = temperature * std::log(theta);
  return accept_common(target_logits, dt, batch, max_nodes, vocab, depth_n, parent, token,
                       depth, n_nodes, accept_len, accept_nodes, bonus_token, err, workspace,
                       workspace_bytes, stream, 1, logit_margin);
}

jt_status jt_commit_kv(void* k_pool, void* v_pool, jt_dtype dt, int batch, int num_kv_heads,
                       int head_dim, const int32_t* page_table, int max_pages_per_seq,
                       int num_pages, int page_size, const int32_t* n_nodes,
                       const int32_t* parent, int max_nodes, int depth_n,
                       const int32_t* accept_len, const int32_t* accept_nodes,
                       int32_t* prefix_len, int32_t* err, void* stream) {
  if (batch < 0 || num_kv_heads < 1 || head_dim < 1 || max_pages_per_seq < 1 || num_pages < 1 ||
      max_nodes < 1 || depth_n < 1 || !valid_dtype(dt))
    return JT_ERR_INVALID_ARG;
  const int row_bytes = head_dim * (dt == JT_F32 ? 4 : 2);
  if (page_size != 16 || row_bytes % 16 != 0 || depth_n > kMaxDepth || max_nodes > kMaxNodes ||
      2LL * depth_n * row_bytes > 64 * 1024)
    return JT_ERR_UNSUPPORTED;
  if (batch == 0) return JT_OK;
  if (!k_pool || !v_pool || !page_table || !n_nodes || !accept_len || !accept_nodes ||
      !prefix_len)
    return JT_ERR_INVALID_ARG;
  return launched(jt::commit_kv_launch(k_pool, v_pool, dt == JT_F32 ? 4 : 2, batch, num_kv_heads,
                                       head_dim, page_table, max_pages_per_seq, num_pages,
                                       n_nodes, parent, max_nodes, depth_n, accept_len,
                                       accept_nodes, prefix_len, err,
                                       static_cast<hipStream_t>(stream)));
}

size_t jt_accept_stochastic_workspace(int batch, int vocab) {
  if (batch <= 0 || vocab < 1) return 0;
  return jt::accept_stochastic_workspace_bytes(batch, vocab);
}

jt_status jt_accept_stochastic(const void* target_logits, const void* draft_logits, jt_dtype dt,
                               int batch, int max_nodes, int vocab, int depth_n,
                               const int32_t* parent, const int32_t* token, const int32_t* depth,
                               const int32_t* n_nodes, float temperature,
                               jt_draft_mode draft_mode, const float* u_accept,
                               const float* u_sample, int32_t* accept_len, int32_t* accept_nodes,
                               int32_t* bonus_token, int32_t* err, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (batch < 0 || max_nodes < 1 || vocab < 1 || depth_n < 1 || !valid_dtype(dt))
    return JT_ERR_INVALID_ARG;
  if (!(temperature > 0.0f) || !std::isfinite(temperature)) return JT_ERR_INVALID_ARG;
  if (draft_mode != JT_DRAFT_TOPW && draft_mode != JT_DRAFT_SAMPLED) return JT_ERR_INVALID_ARG;
  if (max_nodes > kMaxNodes || depth_n > kMaxDepth) return JT_ERR_UNSUPPORTED;
  if (batch == 0) return JT_OK;
  const bool sampled = draft_mode == JT_DRAFT_SAMPLED;
  if (!target_logits || (sampled && !draft_logits) || !parent || !token || !depth || !n_nodes ||
      !u_accept || !u_sample || !accept_len || !accept_nodes || !bonus_token)
    return JT_ERR_INVALID_ARG;
  const size_t need = jt::accept_stochastic_workspace_bytes(batch, vocab);
  if (!workspace || workspace_bytes < need) return JT_ERR_WORKSPACE;
  return launched(jt::accept_stochastic_launch(
      target_logits, draft_logits, dt, batch, max_nodes, vocab, depth_n, parent, token, depth,
      n_nodes, temperature, u_accept, u_sample, sampled ? 1 : 0, accept_len, accept_nodes,
      bonus_token, err, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
