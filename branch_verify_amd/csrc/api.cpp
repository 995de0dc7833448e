// C ABI of libsfv: argument validation, workspace sizing and dispatch.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/sfv.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SFV_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SFV_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool pow2_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

int check_attn_dims(int B1, int N, int L, int Hq, int Hkv, int d) {
  if (B1 < 1 || B1 > SFV_MAX_BRANCHES) return fail(SFV_E_INVAL, "B1=%d not in [1, %d]", B1, SFV_MAX_BRANCHES);
  if (N < 1 || N > SFV_MAX_BLOCK) return fail(SFV_E_INVAL, "N=%d not in [1, %d]", N, SFV_MAX_BLOCK);
  if (L < 0) return fail(SFV_E_INVAL, "L=%d < 0", L);
  if (Hq < 1 || Hkv < 1) return fail(SFV_E_INVAL, "head counts must be positive (Hq=%d, Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(SFV_E_INVAL, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (!pow2_group(Hq / Hkv)) return fail(SFV_E_UNSUPPORTED, "group size Hq/Hkv=%d not in {1,2,4,8}", Hq / Hkv);
  if (d != 32 && d != 64 && d != 128) return fail(SFV_E_UNSUPPORTED, "head dim d=%d not in {32,64,128}", d);
  const double rows = (double)B1 * N * Hq;
  if (rows * d > 2e9 || (double)Hkv * L * d > 2e9) return fail(SFV_E_INVAL, "tensor too large");
  return SFV_OK;
}

// Validates the tree and fills the by-value description the kernels use.
int make_tree(const int32_t* parent_host, int B1, sfv::TreeArgs* tree) {
  if (!parent_host) return fail(SFV_E_INVAL, "parent_host is NULL");
  if (B1 < 1 || B1 > SFV_MAX_BRANCHES) return fail(SFV_E_INVAL, "B1=%d not in [1, %d]", B1, SFV_MAX_BRANCHES);
  if (parent_host[0] != -1) return fail(SFV_E_TREE, "parent[0]=%d, must be -1", parent_host[0]);
  std::memset(tree, 0, sizeof(*tree));
  tree->B1 = B1;
  tree->depth[0] = 0;
  tree->parent[0] = -1;
  int maxd = 0;
  for (int i = 1; i < B1; ++i) {
    const int p = parent_host[i];
    if (p < 0 || p >= i) return fail(SFV_E_TREE, "parent[%d]=%d not in [0, %d)", i, p, i);
    tree->parent[i] = (signed char)p;
    tree->depth[i] = (signed char)(tree->depth[p] + 1);
    if (tree->depth[i] > maxd) maxd = tree->depth[i];
  }
  tree->levels = maxd + 1;
  int pos = 0;
  for (int lv = 0; lv <= maxd; ++lv) {
    tree->level_start[lv] = (unsigned char)pos;
    for (int i = 0; i < B1; ++i)
      if (tree->depth[i] == lv) tree->by_level[pos++] = (unsigned char)i;
  }
  tree->level_start[maxd + 1] = (unsigned char)pos;
  return SFV_OK;
}

int commit_items_max(const sfv::TreeArgs& tree, int N, int M, bool noisy) {
  if (!noisy) return M;
  long bound = 0;
  for (int lv = 0; lv < tree.levels; ++lv) {
    const int width = tree.level_start[lv + 1] - tree.level_start[lv];
    bound += (long)N * ((width + sfv::kItemRowsHost - 1) / sfv::kItemRowsHost);
  }
  return bound < M ? (int)bound : M;
}

int check_commit_dims(int B1, int N, int M, int V) {
  if (B1 < 1 || B1 > SFV_MAX_BRANCHES) return fail(SFV_E_INVAL, "B1=%d not in [1, %d]", B1, SFV_MAX_BRANCHES);
  if (N < 1 || N > SFV_MAX_BLOCK) return fail(SFV_E_INVAL, "N=%d not in [1, %d]", N, SFV_MAX_BLOCK);
  if (M < 0 || M > B1 * N) return fail(SFV_E_INVAL, "M=%d not in [0, B1*N=%d]", M, B1 * N);
  if (V < 1) return fail(SFV_E_INVAL, "V=%d < 1", V);
  if (V % 8 != 0) return fail(SFV_E_UNSUPPORTED, "V=%d is not a multiple of 8", V);
  if (V >= (1 << 28)) return fail(SFV_E_UNSUPPORTED, "V=%d too large", V);
  return SFV_OK;
}

}  // namespace

extern "C" {

const char* sfv_last_error(void) { return g_err; }

int sfv_version(void) { return 100; }

int sfv_attend_workspace_bytes(int B1, int N, int L, int Hq, int Hkv, int d, size_t* bytes) {
  if (!bytes) return fail(SFV_E_INVAL, "bytes is NULL");
  const int rc = check_attn_dims(B1, N, L, Hq, Hkv, d);
  if (rc != SFV_OK) return rc;
  *bytes = sfv::attn_plan(B1, N, L, Hq, Hkv, d).ws_bytes;
  return ok();
}

int sfv_attend_branches(const void* q, const void* k_blk, const void* v_blk, const void* k_ctx,
                        const void* v_ctx, int B1, int N, int L, int Hq, int Hkv, int d,
                        float softmax_scale, void* o, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int rc = check_attn_dims(B1, N, L, Hq, Hkv, d);
  if (rc != SFV_OK) return rc;
  if (!q || !k_blk || !v_blk || !o || !lse) return fail(SFV_E_INVAL, "null tensor pointer");
  if (L > 0 && (!k_ctx || !v_ctx)) return fail(SFV_E_INVAL, "null context pointer with L=%d", L);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f))
    return fail(SFV_E_INVAL, "softmax_scale=%g must be finite and > 0", (double)softmax_scale);
  const sfv::AttnPlan plan = sfv::attn_plan(B1, N, L, Hq, Hkv, d);
  if (workspace_bytes < plan.ws_bytes) {
    return fail(SFV_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, plan.ws_bytes);
  }
  if (plan.ws_bytes > 0 && !workspace) return fail(SFV_E_INVAL, "workspace is NULL");
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k_blk | (uintptr_t)v_blk | (uintptr_t)k_ctx |
                       (uintptr_t)v_ctx | (uintptr_t)o | (uintptr_t)workspace;
  if (al % 16 != 0) return fail(SFV_E_INVAL, "tensor pointers must be 16-byte aligned");
  return hip_status(sfv::launch_attention(q, k_blk, v_blk, k_ctx, v_ctx, B1, N, L, Hq, Hkv, d,
                                          softmax_scale, o, lse, workspace, plan,
                                          (hipStream_t)stream),
                    "sfv_attend_branches");
}

int check_topk_dims(int M, int V, int N, int K) {
  if (N < 1 || N > SFV_MAX_BLOCK) return fail(SFV_E_INVAL, "N=%d not in [1, %d]", N, SFV_MAX_BLOCK);
  if (M < 0 || M > SFV_MAX_BRANCHES * N) return fail(SFV_E_INVAL, "M=%d out of range", M);
  if (V < 1 || V >= (1 << 30)) return fail(SFV_E_INVAL, "V=%d out of range", V);
  if (K < 1 || K > SFV_MAX_TOPK || K > V) return fail(SFV_E_INVAL, "K=%d not in [1, min(%d, V)]", K, SFV_MAX_TOPK);
  if ((double)M * V >= 9.0e15) return fail(SFV_E_INVAL, "too large");
  return SFV_OK;
}

int sfv_stale_topk_workspace_bytes(int M, int V, int N, int K, size_t* bytes) {
  if (!bytes) return fail(SFV_E_INVAL, "bytes is NULL");
  const int rc = check_topk_dims(M, V, N, K);
  if (rc != SFV_OK) return rc;
  *bytes = sfv::topk_plan(M, V, K).ws_bytes;
  return ok();
}

int sfv_stale_topk(const float* logits, const int32_t* rows, const float* conf, int M, int V, int N,
                   int branch, int K, int32_t* top_ids, float* top_logit, float* conf_pos, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const int rc = check_topk_dims(M, V, N, K);
  if (rc != SFV_OK) return rc;
  if (branch < 0 || branch >= SFV_MAX_BRANCHES) return fail(SFV_E_INVAL, "branch=%d out of range", branch);
  if (M > 0 && (!logits || !rows || !conf || !top_ids || !top_logit || !conf_pos || !workspace))
    return fail(SFV_E_INVAL, "null pointer");
  const sfv::TopkPlan plan = sfv::topk_plan(M, V, K);
  if (workspace_bytes < plan.ws_bytes)
    return fail(SFV_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, plan.ws_bytes);
  if ((uintptr_t)workspace % 16 != 0) return fail(SFV_E_INVAL, "workspace must be 16-byte aligned");
  return hip_status(sfv::launch_stale_topk(logits, rows, conf, M, V, N, branch, K, top_ids, top_logit, conf_pos,
                                           workspace, plan, (hipStream_t)stream),
                    "sfv_stale_topk");
}

int sfv_draft_tree(const int32_t* root, const int32_t* top_ids, const float* top_logit, const float* conf,
                   int N, int K, int D, int W, float temperature, uint64_t seed, uint64_t step0, int64_t pos0,
                   int32_t* parent, int32_t* states, int32_t* n_drafts, void* stream) {
  if (N < 1 || N > SFV_MAX_BLOCK) return fail(SFV_E_INVAL, "N=%d not in [1, %d]", N, SFV_MAX_BLOCK);
  if (K < 1 || K > SFV_MAX_TOPK) return fail(SFV_E_INVAL, "K=%d not in [1, %d]", K, SFV_MAX_TOPK);
  if (D < 0 || D > SFV_MAX_BRANCHES - 1) return fail(SFV_E_INVAL, "D=%d not in [0, %d]", D, SFV_MAX_BRANCHES - 1);
  if (W < 0 || W > SFV_MAX_DRAFT_WIDTH) return fail(SFV_E_INVAL, "W=%d not in [0, %d]", W, SFV_MAX_DRAFT_WIDTH);
  if (!(temperature >= 0.f) || !std::isfinite(temperature)) return fail(SFV_E_INVAL, "temperature must be >= 0");
  if (!root || !top_ids || !top_logit || !conf || !parent || !states || !n_drafts)
    return fail(SFV_E_INVAL, "null pointer");
  return hip_status(sfv::launch_draft_tree(root, top_ids, top_logit, conf, N, K, D, W, temperature, seed, step0,
                                           pos0, parent, states, n_drafts, (hipStream_t)stream),
                    "sfv_draft_tree");
}

int sfv_fold_gate(const void* hidden, const int32_t* parent_host, int B1, int N, int D, float delta,
                  int32_t* recompute, int32_t* src, int32_t* rec_rows, int32_t* rec_count,
                  int32_t* rec_pos, int32_t* branch_off, void* stream) {
  sfv::TreeArgs tree;
  const int rc = make_tree(parent_host, B1, &tree);
  if (rc != SFV_OK) return rc;
  if (N < 1 || N > SFV_MAX_BLOCK) return fail(SFV_E_INVAL, "N=%d not in [1, %d]", N, SFV_MAX_BLOCK);
  if (D < 8 || D % 8 != 0) return fail(SFV_E_UNSUPPORTED, "D=%d is not a positive multiple of 8", D);
  if ((double)B1 * N * D > 2e9) return fail(SFV_E_INVAL, "hidden too large");
  if (std::isnan(delta)) return fail(SFV_E_INVAL, "delta is NaN");
  if (!hidden || !recompute || !src || !rec_rows || !rec_count || !rec_pos || !branch_off)
    return fail(SFV_E_INVAL, "null pointer");
  if ((uintptr_t)hidden % 16 != 0) return fail(SFV_E_INVAL, "hidden must be 16-byte aligned");
  return hip_status(sfv::launch_fold_gate(hidden, tree, N, D, delta, recompute, src, rec_rows, rec_count,
                                          rec_pos, branch_off, (hipStream_t)stream),
                    "sfv_fold_gate");
}

int sfv_attend_folded_workspace_bytes(int B1, int N, int L, int Hq, int Hkv, int d, size_t* bytes) {
  if (!bytes) return fail(SFV_E_INVAL, "bytes is NULL");
  const int rc = check_attn_dims(B1, N, L, Hq, Hkv, d);
  if (rc != SFV_OK) return rc;
  *bytes = sfv::attn_plan(B1, N, L, Hq, Hkv, d).ws_bytes_folded;
  return ok();
}

int sfv_attend_folded(const void* q, const void* k_blk, const void* v_blk, const void* k_ctx,
                      const void* v_ctx, int B1, int N, int L, int Hq, int Hkv, int d, float softmax_scale,
                      const int32_t* src, const int32_t* rec_rows, const int32_t* rec_count,
                      const int32_t* rec_pos, void* o, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream) {
  const int rc = check_attn_dims(B1, N, L, Hq, Hkv, d);
  if (rc != SFV_OK) return rc;
  if (!q || !k_blk || !v_blk || !o || !lse || !src || !rec_rows || !rec_count || !rec_pos)
    return fail(SFV_E_INVAL, "null pointer");
  if (L > 0 && (!k_ctx || !v_ctx)) return fail(SFV_E_INVAL, "null context pointer with L=%d", L);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f))
    return fail(SFV_E_INVAL, "softmax_scale=%g must be finite and > 0", (double)softmax_scale);
  const sfv::AttnPlan plan = sfv::attn_plan(B1, N, L, Hq, Hkv, d);
  if (workspace_bytes < plan.ws_bytes_folded) {
    return fail(SFV_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, plan.ws_bytes_folded);
  }
  if (plan.ws_bytes_folded > 0 && !workspace) return fail(SFV_E_INVAL, "workspace is NULL");
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k_blk | (uintptr_t)v_blk | (uintptr_t)k_ctx |
                       (uintptr_t)v_ctx | (uintptr_t)o | (uintptr_t)workspace;
  if (al % 16 != 0) return fail(SFV_E_INVAL, "tensor pointers must be 16-byte aligned");
  return hip_status(sfv::launch_attention(q, k_blk, v_blk, k_ctx, v_ctx, B1, N, L, Hq, Hkv, d, softmax_scale,
                                          o, lse, workspace, plan, (hipStream_t)stream, rec_rows, src, rec_count,
                                          rec_pos),
                    "sfv_attend_folded");
}

int sfv_attend_trays(const void* q, const void* k_blk, const void* v_blk, const void* k_ctx, const void* v_ctx,
                     int B1, int N, int L, int Hq, int Hkv, int d, float softmax_scale, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_attn_dims(B1, N, L, Hq, Hkv, d);
  if (rc != SFV_OK) return rc;
  if (!q || !k_blk || !v_blk || !o || !lse) return fail(SFV_E_INVAL, "null tensor pointer");
  if (L > 0 && (!k_ctx || !v_ctx)) return fail(SFV_E_INVAL, "null context pointer with L=%d", L);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f))
    return fail(SFV_E_INVAL, "softmax_scale=%g must be finite and > 0", (double)softmax_scale);
  const sfv::AttnPlan plan = sfv::attn_plan(B1, N, L, Hq, Hkv, d);
  if (workspace_bytes < plan.ws_bytes) {
    return fail(SFV_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, plan.ws_bytes);
  }
  if (plan.ws_bytes > 0 && !workspace) return fail(SFV_E_INVAL, "workspace is NULL");
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k_blk | (uintptr_t)v_blk | (uintptr_t)k_ctx |
                       (uintptr_t)v_ctx | (uintptr_t)o | (uintptr_t)workspace;
  if (al % 16 != 0) return fail(SFV_E_INVAL, "tensor pointers must be 16-byte aligned");
  return hip_status(sfv::launch_attention(q, k_blk, v_blk, k_ctx, v_ctx, B1, N, L, Hq, Hkv, d, softmax_scale,
                                          o, lse, workspace, plan, (hipStream_t)stream, nullptr, nullptr,
                                          nullptr, nullptr, true),
                    "sfv_attend_trays");
}

int check_reject_dims(int n_trays, int B, int V) {
  if (n_trays < 1 || n_trays > SFV_MAX_BRANCHES) return fail(SFV_E_INVAL, "n_trays=%d not in [1, %d]", n_trays,
                                                              SFV_MAX_BRANCHES);
  if (B < 1 || B > SFV_MAX_BLOCK) return fail(SFV_E_INVAL, "B=%d not in [1, %d]", B, SFV_MAX_BLOCK);
  if (V < 1 || V >= (1 << 30)) return fail(SFV_E_INVAL, "V=%d out of range", V);
  if ((double)n_trays * (B + 1) * V >= 9.0e15) return fail(SFV_E_INVAL, "too large");
  return SFV_OK;
}

int sfv_reject_workspace_bytes(int n_trays, int B, int V, size_t* bytes) {
  if (!bytes) return fail(SFV_E_INVAL, "bytes is NULL");
  const int rc = check_reject_dims(n_trays, B, V);
  if (rc != SFV_OK) return rc;
  *bytes = sfv::reject_plan(n_trays, B, V).ws_bytes;
  return ok();
}

int sfv_reject_verify(const float* logits, const float* q, const int32_t* tokens, int n_trays, int B, int V,
                      float temperature, uint64_t seed, uint64_t step0, int64_t pos0, int32_t* n_accept,
                      int32_t* next_token, void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = check_reject_dims(n_trays, B, V);
  if (rc != SFV_OK) return rc;
  if (!(temperature >= 0.f) || !std::isfinite(temperature)) return fail(SFV_E_INVAL, "temperature must be >= 0");
  if (!logits || !q || !tokens || !n_accept || !next_token || !workspace) return fail(SFV_E_INVAL, "null pointer");
  const sfv::RejectPlan plan = sfv::reject_plan(n_trays, B, V);
  if (workspace_bytes < plan.ws_bytes)
    return fail(SFV_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, plan.ws_bytes);
  if ((uintptr_t)workspace % 256 != 0) return fail(SFV_E_INVAL, "workspace must be 256-byte aligned");
  return hip_status(sfv::launch_reject(logits, q, tokens, n_trays, B, V, temperature, seed, step0, pos0, n_accept,
                                       next_token, workspace, plan, (hipStream_t)stream),
                    "sfv_reject_verify");
}

int sfv_match_trays(const int32_t* n_accept, const int32_t* next_token, int verified, const int32_t* tray_k,
                    const int32_t* tray_alt, int n_prepared, int32_t* served, void* stream) {
  if (verified < 0 || verified >= SFV_MAX_BRANCHES) return fail(SFV_E_INVAL, "verified=%d out of range", verified);
  if (n_prepared < 0 || n_prepared > (1 << 20)) return fail(SFV_E_INVAL, "n_prepared=%d out of range", n_prepared);
  if (!n_accept || !next_token || !served || (n_prepared > 0 && (!tray_k || !tray_alt)))
    return fail(SFV_E_INVAL, "null pointer");
  return hip_status(sfv::launch_match_trays(n_accept, next_token, verified, tray_k, tray_alt, n_prepared, served,
                                            (hipStream_t)stream),
                    "sfv_match_trays");
}

int sfv_masked_rows(const int32_t* state, int B1, int N, int32_t* rows, int32_t* count, void* stream) {
  if (!state || !rows || !count) return fail(SFV_E_INVAL, "null pointer");
  if (B1 < 1 || B1 > SFV_MAX_BRANCHES) return fail(SFV_E_INVAL, "B1=%d not in [1, %d]", B1, SFV_MAX_BRANCHES);
  if (N < 1 || N > SFV_MAX_BLOCK) return fail(SFV_E_INVAL, "N=%d not in [1, %d]", N, SFV_MAX_BLOCK);
  return hip_status(sfv::launch_masked_rows(state, B1, N, rows, count, (hipStream_t)stream),
                    "sfv_masked_rows");
}

int sfv_lm_head(const void* hidden, const int32_t* rows, int M, int R, const void* w, int D, int V,
                float* logits, int32_t* status, void* stream) {
  if (M < 0) return fail(SFV_E_INVAL, "M=%d < 0", M);
  if (R < 1) return fail(SFV_E_INVAL, "R=%d < 1", R);
  if (D < 1 || V < 1) return fail(SFV_E_INVAL, "D=%d, V=%d must be positive", D, V);
  if (D % 64 != 0) return fail(SFV_E_UNSUPPORTED, "D=%d is not a multiple of 64", D);
  if ((double)M * V >= 9.0e15 || (double)V * D >= 9.0e15) return fail(SFV_E_INVAL, "too large");
  if (M > 0 && (!hidden || !rows || !w || !logits)) return fail(SFV_E_INVAL, "null tensor pointer");
  const uintptr_t al = (uintptr_t)hidden | (uintptr_t)w | (uintptr_t)logits;
  if (al % 16 != 0) return fail(SFV_E_INVAL, "tensor pointers must be 16-byte aligned");
  if ((uintptr_t)status % 4 != 0) return fail(SFV_E_INVAL, "status must be 4-byte aligned");
  if (status) {
    const hipError_t e = sfv::launch_rows_status(rows, M, R, status, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "sfv_lm_head: row check");
  }
  return hip_status(sfv::launch_lm_head(hidden, rows, M, R, w, D, V, logits, (hipStream_t)stream),
                    "sfv_lm_head");
}

int sfv_commit_workspace_bytes(int B1, int N, int M, int V, size_t* bytes) {
  if (!bytes) return fail(SFV_E_INVAL, "bytes is NULL");
  const int rc = check_commit_dims(B1, N, M, V);
  if (rc != SFV_OK) return rc;
  // Worst case over trees and temperatures: M items (T = 0 uses exactly M).
  const sfv::CommitPlan a = sfv::commit_plan(B1, N, M, V, M, false);
  size_t worst = a.ws_bytes;
  for (int items = 1; items <= M; items = items < 16 ? items + 1 : items * 2) {
    const sfv::CommitPlan b = sfv::commit_plan(B1, N, M, V, items, true);
    if (b.ws_bytes > worst) worst = b.ws_bytes;
  }
  const sfv::CommitPlan c = sfv::commit_plan(B1, N, M, V, M, true);
  if (c.ws_bytes > worst) worst = c.ws_bytes;
  *bytes = worst;
  return ok();
}

}  // extern "C"

namespace {

// Argument checks shared by sfv_commit and sfv_commit_noalloc; fills the tree
// and the launch plan (whose ws_bytes is the workspace this call needs).
int prepare_commit(const float* logits, const int32_t* rows, int M, const int32_t* state,
                   const int32_t* parent_host, int B1, int N, int V, float temperature, int k_max,
                   float tau, int32_t* next_state, int32_t* commit_pos, int32_t* token, float* conf,
                   sfv::TreeArgs* tree, sfv::CommitPlan* plan) {
  int rc = check_commit_dims(B1, N, M, V);
  if (rc != SFV_OK) return rc;
  if (!state || !next_state || !commit_pos) return fail(SFV_E_INVAL, "null pointer");
  if (M > 0 && (!logits || !rows || !token || !conf)) return fail(SFV_E_INVAL, "null pointer");
  if (!(temperature >= 0.f) || !std::isfinite(temperature)) {
    return fail(SFV_E_INVAL, "temperature must be finite and >= 0");
  }
  if (k_max < 1) return fail(SFV_E_INVAL, "k_max=%d < 1", k_max);
  if (k_max > N) return fail(SFV_E_INVAL, "k_max=%d > N=%d", k_max, N);
  if (k_max > 1 && !std::isfinite(tau)) return fail(SFV_E_INVAL, "tau must be finite");
  if ((uintptr_t)logits % 16 != 0) return fail(SFV_E_INVAL, "logits must be 16-byte aligned");
  rc = make_tree(parent_host, B1, tree);
  if (rc != SFV_OK) return rc;
  const bool noisy = temperature > 0.f;
  const int items = commit_items_max(*tree, N, M, noisy);
  *plan = sfv::commit_plan(B1, N, M, V, items, noisy);
  return SFV_OK;
}

}  // namespace

extern "C" {

int sfv_commit(const float* logits, const int32_t* rows, int M, const int32_t* state,
               const int32_t* parent_host, int B1, int N, int V, float temperature, uint64_t seed,
               uint64_t step0, int64_t pos0, int k_max, float tau, int32_t* next_state,
               int32_t* commit_pos, int32_t* token, float* conf, void* workspace,
               size_t workspace_bytes, void* stream) {
  sfv::TreeArgs tree;
  sfv::CommitPlan plan;
  const int rc = prepare_commit(logits, rows, M, state, parent_host, B1, N, V, temperature, k_max, tau,
                                next_state, commit_pos, token, conf, &tree, &plan);
  if (rc != SFV_OK) return rc;
  if (!workspace) return fail(SFV_E_INVAL, "null pointer");
  if (workspace_bytes < plan.ws_bytes) {
    return fail(SFV_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, plan.ws_bytes);
  }
  return hip_status(sfv::launch_commit(logits, rows, M, state, tree, N, V, temperature, seed, step0,
                                       pos0, k_max, tau, next_state, commit_pos, token, conf,
                                       workspace, plan,
                                       (hipStream_t)stream),
                    "sfv_commit");
}

int sfv_commit_noalloc(const float* logits, const int32_t* rows, int M, const int32_t* state,
                       const int32_t* parent_host, int B1, int N, int V, float temperature, uint64_t seed,
                       uint64_t step0, int64_t pos0, int k_max, float tau, int32_t* next_state,
                       int32_t* commit_pos, int32_t* token, float* conf, void* stream) {
  sfv::TreeArgs tree;
  sfv::CommitPlan plan;
  const int rc = prepare_commit(logits, rows, M, state, parent_host, B1, N, V, temperature, k_max, tau,
                                next_state, commit_pos, token, conf, &tree, &plan);
  if (rc != SFV_OK) return rc;
  if (plan.ws_bytes > sfv::kCommitScratchBytes) {
    return fail(SFV_E_WORKSPACE, "this call needs %zu bytes of workspace; the static one holds %zu",
                plan.ws_bytes, sfv::kCommitScratchBytes);
  }
  if (stream != nullptr) {
    int cur = -1, sdev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return hip_status(e, "sfv_commit_noalloc");
    if (sdev != cur) {
      return fail(SFV_E_INVAL, "stream is on device %d, the current device is %d", sdev, cur);
    }
  }
  void* ws = nullptr;
  const hipError_t e = sfv::commit_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "sfv_commit_noalloc: static workspace address");
  return hip_status(sfv::launch_commit(logits, rows, M, state, tree, N, V, temperature, seed, step0,
                                       pos0, k_max, tau, next_state, commit_pos, token, conf, ws, plan,
                                       (hipStream_t)stream),
                    "sfv_commit_noalloc");
}

int sfv_lm_head_greedy_bytes(int M, int V, int D, size_t* bytes) {
  if (!bytes) return fail(SFV_E_INVAL, "bytes is NULL");
  if (M < 0 || V < 1 || D < 1) return fail(SFV_E_INVAL, "M=%d, V=%d, D=%d out of range", M, V, D);
  const int ns = sfv::lm_head_greedy_parts(M, V, D);
  if (ns == 0) {
    return fail(SFV_E_UNSUPPORTED,
                "greedy partials need M >= 33 and D %% 64 == 0 (M=%d, D=%d)", M, D);
  }
  *bytes = (size_t)ns * M * sizeof(sfv::GreedyPart);
  return ok();
}

int sfv_lm_head_greedy(const void* hidden, const int32_t* rows, int M, int R, const void* w, int D, int V,
                       float* logits, void* partials, size_t partials_bytes, int32_t* status, void* stream) {
  size_t need = 0;
  int rc = sfv_lm_head_greedy_bytes(M, V, D, &need);
  if (rc != SFV_OK) return rc;
  if (R < 1) return fail(SFV_E_INVAL, "R=%d < 1", R);
  if ((double)M * V >= 9.0e15 || (double)V * D >= 9.0e15) return fail(SFV_E_INVAL, "too large");
  if (!hidden || !rows || !w || !logits || !partials) return fail(SFV_E_INVAL, "null pointer");
  const uintptr_t al = (uintptr_t)hidden | (uintptr_t)w | (uintptr_t)logits | (uintptr_t)partials;
  if (al % 16 != 0) return fail(SFV_E_INVAL, "tensor pointers must be 16-byte aligned");
  if (partials_bytes < need) return fail(SFV_E_WORKSPACE, "partials %zu bytes < %zu needed", partials_bytes, need);
  if ((uintptr_t)status % 4 != 0) return fail(SFV_E_INVAL, "status must be 4-byte aligned");
  if (status) {
    const hipError_t e = sfv::launch_rows_status(rows, M, R, status, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "sfv_lm_head_greedy: row check");
  }
  return hip_status(sfv::launch_lm_head_greedy(hidden, rows, M, R, w, D, V, logits,
                                               (sfv::GreedyPart*)partials, (hipStream_t)stream),
                    "sfv_lm_head_greedy");
}

int sfv_commit_greedy_workspace_bytes(int B1, int N, int M, int V, size_t* bytes) {
  if (!bytes) return fail(SFV_E_INVAL, "bytes is NULL");
  const int rc = check_commit_dims(B1, N, M, V);
  if (rc != SFV_OK) return rc;
  *bytes = sfv::commit_greedy_ws_bytes(B1, N, M);
  return ok();
}

int sfv_commit_greedy(const void* partials, size_t partials_bytes, int D, const float* logits,
                      const int32_t* rows, int M, const int32_t* state, const int32_t* parent_host, int B1,
                      int N, int V, int k_max, float tau, int32_t* next_state, int32_t* commit_pos,
                      int32_t* token, float* conf, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_commit_dims(B1, N, M, V);
  if (rc != SFV_OK) return rc;
  size_t need_parts = 0;
  rc = sfv_lm_head_greedy_bytes(M, V, D, &need_parts);
  if (rc != SFV_OK) return rc;
  if (!state || !next_state || !commit_pos || !workspace || !partials) return fail(SFV_E_INVAL, "null pointer");
  if (!logits || !rows || !token || !conf) return fail(SFV_E_INVAL, "null pointer");
  if (((uintptr_t)partials | (uintptr_t)logits) % 16 != 0) {
    return fail(SFV_E_INVAL, "partials and logits must be 16-byte aligned");
  }
  if (partials_bytes < need_parts) {
    return fail(SFV_E_WORKSPACE, "partials %zu bytes < %zu needed", partials_bytes, need_parts);
  }
  if (k_max < 1) return fail(SFV_E_INVAL, "k_max=%d < 1", k_max);
  if (k_max > N) return fail(SFV_E_INVAL, "k_max=%d > N=%d", k_max, N);
  if (k_max > 1 && !std::isfinite(tau)) return fail(SFV_E_INVAL, "tau must be finite");
  sfv::TreeArgs tree;
  rc = make_tree(parent_host, B1, &tree);
  if (rc != SFV_OK) return rc;
  const size_t need = sfv::commit_greedy_ws_bytes(B1, N, M);
  if (workspace_bytes < need) return fail(SFV_E_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  return hip_status(sfv::launch_commit_greedy((const sfv::GreedyPart*)partials, sfv::lm_head_greedy_parts(M, V, D),
                                              logits, rows, M, state, tree, N, V, k_max, tau, next_state,
                                              commit_pos, token, conf, workspace, (hipStream_t)stream),
                    "sfv_commit_greedy");
}

int sfv_match_tree(const int32_t* state, const int32_t* next_state, const int32_t* commit_pos,
                   const int32_t* parent_host, int B1, int N, int k_max, int S_max, int32_t* chain,
                   int32_t* n_accepted, int32_t* status, void* stream) {
  if (!state || !next_state || !commit_pos || !chain || !n_accepted || !status) {
    return fail(SFV_E_INVAL, "null pointer");
  }
  if (N < 1 || N > SFV_MAX_BLOCK) return fail(SFV_E_INVAL, "N=%d not in [1, %d]", N, SFV_MAX_BLOCK);
  if (k_max < 1) return fail(SFV_E_INVAL, "k_max=%d < 1", k_max);
  sfv::TreeArgs tree;
  const int rc = make_tree(parent_host, B1, &tree);
  if (rc != SFV_OK) return rc;
  return hip_status(sfv::launch_match(state, next_state, commit_pos, tree, N, k_max, S_max, chain,
                                      n_accepted, status, (hipStream_t)stream),
                    "sfv_match_tree");
}

int sfv_gumbel_words(uint32_t first, uint32_t count, float* out, void* stream) {
  if (!out && count > 0) return fail(SFV_E_INVAL, "out is NULL");
  if ((uintptr_t)out % 4 != 0) return fail(SFV_E_INVAL, "out must be 4-byte aligned");
  if ((uint64_t)first + count > (1ull << 32)) {
    return fail(SFV_E_INVAL, "words %u + %u run past 2^32", first, count);
  }
  return hip_status(sfv::launch_gumbel_words(first, count, out, (hipStream_t)stream), "sfv_gumbel_words");
}

int sfv_selfcheck_bounds(double* out, void* stream) {
  if (!out) return fail(SFV_E_INVAL, "out is NULL");
  return hip_status(sfv::launch_selfcheck(out, (hipStream_t)stream), "sfv_selfcheck_bounds");
}

}  // extern "C"
