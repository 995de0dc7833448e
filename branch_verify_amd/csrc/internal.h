// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sfv {

struct AttnPlan {
  int rows_total;  // B1 * N * G query rows per kv head
  int row_tiles;   // ceil(rows_total / 128)
  int splits;      // context key ranges
  int chunk;       // context keys per range (multiple of 64)
  int tail_tiles;  // dense path: the last row tiles of every kv head, split apart (0: none)
  int tail_splits, tail_chunk;  // their context ranges
  size_t ws_bytes;
  size_t ws_bytes_folded;  // folded path: context states of every row slot
};

AttnPlan attn_plan(int B1, int N, int L, int Hq, int Hkv, int d);

// With rec_rows non-null (folded verification): the context is attended by
// the rec_count[0] slots listed in rec_rows only, and every slot attends its
// branch's block keys (read through src) with its source's query, merged
// with its source row's context state (rec_pos maps a slot to its index in
// rec_rows).  The workspace is then plan.ws_bytes_folded.
hipError_t launch_attention(const void* q, const void* k_blk, const void* v_blk,
                            const void* k_ctx, const void* v_ctx, int B1, int N, int L,
                            int Hq, int Hkv, int d, float scale, void* o, float* lse,
                            void* ws, const AttnPlan& plan, hipStream_t stream,
                            const int32_t* rec_rows = nullptr, const int32_t* src = nullptr,
                            const int32_t* rec_count = nullptr, const int32_t* rec_pos = nullptr,
                            bool causal = false);

hipError_t launch_masked_rows(const int32_t* state, int B1, int N, int32_t* rows,
                              int32_t* count, hipStream_t stream);

hipError_t launch_lm_head(const void* hidden, const int32_t* rows, int M, int R, const void* w,
                          int D, int V, float* logits, hipStream_t stream);

// *status = -1 (SFV_E_INVAL) if any of rows[0 .. M) lies outside [0, R), else 0.
hipError_t launch_rows_status(const int32_t* rows, int M, int R, int32_t* status, hipStream_t stream);

// Error model of a fast confidence term t = exp2(fl32(fl32(x - m) * log2e))
// against exp(x - m), for a = m - x:  |t / exp(x - m) - 1| <= kExpC1 * |a| +
// kExpC2.  kExpC1 covers the two fp32 roundings of the argument and log2e's
// own, kExpC2 the hardware exp2 (certified below 2^-22 by sfv_selfcheck_bounds
// for every argument in [-126, kExp2ArgMax]; 2^-20 is used).  The greedy terms
// have a >= 0; the sampled sweep takes them against a reference at most
// kLazyMargin below its running max, so a >= -kLazyMargin and the argument
// stays below kLazyMargin * log2e < kExp2ArgMax.
constexpr float kLog2eF = 1.44269504088896341f;
constexpr float kExpC1 = 3.5f / 16777216.0f;
constexpr float kExpC2 = 1.0f / 1048576.0f;
constexpr float kLazyMargin = 4.0f;
constexpr float kExp2ArgMax = 6.0f;

// Greedy partial of one row over a range of vocabulary ids (a 128-id vocab
// tile when written by the fused LM head): the max logit, the lowest id
// attaining it, the fp32 sum of exp(l - max) over the range and a bound on
// that sum's error.
struct GreedyPart {
  float m;
  int idx;
  float S;
  float E;
};

// Fused LM head + greedy partials: served for these shapes when the result
// is > 0 (the number of partials per row, one per vocab tile; `gpart` is
// [tiles][M]), else 0.
int lm_head_greedy_parts(int M, int V, int D);
hipError_t launch_lm_head_greedy(const void* hidden, const int32_t* rows, int M, int R, const void* w,
                                 int D, int V, float* logits, GreedyPart* gpart, hipStream_t stream);

constexpr int kMaxBranches = 64;
constexpr int kMaxBlock = 256;

struct CommitPlan {
  int splits;        // vocabulary ranges per row
  int chunk;         // vocab ids per range (multiple of 2048)
  int items_max;     // upper bound of work items (rows, or row groups at T > 0)
  size_t ws_bytes;
};

// Tree description passed by value to the kernels.
struct TreeArgs {
  int B1;
  int levels;
  signed char depth[kMaxBranches];
  signed char parent[kMaxBranches];
  unsigned char by_level[kMaxBranches];    // branches sorted by depth
  unsigned char level_start[kMaxBranches + 1];
};

// Rows of equal (depth, position) share one noise sweep at T > 0, up to 4 per
// item (with 8, the per-row sweep state leaves room for only three waves per
// SIMD, and the sweep runs slower despite fewer noise evaluations).
constexpr int kItemRowsHost = 4;
CommitPlan commit_plan(int B1, int N, int M, int V, int items_max, bool noisy);

hipError_t launch_commit(const float* logits, const int32_t* rows, int M, const int32_t* state,
                         const TreeArgs& tree, int N, int V, float temperature, uint64_t seed,
                         uint64_t step0, int64_t pos0, int k_max, float tau, int32_t* next_state,
                         int32_t* commit_pos,
                         int32_t* token, float* conf, void* ws, const CommitPlan& plan,
                         hipStream_t stream);

// Device address, on the current GPU, of the static workspace that
// sfv_commit_noalloc uses in place of a caller's (kCommitScratchBytes).
constexpr size_t kCommitScratchBytes = 1u << 20;
hipError_t commit_scratch(void** ptr);

// Greedy commit from the fused LM head's tile partials: a merge kernel
// reduces the partials of every row to kGreedyChunks, then the commit's
// finalize kernel (the same one the vocabulary sweep feeds) decides.
constexpr int kGreedyChunks = 2;
size_t commit_greedy_ws_bytes(int B1, int N, int M);
hipError_t launch_commit_greedy(const GreedyPart* gpart, int nparts, const float* logits,
                                const int32_t* rows, int M, const int32_t* state, const TreeArgs& tree,
                                int N, int V, int k_max, float tau, int32_t* next_state, int32_t* commit_pos,
                                int32_t* token, float* conf, void* ws, hipStream_t stream);

hipError_t launch_match(const int32_t* state, const int32_t* next_state, const int32_t* commit_pos,
                        const TreeArgs& tree, int N, int k_max, int S_max, int32_t* chain,
                        int32_t* n_accepted, int32_t* status, hipStream_t stream);

hipError_t launch_selfcheck(double* out, hipStream_t stream);
hipError_t launch_gumbel_words(uint32_t first, uint32_t count, float* out, hipStream_t stream);

constexpr int kMaxTopk = 32;            // stale conditionals per position
constexpr int kMaxTopkChunks = 16;      // workgroups per row of the stale top-K
constexpr int kTopkChunkTarget = 4096;  // ids per chunk it aims for
struct TopkPlan {
  int S, C;  // chunks per row, ids per chunk
  size_t ws_bytes;
};
TopkPlan topk_plan(int M, int V, int K);

hipError_t launch_stale_topk(const float* logits, const int32_t* rows, const float* conf, int M, int V, int N,
                             int branch, int K, int32_t* top_ids, float* top_logit, float* conf_pos, void* ws,
                             const TopkPlan& plan, hipStream_t stream);

hipError_t launch_draft_tree(const int32_t* root, const int32_t* top_ids, const float* top_logit,
                             const float* conf, int N, int K, int D, int W, float temperature, uint64_t seed,
                             uint64_t step0, int64_t pos0, int32_t* parent, int32_t* states, int32_t* n_drafts,
                             hipStream_t stream);

// Rejection-sampling verification of drafted trays.
constexpr int kMaxRejectChunks = 16;
constexpr int kRejectChunkTarget = 8192;
struct RejectPlan {
  int S, C;  // chunks per emitting row, ids per chunk
  size_t ws_bytes;
};
struct RejectWs {
  float* row_max;    // [n][B+1] max of the (scaled) logits
  int* row_arg;      // [n][B+1] first index attaining it
  int* accept;       // [n][B+1] drafted token accepted (positions < B)
  double* chunk_sum; // [n][S] exact partial denominators of the emitting row
  double* chunk_key; // [n][S]
  int* chunk_id;     // [n][S]
  float* chunk_max;  // [n][B+1][S] per-chunk max of z
  int* chunk_arg;    // [n][B+1][S] its first index
  double* chunk_sum_f;  // [n][B+1][S] fast sum of exp(z - chunk max)
  double* chunk_err;    // [n][B+1][S] bound on its error
};
RejectPlan reject_plan(int n, int B, int V);
hipError_t launch_reject(const float* logits, const float* q, const int32_t* tokens, int n, int B, int V,
                         float temperature, uint64_t seed, uint64_t step0, int64_t pos0, int32_t* n_accept,
                         int32_t* next_token, void* ws, const RejectPlan& plan, hipStream_t stream);
hipError_t launch_match_trays(const int32_t* n_accept, const int32_t* next_token, int verified,
                              const int32_t* tray_k, const int32_t* tray_alt, int n_prepared, int32_t* served,
                              hipStream_t stream);

hipError_t launch_fold_gate(const void* H, const TreeArgs& tree, int N, int D, float delta,
                            int32_t* recompute, int32_t* src, int32_t* rec_rows, int32_t* rec_count,
                            int32_t* rec_pos, int32_t* branch_off, hipStream_t stream);



}  // namespace sfv
