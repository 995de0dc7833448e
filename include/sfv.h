/*
 * sfv.h — C ABI of libsfv: one multi-branch draft-verification step of
 * speculative decoding for masked diffusion language models, on one MI355X
 * (gfx950).
 *
 * The step (SpecFold: "Folding Multi-Branch Redundancy for Faster Speculative
 * Decoding in Diffusion Language Models", introduction and Fig. 1-(b); "On the
 * SPOT: Enhancing Speculative Decoding for Diffusion Language Models via
 * Commit-Order Prediction", coupled-noise match and Propositions 1-2):
 *   B1 = B + 1 block states of length N — the main branch (index 0) and B
 *   drafts whose parents have smaller indices — are verified in one batched
 *   pass against a shared cached context of L positions, then the target's
 *   own commit is taken on every branch and the main branch's next state is
 *   matched against the drafted states.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers unless their name ends in _host.
 *     bf16 tensors are passed as const void* holding IEEE bfloat16 bits.
 *     All tensors are dense, row-major, in the layout given beside them.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is launched and the return value says why
 *     (sfv_last_error() gives a message).  On success the work is enqueued
 *     on `stream` (a hipStream_t passed as void*; NULL = the null stream)
 *     and the call returns at once; outputs are valid after the stream is
 *     synchronised.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no state between calls; calls on distinct streams with
 *     distinct outputs and workspaces may overlap.
 *   - The mask token is SFV_MASK (-1); tokens lie in [0, V).
 */
#ifndef SFV_H
#define SFV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SFV_OK = 0,
  SFV_E_INVAL = -1,        /* null pointer, size out of range */
  SFV_E_UNSUPPORTED = -2,  /* valid but not implemented (head dim, group size, ...) */
  SFV_E_TREE = -3,         /* parent_host[0] != -1 or parent_host[i] not in [0, i) */
  SFV_E_STATE = -4,        /* device-detected: a draft does not extend its parent */
  SFV_E_WORKSPACE = -5,    /* workspace smaller than the *_workspace_bytes size */
  SFV_E_HIP = -6           /* a HIP launch failed */
};

#define SFV_MASK (-1)
#define SFV_MAX_BRANCHES 64  /* B1 limit: the tree is host control data */
#define SFV_MAX_BLOCK 256    /* N limit */
#define SFV_MAX_TOPK 32      /* stale conditionals per position */
#define SFV_MAX_DRAFT_WIDTH 16  /* children offered per draft-tree node */

/* Message of the last non-OK return on this thread ("" if none). */
const char* sfv_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int sfv_version(void);

/*
 * Shared-prefix attention of every branch.
 * SpecFold, introduction (bidirectional in-block attention; the shared-prefix
 * KV cache reused across all branches) and App. A.1 (streaming-softmax state
 * (m, Z, O) over the concatenated prefix and block keys).
 *
 * For every branch i, position n and query head h, with kv head g = h / (Hq/Hkv):
 *   keys = the L context keys of head g followed by the N block keys of
 *   branch i, head g; no key is masked (bidirectional block).
 *   s_j = softmax_scale * <q, k_j>;  o = sum_j e^{s_j} v_j / sum_j e^{s_j};
 *   lse = ln sum_j e^{s_j}  (natural log).
 *
 *   q      [B1][N][Hq][d]  bf16      k_blk, v_blk [B1][N][Hkv][d] bf16
 *   k_ctx, v_ctx [Hkv][L][d] bf16 — one copy shared by all branches
 *   o      [B1][N][Hq][d]  bf16 (round to nearest even)
 *   lse    [B1][N][Hq]     fp32
 * Supported: d in {32, 64, 128}; Hq/Hkv in {1, 2, 4, 8}; 1 <= B1 <= 64;
 * 1 <= N <= 256; L >= 0.  fp32 accumulation.  softmax_scale must be finite
 * and > 0 (the kernel tracks the running maximum of the unscaled scores), else
 * SFV_E_INVAL; this holds for sfv_attend_trays and sfv_attend_folded too.
 * `workspace` holds split-context partial states; its size comes from
 * sfv_attend_workspace_bytes (may be 0, then workspace may be NULL).
 */
int sfv_attend_workspace_bytes(int B1, int N, int L, int Hq, int Hkv, int d, size_t* bytes);
int sfv_attend_branches(const void* q, const void* k_blk, const void* v_blk,
                        const void* k_ctx, const void* v_ctx,
                        int B1, int N, int L, int Hq, int Hkv, int d, float softmax_scale,
                        void* o, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal attention of drafted trays for an autoregressive target.  D3D
 * explainer: the target verifies each prepared tray (a continuation of the
 * shared prefix) in one packed pass.
 *
 * As sfv_attend_branches (branch = tray, position = token of the tray), but
 * the row at position n of tray i sees the L context keys and the block keys
 * of tray i at positions 0..n only.  Same shapes, dtypes, workspace
 * (sfv_attend_workspace_bytes) and limits.
 */
int sfv_attend_trays(const void* q, const void* k_blk, const void* v_blk,
                     const void* k_ctx, const void* v_ctx,
                     int B1, int N, int L, int Hq, int Hkv, int d, float softmax_scale,
                     void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Rejection-sampling verification of drafted trays for an autoregressive
 * target.  D3D explainer: verification by rejection sampling with the
 * proposal probabilities, the standard rule that preserves the target's
 * distribution.
 *
 * For tray j (noise step step0 + j) with drafted tokens x_0..x_{B-1}:
 *   T > 0: p_t = softmax(fl32(l_t * fl32(1/T))) in fp64 (exact exp);
 *   x_t is accepted iff u_t * q_t(x_t) < p_t(x_t), u_t = (w + 1/2) 2^-32 with
 *   w the noise word of id 0 on stream 1 at position pos0 + t; a = the first
 *   rejected t (B if none).  a < B emits argmax over v with p_a(v) > q_a(v)
 *   of ln(p_a(v) - q_a(v)) + g(v); a = B emits argmax_v fl32(l_B(v) / T) +
 *   g(v); g = -ln(-ln u) in fp64 from stream 2 at position pos0 + a; ties to
 *   the lower id; an empty residual emits the first argmax of fl32(l_a / T).
 *   T = 0: x_t accepted iff it is the first argmax of l_t; emits the first
 *   argmax of l_a.
 *   logits [n_trays][B+1][V] fp32 (the target's distributions at the B
 *   drafted positions and the bonus position); q [n_trays][B][V] fp32 (the
 *   drafter's probabilities); tokens [n_trays][B] int32
 *   n_accept [n_trays] int32 out (a); next_token [n_trays] int32 out
 *   workspace: sfv_reject_workspace_bytes(n_trays, B, V), 256-byte aligned
 * Supported: 1 <= n_trays <= 64, 1 <= B <= 256, T >= 0 finite.
 */
int sfv_reject_workspace_bytes(int n_trays, int B, int V, size_t* bytes);
int sfv_reject_verify(const float* logits, const float* q, const int32_t* tokens, int n_trays, int B, int V,
                      float temperature, uint64_t seed, uint64_t step0, int64_t pos0, int32_t* n_accept,
                      int32_t* next_token, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Serving a prepared tray.  D3D explainer: each prepared tray extends the
 * prefix by the tokens accepted before a rejection point and another token
 * there; the tray matching the verified prefix is served (a cache hit).
 *
 * served[0] = the lowest k with tray_k[k] == n_accept[verified] and
 * tray_alt[k] == next_token[verified], or -1 (a miss).
 *   n_accept, next_token: as from sfv_reject_verify; tray_k, tray_alt
 *   [n_prepared] int32 (device); served [1] int32 out.
 */
int sfv_match_trays(const int32_t* n_accept, const int32_t* next_token, int verified, const int32_t* tray_k,
                    const int32_t* tray_alt, int n_prepared, int32_t* served, void* stream);

/*
 * Stale conditionals for drafting.  SPOT, "How does SPOT draft and verify?"
 * (the drafter reads the target's latest top-32 probabilities at each masked
 * position) and "Important context" (stale conditionals).
 *
 * For every masked row r (rows as from sfv_masked_rows) of branch `branch`,
 * n = rows[r] % N: top_ids[n][0..K) = the K vocab ids with the largest
 * logits[r][.], by value, ties to the lower id; top_logit[n][k] their fp32
 * logits; conf_pos[n] = conf[r] (as sfv_commit wrote it).  Entries of
 * positions with no row are left untouched.
 *   logits [M][V] fp32; rows [M] int32; conf [M] fp32
 *   top_ids [N][K] int32 out; top_logit [N][K] fp32 out; conf_pos [N] fp32 out
 *   workspace: sfv_stale_topk_workspace_bytes(M, V, N, K) bytes, 16-byte aligned
 * Supported: 1 <= K <= min(32, V), V < 2^30.  Up to 16 workgroups per row
 * (two passes over their chunk), then one per row to merge.
 */
int sfv_stale_topk_workspace_bytes(int M, int V, int N, int K, size_t* bytes);
int sfv_stale_topk(const float* logits, const int32_t* rows, const float* conf, int M, int V, int N,
                   int branch, int K, int32_t* top_ids, float* top_logit, float* conf_pos,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Draft tree from stale conditionals.  SPOT, "Important context" (block
 * states grown by predicting the next committed position, high-probability
 * branches first, up to D drafted states; coupled-noise match) and "How does
 * SPOT differ from Spiffy, SSD and BlockSpec?" (SSD-style confidence chain,
 * BlockSpec-style confidence tree).
 *
 * From root [N] (SFV_MASK = masked) with, per masked position n, its top-K
 * ids/logits and confidence c_n: a node u offers its W most confident masked
 * positions (c descending, ties to the lower position) as children; child
 * u+n has probability P(u) * c_n / sum_{m masked in u} c_m (fp64; the sum a
 * pairwise tree over 256 leaves, leaf m = c_m or 0, level by level element
 * 2j plus 2j+1); nodes are added best-first (probability, then lower parent
 * index, then lower position) until D drafts.  W = 0 or 1 gives the chain.
 * Drafted token at n from a node of depth d: T = 0, top_ids[n][0]; T > 0, the
 * id maximising fl32(fl32(l * fl32(1/T)) + g(seed, step0 + d, pos0 + n, id))
 * over the K candidates (the commit's noise), ties to the lower id.
 *   parent [D+1] int32 out (parent[0] = -1); states [D+1][N] int32 out
 *   n_drafts [1] int32 out: drafts built; branches past it copy the root
 *   (parent 0).
 * Supported: 0 <= D <= 63, 0 <= W <= 16, 1 <= K <= 32, T >= 0 finite.
 * One workgroup; no workspace.
 */
int sfv_draft_tree(const int32_t* root, const int32_t* top_ids, const float* top_logit, const float* conf,
                   int N, int K, int D, int W, float temperature, uint64_t seed, uint64_t step0, int64_t pos0,
                   int32_t* parent, int32_t* states, int32_t* n_drafts, void* stream);

/*
 * Fold gate for folded verification.  SpecFold, Sec. 3.2 (Eq. 4-5: the
 * per-token parent-child relative residual of the layer-input hidden state,
 * fold iff rho <= delta) and App. B (the main branch recomputes everything;
 * sources resolved to the nearest recomputed ancestor; compacted lists).
 *
 * For draft i >= 1 with parent p and position n:
 *   num = ||H_i[n] - H_p[n]||^2, den = ||H_p[n]||^2 (fp64 sums of the bf16
 *   values); recompute[i][n] = !(delta >= 0 && num <= delta^2 * den), with
 *   delta^2 formed in fp64 from the fp32 argument.  recompute[0][n] = 1.
 *   src[i][n] = i if recompute[i][n], else src[p][n] (nearest recomputed
 *   ancestor; the slot's Q/K/V are that branch's).
 *   rec_rows: flat i*N + n of every recomputed slot, in increasing order;
 *   rec_count[0] = their number; rec_pos[i][n] = the slot's index in
 *   rec_rows, -1 when folded; branch i's entries are
 *   rec_rows[branch_off[i] .. branch_off[i+1]).
 *
 *   hidden [B1][N][D] bf16, 16-byte aligned; parent_host as for sfv_commit
 *   recompute, src, rec_pos [B1][N] int32 out; rec_rows [B1*N] int32 out
 *   rec_count [1] int32 out; branch_off [B1+1] int32 out
 * Supported: D % 8 == 0; 1 <= B1 <= 64; 1 <= N <= 256; delta not NaN
 * (a negative delta folds nothing).  Two kernels on `stream`, no workspace.
 */
int sfv_fold_gate(const void* hidden, const int32_t* parent_host, int B1, int N, int D, float delta,
                  int32_t* recompute, int32_t* src, int32_t* rec_rows, int32_t* rec_count,
                  int32_t* rec_pos, int32_t* branch_off, void* stream);

/*
 * Folded-verification attention.  SpecFold, Sec. 3.2 and App. A.1 (a folded
 * position inherits its parent's query, key and value, and its attention
 * output stays exact with respect to its branch's own K/V table) and App. B
 * (only recomputed rows stream the shared prefix; folded rows reuse their
 * source row's streaming-softmax state).
 *
 * With the tables resolved by src (slot (i, n) holds the q/k/v of branch
 * src[i][n] at n), every (i, n, h) gets the output sfv_attend_branches would
 * give for the resolved q over [context | branch i's resolved block keys].
 * The recomputed slots (rec_rows, rec_count) attend the context; every slot
 * then attends its branch's resolved block keys with its resolved query and
 * merges in the context state (m, Z, O) of its source row (rec_pos).  A
 * folded slot's query and the context are its source's, so that state is
 * its own: folded rows never read the context and nothing is subtracted.
 * q/k/v at folded slots are never read.
 *
 *   Shapes and dtypes as sfv_attend_branches; src, rec_rows, rec_count,
 *   rec_pos as written by sfv_fold_gate.  Other index values give
 *   unspecified outputs but never an out-of-bounds access.
 *   workspace: sfv_attend_folded_workspace_bytes (0 when L = 0) bytes, holding
 *   the context states of the recomputed rows.
 */
int sfv_attend_folded_workspace_bytes(int B1, int N, int L, int Hq, int Hkv, int d, size_t* bytes);
int sfv_attend_folded(const void* q, const void* k_blk, const void* v_blk,
                      const void* k_ctx, const void* v_ctx,
                      int B1, int N, int L, int Hq, int Hkv, int d, float softmax_scale,
                      const int32_t* src, const int32_t* rec_rows, const int32_t* rec_count,
                      const int32_t* rec_pos, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Masked-row list.  SpecFold, introduction: the forward map returns token
 * distributions for the masked positions of the active block.
 *   state [B1][N] int32 (SFV_MASK = masked)
 *   rows  [B1*N] int32 out: flat ids i*N + n of masked positions in (i, n)
 *         order, the first *count entries valid
 *   count [1] int32 out
 */
int sfv_masked_rows(const int32_t* state, int B1, int N, int32_t* rows, int32_t* count,
                    void* stream);

/*
 * LM head over the masked rows.  SpecFold, Appendix B (the language-model
 * head is a plain dense product): logits[r][v] = sum_k hidden[rows[r]][k] * w[v][k].
 *   hidden [R][D] bf16 (R = B1*N, rows index it); rows [M] int32, each in [0, R)
 *   w      [V][D] bf16;  logits [M][V] fp32 (fp32 accumulation)
 * Supported: D % 64 == 0, 1 <= V, 0 <= M.  Row ids must lie in [0, R).  The
 * kernels read an id outside it as the nearest id inside it (never an access
 * outside hidden), so such a row's logits are another row's.  To detect them,
 * pass `status` (device int32, or NULL): before the product a one-workgroup
 * scan of rows writes *status = SFV_E_INVAL if any id is outside [0, R), else
 * SFV_OK.  Kernel by M: up to 32 rows a tiled kernel, above that 256-id vocab
 * tiles of 256 or 192 rows (the row tiles of a vocab tile side by side, so
 * the weight is read from HBM once).
 */
int sfv_lm_head(const void* hidden, const int32_t* rows, int M, int R,
                const void* w, int D, int V, float* logits, int32_t* status, void* stream);

/*
 * Commit of every branch: token per masked row, confidence, unmask-argmax.
 * SPOT, "Important context" (exact decoding commits one position per pass;
 * coupled-noise match) and Proposition 2; SpecFold, introduction (an
 * unmasking rule picks high-confidence masked positions).
 *
 * For masked row r = (i, n) with fp32 logits l:
 *   T == 0: token = lowest v attaining max l.
 *   T  > 0: invT = fl32(1/T); g_v = fl32(-ln(-ln u_v)), u_v = (w_v + 1/2) 2^-32,
 *           w_v the 32-bit Philox4x64-10 word for (seed, step0 + depth(i),
 *           pos0 + n, v) (key (seed, 0), counter (v>>3, pos, step, 0), word
 *           (v&7)>>1, low half for even v); key_v = fl32(fl32(l_v*invT) + g_v);
 *           token = lowest v attaining max key.  Branches at equal depth share
 *           the noise of a position.
 *   S = sum_v exp(l_v - max l) (fp64 decision); conf = fl32(1/S) (fp32 fast
 *   path, relative error below 1e-5).
 * Per branch, masked positions are ranked by S ascending (ties: lowest n).
 * The first is committed; after it, further positions in that order while
 * fewer than k_max are taken and fl32(1/S) >= tau, stopping at the first that
 * fails (SpecFold, evaluation setup, "Models and baselines": confidence-
 * threshold unmasking).  next_state[i][n] = token
 * for each committed n, else state[i][n]; commit_pos[i][0..k_max) = the
 * committed positions in rank order, -1 padded (all -1 when the branch has no
 * masked position).  With k_max = 1, tau is ignored.  Where the fp32 bound on
 * S leaves the ranking or a tau decision open, S is recomputed in fp64.
 *
 *   logits [M][V] fp32; rows [M] int32 = sfv_masked_rows(state) order
 *   state, next_state [B1][N] int32; parent_host [B1] host int32, parent[0] = -1
 *   commit_pos [B1][k_max] int32; token [M] int32; conf [M] fp32
 *   workspace: sfv_commit_workspace_bytes(B1, N, M, V) bytes
 * Supported: V % 8 == 0, V < 2^31 / 8, T >= 0 and finite, 1 <= k_max <= N,
 * tau finite when k_max > 1.
 */
int sfv_commit_workspace_bytes(int B1, int N, int M, int V, size_t* bytes);
int sfv_commit(const float* logits, const int32_t* rows, int M,
               const int32_t* state, const int32_t* parent_host,
               int B1, int N, int V, float temperature,
               uint64_t seed, uint64_t step0, int64_t pos0, int k_max, float tau,
               int32_t* next_state, int32_t* commit_pos, int32_t* token, float* conf,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * sfv_commit without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments (minus workspace and
 * workspace_bytes), checks and outputs as sfv_commit; it runs the same
 * kernels.  It calls no hipMalloc, hipFree or allocating library routine.
 *
 * The workspace is a static device array of SFV_COMMIT_SCRATCH_BYTES per GPU
 * that the library holds until the process ends; its address on a GPU is
 * looked up on the first call there.  A call whose workspace need (at most
 * sfv_commit_workspace_bytes(B1, N, M, V); about 0.2 MB at 33 branches x 64
 * positions with 1482 masked rows) exceeds it returns SFV_E_WORKSPACE before
 * launching anything.  Every call on one GPU uses that one array, and each
 * call writes what it reads, so nothing carries over between calls; but calls
 * whose executions overlap on one GPU (on different streams, or unordered
 * from several threads) race on it and give undefined results.  `stream`
 * must be NULL or a stream of the current device (else SFV_E_INVAL).
 */
#define SFV_COMMIT_SCRATCH_BYTES (1u << 20)
int sfv_commit_noalloc(const float* logits, const int32_t* rows, int M,
                       const int32_t* state, const int32_t* parent_host,
                       int B1, int N, int V, float temperature,
                       uint64_t seed, uint64_t step0, int64_t pos0, int k_max, float tau,
                       int32_t* next_state, int32_t* commit_pos, int32_t* token, float* conf,
                       void* stream);

/*
 * Greedy (T = 0) LM head and commit over tile partials: sfv_lm_head_greedy
 * then sfv_commit_greedy give the outputs of sfv_lm_head then sfv_commit at
 * temperature 0 (the same logits, tokens, committed positions and next
 * states; conf within the same fp32 fast-path bound), without a second pass
 * over the logits.  SpecFold, Appendix B (the head is a dense product over the
 * masked rows); SPOT, "Important context" (at T = 0 the commit is the greedy
 * argmax).
 *
 * sfv_lm_head_greedy: as sfv_lm_head (status included), and the kernel also reduces every
 * vocabulary tile of 256 ids of every row to its
 * max, the lowest id attaining it and a fast fp32 sum of exp(l - max) with a
 * bound on its error.
 *   partials: device buffer of sfv_lm_head_greedy_bytes(M, V, D) bytes,
 *   16-byte aligned, written whole (contents are internal to the pair).
 * sfv_commit_greedy: merges the partials of each row (fast factors within the
 * same bound, then fp64) and ranks, selects and writes exactly as sfv_commit
 * does at T = 0, recomputing S in fp64 from the logits wherever the bound
 * leaves the ranking or a tau decision open.
 *   partials, D: as written by sfv_lm_head_greedy for the same M, V, D;
 *   logits, rows, state, parent_host, outputs: as for sfv_commit;
 *   workspace: sfv_commit_greedy_workspace_bytes(B1, N, M, V) bytes.
 * Supported: M >= 33 and D % 64 == 0 (other shapes return
 * SFV_E_UNSUPPORTED), V % 8 == 0, V < 2^31 / 8, 1 <= k_max <= N, tau
 * finite when k_max > 1.
 */
int sfv_lm_head_greedy_bytes(int M, int V, int D, size_t* bytes);
int sfv_lm_head_greedy(const void* hidden, const int32_t* rows, int M, int R, const void* w, int D, int V,
                       float* logits, void* partials, size_t partials_bytes, int32_t* status, void* stream);
int sfv_commit_greedy_workspace_bytes(int B1, int N, int M, int V, size_t* bytes);
int sfv_commit_greedy(const void* partials, size_t partials_bytes, int D, const float* logits,
                      const int32_t* rows, int M, const int32_t* state, const int32_t* parent_host, int B1,
                      int N, int V, int k_max, float tau, int32_t* next_state, int32_t* commit_pos,
                      int32_t* token, float* conf, void* workspace, size_t workspace_bytes, void* stream);

/*
 * State-equality walk over the draft tree.  SpecFold, introduction (a later
 * main-branch state equal to a cached draft reuses its logits); SPOT, "How
 * does SPOT draft and verify?" (accept the longest prefix consistent with the
 * target's own trajectory).
 *
 * cur = 0; repeat at most B1-1 times: stop if commit_pos[cur][0] == -1;
 * j = lowest draft index >= 1 with depth(j) == depth(cur) + 1 and
 * state[j] == next_state[cur] (64-bit state hash, confirmed by full
 * comparison); stop if none; append j; cur = j.  depth() is the distance to
 * the root in parent_host.  Only the next tree level is searched because a
 * draft at depth d commits with the noise of step step0 + d (sfv_commit): a
 * draft at another depth would continue with another step's noise, and the
 * accepted run would no longer be the draft-free trajectory (SPOT, "Is the
 * output exact when the target samples?", Proposition 2).
 *   chain [B1] int32 out (-1 padded); n_accepted [1] int32 out (h)
 *   status [1] int32 out: SFV_OK, or SFV_E_STATE when S_max >= 0 and some
 *   draft changes or re-masks a parent position or unmasks more than S_max
 *   positions over its parent (then h = 0).  S_max < 0 skips that check.
 * A miss is not an error: h = 0.
 */
int sfv_match_tree(const int32_t* state, const int32_t* next_state, const int32_t* commit_pos,
                   const int32_t* parent_host, int B1, int N, int k_max, int S_max,
                   int32_t* chain, int32_t* n_accepted, int32_t* status, void* stream);

/*
 * Device self-check of the fast-path bounds the commit relies on.  Sweeps
 * every 32-bit noise word and every fp32 argument in [-126, 6] of the fast
 * exp2 and writes out[0] = max over all words of how far the exact Gumbel
 * value (fp64 logarithms, as the commit defines it) lies outside the bounds
 * of its bucket in the sweep's table (0: every word inside), and out[1] = max
 * relative error of the fast exp2 (fp64 reference on the device).
 *   out [2] fp64 device.  Synchronous on `stream`'s work only.
 */
int sfv_selfcheck_bounds(double* out, void* stream);

/*
 * The Gumbel noise value of noise words, as the commit's exact path computes
 * it: out[i] = fl32(-ln(-ln u)) with u = (w + 1/2) 2^-32, w = first + i, both
 * logarithms in fp64 (SPOT, "Is the output exact when the target samples?":
 * the drafter and the target must draw the same noise, Proposition 2).  For
 * checking the device's values against an independent implementation, word by
 * word.
 *   out [count] fp32 device, 4-byte aligned.  first + count <= 2^32, else
 *   SFV_E_INVAL.  count = 0 launches nothing.
 */
int sfv_gumbel_words(uint32_t first, uint32_t count, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SFV_H */
