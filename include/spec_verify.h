/*
 * spec_verify.h -- C ABI of libspecverify, batched draft-token verification
 * (speculative sampling) on AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are cited by page title and section):
 *   "Ling-3.0-flash-dspark" draft-model tutorial (mlqm.cn/news/1205650):
 *     sec. 3.1 -- the draft proposes gamma tokens; the target scores gamma+1
 *       positions in one pass; draft token i is accepted with probability
 *       min(1, p_i(x_i) / q_i(x_i)); the first rejection is replaced by a draw
 *       from norm(max(0, p - q)) and the later drafts are dropped; when every
 *       draft is accepted an extra token is drawn from the last target row.
 *     sec. 4.2 -- both distributions are softmax(logits / temperature) after
 *       the same top-p filter (_apply_top_p), p from the target rows, q from
 *       the draft rows.
 *     sec. 6.2 -- batching: every sequence keeps its own acceptance position.
 *     sec. 6.4 -- draft length 0 is a boundary case (bonus draw only).
 *   SSD inference-engine guide (lpnh.cn/news/2716086):
 *     sec. 6 -- an EAGLE3 draft head covers a reduced vocabulary that d2t maps
 *       into the target vocabulary; ids off the map have draft probability 0.
 *     sec. 7 -- temperature-0 runs: greedy verification.
 *   "基于1层Llama草稿模型实现2.16推测解码加速" (the 2.16x EAGLE blog):
 *     sec. 5 -- a draft tree (32 nodes, depth 5, top-k 8) verified by one target
 *       pass; the speed-up table's Match = True asks for output identical to
 *       the target's own greedy decoding.
 *
 * Readings fixed where the pages leave a step open:
 *   - Each sequence supplies its uniforms: u_accept[b, i] for the accept test
 *     of draft i and one u_sample[b] for whichever draw (replacement or bonus)
 *     happens.  The accept test is u * q < p (the q = 0 limit accepts iff p > 0).
 *   - Draws are inverse-CDF in ascending token id: the first id whose
 *     inclusive cumulative weight exceeds u * (total weight).
 *   - Top-p keeps sorted position s >= 1 iff the cumulative softmax of
 *     positions < s is <= top_p; equal logits are ordered by lower id first.
 *     top_p >= 1 switches the filter off.
 *   - Argmax ties go to the lowest id; -0 and +0 are equal.
 *   - Tree: the deepest accepted node wins, ties to the lowest node index.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, never synchronizes, and enqueues its kernels on
 *     `stream` only (0 = the null stream).  Outputs are written by the kernels;
 *     they are valid once the stream reaches that point.
 *   - Layouts are row-major and contiguous.  Logits rows may have any length
 *     and alignment (only element alignment is required).
 *   - Host-detectable argument errors return an sv_status != SV_OK with NO
 *     launch.  A failed launch returns SV_ERR_HIP.  No C++ exception crosses
 *     the ABI.
 *   - Device-detected per-sequence conditions are reported in out_status[b]
 *     (when out_status is not NULL) as SV_SEQ_* bits; the call still completes.
 *   - The workspace is caller memory of workspace_bytes >=
 *     sv_workspace_bytes_*() bytes that must be ZEROED ONCE when allocated.
 *     Its first part (a fixed fraction of workspace_bytes) holds per-sequence
 *     arrival counters that every call returns to zero; the rest holds
 *     scratch data.  So one workspace serves later calls of every entry point
 *     and every size on the same stream, provided each call passes the same
 *     workspace_bytes (zero it again before passing a different value).
 *     Calls that may run concurrently need separate workspaces.  After a
 *     call that failed on the device, zero the workspace again.
 *   - Inputs containing NaN are outside the contract; -inf logits (masked
 *     tokens) are allowed.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SV_OK = 0,
    SV_ERR_INVALID_ARG = 1,         /* a null pointer, a size out of range, a bad scalar  */
    SV_ERR_UNSUPPORTED_DTYPE = 2,   /* a dtype code other than SV_F32 / SV_BF16            */
    SV_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below sv_workspace_bytes_*()       */
    SV_ERR_HIP = 4,                 /* the HIP runtime reported an error at launch        */
    SV_ERR_TOO_LARGE = 5            /* a size beyond the library's documented limits      */
} sv_status;

typedef enum {
    SV_F32 = 0,    /* IEEE float32 */
    SV_BF16 = 1    /* bfloat16 (the high 16 bits of a float32) */
} sv_dtype;

/* out_status bits (per sequence). */
#define SV_SEQ_TOKEN_RANGE 1  /* a draft/node token id outside [0, V): treated as p = q = 0 (rejected / unmatched) */
#define SV_SEQ_D2T         2  /* sampling with d2t and gamma > 0: the map is not strictly increasing inside
                                 [0, Vt) (SSD guide sec. 6); set on every sequence, whose other outputs are
                                 then unspecified (tokens still lie in [-1, Vt))                              */
#define SV_SEQ_NO_MASS     4  /* a logits row whose maximum is not finite; draws from it return -1             */
#define SV_SEQ_BAD_PARENT  8  /* tree: parents[b][k] outside [0, k) for k >= 1; that node is never accepted     */

/* Limits.  Sizes beyond them return SV_ERR_TOO_LARGE. */
#define SV_MAX_GAMMA      255       /* draft tokens per sequence                     */
#define SV_MAX_TREE_NODES 4096      /* nodes per tree                                */
#define SV_MAX_VOCAB      (1 << 24) /* logits row length (target and draft)          */

/*
 * Workspace sizes in bytes for a call with these sizes (0 only for invalid sizes).
 * The result depends only on the arguments and never decreases as any size
 * argument grows (top_p held on the same side of 1), so a workspace sized for
 * the largest call serves every smaller one.  The same holds for every other
 * sv_workspace_bytes_*() below.
 */
size_t sv_workspace_bytes_sample(int32_t B, int32_t gamma, int32_t Vt, int32_t Vd, float top_p);
size_t sv_workspace_bytes_greedy(int32_t B, int32_t gamma, int32_t V);
size_t sv_workspace_bytes_tree(int32_t B, int32_t N, int32_t V);

/*
 * Sampling verification (Ling tutorial sec. 3.1 and sec. 4.2; SSD guide sec. 6
 * for d2t).
 *
 *   target_logits  [B, gamma+1, Vt] of target_dtype.  Row i (< gamma) is the
 *                  target's distribution for draft token i; row gamma is the
 *                  bonus position.
 *   draft_logits   [B, gamma, Vd] of draft_dtype.  May be NULL when gamma == 0.
 *   draft_tokens   [B, gamma] int32, TARGET-vocabulary ids.  May be NULL when gamma == 0.
 *   d2t            [Vd] int32, strictly increasing ids in [0, Vt): draft id j
 *                  is target id d2t[j].  NULL means Vd == Vt and the identity.
 *                  The kernels check the map on every call with gamma > 0: one
 *                  that is not strictly increasing or leaves [0, Vt) sets
 *                  SV_SEQ_D2T on every sequence (memory stays safe; the other
 *                  outputs are unspecified, tokens in [-1, Vt)).
 *   u_accept       [B, gamma] float32 in [0, 1).  May be NULL when gamma == 0.
 *   u_sample       [B] float32 in [0, 1).
 *   temperature    > 0 and finite (temperature 0 is spec_verify_greedy).
 *   top_p          in (0, 1) filters p and q alike; >= 1 switches top-p off.
 *   out_tokens     [B, gamma+1] int32: the accepted drafts, then the drawn
 *                  token, then -1 padding.
 *   out_accept_len [B] int32 in [0, gamma].
 *   out_p_tok, out_q_tok  [B, gamma] float32 or NULL: p_i(x_i) and q_i(x_i)
 *                  for every i < gamma (also past the first rejection).
 *   out_status     [B] int32 or NULL: SV_SEQ_* bits.
 *   workspace      >= sv_workspace_bytes_sample(B, gamma, Vt, Vd, top_p) bytes.
 * Errors: SV_ERR_INVALID_ARG (null required pointer, B < 0, gamma < 0, V < 1,
 * Vd != Vt without d2t, temperature <= 0 or not finite, top_p <= 0 or NaN),
 * SV_ERR_UNSUPPORTED_DTYPE, SV_ERR_TOO_LARGE, SV_ERR_WORKSPACE_TOO_SMALL,
 * SV_ERR_HIP.  B == 0 returns SV_OK without a launch.
 */
sv_status spec_verify_sample(
    const void *target_logits, sv_dtype target_dtype,
    const void *draft_logits, sv_dtype draft_dtype,
    const int32_t *draft_tokens, const int32_t *d2t,
    const float *u_accept, const float *u_sample,
    int32_t B, int32_t gamma, int32_t Vt, int32_t Vd,
    float temperature, float top_p,
    int32_t *out_tokens, int32_t *out_accept_len,
    float *out_p_tok, float *out_q_tok, int32_t *out_status,
    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Greedy (temperature 0) verification (SSD guide sec. 7; EAGLE blog table).
 *   target_logits  [B, gamma+1, V] of dtype; g_i = argmax of row i (lowest id on ties).
 *   draft_tokens   [B, gamma] int32.  May be NULL when gamma == 0.
 *   out_tokens     [B, gamma+1] int32: x_0..x_{n-1}, g_n, then -1 padding,
 *                  where n is the first i with x_i != g_i (gamma if none).
 *   out_accept_len [B] int32 = n.   out_status [B] int32 or NULL.
 *   workspace      >= sv_workspace_bytes_greedy(B, gamma, V) bytes.
 * Errors as for spec_verify_sample where they apply.
 */
sv_status spec_verify_greedy(
    const void *target_logits, sv_dtype dtype,
    const int32_t *draft_tokens, int32_t B, int32_t gamma, int32_t V,
    int32_t *out_tokens, int32_t *out_accept_len, int32_t *out_status,
    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Greedy tree verification (EAGLE blog sec. 5).
 *   target_logits  [B, N, V] of dtype; row k is the target's distribution
 *                  after node k (node 0 is the root, the last committed token).
 *   node_tokens    [B, N] int32; entry 0 (the root) is ignored.
 *   parents        [B, N] int32; parents[b][0] is ignored; 0 <= parents[b][k] < k.
 *   Node k is accepted iff its parent is accepted (the root always is) and
 *   node_tokens[b][k] equals the argmax of the parent's row.  The deepest
 *   accepted node wins (ties to the lowest index).
 *   out_path_nodes [B, N] int32: node indices of the root->winner path, root
 *                  excluded, then -1 padding.
 *   out_tokens     [B, N] int32: the path's tokens, then the argmax of the
 *                  winner's row (the bonus), then -1 padding.
 *   out_accept_len [B] int32: depth of the winner.   out_status [B] or NULL.
 *   workspace      >= sv_workspace_bytes_tree(B, N, V) bytes.
 * Errors as for spec_verify_sample where they apply; N must be >= 1.
 */
sv_status spec_verify_tree_greedy(
    const void *target_logits, sv_dtype dtype,
    const int32_t *node_tokens, const int32_t *parents,
    int32_t B, int32_t N, int32_t V,
    int32_t *out_path_nodes, int32_t *out_tokens, int32_t *out_accept_len,
    int32_t *out_status, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Draft-side sampler ("Ling-3.0-flash-dspark" tutorial sec. 4.2: the draft
 * loop of generate() -- logits / temperature, _apply_top_p, softmax,
 * multinomial; sec. 3.1: draft tokens by argmax or top-p/top-k).  One token
 * per row: p = softmax(logits[b] / temperature) over the first
 * min(top_k, k_p) positions of the stable order (logit descending, lower id
 * first), where k_p is the top-p count of spec_verify_sample's rule (top-p
 * and top-k cut the same order; the pages give no other rule for combining
 * them).  The token is the inverse-CDF draw in ascending id with u[b], the
 * rule of spec_verify_sample's draws.
 *   logits      [B, V] of dtype (row-major, any row alignment).
 *   d2t         [V] int32 or NULL: report draft id j as target id d2t[j]
 *               (SSD guide sec. 6); the entry is reported as it is.
 *   u           [B] float32 in [0, 1).
 *   temperature > 0 and finite.  top_p in (0, 1), >= 1 = off.
 *   top_k       <= 0 or >= V = off.
 *   out_tokens  [B] int32: the drawn id (through d2t), -1 for a row whose
 *               maximum is not finite.
 *   out_prob    [B] float32 or NULL: p of the drawn id (the draft
 *               probability q(x) that verification compares with).
 *   out_status  [B] int32 or NULL: SV_SEQ_NO_MASS.
 *   workspace   >= sv_workspace_bytes_draft(B, V) bytes, zeroed once when
 *               allocated, as for the other entry points.
 * Errors: SV_ERR_INVALID_ARG (null required pointer, B < 0, V < 1, a bad
 * temperature or top_p), SV_ERR_UNSUPPORTED_DTYPE, SV_ERR_TOO_LARGE
 * (V > SV_MAX_VOCAB), SV_ERR_WORKSPACE_TOO_SMALL, SV_ERR_HIP.
 */
size_t sv_workspace_bytes_draft(int32_t B, int32_t V);
sv_status spec_draft_sample(
    const void *logits, sv_dtype dtype, const int32_t *d2t, const float *u,
    int32_t B, int32_t V, float temperature, float top_p, int32_t top_k,
    int32_t *out_tokens, float *out_prob, int32_t *out_status,
    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Acceptance counters ("Ling-3.0-flash-dspark" tutorial sec. 4.2: the
 * statistics generate() returns -- total tokens, target calls, draft calls,
 * avg_acceptance_rate = accepted / (rounds * draft_length) and
 * speedup_estimate = tokens / target calls).  Adds one verification call's
 * out_accept_len [B] (draft length gamma) to counters [5] uint64 (device
 * memory, zeroed by the caller before the first call):
 *   counters[0] += target calls (one per sequence),
 *   counters[1] += drafts proposed (gamma per sequence),
 *   counters[2] += drafts accepted (sum of accept_len),
 *   counters[3] += tokens emitted (accept_len + 1 per sequence),
 *   counters[4] += entries outside [0, gamma] (which add to no other counter).
 * Acceptance rate = counters[2] / counters[1]; tokens per target call =
 * counters[3] / counters[0].  Integer sums: exact in any order.  Calls on
 * several streams may share counters (64-bit atomic adds).
 * Errors: SV_ERR_INVALID_ARG (B < 0, gamma < 0, null pointers, counters not
 * 8-byte aligned), SV_ERR_TOO_LARGE (gamma > SV_MAX_GAMMA), SV_ERR_HIP.
 */
sv_status spec_verify_count(const int32_t *accept_len, int32_t B, int32_t gamma, uint64_t *counters,
                            hipStream_t stream);

/*
 * SSD fan-out lookup (SSD guide sec. 1: while the target verifies, the draft
 * pre-speculates the possible verification outcomes and drafts every branch
 * at once; a branch that matches the outcome makes the next round's drafting
 * free.  sec. 7 runs it with a fan-out of 3).  After a verification call, the
 * outcome of sequence b is (n, t) = (accept_len[b], out_tokens[b, n]).
 *   out_tokens     [B, gamma+1] int32 and accept_len [B] int32: the outputs
 *                  of spec_verify_sample / spec_verify_greedy.
 *   cand           [B, gamma+1, f] int32: the f candidate tokens
 *                  pre-speculated for each accepted length n (-1 = empty).
 *   branch_drafts  [B, (gamma+1) * f, L] int32: the L tokens drafted ahead
 *                  for branch n * f + j.  May be NULL when out_next is.
 *   out_branch     [B] int32: n * f + j for the lowest slot j with
 *                  cand[b, n, j] == t, -1 when none matches or n is outside
 *                  [0, gamma] (a miss: the next round drafts anew).
 *   out_next       [B, L] int32 or NULL: the matching branch's drafts, -1 on
 *                  a miss.
 *   counters       [2] uint64 or NULL (device, zeroed by the caller once):
 *                  += lookups, += hits (64-bit atomic adds).
 * Limits: f <= SV_MAX_FANOUT, L <= SV_MAX_BRANCH_DRAFTS.  No workspace.
 * Errors: SV_ERR_INVALID_ARG (negative sizes, f < 1, null required
 * pointers, counters not 8-byte aligned), SV_ERR_TOO_LARGE, SV_ERR_HIP.
 */
#define SV_MAX_FANOUT        64
#define SV_MAX_BRANCH_DRAFTS 4096
sv_status spec_fanout_lookup(const int32_t *out_tokens, const int32_t *accept_len, const int32_t *cand,
                             const int32_t *branch_drafts, int32_t B, int32_t gamma, int32_t f, int32_t L,
                             int32_t *out_branch, int32_t *out_next, uint64_t *counters, hipStream_t stream);

/*
 * Vocabulary-trim d2t builder (the 2.16x EAGLE blog sec. 6: from corpus token
 * frequencies keep the core vocabulary whose cumulative probability reaches
 * P >= 0.95, so the draft head scores fewer ids; SSD guide sec. 6 maps them
 * back through d2t).  Ids of tokens[0..N) in [0, Vt) are counted (others are
 * invalid), ordered by count descending with lower ids first, and the
 * smallest prefix whose count sum reaches P * (valid tokens) is kept (in
 * float64 from the float32 P); ids of count 0 are never kept, so P >= 1 keeps
 * every observed id.
 *   tokens     [N] int32 (device).  N <= INT32_MAX.
 *   out_d2t    [Vt] int32: the kept ids in ascending order in its first
 *              *out_vd entries -- a map spec_verify_sample accepts.
 *   out_t2d    [Vt] int32 or NULL: the position of id t in d2t, -1 if not kept.
 *   out_vd     [1] int32: the number of kept ids (device memory).
 *   out_info   [3] int64 or NULL: kept count mass, valid tokens, invalid tokens.
 *   workspace  >= sv_workspace_bytes_vocab_trim(Vt) bytes, zeroed once when
 *              allocated (its totals and per-id overflow counts are returned
 *              to zero by every call).
 * Errors: SV_ERR_INVALID_ARG (N < 0, Vt < 1, P <= 0 or NaN, null required
 * pointers), SV_ERR_TOO_LARGE (Vt > SV_MAX_VOCAB or N > INT32_MAX),
 * SV_ERR_WORKSPACE_TOO_SMALL, SV_ERR_HIP.
 */
size_t sv_workspace_bytes_vocab_trim(int32_t Vt);
sv_status spec_vocab_trim(const int32_t *tokens, int64_t N, int32_t Vt, float P, int32_t *out_d2t,
                          int32_t *out_t2d, int32_t *out_vd, int64_t *out_info, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * Fused lm_head -> greedy verification (SSD guide sec. 6: compute_logits turns
 * the target's hidden states into logits; sec. 7: temperature-0 runs; the
 * 2.16x EAGLE blog sec. 6 ties the cost of this classification matmul to the
 * vocabulary).  logits[m][v] = sum_k hidden[m][k] * W[v][k] with bfloat16
 * inputs and float32 accumulation on the matrix cores; only each row's
 * argmax (largest logit, lowest id on ties) is kept -- the logits are never
 * written -- and the greedy chain (spec_verify_greedy) or tree walk
 * (spec_verify_tree_greedy) follows on those argmaxes.
 *   hidden        [B, R, d] bfloat16 (R = gamma + 1 for the chain, N for the
 *                 tree), 16-byte aligned, d a multiple of 8.
 *   W             [V, d] bfloat16, 16-byte aligned.
 *   out_argmax    [B * R] int32 or NULL: each row's argmax id.
 *   out_maxlogit  [B * R] float32 or NULL: each row's largest logit.
 *   The other arguments and outputs are those of spec_verify_greedy /
 *   spec_verify_tree_greedy.
 *   workspace     >= sv_workspace_bytes_lmhead(B * R, V) bytes.
 * Float32 accumulation can order two logits that are within its rounding
 * differently from exact arithmetic; such near-ties are the only way the
 * argmax can differ from that of exact logits.
 * Errors: SV_ERR_INVALID_ARG (null required pointer, B < 0, R < 1, d not a
 * positive multiple of 8, misaligned hidden or W, V < 1), SV_ERR_TOO_LARGE,
 * SV_ERR_WORKSPACE_TOO_SMALL, SV_ERR_HIP.
 */
size_t sv_workspace_bytes_lmhead(int32_t M, int32_t V);
sv_status spec_lmhead_verify_greedy(const void *hidden, const void *W, const int32_t *draft_tokens, int32_t B,
                                    int32_t gamma, int32_t d, int32_t V, int32_t *out_tokens, int32_t *out_accept_len,
                                    int32_t *out_argmax, float *out_maxlogit, int32_t *out_status, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);
sv_status spec_lmhead_verify_tree(const void *hidden, const void *W, const int32_t *node_tokens,
                                  const int32_t *parents, int32_t B, int32_t N, int32_t d, int32_t V,
                                  int32_t *out_path_nodes, int32_t *out_tokens, int32_t *out_accept_len,
                                  int32_t *out_argmax, float *out_maxlogit, int32_t *out_status, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * Sampling verification without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, outputs and results are those
 * of spec_verify_sample; the scratch is a static device array of
 * SV_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.
 *   - Set-up, on the first call on a device: the array's address is looked up
 *     and its counter region cleared by a small kernel on `stream`.  The call
 *     allocates nothing (no hipMalloc / hipFree) and never synchronizes.
 *   - Every call on one GPU shares that GPU's array and returns its counters
 *     to zero; calls that may overlap on one GPU (different streams, host
 *     threads) race and must be serialized by the caller.
 *   - A call whose sv_workspace_bytes_sample() exceeds
 *     SV_NOALLOC_SCRATCH_BYTES returns SV_ERR_TOO_LARGE with no launch (e.g.
 *     B = 128, gamma = 5, Vt = Vd = 151936 with top-p fits; B = 256 does not).
 * Errors: those of spec_verify_sample, SV_ERR_TOO_LARGE as above, SV_ERR_HIP
 * when the scratch address cannot be obtained.
 */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
sv_status spec_verify_sample_noalloc(
    const void *target_logits, sv_dtype target_dtype,
    const void *draft_logits, sv_dtype draft_dtype,
    const int32_t *draft_tokens, const int32_t *d2t,
    const float *u_accept, const float *u_sample,
    int32_t B, int32_t gamma, int32_t Vt, int32_t Vd,
    float temperature, float top_p,
    int32_t *out_tokens, int32_t *out_accept_len,
    float *out_p_tok, float *out_q_tok, int32_t *out_status,
    hipStream_t stream);

/* A static, human-readable name for a status code. */
const char *spec_verify_strerror(sv_status s);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
