/*
 * libddtree -- DDTree's per-round draft-tree hot path on AMD MI355X (gfx950).
 *
 * One decode round of block-diffusion speculative decoding with draft trees:
 *
 *   ddtree_topk         log-softmax + top-K of the drafter's per-position logits
 *   ddtree_build        best-first top-B prefix tree, node arrays, ancestor mask
 *   ddtree_tree_attn    ancestor-only GQA attention of the tree nodes (per layer)
 *   ddtree_target_argmax  the target's greedy token after every tree node
 *   ddtree_target_sample  the target's sampled token (temperature > 0)
 *   ddtree_budget_select  cost-aware node budget from the build's scores
 *   ddtree_accept_walk  greedy walk of the target's argmax down the tree
 *   ddtree_kv_compact   in-place gather of the accepted path's K/V rows
 *   ..._batched         the same for R requests in one call (a tree and a
 *                       prefix length per request)
 *
 * Sources (the web pages on DDTree; cited by page title and section):
 *   [DD]  "DDTree Deep Dive: Algorithm, Code, and Engineering Philosophy of
 *         Block Diffusion Draft Trees" (zhichai.net forum topic).
 *   [AH]  "DDTree: Turning Block Diffusion Drafters into Tree-Based Speculative
 *         Decoders" (alanhou.org blog summary).
 *   [AB]  "Qwen3-Coder-30B-A3B - DDTree vs DFlash vs autoregressive -
 *         single-stream (batch-1)" (autobench config page).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer is a DEVICE pointer unless its comment says "host".
 * - bf16 tensors are passed as uint16_t bit patterns (IEEE bfloat16).
 * - All arrays are dense row-major with the shapes given; the caller owns
 *   every buffer. The library allocates nothing and keeps no pointer after
 *   a call returns; its only state is a per-thread cache of the last
 *   attention launch plan (a pure function of the shapes and prefix
 *   lengths), so calls are re-entrant and thread-safe.
 * - Every call validates its arguments on the host first; on error it
 *   returns a non-zero ddtree_status and enqueues nothing. On success the
 *   work is enqueued on `stream` (may be 0 = null stream) and the call
 *   returns without synchronising; outputs are valid once the stream has
 *   reached that point. Kernel launch failures return DDTREE_ERR_HIP.
 * - Device-resident inputs (token ids, parents, counts) are trusted: they
 *   must satisfy the documented ranges; the host cannot check them.
 * - Vector loads need 16-byte aligned q/k/v/out pointers (checked).
 */
#ifndef DDTREE_H
#define DDTREE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ddtree_status {
  DDTREE_OK = 0,
  DDTREE_ERR_INVALID_ARGUMENT = 1,   /* a size, pointer or alignment is wrong */
  DDTREE_ERR_UNSUPPORTED = 2,        /* valid but outside what the kernels do */
  DDTREE_ERR_WORKSPACE_TOO_SMALL = 3,/* ws_bytes below the queried size        */
  DDTREE_ERR_HIP = 4                 /* a HIP launch or runtime call failed    */
} ddtree_status;

/* Element types of ddtree_target_argmax's logits. */
#define DDTREE_DTYPE_F32 0
#define DDTREE_DTYPE_BF16 1

/* Limits checked by the calls below. */
#define DDTREE_MAX_L 32        /* drafted block positions (the pages use 16) */
#define DDTREE_MAX_K 1024      /* top-K kept per position                    */
#define DDTREE_MAX_B 1024      /* node budget (the pages sweep 16..1024)     */
#define DDTREE_MAX_LK 32768    /* L * K: the whole top-K table sits in LDS   */
#define DDTREE_MAX_V 4194304   /* vocabulary (1024 chunks of 4096 logits)    */
#define DDTREE_MAX_REQ 64      /* requests in one batched call               */
#define DDTREE_NOALLOC_SCRATCH_BYTES (32u << 20) /* ddtree_tree_attn_noalloc's scratch */

/* Human-readable name of a status code (static string, never NULL). */
const char* ddtree_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int ddtree_version(void);

/* ------------------------------------------------------------------------
 * ddtree_topk -- fused log-softmax and top-K per drafted block position.
 *
 * Source: [DD] section 1 (one drafter pass gives a marginal q_i per block
 * position), section 2 Lemma 1 (only the top K = min(B, |V|) tokens of each
 * position matter); [AH] Key Concepts (node scores are sums of log-probs).
 *
 * logits      fp32 [L, row_stride]; row i holds V logits of block position i
 *             (0-based). Values must be finite. Rows are independent: for R
 *             requests pass their rows stacked (request r's block positions
 *             at rows r * L_req ... r * L_req + L_req - 1), and the output
 *             is the [R, L_req, K] table ddtree_build_batched reads.
 * row_stride  elements between rows, >= V.
 * L, V, K     1 <= L <= DDTREE_MAX_L * DDTREE_MAX_REQ, 1 <= V <= DDTREE_MAX_V,
 *             1 <= K <= min(V, DDTREE_MAX_K).
 * logp        out fp32 [L, K]: log q_i of the selected tokens, rank order.
 * token       out int32 [L, K]: their token ids.
 * ws/ws_bytes device scratch of at least ddtree_topk_workspace_bytes().
 *
 * Ranking is by logit, larger first; exact ties go to the smaller token id
 * (+0 and -0 are equal). logp = x - lse_i with lse_i = log sum_v exp x[i,v]
 * computed in fp32 (max-subtracted); |error| <= 1e-5 against fp64.
 * ---------------------------------------------------------------------- */
int ddtree_topk_workspace_bytes(int L, int V, int K, size_t* bytes /* host */);
int ddtree_topk(const float* logits, int64_t row_stride, int L, int V, int K,
                float* logp, int32_t* token, void* ws, size_t ws_bytes,
                hipStream_t stream);

/* ------------------------------------------------------------------------
 * ddtree_build -- best-first selection of the top-B prefixes and the tree.
 *
 * Source: [DD] section 2, Proposition 3 (max-heap over rank tuples; each pop
 * pushes the next sibling and the first child; pops exactly the top-B
 * prefixes, which by Proposition 2 form a prefix-closed optimal tree);
 * section 3 (tree encoded as position/parent pairs); section 4 and [AH] Key
 * Concepts (each node sees the root, its ancestors and itself).
 *
 * logp, token  fp32 / int32 [L, K], each row non-increasing in logp (the
 *              output of ddtree_topk); logp <= 0.
 * B            node budget, 1 <= B <= min(DDTREE_MAX_B, sum_{d=1..L} K^d);
 *              the tree has N = B + 1 nodes.
 * root_token   int32 device scalar: the round's bonus token (node 0).
 * parent       out int32 [N]: parent node, -1 for the root; parent[n] < n.
 * depth        out int32 [N]: 0 for the root, else 1..L.
 * node_token   out int32 [N]: node 0 = *root_token; node n at depth d with
 *              last rank r has token[(d-1)*K + r].
 * score        out fp32 [N] or NULL: 0 for the root, else the fp32
 *              left-to-right sum of logp along the rank tuple.
 * anc          out uint32 [N, mask_words]: bit j of row n (word j>>5, bit
 *              j&31) is set iff node j is n or an ancestor of n; other bits 0.
 * mask_words   >= ceil(N / 32).
 *
 * Nodes 1..B are the selected prefixes in pop order: higher score first;
 * equal scores by lexicographically smaller rank tuple (a proper prefix is
 * smaller). The result is unique and bit-exact. Runs as one workgroup.
 * ---------------------------------------------------------------------- */
int ddtree_build(const float* logp, const int32_t* token, int L, int K, int B,
                 const int32_t* root_token, int32_t* parent, int32_t* depth,
                 int32_t* node_token, float* score, uint32_t* anc,
                 int mask_words, hipStream_t stream);

/* ddtree_build_batched -- ddtree_build for R requests (one workgroup each),
 * 1 <= R <= DDTREE_MAX_REQ, all with the same L, K, B: logp and token are
 * [R, L, K], root_token [R], parent/depth/node_token/score [R, B + 1] and
 * anc [R, B + 1, mask_words]; request r's slices are exactly what
 * ddtree_build would produce from its own slices. */
int ddtree_build_batched(const float* logp, const int32_t* token, int L, int K, int B, int R,
                         const int32_t* root_token, int32_t* parent, int32_t* depth,
                         int32_t* node_token, float* score, uint32_t* anc, int mask_words,
                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * ddtree_tree_attn -- ancestor-only tree attention of one layer (GQA, bf16).
 *
 * Source: [DD] section 4 (a node attends to the cached past context, the
 * root, its ancestors and itself, never to other branches), section 10
 * (the verifier attention is Qwen3's grouped-query attention); [AH] Core
 * Mechanism (all nodes are verified in one target forward pass); [AB] (the
 * ancestor mask is why the verifier cannot use a plain causal kernel).
 *
 * q        bf16 [N, Hq, D]: node n's query for head h (RoPE already applied).
 * k, v     bf16 [Hkv, S_cap, D] each: rows [0, S) are the cached prefix,
 *          row S + m holds tree node m (m < N).
 * S        prefix length, >= 0; S + N <= S_cap.
 * N        tree nodes incl. the root, 1 <= N <= DDTREE_MAX_B + 1.
 * Hq, Hkv  Hq % Hkv == 0; query head h reads kv-head h / (Hq / Hkv).
 * D        64 or 128.
 * scale    softmax scale (typically 1/sqrt(D)).
 * anc      uint32 [N, mask_words] as produced by ddtree_build.
 * out      out bf16 [N, Hq, D]; must not alias q, k or v.
 * ws       scratch of at least ddtree_tree_attn_workspace_bytes() for this
 *          S or any larger prefix length: the query is non-decreasing in S,
 *          so a decode loop can size one workspace at its largest S.
 *          Holds no state between calls.
 *
 * Range: when the key range is split (S + N > 128), every element of V
 * must satisfy |v| <= 65504 (the fp16 range of the split outputs, which
 * are convex combinations of V rows); larger values may overflow to inf.
 *
 * out[n,h] = sum_j softmax_j(scale * q[n,h] . k[g,j]) v[g,j] over rows
 * j in [0,S) and j = S + m for every m set in anc[n]; fp32 accumulation and
 * online softmax, bf16 rounding of the softmax weights before the P.V
 * product; when the key range is split over workgroups, each split's
 * output is normalised by its own sum and kept in fp16 (2^-11 relative)
 * until the fp32 merge; output rounded to bf16 (to nearest even).
 * ---------------------------------------------------------------------- */
int ddtree_tree_attn_workspace_bytes(int N, int Hq, int Hkv, int D, int S,
                                     size_t* bytes /* host */);
int ddtree_tree_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int S, int S_cap, int N, int Hq, int Hkv, int D,
                     float scale, const uint32_t* anc, int mask_words,
                     uint16_t* out, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* ddtree_tree_attn_noalloc -- ddtree_tree_attn with no workspace argument and
 * no allocation, for callers that cannot allocate device memory or call
 * hipMalloc: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.
 *
 * Arguments, semantics and results are those of ddtree_tree_attn (same
 * kernels, same launch plan, bit-identical output). The split partials go
 * to a static device array of DDTREE_NOALLOC_SCRATCH_BYTES (32 MiB) that
 * the library holds on every GPU it runs on until the process ends; its
 * address is looked up once per device, on the first call that needs it
 * with that device current. `stream` must belong to the current device.
 * Returns DDTREE_ERR_WORKSPACE_TOO_SMALL (nothing enqueued) when the plan
 * needs more than the array, i.e. when ddtree_tree_attn would need a
 * workspace larger than 32 MiB for this shape and S.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (nothing in it needs clearing): calls that overlap on one GPU
 * (other streams, other threads) race and must be serialised by the
 * caller. */
int ddtree_tree_attn_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             int S, int S_cap, int N, int Hq, int Hkv, int D,
                             float scale, const uint32_t* anc, int mask_words,
                             uint16_t* out, hipStream_t stream);

/* ddtree_tree_attn_batched -- ddtree_tree_attn for R requests in one launch
 * (1 <= R <= DDTREE_MAX_REQ), each with its own tree and its own prefix
 * length; all share N, Hq, Hkv, D and S_cap.
 *
 * q, out      bf16 [R, N, Hq, D].
 * k, v        request r's [Hkv, S_cap, D] block starts kv_req_stride
 *             elements after request r - 1's (a multiple of 8, and at least
 *             Hkv * S_cap * D when R > 1); e.g. a cache laid out
 *             [R][layers][2][Hkv][S_cap][D] passes k = its layer's K block of
 *             request 0 and kv_req_stride = layers * 2 * Hkv * S_cap * D.
 * S           host int32 [R]: request r's prefix length, S[r] + N <= S_cap.
 * anc         uint32 [R, N, mask_words].
 * ws          scratch of at least ddtree_tree_attn_batched_workspace_bytes()
 *             for the same R, N, Hq, Hkv, D and prefix lengths at least
 *             S[r] each (the query is non-decreasing in every S[r]).
 * The key range of every request is cut into splits of one common length,
 * so the launch's workgroups follow the total work; request r's output
 * equals ddtree_tree_attn on its own slices. */
int ddtree_tree_attn_batched_workspace_bytes(int R, const int32_t* S /* host */, int N, int Hq,
                                             int Hkv, int D, size_t* bytes /* host */);
int ddtree_tree_attn_batched(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             int64_t kv_req_stride, int R, const int32_t* S /* host */,
                             int S_cap, int N, int Hq, int Hkv, int D, float scale,
                             const uint32_t* anc, int mask_words, uint16_t* out, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * ddtree_target_argmax -- the target's greedy choice after every tree node.
 *
 * Source: [DD] section 6 (the walk compares each node's drafted children
 * with the token the target picks after that node; at temperature 0 the
 * pick is the argmax of the target head's logits for the node); [AH] Core
 * Mechanism (one target pass scores every node).
 *
 * logits      [N, row_stride] elements of type `dtype` (DDTREE_DTYPE_F32:
 *             float; DDTREE_DTYPE_BF16: uint16_t bfloat16 bits); row n holds
 *             the V logits of node n. Aligned to the element size; NaN is
 *             not allowed (the result is then unspecified), -inf is.
 * row_stride  elements between rows, >= V.
 * N, V        1 <= N <= DDTREE_MAX_B + 1, 1 <= V <= DDTREE_MAX_V.
 * out         out int32 [N]: out[n] = the smallest v with logits[n][v] equal
 *             to the row's maximum, compared as fp32 (bf16 widens exactly;
 *             -0 equals +0). It is the target_argmax of ddtree_accept_walk.
 *
 * ws/ws_bytes device scratch of at least ddtree_target_argmax_workspace_bytes()
 *             bytes (N * S * 8 with S <= 32 chunks per row), 8-byte aligned;
 *             no state is kept in it between calls.
 *
 * One streaming pass over N * V elements, each row split over S workgroups
 * whose bests a second small kernel combines.
 * ---------------------------------------------------------------------- */
int ddtree_target_argmax_workspace_bytes(int dtype, int N, int V, size_t* bytes /* host */);
int ddtree_target_argmax(const void* logits, int dtype, int64_t row_stride, int N, int V,
                         int32_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * ddtree_target_sample -- the target's token per tree node at temperature > 0.
 *
 * Source: [DD] section 6 (the target samples its token at each node, the
 * walk descends into the child holding it, the first token with no such
 * child is the bonus; at temperature > 0 the usual speculative-sampling
 * rules keep the output distributed as the target's). The children of a
 * node are fixed drafts, for which that rule reduces to: draw the token from
 * the target and follow it, so ddtree_accept_walk run on these samples is
 * the temperature > 0 verification.
 *
 * Draws out[n] from softmax(logits[n] / temperature) by the Gumbel-max rule,
 * out[n] = argmax_v (logits[n][v] / T - ln(-ln u[n][v])), with the uniforms
 * from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011):
 *   key     = (seed mod 2^32, seed >> 32)
 *   counter = (v >> 2, n, offset mod 2^32, offset >> 32), output word v & 3
 *   u       = ((word >> 9) + 0.5) * 2^-23   (exact in fp32, inside (0, 1))
 * so a result is a pure function of (logits, T, seed, offset): pass a new
 * offset every round. For several requests pass their rows stacked (N is
 * then the total): row n's draws use counter word n, so every request's
 * nodes draw independent numbers. The key is formed in fp32 (in base 2, the same
 * argmax); it can pick differently from an exact evaluation only where two
 * tokens' keys are within fp32 rounding of each other.
 *
 * logits, dtype, row_stride, N, V  as for ddtree_target_argmax; -inf marks
 *             a token that is never drawn; each row needs a finite logit.
 *             |logit| * log2(e) / T must stay below 3e38.
 * temperature T > 0, with log2(e) / T a normal fp32 number.
 * seed, offset  the draw's Philox key and counter words (see above).
 * out         out int32 [N]: the sampled token per node; the target_argmax
 *             argument of ddtree_accept_walk.
 * ws/ws_bytes as for ddtree_target_argmax (same size query).
 *
 * One streaming pass over N * V elements plus one Philox block per four
 * tokens; ALU-bound at the 30B shape.
 * ---------------------------------------------------------------------- */
int ddtree_target_sample(const void* logits, int dtype, int64_t row_stride, int N, int V,
                         float temperature, uint64_t seed, uint64_t offset, int32_t* out,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * ddtree_budget_select -- the node budget with the most expected tokens per
 * unit of round time.
 *
 * Source: [DD] section 2, Proposition 1 (the expected accepted length of a
 * tree under the drafter's distribution is the sum of q(u) = exp(score(u))
 * over its nodes) and Propositions 2-3 (best-first pops are the top-B
 * prefixes, so the budget-B tree is the first B + 1 nodes of one build with
 * the largest budget, and its mask rows are unchanged); [AB] results and
 * notes (the budget has an optimum where verification cost outgrows the
 * acceptance gain; a cost-aware variant picks it).
 *
 * score     fp32 [B_max + 1] from ddtree_build (pop order, root first).
 * B_max     1 <= B_max <= DDTREE_MAX_B; B_min: 0 <= B_min <= B_max.
 * t0, t1    round time model t0 + t1 * (B + 1) (any unit), both finite,
 *           >= 0, not both 0.
 * expected  out fp32 [B_max + 1] or NULL: expected[B] = E[alpha] of the
 *           budget-B tree = sum_{n=1..B} exp(score[n]) (summed in fp64).
 * budget    out int32 [1]: the smallest B in [B_min, B_max] maximising
 *           (1 + expected[B]) / (t0 + t1 * (B + 1)) (fp64).
 * ---------------------------------------------------------------------- */
int ddtree_budget_select(const float* score, int B_max, int B_min, double t0, double t1,
                         float* expected, int32_t* budget, hipStream_t stream);

/* ------------------------------------------------------------------------
 * ddtree_tree_prune -- keep the budget-B' tree inside a built tree.
 *
 * Source: [DD] section 2, Propositions 2-3 (best-first pops come in score
 * order, so the budget-B' tree is the first B' + 1 nodes of a build with a
 * larger budget); [AB] results and notes (the budget optimum; the verifier
 * should spend work only on the nodes it keeps).
 *
 * budget     device int32 [1]: B', 0 <= B' (e.g. ddtree_budget_select's
 *            output); values >= N - 1 keep every node.
 * N          nodes of the built tree, 1 <= N <= DDTREE_MAX_B + 1.
 * parent     in/out int32 [N]: parent[n] = -1 for every n > B', so that
 *            ddtree_accept_walk never reaches them.
 * anc        in/out uint32 [N, mask_words]: rows of nodes n > B' cleared.
 * With the rows cleared, ddtree_tree_attn skips the query tiles that hold
 * only pruned nodes; the output rows of pruned nodes are unspecified. The
 * kept nodes' rows, parents and mask rows are those of a build with budget
 * B' (prefix-closed: every kept node's ancestors are kept), so the walk and
 * the kept outputs equal those of the budget-B' round.
 * ---------------------------------------------------------------------- */
int ddtree_tree_prune(const int32_t* budget, int N, int32_t* parent, uint32_t* anc,
                      int mask_words, hipStream_t stream);

/* ------------------------------------------------------------------------
 * ddtree_accept_walk -- greedy verification walk down the tree.
 *
 * Source: [DD] section 6 (walk state machine: follow the child whose token
 * matches the target's choice; the first unmatched target token becomes the
 * next bonus token); [AH] Core Mechanism (the longest matching path is
 * accepted).
 *
 * parent, node_token  int32 [N] from ddtree_build (parent[n] < n; sibling
 *                     tokens distinct).
 * target_argmax       int32 [N]: the target's greedy token after node n.
 * L                   tree depth bound (1..DDTREE_MAX_L).
 * acc                 out int32 [L + 1]: acc[0] = 0 (root), acc[1..a] the
 *                     accepted nodes root-to-leaf, acc[a+1..L] = -1.
 * n_acc               out int32 device scalar: a = accepted drafted tokens.
 * next_bonus          out int32 device scalar: target_argmax[acc[a]]; may be
 *                     passed as the next round's root_token.
 * ---------------------------------------------------------------------- */
int ddtree_accept_walk(const int32_t* parent, const int32_t* node_token, int N,
                       int L, const int32_t* target_argmax, int32_t* acc,
                       int32_t* n_acc, int32_t* next_bonus, hipStream_t stream);

/* ddtree_accept_walk_batched -- ddtree_accept_walk for R requests (one wave
 * each), 1 <= R <= DDTREE_MAX_REQ: parent, node_token and target are
 * [R, N], acc [R, L + 1], n_acc and next_bonus [R]. */
int ddtree_accept_walk_batched(const int32_t* parent, const int32_t* node_token, int N, int L,
                               int R, const int32_t* target, int32_t* acc, int32_t* n_acc,
                               int32_t* next_bonus, hipStream_t stream);

/* ------------------------------------------------------------------------
 * ddtree_kv_compact -- keep only the accepted path in the KV cache, in place.
 *
 * Source: [DD] section 5 (tree tokens are interleaved in the cache tail, so
 * the accepted rows are gathered in place; without it the cache grows by
 * the budget every round); [AB] (the in-place tail compaction is the
 * method's fair path).
 *
 * kv       bf16 [layers, 2, Hkv, S_cap, D]: every layer's K then V half.
 * S        prefix length of this round; rows S..S+N-1 hold the tree.
 * acc      int32 [L + 1] and n_acc (device scalar, 0..L) from the walk.
 *
 * For every layer, half and kv-head: row S + k <- row S + acc[k] for
 * k = 1..a (all reads happen before any write of a slice). Rows below S + 1
 * and from S + 1 + a on are untouched. The new cache length is S + 1 + a.
 * ---------------------------------------------------------------------- */
int ddtree_kv_compact(uint16_t* kv, int layers, int Hkv, int S_cap, int D,
                      int S, int N, int L, const int32_t* acc,
                      const int32_t* n_acc, hipStream_t stream);

/* ddtree_kv_compact_batched -- ddtree_kv_compact for R requests in one
 * launch, 1 <= R <= DDTREE_MAX_REQ: kv is [R][layers][2][Hkv][S_cap][D]
 * (16-byte aligned), S a host int32 [R] of prefix lengths (S[r] + N <=
 * S_cap), acc [R, L + 1] and n_acc [R] from ddtree_accept_walk_batched. */
int ddtree_kv_compact_batched(uint16_t* kv, int layers, int Hkv, int S_cap, int D, int R,
                              const int32_t* S /* host */, int N, int L, const int32_t* acc,
                              const int32_t* n_acc, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DDTREE_H */
