/*
 * medusa.h -- C ABI of libmedusa, the Medusa speculate-and-verify step on
 * AMD MI355X (gfx950).
 *
 * One verify step is, in order (every call enqueues on one HIP stream):
 *   medusa_heads               K Medusa heads: ResBlock, lm_head, top-k
 *                              (or medusa_heads_packed on weights packed
 *                              once by medusa_heads_pack: batch > 2)
 *   medusa_build_tree          candidate tree from a medusa_choices spec,
 *                              once per spec; then every step
 *   medusa_tree_candidates     this step's candidates and positions
 *                              (or medusa_heads_tree / medusa_lm_head_topk_tree:
 *                              the heads' top-k and this gather in one call)
 *   medusa_tree_attention      tree-masked attention over the KV prefix
 *   medusa_base_lm_head        base lm_head at the tree nodes -> logits
 *                              (or medusa_base_posterior: both fused)
 *   medusa_evaluate_posterior  greedy / typical acceptance, best path
 *                              (or medusa_evaluate_posterior_nucleus: top-p,
 *                              its draws from medusa_philox_uniforms)
 *   medusa_sample_typical      typical mode: the sampled next token
 *   medusa_commit_kv           gather the accepted rows into contiguous slots
 *
 * Conventions shared by every call
 *  - Tensor pointers are DEVICE memory owned by the caller.  The library
 *    never allocates, frees or synchronises, and keeps no state between
 *    calls.  Outputs are valid once the stream reaches the call.
 *  - `stream` is a hipStream_t (NULL = the default stream).
 *  - Every call validates its arguments on the host BEFORE any HIP call and
 *    returns a medusa_status synchronously; on a negative status nothing was
 *    enqueued.  MEDUSA_ERR_HIP means a launch failed; medusa_last_error()
 *    then holds the HIP message (per calling thread).
 *  - Tensor pointers must be 16-byte aligned (MEDUSA_ERR_ALIGN).  Layouts
 *    are dense row-major in the order given; no strides.
 *  - Supported sizes: batch B <= 16, heads K <= 8, topk <= 64, tree nodes
 *    T <= 256 (so at most 255 spec entries), head dim d in {64, 128}.
 *  - bf16 tensors are raw bf16 bit patterns (uint16); f32 tensors are IEEE
 *    float32.  Accumulation is always float32.
 *
 * Citations name the pages the operations come from:
 *  [API] "Medusa API参考：核心函数与类详解" (jsqmd.com)
 *  [NOTES] "Medusa — 让大模型自己同时猜好几个 token" (estelledc.github.io)
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MEDUSA_OK = 0,
  MEDUSA_ERR_NULL = -1,      /* a required pointer is NULL                  */
  MEDUSA_ERR_SHAPE = -2,     /* a size is outside the supported range       */
  MEDUSA_ERR_DTYPE = -3,     /* unknown or unsupported dtype                */
  MEDUSA_ERR_VALUE = -4,     /* a scalar argument is out of range           */
  MEDUSA_ERR_WORKSPACE = -5, /* workspace smaller than the *_workspace size */
  MEDUSA_ERR_HIP = -6,       /* a HIP launch failed (see medusa_last_error) */
  MEDUSA_ERR_ALIGN = -7,     /* a tensor pointer is not 16-byte aligned     */
  MEDUSA_ERR_ALIAS = -8      /* an output aliases an input it must not      */
} medusa_status;

typedef enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 } medusa_dtype;

/* Values of status[0] written on the device by medusa_build_tree.
 * status[1] holds the offending spec entry (or the leaf count for
 * MEDUSA_SPEC_TOO_MANY_PATHS), -1 when MEDUSA_SPEC_OK.  Entries are checked
 * in this order: for each entry (in the given order) padding, then empty,
 * then rank; then duplicates (the first entry repeating an earlier one);
 * then missing prefixes (the first entry lacking a proper prefix); then the
 * leaf count against p_max. */
enum {
  MEDUSA_SPEC_OK = 0,
  MEDUSA_SPEC_PADDING = 1,        /* a -1 followed by a rank            */
  MEDUSA_SPEC_EMPTY = 2,          /* an all -1 entry                    */
  MEDUSA_SPEC_RANK = 3,           /* a rank outside [0, topk)           */
  MEDUSA_SPEC_DUPLICATE = 4,      /* the same tuple twice               */
  MEDUSA_SPEC_PREFIX = 5,         /* a proper prefix is not an entry    */
  MEDUSA_SPEC_TOO_MANY_PATHS = 6  /* more leaves than p_max             */
};

/* ---------------------------------------------------------------------
 * Medusa heads.  [API] MedusaModelABC (medusa_head: residual blocks and
 * linear layers; MedusaConfig medusa_num_heads = 5, medusa_num_layers = 1);
 * [NOTES] 是什么 / 核心要点 (K parallel heads on the last hidden state,
 * each a one-layer MLP with a residual, head k proposing token t+k+1, the
 * per-head top-k forming the candidate tree).
 *
 * For every sequence b and head j:
 *   r[b][j]      = h[b] + SiLU(W1[j] h[b] + b1[j])           (float32)
 *   logits[b][j] = Wlm[j] r[b][j]                             (no bias)
 *   topk_ids[b][j][0..topk) = the topk largest logits, ordered by value
 *   descending, equal values (+0 and -0 included) by lower token id first.
 *   A NaN logit is never selected; slots left without a candidate (only
 *   possible with NaN logits) hold id -1 and value -inf.
 *
 * Layouts: hidden [B][H]; w1 [K][H][H] (out x in: row i makes output i);
 * b1 [K][H]; w_lm [K][V][H] (out x in); r [B][K][H] float32;
 * topk_ids int32 and topk_logits float32 [B][K][topk]; logits float32
 * [B][K][V].  `dtype` applies to hidden, w1, b1 and w_lm.  bf16 needs
 * H % 8 == 0, f32 needs H % 4 == 0; 1 <= topk <= min(64, V).
 *
 * Workspace: medusa_heads_workspace() bytes of device memory (per-wave
 * candidate lists, one arrival count per head, one row-pool counter per
 * head and, in medusa_heads, r).  Its first 2304 bytes (the counts) must be
 * zero before the first call that uses it (allocate it zeroed once); every
 * call leaves them zero again.  The rest needs no initialisation.
 * medusa_lm_head_topk streams the weights in one kernel on `stream`; each
 * wave leaves a sorted top-k list, and the merge of a head's lists (radix
 * selection on unique value/id keys) runs in the last workgroup of that
 * head to finish when they fit its 2048-key budget, in a second kernel
 * otherwise.  With that in-kernel merge and H > 2048 the last seventh of
 * each head's rows is handed out at run time in blocks of four rows.  Calls
 * that share a workspace must not run concurrently.
 * ------------------------------------------------------------------- */
size_t medusa_heads_workspace(int dtype, int B, int H, int V, int K, int topk);

/* ResBlock of every head: writes r (float32 [B][K][H]). */
int medusa_resblock(int dtype, int B, int H, int K,
                    const void* hidden, const void* w1, const void* b1,
                    float* r, void* stream);

/* lm_head of every head on a float32 r [B][K][H], with fused top-k.
 * logits_or_null: optional float32 [B][K][V] copy of every logit. */
int medusa_lm_head_topk(int dtype, int B, int H, int V, int K, int topk,
                        const float* r, const void* w_lm,
                        int32_t* topk_ids, float* topk_logits, float* logits_or_null,
                        void* ws, size_t ws_bytes, void* stream);

/* The same lm_head + top-k on head weights packed once by
 * medusa_heads_pack (bf16 only, H <= 65536): the skinny-GEMM kernel at any
 * batch (per head, r's hi/lo bf16 planes as 2B rows; every 128-entry
 * vocabulary block publishes each sequence's top-k, merged in a second
 * kernel).  From the packed layout one wave instruction reads 1 KB of
 * weights contiguously; meant for batch > 2, where the row-major call runs
 * the same GEMM on row-major weights.  Same outputs as medusa_lm_head_topk;
 * workspace: medusa_heads_workspace() bytes (it covers both calls). */
int medusa_lm_head_topk_packed(int dtype, int B, int H, int V, int K, int topk,
                               const float* r, const void* w_lm_packed,
                               int32_t* topk_ids, float* topk_logits, float* logits_or_null,
                               void* ws, size_t ws_bytes, void* stream);

/* Pack w_lm [K][V][H] (bf16) into w_packed: each head in the layout of
 * medusa_base_lm_head_pack, heads one after another.  Size:
 * medusa_heads_packed_bytes() (0 for invalid sizes).  The buffers must not
 * alias. */
size_t medusa_heads_packed_bytes(int K, int H, int V);
int medusa_heads_pack(int dtype, int K, int H, int V, const void* w_lm, void* w_packed, void* stream);

/* Both stages on packed weights (bf16 only, H <= 65536): w1_packed is
 * medusa_heads_pack(K, H, V = H) of W1 [K][H][H], w_lm_packed that of
 * w_lm [K][V][H].  The ResBlock products run on the skinny-GEMM kernel with
 * the reduction split into slices (float32 partial sums in the workspace),
 * a second kernel finishes r = h + SiLU(sum + b1) and its bf16 planes, then
 * the lm_head + top-k as medusa_lm_head_topk_packed.  Same outputs as
 * medusa_heads; workspace: medusa_heads_workspace() bytes. */
int medusa_heads_packed(int dtype, int B, int H, int V, int K, int topk, const void* hidden,
                        const void* w1_packed, const void* b1, const void* w_lm_packed,
                        int32_t* topk_ids, float* topk_logits, float* logits_or_null, float* r_or_null,
                        void* ws, size_t ws_bytes, void* stream);

/* Both stages.  r_or_null: optional float32 [B][K][H] output of the
 * ResBlocks (kept inside the workspace otherwise). */
int medusa_heads(int dtype, int B, int H, int V, int K, int topk,
                 const void* hidden, const void* w1, const void* b1, const void* w_lm,
                 int32_t* topk_ids, float* topk_logits, float* logits_or_null,
                 float* r_or_null, void* ws, size_t ws_bytes, void* stream);

/* medusa_heads without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, outputs, kernels and
 * results as medusa_heads; the workspace is instead a scratch array of
 * MEDUSA_HEADS_NOALLOC_SCRATCH_BYTES held by the library on each GPU it
 * runs on until the process ends.  The call itself allocates and frees
 * nothing.  A shape whose medusa_heads_workspace() exceeds that size
 * returns MEDUSA_ERR_WORKSPACE (before any HIP call).  The first call on a
 * device (the current device) looks the array up and enqueues a small
 * kernel on `stream` that zeroes its arrival counts; a failure there
 * returns MEDUSA_ERR_HIP.  Every call on one GPU shares that GPU's array
 * and leaves it holding the last call's lists: calls that overlap on one
 * GPU (concurrent streams, threads) race and must be serialised by the
 * caller. */
#define MEDUSA_HEADS_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int medusa_heads_noalloc(int dtype, int B, int H, int V, int K, int topk,
                         const void* hidden, const void* w1, const void* b1, const void* w_lm,
                         int32_t* topk_ids, float* topk_logits, float* logits_or_null,
                         float* r_or_null, void* stream);

/* ---------------------------------------------------------------------
 * Candidate tree.  [API] medusa_generate (medusa_choices),
 * generate_candidates (tree_indices, retrieve_indices), tree_decoding
 * (tree_candidates, medusa_position_ids); [NOTES] 核心要点 (prefix tree of
 * the per-head top-k) and 实践案例 案例 3 (the worked mask: P, A, B, X, Y,
 * X, Y with each continuation seeing only the prompt and its own branch).
 *
 * choices int32 [n_choices][K]: rank tuples (r1, ..., rd) padded with -1,
 * in any order; tuple (r1..rd) is the r1-th token of head 1 followed by the
 * r2-th token of head 2, etc.  T = n_choices + 1 nodes: node 0 is the root
 * (the base model's next token, root_token[b]); the others are the tuples
 * sorted by (length, lexicographic order).  One tree serves the whole
 * batch; candidates and positions are per sequence.
 *
 * Outputs:
 *   tree_candidates int32 [B][T]  token at each node
 *   tree_indices    int32 [T]     0 for the root, else 1+(depth-1)*topk+rank:
 *                                 index into [root, head-1 top-k, head-2 top-k, ...]
 *   parent, depth   int32 [T]     parent[0] = -1
 *   position_ids    int32 [B][T]  prefix_len[b] + depth
 *   tree_mask       uint8 [T][T]  1 where node j is an ancestor of node i or i
 *   retrieve        int32 [p_max][K+1]  leaf paths in ascending leaf order,
 *                                 root first, -1 padded; rows >= num_paths are -1
 *   num_paths       int32 [1]
 *   status          int32 [2]     see MEDUSA_SPEC_*
 * On a spec error the outputs describe the root alone (num_paths = 1,
 * retrieve row 0 = (0, -1, ...), identity mask, every node the root token,
 * depth 0), so later stages stay in bounds and accept nothing.
 * ------------------------------------------------------------------- */
int medusa_build_tree(int B, int K, int topk, int n_choices,
                      const int32_t* choices, const int32_t* topk_ids,
                      const int32_t* root_token, const int32_t* prefix_len,
                      int32_t* tree_candidates, int32_t* tree_indices,
                      int32_t* parent, int32_t* depth, int32_t* position_ids,
                      uint8_t* tree_mask, int32_t* retrieve, int32_t* num_paths,
                      int p_max, int32_t* status, void* stream);

/* The per-step half of the candidate tree.  [API] generate_candidates:
 * the tree's buffers (mask, tree_indices, retrieve paths, depths) depend
 * only on medusa_choices and are built once; each step only gathers the new
 * top-k through tree_indices and offsets the positions.  Given tree_indices
 * and depth from a medusa_build_tree call on the same spec, K and topk:
 *   tree_candidates[b][t] = [root_token[b], topk_ids[b][0][..], topk_ids[b][1][..], ...][tree_indices[t]]
 *   position_ids[b][t]    = prefix_len[b] + depth[t]
 * exactly the tree_candidates and position_ids medusa_build_tree writes for
 * these topk_ids, root_token and prefix_len.  An index outside
 * [0, 1 + K * topk) reads the root token.  int32 throughout; topk_ids
 * [B][K][topk]; outputs [B][T] must not alias each other or the inputs. */
int medusa_tree_candidates(int B, int T, int K, int topk, const int32_t* tree_indices, const int32_t* depth,
                           const int32_t* topk_ids, const int32_t* root_token, const int32_t* prefix_len,
                           int32_t* tree_candidates, int32_t* position_ids, void* stream);

/* medusa_lm_head_topk followed by medusa_tree_candidates, in one call (and
 * medusa_heads_tree below: medusa_heads followed by it).  [API]
 * generate_candidates: each step takes the heads' top-k and gathers the
 * tree's candidates through tree_indices.  Arguments as in the two calls
 * (topk_ids is both the heads' output and the gather's input; T, tree_indices,
 * depth, root_token, prefix_len, tree_candidates and position_ids as in
 * medusa_tree_candidates); outputs identical to the two calls in sequence.
 * Where the lm_head's top-k merge runs inside its kernel (bf16 at batch
 * <= 2), the merging workgroup of the last head to finish also does the
 * gather, so the step saves the gather's launch; otherwise the gather is a
 * launch of its own after the merge.  tree_candidates, position_ids and
 * topk_ids must not alias (MEDUSA_ERR_ALIAS).  Workspace:
 * medusa_heads_workspace() bytes; every call leaves its arrival counts at
 * zero, as medusa_heads does. */
int medusa_lm_head_topk_tree(int dtype, int B, int H, int V, int K, int topk,
                             const float* r, const void* w_lm,
                             int32_t* topk_ids, float* topk_logits, float* logits_or_null,
                             int T, const int32_t* tree_indices, const int32_t* depth,
                             const int32_t* root_token, const int32_t* prefix_len,
                             int32_t* tree_candidates, int32_t* position_ids,
                             void* ws, size_t ws_bytes, void* stream);
int medusa_heads_tree(int dtype, int B, int H, int V, int K, int topk,
                      const void* hidden, const void* w1, const void* b1, const void* w_lm,
                      int32_t* topk_ids, float* topk_logits, float* logits_or_null,
                      float* r_or_null, int T, const int32_t* tree_indices, const int32_t* depth,
                      const int32_t* root_token, const int32_t* prefix_len,
                      int32_t* tree_candidates, int32_t* position_ids,
                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Tree attention.  [NOTES] 核心要点 (tree attention verifies every
 * candidate in one forward) and 实践案例 案例 3 (ancestor-only mask);
 * [API] tree_decoding (the tree runs against past_key_values).
 *
 * For sequence b, head h and tree node i (L = prefix_len[b]):
 *   out[b][i][h] = softmax_m(scale * q[b][i][h] . K[m]) V[m]
 * over the prefix slots m in [0, L) and the tree slots L + j with
 * tree_mask[i][j] = 1.  The caller has written the tree's K/V at slots
 * L .. L+T-1 and applied position encoding (positions prefix_len + depth)
 * to q and the tree keys.  Slots past L+T are never read.
 *
 * Layouts: q, out [B][T][Hq][d]; k_cache, v_cache [B][Hq][max_slots][d]
 * (one layer; pass a layer's base pointer for a multi-layer cache);
 * tree_mask uint8 [T][T].  Requires L + T <= max_slots for every b (a larger
 * L is clamped to max_slots - T).  scale is usually 1/sqrt(d).
 * Workspace: medusa_tree_attention_workspace() bytes (no initialisation).
 * ------------------------------------------------------------------- */
size_t medusa_tree_attention_workspace(int dtype, int B, int T, int Hq, int d, int max_slots);

int medusa_tree_attention(int dtype, int B, int T, int Hq, int d, int max_slots,
                          const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* prefix_len, const uint8_t* tree_mask, float scale,
                          void* out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Acceptance.  [API] evaluate_posterior (temperature, posterior_threshold
 * = eps, posterior_alpha = delta; medusa_generate defaults 0.0, 0.09, 0.3);
 * [NOTES] 核心要点 (typical acceptance) and 实践案例 案例 1 (keep the
 * longest acceptable prefix from the root); 学到什么 (a verify step also
 * yields the base model's next token).
 *
 * logits float32 [B][T][V]: base logits at every tree node.
 * A candidate c with parent n is accepted when
 *   temperature == 0: tree_candidates[b][c] == argmax logits[b][n]
 *   temperature  > 0: p_n(x) > min(eps, delta * exp(-H(p_n))), where
 *                     p_n = softmax(logits[b][n] / temperature), x is c's
 *                     token and H the natural-log entropy.
 * A path's length is its count of accepted nodes from the root's child on,
 * stopping at the first reject or -1.  best_path = the lowest-index path of
 * maximal length, accept_len its length, next_token = argmax of the logits
 * at the path's last accepted node (ties: lowest token id).
 * retrieve [p_max][D] and num_paths come from medusa_build_tree (D = K+1).
 * Workspace: medusa_posterior_workspace() bytes (no initialisation).
 * ------------------------------------------------------------------- */
size_t medusa_posterior_workspace(int B, int T, int V);

int medusa_evaluate_posterior(int B, int T, int V, int p_max, int D,
                              const float* logits, const int32_t* tree_candidates,
                              const int32_t* retrieve, const int32_t* num_paths,
                              float temperature, float eps, float delta,
                              int32_t* best_path, int32_t* accept_len, int32_t* next_token,
                              void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Nucleus (top-p) acceptance.  [API] medusa_generate, generate_candidates
 * and evaluate_posterior take top_p (default 0.8) beside the sampling
 * mode; the pages define nothing further, and this call takes the plain
 * reading:
 *   p_n = softmax(logits[b][n] / temperature) (temperature > 0);
 *   the nucleus of node n is the shortest prefix of the vocabulary ordered
 *   by p_n descending (ties: lower token id first) whose mass reaches top_p;
 *   s_n = the token drawn from the nucleus with uniforms[b][n]: walking the
 *   nucleus in token-id order, the first token whose running mass exceeds
 *   u * (nucleus mass), u clamped to [0, 1] (if rounding leaves none, the
 *   nucleus's highest id).
 * A candidate c with parent n is accepted when tree_candidates[b][c] ==
 * s_n; best_path and accept_len as in medusa_evaluate_posterior, and
 * next_token = s at the path's last accepted node.  Each accepted token is
 * a draw from the base model's nucleus, so the tokens a step emits follow
 * nucleus sampling of the base model.
 *
 * logits float32 [B][T][V] (finite), V <= 262144; uniforms float32 [B][T]
 * (the caller's random numbers, one per node); samples int32 [B][T] (may be
 * NULL): every node's draw.  0 < top_p <= 1.  Workspace:
 * medusa_posterior_nucleus_workspace() bytes (no initialisation).
 * ------------------------------------------------------------------- */
size_t medusa_posterior_nucleus_workspace(int B, int T);

int medusa_evaluate_posterior_nucleus(int B, int T, int V, int p_max, int D,
                                      const float* logits, const int32_t* tree_candidates,
                                      const int32_t* retrieve, const int32_t* num_paths,
                                      float temperature, float top_p, const float* uniforms,
                                      int32_t* best_path, int32_t* accept_len, int32_t* next_token,
                                      int32_t* samples, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Random numbers and the sampled next token.  [API] medusa_generate and
 * generate_candidates (temperature, posterior_threshold, posterior_alpha,
 * top_p, sampling='typical'): with a positive temperature the tree's root
 * -- the base model's token after the last accepted one, which is also the
 * step's bonus token -- is drawn under the sampling mode, not taken as the
 * argmax.
 *
 * medusa_philox_uniforms: out[b][n] (float32 [B][T]) = the uniform of
 * (seed, step, b, n, purpose) in [0, 1): the top 24 bits of the first
 * output word of Philox4x64-10 (Salmon, Moraes, Dror and Shaw, SC 2011)
 * with counter (n, b, step, purpose) and key (seed, 0), times 2^-24 --
 * bit-identical on any machine.  Purpose 0 is the nucleus draw of each node
 * (the `uniforms` of medusa_evaluate_posterior_nucleus), purpose 1 the
 * typical-mode next token.  B <= 16, T <= 256, purpose >= 0.
 *
 * medusa_sample_typical: for each sequence b, n = retrieve[best_path[b]]
 * [accept_len[b]] (clamped into the tables; an entry outside [0, T) reads
 * node 0), p = softmax(logits[b][n] / temperature); the allowed tokens are
 * those with p(x) > min(eps, delta * exp(-H(p))) -- the typical acceptance
 * test -- and next_token[b] is drawn from them renormalised with the
 * purpose-1 uniform u of (seed, step, b, node 0): walking the allowed tokens
 * in id order, the first whose running mass exceeds u times their total.
 * Masses are e^(z - max) in fixed point with 40 fraction bits (exact sums);
 * the test p > threshold is taken in float32.  Requires temperature > 0,
 * eps > 0 and 0 < delta < 1 (the argmax is then always allowed), else
 * MEDUSA_ERR_VALUE.  Layouts as medusa_evaluate_posterior; best_path and
 * accept_len are that call's outputs.  For a plain (non-tree) draw pass
 * T = 1, a one-entry retrieve {0} (p_max = D = 1) and zero best_path and
 * accept_len.  One workgroup per sequence; no workspace.
 * ------------------------------------------------------------------- */
int medusa_philox_uniforms(uint64_t seed, uint64_t step, int purpose, int B, int T, float* out,
                           void* stream);

int medusa_sample_typical(int B, int T, int V, int p_max, int D, const float* logits,
                          const int32_t* retrieve, const int32_t* best_path, const int32_t* accept_len,
                          float temperature, float eps, float delta, uint64_t seed, uint64_t step,
                          int32_t* next_token, void* stream);

/* ---------------------------------------------------------------------
 * KV commit.  [API] tree_decoding (tree K/V appended to past_key_values);
 * [NOTES] 实践案例 案例 1 (only the accepted prefix is kept).
 *
 * For every layer, sequence b (L = prefix_len[b], path = retrieve[best_path[b]]),
 * head and both caches, slot L + j receives the row that was at slot
 * L + path[j] before the call, for j = 0 .. accept_len[b] (every source is
 * read before any destination is written).  new_prefix_len[b] =
 * L + accept_len[b] + 1.  Other slots are untouched.
 *
 * Layouts: k_cache, v_cache [n_layers][B][H][max_slots][d] (dtype sets the
 * element size), updated in place; retrieve [p_max][D].  new_prefix_len must
 * not alias prefix_len.  Rows whose source or destination would fall outside
 * the cache are skipped.
 * ------------------------------------------------------------------- */
int medusa_commit_kv(int dtype, int B, int n_layers, int H, int d, int max_slots,
                     void* k_cache, void* v_cache, const int32_t* prefix_len,
                     const int32_t* retrieve, int p_max, int D,
                     const int32_t* best_path, const int32_t* accept_len,
                     int32_t* new_prefix_len, void* stream);

/* ---------------------------------------------------------------------
 * Base lm_head over the tree nodes.  [API] tree_decoding (the base model's
 * logits at every tree node) and evaluate_posterior (which takes them).
 * The step that produces medusa_evaluate_posterior's `logits`.
 *
 * logits[m][v] = sum_k hidden[m][k] * W[v][k] for every m < M and v < V:
 * float32 accumulation of the bf16 products, no bias.  Rows m are the B*T
 * final hidden states of the tree nodes in node order.
 *
 * Layouts: hidden bf16 [M][H]; logits float32 [M][V].  W is bf16, out x in
 * (row v makes logit v), given either row-major [V][H] (w_packed = 0) or in
 * the packed layout written by medusa_base_lm_head_pack (w_packed = 1),
 * which streams faster.  dtype must be MEDUSA_BF16.  1 <= M <= 4096,
 * 8 <= H <= 65536 with H % 8 == 0, 1 <= V <= 2^24.  No workspace; one
 * kernel on `stream`.
 *
 * Packed layout (medusa_base_lm_head_packed_bytes(H, V) bytes): for tile
 * t = v / 16, k step s = k / 32 and lane l = 16 g + n, the 16 bytes
 * W[16 t + n][32 s + 8 g .. 32 s + 8 g + 7] sit at byte offset
 * ((s * P + t / 2) * 2 + t % 2) * 1024 + l * 16, with P = ceil(V / 32)
 * tile pairs (the tile count padded to an even number); entries past V or
 * H are zero.  k steps outermost: all workgroups stream one k range of the
 * whole matrix at a time.
 * The weights are static, so a caller packs them once.
 * medusa_base_lm_head_packed_bytes returns 0 for invalid sizes.
 * ------------------------------------------------------------------- */
size_t medusa_base_lm_head_packed_bytes(int H, int V);

int medusa_base_lm_head_pack(int dtype, int H, int V, const void* w_base, void* w_packed, void* stream);

int medusa_base_lm_head(int dtype, int M, int H, int V, const void* hidden, const void* w_base,
                        int w_packed, float* logits, void* stream);

/* The same product, y[m][v] = x[m] . W[v] (float32 out), for the base
 * model's other projections (QKV, O, gate/up, down: [API] tree_decoding runs
 * the whole base model over the tree), whose outputs can be too narrow to
 * fill the chip: with at most 64 rows and fewer than 128 blocks of 128
 * outputs, the reduction over H is split into slices (float32 partial sums
 * [S][M][V] in the workspace, summed by a second kernel in slice order, so
 * results are deterministic); otherwise it is medusa_base_lm_head.
 * w_packed: medusa_base_lm_head_pack layout (bf16 only).  Workspace:
 * medusa_linear_workspace(M, H, V) bytes (256 when no split is taken; no
 * initialisation); calls sharing it must not overlap. */
size_t medusa_linear_workspace(int M, int H, int V);
int medusa_linear(int dtype, int M, int H, int V, const void* x, const void* w_packed, float* y, void* ws,
                  size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Base lm_head fused with the acceptance test.  [API] tree_decoding
 * (base logits at every tree node) and evaluate_posterior.
 *
 * The result of medusa_base_lm_head followed by medusa_evaluate_posterior
 * (same arguments and readings; logits = hidden . W^T of the B*T node
 * rows), without the logits ever reaching memory: each block of 128
 * vocabulary entries leaves, per node, its maximum, first argmax and
 * (temperature > 0) the softmax sums of logits / temperature, plus the
 * logits of the tree candidates whose tokens it holds; a merge and the
 * path decision follow.  Three kernels on `stream`.
 *
 * hidden bf16 [B][T][H] (node order); W bf16 row-major or packed as in
 * medusa_base_lm_head (w_packed); tree_candidates [B][T], retrieve
 * [p_max][D], num_paths, temperature, eps, delta and the outputs as in
 * medusa_evaluate_posterior.  V <= 131072.  Workspace:
 * medusa_base_posterior_workspace() bytes (no initialisation; 0 for
 * invalid sizes).
 * ------------------------------------------------------------------- */
size_t medusa_base_posterior_workspace(int B, int T, int H, int V);

int medusa_base_posterior(int B, int T, int H, int V, int p_max, int D,
                          const void* hidden, const void* w_base, int w_packed,
                          const int32_t* tree_candidates, const int32_t* retrieve,
                          const int32_t* num_paths, float temperature, float eps, float delta,
                          int32_t* best_path, int32_t* accept_len, int32_t* next_token,
                          void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Base model forward pieces.  [API] tree_decoding runs the base model over
 * the tree tokens with the prefix's KV cache; [NOTES] 学到什么 (greedy
 * Medusa decoding keeps exactly what the base model would produce).  The
 * pages do not spell the base model out; these calls follow a LLaMA layer
 * (pre-norm RMSNorm, rotate-half RoPE, SwiGLU MLP), and its linear layers
 * are medusa_base_lm_head (float32 out = bf16 in . W^T).  Per layer:
 *   medusa_add_rmsnorm (x += previous block output; n = rmsnorm(x))
 *   medusa_base_lm_head (n . Wqkv^T) -> medusa_rope_qkv -> medusa_tree_attention
 *   medusa_base_lm_head (attn . Wo^T) -> medusa_add_rmsnorm
 *   medusa_base_lm_head (n . [Wgate; Wup]^T) -> medusa_silu_mul
 *   medusa_base_lm_head (. Wdown^T)
 *
 * medusa_embed: x [M][H] float32 = embed [V][H] bf16 rows of tokens [M]
 *   (int32); a token outside [0, V) gives a zero row.  H % 8 == 0.
 * medusa_add_rmsnorm: for each of M rows, x += y (y may be NULL: no add),
 *   then out = bf16(x / sqrt(mean(x^2) + eps) * gain); x, y float32 [M][H],
 *   gain bf16 [H], out bf16 [M][H].  x is updated in place.
 * medusa_rope_qkv: qkv float32 [B][T][3][heads][d] (q, k, v as one GEMM
 *   output row); positions int32 [B][T]; dims i and i + d/2 of every head of
 *   q and k are rotated by positions[b][t] * theta^(-2i/d) (x1 cos - x2 sin,
 *   x2 cos + x1 sin).  q -> bf16 [B][T][heads][d]; k and v -> bf16 cache
 *   slots prefix_len[b] + t of k_cache, v_cache [B][heads][max_slots][d]
 *   (slots outside [0, max_slots) are not written).  d even.
 * medusa_silu_mul: gate_up float32 [M][2I] (gate in columns [0, I), up in
 *   [I, 2I)) -> out bf16 [M][I] = silu(gate) * up.  I % 8 == 0.
 * ------------------------------------------------------------------- */
int medusa_embed(int M, int H, int V, const int32_t* tokens, const void* embed, float* x, void* stream);

int medusa_add_rmsnorm(int M, int H, float* x, const float* y, const void* gain, float eps, void* out,
                       void* stream);

int medusa_rope_qkv(int B, int T, int heads, int d, int max_slots, const float* qkv,
                    const int32_t* positions, const int32_t* prefix_len, float theta, void* q,
                    void* k_cache, void* v_cache, void* stream);

int medusa_silu_mul(int M, int I, const float* gate_up, void* out, void* stream);

/* Text for a medusa_status value. */
const char* medusa_status_string(int status);
/* Detail of the last failing call on this thread ("" if none). */
const char* medusa_last_error(void);
/* ABI version of this header (major * 100 + minor). */
int medusa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MEDUSA_H */
