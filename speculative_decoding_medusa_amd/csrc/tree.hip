// Candidate tree from a medusa_choices spec, in one workgroup.
//
// Thread e owns spec entry e.  Each valid tuple (r1..rl) is packed into one
// 64-bit key: the length in bits 60..63, then r_m + 1 in 7-bit fields from
// bit 60 downwards, zeros after the last rank.  Unsigned key order is then
// the node order (length, then lexicographic), equal keys are equal tuples,
// and a key of length m is a proper prefix of another exactly when it is
// shorter and agrees on the top 4 + 7m bits below the length field.  One
// pass of every entry over all keys yields its duplicate flag, which prefix
// lengths are present, its node rank and its parent's entry.  The spec is
// validated in the documented order with one atomicMin over (phase, entry,
// kind) keys.  Work is O(N) per thread for N <= 255 entries.
#include "common.hpp"

namespace medusa {

constexpr int kTreeThreads = 256;
constexpr int kMaxDepth = kMaxHeads;
constexpr int kRankBits = 7;
constexpr uint64_t kRanksMask = (1ull << 60) - 1;

// bits of the first m ranks of a key (m <= 8)
__device__ __forceinline__ uint64_t rank_field_mask(int m) {
  const int sh = 60 - kRankBits * m;
  return (kRanksMask >> sh) << sh;
}

__global__ __launch_bounds__(kTreeThreads) void build_tree_kernel(
    int B, int K, int topk, int N, int p_max, const int32_t* __restrict__ choices,
    const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ root_token,
    const int32_t* __restrict__ prefix_len, int32_t* __restrict__ tree_candidates,
    int32_t* __restrict__ tree_indices, int32_t* __restrict__ parent_out, int32_t* __restrict__ depth_out,
    int32_t* __restrict__ position_ids, uint8_t* __restrict__ tree_mask, int32_t* __restrict__ retrieve,
    int32_t* __restrict__ num_paths, int32_t* __restrict__ status) {
  __shared__ uint64_t skey[kMaxNodes];           // by entry
  __shared__ int16_t node_of[kMaxNodes];         // entry -> node
  __shared__ int16_t par[kMaxNodes];             // by node
  __shared__ int8_t dep[kMaxNodes];
  __shared__ uint8_t has_child[kMaxNodes];
  __shared__ int16_t leaf_at[kMaxNodes];         // path -> leaf node
  __shared__ uint64_t anc[kMaxNodes][kMaxNodes / 64];
  __shared__ int wave_leaves[kTreeThreads / kWave];
  __shared__ int err_key;
  __shared__ int s_ids[kMaxBatch * kMaxHeads * kMaxTopk];   // topk_ids [B][K][topk]
  __shared__ int s_root[kMaxBatch], s_plen[kMaxBatch];
  __shared__ uint32_t s_pfound[kTreeThreads];   // key-pass partials (bit 31: duplicate)
  __shared__ int s_prank[kTreeThreads];
  __shared__ int16_t s_ppe[kTreeThreads];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int T = N + 1;
  const int D = K + 1;
  const int NONE = 0x7fffffff;

  // Inputs first, all independent loads in one round trip: the entry's row,
  // and into LDS the whole top-k table, the root tokens and the prefix
  // lengths (clamped indices, masked at use); every later read is LDS.
  int row[kMaxDepth];
  const int e_row = min(tid, max(N - 1, 0));
#pragma unroll
  for (int m = 0; m < kMaxDepth; ++m) row[m] = N > 0 ? choices[static_cast<size_t>(e_row) * K + min(m, K - 1)] : -1;
  const int n_ids = B * K * topk;
  for (int x0 = 0; x0 < n_ids; x0 += kTreeThreads * 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = topk_ids[min(x0 + u * kTreeThreads + tid, n_ids - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (x0 + u * kTreeThreads + tid < n_ids) s_ids[x0 + u * kTreeThreads + tid] = v[u];
  }
  if (tid < B) {
    s_root[tid] = root_token[tid];
    s_plen[tid] = prefix_len[tid];
  }
  if (tid == 0) err_key = NONE;
  has_child[tid] = 0;

  // phase 0: per-entry format (padding, then empty, then rank) and the key
  const bool is_entry = tid < N;
  int l = 0;
  uint64_t key = 0;
  int my_err = 0;
  {
    int n = 0;
#pragma unroll
    for (int m = 0; m < kMaxDepth; ++m)
      if (m < K && row[m] != -1) n = m + 1;  // length after trimming trailing -1
    bool pad = false, bad = false;
#pragma unroll
    for (int m = 0; m < kMaxDepth; ++m) {
      if (m < n) {
        if (row[m] == -1) pad = true;
        else if (row[m] < 0 || row[m] >= topk) bad = true;
        else key |= static_cast<uint64_t>(row[m] + 1) << (60 - kRankBits * (m + 1));
      }
    }
    l = n;
    key |= static_cast<uint64_t>(n) << 60;
    my_err = pad ? MEDUSA_SPEC_PADDING : (n == 0 ? MEDUSA_SPEC_EMPTY : (bad ? MEDUSA_SPEC_RANK : 0));
  }
  if (is_entry) skey[tid] = key;
  __syncthreads();
  if (is_entry && my_err) atomicMin(&err_key, (0 << 24) | (tid << 8) | my_err);

  // One pass over every key, for entry q: duplicates before q, the prefix
  // lengths present, q's rank in node order, q's parent's entry.  For small
  // specs the keys are split over P threads per entry (thread t scans part
  // t / EPP of the keys for entry t % EPP) and the partials are combined.
  const int P = N <= 64 ? 4 : (N <= 128 ? 2 : 1);
  const int EPP = kTreeThreads / P;
  const int q_ent = tid % EPP, part = tid / EPP;
  const int span = (N + P - 1) / P;
  const int e_lo = part * span, e_hi = min(N, e_lo + span);
  bool dup_p = false;
  uint32_t found_p = 0;
  int rank_p = 0, pe_p = -1;
  if (q_ent < N) {
    const uint64_t qk = skey[q_ent];
    const int ql = static_cast<int>(qk >> 60);
    int e = e_lo;
    for (; e + 4 <= e_hi; e += 4) {
      uint64_t ke[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) ke[u] = skey[e + u];
      // branch-free (bitwise & on the conditions, no short circuits)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int le = static_cast<int>(ke[u] >> 60);
        const bool pre = (le >= 1) & (le < ql) & (((ke[u] ^ qk) & rank_field_mask(le)) == 0);
        dup_p |= (e + u < q_ent) & (ke[u] == qk);
        found_p |= static_cast<uint32_t>(pre) << le;
        pe_p = (pre & (le == ql - 1)) ? e + u : pe_p;
        rank_p += static_cast<int>(ke[u] < qk);
      }
    }
    for (; e < e_hi; ++e) {
      const uint64_t k1 = skey[e];
      const int le = static_cast<int>(k1 >> 60);
      const bool pre = (le >= 1) & (le < ql) & (((k1 ^ qk) & rank_field_mask(le)) == 0);
      dup_p |= (e < q_ent) & (k1 == qk);
      found_p |= static_cast<uint32_t>(pre) << le;
      pe_p = (pre & (le == ql - 1)) ? e : pe_p;
      rank_p += static_cast<int>(k1 < qk);
    }
  }
  s_pfound[tid] = found_p | (static_cast<uint32_t>(dup_p) << 31);
  s_prank[tid] = rank_p;
  s_ppe[tid] = static_cast<int16_t>(pe_p);
  __syncthreads();
  bool dup = false;
  uint32_t found = 0;
  int rank = 0, pe = -1;
  if (is_entry) {
    for (int pp = 0; pp < P; ++pp) {
      const int x = pp * EPP + tid;
      found |= s_pfound[x];
      rank += s_prank[x];
      pe = max(pe, static_cast<int>(s_ppe[x]));
    }
    dup = (found >> 31) != 0;
    found &= 0x7fffffffu;
    const uint32_t want = (1u << l) - 2u;  // lengths 1 .. l-1
    if (dup) atomicMin(&err_key, (1 << 24) | (tid << 8) | MEDUSA_SPEC_DUPLICATE);
    else if ((found & want) != want) atomicMin(&err_key, (2 << 24) | (tid << 8) | MEDUSA_SPEC_PREFIX);
    node_of[tid] = static_cast<int16_t>(rank + 1);
  }
  __syncthreads();
  bool ok = err_key == NONE;

  // structure in LDS first; global outputs are written once, at the end,
  // after the leaf count is checked against p_max
  int last = 0;
#pragma unroll
  for (int m = 0; m < kMaxDepth; ++m)
    if (m == l - 1) last = row[m];
  const int node = rank + 1;
  if (ok) {
    if (is_entry) {
      const int pnode = l == 1 ? 0 : node_of[pe];
      par[node] = static_cast<int16_t>(pnode);
      dep[node] = static_cast<int8_t>(l);
      has_child[pnode] = 1;
    }
    if (tid == 0) {
      par[0] = -1;
      dep[0] = 0;
    }
  }
  __syncthreads();

  // ancestors (a walk of at most K parents) and leaf numbering by ballot;
  // an invalid spec leaves the root alone (every later stage stays in
  // bounds and accepts nothing)
  const bool is_node = tid < T;
  if (is_node) {
    uint64_t w[kMaxNodes / 64] = {0, 0, 0, 0};
    int a = tid;
    while (ok && a >= 0) {
      w[a >> 6] |= 1ull << (a & 63);
      a = par[a];
    }
    if (!ok) w[tid >> 6] = 1ull << (tid & 63);
#pragma unroll
    for (int q = 0; q < kMaxNodes / 64; ++q) anc[tid][q] = w[q];
  }
  const bool leaf = is_node && (ok ? !has_child[tid] : tid == 0);
  const uint64_t lm = ballot(leaf);
  if (lane == 0) wave_leaves[wave] = __popcll(lm);
  __syncthreads();
  int before = __popcll(lm & ((1ull << lane) - 1));
  int total = 0;
#pragma unroll
  for (int w = 0; w < kTreeThreads / kWave; ++w) {
    before += w < wave ? wave_leaves[w] : 0;
    total += wave_leaves[w];
  }
  if (ok && total > p_max) {
    // too many paths: the root alone as well
    ok = false;
    if (tid == 0) err_key = (3 << 24) | ((total & 0xffff) << 8) | MEDUSA_SPEC_TOO_MANY_PATHS;
    if (is_node) {
#pragma unroll
      for (int q = 0; q < kMaxNodes / 64; ++q) anc[tid][q] = q == (tid >> 6) ? 1ull << (tid & 63) : 0;
    }
    total = 1;
    if (tid == 0) leaf_at[0] = 0;
  } else if (leaf) {
    leaf_at[before] = static_cast<int16_t>(tid);
  }
  if (!ok && is_node) {
    par[tid] = -1;
    dep[tid] = 0;
  }
  __syncthreads();

  // per-node outputs: the entry's thread writes its node, thread 0 the root
  // (or every thread its own node when only the root is kept)
  if (ok && is_entry) {
    tree_indices[node] = 1 + (l - 1) * topk + last;
    parent_out[node] = par[node];
    depth_out[node] = l;
    for (int b = 0; b < B; ++b) {
      tree_candidates[static_cast<size_t>(b) * T + node] = s_ids[(b * K + (l - 1)) * topk + last];
      position_ids[static_cast<size_t>(b) * T + node] = s_plen[b] + l;
    }
  }
  if ((ok && tid == 0) || (!ok && is_node)) {
    tree_indices[tid] = 0;
    parent_out[tid] = -1;
    depth_out[tid] = 0;
    for (int b = 0; b < B; ++b) {
      tree_candidates[static_cast<size_t>(b) * T + tid] = s_root[b];
      position_ids[static_cast<size_t>(b) * T + tid] = s_plen[b];
    }
  }
  // mask rows over the flat [T][T] byte array, four bytes per store
  const int nbytes = T * T;
  uint32_t* mask_words = reinterpret_cast<uint32_t*>(tree_mask);
  for (int w = tid; w * 4 < nbytes; w += kTreeThreads) {
    uint32_t word = 0;
    int i = (4 * w) / T, jj = 4 * w - i * T;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (4 * w + c < nbytes) word |= static_cast<uint32_t>((anc[i][jj >> 6] >> (jj & 63)) & 1ull) << (8 * c);
      if (++jj == T) { jj = 0; ++i; }
    }
    if (4 * w + 4 <= nbytes) {
      mask_words[w] = word;
    } else {
      for (int c = 0; 4 * w + c < nbytes; ++c) tree_mask[4 * w + c] = static_cast<uint8_t>(word >> (8 * c));
    }
  }
  // retrieve[p][j]: the depth-j node on leaf p's path; -1 past the leaf
  // and on rows >= num_paths
  for (int x = tid; x < p_max * D; x += kTreeThreads) {
    const int p = x / D, j = x - p * D;
    int v = -1;
    if (p < total) {
      int a = leaf_at[p];
      const int da = dep[a];
      if (j <= da) {
        for (int s2 = da; s2 > j; --s2) a = par[a];
        v = a;
      }
    }
    retrieve[x] = v;
  }
  if (tid == 0) {
    *num_paths = total;
    const int k2 = err_key;
    status[0] = k2 == NONE ? MEDUSA_SPEC_OK : (k2 & 0xff);
    status[1] = k2 == NONE ? -1 : ((k2 >> 8) & 0xffff);
  }
}

// The per-step gather: one thread per (sequence, node).  Node t's token is
// entry tree_indices[t] of [root, head-1 top-k, head-2 top-k, ...]; indices
// outside that range read the root.
__global__ __launch_bounds__(256) void tree_candidates_kernel(int B, int T, int K, int topk,
                                                              const int32_t* __restrict__ tree_indices,
                                                              const int32_t* __restrict__ depth,
                                                              const int32_t* __restrict__ topk_ids,
                                                              const int32_t* __restrict__ root_token,
                                                              const int32_t* __restrict__ prefix_len,
                                                              int32_t* __restrict__ tree_candidates,
                                                              int32_t* __restrict__ position_ids) {
  const int x = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
  if (x >= B * T) return;
  const int b = x / T, t = x - b * T;
  const int ti = tree_indices[t];
  const int dp = depth[t];
  const int root = root_token[b];
  const int L = prefix_len[b];
  const bool in = ti >= 1 && ti <= K * topk;
  const int tok = in ? topk_ids[static_cast<size_t>(b) * K * topk + (ti - 1)] : root;
  tree_candidates[x] = tok;
  position_ids[x] = L + dp;
}

}  // namespace medusa

extern "C" int medusa_tree_candidates(int B, int T, int K, int topk, const int32_t* tree_indices,
                                      const int32_t* depth, const int32_t* topk_ids, const int32_t* root_token,
                                      const int32_t* prefix_len, int32_t* tree_candidates, int32_t* position_ids,
                                      void* stream) {
  using namespace medusa;
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d", __func__, B);
  MEDUSA_REQUIRE(T >= 1 && T <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: T=%d", __func__, T);
  MEDUSA_REQUIRE(K >= 1 && K <= kMaxHeads, MEDUSA_ERR_SHAPE, "%s: K=%d", __func__, K);
  MEDUSA_REQUIRE(topk >= 1 && topk <= kMaxTopk, MEDUSA_ERR_SHAPE, "%s: topk=%d", __func__, topk);
  MEDUSA_REQUIRE_PTR(tree_indices);
  MEDUSA_REQUIRE_PTR(depth);
  MEDUSA_REQUIRE_PTR(topk_ids);
  MEDUSA_REQUIRE_PTR(root_token);
  MEDUSA_REQUIRE_PTR(prefix_len);
  MEDUSA_REQUIRE_PTR(tree_candidates);
  MEDUSA_REQUIRE_PTR(position_ids);
  MEDUSA_REQUIRE(tree_candidates != position_ids, MEDUSA_ERR_ALIAS, "%s: outputs must not alias", __func__);
  const TreeGather tg{T, tree_indices, depth, root_token, prefix_len, tree_candidates, position_ids};
  return medusa_host::launch_tree_candidates(B, K, topk, topk_ids, tg, static_cast<hipStream_t>(stream));
}

int medusa_host::launch_tree_candidates(int B, int K, int topk, const int32_t* topk_ids,
                                        const medusa::TreeGather& tg, hipStream_t st) {
  using namespace medusa;
  hipLaunchKernelGGL(tree_candidates_kernel, dim3(static_cast<unsigned>((B * tg.T + 255) / 256)), dim3(256), 0, st,
                     B, tg.T, K, topk, tg.tree_indices, tg.depth, topk_ids, tg.root_token, tg.prefix_len,
                     tg.tree_candidates, tg.position_ids);
  return medusa_host::hip_check("medusa_tree_candidates launch");
}

extern "C" int medusa_build_tree(int B, int K, int topk, int n_choices, const int32_t* choices,
                                 const int32_t* topk_ids, const int32_t* root_token,
                                 const int32_t* prefix_len, int32_t* tree_candidates,
                                 int32_t* tree_indices, int32_t* parent, int32_t* depth,
                                 int32_t* position_ids, uint8_t* tree_mask, int32_t* retrieve,
                                 int32_t* num_paths, int p_max, int32_t* status, void* stream) {
  using namespace medusa;
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d", __func__, B);
  MEDUSA_REQUIRE(K >= 1 && K <= kMaxHeads, MEDUSA_ERR_SHAPE, "%s: K=%d", __func__, K);
  MEDUSA_REQUIRE(topk >= 1 && topk <= kMaxTopk, MEDUSA_ERR_SHAPE, "%s: topk=%d", __func__, topk);
  MEDUSA_REQUIRE(n_choices >= 0 && n_choices <= kMaxNodes - 1, MEDUSA_ERR_SHAPE,
                 "%s: n_choices=%d not in [0, %d]", __func__, n_choices, kMaxNodes - 1);
  MEDUSA_REQUIRE(p_max >= 1 && p_max <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: p_max=%d", __func__, p_max);
  if (n_choices > 0) MEDUSA_REQUIRE_PTR(choices);
  MEDUSA_REQUIRE_PTR(topk_ids);
  MEDUSA_REQUIRE_PTR(root_token);
  MEDUSA_REQUIRE_PTR(prefix_len);
  MEDUSA_REQUIRE_PTR(tree_candidates);
  MEDUSA_REQUIRE_PTR(tree_indices);
  MEDUSA_REQUIRE_PTR(parent);
  MEDUSA_REQUIRE_PTR(depth);
  MEDUSA_REQUIRE_PTR(position_ids);
  MEDUSA_REQUIRE_PTR(tree_mask);
  MEDUSA_REQUIRE_PTR(retrieve);
  MEDUSA_REQUIRE_PTR(num_paths);
  MEDUSA_REQUIRE_PTR(status);
  hipLaunchKernelGGL(build_tree_kernel, dim3(1), dim3(kTreeThreads), 0, static_cast<hipStream_t>(stream), B,
                     K, topk, n_choices, p_max, choices, topk_ids, root_token, prefix_len, tree_candidates,
                     tree_indices, parent, depth, position_ids, tree_mask, retrieve, num_paths, status);
  return medusa_host::hip_check("medusa_build_tree launch");
}
