// Candidate tree from a medusa_choices spec, in one workgroup.
//
// Thread e owns spec entry e (and later node e).  The spec is validated in
// the documented order with one atomicMin over (phase, entry, kind) keys, nodes
// are ordered by counting the entries that sort before each one (length,
// then lexicographic), parents are found by matching the tuple minus its
// last rank, and every output is written from LDS.  Work is O(N^2 K) with
// N <= 255: a few microseconds of integer work, bound by launch latency.
#include "common.hpp"

namespace medusa {

constexpr int kTreeThreads = 256;
constexpr int kMaxDepth = kMaxHeads;

__device__ __forceinline__ bool tuple_less(const int8_t* a, int la, const int8_t* b, int lb) {
  if (la != lb) return la < lb;
  for (int m = 0; m < la; ++m)
    if (a[m] != b[m]) return a[m] < b[m];
  return false;
}

__device__ __forceinline__ bool tuple_eq_prefix(const int8_t* a, const int8_t* b, int len) {
  for (int m = 0; m < len; ++m)
    if (a[m] != b[m]) return false;
  return true;
}

__global__ __launch_bounds__(kTreeThreads) void build_tree_kernel(
    int B, int K, int topk, int N, int p_max, const int32_t* __restrict__ choices,
    const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ root_token,
    const int32_t* __restrict__ prefix_len, int32_t* __restrict__ tree_candidates,
    int32_t* __restrict__ tree_indices, int32_t* __restrict__ parent_out, int32_t* __restrict__ depth_out,
    int32_t* __restrict__ position_ids, uint8_t* __restrict__ tree_mask, int32_t* __restrict__ retrieve,
    int32_t* __restrict__ num_paths, int32_t* __restrict__ status) {
  __shared__ int8_t tup[kMaxNodes][kMaxDepth];   // by entry
  __shared__ int8_t len[kMaxNodes];
  __shared__ int16_t node_entry[kMaxNodes];      // node -> entry (node 0 = root = -1)
  __shared__ int16_t par[kMaxNodes];
  __shared__ int8_t dep[kMaxNodes];
  __shared__ uint8_t has_child[kMaxNodes];
  __shared__ int16_t path_of[kMaxNodes];
  __shared__ uint64_t anc[kMaxNodes][kMaxNodes / 64];
  __shared__ int err_key;
  __shared__ int n_leaves;

  const int tid = threadIdx.x;
  const int T = N + 1;
  const int D = K + 1;
  if (tid == 0) { err_key = 0x7fffffff; n_leaves = 0; }
  if (tid < kMaxNodes) has_child[tid] = 0;
  __syncthreads();

  // phase 0: per-entry format (padding, then empty, then rank)
  int my_err = 0;
  if (tid < N) {
    int row[kMaxDepth];
    for (int m = 0; m < K; ++m) row[m] = choices[static_cast<size_t>(tid) * K + m];
    int n = K;
    while (n > 0 && row[n - 1] == -1) --n;
    bool pad = false, rank = false;
    for (int m = 0; m < n; ++m) {
      if (row[m] == -1) pad = true;
      else if (row[m] < 0 || row[m] >= topk) rank = true;
    }
    if (pad) my_err = MEDUSA_SPEC_PADDING;
    else if (n == 0) my_err = MEDUSA_SPEC_EMPTY;
    else if (rank) my_err = MEDUSA_SPEC_RANK;
    for (int m = 0; m < kMaxDepth; ++m) tup[tid][m] = static_cast<int8_t>(m < n ? row[m] : -1);
    len[tid] = static_cast<int8_t>(n);
    if (my_err) atomicMin(&err_key, (0 << 24) | (tid << 8) | my_err);
  }
  __syncthreads();
  if (err_key == 0x7fffffff && tid < N) {
    // phase 1: duplicates (first entry equal to an earlier one)
    const int l = len[tid];
    for (int e = 0; e < tid; ++e) {
      if (len[e] == l && tuple_eq_prefix(tup[e], tup[tid], l)) {
        atomicMin(&err_key, (1 << 24) | (tid << 8) | MEDUSA_SPEC_DUPLICATE);
        break;
      }
    }
    // phase 2: every proper prefix must be an entry
    for (int m = 1; m < l; ++m) {
      bool found = false;
      for (int e = 0; e < N && !found; ++e) found = len[e] == m && tuple_eq_prefix(tup[e], tup[tid], m);
      if (!found) {
        atomicMin(&err_key, (2 << 24) | (tid << 8) | MEDUSA_SPEC_PREFIX);
        break;
      }
    }
  }
  __syncthreads();

  bool ok = err_key == 0x7fffffff;
  if (ok) {
    // node order: rank among entries by (length, lexicographic)
    if (tid < N) {
      int rank = 0;
      for (int e = 0; e < N; ++e) rank += tuple_less(tup[e], len[e], tup[tid], len[tid]) ? 1 : 0;
      node_entry[rank + 1] = static_cast<int16_t>(tid);
    }
    if (tid == 0) { node_entry[0] = -1; par[0] = -1; dep[0] = 0; }
    __syncthreads();
    // parent of node i: the node whose tuple is node i's minus its last rank
    if (tid >= 1 && tid < T) {
      const int e = node_entry[tid];
      const int l = len[e];
      dep[tid] = static_cast<int8_t>(l);
      int p = 0;
      if (l > 1) {
        for (int q = 1; q < T; ++q) {
          const int f = node_entry[q];
          if (len[f] == l - 1 && tuple_eq_prefix(tup[f], tup[e], l - 1)) { p = q; break; }
        }
      }
      par[tid] = static_cast<int16_t>(p);
      has_child[p] = 1;
    }
    __syncthreads();
    // ancestor bitmasks (walk parents; depth <= K)
    if (tid < T) {
      uint64_t w[kMaxNodes / 64] = {0, 0, 0, 0};
      int a = tid;
      while (a >= 0) {
        w[a >> 6] |= 1ull << (a & 63);
        a = par[a];
      }
      for (int q = 0; q < kMaxNodes / 64; ++q) anc[tid][q] = w[q];
    }
    // leaf order: a leaf's path index is the number of leaves before it
    if (tid < T && !has_child[tid]) {
      int before = 0;
      for (int q = 0; q < tid; ++q) before += has_child[q] ? 0 : 1;
      path_of[tid] = static_cast<int16_t>(before);
      atomicAdd(&n_leaves, 1);
    }
    __syncthreads();
    if (n_leaves > p_max) {
      if (tid == 0) err_key = (3 << 24) | ((n_leaves & 0xffff) << 8) | MEDUSA_SPEC_TOO_MANY_PATHS;
      ok = false;
    }
  }
  __syncthreads();

  if (!ok) {
    // the root alone: every later stage stays in bounds and accepts nothing
    if (tid < T) {
      par[tid] = -1;
      dep[tid] = 0;
      for (int q = 0; q < kMaxNodes / 64; ++q) anc[tid][q] = 0;
      anc[tid][tid >> 6] = 1ull << (tid & 63);
      has_child[tid] = 1;
    }
    __syncthreads();
    if (tid == 0) { has_child[0] = 0; path_of[0] = 0; n_leaves = 1; }
    __syncthreads();
  }

  // per-node outputs
  if (tid < T) {
    const int d = dep[tid];
    int ti = 0;
    if (ok && tid > 0) {
      const int e = node_entry[tid];
      ti = 1 + (d - 1) * topk + tup[e][d - 1];
    }
    tree_indices[tid] = ti;
    parent_out[tid] = par[tid];
    depth_out[tid] = d;
    for (int b = 0; b < B; ++b) {
      const int tok = ti == 0 ? root_token[b]
                              : topk_ids[(static_cast<size_t>(b) * K + (d - 1)) * topk + (ti - 1 - (d - 1) * topk)];
      tree_candidates[static_cast<size_t>(b) * T + tid] = tok;
      position_ids[static_cast<size_t>(b) * T + tid] = prefix_len[b] + d;
    }
  }
  // mask rows, written as bytes over the flat [T][T] array
  for (int x = tid; x < T * T; x += kTreeThreads) {
    const int i = x / T, jj = x - i * T;
    tree_mask[x] = static_cast<uint8_t>((anc[i][jj >> 6] >> (jj & 63)) & 1ull);
  }
  // retrieve: rows >= num_paths are all -1
  for (int x = tid; x < p_max * D; x += kTreeThreads) retrieve[x] = -1;
  __syncthreads();
  if (tid < T && !has_child[tid]) {
    const int p = path_of[tid];
    int a = tid;
    while (a >= 0) {
      retrieve[static_cast<size_t>(p) * D + dep[a]] = a;
      a = par[a];
    }
  }
  if (tid == 0) {
    *num_paths = n_leaves;
    const int key = err_key;
    status[0] = key == 0x7fffffff ? MEDUSA_SPEC_OK : (key & 0xff);
    status[1] = key == 0x7fffffff ? -1 : ((key >> 8) & 0xffff);
  }
}

}  // namespace medusa

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
