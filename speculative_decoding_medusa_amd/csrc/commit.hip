// KV commit on gfx950: gather the accepted path's rows into the slots right
// after the prefix, in place.
//
// One wave per (layer, sequence, head, K|V) group.  Row j = 1 .. accept_len
// moves from slot L + path[j] to slot L + j (row 0, the root, never moves);
// rows whose source already is their destination are skipped.  A source
// slot can be another row's destination (path (0, 2, 11): slot L+2 is both
// read for row 1 and written for row 2), so the wave loads every row it
// moves into registers, waits for all loads, and only then stores.  Groups
// touch disjoint memory, so no cross-wave ordering is needed.
#include "common.hpp"

namespace medusa {

constexpr int kCommitThreads = 256;
constexpr int kCommitMaxRows = kMaxHeads;   // accept_len <= K <= 8

template <int RowBytes>
__global__ __launch_bounds__(kCommitThreads) void commit_kv_kernel(
    int B, int H, int max_slots, int p_max, int D, long long n_groups, char* __restrict__ k_cache,
    char* __restrict__ v_cache, const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ retrieve,
    const int32_t* __restrict__ best_path, const int32_t* __restrict__ accept_len,
    int32_t* __restrict__ new_prefix_len) {
  constexpr int PIECES = RowBytes / 16;                  // 16-byte pieces per row
  constexpr int SLOTS = kCommitMaxRows * PIECES;         // pieces a group may move
  constexpr int PER_LANE = (SLOTS + kWave - 1) / kWave;
  const long long grp = static_cast<long long>(blockIdx.x) * (kCommitThreads / kWave) + (threadIdx.x >> 6);
  if (grp >= n_groups) return;
  const int lane = threadIdx.x & 63;
  // group = ((layer * B + b) * H + head) * 2 + kv
  const int kv = static_cast<int>(grp & 1);
  const long long lbh = grp >> 1;
  const int b = static_cast<int>((lbh / H) % B);
  const int L = prefix_len[b];
  int acc = accept_len[b];
  const int bp = best_path[b];
  if (grp == static_cast<long long>(b) * H * 2 && lane == 0) new_prefix_len[b] = L + acc + 1;
  if (bp < 0 || bp >= p_max || L < 0) return;
  if (acc > D - 1) acc = D - 1;
  if (acc > kCommitMaxRows) acc = kCommitMaxRows;
  char* base = (kv ? v_cache : k_cache) + static_cast<size_t>(lbh) * max_slots * RowBytes;
  const int32_t* path = retrieve + static_cast<size_t>(bp) * D;

  u32x4 data[PER_LANE];
  int dst[PER_LANE];
#pragma unroll
  for (int r = 0; r < PER_LANE; ++r) {
    const int slot = r * kWave + lane;
    const int j = 1 + slot / PIECES, pc = slot % PIECES;
    dst[r] = -1;
    if (j <= acc) {
      const int src = path[j];
      if (src >= 0 && src != j && L + src < max_slots && L + j < max_slots) {
        data[r] = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(L + src) * RowBytes + pc * 16);
        dst[r] = (L + j) * PIECES + pc;
      }
    }
  }
  // every load of the wave completes before any store is issued
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int r = 0; r < PER_LANE; ++r) {
    if (dst[r] >= 0) {
      const int slot = dst[r] / PIECES, pc = dst[r] % PIECES;
      *reinterpret_cast<u32x4*>(base + static_cast<size_t>(slot) * RowBytes + pc * 16) = data[r];
    }
  }
}

}  // namespace medusa

extern "C" int medusa_commit_kv(int dtype, int B, int n_layers, int H, int d, int max_slots, void* k_cache,
                                void* v_cache, const int32_t* prefix_len, const int32_t* retrieve, int p_max, int D,
                                const int32_t* best_path, const int32_t* accept_len, int32_t* new_prefix_len,
                                void* stream) {
  using namespace medusa;
  MEDUSA_REQUIRE(dtype == MEDUSA_F32 || dtype == MEDUSA_BF16, MEDUSA_ERR_DTYPE, "%s: dtype %d", __func__, dtype);
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d", __func__, B);
  MEDUSA_REQUIRE(n_layers >= 1 && n_layers <= 4096, MEDUSA_ERR_SHAPE, "%s: n_layers=%d", __func__, n_layers);
  MEDUSA_REQUIRE(H >= 1 && H <= 1024, MEDUSA_ERR_SHAPE, "%s: H=%d", __func__, H);
  MEDUSA_REQUIRE(d == 64 || d == 128, MEDUSA_ERR_SHAPE, "%s: d=%d not 64 or 128", __func__, d);
  MEDUSA_REQUIRE(max_slots >= 1 && max_slots <= (1 << 24), MEDUSA_ERR_SHAPE, "%s: max_slots=%d", __func__,
                 max_slots);
  MEDUSA_REQUIRE(p_max >= 1 && p_max <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: p_max=%d", __func__, p_max);
  MEDUSA_REQUIRE(D >= 1 && D <= kMaxHeads + 1, MEDUSA_ERR_SHAPE, "%s: D=%d", __func__, D);
  MEDUSA_REQUIRE_PTR(k_cache);
  MEDUSA_REQUIRE_PTR(v_cache);
  MEDUSA_REQUIRE_PTR(prefix_len);
  MEDUSA_REQUIRE_PTR(retrieve);
  MEDUSA_REQUIRE_PTR(best_path);
  MEDUSA_REQUIRE_PTR(accept_len);
  MEDUSA_REQUIRE_PTR(new_prefix_len);
  MEDUSA_REQUIRE(static_cast<const void*>(new_prefix_len) != static_cast<const void*>(prefix_len),
                 MEDUSA_ERR_ALIAS, "%s: new_prefix_len aliases prefix_len", __func__);
  MEDUSA_REQUIRE(k_cache != v_cache, MEDUSA_ERR_ALIAS, "%s: k_cache and v_cache alias", __func__);
  const int row_bytes = d * medusa_host::dtype_size(dtype);
  const long long n_groups = static_cast<long long>(n_layers) * B * H * 2;
  const long long per_block = kCommitThreads / kWave;
  const long long blocks = (n_groups + per_block - 1) / per_block;
  MEDUSA_REQUIRE(blocks <= 0x7fffffffLL, MEDUSA_ERR_SHAPE, "%s: too many groups", __func__);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* kc = static_cast<char*>(k_cache);
  char* vc = static_cast<char*>(v_cache);
  switch (row_bytes) {
    case 128:
      hipLaunchKernelGGL(commit_kv_kernel<128>, dim3(static_cast<unsigned>(blocks)), dim3(kCommitThreads), 0, st, B,
                         H, max_slots, p_max, D, n_groups, kc, vc, prefix_len, retrieve, best_path, accept_len,
                         new_prefix_len);
      break;
    case 256:
      hipLaunchKernelGGL(commit_kv_kernel<256>, dim3(static_cast<unsigned>(blocks)), dim3(kCommitThreads), 0, st, B,
                         H, max_slots, p_max, D, n_groups, kc, vc, prefix_len, retrieve, best_path, accept_len,
                         new_prefix_len);
      break;
    default:
      hipLaunchKernelGGL(commit_kv_kernel<512>, dim3(static_cast<unsigned>(blocks)), dim3(kCommitThreads), 0, st, B,
                         H, max_slots, p_max, D, n_groups, kc, vc, prefix_len, retrieve, best_path, accept_len,
                         new_prefix_len);
      break;
  }
  return medusa_host::hip_check("medusa_commit_kv launch");
}
