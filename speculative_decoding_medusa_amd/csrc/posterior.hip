// Acceptance of the candidate tree on gfx950.
//
// Stage 1 (rows): grid (chunks, B*T).  Each workgroup reads one chunk of one
// node's logits into registers once (16-byte loads), reduces max / argmax
// (ties: lowest token id) and, for temperature > 0, the softmax statistics
// S = sum exp(z - m) and A = sum (z - m) exp(z - m) of z = logits / temperature
// relative to its own chunk maximum.  Wave reductions on DPP lane moves, then
// LDS across waves.
//
// Stage 2 (decide): one workgroup per sequence merges the chunk statistics
// per node (log-sum-exp rescaling), derives H = log S - A / S and the
// threshold min(eps, delta * exp(-H)), walks every retrieve path with one
// thread, and picks the lowest-index longest path with a block reduction.
#include "common.hpp"

namespace medusa {

constexpr int kPostThreads = 256;
constexpr int kPostVec = 4;         // float4 loads per thread per chunk
constexpr int kPostChunk = kPostThreads * kPostVec * 4;

__global__ __launch_bounds__(kPostThreads) void posterior_rows_kernel(
    int T, int V, int nchunk, const float* __restrict__ logits, float temperature, RowStat* __restrict__ stats) {
  const int chunk = blockIdx.x, row = blockIdx.y;   // row = b * T + node
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* x = logits + static_cast<size_t>(row) * V;
  const int lo = chunk * kPostChunk;
  const float NEG = -__builtin_huge_valf();
  float v[kPostVec * 4];
  const bool vec_ok = (V & 3) == 0;
#pragma unroll
  for (int r = 0; r < kPostVec; ++r) {
    const int e = lo + (r * kPostThreads + tid) * 4;
    if (vec_ok && e + 3 < V) {
      const float4 f = *reinterpret_cast<const float4*>(x + e);
      v[4 * r] = f.x; v[4 * r + 1] = f.y; v[4 * r + 2] = f.z; v[4 * r + 3] = f.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * r + c] = e + c < V ? x[e + c] : NEG;
    }
  }
  // max / argmax over this thread's elements (ascending index order)
  float mx = NEG;
  int arg = 0x7fffffff;
#pragma unroll
  for (int r = 0; r < kPostVec; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lo + (r * kPostThreads + tid) * 4 + c;
      if (e < V && beats(v[4 * r + c], e, mx, arg)) { mx = v[4 * r + c]; arg = e; }
    }
  wave_argmax_dpp(mx, arg);
  __shared__ float smx[kPostThreads / kWave];
  __shared__ int sarg[kPostThreads / kWave];
  __shared__ float sS[kPostThreads / kWave], sA[kPostThreads / kWave];
  if (lane == 0) { smx[wave] = mx; sarg[wave] = arg; }
  __syncthreads();
  mx = smx[0];
  arg = sarg[0];
  for (int w = 1; w < kPostThreads / kWave; ++w)
    if (beats(smx[w], sarg[w], mx, arg)) { mx = smx[w]; arg = sarg[w]; }
  RowStat out;
  out.mx = mx;
  out.arg = arg;
  out.m = NEG;
  out.S = 0.f;
  out.A = 0.f;
  if (temperature > 0.f) {
    // division by a positive temperature is monotonic, so max z = max x / t
    const float m = mx / temperature;
    float S = 0.f, A = 0.f;
#pragma unroll
    for (int r = 0; r < kPostVec; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = lo + (r * kPostThreads + tid) * 4 + c;
        if (e < V) {
          const float dz = v[4 * r + c] / temperature - m;
          const float p = expf(dz);
          S += p;
          A += dz * p;
        }
      }
    S = wave_reduce_dpp<false>(S);
    A = wave_reduce_dpp<false>(A);
    if (lane == 0) { sS[wave] = S; sA[wave] = A; }
    __syncthreads();
    S = 0.f;
    A = 0.f;
    for (int w = 0; w < kPostThreads / kWave; ++w) { S += sS[w]; A += sA[w]; }
    out.m = m;
    out.S = S;
    out.A = A;
  }
  if (tid == 0) stats[static_cast<size_t>(row) * nchunk + chunk] = out;
}

// Decide, in three phases of independent loads: (1) the sequence's
// candidates and the retrieve paths into LDS, and every node's chunk
// statistics (all chunks of a node loaded together) merged into its argmax
// and threshold; (2) the accept flag of every (path, depth) pair at once --
// the child's token against its parent's argmax, or its tempered
// probability against the parent's threshold (one logit load); (3) each
// path's run of leading accepted steps, and the lowest-index longest path.
constexpr int kDecideUnroll = 8;   // chunk statistics loaded per batch

//
// child_z (optional, [B][T][T]): child_z[b][n][c] = the logit of node c's
// token at node n, supplied by the fused base lm_head instead of `logits`.
__global__ __launch_bounds__(kPostThreads) void posterior_decide_kernel(
    int T, int V, int nchunk, int p_max, int D, const float* __restrict__ logits,
    const int32_t* __restrict__ tree_candidates, const int32_t* __restrict__ retrieve,
    const int32_t* __restrict__ num_paths, float temperature, float eps, float delta,
    const RowStat* __restrict__ stats, int32_t* __restrict__ best_path, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ next_token, const float* __restrict__ child_z) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_tok[kMaxNodes], s_arg[kMaxNodes];
  __shared__ float s_m[kMaxNodes], s_S[kMaxNodes], s_thr[kMaxNodes];
  __shared__ int16_t s_ret[kMaxNodes * (kMaxHeads + 1)];
  __shared__ uint8_t s_acc[kMaxNodes * (kMaxHeads + 1)];
  __shared__ int s_len[kPostThreads / kWave], s_path[kPostThreads / kWave];
  const bool typical = temperature > 0.f;
  const float NEG = -__builtin_huge_valf();

  int P = *num_paths;
  if (P > p_max) P = p_max;
  if (P < 0) P = 0;
  const int nret = P * D;
  // (1) one round trip: this thread's candidate, its share of the paths and
  // the first batch of its node's chunk statistics are all requested before
  // anything waits (clamped indices, masked at use)
  constexpr int RPER = (kMaxNodes * (kMaxHeads + 1) + kPostThreads - 1) / kPostThreads;
  const int node = min(tid, T - 1);
  const int tokv = tree_candidates[static_cast<size_t>(b) * T + node];
  int retv[RPER];
#pragma unroll
  for (int u = 0; u < RPER; ++u) retv[u] = retrieve[max(min(u * kPostThreads + tid, nret - 1), 0)];
  const RowStat* st = stats + (static_cast<size_t>(b) * T + node) * nchunk;
  RowStat r[kDecideUnroll];
#pragma unroll
  for (int u = 0; u < kDecideUnroll; ++u) r[u] = st[min(u, nchunk - 1)];

  // candidates and paths into LDS (entries outside [0, T) end a path)
  if (tid < T) s_tok[tid] = tokv;
#pragma unroll
  for (int u = 0; u < RPER; ++u) {
    const int x = u * kPostThreads + tid;
    if (x < nret) s_ret[x] = static_cast<int16_t>(retv[u] >= 0 && retv[u] < T ? retv[u] : -1);
  }
  // node statistics: chunks merged with log-sum-exp rescaling, a batch of
  // kDecideUnroll chunks at a time (one batch for V <= 32768)
  if (tid < T) {
    float mx = NEG, m = NEG, S = 0.f, A = 0.f;
    int arg = 0x7fffffff;
    for (int c0 = 0; c0 < nchunk; c0 += kDecideUnroll) {
      if (c0 > 0) {
#pragma unroll
        for (int u = 0; u < kDecideUnroll; ++u) r[u] = st[min(c0 + u, nchunk - 1)];
      }
      float mb = m;
#pragma unroll
      for (int u = 0; u < kDecideUnroll; ++u) {
        if (c0 + u < nchunk) {
          if (beats(r[u].mx, r[u].arg, mx, arg)) { mx = r[u].mx; arg = r[u].arg; }
          mb = fmaxf(mb, r[u].m);
        }
      }
      if (typical) {
        // rescale the running sums to the new maximum, then add this batch
        if (m != NEG) {
          const float w0 = expf(m - mb);
          A = w0 * (A + (m - mb) * S);
          S *= w0;
        }
#pragma unroll
        for (int u = 0; u < kDecideUnroll; ++u) {
          if (c0 + u < nchunk) {
            const float w = expf(r[u].m - mb);
            S += r[u].S * w;
            A += w * (r[u].A + (r[u].m - mb) * r[u].S);
          }
        }
      }
      m = mb;
    }
    s_arg[tid] = arg;
    if (typical) {
      const float H = logf(S) - A / S;
      s_m[tid] = m;
      s_S[tid] = S;
      s_thr[tid] = fminf(eps, delta * expf(-H));
    }
  }
  __syncthreads();

  // (2) accept flag of step j of path p: child c = ret[p][j], parent ret[p][j-1]
  for (int x0 = 0; x0 < nret; x0 += kPostThreads * 4) {
    float z[4];
    int c[4], prev[4], tok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = min(x0 + u * kPostThreads + tid, nret - 1);
      const int j = x % D;
      c[u] = j > 0 ? s_ret[x] : -1;
      prev[u] = j > 0 ? s_ret[x - 1] : -1;
      tok[u] = c[u] >= 0 ? s_tok[c[u]] : -1;
      const bool ok = prev[u] >= 0 && tok[u] >= 0 && tok[u] < V;
      z[u] = 0.f;
      if (typical) {
        if (child_z != nullptr)
          z[u] = child_z[(static_cast<size_t>(b) * T + (ok ? prev[u] : 0)) * T + (ok ? c[u] : 0)];
        else
          z[u] = logits[(static_cast<size_t>(b) * T + (ok ? prev[u] : 0)) * V + (ok ? tok[u] : 0)];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = x0 + u * kPostThreads + tid;
      if (x >= nret) continue;
      const bool ok = c[u] >= 0 && prev[u] >= 0 && tok[u] >= 0 && tok[u] < V;
      bool acc = false;
      if (ok) {
        if (!typical) {
          acc = tok[u] == s_arg[prev[u]];
        } else {
          const float pr = expf(z[u] / temperature - s_m[prev[u]]) / s_S[prev[u]];
          acc = pr > s_thr[prev[u]];
        }
      }
      s_acc[x] = acc ? 1 : 0;
    }
  }
  __syncthreads();

  // (3) accepted length of every path; lowest-index longest path
  int best_len = -1, best_p = 0x7fffffff;
  for (int p = tid; p < P; p += kPostThreads) {
    int ell = 0;
    if (s_ret[p * D] >= 0) {
      for (int j = 1; j < D && s_acc[p * D + j]; ++j) ++ell;
    }
    if (ell > best_len || (ell == best_len && p < best_p)) { best_len = ell; best_p = p; }
  }
  {
    // the wave's longest (lowest-index on ties) on DPP lane moves; the fill
    // (-1, INT_MAX) never wins
    auto take = [&](uint32_t ol, uint32_t op) {
      const int l = static_cast<int>(ol), q = static_cast<int>(op);
      if (l > best_len || (l == best_len && q < best_p)) { best_len = l; best_p = q; }
    };
    const uint32_t fl = 0xffffffffu, fp = 0x7fffffffu;
    take(dpp_u32<0x111, 0xf>(best_len, fl), dpp_u32<0x111, 0xf>(best_p, fp));
    take(dpp_u32<0x112, 0xf>(best_len, fl), dpp_u32<0x112, 0xf>(best_p, fp));
    take(dpp_u32<0x114, 0xf>(best_len, fl), dpp_u32<0x114, 0xf>(best_p, fp));
    take(dpp_u32<0x118, 0xf>(best_len, fl), dpp_u32<0x118, 0xf>(best_p, fp));
    take(dpp_u32<0x142, 0xa>(best_len, fl), dpp_u32<0x142, 0xa>(best_p, fp));
    take(dpp_u32<0x143, 0xc>(best_len, fl), dpp_u32<0x143, 0xc>(best_p, fp));
    best_len = __builtin_amdgcn_readlane(best_len, kWave - 1);
    best_p = __builtin_amdgcn_readlane(best_p, kWave - 1);
  }
  if (lane == 0) { s_len[wave] = best_len; s_path[wave] = best_p; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kPostThreads / kWave; ++w)
      if (s_len[w] > best_len || (s_len[w] == best_len && s_path[w] < best_p)) {
        best_len = s_len[w];
        best_p = s_path[w];
      }
    if (best_len < 0) { best_len = 0; best_p = 0; }   // no paths: the root alone
    int last = 0;
    if (P > 0) {
      last = s_ret[best_p * D + best_len];
      if (last < 0) last = 0;
    }
    best_path[b] = best_p;
    accept_len[b] = best_len;
    next_token[b] = s_arg[last];
  }
}

}  // namespace medusa

namespace {
using namespace medusa;
int post_chunks(int V) { return (V + kPostChunk - 1) / kPostChunk; }
size_t post_ws(int B, int T, int V) {
  return medusa_host::round_up(static_cast<size_t>(B) * T * post_chunks(V) * sizeof(RowStat), 256);
}
}  // namespace

extern "C" size_t medusa_posterior_workspace(int B, int T, int V) {
  if (B < 1 || B > kMaxBatch || T < 1 || T > kMaxNodes || V < 1) return 0;
  return post_ws(B, T, V);
}

extern "C" int medusa_evaluate_posterior(int B, int T, int V, int p_max, int D, const float* logits,
                                         const int32_t* tree_candidates, const int32_t* retrieve,
                                         const int32_t* num_paths, float temperature, float eps, float delta,
                                         int32_t* best_path, int32_t* accept_len, int32_t* next_token,
                                         void* ws, size_t ws_bytes, void* stream) {
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d", __func__, B);
  MEDUSA_REQUIRE(T >= 1 && T <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: T=%d", __func__, T);
  MEDUSA_REQUIRE(V >= 1 && V <= (1 << 24), MEDUSA_ERR_SHAPE, "%s: V=%d", __func__, V);
  MEDUSA_REQUIRE(p_max >= 1 && p_max <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: p_max=%d", __func__, p_max);
  MEDUSA_REQUIRE(D >= 1 && D <= kMaxHeads + 1, MEDUSA_ERR_SHAPE, "%s: D=%d", __func__, D);
  MEDUSA_REQUIRE(temperature == temperature && temperature >= 0.f, MEDUSA_ERR_VALUE,
                 "%s: temperature must be >= 0", __func__);
  MEDUSA_REQUIRE(temperature == 0.f || (eps == eps && eps > 0.f && delta == delta && delta > 0.f),
                 MEDUSA_ERR_VALUE, "%s: eps and delta must be positive", __func__);
  MEDUSA_REQUIRE_PTR(logits);
  MEDUSA_REQUIRE_PTR(tree_candidates);
  MEDUSA_REQUIRE_PTR(retrieve);
  MEDUSA_REQUIRE_PTR(num_paths);
  MEDUSA_REQUIRE_PTR(best_path);
  MEDUSA_REQUIRE_PTR(accept_len);
  MEDUSA_REQUIRE_PTR(next_token);
  MEDUSA_REQUIRE_PTR(ws);
  MEDUSA_REQUIRE(ws_bytes >= post_ws(B, T, V), MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__,
                 ws_bytes, post_ws(B, T, V));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int nchunk = post_chunks(V);
  RowStat* stats = static_cast<RowStat*>(ws);
  hipLaunchKernelGGL(posterior_rows_kernel, dim3(nchunk, B * T), dim3(kPostThreads), 0, st, T, V, nchunk, logits,
                     temperature, stats);
  int rc = medusa_host::hip_check("medusa_evaluate_posterior rows launch");
  if (rc != MEDUSA_OK) return rc;
  hipLaunchKernelGGL(posterior_decide_kernel, dim3(B), dim3(kPostThreads), 0, st, T, V, nchunk, p_max, D, logits,
                     tree_candidates, retrieve, num_paths, temperature, eps, delta, stats, best_path, accept_len,
                     next_token, static_cast<const float*>(nullptr));
  return medusa_host::hip_check("medusa_evaluate_posterior decide launch");
}

namespace medusa {

// Per-row statistics from `nparts` partial ones (disjoint vocabulary
// blocks): one workgroup per row, every part requested in one round trip,
// merged in registers, across the wave on DPP lane moves, then across waves.
constexpr int kMergeParts = 4;   // parts per thread: nparts <= 1024

// `a` of the lane that DPP control C (row mask M) selects; the empty set
// where there is none
template <int C, int M>
__device__ __forceinline__ RowStat rowstat_dpp(const RowStat& a) {
  const float NEG = -__builtin_huge_valf();
  RowStat y;
  y.mx = dpp_f32<C, M>(a.mx, NEG);
  y.arg = static_cast<int>(dpp_u32<C, M>(static_cast<uint32_t>(a.arg), 0x7fffffffu));
  y.m = dpp_f32<C, M>(a.m, NEG);
  y.S = dpp_f32<C, M>(a.S, 0.f);
  y.A = dpp_f32<C, M>(a.A, 0.f);
  return y;
}

__global__ __launch_bounds__(kPostThreads) void posterior_merge_kernel(int nparts, int typical,
                                                                     const RowStat* __restrict__ parts,
                                                                     RowStat* __restrict__ out) {
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const RowStat* pr = parts + static_cast<size_t>(row) * nparts;
  const float NEG = -__builtin_huge_valf();
  RowStat x[kMergeParts];
#pragma unroll
  for (int u = 0; u < kMergeParts; ++u) x[u] = pr[min(u * kPostThreads + tid, nparts - 1)];
  RowStat acc = {NEG, 0x7fffffff, NEG, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMergeParts; ++u)
    if (u * kPostThreads + tid < nparts) rowstat_merge(acc, x[u], typical != 0);
  // across the wave on DPP lane moves (lanes with no source bring the empty
  // set); lane 63 ends with the wave's statistics
  rowstat_merge(acc, rowstat_dpp<0x111, 0xf>(acc), typical != 0);
  rowstat_merge(acc, rowstat_dpp<0x112, 0xf>(acc), typical != 0);
  rowstat_merge(acc, rowstat_dpp<0x114, 0xf>(acc), typical != 0);
  rowstat_merge(acc, rowstat_dpp<0x118, 0xf>(acc), typical != 0);
  rowstat_merge(acc, rowstat_dpp<0x142, 0xa>(acc), typical != 0);
  rowstat_merge(acc, rowstat_dpp<0x143, 0xc>(acc), typical != 0);
  __shared__ RowStat s_part[kPostThreads / kWave];
  if (lane == kWave - 1) s_part[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    acc = s_part[0];
    for (int w = 1; w < kPostThreads / kWave; ++w) rowstat_merge(acc, s_part[w], typical != 0);
    out[row] = acc;
  }
}

}  // namespace medusa

namespace medusa_host {

// Acceptance from per-(row, part) statistics and the children's logits
// (rows = B * T nodes): merge kernel, then the decide kernel on one
// statistic per row.  `merged` holds B * T statistics.
int posterior_from_parts(int B, int T, int V, int p_max, int D, int nparts, const medusa::RowStat* parts,
                         medusa::RowStat* merged, const float* child_z, const int32_t* tree_candidates,
                         const int32_t* retrieve, const int32_t* num_paths, float temperature, float eps,
                         float delta, int32_t* best_path, int32_t* accept_len, int32_t* next_token,
                         hipStream_t st) {
  using namespace medusa;
  hipLaunchKernelGGL(posterior_merge_kernel, dim3(B * T), dim3(kPostThreads), 0, st, nparts,
                     temperature > 0.f ? 1 : 0, parts, merged);
  int rc = hip_check("posterior merge launch");
  if (rc != MEDUSA_OK) return rc;
  hipLaunchKernelGGL(posterior_decide_kernel, dim3(B), dim3(kPostThreads), 0, st, T, V, 1, p_max, D,
                     static_cast<const float*>(nullptr), tree_candidates, retrieve, num_paths, temperature, eps,
                     delta, merged, best_path, accept_len, next_token, child_z);
  return hip_check("posterior decide launch");
}

// Acceptance on one drawn token per node (RowStat.arg): the greedy
// decision with the draw in place of the argmax (nucleus acceptance).
int decide_on_draws(int B, int T, int V, int p_max, int D, const medusa::RowStat* draws,
                    const int32_t* tree_candidates, const int32_t* retrieve, const int32_t* num_paths,
                    int32_t* best_path, int32_t* accept_len, int32_t* next_token, hipStream_t st) {
  using namespace medusa;
  hipLaunchKernelGGL(posterior_decide_kernel, dim3(B), dim3(kPostThreads), 0, st, T, V, 1, p_max, D,
                     static_cast<const float*>(nullptr), tree_candidates, retrieve, num_paths, 0.f, 0.f, 0.f, draws,
                     best_path, accept_len, next_token, static_cast<const float*>(nullptr));
  return hip_check("posterior decide launch");
}

}  // namespace medusa_host
