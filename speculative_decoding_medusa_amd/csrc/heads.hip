// Medusa heads on gfx950: ResBlock GEMV and lm_head GEMV with fused top-k.
//
// Both stages are skinny matrix products (B <= 16 rows of activations
// against K*H resp. K*V weight rows) and bound by streaming the weights
// from HBM.  The bf16 path feeds them through v_mfma_f32_16x16x32_bf16 with
// the batch on the M side: lane l supplies 16 contiguous bytes of weight row
// (l % 16) at hidden offset 8 * (l / 16) of each 32-wide K step, so every
// weight byte is loaded once with 16-byte loads and the MFMA does the
// multiply-accumulate (no bf16 -> f32 conversions on the VALU).  A workgroup
// of four waves splits each 16-row tile's K range and reduces through LDS.
//
// The ResBlock output r is float32.  For the lm_head product the bf16 MFMA
// needs bf16 A operands, so r is split exactly into hi = bf16(r) and
// lo = bf16(r - hi) and both go through the MFMA as separate M rows; their
// products with the (exact) bf16 weights are summed in float32, which keeps
// about 16 significant bits of r instead of 8.
//
// Top-k: wave 0 of each workgroup keeps a sorted list per sequence in LDS
// and inserts the rare tile logits that beat its current k-th entry; the
// workgroup then publishes its list and the last workgroup of each head
// (completion counter) merges them.
#include "common.hpp"

namespace medusa {

constexpr int kHeadsThreads = 256;
constexpr int kHeadsWaves = kHeadsThreads / kWave;
constexpr int kUnroll = 8;          // 32-wide K steps issued back to back per wave
constexpr int kMergeCap = 1024;     // LDS survivors in the final merge

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ------------------------------------------------------------------ K1 bf16
// Grid (ceil(H/16), K).  r[b][j][i] = h[b][i] + SiLU(W1[j][i] . h[b] + b1[j][i]).
__global__ __launch_bounds__(kHeadsThreads) void resblock_bf16_kernel(
    int B, int H, int K, const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w1,
    const uint16_t* __restrict__ b1, float* __restrict__ r) {
  const int j = blockIdx.y;
  const int row0 = blockIdx.x * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = row0 + n;
  const bool row_ok = row < H;
  const bool a_ok = n < B;
  const uint16_t* wrow = w1 + (static_cast<size_t>(j) * H + (row_ok ? row : 0)) * H;
  const uint16_t* arow = hidden + static_cast<size_t>(a_ok ? n : 0) * H;
  const int nsteps = (H + 31) / 32;
  const int s0 = wave * nsteps / kHeadsWaves, s1 = (wave + 1) * nsteps / kHeadsWaves;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = s0; s < s1; s += kUnroll) {
    u32x4 wv[kUnroll], av[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k0 = (s + u) * 32 + g * 8;
      const bool ok = (s + u < s1) && (k0 < H);
      wv[u] = (ok && row_ok) ? ld16_stream(wrow + k0) : zero;
      av[u] = (ok && a_ok) ? ld16(arow + k0) : zero;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u]), as_bf16x8(wv[u]), acc, 0, 0, 0);
  }

  __shared__ f32x4 red[kHeadsWaves][kWave];
  red[wave][lane] = acc;
  __syncthreads();
  // thread t: accumulator element (t & 3) of lane (t >> 2) = u[b][row]
  const int L = threadIdx.x >> 2, i = threadIdx.x & 3;
  float u = 0.f;
#pragma unroll
  for (int w = 0; w < kHeadsWaves; ++w) u += red[w][L][i];
  const int b = 4 * (L >> 4) + i;
  const int rr = row0 + (L & 15);
  if (b < B && rr < H) {
    u += bf16_to_f32(b1[static_cast<size_t>(j) * H + rr]);
    const float h = bf16_to_f32(hidden[static_cast<size_t>(b) * H + rr]);
    r[(static_cast<size_t>(b) * K + j) * H + rr] = h + u / (1.0f + expf(-u));
  }
}

// ------------------------------------------------------------------ K1 f32
// Grid (ceil(H/16), K); each wave computes four rows of the tile on the VALU.
__global__ __launch_bounds__(kHeadsThreads) void resblock_f32_kernel(
    int B, int H, int K, const float* __restrict__ hidden, const float* __restrict__ w1,
    const float* __restrict__ b1, float* __restrict__ r) {
  const int j = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int q = 0; q < 4; ++q) {
    const int row = blockIdx.x * 16 + wave * 4 + q;
    if (row >= H) break;
    const float* wrow = w1 + (static_cast<size_t>(j) * H + row) * H;
    float acc[kMaxBatch];
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) acc[b] = 0.f;
    for (int k = lane * 4; k < H; k += kWave * 4) {
      const float4 w = *reinterpret_cast<const float4*>(wrow + k);
#pragma unroll
      for (int b = 0; b < kMaxBatch; ++b) {
        if (b < B) {
          const float4 h = *reinterpret_cast<const float4*>(hidden + static_cast<size_t>(b) * H + k);
          acc[b] += w.x * h.x + w.y * h.y + w.z * h.z + w.w * h.w;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) {
      if (b < B) {
        float u = wave_sum(acc[b]);
        if (lane == 0) {
          u += b1[static_cast<size_t>(j) * H + row];
          r[(static_cast<size_t>(b) * K + j) * H + row] =
              hidden[static_cast<size_t>(b) * H + row] + u / (1.0f + expf(-u));
        }
      }
    }
  }
}

// ------------------------------------------------------------- top-k lists
struct TopkLists {
  float v[kMaxBatch][kMaxTopk];
  int id[kMaxBatch][kMaxTopk];
  int count[kMaxBatch];
};

// Wave-uniform insertion of the candidates held by the lanes in `mask`.
// The lists are shared by the lanes of wave 0 through LDS without a
// barrier, so every access is volatile: each read is a real LDS read issued
// after the wave's earlier writes (LDS operations of one wave complete in
// order).
__device__ void topk_insert(TopkLists& tl_, int b, int k, float v, int id, uint64_t mask, int lane) {
  volatile TopkLists& tl = tl_;
  while (mask) {
    const int src = __ffsll(static_cast<unsigned long long>(mask)) - 1;
    mask &= mask - 1;
    const float cv = __shfl(v, src);
    const int ci = __shfl(id, src);
    const int c = tl.count[b];
    if (c == k && !beats(cv, ci, tl.v[b][k - 1], tl.id[b][k - 1])) continue;
    const float ev = lane < c ? tl.v[b][lane] : 0.f;
    const int ei = lane < c ? tl.id[b][lane] : 0;
    const int pos = __popcll(ballot(lane < c && beats(ev, ei, cv, ci)));
    const float pv = __shfl(ev, lane > 0 ? lane - 1 : 0);
    const int pi = __shfl(ei, lane > 0 ? lane - 1 : 0);
    const int nc = c + 1 < k ? c + 1 : k;
    if (lane < nc) {
      if (lane == pos) {
        tl.v[b][lane] = cv;
        tl.id[b][lane] = ci;
      } else if (lane > pos) {
        tl.v[b][lane] = pv;
        tl.id[b][lane] = pi;
      }
    }
    tl.count[b] = nc;  // every lane stores the same value
  }
}

// Block-wide best (by `beats`) of one (value, id) per thread; all threads get it.
__device__ void block_best(float& v, int& id, float* sv, int* si) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(id, o);
    if (beats(ov, oi, v, id)) { v = ov; id = oi; }
  }
  __syncthreads();
  if (lane == 0) { sv[wave] = v; si[wave] = id; }
  __syncthreads();
  v = sv[0];
  id = si[0];
  for (int w = 1; w < static_cast<int>(blockDim.x) / kWave; ++w)
    if (beats(sv[w], si[w], v, id)) { v = sv[w]; id = si[w]; }
}

// The last workgroup of head j merges the G published lists of each sequence.
__device__ void merge_head_lists(int B, int K, int V, int k, int G, int j,
                                 const float* cand_v, const int* cand_i,
                                 int32_t* topk_ids, float* topk_vals) {
  __shared__ float mv[kMergeCap];
  __shared__ int mi[kMergeCap];
  __shared__ float redv[16];
  __shared__ int redi[16];
  __shared__ int mcount;
  const int tid = threadIdx.x;
  const float NEG = -__builtin_huge_valf();
  for (int b = 0; b < B; ++b) {
    const size_t base = (static_cast<size_t>(j) * B + b) * G * k;
    // lower bound of the k-th best: the best of the per-list k-th entries
    float tv = NEG;
    int ti = 0x7fffffff;
    bool have = false;
    for (int w = tid; w < G; w += blockDim.x) {
      const int e = cand_i[base + static_cast<size_t>(w) * k + (k - 1)];
      if (e >= 0) {
        const float ev = cand_v[base + static_cast<size_t>(w) * k + (k - 1)];
        if (!have || beats(ev, e, tv, ti)) { tv = ev; ti = e; have = true; }
      }
    }
    block_best(tv, ti, redv, redi);
    const bool any_full = ti != 0x7fffffff;
    if (tid == 0) mcount = 0;
    __syncthreads();
    for (int e = tid; e < G * k; e += blockDim.x) {
      const int id = cand_i[base + e];
      if (id < 0) continue;
      const float v = cand_v[base + e];
      if (!any_full || !beats(tv, ti, v, id)) {
        const int slot = atomicAdd(&mcount, 1);
        if (slot < kMergeCap) { mv[slot] = v; mi[slot] = id; }
      }
    }
    __syncthreads();
    const int S = mcount;
    int32_t* oid = topk_ids + (static_cast<size_t>(b) * K + j) * k;
    float* oval = topk_vals + (static_cast<size_t>(b) * K + j) * k;
    if (S <= kMergeCap) {
      for (int s = tid; s < S; s += blockDim.x) {
        int rank = 0;
        for (int t = 0; t < S; ++t) rank += beats(mv[t], mi[t], mv[s], mi[s]) ? 1 : 0;
        if (rank < k) { oid[rank] = mi[s]; oval[rank] = mv[s]; }
      }
      for (int s = S + tid; s < k; s += blockDim.x) { oid[s] = -1; oval[s] = NEG; }
    } else {
      // many exact ties: k rounds of "best entry ranked after the last pick"
      float lv = __builtin_huge_valf();
      int li = -1;
      for (int round = 0; round < k; ++round) {
        float bv = NEG;
        int bi = 0x7fffffff;
        bool found = false;
        for (int e = tid; e < G * k; e += blockDim.x) {
          const int id = cand_i[base + e];
          if (id < 0) continue;
          const float v = cand_v[base + e];
          if ((round == 0 || beats(lv, li, v, id)) && (!found || beats(v, id, bv, bi))) {
            bv = v; bi = id; found = true;
          }
        }
        block_best(bv, bi, redv, redi);
        if (tid == 0) { oid[round] = bi == 0x7fffffff ? -1 : bi; oval[round] = bv; }
        lv = bv;
        li = bi;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ K2
// Grid (G, K).  Workgroup wg of head j owns rows [wg*rows_per_wg, ...) of
// Wlm[j], walked in 16-row tiles.  NP = partial sums per tile (one per wave
// for the split-K MFMA path, one for the f32 path).
template <bool kBF16, int MT>
__global__ __launch_bounds__(kHeadsThreads) void lm_topk_kernel(
    int B, int H, int V, int K, int k, int rows_per_wg, int G,
    const float* __restrict__ r, const void* __restrict__ wlm_v,
    float* __restrict__ logits_out, int32_t* __restrict__ topk_ids, float* __restrict__ topk_vals,
    float* __restrict__ cand_v, int32_t* __restrict__ cand_i, unsigned* __restrict__ counters) {
  constexpr int NP = kBF16 ? kHeadsWaves : 1;
  const int j = blockIdx.y, wg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int r_begin = wg * rows_per_wg;
  const int r_end = min(V, r_begin + rows_per_wg);
  const float NEG = -__builtin_huge_valf();

  __shared__ float red[2][NP][kMaxBatch][16];
  __shared__ TopkLists tl;
  __shared__ unsigned s_ticket;
  if (threadIdx.x < kMaxBatch) tl.count[threadIdx.x] = 0;
  __syncthreads();

  const int nsteps = (H + 31) / 32;
  const int s0 = wave * nsteps / kHeadsWaves, s1 = (wave + 1) * nsteps / kHeadsWaves;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  int buf = 0;
  for (int row0 = r_begin; row0 < r_end; row0 += 16) {
    if constexpr (kBF16) {
      const uint16_t* wlm = static_cast<const uint16_t*>(wlm_v);
      const int row = row0 + n;
      const bool row_ok = row < r_end;
      const uint16_t* wrow = wlm + (static_cast<size_t>(j) * V + (row_ok ? row : r_begin)) * H;
      // A operand: M row m = 2*bb + part of tile t holds the hi (part 0) or lo
      // (part 1) half of r[b = 8t + bb]; rows past the batch are zero.
      const float* arow[MT];
      bool a_ok[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int b = 8 * t + (n >> 1);
        a_ok[t] = b < B;
        arow[t] = r + (static_cast<size_t>(a_ok[t] ? b : 0) * K + j) * H;
      }
      const bool lo_part = (n & 1) != 0;
      f32x4 acc[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int s = s0; s < s1; s += kUnroll) {
        u32x4 wv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int k0 = (s + u) * 32 + g * 8;
          const bool ok = (s + u < s1) && (k0 < H) && row_ok;
          wv[u] = ok ? ld16_stream(wrow + k0) : zero;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int k0 = (s + u) * 32 + g * 8;
          const bool kok = (s + u < s1) && (k0 < H);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            u32x4 av = zero;
            if (kok && a_ok[t]) {
              const float4 x0 = *reinterpret_cast<const float4*>(arow[t] + k0);
              const float4 x1 = *reinterpret_cast<const float4*>(arow[t] + k0 + 4);
              const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
              uint32_t hb[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t hi = f32_to_bf16_bits(xs[e]);
                hb[e] = lo_part ? f32_to_bf16_bits(xs[e] - __uint_as_float(hi << 16)) : hi;
              }
              av = u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16),
                         hb[6] | (hb[7] << 16)};
            }
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(wv[u]), acc[t],
                                                              0, 0, 0);
          }
        }
      }
      // lane (g, n) holds C[4g + i][n]: sequences 8t + 2g (i = 0 hi, 1 lo)
      // and 8t + 2g + 1 (i = 2 hi, 3 lo) of row row0 + n.
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        red[buf][wave][8 * t + 2 * g][n] = acc[t][0] + acc[t][1];
        red[buf][wave][8 * t + 2 * g + 1][n] = acc[t][2] + acc[t][3];
      }
    } else {
      // f32 weights: wave w computes rows row0 + 4w .. +3 over the full H.
      const float* wlm = static_cast<const float*>(wlm_v);
      for (int q = 0; q < 4; ++q) {
        const int rn = wave * 4 + q;
        const int row = row0 + rn;
        float acc[kMaxBatch];
#pragma unroll
        for (int b = 0; b < kMaxBatch; ++b) acc[b] = 0.f;
        if (row < r_end) {
          const float* wrow = wlm + (static_cast<size_t>(j) * V + row) * H;
          for (int kk = lane * 4; kk < H; kk += kWave * 4) {
            const float4 w = *reinterpret_cast<const float4*>(wrow + kk);
#pragma unroll
            for (int b = 0; b < kMaxBatch; ++b) {
              if (b < B) {
                const float4 x = *reinterpret_cast<const float4*>(r + (static_cast<size_t>(b) * K + j) * H + kk);
                acc[b] += w.x * x.x + w.y * x.y + w.z * x.z + w.w * x.w;
              }
            }
          }
        }
#pragma unroll
        for (int b = 0; b < kMaxBatch; ++b) {
          if (b < B) {
            const float s = wave_sum(acc[b]);
            if (lane == 0) red[buf][0][b][rn] = s;
          }
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int row = row0 + n;
      const bool valid = lane < 16 && row < r_end;
      for (int b = 0; b < B; ++b) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NP; ++w) v += red[buf][w][b][n];
        if (valid && logits_out != nullptr)
          logits_out[(static_cast<size_t>(b) * K + j) * V + row] = v;
        volatile TopkLists& vtl = tl;
        const int c = vtl.count[b];
        const bool ok = valid && (v == v) &&
                        (c < k || beats(v, row, vtl.v[b][k - 1], vtl.id[b][k - 1]));
        const uint64_t m = ballot(ok);
        if (m) topk_insert(tl, b, k, v, row, m, lane);
      }
    }
    buf ^= 1;
  }
  __syncthreads();

  // publish this workgroup's lists
  if (wave == 0) {
    for (int b = 0; b < B; ++b) {
      const size_t base = ((static_cast<size_t>(j) * B + b) * G + wg) * k;
      if (lane < k) {
        volatile TopkLists& vtl = tl;
        const bool have = lane < vtl.count[b];
        cand_v[base + lane] = have ? vtl.v[b][lane] : NEG;
        cand_i[base + lane] = have ? vtl.id[b][lane] : -1;
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_ticket = atomicAdd(&counters[j], 1u);
  __syncthreads();
  if (s_ticket != static_cast<unsigned>(G - 1)) return;
  __threadfence();
  merge_head_lists(B, K, V, k, G, j, cand_v, cand_i, topk_ids, topk_vals);
  if (threadIdx.x == 0) counters[j] = 0u;
}

}  // namespace medusa

// ---------------------------------------------------------------- host side
namespace {

using namespace medusa;

constexpr size_t kCounterBytes = 256;

struct LmGrid {
  int rows_per_wg;
  int G;
};

// About four resident workgroups per CU over the whole grid; rows per
// workgroup a multiple of the 16-row tile.
LmGrid lm_grid(int V, int K) {
  const int target = 1024;
  int g0 = (target + K - 1) / K;
  if (g0 < 1) g0 = 1;
  int rows = (V + g0 - 1) / g0;
  rows = (rows + 15) / 16 * 16;
  if (rows < 16) rows = 16;
  LmGrid lg;
  lg.rows_per_wg = rows;
  lg.G = (V + rows - 1) / rows;
  return lg;
}

size_t cand_bytes(int B, int V, int K, int topk) {
  const LmGrid lg = lm_grid(V, K);
  return medusa_host::round_up(static_cast<size_t>(K) * B * lg.G * topk * 4, 256);
}

size_t r_bytes(int B, int K, int H) {
  return medusa_host::round_up(static_cast<size_t>(B) * K * H * 4, 256);
}

int check_heads_shape(const char* fn, int dtype, int B, int H, int V, int K, int topk) {
  MEDUSA_REQUIRE(dtype == MEDUSA_F32 || dtype == MEDUSA_BF16, MEDUSA_ERR_DTYPE, "%s: dtype %d", fn, dtype);
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d not in [1,%d]", fn, B, kMaxBatch);
  MEDUSA_REQUIRE(K >= 1 && K <= kMaxHeads, MEDUSA_ERR_SHAPE, "%s: K=%d not in [1,%d]", fn, K, kMaxHeads);
  MEDUSA_REQUIRE(H >= 8 && H <= (1 << 20), MEDUSA_ERR_SHAPE, "%s: H=%d", fn, H);
  MEDUSA_REQUIRE(H % (dtype == MEDUSA_BF16 ? 8 : 4) == 0, MEDUSA_ERR_SHAPE,
                 "%s: H=%d must be a multiple of %d", fn, H, dtype == MEDUSA_BF16 ? 8 : 4);
  if (V >= 0) {
    MEDUSA_REQUIRE(V >= 1 && V <= (1 << 24), MEDUSA_ERR_SHAPE, "%s: V=%d", fn, V);
    MEDUSA_REQUIRE(topk >= 1 && topk <= kMaxTopk && topk <= V, MEDUSA_ERR_SHAPE,
                   "%s: topk=%d not in [1, min(%d, V)]", fn, topk, kMaxTopk);
  }
  return MEDUSA_OK;
}

int launch_resblock(int dtype, int B, int H, int K, const void* hidden, const void* w1, const void* b1,
                    float* r, hipStream_t st) {
  dim3 grid((H + 15) / 16, K);
  if (dtype == MEDUSA_BF16) {
    hipLaunchKernelGGL(resblock_bf16_kernel, grid, dim3(kHeadsThreads), 0, st, B, H, K,
                       static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(w1),
                       static_cast<const uint16_t*>(b1), r);
  } else {
    hipLaunchKernelGGL(resblock_f32_kernel, grid, dim3(kHeadsThreads), 0, st, B, H, K,
                       static_cast<const float*>(hidden), static_cast<const float*>(w1),
                       static_cast<const float*>(b1), r);
  }
  return medusa_host::hip_check("medusa_resblock launch");
}

int launch_lm_topk(int dtype, int B, int H, int V, int K, int topk, const float* r, const void* w_lm,
                   int32_t* ids, float* vals, float* logits, void* ws, hipStream_t st) {
  const LmGrid lg = lm_grid(V, K);
  char* base = static_cast<char*>(ws);
  unsigned* counters = reinterpret_cast<unsigned*>(base);
  const size_t cb = cand_bytes(B, V, K, topk);
  float* cand_v = reinterpret_cast<float*>(base + kCounterBytes);
  int32_t* cand_i = reinterpret_cast<int32_t*>(base + kCounterBytes + cb);
  dim3 grid(lg.G, K);
  if (dtype == MEDUSA_BF16) {
    if (B <= 8)
      hipLaunchKernelGGL((lm_topk_kernel<true, 1>), grid, dim3(kHeadsThreads), 0, st, B, H, V, K, topk,
                         lg.rows_per_wg, lg.G, r, w_lm, logits, ids, vals, cand_v, cand_i, counters);
    else
      hipLaunchKernelGGL((lm_topk_kernel<true, 2>), grid, dim3(kHeadsThreads), 0, st, B, H, V, K, topk,
                         lg.rows_per_wg, lg.G, r, w_lm, logits, ids, vals, cand_v, cand_i, counters);
  } else {
    hipLaunchKernelGGL((lm_topk_kernel<false, 1>), grid, dim3(kHeadsThreads), 0, st, B, H, V, K, topk,
                       lg.rows_per_wg, lg.G, r, w_lm, logits, ids, vals, cand_v, cand_i, counters);
  }
  return medusa_host::hip_check("medusa_lm_head_topk launch");
}

size_t lm_ws_bytes(int B, int V, int K, int topk) { return kCounterBytes + 2 * cand_bytes(B, V, K, topk); }

}  // namespace

extern "C" size_t medusa_heads_workspace(int dtype, int B, int H, int V, int K, int topk) {
  if (check_heads_shape("medusa_heads_workspace", dtype, B, H, V, K, topk) != MEDUSA_OK) return 0;
  return lm_ws_bytes(B, V, K, topk) + r_bytes(B, K, H);
}

extern "C" int medusa_resblock(int dtype, int B, int H, int K, const void* hidden, const void* w1,
                               const void* b1, float* r, void* stream) {
  int rc = check_heads_shape(__func__, dtype, B, H, -1, K, 1);
  if (rc != MEDUSA_OK) return rc;
  MEDUSA_REQUIRE_PTR(hidden);
  MEDUSA_REQUIRE_PTR(w1);
  MEDUSA_REQUIRE_PTR(b1);
  MEDUSA_REQUIRE_PTR(r);
  return launch_resblock(dtype, B, H, K, hidden, w1, b1, r, static_cast<hipStream_t>(stream));
}

extern "C" int medusa_lm_head_topk(int dtype, int B, int H, int V, int K, int topk, const float* r,
                                   const void* w_lm, int32_t* topk_ids, float* topk_logits,
                                   float* logits_or_null, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_heads_shape(__func__, dtype, B, H, V, K, topk);
  if (rc != MEDUSA_OK) return rc;
  MEDUSA_REQUIRE_PTR(r);
  MEDUSA_REQUIRE_PTR(w_lm);
  MEDUSA_REQUIRE_PTR(topk_ids);
  MEDUSA_REQUIRE_PTR(topk_logits);
  MEDUSA_REQUIRE_PTR(ws);
  if (logits_or_null != nullptr) MEDUSA_REQUIRE_PTR(logits_or_null);
  MEDUSA_REQUIRE(ws_bytes >= lm_ws_bytes(B, V, K, topk), MEDUSA_ERR_WORKSPACE,
                 "%s: workspace %zu < %zu bytes", __func__, ws_bytes, lm_ws_bytes(B, V, K, topk));
  return launch_lm_topk(dtype, B, H, V, K, topk, r, w_lm, topk_ids, topk_logits, logits_or_null, ws,
                        static_cast<hipStream_t>(stream));
}

extern "C" int medusa_heads(int dtype, int B, int H, int V, int K, int topk, const void* hidden,
                            const void* w1, const void* b1, const void* w_lm, int32_t* topk_ids,
                            float* topk_logits, float* logits_or_null, float* r_or_null, void* ws,
                            size_t ws_bytes, void* stream) {
  int rc = check_heads_shape(__func__, dtype, B, H, V, K, topk);
  if (rc != MEDUSA_OK) return rc;
  MEDUSA_REQUIRE_PTR(hidden);
  MEDUSA_REQUIRE_PTR(w1);
  MEDUSA_REQUIRE_PTR(b1);
  MEDUSA_REQUIRE_PTR(w_lm);
  MEDUSA_REQUIRE_PTR(topk_ids);
  MEDUSA_REQUIRE_PTR(topk_logits);
  MEDUSA_REQUIRE_PTR(ws);
  if (logits_or_null != nullptr) MEDUSA_REQUIRE_PTR(logits_or_null);
  if (r_or_null != nullptr) MEDUSA_REQUIRE_PTR(r_or_null);
  const size_t need = lm_ws_bytes(B, V, K, topk) + r_bytes(B, K, H);
  MEDUSA_REQUIRE(ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__,
                 ws_bytes, need);
  float* r = r_or_null != nullptr
                 ? r_or_null
                 : reinterpret_cast<float*>(static_cast<char*>(ws) + lm_ws_bytes(B, V, K, topk));
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = launch_resblock(dtype, B, H, K, hidden, w1, b1, r, st);
  if (rc != MEDUSA_OK) return rc;
  return launch_lm_topk(dtype, B, H, V, K, topk, r, w_lm, topk_ids, topk_logits, logits_or_null, ws, st);
}
