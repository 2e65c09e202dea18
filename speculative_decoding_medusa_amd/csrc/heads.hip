// Medusa heads on gfx950: ResBlock GEMV and lm_head GEMV with fused top-k.
//
// Both stages are skinny matrix products (B <= 16 rows of activations
// against K*H resp. K*V weight rows), bound by streaming the weights from
// HBM once.  By shape:
//
//  * bf16, batch <= 2, H <= 8192 (the verify step's shape): row-diagonal
//    kernels.  Each wave streams whole weight rows (one 1 KB wave
//    instruction per 512 elements; the ResBlock's waves take contiguous
//    blocks of rows, the lm_head's interleave) and takes each row's dot
//    product as the trace of a v_mfma_f32_16x16x32_bf16 whose A operand
//    holds the activations at the same positions.  lm_head logits go into
//    per-wave top-k lists in registers; the last workgroup of each head to
//    finish (a device-scope arrival count; lists published with
//    write-through stores) merges them, so the call is one kernel.  With
//    that in-kernel merge, and H > 2048, the last seventh of each head's
//    rows is a pool handed out in blocks of four rows from a device-scope
//    counter, so that compute units whose loads return faster (some XCDs
//    stream about 10% faster than others) take more rows and all finish
//    together.
//  * bf16 otherwise: the ResBlock on a split-K MFMA kernel (four waves split
//    each 16-row tile's K range and reduce through LDS), and the lm_head on
//    the skinny-GEMM kernel of base_head.hip, the batch's hi/lo planes as
//    2B GEMM rows, each workgroup publishing the top-k of its 128-entry
//    vocabulary block; a merge kernel then finishes each (sequence, head).
//  * float32 weights: VALU kernels.
//
// The ResBlock output r is float32.  The bf16 MFMA needs bf16 operands, so
// r enters the lm_head as hi = bf16(r) and lo = bf16(r - hi), both against
// the exact bf16 weights with float32 sums: about 16 significant bits of r
// instead of 8.
#include <mutex>

#include "common.hpp"

namespace medusa {

constexpr int kHeadsThreads = 256;
constexpr int kHeadsWaves = kHeadsThreads / kWave;
constexpr int kUnroll = 8;          // 32-wide K steps issued back to back per wave

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

#ifndef MEDUSA_STREAM_NT
#define MEDUSA_STREAM_NT 1
#endif
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
#if MEDUSA_STREAM_NT
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}


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

// Wave-uniform insertion of the candidates held by the lanes in `mask` into
// one sorted list (values lv, ids li, length *cnt <= k).  A list is only
// touched by one wave, through LDS and without a barrier, so every access is
// volatile: each read is a real LDS read issued after the wave's earlier
// writes (LDS operations of one wave complete in order).
__device__ __forceinline__ void topk_insert_list(lds_vfloat* lv, lds_vint* li, lds_vint* cnt, int k, float v, int id,
                                                 uint64_t mask, int lane) {
  while (mask) {
    const int src = __ffsll(static_cast<unsigned long long>(mask)) - 1;
    mask &= mask - 1;
    const float cv = __shfl(v, src);
    const int ci = __shfl(id, src);
    const int c = *cnt;
    if (c == k && !beats(cv, ci, lv[k - 1], li[k - 1])) continue;
    const float ev = lane < c ? lv[lane] : 0.f;
    const int ei = lane < c ? li[lane] : 0;
    const int pos = __popcll(ballot(lane < c && beats(ev, ei, cv, ci)));
    const float pv = __shfl(ev, lane > 0 ? lane - 1 : 0);
    const int pi = __shfl(ei, lane > 0 ? lane - 1 : 0);
    const int nc = c + 1 < k ? c + 1 : k;
    if (lane < nc) {
      if (lane == pos) {
        lv[lane] = cv;
        li[lane] = ci;
      } else if (lane > pos) {
        lv[lane] = pv;
        li[lane] = pi;
      }
    }
    *cnt = nc;  // every lane stores the same value
  }
}

__device__ __forceinline__ void topk_insert(TopkLists& tl, int b, int k, float v, int id, uint64_t mask, int lane) {
  topk_insert_list((lds_vfloat*)tl.v[b], (lds_vint*)tl.id[b], (lds_vint*)&tl.count[b], k, v, id, mask, lane);
}

// The same insertion into a sorted list held in registers: lane t < cnt
// holds the list's t-th entry (cnt wave-uniform, k <= 64).  Each candidate
// and a full list's last entry are read out as scalars, so a candidate costs
// a few ALU operations and no memory access; one that beats entries moves
// them down one lane.
__device__ __forceinline__ void topk_reg_insert(float& lv, int& li, int& cnt, int k, float v, int id,
                                                uint64_t mask, int lane) {
  while (mask) {
    const int src = __ffsll(static_cast<unsigned long long>(mask)) - 1;
    mask &= mask - 1;
    const float cv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
    const int ci = __builtin_amdgcn_readlane(id, src);
    if (cnt == k && !beats(cv, ci, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), k - 1)),
                           __builtin_amdgcn_readlane(li, k - 1)))
      continue;
    const int pos = __popcll(ballot(lane < cnt && beats(lv, li, cv, ci)));
    const float pv = __shfl(lv, lane > 0 ? lane - 1 : 0);
    const int pi = __shfl(li, lane > 0 ? lane - 1 : 0);
    if (lane == pos) {
      lv = cv;
      li = ci;
    } else if (lane > pos) {
      lv = pv;
      li = pi;
    }
    cnt = cnt + 1 < k ? cnt + 1 : k;
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

// ------------------------------------------------------------- top-k merge
// Final top-k of one (sequence b, head j) from the `lists` sorted lists of k
// entries that the lm_head kernel published (a separate launch: the kernel
// boundary makes every list visible to this workgroup whatever XCD wrote
// it).  Selection runs on unique 64-bit keys whose unsigned order is the
// order of `beats`: the high word is the value's bit pattern made monotonic
// (+0 and -0 merged, as they compare equal), the low word the inverted
// token id, so equal values rank the smaller id first.  Key 0 means "no
// candidate" (an unused list slot; NaN is never a candidate).  The k-th
// largest key is found by radix selection, 8 bits per pass from the top:
// each pass histograms the keys that share the prefix chosen so far, one
// wave scans the 256 bins from the top to pick the bucket holding the
// still-needed rank, and selection stops as soon as the whole bucket is
// needed.  The keys >= the selected prefix are then exactly the top k
// (or every candidate, when there are fewer than k); each ranks itself
// against the others.
constexpr int kMergeThreads = 1024;
constexpr int kMergeMaxKeys = 32;  // keys per thread: lists * k <= 32768
constexpr int kFusedMergeKeys = 8;  // in-kernel merge: lists * k <= 256 * 8
constexpr int kGatherCounter = 32;  // arrival count of merged heads, after the per-head counts
// Dynamic row pool of the row-diagonal lm_head: per head a counter of handed
// out blocks, each counter in a 256-byte line of its own (heads do not
// contend for one atomic unit), after the 256 bytes of arrival counts.  The
// pool is about the last seventh of each head's rows, in blocks of four
// (measured at the Vicuna-7B shape against a static split: pools of 1/16,
// 1/10, 1/8, 1/7 and 1/5 with blocks of four: +1.1, -3.0, -3.0, -4.0, -3.9
// us; 1/10 with blocks of eight: -0.3 to +1.4 us).
constexpr int kDynCounterBase = 64;      // ints
constexpr int kDynCounterStride = 64;    // ints
constexpr int kDynBlock = 4;             // rows per block
constexpr int kDynPoolDiv = 7;           // pool: the last V / kDynPoolDiv rows, rounded down to whole strides

__device__ __forceinline__ uint64_t merge_key(float v, int id) {
  if (id < 0 || v != v) return 0;
  const uint32_t u = __float_as_uint(v);
  const uint32_t m = v == 0.f ? 0x80000000u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
  return (static_cast<uint64_t>(m) << 32) | static_cast<uint32_t>(~id);
}

__device__ __forceinline__ float merge_key_value(uint64_t x) {
  const uint32_t m = static_cast<uint32_t>(x >> 32);
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}

// Shared state of one radix selection.
struct MergeSmem {
  int hist[2][256];
  uint64_t prefix;
  int need, done, nsel;
  uint64_t keys[kMaxTopk];
};

// Top-k of the n candidates (cv, ci) by radix selection with NT threads
// (E keys each, n <= NT * E); writes k entries of oid / oval (-1 / -inf
// past the candidates).  Every thread of the workgroup calls it.
// COHERENT: the candidates are read, and the results written, with
// device-scope accesses (other workgroups of the running kernel wrote the
// lists, and may read the results).
template <int NT, int E, bool COHERENT>
__device__ __forceinline__ void radix_topk(const float* __restrict__ cv, const int* __restrict__ ci, int n, int k,
                                           int32_t* __restrict__ oid, float* __restrict__ oval, MergeSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // all loads first (clamped index, masked at use): one memory round trip;
  // COHERENT: lists written by other workgroups of the running kernel, read
  // with device-scope loads
  float v[E];
  int id[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int e = min(i * NT + tid, n - 1);
    if (COHERENT) {
      v[i] = __hip_atomic_load(cv + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      id[i] = __hip_atomic_load(ci + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      v[i] = cv[e];
      id[i] = ci[e];
    }
  }
  for (int x = tid; x < 256; x += NT) sm.hist[0][x] = 0;
  if (tid == 0) {
    sm.prefix = 0;
    sm.need = k;
    sm.done = 0;
    sm.nsel = 0;
  }
  uint64_t key[E];
#pragma unroll
  for (int i = 0; i < E; ++i) key[i] = i * NT + tid < n ? merge_key(v[i], id[i]) : 0;
  __syncthreads();

  for (int p = 0; p < 8; ++p) {
    const int shift = 56 - 8 * p;
    const uint64_t prefix = sm.prefix;
    int* h = sm.hist[p & 1];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint64_t x = key[i];
      const bool match = x != 0 && (p == 0 || (x >> (shift + 8)) == (prefix >> (shift + 8)));
      if (match) atomicAdd(&h[static_cast<int>(x >> shift) & 255], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 255-4l .. 252-4l (best first)
      int c[4];
      int sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = h[255 - 4 * lane - q];
        sum += c[q];
      }
      const int incl = wave_incl_scan_i32(sum);
      const int need = sm.need;
      const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
      if (total < need) {
        // fewer candidates than k (first pass only): take them all
        if (lane == 0) {
          sm.prefix = 1;
          sm.done = 1;
        }
      } else if (incl - sum < need && need <= incl) {
        int acc = incl - sum;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (acc < need && need <= acc + c[q]) {
            const int rest = need - acc;
            sm.prefix = prefix | (static_cast<uint64_t>(255 - 4 * lane - q) << shift);
            sm.need = rest;
            sm.done = c[q] == rest ? 1 : 0;
          }
          acc += c[q];
        }
      }
    } else {
      for (int x = tid - kWave; x < 256; x += NT - kWave) sm.hist[(p + 1) & 1][x] = 0;
    }
    __syncthreads();
    if (sm.done) break;
  }

  const uint64_t thr = sm.prefix;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (key[i] != 0 && key[i] >= thr) sm.keys[atomicAdd(&sm.nsel, 1)] = key[i];
  }
  __syncthreads();
  const int S = sm.nsel;  // <= k
  int slot = -1, oi = -1;
  float ov = -__builtin_huge_valf();
  if (tid < S) {
    const uint64_t x = sm.keys[tid];
    int rank = 0;
    for (int t = 0; t < S; ++t) rank += sm.keys[t] > x ? 1 : 0;
    slot = rank;
    oi = static_cast<int32_t>(~static_cast<uint32_t>(x));
    ov = merge_key_value(x);
  } else if (tid < k) {
    slot = tid;
  }
  if (slot >= 0) {
    if (COHERENT) {   // write-through: read back by another workgroup of the running kernel
      __hip_atomic_store(oid + slot, oi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(oval + slot, ov, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      oid[slot] = oi;
      oval[slot] = ov;
    }
  }
}

template <int E>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(int B, int K, int k, int lists,
                                                                   const float* __restrict__ cand_v,
                                                                   const int* __restrict__ cand_i,
                                                                   int32_t* __restrict__ topk_ids,
                                                                   float* __restrict__ topk_vals) {
  const int b = blockIdx.x, j = blockIdx.y;
  const int n = lists * k;
  const size_t base = (static_cast<size_t>(j) * B + b) * n;
  __shared__ MergeSmem sm;
  radix_topk<kMergeThreads, E, false>(cand_v + base, cand_i + base, n, k,
                                      topk_ids + (static_cast<size_t>(b) * K + j) * k,
                               topk_vals + (static_cast<size_t>(b) * K + j) * k, sm);
}

// Candidate sets beyond kMergeThreads * kMergeMaxKeys: k rounds of
// block-wide "best entry ranked after the previous pick" over global memory.
__global__ __launch_bounds__(kMergeThreads) void topk_merge_rounds_kernel(int B, int K, int k, int lists,
                                                                          const float* __restrict__ cand_v,
                                                                          const int* __restrict__ cand_i,
                                                                          int32_t* __restrict__ topk_ids,
                                                                          float* __restrict__ topk_vals) {
  const int b = blockIdx.x, j = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = lists * k;
  const size_t base = (static_cast<size_t>(j) * B + b) * n;
  int32_t* oid = topk_ids + (static_cast<size_t>(b) * K + j) * k;
  float* oval = topk_vals + (static_cast<size_t>(b) * K + j) * k;
  __shared__ float redv[kMergeThreads / kWave];
  __shared__ int redi[kMergeThreads / kWave];
  const float NEG = -__builtin_huge_valf();
  const int NONE = 0x7fffffff;
  float lv = __builtin_huge_valf();
  int li = -1;
  for (int round = 0; round < k; ++round) {
    float bv = NEG;
    int bi = NONE;
    bool found = false;
    for (int e = tid; e < n; e += kMergeThreads) {
      const int id = cand_i[base + e];
      const float v = cand_v[base + e];
      if (id < 0 || v != v) continue;
      if ((round == 0 || beats(lv, li, v, id)) && (!found || beats(v, id, bv, bi))) {
        bv = v;
        bi = id;
        found = true;
      }
    }
    block_best(bv, bi, redv, redi);
    if (tid == 0) {
      oid[round] = bi == NONE ? -1 : bi;
      oval[round] = bi == NONE ? NEG : bv;
    }
    lv = bv;
    li = bi;
  }
}

// ------------------------------------------------------------------ K2
// float32 weights.  Grid (G, K).  Workgroup wg of head j owns rows
// [wg*rows_per_wg, ...) of Wlm[j], walked in 16-row tiles; wave w computes
// rows row0 + 4w .. +3 over the full H.  (bf16 weights take the row-diagonal
// kernel at batch <= 2 and the skinny-GEMM kernel otherwise.)
__global__ __launch_bounds__(kHeadsThreads) void lm_topk_f32_kernel(
    int B, int H, int V, int K, int k, int rows_per_wg, int G,
    const float* __restrict__ r, const float* __restrict__ wlm,
    float* __restrict__ logits_out, int32_t* __restrict__ topk_ids, float* __restrict__ topk_vals,
    float* __restrict__ cand_v, int32_t* __restrict__ cand_i) {
  const int j = blockIdx.y, wg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int r_begin = wg * rows_per_wg;
  const int r_end = min(V, r_begin + rows_per_wg);
  const float NEG = -__builtin_huge_valf();

  __shared__ float red[2][kMaxBatch][16];
  __shared__ TopkLists tl;
  if (threadIdx.x < kMaxBatch) tl.count[threadIdx.x] = 0;
  __syncthreads();

  int buf = 0;
  for (int row0 = r_begin; row0 < r_end; row0 += 16) {
    {
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
            if (lane == 0) red[buf][b][rn] = s;
          }
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int row = row0 + n;
      const bool valid = lane < 16 && row < r_end;
      for (int b = 0; b < B; ++b) {
        const float v = red[buf][b][n];
        if (valid && logits_out != nullptr)
          logits_out[(static_cast<size_t>(b) * K + j) * V + row] = v;
        lds_vfloat* lvb = (lds_vfloat*)tl.v[b];
        lds_vint* lib = (lds_vint*)tl.id[b];
        const int c = *(lds_vint*)&tl.count[b];
        const bool ok = valid && (v == v) && (c < k || beats(v, row, lvb[k - 1], lib[k - 1]));
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
        const bool have = lane < *(lds_vint*)&tl.count[b];
        cand_v[base + lane] = have ? ((lds_vfloat*)tl.v[b])[lane] : NEG;
        cand_i[base + lane] = have ? ((lds_vint*)tl.id[b])[lane] : -1;
      }
    }
  }
}

// ------------------------------------------------------- K2, row-diagonal
// bf16 lm_head for B <= 2 and H <= 512 * 16, streaming whole weight rows.
//
// Lane l = 16g + n loads the 16 bytes of a row at element 512s + 8l, so one
// wave instruction reads 1 KB of one row contiguously, in lane order, and a
// row is NST = H/512 such loads.  The A operand holds r at the same
// positions, so in C = A B the diagonal entry C[n][n] sums the products of
// the four lanes with that n (the MFMA pairs A lane (g, m) with B lane
// (g, n) over k): the trace of C accumulated over s is the row's logit.
// Only the diagonal is used, but at two MFMAs (r's hi and lo bf16 halves)
// per KB the matrix cores stay far below the time the KB takes to arrive.
// Each wave streams rows w, w + S, w + 2S, ... of its head (w its index
// among the head's S waves: see DiagRows), row loads double-buffered in
// registers; r's split planes stay in registers for
// the whole kernel.  Logits of 64 consecutive rows gather one per lane and
// are offered to the wave's top-k lists together.
// The rows a wave streams: n rows r0, r0 + rs, ... of `total`.  With
// row_stride 1 each wave takes its own contiguous block of rows_per_wave
// rows; with row_stride = the waves per head, wave w takes rows w, w + rs,
// ..., so at any moment the waves of a head read neighbouring rows and the
// head's reads sweep its weights front to back (fewer DRAM pages and
// translations open at once than a thousand scattered streams).  row(i)
// clamps to the wave's last row (to row `total` - 1 for a wave with none),
// so prefetches past the end stay in bounds.
struct DiagRows {
  int r0, rs, n;
  __device__ __forceinline__ int row(int i) const {
    const int last = n > 0 ? r0 + (n - 1) * rs : r0;
    return min(min(r0 + i * rs, last), total_m1);
  }
  int total_m1;
};

__device__ __forceinline__ DiagRows diag_rows(int wv, int rows_per_wave, int row_stride, int total) {
  DiagRows d;
  d.total_m1 = total - 1;
  if (row_stride <= 1) {
    d.r0 = wv * rows_per_wave;
    d.rs = 1;
    d.n = max(0, min(rows_per_wave, total - d.r0));
  } else {
    d.r0 = wv;
    d.rs = row_stride;
    d.n = wv < total ? (total - 1 - wv) / row_stride + 1 : 0;
  }
  return d;
}

__host__ __device__ constexpr int diag_nstmax(int nst) { return nst <= 4 ? 4 : (nst <= 8 ? 8 : (nst <= 13 ? 13 : 16)); }

template <int NSTMAX>
__device__ __forceinline__ void diag_load_row(const uint16_t* __restrict__ wrow, int H, int e0, u32x4 (&buf)[NSTMAX]) {
#pragma unroll
  for (int s = 0; s < NSTMAX; ++s) buf[s] = ld16_stream(wrow + static_cast<uint32_t>(min(512 * s + e0, H - 8)));
}

// Trace of a 16x16 MFMA result.  Lane (g, n) holds C[4g + i][n] in a[i], so
// C[n][n] is component n % 4 of lane 16 (n / 4) + n: the diagonal fills the
// four whole quads of lanes 0-3, 20-23, 40-43 and 60-63, quad lane i holding
// it in a[i].  Each quad's first lane gathers its neighbours' components with
// DPP quad broadcasts; the four quad sums are read as scalars.  The result
// is wave-uniform.
__device__ __forceinline__ float diag_trace(const f32x4& a) {
  float d = a[0];
  d += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a[1]), 0x55, 0xf, 0xf, true));  // quad_perm(1,1,1,1)
  d += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a[2]), 0xAA, 0xf, 0xf, true));  // quad_perm(2,2,2,2)
  d += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a[3]), 0xFF, 0xf, 0xf, true));  // quad_perm(3,3,3,3)
  const int x = __float_as_int(d);
  return (__int_as_float(__builtin_amdgcn_readlane(x, 0)) + __int_as_float(__builtin_amdgcn_readlane(x, 20))) +
         (__int_as_float(__builtin_amdgcn_readlane(x, 40)) + __int_as_float(__builtin_amdgcn_readlane(x, 60)));
}

// Logits of one streamed row against r's hi and lo bf16 planes: both planes
// accumulate into one chain (the matrix core pipelines a dependent
// accumulator), then one trace.  With REFILL, each 16-byte piece of the
// buffer is reloaded from `next` as soon as its two MFMAs have read it, so a
// wave keeps close to two rows of loads in flight through the chain instead
// of one (the scheduling barriers pin that order).  FULL: H is exactly
// NSTMAX * 512, so no piece lies past the row and no select is needed;
// otherwise such pieces (clamped reloads of the row's last 16 bytes) are
// replaced by zeros.
template <int NSTMAX, int NB, bool FULL, bool REFILL>
__device__ __forceinline__ void diag_row_logits(u32x4 (&buf)[NSTMAX], const u32x4 (&ahi)[NB][NSTMAX],
                                                const u32x4 (&alo)[NB][NSTMAX], int H, int e0,
                                                const uint16_t* __restrict__ next, float (&logit)[NB]) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NSTMAX; ++s) {
    const u32x4 w = (FULL || 512 * s + e0 < H) ? buf[s] : zero;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ahi[b][s]), as_bf16x8(w), acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(alo[b][s]), as_bf16x8(w), acc[b], 0, 0, 0);
    }
    if (REFILL) {
      buf[s] = ld16_stream(next + static_cast<uint32_t>(min(512 * s + e0, H - 8)));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) logit[b] = diag_trace(acc[b]);
}

// Dot products of one streamed row with a bf16 vector held in one plane
// (exact): same lane layout, trace and piecewise refill as diag_row_logits.
template <int NSTMAX, int NB, bool FULL, bool REFILL>
__device__ __forceinline__ void diag_row_dot(u32x4 (&buf)[NSTMAX], const u32x4 (&a)[NB][NSTMAX], int H, int e0,
                                             const uint16_t* __restrict__ next, float (&dot)[NB]) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NSTMAX; ++s) {
    const u32x4 w = (FULL || 512 * s + e0 < H) ? buf[s] : zero;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[b][s]), as_bf16x8(w), acc[b], 0, 0, 0);
    if (REFILL) {
      buf[s] = ld16_stream(next + static_cast<uint32_t>(min(512 * s + e0, H - 8)));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) dot[b] = diag_trace(acc[b]);
}

// Put a wave-uniform value into lane `slot` (uniform) of v.
__device__ __forceinline__ float put_lane(float v, float x, int slot) {
  return static_cast<int>(threadIdx.x & 63) == slot ? x : v;
}

// ------------------------------------------------------- K1, row-diagonal
// bf16 ResBlock for B <= 2 and H <= 512 * 16: each wave streams its own
// contiguous block of W1[j] rows (double-buffered whole rows, 1 KB per wave
// instruction) against h, gathers one row's dot product per lane, and every
// 64 rows (and at the end) applies r = h + SiLU(dot + b1) to the gathered
// rows in parallel, one coalesced store per sequence.
template <int NSTMAX, int NB, bool FULL>
__global__ __launch_bounds__(kHeadsThreads) void resblock_diag_kernel(int B, int H, int K, int rows_per_wave,
                                                                      int row_stride,
                                                                      const uint16_t* __restrict__ hidden,
                                                                      const uint16_t* __restrict__ w1,
                                                                      const uint16_t* __restrict__ b1,
                                                                      float* __restrict__ r) {
  const int j = blockIdx.y, wg = blockIdx.x;
  // the wave index made uniform: rows, addresses and gather slots in scalars
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e0 = 8 * lane;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 ah[NB][NSTMAX];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int s = 0; s < NSTMAX; ++s)
      ah[b][s] = (b < B && 512 * s + e0 < H) ? ld16(hidden + static_cast<size_t>(b) * H + 512 * s + e0) : zero;

  const DiagRows dr = diag_rows(wg * kHeadsWaves + wave, rows_per_wave, row_stride, H);
  if (dr.n == 0) return;
  const uint16_t* wbase = w1 + static_cast<size_t>(j) * H * H;
  float gath[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) gath[b] = 0.f;

  // row i of the wave's sequence: its dot product into lane i % 64; every
  // 64 rows (and at the end) the gathered rows are finished in parallel
  auto take = [&](int i, const float (&dot)[NB]) {
    const int slot = i & 63;
#pragma unroll
    for (int b = 0; b < NB; ++b) gath[b] = put_lane(gath[b], dot[b], slot);
    if (slot == 63 || i == dr.n - 1) {
      const int myrow = dr.r0 + (i - slot + lane) * dr.rs;
      if (lane <= slot) {
        const float bias = bf16_to_f32(b1[static_cast<size_t>(j) * H + myrow]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < B) {
            const float u = gath[b] + bias;
            const float h = bf16_to_f32(hidden[static_cast<size_t>(b) * H + myrow]);
            r[(static_cast<size_t>(b) * K + j) * H + myrow] = h + u / (1.0f + expf(-u));
          }
        }
      }
    }
  };

  // rotated double buffer, as in the row-diagonal lm_head kernel
  u32x4 wa[NSTMAX], wb[NSTMAX];
  float dot[NB];
  diag_load_row<NSTMAX>(wbase + static_cast<size_t>(dr.row(0)) * H, H, e0, wa);
  diag_load_row<NSTMAX>(wbase + static_cast<size_t>(dr.row(1)) * H, H, e0, wb);
  int i = 0;
  for (; i + 1 < dr.n; i += 2) {
    __builtin_amdgcn_sched_barrier(0);
    diag_row_dot<NSTMAX, NB, FULL, true>(wa, ah, H, e0, wbase + static_cast<size_t>(dr.row(i + 2)) * H, dot);
    take(i, dot);
    __builtin_amdgcn_sched_barrier(0);
    diag_row_dot<NSTMAX, NB, FULL, true>(wb, ah, H, e0, wbase + static_cast<size_t>(dr.row(i + 3)) * H, dot);
    take(i + 1, dot);
  }
  if (i < dr.n) {
    diag_row_dot<NSTMAX, NB, FULL, false>(wa, ah, H, e0, wbase, dot);
    take(i, dot);
  }
}

template <int NSTMAX, int NB, bool FULL>
__global__ __launch_bounds__(kHeadsThreads) void lm_topk_diag_kernel(
    int B, int H, int V, int K, int k, int rows_per_wave, int row_stride, int G, const float* __restrict__ r,
    const uint16_t* __restrict__ wlm, float* __restrict__ logits_out, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_vals, float* __restrict__ cand_v, int32_t* __restrict__ cand_i,
    int* __restrict__ counters, int fuse, TreeGather tg) {
  const int j = blockIdx.y, wg = blockIdx.x;
  // the wave index made uniform: rows, addresses and gather slots in scalars
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // lane l owns elements [512s + 8l, +8): one wave instruction reads 1 KB in
  // lane order (fully coalesced); any one-to-one assignment of 8-element
  // pieces to lanes gives the same trace as long as A uses the same one
  const int e0 = 8 * lane;
  const float NEG = -__builtin_huge_valf();
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // a wave with no rows (n == 0) still loads a valid row (dr.row clamps)
  const DiagRows dr = diag_rows(wg * kHeadsWaves + wave, rows_per_wave, row_stride, V);
  const uint16_t* wbase = wlm + static_cast<size_t>(j) * V * H;
  // With the in-kernel merge the head's rows split into a static part, rows
  // [0, pool0) interleaved over its waves as above, and a pool [pool0, V)
  // handed out in blocks of kDynBlock rows, in order, from a device-scope
  // counter: compute units whose loads return faster take more blocks.
  // (rows of H > 2048 only: shorter rows make a block too short to hide its
  // grab, and at H 1024 the pool cost 10 us a call, 47.8 against 58.2 us)
  const bool dyn = NSTMAX >= 8 && fuse != 0 && row_stride > 1;
  const int pool0 = dyn ? ((V - V / kDynPoolDiv) / row_stride) * row_stride : V;
  const int ns = dyn ? min(dr.n, (pool0 - dr.r0 + row_stride - 1) / row_stride) : dr.n;
  int* const dyn_ctr = counters + kDynCounterBase + j * kDynCounterStride;
  int graw = 0;   // lane 0: the block index of the pending grab
  if (dyn && lane == 0) graw = __hip_atomic_fetch_add(dyn_ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // Prologue in one memory round trip: a round of r loads (clamped, with no
  // branch, so all are in flight together), the block's first two weight
  // rows, then r's split into exact bf16 hi/lo planes at this lane's
  // positions while the rows arrive.  Larger r (two sequences, wide rows)
  // takes further rounds of eight 32-byte pieces.
  constexpr int P = NB * NSTMAX;
  constexpr int GR = P < 8 ? P : 8;
  u32x4 ahi[NB][NSTMAX], alo[NB][NSTMAX];
  u32x4 wa[NSTMAX], wb[NSTMAX];
#pragma unroll
  for (int p0 = 0; p0 < P; p0 += GR) {
    float4 x[GR][2];
#pragma unroll
    for (int q = 0; q < GR; ++q) {
      const int p = p0 + q;
      if (p < P) {
        const int b = p / NSTMAX, s = p % NSTMAX;
        const float* src = r + (static_cast<size_t>(min(b, B - 1)) * K + j) * H + min(512 * s + e0, H - 8);
        x[q][0] = *reinterpret_cast<const float4*>(src);
        x[q][1] = *reinterpret_cast<const float4*>(src + 4);
      }
    }
    if (p0 == 0) {
      diag_load_row<NSTMAX>(wbase + static_cast<size_t>(dr.row(0)) * H, H, e0, wa);
      diag_load_row<NSTMAX>(wbase + static_cast<size_t>(dr.row(1)) * H, H, e0, wb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < GR; ++q) {
      const int p = p0 + q;
      if (p < P) {
        const int b = p / NSTMAX, s = p % NSTMAX;
        const bool valid = b < B && 512 * s + e0 < H;
        const float xs[8] = {x[q][0].x, x[q][0].y, x[q][0].z, x[q][0].w,
                             x[q][1].x, x[q][1].y, x[q][1].z, x[q][1].w};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hw[e] = pack_bf16x2(xs[2 * e], xs[2 * e + 1]);
          lw[e] = pack_bf16x2(xs[2 * e] - __uint_as_float(hw[e] << 16),
                              xs[2 * e + 1] - __uint_as_float(hw[e] & 0xffff0000u));
        }
        ahi[b][s] = valid ? u32x4{hw[0], hw[1], hw[2], hw[3]} : zero;
        alo[b][s] = valid ? u32x4{lw[0], lw[1], lw[2], lw[3]} : zero;
      }
    }
  }

  // per sequence: gathered logits, and the wave's sorted top-k list in
  // registers (lane t holds entry t)
  float gath[NB], lv[NB];
  int li[NB], cnt[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    gath[b] = NEG;
    lv[b] = NEG;
    li[b] = -1;
    cnt[b] = 0;
  }

  // gather the logits of row i of the wave's sequence into lane i % 64;
  // flush every 64 rows
  int gid = 0;   // the row whose logit this lane's slot holds
  auto flush = [&](int slot) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b >= B) continue;
      const float v = gath[b];
      bool ok = lane <= slot && (v == v);
      if (cnt[b] == k)
        ok = ok && beats(v, gid, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv[b]), k - 1)),
                         __builtin_amdgcn_readlane(li[b], k - 1));
      const uint64_t m = ballot(ok);
      if (m) topk_reg_insert(lv[b], li[b], cnt[b], k, v, gid, m, lane);
      gath[b] = NEG;
    }
  };
  // the i-th row of the wave (row id `row`) into slot i % 64; flush every 64
  auto offer = [&](int i, int row, const float (&lg)[NB]) {
    const int slot = i & 63;
    gid = lane == slot ? row : gid;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      gath[b] = put_lane(gath[b], lg[b], slot);
      if (logits_out != nullptr && lane == 0 && b < B) logits_out[(static_cast<size_t>(b) * K + j) * V + row] = lg[b];
    }
    if (slot == 63) flush(63);
  };

  // Rotated double buffer: both buffers are in flight before the loop, and
  // each piece is refilled with the row two ahead as soon as its MFMAs have
  // read it, so every MFMA waits only for the piece it consumes, with about
  // two rows of loads still in flight.  Loads past the block reload its last
  // row (an L2 hit) so that no load is conditional.  An empty block runs
  // neither the loop nor the tail; with no branch around both, the
  // prologue's loads cannot be sunk below its conversions.
  float lg[NB];
  int i = 0;
  for (; i + 1 < ns; i += 2) {
    __builtin_amdgcn_sched_barrier(0);
    diag_row_logits<NSTMAX, NB, FULL, true>(wa, ahi, alo, H, e0,
                                            wbase + static_cast<size_t>(dr.row(min(i + 2, ns - 1))) * H, lg);
    offer(i, dr.r0 + i * dr.rs, lg);
    __builtin_amdgcn_sched_barrier(0);
    diag_row_logits<NSTMAX, NB, FULL, true>(wb, ahi, alo, H, e0,
                                            wbase + static_cast<size_t>(dr.row(min(i + 3, ns - 1))) * H, lg);
    offer(i + 1, dr.r0 + (i + 1) * dr.rs, lg);
  }
  if (i < ns) {
    diag_row_logits<NSTMAX, NB, FULL, false>(wa, ahi, alo, H, e0, wbase, lg);
    offer(i, dr.r0 + i * dr.rs, lg);
    ++i;
  }
  if (dyn) {
    // The pool, a block at a time.  The grab for the next block goes out as
    // a block starts and its value is first read (through an empty asm, so
    // the read is not hoisted) when the refills reach the block's end:
    // those loads of the next block's first rows keep the pipeline full.
    asm volatile("" : "+v"(graw));
    int blk = pool0 + __builtin_amdgcn_readfirstlane(graw) * kDynBlock;
    if (blk < V) {
      diag_load_row<NSTMAX>(wbase + static_cast<size_t>(blk) * H, H, e0, wa);
      diag_load_row<NSTMAX>(wbase + static_cast<size_t>(min(blk + 1, V - 1)) * H, H, e0, wb);
    }
    while (blk < V) {
      int nraw = 0;
      if (lane == 0) nraw = __hip_atomic_fetch_add(dyn_ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int nblk = V;
#pragma unroll
      for (int t = 0; t < kDynBlock; t += 2) {
        if (t + 2 == kDynBlock) {
          asm volatile("" : "+v"(nraw));
          nblk = pool0 + __builtin_amdgcn_readfirstlane(nraw) * kDynBlock;
        }
        const int ra = t + 2 < kDynBlock ? blk + t + 2 : nblk;
        const int rb = t + 3 < kDynBlock ? blk + t + 3 : nblk + 1;
        __builtin_amdgcn_sched_barrier(0);
        diag_row_logits<NSTMAX, NB, FULL, true>(wa, ahi, alo, H, e0, wbase + static_cast<size_t>(min(ra, V - 1)) * H,
                                                lg);
        if (blk + t < V) offer(i++, blk + t, lg);
        __builtin_amdgcn_sched_barrier(0);
        diag_row_logits<NSTMAX, NB, FULL, true>(wb, ahi, alo, H, e0, wbase + static_cast<size_t>(min(rb, V - 1)) * H,
                                                lg);
        if (blk + t + 1 < V) offer(i++, blk + t + 1, lg);
      }
      blk = nblk;
    }
  }
  if ((i & 63) != 0) flush((i - 1) & 63);
  // every wave publishes its own lists (list wg * 4 + wave of head j)
  const int nlists = G * kHeadsWaves;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b >= B) continue;
    const size_t base = ((static_cast<size_t>(j) * B + b) * nlists + wg * kHeadsWaves + wave) * k;
    if (lane < k) {
      const bool have = lane < cnt[b];
      const float pv = have ? lv[b] : NEG;
      const int pi = have ? li[b] : -1;
      if (fuse) {
        __hip_atomic_store(cand_v + base + lane, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(cand_i + base + lane, pi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        cand_v[base + lane] = pv;
        cand_i[base + lane] = pi;
      }
    }
  }
  if (!fuse) return;
  // The last workgroup of head j to finish merges the head's lists.  Lists
  // are written and read with device-scope (write-through) accesses, so no
  // cache-wide writeback or invalidation is needed: each wave waits for its
  // stores to complete before the workgroup's arrival is counted, and the
  // count is reset for the next call.
  __shared__ MergeSmem sm;
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(counters + j, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1 ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) __hip_atomic_store(counters + kDynCounterBase + j * kDynCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int n = nlists * k;
  for (int b = 0; b < B; ++b) {
    const size_t base = (static_cast<size_t>(j) * B + b) * n;
    radix_topk<kHeadsThreads, kFusedMergeKeys, true>(cand_v + base, cand_i + base, n, k,
                                                     topk_ids + (static_cast<size_t>(b) * K + j) * k,
                                                     topk_vals + (static_cast<size_t>(b) * K + j) * k, sm);
    __syncthreads();
  }
  if (threadIdx.x == 0) __hip_atomic_store(counters + j, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tg.T == 0) return;
  // The tree gather, by the merging workgroup of the last head to finish:
  // this head's top-k is written through; count it, and the workgroup that
  // completes the count reads every head's (device scope) and gathers.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(counters + kGatherCounter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     K - 1
                 ? 1
                 : 0;
  __syncthreads();
  if (!s_last) return;
  for (int x = threadIdx.x; x < B * tg.T; x += kHeadsThreads) {
    const int b = x / tg.T, t = x - b * tg.T;
    const int ti = tg.tree_indices[t];
    const bool in = ti >= 1 && ti <= K * k;
    const int tok = in ? __hip_atomic_load(topk_ids + static_cast<size_t>(b) * K * k + (ti - 1), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)
                       : tg.root_token[b];
    tg.tree_candidates[x] = tok;
    tg.position_ids[x] = tg.prefix_len[b] + tg.depth[t];
  }
  if (threadIdx.x == 0) __hip_atomic_store(counters + kGatherCounter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace medusa

// ---------------------------------------------------------------- host side
namespace {

using namespace medusa;

// Workspace header: one arrival count per head for the in-kernel merge
// (zero before the first call; every call leaves it zero).
constexpr size_t kCounterBytes = 256 + kMaxHeads * kDynCounterStride * 4;

struct LmGrid {
  bool diag;       // row-diagonal kernel (B <= 2)
  bool gemm;       // bf16 otherwise: the skinny-GEMM kernel with a top-k epilogue
  int nst;         // 512-element steps per row
  int rows_per_wave;
  int rows_per_wg; // f32 kernel
  int G;           // workgroups per head
  int lists;       // published top-k lists per head (per wave, per vocabulary block or per workgroup)
};

// Resident waves per SIMD the row-diagonal lm_head grid is sized for: one
// measured best at the Vicuna-7B shape (fewer loads in flight per compute
// unit, fewer lists to merge; two per SIMD: 207 us against 204.6 us).
constexpr int kDiagWavesPerSimd = 1;
constexpr int kMaxWavesPerSimd = 8;

// Grid of the lm_head kernel for `wps` resident waves per SIMD: sized so that
// every wave is resident at once (one round, no tail).  The launch passes the
// kernel's actual occupancy; workspace sizes use kMaxWavesPerSimd, an upper
// bound on G.
LmGrid lm_grid(int dtype, int B, int H, int V, int K, int topk, int wps) {
  LmGrid lg{};
  lg.nst = (H + 511) / 512;
  lg.diag = dtype == MEDUSA_BF16 && B <= 2 && lg.nst <= 16;
  // workgroups per head: the K heads share 256 CUs x wps resident
  // workgroups, rounded down so the whole grid is one round
  long long wgh = 256LL * wps / K;
  if (wgh < 1) wgh = 1;
  lg.gemm = dtype == MEDUSA_BF16 && !lg.diag;
  if (lg.gemm) {   // one list per (head, sequence, 128-entry vocabulary block)
    lg.G = medusa_host::heads_gemm_lists(V);
    lg.lists = lg.G;
    return lg;
  }
  if (lg.diag) {
    long long rpw = (V + kHeadsWaves * wgh - 1) / (kHeadsWaves * wgh);
    const long long min_rpw = (V + kHeadsWaves * 1024LL - 1) / (kHeadsWaves * 1024LL);
    if (rpw < min_rpw) rpw = min_rpw;
    lg.rows_per_wave = static_cast<int>(rpw);
    lg.G = static_cast<int>((V + kHeadsWaves * rpw - 1) / (kHeadsWaves * rpw));
    lg.lists = lg.G * kHeadsWaves;
    return lg;
  }
  // float32 weights: about four resident workgroups per CU over the grid
  const int target = 1024;
  int g0 = (target + K - 1) / K;
  if (g0 < 1) g0 = 1;
  int rows = (V + g0 - 1) / g0;
  rows = (rows + 15) / 16 * 16;
  if (rows < 16) rows = 16;
  lg.rows_per_wg = rows;
  lg.G = (V + rows - 1) / rows;
  lg.lists = lg.G;
  return lg;
}

// Resident workgroups (= waves per SIMD for 4-wave workgroups) of a kernel,
// queried once per kernel and cached.
template <typename F>
int occupancy_wps(F kernel, size_t dyn_lds) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, kHeadsThreads, dyn_lds) != hipSuccess ||
      blocks < 1)
    blocks = 1;
  return blocks > kMaxWavesPerSimd ? kMaxWavesPerSimd : blocks;
}

size_t cand_bytes(int dtype, int B, int H, int V, int K, int topk) {
  const LmGrid lg = lm_grid(dtype, B, H, V, K, topk, kMaxWavesPerSimd);
  return medusa_host::round_up(static_cast<size_t>(K) * B * lg.lists * topk * 4, 256);
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

// Rows of W1 per wave for the row-diagonal ResBlock: `wps` waves per SIMD,
// all resident at once, at least one row each.  One wave per SIMD measured
// best at the Vicuna-7B shape: fewer, longer contiguous streams.
constexpr int kResblockWavesPerSimd = 1;

int resblock_rows_per_wave(int H, int K, int wps) {
  long long wgh = 256LL * wps / K;   // workgroups per head, one round over 256 CUs
  if (wgh < 1) wgh = 1;
  long long rpw = (H + kHeadsWaves * wgh - 1) / (kHeadsWaves * wgh);
  return static_cast<int>(rpw < 1 ? 1 : rpw);
}

// Row order of the row-diagonal kernels with G workgroups per head.  The
// lm_head (V rows of 8 KB per head at H 4096) interleaves its waves over the
// rows: 204.6 us per call at the Vicuna-7B shape against 207.6-209 us with a
// contiguous block per wave.  The ResBlock (H rows, about twenty per wave)
// measured 0.3-0.6 us faster with contiguous blocks, and keeps them.
int lm_row_stride(int G) { return G * kHeadsWaves; }
int res_row_stride(int /*G*/) { return 1; }

int launch_resblock(int dtype, int B, int H, int K, const void* hidden, const void* w1, const void* b1,
                    float* r, hipStream_t st) {
  const int nst = (H + 511) / 512;
  if (dtype == MEDUSA_BF16 && B <= 2 && nst <= 16) {
    const uint16_t* hh = static_cast<const uint16_t*>(hidden);
    const uint16_t* ww = static_cast<const uint16_t*>(w1);
    const uint16_t* bb = static_cast<const uint16_t*>(b1);
#define MEDUSA_RES_LAUNCH(NS, NB)                                                                          \
  do {                                                                                                     \
    const int rpw = resblock_rows_per_wave(H, K, kResblockWavesPerSimd);                                   \
    const int G = (H + kHeadsWaves * rpw - 1) / (kHeadsWaves * rpw);                                       \
    if (H == (NS) * 512)                                                                                   \
      hipLaunchKernelGGL((resblock_diag_kernel<NS, NB, true>), dim3(G, K), dim3(kHeadsThreads), 0, st, B, H, \
                         K, rpw, res_row_stride(G), hh, ww, bb, r);                                         \
    else                                                                                                   \
      hipLaunchKernelGGL((resblock_diag_kernel<NS, NB, false>), dim3(G, K), dim3(kHeadsThreads), 0, st, B, \
                         H, K, rpw, res_row_stride(G), hh, ww, bb, r);                                      \
  } while (0)
    const int ns = diag_nstmax(nst);
    if (ns == 4) {
      if (B == 1) MEDUSA_RES_LAUNCH(4, 1); else MEDUSA_RES_LAUNCH(4, 2);
    } else if (ns == 8) {
      if (B == 1) MEDUSA_RES_LAUNCH(8, 1); else MEDUSA_RES_LAUNCH(8, 2);
    } else if (ns == 13) {
      if (B == 1) MEDUSA_RES_LAUNCH(13, 1); else MEDUSA_RES_LAUNCH(13, 2);
    } else {
      if (B == 1) MEDUSA_RES_LAUNCH(16, 1); else MEDUSA_RES_LAUNCH(16, 2);
    }
#undef MEDUSA_RES_LAUNCH
    return medusa_host::hip_check("medusa_resblock launch");
  }
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

// The merge kernel over `lists` published lists of k per (sequence, head).
int launch_topk_merge(int B, int K, int topk, int lists, const float* cand_v, const int32_t* cand_i, int32_t* ids,
                      float* vals, hipStream_t st) {
  const int per = (lists * topk + kMergeThreads - 1) / kMergeThreads;
  const dim3 mg(B, K), mb(kMergeThreads);
  if (per <= 1)
    hipLaunchKernelGGL(topk_merge_kernel<1>, mg, mb, 0, st, B, K, topk, lists, cand_v, cand_i, ids, vals);
  else if (per <= 2)
    hipLaunchKernelGGL(topk_merge_kernel<2>, mg, mb, 0, st, B, K, topk, lists, cand_v, cand_i, ids, vals);
  else if (per <= 4)
    hipLaunchKernelGGL(topk_merge_kernel<4>, mg, mb, 0, st, B, K, topk, lists, cand_v, cand_i, ids, vals);
  else if (per <= 8)
    hipLaunchKernelGGL(topk_merge_kernel<8>, mg, mb, 0, st, B, K, topk, lists, cand_v, cand_i, ids, vals);
  else if (per <= 16)
    hipLaunchKernelGGL(topk_merge_kernel<16>, mg, mb, 0, st, B, K, topk, lists, cand_v, cand_i, ids, vals);
  else if (per <= kMergeMaxKeys)
    hipLaunchKernelGGL(topk_merge_kernel<kMergeMaxKeys>, mg, mb, 0, st, B, K, topk, lists, cand_v, cand_i, ids,
                       vals);
  else
    hipLaunchKernelGGL(topk_merge_rounds_kernel, mg, mb, 0, st, B, K, topk, lists, cand_v, cand_i, ids, vals);
  return medusa_host::hip_check("medusa_lm_head_topk merge launch");
}

// tg (optional): the tree gather after the top-k, inside the lm_head kernel
// where its merge runs there, else as a launch of its own.
int launch_lm_topk(int dtype, int B, int H, int V, int K, int topk, const float* r, const void* w_lm,
                   int32_t* ids, float* vals, float* logits, void* ws, hipStream_t st,
                   const TreeGather* tg = nullptr) {
  const TreeGather none{};
  LmGrid lg = lm_grid(dtype, B, H, V, K, topk, kMaxWavesPerSimd);
  char* base = static_cast<char*>(ws);
  const size_t cb = cand_bytes(dtype, B, H, V, K, topk);
  int* counters = reinterpret_cast<int*>(base);
  float* cand_v = reinterpret_cast<float*>(base + kCounterBytes);
  int32_t* cand_i = reinterpret_cast<int32_t*>(base + kCounterBytes + cb);
  bool fused = false;
  if (lg.gemm) {
    uint16_t* planes = reinterpret_cast<uint16_t*>(base + kCounterBytes + 2 * cb);
    int rc = medusa_host::heads_lm_gemm(B, H, V, K, topk, r, w_lm, 0, logits, planes, cand_v, cand_i, st);
    if (rc != MEDUSA_OK) return rc;
  } else if (lg.diag) {
    const uint16_t* w = static_cast<const uint16_t*>(w_lm);
#define MEDUSA_DIAG_LAUNCH(NS, NB)                                                                            \
  do {                                                                                                        \
    lg = lm_grid(dtype, B, H, V, K, topk, kDiagWavesPerSimd);                                                 \
    fused = lg.lists * topk <= kHeadsThreads * kFusedMergeKeys;                                               \
    if (H == (NS) * 512)                                                                                      \
      hipLaunchKernelGGL((lm_topk_diag_kernel<NS, NB, true>), dim3(lg.G, K), dim3(kHeadsThreads), 0, st, B, H,  \
                         V, K, topk, lg.rows_per_wave, lm_row_stride(lg.G), lg.G, r, w, logits, ids, vals,    \
                         cand_v, cand_i, counters, fused ? 1 : 0, fused && tg != nullptr ? *tg : none);         \
    else                                                                                                      \
      hipLaunchKernelGGL((lm_topk_diag_kernel<NS, NB, false>), dim3(lg.G, K), dim3(kHeadsThreads), 0, st, B, H, \
                         V, K, topk, lg.rows_per_wave, lm_row_stride(lg.G), lg.G, r, w, logits, ids, vals,    \
                         cand_v, cand_i, counters, fused ? 1 : 0, fused && tg != nullptr ? *tg : none);         \
  } while (0)
    const int ns = diag_nstmax(lg.nst);
    if (ns == 4) {
      if (B == 1) MEDUSA_DIAG_LAUNCH(4, 1); else MEDUSA_DIAG_LAUNCH(4, 2);
    } else if (ns == 8) {
      if (B == 1) MEDUSA_DIAG_LAUNCH(8, 1); else MEDUSA_DIAG_LAUNCH(8, 2);
    } else if (ns == 13) {
      if (B == 1) MEDUSA_DIAG_LAUNCH(13, 1); else MEDUSA_DIAG_LAUNCH(13, 2);
    } else {
      if (B == 1) MEDUSA_DIAG_LAUNCH(16, 1); else MEDUSA_DIAG_LAUNCH(16, 2);
    }
#undef MEDUSA_DIAG_LAUNCH
  } else {
    hipLaunchKernelGGL(lm_topk_f32_kernel, dim3(lg.G, K), dim3(kHeadsThreads), 0, st, B, H, V, K, topk,
                       lg.rows_per_wg, lg.G, r, static_cast<const float*>(w_lm), logits, ids, vals, cand_v, cand_i);
  }
  int rc = medusa_host::hip_check("medusa_lm_head_topk launch");
  if (rc != MEDUSA_OK) return rc;
  if (!fused) {
    rc = launch_topk_merge(B, K, topk, lg.lists, cand_v, cand_i, ids, vals, st);
    if (rc != MEDUSA_OK) return rc;
  }
  if (tg != nullptr && !fused) return medusa_host::launch_tree_candidates(B, K, topk, ids, *tg, st);
  return MEDUSA_OK;
}

// the GEMM path's hi/lo planes of r, [K][2B][H] bf16
size_t planes_bytes(int dtype, int B, int H, int V, int K, int topk) {
  if (!lm_grid(dtype, B, H, V, K, topk, kMaxWavesPerSimd).gemm) return 0;
  return medusa_host::round_up(static_cast<size_t>(K) * 2 * B * H * 2, 256);
}

// the skinny-GEMM path as medusa_lm_head_topk_packed takes it at any batch
size_t gemm_cand_bytes(int B, int V, int K, int topk) {
  return medusa_host::round_up(static_cast<size_t>(K) * B * medusa_host::heads_gemm_lists(V) * topk * 4, 256);
}
size_t gemm_ws_bytes(int B, int H, int V, int K, int topk) {
  return kCounterBytes + 2 * gemm_cand_bytes(B, V, K, topk) +
         medusa_host::round_up(static_cast<size_t>(K) * 2 * B * H * 2, 256);
}

size_t lm_ws_bytes(int dtype, int B, int H, int V, int K, int topk) {
  const size_t own = kCounterBytes + 2 * cand_bytes(dtype, B, H, V, K, topk) + planes_bytes(dtype, B, H, V, K, topk);
  if (dtype != MEDUSA_BF16) return own;
  const size_t g = gemm_ws_bytes(B, H, V, K, topk);
  return own > g ? own : g;
}

// medusa_heads_packed: the ResBlock's split partial sums, [S][K][B][H] float32
size_t res_part_bytes(int B, int H, int K) {
  return medusa_host::round_up(
      static_cast<size_t>(medusa_host::heads_res_splits(H, K)) * K * B * H * sizeof(float), 256);
}

// the tail of the workspace: r (medusa_heads) or the partial sums (packed)
size_t tail_bytes(int dtype, int B, int H, int K) {
  const size_t rb = r_bytes(B, K, H);
  if (dtype != MEDUSA_BF16) return rb;
  const size_t pb = res_part_bytes(B, H, K);
  return rb > pb ? rb : pb;
}

}  // namespace

extern "C" size_t medusa_heads_workspace(int dtype, int B, int H, int V, int K, int topk) {
  if (check_heads_shape("medusa_heads_workspace", dtype, B, H, V, K, topk) != MEDUSA_OK) return 0;
  return lm_ws_bytes(dtype, B, H, V, K, topk) + tail_bytes(dtype, B, H, K);
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

namespace {

// Arguments of the tree gather shared by the *_tree calls.
int check_tree_gather(const char* fn, int T, const int32_t* tree_indices, const int32_t* depth,
                      const int32_t* root_token, const int32_t* prefix_len, const int32_t* tree_candidates,
                      const int32_t* position_ids, const int32_t* topk_ids) {
  MEDUSA_REQUIRE(T >= 1 && T <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: T=%d", fn, T);
#define MEDUSA_ARG_PTR(p)                                                                   \
  do {                                                                                     \
    MEDUSA_REQUIRE((p) != nullptr, MEDUSA_ERR_NULL, "%s: %s is NULL", fn, #p);             \
    MEDUSA_REQUIRE(medusa_host::aligned16(p), MEDUSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)
  MEDUSA_ARG_PTR(tree_indices);
  MEDUSA_ARG_PTR(depth);
  MEDUSA_ARG_PTR(root_token);
  MEDUSA_ARG_PTR(prefix_len);
  MEDUSA_ARG_PTR(tree_candidates);
  MEDUSA_ARG_PTR(position_ids);
#undef MEDUSA_ARG_PTR
  MEDUSA_REQUIRE(tree_candidates != position_ids && tree_candidates != topk_ids && position_ids != topk_ids,
                 MEDUSA_ERR_ALIAS, "%s: tree_candidates, position_ids and topk_ids must not alias", fn);
  return MEDUSA_OK;
}

}  // namespace

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
  MEDUSA_REQUIRE(ws_bytes >= lm_ws_bytes(dtype, B, H, V, K, topk), MEDUSA_ERR_WORKSPACE,
                 "%s: workspace %zu < %zu bytes", __func__, ws_bytes, lm_ws_bytes(dtype, B, H, V, K, topk));
  return launch_lm_topk(dtype, B, H, V, K, topk, r, w_lm, topk_ids, topk_logits, logits_or_null, ws,
                        static_cast<hipStream_t>(stream));
}

extern "C" int medusa_lm_head_topk_tree(int dtype, int B, int H, int V, int K, int topk, const float* r,
                                        const void* w_lm, int32_t* topk_ids, float* topk_logits,
                                        float* logits_or_null, int T, const int32_t* tree_indices,
                                        const int32_t* depth, const int32_t* root_token, const int32_t* prefix_len,
                                        int32_t* tree_candidates, int32_t* position_ids, void* ws, size_t ws_bytes,
                                        void* stream) {
  int rc = check_heads_shape(__func__, dtype, B, H, V, K, topk);
  if (rc != MEDUSA_OK) return rc;
  MEDUSA_REQUIRE_PTR(r);
  MEDUSA_REQUIRE_PTR(w_lm);
  MEDUSA_REQUIRE_PTR(topk_ids);
  MEDUSA_REQUIRE_PTR(topk_logits);
  if (logits_or_null != nullptr) MEDUSA_REQUIRE_PTR(logits_or_null);
  rc = check_tree_gather(__func__, T, tree_indices, depth, root_token, prefix_len, tree_candidates, position_ids,
                         topk_ids);
  if (rc != MEDUSA_OK) return rc;
  MEDUSA_REQUIRE_PTR(ws);
  MEDUSA_REQUIRE(ws_bytes >= lm_ws_bytes(dtype, B, H, V, K, topk), MEDUSA_ERR_WORKSPACE,
                 "%s: workspace %zu < %zu bytes", __func__, ws_bytes, lm_ws_bytes(dtype, B, H, V, K, topk));
  const TreeGather tg{T, tree_indices, depth, root_token, prefix_len, tree_candidates, position_ids};
  return launch_lm_topk(dtype, B, H, V, K, topk, r, w_lm, topk_ids, topk_logits, logits_or_null, ws,
                        static_cast<hipStream_t>(stream), &tg);
}

extern "C" int medusa_lm_head_topk_packed(int dtype, int B, int H, int V, int K, int topk, const float* r,
                                          const void* w_lm_packed, int32_t* topk_ids, float* topk_logits,
                                          float* logits_or_null, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_heads_shape(__func__, dtype, B, H, V, K, topk);
  if (rc != MEDUSA_OK) return rc;
  MEDUSA_REQUIRE(dtype == MEDUSA_BF16, MEDUSA_ERR_DTYPE, "%s: packed weights are bf16", __func__);
  MEDUSA_REQUIRE(H <= (1 << 16), MEDUSA_ERR_SHAPE, "%s: H=%d", __func__, H);
  MEDUSA_REQUIRE_PTR(r);
  MEDUSA_REQUIRE_PTR(w_lm_packed);
  MEDUSA_REQUIRE_PTR(topk_ids);
  MEDUSA_REQUIRE_PTR(topk_logits);
  MEDUSA_REQUIRE_PTR(ws);
  if (logits_or_null != nullptr) MEDUSA_REQUIRE_PTR(logits_or_null);
  MEDUSA_REQUIRE(ws_bytes >= lm_ws_bytes(dtype, B, H, V, K, topk), MEDUSA_ERR_WORKSPACE,
                 "%s: workspace %zu < %zu bytes", __func__, ws_bytes, lm_ws_bytes(dtype, B, H, V, K, topk));
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const size_t cb = gemm_cand_bytes(B, V, K, topk);
  float* cand_v = reinterpret_cast<float*>(base + kCounterBytes);
  int32_t* cand_i = reinterpret_cast<int32_t*>(base + kCounterBytes + cb);
  uint16_t* planes = reinterpret_cast<uint16_t*>(base + kCounterBytes + 2 * cb);
  rc = medusa_host::heads_lm_gemm(B, H, V, K, topk, r, w_lm_packed, 1, logits_or_null, planes, cand_v, cand_i, st);
  if (rc != MEDUSA_OK) return rc;
  return launch_topk_merge(B, K, topk, medusa_host::heads_gemm_lists(V), cand_v, cand_i, topk_ids, topk_logits, st);
}

namespace {

// Both stages of medusa_heads on a validated workspace of at least
// lm_ws_bytes + tail_bytes bytes.
int run_heads(int dtype, int B, int H, int V, int K, int topk, const void* hidden, const void* w1, const void* b1,
              const void* w_lm, int32_t* topk_ids, float* topk_logits, float* logits_or_null, float* r_or_null,
              void* ws, hipStream_t st, const TreeGather* tg = nullptr) {
  float* r = r_or_null != nullptr
                 ? r_or_null
                 : reinterpret_cast<float*>(static_cast<char*>(ws) + lm_ws_bytes(dtype, B, H, V, K, topk));
  int rc = launch_resblock(dtype, B, H, K, hidden, w1, b1, r, st);
  if (rc != MEDUSA_OK) return rc;
  return launch_lm_topk(dtype, B, H, V, K, topk, r, w_lm, topk_ids, topk_logits, logits_or_null, ws, st, tg);
}

int check_heads_args(const char* fn, int dtype, int B, int H, int V, int K, int topk, const void* hidden,
                     const void* w1, const void* b1, const void* w_lm, const int32_t* topk_ids,
                     const float* topk_logits, const float* logits_or_null, const float* r_or_null) {
  int rc = check_heads_shape(fn, dtype, B, H, V, K, topk);
  if (rc != MEDUSA_OK) return rc;
#define MEDUSA_ARG_PTR(p)                                                                   \
  do {                                                                                     \
    MEDUSA_REQUIRE((p) != nullptr, MEDUSA_ERR_NULL, "%s: %s is NULL", fn, #p);             \
    MEDUSA_REQUIRE(medusa_host::aligned16(p), MEDUSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)
  MEDUSA_ARG_PTR(hidden);
  MEDUSA_ARG_PTR(w1);
  MEDUSA_ARG_PTR(b1);
  MEDUSA_ARG_PTR(w_lm);
  MEDUSA_ARG_PTR(topk_ids);
  MEDUSA_ARG_PTR(topk_logits);
  if (logits_or_null != nullptr) MEDUSA_ARG_PTR(logits_or_null);
  if (r_or_null != nullptr) MEDUSA_ARG_PTR(r_or_null);
#undef MEDUSA_ARG_PTR
  return MEDUSA_OK;
}

}  // namespace

extern "C" int medusa_heads(int dtype, int B, int H, int V, int K, int topk, const void* hidden,
                            const void* w1, const void* b1, const void* w_lm, int32_t* topk_ids,
                            float* topk_logits, float* logits_or_null, float* r_or_null, void* ws,
                            size_t ws_bytes, void* stream) {
  int rc = check_heads_args(__func__, dtype, B, H, V, K, topk, hidden, w1, b1, w_lm, topk_ids, topk_logits,
                            logits_or_null, r_or_null);
  if (rc != MEDUSA_OK) return rc;
  MEDUSA_REQUIRE_PTR(ws);
  const size_t need = lm_ws_bytes(dtype, B, H, V, K, topk) + tail_bytes(dtype, B, H, K);
  MEDUSA_REQUIRE(ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__,
                 ws_bytes, need);
  return run_heads(dtype, B, H, V, K, topk, hidden, w1, b1, w_lm, topk_ids, topk_logits, logits_or_null, r_or_null,
                   ws, static_cast<hipStream_t>(stream));
}

extern "C" int medusa_heads_tree(int dtype, int B, int H, int V, int K, int topk, const void* hidden,
                                 const void* w1, const void* b1, const void* w_lm, int32_t* topk_ids,
                                 float* topk_logits, float* logits_or_null, float* r_or_null, int T,
                                 const int32_t* tree_indices, const int32_t* depth, const int32_t* root_token,
                                 const int32_t* prefix_len, int32_t* tree_candidates, int32_t* position_ids,
                                 void* ws, size_t ws_bytes, void* stream) {
  int rc = check_heads_args(__func__, dtype, B, H, V, K, topk, hidden, w1, b1, w_lm, topk_ids, topk_logits,
                            logits_or_null, r_or_null);
  if (rc != MEDUSA_OK) return rc;
  rc = check_tree_gather(__func__, T, tree_indices, depth, root_token, prefix_len, tree_candidates, position_ids,
                         topk_ids);
  if (rc != MEDUSA_OK) return rc;
  MEDUSA_REQUIRE_PTR(ws);
  const size_t need = lm_ws_bytes(dtype, B, H, V, K, topk) + tail_bytes(dtype, B, H, K);
  MEDUSA_REQUIRE(ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__,
                 ws_bytes, need);
  const TreeGather tg{T, tree_indices, depth, root_token, prefix_len, tree_candidates, position_ids};
  return run_heads(dtype, B, H, V, K, topk, hidden, w1, b1, w_lm, topk_ids, topk_logits, logits_or_null, r_or_null,
                   ws, static_cast<hipStream_t>(stream), &tg);
}

extern "C" int medusa_heads_packed(int dtype, int B, int H, int V, int K, int topk, const void* hidden,
                                   const void* w1_packed, const void* b1, const void* w_lm_packed,
                                   int32_t* topk_ids, float* topk_logits, float* logits_or_null, float* r_or_null,
                                   void* ws, size_t ws_bytes, void* stream) {
  int rc = check_heads_shape(__func__, dtype, B, H, V, K, topk);
  if (rc != MEDUSA_OK) return rc;
  MEDUSA_REQUIRE(dtype == MEDUSA_BF16, MEDUSA_ERR_DTYPE, "%s: packed weights are bf16", __func__);
  MEDUSA_REQUIRE(H <= (1 << 16), MEDUSA_ERR_SHAPE, "%s: H=%d", __func__, H);
  MEDUSA_REQUIRE_PTR(hidden);
  MEDUSA_REQUIRE_PTR(w1_packed);
  MEDUSA_REQUIRE_PTR(b1);
  MEDUSA_REQUIRE_PTR(w_lm_packed);
  MEDUSA_REQUIRE_PTR(topk_ids);
  MEDUSA_REQUIRE_PTR(topk_logits);
  MEDUSA_REQUIRE_PTR(ws);
  if (logits_or_null != nullptr) MEDUSA_REQUIRE_PTR(logits_or_null);
  if (r_or_null != nullptr) MEDUSA_REQUIRE_PTR(r_or_null);
  const size_t lm = lm_ws_bytes(dtype, B, H, V, K, topk), need = lm + tail_bytes(dtype, B, H, K);
  MEDUSA_REQUIRE(ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes,
                 need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const size_t cb = gemm_cand_bytes(B, V, K, topk);
  float* cand_v = reinterpret_cast<float*>(base + kCounterBytes);
  int32_t* cand_i = reinterpret_cast<int32_t*>(base + kCounterBytes + cb);
  uint16_t* planes = reinterpret_cast<uint16_t*>(base + kCounterBytes + 2 * cb);
  float* part = reinterpret_cast<float*>(base + lm);
  rc = medusa_host::heads_res_gemm(B, H, K, static_cast<const uint16_t*>(hidden), w1_packed,
                                   static_cast<const uint16_t*>(b1), r_or_null, part, planes, st);
  if (rc != MEDUSA_OK) return rc;
  rc = medusa_host::heads_lm_gemm(B, H, V, K, topk, nullptr, w_lm_packed, 1, logits_or_null, planes, cand_v, cand_i,
                                  st);
  if (rc != MEDUSA_OK) return rc;
  return launch_topk_merge(B, K, topk, medusa_host::heads_gemm_lists(V), cand_v, cand_i, topk_ids, topk_logits, st);
}

// ---------------------------------------------------------------- medusa_heads_noalloc
// medusa_heads for callers that cannot allocate (code under graph capture,
// tight serving loops): the workspace is one file-scope device array per
// GPU instead of a caller buffer.  In host code the array's name is only a
// stand-in; its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept, and only that
// address is ever handed to a kernel.

namespace {
constexpr size_t kHeadsScratchBytes = MEDUSA_HEADS_NOALLOC_SCRATCH_BYTES;   // per GPU
constexpr int kScratchDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kHeadsScratchBytes];

namespace {

// The arrival counts at the head of the scratch start at zero.
__global__ __launch_bounds__(64) void scratch_clear_kernel(uint32_t* p, int n) {
  for (int x = static_cast<int>(threadIdx.x); x < n; x += 64) p[x] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];

// Device address of this GPU's scratch.  The first call on a device looks
// it up (with that device current) and clears the arrival counts with a
// fill kernel on `st`; every later call on the device reuses the address.
int heads_scratch(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kScratchDevices) {
    medusa_host::set_error("medusa_heads_noalloc: no usable current device (%s, device %d)",
                           hipGetErrorString(e), dev);
    return MEDUSA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      medusa_host::set_error("medusa_heads_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
      return MEDUSA_ERR_HIP;
    }
    hipLaunchKernelGGL(scratch_clear_kernel, dim3(1), dim3(64), 0, st, static_cast<uint32_t*>(p),
                       static_cast<int>(kCounterBytes / 4));
    const int rc = medusa_host::hip_check("medusa_heads_noalloc scratch clear");
    if (rc != MEDUSA_OK) return rc;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MEDUSA_OK;
}

}  // namespace

extern "C" int medusa_heads_noalloc(int dtype, int B, int H, int V, int K, int topk, const void* hidden,
                                    const void* w1, const void* b1, const void* w_lm, int32_t* topk_ids,
                                    float* topk_logits, float* logits_or_null, float* r_or_null, void* stream) {
  int rc = check_heads_args(__func__, dtype, B, H, V, K, topk, hidden, w1, b1, w_lm, topk_ids, topk_logits,
                            logits_or_null, r_or_null);
  if (rc != MEDUSA_OK) return rc;
  const size_t need = lm_ws_bytes(dtype, B, H, V, K, topk) + tail_bytes(dtype, B, H, K);
  MEDUSA_REQUIRE(need <= kHeadsScratchBytes, MEDUSA_ERR_WORKSPACE,
                 "%s: this shape needs %zu bytes of scratch, more than the %zu bytes held per GPU", __func__, need,
                 kHeadsScratchBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  rc = heads_scratch(st, &ws);
  if (rc != MEDUSA_OK) return rc;
  return run_heads(dtype, B, H, V, K, topk, hidden, w1, b1, w_lm, topk_ids, topk_logits, logits_or_null, r_or_null,
                   ws, st);
}
