// Nucleus (top-p) acceptance on gfx950.
//
// Per tree node: p = softmax(logits / temperature); the nucleus is the
// shortest prefix of the vocabulary ordered by p descending (ties by token
// id) whose mass reaches top_p; one token is drawn from it by inverse CDF
// in token-id order with the caller's uniform.  A child is then accepted
// exactly when its token equals its parent's draw, and the step's next
// token is the draw at the last accepted node -- the greedy decision with
// the draw in place of the argmax, so the decide kernel of the posterior
// runs unchanged on the draws.
//
// One workgroup per node; each thread holds a contiguous chunk of the row
// in registers (loaded once when the row fits 256 x 128 tokens) and every
// walk runs over the chunks:
//   0. the row maximum (masses are exp((x - max) / temperature), held as
//      fixed-point integers so every sum is exact and order-independent);
//   1-3. radix select by MASS on the order key of x: 11, 11, then 10 bits;
//      each walk adds the masses of the keys that share the digits chosen
//      so far into per-wave LDS histograms (the whole mass S on the first
//      walk), and one wave then picks the highest bucket at which the mass
//      from the top reaches what is still needed.  The result is the
//      boundary key kappa: every key above it is in the nucleus, and the
//      first c tokens (by id) with key kappa complete it;
//   4. the nucleus mass Z, and target = floor(u * Z);
//   5. a workgroup scan of the chunks' nucleus masses in id order: the one
//      thread whose interval holds the target walks its chunk to the token.
#include "common.hpp"

namespace medusa {

constexpr int kNucThreads = 256;
constexpr int kNucWaves = kNucThreads / kWave;
constexpr int kNucBuckets = 2048;           // 11-bit digits
constexpr int kNucMaxV = 1 << 18;           // fixed-point sums stay below 2^58
static_assert(kNucWaves == 4, "the block reductions below combine four waves");

// Masses are exp((x - max) / temperature) in (0, 1], held as fixed-point
// integers with 40 fraction bits: every sum below is exact and independent
// of the order of the additions (at most 2^18 tokens: sums < 2^58).
typedef unsigned long long u64;

// Order key of a float: larger value, larger key (both zeros map to +0).
__device__ __forceinline__ uint32_t nuc_key(float x) {
  const uint32_t b = x == 0.f ? 0u : __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float nuc_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Wave reductions and scans on DPP lane moves (common.hpp).
__device__ __forceinline__ int wave_min_i(int v) { return wave_reduce_i32_dpp<false>(v); }

__device__ __forceinline__ int wave_max_i(int v) { return wave_reduce_i32_dpp<true>(v); }

__device__ __forceinline__ u64 wave_sum_u64(u64 v) { return readlane_u64(wave_incl_scan_u64(v), kWave - 1); }

// Inclusive scan across the wave's lanes in lane order.
template <typename X>
__device__ __forceinline__ X wave_incl_scan(X v, int) {
  static_assert(sizeof(X) == 8 || sizeof(X) == 4, "64- or 32-bit sums");
  if constexpr (sizeof(X) == 8)
    return static_cast<X>(wave_incl_scan_u64(static_cast<uint64_t>(v)));
  else
    return static_cast<X>(wave_incl_scan_i32(static_cast<int>(v)));
}

// Bucket choice for one digit (called by one whole wave): among buckets
// [0, nb) of `h` (masses), the highest d with h[d] > 0 whose mass from the
// top through d reaches `need`; if there is none, the lowest d with
// h[d] > 0.  Returns d and, in `above`, the mass of the buckets above d.
__device__ __forceinline__ int nuc_pick(const u64* h, int nb, u64 need, int lane, u64& above) {
  const int per = nb / kWave;
  const int lo = lane * per;
  u64 local = 0;
  for (int i = 0; i < per; ++i) local += h[lo + i];
  // mass of the lanes above this one: the wave's total less the lanes up to
  // and including this one
  const u64 incl = wave_incl_scan(local, lane);
  u64 run = readlane_u64(incl, kWave - 1) - incl;
  int cand = -1, low = 0x7fffffff;
  u64 cand_above = 0, low_above = 0;
  for (int i = per - 1; i >= 0; --i) {
    const u64 m = h[lo + i];
    if (m > 0) {
      if (cand < 0 && run + m >= need) {
        cand = lo + i;
        cand_above = run;
      }
      low = lo + i;
      low_above = run;
    }
    run += m;
  }
  int d = wave_max_i(cand);
  u64 a = cand_above;
  if (d < 0) {
    d = wave_min_i(low);
    a = low_above;
  }
  // the owning lane's value to every lane
  const uint64_t owner = ballot(lo <= d && d < lo + per);
  above = readlane_u64(a, owner ? __builtin_ctzll(owner) : 0);
  return d;
}

__device__ __forceinline__ u64 block_sum_u64(u64 v, u64* sh, int lane, int wave) {
  v = wave_sum_u64(v);
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  const u64 r = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return r;
}

// Exclusive scan over the workgroup's threads in thread order; `total` gets
// the sum of all.
template <typename X>
__device__ __forceinline__ X block_excl_scan(X v, X* sh, int lane, int wave, X& total) {
  const X inc = wave_incl_scan(v, lane);
  if (lane == kWave - 1) sh[wave] = inc;
  __syncthreads();
  X off = 0;
  for (int w = 0; w < wave; ++w) off += sh[w];
  total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return off + inc - v;
}

// One workgroup per node.  Thread tid holds tokens [SEG s + E tid, + E) of
// segment s in registers (SEG = 256 E); a row of at most SEG tokens is
// loaded once and every walk runs from registers, a longer one is reloaded
// segment by segment on each walk.
template <int E>
__global__ __launch_bounds__(kNucThreads) void nucleus_sample_kernel(int V, const float* __restrict__ logits,
                                                                   float temperature, float top_p,
                                                                   const float* __restrict__ uniforms,
                                                                   RowStat* __restrict__ stats,
                                                                   int32_t* __restrict__ samples) {
  constexpr int SEG = kNucThreads * E;
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* x = logits + static_cast<size_t>(row) * V;
  const int nseg = (V + SEG - 1) / SEG;
  __shared__ u64 s_hist[kNucWaves][kNucBuckets];
  __shared__ u64 s_u64[kNucWaves];
  __shared__ int s_int[kNucWaves];
  __shared__ float s_max[kNucWaves];
  __shared__ int s_digit;
  __shared__ u64 s_need;
  __shared__ int s_sample;

  float xr[E];
  auto load = [&](int s) {
    const int b = s * SEG + E * tid;
#pragma unroll
    for (int j = 0; j < E; ++j) xr[j] = x[min(b + j, V - 1)];
  };
  auto ok = [&](int s, int j) { return s * SEG + E * tid + j < V; };
  if (nseg == 1) load(0);

  // (0) row maximum
  float mx = -__builtin_huge_valf();
  for (int s = 0; s < nseg; ++s) {
    if (nseg > 1) load(s);
#pragma unroll
    for (int j = 0; j < E; ++j)
      if (ok(s, j)) mx = fmaxf(mx, xr[j]);
  }
  mx = wave_max(mx);
  if (lane == 0) s_max[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float sc = (1.f / temperature) * 1.44269504088896341f;   // log2(e) / temperature
  // mass of a token, 40 fraction bits: exp((x - max) / temperature)
  auto mass = [&](float v) -> u64 { return static_cast<u64>(exp2f((v - mx) * sc) * 0x1p40f); };

  // (1-3) radix select by mass: digits [31:21], [20:10], [9:0]
  uint32_t prefix = 0;
  u64 need = 0;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    const int hi_shift = pass == 1 ? 21 : 10;   // bits above this digit (passes 1, 2)
    for (int i = tid; i < kNucWaves * kNucBuckets; i += kNucThreads) (&s_hist[0][0])[i] = 0;
    __syncthreads();
    u64 S = 0;
    for (int s = 0; s < nseg; ++s) {
      if (nseg > 1) load(s);
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const uint32_t k = nuc_key(xr[j]);
        if (ok(s, j) && (pass == 0 || (k >> hi_shift) == (prefix >> hi_shift))) {
          const u64 m = mass(xr[j]);
          if (m) atomicAdd(&s_hist[wave][(k >> shift) & (nb - 1)], m);
          S += m;
        }
      }
    }
    __syncthreads();
    for (int b = tid; b < nb; b += kNucThreads)
      s_hist[0][b] = s_hist[0][b] + s_hist[1][b] + s_hist[2][b] + s_hist[3][b];
    if (pass == 0) {
      const u64 total = block_sum_u64(S, s_u64, lane, wave);
      need = static_cast<u64>(ceil(static_cast<double>(top_p) * static_cast<double>(total)));
    } else {
      __syncthreads();
    }
    if (wave == 0) {
      u64 above;
      const int d = nuc_pick(s_hist[0], nb, need, lane, above);
      if (lane == 0) {
        s_digit = d;
        s_need = need > above ? need - above : 0;
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(s_digit) << shift;
    need = s_need;
    __syncthreads();   // s_hist is cleared by the next pass
  }
  const uint32_t kappa = prefix;   // every key above it is in the nucleus
  const u64 m_kappa = mass(nuc_value(kappa));

  // (4) the nucleus: keys above kappa, and the first c kappa tokens (by id)
  // with c the fewest whose mass covers what is still needed
  u64 ma_all = 0;
  int cnt_all = 0;
  for (int s = 0; s < nseg; ++s) {
    if (nseg > 1) load(s);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const uint32_t k = nuc_key(xr[j]);
      if (ok(s, j) && k > kappa) ma_all += mass(xr[j]);
      if (ok(s, j) && k == kappa) ++cnt_all;
    }
  }
  const u64 MA = block_sum_u64(ma_all, s_u64, lane, wave);
  int count_kappa;
  block_excl_scan(cnt_all, s_int, lane, wave, count_kappa);
  long long cq = m_kappa > 0 ? static_cast<long long>((need + m_kappa - 1) / m_kappa) : count_kappa;
  const int c = static_cast<int>(cq < 1 ? 1 : (cq > count_kappa ? count_kappa : cq));
  const u64 Z = MA + static_cast<u64>(c) * m_kappa;
  const float u = fminf(fmaxf(uniforms[row], 0.f), 1.f);
  u64 target = static_cast<u64>(floor(static_cast<double>(u) * static_cast<double>(Z)));
  if (target >= Z) target = Z - 1;   // u = 1: the nucleus's highest id

  // (5) the draw: the nucleus token whose id-ordered mass interval holds
  // target; the sums are exact, so exactly one thread's chunk holds it
  if (tid == 0) s_sample = -1;
  u64 carry = 0;
  int kcarry = 0;
  for (int s = 0; s < nseg; ++s) {
    if (nseg > 1) load(s);
    u64 ma = 0;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const uint32_t k = nuc_key(xr[j]);
      if (ok(s, j) && k > kappa) ma += mass(xr[j]);
      if (ok(s, j) && k == kappa) ++cnt;
    }
    int cnt_seg;
    const int ord = kcarry + block_excl_scan(cnt, s_int, lane, wave, cnt_seg);
    const int take = min(max(c - ord, 0), cnt);
    const u64 w = ma + static_cast<u64>(take) * m_kappa;
    u64 w_seg;
    const u64 run0 = carry + block_excl_scan(w, s_u64, lane, wave, w_seg);
    if (w > 0 && run0 <= target && target < run0 + w) {
      u64 run = run0;
      int kord = ord, found = -1;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const uint32_t k = nuc_key(xr[j]);
        bool inc = false;
        if (ok(s, j) && k > kappa) inc = true;
        if (ok(s, j) && k == kappa) {
          inc = kord < c;
          ++kord;
        }
        if (inc) {
          run += mass(xr[j]);
          if (found < 0 && run > target) found = s * SEG + E * tid + j;
        }
      }
      s_sample = found;
    }
    carry += w_seg;
    kcarry += cnt_seg;
  }
  __syncthreads();
  if (tid == 0) {
    const int sample = s_sample >= 0 ? s_sample : 0;   // always found: the sums are exact
    stats[row] = RowStat{0.f, sample, 0.f, 0.f, 0.f};
    if (samples != nullptr) samples[row] = sample;
  }
}

// ---------------------------------------------------------------------------
// Rows of at most 32768 tokens: the whole row's order keys stay in LDS
// (padded by one word per 32 so that a thread's contiguous chunk is read
// without bank conflicts), 1024 threads.  The boundary key kappa is found in
// five walks, each a 256-bucket histogram of masses followed by a pick on
// one wave:
//   A. over every token, buckets linear in (max - x) / temperature over the
//      row's range (at most 40 binary orders of magnitude of mass: below
//      that masses are zero), so equal values share a bucket and a higher
//      bucket holds only larger values; the masses spread over many
//      buckets, so the LDS atomics rarely collide;
//   B-E. 8-bit radix digits of the order key over the tokens of the bucket
//      chosen in A (a contiguous range of keys), first gathered into a short
//      LDS list when they are few, so that these walks touch only them.  A
//      bucket of at most 256 tokens (the usual case) skips B-E: each of its
//      tokens sums the masses above and at its own key over the bucket.
// The first c kappa tokens (by id) complete the nucleus as in the kernel
// above.  The draw is one workgroup scan of every thread's (mass above
// kappa, kappa count) over its chunk of 32 tokens in id order; the one
// thread whose interval holds the target walks its chunk.  The same
// fixed-point masses give the same draws as the kernel above.
constexpr int kNlThreads = 1024;
constexpr int kNlWaves = kNlThreads / kWave;
constexpr int kNlMaxV = 32768;
constexpr int kNlChunk = kNlMaxV / kNlThreads;   // tokens per thread in the id-ordered walk
constexpr int kNlBuckets = 256;
constexpr int kNlList = 4096;                    // bucket A's tokens gathered for walks B-E
constexpr int kNlSmall = 256;                    // a bucket this small is resolved directly

__device__ __forceinline__ int nl_pad(int i) { return i + (i >> 5); }

__global__ __launch_bounds__(kNlThreads) void nucleus_sample_lds_kernel(int V, const float* __restrict__ logits,
                                                                      float temperature, float top_p,
                                                                      const float* __restrict__ uniforms,
                                                                      RowStat* __restrict__ stats,
                                                                      int32_t* __restrict__ samples) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* x = logits + static_cast<size_t>(row) * V;
  __shared__ uint32_t s_key[kNlMaxV + kNlMaxV / 32];
  __shared__ uint32_t s_list[kNlList];
  __shared__ u64 s_hist[kNlBuckets];
  __shared__ float s_red[2][kNlWaves];
  __shared__ u64 s_wm[kNlWaves];
  __shared__ int s_wc[kNlWaves];
  __shared__ u64 s_lm[kNlSmall];
  __shared__ int s_digit, s_count, s_sample, s_owner, s_kbefore;
  __shared__ uint32_t s_kappa;
  __shared__ u64 s_above, s_hd, s_base;

  // load: order keys into LDS, the row's maximum and minimum
  float mx = -__builtin_huge_valf(), mn = __builtin_huge_valf();
#pragma unroll 8
  for (int v = tid; v < V; v += kNlThreads) {
    const float xv = x[v];
    mx = fmaxf(mx, xv);
    mn = fminf(mn, xv);
    s_key[nl_pad(v)] = nuc_key(xv);
  }
  static_assert(kNlBuckets <= kNlThreads, "one thread per bucket clears the histogram");
  if (tid < kNlBuckets) s_hist[tid] = 0;
  if (tid == 0) {
    s_count = 0;
    s_sample = -1;
    s_owner = 0;
    s_base = 0;
    s_kbefore = 0;
    s_kappa = 0;
  }
  mx = wave_reduce_dpp<true>(mx);
  mn = -wave_reduce_dpp<true>(-mn);
  if (lane == 0) {
    s_red[0][wave] = mx;
    s_red[1][wave] = mn;
  }
  __syncthreads();
  mx = s_red[0][0];
  mn = s_red[1][0];
  for (int w = 1; w < kNlWaves; ++w) {
    mx = fmaxf(mx, s_red[0][w]);
    mn = fminf(mn, s_red[1][w]);
  }
  const float sc = (1.f / temperature) * 1.44269504088896341f;   // log2(e) / temperature
  auto mass = [&](uint32_t k) -> u64 { return static_cast<u64>(exp2f((nuc_value(k) - mx) * sc) * 0x1p40f); };
  // walk A's bucket as a digit (higher digit: larger values): linear in
  // d = (max - x) * log2(e) / temperature over [0, min(span, 40)]; every
  // step is monotone in x, so equal values share a digit
  const float span = fminf((mx - mn) * sc, 40.f);
  const float bscale = span > 1e-20f ? static_cast<float>(kNlBuckets - 1) / span : 0.f;
  auto digit_a = [&](uint32_t k) -> int {
    const float d = (mx - nuc_value(k)) * sc;
    return kNlBuckets - 1 - static_cast<int>(fminf(d * bscale, static_cast<float>(kNlBuckets - 1)));
  };

  // (A) masses by value bucket, and the row's total mass.  Thread tid walks
  // its own chunk [kNlChunk tid, + kNlChunk) in id order and keeps each
  // token's mass (as the float it converts from) and bucket in registers
  // for the gather and the draw.
  const int v0 = kNlChunk * tid;
  float fm[kNlChunk];          // exp2((x - max) / T) * 2^40; u64(fm) is the mass
  uint32_t dg[kNlChunk / 4];   // walk A's digits, four per word
  u64 S = 0;
#pragma unroll
  for (int j = 0; j < kNlChunk; ++j) {
    const int v = v0 + j;
    const uint32_t k = v < V ? s_key[nl_pad(v)] : 0x007fffffu;   // past V: -inf, mass zero
    fm[j] = exp2f((nuc_value(k) - mx) * sc) * 0x1p40f;
    const int d = digit_a(k);
    if ((j & 3) == 0) dg[j >> 2] = 0;
    dg[j >> 2] |= static_cast<uint32_t>(d) << (8 * (j & 3));
    const u64 m = static_cast<u64>(fm[j]);
    if (m) atomicAdd(&s_hist[d], m);
    S += m;
  }
  S = wave_sum_u64(S);
  if (lane == 0) s_wm[wave] = S;
  __syncthreads();
  u64 total = 0;
  for (int w = 0; w < kNlWaves; ++w) total += s_wm[w];
  u64 need = static_cast<u64>(ceil(static_cast<double>(top_p) * static_cast<double>(total)));

  // pick on one wave, then every thread takes the digit; the histogram is
  // cleared for the next walk
  u64 MA = 0, h_kappa = 0;
  auto pick = [&]() -> int {
    if (wave == 0) {
      u64 above;
      const int d = nuc_pick(s_hist, kNlBuckets, need, lane, above);
      if (lane == 0) {
        s_digit = d;
        s_above = above;
        s_hd = s_hist[min(max(d, 0), kNlBuckets - 1)];
      }
    }
    __syncthreads();
    const int d = min(max(s_digit, 0), kNlBuckets - 1);   // always in range: some bucket holds mass
    const u64 above = s_above;
    h_kappa = s_hd;
    MA += above;
    need = need > above ? need - above : 0;
    if (tid < kNlBuckets) s_hist[tid] = 0;
    __syncthreads();
    return d;
  };
  const int da = pick();

  // bucket da's keys gathered into s_list (any order: the walks below only
  // build histograms); past kNlList of them the walks read the whole row
#pragma unroll
  for (int j = 0; j < kNlChunk; ++j) {
    const int v = v0 + j;
    const bool in = v < V && static_cast<int>((dg[j >> 2] >> (8 * (j & 3))) & 0xffu) == da;
    const uint64_t bal = ballot(in);
    if (bal) {
      const int leader = __builtin_ctzll(bal);
      int base = 0;
      if (lane == leader) base = atomicAdd(&s_count, __popcll(bal));
      base = __builtin_amdgcn_readlane(base, leader);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1));
      if (in && pos < kNlList) s_list[pos] = s_key[nl_pad(v)];
      if (in && pos < kNlSmall) s_lm[pos] = static_cast<u64>(fm[j]);
    }
  }
  __syncthreads();
  const int nb = s_count;
  const bool listed = nb <= kNlList;

  uint32_t kappa;
  if (nb <= kNlSmall) {
    // a small bucket: each of its tokens (thread i, entry i) sums the masses
    // above its key and at its key over the bucket; the key whose interval
    // of cumulative mass holds what is still needed is kappa
    if (tid < nb) {
      const uint32_t ki = s_list[tid];
      u64 above = 0, at = 0;
      for (int j = 0; j < nb; ++j) {
        const uint32_t kj = s_list[j];
        const u64 mj = s_lm[j];
        above += kj > ki ? mj : 0;
        at += kj == ki ? mj : 0;
      }
      if (above < need && need <= above + at) {   // every entry with key ki agrees
        s_kappa = ki;
        s_above = above;
        s_hd = at;
      }
    }
    __syncthreads();
    kappa = s_kappa;
    const u64 above = s_above;
    h_kappa = s_hd;
    MA += above;
    need = need > above ? need - above : 0;
  } else {
    // (B-E) radix digits of the key over bucket da
    uint32_t prefix = 0;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      auto add = [&](uint32_t k) {
        if (pass == 0 || (k >> (shift + 8)) == (prefix >> (shift + 8))) {
          const u64 m = mass(k);
          if (m) atomicAdd(&s_hist[(k >> shift) & (kNlBuckets - 1)], m);
        }
      };
      if (listed) {
        for (int i = tid; i < nb; i += kNlThreads) add(s_list[i]);
      } else {
        for (int v = tid; v < V; v += kNlThreads) {
          const uint32_t k = s_key[nl_pad(v)];
          if (digit_a(k) == da) add(k);
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(pick()) << shift;
    }
    kappa = prefix;
  }
  const u64 m_kappa = mass(kappa);
  // the last histogram's bucket is exactly key kappa: count x m_kappa
  const int count_kappa = m_kappa > 0 ? static_cast<int>(h_kappa / m_kappa) : 1;
  long long cq = m_kappa > 0 ? static_cast<long long>((need + m_kappa - 1) / m_kappa) : count_kappa;
  const int c = static_cast<int>(cq < 1 ? 1 : (cq > count_kappa ? count_kappa : cq));
  const u64 Z = MA + static_cast<u64>(c) * m_kappa;
  const float u = fminf(fmaxf(uniforms[row], 0.f), 1.f);
  u64 target = static_cast<u64>(floor(static_cast<double>(u) * static_cast<double>(Z)));
  if (target >= Z) target = Z - 1;   // u = 1: the nucleus's highest id

  // the draw, over each thread's chunk in id order: one scan of (mass above
  // kappa, kappa count), since the kappa tokens taken before a thread's
  // chunk are the first c of them
  u64 ma = 0;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kNlChunk; ++j) {
    const int v = v0 + j;
    if (v < V) {
      const uint32_t k = s_key[nl_pad(v)];
      if (k > kappa) ma += static_cast<u64>(fm[j]);
      cnt += k == kappa ? 1 : 0;
    }
  }
  const u64 ma_inc = wave_incl_scan(ma, lane);
  const int cnt_inc = wave_incl_scan(cnt, lane);
  if (lane == kWave - 1) {
    s_wm[wave] = ma_inc;
    s_wc[wave] = cnt_inc;
  }
  __syncthreads();
  u64 off_m = 0;
  int off_c = 0;
  for (int w = 0; w < wave; ++w) {
    off_m += s_wm[w];
    off_c += s_wc[w];
  }
  const u64 ma_before = off_m + ma_inc - ma;
  const int cnt_before = off_c + cnt_inc - cnt;
  const int take = min(max(c - cnt_before, 0), cnt);
  const u64 w = ma + static_cast<u64>(take) * m_kappa;
  const u64 run0 = ma_before + static_cast<u64>(min(cnt_before, c)) * m_kappa;
  // exactly one thread's interval holds the target (the sums are exact); it
  // hands its chunk to wave 0, whose lane j takes token j of the chunk
  if (w > 0 && run0 <= target && target < run0 + w) {
    s_owner = tid;
    s_base = run0;
    s_kbefore = cnt_before;
  }
  __syncthreads();
  if (wave == 0) {
    const int owner = s_owner;
    const u64 base = s_base;
    const int kbefore = s_kbefore;
    const int v = kNlChunk * owner + lane;
    const bool live = lane < kNlChunk && v < V;
    const uint32_t k = live ? s_key[nl_pad(v)] : 0u;
    // kappa tokens of the chunk up to and including this lane
    const uint64_t kap = ballot(live && k == kappa);
    const int kord = kbefore + __popcll(kap & ((2ull << lane) - 1)) - 1;   // this token's ordinal if k == kappa
    const bool in = live && (k > kappa || (k == kappa && kord < c));
    // inclusive prefix of the masses over the lanes
    const u64 m = wave_incl_scan(in ? mass(k) : u64{0}, lane);
    const uint64_t hit = ballot(in && base + m > target);
    if (lane == 0) s_sample = hit ? kNlChunk * owner + __builtin_ctzll(hit) : -1;
  }
  __syncthreads();
  if (tid == 0) {
    const int sample = s_sample >= 0 ? s_sample : 0;   // always found: the sums are exact
    stats[row] = RowStat{0.f, sample, 0.f, 0.f, 0.f};
    if (samples != nullptr) samples[row] = sample;
  }
}

}  // namespace medusa

namespace {
using namespace medusa;
size_t nuc_ws(int B, int T) { return medusa_host::round_up(static_cast<size_t>(B) * T * sizeof(RowStat), 256); }
}  // namespace

extern "C" size_t medusa_posterior_nucleus_workspace(int B, int T) {
  if (B < 1 || B > kMaxBatch || T < 1 || T > kMaxNodes) return 0;
  return nuc_ws(B, T);
}

extern "C" int medusa_evaluate_posterior_nucleus(int B, int T, int V, int p_max, int D, const float* logits,
                                                 const int32_t* tree_candidates, const int32_t* retrieve,
                                                 const int32_t* num_paths, float temperature, float top_p,
                                                 const float* uniforms, int32_t* best_path, int32_t* accept_len,
                                                 int32_t* next_token, int32_t* samples, void* ws, size_t ws_bytes,
                                                 void* stream) {
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d", __func__, B);
  MEDUSA_REQUIRE(T >= 1 && T <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: T=%d", __func__, T);
  MEDUSA_REQUIRE(V >= 1 && V <= kNucMaxV, MEDUSA_ERR_SHAPE, "%s: V=%d (at most %d)", __func__, V, kNucMaxV);
  MEDUSA_REQUIRE(p_max >= 1 && p_max <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: p_max=%d", __func__, p_max);
  MEDUSA_REQUIRE(D >= 1 && D <= kMaxHeads + 1, MEDUSA_ERR_SHAPE, "%s: D=%d", __func__, D);
  MEDUSA_REQUIRE(temperature == temperature && temperature > 0.f && temperature < __builtin_huge_valf(),
                 MEDUSA_ERR_VALUE, "%s: temperature must be positive and finite", __func__);
  MEDUSA_REQUIRE(top_p > 0.f && top_p <= 1.f, MEDUSA_ERR_VALUE, "%s: top_p must lie in (0, 1]", __func__);
  MEDUSA_REQUIRE_PTR(logits);
  MEDUSA_REQUIRE_PTR(tree_candidates);
  MEDUSA_REQUIRE_PTR(retrieve);
  MEDUSA_REQUIRE_PTR(num_paths);
  MEDUSA_REQUIRE_PTR(uniforms);
  MEDUSA_REQUIRE_PTR(best_path);
  MEDUSA_REQUIRE_PTR(accept_len);
  MEDUSA_REQUIRE_PTR(next_token);
  MEDUSA_REQUIRE(samples == nullptr || medusa_host::aligned16(samples), MEDUSA_ERR_ALIGN,
                 "%s: samples is not 16-byte aligned", __func__);
  MEDUSA_REQUIRE_PTR(ws);
  MEDUSA_REQUIRE(ws_bytes >= nuc_ws(B, T), MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__,
                 ws_bytes, nuc_ws(B, T));
  hipStream_t st = static_cast<hipStream_t>(stream);
  RowStat* draws = static_cast<RowStat*>(ws);
  const dim3 grid(B * T), block(kNucThreads);
  if (V <= kNlMaxV)
    hipLaunchKernelGGL(nucleus_sample_lds_kernel, grid, dim3(kNlThreads), 0, st, V, logits, temperature, top_p,
                       uniforms, draws, samples);
  else if (V <= kNucThreads * 16)
    hipLaunchKernelGGL(nucleus_sample_kernel<16>, grid, block, 0, st, V, logits, temperature, top_p, uniforms, draws,
                       samples);
  else if (V <= kNucThreads * 32)
    hipLaunchKernelGGL(nucleus_sample_kernel<32>, grid, block, 0, st, V, logits, temperature, top_p, uniforms, draws,
                       samples);
  else if (V <= kNucThreads * 64)
    hipLaunchKernelGGL(nucleus_sample_kernel<64>, grid, block, 0, st, V, logits, temperature, top_p, uniforms, draws,
                       samples);
  else
    hipLaunchKernelGGL(nucleus_sample_kernel<128>, grid, block, 0, st, V, logits, temperature, top_p, uniforms, draws,
                       samples);
  int rc = medusa_host::hip_check("medusa_evaluate_posterior_nucleus sample launch");
  if (rc != MEDUSA_OK) return rc;
  return medusa_host::decide_on_draws(B, T, V, p_max, D, draws, tree_candidates, retrieve, num_paths, best_path,
                                      accept_len, next_token, st);
}
