// Counter-based uniforms (Philox4x64-10) and the typical-mode sampled next
// token on gfx950.
//
// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, SC 2011): a 4 x 64-bit
// counter and a 2 x 64-bit key; each of ten rounds takes the full 128-bit
// products of counter words 0 and 2 with two fixed multipliers, exchanges
// halves and xors in the key, and the key is bumped by two Weyl constants
// between rounds.  The uniform of (seed, step, sequence b, node n, purpose)
// is the top 24 bits of the first output word for counter (n, b, step,
// purpose) and key (seed, 0), times 2^-24: exact in float32, the same bits
// on any machine.
//
// Typical-mode next token: one workgroup per sequence reads the base logits
// at its last accepted node (retrieve[best_path][accept_len]) and computes
// the maximum; S = sum e^(z - m) and A = sum (z - m) e^(z - m) with
// z = logit / temperature, hence H and the threshold min(eps, delta e^-H);
// then the mass e^(z - m) of every token with e^(z - m) / S above the
// threshold (the acceptance rule's own test), as an integer with 40
// fraction bits so that sums are exact and independent of order.  The draw
// is the first token in id order whose running mass exceeds floor(u * Z),
// Z the total.
//
// Rows of up to 32768 tokens stay in registers: the row is cut into chunks
// of 4096 ids, thread t holds ids 4t .. 4t + 3 of every chunk (one 16-byte
// load per chunk, coalesced across the wave), so id order is (chunk,
// thread, element).  Per chunk a 64-bit wave scan of the threads' masses
// and one scan over the 8 x 16 (chunk, wave) totals give every thread the
// mass before each of its four-token runs; the one run whose interval holds
// floor(u * Z) is walked element by element.  Longer rows take a streaming
// kernel in which thread t owns a contiguous block of ids and re-reads it
// for each pass.
#include "common.hpp"

namespace medusa {

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull, kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull, kPhiloxW1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                                 uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t hi0 = __umul64hi(kPhiloxM0, c0), lo0 = kPhiloxM0 * c0;
    const uint64_t hi1 = __umul64hi(kPhiloxM1, c2), lo1 = kPhiloxM1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

// the 24-bit integer behind a uniform
__device__ __forceinline__ uint32_t philox_bits24(uint64_t seed, uint64_t step, int b, int node, int purpose) {
  return static_cast<uint32_t>(philox_word0(static_cast<uint64_t>(node), static_cast<uint64_t>(b), step,
                                            static_cast<uint64_t>(purpose), seed, 0ull) >> 40);
}

__global__ __launch_bounds__(256) void philox_uniforms_kernel(uint64_t seed, uint64_t step, int purpose, int B, int T,
                                                              float* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= B * T) return;
  out[i] = static_cast<float>(philox_bits24(seed, step, i / T, i % T, purpose)) * 0x1p-24f;
}

constexpr int kSampleThreads = 1024;
constexpr int kPurposeNextToken = 1;
constexpr int kStWaves = kSampleThreads / kWave;
constexpr int kStChunk = kSampleThreads * 4;     // ids per chunk: four per thread
constexpr int kStChunks = 8;
constexpr int kStRegMaxV = kStChunk * kStChunks;  // rows the register kernel takes

// kVec4: V % 4 == 0 and a 16-byte aligned logits base, so that each
// thread's four ids of a chunk are one aligned 16-byte load.  In base 2:
// with k = log2(e) / temperature, e^(z - m) = 2^(x k - mx k) for logit x
// and maximum logit mx, A = ln 2 * sum (x k - mx k) 2^(x k - mx k), and a
// token is allowed when its e^(z - m) exceeds thr * S.
template <bool kVec4>
__global__ __launch_bounds__(kSampleThreads) void sample_typical_reg_kernel(
    int T, int V, int p_max, int D, const float* __restrict__ logits, const int32_t* __restrict__ retrieve,
    const int32_t* __restrict__ best_path, const int32_t* __restrict__ accept_len, float temperature, float eps,
    float delta, uint64_t seed, uint64_t step, int32_t* __restrict__ next_token) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __shared__ float s_red[2][kStWaves];
  __shared__ uint64_t s_scan[kStChunks * kStWaves];   // (chunk, wave) mass totals in id order
  __shared__ int s_tok, s_last;
  const int best = min(max(best_path[b], 0), p_max - 1);
  const int acc = min(max(accept_len[b], 0), D - 1);
  int node = retrieve[best * D + acc];
  if (node < 0 || node >= T) node = 0;
  const float* row = logits + (static_cast<size_t>(b) * T + node) * V;
  const float NEG = -__builtin_huge_valf();
  if (tid == 0) {
    s_tok = -1;
    s_last = -1;
  }

  float z[kStChunks][4];
#pragma unroll
  for (int c = 0; c < kStChunks; ++c) {
    const int v0 = c * kStChunk + 4 * tid;
    if constexpr (kVec4) {
      if (v0 < V) {   // V % 4 == 0: the whole run is inside the row
        const float4 q = *reinterpret_cast<const float4*>(row + v0);
        z[c][0] = q.x;
        z[c][1] = q.y;
        z[c][2] = q.z;
        z[c][3] = q.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) z[c][i] = NEG;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) z[c][i] = v0 + i < V ? row[v0 + i] : NEG;
    }
  }

  // maximum of the raw logits (a positive temperature keeps the order)
  float mx = NEG;
#pragma unroll
  for (int c = 0; c < kStChunks; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[c][i]);
  mx = wave_reduce_dpp<true>(mx);
  if (lane == 0) s_red[0][wave] = mx;
  __syncthreads();
  mx = s_red[0][0];
#pragma unroll
  for (int w = 1; w < kStWaves; ++w) mx = fmaxf(mx, s_red[0][w]);
  const float kl = 1.4426950408889634f / temperature;
  const float m2 = mx * kl;
  __syncthreads();

  // S and A, hence the entropy and the threshold; z becomes e^(z - m)
  float S = 0.f, A2 = 0.f;
#pragma unroll
  for (int c = 0; c < kStChunks; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (c * kStChunk + 4 * tid + i < V) {
        const float d2 = fmaf(z[c][i], kl, -m2);
        const float e = __builtin_amdgcn_exp2f(d2);
        S += e;
        A2 = fmaf(d2, e, A2);
        z[c][i] = e;
      } else {
        z[c][i] = 0.f;
      }
    }
  S = wave_reduce_dpp<false>(S);
  A2 = wave_reduce_dpp<false>(A2);
  if (lane == 0) {
    s_red[0][wave] = S;
    s_red[1][wave] = A2;
  }
  __syncthreads();
  S = 0.f;
  A2 = 0.f;
#pragma unroll
  for (int w = 0; w < kStWaves; ++w) {
    S += s_red[0][w];
    A2 += s_red[1][w];
  }
  const float H = logf(S) - 0.6931471805599453f * A2 / S;
  const float thrS = fminf(eps, delta * expf(-H)) * S;

  // allowed flags (bit 4c + i) and fixed-point masses, per four-token run;
  // per chunk the mass of the wave's earlier lanes (excl) and the wave's
  // total
  uint64_t excl[kStChunks];
  uint32_t allow = 0;
#pragma unroll
  for (int c = 0; c < kStChunks; ++c) {
    uint64_t own = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool a = z[c][i] > thrS;
      allow |= static_cast<uint32_t>(a) << (4 * c + i);
      own += a ? static_cast<uint64_t>(z[c][i] * 0x1p40f) : 0ull;
    }
    const uint64_t inc = wave_incl_scan_u64(own);
    excl[c] = inc - own;
    if (lane == kWave - 1) s_scan[c * kStWaves + wave] = inc;
  }
  if (allow != 0) {
    const int j = 31 - __builtin_clz(allow);
    atomicMax(&s_last, (j >> 2) * kStChunk + 4 * tid + (j & 3));
  }
  __syncthreads();

  // exclusive prefix of the 128 (chunk, wave) totals: lane l holds entries
  // 2l and 2l + 1
  const uint64_t e0 = s_scan[2 * lane], e1 = s_scan[2 * lane + 1];
  const uint64_t pair_inc = wave_incl_scan_u64(e0 + e1);
  const uint64_t pair_ex = pair_inc - (e0 + e1);
  const uint64_t Z = readlane_u64(pair_inc, kWave - 1);
  // target = floor(u * Z), u = bits * 2^-24: the 24 bits times Z, shifted
  const uint64_t ub = philox_bits24(seed, step, b, 0, kPurposeNextToken);
  const uint64_t plo = ub * Z, phi = __umul64hi(ub, Z);
  const uint64_t target = (phi << 40) | (plo >> 24);
#pragma unroll
  for (int c = 0; c < kStChunks; ++c) {
    // this wave's entry k = 16c + wave sits in lane k / 2, slot wave & 1
    const int src = (c * kStWaves + wave) >> 1;
    const uint64_t f0 = readlane_u64(e0, src);
    const uint64_t wbase = readlane_u64(pair_ex, src) + ((wave & 1) ? f0 : 0ull);
    const uint64_t wtotal = (wave & 1) ? readlane_u64(e1, src) : f0;
    if (wbase <= target && target < wbase + wtotal) {   // the crossing is in this wave's run of chunk c
      // the last lane with a non-empty run starting at or before the target
      const uint64_t before = wbase + excl[c];
      const uint64_t hit = __ballot(((allow >> (4 * c)) & 0xfu) != 0 && before <= target);
      if (lane == kWave - 1 - __builtin_clzll(hit)) {
        uint64_t run = before;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // the same mass as above, recomputed: the empty asm hides that,
          // so the compiler keeps 32 floats live rather than 32 64-bit masses
          float e = z[c][i];
          asm volatile("" : "+v"(e));
          if ((allow >> (4 * c + i)) & 1u) run += static_cast<uint64_t>(e * 0x1p40f);
          if (run > target) {
            s_tok = c * kStChunk + 4 * tid + i;
            break;
          }
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    // no crossing (not reached for u < 1): the highest allowed id
    const int tok = s_tok >= 0 ? s_tok : s_last;
    next_token[b] = tok < 0 ? 0 : tok;
  }
}

__global__ __launch_bounds__(kSampleThreads) void sample_typical_stream_kernel(
    int T, int V, int p_max, int D, const float* __restrict__ logits, const int32_t* __restrict__ retrieve,
    const int32_t* __restrict__ best_path, const int32_t* __restrict__ accept_len, float temperature, float eps,
    float delta, uint64_t seed, uint64_t step, int32_t* __restrict__ next_token) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = kSampleThreads / kWave;
  __shared__ float s_red[2][NW];
  __shared__ uint64_t s_scan[NW];
  __shared__ int s_tok;
  const int best = min(max(best_path[b], 0), p_max - 1);
  const int acc = min(max(accept_len[b], 0), D - 1);
  int node = retrieve[best * D + acc];
  if (node < 0 || node >= T) node = 0;
  const float* row = logits + (static_cast<size_t>(b) * T + node) * V;
  const int per = (V + kSampleThreads - 1) / kSampleThreads;
  const int lo = min(tid * per, V), hi = min(lo + per, V);
  const float NEG = -__builtin_huge_valf();

  // (1) maximum of the raw logits (division by a positive temperature is monotonic)
  float mx = NEG;
  for (int v = lo; v < hi; ++v) mx = fmaxf(mx, row[v]);
  mx = wave_max(mx);
  if (lane == 0) s_red[0][wave] = mx;
  __syncthreads();
  mx = s_red[0][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, s_red[0][w]);
  const float m = mx / temperature;
  __syncthreads();

  // (2) S and A, hence the entropy and the threshold
  float S = 0.f, A = 0.f;
  for (int v = lo; v < hi; ++v) {
    const float dz = row[v] / temperature - m;
    const float e = expf(dz);
    S += e;
    A += dz * e;
  }
  S = wave_sum(S);
  A = wave_sum(A);
  if (lane == 0) {
    s_red[0][wave] = S;
    s_red[1][wave] = A;
  }
  __syncthreads();
  S = 0.f;
  A = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    S += s_red[0][w];
    A += s_red[1][w];
  }
  const float H = logf(S) - A / S;
  const float thr = fminf(eps, delta * expf(-H));

  // (3) fixed-point masses of the allowed tokens in this thread's block
  uint64_t own = 0;
  for (int v = lo; v < hi; ++v) {
    const float e = expf(row[v] / temperature - m);
    if (e / S > thr) own += static_cast<uint64_t>(e * 0x1p40f);
  }
  // exclusive prefix of the blocks' masses, in id order
  uint64_t inc = own;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint64_t x = __shfl_up(inc, o);
    if (lane >= o) inc += x;
  }
  if (lane == kWave - 1) s_scan[wave] = inc;
  if (tid == 0) s_tok = -1;
  __syncthreads();
  uint64_t before = 0, Z = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += w < wave ? s_scan[w] : 0ull;
    Z += s_scan[w];
  }
  const uint64_t prefix = before + inc - own;
  // target = floor(u * Z), u = bits * 2^-24: the 24 bits times Z, shifted
  const uint64_t ub = philox_bits24(seed, step, b, 0, kPurposeNextToken);
  const uint64_t plo = ub * Z, phi = __umul64hi(ub, Z);
  const uint64_t target = (phi << 40) | (plo >> 24);
  if (own != 0 && prefix <= target && target < prefix + own) {
    uint64_t run = prefix;
    for (int v = lo; v < hi; ++v) {
      const float e = expf(row[v] / temperature - m);
      if (e / S > thr) {
        run += static_cast<uint64_t>(e * 0x1p40f);
        if (run > target) {
          s_tok = v;
          break;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int tok = s_tok;
    if (tok < 0) {   // no crossing (not reached for u < 1): the highest allowed id
      for (int v = V - 1; v >= 0; --v) {
        const float e = expf(row[v] / temperature - m);
        if (e / S > thr) {
          tok = v;
          break;
        }
      }
    }
    next_token[b] = tok < 0 ? 0 : tok;
  }
}

}  // namespace medusa

using namespace medusa;

extern "C" int medusa_philox_uniforms(uint64_t seed, uint64_t step, int purpose, int B, int T, float* out,
                                      void* stream) {
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d", __func__, B);
  MEDUSA_REQUIRE(T >= 1 && T <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: T=%d", __func__, T);
  MEDUSA_REQUIRE(purpose >= 0, MEDUSA_ERR_VALUE, "%s: purpose=%d", __func__, purpose);
  MEDUSA_REQUIRE_PTR(out);
  hipLaunchKernelGGL(philox_uniforms_kernel, dim3((B * T + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                     seed, step, purpose, B, T, out);
  return medusa_host::hip_check("medusa_philox_uniforms launch");
}

extern "C" int medusa_sample_typical(int B, int T, int V, int p_max, int D, const float* logits,
                                     const int32_t* retrieve, const int32_t* best_path, const int32_t* accept_len,
                                     float temperature, float eps, float delta, uint64_t seed, uint64_t step,
                                     int32_t* next_token, void* stream) {
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d", __func__, B);
  MEDUSA_REQUIRE(T >= 1 && T <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: T=%d", __func__, T);
  MEDUSA_REQUIRE(V >= 1 && V <= (1 << 24), MEDUSA_ERR_SHAPE, "%s: V=%d", __func__, V);
  MEDUSA_REQUIRE(p_max >= 1 && p_max <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: p_max=%d", __func__, p_max);
  MEDUSA_REQUIRE(D >= 1 && D <= kMaxHeads + 1, MEDUSA_ERR_SHAPE, "%s: D=%d", __func__, D);
  MEDUSA_REQUIRE(temperature > 0.f && temperature < __builtin_huge_valf(), MEDUSA_ERR_VALUE,
                 "%s: temperature must be positive", __func__);
  MEDUSA_REQUIRE(eps > 0.f && delta > 0.f && delta < 1.f, MEDUSA_ERR_VALUE,
                 "%s: need eps > 0 and 0 < delta < 1 (eps %g, delta %g)", __func__, eps, delta);
  MEDUSA_REQUIRE_PTR(logits);
  MEDUSA_REQUIRE_PTR(retrieve);
  MEDUSA_REQUIRE_PTR(best_path);
  MEDUSA_REQUIRE_PTR(accept_len);
  MEDUSA_REQUIRE_PTR(next_token);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (V <= kStRegMaxV) {
    if (V % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0)
      hipLaunchKernelGGL(sample_typical_reg_kernel<true>, dim3(B), dim3(kSampleThreads), 0, st, T, V, p_max, D, logits,
                         retrieve, best_path, accept_len, temperature, eps, delta, seed, step, next_token);
    else
      hipLaunchKernelGGL(sample_typical_reg_kernel<false>, dim3(B), dim3(kSampleThreads), 0, st, T, V, p_max, D,
                         logits, retrieve, best_path, accept_len, temperature, eps, delta, seed, step, next_token);
  } else {
    hipLaunchKernelGGL(sample_typical_stream_kernel, dim3(B), dim3(kSampleThreads), 0, st, T, V, p_max, D, logits,
                       retrieve, best_path, accept_len, temperature, eps, delta, seed, step, next_token);
  }
  return medusa_host::hip_check("medusa_sample_typical launch");
}
