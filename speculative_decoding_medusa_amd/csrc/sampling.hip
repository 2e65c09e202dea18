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
// at its last accepted node (retrieve[best_path][accept_len]) in three
// passes -- maximum; S = sum e^(z - m) and A = sum (z - m) e^(z - m) with
// z = logit / temperature, hence H and the threshold min(eps, delta e^-H);
// then the mass e^(z - m) of every token with e^(z - m) / S above the
// threshold (the acceptance rule's own test), as an integer with 40
// fraction bits so that sums are exact and independent of order.  Thread t
// owns a contiguous block of token ids; a workgroup scan of the blocks'
// masses finds the one block whose interval holds floor(u * Z), and its
// thread walks its tokens in id order to the first whose running mass
// exceeds it.
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

__global__ __launch_bounds__(kSampleThreads) void sample_typical_kernel(
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
  hipLaunchKernelGGL(sample_typical_kernel, dim3(B), dim3(kSampleThreads), 0, static_cast<hipStream_t>(stream), T, V,
                     p_max, D, logits, retrieve, best_path, accept_len, temperature, eps, delta, seed, step,
                     next_token);
  return medusa_host::hip_check("medusa_sample_typical launch");
}
