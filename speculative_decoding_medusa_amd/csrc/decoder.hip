// The elementwise and row-wise pieces of a LLaMA-style base model forward
// on gfx950, around the skinny GEMM of base_head.hip (which runs every
// linear layer, packed weights, float32 out):
//
//   medusa_embed        x[m] = embed[token[m]]                 (float32 rows)
//   medusa_add_rmsnorm  x[m] += y[m]; out[m] = bf16(x[m] / rms(x[m]) * g)
//   medusa_rope_qkv     rotate q and k (rotate-half RoPE at each token's
//                       position), q -> bf16, k and v -> bf16 KV-cache slots
//                       prefix_len[b] + t
//   medusa_silu_mul     out = bf16(silu(gate) * up)
//
// All are one pass over HBM-resident rows of a few KB: one workgroup per
// row for the reductions, one thread per pair (RoPE) or per 8 elements
// otherwise.
#include "common.hpp"

namespace medusa {

constexpr int kDecThreads = 256;

__global__ __launch_bounds__(kDecThreads) void embed_kernel(int M, int H, int V, const int32_t* __restrict__ tokens,
                                                          const uint16_t* __restrict__ embed, float* __restrict__ x) {
  const long long i = static_cast<long long>(blockIdx.x) * kDecThreads + threadIdx.x;   // 8 elements each
  const int per_row = H / 8;
  if (i >= static_cast<long long>(M) * per_row) return;
  const int m = static_cast<int>(i / per_row), c = static_cast<int>(i % per_row) * 8;
  const int tok = tokens[m];
  float4 lo = {0.f, 0.f, 0.f, 0.f}, hi = lo;
  if (tok >= 0 && tok < V) {
    const u32x4 e = *reinterpret_cast<const u32x4*>(embed + static_cast<size_t>(tok) * H + c);
    lo = {__uint_as_float(e[0] << 16), __uint_as_float(e[0] & 0xffff0000u), __uint_as_float(e[1] << 16),
          __uint_as_float(e[1] & 0xffff0000u)};
    hi = {__uint_as_float(e[2] << 16), __uint_as_float(e[2] & 0xffff0000u), __uint_as_float(e[3] << 16),
          __uint_as_float(e[3] & 0xffff0000u)};
  }
  float4* dst = reinterpret_cast<float4*>(x + static_cast<size_t>(m) * H + c);
  dst[0] = lo;
  dst[1] = hi;
}

// One workgroup per row; each thread owns 8-element groups c = 8 (tid + 256 j).
__global__ __launch_bounds__(kDecThreads) void add_rmsnorm_kernel(int H, float* __restrict__ x,
                                                                const float* __restrict__ y,
                                                                const uint16_t* __restrict__ g, float eps,
                                                                uint16_t* __restrict__ out) {
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* xr = x + static_cast<size_t>(m) * H;
  const float* yr = y != nullptr ? y + static_cast<size_t>(m) * H : nullptr;
  __shared__ float s_red[kDecThreads / kWave];
  float ss = 0.f;
  for (int c = 8 * tid; c < H; c += 8 * kDecThreads) {
    float4 a = *reinterpret_cast<const float4*>(xr + c), b = *reinterpret_cast<const float4*>(xr + c + 4);
    if (yr != nullptr) {
      const float4 p = *reinterpret_cast<const float4*>(yr + c), q = *reinterpret_cast<const float4*>(yr + c + 4);
      a = {a.x + p.x, a.y + p.y, a.z + p.z, a.w + p.w};
      b = {b.x + q.x, b.y + q.y, b.z + q.z, b.w + q.w};
      *reinterpret_cast<float4*>(xr + c) = a;
      *reinterpret_cast<float4*>(xr + c + 4) = b;
    }
    ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
  }
  ss = wave_sum(ss);
  if (lane == 0) s_red[wave] = ss;
  __syncthreads();
  ss = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  const float r = 1.f / sqrtf(ss / static_cast<float>(H) + eps);
  for (int c = 8 * tid; c < H; c += 8 * kDecThreads) {
    const float4 a = *reinterpret_cast<const float4*>(xr + c), b = *reinterpret_cast<const float4*>(xr + c + 4);
    const u32x4 gv = *reinterpret_cast<const u32x4*>(g + c);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float g0 = __uint_as_float(gv[p] << 16), g1 = __uint_as_float(gv[p] & 0xffff0000u);
      o[p] = pack_bf16x2(v[2 * p] * r * g0, v[2 * p + 1] * r * g1);
    }
    *reinterpret_cast<u32x4*>(out + static_cast<size_t>(m) * H + c) = o;
  }
}

// Thread per (b, t, head, pair i < d/2): dims i and i + d/2 of q and k are
// rotated by position * theta^(-2i/d) (angle and its sine and cosine in
// double precision, then rounded); v is copied.
__global__ __launch_bounds__(kDecThreads) void rope_qkv_kernel(int B, int T, int heads, int d, int max_slots,
                                                             const float* __restrict__ qkv,
                                                             const int32_t* __restrict__ positions,
                                                             const int32_t* __restrict__ prefix_len, float theta,
                                                             uint16_t* __restrict__ q, uint16_t* __restrict__ kc,
                                                             uint16_t* __restrict__ vc) {
  const int half = d / 2;
  const long long idx = static_cast<long long>(blockIdx.x) * kDecThreads + threadIdx.x;
  if (idx >= static_cast<long long>(B) * T * heads * half) return;
  const int i = static_cast<int>(idx % half);
  const int h = static_cast<int>((idx / half) % heads);
  const int t = static_cast<int>((idx / half / heads) % T);
  const int b = static_cast<int>(idx / half / heads / T);
  const int H = heads * d;
  const float* row = qkv + (static_cast<size_t>(b) * T + t) * 3 * H;
  const double ang = static_cast<double>(positions[static_cast<size_t>(b) * T + t]) *
                     pow(static_cast<double>(theta), -2.0 * i / d);
  const float c = static_cast<float>(cos(ang)), s = static_cast<float>(sin(ang));
  auto bf = [](float v) { return static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu); };
  const float q1 = row[h * d + i], q2 = row[h * d + i + half];
  uint16_t* qo = q + ((static_cast<size_t>(b) * T + t) * heads + h) * d;
  qo[i] = bf(q1 * c - q2 * s);
  qo[i + half] = bf(q2 * c + q1 * s);
  const int slot = prefix_len[b] + t;
  if (slot < 0 || slot >= max_slots) return;   // outside the cache: not written
  const float k1 = row[H + h * d + i], k2 = row[H + h * d + i + half];
  const size_t off = ((static_cast<size_t>(b) * heads + h) * max_slots + slot) * d;
  kc[off + i] = bf(k1 * c - k2 * s);
  kc[off + i + half] = bf(k2 * c + k1 * s);
  vc[off + i] = bf(row[2 * H + h * d + i]);
  vc[off + i + half] = bf(row[2 * H + h * d + i + half]);
}

__global__ __launch_bounds__(kDecThreads) void silu_mul_kernel(int M, int I, const float* __restrict__ gu,
                                                             uint16_t* __restrict__ out) {
  const long long idx = static_cast<long long>(blockIdx.x) * kDecThreads + threadIdx.x;   // 8 elements each
  const int per_row = I / 8;
  if (idx >= static_cast<long long>(M) * per_row) return;
  const int m = static_cast<int>(idx / per_row), c = static_cast<int>(idx % per_row) * 8;
  const float* gr = gu + static_cast<size_t>(m) * 2 * I + c;
  const float* ur = gr + I;
  u32x4 o;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float g0 = gr[2 * p], g1 = gr[2 * p + 1];
    o[p] = pack_bf16x2(g0 / (1.f + expf(-g0)) * ur[2 * p], g1 / (1.f + expf(-g1)) * ur[2 * p + 1]);
  }
  *reinterpret_cast<u32x4*>(out + static_cast<size_t>(m) * I + c) = o;
}

}  // namespace medusa

using namespace medusa;

namespace {
int blocks_for(long long n) { return static_cast<int>((n + kDecThreads - 1) / kDecThreads); }
}  // namespace

extern "C" int medusa_embed(int M, int H, int V, const int32_t* tokens, const void* embed, float* x, void* stream) {
  MEDUSA_REQUIRE(M >= 1 && M <= (1 << 20), MEDUSA_ERR_SHAPE, "%s: M=%d", __func__, M);
  MEDUSA_REQUIRE(H >= 8 && H % 8 == 0 && H <= (1 << 16), MEDUSA_ERR_SHAPE, "%s: H=%d", __func__, H);
  MEDUSA_REQUIRE(V >= 1, MEDUSA_ERR_SHAPE, "%s: V=%d", __func__, V);
  MEDUSA_REQUIRE_PTR(tokens);
  MEDUSA_REQUIRE_PTR(embed);
  MEDUSA_REQUIRE_PTR(x);
  hipLaunchKernelGGL(embed_kernel, dim3(blocks_for(static_cast<long long>(M) * H / 8)), dim3(kDecThreads), 0,
                     static_cast<hipStream_t>(stream), M, H, V, tokens, static_cast<const uint16_t*>(embed), x);
  return medusa_host::hip_check("medusa_embed launch");
}

extern "C" int medusa_add_rmsnorm(int M, int H, float* x, const float* y, const void* gain, float eps, void* out,
                                  void* stream) {
  MEDUSA_REQUIRE(M >= 1 && M <= (1 << 20), MEDUSA_ERR_SHAPE, "%s: M=%d", __func__, M);
  MEDUSA_REQUIRE(H >= 8 && H % 8 == 0 && H <= (1 << 16), MEDUSA_ERR_SHAPE, "%s: H=%d", __func__, H);
  MEDUSA_REQUIRE(eps == eps && eps >= 0.f, MEDUSA_ERR_VALUE, "%s: eps must be >= 0", __func__);
  MEDUSA_REQUIRE_PTR(x);
  MEDUSA_REQUIRE(y == nullptr || medusa_host::aligned16(y), MEDUSA_ERR_ALIGN, "%s: y is not 16-byte aligned",
                 __func__);
  MEDUSA_REQUIRE_PTR(gain);
  MEDUSA_REQUIRE_PTR(out);
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(M), dim3(kDecThreads), 0, static_cast<hipStream_t>(stream), H, x, y,
                     static_cast<const uint16_t*>(gain), eps, static_cast<uint16_t*>(out));
  return medusa_host::hip_check("medusa_add_rmsnorm launch");
}

extern "C" int medusa_rope_qkv(int B, int T, int heads, int d, int max_slots, const float* qkv,
                               const int32_t* positions, const int32_t* prefix_len, float theta, void* q,
                               void* k_cache, void* v_cache, void* stream) {
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d", __func__, B);
  MEDUSA_REQUIRE(T >= 1 && T <= (1 << 16), MEDUSA_ERR_SHAPE, "%s: T=%d", __func__, T);
  MEDUSA_REQUIRE(heads >= 1 && heads <= 256, MEDUSA_ERR_SHAPE, "%s: heads=%d", __func__, heads);
  MEDUSA_REQUIRE(d >= 2 && d % 2 == 0 && d <= 512, MEDUSA_ERR_SHAPE, "%s: d=%d", __func__, d);
  MEDUSA_REQUIRE(max_slots >= 1, MEDUSA_ERR_SHAPE, "%s: max_slots=%d", __func__, max_slots);
  MEDUSA_REQUIRE(theta == theta && theta > 0.f, MEDUSA_ERR_VALUE, "%s: theta must be positive", __func__);
  MEDUSA_REQUIRE_PTR(qkv);
  MEDUSA_REQUIRE_PTR(positions);
  MEDUSA_REQUIRE_PTR(prefix_len);
  MEDUSA_REQUIRE_PTR(q);
  MEDUSA_REQUIRE_PTR(k_cache);
  MEDUSA_REQUIRE_PTR(v_cache);
  hipLaunchKernelGGL(rope_qkv_kernel, dim3(blocks_for(static_cast<long long>(B) * T * heads * (d / 2))),
                     dim3(kDecThreads), 0, static_cast<hipStream_t>(stream), B, T, heads, d, max_slots, qkv,
                     positions, prefix_len, theta, static_cast<uint16_t*>(q), static_cast<uint16_t*>(k_cache),
                     static_cast<uint16_t*>(v_cache));
  return medusa_host::hip_check("medusa_rope_qkv launch");
}

extern "C" int medusa_silu_mul(int M, int I, const float* gate_up, void* out, void* stream) {
  MEDUSA_REQUIRE(M >= 1 && M <= (1 << 20), MEDUSA_ERR_SHAPE, "%s: M=%d", __func__, M);
  MEDUSA_REQUIRE(I >= 8 && I % 8 == 0 && I <= (1 << 18), MEDUSA_ERR_SHAPE, "%s: I=%d", __func__, I);
  MEDUSA_REQUIRE_PTR(gate_up);
  MEDUSA_REQUIRE_PTR(out);
  hipLaunchKernelGGL(silu_mul_kernel, dim3(blocks_for(static_cast<long long>(M) * I / 8)), dim3(kDecThreads), 0,
                     static_cast<hipStream_t>(stream), M, I, gate_up, static_cast<uint16_t*>(out));
  return medusa_host::hip_check("medusa_silu_mul launch");
}
