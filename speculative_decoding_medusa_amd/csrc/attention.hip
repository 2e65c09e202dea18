// Tree attention on gfx950: T tree queries against a KV prefix plus the
// ancestor-only mask among the tree's own keys.
//
// bf16 path.  The key range [0, L+T) of each (sequence, head) is cut into
// splits of kSplit keys (the last split takes the remainder), one workgroup
// each, so a 32-head layer at L = 2048 fills the chip.  A workgroup holds up
// to 64 queries (four waves of 16) and walks its split in 64-key chunks
// staged through LDS: K row-major, V transposed (d-major) on the way in.
// Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16: a lane then holds four consecutive keys of one
// query, which is exactly the B-operand layout P^T needs for O^T += V^T P^T,
// so probabilities never leave registers.  Online softmax in base 2, fp32
// accumulators.  Each split writes (O unnormalised, m, l) and a second
// kernel merges the splits (log-sum-exp).
//
// f32 path: one wave per (sequence, head, query), online softmax over
// 64-key chunks on the VALU.
#include "common.hpp"

namespace medusa {

constexpr int kAttnThreads = 256;
constexpr int kQBlock = 64;        // queries per workgroup
constexpr int kChunk = 64;         // keys per LDS chunk
constexpr int kSplit = 256;        // keys per split
constexpr float kLog2e = 1.4426950408889634f;

__host__ __device__ inline int num_splits(int total_keys) {
  const int s = total_keys / kSplit;
  return s < 1 ? 1 : s;
}

__device__ __forceinline__ u32x4 ld16g(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

template <int D>
__global__ __launch_bounds__(kAttnThreads) void tree_attn_bf16_kernel(
    int T, int Hq, int max_slots, int nsplit_max, int nqb,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ prefix_len, const uint8_t* __restrict__ tree_mask, float scale_log2,
    float* __restrict__ part_o, float2* __restrict__ part_ml) {
  constexpr int KS = D + 8;            // K row stride in LDS (elements)
  constexpr int VS = kChunk + 8;       // V^T row stride in LDS (elements)
  constexpr int PIECES = D / 8;        // 16-byte pieces per row
  constexpr int PER_THREAD = kChunk * PIECES / kAttnThreads;
  constexpr int DT = D / 16;           // output d tiles
  constexpr int DS = D / 32;           // K steps of the score MFMA
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kChunk * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS];
  __shared__ uint64_t mbits[kQBlock][kMaxNodes / 64];

  const int split = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z / nqb, qb = blockIdx.z - b * nqb;
  int L = prefix_len[b];
  if (L > max_slots - T) L = max_slots - T;
  if (L < 0) L = 0;
  const int total = L + T;
  const int ns = num_splits(total);
  if (split >= ns) return;
  const int k_lo = split * kSplit;
  const int k_hi = split == ns - 1 ? total : k_lo + kSplit;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int qi = qb * kQBlock + wave * 16 + n;     // this lane's query
  const bool q_ok = qi < T;
  const size_t bh = static_cast<size_t>(b) * Hq + h;
  const uint16_t* kbase = kc + bh * max_slots * D;
  const uint16_t* vbase = vc + bh * max_slots * D;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // Q as the B operand of S^T: Q[qi][s*32 + 8g .. +8]
  u32x4 qv[DS];
  {
    const uint16_t* qrow = q + ((static_cast<size_t>(b) * T + (q_ok ? qi : 0)) * Hq + h) * D;
#pragma unroll
    for (int s = 0; s < DS; ++s) qv[s] = q_ok ? ld16g(qrow + s * 32 + g * 8) : zero;
  }

  // ancestor bits of the block's queries (only splits that reach the tree)
  const bool has_tree = k_hi > L;
  if (has_tree) {
    const int ql = tid >> 2, w = tid & 3;
    const int qq = qb * kQBlock + ql;
    uint64_t word = 0;
    if (qq < T) {
      for (int jj = 0; jj < 64; ++jj) {
        const int j = w * 64 + jj;
        if (j < T && tree_mask[static_cast<size_t>(qq) * T + j]) word |= 1ull << jj;
      }
    }
    mbits[ql][w] = word;
  }

  float m_run = -__builtin_huge_valf();
  float l_part = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 kreg[PER_THREAD], vreg[PER_THREAD];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int p = tid + r * kAttnThreads;
      const int key = c0 + p / PIECES, pc = p % PIECES;
      const bool ok = key < k_hi;
      kreg[r] = ok ? ld16g(kbase + static_cast<size_t>(key) * D + pc * 8) : zero;
      vreg[r] = ok ? ld16g(vbase + static_cast<size_t>(key) * D + pc * 8) : zero;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int p = tid + r * kAttnThreads;
      const int key = p / PIECES, pc = p % PIECES;
      *reinterpret_cast<u32x4*>(&Ks[key * KS + pc * 8]) = kreg[r];
      const uint32_t w4[4] = {vreg[r][0], vreg[r][1], vreg[r][2], vreg[r][3]};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        Vt[(pc * 8 + e) * VS + key] = static_cast<uint16_t>(w4[e >> 1] >> ((e & 1) * 16));
    }
  };

  const int nchunks = (k_hi - k_lo + kChunk - 1) / kChunk;
  fetch(k_lo);
  uint64_t my_bits[kMaxNodes / 64] = {0, 0, 0, 0};
  for (int c = 0; c < nchunks; ++c) {
    const int c0 = k_lo + c * kChunk;
    __syncthreads();
    stage();
    __syncthreads();
    if (c == 0 && has_tree) {
#pragma unroll
      for (int w = 0; w < kMaxNodes / 64; ++w) my_bits[w] = mbits[wave * 16 + n][w];
    }
    if (c + 1 < nchunks) fetch(c0 + kChunk);

    // scores S^T[key = kt*16 + 4g + i][query n]
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < DS; ++st) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Ks[(kt * 16 + n) * KS + st * 32 + g * 8]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, qv[st]), acc, 0, 0, 0);
      }
      s[kt] = acc;
    }
    float mloc = -__builtin_huge_valf();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = c0 + kt * 16 + 4 * g + i;
        float x = s[kt][i] * scale_log2;
        bool allowed = key < k_hi;
        if (key >= L) {
          const int j = key - L;
          allowed = allowed && ((my_bits[(j >> 6) & 3] >> (j & 63)) & 1ull);
        }
        x = allowed ? x : -__builtin_huge_valf();
        s[kt][i] = x;
        mloc = fmaxf(mloc, x);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float ref = m_new == -__builtin_huge_valf() ? 0.f : m_new;
    const float alpha = exp2f(m_run - ref);
    float psum = 0.f;
    uint32_t pb[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = exp2f(s[kt][i] - ref);
        psum += p[i];
      }
      pb[kt][0] = f32_to_bf16_bits(p[0]) | (f32_to_bf16_bits(p[1]) << 16);
      pb[kt][1] = f32_to_bf16_bits(p[2]) | (f32_to_bf16_bits(p[3]) << 16);
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      o[t][0] *= alpha;
      o[t][1] *= alpha;
      o[t][2] *= alpha;
      o[t][3] *= alpha;
    }
    // O^T[d][q] += V^T[d][keys] P^T[keys][q]; K slots of group g are keys
    // 32c + 4g + (0..3) and 32c + 16 + 4g + (0..3)
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const u32x4 pv = {pb[2 * c2][0], pb[2 * c2][1], pb[2 * c2 + 1][0], pb[2 * c2 + 1][1]};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const uint16_t* vrow = &Vt[(t * 16 + n) * VS + 32 * c2 + 4 * g];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
        const u32x4 av = {lo.x, lo.y, hi.x, hi.y};
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                       __builtin_bit_cast(bf16x8, pv), o[t], 0, 0, 0);
      }
    }
  }

  float l = l_part + __shfl_xor(l_part, 16);
  l += __shfl_xor(l, 32);
  if (q_ok) {
    const size_t row = (bh * nsplit_max + split) * T + qi;
    float* orow = part_o + row * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      *reinterpret_cast<float4*>(orow + t * 16 + 4 * g) = float4{o[t][0], o[t][1], o[t][2], o[t][3]};
    if (g == 0) part_ml[row] = float2{m_run, l};
  }
}

// Merge the splits of one (sequence, query, head): grid (T, Hq, B), D threads.
template <typename OutT>
__global__ void tree_attn_combine_kernel(int T, int Hq, int D, int max_slots, int nsplit_max,
                                         const int32_t* __restrict__ prefix_len,
                                         const float* __restrict__ part_o, const float2* __restrict__ part_ml,
                                         OutT* __restrict__ out) {
  const int qi = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int L = prefix_len[b];
  if (L > max_slots - T) L = max_slots - T;
  if (L < 0) L = 0;
  const int ns = num_splits(L + T);
  const size_t bh = static_cast<size_t>(b) * Hq + h;
  float M = -__builtin_huge_valf();
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[(bh * nsplit_max + s) * T + qi].x);
  const float ref = M == -__builtin_huge_valf() ? 0.f : M;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f, den = 0.f;
    for (int s = 0; s < ns; ++s) {
      const size_t row = (bh * nsplit_max + s) * T + qi;
      const float2 ml = part_ml[row];
      const float w = exp2f(ml.x - ref);
      acc += w * part_o[row * D + d];
      den += w * ml.y;
    }
    const float v = acc / den;
    const size_t o = ((static_cast<size_t>(b) * T + qi) * Hq + h) * D + d;
    if constexpr (sizeof(OutT) == 2) out[o] = static_cast<uint16_t>(f32_to_bf16_bits(v));
    else out[o] = v;
  }
}

// f32: one wave per (sequence, head, query); lanes over keys for scores,
// lanes over d for the output.
__global__ __launch_bounds__(64) void tree_attn_f32_kernel(
    int T, int Hq, int D, int max_slots, const float* __restrict__ q, const float* __restrict__ kc,
    const float* __restrict__ vc, const int32_t* __restrict__ prefix_len,
    const uint8_t* __restrict__ tree_mask, float scale, float* __restrict__ out) {
  const int qi = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  int L = prefix_len[b];
  if (L > max_slots - T) L = max_slots - T;
  if (L < 0) L = 0;
  const int total = L + T;
  const size_t bh = static_cast<size_t>(b) * Hq + h;
  const float* qrow = q + ((static_cast<size_t>(b) * T + qi) * Hq + h) * D;
  const float* kb = kc + bh * max_slots * D;
  const float* vb = vc + bh * max_slots * D;
  float m_run = -__builtin_huge_valf(), l = 0.f;
  float o0 = 0.f, o1 = 0.f;   // d = lane, lane + 64
  for (int c0 = 0; c0 < total; c0 += 64) {
    const int key = c0 + lane;
    bool allowed = key < total;
    if (allowed && key >= L) allowed = tree_mask[static_cast<size_t>(qi) * T + (key - L)] != 0;
    float sc = -__builtin_huge_valf();
    if (allowed) {
      float acc = 0.f;
      for (int d = 0; d < D; d += 4) {
        const float4 a = *reinterpret_cast<const float4*>(qrow + d);
        const float4 k = *reinterpret_cast<const float4*>(kb + static_cast<size_t>(key) * D + d);
        acc += a.x * k.x + a.y * k.y + a.z * k.z + a.w * k.w;
      }
      sc = acc * scale;
    }
    const float m_new = fmaxf(m_run, wave_max(sc));
    const float ref = m_new == -__builtin_huge_valf() ? 0.f : m_new;
    const float alpha = expf(m_run - ref);
    const float p = allowed ? expf(sc - ref) : 0.f;
    l = l * alpha + wave_sum(p);
    o0 *= alpha;
    o1 *= alpha;
    const int nk = total - c0 < 64 ? total - c0 : 64;
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = __shfl(p, jj);
      if (pj != 0.f) {
        const float* vrow = vb + static_cast<size_t>(c0 + jj) * D;
        o0 += pj * vrow[lane];
        if (D > 64) o1 += pj * vrow[lane + 64];
      }
    }
    m_run = m_new;
  }
  float* orow = out + ((static_cast<size_t>(b) * T + qi) * Hq + h) * D;
  orow[lane] = o0 / l;
  if (D > 64) orow[lane + 64] = o1 / l;
}

}  // namespace medusa

namespace {

using namespace medusa;

size_t attn_part_o_bytes(int B, int T, int Hq, int d, int max_slots) {
  const size_t nsm = static_cast<size_t>(num_splits(max_slots));
  return medusa_host::round_up(static_cast<size_t>(B) * Hq * nsm * T * d * 4, 256);
}
size_t attn_part_ml_bytes(int B, int T, int Hq, int max_slots) {
  const size_t nsm = static_cast<size_t>(num_splits(max_slots));
  return medusa_host::round_up(static_cast<size_t>(B) * Hq * nsm * T * 8, 256);
}

int check_attn(const char* fn, int dtype, int B, int T, int Hq, int d, int max_slots) {
  MEDUSA_REQUIRE(dtype == MEDUSA_F32 || dtype == MEDUSA_BF16, MEDUSA_ERR_DTYPE, "%s: dtype %d", fn, dtype);
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d", fn, B);
  MEDUSA_REQUIRE(T >= 1 && T <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: T=%d", fn, T);
  MEDUSA_REQUIRE(Hq >= 1 && Hq <= 1024, MEDUSA_ERR_SHAPE, "%s: Hq=%d", fn, Hq);
  MEDUSA_REQUIRE(d == 64 || d == 128, MEDUSA_ERR_SHAPE, "%s: d=%d not 64 or 128", fn, d);
  MEDUSA_REQUIRE(max_slots >= T && max_slots <= (1 << 24), MEDUSA_ERR_SHAPE, "%s: max_slots=%d", fn,
                 max_slots);
  return MEDUSA_OK;
}

}  // namespace

extern "C" size_t medusa_tree_attention_workspace(int dtype, int B, int T, int Hq, int d, int max_slots) {
  if (check_attn("medusa_tree_attention_workspace", dtype, B, T, Hq, d, max_slots) != MEDUSA_OK) return 0;
  if (dtype == MEDUSA_F32) return 256;
  return attn_part_o_bytes(B, T, Hq, d, max_slots) + attn_part_ml_bytes(B, T, Hq, max_slots);
}

extern "C" int medusa_tree_attention(int dtype, int B, int T, int Hq, int d, int max_slots, const void* q,
                                     const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                                     const uint8_t* tree_mask, float scale, void* out, void* ws,
                                     size_t ws_bytes, void* stream) {
  int rc = check_attn(__func__, dtype, B, T, Hq, d, max_slots);
  if (rc != MEDUSA_OK) return rc;
  MEDUSA_REQUIRE_PTR(q);
  MEDUSA_REQUIRE_PTR(k_cache);
  MEDUSA_REQUIRE_PTR(v_cache);
  MEDUSA_REQUIRE_PTR(prefix_len);
  MEDUSA_REQUIRE_PTR(tree_mask);
  MEDUSA_REQUIRE_PTR(out);
  MEDUSA_REQUIRE(scale == scale && scale > 0.f, MEDUSA_ERR_VALUE, "%s: scale must be positive", __func__);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == MEDUSA_F32) {
    hipLaunchKernelGGL(tree_attn_f32_kernel, dim3(T, Hq, B), dim3(64), 0, st, T, Hq, d, max_slots,
                       static_cast<const float*>(q), static_cast<const float*>(k_cache),
                       static_cast<const float*>(v_cache), prefix_len, tree_mask, scale,
                       static_cast<float*>(out));
    return medusa_host::hip_check("medusa_tree_attention launch");
  }
  MEDUSA_REQUIRE_PTR(ws);
  const size_t need = attn_part_o_bytes(B, T, Hq, d, max_slots) + attn_part_ml_bytes(B, T, Hq, max_slots);
  MEDUSA_REQUIRE(ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes,
                 need);
  const int nsm = num_splits(max_slots);
  const int nqb = (T + kQBlock - 1) / kQBlock;
  float* part_o = static_cast<float*>(ws);
  float2* part_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + attn_part_o_bytes(B, T, Hq, d, max_slots));
  const float sl2 = scale * kLog2e;
  dim3 grid(nsm, Hq, B * nqb);
  if (d == 128)
    hipLaunchKernelGGL(tree_attn_bf16_kernel<128>, grid, dim3(kAttnThreads), 0, st, T, Hq, max_slots, nsm, nqb,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                       static_cast<const uint16_t*>(v_cache), prefix_len, tree_mask, sl2, part_o, part_ml);
  else
    hipLaunchKernelGGL(tree_attn_bf16_kernel<64>, grid, dim3(kAttnThreads), 0, st, T, Hq, max_slots, nsm, nqb,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                       static_cast<const uint16_t*>(v_cache), prefix_len, tree_mask, sl2, part_o, part_ml);
  rc = medusa_host::hip_check("medusa_tree_attention launch");
  if (rc != MEDUSA_OK) return rc;
  hipLaunchKernelGGL(tree_attn_combine_kernel<uint16_t>, dim3(T, Hq, B), dim3(d), 0, st, T, Hq, d, max_slots,
                     nsm, prefix_len, part_o, part_ml, static_cast<uint16_t*>(out));
  return medusa_host::hip_check("medusa_tree_attention combine launch");
}
