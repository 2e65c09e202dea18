// Internal helpers shared by the libmedusa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "medusa.h"

namespace medusa {

constexpr int kWave = 64;
constexpr int kMaxBatch = 16;
constexpr int kMaxHeads = 8;
constexpr int kMaxTopk = 64;
constexpr int kMaxNodes = 256;

// MFMA operand/accumulator vector types.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round a float32 to bf16 (nearest, ties to even).  Finite inputs only
// matter here; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats to packed bf16, a in the low half (round to nearest even, one
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Wave-wide scans and reductions on DPP lane moves (register to register,
// no LDS round trip): row_shr:1, 2, 4, 8 (lane i takes lane i - n of its
// row of 16; lanes with no source, and rows outside the row mask, take
// `fill`), then row_bcast:15 into rows 1 and 3 and row_bcast:31 into rows 2
// and 3 carry each row's last lane into the rows above it.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t fill) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(fill), static_cast<int>(v), kCtrl, kRowMask, 0xf, false));
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t dpp_add_u64(uint64_t v) {
  const uint64_t lo = dpp_u32<kCtrl, kRowMask>(static_cast<uint32_t>(v), 0u);
  const uint64_t hi = dpp_u32<kCtrl, kRowMask>(static_cast<uint32_t>(v >> 32), 0u);
  return v + ((hi << 32) | lo);
}

// inclusive prefix sum over the wave's 64 lanes in lane order
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  v = dpp_add_u64<0x111, 0xf>(v);
  v = dpp_add_u64<0x112, 0xf>(v);
  v = dpp_add_u64<0x114, 0xf>(v);
  v = dpp_add_u64<0x118, 0xf>(v);
  v = dpp_add_u64<0x142, 0xa>(v);
  return dpp_add_u64<0x143, 0xc>(v);
}

// inclusive prefix sum over the wave's 64 lanes in lane order
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  v += static_cast<int>(dpp_u32<0x111, 0xf>(static_cast<uint32_t>(v), 0u));
  v += static_cast<int>(dpp_u32<0x112, 0xf>(static_cast<uint32_t>(v), 0u));
  v += static_cast<int>(dpp_u32<0x114, 0xf>(static_cast<uint32_t>(v), 0u));
  v += static_cast<int>(dpp_u32<0x118, 0xf>(static_cast<uint32_t>(v), 0u));
  v += static_cast<int>(dpp_u32<0x142, 0xa>(static_cast<uint32_t>(v), 0u));
  return v + static_cast<int>(dpp_u32<0x143, 0xc>(static_cast<uint32_t>(v), 0u));
}

// the wave's maximum (kMax) or minimum of signed ints, in every lane
template <bool kMax>
__device__ __forceinline__ int wave_reduce_i32_dpp(int v) {
  const uint32_t id = kMax ? 0x80000000u : 0x7fffffffu;
  auto op = [](int a, int b) { return kMax ? max(a, b) : min(a, b); };
  v = op(v, static_cast<int>(dpp_u32<0x111, 0xf>(static_cast<uint32_t>(v), id)));
  v = op(v, static_cast<int>(dpp_u32<0x112, 0xf>(static_cast<uint32_t>(v), id)));
  v = op(v, static_cast<int>(dpp_u32<0x114, 0xf>(static_cast<uint32_t>(v), id)));
  v = op(v, static_cast<int>(dpp_u32<0x118, 0xf>(static_cast<uint32_t>(v), id)));
  v = op(v, static_cast<int>(dpp_u32<0x142, 0xa>(static_cast<uint32_t>(v), id)));
  v = op(v, static_cast<int>(dpp_u32<0x143, 0xc>(static_cast<uint32_t>(v), id)));
  return __builtin_amdgcn_readlane(v, kWave - 1);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l));
  return (hi << 32) | lo;
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_f32(float v, float fill) {
  return __builtin_bit_cast(float, dpp_u32<kCtrl, kRowMask>(__builtin_bit_cast(uint32_t, v),
                                                            __builtin_bit_cast(uint32_t, fill)));
}

// the wave's maximum (kMax) or sum, in every lane
template <bool kMax>
__device__ __forceinline__ float wave_reduce_dpp(float v) {
  const float id = kMax ? -__builtin_huge_valf() : 0.f;
  auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : a + b; };
  v = op(v, dpp_f32<0x111, 0xf>(v, id));
  v = op(v, dpp_f32<0x112, 0xf>(v, id));
  v = op(v, dpp_f32<0x114, 0xf>(v, id));
  v = op(v, dpp_f32<0x118, 0xf>(v, id));
  v = op(v, dpp_f32<0x142, 0xa>(v, id));
  v = op(v, dpp_f32<0x143, 0xc>(v, id));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kWave - 1));
}

// Total order used by every top-k and argmax here: larger value first,
// equal values by smaller index.  NaN never wins.
__device__ __forceinline__ bool beats(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// The wave's (max, first index) under `beats`, in every lane.
__device__ __forceinline__ void wave_argmax_dpp(float& v, int& i) {
  const float fv = -__builtin_huge_valf();
  const uint32_t fi = 0x7fffffffu;
  auto step = [&](float ov, int oi) {
    if (beats(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  };
  step(dpp_f32<0x111, 0xf>(v, fv), static_cast<int>(dpp_u32<0x111, 0xf>(static_cast<uint32_t>(i), fi)));
  step(dpp_f32<0x112, 0xf>(v, fv), static_cast<int>(dpp_u32<0x112, 0xf>(static_cast<uint32_t>(i), fi)));
  step(dpp_f32<0x114, 0xf>(v, fv), static_cast<int>(dpp_u32<0x114, 0xf>(static_cast<uint32_t>(i), fi)));
  step(dpp_f32<0x118, 0xf>(v, fv), static_cast<int>(dpp_u32<0x118, 0xf>(static_cast<uint32_t>(i), fi)));
  step(dpp_f32<0x142, 0xa>(v, fv), static_cast<int>(dpp_u32<0x142, 0xa>(static_cast<uint32_t>(i), fi)));
  step(dpp_f32<0x143, 0xc>(v, fv), static_cast<int>(dpp_u32<0x143, 0xc>(static_cast<uint32_t>(i), fi)));
  v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kWave - 1));
  i = __builtin_amdgcn_readlane(i, kWave - 1);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Statistics of one node's logits over a set of vocabulary entries: the raw
// maximum and its first index and, for a positive temperature t, with
// z = logit / t: m = max z, S = sum exp(z - m), A = sum (z - m) exp(z - m).
// An empty set has mx = m = -inf, S = A = 0.
struct RowStat {
  float mx;     // max of the raw logits
  int arg;      // first index of the max
  float m;      // max of z (temperature > 0)
  float S;      // sum exp(z - m)
  float A;      // sum (z - m) exp(z - m)
};

// The per-step tree gather of medusa_tree_candidates as kernel arguments:
// tree_candidates[b][t] = [root_token[b], topk_ids[b][0][..], ...][tree_indices[t]]
// and position_ids[b][t] = prefix_len[b] + depth[t].  T = 0: no gather.
struct TreeGather {
  int T;
  const int32_t* tree_indices;
  const int32_t* depth;
  const int32_t* root_token;
  const int32_t* prefix_len;
  int32_t* tree_candidates;
  int32_t* position_ids;
};

// a <- statistics of the union of two disjoint sets (log-sum-exp rescaling;
// an empty side contributes nothing).
__device__ __forceinline__ void rowstat_merge(RowStat& a, const RowStat& b, bool typical) {
  if (beats(b.mx, b.arg, a.mx, a.arg)) {
    a.mx = b.mx;
    a.arg = b.arg;
  }
  if (!typical) return;
  const float NEG = -__builtin_huge_valf();
  if (b.m == NEG) return;
  if (a.m == NEG) {
    a.m = b.m;
    a.S = b.S;
    a.A = b.A;
    return;
  }
  const float m = fmaxf(a.m, b.m);
  const float wa = expf(a.m - m), wb = expf(b.m - m);
  a.A = wa * (a.A + (a.m - m) * a.S) + wb * (b.A + (b.m - m) * b.S);
  a.S = wa * a.S + wb * b.S;
  a.m = m;
}

// Pointers into LDS that stay LDS pointers (ds_read/ds_write) even when they
// are volatile or pass through functions; a generic pointer would be lowered
// to flat accesses, which count against the vector-memory counter.
#define MEDUSA_LDS __attribute__((address_space(3)))
typedef volatile MEDUSA_LDS float lds_vfloat;
typedef volatile MEDUSA_LDS int lds_vint;

}  // namespace medusa

// ---------------------------------------------------------------- host side
namespace medusa_host {

void set_error(const char* fmt, ...);
int hip_check(const char* what);  // MEDUSA_OK or MEDUSA_ERR_HIP after a launch

// Acceptance test from per-(node, vocabulary block) statistics and the
// children's logits (posterior.hip; used by the fused base lm_head).
int posterior_from_parts(int B, int T, int V, int p_max, int D, int nparts, const medusa::RowStat* parts,
                         medusa::RowStat* merged, const float* child_z, const int32_t* tree_candidates,
                         const int32_t* retrieve, const int32_t* num_paths, float temperature, float eps,
                         float delta, int32_t* best_path, int32_t* accept_len, int32_t* next_token,
                         hipStream_t st);

// Medusa heads' lm_head + top-k lists at batch > 2 on the skinny-GEMM kernel
// (base_head.hip): r's hi/lo planes into `planes` [K][2B][H], then one
// sorted top-k list per (head, sequence, 128-entry vocabulary block) in
// cand_v / cand_i [K][B][heads_gemm_lists(V)][k].
// r == nullptr: the planes are already in place (heads_res_gemm).
inline int heads_gemm_lists(int V) { return (V + 127) / 128; }
int heads_lm_gemm(int B, int H, int V, int K, int k, const float* r, const void* w_lm, int packed,
                  float* logits_or_null, uint16_t* planes, float* cand_v, int32_t* cand_i, hipStream_t st);

// The heads' ResBlock on packed W1 (medusa_heads_pack with V = H) on the same
// kernel, K split into heads_res_splits(H, K) slices whose float32 partial
// sums go to `part` [S][K][B][H]; a second kernel adds them up, applies bias,
// SiLU and the residual and writes r (optional, [B][K][H]) and its planes.
constexpr int kHeadsResMaxSplits = 8;
int heads_res_splits(int H, int K);
int heads_res_gemm(int B, int H, int K, const uint16_t* hidden, const void* w1_packed, const uint16_t* b1,
                   float* r_or_null, float* part, uint16_t* planes, hipStream_t st);

// The tree gather as its own launch (tree.hip), topk_ids [B][K][topk].
int launch_tree_candidates(int B, int K, int topk, const int32_t* topk_ids, const medusa::TreeGather& tg,
                           hipStream_t st);

// Acceptance from one drawn token per node (posterior.hip; nucleus mode).
int decide_on_draws(int B, int T, int V, int p_max, int D, const medusa::RowStat* draws,
                    const int32_t* tree_candidates, const int32_t* retrieve, const int32_t* num_paths,
                    int32_t* best_path, int32_t* accept_len, int32_t* next_token, hipStream_t st);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int dtype_size(int dtype) {
  return dtype == MEDUSA_F32 ? 4 : (dtype == MEDUSA_BF16 ? 2 : 0);
}

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace medusa_host

// Validation helpers: return the status from the enclosing entry point.
#define MEDUSA_REQUIRE(cond, code, ...)            \
  do {                                             \
    if (!(cond)) {                                 \
      medusa_host::set_error(__VA_ARGS__);         \
      return (code);                               \
    }                                              \
  } while (0)

#define MEDUSA_REQUIRE_PTR(p)                                                           \
  do {                                                                                  \
    MEDUSA_REQUIRE((p) != nullptr, MEDUSA_ERR_NULL, "%s: %s is NULL", __func__, #p);    \
    MEDUSA_REQUIRE(medusa_host::aligned16(p), MEDUSA_ERR_ALIGN,                         \
                   "%s: %s is not 16-byte aligned", __func__, #p);                      \
  } while (0)
