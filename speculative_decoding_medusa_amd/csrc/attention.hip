// Tree attention on gfx950: T tree queries against a KV prefix plus the
// ancestor-only mask among the tree's own keys.
//
// bf16 path, one kernel.  The key range [0, L+T) of each (sequence, head) is
// cut into splits of whole 32-key chunks, one workgroup per (split, 64-query
// block).  A workgroup is eight waves: two halves of the query block (32
// queries, two 16-query MFMA tiles each) times four key groups.  Chunks go
// in rounds of four, one per key group, so every chunk is read from LDS by
// the two waves of its group only, and the four groups work unsynchronised
// within a round.  K and V chunks (and the block's Q) go from HBM straight
// into LDS with 16-byte direct-to-LDS loads: a ring of two rounds (eight
// chunks) in flight, no staging registers, no LDS stores; rows are kept
// whole with their 16-byte pieces XOR-swizzled by row, so the MFMA operand
// reads are free of bank conflicts.  Scores are computed transposed,
// S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: a lane then holds four
// consecutive keys of one query, which is the B-operand layout P^T needs for
// O^T += V^T P^T, so probabilities never leave registers; each K and V
// operand read serves both query tiles of the wave.  The V^T operand comes
// from the row-major V chunk through the LDS transpose read
// (ds_read_b64_tr_b16).  Online softmax in base 2 with fp32 accumulators and
// a lazily raised reference.  After the last round the four key groups'
// states are merged through LDS.  A sequence with one split writes its
// output directly; otherwise each split writes its partial (O / l in half
// precision, m and l in float32) and a second kernel merges the splits
// (log-sum-exp) and writes the output.
//
// f32 path: one wave per (sequence, head, query), online softmax over
// 64-key chunks on the VALU.
#include "common.hpp"

namespace medusa {

constexpr int kAttnThreads = 512;  // eight waves: two query halves x four key groups
constexpr int kQBlock = 64;        // queries per workgroup
constexpr int kChunk = 32;         // keys per LDS stage
constexpr int kGroups = 4;         // key groups = chunks per round
constexpr int kStages = 2 * kGroups;   // LDS ring: two rounds
constexpr int kEarly = 2;          // chunks issued together with Q
constexpr int kMinSplitKeys = 128; // shortest split
constexpr int kMaxSplits = 16;     // most splits of one (sequence, head)
constexpr float kLog2e = 1.4426950408889634f;

// Splits of a (sequence, head): total_keys / split_keys (at least one, at
// most kMaxSplits); the chunks are spread evenly over them.
__host__ __device__ inline int num_splits(int total_keys, int split_keys) {
  const int s = total_keys / split_keys;
  return s < 1 ? 1 : (s > kMaxSplits ? kMaxSplits : s);
}

// Keys per split for a launch.  One workgroup runs per compute unit (its LDS
// ring fills most of one), so W workgroups take ceil(W / 256) rounds.  A
// workgroup's time was measured on MI355X (64 queries, d 128, batch 1) as a
// fixed part (launch, Q, the first round's latency, merge and partial
// write: about 9.6 us) plus about 0.0227 us per key (its K/V stream runs at
// the rate its ring in flight sustains, about 23 GB/s); the split count
// minimising rounds x (fixed + keys per split x rate) is used, splits of at
// least kMinSplitKeys keys, with every sequence taken at max_slots keys.
inline int attn_split_keys(int B, int Hq, int d, int nqb, int max_slots) {
  const double kFixedUs = 9.6, kUsPerKey = 0.0227 * d / 128.0;
  const long long units = static_cast<long long>(B) * Hq * nqb;
  int best_keys = max_slots;
  double best = 1e300;
  for (int ns = 1; ns <= kMaxSplits; ++ns) {
    const long long sk = (static_cast<long long>(max_slots) + ns - 1) / ns;
    if (sk < kMinSplitKeys) break;
    if (num_splits(max_slots, static_cast<int>(sk)) != ns) continue;
    const long long rounds = (units * ns + 255) / 256;
    const double est = static_cast<double>(rounds) * (kFixedUs + kUsPerKey * static_cast<double>(sk));
    if (est < best - 1e-9) {
      best = est;
      best_keys = static_cast<int>(sk);
    }
  }
  return best_keys;
}

typedef short v4s __attribute__((ext_vector_type(4)));
#define LDSB(x) ((MEDUSA_LDS uint8_t*)(x))

// s_waitcnt: at most N vector-memory operations outstanding (N < 64) and
// no LDS operation outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// 16-byte direct load from global memory into LDS: lane l's piece lands at
// lds + 16*l.  Issued from inline assembly so that the compiler does not
// track it: its own bookkeeping cannot tell the ring stages apart and would
// wait for every chunk in flight before any LDS read.  The instruction
// writes no register; completion is counted by vmcnt, and the kernel waits
// for it explicitly (wait_vm) before the barrier that publishes a chunk.
__device__ __forceinline__ void lds_dma16(const void* gptr, MEDUSA_LDS void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(gptr), "{m0}"(m0) : "memory");
}

template <int D>
struct AttnLayout {
  static constexpr int PIECES = D / 8;                       // 16-byte pieces per row
  static constexpr int ROWB = D * 2;                         // bytes per row
  static constexpr int TILE = kChunk * ROWB;                 // bytes of K (or V) per chunk
  static constexpr int PER = 2 * TILE / 16 / kAttnThreads;   // direct loads per thread per chunk (K and V)
  static constexpr int QPER = kQBlock * ROWB / 16 / kAttnThreads;   // direct loads per thread for Q
  static constexpr int SH = D == 128 ? 0 : 1;                // rows sharing a bank base
  // LDS slot of piece pc of row `row`
  __device__ static int k_slot(int row, int pc) { return pc ^ ((row >> SH) & (PIECES - 1)); }
  __device__ static int v_slot(int row, int pc) { return pc ^ (2 * ((row >> SH) & (PIECES / 2 - 1))); }
};

// Issue the direct loads of chunk [c0, c0 + kChunk) into one ring stage.
// The chunk's K and V tiles are 2 * TILE / 16 pieces of 16 bytes; piece x
// (x = i * kAttnThreads + tid) is K piece x, or V piece x - TILE / 16.  A
// wave instruction covers 64 consecutive pieces, one 1 KB block of K or of
// V: lane l fills LDS slot blk * 64 + l, i.e. (row, slot), with the piece
// that slot holds under the swizzle (an involution).  Rows past k_hi repeat
// row k_hi - 1: finite data whose scores are masked.
template <int D>
__device__ __forceinline__ void attn_issue(const uint16_t* kbase, const uint16_t* vbase, int c0, int k_hi, int tid,
                                           uint8_t* kst, uint8_t* vst) {
  using Lay = AttnLayout<D>;
  constexpr int NP = Lay::TILE / 16;      // pieces per tensor
#pragma unroll
  for (int i = 0; i < Lay::PER; ++i) {
    const int x = i * kAttnThreads + tid;
    const bool is_v = x >= NP;              // uniform per wave
    const int sidx = is_v ? x - NP : x;
    const int row = sidx / Lay::PIECES, slot = sidx % Lay::PIECES;
    const size_t key = static_cast<size_t>(min(c0 + row, k_hi - 1));
    const uint16_t* src = is_v ? vbase + key * D + Lay::v_slot(row, slot) * 8
                               : kbase + key * D + Lay::k_slot(row, slot) * 8;
    lds_dma16(src, LDSB(is_v ? vst : kst) + (sidx & ~63) * 16);
  }
}

// Allowed keys of one 32-key chunk for one query, bit p = key c0 + p:
// inside the split, and either in the prefix or an ancestor (or self) in
// the tree.  mb: the query's ancestor words (LDS), bit j = tree key L + j.
__device__ __forceinline__ uint32_t chunk_allowed(int c0, int k_hi, int L, const MEDUSA_LDS uint64_t* mb) {
  const int nvalid = min(max(k_hi - c0, 0), 32);
  uint32_t allow = nvalid == 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
  if (c0 + kChunk > L) {   // the chunk reaches the tree keys (uniform)
    const int j0 = c0 - L;
    uint32_t tree;
    uint32_t prefix = 0;
    if (j0 >= 0) {
      const int w0 = j0 >> 6, sh = j0 & 63;
      const uint64_t lo = mb[w0] >> sh;
      const uint64_t hi = (sh != 0 && w0 < 3) ? (mb[w0 + 1] << (64 - sh)) : 0ull;
      tree = static_cast<uint32_t>(lo | hi);
    } else {
      tree = static_cast<uint32_t>(mb[0] << (-j0));   // -j0 in (0, 32)
      prefix = (1u << (-j0)) - 1u;
    }
    allow &= prefix | tree;
  }
  return allow;
}

// Online-softmax state of one wave: its 32 queries (two tiles of 16; lane
// n + 16g holds query n of each tile, and d rows 16t + 4g .. +3 of O^T).
template <int D>
struct AttnState {
  f32x4 o[2][D / 16];
  float m_run[2];
  float l_part[2];   // this lane's share: its keys of the chunks seen
};

// One chunk [c0, c0 + kChunk) from a ring stage for the wave's two query
// tiles: scores, online softmax, PV.  mrow[u]: the ancestor words of this
// lane's query in tile u (LDS).  The running reference m_run is raised only
// when some lane's chunk maximum exceeds it by more than kLazy (log2
// units): exponentials then stay below 2^kLazy, and O and l, both taken
// against the same reference, stay exact.  `full`: every key of the chunk
// is an allowed prefix key (no mask).
constexpr float kLazy = 8.f;
template <int D>
__device__ __forceinline__ void attn_chunk(const u32x4 (&qv)[2][D / 32], AttnState<D>& st, int c0, int k_hi, int L,
                                           bool full, int lane, float scale_log2,
                                           const MEDUSA_LDS uint64_t* const (&mrow)[2], const uint8_t* kst,
                                           const uint8_t* vst) {
  using Lay = AttnLayout<D>;
  constexpr int DT = D / 16, DS = D / 32;
  const int n = lane & 15, g = lane >> 4;
  const MEDUSA_LDS uint8_t* Kc = (const MEDUSA_LDS uint8_t*)kst;
  const MEDUSA_LDS uint8_t* Vc = (const MEDUSA_LDS uint8_t*)vst;

  // scores S^T[key = kt*16 + 4g + i][query n] of both tiles; each K operand
  // read serves both
  f32x4 s[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[u][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int row = kt * 16 + n;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const u32x4 a = *(const MEDUSA_LDS u32x4*)(Kc + row * Lay::ROWB + Lay::k_slot(row, ds * 4 + g) * 16);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        s[u][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, qv[u][ds]), s[u][kt], 0, 0, 0);
    }
  }
  const float NEG = -__builtin_huge_valf();
  u32x4 pv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!full) {
      const uint32_t allow = chunk_allowed(c0, k_hi, L, mrow[u]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((allow >> (kt * 16 + 4 * g + i)) & 1u)) s[u][kt][i] = NEG;
    }
    // the chunk maximum of this lane's query, in log2 units
    float mloc = fmaxf(fmaxf(fmaxf(s[u][0][0], s[u][0][1]), fmaxf(s[u][0][2], s[u][0][3])),
                       fmaxf(fmaxf(s[u][1][0], s[u][1][1]), fmaxf(s[u][1][2], s[u][1][3])));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    mloc *= scale_log2;
    if (ballot(mloc > st.m_run[u] + kLazy) != 0) {   // uniform: raise the reference
      const float m_new = fmaxf(st.m_run[u], mloc);
      const float alpha = st.m_run[u] == NEG ? 0.f : __builtin_amdgcn_exp2f(st.m_run[u] - m_new);
      st.l_part[u] *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        st.o[u][t][0] *= alpha;
        st.o[u][t][1] *= alpha;
        st.o[u][t][2] *= alpha;
        st.o[u][t][3] *= alpha;
      }
      st.m_run[u] = m_new;
    }
    const float nref = st.m_run[u] == NEG ? 0.f : -st.m_run[u];
    float p[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[kt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][kt][i], scale_log2, nref));
        st.l_part[u] += p[kt][i];
      }
    pv[u] = u32x4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]), pack_bf16x2(p[1][0], p[1][1]),
                  pack_bf16x2(p[1][2], p[1][3])};
  }
  // O^T[d][q] += V^T[d][keys] P^T[keys][q]; the k-slots of group g are keys
  // 4g + (0..3) and 16 + 4g + (0..3).  The transpose read gives lane m of a
  // 16-lane group element m%4 of the 8 bytes addressed by lane 4c + m/4 of
  // the group, as component c; so lane (c, qd) addresses row 16r + 4g + c,
  // columns 16t + 4qd .. +3 of the row-major V chunk.  Each V^T operand
  // serves both query tiles.
  const int vrow = 4 * g + ((lane & 15) >> 2), qd = lane & 3;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    uint32_t w4[4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 16 * r + vrow;
      const int pc = 2 * t + (qd >> 1);
      const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (MEDUSA_LDS v4s*)(Vc + row * Lay::ROWB + Lay::v_slot(row, pc) * 16 + (qd & 1) * 8));
      const uint2 w = __builtin_bit_cast(uint2, x);
      w4[2 * r] = w.x;
      w4[2 * r + 1] = w.y;
    }
    const u32x4 av = {w4[0], w4[1], w4[2], w4[3]};
#pragma unroll
    for (int u = 0; u < 2; ++u)
      st.o[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                           __builtin_bit_cast(bf16x8, pv[u]), st.o[u][t], 0, 0, 0);
  }
}

// Wait until at most k (0 <= k <= K) chunks of PER loads each are still in
// flight for this thread (and no LDS operation); s_waitcnt takes a constant.
template <int PER, int K>
__device__ __forceinline__ void wait_chunks(int k) {
  if constexpr (K == 0) {
    wait_vm<0>();
  } else {
    if (k >= K) wait_vm<PER * K>();
    else wait_chunks<PER, K - 1>(k);
  }
}

// Make the loads waited for visible to every wave: each thread waits for its
// own direct loads (later ones stay in flight), then a bare barrier
// publishes them -- a fenced barrier would also drain the loads in flight.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(kAttnThreads, 1) void tree_attn_bf16_kernel(
    int T, int Hq, int max_slots, int nsplit_max, int split_keys, int nqb, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, const int32_t* __restrict__ prefix_len,
    const uint8_t* __restrict__ tree_mask, float scale_log2, _Float16* __restrict__ part_o,
    float2* __restrict__ part_ml, uint16_t* __restrict__ out) {
  using Lay = AttnLayout<D>;
  constexpr int DT = D / 16, DS = D / 32;
  constexpr int PER = Lay::PER, QPER = Lay::QPER;
  static_assert(PER * kAttnThreads * 16 == 2 * Lay::TILE, "chunk must split into whole loads");
  static_assert(QPER * kAttnThreads * 16 == kQBlock * Lay::ROWB, "Q block must split into whole loads");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages][2][Lay::TILE];   // [stage][K, V]
  __shared__ __attribute__((aligned(1024))) uint8_t qtile[kQBlock * Lay::ROWB];
  __shared__ uint64_t mbits[kQBlock][kMaxNodes / 64];

  // Workgroup i is dispatched to XCD i % 8 (round robin): the splits of a
  // (sequence, head, query block) group take ids congruent mod 8 where the
  // grid allows, so they share one L2 for their Q and mask loads.  Only the
  // placement depends on this; any order is correct.
  int split, gi;
  {
    const int ns_l = static_cast<int>(gridDim.x);
    const int ng = static_cast<int>(gridDim.y * gridDim.z);
    const int i = static_cast<int>(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    const int blk = i / (8 * ns_l), rem = i - blk * 8 * ns_l;
    const int width = min(8, ng - 8 * blk);   // groups in this block of ids
    split = rem / width;
    gi = 8 * blk + rem % width;
  }
  const int h = gi % Hq, bz = gi / Hq;
  const int b = bz / nqb, qb = bz - b * nqb;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qh = wave & 1, kg = wave >> 1;             // query half, key group
  const int n = lane & 15, g = lane >> 4;

  // Q of the block's 64 queries (rows past T repeat row T - 1), swizzled
  // like K; issued before the prefix length is known
#pragma unroll
  for (int i = 0; i < QPER; ++i) {
    const int x = i * kAttnThreads + tid;
    const int row = x / Lay::PIECES, slot = x % Lay::PIECES;
    const int qq = min(qb * kQBlock + row, T - 1);
    const uint16_t* src = q + ((static_cast<size_t>(b) * T + qq) * Hq + h) * D + Lay::k_slot(row, slot) * 8;
    lds_dma16(src, LDSB(qtile) + (x & ~63) * 16);
  }

  int L = prefix_len[b];
  if (L > max_slots - T) L = max_slots - T;
  if (L < 0) L = 0;
  const int total = L + T;
  const int ns = num_splits(total, split_keys);
  if (split >= ns) {
    wait_vm<0>();   // no direct load may land in LDS after the workgroup leaves
    return;
  }
  // whole chunks per split, spread evenly; only a head's last chunk is ragged
  const int nc_all = (total + kChunk - 1) / kChunk;
  const int c_base = nc_all / ns, c_rem = nc_all % ns;
  const int k_lo = kChunk * (split * c_base + min(split, c_rem));
  const int k_hi = min(total, k_lo + kChunk * (c_base + (split < c_rem ? 1 : 0)));
  const size_t bh = static_cast<size_t>(b) * Hq + h;
  const uint16_t* kbase = kc + bh * max_slots * D;
  const uint16_t* vbase = vc + bh * max_slots * D;
  const int nch = (k_hi - k_lo + kChunk - 1) / kChunk;
  const int nrounds = (nch + kGroups - 1) / kGroups;

  // Ancestor words of the block's queries (only in a split that reaches
  // the tree): word ww of query row r is a ballot over a coalesced load of
  // the mask row; each wave builds eight rows.  The bytes of word 0 are
  // loaded here, behind Q and ahead of the K/V stream, so the wait for Q
  // covers them; the ballots wait until the first round that reaches the
  // tree, since the compiler's wait before them is a wait for every load
  // issued so far.
  const bool has_tree = k_hi > L;
  uint8_t mbv[8];
  if (has_tree) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int qq = qb * kQBlock + wave * 8 + r;
      mbv[r] = tree_mask[static_cast<size_t>(min(qq, T - 1)) * T + min(lane, T - 1)];
    }
  }

  // The first kEarly chunks go out with Q; the rest of rounds 0 and 1 only
  // once Q has landed, so that Q and the first chunks are not queued behind
  // the whole burst of every workgroup's loads.
  const int n0 = min(kStages, nch);
  const int ne = min(kEarly, n0);
  for (int c = 0; c < ne; ++c)
    attn_issue<D>(kbase, vbase, k_lo + c * kChunk, k_hi, tid, ring[c][0], ring[c][1]);
  bool mask_ready = !has_tree;
  auto build_mask = [&]() {
    const int nw = (T + 63) >> 6;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int qq = qb * kQBlock + wave * 8 + r;
      const uint64_t word = ballot(qq < T && lane < T && mbv[r] != 0);
      if (lane == 0) mbits[wave * 8 + r][0] = word;
    }
#pragma unroll 1
    for (int ww = 1; ww < nw; ++ww) {   // trees of more than 64 nodes
      const int j = ww * 64 + lane;
      uint8_t mw[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int qq = qb * kQBlock + wave * 8 + r;
        mw[r] = tree_mask[static_cast<size_t>(min(qq, T - 1)) * T + min(j, T - 1)];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int qq = qb * kQBlock + wave * 8 + r;
        const uint64_t word = ballot(qq < T && j < T && mw[r] != 0);
        if (lane == 0) mbits[wave * 8 + r][ww] = word;
      }
    }
  };

  // Q from LDS into registers once its loads (the oldest in flight, with
  // the mask bytes) are in
  wait_chunks<PER, kEarly>(ne);
  ring_barrier();
  for (int c = ne; c < n0; ++c)
    attn_issue<D>(kbase, vbase, k_lo + c * kChunk, k_hi, tid, ring[c][0], ring[c][1]);
  u32x4 qv[2][DS];   // Q[query][s*32 + 8g .. +8]: the B operand of S^T, per tile
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = qh * 32 + u * 16 + n;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qv[u][s] = *(const MEDUSA_LDS u32x4*)(LDSB(qtile) + row * Lay::ROWB + Lay::k_slot(row, s * 4 + g) * 16);
  }
  const MEDUSA_LDS uint64_t* const mrow[2] = {(const MEDUSA_LDS uint64_t*)mbits[qh * 32 + n],
                                              (const MEDUSA_LDS uint64_t*)mbits[qh * 32 + 16 + n]};

  AttnState<D> st;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    st.m_run[u] = -__builtin_huge_valf();
    st.l_part[u] = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t) st.o[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Round r holds chunks 4r .. 4r+3 in ring set r % 2; key group kg takes
  // chunk 4r + kg.  After the barrier of round r (r >= 1) every wave is done
  // with round r - 1, whose set then takes round r + 1.
  for (int r = 0; r < nrounds; ++r) {
    const int need_hi = min(kGroups * r + kGroups - 1, nch - 1);
    const int issued_hi = min(kGroups * (r < 1 ? 2 : r + 1) - 1, nch - 1);
    wait_chunks<PER, kGroups>(issued_hi - need_hi);
    if (!mask_ready && k_lo + kChunk * min(kGroups * r + kGroups, nch) > L) {   // uniform: first round reaching the tree
      build_mask();
      mask_ready = true;
    }
    ring_barrier();
    if (r >= 1) {
#pragma unroll 1
      for (int c = kGroups * (r + 1); c < min(kGroups * (r + 2), nch); ++c) {
        const int sn = c % kStages;
        attn_issue<D>(kbase, vbase, k_lo + c * kChunk, k_hi, tid, ring[sn][0], ring[sn][1]);
      }
    }
    const int c = kGroups * r + kg;
    if (c < nch) {
      const int c0 = k_lo + c * kChunk;
      const bool full = c0 + kChunk <= min(L, k_hi);
      const int sn = c % kStages;
      attn_chunk<D>(qv, st, c0, k_hi, L, full, lane, scale_log2, mrow, ring[sn][0], ring[sn][1]);
    }
  }

  // Key groups 1-3 hand their states to group 0 through LDS (the ring is
  // free: every direct load has landed and every chunk has been read):
  // per lane 2 * DT + 1 16-byte words (O of both tiles, then m and l of
  // both), each wave instruction writing or reading 1 KB contiguously.
  constexpr int NF4 = 2 * DT + 1;
  static_assert(3 * 2 * NF4 * kWave * 16 <= kStages * 2 * Lay::TILE, "merge area must fit the ring");
  f32x4* xfer = reinterpret_cast<f32x4*>(&ring[0][0][0]);
  ring_barrier();
  if (kg != 0) {
    f32x4* xw = xfer + ((kg - 1) * 2 + qh) * NF4 * kWave + lane;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < DT; ++t) xw[(u * DT + t) * kWave] = st.o[u][t];
    xw[2 * DT * kWave] = f32x4{st.m_run[0], st.m_run[1], st.l_part[0], st.l_part[1]};
  }
  ring_barrier();
  const float NEG = -__builtin_huge_valf();
  if (kg == 0) {
    f32x4 ml[kGroups - 1];
#pragma unroll
    for (int k = 1; k < kGroups; ++k) ml[k - 1] = xfer[(((k - 1) * 2 + qh) * NF4 + 2 * DT) * kWave + lane];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float M = st.m_run[u];
#pragma unroll
      for (int k = 1; k < kGroups; ++k) M = fmaxf(M, ml[k - 1][u]);
      const float a0 = st.m_run[u] == NEG ? 0.f : exp2f(st.m_run[u] - M);
      st.l_part[u] *= a0;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.o[u][t][i] *= a0;
#pragma unroll
      for (int k = 1; k < kGroups; ++k) {
        const f32x4* xw = xfer + ((k - 1) * 2 + qh) * NF4 * kWave + lane;
        const float mk = ml[k - 1][u];
        const float ak = mk == NEG ? 0.f : exp2f(mk - M);
        st.l_part[u] += ak * ml[k - 1][2 + u];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const f32x4 x = xw[(u * DT + t) * kWave];
#pragma unroll
          for (int i = 0; i < 4; ++i) st.o[u][t][i] += ak * x[i];
        }
      }
      st.m_run[u] = M;
      float l = st.l_part[u] + __shfl_xor(st.l_part[u], 16);
      st.l_part[u] = l + __shfl_xor(l, 32);     // the query's total over its four lanes
    }
    if (ns == 1) {
      // the only split: normalise and write the output
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qi = qb * kQBlock + qh * 32 + u * 16 + n;
        if (qi < T) {
          const float inv = 1.f / st.l_part[u];
          uint16_t* orow = out + ((static_cast<size_t>(b) * T + qi) * Hq + h) * D;
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            uint2 w;
            w.x = pack_bf16x2(st.o[u][t][0] * inv, st.o[u][t][1] * inv);
            w.y = pack_bf16x2(st.o[u][t][2] * inv, st.o[u][t][3] * inv);
            *reinterpret_cast<uint2*>(orow + t * 16 + 4 * g) = w;
          }
        }
      }
      return;
    }
    // this split's partial: O / l in half precision [group][split][64
    // rows][D] and (m, l) in float32 [group][split][64], group = (sequence,
    // head, query block).  O / l is a convex combination of V rows, so its
    // range is theirs; the merge weights each by l e^(m - M).
    const size_t grp = bh * nqb + qb;
    _Float16* po = part_o + (grp * nsplit_max + split) * kQBlock * D;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = qh * 32 + u * 16 + n;
      const float inv = st.l_part[u] > 0.f ? 1.f / st.l_part[u] : 0.f;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 v = {static_cast<_Float16>(st.o[u][t][0] * inv), static_cast<_Float16>(st.o[u][t][1] * inv),
                      static_cast<_Float16>(st.o[u][t][2] * inv), static_cast<_Float16>(st.o[u][t][3] * inv)};
        *reinterpret_cast<h4*>(po + row * D + t * 16 + 4 * g) = v;
      }
      if (g == 0) part_ml[(grp * nsplit_max + split) * kQBlock + row] = float2{st.m_run[u], st.l_part[u]};
    }
  }
}

// Merge the splits of each (sequence, head, query) by log-sum-exp.  D/4
// threads per query, four output columns each (8-byte half-precision
// partial loads); a 256-thread workgroup takes 1024/D consecutive queries of
// one (sequence, head), so a wave instruction reads 512 bytes of one split
// contiguously.
// Splits are taken eight at a time with all their loads issued together,
// merged online against a running maximum.  The first eight are addressed
// within the workspace's nsplit_max splits, so their loads go out with the
// prefix length's in one round trip; splits at or past the sequence's own
// count (never written by this call) are dropped by selects, never
// multiplied.  A sequence with one split was written by the main kernel.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_combine_kernel(int B, int T, int Hq, int max_slots, int nsplit_max,
                                                              int split_keys, const int32_t* __restrict__ prefix_len,
                                                              const _Float16* __restrict__ part_o,
                                                              const float2* __restrict__ part_ml,
                                                              uint16_t* __restrict__ out) {
  constexpr int TPQ = D / 4, QPW = 256 / TPQ, U = 8;
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const int t = threadIdx.x % TPQ;
  // B * Hq * T * D / 4 stays below 2^31 (B <= 16, Hq <= 1024, T <= 256)
  const unsigned Q = blockIdx.x * QPW + threadIdx.x / TPQ;
  if (Q >= static_cast<unsigned>(B * Hq * T)) return;
  const int qi = static_cast<int>(Q % static_cast<unsigned>(T));
  const int h = static_cast<int>((Q / static_cast<unsigned>(T)) % static_cast<unsigned>(Hq));
  const int b = static_cast<int>(Q / static_cast<unsigned>(T * Hq));
  const int nqb = (T + kQBlock - 1) / kQBlock;
  const size_t grp = (static_cast<size_t>(b) * Hq + h) * nqb + qi / kQBlock;
  const int row = qi % kQBlock;
  const float NEG = -__builtin_huge_valf();
  float M = NEG, den = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float2 ml[U];
  h4 ov[U];
  auto load = [&](int s0, int smax) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t r = (grp * nsplit_max + min(s0 + u, smax - 1)) * kQBlock + row;
      ml[u] = part_ml[r];
      ov[u] = *reinterpret_cast<const h4*>(part_o + r * D + 4 * t);
    }
  };
  load(0, nsplit_max);
  int L = prefix_len[b];
  if (L > max_slots - T) L = max_slots - T;
  if (L < 0) L = 0;
  const int ns = num_splits(L + T, split_keys);
  if (ns == 1) return;
  for (int s0 = 0; s0 < ns; s0 += U) {
    if (s0 > 0) load(s0, ns);
    float bm = NEG;
#pragma unroll
    for (int u = 0; u < U; ++u) bm = fmaxf(bm, s0 + u < ns ? ml[u].x : NEG);
    const float Mn = fmaxf(M, bm);
    const float ref = Mn == NEG ? 0.f : Mn;
    const float f = M == NEG ? 0.f : exp2f(M - ref);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] *= f;
    den *= f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < ns && ml[u].x != NEG) {
        const float w = exp2f(ml[u].x - ref) * ml[u].y;   // the split's weight: l e^(m - M)
        acc[0] += w * static_cast<float>(ov[u][0]);
        acc[1] += w * static_cast<float>(ov[u][1]);
        acc[2] += w * static_cast<float>(ov[u][2]);
        acc[3] += w * static_cast<float>(ov[u][3]);
        den += w;
      }
    }
    M = Mn;
  }
  const size_t o = ((static_cast<size_t>(b) * T + qi) * Hq + h) * D + 4 * t;
  uint2 w;
  w.x = pack_bf16x2(acc[0] / den, acc[1] / den);
  w.y = pack_bf16x2(acc[2] / den, acc[3] / den);
  *reinterpret_cast<uint2*>(out + o) = w;
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

// Workspace: the splits' partials (O / l [group][split][64][d] half
// precision and (m, l) [group][split][64] float32; group = (sequence, head,
// query block)), sized for the most splits any launch at this max_slots uses.
int attn_nsplit_max(int max_slots) { return num_splits(max_slots, kMinSplitKeys); }
size_t attn_part_o_bytes(int B, int T, int Hq, int d, int max_slots) {
  const size_t nqb = static_cast<size_t>((T + kQBlock - 1) / kQBlock);
  return medusa_host::round_up(static_cast<size_t>(B) * Hq * nqb * attn_nsplit_max(max_slots) * kQBlock * d * 2, 256);
}
size_t attn_part_ml_bytes(int B, int T, int Hq, int max_slots) {
  const size_t nqb = static_cast<size_t>((T + kQBlock - 1) / kQBlock);
  return medusa_host::round_up(static_cast<size_t>(B) * Hq * nqb * attn_nsplit_max(max_slots) * kQBlock * 8, 256);
}
size_t attn_ws_bytes(int B, int T, int Hq, int d, int max_slots) {
  return attn_part_o_bytes(B, T, Hq, d, max_slots) + attn_part_ml_bytes(B, T, Hq, max_slots);
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
  return attn_ws_bytes(B, T, Hq, d, max_slots);
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
  const size_t need = attn_ws_bytes(B, T, Hq, d, max_slots);
  MEDUSA_REQUIRE(ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes,
                 need);
  const int nqb = (T + kQBlock - 1) / kQBlock;
  const int sk = attn_split_keys(B, Hq, d, nqb, max_slots);
  const int nsm = attn_nsplit_max(max_slots);
  const int nsl = num_splits(max_slots, sk);   // splits of the launch (no sequence uses more)
  char* base = static_cast<char*>(ws);
  _Float16* part_o = reinterpret_cast<_Float16*>(base);
  float2* part_ml = reinterpret_cast<float2*>(base + attn_part_o_bytes(B, T, Hq, d, max_slots));
  const float sl2 = scale * kLog2e;
  dim3 grid(nsl, Hq, B * nqb);
  uint16_t* o16 = static_cast<uint16_t*>(out);
  if (d == 128)
    hipLaunchKernelGGL(tree_attn_bf16_kernel<128>, grid, dim3(kAttnThreads), 0, st, T, Hq, max_slots, nsm, sk, nqb,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                       static_cast<const uint16_t*>(v_cache), prefix_len, tree_mask, sl2, part_o, part_ml, o16);
  else
    hipLaunchKernelGGL(tree_attn_bf16_kernel<64>, grid, dim3(kAttnThreads), 0, st, T, Hq, max_slots, nsm, sk, nqb,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                       static_cast<const uint16_t*>(v_cache), prefix_len, tree_mask, sl2, part_o, part_ml, o16);
  rc = medusa_host::hip_check("medusa_tree_attention launch");
  if (rc != MEDUSA_OK || nsl == 1) return rc;   // one split everywhere: no merge
  const unsigned cgrid = static_cast<unsigned>((B * Hq * T * (d / 4) + 255) / 256);
  if (d == 128)
    hipLaunchKernelGGL(tree_attn_combine_kernel<128>, dim3(cgrid), dim3(256), 0, st, B, T, Hq, max_slots, nsm, sk,
                       prefix_len, part_o, part_ml, o16);
  else
    hipLaunchKernelGGL(tree_attn_combine_kernel<64>, dim3(cgrid), dim3(256), 0, st, B, T, Hq, max_slots, nsm, sk,
                       prefix_len, part_o, part_ml, o16);
  return medusa_host::hip_check("medusa_tree_attention combine launch");
}
