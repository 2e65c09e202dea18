// Tree attention on gfx950: T tree queries against a KV prefix plus the
// ancestor-only mask among the tree's own keys.
//
// bf16 path.  The key range [0, L+T) of each (sequence, head) is cut into
// num_splits splits of whole 32-key chunks, one workgroup each.  A workgroup
// holds up to 64 queries in two groups of four waves (16 queries a wave);
// the groups take alternate chunks of the split.  K and V chunks go from HBM
// straight into an eight-stage LDS ring with 16-byte direct-to-LDS loads (up
// to six chunks in flight), so the stream needs no registers and no LDS
// stores; rows are kept whole and the 16-byte pieces within a row are
// XOR-swizzled by row so the MFMA operand reads are free of bank conflicts.
// Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16: a lane then holds four consecutive keys of one
// query, which is the B-operand layout P^T needs for O^T += V^T P^T, so
// probabilities never leave registers.  The V^T operand is read from the
// row-major V chunk with the LDS transpose read (ds_read_b64_tr_b16).
// Online softmax in base 2, fp32 accumulators.  The second group hands its
// (O, m, l) to the first through LDS; each split writes (O unnormalised, m,
// l) and a second kernel merges the splits (log-sum-exp).  Every global load
// is unconditional with a clamped index (masked at use), so no load waits
// behind a branch.
//
// f32 path: one wave per (sequence, head, query), online softmax over
// 64-key chunks on the VALU.
#include "common.hpp"

namespace medusa {

constexpr int kAttnThreads = 512;   // two groups of four waves
constexpr int kQBlock = 64;        // queries per workgroup
constexpr int kChunk = 32;         // keys per LDS stage
constexpr int kStages = 8;         // LDS ring depth: up to kStages - 2 chunks in flight
constexpr int kSplit = 256;        // target keys per split
constexpr float kLog2e = 1.4426950408889634f;

// Splits of a (sequence, head): split_keys (a multiple of kChunk, at least
// kSplit) to twice that many keys each, whole chunks.
__host__ __device__ inline int num_splits(int total_keys, int split_keys) {
  const int s = total_keys / split_keys;
  return s < 1 ? 1 : s;
}

// Keys per split for a launch.  A workgroup's ring fills most of a compute
// unit's LDS, so one runs per unit and a launch of W workgroups takes
// ceil(W / 256) rounds; each workgroup costs a fixed part (Q load, ring
// fill, partial-result write: about 11 us measured on MI355X) plus its K/V
// bytes at about 38 GB/s per unit.  With every sequence taken at max_slots
// keys, the number of splits n minimising rounds(n) * (fixed + bytes / n)
// is chosen and split_keys = max_slots / n (whole chunks, at least kSplit).
// Long prefixes at batch 1 get one full round of workgroups; many
// (sequence, head) pairs get one split each.
inline int attn_split_keys(int B, int Hq, int d, int nqb, int max_slots) {
  const double kFixedUs = 11.0, kUsPerByte = 1.0 / 38000.0;
  const long long units = static_cast<long long>(B) * Hq * nqb;
  const int nmax = num_splits(max_slots, kSplit);
  int best_s = kSplit;
  double best = 1e300;
  for (int n = 1; n <= nmax; ++n) {
    long long sk = static_cast<long long>(max_slots) / n / kChunk * kChunk;
    if (sk < kSplit) sk = kSplit;
    const int ns = num_splits(max_slots, static_cast<int>(sk));
    const long long rounds = (units * ns + 255) / 256;
    const double est = static_cast<double>(rounds) * (kFixedUs + kUsPerByte * 4.0 * d * max_slots / ns);
    if (est < best) {
      best = est;
      best_s = static_cast<int>(sk);
    }
  }
  return best_s;
}

__device__ __forceinline__ u32x4 ld16g(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

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

// Allowed keys of one 32-key chunk for this lane's query, bit p = key c0 + p:
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

// One chunk [c0, c0 + kChunk) from a ring stage: scores, online softmax, PV.
// mrow: this lane's query row of ancestor words (LDS).  The running
// reference m_run is raised only when some lane's chunk maximum exceeds it
// by more than kLazy (log2 units): exponentials then stay below 2^kLazy,
// and O and l, both taken against the same reference, stay exact.
constexpr float kLazy = 8.f;
template <int D>
__device__ __forceinline__ void attn_chunk(const u32x4 (&qv)[D / 32], f32x4 (&o)[D / 16], float& m_run,
                                           float& l_part, int c0, int k_hi, int L, int lane, float scale_log2,
                                           const uint64_t* mrow, const uint8_t* kst, const uint8_t* vst) {
  using Lay = AttnLayout<D>;
  constexpr int DT = D / 16, DS = D / 32;
  const int n = lane & 15, g = lane >> 4;
  const MEDUSA_LDS uint8_t* Kc = (const MEDUSA_LDS uint8_t*)kst;
  const MEDUSA_LDS uint8_t* Vc = (const MEDUSA_LDS uint8_t*)vst;
  const uint32_t allow = chunk_allowed(c0, k_hi, L, (const MEDUSA_LDS uint64_t*)mrow);

  // scores S^T[key = kt*16 + 4g + i][query n]
  f32x4 s[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int row = kt * 16 + n;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const u32x4 a = *(const MEDUSA_LDS u32x4*)(Kc + row * Lay::ROWB + Lay::k_slot(row, ds * 4 + g) * 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, qv[ds]), acc, 0, 0, 0);
    }
    s[kt] = acc;
  }
  const float NEG = -__builtin_huge_valf();
  float mloc = NEG;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = ((allow >> (kt * 16 + 4 * g + i)) & 1u) ? s[kt][i] * scale_log2 : NEG;
      s[kt][i] = x;
      mloc = fmaxf(mloc, x);
    }
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  if (ballot(mloc > m_run + kLazy) != 0) {   // uniform: raise the reference
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = m_run == NEG ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_part *= alpha;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      o[t][0] *= alpha;
      o[t][1] *= alpha;
      o[t][2] *= alpha;
      o[t][3] *= alpha;
    }
    m_run = m_new;
  }
  const float ref = m_run == NEG ? 0.f : m_run;
  float p[2][4];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[kt][i] = __builtin_amdgcn_exp2f(s[kt][i] - ref);
      l_part += p[kt][i];
    }
  }
  // O^T[d][q] += V^T[d][keys] P^T[keys][q]; the k-slots of group g are keys
  // 4g + (0..3) and 16 + 4g + (0..3).  The transpose read gives lane m of a
  // 16-lane group element m%4 of the 8 bytes addressed by lane 4c + m/4 of
  // the group, as component c; so lane (c, qd) addresses row 16r + 4g + c,
  // columns 16t + 4qd .. +3 of the row-major V chunk.
  const u32x4 pv = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                    pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
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
      const uint2 u = __builtin_bit_cast(uint2, x);
      w4[2 * r] = u.x;
      w4[2 * r + 1] = u.y;
    }
    const u32x4 av = {w4[0], w4[1], w4[2], w4[3]};
    o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                   __builtin_bit_cast(bf16x8, pv), o[t], 0, 0, 0);
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

// Make chunk c visible to every wave: each thread waits for its own direct
// loads of chunk c (later chunks stay in flight), then a bare barrier
// publishes it -- a fenced barrier would also drain the chunks in flight.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void tree_attn_bf16_kernel(
    int T, int Hq, int max_slots, int nsplit_max, int split_keys, int nqb,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ prefix_len, const uint8_t* __restrict__ tree_mask, float scale_log2,
    float* __restrict__ part_o, float2* __restrict__ part_ml) {
  using Lay = AttnLayout<D>;
  constexpr int DT = D / 16, DS = D / 32;
  constexpr int NW = kAttnThreads / kWave;           // waves: two groups of four
  static_assert(Lay::PER * kAttnThreads * 16 == 2 * Lay::TILE, "chunk must split into whole loads");
  static_assert(kStages >= 4 && kStages % 2 == 0, "chunks are consumed in pairs");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages][2][Lay::TILE];   // [stage][K, V]
  __shared__ uint64_t mbits[NW][16][kMaxNodes / 64];

  const int split = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z / nqb, qb = blockIdx.z - b * nqb;
  int L = prefix_len[b];
  if (L > max_slots - T) L = max_slots - T;
  if (L < 0) L = 0;
  const int total = L + T;
  const int ns = num_splits(total, split_keys);
  if (split >= ns) return;

  // whole chunks per split, spread evenly; only a head's last chunk is ragged
  const int nc_all = (total + kChunk - 1) / kChunk;
  const int c_base = nc_all / ns, c_rem = nc_all % ns;
  const int k_lo = kChunk * (split * c_base + min(split, c_rem));
  const int k_hi = min(total, k_lo + kChunk * (c_base + (split < c_rem ? 1 : 0)));
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2, wq = wave & 3;            // chunk group, query wave
  const int n = lane & 15, g = lane >> 4;
  const int qi = qb * kQBlock + wq * 16 + n;           // this lane's query
  const bool q_ok = qi < T;
  const size_t bh = static_cast<size_t>(b) * Hq + h;
  const uint16_t* kbase = kc + bh * max_slots * D;
  const uint16_t* vbase = vc + bh * max_slots * D;
  constexpr int PER = Lay::PER;
  const int nch = (k_hi - k_lo + kChunk - 1) / kChunk;

  // Q of the block's 64 queries goes through the same direct-load path into
  // the last ring stage (rows 0-31 in its K half, 32-63 in its V half,
  // swizzled like K), ahead of the first chunks; that stage is first
  // refilled after the barrier that ends the Q reads.  Rows past T repeat
  // row T - 1.
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int x = i * kAttnThreads + tid;                // piece of the 64 x D tile
    const int row = x / Lay::PIECES, slot = x % Lay::PIECES;
    const int qq = min(qb * kQBlock + row, T - 1);
    const uint16_t* src = q + ((static_cast<size_t>(b) * T + qq) * Hq + h) * D + Lay::k_slot(row, slot) * 8;
    const int half = x * 16 < Lay::TILE ? 0 : 1;
    lds_dma16(src, LDSB(ring[kStages - 1][half]) + ((x & ~63) * 16 - half * Lay::TILE));
  }
  const int n0 = min(kStages - 2, nch);   // chunks issued ahead of the loop
  for (int c = 0; c < n0; ++c)
    attn_issue<D>(kbase, vbase, k_lo + c * kChunk, k_hi, tid, ring[c][0], ring[c][1]);

  // Ancestor words of the wave's queries (only in a split that reaches the
  // tree): word ww of query row r is a ballot over one coalesced 64-byte
  // load of the mask row; every wave builds the rows of its own 16 queries.
  // The bytes of word 0 are loaded here, but the ballots wait until the
  // wave's first chunk that reaches the tree: waiting for a load waits for
  // every load issued before it, and by then only the split's last chunks
  // are still in flight.
  const bool has_tree = k_hi > L;
  uint8_t mbv[16];
  if (has_tree) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = qb * kQBlock + wq * 16 + r;
      mbv[r] = tree_mask[static_cast<size_t>(min(qq, T - 1)) * T + min(lane, T - 1)];
    }
  }
  bool mask_ready = !has_tree;
  auto build_mask = [&]() {
    const int nw = (T + 63) >> 6;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = qb * kQBlock + wq * 16 + r;
      const uint64_t word = ballot(qq < T && lane < T && mbv[r] != 0);
      if (lane == 0) mbits[wave][r][0] = word;
    }
#pragma unroll 1
    for (int ww = 1; ww < nw; ++ww) {   // trees of more than 64 nodes
      const int j = ww * 64 + lane;
      uint8_t mw[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qq = qb * kQBlock + wq * 16 + r;
        mw[r] = tree_mask[static_cast<size_t>(min(qq, T - 1)) * T + min(j, T - 1)];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qq = qb * kQBlock + wq * 16 + r;
        const uint64_t word = ballot(qq < T && j < T && mw[r] != 0);
        if (lane == 0) mbits[wave][r][ww] = word;
      }
    }
  };
  const uint64_t* mrow = mbits[wave][n];

  // Q from LDS into registers once its loads (the oldest in flight) are in
  wait_chunks<PER, kStages - 2>(n0);
  ring_barrier();
  u32x4 qv[DS];   // Q[qi][s*32 + 8g .. +8]: the B operand of S^T
  {
    const int row = wq * 16 + n;
    const MEDUSA_LDS uint8_t* qt = LDSB(ring[kStages - 1][row < 32 ? 0 : 1]) + (row & 31) * Lay::ROWB;
#pragma unroll
    for (int s = 0; s < DS; ++s) qv[s] = *(const MEDUSA_LDS u32x4*)(qt + Lay::k_slot(row, s * 4 + g) * 16);
  }

  float m_run = -__builtin_huge_valf();
  float l_part = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Chunks go in pairs: group 0 takes chunk c, group 1 chunk c + 1, each
  // with its own online-softmax state.  Chunk c sits in stage c % kStages;
  // after the barrier of pair c the stages of pair c - 2 are free and take
  // chunks c + kStages - 2 and c + kStages - 1.
  for (int c = 0; c < nch; c += 2) {
    const int need_hi = min(c + 1, nch - 1);
    const int issued_hi = min(c + kStages - 3, nch - 1);
    wait_chunks<PER, kStages - 4>(issued_hi - need_hi);
    ring_barrier();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cn = c + kStages - 2 + u;
      if (cn < nch) {
        const int sn = cn % kStages;
        attn_issue<D>(kbase, vbase, k_lo + cn * kChunk, k_hi, tid, ring[sn][0], ring[sn][1]);
      }
    }
    const int cc = c + grp;
    if (cc < nch) {
      if (!mask_ready && k_lo + (cc + 1) * kChunk > L) {   // uniform: the wave's first chunk reaching the tree
        build_mask();
        mask_ready = true;
      }
      const int st = cc % kStages;
      attn_chunk<D>(qv, o, m_run, l_part, k_lo + cc * kChunk, k_hi, L, lane, scale_log2, mrow, ring[st][0],
                    ring[st][1]);
    }
  }

  // Group 1 hands its state to group 0 through LDS (the ring is free: every
  // direct load has landed and every chunk has been read), then group 0
  // merges the two -- each taken against its own reference -- and writes
  // the split's partial.
  constexpr int NF = 4 * DT + 2;                       // floats per lane: O, m, l
  float* xfer = reinterpret_cast<float*>(&ring[0][0][0]);
  ring_barrier();
  if (grp == 1) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) xfer[(wq * NF + 4 * t + i) * kWave + lane] = o[t][i];
    xfer[(wq * NF + 4 * DT) * kWave + lane] = m_run;
    xfer[(wq * NF + 4 * DT + 1) * kWave + lane] = l_part;
  }
  ring_barrier();
  if (grp == 0) {
    const float NEG = -__builtin_huge_valf();
    const float m1 = xfer[(wq * NF + 4 * DT) * kWave + lane];
    const float l1 = xfer[(wq * NF + 4 * DT + 1) * kWave + lane];
    const float M = fmaxf(m_run, m1);
    const float a0 = m_run == NEG ? 0.f : exp2f(m_run - M);
    const float a1 = m1 == NEG ? 0.f : exp2f(m1 - M);
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[t][i] = o[t][i] * a0 + xfer[(wq * NF + 4 * t + i) * kWave + lane] * a1;
    l_part = l_part * a0 + l1 * a1;
    m_run = M;

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
}

// Merge the splits of each (sequence, head, query) by log-sum-exp.  D/4
// threads per query, four output columns each (16-byte partial loads); a
// 256-thread workgroup takes 1024/D consecutive queries of one (sequence,
// head), so its loads of one split are one contiguous run.  Splits are taken
// eight at a time with all their loads issued together, merged online
// against a running maximum.  The first eight are addressed within the
// workspace's nsplit_max splits, so their loads go out with the prefix
// length's in one round trip; splits at or past the sequence's own count
// (never written by this call) are dropped by selects, never multiplied.
template <typename OutT, int D>
__global__ __launch_bounds__(256) void tree_attn_combine_kernel(int B, int T, int Hq, int max_slots, int nsplit_max,
                                                              int split_keys, const int32_t* __restrict__ prefix_len,
                                                              const float* __restrict__ part_o,
                                                              const float2* __restrict__ part_ml,
                                                              OutT* __restrict__ out) {
  constexpr int TPQ = D / 4, QPW = 256 / TPQ, U = 8;
  const int t = threadIdx.x % TPQ;
  // B * Hq * T * D / 4 stays below 2^31 (B <= 16, Hq <= 1024, T <= 256)
  const unsigned Q = blockIdx.x * QPW + threadIdx.x / TPQ;
  if (Q >= static_cast<unsigned>(B * Hq * T)) return;
  const int qi = static_cast<int>(Q % static_cast<unsigned>(T));
  const int h = static_cast<int>((Q / static_cast<unsigned>(T)) % static_cast<unsigned>(Hq));
  const int b = static_cast<int>(Q / static_cast<unsigned>(T * Hq));
  const size_t bh = static_cast<size_t>(b) * Hq + h;
  const float NEG = -__builtin_huge_valf();
  float M = NEG, den = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float2 ml[U];
  float4 ov[U];
  auto load = [&](int s0, int smax) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t row = (bh * nsplit_max + min(s0 + u, smax - 1)) * T + qi;
      ml[u] = part_ml[row];
      ov[u] = *reinterpret_cast<const float4*>(part_o + row * D + 4 * t);
    }
  };
  load(0, nsplit_max);
  int L = prefix_len[b];
  if (L > max_slots - T) L = max_slots - T;
  if (L < 0) L = 0;
  const int ns = num_splits(L + T, split_keys);
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
        const float w = exp2f(ml[u].x - ref);
        acc[0] += w * ov[u].x;
        acc[1] += w * ov[u].y;
        acc[2] += w * ov[u].z;
        acc[3] += w * ov[u].w;
        den += w * ml[u].y;
      }
    }
    M = Mn;
  }
  const size_t o = ((static_cast<size_t>(b) * T + qi) * Hq + h) * D + 4 * t;
  if constexpr (sizeof(OutT) == 2) {
    uint2 w;
    w.x = f32_to_bf16_bits(acc[0] / den) | (f32_to_bf16_bits(acc[1] / den) << 16);
    w.y = f32_to_bf16_bits(acc[2] / den) | (f32_to_bf16_bits(acc[3] / den) << 16);
    *reinterpret_cast<uint2*>(out + o) = w;
  } else {
    *reinterpret_cast<float4*>(out + o) = float4{acc[0] / den, acc[1] / den, acc[2] / den, acc[3] / den};
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
  // sized for the shortest splits (every launch uses at most this many)
  const size_t nsm = static_cast<size_t>(num_splits(max_slots, kSplit));
  return medusa_host::round_up(static_cast<size_t>(B) * Hq * nsm * T * d * 4, 256);
}
size_t attn_part_ml_bytes(int B, int T, int Hq, int max_slots) {
  const size_t nsm = static_cast<size_t>(num_splits(max_slots, kSplit));
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
  const int nqb = (T + kQBlock - 1) / kQBlock;
  const int sk = attn_split_keys(B, Hq, d, nqb, max_slots);
  const int nsm = num_splits(max_slots, sk);
  float* part_o = static_cast<float*>(ws);
  float2* part_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + attn_part_o_bytes(B, T, Hq, d, max_slots));
  const float sl2 = scale * kLog2e;
  dim3 grid(nsm, Hq, B * nqb);
  if (d == 128)
    hipLaunchKernelGGL(tree_attn_bf16_kernel<128>, grid, dim3(kAttnThreads), 0, st, T, Hq, max_slots, nsm, sk, nqb,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                       static_cast<const uint16_t*>(v_cache), prefix_len, tree_mask, sl2, part_o, part_ml);
  else
    hipLaunchKernelGGL(tree_attn_bf16_kernel<64>, grid, dim3(kAttnThreads), 0, st, T, Hq, max_slots, nsm, sk, nqb,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                       static_cast<const uint16_t*>(v_cache), prefix_len, tree_mask, sl2, part_o, part_ml);
  rc = medusa_host::hip_check("medusa_tree_attention launch");
  if (rc != MEDUSA_OK) return rc;
  const unsigned cgrid = static_cast<unsigned>((B * Hq * T * (d / 4) + 255) / 256);
  if (d == 128)
    hipLaunchKernelGGL((tree_attn_combine_kernel<uint16_t, 128>), dim3(cgrid), dim3(256), 0, st, B, T, Hq, max_slots,
                       nsm, sk, prefix_len, part_o, part_ml, static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL((tree_attn_combine_kernel<uint16_t, 64>), dim3(cgrid), dim3(256), 0, st, B, T, Hq, max_slots,
                       nsm, sk, prefix_len, part_o, part_ml, static_cast<uint16_t*>(out));
  return medusa_host::hip_check("medusa_tree_attention combine launch");
}
