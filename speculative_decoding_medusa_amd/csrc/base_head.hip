// The base model's lm_head over the tree nodes on gfx950:
// logits[m][v] = sum_k hidden[m][k] * W[v][k], float32 accumulation, no bias.
//
// A skinny GEMM: M = B*T rows of final hidden states (tens of rows), V weight
// rows of H elements (32000 x 4096 bf16 = 262 MB), so every weight is
// streamed from HBM exactly once and the whole grid is resident at once.
// Workgroup = (a block of 128 vocab rows, an M tile of 64 hidden rows): four
// waves, each owning two 16-row weight tiles, walk K in chunks of 256.
//
//  * The M tile's chunk of hidden states (64 x 256 bf16, 32 KB) is staged in
//    LDS, double-buffered and shared by the four waves; its 16-byte pieces
//    are XOR-swizzled by row so the MFMA operand reads are conflict-free.
//  * Weight tiles go straight from HBM into registers, double-buffered
//    across chunks, each 16-byte piece refilled as soon as its MFMAs have
//    read it.  From the packed layout (medusa_base_lm_head_pack: 32-element
//    k steps, pairs of 16-row tiles, the pair's two tiles, lanes) one wave
//    instruction reads 1 KB contiguously and a wave's two tiles are one
//    2 KB run per k step; from the row-major layout it reads 64 bytes of
//    each of 16 rows.
//  * v_mfma_f32_16x16x32_bf16 with A = 16 hidden rows, B = 16 weight rows:
//    lane (g, n) of a tile holds logits[4g + i][n] in component i.
//  * Chunks are published with an LDS-only wait and a bare barrier, so the
//    weight loads in flight are never drained at a chunk boundary.
#include "common.hpp"

namespace medusa {

constexpr int kBhThreads = 256;
constexpr int kBhWaves = 4;
constexpr int kBhTiles = 2;                           // 16-row weight tiles per wave
constexpr int kBhVBlock = kBhWaves * kBhTiles * 16;   // vocab rows per workgroup
constexpr int kBhMTile = 64;                          // hidden rows per workgroup
constexpr int kBhKC = 256;                            // K elements per chunk
constexpr int kBhSteps = kBhKC / 32;                  // MFMA k-steps per chunk
constexpr int kBhPieces = kBhKC / 8;                  // 16-byte pieces of a row chunk

// Packed weights: tile vt (rows 16 vt ..), k step ks (elements 32 ks ..),
// lane l = 16 g + n -> the 16 bytes W[16 vt + n][32 ks + 8 g .. + 8], zero
// past V or H.  Order: k step, tile pair vt / 2, tile vt % 2, lane -- 1 KB
// per (tile, step), so the two tiles a wave owns form one 2 KB run per k
// step, and at any moment every workgroup reads inside one k range of the
// whole matrix: the grid sweeps the weights front to back instead of each
// workgroup streaming its own megabyte (52.7-52.8 us against 53.3-53.7 us
// per 64 x 4096 x 32000 call, and the fused acceptance 60.9 against 63.0).
// The tile count is padded to an even number.
__host__ __device__ inline int bh_ksteps(int H) { return (H + 31) / 32; }
__host__ __device__ inline int bh_vtiles(int V) { return ((V + 31) / 32) * 2; }
__host__ __device__ inline size_t bh_block(int vt, int ks, int npair) {
  return (static_cast<size_t>(ks) * npair + vt / 2) * 2 + (vt & 1);
}
// elements between one k step of a tile and the next
__host__ __device__ inline size_t bh_kstride(int npair) { return static_cast<size_t>(npair) * 1024; }

// 16-byte slot of piece p of hidden row r in a chunk buffer.
__device__ __forceinline__ int bh_slot(int r, int p) { return r * kBhPieces + (p ^ (r & 7)); }

// Every LDS operation of this thread complete (vector memory left in flight).
__device__ __forceinline__ void bh_wait_lds() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ void bh_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ u32x4 bh_ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 bh_ld16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Epilogues of the GEMM:
//   kEpiLogits  write the float32 logits;
//   kEpiStats   per-row statistics over the workgroup's 128 vocabulary
//               entries and the logits of the tree candidates whose tokens
//               fall among them (the fused acceptance test);
//   kEpiTopk    Medusa heads at batch > 2: grid.y = head; the 2B rows are
//               the hi and lo bf16 planes of the head's float32 inputs, so
//               logit[b][v] = acc[b][v] + acc[B + b][v]; each workgroup
//               publishes every row's top-k of its 128 entries as one
//               sorted list (value desc, id asc) for the heads' merge;
//   kEpiPart    the heads' ResBlock products W1[j] . h on packed W1:
//               grid.y = head, grid.z = a slice of K (split so the grid
//               fills the chip); every row's float32 partial sums go to
//               part[z][head][m][v] for heads_res_finish_kernel.
constexpr int kEpiLogits = 0, kEpiStats = 1, kEpiTopk = 2, kEpiPart = 3;

struct BhEpiArgs {
  // kEpiStats
  int T;                        // nodes per sequence (rows m = b * T + node)
  float temperature;            // > 0: softmax statistics of logits / temperature
  const int32_t* candidates;    // [B][T] token of every node
  RowStat* parts;               // [M][gridDim.x]
  float* child_z;               // [B][T][T]: child_z[b][n][c] = logit of c's token at node n
  // kEpiTopk
  int B, K, k;
  float* cand_v;                // [K][B][gridDim.x][k]
  int32_t* cand_i;
  float* logits;                // optional [B][K][V]
  // kEpiPart
  float* part;                  // [gridDim.z][K][M][V]
};

// MT: 16-row M blocks per workgroup (the statistics epilogue takes 4; the
// heads take 1 or 2, enough for their 2B plane rows).
template <bool PACKED, int EPI, int MT>
__global__ __launch_bounds__(kBhThreads) void base_lm_head_kernel(int M, int H, int V,
                                                                  const uint16_t* __restrict__ hidden_all,
                                                                  const uint16_t* __restrict__ w_all,
                                                                  float* __restrict__ logits, BhEpiArgs sa_args) {
  constexpr int MTILE = 16 * MT;
  constexpr int STAGE = MTILE * kBhPieces / kBhThreads;   // pieces staged per thread
  static_assert(MT == 1 || MT == 2 || MT == 4, "M blocks");
  static_assert(EPI != kEpiStats || MT == 4, "the statistics epilogue assumes 64-row tiles");
  __shared__ __attribute__((aligned(16))) u32x4 sa[2][MTILE * kBhPieces];
  // kEpiTopk / kEpiPart: one head per grid row; its weights and (kEpiTopk)
  // its planes (kEpiPart: every head reads the same hidden rows)
  constexpr bool PER_HEAD = EPI == kEpiTopk || EPI == kEpiPart;
  const int head = PER_HEAD ? static_cast<int>(blockIdx.y) : 0;
  const uint16_t* __restrict__ hidden = hidden_all + (EPI == kEpiTopk ? static_cast<size_t>(head) * M * H : 0);
  const uint16_t* __restrict__ w =
      w_all + static_cast<size_t>(head) *
                  (PACKED ? static_cast<size_t>(bh_vtiles(V)) * bh_ksteps(H) * 512 : static_cast<size_t>(V) * H);
  const int m0 = PER_HEAD ? 0 : blockIdx.y * MTILE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  // this workgroup's chunks [c_begin, c_end) (grid.z > 1: a slice of K)
  const int nch = (H + kBhKC - 1) / kBhKC;
  const int c_per = (nch + static_cast<int>(gridDim.z) - 1) / static_cast<int>(gridDim.z);
  const int c_begin = static_cast<int>(blockIdx.z) * c_per, c_end = min(nch, c_begin + c_per);
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // this lane's weight row in each tile (rows past V reload row V-1 or the
  // last packed tile, and are not written)
  const int ks_n = bh_ksteps(H), vt_n = bh_vtiles(V);
  const size_t kstride = bh_kstride(vt_n / 2);
  int vrow[kBhTiles];
  const uint16_t* wr[kBhTiles];
#pragma unroll
  for (int t = 0; t < kBhTiles; ++t) {
    const int vt = blockIdx.x * (kBhVBlock / 16) + wave * kBhTiles + t;
    vrow[t] = vt * 16 + n;
    if (PACKED)
      wr[t] = w + (bh_block(min(vt, vt_n - 1), 0, vt_n / 2) * 64 + lane) * 8;
    else
      wr[t] = w + static_cast<size_t>(min(vrow[t], V - 1)) * H;
  }
  // the 16 bytes of weight piece (chunk c, step s) of tile t for this lane
  auto wpiece = [&](int t, int c, int s) -> u32x4 {
    if (PACKED) return bh_ld16_stream(wr[t] + static_cast<size_t>(min(c * kBhSteps + s, ks_n - 1)) * kstride);
    return bh_ld16_stream(wr[t] + static_cast<uint32_t>(min(c * kBhKC + 32 * s + 8 * g, H - 8)));
  };

  // staging of the hidden chunk: thread tid moves pieces tid + 256 q
  auto load_a = [&](int c, u32x4 (&ra)[STAGE]) {
#pragma unroll
    for (int q = 0; q < STAGE; ++q) {
      const int x = q * kBhThreads + tid;
      const int r = x / kBhPieces, p = x % kBhPieces;
      ra[q] = bh_ld16(hidden + static_cast<size_t>(min(m0 + r, M - 1)) * H + min(c * kBhKC + 8 * p, H - 8));
    }
  };
  auto store_a = [&](int buf, int c, const u32x4 (&ra)[STAGE]) {
#pragma unroll
    for (int q = 0; q < STAGE; ++q) {
      const int x = q * kBhThreads + tid;
      const int r = x / kBhPieces, p = x % kBhPieces;
      const bool ok = m0 + r < M && c * kBhKC + 8 * p < H;
      sa[buf][bh_slot(r, p)] = ok ? ra[q] : zero;
    }
  };
  // weight pieces of chunk c: step s, lane group g -> k = 256 c + 32 s + 8 g,
  // issued in step order so step s waits only for its own two pieces
  auto load_w = [&](int c, u32x4 (&bw)[kBhTiles][kBhSteps]) {
#pragma unroll
    for (int s = 0; s < kBhSteps; ++s)
#pragma unroll
      for (int t = 0; t < kBhTiles; ++t) bw[t][s] = wpiece(t, c, s);
  };

  // STATS: the tokens of the (sequence, node) pairs this M tile covers,
  // requested now so the epilogue does not wait on them.  A 64-row tile
  // spans at most ceil(63 / T) + 1 sequences: at most 2 * kMaxNodes pairs,
  // two per thread (clamped addresses, masked at use).
  constexpr bool STATS = EPI == kEpiStats;
  const int Tn = STATS ? sa_args.T : 1;
  const int b_lo = m0 / Tn;
  const int npair = STATS ? ((min(m0 + kBhMTile, M) - 1) / Tn - b_lo + 1) * Tn : 0;
  int ctok[2] = {-1, -1};
  static_assert(2 * kBhThreads >= 2 * kMaxNodes, "two candidate tokens per thread cover a tile's pairs");
  if constexpr (STATS) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      ctok[u] = sa_args.candidates[static_cast<size_t>(b_lo) * Tn + min(u * kBhThreads + tid, npair - 1)];
  }

  f32x4 acc[kBhTiles][MT];
#pragma unroll
  for (int t = 0; t < kBhTiles; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // chunk c from LDS buffer buf and weight buffer bw; each piece of bw is
  // refilled with chunk cn right after its MFMAs (cn < 0: no refill)
  auto compute = [&](int buf, int c, u32x4 (&bw)[kBhTiles][kBhSteps], int cn) {
#pragma unroll
    for (int s = 0; s < kBhSteps; ++s) {
      u32x4 a[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[mt] = sa[buf][bh_slot(mt * 16 + n, 4 * s + g)];
      const bool kin = c * kBhKC + 32 * s + 8 * g < H;   // K tail: the hidden side is zero too
#pragma unroll
      for (int t = 0; t < kBhTiles; ++t) {
        const u32x4 b = kin ? bw[t][s] : zero;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[mt]), as_bf16x8(b), acc[t][mt], 0, 0, 0);
      }
      if (cn >= 0) {
#pragma unroll
        for (int t = 0; t < kBhTiles; ++t) bw[t][s] = wpiece(t, cn, s);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Issue order keeps every wait on the oldest loads: hidden chunk 0, weight
  // chunks 0 and 1, hidden chunk 1; then per chunk: compute (refilling the
  // weights two chunks ahead piece by piece), stage the next hidden chunk,
  // prefetch the one after.  An LDS buffer is rewritten only after the
  // barrier that follows its last reads.
  u32x4 ra[STAGE];
  u32x4 wa[kBhTiles][kBhSteps], wb[kBhTiles][kBhSteps];
  const int lastc = c_end - 1;
  if (c_begin < c_end) {   // uniform per workgroup (the host leaves no slice empty)
  load_a(c_begin, ra);
  load_w(c_begin, wa);
  load_w(min(c_begin + 1, lastc), wb);
  store_a(0, c_begin, ra);
  load_a(min(c_begin + 1, lastc), ra);
  int c = c_begin;
  for (; c + 1 < c_end; c += 2) {
    bh_wait_lds();
    bh_barrier();
    compute(0, c, wa, min(c + 2, lastc));
    store_a(1, c + 1, ra);
    load_a(min(c + 2, lastc), ra);
    bh_wait_lds();
    bh_barrier();
    compute(1, c + 1, wb, min(c + 3, lastc));
    store_a(0, c + 2, ra);
    load_a(min(c + 3, lastc), ra);
  }
  if (c < c_end) {
    bh_wait_lds();
    bh_barrier();
    compute(0, c, wa, -1);
  }
  }

  if constexpr (EPI == kEpiPart) {
    float* out = sa_args.part + (static_cast<size_t>(blockIdx.z) * sa_args.K + head) * M * V;
#pragma unroll
    for (int t = 0; t < kBhTiles; ++t) {
      if (vrow[t] >= V) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mt * 16 + 4 * g + i;
          if (m < M) out[static_cast<size_t>(m) * V + vrow[t]] = acc[t][mt][i];
        }
    }
    return;
  }

  if constexpr (EPI == kEpiLogits) {
    // logits[m][v]: lane (g, n) of tile (t, mt) holds rows mt*16 + 4g + i
#pragma unroll
    for (int t = 0; t < kBhTiles; ++t) {
      if (vrow[t] >= V) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + mt * 16 + 4 * g + i;
          if (m < M) logits[static_cast<size_t>(m) * V + vrow[t]] = acc[t][mt][i];
        }
    }
    return;
  }

  // ---- fused epilogues: the workgroup's 64 x 128 logits go to LDS (over the
  // hidden-state buffers, once every wave is past its last chunk)
  bh_wait_lds();
  bh_barrier();
  constexpr int LD = kBhVBlock + 1;   // padded row
  float* lg = reinterpret_cast<float*>(&sa[0][0]);
  static_assert(MTILE * LD * 4 <= 2 * MTILE * kBhPieces * 16, "logit tile fits the LDS buffers");
#pragma unroll
  for (int t = 0; t < kBhTiles; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) lg[(mt * 16 + 4 * g + i) * LD + (wave * kBhTiles + t) * 16 + n] = acc[t][mt][i];

  if constexpr (EPI == kEpiTopk) {
    // one wave per row b: lane l holds entries l and l + 64 of the block;
    // k rounds of a wave arg-best (value desc, id asc) build the sorted list
    // in lanes 0 .. k-1.  Entries past V and NaN logits never win; slots no
    // entry fills hold (-inf, -1).
    bh_wait_lds();
    bh_barrier();
    const int Bn = sa_args.B, kk = sa_args.k;
    const int v0 = blockIdx.x * kBhVBlock;
    const float NEG = -__builtin_huge_valf();
    const int NONE = 0x7fffffff;
    for (int b = wave; b < Bn; b += kBhWaves) {
      float z0 = NEG, z1 = NEG;
      int i0 = NONE, i1 = NONE;
      if (v0 + lane < V) {
        z0 = lg[b * LD + lane] + lg[(Bn + b) * LD + lane];
        i0 = v0 + lane;
      }
      if (v0 + lane + 64 < V) {
        z1 = lg[b * LD + lane + 64] + lg[(Bn + b) * LD + lane + 64];
        i1 = v0 + lane + 64;
      }
      if (sa_args.logits != nullptr) {
        float* lr = sa_args.logits + (static_cast<size_t>(b) * sa_args.K + head) * V;
        if (i0 != NONE) lr[i0] = z0;
        if (i1 != NONE) lr[i1] = z1;
      }
      float myv = NEG;
      int myi = -1;
      for (int r = 0; r < kk; ++r) {
        float bv = z0;
        int bi = i0;
        if (beats(z1, i1, bv, bi)) {
          bv = z1;
          bi = i1;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float ov = __shfl_xor(bv, o);
          const int oi = __shfl_xor(bi, o);
          if (beats(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
          }
        }
        if (lane == r && bi != NONE) {
          myv = bv;
          myi = bi;
        }
        if (bi != NONE && i0 == bi) {
          z0 = NEG;
          i0 = NONE;
        }
        if (bi != NONE && i1 == bi) {
          z1 = NEG;
          i1 = NONE;
        }
      }
      if (lane < kk) {
        const size_t off = ((static_cast<size_t>(head) * Bn + b) * gridDim.x + blockIdx.x) * kk + lane;
        sa_args.cand_v[off] = myv;
        sa_args.cand_i[off] = myi;
      }
    }
    return;
  }
  // tree candidates whose token lies in this block: (sequence, node, column);
  // a 64-row tile spans at most 63 / T + 2 sequences, so at most 2 * kMaxNodes
  // (sequence, node) pairs are checked
  __shared__ int s_hits[2 * kMaxNodes];
  __shared__ int s_nhit;
  const int v0 = blockIdx.x * kBhVBlock;
  if (tid == 0) s_nhit = 0;
  bh_wait_lds();
  bh_barrier();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int x = u * kBhThreads + tid, tok = ctok[u];
    if (x < npair && tok >= v0 && tok < v0 + kBhVBlock && tok < V) {
      const int slot = atomicAdd(&s_nhit, 1);
      if (slot < 2 * kMaxNodes) s_hits[slot] = ((x / Tn) << 24) | ((x % Tn) << 8) | (tok - v0);
    }
  }
  bh_wait_lds();
  bh_barrier();

  // four threads per row, 32 columns each: max / argmax, then (temperature
  // > 0) S and A against the quarter's own maximum; quarters merged by
  // shuffles
  const int r = tid >> 2, q = tid & 3;
  const float NEG = -__builtin_huge_valf();
  RowStat st = {NEG, 0x7fffffff, NEG, 0.f, 0.f};
  const float* lr = lg + r * LD + q * 32;
#pragma unroll 8
  for (int j = 0; j < 32; ++j) {
    const int v = v0 + q * 32 + j;
    const float z = lr[j];
    if (v < V && beats(z, v, st.mx, st.arg)) {
      st.mx = z;
      st.arg = v;
    }
  }
  const float temp = sa_args.temperature;
  const bool typical = temp > 0.f;
  if (typical && st.mx != NEG && st.mx == st.mx) {
    const float mq = st.mx / temp;   // positive temperature: max z = max logit / t
    float S = 0.f, A = 0.f;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      if (v0 + q * 32 + j < V) {
        const float dz = lr[j] / temp - mq;
        const float p = expf(dz);
        S += p;
        A += dz * p;
      }
    }
    st.m = mq;
    st.S = S;
    st.A = A;
  }
#pragma unroll
  for (int o = 1; o < 4; o <<= 1) {
    RowStat y;
    y.mx = __shfl_xor(st.mx, o);
    y.arg = __shfl_xor(st.arg, o);
    y.m = __shfl_xor(st.m, o);
    y.S = __shfl_xor(st.S, o);
    y.A = __shfl_xor(st.A, o);
    rowstat_merge(st, y, typical);
  }
  if (q == 0 && m0 + r < M) sa_args.parts[static_cast<size_t>(m0 + r) * gridDim.x + blockIdx.x] = st;

  // the candidates' logits at every node of their sequence in this tile
  const int nhit = min(s_nhit, 2 * kMaxNodes);
  for (int e = 0; e < nhit; ++e) {
    const int code = s_hits[e];
    const int b = b_lo + (code >> 24), c = (code >> 8) & 0xffff, col = code & 0xff;
    if (tid < kBhMTile) {
      const int m = m0 + tid;
      if (m < M && m / Tn == b)
        sa_args.child_z[(static_cast<size_t>(b) * Tn + m % Tn) * Tn + c] = lg[tid * LD + col];
    }
  }
}

// Medusa heads at batch > 2: r [B][K][H] float32 -> per head the hi and lo
// bf16 planes [K][2B][H] (hi = r rounded to nearest even, lo = the rest
// rounded; the GEMM sums both rows' products).  Eight elements per thread.
__global__ __launch_bounds__(256) void heads_planes_kernel(int B, int K, int H, const float* __restrict__ r,
                                                           uint16_t* __restrict__ planes) {
  const long long x = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int per = H / 8;
  if (x >= static_cast<long long>(B) * K * per) return;
  const int c = static_cast<int>(x % per) * 8;
  const int j = static_cast<int>((x / per) % K), b = static_cast<int>(x / per / K);
  const float* src = r + (static_cast<size_t>(b) * K + j) * H + c;
  u32x4 hi, lo;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = src[2 * p], e = src[2 * p + 1];
    const uint32_t h2 = pack_bf16x2(a, e);
    hi[p] = h2;
    lo[p] = pack_bf16x2(a - __uint_as_float(h2 << 16), e - __uint_as_float(h2 & 0xffff0000u));
  }
  uint16_t* base = planes + static_cast<size_t>(j) * 2 * B * H;
  *reinterpret_cast<u32x4*>(base + static_cast<size_t>(b) * H + c) = hi;
  *reinterpret_cast<u32x4*>(base + static_cast<size_t>(B + b) * H + c) = lo;
}

// The ResBlock from the split products: u = sum_z part[z][j][b] + b1[j],
// r[b][j] = h[b] + SiLU(u), written as float32 (optional) and as the hi/lo
// bf16 planes [K][2B][H] of the heads' lm_head.  Eight elements per thread.
__global__ __launch_bounds__(256) void heads_res_finish_kernel(int B, int K, int H, int S,
                                                               const float* __restrict__ part,
                                                               const uint16_t* __restrict__ hidden,
                                                               const uint16_t* __restrict__ b1, float* __restrict__ r,
                                                               uint16_t* __restrict__ planes) {
  const long long x = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int per = H / 8;
  if (x >= static_cast<long long>(K) * B * per) return;
  const int c = static_cast<int>(x % per) * 8;
  const int b = static_cast<int>((x / per) % B), j = static_cast<int>(x / per / B);
  const u32x4 bw = *reinterpret_cast<const u32x4*>(b1 + static_cast<size_t>(j) * H + c);
  const u32x4 hw = *reinterpret_cast<const u32x4*>(hidden + static_cast<size_t>(b) * H + c);
  float u[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    u[2 * p] = 0.f;
    u[2 * p + 1] = 0.f;
  }
  for (int z = 0; z < S; ++z) {
    const f32x4* src = reinterpret_cast<const f32x4*>(part + ((static_cast<size_t>(z) * K + j) * B + b) * H + c);
    const f32x4 lo4 = src[0], hi4 = src[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[e] += lo4[e];
      u[4 + e] += hi4[e];
    }
  }
  float v[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float u0 = u[2 * p] + __uint_as_float(bw[p] << 16);
    const float u1 = u[2 * p + 1] + __uint_as_float(bw[p] & 0xffff0000u);
    v[2 * p] = __uint_as_float(hw[p] << 16) + u0 / (1.0f + expf(-u0));
    v[2 * p + 1] = __uint_as_float(hw[p] & 0xffff0000u) + u1 / (1.0f + expf(-u1));
  }
  if (r != nullptr) {
    f32x4* dst = reinterpret_cast<f32x4*>(r + (static_cast<size_t>(b) * K + j) * H + c);
    dst[0] = f32x4{v[0], v[1], v[2], v[3]};
    dst[1] = f32x4{v[4], v[5], v[6], v[7]};
  }
  u32x4 hi, lo;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t h2 = pack_bf16x2(v[2 * p], v[2 * p + 1]);
    hi[p] = h2;
    lo[p] = pack_bf16x2(v[2 * p] - __uint_as_float(h2 << 16), v[2 * p + 1] - __uint_as_float(h2 & 0xffff0000u));
  }
  uint16_t* base = planes + static_cast<size_t>(j) * 2 * B * H;
  *reinterpret_cast<u32x4*>(base + static_cast<size_t>(b) * H + c) = hi;
  *reinterpret_cast<u32x4*>(base + static_cast<size_t>(B + b) * H + c) = lo;
}

// y[i] = sum over z of part[z][i], z in order (medusa_linear's split path).
__global__ __launch_bounds__(256) void linear_reduce_kernel(int S, long long n, const float* __restrict__ part,
                                                            float* __restrict__ y) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = part[i];
  for (int z = 1; z < S; ++z) acc += part[static_cast<size_t>(z) * n + i];
  y[i] = acc;
}

// Row-major weights [V][H] -> the packed layout, one 16-byte piece per
// thread (zeros past V or H).
__global__ __launch_bounds__(256) void base_lm_head_pack_kernel(int H, int V, const uint16_t* __restrict__ w,
                                                               uint16_t* __restrict__ wp, long long npieces) {
  const long long x = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (x >= npieces) return;
  const int l = static_cast<int>(x & 63);
  const long long blk = x >> 6;                 // (ks * npair + pair) * 2 + half
  const int half = static_cast<int>(blk & 1);
  const int npair = bh_vtiles(V) / 2;
  const int ks = static_cast<int>((blk >> 1) / npair);
  const int vt = static_cast<int>((blk >> 1) % npair) * 2 + half;
  const int row = vt * 16 + (l & 15), k = ks * 32 + 8 * (l >> 4);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < V && k < H) v = *reinterpret_cast<const u32x4*>(w + static_cast<size_t>(row) * H + k);
  *reinterpret_cast<u32x4*>(wp + x * 8) = v;
}

}  // namespace medusa

namespace medusa_host {
namespace {
// One launch of the GEMM with the smallest M tile that holds min(M, 64) rows
// (a 16- or 32-row tile stages less, skips the empty MFMA blocks and lets
// more workgroups share a compute unit).
template <bool PACKED, int EPI>
void bh_launch(int M, int H, int V, dim3 grid, const uint16_t* hidden, const uint16_t* w, float* logits,
               const medusa::BhEpiArgs& ea, hipStream_t st) {
  using namespace medusa;
  if constexpr (EPI != kEpiStats) {
    const int rows = EPI == kEpiTopk || EPI == kEpiPart ? M : min(M, kBhMTile);
    if (rows <= 16) {
      hipLaunchKernelGGL((base_lm_head_kernel<PACKED, EPI, 1>), grid, dim3(kBhThreads), 0, st, M, H, V, hidden, w,
                         logits, ea);
      return;
    }
    if (rows <= 32) {
      hipLaunchKernelGGL((base_lm_head_kernel<PACKED, EPI, 2>), grid, dim3(kBhThreads), 0, st, M, H, V, hidden, w,
                         logits, ea);
      return;
    }
  }
  hipLaunchKernelGGL((base_lm_head_kernel<PACKED, EPI, 4>), grid, dim3(kBhThreads), 0, st, M, H, V, hidden, w,
                     logits, ea);
}
int bh_mtile(int M) { return M <= 16 ? 16 : M <= 32 ? 32 : medusa::kBhMTile; }
}  // namespace

#ifndef MEDUSA_RES_WG_TARGET
#define MEDUSA_RES_WG_TARGET 1024   // about four workgroups per compute unit
#endif
int heads_res_splits(int H, int K) {
  const int nch = (H + medusa::kBhKC - 1) / medusa::kBhKC;
  const int wg = heads_gemm_lists(H) * K;
  int s = (MEDUSA_RES_WG_TARGET + wg - 1) / wg;
  if (s > kHeadsResMaxSplits) s = kHeadsResMaxSplits;
  if (s > nch) s = nch;
  const int per = (nch + s - 1) / s;
  return (nch + per - 1) / per;   // no empty slice
}

int heads_res_gemm(int B, int H, int K, const uint16_t* hidden, const void* w1_packed, const uint16_t* b1,
                   float* r_or_null, float* part, uint16_t* planes, hipStream_t st) {
  using namespace medusa;
  const int S = heads_res_splits(H, K);
  BhEpiArgs ea{};
  ea.B = B;
  ea.K = K;
  ea.part = part;
  bh_launch<true, kEpiPart>(B, H, H, dim3(heads_gemm_lists(H), K, S), hidden, static_cast<const uint16_t*>(w1_packed),
                            nullptr, ea, st);
  int rc = hip_check("medusa_heads_packed resblock launch");
  if (rc != MEDUSA_OK) return rc;
  const long long n = static_cast<long long>(B) * K * (H / 8);
  hipLaunchKernelGGL(heads_res_finish_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, B, K, H,
                     S, part, hidden, b1, r_or_null, planes);
  return hip_check("medusa_heads_packed resblock finish launch");
}

int heads_lm_gemm(int B, int H, int V, int K, int k, const float* r, const void* w_lm, int packed,
                  float* logits_or_null, uint16_t* planes, float* cand_v, int32_t* cand_i, hipStream_t st) {
  using namespace medusa;
  if (r != nullptr) {
    const long long n = static_cast<long long>(B) * K * (H / 8);
    hipLaunchKernelGGL(heads_planes_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, B, K, H,
                       r, planes);
    int rc = hip_check("medusa_lm_head_topk planes launch");
    if (rc != MEDUSA_OK) return rc;
  }
  BhEpiArgs ea{};
  ea.B = B;
  ea.K = K;
  ea.k = k;
  ea.cand_v = cand_v;
  ea.cand_i = cand_i;
  ea.logits = logits_or_null;
  // the 2B plane rows of a head fit one tile (B <= 16)
  const dim3 grid(heads_gemm_lists(V), K);
  if (packed)
    bh_launch<true, kEpiTopk>(2 * B, H, V, grid, planes, static_cast<const uint16_t*>(w_lm), nullptr, ea, st);
  else
    bh_launch<false, kEpiTopk>(2 * B, H, V, grid, planes, static_cast<const uint16_t*>(w_lm), nullptr, ea, st);
  return hip_check("medusa_lm_head_topk gemm launch");
}

}  // namespace medusa_host

namespace {
// medusa_linear: slices of the reduction when the output alone gives too few
// workgroups (one M tile of at most 64 rows, fewer than 128 vocabulary
// blocks): enough slices for about 256 workgroups, at most 16, none empty.
constexpr int kLinearMaxSplits = 16;
int linear_splits(int M, int H, int V) {
  using namespace medusa;
  const int blocks = (V + kBhVBlock - 1) / kBhVBlock;
  const int nch = (H + kBhKC - 1) / kBhKC;
  if (M > kBhMTile || blocks >= 128 || nch < 2) return 1;
  int s = (256 + blocks - 1) / blocks;
  if (s > kLinearMaxSplits) s = kLinearMaxSplits;
  if (s > nch) s = nch;
  const int per = (nch + s - 1) / s;
  return (nch + per - 1) / per;
}
size_t linear_ws(int M, int H, int V) {
  const int S = linear_splits(M, H, V);
  if (S <= 1) return 256;
  return medusa_host::round_up(static_cast<size_t>(S) * M * V * sizeof(float), 256);
}
}  // namespace

extern "C" size_t medusa_linear_workspace(int M, int H, int V) {
  using namespace medusa;
  if (M < 1 || M > kMaxBatch * kMaxNodes || H < 8 || H > (1 << 16) || H % 8 != 0 || V < 1 || V > (1 << 24))
    return 0;
  return linear_ws(M, H, V);
}

extern "C" int medusa_linear(int dtype, int M, int H, int V, const void* x, const void* w_packed, float* y, void* ws,
                             size_t ws_bytes, void* stream) {
  using namespace medusa;
  MEDUSA_REQUIRE(dtype == MEDUSA_BF16, MEDUSA_ERR_DTYPE, "%s: dtype %d (bf16 only)", __func__, dtype);
  MEDUSA_REQUIRE(M >= 1 && M <= kMaxBatch * kMaxNodes, MEDUSA_ERR_SHAPE, "%s: M=%d", __func__, M);
  MEDUSA_REQUIRE(H >= 8 && H <= (1 << 16) && H % 8 == 0, MEDUSA_ERR_SHAPE, "%s: H=%d", __func__, H);
  MEDUSA_REQUIRE(V >= 1 && V <= (1 << 24), MEDUSA_ERR_SHAPE, "%s: V=%d", __func__, V);
  MEDUSA_REQUIRE_PTR(x);
  MEDUSA_REQUIRE_PTR(w_packed);
  MEDUSA_REQUIRE_PTR(y);
  MEDUSA_REQUIRE_PTR(ws);
  MEDUSA_REQUIRE(ws_bytes >= linear_ws(M, H, V), MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__,
                 ws_bytes, linear_ws(M, H, V));
  const int S = linear_splits(M, H, V);
  if (S <= 1) return medusa_base_lm_head(dtype, M, H, V, x, w_packed, 1, y, stream);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(ws);
  BhEpiArgs ea{};
  ea.B = M;
  ea.K = 1;
  ea.part = part;
  medusa_host::bh_launch<true, kEpiPart>(M, H, V, dim3((V + kBhVBlock - 1) / kBhVBlock, 1, S),
                                         static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_packed),
                                         nullptr, ea, st);
  int rc = medusa_host::hip_check("medusa_linear launch");
  if (rc != MEDUSA_OK) return rc;
  const long long n = static_cast<long long>(M) * V;
  hipLaunchKernelGGL(linear_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, S, n, part,
                     y);
  return medusa_host::hip_check("medusa_linear reduce launch");
}

extern "C" size_t medusa_base_lm_head_packed_bytes(int H, int V) {
  using namespace medusa;
  if (H < 8 || H > (1 << 16) || H % 8 != 0 || V < 1 || V > (1 << 24)) return 0;
  return static_cast<size_t>(bh_vtiles(V)) * bh_ksteps(H) * 1024;
}

extern "C" int medusa_base_lm_head_pack(int dtype, int H, int V, const void* w_base, void* w_packed, void* stream) {
  using namespace medusa;
  MEDUSA_REQUIRE(dtype == MEDUSA_BF16, MEDUSA_ERR_DTYPE, "%s: dtype %d (bf16 only)", __func__, dtype);
  MEDUSA_REQUIRE(H >= 8 && H <= (1 << 16) && H % 8 == 0, MEDUSA_ERR_SHAPE, "%s: H=%d", __func__, H);
  MEDUSA_REQUIRE(V >= 1 && V <= (1 << 24), MEDUSA_ERR_SHAPE, "%s: V=%d", __func__, V);
  MEDUSA_REQUIRE_PTR(w_base);
  MEDUSA_REQUIRE_PTR(w_packed);
  MEDUSA_REQUIRE(w_packed != w_base, MEDUSA_ERR_ALIAS, "%s: w_packed must not alias w_base", __func__);
  const long long npieces = static_cast<long long>(bh_vtiles(V)) * bh_ksteps(H) * 64;
  hipLaunchKernelGGL(base_lm_head_pack_kernel, dim3(static_cast<unsigned>((npieces + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), H, V, static_cast<const uint16_t*>(w_base),
                     static_cast<uint16_t*>(w_packed), npieces);
  return medusa_host::hip_check("medusa_base_lm_head_pack launch");
}

extern "C" size_t medusa_heads_packed_bytes(int K, int H, int V) {
  using namespace medusa;
  if (K < 1 || K > kMaxHeads) return 0;
  return static_cast<size_t>(K) * medusa_base_lm_head_packed_bytes(H, V);
}

extern "C" int medusa_heads_pack(int dtype, int K, int H, int V, const void* w_lm, void* w_packed, void* stream) {
  using namespace medusa;
  MEDUSA_REQUIRE(K >= 1 && K <= kMaxHeads, MEDUSA_ERR_SHAPE, "%s: K=%d", __func__, K);
  MEDUSA_REQUIRE(dtype == MEDUSA_BF16, MEDUSA_ERR_DTYPE, "%s: dtype %d (bf16 only)", __func__, dtype);
  MEDUSA_REQUIRE(H >= 8 && H <= (1 << 16) && H % 8 == 0, MEDUSA_ERR_SHAPE, "%s: H=%d", __func__, H);
  MEDUSA_REQUIRE(V >= 1 && V <= (1 << 24), MEDUSA_ERR_SHAPE, "%s: V=%d", __func__, V);
  MEDUSA_REQUIRE_PTR(w_lm);
  MEDUSA_REQUIRE_PTR(w_packed);
  MEDUSA_REQUIRE(w_packed != w_lm, MEDUSA_ERR_ALIAS, "%s: w_packed must not alias w_lm", __func__);
  const size_t head_in = static_cast<size_t>(V) * H, head_out = medusa_base_lm_head_packed_bytes(H, V) / 2;
  for (int j = 0; j < K; ++j) {
    const int rc = medusa_base_lm_head_pack(dtype, H, V, static_cast<const uint16_t*>(w_lm) + j * head_in,
                                            static_cast<uint16_t*>(w_packed) + j * head_out, stream);
    if (rc != MEDUSA_OK) return rc;
  }
  return MEDUSA_OK;
}

extern "C" int medusa_base_lm_head(int dtype, int M, int H, int V, const void* hidden, const void* w_base,
                                   int w_packed, float* logits, void* stream) {
  using namespace medusa;
  MEDUSA_REQUIRE(dtype == MEDUSA_BF16, MEDUSA_ERR_DTYPE, "%s: dtype %d (bf16 only)", __func__, dtype);
  MEDUSA_REQUIRE(M >= 1 && M <= kMaxBatch * kMaxNodes, MEDUSA_ERR_SHAPE, "%s: M=%d", __func__, M);
  MEDUSA_REQUIRE(H >= 8 && H <= (1 << 16) && H % 8 == 0, MEDUSA_ERR_SHAPE, "%s: H=%d", __func__, H);
  MEDUSA_REQUIRE(V >= 1 && V <= (1 << 24), MEDUSA_ERR_SHAPE, "%s: V=%d", __func__, V);
  MEDUSA_REQUIRE_PTR(hidden);
  MEDUSA_REQUIRE_PTR(w_base);
  MEDUSA_REQUIRE_PTR(logits);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int mt = medusa_host::bh_mtile(M);
  dim3 grid((V + kBhVBlock - 1) / kBhVBlock, (M + mt - 1) / mt);
  BhEpiArgs none{};
  none.T = 1;
  const auto* h16 = static_cast<const uint16_t*>(hidden);
  const auto* w16 = static_cast<const uint16_t*>(w_base);
  if (w_packed)
    medusa_host::bh_launch<true, kEpiLogits>(M, H, V, grid, h16, w16, logits, none, st);
  else
    medusa_host::bh_launch<false, kEpiLogits>(M, H, V, grid, h16, w16, logits, none, st);
  return medusa_host::hip_check("medusa_base_lm_head launch");
}

namespace {
size_t bp_parts_bytes(int B, int T, int V) {
  return medusa_host::round_up(static_cast<size_t>(B) * T * ((V + medusa::kBhVBlock - 1) / medusa::kBhVBlock) *
                                   sizeof(medusa::RowStat), 256);
}
size_t bp_merged_bytes(int B, int T) {
  return medusa_host::round_up(static_cast<size_t>(B) * T * sizeof(medusa::RowStat), 256);
}
size_t bp_childz_bytes(int B, int T) {
  return medusa_host::round_up(static_cast<size_t>(B) * T * T * sizeof(float), 256);
}
constexpr int kBpMaxParts = 1024;   // vocabulary blocks the merge takes: V <= 131072
}  // namespace

extern "C" size_t medusa_base_posterior_workspace(int B, int T, int H, int V) {
  using namespace medusa;
  if (B < 1 || B > kMaxBatch || T < 1 || T > kMaxNodes || H < 8 || H > (1 << 16) || H % 8 != 0 || V < 1 ||
      (V + kBhVBlock - 1) / kBhVBlock > kBpMaxParts)
    return 0;
  return bp_parts_bytes(B, T, V) + bp_merged_bytes(B, T) + bp_childz_bytes(B, T);
}

extern "C" int medusa_base_posterior(int B, int T, int H, int V, int p_max, int D, const void* hidden,
                                     const void* w_base, int w_packed, const int32_t* tree_candidates,
                                     const int32_t* retrieve, const int32_t* num_paths, float temperature,
                                     float eps, float delta, int32_t* best_path, int32_t* accept_len,
                                     int32_t* next_token, void* ws, size_t ws_bytes, void* stream) {
  using namespace medusa;
  MEDUSA_REQUIRE(B >= 1 && B <= kMaxBatch, MEDUSA_ERR_SHAPE, "%s: B=%d", __func__, B);
  MEDUSA_REQUIRE(T >= 1 && T <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: T=%d", __func__, T);
  MEDUSA_REQUIRE(H >= 8 && H <= (1 << 16) && H % 8 == 0, MEDUSA_ERR_SHAPE, "%s: H=%d", __func__, H);
  MEDUSA_REQUIRE(V >= 1 && (V + kBhVBlock - 1) / kBhVBlock <= kBpMaxParts, MEDUSA_ERR_SHAPE,
                 "%s: V=%d (at most %d)", __func__, V, kBpMaxParts * kBhVBlock);
  MEDUSA_REQUIRE(p_max >= 1 && p_max <= kMaxNodes, MEDUSA_ERR_SHAPE, "%s: p_max=%d", __func__, p_max);
  MEDUSA_REQUIRE(D >= 1 && D <= kMaxHeads + 1, MEDUSA_ERR_SHAPE, "%s: D=%d", __func__, D);
  MEDUSA_REQUIRE(temperature == temperature && temperature >= 0.f, MEDUSA_ERR_VALUE,
                 "%s: temperature must be >= 0", __func__);
  MEDUSA_REQUIRE(temperature == 0.f || (eps == eps && eps > 0.f && delta == delta && delta > 0.f),
                 MEDUSA_ERR_VALUE, "%s: eps and delta must be positive", __func__);
  MEDUSA_REQUIRE_PTR(hidden);
  MEDUSA_REQUIRE_PTR(w_base);
  MEDUSA_REQUIRE_PTR(tree_candidates);
  MEDUSA_REQUIRE_PTR(retrieve);
  MEDUSA_REQUIRE_PTR(num_paths);
  MEDUSA_REQUIRE_PTR(best_path);
  MEDUSA_REQUIRE_PTR(accept_len);
  MEDUSA_REQUIRE_PTR(next_token);
  MEDUSA_REQUIRE_PTR(ws);
  const size_t need = medusa_base_posterior_workspace(B, T, H, V);
  MEDUSA_REQUIRE(ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes,
                 need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  RowStat* parts = reinterpret_cast<RowStat*>(base);
  RowStat* merged = reinterpret_cast<RowStat*>(base + bp_parts_bytes(B, T, V));
  float* child_z = reinterpret_cast<float*>(base + bp_parts_bytes(B, T, V) + bp_merged_bytes(B, T));
  const int M = B * T;
  dim3 grid((V + kBhVBlock - 1) / kBhVBlock, (M + kBhMTile - 1) / kBhMTile);
  BhEpiArgs args{};
  args.T = T;
  args.temperature = temperature;
  args.candidates = tree_candidates;
  args.parts = parts;
  args.child_z = child_z;
  if (w_packed)
    medusa_host::bh_launch<true, kEpiStats>(M, H, V, grid, static_cast<const uint16_t*>(hidden),
                                            static_cast<const uint16_t*>(w_base), nullptr, args, st);
  else
    medusa_host::bh_launch<false, kEpiStats>(M, H, V, grid, static_cast<const uint16_t*>(hidden),
                                             static_cast<const uint16_t*>(w_base), nullptr, args, st);
  int rc = medusa_host::hip_check("medusa_base_posterior launch");
  if (rc != MEDUSA_OK) return rc;
  return medusa_host::posterior_from_parts(B, T, V, p_max, D, static_cast<int>(grid.x), parts, merged, child_z,
                                           tree_candidates, retrieve, num_paths, temperature, eps, delta,
                                           best_path, accept_len, next_token, st);
}
