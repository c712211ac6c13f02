// Paged prefill attention for gfx950: the newest tokens of each sequence,
// already written to the cache, attend causally to the sequence's cached
// tokens, their own included.
//
// What is computed ("PagedAttention: paging the KV cache like an OS pages
// memory", "How it works": attention is standard causal attention and only
// the storage changes; "Paged Attention Explained", "How Paged Attention
// Works", Steps 2-4: blocks for the new tokens are allocated and filled, then
// attention gathers K/V through the block table).  Sequence i with context
// length T_i whose last n_i tokens are new: new token k sits at position
// T_i - n_i + k and attends to positions 0 .. T_i - n_i + k.
//
// Query rows.  The rows of one (sequence, kv head) are the pairs (new token
// k, query head g of the group), row = k * G + g, so the 16 columns of an
// MFMA tile are full whatever the group size; a wave owns NB such tiles and
// keeps one online softmax per row (reference raised lazily, only when a
// score passes it by 2^8).  Scores are S = K.Q^T with
// v_mfma_f32_16x16x32_{bf16,f16} (tokens x rows, head_dim reduced).
//
// Two kernels:
//   * 16-bit pools (prefill_lds_kernel): a workgroup of eight waves stages
//     each 64-token stage of K/V in LDS once, with the next stage's loads in
//     flight, and reduces P.V as O^T = V^T.P^T with v_mfma_f32_16x16x32 over
//     32-token pairs; workgroups are ordered so that one XCD runs all row
//     tiles of a (sequence, kv head) pair back to back (they share its L2).
//   * float32 pools (prefill_kernel): each wave streams its own K/V units from
//     the pool (v_mfma_f32_16x16x4_f32), with O += P.V per 16-token unit.
//
// Memory safety: lengths and query offsets are clamped to the buffers the
// caller declared, table reads stay inside the row and block ids outside
// [0, N) read block 0 and are masked.
#include <algorithm>
#include <type_traits>

#include "../launch.hpp"
#include "common.hpp"
#include "stream.hpp"

namespace pa {

namespace {

constexpr int kPrefillWaves = 4;
constexpr int kPrefillThreads = 64 * kPrefillWaves;
constexpr float kNegInfP = -__builtin_inff();
constexpr float kRescaleLog2P = 8.0f;

// Row tiles per wave and units in flight ahead of the one being computed.
#ifndef PA_PREFILL_TILES
#define PA_PREFILL_TILES 2
#endif
#ifndef PA_PREFILL_PREFETCH
#define PA_PREFILL_PREFETCH 1
#endif
constexpr int kTilesPerWave = PA_PREFILL_TILES;

constexpr int kPrefillPrefetch = PA_PREFILL_PREFETCH;

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

template <typename T, int D, int NB>
struct PrefillState {
  static constexpr int kBytes = T::kBytes;
  static constexpr int E = 16 / kBytes;
  static constexpr int NCH = D / (4 * E);  // 16-byte chunks per lane per unit
  static constexpr int NT = D / 16;        // 16-wide head_dim tiles of the output
  uint4 qb[NB][NCH];                       // B operand of S = K.Q^T per tile
  f32x4_t acc[NB][NT];
  float m_col[NB];                         // reference max of this lane's row (log2 units)
  float l_part[NB];                        // this lane's share of the row's sum
  int qpos[NB];                            // position of this lane's row, -1 for a padding row
};

// One unit for one row tile: scores, mask, online softmax, P.V.
template <typename T, int D, int NB>
__device__ __forceinline__ void prefill_tile(PrefillState<T, D, NB>& st, int b,
                                             Frag<PrefillState<T, D, NB>::NCH>& f, int key0, int valid_tok,
                                             int grp, float sl2) {
  using S = PrefillState<T, D, NB>;
  constexpr int kBytes = S::kBytes, NCH = S::NCH, NT = S::NT;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kBytes == 2) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) s = mfma_k32<T>(f.k[c], st.qb[b][c], s);
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      s = mfma_f32_k4(__uint_as_float(f.k[c].x), __uint_as_float(st.qb[b][c].x), s);
      s = mfma_f32_k4(__uint_as_float(f.k[c].y), __uint_as_float(st.qb[b][c].y), s);
      s = mfma_f32_k4(__uint_as_float(f.k[c].z), __uint_as_float(st.qb[b][c].z), s);
      s = mfma_f32_k4(__uint_as_float(f.k[c].w), __uint_as_float(st.qb[b][c].w), s);
    }
  }
  // s[r]: score of token key0 + 4*grp + r for this lane's row (column).
  float sv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * grp + r;
    sv[r] = (t < valid_tok && key0 + t <= st.qpos[b]) ? s[r] * sl2 : kNegInfP;
  }
  const float mloc = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  if (wave_any(mloc > st.m_col[b] + kRescaleLog2P)) {
    float mx = fmaxf(mloc, __shfl_xor(mloc, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m_col[b], mx);
    const float alpha = m_new == kNegInfP ? 1.f : fast_exp2(st.m_col[b] - m_new);
    st.m_col[b] = m_new;
    st.l_part[b] *= alpha;
    // Output rows 4*grp + r of the tile take the factor of the lane whose
    // column is that row.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a = __shfl(alpha, 4 * grp + r);
#pragma unroll
      for (int t = 0; t < NT; ++t) st.acc[b][t][r] *= a;
    }
  }
  float pr[4];
  uint32_t pbits[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float e = sv[r] == kNegInfP ? 0.f : fast_exp2(sv[r] - st.m_col[b]);
    if constexpr (kBytes == 2) {
      pbits[r] = to_storage<T>(e);
      pr[r] = from_storage<T>(pbits[r]);
    } else {
      pr[r] = e;
    }
  }
  st.l_part[b] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  if constexpr (kBytes == 2) {
    const uint2 pa = make_uint2(pbits[0] | (pbits[1] << 16), pbits[2] | (pbits[3] << 16));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint4 vc = f.v[t >> 1];
      const uint2 vb = (t & 1) ? make_uint2(vc.z, vc.w) : make_uint2(vc.x, vc.y);
      st.acc[b][t] = mfma_k16<T>(pa, vb, st.acc[b][t]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      st.acc[b][t] = mfma_f32_k4(pr[0], __uint_as_float(f.v[t].x), st.acc[b][t]);
      st.acc[b][t] = mfma_f32_k4(pr[1], __uint_as_float(f.v[t].y), st.acc[b][t]);
      st.acc[b][t] = mfma_f32_k4(pr[2], __uint_as_float(f.v[t].z), st.acc[b][t]);
      st.acc[b][t] = mfma_f32_k4(pr[3], __uint_as_float(f.v[t].w), st.acc[b][t]);
    }
  }
}

template <typename T, int D, int NB, int PF>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillParams p) {
  using St = PrefillState<T, D, NB>;
  constexpr int kBytes = St::kBytes, E = St::E, NCH = St::NCH, NT = St::NT;
  constexpr int kRowsWave = 16 * NB;
  constexpr int kRowsWG = kRowsWave * kPrefillWaves;
  using B = typename T::bits;

  const int lane = threadIdx.x & 63;
  const int wave = rfl(threadIdx.x >> 6);
  const int i = blockIdx.x / p.H;
  const int h = blockIdx.x - i * p.H;
  const int G = p.G;

  // This sequence's new tokens, clamped to the declared buffers.
  const int qs = clampi(p.query_start[i], 0, p.num_q_tokens);
  const int qe = clampi(p.query_start[i + 1], qs, p.num_q_tokens);
  const int c = clampi(p.ctx[i], 0, p.ctx_cap);
  int n = qe - qs;
  n = n < p.max_query_len ? n : p.max_query_len;
  n = n < c ? n : c;
  const int rows = rfl(n * G);
  const int ntiles = (rows + kRowsWG - 1) / kRowsWG;
  const int tile = ntiles - 1 - static_cast<int>(blockIdx.y);
  if (tile < 0) return;
  const int r0 = tile * kRowsWG + wave * kRowsWave;
  if (r0 >= rows) return;
  const int last_row = (r0 + kRowsWave < rows ? r0 + kRowsWave : rows) - 1;
  const int first_pos = c - n;  // position of new token 0
  const int nunits = (first_pos + last_row / G + 16) >> 4;

  const int col = lane & 15, grp = lane >> 4;
  St st;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int row = r0 + 16 * b + col;
    const bool valid = row < rows;
    const int k = row / G, g = row - (row / G) * G;
    st.qpos[b] = valid ? first_pos + k : -1;
    const char* qbase = static_cast<const char*>(p.q) +
                        ((static_cast<size_t>(qs) + (valid ? k : 0)) * p.Hq + static_cast<size_t>(h) * G + g) * D *
                            kBytes;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc)
      st.qb[b][cc] = valid ? *reinterpret_cast<const uint4*>(qbase + ((cc * 4 + grp) * E) * kBytes)
                           : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) st.acc[b][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.m_col[b] = kNegInfP;
    st.l_part[b] = 0.f;
  }

  const int32_t* trow = p.tables + static_cast<size_t>(i) * p.max_blocks;
  UnitStream<D, kBytes> us;
  us.begin(p, trow, 0, 0, h);
  us.ids = us.fetch_ids(lane);
  Frag<NCH> f[PF + 1];
  bool ok[PF + 1];
  prologue<PF, NCH>(us, f, ok, lane);
  const float sl2 = p.scale_log2;
  stream_run<PF, NCH>(p, us, f, ok, trow, 0, 0, nunits, h, lane, [&](Frag<NCH>& fr, int u, bool okk) {
    const int key0 = u * 16;
    int valid_tok = c - key0;
    valid_tok = !okk ? 0 : (valid_tok < 16 ? valid_tok : 16);
    if (valid_tok < 16) mask_v_tail<kBytes, NCH>(fr, grp, valid_tok);
#pragma unroll
    for (int b = 0; b < NB; ++b) prefill_tile<T, D, NB>(st, b, fr, key0, valid_tok, grp, sl2);
  });

  // Normalise and store: accumulator row 4*grp + r of tile b, head_dim
  // entry t*16 + col; the row's sum sits in the lane whose column is that row.
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float l_col = st.l_part[b] + __shfl_xor(st.l_part[b], 16);
    l_col += __shfl_xor(l_col, 32);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = 4 * grp + r;
      const float L = __shfl(l_col, rr);
      const int row = r0 + 16 * b + rr;
      if (row < rows) {
        const int k = row / G, g = row - (row / G) * G;
        B* orow = static_cast<B*>(p.out) +
                  ((static_cast<size_t>(qs) + k) * p.Hq + static_cast<size_t>(h) * G + g) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float o = L > 0.f ? st.acc[b][t][r] / L : 0.f;
          orow[t * 16 + col] = static_cast<B>(to_storage<T>(o));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 16-bit pools: K/V staged once per workgroup in LDS.
//
// A stage is NP pairs of consecutive units (32 * NP tokens).  Each wave loads
// its share of the stage's sub-tiles (K or V of one unit, 1 KiB per load
// instruction, in flight while the previous stage is computed), zeroes tokens past the
// context and units of invalid blocks, and writes it to one of two LDS
// buffers; after a barrier every wave reads the stage's fragments.  K keeps
// the pool's operand layout (A operand of S = K.Q^T, tokens x rows).  V is
// stored interleaved per pair so that one 16-byte read is, for head_dim tile
// t and lane (col, grp), the entries d = t*16 + col of tokens 4*grp .. 4*grp+3
// of the pair's first unit, then of its second: the A operand of
// O^T += V^T.P^T with v_mfma_f32_16x16x32 over the pair's 32 tokens, whose B
// operand -- P of row col at those tokens -- is exactly what the lane holds
// after S = K.Q^T.  The result has query rows along the lanes: a lane owns
// one row (its softmax reference, its rescale factor, its sum) and four
// consecutive head_dim entries per tile, stored with 8-byte writes.
//
// The softmax work per score is a max, one FMA (scale and reference folded),
// one exp2 and half a packed convert: stages that lie wholly below every row's
// position and inside the context take no mask, and the row sums come from
// one more MFMA of P against ones.
// ---------------------------------------------------------------------------
template <int D, int NP>
struct PrefillLds {
  static constexpr int NCH = D / 32;
  static constexpr int NT = D / 16;
  uint4 k[2][2 * NP][NCH][64];  // [buffer][unit][chunk][lane]
  uint2 v[2][NP][NT][64][2];    // [buffer][pair][head_dim tile][lane][unit of the pair]
};

// Zero the 16-bit entries of tokens >= valid in a V chunk: lane group grp
// holds tokens 4*grp .. 4*grp+3 (two per 32-bit word), for two head_dim tiles.
__device__ __forceinline__ uint4 zero_v_tail(uint4 x, int grp, int valid) {
  const int t0 = 4 * grp;
  const uint32_t m01 = (t0 + 0 < valid ? 0x0000ffffu : 0u) | (t0 + 1 < valid ? 0xffff0000u : 0u);
  const uint32_t m23 = (t0 + 2 < valid ? 0x0000ffffu : 0u) | (t0 + 3 < valid ? 0xffff0000u : 0u);
  return make_uint4(x.x & m01, x.y & m23, x.z & m01, x.w & m23);
}

// Heaviest-first order of the 16-bit kernel's workgroups.  Its work items
// are the (sequence, row tile) pairs, each run once per kv head; an item
// costs about as many stages as its last row has keys / stage.  The hardware
// hands workgroups to the CUs in grid order as they free up, so a grid in
// plain order can end with a few long items on few CUs (prompts of very
// different lengths, or short chunks over very different contexts).  Every
// workgroup computes the same order in LDS (a counting sort of the items by
// stage count, heaviest first, ties in item order) and takes its own entry:
// rank r of that order, kv head h.  Workgroups past the last non-empty item
// exit at once.
constexpr int kLptMaxItems = 4096;  // sequences x row tiles; more: plain order
// With more row tiles per (sequence, kv head) pair than this (long prompts)
// the plain order is kept: it already runs each pair's tiles heaviest first,
// back to back on one XCD (sharing its L2), and a grid sized for the longest
// prompt holds many empty slots that would each pay for the sort.  Fewer
// tiles per pair (chunks of new tokens over cached contexts) leave the
// spread of context lengths to decide the finishing time: sorted there.
constexpr int kLptMaxTiles = 8;
constexpr int kLptKeys = 1024;      // sort keys: 1023 - min(stages, 1023)

struct LptLds {
  int start[kLptKeys];         // items per key, then the first rank of each key
  uint16_t key[kLptMaxItems];  // key of each item
  int wsum[16];                // per-wave sums
  int pick;                    // the item chosen for this workgroup
};

// Stages of item (sequence i, grid row y) in prefill_lds_kernel; 0: no rows.
template <int kRowsWG, int kKeys>
__device__ __forceinline__ int item_stages(const PrefillParams& p, int i, int y) {
  const int qs = clampi(p.query_start[i], 0, p.num_q_tokens);
  const int qe = clampi(p.query_start[i + 1], qs, p.num_q_tokens);
  const int c = clampi(p.ctx[i], 0, p.ctx_cap);
  int n = qe - qs;
  n = n < p.max_query_len ? n : p.max_query_len;
  n = n < c ? n : c;
  const int rows = n * p.G;
  const int tile = (rows + kRowsWG - 1) / kRowsWG - 1 - y;
  if (tile < 0) return 0;
  const int last_row = (tile * kRowsWG + kRowsWG < rows ? tile * kRowsWG + kRowsWG : rows) - 1;
  return (c - n + last_row / p.G + kKeys) / kKeys;
}

// This workgroup's (sequence, kv head, grid row) in heaviest-first order;
// false when it has none.  With H a multiple of 8, consecutive workgroups go
// to the eight XCDs in turn and XCD x runs kv heads x, x + 8, ... of every
// item, so all XCDs see the same order and the workgroups of one (sequence,
// kv head) pair share an L2.  Called by every thread of the workgroup.
template <int NW, int kRowsWG, int kKeys>
__device__ bool lpt_item(const PrefillParams& p, LptLds& L, int& i, int& h, int& y) {
  constexpr int kThreads = 64 * NW;
  constexpr int kRun = kLptKeys / kThreads;
  static_assert(kRun * kThreads == kLptKeys && NW <= 16, "key runs");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int U = p.S * p.tiles;
  for (int k = tid; k < kLptKeys; k += kThreads) L.start[k] = 0;
  if (tid == 0) L.pick = -1;
  __syncthreads();
  for (int u = tid; u < U; u += kThreads) {
    const int si = u / p.tiles;
    const int st = item_stages<kRowsWG, kKeys>(p, si, u - si * p.tiles);
    const int key = kLptKeys - 1 - (st < kLptKeys - 1 ? st : kLptKeys - 1);
    L.key[u] = static_cast<uint16_t>(key);
    atomicAdd(&L.start[key], 1);
  }
  __syncthreads();
  // Exclusive scan of the key counts: thread t owns keys t*kRun .. t*kRun+kRun-1.
  int run[kRun];
  int tot = 0;
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    run[r] = L.start[tid * kRun + r];
    tot += run[r];
  }
  int inc = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o);
    if (lane >= o) inc += v;
  }
  if (lane == 63) L.wsum[wave] = inc;
  __syncthreads();
  int ex = inc - tot;
  for (int w = 0; w < wave; ++w) ex += L.wsum[w];
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    L.start[tid * kRun + r] = ex;
    ex += run[r];
  }
  __syncthreads();
  const int nonempty = L.start[kLptKeys - 1];  // items with stages sort before the empty key
  int rank, hh;
  if ((p.H & 7) == 0) {
    const int hx = p.H >> 3, j = blockIdx.x >> 3;
    rank = j / hx;
    hh = (j - rank * hx) * 8 + (blockIdx.x & 7);
  } else {
    rank = blockIdx.x / p.H;
    hh = blockIdx.x - rank * p.H;
  }
  if (rank >= nonempty) return false;  // whole workgroup
  // The key holding this rank: the last key whose first rank is <= rank.
  int lo = 0, hi = kLptKeys - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (L.start[mid] <= rank) lo = mid;
    else hi = mid - 1;
  }
  const int kb = lo;
  int want = rank - L.start[kb];
  // The want-th item with key kb, in item order.
  for (int c0 = 0; c0 < U; c0 += kThreads) {
    const int u = c0 + tid;
    const bool f = u < U && L.key[u] == kb;
    const uint64_t m = __builtin_amdgcn_ballot_w64(f);
    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
    if (lane == 0) L.wsum[wave] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < NW; ++w) {
      const int v = L.wsum[w];
      total += v;
      before += w < wave ? v : 0;
    }
    if (f && before + below == want) L.pick = u;
    __syncthreads();
    if (want < total) break;  // uniform: every thread read the same sums
    want -= total;
  }
  const int u = L.pick;
  if (u < 0 || u >= U) return false;  // not reached: the counts above place every rank
  i = u / p.tiles;
  y = u - i * p.tiles;
  h = hh;
  return true;
}

// Row tiles of sequence i's new tokens (rows = new tokens x G) in the 16-bit
// kernel's workgroups of kRowsWG rows.
template <int kRowsWG>
__device__ __forceinline__ int seq_tiles(const PrefillParams& p, int i) {
  const int qs = clampi(p.query_start[i], 0, p.num_q_tokens);
  const int qe = clampi(p.query_start[i + 1], qs, p.num_q_tokens);
  const int c = clampi(p.ctx[i], 0, p.ctx_cap);
  int n = qe - qs;
  n = n < p.max_query_len ? n : p.max_query_len;
  n = n < c ? n : c;
  return (n * p.G + kRowsWG - 1) / kRowsWG;
}

// Plain order over the row tiles that hold rows: consecutive workgroups go
// to the eight XCDs in turn, and slot s of XCD x is the s-th (pair, tile)
// among the (sequence, kv head) pairs x, x + 8, x + 16, ..., each pair's
// tiles heaviest first.  The grid is sized for the longest prompt; its slots
// past the real tiles come last and exit at once, instead of sitting between
// the real ones.  Each wave computes the mapping alone (a scan of the XCD's
// pairs, 64 per step), so no barrier is needed.  False: no tile.
template <int kRowsWG>
__device__ bool compact_item(const PrefillParams& p, int& i, int& h, int& y) {
  const int lane = threadIdx.x & 63;
  const int xcd = blockIdx.x & 7;
  const int s = static_cast<int>(blockIdx.x >> 3);
  const int npairs = p.S * p.H;
  const int nk = npairs > xcd ? (npairs - xcd + 7) / 8 : 0;  // pairs of this XCD
  int base = 0;
  for (int k0 = 0; k0 < nk; k0 += 64) {
    const int k = k0 + lane;
    const int nt = k < nk ? seq_tiles<kRowsWG>(p, (xcd + 8 * k) / p.H) : 0;
    int inc = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o);
      if (lane >= o) inc += v;
    }
    const int tot = __shfl(inc, 63);
    if (s < base + tot) {
      // the first lane whose run ends past s holds it (that lane has tiles)
      const int L = static_cast<int>(__builtin_ctzll(__builtin_amdgcn_ballot_w64(s < base + inc)));
      const int first = base + __shfl(inc - nt, L);
      const int pair = xcd + 8 * (k0 + L);
      i = pair / p.H;
      h = pair - i * p.H;
      y = s - first;
      return true;
    }
    base += tot;
  }
  return false;
}

#ifndef PA_PREFILL_COMPACT
#define PA_PREFILL_COMPACT 1
#endif
#ifndef PA_PREFILL_LPT
#define PA_PREFILL_LPT 1
#endif
#ifndef PA_PREFILL_WAVES_PER_EU
#define PA_PREFILL_WAVES_PER_EU 2
#endif
template <typename T, int D, int NW, int NB, int NP>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(PA_PREFILL_WAVES_PER_EU,
                                                                         PA_PREFILL_WAVES_PER_EU))) void prefill_lds_kernel(
    PrefillParams p, const int32_t* __restrict__ tables) {
  static_assert(T::kBytes == 2, "16-bit pools only");
  constexpr int NCH = D / 32;  // 1 KiB chunks per sub-tile
  constexpr int NT = D / 16;
  constexpr int kUnits = 2 * NP;         // units per stage
  constexpr int kKeys = 16 * kUnits;     // keys per stage
  constexpr int kRowsWave = 16 * NB;
  constexpr int kRowsWG = kRowsWave * NW;
  // Sub-tiles (the K or the V of one unit) per wave per stage: one (eight
  // waves), or the K and the V of one unit (four waves).
  constexpr int kSPW = 2 * kUnits / NW;
  static_assert(kSPW * NW == 2 * kUnits && (kSPW == 1 || kSPW == 2), "whole sub-tiles per wave");
  constexpr int kLoads = kSPW * NCH;  // chunk loads per wave per stage
  using B = typename T::bits;
  __shared__ PrefillLds<D, NP> sm;

  const int lane = threadIdx.x & 63;
  const int wave = rfl(threadIdx.x >> 6);
  // Workgroup -> (sequence, kv head, row tile).  In plain order consecutive
  // workgroups go to the eight XCDs in turn; XCD x runs the (sequence, kv
  // head) pairs x, x + 8, x + 16, ... one after the other, each pair's row
  // tiles back to back and the last (heaviest) first, so the workgroups that
  // run at the same time on an XCD read the same K/V through its L2.  The
  // heaviest-first order (lpt_item) keeps the XCD of each pair.
  int i, h, y;
  if (p.lpt) {
    __shared__ LptLds lpt;
    if (!lpt_item<NW, kRowsWG, kKeys>(p, lpt, i, h, y)) return;  // whole workgroup
  } else {
#if PA_PREFILL_COMPACT
    if (!compact_item<kRowsWG>(p, i, h, y)) return;  // whole workgroup (every wave finds the same)
#else
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int pair = (slot / p.tiles) * 8 + xcd;
    y = slot - (slot / p.tiles) * p.tiles;
    if (pair >= p.S * p.H) return;  // whole workgroup
    i = pair / p.H;
    h = pair - i * p.H;
#endif
  }
  i = rfl(i);
  h = rfl(h);
  y = rfl(y);
  const int G = p.G;
  const int qs = clampi(p.query_start[i], 0, p.num_q_tokens);
  const int qe = clampi(p.query_start[i + 1], qs, p.num_q_tokens);
  const int c = clampi(p.ctx[i], 0, p.ctx_cap);
  int n = qe - qs;
  n = n < p.max_query_len ? n : p.max_query_len;
  n = n < c ? n : c;
  const int rows = rfl(n * G);
  const int ntiles = (rows + kRowsWG - 1) / kRowsWG;
  const int tile = ntiles - 1 - y;
  if (tile < 0) return;  // whole workgroup
  const int first_pos = c - n;
  const int wg_last_row = (tile * kRowsWG + kRowsWG < rows ? tile * kRowsWG + kRowsWG : rows) - 1;
  const int nst = (first_pos + wg_last_row / G + kKeys) / kKeys;  // stages covering the workgroup's keys
  const int r0 = tile * kRowsWG + wave * kRowsWave;
  const bool active = r0 < rows;
  const int last_row = (r0 + kRowsWave < rows ? r0 + kRowsWave : rows) - 1;
  const int kmax = active ? first_pos + last_row / G : -1;  // last key this wave attends to

  const int col = lane & 15, grp = lane >> 4;
  uint4 qb[NB][NCH];
  f32x4_t acc[NB][NT];  // O^T: head_dim t*16 + 4*grp + r of row col
  f32x4_t lsum[NB];     // the row's sum (every entry)
  float m_ref[NB];      // reference max of the row, log2 units
  int qpos[NB];         // position of the lane's row (-1: padding row)
  int qmin[NB];         // position of the tile's first row (wave-uniform)
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int row = r0 + 16 * b + col;
    const bool valid = row < rows;
    const int k = row / G, g = row - (row / G) * G;
    qpos[b] = valid ? first_pos + k : -1;
    qmin[b] = first_pos + (r0 + 16 * b) / G;
    const char* qbase = static_cast<const char*>(p.q) +
                        ((static_cast<size_t>(qs) + (valid ? k : 0)) * p.Hq + static_cast<size_t>(h) * G + g) * D * 2;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc)
      qb[b][cc] = valid ? *reinterpret_cast<const uint4*>(qbase + (cc * 4 + grp) * 16) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[b][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lsum[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_ref[b] = kNegInfP;
  }

  // Load assignment: sub-tiles wave * kSPW .. (unit = sub-tile >> 1, K or V
  // by its low bit), every chunk of each.
  const int unit = (wave * kSPW) >> 1;
  auto sub_is_v = [&](int j) { return kSPW == 2 ? j == 1 : (wave & 1) == 1; };
  // The table row is read with scalar loads (a __restrict__ argument), so
  // that locating a unit never waits on the vector loads in flight.
  const int32_t* trow = tables + static_cast<size_t>(i) * p.max_blocks;
  const char* layer_base = static_cast<const char*>(p.pool) + p.layer_off * 2;
  uint4 stg[kLoads];  // this wave's loads of the next stage
  int valid_st;       // tokens of this wave's unit to keep (0 for an invalid block)

  // This wave's unit of the next stage: logical block and 16-token sub-tile.
  const int subs = p.bs >> 4;  // sub-tiles per block
  int my_lb = unit / subs, my_sub = unit - (unit / subs) * subs;
  // Locate this wave's unit of stage s (stages are issued in order) and
  // issue its loads.
  auto issue = [&](int s, uint4 (&r)[kLoads], int& valid) {
    const int32_t bid = my_lb < p.max_blocks ? trow[my_lb] : -1;
    const bool ok = bid >= 0 && bid < p.N;
    const size_t region = (static_cast<size_t>(ok ? bid : 0) * p.H + h) * (2 * static_cast<size_t>(p.bs) * D);
    const char* kv = layer_base + (region + static_cast<size_t>(my_sub) * 16 * D) * 2;
    my_sub += kUnits;
    while (my_sub >= subs) {
      my_sub -= subs;
      ++my_lb;
    }
#pragma unroll
    for (int j = 0; j < kSPW; ++j) {
      const uint4* sp = reinterpret_cast<const uint4*>(kv + (sub_is_v(j) ? static_cast<size_t>(p.bs) * D * 2 : 0)) +
                        lane;
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) r[j * NCH + cc] = sp[64 * cc];
    }
    const int left = c - s * kKeys - unit * 16;
    valid = !ok ? 0 : (left < 0 ? 0 : (left < 16 ? left : 16));
  };
  auto to_lds = [&](uint4 (&r)[kLoads], int valid, int buf) {
#pragma unroll
    for (int j = 0; j < kSPW; ++j) {
      uint4* rj = r + j * NCH;
      const bool is_v = sub_is_v(j);
      if (valid < 16) {  // wave-uniform: the context's last unit, or an invalid block
        if (is_v) {
#pragma unroll
          for (int cc = 0; cc < NCH; ++cc) rj[cc] = zero_v_tail(rj[cc], grp, valid);
        } else {
#pragma unroll
          for (int cc = 0; cc < NCH; ++cc)
            if (col >= valid) rj[cc] = make_uint4(0, 0, 0, 0);
        }
      }
      if (is_v) {
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
          sm.v[buf][unit >> 1][2 * cc][lane][unit & 1] = make_uint2(rj[cc].x, rj[cc].y);
          sm.v[buf][unit >> 1][2 * cc + 1][lane][unit & 1] = make_uint2(rj[cc].z, rj[cc].w);
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) sm.k[buf][unit][cc][lane] = rj[cc];
      }
    }
  };

  const float sl2 = p.scale_log2;
  const uint4 ones = make_uint4(ones2<T>(), ones2<T>(), ones2<T>(), ones2<T>());
  // One stage from LDS buffer `buf`: keys key0 .. key0 + kKeys - 1.  The
  // masked form is needed only where the stage reaches past some row's
  // position (the causal diagonal and the context's end).
  auto compute = [&](int buf, int key0, bool masked) {
    // The stage's K fragments, read once and used by every row tile.
    uint4 kf[kUnits][NCH];
#pragma unroll
    for (int u = 0; u < kUnits; ++u)
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) kf[u][cc] = sm.k[buf][u][cc][lane];
    f32x4_t sc[NB][kUnits];  // scores: token key0 + 16*u + 4*grp + r of row col
    auto scores = [&](int b) {
#pragma unroll
      for (int u = 0; u < kUnits; ++u) {
        sc[b][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) sc[b][u] = mfma_k32<T>(kf[u][cc], qb[b][cc], sc[b][u]);
      }
    };
    // Mask and reference of tile b.  Keys past the context were zeroed by the
    // loader; they and the keys beyond a row's position are masked where
    // some row of the tile can see them.
    auto prep = [&](int b) {
      if (masked && key0 + kKeys - 1 > qmin[b]) {
        asm volatile("");  // keep the branch: most stages skip it
        const int lim = qpos[b] - key0 - 4 * grp;
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[b][u][r] = 16 * u + r <= lim ? sc[b][u][r] : kNegInfP;
      }
      float mraw = kNegInfP;
#pragma unroll
      for (int u = 0; u < kUnits; ++u)
        mraw = fmaxf(mraw, fmaxf(fmaxf(sc[b][u][0], sc[b][u][1]), fmaxf(sc[b][u][2], sc[b][u][3])));
      const float mloc = mraw * sl2;  // this lane's share of the row
      if (wave_any(mloc > m_ref[b] + kRescaleLog2P)) {
        // The row's maximum over its four lane groups, so that the row keeps
        // one reference.
        float mx = fmaxf(mloc, __shfl_xor(mloc, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_ref[b], mx);
        const float alpha = m_new == kNegInfP ? 1.f : fast_exp2(m_ref[b] - m_new);
        m_ref[b] = m_new;
        lsum[b] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[b][t] *= alpha;
      }
    };
    // Weights of tile b at pair q (the B operand of O^T += V^T.P^T).
    auto weights = [&](int b, int q) {
      const float nm = m_ref[b] == kNegInfP ? 0.f : -m_ref[b];
      float e[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e[r] = fast_exp2(fmaf(sc[b][2 * q][r], sl2, nm));
        e[4 + r] = fast_exp2(fmaf(sc[b][2 * q + 1][r], sl2, nm));
      }
      return make_uint4(pack2<T>(e[0], e[1]), pack2<T>(e[2], e[3]), pack2<T>(e[4], e[5]), pack2<T>(e[6], e[7]));
    };
    auto pv = [&](int b, const uint4 (&vv)[NT], uint4 pb) {
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[b][t] = mfma_k32<T>(vv[t], pb, acc[b][t]);
      lsum[b] = mfma_k32<T>(ones, pb, lsum[b]);
    };
    // Software pipeline over the row tiles: the score products of tile b go
    // out while the weights of tile b - 1 are exponentiated, and the P.V
    // products of the earlier tiles while the last tile's weights are.
    uint4 pb[NB][NP];
    scores(0);
    prep(0);
#pragma unroll
    for (int b = 1; b < NB; ++b) {
      scores(b);
#pragma unroll
      for (int q = 0; q < NP; ++q) pb[b - 1][q] = weights(b - 1, q);
      // Scheduling: one score MFMA, then three VALU instructions of the weights.
#pragma unroll
      for (int k = 0; k < kUnits * NCH; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
      prep(b);
    }
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      uint4 vv[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) vv[t] = *reinterpret_cast<const uint4*>(&sm.v[buf][q][t][lane][0]);
#pragma unroll
      for (int b = 0; b < NB - 1; ++b) pv(b, vv, pb[b][q]);
      pv(NB - 1, vv, weights(NB - 1, q));
      // Scheduling: the V reads first, then one P.V MFMA of the earlier tiles
      // and two VALU instructions of the last tile's weights, in turn.
      __builtin_amdgcn_sched_group_barrier(0x100, NT, 1);
#pragma unroll
      for (int k = 0; k < (NB - 1) * (NT + 1); ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 1);
      }
    }
  };

  // Pipeline: the loads of stage s + 1 are in flight in registers while
  // stage s is computed from LDS; they are written to the other buffer after
  // it, and one barrier per stage publishes them.
  // Stages below this wave's first row need no mask.
  const int kfull = active ? qmin[0] - kKeys + 1 : -1;
  issue(0, stg, valid_st);
  to_lds(stg, valid_st, 0);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    if (s + 1 < nst) issue(s + 1, stg, valid_st);
    const int key0 = s * kKeys;
    if (key0 <= kmax) compute(s & 1, key0, key0 > kfull);
    if (s + 1 < nst) to_lds(stg, valid_st, (s + 1) & 1);
    __syncthreads();
  }

  if (!active) return;
  // Row col of tile b: head_dim entries t*16 + 4*grp .. +3, 8 bytes per store.
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int row = r0 + 16 * b + col;
    if (row < rows) {
      const float L = lsum[b][0];
      const float inv = L > 0.f ? 1.f / L : 0.f;
      const int k = row / G, g = row - (row / G) * G;
      B* orow = static_cast<B*>(p.out) + ((static_cast<size_t>(qs) + k) * p.Hq + static_cast<size_t>(h) * G + g) * D;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint2 w = make_uint2(pack2<T>(acc[b][t][0] * inv, acc[b][t][1] * inv),
                                   pack2<T>(acc[b][t][2] * inv, acc[b][t][3] * inv));
        *reinterpret_cast<uint2*>(orow + t * 16 + 4 * grp) = w;
      }
    }
  }
}

#ifndef PA_PREFILL_LDS_WAVES
#define PA_PREFILL_LDS_WAVES 8
#endif
#ifndef PA_PREFILL_LDS_TILES
#define PA_PREFILL_LDS_TILES 2
#endif
#ifndef PA_PREFILL_LDS_PAIRS
#define PA_PREFILL_LDS_PAIRS 2
#endif
constexpr int kLdsWaves = PA_PREFILL_LDS_WAVES;
constexpr int kLdsTiles = PA_PREFILL_LDS_TILES;
constexpr int kLdsPairs = PA_PREFILL_LDS_PAIRS;

template <typename T, int D>
hipError_t launch_prefill_typed(const PrefillParams& p, hipStream_t stream) {
  constexpr bool kLds = T::kBytes == 2;
  constexpr int kRowsWG = kLds ? 16 * kLdsTiles * kLdsWaves : 16 * kTilesPerWave * kPrefillWaves;
  const int64_t tiles = (static_cast<int64_t>(p.max_query_len) * p.G + kRowsWG - 1) / kRowsWG;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.S) * p.H, static_cast<unsigned>(tiles));
  if constexpr (kLds) {
    // One dimension: eight XCD lanes of ceil(S * H / 8) pairs x tiles slots.
    PrefillParams q = p;
    q.tiles = static_cast<int32_t>(tiles);
    q.lpt = PA_PREFILL_LPT && tiles <= kLptMaxTiles && static_cast<int64_t>(p.S) * tiles <= kLptMaxItems;
    const int64_t pairs8 = (static_cast<int64_t>(p.S) * p.H + 7) / 8;
    const int64_t wgs = 8 * pairs8 * tiles;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_lds_kernel<T, D, kLdsWaves, kLdsTiles, kLdsPairs>), dim3(static_cast<unsigned>(wgs)),
                       dim3(64 * kLdsWaves), 0, stream, q, p.tables);
  } else {
    hipLaunchKernelGGL((prefill_kernel<T, D, kTilesPerWave, kPrefillPrefetch>), grid, dim3(kPrefillThreads), 0,
                       stream, p);
  }
  return hipGetLastError();
}

}  // namespace

int64_t prefill_max_query_len(int G) {
  // The smaller row tile of the two kernels bounds the grid's y extent.
  const int64_t rows_wg = std::min(16 * kLdsTiles * kLdsWaves, 16 * kTilesPerWave * kPrefillWaves);
  return static_cast<int64_t>(65535) * rows_wg / (G > 0 ? G : 1);
}

hipError_t launch_prefill(const PrefillParams& p, int dtype, int D, hipStream_t stream) {
  if (!decode_supported(dtype, D, p.G)) return hipErrorInvalidValue;
  if (p.S <= 0 || p.max_query_len <= 0) return hipSuccess;
  switch (dtype) {
    case 0:
      return D == 64 ? launch_prefill_typed<F32, 64>(p, stream) : launch_prefill_typed<F32, 128>(p, stream);
    case 1:
      return D == 64 ? launch_prefill_typed<F16, 64>(p, stream) : launch_prefill_typed<F16, 128>(p, stream);
    default:
      return D == 64 ? launch_prefill_typed<BF16, 64>(p, stream) : launch_prefill_typed<BF16, 128>(p, stream);
  }
}

}  // namespace pa
