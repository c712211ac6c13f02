// Paged single-token decode attention for gfx950.
//
// What is computed ("Paged Attention Explained", "How Paged Attention Works",
// Step 4; "PagedAttention: paging the KV cache like an OS pages memory", "How
// it works"): for every sequence and query head, softmax attention of the new
// token's query over the sequence's cached K/V, which the kernel gathers block
// by block through the sequence's block table.  The softmax is evaluated
// online (running max and sum, the technique the first page attributes to
// FlashAttention) so K/V are read exactly once.
//
// Launch sequence of one pa_decode call:
//   1. plan_kernel (one workgroup; plan_share_kernel when the pool holds
//      shared blocks) cuts every context into work items of P tokens (P
//      chosen from the total work when the caller asks for automatic
//      partitioning; with many small explicit partitions an item is four
//      consecutive partitions, one per wave) and writes the list of
//      (sequence, item, context) records, full items first and the partial
//      ones by decreasing size, so the tail of the decode consists of the
//      smallest items.  Small batches whose contexts all fit one partition
//      skip this kernel (direct launch).
//   2. the decode kernel is persistent: one workgroup of four wave64s per CU
//      takes work indices (item, kv head) from an atomic counter.  For many
//      small items it runs two indices ahead and streams item after item:
//      while it computes one item it reads the next item's record (scalar
//      load), query rows and block ids, and it issues the next item's first
//      K/V loads before merging the current item's four wave states.  For
//      the few long items of an automatic partition size it takes one index
//      at a time, which balances the end of the queue better.  The sharing
//      plan's items (a prefix several forked sequences share, read once for
//      all of them) run two workgroups per CU.
//   3. merge_kernel combines the partition states of multi-partition
//      sequences by log-sum-exp weighting, one wave per (sequence, query head).
//      (Merging inside the decode kernel, by the workgroup that finishes a
//      sequence's last partition, needs either agent-scope fences -- a whole-L2
//      writeback and invalidate per partition on gfx950 -- or a wait for
//      device-coherent stores per partition; both cost more than this launch.)
//
// Inside an item the partition is cut into 16-token units (a 16-token
// sub-tile of one block); wave w takes a contiguous run of units, keeping the
// loads of the next units in flight (16-byte loads, 1 KiB per instruction)
// while it computes the current one.
//
// Two inner paths read the same pool layout:
//   * MFMA (G = query heads per kv head >= 3): S = K.Q^T with
//     v_mfma_f32_16x16x32_{bf16,f16} (tokens x heads, head_dim reduced) and
//     O += P.V with v_mfma_f32_16x16x16 (heads x head_dim, tokens reduced);
//     float32 pools use v_mfma_f32_16x16x4_f32.  The 16x16 result layout of
//     the first product is exactly the A-operand layout of the second, so P
//     never leaves registers.
//   * VALU (G <= 2, e.g. multi-head attention): packed dot2 for Q.K, wave
//     shuffles for the per-token reduction and the block max, dot2/FMA for P.V.
//
// Online softmax with a lazily moved reference: exponentials are taken
// relative to a reference max that is raised only when a score exceeds it by
// more than 2^8; the accumulators are rescaled only then.  The result is the
// same softmax (the final division uses the same reference) while the common
// unit needs no cross-lane max and no accumulator traffic.
//
// Memory safety: context lengths are clamped to the table capacity, table
// reads stay inside the row, and block ids outside [0, N) are replaced by
// block 0 and masked, so bad inputs give unspecified values but never an
// out-of-bounds access.
#include <mutex>

#include "../launch.hpp"
#include "common.hpp"
#include "stream.hpp"
#include "write.hpp"

namespace pa {

namespace {

constexpr int kWaves = 4;  // waves of a decode workgroup, sharing one work item
constexpr int kThreads = 64 * kWaves;
constexpr int kMergeWaves = 4;
constexpr int kMergeThreads = 64 * kMergeWaves;
constexpr int kWideMergeParts = 16;  // from this many partitions, a workgroup merges one row
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleLog2 = 8.0f;  // raise the reference only past 2^8
constexpr int kPlanThreads = 1024;
constexpr int kPlanBins = 1024;       // partial items sorted by 16-token units

// Units whose loads are in flight ahead of the one being computed, and
// decode workgroups per CU.  Measured on MI355X: one workgroup of four waves
// per CU with two units (16 KiB) in flight per wave reads the paged cache
// faster than two or three workgroups per CU with one or two units each --
// fewer, deeper streams suit HBM3E here better than more, shallower ones.
#ifndef PA_PREFETCH_UNITS
#define PA_PREFETCH_UNITS 2
#endif
#ifndef PA_WG_PER_CU
#define PA_WG_PER_CU 1
#endif
constexpr int kPrefetch = PA_PREFETCH_UNITS;
constexpr int kWorkgroupsPerCU = PA_WG_PER_CU;
#ifndef PA_ITEMS_PER_WG
#define PA_ITEMS_PER_WG 2
#endif


// ---------------------------------------------------------------------------
// Work items.
// ---------------------------------------------------------------------------

// Sequences one shared work item covers at most (their G query heads each
// take a column of the 16-wide score tile).
constexpr int kShareMaxMembers = 4;

// One work item as one wave of the workgroup sees it (all values uniform).
// An item covers the tokens [start, start + ntok) of one sequence or, with
// the sharing plan, possibly of a prefix that several sequences share (x < 0:
// shared group ~x).  The members of a shared group are looked up where they
// are needed -- query rows at the start, outputs at the end -- so that no
// more registers stay live through the item than for a single sequence.
struct Item {
  int i, j, h;     // sequence (a shared group's first member), partition slot, kv head
  int ctx;         // context length (clamped)
  int start;       // first token of the item
  int ntok;        // tokens in the item
  int u0, u1;      // this wave's run of 16-token units
  int np;          // work items of the sequence
  int x;           // record's first field: the sequence, or ~group with the sharing plan
  int cols;        // query-head columns of the score tile: G per member sequence
  const int32_t* trow;  // block-table row the K/V ids are read from
};

__device__ __forceinline__ void split_units(Item& it, int per_fixed, int wave) {
  const int nunits = (it.ntok + 15) >> 4;
  const int per = per_fixed > 0 ? per_fixed : (nunits + kWaves - 1) / kWaves;
  it.u0 = wave * per;
  it.u1 = it.u0 + per < nunits ? it.u0 + per : nunits;
}

// rec = (sequence, item, clamped context, items of the sequence) as written
// by plan_kernel; an item holds PI tokens.  With group == 1 the four waves
// split the item evenly.  Otherwise the item is `group` consecutive
// partitions of PI / group tokens and wave w computes partition w of it.
// Either way the waves' states are then combined through LDS.
__device__ __forceinline__ Item make_item(const DecodeParams& p, int4 rec, int h, int PI, int group, int wave) {
  Item it;
  it.i = rfl(rec.x);
  it.j = rfl(rec.y);
  it.ctx = rfl(rec.z);
  it.np = rfl(rec.w);
  it.h = h;
  it.start = it.j * PI;
  const int left = it.ctx - it.start;
  it.ntok = left < PI ? (left > 0 ? left : 0) : PI;
  split_units(it, group > 1 ? (PI / group) >> 4 : 0, wave);
  it.trow = p.tables + static_cast<size_t>(it.i) * p.max_blocks;
  it.x = it.i;
  it.cols = p.G;
  return it;
}

// Member sequences of an item of the sharing plan (-1 = none).
__device__ __forceinline__ int4 item_members(const Item& it, const int4* __restrict__ groups) {
  if (it.x >= 0) return make_int4(it.x, -1, -1, -1);
  const int4 g = groups[~it.x];
  return make_int4(rfl(g.x), rfl(g.y), rfl(g.z), rfl(g.w));
}

// Sharing plan: rec = (sequence, partition slot, first token, end token), or
// (~group, ...) for an item over a prefix that the group's members share;
// groups[g] lists those members.
__device__ __forceinline__ Item make_item_share(const DecodeParams& p, int4 rec, int h, int wave,
                                                const int4* __restrict__ groups) {
  Item it;
  it.x = rfl(rec.x);
  it.j = rfl(rec.y);
  it.start = rfl(rec.z);
  const int end = rfl(rec.w);
  it.ntok = end > it.start ? end - it.start : 0;
  it.ctx = end;
  it.h = h;
  it.np = 0;  // per member, read where the item's states are written
  split_units(it, 0, wave);
  const int4 m = item_members(it, groups);
  it.i = m.x;
  it.cols = (1 + (m.y >= 0) + (m.z >= 0) + (m.w >= 0)) * p.G;
  it.trow = p.tables + static_cast<size_t>(it.i) * p.max_blocks;
  return it;
}

// The whole run of one item, its first piece's prologue already issued.
template <int PF, int NCH, typename Stream, typename Compute>
__device__ __forceinline__ void stream_item(const DecodeParams& p, Stream& st,
                                            Frag<NCH> (&f)[PF + 1], bool (&ok)[PF + 1], const Item& it,
                                            int lane, Compute&& compute) {
  stream_run<PF, NCH>(p, st, f, ok, it.trow, it.start, it.u0, it.u1, it.h, lane, compute);
}

// ---------------------------------------------------------------------------
// Merging the four waves' states of an item.
// ---------------------------------------------------------------------------

// LDS merge of the four waves' states, then either the final output or the
// partition's workspace entry.  Rows are the query heads of this kv head.
// `slot` carries work indices from thread 0 to the workgroup.
template <int D, int GMAX>
struct MergeSmem {
  static constexpr int kRows = GMAX;
  float m[kWaves][GMAX];
  float l[kWaves][GMAX];
  float o[kWaves][GMAX][D];
  float wt[kWaves][GMAX];  // each wave's weight in a column's merged output (2^(m_w - M) / L)
  float cm[GMAX], cl[GMAX];  // a column's merged maximum and sum
  int slot[4];
};

template <typename T>
__device__ __forceinline__ void store_out(const DecodeParams& p, size_t row, int d, int D, float o) {
  using B = typename T::bits;
  static_cast<B*>(p.out)[row * D + d] = static_cast<B>(to_storage<T>(o));
}

template <typename T, int D, int GMAX, bool kShare = false>
__device__ __forceinline__ void finish_partition(const DecodeParams& p, MergeSmem<D, GMAX>& sm, const Item& it,
                                                 const int4* __restrict__ groups = nullptr,
                                                 const int32_t* __restrict__ seq_np = nullptr) {
  // Sharing plan: column c is query head c % G of member c / G, and each
  // member has its own number of states.
  int4 mem = make_int4(it.i, -1, -1, -1), mnp = make_int4(it.np, -1, -1, -1);
  if constexpr (kShare) {
    mem = item_members(it, groups);
    mnp.x = rfl(seq_np[mem.x]);
    mnp.y = mem.y >= 0 ? rfl(seq_np[mem.y]) : -1;
    mnp.z = mem.z >= 0 ? rfl(seq_np[mem.z]) : -1;
    mnp.w = mem.w >= 0 ? rfl(seq_np[mem.w]) : -1;
  }
  __syncthreads();
  const int G = p.G;
  const int rows = kShare ? it.cols : G;
  // Per column (one thread each): the merged maximum and sum, and each
  // wave's weight in the merged output; then every (column, head_dim) entry
  // is one weighted sum of the four waves' entries.
  if (threadIdx.x < rows) {
    const int c = threadIdx.x;
    float M = sm.m[0][c];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.m[w][c]);
    float f[kWaves], L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.m[w][c];
      f[w] = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
      L += f[w] * sm.l[w][c];
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sm.wt[w][c] = f[w] * inv;
    sm.cm[c] = M;
    sm.cl[c] = L;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < rows * D; idx += kThreads) {
    const int c = idx / D, d = idx - c * D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o = fmaf(sm.wt[w][c], sm.o[w][c][d], o);
    const float M = sm.cm[c], L = sm.cl[c];
    int seq = it.i, np = it.np, g = c;
    if constexpr (kShare) {
      const int m = c / G;
      g = c - m * G;
      seq = m == 0 ? mem.x : m == 1 ? mem.y : m == 2 ? mem.z : mem.w;
      np = m == 0 ? mnp.x : m == 1 ? mnp.y : m == 2 ? mnp.z : mnp.w;
    }
    const size_t row = static_cast<size_t>(seq) * p.Hq + it.h * G + g;
    if (np == 1) {
      store_out<T>(p, row, d, D, o);
    } else {
      const size_t e = row * p.ws_stride + it.j;
      p.ws_o[e * D + d] = o;
      if (d == 0) {
        p.ws_ml[2 * e] = M;
        p.ws_ml[2 * e + 1] = L;
      }
    }
  }
}

// Context length of sequence i clamped to [0, ctx_cap] (per lane).
__device__ __forceinline__ int clamp_ctx(const DecodeParams& p, int i) {
  int c = p.ctx[i];
  c = c < 0 ? 0 : c;
  return c > p.ctx_cap ? p.ctx_cap : c;
}

// ---------------------------------------------------------------------------
// Work items: plan kernel.
// ---------------------------------------------------------------------------

// Partition size of an automatic decode: as large as keeps about
// kItemsPerWorkgroup work items per workgroup of the persistent grid (fewer,
// longer items cost fewer item starts and fewer partition merges; the sorted
// work list keeps the tail short), never below the caller's minimum, at most
// kMaxAutoPartition tokens, a multiple of the block size.  Measured on
// MI355X: two items per workgroup against four leave the Llama-3-8B- and
// OPT-13B-shaped batches unchanged (the 4096-token cap decides there) and
// make the shared-prefix batch 11% faster (each 2304-token branch is one
// item instead of two).
constexpr int kItemsPerWorkgroup = PA_ITEMS_PER_WG;
constexpr int kMaxAutoPartition = 4096;

__device__ __forceinline__ void plan_plain(const DecodeParams& p) {
  __shared__ int cnt[kPlanBins];
  __shared__ int off[kPlanBins];
  __shared__ int wsum[kPlanThreads / 64];
  __shared__ long long wtok[kPlanThreads / 64];
  __shared__ int sP;
  __shared__ int4 longs[kPlanThreads];  // (sequence, first item, full items, context)
  __shared__ int long_np[kPlanThreads];
  __shared__ int nlong;
  constexpr int kCached = 4;  // context lengths kept in registers per thread
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int cc[kCached];
  long long tok = 0;
#pragma unroll
  for (int k = 0; k < kCached; ++k) {
    const int i = threadIdx.x + k * kPlanThreads;
    cc[k] = i < p.S ? clamp_ctx(p, i) : 0;
    tok += cc[k];
  }
  for (int i = threadIdx.x + kCached * kPlanThreads; i < p.S; i += kPlanThreads) tok += clamp_ctx(p, i);
  auto ctx_of = [&](int k, int i) { return k < kCached ? cc[k] : clamp_ctx(p, i); };
  for (int b = threadIdx.x; b < kPlanBins; b += kPlanThreads) cnt[b] = 0;
  if (p.auto_partition) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tok += __shfl_xor(tok, o);
    if (lane == 0) wtok[wave] = tok;
    __syncthreads();
    if (threadIdx.x == 0) {
      long long total = 0;
      for (int w = 0; w < kPlanThreads / 64; ++w) total += wtok[w];
      total *= p.H;
      const long long per = (total + static_cast<long long>(p.grid) * kItemsPerWorkgroup - 1) /
                            (static_cast<long long>(p.grid) * kItemsPerWorkgroup);
      long long P = (per + p.bs - 1) / p.bs * p.bs;
      const int cap = kMaxAutoPartition / p.bs * p.bs;
      P = P > cap ? cap : P;
      sP = static_cast<int>(P < p.P ? p.P : P);
    }
  } else if (threadIdx.x == 0) {
    sP = p.P;
  }
  __syncthreads();
  const int P = sP * p.group;  // tokens per work item (header[2]; the merge's unit)
  const int top = (P >> 4) - 1 < kPlanBins - 1 ? (P >> 4) - 1 : kPlanBins - 1;
  auto bin_of = [&](int ntok) {
    const int units = (ntok + 15) >> 4;
    const int b = units > 0 ? units - 1 : 0;
    return b < top ? b : top;
  };
  for (int k = 0, i = threadIdx.x; i < p.S; ++k, i += kPlanThreads) {
    const int c = ctx_of(k, i);
    const int nfull = c / P, rem = c - nfull * P;
    if (nfull > 0) atomicAdd(&cnt[bin_of(P)], nfull);
    if (rem > 0 || c == 0) atomicAdd(&cnt[bin_of(rem)], 1);
  }
  __syncthreads();
  // off[b] = sum of cnt[b'] over b' > b: an exclusive scan in descending bin
  // order, thread t owning bin kPlanBins - 1 - t.
  static_assert(kPlanBins == kPlanThreads, "one bin per thread");
  const int bin = kPlanBins - 1 - threadIdx.x;
  const int val = cnt[bin];
  int x = val;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  off[bin] = before + x - val;
  if (threadIdx.x == kPlanThreads - 1) {
    p.header[0] = before + x;
    p.header[1] = p.first_taken;
    p.header[2] = P;
  }
  __syncthreads();
  // Each thread writes its sequence's first kDirect full items and its
  // partial one; the further full items of long sequences are written by the
  // whole workgroup, so that a few long contexts do not serialise the plan.
  constexpr int kDirect = 4;
  const int rounds = (p.S + kPlanThreads - 1) / kPlanThreads;
  for (int k = 0; k < rounds; ++k) {
    const int i = threadIdx.x + k * kPlanThreads;
    if (threadIdx.x == 0) nlong = 0;
    __syncthreads();
    if (i < p.S) {
      const int c = ctx_of(k, i);
      const int nfull = c / P, rem = c - nfull * P;
      const int np = nfull + (rem > 0 || c == 0 ? 1 : 0);
      if (nfull > 0) {
        const int base = atomicAdd(&off[bin_of(P)], nfull);
        const int direct = nfull < kDirect ? nfull : kDirect;
        for (int j = 0; j < direct; ++j) p.items[base + j] = make_int4(i, j, c, np);
        if (nfull > kDirect) {
          const int e = atomicAdd(&nlong, 1);
          longs[e] = make_int4(i, base, nfull, c);
          long_np[e] = np;
        }
      }
      if (rem > 0 || c == 0) p.items[atomicAdd(&off[bin_of(rem)], 1)] = make_int4(i, nfull, c, np);
    }
    __syncthreads();
    const int nl = nlong;
    for (int e = 0; e < nl; ++e) {
      const int4 L = longs[e];
      const int np = long_np[e];
      for (int j = kDirect + static_cast<int>(threadIdx.x); j < L.z; j += kPlanThreads)
        p.items[L.y + j] = make_int4(L.x, j, L.w, np);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Sharing plan: one workgroup, one sequence per thread.
//
// Sequences that share blocks (forked branches, cached prompt prefixes) hold
// the same block ids at the start of their tables ("Support for Prefix
// Sharing"; blocks are shared by reference count and only the storage is
// shared, "How it works").  The plan finds, for each group of sequences whose
// tables begin with the same block, the full blocks every member has in
// common with the group's lowest sequence (checked id by id), and cuts the
// group into subgroups of up to share_nmax members.  A subgroup's common
// prefix becomes work items of its own whose score tile holds the query heads
// of all its members, so those K/V tiles are read from HBM once for the
// subgroup; each member's remaining tokens are ordinary items.  The states of
// both kinds are combined by the merge kernel like any partitions.
//
// Records: (sequence, partition slot, first token, end token) for a
// sequence's own tokens, (~subgroup, slot, first, end) for a shared prefix.
// seq_np[i] is the number of states of sequence i; groups[g] its members.
// ---------------------------------------------------------------------------
constexpr int kShareMaxSeqs = kPlanThreads;  // batches up to this size are examined
constexpr int kShareHashBits = 11;
constexpr int kShareHash = 1 << kShareHashBits;  // open addressing at load factor <= 1/2
static_assert(kShareHash >= 2 * kShareMaxSeqs, "hash load factor");
static_assert(kShareHash >= kPlanBins, "the hash arrays hold the size bins afterwards");
constexpr int kMinSharedTokens = 256;  // shorter common prefixes are read per sequence
// Work items per workgroup that size the sharing plan's partitions (two
// workgroups per CU run its decode, so two items per CU).
#ifndef PA_SHARE_ITEMS_PER_WG
#define PA_SHARE_ITEMS_PER_WG 1
#endif
constexpr int kShareItemsPerWorkgroup = PA_SHARE_ITEMS_PER_WG;
constexpr int kCmpBatch = 8;           // comparison tasks whose loads a wave issues together
constexpr int kMaxCmpTasks = kShareHash;  // 64-entry comparison tasks checked per call

// Exclusive prefix sum of one value per thread in thread order; `total`
// receives the sum.  Ends with a barrier, so `wsum` can be reused at once.
__device__ __forceinline__ int block_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    const int s = wsum[w];
    before += w < wave ? s : 0;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

__device__ __forceinline__ void plan_share(const DecodeParams& p) {
  __shared__ int hk[kShareHash];          // first block ids (-1 = empty), then size bins
  __shared__ int hv[kShareHash];          // lowest sequence per first block, then bin offsets
  __shared__ int lead[kShareMaxSeqs];     // lowest sequence of each sequence's group
  __shared__ int gcount[kShareMaxSeqs];   // sequences beside the leader in its group
  __shared__ int cpre[kShareMaxSeqs];     // full blocks in common with the leader
  __shared__ int sbase[kShareMaxSeqs];    // first subgroup id of a leader's group
  __shared__ int mlist[kShareMaxSeqs];    // the non-leaders, in index order
  __shared__ int mcap[kShareMaxSeqs];     // blocks to compare for each of them
  __shared__ int tbase[kShareMaxSeqs];    // first comparison task of each of them
  __shared__ int sls[kShareMaxSeqs / 2];  // shared full blocks of each subgroup
  __shared__ int smem[kShareMaxSeqs / 2][kShareMaxMembers];
  __shared__ int wsum[kPlanThreads / 64];
  __shared__ long long wtok[kPlanThreads / 64];
  __shared__ int sP, sact;
  const int t = threadIdx.x, lane = t & 63, wave = rfl(t >> 6);
  const int bs = p.bs, nmax = p.share_nmax;
  const bool live = t < p.S;
  // the first table entry is read beside the length (every row has one)
  const int b0 = live ? p.tables[static_cast<size_t>(t) * p.max_blocks] : -1;
  const int c = live ? clamp_ctx(p, t) : 0;
  const int nfb = c / bs;  // full blocks
  const bool keyed = nfb > 0 && b0 >= 0 && b0 < p.N;
  int sid = -1, Ls = 0;  // subgroup, shared tokens
  bool head = false;     // first member of an active subgroup
  // Groups found on the host: used when made for this batch size and group
  // size (words 1 and 2), else found here.
  const bool from_host = p.host_plan != nullptr && p.host_plan[1] == p.S && p.host_plan[2] == nmax;
  if (from_host) {
    // Steps 1-4 done on the host from the block manager's tables: row t's
    // subgroup and shared tokens, each subgroup's members.  Every value is
    // clamped into range, so a plan that does not fit the batch gives wrong
    // attention but no access outside the buffers.
    const int32_t* hp = p.host_plan + 2;  // hp[1 + i] is word 3 + i
    const int nsub = p.S / 2;  // at most one subgroup per two rows
    for (int k = t; k < nsub; k += kPlanThreads) sls[k] = 0x7fffffff;
    __syncthreads();
    if (live) {
      const int s = hp[1 + t];
      sid = (s >= 0 && s < nsub) ? s : -1;
      if (sid >= 0) {
        const int lt = hp[1 + p.S + t];
        atomicMin(&sls[sid], lt > 0 ? min(lt / bs, nfb) : 0);
      }
    }
    __syncthreads();
    if (sid >= 0 && sls[sid] * bs >= kMinSharedTokens) {
      Ls = sls[sid] * bs;
      const int32_t* mem = hp + 1 + 2 * static_cast<size_t>(p.S) + 4 * static_cast<size_t>(sid);
      head = mem[0] == t;
      if (head) {
        // at most nmax members, so that their query heads fit the score tile
        smem[sid][0] = t;
#pragma unroll
        for (int m = 1; m < kShareMaxMembers; ++m)
          smem[sid][m] = (m < nmax && mem[m] >= 0 && mem[m] < p.S) ? mem[m] : -1;
      }
    }
  } else {
    for (int k = t; k < kShareHash; k += kPlanThreads) {
      hk[k] = -1;
      hv[k] = 0x7fffffff;
    }
    gcount[t] = 0;
    cpre[t] = nfb;
    __syncthreads();

    // 1. Groups: sequences whose first block is the same physical block.
    int slot = 0;
    if (keyed) {
      uint32_t hh = (static_cast<uint32_t>(b0) * 2654435761u) >> (32 - kShareHashBits);
      for (;;) {  // ends: at most kShareMaxSeqs keys in kShareHash slots
        const int old = atomicCAS(&hk[hh], -1, b0);
        if (old == -1 || old == b0) break;
        hh = (hh + 1) & (kShareHash - 1);
      }
      slot = static_cast<int>(hh);
      atomicMin(&hv[slot], t);
    }
    __syncthreads();
    const int L = keyed ? hv[slot] : t;
    lead[t] = L;
    if (L != t) atomicAdd(&gcount[L], 1);
    __syncthreads();

    // 2. Rank in the group by sequence index; subgroups of nmax consecutive
    //    ranks (a lone last member stays on its own).
    int rank = 0;
    if (L != t) {
      rank = 1;
      for (int j = L + 1; j < t; ++j) rank += lead[j] == L ? 1 : 0;
    }
    const int gn = live ? gcount[L] + 1 : 0;
    const int gsub = gn >= 2 ? gn / nmax + (gn % nmax >= 2 ? 1 : 0) : 0;
    // one scan for both: subgroups per leader (low 16 bits), members (high)
    const bool member = live && L != t;
    int both = 0;
    const int sc = block_scan((L == t ? gsub : 0) | (member ? 1 << 16 : 0), wsum, both);
    const int nsub_total = both & 0xffff, nmem = both >> 16;
    sbase[t] = sc & 0xffff;
    if (member) mlist[sc >> 16] = t;
    for (int k = t; k < nsub_total; k += kPlanThreads) {
      sls[k] = 0x7fffffff;
#pragma unroll
      for (int m = 0; m < kShareMaxMembers; ++m) smem[k][m] = -1;
    }
    __syncthreads();
    const int sub = rank / nmax;
    sid = (live && sub < gsub) ? sbase[L] + sub : -1;
    if (sid >= 0) smem[sid][rank - sub * nmax] = t;

    // 3. Each non-leader's table against its leader's, over the full blocks
    //    both hold: tasks of 64 entries (one per lane), each task's member
    //    found in an owner array (the hash arrays are free now), the loads of
    //    kCmpBatch tasks per wave issued together.  At most kMaxCmpTasks tasks
    //    are checked; a member whose tasks lie beyond shares only what was
    //    checked.
    int ntk = 0, cap = 0;
    if (t < nmem) {
      const int m = mlist[t];
      cap = min(cpre[m], cpre[lead[m]]);
      ntk = (cap + 63) / 64;
    }
    int ntask = 0;
    const int tb = block_scan(ntk, wsum, ntask);
    int* towner = hk;
    if (t < nmem) {
      const int e = min(tb + ntk, kMaxCmpTasks);
      for (int k = tb; k < e; ++k) towner[k] = t;
      cap = min(cap, max(e - tb, 0) * 64);
      mcap[t] = cap;
      tbase[t] = tb;
      cpre[mlist[t]] = cap;
    }
    __syncthreads();
    ntask = min(ntask, kMaxCmpTasks);
    constexpr int kWavesPlan = kPlanThreads / 64;
    for (int base = wave; base < ntask; base += kWavesPlan * kCmpBatch) {
      // Lane r < kCmpBatch looks up task base + r * kWavesPlan (three LDS round
      // trips for the whole batch); the values are then broadcast by readlane.
      const int mtk = base + (lane % kCmpBatch) * kWavesPlan;
      const int own = towner[mtk < ntask ? mtk : 0];
      const int mm = mlist[own];
      const int ml = lead[mm];
      const int mcp = mtk < ntask ? mcap[own] : 0;
      const int mk0 = (mtk - tbase[own]) * 64;
      int tm[kCmpBatch], tk0[kCmpBatch], tcap[kCmpBatch], va[kCmpBatch], vb[kCmpBatch];
#pragma unroll
      for (int r = 0; r < kCmpBatch; ++r) {
        tm[r] = __builtin_amdgcn_readlane(mm, r);
        tk0[r] = __builtin_amdgcn_readlane(mk0, r);
        tcap[r] = __builtin_amdgcn_readlane(mcp, r);
        const int tl = __builtin_amdgcn_readlane(ml, r);
        const int k = tk0[r] + lane;
        const int kk = k < tcap[r] ? k : 0;  // tcap <= both rows' full blocks <= max_blocks
        va[r] = p.tables[static_cast<size_t>(tm[r]) * p.max_blocks + kk];
        vb[r] = p.tables[static_cast<size_t>(tl) * p.max_blocks + kk];
      }
#pragma unroll
      for (int r = 0; r < kCmpBatch; ++r) {
        const uint64_t bad = __builtin_amdgcn_ballot_w64(tk0[r] + lane < tcap[r] && va[r] != vb[r]);
        if (lane == 0 && bad != 0) atomicMin(&cpre[tm[r]], tk0[r] + static_cast<int>(__builtin_ctzll(bad)));
      }
    }
    __syncthreads();

    // 4. A subgroup shares the full blocks all its members hold in common with
    //    the leader (the leader's own full blocks when it is a member).
    if (sid >= 0) atomicMin(&sls[sid], cpre[t]);
    __syncthreads();
    if (sid >= 0 && sls[sid] * bs >= kMinSharedTokens) {
      Ls = sls[sid] * bs;
      head = rank == sub * nmax;
    }
  }

  // 5. Partition size from the work that remains: each sequence's own
  //    tokens once and each shared prefix once.
  long long tok = live ? c - Ls : 0;
  if (head) tok += Ls;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tok += __shfl_xor(tok, o);
  if (lane == 0) wtok[wave] = tok;
  __syncthreads();
  if (wave == 0) {
    long long total = lane < kPlanThreads / 64 ? wtok[lane] : 0;
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) total += __shfl_xor(total, o);
    total *= p.H;
    // 32-bit arithmetic once the cap is known not to apply
    const int cap_p = kMaxAutoPartition / bs * bs;
    const int slots = p.grid * kShareItemsPerWorkgroup;
    int P = cap_p;
    if (total <= static_cast<long long>(slots) * cap_p) {
      const int per = (static_cast<int>(total) + slots - 1) / slots;
      P = (per + bs - 1) / bs * bs;
      P = P > cap_p ? cap_p : P;
    }
    if (lane == 0) sP = P < p.P ? p.P : P;
  }
  int* cnt = hk;  // the hash is no longer read
  int* off = hv;
  for (int b = t; b < kPlanBins; b += kPlanThreads) cnt[b] = 0;
  if (t == 0) sact = 0;
  __syncthreads();
  const int P = sP;
  const int top = (P >> 4) - 1 < kPlanBins - 1 ? (P >> 4) - 1 : kPlanBins - 1;
  auto bin_of = [&](int ntok) {
    const int units = (ntok + 15) >> 4;
    const int b = units > 0 ? units - 1 : 0;
    return b < top ? b : top;
  };

  // 6. Items: the sequence's own tokens [Ls, c) in P-token pieces (an empty
  //    context still gets one item, which writes zeros), and for a
  //    subgroup's first member the shared prefix [0, Ls).
  const int tail = c - Ls;
  const int nsh = Ls > 0 ? (Ls + P - 1) / P : 0;
  const int tfull = tail / P, trem = tail - tfull * P;
  const bool tlast = trem > 0 || (live && c == 0);
  if (live) p.seq_np[t] = nsh + tfull + (tlast ? 1 : 0);
  const int sfull = head ? Ls / P : 0, srem = head ? Ls - sfull * P : 0;
  if (tfull + sfull > 0) atomicAdd(&cnt[bin_of(P)], tfull + sfull);
  if (tlast) atomicAdd(&cnt[bin_of(trem)], 1);
  if (srem > 0) atomicAdd(&cnt[bin_of(srem)], 1);
  if (head) atomicAdd(&sact, 1);
  __syncthreads();
  // bin offsets in descending size order: thread t owns bin kPlanBins - 1 - t
  static_assert(kPlanBins == kPlanThreads, "one bin per thread");
  const int bin = kPlanBins - 1 - t;
  int nitems = 0;
  const int o = block_scan(cnt[bin], wsum, nitems);
  const int nactive = sact;
  off[bin] = o;
  if (t == 0) {
    p.header[0] = nitems;
    p.header[1] = p.first_taken;
    p.header[2] = P;
    p.header[3] = nactive;
  }
  __syncthreads();
  if (tfull > 0) {
    const int base = atomicAdd(&off[bin_of(P)], tfull);
    for (int j = 0; j < tfull; ++j) p.items[base + j] = make_int4(t, nsh + j, Ls + j * P, Ls + (j + 1) * P);
  }
  if (tlast) p.items[atomicAdd(&off[bin_of(trem)], 1)] = make_int4(t, nsh + tfull, Ls + tfull * P, c);
  if (head) {
    p.groups[sid] = make_int4(smem[sid][0], smem[sid][1], smem[sid][2], smem[sid][3]);
    if (sfull > 0) {
      const int base = atomicAdd(&off[bin_of(P)], sfull);
      for (int j = 0; j < sfull; ++j) p.items[base + j] = make_int4(~sid, j, j * P, (j + 1) * P);
    }
    if (srem > 0) p.items[atomicAdd(&off[bin_of(srem)], 1)] = make_int4(~sid, sfull, sfull * P, Ls);
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(DecodeParams p) { plan_plain(p); }

__global__ __launch_bounds__(kPlanThreads) void plan_share_kernel(DecodeParams p) { plan_share(p); }

// Prologue of pa_decode_step: workgroup 0 plans the decode while the others
// write the new tokens' K/V (one wave per group of four tokens and kv head,
// as the write kernel does).  The plan reads no K/V, so the two are
// independent; the decode kernel that follows sees both.
// Write tasks per prologue workgroup: the others of its 16 waves exit at
// once, so the write spreads over many CUs.  Measured on MI355X (cfg3 step,
// 256 new tokens x 8 kv heads): 16 tasks per workgroup 250.3 us per step, 4
// tasks 247.9, 2 tasks 247.8, 1 task 247.5.
#ifndef PA_PROLOGUE_WRITE_WAVES
#define PA_PROLOGUE_WRITE_WAVES 2
#endif
constexpr int kWriteWaves = PA_PROLOGUE_WRITE_WAVES;

template <int kBytes, int D, bool kShare>
__global__ __launch_bounds__(kPlanThreads) void prologue_kernel(DecodeParams p) {
  if (blockIdx.x == 0) {
    if constexpr (kShare) plan_share(p);
    else plan_plain(p);
    return;
  }
  if (static_cast<int>(threadIdx.x >> 6) >= kWriteWaves) return;
  const int task = (blockIdx.x - 1) * kWriteWaves + static_cast<int>(threadIdx.x >> 6);
  const int groups = (p.w_tokens + 3) / 4;
  if (task >= groups * p.H) return;
  char* base = static_cast<char*>(const_cast<void*>(p.pool)) + p.layer_off * kBytes;
  write_token_group<kBytes>(static_cast<const uint4*>(p.w_k), static_cast<const uint4*>(p.w_v), p.w_slots,
                            p.w_tokens, base, p.N, p.H, p.bs, D, task / p.H, task % p.H, threadIdx.x & 63);
}

// Plan of a decode call, with the new tokens' write beside it when the call
// carries one (pa_decode_step).
template <int kBytes, int D, bool kShare>
hipError_t launch_plan(const DecodeParams& p, hipStream_t stream) {
  if (p.w_tokens > 0) {
    const int64_t tasks = static_cast<int64_t>((p.w_tokens + 3) / 4) * p.H;
    const int64_t blocks = 1 + (tasks + kWriteWaves - 1) / kWriteWaves;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prologue_kernel<kBytes, D, kShare>), dim3(static_cast<unsigned>(blocks)), dim3(kPlanThreads),
                       0, stream, p);
  } else if constexpr (kShare) {
    hipLaunchKernelGGL(plan_share_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MFMA path: 3 <= G <= 16 query heads per kv head (GM = G rounded up to 4, 8
// or 16 sizes the LDS merge).
// ---------------------------------------------------------------------------
template <typename T, int D, int GM>
struct MfmaPath {
  static constexpr int kBytes = T::kBytes;
  static constexpr int E = 16 / kBytes;
  static constexpr int NCH = D / (4 * E);  // 16-byte chunks per lane per sub-tile
  static constexpr int NT = D / 16;        // 16-wide head_dim tiles of the output
  using Smem = MergeSmem<D, GM>;

  // Query rows as the B operand of S = K.Q^T: lane holds head `col`, the
  // head_dim entries matching its K chunk entries.
  struct Q {
    uint4 b[NCH];
  };
  struct State {
    f32x4_t acc[NT];
    float m_col, l_part;
  };

  __device__ static void load_q(Q& q, const DecodeParams& p, const Item& it, int lane) {
    const int col = lane & 15, grp = lane >> 4;
    const int G = p.G;
    const char* qbase = static_cast<const char*>(p.q) +
                        (static_cast<size_t>(it.i) * p.Hq + static_cast<size_t>(it.h) * G + col) * D * kBytes;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      q.b[c] = (col < G) ? *reinterpret_cast<const uint4*>(qbase + ((c * 4 + grp) * E) * kBytes)
                         : make_uint4(0, 0, 0, 0);
  }

  // Sharing plan: column col is query head col % G of member col / G.
  __device__ static void load_q_members(Q& q, const DecodeParams& p, const Item& it, int4 mem, int lane) {
    const int col = lane & 15, grp = lane >> 4;
    const int G = p.G;
    const int m = col / G, g = col - m * G;
    const int seq = m == 0 ? mem.x : m == 1 ? mem.y : m == 2 ? mem.z : mem.w;
    const bool live = col < it.cols;
    const char* qbase = static_cast<const char*>(p.q) +
                        (static_cast<size_t>(live ? seq : 0) * p.Hq + static_cast<size_t>(it.h) * G + g) * D * kBytes;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      q.b[c] = live ? *reinterpret_cast<const uint4*>(qbase + ((c * 4 + grp) * E) * kBytes)
                    : make_uint4(0, 0, 0, 0);
  }

  __device__ static void reset(State& s) {
#pragma unroll
    for (int t = 0; t < NT; ++t) s.acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    s.m_col = kNegInf;
    s.l_part = 0.f;
  }

  __device__ static void compute(State& st, const Q& q, Frag<NCH>& f, int valid, int lane, float sl2) {
    const int grp = lane >> 4;
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kBytes == 2) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) s = mfma_k32<T>(f.k[c], q.b[c], s);
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        s = mfma_f32_k4(__uint_as_float(f.k[c].x), __uint_as_float(q.b[c].x), s);
        s = mfma_f32_k4(__uint_as_float(f.k[c].y), __uint_as_float(q.b[c].y), s);
        s = mfma_f32_k4(__uint_as_float(f.k[c].z), __uint_as_float(q.b[c].z), s);
        s = mfma_f32_k4(__uint_as_float(f.k[c].w), __uint_as_float(q.b[c].w), s);
      }
    }
    // s[r] = score of token 4*grp + r for query head col (log2 units).
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = (4 * grp + r < valid) ? s[r] * sl2 : kNegInf;
    const float mloc = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    if (wave_any(mloc > st.m_col + kRescaleLog2)) {
      float mx = fmaxf(mloc, __shfl_xor(mloc, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(st.m_col, mx);
      const float alpha = fast_exp2(st.m_col - m_new);
      st.m_col = m_new;
      st.l_part *= alpha;
      // Output rows 4*grp + r belong to query heads whose alpha sits in lane 4*grp + r.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = __shfl(alpha, 4 * grp + r);
#pragma unroll
        for (int t = 0; t < NT; ++t) st.acc[t][r] *= a;
      }
    }
    float pr[4];
    uint32_t pbits[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = sv[r] == kNegInf ? 0.f : fast_exp2(sv[r] - st.m_col);
      if constexpr (kBytes == 2) {
        pbits[r] = to_storage<T>(e);
        pr[r] = from_storage<T>(pbits[r]);
      } else {
        pr[r] = e;
      }
    }
    st.l_part += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    if (valid < 16) mask_v_tail<kBytes, NCH>(f, grp, valid);
    if constexpr (kBytes == 2) {
      const uint2 pa = make_uint2(pbits[0] | (pbits[1] << 16), pbits[2] | (pbits[3] << 16));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint4 vc = f.v[t >> 1];
        const uint2 vb = (t & 1) ? make_uint2(vc.z, vc.w) : make_uint2(vc.x, vc.y);
        st.acc[t] = mfma_k16<T>(pa, vb, st.acc[t]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        st.acc[t] = mfma_f32_k4(pr[0], __uint_as_float(f.v[t].x), st.acc[t]);
        st.acc[t] = mfma_f32_k4(pr[1], __uint_as_float(f.v[t].y), st.acc[t]);
        st.acc[t] = mfma_f32_k4(pr[2], __uint_as_float(f.v[t].z), st.acc[t]);
        st.acc[t] = mfma_f32_k4(pr[3], __uint_as_float(f.v[t].w), st.acc[t]);
      }
    }
  }

  // This wave's (max, sum, weighted V) per query head into LDS.
  __device__ static void to_lds(const State& st, Smem& sm, int wave, int lane, int G) {
    const int col = lane & 15, grp = lane >> 4;
    // Column sums over the four lane groups.
    float l_col = st.l_part + __shfl_xor(st.l_part, 16);
    l_col += __shfl_xor(l_col, 32);
    if (lane < GM) {  // lane = query-head column
      sm.m[wave][lane] = st.m_col;
      sm.l[wave][lane] = l_col;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * grp + r;
      if (g < GM && g < G) {
#pragma unroll
        for (int t = 0; t < NT; ++t) sm.o[wave][g][t * 16 + col] = st.acc[t][r];
      }
    }
  }
};

// ---------------------------------------------------------------------------
// VALU path: NG (1 or 2) query heads per kv head.
// ---------------------------------------------------------------------------
template <typename T, int D, int NG>
struct ValuPath {
  static constexpr int kBytes = T::kBytes;
  static constexpr int E = 16 / kBytes;
  static constexpr int NCH = D / (4 * E);
  static constexpr int R = E / 4;    // 16-wide d tiles per V chunk
  static constexpr int NT = D / 16;  // d values per lane in P.V (d = t*16 + col)
  using Smem = MergeSmem<D, NG>;

  // q entries matching this lane's K chunk entries: d = (c*4 + grp)*E + e.
  struct Q {
    uint4 v[NG][NCH];
  };
  struct State {
    float acc[NG][NT];
    float m_run[NG], l_run[NG];
  };

  __device__ static void load_q(Q& q, const DecodeParams& p, const Item& it, int lane) {
    const int grp = lane >> 4;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const char* qrow = static_cast<const char*>(p.q) +
                         (static_cast<size_t>(it.i) * p.Hq + static_cast<size_t>(it.h) * NG + g) * D * kBytes;
#pragma unroll
      for (int c = 0; c < NCH; ++c) q.v[g][c] = *reinterpret_cast<const uint4*>(qrow + ((c * 4 + grp) * E) * kBytes);
    }
  }

  __device__ static void reset(State& s) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      s.m_run[g] = kNegInf;
      s.l_run[g] = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) s.acc[g][t] = 0.f;
    }
  }

  __device__ static void compute(State& st, const Q& q, Frag<NCH>& f, int valid, int lane, float sl2) {
    const int col = lane & 15, grp = lane >> 4;
    if (valid < 16) mask_v_tail<kBytes, NCH>(f, grp, valid);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      // Partial dot over this lane's head_dim entries of token `col`.
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if constexpr (kBytes == 2) {
          dot = dot2<T>(f.k[c].x, q.v[g][c].x, dot);
          dot = dot2<T>(f.k[c].y, q.v[g][c].y, dot);
          dot = dot2<T>(f.k[c].z, q.v[g][c].z, dot);
          dot = dot2<T>(f.k[c].w, q.v[g][c].w, dot);
        } else {
          dot = fmaf(__uint_as_float(f.k[c].x), __uint_as_float(q.v[g][c].x), dot);
          dot = fmaf(__uint_as_float(f.k[c].y), __uint_as_float(q.v[g][c].y), dot);
          dot = fmaf(__uint_as_float(f.k[c].z), __uint_as_float(q.v[g][c].z), dot);
          dot = fmaf(__uint_as_float(f.k[c].w), __uint_as_float(q.v[g][c].w), dot);
        }
      }
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      const float s = (col < valid) ? dot * sl2 : kNegInf;
      if (wave_any(s > st.m_run[g] + kRescaleLog2)) {
        float mx = fmaxf(s, __shfl_xor(s, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        mx = fmaxf(mx, __shfl_xor(mx, 4));
        mx = fmaxf(mx, __shfl_xor(mx, 8));
        const float m_new = fmaxf(st.m_run[g], mx);
        const float alpha = fast_exp2(st.m_run[g] - m_new);
        st.m_run[g] = m_new;
        st.l_run[g] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) st.acc[g][t] *= alpha;
      }
      const float e = s == kNegInf ? 0.f : fast_exp2(s - st.m_run[g]);
      uint32_t pb;
      float pr;
      if constexpr (kBytes == 2) {
        pb = to_storage<T>(e);
        pr = from_storage<T>(pb);
      } else {
        pb = __float_as_uint(e);
        pr = e;
      }
      st.l_run[g] += pr;  // token `col`'s weight; summed over lanes at the end
      // Weights of tokens 4*grp .. 4*grp+3, the tokens this lane's V entries hold.
      const uint32_t w0 = __shfl(pb, 4 * grp + 0), w1 = __shfl(pb, 4 * grp + 1);
      const uint32_t w2 = __shfl(pb, 4 * grp + 2), w3 = __shfl(pb, 4 * grp + 3);
      if constexpr (kBytes == 2) {
        const uint32_t p01 = w0 | (w1 << 16), p23 = w2 | (w3 << 16);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          // chunk c holds d tiles c*R + 0 (dwords x, y) and c*R + 1 (z, w)
          st.acc[g][c * R + 0] = dot2<T>(f.v[c].x, p01, st.acc[g][c * R + 0]);
          st.acc[g][c * R + 0] = dot2<T>(f.v[c].y, p23, st.acc[g][c * R + 0]);
          st.acc[g][c * R + 1] = dot2<T>(f.v[c].z, p01, st.acc[g][c * R + 1]);
          st.acc[g][c * R + 1] = dot2<T>(f.v[c].w, p23, st.acc[g][c * R + 1]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          float a = st.acc[g][c];
          a = fmaf(__uint_as_float(w0), __uint_as_float(f.v[c].x), a);
          a = fmaf(__uint_as_float(w1), __uint_as_float(f.v[c].y), a);
          a = fmaf(__uint_as_float(w2), __uint_as_float(f.v[c].z), a);
          a = fmaf(__uint_as_float(w3), __uint_as_float(f.v[c].w), a);
          st.acc[g][c] = a;
        }
      }
    }
  }

  __device__ static void to_lds(State& st, Smem& sm, int wave, int lane, int) {
    const int col = lane & 15;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float l = st.l_run[g];
      l += __shfl_xor(l, 1);
      l += __shfl_xor(l, 2);
      l += __shfl_xor(l, 4);
      l += __shfl_xor(l, 8);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float a = st.acc[g][t];
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 32);
        st.acc[g][t] = a;
      }
      if (lane < 16) {
        if (lane == 0) {
          sm.m[wave][g] = st.m_run[g];
          sm.l[wave][g] = l;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) sm.o[wave][g][t * 16 + col] = st.acc[g][t];
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Persistent decode kernel, in two schedules.
//
// Deep (kDeep = true), for many small items (an explicit small partition
// size): work indices run two ahead of the item being computed.  Timeline of
// one workgroup for item k:
//   - thread 0 fetches the index of item k+2 from the counter;
//   - every wave reads item k+1's record (a scalar load through the
//     __restrict__ items argument, which does not disturb the vector-load
//     waits), then loads item k+1's query rows and this wave's block ids;
//   - the waves stream and compute item k's units;
//   - thread 0 posts item k+2's index; the waves issue item k+1's first units;
//   - the four wave states of item k are merged through LDS and written while
//     those loads are in flight.
// Shallow (kDeep = false), for the few long items of an automatic partition
// size: one index ahead, so the last items of the queue stay free for
// whichever workgroup finishes first (measured: holding two indices per
// workgroup costs more in the tail than it saves between items there).
// ---------------------------------------------------------------------------
template <typename Path, typename T, int D, bool kDeep, bool kShare, bool kFlat = false>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p, const int4* __restrict__ items,
                                                          const int4* __restrict__ groups,
                                                          const int32_t* __restrict__ seq_np) {
  constexpr int kBytes = T::kBytes;
  constexpr int NCH = Path::NCH;
  constexpr int PF = kPrefetch;
  using Smem = typename Path::Smem;
  __shared__ Smem sm;
  const int lane = threadIdx.x & 63;
  const int wave = rfl(threadIdx.x >> 6);
  const int H = p.H;
  const bool direct = p.direct != 0;
  const int P = direct ? p.P : rfl(p.header[2]);
  const int total = direct ? p.S * H : rfl(p.header[0]) * H;
  const float sl2 = p.scale_log2;
  // Item record of work index w: from the plan's list, or (direct launch:
  // every context within one partition) the sequence itself.
  auto record = [&](int w) {
    if (!direct) return items[w / H];
    const int i = w / H;
    return make_int4(i, 0, rfl(clamp_ctx(p, i)), 1);
  };

  // The first index (two in the deep schedule) comes from the workgroup id;
  // the plan kernel starts the counter past them.  A direct launch has one
  // index per workgroup and never touches the counter.
  int cur = blockIdx.x;
  int nxt = kDeep ? static_cast<int>(blockIdx.x + gridDim.x) : 0;
  if (cur >= total) return;

  const int group = p.group;
  auto item_at = [&](int w) {
    if constexpr (kShare) return make_item_share(p, record(w), w % H, wave, groups);
    else return make_item(p, record(w), w % H, P, group, wave);
  };
  auto load_q = [&](typename Path::Q& qq, const Item& ii) {
    if constexpr (kShare) Path::load_q_members(qq, p, ii, item_members(ii, groups), lane);
    else Path::load_q(qq, p, ii, lane);
  };
  Item it = item_at(cur);
  typename Path::Q q;
  load_q(q, it);
  UnitStream<D, kBytes, kFlat> st;
  Frag<NCH> f[PF + 1];
  bool ok[PF + 1];
  st.begin(p, it.trow, it.start, it.u0, it.h);
  st.ids = st.fetch_ids(lane);
  prologue<PF, NCH>(st, f, ok, lane);

  auto run_item = [&](typename Path::State& s) {
    Path::reset(s);
    stream_item<PF, NCH>(p, st, f, ok, it, lane, [&](Frag<NCH>& fr, int u, bool okk) {
      // A unit whose block id is invalid counts as having no valid token (its
      // registers are still consumed, which keeps the load waits exact).
      const int valid = !okk ? 0 : it.ntok - u * 16 < 16 ? it.ntok - u * 16 : 16;
      Path::compute(s, q, fr, valid, lane, sl2);
    });
  };

  for (int k = 0;; ++k) {
    int nn = total;
    if (threadIdx.x == 0 && !direct) nn = atomicAdd(&p.header[1], 1);
    if constexpr (kDeep) {
      // The next item (the current one again after the last: the loads below
      // are then harmless repeats, and always issuing them keeps the waits in
      // the stream exact).
      const bool has_next = nxt < total;
      const Item nit = item_at(has_next ? nxt : cur);
      typename Path::Q qn;
      load_q(qn, nit);
      int32_t ids_n;
      {
        const int kk = (nit.start + nit.u0 * 16) / p.bs + lane;
        ids_n = kk < p.max_blocks ? nit.trow[kk] : -1;
      }
      typename Path::State s;
      run_item(s);
      if (threadIdx.x == 0) sm.slot[k & 1] = nn;
      // The next item's first units go out before this item's merge.  After
      // the last item every id reads as invalid, so these loads all hit block
      // 0 (a cached address); issuing them regardless keeps the waits exact.
      st.begin(p, nit.trow, nit.start, nit.u0, nit.h);
      st.ids = has_next ? ids_n : -1;
      prologue<PF, NCH>(st, f, ok, lane);
      Path::to_lds(s, sm, wave, lane, it.cols);
      finish_partition<T, D, Smem::kRows, kShare>(p, sm, it, groups, seq_np);
      __syncthreads();
      if (!has_next) break;
      cur = nxt;
      nxt = rfl(sm.slot[k & 1]);
      it = nit;
      q = qn;
    } else {
      typename Path::State s;
      run_item(s);
      if (threadIdx.x == 0) sm.slot[k & 1] = nn;
      Path::to_lds(s, sm, wave, lane, it.cols);
      finish_partition<T, D, Smem::kRows, kShare>(p, sm, it, groups, seq_np);
      __syncthreads();
      cur = rfl(sm.slot[k & 1]);
      if (cur >= total) break;
      it = item_at(cur);
      load_q(q, it);
      st.begin(p, it.trow, it.start, it.u0, it.h);
      st.ids = st.fetch_ids(lane);
      prologue<PF, NCH>(st, f, ok, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partition states: one wave per (sequence, query head).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (pair >= p.S * p.Hq) return;
  // Partition states of this row: from the sharing plan's count, or one per
  // P tokens of the context.  A row with one state was written directly.
  int np;
  if (p.share) {
    np = rfl(p.seq_np[pair / p.Hq]);
  } else {
    const int P = rfl(p.header[2]);
    const int ctx = rfl(clamp_ctx(p, pair / p.Hq));
    np = (ctx + P - 1) / P;
  }
  if (np <= 1) return;
  np = np > p.ws_stride ? p.ws_stride : np;
  const size_t e0 = static_cast<size_t>(pair) * p.ws_stride;
  const float* ml = p.ws_ml + 2 * e0;

  constexpr int PER = D / 64;  // head_dim entries per lane
  // Eight partitions' rows per step, their loads issued together; the first
  // eight go out with the (m, l) pairs.
  float orow[8][PER];
  auto load_rows = [&](int c0, int t, int n) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = t + u < n ? t + u : n - 1;
      const float* src = p.ws_o + (e0 + c0 + r) * D + lane;
#pragma unroll
      for (int k = 0; k < PER; ++k) orow[u][k] = src[64 * k];
    }
  };
  load_rows(0, 0, np < 64 ? np : 64);

  // Partition states are held one per lane, 64 partitions at a time.
  float M = kNegInf;
  for (int c0 = 0; c0 < np; c0 += 64)
    if (c0 + lane < np) M = fmaxf(M, ml[2 * (c0 + lane)]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));

  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float L = 0.f;
  for (int c0 = 0; c0 < np; c0 += 64) {
    const int jj = c0 + lane;
    const float mj = jj < np ? ml[2 * jj] : kNegInf;
    const float wj = (mj == kNegInf) ? 0.f : ml[2 * jj + 1] * fast_exp2(mj - M);
    L += wj;
    const int n = np - c0 < 64 ? np - c0 : 64;
    for (int t = 0; t < n; t += 8) {
      if (c0 + t > 0) load_rows(c0, t, n);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = t + u < n ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                         __builtin_bit_cast(int, wj), t + u))
                                  : 0.f;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = fmaf(w, orow[u][k], acc[k]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  using B = typename T::bits;
  B* out = static_cast<B*>(p.out);
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k)
    out[static_cast<size_t>(pair) * D + lane + 64 * k] = static_cast<B>(to_storage<T>(acc[k] * inv));
}

// Merge for contexts of many partitions: a workgroup of four waves per
// (sequence, query head).  Wave w merges a contiguous quarter of the
// partitions against its own maximum, loading eight partitions' rows at a
// time (D / 64 consecutive floats per lane); the four results are then
// combined through LDS with the same log-sum-exp weights.
template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_wide_kernel(DecodeParams p) {
  constexpr int VEC = D / 64;  // consecutive head_dim entries per lane
  __shared__ float s_m[kMergeWaves], s_l[kMergeWaves];
  __shared__ float s_o[kMergeWaves][D];
  const int lane = threadIdx.x & 63;
  const int wave = rfl(threadIdx.x >> 6);
  const int pair = blockIdx.x;
  const int P = rfl(p.header[2]);
  const int ctx = rfl(clamp_ctx(p, pair / p.Hq));
  if (ctx <= P) return;  // written directly by the partition kernel
  int np = (ctx + P - 1) / P;
  np = np > p.ws_stride ? p.ws_stride : np;
  const int per = (np + kMergeWaves - 1) / kMergeWaves;
  const int j0 = wave * per;
  const int j1 = j0 + per < np ? j0 + per : np;
  const size_t e0 = static_cast<size_t>(pair) * p.ws_stride;
  const float* ml = p.ws_ml + 2 * e0;

  // Rows eight at a time, the first eight requested with the (m, l) pairs.
  // A wave with no partitions (j0 >= j1) loads nothing.
  float orow[8][VEC];
  auto load_rows = [&](int c0, int t, int n) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = t + u < n ? t + u : n - 1;
      const float* src = p.ws_o + (e0 + c0 + r) * D + VEC * lane;
      if constexpr (VEC == 2) {
        const float2 x = *reinterpret_cast<const float2*>(src);
        orow[u][0] = x.x;
        orow[u][1] = x.y;
      } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) orow[u][k] = src[k];
      }
    }
  };
  if (j0 < j1) load_rows(j0, 0, j1 - j0 < 64 ? j1 - j0 : 64);
  float M = kNegInf;
  for (int c0 = j0; c0 < j1; c0 += 64)
    if (c0 + lane < j1) M = fmaxf(M, ml[2 * (c0 + lane)]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float acc[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) acc[k] = 0.f;
  float L = 0.f;
  for (int c0 = j0; c0 < j1; c0 += 64) {
    const int jj = c0 + lane;
    const float mj = jj < j1 ? ml[2 * jj] : kNegInf;
    const float wj = (mj == kNegInf) ? 0.f : ml[2 * jj + 1] * fast_exp2(mj - M);
    L += wj;
    const int n = j1 - c0 < 64 ? j1 - c0 : 64;
    for (int t = 0; t < n; t += 8) {
      if (c0 + t > j0) load_rows(c0, t, n);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = t + u < n ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                         __builtin_bit_cast(int, wj), t + u))
                                  : 0.f;
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[k] = fmaf(w, orow[u][k], acc[k]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  if (lane == 0) {
    s_m[wave] = M;
    s_l[wave] = L;
  }
#pragma unroll
  for (int k = 0; k < VEC; ++k) s_o[wave][VEC * lane + k] = acc[k];
  __syncthreads();
  if (wave != 0) return;
  float Mt = s_m[0];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) Mt = fmaxf(Mt, s_m[w]);
  float Lt = 0.f, o[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) o[k] = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    const float f = s_m[w] == kNegInf ? 0.f : fast_exp2(s_m[w] - Mt);
    Lt += f * s_l[w];
#pragma unroll
    for (int k = 0; k < VEC; ++k) o[k] += f * s_o[w][VEC * lane + k];
  }
  using B = typename T::bits;
  B* out = static_cast<B*>(p.out);
  const float inv = (Lt > 0.f) ? 1.f / Lt : 0.f;
#pragma unroll
  for (int k = 0; k < VEC; ++k)
    out[static_cast<size_t>(pair) * D + VEC * lane + k] = static_cast<B>(to_storage<T>(o[k] * inv));
}

// Persistent grid: kWorkgroupsPerCU workgroups per CU (never more than the
// kernel's occupancy allows), cached per device.
int persistent_grid(const void* kernel, int wg_per_cu = kWorkgroupsPerCU) {
  static std::mutex mu;
  static struct {
    const void* k;
    int dev, cap, grid;
  } cache[64];
  static int n = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int c = 0; c < n; ++c)
    if (cache[c].k == kernel && cache[c].dev == dev && cache[c].cap == wg_per_cu) return cache[c].grid;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, 0) != hipSuccess) return 0;
  const int per_cu = occ > 0 && occ < wg_per_cu ? occ : wg_per_cu;
  const int grid = (cus > 0 ? cus : 1) * per_cu;
  if (n < 64) cache[n++] = {kernel, dev, wg_per_cu, grid};
  return grid;
}

// Items per workgroup from which the deep schedule pays (an upper bound
// from the host's view: every sequence at the maximum context length).
constexpr int kDeepItemsPerWorkgroup = 16;
// Largest partition that a single wave streams alone in grouped items.
constexpr int kMaxGroupedPartition = 1024;

template <typename Path, typename T, int D>
hipError_t launch_decode_kernel(DecodeParams p, hipStream_t stream) {
  const int64_t work_bound = static_cast<int64_t>(p.S) * p.max_parts * p.H;
  const void* k_shallow = p.flat ? reinterpret_cast<const void*>(&decode_kernel<Path, T, D, false, false, true>)
                                 : reinterpret_cast<const void*>(&decode_kernel<Path, T, D, false, false>);
  const void* k_deep = reinterpret_cast<const void*>(&decode_kernel<Path, T, D, true, false>);
  int grid = persistent_grid(k_shallow);
  if (grid <= 0) return hipErrorInvalidValue;
  // Direct launch: every context fits one partition and every (sequence,
  // kv head) pair gets a workgroup of its own, so the work list is the
  // sequences in order and needs neither the plan kernel nor the counter.
  p.direct = (p.max_parts == 1 && work_bound <= grid) ? 1 : 0;
  // (the table-free comparison instance exists in the shallow schedule only)
  const bool deep = !p.direct && !p.auto_partition && !p.flat &&
                    work_bound >= static_cast<int64_t>(kDeepItemsPerWorkgroup) * grid;
  if (deep) grid = persistent_grid(k_deep);
  if (grid <= 0) return hipErrorInvalidValue;
  if (grid > work_bound) grid = static_cast<int>(work_bound);
  p.grid = grid;
  p.first_taken = deep ? 2 * grid : grid;
  // Many small explicit partitions: a work item is four consecutive
  // partitions, one per wave (the workspace keeps its per-partition stride,
  // which bounds the number of items).  Each wave computes its partition's
  // softmax state; the four states are combined through LDS (the first
  // level of the log-sum-exp merge) and the item's state goes to the
  // workspace for the merge kernel (the second level).  Measured on the
  // long-context batch (8 x 32K-128K tokens, 512-token partitions): one
  // partition per item, split over the four waves, wrote and merged four
  // times as many states and took 7% longer.
  p.group = (deep && p.P <= kMaxGroupedPartition) ? kWaves : 1;
  if (!p.direct) {
    hipError_t e = launch_plan<T::kBytes, D, false>(p, stream);
    if (e != hipSuccess) return e;
  } else if (p.w_tokens > 0) {  // no plan to run beside: the write kernel first
    PoolGeom g{const_cast<void*>(p.pool), 1, p.N, p.bs, p.H, D, 0, T::kBytes};
    hipError_t e = launch_write_kv(g, 0, p.w_k, p.w_v, p.w_slots, p.w_tokens, stream, p.layer_off * T::kBytes);
    if (e != hipSuccess) return e;
  }
  const int4* items = static_cast<const int4*>(p.items);
  if (deep) {
    hipLaunchKernelGGL((decode_kernel<Path, T, D, true, false>), dim3(grid), dim3(kThreads), 0, stream, p, items,
                       p.groups, p.seq_np);
  } else if (p.flat) {
    hipLaunchKernelGGL((decode_kernel<Path, T, D, false, false, true>), dim3(grid), dim3(kThreads), 0, stream, p,
                       items, p.groups, p.seq_np);
  } else {
    hipLaunchKernelGGL((decode_kernel<Path, T, D, false, false>), dim3(grid), dim3(kThreads), 0, stream, p, items,
                       p.groups, p.seq_np);
  }
  return hipGetLastError();
}

// The sharing plan's items take the shallow schedule: measured on MI355X
// (64 branches over 16 shared 2,048-token prefixes), 60.0 against 61.2 us per
// call with the deep one, whose second held index lengthens the tail.
#ifndef PA_SHARE_DEEP
#define PA_SHARE_DEEP 0
#endif
constexpr bool kShareDeep = PA_SHARE_DEEP != 0;
// Two workgroups per CU for the sharing plan's decode: its items are short
// (about 3.5 per CU), and while one workgroup merges an item's wave states
// and starts the next, the other streams.  Measured on MI355X (64 branches
// over 16 shared 2,048-token prefixes, groups from the host): 54.3 us per
// step with one workgroup per CU and two items each, 50.7 us with two
// workgroups and one item each (copy-on-write batch 53.6 -> 51.8 us); two
// workgroups with two items each, or with the partition size doubled, were no
// better than one.  The other instances keep one workgroup per CU.
#ifndef PA_SHARE_WG_PER_CU
#define PA_SHARE_WG_PER_CU 2
#endif
constexpr int kShareWorkgroupsPerCU = PA_SHARE_WG_PER_CU;

// Sharing plan and decode: the MFMA path with a 16-column tile for every G,
// so that the query heads of up to four sequences that share a prefix fill
// one score tile.
template <typename T, int D>
hipError_t launch_share(DecodeParams p, hipStream_t stream) {
  using Path = MfmaPath<T, D, 16>;
  const void* k = reinterpret_cast<const void*>(&decode_kernel<Path, T, D, kShareDeep, true>);
  int grid = persistent_grid(k, kShareWorkgroupsPerCU);
  if (grid <= 0) return hipErrorInvalidValue;
  const int64_t work_bound = static_cast<int64_t>(p.S) * p.ws_stride * p.H;
  if (grid > work_bound) grid = static_cast<int>(work_bound);
  p.grid = grid;
  p.first_taken = kShareDeep ? 2 * grid : grid;
  p.group = 1;
  p.direct = 0;
  p.share_nmax = 16 / p.G < kShareMaxMembers ? 16 / p.G : kShareMaxMembers;
  hipError_t e = launch_plan<T::kBytes, D, true>(p, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<Path, T, D, kShareDeep, true>), dim3(grid), dim3(kThreads), 0, stream, p,
                     static_cast<const int4*>(p.items), p.groups, p.seq_np);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(DecodeParams p, hipStream_t stream) {
  hipError_t e;
  // Sharing detection: the block manager holds shared blocks, the partition
  // size is automatic (the plan sizes items from the unique work) and the
  // contexts can span partitions (the split at a shared prefix's end needs
  // the partition-state workspace); small enough batches for the one-
  // workgroup plan, and at least two sequences per 16-column tile.
  p.share = (p.share && !p.flat && p.auto_partition && p.max_parts > 1 && p.S <= kShareMaxSeqs && p.G <= 8) ? 1 : 0;
  if (p.share) {
    e = launch_share<T, D>(p, stream);
  } else if (p.G == 1) {
    e = launch_decode_kernel<ValuPath<T, D, 1>, T, D>(p, stream);
  } else if (p.G == 2) {
    e = launch_decode_kernel<ValuPath<T, D, 2>, T, D>(p, stream);
  } else if (p.G <= 4) {
    e = launch_decode_kernel<MfmaPath<T, D, 4>, T, D>(p, stream);
  } else if (p.G <= 8) {
    e = launch_decode_kernel<MfmaPath<T, D, 8>, T, D>(p, stream);
  } else {
    e = launch_decode_kernel<MfmaPath<T, D, 16>, T, D>(p, stream);
  }
  if (e != hipSuccess || p.max_parts <= 1) return e;
  const int pairs = p.S * p.Hq;
  if (!p.auto_partition && p.max_parts >= kWideMergeParts) {
    hipLaunchKernelGGL((merge_wide_kernel<T, D>), dim3(pairs), dim3(kMergeThreads), 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3((pairs + kMergeWaves - 1) / kMergeWaves), dim3(kMergeThreads),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int dtype, int D, int G) {
  if (D != 64 && D != 128) return false;
  if (G < 1 || G > 16) return false;
  return dtype == 0 || dtype == 1 || dtype == 2;
}

hipError_t launch_decode(const DecodeParams& p, int dtype, int D, hipStream_t stream) {
  if (!decode_supported(dtype, D, p.G)) return hipErrorInvalidValue;
  if (p.S <= 0) return hipSuccess;
  switch (dtype) {
    case 0:
      return D == 64 ? launch_typed<F32, 64>(p, stream) : launch_typed<F32, 128>(p, stream);
    case 1:
      return D == 64 ? launch_typed<F16, 64>(p, stream) : launch_typed<F16, 128>(p, stream);
    default:
      return D == 64 ? launch_typed<BF16, 64>(p, stream) : launch_typed<BF16, 128>(p, stream);
  }
}

}  // namespace pa
