// Streaming of 16-token K/V units from the paged pool for the gfx950
// attention kernels (decode and prefill): per-lane block ids read out with
// v_readlane, 16-byte loads of whole MFMA operand chunks, and a software
// pipeline that keeps a fixed number of units in flight per wave.
#pragma once

#include "common.hpp"

namespace pa {

__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Wave-uniform "any lane" test.
__device__ __forceinline__ bool wave_any(bool x) { return __builtin_amdgcn_ballot_w64(x) != 0; }

// Per-thread view of one unit: NCH 16-byte chunks of K and of V.
template <int NCH>
struct Frag {
  uint4 k[NCH];
  uint4 v[NCH];
};

// ---------------------------------------------------------------------------
// Unit streaming.
// ---------------------------------------------------------------------------

// The 16-token units of one wave's run of a partition, located in issue order.
// The block ids of a piece of the run (at most 64 logical blocks) are held one
// per lane and read out with v_readlane, so locating a unit is scalar
// arithmetic with no memory access.
// kFlat: no block table -- the sequence's blocks are consecutive physical
// blocks from its first one (a contiguous range, the comparison point for
// what the table costs); `trow` then points at that first block id.
template <int D, int kBytes, bool kFlat = false>
struct UnitStream {
  const char* layer_base;  // pool base + layer offset (bytes)
  const int32_t* trow;     // block-table row of the sequence
  int max_blocks, bs, N, H, h;
  int lb, sub;             // logical block and 16-token sub-tile of the next unit
  int lb_base;             // logical block of ids lane 0
  int32_t ids;

  // Position at unit u of the token range starting at `start`.  Params
  // carries the pool base, layer offset and geometry.
  template <typename Params>
  __device__ __forceinline__ void begin(const Params& p, const int32_t* row, int start, int u, int head) {
    layer_base = static_cast<const char*>(p.pool) + p.layer_off * kBytes;
    trow = row;
    max_blocks = p.max_blocks;
    bs = p.bs;
    N = p.N;
    H = p.H;
    h = head;
    const int p0 = start + u * 16;
    lb = p0 / bs;
    sub = (p0 - lb * bs) >> 4;
    lb_base = lb;
  }

  // Block id of logical block lb_base + lane (-1 past the row); with kFlat,
  // the sequence's first block id (uniform).
  __device__ __forceinline__ int32_t fetch_ids(int lane) const {
    if constexpr (kFlat) return __builtin_amdgcn_readfirstlane(trow[0]);
    const int k = lb_base + lane;
    return k < max_blocks ? trow[k] : -1;
  }

  // Bases of the K and V sub-tiles of the next unit, then advance.  Returns
  // false for an invalid block id (the bases then point at block 0 of the
  // layer, a valid address; such a unit is masked).
  __device__ __forceinline__ bool locate(const char*& kp, const char*& vp) {
    const int32_t b = kFlat ? static_cast<int32_t>(static_cast<uint32_t>(ids) + static_cast<uint32_t>(lb))
                            : __builtin_amdgcn_readlane(ids, lb - lb_base);
    const int s = sub;
    if (++sub * 16 == bs) {
      sub = 0;
      ++lb;
    }
    const bool ok = b >= 0 && b < N;
    const size_t region = (static_cast<size_t>(ok ? b : 0) * H + h) * (2 * static_cast<size_t>(bs) * D);
    kp = layer_base + (region + static_cast<size_t>(s) * 16 * D) * kBytes;
    vp = layer_base + (region + static_cast<size_t>(bs) * D + static_cast<size_t>(s) * 16 * D) * kBytes;
    return ok;
  }

  template <int NCH>
  __device__ __forceinline__ bool issue(Frag<NCH>& f, int lane) {
    const char *kb, *vb;
    const bool ok = locate(kb, vb);
    const uint32_t lane_off = static_cast<uint32_t>(lane) * 16u;
    const uint4* kp = reinterpret_cast<const uint4*>(kb + lane_off);
    const uint4* vp = reinterpret_cast<const uint4*>(vb + lane_off);
#pragma unroll
    for (int c = 0; c < NCH; ++c) f.k[c] = load_stream16(kp + 64 * c);
#pragma unroll
    for (int c = 0; c < NCH; ++c) f.v[c] = load_stream16(vp + 64 * c);
    return ok;
  }
};

// Issues the first PF units of a piece into f[0 .. PF-1].  Always PF units:
// units past the run only cost a wasted load of a valid address, and a fixed
// count keeps the compiler's waits exact in every loop that follows.
template <int PF, int NCH, typename Stream>
__device__ __forceinline__ void prologue(Stream& st, Frag<NCH> (&f)[PF + 1], bool (&ok)[PF + 1], int lane) {
#pragma unroll
  for (int s = 0; s < PF; ++s) ok[s] = st.template issue<NCH>(f[s], lane);
}

// Runs compute(frag, u, ok) over the units [u0, u1) of one piece whose first
// PF units are already in flight.  In the main loop every step issues one
// unit's loads, so the wait before each unit covers exactly that unit's
// loads; the last steps (fewer than PF + NB units) issue what is left and
// drain.
template <int PF, int NCH, typename Stream, typename Compute>
__device__ __forceinline__ void stream_piece(Stream& st, Frag<NCH> (&f)[PF + 1], bool (&ok)[PF + 1],
                                             int u0, int u1, int lane, Compute&& compute) {
  constexpr int NB = PF + 1;
  int u = u0;
  for (; u + NB - 1 + PF < u1; u += NB) {
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      ok[(s + PF) % NB] = st.template issue<NCH>(f[(s + PF) % NB], lane);
      compute(f[s], u + s, ok[s]);
    }
  }
  for (; u < u1; u += NB) {
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      if (u + s + PF < u1) ok[(s + PF) % NB] = st.template issue<NCH>(f[(s + PF) % NB], lane);
      if (u + s < u1) compute(f[s], u + s, ok[s]);
    }
  }
}

// First unit of the logical block 64 blocks after that of unit u: runs are
// cut there, so that one load of block ids covers each piece.
__device__ __forceinline__ int piece_end(int bs, int start, int u) {
  const int p0 = start + u * 16;
  return ((p0 / bs + 64) * bs - start) >> 4;
}

// Units [u0, u1) of the token range starting at `start` of one table row,
// the first piece's prologue already issued.  Runs longer than 64 blocks load
// the ids of each further piece where it starts.
template <int PF, int NCH, typename Stream, typename Params, typename Compute>
__device__ __forceinline__ void stream_run(const Params& p, Stream& st, Frag<NCH> (&f)[PF + 1],
                                           bool (&ok)[PF + 1], const int32_t* trow, int start, int u0, int u1,
                                           int head, int lane, Compute&& compute) {
  int a = u0;
  int b = piece_end(p.bs, start, a);
  b = b < u1 ? b : u1;
  stream_piece<PF, NCH>(st, f, ok, a, b, lane, compute);
  for (a = b; a < u1; a = b) {
    b = piece_end(p.bs, start, a);
    b = b < u1 ? b : u1;
    st.begin(p, trow, start, a, head);
    st.ids = st.fetch_ids(lane);
    prologue<PF, NCH>(st, f, ok, lane);
    stream_piece<PF, NCH>(st, f, ok, a, b, lane, compute);
  }
}

// Zero V elements of tokens >= valid (their slots may hold anything, and
// 0 * NaN would poison the product).  Lane group `grp` holds tokens
// 4*grp .. 4*grp+3 of the unit, token-inner.
template <int kBytes, int NCH>
__device__ __forceinline__ void mask_v_tail(Frag<NCH>& f, int grp, int valid) {
  const int t0 = 4 * grp;
  if constexpr (kBytes == 2) {
    const uint32_t m01 = (t0 + 0 < valid ? 0x0000ffffu : 0u) | (t0 + 1 < valid ? 0xffff0000u : 0u);
    const uint32_t m23 = (t0 + 2 < valid ? 0x0000ffffu : 0u) | (t0 + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      f.v[c].x &= m01;
      f.v[c].y &= m23;
      f.v[c].z &= m01;
      f.v[c].w &= m23;
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      f.v[c].x = t0 + 0 < valid ? f.v[c].x : 0u;
      f.v[c].y = t0 + 1 < valid ? f.v[c].y : 0u;
      f.v[c].z = t0 + 2 < valid ? f.v[c].z : 0u;
      f.v[c].w = t0 + 3 < valid ? f.v[c].w : 0u;
    }
  }
}

}  // namespace pa
