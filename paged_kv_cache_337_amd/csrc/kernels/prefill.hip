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
// Work split.  The query rows of one (sequence, kv head) are the pairs
// (new token k, query head g of the group), row = k * G + g, so the 16
// columns of an MFMA tile are always full whatever the group size.  A wave
// owns NB tiles of 16 rows and streams the K/V units (16 tokens of one block)
// from position 0 up to the last position its rows attend to; it keeps
// NB independent online-softmax states and never exchanges data with the
// other waves.  A workgroup is four such waves on consecutive rows; the grid
// is (sequence x kv head, row tile) with the heaviest (last) row tiles of
// every sequence dispatched first.
//
// Per unit and tile: S = K.Q^T with v_mfma_f32_16x16x32_{bf16,f16} (tokens x
// rows, head_dim reduced; v_mfma_f32_16x16x4_f32 for float32 pools), the
// causal mask per row by select, the online softmax with a lazily raised
// reference (rescale only when a score passes the reference by 2^8), then
// O += P.V with v_mfma_f32_16x16x16 (rows x head_dim, tokens reduced).  The K
// and V fragments of a unit are loaded once and used for all NB tiles.
//
// Memory safety: lengths and query offsets are clamped to the buffers the
// caller declared, table reads stay inside the row and block ids outside
// [0, N) read block 0 and are masked.
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

template <typename T, int D>
hipError_t launch_prefill_typed(const PrefillParams& p, hipStream_t stream) {
  constexpr int kRowsWG = 16 * kTilesPerWave * kPrefillWaves;
  const int64_t tiles = (static_cast<int64_t>(p.max_query_len) * p.G + kRowsWG - 1) / kRowsWG;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.S) * p.H, static_cast<unsigned>(tiles));
  hipLaunchKernelGGL((prefill_kernel<T, D, kTilesPerWave, kPrefillPrefetch>), grid, dim3(kPrefillThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

int64_t prefill_max_query_len(int G) {
  return static_cast<int64_t>(65535) * (16 * kTilesPerWave * kPrefillWaves) / (G > 0 ? G : 1);
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
