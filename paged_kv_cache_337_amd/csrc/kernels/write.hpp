// The cache write of one wave: the K and V rows of a group of four
// consecutive new tokens for one kv head, scattered into their slots in the
// pool layout documented in pa.h.  Used by the write kernel and by the
// prologue of pa_decode_step.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace pa {

// One wave per (group of four consecutive input tokens, kv head).
//
// K: a token's row is D / E chunks of 16 bytes, each one 16-byte store (E
// consecutive d stay consecutive in a K sub-tile).
// V: the sub-tile keeps four tokens side by side (token-inner order), so one
// 16-byte chunk holds tokens 4m .. 4m+3 of R = E / 4 head_dim tiles at one
// d % 16.  When the group's four slots are consecutive and start at a
// multiple of four (the tokens of a prompt chunk), the wave assembles whole
// chunks and stores 16 bytes at a time; otherwise (for example one new token
// per sequence in decode) each token's V elements are stored one by one.
template <int kBytes>
__device__ __forceinline__ void write_token_group(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                  const int32_t* __restrict__ slots, int num_tokens,
                                                  char* __restrict__ layer_base, int N, int H, int bs, int D,
                                                  int group_id, int h, int lane) {
  using Bits = typename std::conditional<kBytes == 4, uint32_t, uint16_t>::type;
  constexpr int E = 16 / kBytes;
  constexpr int R = E / 4;
  const int cpr = D / E;  // 16-byte chunks per (token, head) row
  const int t0 = group_id * 4;
  const int ntok = num_tokens - t0 < 4 ? num_tokens - t0 : 4;
  int32_t sl[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) sl[q] = q < ntok ? slots[t0 + q] : -1;
  const int32_t s0 = sl[0];
  const bool group = ntok == 4 && s0 >= 0 && (s0 & 3) == 0 && sl[1] == s0 + 1 && sl[2] == s0 + 2 &&
                     sl[3] == s0 + 3 && s0 / bs < N;

  // K rows: one 16-byte store per chunk.
  for (int x = lane; x < 4 * cpr; x += 64) {
    const int q = x / cpr, c = x - (x / cpr) * cpr;
    const int32_t slot = sl[q];
    if (slot < 0 || slot / bs >= N) continue;
    const int32_t b = slot / bs;
    const int t = slot - b * bs, sub = t / 16, r = t % 16;
    const size_t region = (static_cast<size_t>(b) * H + h) * (2 * static_cast<size_t>(bs) * D);
    const int d0 = c * E;
    const int k_off = ((d0 / (4 * E)) * 64 + r + 16 * ((d0 % (4 * E)) / E)) * E;
    const size_t row = (static_cast<size_t>(t0 + q) * H + h) * cpr + c;
    *reinterpret_cast<uint4*>(layer_base + (region + static_cast<size_t>(sub) * 16 * D + k_off) * kBytes) = k[row];
  }

  const Bits* vin = reinterpret_cast<const Bits*>(v);
  if (group) {
    // Chunk (P, j) of the group's token quad: head_dim tiles P*R .. P*R+R-1
    // at d % 16 = j, four tokens each.
    const int32_t b = s0 / bs;
    const int t = s0 - b * bs, sub = t / 16, m = (t % 16) / 4;
    const size_t vbase = (static_cast<size_t>(b) * H + h) * (2 * static_cast<size_t>(bs) * D) +
                         static_cast<size_t>(bs) * D + static_cast<size_t>(sub) * 16 * D;
    for (int x = lane; x < D / R; x += 64) {
      const int P = x / 16, j = x % 16;
      Bits e[E];
#pragma unroll
      for (int mm = 0; mm < R; ++mm)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          e[mm * 4 + q] = vin[(static_cast<size_t>(t0 + q) * H + h) * D + (P * R + mm) * 16 + j];
      const size_t off = vbase + static_cast<size_t>((P * 64 + j + 16 * m) * E);
      uint4 w;
      __builtin_memcpy(&w, e, sizeof(w));
      *reinterpret_cast<uint4*>(layer_base + off * kBytes) = w;
    }
  } else {
    for (int x = lane; x < 4 * D; x += 64) {
      const int q = x / D, d = x - (x / D) * D;
      const int32_t slot = sl[q];
      if (slot < 0 || slot / bs >= N) continue;
      const int32_t b = slot / bs;
      const int t = slot - b * bs, sub = t / 16, r = t % 16;
      const size_t vbase = (static_cast<size_t>(b) * H + h) * (2 * static_cast<size_t>(bs) * D) +
                           static_cast<size_t>(bs) * D + static_cast<size_t>(sub) * 16 * D;
      const int nd = d / 16;
      const int v_off = (((nd / R) * 64 + d % 16 + 16 * (r / 4)) * R + nd % R) * 4 + r % 4;
      *reinterpret_cast<Bits*>(layer_base + (vbase + v_off) * kBytes) =
          vin[(static_cast<size_t>(t0 + q) * H + h) * D + d];
    }
  }
}

}  // namespace pa
