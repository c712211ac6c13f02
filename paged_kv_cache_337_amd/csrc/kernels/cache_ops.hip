// Cache update kernels: scatter new tokens' K/V rows into their slots, and
// copy whole blocks for copy-on-write.
//
// "Paged Attention Explained", "Practical Example" lists cache updates among
// what a paged implementation must do; "PagedAttention: paging the KV cache like
// an OS pages memory", "How it works", copies a shared block when it must be
// modified.  The element placement follows the pool layout documented in pa.h.
#include <type_traits>

#include "../launch.hpp"
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
__global__ __launch_bounds__(64) void write_kv_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                      const int32_t* __restrict__ slots, int num_tokens,
                                                      char* __restrict__ layer_base, int N, int H, int bs, int D) {
  using Bits = typename std::conditional<kBytes == 4, uint32_t, uint16_t>::type;
  constexpr int E = 16 / kBytes;
  constexpr int R = E / 4;
  const int cpr = D / E;  // 16-byte chunks per (token, head) row
  const int lane = threadIdx.x;
  const int t0 = blockIdx.x * 4;
  const int h = blockIdx.y;
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

hipError_t launch_write_kv(const PoolGeom& g, int layer, const void* k, const void* v,
                           const int32_t* slots, int num_tokens, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  if (g.H > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((num_tokens + 3) / 4), static_cast<unsigned>(g.H));
  char* base = static_cast<char*>(g.base) + static_cast<size_t>(layer) * g.layer_elems() * g.elem_bytes;
  if (g.elem_bytes == 4) {
    hipLaunchKernelGGL(write_kv_kernel<4>, grid, dim3(64), 0, stream, static_cast<const uint4*>(k),
                       static_cast<const uint4*>(v), slots, num_tokens, base, g.N, g.H, g.bs, g.D);
  } else {
    hipLaunchKernelGGL(write_kv_kernel<2>, grid, dim3(64), 0, stream, static_cast<const uint4*>(k),
                       static_cast<const uint4*>(v), slots, num_tokens, base, g.N, g.H, g.bs, g.D);
  }
  return hipGetLastError();
}

// grid.x = pair index, grid.y = layer.  Each (layer, block) is one contiguous
// run of H * 2 * bs * D elements, copied with 16-byte loads and stores.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ base,
                                                          const int32_t* __restrict__ pairs, int N,
                                                          size_t block_bytes, size_t layer_bytes) {
  const int32_t src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || dst < 0 || src >= N || dst >= N || src == dst) return;
  const size_t lo = static_cast<size_t>(blockIdx.y) * layer_bytes;
  const uint4* s = reinterpret_cast<const uint4*>(base + lo + static_cast<size_t>(src) * block_bytes);
  uint4* d = reinterpret_cast<uint4*>(base + lo + static_cast<size_t>(dst) * block_bytes);
  const size_t n16 = block_bytes / 16;
  for (size_t i = threadIdx.x; i < n16; i += blockDim.x) d[i] = s[i];
}

hipError_t launch_copy_blocks(const PoolGeom& g, const int32_t* pairs, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const size_t block_bytes = static_cast<size_t>(g.H) * 2 * g.bs * g.D * g.elem_bytes;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, g.L), dim3(256), 0, stream,
                     static_cast<char*>(g.base), pairs, g.N, block_bytes,
                     g.layer_elems() * g.elem_bytes);
  return hipGetLastError();
}

// Swap copies between the pool and a host tier.  grid.x = pair index,
// grid.y = layer.  A device block of one layer is one contiguous run of
// H * 2 * bs * D elements; a host block holds the runs of every layer side
// by side.  dir 0 copies (device, host) pairs out, dir 1 (host, device) pairs
// in.  Pairs with an id out of range are skipped.
__global__ __launch_bounds__(256) void swap_blocks_kernel(char* __restrict__ pool, char* __restrict__ host,
                                                          const int32_t* __restrict__ pairs, int N, int64_t host_n,
                                                          size_t block_bytes, size_t layer_bytes, int L, int dir) {
  const int32_t a = pairs[2 * blockIdx.x], b = pairs[2 * blockIdx.x + 1];
  const int32_t dev = dir == 0 ? a : b;
  const int32_t hb = dir == 0 ? b : a;
  if (dev < 0 || dev >= N || hb < 0 || hb >= host_n) return;
  const size_t l = blockIdx.y;
  uint4* d = reinterpret_cast<uint4*>(pool + l * layer_bytes + static_cast<size_t>(dev) * block_bytes);
  uint4* h = reinterpret_cast<uint4*>(host + (static_cast<size_t>(hb) * L + l) * block_bytes);
  const uint4* src = dir == 0 ? d : h;
  uint4* dst = dir == 0 ? h : d;
  const size_t n16 = block_bytes / 16;
  for (size_t i = threadIdx.x; i < n16; i += blockDim.x) dst[i] = src[i];
}

hipError_t launch_swap_blocks(const PoolGeom& g, const int32_t* pairs, int n, void* host, int64_t host_blocks,
                              int dir, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (g.L > 65535) return hipErrorInvalidValue;
  const size_t block_bytes = static_cast<size_t>(g.H) * 2 * g.bs * g.D * g.elem_bytes;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(n, g.L), dim3(256), 0, stream, static_cast<char*>(g.base),
                     static_cast<char*>(host), pairs, g.N, host_blocks, block_bytes, g.layer_elems() * g.elem_bytes,
                     g.L, dir);
  return hipGetLastError();
}

}  // namespace pa
