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
#include "write.hpp"

namespace pa {

// One wave per (group of four consecutive input tokens, kv head).
template <int kBytes>
__global__ __launch_bounds__(64) void write_kv_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                      const int32_t* __restrict__ slots, int num_tokens,
                                                      char* __restrict__ layer_base, int N, int H, int bs, int D) {
  write_token_group<kBytes>(k, v, slots, num_tokens, layer_base, N, H, bs, D, blockIdx.x, blockIdx.y, threadIdx.x);
}

hipError_t launch_write_kv(const PoolGeom& g, int layer, const void* k, const void* v,
                           const int32_t* slots, int num_tokens, hipStream_t stream, int64_t layer_byte_off) {
  if (num_tokens <= 0) return hipSuccess;
  if (g.H > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((num_tokens + 3) / 4), static_cast<unsigned>(g.H));
  char* base = static_cast<char*>(g.base) + (layer_byte_off >= 0 ? static_cast<size_t>(layer_byte_off)
                                                                  : static_cast<size_t>(layer) * g.layer_elems() *
                                                                        g.elem_bytes);
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
