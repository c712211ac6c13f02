// Cache update kernels: scatter new tokens' K/V rows into their slots, and
// copy whole blocks for copy-on-write.
//
// "Paged Attention Explained", "Practical Example" lists cache updates among
// what a paged implementation must do; "PagedAttention: paging the KV cache like
// an OS pages memory", "How it works", copies a shared block when it must be
// modified.  The element placement follows the pool layout documented in pa.h.
#include "../launch.hpp"
#include "common.hpp"

namespace pa {

// One thread per (token, kv head, 16-byte chunk of the row).  The K chunk is a
// single 16-byte store (E consecutive d stay consecutive in a K sub-tile);
// the V elements of one token are 4 elements apart (token-inner order), so
// they are stored one by one.
template <int kBytes>
__global__ __launch_bounds__(256) void write_kv_kernel(const uint4* __restrict__ k,
                                                       const uint4* __restrict__ v,
                                                       const int32_t* __restrict__ slots,
                                                       int num_tokens, char* __restrict__ layer_base,
                                                       int N, int H, int bs, int D) {
  constexpr int E = 16 / kBytes;
  constexpr int R = E / 4;
  const int cpr = D / E;  // 16-byte chunks per (token, head) row
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(num_tokens) * H * cpr;
  if (gid >= total) return;
  const int tok = static_cast<int>(gid / (H * cpr));
  const int rem = static_cast<int>(gid % (H * cpr));
  const int h = rem / cpr, c = rem % cpr;
  const int32_t slot = slots[tok];
  if (slot < 0) return;
  const int32_t b = slot / bs;
  if (b >= N) return;
  const int t = slot % bs, sub = t / 16, r = t % 16;

  const size_t region = (static_cast<size_t>(b) * H + h) * (2 * static_cast<size_t>(bs) * D);
  const size_t kbase = region + static_cast<size_t>(sub) * 16 * D;
  const size_t vbase = region + static_cast<size_t>(bs) * D + static_cast<size_t>(sub) * 16 * D;
  const int d0 = c * E;
  const int k_off = ((d0 / (4 * E)) * 64 + r + 16 * ((d0 % (4 * E)) / E)) * E;
  const uint4 kv = k[gid];
  const uint4 vv = v[gid];
  *reinterpret_cast<uint4*>(layer_base + (kbase + k_off) * kBytes) = kv;

  const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int d = d0 + e;
    const int nd = d / 16;
    const int v_off = (((nd / R) * 64 + d % 16 + 16 * (r / 4)) * R + nd % R) * 4 + r % 4;
    char* dst = layer_base + (vbase + v_off) * kBytes;
    if constexpr (kBytes == 4) {
      *reinterpret_cast<uint32_t*>(dst) = w[e];
    } else {
      *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(w[e / 2] >> (16 * (e % 2)));
    }
  }
}

hipError_t launch_write_kv(const PoolGeom& g, int layer, const void* k, const void* v,
                           const int32_t* slots, int num_tokens, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  const int E = 16 / g.elem_bytes;
  const int64_t total = static_cast<int64_t>(num_tokens) * g.H * (g.D / E);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  char* base = static_cast<char*>(g.base) + static_cast<size_t>(layer) * g.layer_elems() * g.elem_bytes;
  if (g.elem_bytes == 4) {
    hipLaunchKernelGGL(write_kv_kernel<4>, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                       stream, static_cast<const uint4*>(k), static_cast<const uint4*>(v), slots,
                       num_tokens, base, g.N, g.H, g.bs, g.D);
  } else {
    hipLaunchKernelGGL(write_kv_kernel<2>, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                       stream, static_cast<const uint4*>(k), static_cast<const uint4*>(v), slots,
                       num_tokens, base, g.N, g.H, g.bs, g.D);
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

}  // namespace pa
