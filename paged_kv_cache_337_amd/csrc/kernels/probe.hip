// Read-bandwidth probe: the access pattern of the decode kernel without its
// arithmetic.  Each wave reads whole 8 KiB chunks (eight 16-byte loads per
// lane, 1 KiB per instruction) in the order given by a chunk list, two chunks
// in flight, and folds the data into one word so the loads stay live.  It
// gives the HBM read rate that paged 8 KiB runs can reach on this GPU, the
// practical ceiling the decode kernel is compared with.
#include "../launch.hpp"
#include "common.hpp"

namespace pa {

namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ buf, int64_t nchunks_buf,
                                                                   const int32_t* __restrict__ ids, int n,
                                                                   uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = static_cast<int>((blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x) >> 6);
  const int W = static_cast<int>((static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6);
  uint32_t acc = 0;
  for (int c = wave; c < n; c += 2 * W) {
    uint4 v[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = c + u * W;
      int32_t id = k < n ? ids[k] : -1;
      id = (id >= 0 && id < nchunks_buf) ? id : 0;
      const uint4* b = buf + static_cast<size_t>(id) * 512 + lane;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[u][j] = load_stream16(b + 64 * j);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc ^= v[u][j].x ^ v[u][j].y ^ v[u][j].z ^ v[u][j].w;
  }
  // Almost never true; keeps the loads from being removed.
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_probe_read(const void* buf, int64_t nchunks_buf, const int32_t* ids, int n, void* sink,
                             hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // Two workgroups of four waves per CU: the configuration that read paged
  // 8 KiB chunks fastest on MI355X.
  const int grid = 2 * cus;
  hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, static_cast<const uint4*>(buf),
                     nchunks_buf, ids, n, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace pa
