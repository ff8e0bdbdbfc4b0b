// Read-bandwidth probe: how fast this device delivers a large buffer read as
// 4 or 8 KiB blocks in a given order, the access pattern of the attention
// kernels (each (block, KV head) slice of a pool is 8 KiB at block size 32,
// 4 KiB at block size 16, head dimension 128, bf16). It measures the practical
// ceiling under the HBM roofline; it is not part of the attention path.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "pa_internal.h"

namespace {

constexpr int kProbeThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each wave reads DEPTH blocks of KIB KiB per round (KIB non-temporal 16-byte
// loads per lane per block, all in flight together), rounds spread over the
// grid.
template <int DEPTH, int KIB>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const char* __restrict__ buf,
                                                                   const int32_t* __restrict__ order,
                                                                   int64_t num_blocks, uint32_t* sink) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int64_t wid = int64_t(blockIdx.x) * (kProbeThreads / 64) + wave;
  const int64_t nw = int64_t(gridDim.x) * (kProbeThreads / 64);
  const int64_t rounds = num_blocks / DEPTH;
  uint32_t acc = 0;
  for (int64_t g = wid; g < rounds; g += nw) {
    u32x4 v[DEPTH][KIB];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      // entries outside [0, num_blocks) are clamped: the probe never reads past buf
      const int64_t blk = std::min<int64_t>(uint32_t(order[g * DEPTH + d]), num_blocks - 1);
      const char* base = buf + blk * (KIB * 1024);
#pragma unroll
      for (int u = 0; u < KIB; ++u)
        v[d][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (u * 64 + lane) * 16));
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int u = 0; u < KIB; ++u) acc ^= v[d][u].x ^ v[d][u].y ^ v[d][u].z ^ v[d][u].w;
  }
  // the loads must not be optimised away: a store that depends on them
  if (acc == 0x9e3779b9u) __hip_atomic_store(sink, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int KIB>
void launch_probe(int depth, int workgroups, hipStream_t s, const char* b, const int32_t* order,
                  int64_t num_blocks, uint32_t* sink) {
  switch (depth) {
    case 1: hipLaunchKernelGGL((read_probe_kernel<1, KIB>), dim3(workgroups), dim3(kProbeThreads), 0, s, b, order, num_blocks, sink); break;
    case 2: hipLaunchKernelGGL((read_probe_kernel<2, KIB>), dim3(workgroups), dim3(kProbeThreads), 0, s, b, order, num_blocks, sink); break;
    case 4: hipLaunchKernelGGL((read_probe_kernel<4, KIB>), dim3(workgroups), dim3(kProbeThreads), 0, s, b, order, num_blocks, sink); break;
  }
}

}  // namespace

extern "C" pa_status pa_read_probe(const void* buf, int64_t num_blocks, int32_t block_bytes,
                                   const int32_t* order, int32_t blocks_in_flight, int32_t workgroups,
                                   uint32_t* sink, void* stream) {
  if (!buf || !order || !sink || num_blocks < 1 || workgroups < 1) return PA_ERR_INVALID_ARG;
  if (block_bytes != 4096 && block_bytes != 8192) return PA_ERR_INVALID_ARG;
  if (blocks_in_flight != 1 && blocks_in_flight != 2 && blocks_in_flight != 4) return PA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* b = static_cast<const char*>(buf);
  if (block_bytes == 4096)
    launch_probe<4>(blocks_in_flight, workgroups, s, b, order, num_blocks, sink);
  else
    launch_probe<8>(blocks_in_flight, workgroups, s, b, order, num_blocks, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : pa::hip_failed(e);
}
