// Block transfers between the packed cache (HBM) and host memory for gfx950.
//
// Source (page and section): qiita article on AMD 4-bit KV caching in LMCache,
// the sections on the transfer side not interpreting the quantized contents (the
// connector moves packed slots as bytes, with their strides) and on what equal
// bytes guarantee (a save/restore round trip T must give T(Q(X)) = Q(X), and must
// leave adjacent regions untouched).
//
// A block is the num_kv_heads pages of one block id, contiguous in the cache
// ([num_blocks][num_kv_heads][page_bytes]), so a transfer is a gather (or
// scatter) of equal-sized contiguous byte ranges.  Host memory is pinned and
// mapped into the device's address space: the kernels read or write it directly
// with 16-byte accesses (non-temporal on the host side), and many work-groups
// keep enough requests in flight to cover the host link's latency.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {

namespace {

// Copy n blocks of `row` 16-byte units: block_ids[i] of `cache` <-> unit range i
// of `host`.  TO_HOST: cache -> host.  Ids outside [0, num_blocks) are skipped.
template <bool TO_HOST>
__global__ __launch_bounds__(256) void transfer_kernel(uint4* cache, uint4* host, const int32_t* block_ids,
                                                       int64_t n, int64_t num_blocks, int64_t row) {
  const int64_t total = n * row;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = u / row, r = u - i * row;
    const int64_t blk = block_ids[i];
    if (blk < 0 || blk >= num_blocks) continue;
    uint4* c = cache + blk * row + r;
    uint4* h = host + u;
    if constexpr (TO_HOST) {
      const uint4 v = *c;
      __builtin_nontemporal_store(v.x, &h->x);
      __builtin_nontemporal_store(v.y, &h->y);
      __builtin_nontemporal_store(v.z, &h->z);
      __builtin_nontemporal_store(v.w, &h->w);
    } else {
      uint4 v;
      v.x = __builtin_nontemporal_load(&h->x);
      v.y = __builtin_nontemporal_load(&h->y);
      v.z = __builtin_nontemporal_load(&h->z);
      v.w = __builtin_nontemporal_load(&h->w);
      *c = v;
    }
  }
}

}  // namespace

hipError_t launch_transfer(bool to_host, void* cache, void* host, const int32_t* block_ids, int64_t n,
                           int64_t num_blocks, int64_t block_bytes, int grid, hipStream_t s) {
  const int64_t row = block_bytes / 16;
  const int64_t units = n * row;
  const unsigned g = (unsigned)std::max<int64_t>(1, std::min<int64_t>((units + 255) / 256, grid));
  if (to_host)
    hipLaunchKernelGGL(transfer_kernel<true>, dim3(g), dim3(256), 0, s, static_cast<uint4*>(cache),
                       static_cast<uint4*>(host), block_ids, n, num_blocks, row);
  else
    hipLaunchKernelGGL(transfer_kernel<false>, dim3(g), dim3(256), 0, s, static_cast<uint4*>(cache),
                       static_cast<uint4*>(host), block_ids, n, num_blocks, row);
  return hipGetLastError();
}

}  // namespace tq
