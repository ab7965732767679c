// Plain streaming kernels that set the memory-system ceilings beside the roofline
// figures: read only, write only, copy, and a mixed stream that reads m words for
// every word it writes, each with 16-byte accesses and a grid-stride loop over
// whole 16-byte words.  Built into their own library
// (libtqstream.so), used by bench.py only; not part of the C ABI in tq.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Read every word; the XOR of a lane's words is stored only when it equals a
// value no input holds, so the loads stay (the compiler cannot drop them) and
// nothing is written.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, size_t n, uint32_t never,
                                                   uint32_t* __restrict__ sink) {
  uint32_t x = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const u32x4 w = __builtin_nontemporal_load(src + i);
    x ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  if (x == never) sink[0] = x;
}

__global__ __launch_bounds__(256) void write_kernel(u32x4* __restrict__ dst, size_t n, uint32_t v) {
  const u32x4 w = {v, v, v, v};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    __builtin_nontemporal_store(w, dst + i);
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Read M consecutive words and write their XOR as one word: reads and writes in
// the ratio M : 1, interleaved as a kernel that quantizes what it reads would
// interleave them.  The M loads of a lane are issued together.  Plain (temporal)
// accesses: the nontemporal forms are slower for this mix.
template <int M>
__global__ __launch_bounds__(256) void mix_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                  size_t n_out) {
  for (size_t o = (size_t)blockIdx.x * 256 + threadIdx.x; o < n_out; o += (size_t)gridDim.x * 256) {
    u32x4 w[M];
#pragma unroll
    for (int q = 0; q < M; ++q) w[q] = src[o * M + q];
#pragma unroll
    for (int q = 1; q < M; ++q) w[0] ^= w[q];
    dst[o] = w[0];
  }
}

unsigned grid_for(size_t n, int blocks) {
  const size_t need = (n + 255) / 256;
  return (unsigned)(need < (size_t)blocks ? (need > 0 ? need : 1) : (size_t)blocks);
}

}  // namespace

// Each returns the launch status (hipSuccess = 0).  Buffers are device memory,
// 16-byte aligned, of `bytes` bytes (a multiple of 16); `blocks` caps the grid.
extern "C" int tqs_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(read_kernel, dim3(grid_for(bytes / 16, blocks)), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), bytes / 16, 0x9E3779B9u, sink);
  return (int)hipGetLastError();
}

extern "C" int tqs_write(void* dst, size_t bytes, uint32_t value, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(write_kernel, dim3(grid_for(bytes / 16, blocks)), dim3(256), 0, s, static_cast<u32x4*>(dst),
                     bytes / 16, value);
  return (int)hipGetLastError();
}

extern "C" int tqs_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(bytes / 16, blocks)), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return (int)hipGetLastError();
}

// Reads (bytes / 16 / m) * m words of src and writes bytes / 16 / m words of dst;
// m from 1 to 8.
extern "C" int tqs_mix(const void* src, void* dst, size_t bytes, int m, int blocks, hipStream_t s) {
  if (m < 1 || m > 8) return (int)hipErrorInvalidValue;
  const size_t n_out = bytes / 16 / (size_t)m;
  const dim3 grid(grid_for(n_out, blocks));
  const u32x4* in = static_cast<const u32x4*>(src);
  u32x4* out = static_cast<u32x4*>(dst);
  switch (m) {
    case 1: hipLaunchKernelGGL(mix_kernel<1>, grid, dim3(256), 0, s, in, out, n_out); break;
    case 2: hipLaunchKernelGGL(mix_kernel<2>, grid, dim3(256), 0, s, in, out, n_out); break;
    case 3: hipLaunchKernelGGL(mix_kernel<3>, grid, dim3(256), 0, s, in, out, n_out); break;
    case 4: hipLaunchKernelGGL(mix_kernel<4>, grid, dim3(256), 0, s, in, out, n_out); break;
    case 5: hipLaunchKernelGGL(mix_kernel<5>, grid, dim3(256), 0, s, in, out, n_out); break;
    case 6: hipLaunchKernelGGL(mix_kernel<6>, grid, dim3(256), 0, s, in, out, n_out); break;
    case 7: hipLaunchKernelGGL(mix_kernel<7>, grid, dim3(256), 0, s, in, out, n_out); break;
    default: hipLaunchKernelGGL(mix_kernel<8>, grid, dim3(256), 0, s, in, out, n_out); break;
  }
  return (int)hipGetLastError();
}
