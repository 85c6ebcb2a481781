// Read-stream reference kernel: the attainable HBM read rate of this GPU,
// against which the attention kernel's KV rate is also reported (the
// attention kernel streams every KV byte once, so a plain read of the same
// kind of traffic is its practical ceiling).  Not part of the attention
// method.
//
// gfx950 mapping: workgroup b reads one contiguous chunk of the buffer,
// 256 threads x 16 bytes per load with eight loads in flight per thread,
// all non-temporal (read once, like KV).  The loaded words are folded with
// XOR into one value per workgroup, written to sink[b], so the loads stay
// live.
#include "lbp_internal.h"

namespace lbp {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

typedef int i32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kStreamThreads) void read_stream_kernel(const i32x4_t* __restrict__ src,
                                                                     int64_t n16,
                                                                     int32_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t begin = int64_t(blockIdx.x) * per;
  const int64_t end = begin + per < n16 ? begin + per : n16;
  i32x4_t acc = {0, 0, 0, 0};
  for (int64_t i = begin + threadIdx.x; i < end; i += int64_t(kStreamThreads) * kStreamUnroll) {
    i32x4_t v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t j = i + int64_t(u) * kStreamThreads;
      v[u] = j < end ? __builtin_nontemporal_load(src + j) : i32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
  }
  int x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
  __shared__ int part[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_read_stream(const void* src, int64_t n16, int32_t* sink, int blocks,
                              hipStream_t s) {
  if (n16 <= 0 || blocks <= 0) return hipSuccess;
  const i32x4_t* p = static_cast<const i32x4_t*>(src);
  void* args[] = {&p, &n16, &sink};
  return hipLaunchKernel(reinterpret_cast<const void*>(&read_stream_kernel), dim3(blocks),
                         dim3(kStreamThreads), args, 0, s);
}

}  // namespace lbp
