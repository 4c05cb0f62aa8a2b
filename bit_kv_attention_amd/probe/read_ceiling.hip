// read_ceiling.hip -- the plain HBM read ceiling, for judging the scan's
// fraction of the read bandwidth it could reach: every workgroup streams a
// contiguous slice of a buffer with 16-byte loads, four in flight per lane,
// and folds what it read into one word (so no load is dead).  Measurement
// infrastructure for bench.py --read-ceiling; not part of libbitkv.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512) void read_kernel(const u32x4* __restrict__ src, size_t n16, uint32_t* __restrict__ out) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;  // 16-byte items per workgroup
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = lo + threadIdx.x;
  for (; i + 3 * 512 < hi; i += 4 * 512) {
    const u32x4 a = src[i], b = src[i + 512], c = src[i + 1024], d = src[i + 1536];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < hi; i += 512) acc ^= src[i];
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == 0x9E3779B9u) out[blockIdx.x] = v;  // (data-dependent, so the loads stay)
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at device address src once with `grid`
// workgroups of 512 threads on `stream`; out: grid words of device memory.
// Returns the launch's hipError_t.
int bkv_probe_read(const void* src, size_t bytes, uint32_t* out, int grid, void* stream) {
  if (!src || !out || grid <= 0 || bytes % 16) return (int)hipErrorInvalidValue;
  (void)hipGetLastError();
  read_kernel<<<grid, 512, 0, (hipStream_t)stream>>>(static_cast<const u32x4*>(src), bytes / 16, out);
  return (int)hipGetLastError();
}

}
