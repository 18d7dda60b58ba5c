// Calibration kernel for the benchmark (not part of the MLA path): a plain
// streaming read of a device buffer, the rate against which the decode
// kernels' cache stream is compared. Every lane reads 16-byte pieces in a
// grid-stride loop, four independent loads in flight per iteration, and
// folds them into one word per thread so the loads are not removed.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n,
                                                         uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n; i += stride) acc ^= p[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned) of `buf` once with
// `grid` workgroups of 256 threads; `out` receives grid * 256 words. Between
// the optional events (recorded by the launch itself) lies exactly the
// kernel. Returns 0, or -1 on invalid arguments, -2 on a launch failure.
int mla_calib_stream_read(const void* buf, size_t bytes, void* out, int grid,
                          hipEvent_t begin, hipEvent_t end, hipStream_t stream) {
  if (!buf || !out || grid <= 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0) return -1;
  (void)hipGetLastError();
  hipExtLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, stream, begin, end, 0,
                        (const u32x4*)buf, bytes / 16, (uint32_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
