// mla_stream_read: a plain, contiguous read of device memory, as the
// reference for what a launch that only reads can reach on this device at a
// given byte count. It is not part of the decode; the benchmark times it
// over the same bytes as each partition launch and reports the kernel's
// rate against it as well as against the 8 TB/s data-sheet peak.
//
// 4096 workgroups of 256 threads (16 per CU) stride through the buffer with
// one 16-byte load per thread and iteration: the launch shape that read
// fastest among 256..4096 workgroups and 1..4 loads per iteration at
// 40-600 MB on MI355X. Each thread folds the words it loaded with XOR and
// stores the fold only if it equals a value the caller passes and no fold
// of the data can take, so the loads cannot be dropped and nothing is
// written.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kGrid = 4096;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* src, size_t bytes,
                                                               uint32_t* sink, uint32_t never) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * kThreads * 16;
  for (size_t off = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 16; off + 16 <= bytes;
       off += stride)
    acc ^= *reinterpret_cast<const u32x4*>(src + off);
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == never) sink[0] = v;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int mla_stream_read(const void* src, size_t bytes, uint32_t* sink, uint32_t never,
                               hipStream_t stream) {
  clear_error();
  if (bytes == 0) return MLA_OK;
  if (!src || !sink) return fail(MLA_E_NULL, "null pointer");
  if (reinterpret_cast<uintptr_t>(src) % 16 || bytes % 16)
    return fail(MLA_E_ALIGN, "source and byte count must be multiples of 16");
  hipLaunchKernelGGL(stream_read_kernel, dim3(kGrid), dim3(kThreads), 0, stream,
                     static_cast<const char*>(src), bytes, sink, never);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_E_HIP, "stream read launch: %s", hipGetErrorString(e));
  return MLA_OK;
}
