// mla_copy_probe: a measurement helper, not part of the decode. It moves
// the KV of paged rows into LDS the way the partition kernels' copies do
// (global_load_lds_dwordx4, 1 KB per instruction: the 32 ckv rows and 4 kpe
// pieces of each 32-token block), and nothing else, so that the rate the
// memory path gives such copies can be measured apart from any arithmetic:
// with one workgroup per row (every block read by one CU) or with G
// workgroups per row on one XCD (every block read by G CUs, as the 64-head
// workgroups of a 128-head row do), and with a given number of copying
// waves and copies each wave keeps in flight.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

using namespace dev;

constexpr int THREADS = 512;
constexpr int RING_KB = 128;   // LDS ring, split among the copying waves

template <int WAVES, int INFLIGHT>
__global__ __launch_bounds__(THREADS, 1) void copy_probe_kernel(const char* ckv, const char* kpe,
                                                               const int32_t* table, int rows,
                                                               int blocks, int groups,
                                                               int num_blocks) {
  __shared__ __attribute__((aligned(1024))) char ring[RING_KB * 1024];
  // The partition kernels' layout: slot u = row, head group hg, and the G
  // groups of one row on one XCD.
  const int sl = blockIdx.x >> 3;
  const int u = (sl / groups) * 8 + (blockIdx.x & 7);
  if (u >= rows) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= WAVES) return;
  constexpr int SLOTS = RING_KB / WAVES;   // 1 KB slots per wave
  const uint32_t lds0 = lds_addr((MLA_LDS char*)ring) + wave * SLOTS * 1024;
  int j = 0;
  for (int k = 0; k < blocks; ++k) {
    const int64_t phys =
        max(0, min(load_const(table, (int64_t)u * blocks + k), num_blocks - 1));
    for (int c = wave; c < 36; c += WAVES) {
      const char* src = c < 32 ? ckv + phys * 32768 + c * 1024 : kpe + phys * 4096 + (c - 32) * 1024;
      dma16s(lane * 16, src, lds0 + (j % SLOTS) * 1024);
      ++j;
      wait_vmcnt<INFLIGHT - 1>();
    }
  }
  wait_vmcnt<0>();
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int mla_copy_probe(const void* ckv_pool, const void* kpe_pool, int32_t num_blocks,
                              const int32_t* table, int32_t rows, int32_t blocks_per_row,
                              int32_t groups, int32_t waves, int32_t inflight,
                              hipStream_t stream) {
  clear_error();
  if (!ckv_pool || !kpe_pool || !table) return fail(MLA_E_NULL, "null pointer");
  if (rows < 1 || blocks_per_row < 1 || num_blocks < 1 || (groups != 1 && groups != 2 &&
                                                           groups != 4))
    return fail(MLA_E_SHAPE, "rows %d, blocks per row %d, num_blocks %d, groups %d", rows,
                blocks_per_row, num_blocks, groups);
  if ((int64_t)rows * blocks_per_row > INT32_MAX || (int64_t)rows * groups > INT32_MAX / 2)
    return fail(MLA_E_SHAPE, "too large");
  using K = void (*)(const char*, const char*, const int32_t*, int, int, int, int);
  K k = nullptr;
  if (waves == 4 && inflight == 4) k = copy_probe_kernel<4, 4>;
  else if (waves == 4 && inflight == 8) k = copy_probe_kernel<4, 8>;
  else if (waves == 4 && inflight == 16) k = copy_probe_kernel<4, 16>;
  else if (waves == 8 && inflight == 4) k = copy_probe_kernel<8, 4>;
  else if (waves == 8 && inflight == 8) k = copy_probe_kernel<8, 8>;
  else if (waves == 8 && inflight == 16) k = copy_probe_kernel<8, 16>;
  else return fail(MLA_E_UNSUPPORTED, "waves %d, inflight %d (4 or 8; 4, 8 or 16)", waves, inflight);
  const int64_t wgs = (((int64_t)rows + 7) / 8) * 8 * groups;
  hipLaunchKernelGGL(k, dim3((unsigned)wgs), dim3(THREADS), 0, stream,
                     static_cast<const char*>(ckv_pool), static_cast<const char*>(kpe_pool), table,
                     rows, blocks_per_row, groups, num_blocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_E_HIP, "copy probe launch: %s", hipGetErrorString(e));
  return MLA_OK;
}
