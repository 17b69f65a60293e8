// mla_decode_noalloc: the split decode (partition launch, then the reduce)
// with its fp32 partial workspace in a fixed device array of this library
// instead of caller memory, for callers that cannot allocate.
//
// The array lives in the code object (one copy per GPU the library runs
// on, held until the process ends). Host code never passes the array's name
// to a kernel: on the host that name is only a stand-in, not a device
// address. Each device's address of the array is looked up once, with that
// device current, and every launch takes that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace mla {
namespace {

constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device, with that device current).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_E_HIP, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MLA_E_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

constexpr size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" size_t mla_noalloc_scratch_bytes(int32_t total_rows, int32_t num_heads,
                                            int32_t q_len) {
  if (total_rows < 0 || num_heads < 0 || q_len < 0) return 0;
  const size_t qrows = (size_t)num_heads * (size_t)q_len;
  return align256((size_t)total_rows * qrows * MLA_KV_LORA_RANK * sizeof(float)) +
         (size_t)total_rows * qrows * sizeof(float);
}

extern "C" int mla_decode_noalloc(
    const void* q_absorbed, const void* q_pe, const void* ckv_cache, const void* kpe_cache,
    int32_t num_blocks, int32_t block_size, const int32_t* block_table,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch, int32_t num_heads,
    int32_t q_len, float scale, int32_t dtype, const int32_t* partitions, const int32_t* splits,
    const int32_t* row_indptr, int32_t total_rows, int32_t max_rows_per_req,
    int32_t heads_per_wg, void* out, float* lse2_out, hipStream_t stream) {
  clear_error();
  if (batch < 0 || total_rows < 0 || num_heads < 0 || q_len < 0)
    return fail(MLA_E_SHAPE, "batch %d, total_rows %d, num_heads %d, q_len %d", batch,
                total_rows, num_heads, q_len);
  if (batch == 0) return MLA_OK;
  if (total_rows == batch) {
    // Single pass: every request is one row, written straight into `out`.
    return mla_decode_partition(q_absorbed, q_pe, ckv_cache, kpe_cache, num_blocks, block_size,
                                block_table, max_blocks_per_seq, context_lens, batch, num_heads,
                                q_len, scale, dtype, partitions, splits, row_indptr, total_rows,
                                max_rows_per_req, heads_per_wg, nullptr, nullptr, out, lse2_out,
                                nullptr, stream);
  }
  const size_t need = mla_noalloc_scratch_bytes(total_rows, num_heads, q_len);
  if (need > kScratchBytes)
    return fail(MLA_E_WORKSPACE,
                "partials of %d rows x %d query rows need %zu bytes; the fixed scratch holds %zu",
                total_rows, num_heads * q_len, need, kScratchBytes);
  // What the reduce will check, checked before the partition launch, so a
  // refused call launches nothing.
  if (!out) return fail(MLA_E_NULL, "null `out`");
  if (reinterpret_cast<uintptr_t>(out) % 16 || reinterpret_cast<uintptr_t>(lse2_out) % 4)
    return fail(MLA_E_ALIGN, "out (16 bytes) or lse2_out (4 bytes) misaligned");
  if ((int64_t)batch * num_heads * q_len * (MLA_KV_LORA_RANK / 32) > INT32_MAX)
    return fail(MLA_E_SHAPE, "reduce grid too large");
  void* base = nullptr;
  int rc = scratch_address(&base);
  if (rc != MLA_OK) return rc;
  const size_t qrows = (size_t)num_heads * (size_t)q_len;
  float* partial_out = static_cast<float*>(base);
  float* partial_lse2 = reinterpret_cast<float*>(
      static_cast<char*>(base) + align256((size_t)total_rows * qrows * MLA_KV_LORA_RANK * 4));
  rc = mla_decode_partition(q_absorbed, q_pe, ckv_cache, kpe_cache, num_blocks, block_size,
                            block_table, max_blocks_per_seq, context_lens, batch, num_heads,
                            q_len, scale, dtype, partitions, splits, row_indptr, total_rows,
                            max_rows_per_req, heads_per_wg, partial_out, partial_lse2, nullptr,
                            nullptr, nullptr, stream);
  if (rc != MLA_OK) return rc;
  return mla_decode_reduce(partial_out, partial_lse2, row_indptr, batch, (int32_t)qrows,
                           total_rows, dtype, out, lse2_out, stream);
}
