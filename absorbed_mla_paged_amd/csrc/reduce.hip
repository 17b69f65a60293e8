// LSE-weighted reduce of split-KV partials on gfx950.
//
// For request b and head h, over its rows r (request-major, row_indptr):
//   M = max_r lse2_r;  w_r = 2^(lse2_r - M);
//   out = (sum_r w_r O_r) / (sum_r w_r)  rounded once to fp16 / bf16;
//   lse2_out = M + log2(sum_r w_r);  M = -inf gives out = 0, lse2 = -inf.
// (vllm-metal pull request 601 "[kernel] Wire MLA split-KV decode", "What
// changed"; base-2 LSEs and request-major rows per mlxcel pull request 995,
// "How #898's merge kernel is reused"; zero weight for rows with no visible
// key and a single rounding after the merge per MTPLX pull request 639.)
//
// One workgroup handles (b, h, a 32-dim slice): 32 row lanes x 8 threads,
// each thread owning 4 consecutive dims (one 16-byte load per row), so a
// row's slice is one 128-byte line. Row lane k takes rows k, k+32, ... in
// order, with 8 rows' loads issued before any is used, so a request's whole
// partial set is in flight at once; the 32 row-lane sums are then added in a
// fixed order, so the result is bit-identical run to run.
#include "device_common.h"
#include "internal.h"

#include <cmath>

namespace mla {
namespace {

using namespace dev;

constexpr int LAT = MLA_KV_LORA_RANK;
constexpr int SLICE = 32;                 // dims per workgroup
constexpr int SLICES = LAT / SLICE;       // 16
constexpr int TPR = SLICE / 4;            // threads per row: 8
constexpr int RL = 32;                    // row lanes
constexpr int THREADS = TPR * RL;         // 256
constexpr int UNROLL = 8;                 // rows in flight per thread

struct ReduceArgs {
  const float* partial_out;
  const float* partial_lse2;
  const int32_t* row_indptr;
  void* out;
  float* lse2_out;
  int32_t batch;
  int32_t heads;
  int32_t total_rows;
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int DT>
__global__ __launch_bounds__(THREADS) void reduce_kernel(ReduceArgs a) {
  typedef Elem<DT> E;
  __shared__ float red[THREADS / 64];
  __shared__ f32x4 part[RL][TPR];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x / SLICES;
  const int slice = blockIdx.x % SLICES;
  const int b = bh / a.heads;
  const int h = bh % a.heads;
  if (b >= a.batch) return;
  int r0 = a.row_indptr[b];
  int r1 = a.row_indptr[b + 1];
  r0 = max(0, min(r0, a.total_rows));
  r1 = max(r0, min(r1, a.total_rows));
  const int nr = r1 - r0;

  // M and W = sum_r 2^(lse2_r - M), each in a fixed order.
  float mx = -INFINITY;
  for (int r = tid; r < nr; r += THREADS)
    mx = fmaxf(mx, a.partial_lse2[(int64_t)(r0 + r) * a.heads + h]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < THREADS / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();

  const int c4 = tid % TPR;    // which 4 dims of the slice
  const int rl = tid / TPR;    // which row lane
  const int d0 = slice * SLICE + c4 * 4;
  const int64_t oidx = ((int64_t)b * a.heads + h) * LAT + d0;

  if (M == -INFINITY) {
    // Nothing visible in any row: zeros and -inf, never NaN.
    if (rl == 0) {
      typename E::vec4 z;
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] = static_cast<typename E::scalar>(0.0f);
      *reinterpret_cast<typename E::vec4*>(reinterpret_cast<uint16_t*>(a.out) + oidx) = z;
    }
    if (a.lse2_out && slice == 0 && tid == 0) a.lse2_out[(int64_t)b * a.heads + h] = -INFINITY;
    return;
  }

  float wsum = 0.f;
  for (int r = tid; r < nr; r += THREADS)
    wsum += __builtin_amdgcn_exp2f(a.partial_lse2[(int64_t)(r0 + r) * a.heads + h] - M);
  wsum = wave_sum(wsum);
  if ((tid & 63) == 0) red[tid >> 6] = wsum;
  __syncthreads();
  float W = red[0];
#pragma unroll
  for (int w = 1; w < THREADS / 64; ++w) W += red[w];

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int rb = rl; rb < nr; rb += RL * UNROLL) {
    f32x4 v[UNROLL];
    float lw[UNROLL];
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int r = rb + j * RL;
      const int64_t row = r0 + min(r, nr - 1);
      lw[j] = a.partial_lse2[row * a.heads + h];
      v[j] = *reinterpret_cast<const f32x4*>(a.partial_out + (row * a.heads + h) * LAT + d0);
    }
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      if (rb + j * RL < nr) acc += __builtin_amdgcn_exp2f(lw[j] - M) * v[j];
    }
  }
  part[rl][c4] = acc;
  __syncthreads();
  if (rl == 0) {
    f32x4 tot = part[0][c4];
#pragma unroll
    for (int k = 1; k < RL; ++k) tot += part[k][c4];
    const float inv = 1.0f / W;
    typename E::vec4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = static_cast<typename E::scalar>(tot[j] * inv);
    *reinterpret_cast<typename E::vec4*>(reinterpret_cast<uint16_t*>(a.out) + oidx) = o;
    if (a.lse2_out && slice == 0 && c4 == 0)
      a.lse2_out[(int64_t)b * a.heads + h] = M + __builtin_amdgcn_logf(W);
  }
}

bool aligned(const void* p, uintptr_t k) { return (reinterpret_cast<uintptr_t>(p) % k) == 0; }

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int mla_decode_reduce(const float* partial_out, const float* partial_lse2,
                                 const int32_t* row_indptr, int32_t batch, int32_t num_heads,
                                 int32_t total_rows, int32_t dtype, void* out, float* lse2_out,
                                 hipStream_t stream) {
  clear_error();
  if (batch < 0 || total_rows < 0) return fail(MLA_E_SHAPE, "batch %d, total_rows %d", batch, total_rows);
  if (num_heads < MLA_MIN_HEADS || num_heads > MLA_MAX_HEADS || num_heads % 16)
    return fail(MLA_E_UNSUPPORTED, "num_heads %d (need a multiple of 16 in [16, 128])",
                num_heads);
  if (dtype != MLA_F16 && dtype != MLA_BF16) return fail(MLA_E_UNSUPPORTED, "dtype %d", dtype);
  if (batch == 0) return MLA_OK;
  if (!row_indptr || !out || (total_rows > 0 && (!partial_out || !partial_lse2)))
    return fail(MLA_E_NULL, "null pointer");
  if (!aligned(out, 16) || (partial_out && !aligned(partial_out, 16)) ||
      (partial_lse2 && !aligned(partial_lse2, 4)) || !aligned(row_indptr, 4) ||
      (lse2_out && !aligned(lse2_out, 4)))
    return fail(MLA_E_ALIGN, "misaligned buffer");
  const int64_t wgs = (int64_t)batch * num_heads * SLICES;
  if (wgs > INT32_MAX) return fail(MLA_E_SHAPE, "grid too large");
  ReduceArgs a;
  a.partial_out = partial_out;
  a.partial_lse2 = partial_lse2;
  a.row_indptr = row_indptr;
  a.out = out;
  a.lse2_out = lse2_out;
  a.batch = batch;
  a.heads = num_heads;
  a.total_rows = total_rows;
  if (dtype == MLA_F16)
    hipLaunchKernelGGL(reduce_kernel<0>, dim3((unsigned)wgs), dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(reduce_kernel<1>, dim3((unsigned)wgs), dim3(THREADS), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_E_HIP, "reduce launch: %s", hipGetErrorString(e));
  count(2, 1);
  return MLA_OK;
}
