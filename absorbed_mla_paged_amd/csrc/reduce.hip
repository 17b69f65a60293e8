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
// One workgroup handles (b, h, a slice of 32, 64 or 256 dims): 256 threads
// as row lanes x (slice / 4) threads, each thread owning 4 consecutive dims
// (one 16-byte load per row), so a row's slice is one 128-, 256- or
// 1024-byte piece. Row lane k takes rows k, k + RL, ... in order, with 8 rows' loads
// (slice and lse2) issued before any is used, so a request's whole partial
// set is in flight at once, in a single round trip. Each row lane keeps its
// own running maximum, weighted sum and weight; the row lanes are then
// merged in a fixed tree order (lane shuffles, then the four waves), so the
// result is bit-identical run to run. The launch takes 64-dim slices when
// that still gives at least 1024 workgroups (many heads: fewer, wider
// workgroups), else 32-dim ones (16 heads: more workgroups in flight); and
// 256-dim slices when requests have 32 rows or fewer on average (a batch of
// many requests: 4 row lanes x 8 rows hold them, and far fewer workgroups
// of mostly idle lanes are launched).
#include "device_common.h"
#include "internal.h"

#include <cmath>

namespace mla {
namespace {

using namespace dev;

constexpr int LAT = MLA_KV_LORA_RANK;
constexpr int THREADS = 256;
constexpr int UNROLL = 8;                 // rows in flight per thread
constexpr int WIDE_MIN_WGS = 1024;        // 64-dim slices from this many workgroups
// Requests of at most this many rows on average (all of them one load batch
// of 4 row lanes x 8) take 256-dim slices: 4 waves, one row lane each.
constexpr int FEW_ROWS = 32;
constexpr int FEW_ROWS_MIN_WGS = 256;

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

template <int DT, int SLICE>
__global__ __launch_bounds__(THREADS) void reduce_kernel(ReduceArgs a) {
  constexpr int SLICES = LAT / SLICE;     // workgroups per (request, head)
  constexpr int TPR = SLICE / 4;          // threads per row
  constexpr int RL = THREADS / TPR;       // row lanes
  static_assert(SLICE == 32 || SLICE == 64 || SLICE == 256, "slice width");
  typedef Elem<DT> E;
  __shared__ f32x4 part[THREADS / 64][TPR];
  __shared__ float lane_m[THREADS / 64], lane_w[THREADS / 64];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x / SLICES;
  const int slice = blockIdx.x % SLICES;
  const int b = bh / a.heads;
  const int h = bh % a.heads;
  if (b >= a.batch) return;
  // row_indptr[0] = 0 and row_indptr[batch] = total_rows by contract, so a
  // single request needs no load before its partials.
  int r0 = b == 0 ? 0 : a.row_indptr[b];
  int r1 = b == a.batch - 1 ? a.total_rows : a.row_indptr[b + 1];
  r0 = max(0, min(r0, a.total_rows));
  r1 = max(r0, min(r1, a.total_rows));
  const int nr = r1 - r0;

  const int c4 = tid % TPR;    // which 4 dims of the slice
  const int rl = tid / TPR;    // which row lane
  const int d0 = slice * SLICE + c4 * 4;
  const int64_t oidx = ((int64_t)b * a.heads + h) * LAT + d0;

  // Running merge of this row lane's rows: maximum m, sum of 2^(lse - m) O
  // and of 2^(lse - m). Rows with lse2 = -inf (no visible token) weigh 0.
  float m = -INFINITY, w = 0.f;
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
    float bm = m;
#pragma unroll
    for (int j = 0; j < UNROLL; ++j)
      if (rb + j * RL < nr) bm = fmaxf(bm, lw[j]);
    if (bm > m) {   // bm is finite here
      const float alpha = __builtin_amdgcn_exp2f(m - bm);   // 0 when m = -inf
      acc *= alpha;
      w *= alpha;
      m = bm;
    }
    if (m != -INFINITY) {
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        if (rb + j * RL < nr) {
          const float e = __builtin_amdgcn_exp2f(lw[j] - m);
          acc += e * v[j];
          w += e;
        }
      }
    }
  }
  // Merge the row lanes: first those of each wave through lane shuffles
  // (the lane bits above the thread-in-row bits), then the 4 waves through
  // LDS, each in a fixed order.
  auto merge = [&](float m2, float w2, f32x4 acc2) {
    const float mn = fmaxf(m, m2);
    const float s1 = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    const float s2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
    acc = s1 * acc + s2 * acc2;
    w = s1 * w + s2 * w2;
    m = mn;
  };
#pragma unroll
  for (int x = TPR; x < 64; x <<= 1) {
    f32x4 acc2;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc2[j] = shfl_xor(acc[j], x);
    merge(shfl_xor(m, x), shfl_xor(w, x), acc2);
  }
  const int wv = tid >> 6;
  if ((tid & 63) < TPR) {
    part[wv][c4] = acc;
    if (c4 == 0) {
      lane_m[wv] = m;
      lane_w[wv] = w;
    }
  }
  __syncthreads();
  if (tid >= TPR) return;
  // Thread c4 of wave 0 (its own merged state is wave 0's entry).
#pragma unroll
  for (int k = 1; k < THREADS / 64; ++k) merge(lane_m[k], lane_w[k], part[k][c4]);
  const float M = m;
  if (M == -INFINITY) {
    // Nothing visible in any row: zeros and -inf, never NaN.
    typename E::vec4 z;
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = static_cast<typename E::scalar>(0.0f);
    *reinterpret_cast<typename E::vec4*>(reinterpret_cast<uint16_t*>(a.out) + oidx) = z;
    if (a.lse2_out && slice == 0 && c4 == 0) a.lse2_out[(int64_t)b * a.heads + h] = -INFINITY;
    return;
  }
  const f32x4 tot = acc;
  const float W = w;
  const float inv = 1.0f / W;
  typename E::vec4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = static_cast<typename E::scalar>(tot[j] * inv);
  *reinterpret_cast<typename E::vec4*>(reinterpret_cast<uint16_t*>(a.out) + oidx) = o;
  if (a.lse2_out && slice == 0 && c4 == 0)
    a.lse2_out[(int64_t)b * a.heads + h] = M + __builtin_amdgcn_logf(W);
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
  // num_heads counts query rows per request: q_len * heads.
  if (num_heads < MLA_MIN_HEADS || num_heads > MLA_MAX_HEADS * MLA_MAX_QLEN || num_heads % 16)
    return fail(MLA_E_UNSUPPORTED, "num_heads %d (need a multiple of 16 in [16, %d])",
                num_heads, MLA_MAX_HEADS * MLA_MAX_QLEN);
  if (dtype != MLA_F16 && dtype != MLA_BF16) return fail(MLA_E_UNSUPPORTED, "dtype %d", dtype);
  if (batch == 0) return MLA_OK;
  if (!row_indptr || !out || (total_rows > 0 && (!partial_out || !partial_lse2)))
    return fail(MLA_E_NULL, "null pointer");
  if (!aligned(out, 16) || (partial_out && !aligned(partial_out, 16)) ||
      (partial_lse2 && !aligned(partial_lse2, 4)) || !aligned(row_indptr, 4) ||
      (lse2_out && !aligned(lse2_out, 4)))
    return fail(MLA_E_ALIGN, "misaligned buffer");
  const bool wide = (int64_t)batch * num_heads * (LAT / 64) >= WIDE_MIN_WGS;
  const bool few = total_rows <= (int64_t)FEW_ROWS * batch &&
                   (int64_t)batch * num_heads * (LAT / 256) >= FEW_ROWS_MIN_WGS;
  const int slice = few ? 256 : wide ? 64 : 32;
  const int64_t wgs = (int64_t)batch * num_heads * (LAT / slice);
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
  auto kernel = dtype == MLA_F16
                    ? (few ? reduce_kernel<0, 256> : wide ? reduce_kernel<0, 64> : reduce_kernel<0, 32>)
                    : (few ? reduce_kernel<1, 256> : wide ? reduce_kernel<1, 64> : reduce_kernel<1, 32>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(THREADS), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_E_HIP, "reduce launch: %s", hipGetErrorString(e));
  count(2, 1);
  return MLA_OK;
}
