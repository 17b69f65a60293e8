// The per-head products on either side of absorbed decode, on gfx950:
//   fold:    q_absorbed[b, h, :] = q_nope[b, h, :] . W_UK[h]     (128 -> 512)
//   unfold:  o[b, h, :]          = out[b, h, :]    . W_UV^T[h]   (512 -> 128)
// (mlxcel pull request 995, "What changed", the absorb.rs bullet: kv_b_proj
// splits into W_UK [H, qk_nope, r] applied on the query side and W_UV^T
// [H, r, v_head] applied to the latent output; qk_nope = v_head = 128.)
//
// At decode sizes each weight element meets a handful of rows, so both are
// bound by reading the weights once from HBM (H x 128 x 512 x 2 bytes per
// call). They still run on the matrix cores: a vector-ALU version (fp32
// multiply-adds per weight element, then cross-lane sums of each row's
// slices) measured 11.2 and 15.8 us for 8 rows of 128 heads, where these
// take 6.5 and 6.7 us, and it was no faster for one row.
#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

using namespace dev;

constexpr int THREADS = 256;
constexpr int NOPE = 128;              // qk_nope = v_head

struct ProjArgs {
  const uint16_t* x;   // [rows, H, K]
  const uint16_t* w;   // [H, K, N]
  uint16_t* y;         // [rows, H, N]
  int32_t rows;
  int32_t heads;
};

// Per head, Y^T = W^T X^T: the weight chunk W[:, c0 .. c0 + NC) is the A
// operand (NC output columns x K inputs, read from LDS with the transposing 16-bit
// read, as V^T is in the decode kernels), the rows of X are the B operand
// (K x up to 16 rows, read straight from memory), and v_mfma_f32_16x16x32
// sums over K in fp32, so no cross-lane sums remain. Lane (j, g) of a result
// tile holds output columns 4 g .. + 4 of row j: one 8-byte store, after one
// rounding to the 16-bit type.
//
// One workgroup (4 waves) takes head h and NC columns: it copies the chunk
// (K x NC, 32 KB at most) into LDS once and keeps it for every 16-row tile
// of X. With at least 4 column tiles and at most 4 K-steps (the fold) the
// waves split the column tiles; otherwise they split the K-steps and their
// sums are added through LDS in wave order, so results are bit-identical
// run to run.
//
// LDS row k of the chunk holds its NC columns; 16-byte chunk c sits at
// c ^ mswz(k), so the 8 rows one transposing read takes from a pair of
// 16-lane groups ({0..3, 8..11} or {4..7, 12..15} of a K-step half) fall in
// distinct banks when the row has 16 chunks.
template <int CHUNKS>
__device__ __forceinline__ int mswz(int k) {
  if constexpr (CHUNKS >= 16) return (((k & 3) << 1) | ((k >> 3) & 1)) & (CHUNKS - 1);
  else return ((k >> 3) & 1) * (CHUNKS / 2);
}

template <int DT, int K, int N, int NC>
__global__ __launch_bounds__(THREADS) void head_mfma_kernel(ProjArgs a) {
  typedef Elem<DT> E;
  typedef typename E::vec8 vec8;
  typedef typename E::vec4 vec4;
  typedef typename E::scalar scalar;
  constexpr int ROWB = NC * 2;            // bytes per LDS row of the chunk
  constexpr int CHUNKS = ROWB / 16;
  constexpr int CT = NC / 16;             // column tiles
  constexpr int KST = K / 32;             // K-steps
  constexpr bool SPLIT_COLS = CT >= 4 && KST <= 4;
  constexpr int CT_W = SPLIT_COLS ? CT / 4 : CT;     // column tiles per wave
  constexpr int KS_W = SPLIT_COLS ? KST : KST / 4;   // K-steps per wave
  static_assert(SPLIT_COLS ? CT % 4 == 0 : KST % 4 == 0, "wave split");
  __shared__ __attribute__((aligned(16))) char wt[K * ROWB];
  __shared__ f32x4 red[SPLIT_COLS ? 1 : 4][CT][64];
  MLA_LDS char* wl = (MLA_LDS char*)wt;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int chunks = N / NC;
  const int h = blockIdx.x / chunks;
  const int c0 = (blockIdx.x % chunks) * NC;
  if (h >= a.heads) return;

  // B fragments of the first row tile: X[row, 32 ks + {4 lg .. + 4,
  // 16 + 4 lg .. + 4}] for this wave's K-steps, loaded together with the
  // weights so that both round trips overlap.
  auto xload = [&](int r0, u32x2 (&xl)[KS_W], u32x2 (&xh)[KS_W]) {
    const int row = r0 + ln;
    const uint16_t* xrow = a.x + ((int64_t)min(row, a.rows - 1) * a.heads + h) * K;
#pragma unroll
    for (int kk = 0; kk < KS_W; ++kk) {
      const int ks = SPLIT_COLS ? kk : wave * KS_W + kk;
      xl[kk] = u32x2{0u, 0u};
      xh[kk] = u32x2{0u, 0u};
      if (row < a.rows) {
        xl[kk] = *reinterpret_cast<const u32x2*>(xrow + 32 * ks + 4 * lg);
        xh[kk] = *reinterpret_cast<const u32x2*>(xrow + 32 * ks + 16 + 4 * lg);
      }
    }
  };
  u32x2 xl[KS_W], xh[KS_W];
  // The weight chunk: every thread's loads issued at once (16 bytes each),
  // then stored into swizzled LDS rows.
  constexpr int WLOADS = K * CHUNKS / THREADS;
  static_assert(K * CHUNKS % THREADS == 0, "chunk loads per thread");
  const uint16_t* wsrc = a.w + (int64_t)h * K * N + c0;
  u32x4 wv[WLOADS];
#pragma unroll
  for (int j = 0; j < WLOADS; ++j) {
    const int i = tid + j * THREADS;
    wv[j] = *reinterpret_cast<const u32x4*>(wsrc + (int64_t)(i / CHUNKS) * N + (i % CHUNKS) * 8);
  }
  xload(0, xl, xh);
#pragma unroll
  for (int j = 0; j < WLOADS; ++j) {
    const int i = tid + j * THREADS;
    const int k = i / CHUNKS, c = i % CHUNKS;
    *(MLA_LDS u32x4*)(wl + k * ROWB + ((c ^ mswz<CHUNKS>(k)) * 16)) = wv[j];
  }
  __syncthreads();

  // A fragment (column tile ct, K-step ks): in each 16-lane group, lane
  // 4 t + p addresses row 32 ks + 4 lg + t (then + 16), columns
  // 16 ct + 4 p .. + 4; the read hands lane (j, lg) column 16 ct + j at
  // K = 32 ks + {4 lg .. + 4, 16 + 4 lg .. + 4}.
  auto afrag = [&](int ct, int ks) {
    const int t = ln >> 2, p = ln & 3;
    const int k1 = 32 * ks + 4 * lg + t;
    const int c = (32 * ct + 8 * p) / 16, half = p & 1;
    const uint32_t a1 = lds_addr(wl) + k1 * ROWB + ((c ^ mswz<CHUNKS>(k1)) * 16) + half * 8;
    const int k2 = k1 + 16;
    const uint32_t a2 = lds_addr(wl) + k2 * ROWB + ((c ^ mswz<CHUNKS>(k2)) * 16) + half * 8;
    const u32x2 lo = lds_read_tr_b16(a1);
    const u32x2 hi = lds_read_tr_b16(a2);
    u32x2 l2 = lo, h2 = hi;
    lds_wait<0>(l2, h2);
    return __builtin_bit_cast(vec8, u32x4{l2[0], l2[1], h2[0], h2[1]});
  };

  for (int r0 = 0; r0 < a.rows; r0 += 16) {
    const int row = r0 + ln;              // this lane's row of X (B operand column)
    const bool live = row < a.rows;
    if (r0 > 0) xload(r0, xl, xh);
    f32x4 acc[CT_W];
#pragma unroll
    for (int c = 0; c < CT_W; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS_W; ++kk) {
      const int ks = SPLIT_COLS ? kk : wave * KS_W + kk;
      const vec8 xb = __builtin_bit_cast(vec8, u32x4{xl[kk][0], xl[kk][1], xh[kk][0], xh[kk][1]});
#pragma unroll
      for (int c = 0; c < CT_W; ++c) {
        const int ct = SPLIT_COLS ? wave * CT_W + c : c;
        acc[c] = E::mfma(afrag(ct, ks), xb, acc[c]);
      }
    }
    // Lane (j, g) of tile ct: columns 16 ct + 4 g .. + 4 of row r0 + j.
    auto put = [&](int ct, f32x4 v) {
      if (!live) return;
      vec4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = static_cast<scalar>(v[e]);
      *reinterpret_cast<vec4*>(a.y + ((int64_t)row * a.heads + h) * N + c0 + 16 * ct + 4 * lg) = o;
    };
    if constexpr (SPLIT_COLS) {
#pragma unroll
      for (int c = 0; c < CT_W; ++c) put(wave * CT_W + c, acc[c]);
    } else {
      // Sum the waves' K-step shares in wave order.
#pragma unroll
      for (int c = 0; c < CT_W; ++c) red[wave][c][lane] = acc[c];
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int c = 0; c < CT_W; ++c) {
          f32x4 s = red[0][c][lane];
#pragma unroll
          for (int w = 1; w < 4; ++w) s += red[w][c][lane];
          put(c, s);
        }
      }
      __syncthreads();   // red is reused by the next row tile
    }
  }
}

bool aligned(const void* p, uintptr_t k) { return (reinterpret_cast<uintptr_t>(p) % k) == 0; }

// Workgroups that fill the 256 CUs of one MI355X.
constexpr int64_t kFillWorkgroups = 256;

// Column chunks of NC when that still fills the device (half as many
// workgroups for chunks of 64+ columns, which hold more LDS), else of
// NC_NARROW.
template <int K, int N, int NC, int NC_NARROW>
int launch(const char* what, const void* x, const void* w, void* y, int32_t rows, int32_t heads,
           int32_t dtype, hipStream_t stream) {
  clear_error();
  if (rows < 0 || heads < 1 || heads > MLA_MAX_HEADS * MLA_MAX_QLEN)
    return fail(MLA_E_SHAPE, "%s: rows %d, heads %d", what, rows, heads);
  if (dtype != MLA_F16 && dtype != MLA_BF16) return fail(MLA_E_UNSUPPORTED, "dtype %d", dtype);
  if (rows == 0) return MLA_OK;
  if (!x || !w || !y) return fail(MLA_E_NULL, "%s: null pointer", what);
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16))
    return fail(MLA_E_ALIGN, "%s: tensors must be 16-byte aligned", what);
  ProjArgs a{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
             static_cast<uint16_t*>(y), rows, heads};
  const bool big = (int64_t)heads * (N / NC) >= kFillWorkgroups / (NC > 32 ? 2 : 1);
  const dim3 grid((unsigned)((int64_t)heads * (N / (big ? NC : NC_NARROW))));
  if (dtype == MLA_F16 && big)
    hipLaunchKernelGGL((head_mfma_kernel<0, K, N, NC>), grid, dim3(THREADS), 0, stream, a);
  else if (dtype == MLA_F16)
    hipLaunchKernelGGL((head_mfma_kernel<0, K, N, NC_NARROW>), grid, dim3(THREADS), 0, stream, a);
  else if (big)
    hipLaunchKernelGGL((head_mfma_kernel<1, K, N, NC>), grid, dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((head_mfma_kernel<1, K, N, NC_NARROW>), grid, dim3(THREADS), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int mla_absorb_query(const void* q_nope, const void* w_uk, void* q_absorbed,
                                int32_t rows, int32_t num_heads, int32_t dtype,
                                hipStream_t stream) {
  return launch<NOPE, MLA_KV_LORA_RANK, 128, 32>("mla_absorb_query", q_nope, w_uk, q_absorbed,
                                                rows, num_heads, dtype, stream);
}

extern "C" int mla_unabsorb_output(const void* out_latent, const void* w_uv_t, void* o,
                                   int32_t rows, int32_t num_heads, int32_t dtype,
                                   hipStream_t stream) {
  return launch<MLA_KV_LORA_RANK, NOPE, 64, 16>("mla_unabsorb_output", out_latent, w_uv_t, o,
                                               rows, num_heads, dtype, stream);
}
