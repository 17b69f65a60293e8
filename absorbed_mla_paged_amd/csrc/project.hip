// The per-head products on either side of absorbed decode, on gfx950:
//   fold:    q_absorbed[b, h, :] = q_nope[b, h, :] . W_UK[h]     (128 -> 512)
//   unfold:  o[b, h, :]          = out[b, h, :]    . W_UV^T[h]   (512 -> 128)
// (mlxcel pull request 995, "What changed", the absorb.rs bullet: kv_b_proj
// splits into W_UK [H, qk_nope, r] applied on the query side and W_UV^T
// [H, r, v_head] applied to the latent output; qk_nope = v_head = 128.)
//
// At decode sizes (a handful of rows per head) these are bound by reading
// the weights once from HBM, so the kernel streams each weight element once
// and does the few multiply-adds per element on the vector ALUs; matrix
// cores would wait on the same bytes.
//
// One workgroup (256 threads) takes head h and COLS output columns. Thread
// (ct, ks): columns 8 ct .. 8 ct + 8 (one 16-byte load per weight row) and
// the ks-th of 256 / (COLS / 8) slices of the K rows. The rows of X (up to 8
// per pass) sit in LDS as fp32. Each thread accumulates its slice in fp32,
// the slices are summed by lane shuffles inside a wave and then across the 4
// waves through LDS, in a fixed order, and the sum is rounded once to the
// 16-bit output type. Wide column chunks (256 fold, 64 unfold columns) leave
// fewer slices to sum across lanes, which is what costs when a pass has
// several rows; they are used when they still give a workgroup per CU, the
// narrow ones (64, 32) otherwise.
#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

using namespace dev;

constexpr int THREADS = 256;
constexpr int BPASS = 8;               // rows of X per pass
constexpr int NOPE = 128;              // qk_nope = v_head

struct ProjArgs {
  const uint16_t* x;   // [rows, H, K]
  const uint16_t* w;   // [H, K, N]
  uint16_t* y;         // [rows, H, N]
  int32_t rows;
  int32_t heads;
};

template <int DT, int K, int N, int COLS>
__global__ __launch_bounds__(THREADS) void head_matmul_kernel(ProjArgs a) {
  typedef Elem<DT> E;
  typedef typename E::vec8 vec8;
  constexpr int CT = COLS / 8;         // column threads (8 columns each)
  constexpr int KS = THREADS / CT;     // K slices
  constexpr int RPS = K / KS;          // weight rows per slice
  __shared__ __attribute__((aligned(16))) float xs[BPASS][K];
  static_assert(RPS % 4 == 0, "rows per slice in fours");
  __shared__ f32x4 part[THREADS / 64][BPASS][COLS / 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ct = tid % CT;
  const int ks = tid / CT;
  const int chunks = N / COLS;
  const int h = blockIdx.x / chunks;
  const int c0 = (blockIdx.x % chunks) * COLS + 8 * ct;
  if (h >= a.heads) return;

  // This thread's weight rows, loaded once for every pass.
  vec8 wv[RPS];
  const uint16_t* wrow = a.w + ((int64_t)h * K + ks * RPS) * N + c0;
#pragma unroll
  for (int r = 0; r < RPS; ++r) wv[r] = *reinterpret_cast<const vec8*>(wrow + (int64_t)r * N);

  for (int b0 = 0; b0 < a.rows; b0 += BPASS) {
    const int nb = min(BPASS, a.rows - b0);
    __syncthreads();   // the previous pass is done with xs and part
    for (int i = tid; i < nb * K; i += THREADS) {
      const int bb = i / K, k = i % K;
      const uint16_t bits = a.x[((int64_t)(b0 + bb) * a.heads + h) * K + k];
      xs[bb][k] = static_cast<float>(__builtin_bit_cast(typename E::scalar, bits));
    }
    __syncthreads();
    float acc[BPASS][8];
#pragma unroll
    for (int bb = 0; bb < BPASS; ++bb)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[bb][c] = 0.f;
#pragma unroll
    for (int r4 = 0; r4 < RPS; r4 += 4) {
#pragma unroll
      for (int bb = 0; bb < BPASS; ++bb) {
        if (bb < nb) {
          const f32x4 xk = *reinterpret_cast<const f32x4*>(&xs[bb][ks * RPS + r4]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c)
              acc[bb][c] = __builtin_fmaf(xk[r], static_cast<float>(wv[r4 + r][c]), acc[bb][c]);
        }
      }
    }
    // Slices inside a wave: lanes CT apart hold the same columns. Only the
    // pass's live rows are summed (nb is uniform over the workgroup).
#pragma unroll
    for (int x = CT; x < 64; x <<= 1)
#pragma unroll
      for (int bb = 0; bb < BPASS; ++bb)
        if (bb < nb) {
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[bb][c] += shfl_xor(acc[bb][c], x);
        }
    if (lane < CT) {
#pragma unroll
      for (int bb = 0; bb < BPASS; ++bb) {
        if (bb >= nb) continue;
        part[wave][bb][2 * ct] = f32x4{acc[bb][0], acc[bb][1], acc[bb][2], acc[bb][3]};
        part[wave][bb][2 * ct + 1] = f32x4{acc[bb][4], acc[bb][5], acc[bb][6], acc[bb][7]};
      }
    }
    __syncthreads();
    // Item (bb, q): 4 columns of row bb, summed over the waves in order.
    for (int i = tid; i < nb * CT * 2; i += THREADS) {
      const int bb = i / (CT * 2), q = i % (CT * 2);
      {
        f32x4 s = part[0][bb][q];
#pragma unroll
        for (int w = 1; w < THREADS / 64; ++w) s += part[w][bb][q];
        typename E::vec4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = static_cast<typename E::scalar>(s[c]);
        const int col = (blockIdx.x % chunks) * COLS + 4 * q;
        *reinterpret_cast<typename E::vec4*>(a.y + ((int64_t)(b0 + bb) * a.heads + h) * N + col) = o;
      }
    }
  }
}

bool aligned(const void* p, uintptr_t k) { return (reinterpret_cast<uintptr_t>(p) % k) == 0; }

// Workgroups that fill the 256 CUs of one MI355X.
constexpr int64_t kFillWorkgroups = 256;

template <int K, int N, int COLS, int COLS_WIDE>
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
  const bool wide = (int64_t)heads * (N / COLS_WIDE) >= kFillWorkgroups;
  const dim3 grid((unsigned)((int64_t)heads * (N / (wide ? COLS_WIDE : COLS))));
  if (dtype == MLA_F16 && wide)
    hipLaunchKernelGGL((head_matmul_kernel<0, K, N, COLS_WIDE>), grid, dim3(THREADS), 0, stream, a);
  else if (dtype == MLA_F16)
    hipLaunchKernelGGL((head_matmul_kernel<0, K, N, COLS>), grid, dim3(THREADS), 0, stream, a);
  else if (wide)
    hipLaunchKernelGGL((head_matmul_kernel<1, K, N, COLS_WIDE>), grid, dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((head_matmul_kernel<1, K, N, COLS>), grid, dim3(THREADS), 0, stream, a);
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
  return launch<NOPE, MLA_KV_LORA_RANK, 64, 256>("mla_absorb_query", q_nope, w_uk, q_absorbed, rows,
                                        num_heads, dtype, stream);
}

extern "C" int mla_unabsorb_output(const void* out_latent, const void* w_uv_t, void* o,
                                   int32_t rows, int32_t num_heads, int32_t dtype,
                                   hipStream_t stream) {
  return launch<MLA_KV_LORA_RANK, NOPE, 32, 64>("mla_unabsorb_output", out_latent, w_uv_t, o, rows,
                                        num_heads, dtype, stream);
}
