// Partition kernel of split-KV, matrix-absorbed MLA decode on gfx950.
//
// What it computes (mlxcel pull request 995, "What changed", Stage 1 and
// the split_kv.rs bullet; vllm-metal pull request 601 "[kernel] Wire MLA
// split-KV decode", "What changed"): for one row -- a block-aligned token
// range of one request -- and 16 heads, the softmax over
//   s_t = scale * (q_absorbed . ckv_t + q_pe . kpe_t)
// of the row's tokens, applied to the 512-wide ckv rows, written as a
// normalised fp32 partial and its base-2 log-sum-exp, or rounded straight
// into `out` when the request is a single row.
//
// Mapping onto one CU (256 threads = 4 wave64):
//  * Paged gather: each 32-token cache block (32 KB of ckv + 4 KB of kpe,
//    contiguous per physical block) is copied by global_load_lds_dwordx4
//    (16 B per lane, whole 128 B lines per instruction) into one of 4 LDS
//    stages of a ring, so up to 4 blocks per CU are in flight. Within a
//    row, the 16-byte chunk c sits at chunk position c ^ swz(row), which
//    keeps both the row-wise reads of the score product and the transposed
//    reads of the value product free of bank conflicts.
//  * Scores: S^T[token, head] = K[token, :] . Q^T[:, head] on
//    v_mfma_f32_16x16x32 (K = 576 = 18 steps of 32), tokens as the M side
//    and the 16 heads as the N side. Q (16 x 576) stays in registers.
//  * Online softmax in the base-2 domain: each lane owns one head and 8
//    tokens of a block; the block maximum needs two cross-lane steps. The
//    running reference maximum is only moved when a block beats it by more
//    than 2^8, so rescaling the fp32 accumulators is rare; the final O/l is
//    unchanged by that choice.
//  * Values: O^T[dim, head] += V^T[dim, token] . P^T[token, head], with the
//    probabilities P^T taken straight from the score accumulators (the MFMA
//    output layout of S^T is exactly the B-operand layout of this product
//    once the 32 tokens are ordered to match) and V^T read from the same
//    LDS tile with ds_read_b64_tr_b16. The 4 waves split the 512 output
//    dims (128 each), so every wave computes the scores of all 32 tokens --
//    cheap at 16 heads, where the kernel is bound by HBM many times over.
#include "device_common.h"
#include "internal.h"

#include <cmath>

namespace mla {
namespace {

using namespace dev;

constexpr int BS = MLA_BLOCK_SIZE;            // tokens per cache block
constexpr int LAT = MLA_KV_LORA_RANK;         // 512
constexpr int ROPE = MLA_ROPE_DIM;            // 64
constexpr int CKV_ROW = LAT * 2;              // bytes per ckv row
constexpr int KPE_ROW = ROPE * 2;             // bytes per kpe row
constexpr int CKV_TILE = BS * CKV_ROW;        // 32 KB
constexpr int KPE_TILE = BS * KPE_ROW;        // 4 KB
constexpr int STAGE = CKV_TILE + KPE_TILE;    // 36 KB per cache block
constexpr int NSTAGE = 4;
constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int HG = 16;                        // heads per workgroup
constexpr int KSTEPS = (LAT + ROPE) / 32;     // 18 MFMA K-steps per score
constexpr int DT_PER_WAVE = LAT / 16 / WAVES; // 8 output dim tiles per wave
constexpr int LOADS_PER_BLOCK = STAGE / 1024 / WAVES;  // 9 DMA ops per wave
constexpr float RESCALE_LOG2 = 8.0f;          // lazy-rescale threshold
static_assert(LOADS_PER_BLOCK * WAVES * 1024 == STAGE, "stage split");
static_assert(NSTAGE * STAGE <= 160 * 1024, "LDS budget");
// Q (16 heads x 1152 B) is staged through the last ring stage at start.
static_assert(HG * (CKV_ROW + KPE_ROW) <= STAGE, "Q staging fits a stage");

struct PartitionArgs {
  const uint16_t* q_absorbed;
  const uint16_t* q_pe;
  const uint16_t* ckv;
  const uint16_t* kpe;
  const int32_t* block_table;
  const int32_t* context_lens;
  const int32_t* partitions;
  const int32_t* splits;
  const int32_t* row_indptr;
  float* partial_out;
  float* partial_lse2;
  void* out;
  float* lse2_out;
  int32_t* debug_ranges;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t batch;
  int32_t heads;
  int32_t groups;        // heads / HG
  int32_t rows_per_req;  // grid rows per request (max_rows_per_req)
  int32_t slots;         // batch * rows_per_req
  int32_t total_rows;
  int32_t direct;        // 1: one row per request, write `out`
  float scale_log2;      // scale * log2(e)
};

// XOR swizzles of the 16-byte chunk index inside an LDS row (see header).
__device__ __forceinline__ int swz_ckv(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int swz_kpe(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Issue the DMA of one 32-token cache block into `stage` (9 ops per wave).
__device__ __forceinline__ void issue_block(const PartitionArgs& a, int64_t phys,
                                            uint32_t stage, int wave, int lane) {
  const char* ckv = reinterpret_cast<const char*>(a.ckv) + phys * CKV_TILE;
  const char* kpe = reinterpret_cast<const char*>(a.kpe) + phys * KPE_TILE;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wave * 8 + j;
    const int chunk = (lane & ~15) | ((lane & 15) ^ swz_ckv(r));
    dma16(ckv + r * CKV_ROW + chunk * 16, stage + r * CKV_ROW);
  }
  {
    const int r = wave * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz_kpe(r);
    dma16(kpe + r * KPE_ROW + chunk * 16, stage + CKV_TILE + wave * 1024);
  }
}

// Wait until this wave's DMA ops older than the newest `ahead` blocks are
// complete (ahead = blocks issued after the one we need).
__device__ __forceinline__ void wait_blocks_ahead(int ahead) {
  if (ahead >= 3) wait_vmcnt<3 * LOADS_PER_BLOCK>();
  else if (ahead == 2) wait_vmcnt<2 * LOADS_PER_BLOCK>();
  else if (ahead == 1) wait_vmcnt<LOADS_PER_BLOCK>();
  else wait_vmcnt<0>();
}

template <int DT>
__global__ __launch_bounds__(THREADS) void partition_kernel(PartitionArgs a) {
  typedef Elem<DT> E;
  typedef typename E::vec8 vec8;
  typedef typename E::vec4 vec4;
  __shared__ __attribute__((aligned(1024))) char smem_raw[NSTAGE * STAGE];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15;   // MFMA row/column inside a 16-wide tile
  const int lg = lane >> 4;   // MFMA k-group (0..3)

  // ---- which (request, local row, head group) this workgroup owns -------
  // Workgroups are dealt to the 8 XCDs round-robin by linear id. Row slot
  // u = b * rows_per_req + x; the id layout L = ((u / 8) * G + hg) * 8 + u % 8
  // keeps the G head groups of one row on one XCD, so they share its L2.
  const int L = blockIdx.x;
  const int sl = L >> 3;
  const int hg = sl % a.groups;
  const int u = (sl / a.groups) * 8 + (L & 7);
  if (u >= a.slots) return;
  const int b = u / a.rows_per_req;
  const int x = u % a.rows_per_req;

  int n = load_const(a.context_lens, b);
  n = max(0, min(n, a.max_blocks * BS));
  int P = 1, S = 1, row = b, nrows = 1;
  if (!a.direct) {
    const int r0 = load_const(a.row_indptr, b);
    nrows = load_const(a.row_indptr, b + 1) - r0;
    P = max(1, min(load_const(a.partitions, b), 1 << 25));
    S = max(1, min(load_const(a.splits, b), 1 << 25));
    row = r0 + x;
  }
  if (x >= nrows || row < 0 || row >= a.total_rows) return;
  const int p = x / S;
  const int s = x % S;
  // Index math of mla_partition_range (must agree bit for bit).
  const int nblk = cdiv(n, BS);
  const int bpp = cdiv(nblk, P);
  const int pb0 = min(p * bpp, nblk);
  const int pb1 = min((p + 1) * bpp, nblk);
  const int m = pb1 - pb0;
  const int bps = m > 0 ? cdiv(m, S) : 0;
  const int blk_lo = (p < P) ? pb0 + min(s * bps, m) : nblk;
  const int blk_hi = (p < P) ? pb0 + min((s + 1) * bps, m) : nblk;
  const int tok_lo = min(blk_lo * BS, n);
  const int tok_hi = min(blk_hi * BS, n);
  const int nb = blk_hi - blk_lo;

  const int head0 = hg * HG;
  const int64_t qrow0 = (int64_t)b * a.heads + head0;   // first (b, head) row
  const int my_head = head0 + ln;

  if (a.debug_ranges && hg == 0 && tid == 0) {
    // Stored before any DMA is issued only on the empty path; otherwise in
    // the epilogue, so no store is outstanding while stages are awaited.
    if (nb <= 0 || tok_hi <= tok_lo) {
      a.debug_ranges[2 * row] = tok_lo;
      a.debug_ranges[2 * row + 1] = tok_hi;
    }
  }
  if (nb <= 0 || tok_hi <= tok_lo) {
    // No visible token: zero output, lse2 = -inf.
#pragma unroll
    for (int dt = 0; dt < DT_PER_WAVE; ++dt) {
      const int d0 = (wave * DT_PER_WAVE + dt) * 16 + lg * 4;
      const int64_t off = ((int64_t)b * a.heads + my_head) * LAT + d0;
      if (a.direct) {
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + off;
        *reinterpret_cast<u32x2*>(o) = u32x2{0u, 0u};
      } else {
        float* o = a.partial_out + ((int64_t)row * a.heads + my_head) * LAT + d0;
        *reinterpret_cast<f32x4*>(o) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (wave == 0 && lg == 0) {
      if (a.direct) {
        if (a.lse2_out) a.lse2_out[(int64_t)b * a.heads + my_head] = -INFINITY;
      } else {
        a.partial_lse2[(int64_t)row * a.heads + my_head] = -INFINITY;
      }
    }
    return;
  }

  const int64_t tbl0 = (int64_t)b * a.max_blocks;
  const int last_blk = a.num_blocks - 1;
  auto phys_of = [&](int blk) -> int64_t {
    int v = __builtin_amdgcn_readfirstlane(load_const(a.block_table, tbl0 + blk));
    return (int64_t)max(0, min(v, last_blk));
  };
  const uint32_t lds0 = lds_addr(smem);

  // ---- prologue: Q into the last stage, first blocks into the others ----
  {
    const uint32_t qst = lds0 + (NSTAGE - 1) * STAGE;
    const char* qa = reinterpret_cast<const char*>(a.q_absorbed) + qrow0 * CKV_ROW;
#pragma unroll
    for (int j = 0; j < HG / WAVES; ++j) {
      const int h = wave * (HG / WAVES) + j;
      const int chunk = (lane & ~15) | ((lane & 15) ^ swz_ckv(h));
      dma16(qa + h * CKV_ROW + chunk * 16, qst + h * CKV_ROW);
    }
    if (wave < HG * KPE_ROW / 1024) {
      const char* qp = reinterpret_cast<const char*>(a.q_pe) + qrow0 * KPE_ROW;
      const int h = wave * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ swz_kpe(h);
      dma16(qp + h * KPE_ROW + chunk * 16, qst + HG * CKV_ROW + wave * 1024);
    }
  }
  int issued = 0;
  for (; issued < NSTAGE - 1 && issued < nb; ++issued)
    issue_block(a, phys_of(blk_lo + issued), lds0 + issued * STAGE, wave, lane);

  // Q lands first (oldest ops); wait for it alone.
  wait_blocks_ahead(issued);
  __syncthreads();
  vec8 q[KSTEPS];
  {
    const MLA_LDS char* qs = smem + (NSTAGE - 1) * STAGE;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      const MLA_LDS char* pq;
      if (k < LAT / 32) {
        const int c = (4 * k + lg) ^ swz_ckv(ln);
        pq = qs + ln * CKV_ROW + c * 16;
      } else {
        const int c = (4 * (k - LAT / 32) + lg) ^ swz_kpe(ln);
        pq = qs + HG * CKV_ROW + ln * KPE_ROW + c * 16;
      }
      q[k] = *(const MLA_LDS vec8*)pq;
    }
  }
  __syncthreads();   // everyone holds Q before the last stage is reused
  if (issued < nb) {
    issue_block(a, phys_of(blk_lo + issued), lds0 + issued * STAGE, wave, lane);
    ++issued;
  }

  // ---- main loop over the row's cache blocks -----------------------------
  f32x4 o[DT_PER_WAVE];
#pragma unroll
  for (int dt = 0; dt < DT_PER_WAVE; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference maximum (base-2 domain) of my head
  float l_part = 0.f;       // my 8-token share of the running sum
  const float c2 = a.scale_log2;

  for (int i = 0; i < nb; ++i) {
    const int st = i % NSTAGE;
    const MLA_LDS char* stg = smem + st * STAGE;
    // Prefetch the table entry of the block this stage gets next.
    const bool more = issued < nb;
    const int64_t next_phys = more ? phys_of(blk_lo + issued) : 0;

    wait_blocks_ahead(issued - i - 1);
    __syncthreads();

    const int tok0 = (blk_lo + i) * BS;
    const int valid = min(BS, tok_hi - tok0);  // visible tokens of this block
    if (valid < BS) {
      // Rows past the context end may hold anything (NaN included); zero
      // their latent values so that 0-probability tokens add exactly 0.
      for (int idx = tid; idx < (BS - valid) * (CKV_ROW / 16); idx += THREADS) {
        const int r = valid + idx / (CKV_ROW / 16);
        const int c = idx % (CKV_ROW / 16);
        *(MLA_LDS u32x4*)(smem + st * STAGE + r * CKV_ROW + c * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }

    // Scores of the 32 tokens for the 16 heads: two 16-token M-tiles, two
    // accumulators each (even / odd K-steps) to keep MFMA chains short.
    f32x4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      acc[mt][0] = acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int r = mt * 16 + ln;
        const MLA_LDS char* pk;
        if (k < LAT / 32) {
          pk = stg + r * CKV_ROW + (((4 * k + lg) ^ swz_ckv(r)) * 16);
        } else {
          pk = stg + CKV_TILE + r * KPE_ROW + (((4 * (k - LAT / 32) + lg) ^ swz_kpe(r)) * 16);
        }
        const vec8 kf = *(const MLA_LDS vec8*)pk;
        acc[mt][k & 1] = E::mfma(kf, q[k], acc[mt][k & 1]);
      }
    }
    // Lane (ln, lg) now holds, for head head0+ln, the tokens
    // 4*lg+j (j < 4, from M-tile 0) and 16+4*lg+(j-4) (j >= 4, M-tile 1).
    float xs[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xs[j] = (acc[0][0][j] + acc[0][1][j]) * c2;
      xs[4 + j] = (acc[1][0][j] + acc[1][1][j]) * c2;
    }
    if (valid < BS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tk = (j < 4) ? (4 * lg + j) : (16 + 4 * lg + (j - 4));
        if (tk >= valid) xs[j] = -INFINITY;
      }
    }
    float bm = xs[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) bm = fmaxf(bm, xs[j]);
    bm = fmaxf(bm, shfl_xor(bm, 16));
    bm = fmaxf(bm, shfl_xor(bm, 32));
    const bool need = bm > m_ref + RESCALE_LOG2;
    if (__any(need)) {
      const float m_new = need ? bm : m_ref;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
#pragma unroll
      for (int dt = 0; dt < DT_PER_WAVE; ++dt) o[dt] *= alpha;
      l_part *= alpha;
      m_ref = m_new;
    }
    vec8 pv;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const typename E::scalar pj =
          static_cast<typename E::scalar>(__builtin_amdgcn_exp2f(xs[j] - m_ref));
      pv[j] = pj;
      l_part += static_cast<float>(pj);
    }

    // Values: O^T[dims, heads] += V^T[dims, tokens] . P^T[tokens, heads].
    // The A operand of lane (ln, lg) is dim 16*dtg+ln of tokens
    // 4*lg..4*lg+3 and 16+4*lg..16+4*lg+3, read transposed from the tile.
#pragma unroll
    for (int dt = 0; dt < DT_PER_WAVE; ++dt) {
      const int dtg = wave * DT_PER_WAVE + dt;
      const int r1 = 4 * lg + (ln >> 2);
      const int r2 = r1 + 16;
      const int cpos = 2 * dtg + ((ln >> 1) & 1);   // 16-byte chunk holding my dims
      const int half = (ln & 1) * 8;
      const vec4 v1 = E::tr_read(stg + r1 * CKV_ROW + ((cpos ^ swz_ckv(r1)) * 16) + half);
      const vec4 v2 = E::tr_read(stg + r2 * CKV_ROW + ((cpos ^ swz_ckv(r2)) * 16) + half);
      const vec8 vf = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
      o[dt] = E::mfma(vf, pv, o[dt]);
    }

    __syncthreads();   // this stage is free again
    if (more) {
      issue_block(a, next_phys, lds0 + st * STAGE, wave, lane);
      ++issued;
    }
  }

  // ---- epilogue: normalise and write --------------------------------------
  float l_tot = l_part + shfl_xor(l_part, 16);
  l_tot = l_tot + shfl_xor(l_tot, 32);
  const float inv = 1.0f / l_tot;
  const float lse2 = m_ref + __builtin_amdgcn_logf(l_tot);
#pragma unroll
  for (int dt = 0; dt < DT_PER_WAVE; ++dt) {
    const int d0 = (wave * DT_PER_WAVE + dt) * 16 + lg * 4;
    const f32x4 v = o[dt] * inv;
    if (a.direct) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) +
                      ((int64_t)b * a.heads + my_head) * LAT + d0;
      typename E::vec4 h;
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = static_cast<typename E::scalar>(v[j]);
      *reinterpret_cast<typename E::vec4*>(dst) = h;
    } else {
      float* dst = a.partial_out + ((int64_t)row * a.heads + my_head) * LAT + d0;
      *reinterpret_cast<f32x4*>(dst) = v;
    }
  }
  if (wave == 0 && lg == 0) {
    if (a.direct) {
      if (a.lse2_out) a.lse2_out[(int64_t)b * a.heads + my_head] = lse2;
    } else {
      a.partial_lse2[(int64_t)row * a.heads + my_head] = lse2;
    }
  }
  if (a.debug_ranges && hg == 0 && tid == 0) {
    a.debug_ranges[2 * row] = tok_lo;
    a.debug_ranges[2 * row + 1] = tok_hi;
  }
}

bool aligned(const void* p, uintptr_t k) { return (reinterpret_cast<uintptr_t>(p) % k) == 0; }

}  // namespace

int device_compute_units(int64_t* cus) {
  int dev = 0, v = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || v <= 0)
    return fail(MLA_E_HIP, "compute-unit query failed: %s", hipGetErrorString(e));
  *cus = v;
  return MLA_OK;
}

}  // namespace mla

using namespace mla;

extern "C" int mla_decode_partition(
    const void* q_absorbed, const void* q_pe, const void* ckv_cache, const void* kpe_cache,
    int32_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t batch, int32_t num_heads, float scale, int32_t dtype,
    const int32_t* partitions, const int32_t* splits, const int32_t* row_indptr,
    int32_t total_rows, int32_t max_rows_per_req, int32_t heads_per_wg, float* partial_out,
    float* partial_lse2, void* out, float* lse2_out, int32_t* debug_ranges,
    hipStream_t stream) {
  clear_error();
  if (batch < 0) return fail(MLA_E_SHAPE, "batch %d < 0", batch);
  if (num_heads < MLA_MIN_HEADS || num_heads > MLA_MAX_HEADS || num_heads % 16)
    return fail(MLA_E_UNSUPPORTED, "num_heads %d (need a multiple of 16 in [16, 128])",
                num_heads);
  if (dtype != MLA_F16 && dtype != MLA_BF16) return fail(MLA_E_UNSUPPORTED, "dtype %d", dtype);
  const int32_t hpw = heads_per_wg ? heads_per_wg : default_heads_per_wg(num_heads);
  if (hpw != HG || num_heads % hpw)
    return fail(MLA_E_UNSUPPORTED, "heads_per_wg %d (this build has 16-head workgroups)", hpw);
  if (!std::isfinite(scale)) return fail(MLA_E_RANGE, "scale is not finite");
  if (batch == 0) return MLA_OK;
  if (!q_absorbed || !q_pe || !ckv_cache || !kpe_cache || !block_table || !context_lens)
    return fail(MLA_E_NULL, "null input pointer");
  if (num_blocks < 1 || max_blocks_per_seq < 1 || max_blocks_per_seq > (1 << 25))
    return fail(MLA_E_SHAPE, "num_blocks %d, max_blocks_per_seq %d", num_blocks,
                max_blocks_per_seq);
  if (total_rows < batch || max_rows_per_req < 1 ||
      (int64_t)max_rows_per_req * batch < total_rows)
    return fail(MLA_E_SHAPE, "total_rows %d / max_rows_per_req %d for batch %d", total_rows,
                max_rows_per_req, batch);
  const bool direct = total_rows == batch;
  if (direct) {
    if (!out) return fail(MLA_E_NULL, "single-pass plan needs `out`");
    if (!aligned(out, 16)) return fail(MLA_E_ALIGN, "out not 16-byte aligned");
  } else {
    if (!partitions || !splits || !row_indptr || !partial_out || !partial_lse2)
      return fail(MLA_E_NULL, "split plan needs plan arrays and partial buffers");
    if (!aligned(partial_out, 16) || !aligned(partial_lse2, 4))
      return fail(MLA_E_ALIGN, "partial buffers misaligned");
  }
  if (!aligned(q_absorbed, 16) || !aligned(q_pe, 16) || !aligned(ckv_cache, 16) ||
      !aligned(kpe_cache, 16))
    return fail(MLA_E_ALIGN, "16-bit tensors must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4) || (lse2_out && !aligned(lse2_out, 4)) ||
      (debug_ranges && !aligned(debug_ranges, 8)))
    return fail(MLA_E_ALIGN, "int32/fp32 arrays misaligned");

  PartitionArgs a;
  a.q_absorbed = static_cast<const uint16_t*>(q_absorbed);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.ckv = static_cast<const uint16_t*>(ckv_cache);
  a.kpe = static_cast<const uint16_t*>(kpe_cache);
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.partitions = partitions;
  a.splits = splits;
  a.row_indptr = row_indptr;
  a.partial_out = partial_out;
  a.partial_lse2 = partial_lse2;
  a.out = out;
  a.lse2_out = lse2_out;
  a.debug_ranges = debug_ranges;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.batch = batch;
  a.heads = num_heads;
  a.groups = num_heads / HG;
  a.rows_per_req = direct ? 1 : max_rows_per_req;
  a.direct = direct ? 1 : 0;
  a.total_rows = total_rows;
  a.scale_log2 = scale * 1.4426950408889634f;

  const int64_t slots = (int64_t)batch * a.rows_per_req;
  const int64_t wgs = ((slots + 7) / 8) * 8 * a.groups;
  if (wgs > INT32_MAX || slots > INT32_MAX)
    return fail(MLA_E_SHAPE, "grid too large (%lld workgroups)", (long long)wgs);
  a.slots = (int32_t)slots;
  if (dtype == MLA_F16)
    hipLaunchKernelGGL(partition_kernel<0>, dim3((unsigned)wgs), dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(partition_kernel<1>, dim3((unsigned)wgs), dim3(THREADS), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_E_HIP, "partition launch: %s", hipGetErrorString(e));
  count(direct ? 0 : 1, 1);
  count(3, (uint64_t)total_rows);
  return MLA_OK;
}
