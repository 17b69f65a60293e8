// Wide partition kernel of split-KV, matrix-absorbed MLA decode on gfx950:
// 64 heads per workgroup (used when 64 divides the head count, e.g. the
// 128-head DeepSeek-V3 shape as two workgroups per row).
//
// Same computation as the 16-head kernel (mlxcel pull request 995, "What
// changed", Stage 1; vllm-metal pull request 601 "[kernel] Wire MLA
// split-KV decode", "What changed"): for one row (a block-aligned token
// range of one request) and a group of heads, the base-2 online softmax over
//   s_t = scale * (q_absorbed . ckv_t + q_pe . kpe_t)
// applied to the 512-wide ckv rows, written as a normalised fp32 partial and
// its log2-sum-exp, or rounded into `out` for a single-row request.
//
// With 64 heads the work per cached token is dense enough for the matrix
// cores to matter, so each LDS fragment should feed as many heads as the
// registers allow:
//  * 256 threads = 4 wave64, one per SIMD. Waves 2p and 2p+1 form pair p,
//    which owns heads 32p .. 32p+31 of the workgroup; wave 2p+h owns head
//    tile h of the pair (16 heads), whose Q (16 x 576, the score B operand)
//    sits in 72 VGPRs.
//  * Scores: each wave scores all 32 tokens of the block for its 16 heads,
//    S^T[token, head] = K[token, :] . Q^T[:, head] on v_mfma_f32_16x16x32
//    (2 token tiles x 18 K-steps), and runs the softmax of those heads.
//    The pair then swaps its 16-bit probabilities through LDS.
//  * Values: wave 2p+h accumulates O^T[dim, head] for dims 256h .. 256h+255
//    and both head tiles of the pair (128 registers) on v_mfma_f32_16x16x32;
//    the MFMA result layout of S^T is already the B-operand layout of P^T,
//    and V^T comes from the same LDS tile through ds_read_b64_tr_b16, each
//    fragment feeding both head tiles. The running sums are swapped once,
//    at the end.
//  * LDS holds a ring of 4 one-block slots (32 KB ckv + 4 KB kpe each);
//    block k lives in slot k % 4, so three blocks are in flight while one is
//    used. Every wave copies a quarter of each block with
//    global_load_lds_dwordx4 (16 B per lane) and waits only for its own
//    copies; one s_barrier per block then makes the block visible to all and
//    also proves that every wave is done with the previous block, whose slot
//    is refilled right away with block k + 3. A second s_barrier per block
//    publishes the swapped probabilities.
//  * No rescaling inside the loop: every head's reference maximum is fixed
//    by the first block, and probabilities relative to it may grow up to
//    2^15 (finite in fp16 and bf16, exact to the format's precision). The
//    true running maximum is tracked alongside; if it ends more than 15
//    (base 2) above the reference for any head, the workgroup makes a
//    second pass over the row with the exact maximum as reference. The
//    accumulators thus only ever see MFMA updates and stay in AGPRs.
#include "partition_common.h"

#include <cmath>

namespace mla {
namespace part {
namespace {

using namespace dev;

constexpr int HPW = 64;                         // heads per workgroup
constexpr int SLOT = BS * (CKV_ROW + KPE_ROW);  // 36 KB per one-block slot
constexpr int SLOT_KPE = BS * CKV_ROW;          // kpe rows after the ckv rows
constexpr int NSLOT = 4;
constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int DT_WAVE = LAT / 16 / 2;           // 16 output dim tiles per wave
constexpr int OPS = BS + BS * KPE_ROW / 1024;   // 36 copy instructions per block
constexpr int OPW = OPS / WAVES;                // 9 per wave
constexpr int XP = NSLOT * SLOT;                // swapped probabilities [wave][lane]
constexpr int XML = XP + WAVES * 64 * 16;       // swapped (max, sum) [wave][16 heads]
constexpr int XFLAG = XML + WAVES * 16 * 8;     // "second pass needed" flag
constexpr int LDS_BYTES = XFLAG + 16;
constexpr float HEADROOM_LOG2 = 15.0f;          // p <= 2^15 against the reference
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(OPS % WAVES == 0 && 3 * OPW < 64, "copy split / vmcnt range");

// Wait until at most `later` blocks' worth of this wave's copies are still
// in flight (copies complete in issue order).
__device__ __forceinline__ void wait_blocks(int later) {
  switch (later) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<OPW>(); break;
    case 2: wait_vmcnt<2 * OPW>(); break;
    default: wait_vmcnt<3 * OPW>(); break;
  }
}

// Make this wave's LDS writes visible, then meet the other waves. No memory
// fence: the in-flight LDS copies must not be waited for here.
__device__ __forceinline__ void meet() {
  wait_lgkmcnt0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int DT>
__global__ __launch_bounds__(THREADS, 1) void wide_kernel(
    int32_t groups, int32_t rows_per_req, int32_t slots, int32_t direct, int32_t total_rows,
    int32_t max_blocks, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ row_indptr, const int32_t* __restrict__ partitions,
    const int32_t* __restrict__ splits, const int32_t* __restrict__ block_table,
    PartitionArgs a) {
  typedef Elem<DT> E;
  typedef typename E::vec8 vec8;
  typedef typename E::vec4 vec4;
  typedef typename E::scalar scalar;

  __shared__ __attribute__((aligned(1024))) char smem_raw[LDS_BYTES];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15;   // MFMA row/column inside a 16-wide tile
  const int lg = lane >> 4;   // MFMA k-group (0..3)
  const int half = wave & 1;  // my head tile of the pair; my dim half

  int b, x, hg;
  if (!slot_of(blockIdx.x, groups, rows_per_req, slots, &b, &x, &hg)) return;
  const int head0 = hg * HPW + (wave >> 1) * 32;   // this pair's first head
  const int64_t qrow0 = (int64_t)b * a.heads + head0;

  // Q first (its address needs no metadata): lane (ln, lg) holds head
  // head0 + 16 half + ln, dims 32 k + 8 lg .. + 8.
  vec8 q[KSTEPS];
  {
    const int64_t qr = qrow0 + 16 * half + ln;
    const vec8* qa = reinterpret_cast<const vec8*>(a.q_absorbed + qr * LAT);
    const vec8* qp = reinterpret_cast<const vec8*>(a.q_pe + qr * ROPE);
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k)
      q[k] = (k < LAT / 32) ? qa[4 * k + lg] : qp[4 * (k - LAT / 32) + lg];
  }

  RowInfo ri;
  if (!find_row(b, x, direct, total_rows, max_blocks, context_lens, row_indptr, partitions,
                splits, &ri))
    return;
  const int row = ri.row;
  const int nblocks = ri.nblocks;
  // Lane (ln, lg) of head tile ht and dim tile dt holds head head0 + 16 ht +
  // ln, dims 16 dt + 4 lg .. + 4.
  auto store = [&](int ht, int dt, f32x4 v) {
    const int64_t h = head0 + 16 * ht + ln;
    const int d0 = dt * 16 + lg * 4;
    if (direct) {
      vec4 hv;
#pragma unroll
      for (int j = 0; j < 4; ++j) hv[j] = static_cast<scalar>(v[j]);
      *reinterpret_cast<vec4*>(reinterpret_cast<uint16_t*>(a.out) +
                               ((int64_t)b * a.heads + h) * LAT + d0) = hv;
    } else {
      *reinterpret_cast<f32x4*>(a.partial_out + ((int64_t)row * a.heads + h) * LAT + d0) = v;
    }
  };
  auto store_lse = [&](int ht, float v) {
    const int64_t i = (int64_t)(direct ? b : row) * a.heads + head0 + 16 * ht + ln;
    if (direct) {
      if (a.lse2_out) a.lse2_out[i] = v;
    } else {
      a.partial_lse2[i] = v;
    }
  };
  if (a.debug_ranges && hg == 0 && tid == 0) {
    a.debug_ranges[2 * row] = ri.tok_lo;
    a.debug_ranges[2 * row + 1] = ri.tok_hi;
  }

  if (nblocks <= 0) {
    // No visible token: zero output, lse2 = -inf.
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
      for (int d = 0; d < DT_WAVE; ++d) store(ht, half * DT_WAVE + d, f32x4{0.f, 0.f, 0.f, 0.f});
      if (half == 0 && lg == 0) store_lse(ht, -INFINITY);
    }
    return;
  }

  const int64_t tbl0 = (int64_t)b * max_blocks + ri.blk_lo;
  const int last_phys = a.num_blocks - 1;
  const char* ckv_base = reinterpret_cast<const char*>(a.ckv);
  const char* kpe_base = reinterpret_cast<const char*>(a.kpe);
  const uint32_t lds0 = lds_addr(smem);
  auto phys_of = [&](int k) {
    const int v = __builtin_amdgcn_readfirstlane(load_const(block_table, tbl0 + k));
    return (int64_t)max(0, min(v, last_phys));
  };
  // This wave's quarter of block k's copies into slot k % 4: ops 0..31 are
  // ckv rows, 32..35 kpe rows 8 (op - 32) .. + 8. Chunk c of an LDS row sits
  // at position c ^ swizzle(row).
  auto issue = [&](int k, int64_t phys) {
    const uint32_t base = lds0 + (k & (NSLOT - 1)) * SLOT;
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int op = wave * OPW + i;
      if (op < BS) {
        const uint32_t voff = ((lane & ~15) | ((lane & 15) ^ swz_ckv(op))) * 16;
        dma16s(voff, ckv_base + phys * (BS * CKV_ROW) + op * CKV_ROW, base + op * CKV_ROW);
      } else {
        const int t8 = op - BS;
        const int r = t8 * 8 + (lane >> 3);
        const uint32_t voff = (lane >> 3) * KPE_ROW + ((lane & 7) ^ swz_kpe(r)) * 16;
        dma16s(voff, kpe_base + phys * (BS * KPE_ROW) + t8 * 1024, base + SLOT_KPE + t8 * 1024);
      }
    }
  };

  // Loop-invariant LDS byte offsets inside a slot. Score fragments of
  // token tile tt: row 16 tt + ln (tile 1 is 16 KB further, same swizzle),
  // chunk 4 k + lg; chunks 16 apart keep the same swizzled low bits, so
  // k = 4 m + kk is offs_k[kk] + 256 m. Value fragments: rows r1 = 4 lg +
  // ln / 4 and r1 + 16 (16 KB further), chunk 2 dt + (ln / 2) % 2; dt =
  // 8 m + dd is offs_v[dd] + 256 m.
  uint32_t offs_k[4], offs_p[2], offs_v[8];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) offs_k[kk] = ln * CKV_ROW + (((4 * kk + lg) ^ swz_ckv(ln)) * 16);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    offs_p[kk] = SLOT_KPE + ln * KPE_ROW + (((4 * kk + lg) ^ swz_kpe(ln)) * 16);
  const int r1 = 4 * lg + (ln >> 2);
#pragma unroll
  for (int dd = 0; dd < 8; ++dd)
    offs_v[dd] = r1 * CKV_ROW + (((2 * dd + ((ln >> 1) & 1)) ^ swz_ckv(r1)) * 16) + (ln & 1) * 8;
  MLA_LDS char* xp_mine = smem + XP + wave * 1024;
  const MLA_LDS char* xp_pair = smem + XP + (wave ^ 1) * 1024;
  MLA_LDS uint32_t* flag = (MLA_LDS uint32_t*)(smem + XFLAG);
  if (tid == 0) *flag = 0u;   // seen by all after the first meeting below

  const float c2 = a.scale_log2;
  const int ntok = ri.tok_hi - ri.tok_lo;
  f32x4 o[DT_WAVE][2];
  float m_ref = -INFINITY;   // reference max of my head (base 2)
  float m_run = -INFINITY;   // true running max of my head
  float l_part = 0.f;        // this lane's share of my head's sum

  // Q must be in registers before any copy is issued: the copies are
  // invisible to the compiler's own wait counting.
  wait_vmcnt<0>();
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) m_ref = m_run;   // exact maximum: every p <= 1
#pragma unroll
    for (int d = 0; d < DT_WAVE; ++d) o[d][0] = o[d][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_part = 0.f;
    for (int k = 0; k < NSLOT && k < nblocks; ++k) issue(k, phys_of(k));
    int64_t phys_next = nblocks > NSLOT ? phys_of(NSLOT) : 0;

    for (int k = 0; k < nblocks; ++k) {
      const int slot = k & (NSLOT - 1);
      const int valid = min(BS, ntok - k * BS);

      // This wave's copies of block k have landed: copies of blocks up to
      // k + 2 (k + 3 for the first block) were issued before this point.
      wait_blocks(min(k == 0 ? 3 : 2, nblocks - 1 - k));
      if (valid < BS) {
        // Rows past the context end may hold anything (NaN included): zero
        // the ckv rows this wave brought in, so that 0-probability tokens
        // add exactly 0.
        for (int r = max(valid, wave * OPW); r < min(BS, (wave + 1) * OPW); ++r)
          *(MLA_LDS u32x4*)(smem + slot * SLOT + r * CKV_ROW + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      meet();  // block k is in LDS; every wave is done with block k - 1
      if (k >= 1 && k + NSLOT - 1 < nblocks) {
        issue(k + NSLOT - 1, phys_next);   // into the slot of block k - 1
        if (k + NSLOT < nblocks) phys_next = phys_of(k + NSLOT);
      }

      // ---- scores of my 16 heads over the 32 tokens ---------------------
      // 36 K fragments (K-step ks, token tile tt) in the order j = 2 ks + tt,
      // each read KD reads ahead of the MFMA that uses it; four
      // accumulation chains.
      const uint32_t sbase = lds0 + slot * SLOT;
      auto kaddr = [&](int j) {
        const int ks = j >> 1, tt = j & 1;
        return sbase + ((ks < LAT / 32)
                            ? offs_k[ks & 3] + 256 * (ks >> 2) + tt * (16 * CKV_ROW)
                            : offs_p[ks - LAT / 32] + tt * (16 * KPE_ROW));
      };
      constexpr int NK = 2 * KSTEPS;
      constexpr int KD = 6;
      f32x4 acc[2][2];
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[0][c] = acc[1][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      vec8 kf[NK];
#pragma unroll
      for (int j = 0; j < KD; ++j) kf[j] = lds_read_b128<vec8>(kaddr(j));
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        if (j + KD <= NK) lds_wait<KD - 1>(kf[j]);
        else lds_wait<0>(kf[j]);   // tail: reads after j are < KD - 1
        const int ks = j >> 1, tt = j & 1;
        acc[tt][ks & 1] = E::mfma(kf[j], q[ks], acc[tt][ks & 1]);
        if (j + KD < NK) kf[j + KD] = lds_read_b128<vec8>(kaddr(j + KD));
      }
      // First value fragment now: its latency hides behind the softmax.
      // Fragment d: dim tile 16 half + d, tokens 4 lg + (0..3) and
      // 16 + 4 lg + (0..3) of the block.
      auto vaddr = [&](int d) {
        const int dt = half * DT_WAVE + d;
        return sbase + offs_v[dt & 7] + 256 * (dt >> 3);
      };
      u32x2 vr[DT_WAVE][2];
      vr[0][0] = lds_read_tr_b16(vaddr(0));
      vr[0][1] = lds_read_tr_b16(vaddr(0) + 16 * CKV_ROW);

      // ---- softmax weights of my heads (base 2) ----------------------------
      // Lane (ln, lg) holds head 16 half + ln at tokens 16 tt + 4 lg + e.
      float sc[2][4];
      float bm = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 sacc = acc[tt][0] + acc[tt][1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[tt][e] = (16 * tt + 4 * lg + e < valid) ? sacc[e] * c2 : -INFINITY;
          bm = fmaxf(bm, sc[tt][e]);
        }
      }
      bm = fmaxf(bm, shfl_xor(bm, 16));
      bm = fmaxf(bm, shfl_xor(bm, 32));
      m_run = fmaxf(m_run, bm);
      if (pass == 0 && k == 0) m_ref = bm;
      // P^T B operand of lane (ln, lg): head 16 half + ln at tokens 4 lg + e
      // (e < 4) and 16 + 4 lg + (e - 4) -- the order of the V^T reads.
      vec8 pmine;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const scalar p = static_cast<scalar>(__builtin_amdgcn_exp2f(sc[e >> 2][e & 3] - m_ref));
        pmine[e] = p;
        l_part += static_cast<float>(p);
      }
      // Swap with the pair partner (same lane, same layout).
      *(MLA_LDS vec8*)(xp_mine + lane * 16) = pmine;
      meet();   // also completes the first value fragment's reads
      vec8 ppair = lds_read_b128<vec8>(lds_addr(xp_pair) + lane * 16);

      // ---- values: my 256 dims, both head tiles -----------------------------
      // Fragment d + VD is read while fragment d is used.
      constexpr int VD = 3;
#pragma unroll
      for (int d = 1; d <= VD; ++d) {
        vr[d][0] = lds_read_tr_b16(vaddr(d));
        vr[d][1] = lds_read_tr_b16(vaddr(d) + 16 * CKV_ROW);
      }
      lds_wait<2 * VD>(ppair);
      const vec8 pv0 = half ? ppair : pmine;   // head tile 0 of the pair
      const vec8 pv1 = half ? pmine : ppair;   // head tile 1
#pragma unroll
      for (int d = 0; d < DT_WAVE; ++d) {
        // Reads issued after fragment d: fragments d+1 .. min(d+VD, 15).
        if (d > 0) {
          if (d + VD < DT_WAVE) lds_wait<2 * VD>(vr[d][1]);
          else if (d + VD == DT_WAVE) lds_wait<2 * (VD - 1)>(vr[d][1]);
          else if (d + VD == DT_WAVE + 1) lds_wait<2 * (VD - 2)>(vr[d][1]);
          else lds_wait<0>(vr[d][1]);
        }
        const vec8 va = __builtin_bit_cast(vec8, u32x4{vr[d][0][0], vr[d][0][1], vr[d][1][0], vr[d][1][1]});
        o[d][0] = E::mfma(va, pv0, o[d][0]);
        o[d][1] = E::mfma(va, pv1, o[d][1]);
        if (d + VD + 1 < DT_WAVE) {
          vr[d + VD + 1][0] = lds_read_tr_b16(vaddr(d + VD + 1));
          vr[d + VD + 1][1] = lds_read_tr_b16(vaddr(d + VD + 1) + 16 * CKV_ROW);
        }
      }
    }

    // Did any head of any wave outgrow its reference? (The pass count must
    // be the same in all four waves: they share barriers.)
    if (pass == 0) {
      if (__any(m_run > m_ref + HEADROOM_LOG2) && lane == 0) *flag = 1u;
      meet();
      if (*(const volatile MLA_LDS uint32_t*)flag == 0u) break;
    }
  }

  // ---- epilogue: swap the sums, normalise and write my dims ---------------
  float l_tot = l_part + shfl_xor(l_part, 16);
  l_tot += shfl_xor(l_tot, 32);
  MLA_LDS float* xml = (MLA_LDS float*)(smem + XML);
  if (lg == 0) xml[wave * 16 + ln] = l_tot;
  meet();
  const float l_pair = xml[(wave ^ 1) * 16 + ln];
  const float inv0 = 1.0f / (half ? l_pair : l_tot);
  const float inv1 = 1.0f / (half ? l_tot : l_pair);
#pragma unroll
  for (int d = 0; d < DT_WAVE; ++d) {
    store(0, half * DT_WAVE + d, o[d][0] * inv0);
    store(1, half * DT_WAVE + d, o[d][1] * inv1);
  }
  if (lg == 0) store_lse(half, m_ref + __builtin_amdgcn_logf(l_tot));
}

}  // namespace

void launch_wide(int dtype, int hpw, unsigned wgs, hipStream_t stream, int32_t groups,
                 int32_t rows_per_req, int32_t slots, int32_t direct, int32_t total_rows,
                 int32_t max_blocks, const int32_t* context_lens, const int32_t* row_indptr,
                 const int32_t* partitions, const int32_t* splits, const int32_t* block_table,
                 const PartitionArgs& a) {
  (void)hpw;  // 64: the only wide layout
  if (dtype == MLA_F16)
    hipLaunchKernelGGL(wide_kernel<0>, dim3(wgs), dim3(THREADS), 0, stream, groups, rows_per_req,
                       slots, direct, total_rows, max_blocks, context_lens, row_indptr,
                       partitions, splits, block_table, a);
  else
    hipLaunchKernelGGL(wide_kernel<1>, dim3(wgs), dim3(THREADS), 0, stream, groups, rows_per_req,
                       slots, direct, total_rows, max_blocks, context_lens, row_indptr,
                       partitions, splits, block_table, a);
}

}  // namespace part
}  // namespace mla
