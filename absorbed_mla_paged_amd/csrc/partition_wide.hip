// Wide partition kernel of split-KV, matrix-absorbed MLA decode on gfx950:
// 64 heads per workgroup (used when 64 divides the head count, e.g. the
// 128-head DeepSeek-V3 shape as two workgroups per row).
//
// Same computation as the 16-head kernel (mlxcel pull request 995, "What
// changed", Stage 1; vllm-metal pull request 601 "[kernel] Wire MLA
// split-KV decode", "What changed"): for one row (a block-aligned token
// range of one request) and a group of heads, the base-2 softmax over
//   s_t = scale * (q_absorbed . ckv_t + q_pe . kpe_t)
// applied to the 512-wide ckv rows, written as a normalised fp32 partial and
// its log2-sum-exp, or rounded into `out` for a single-row request.
//
// With 64 heads the arithmetic per cached byte is high enough that the
// matrix cores and LDS, not HBM, set the pace, so the layout keeps each
// SIMD's MFMA pipe fed from two waves with different jobs:
//  * 512 threads = 8 wave64, two per SIMD (256 registers each; the MFMA
//    accumulators live in VGPRs). Waves 0-3 score, waves 4-7 apply values.
//  * Score wave s scores tokens 16 (s / 2) .. +16 of a 32-token block for
//    heads 32 (s % 2) .. +32 of the workgroup, S^T[token, head] =
//    K[token, :] . Q^T[:, head] on v_mfma_f32_16x16x32 (18 K-steps); Q of
//    its 32 heads (the B operand) sits in 144 VGPRs, so each K fragment read
//    from LDS feeds two MFMAs. It then turns its scores into 16-bit
//    probabilities and publishes them in LDS.
//  * Value wave v accumulates O^T[dim, head] for dims 128 v .. +128 and all
//    64 heads (128 VGPRs) on v_mfma_f32_16x16x32. The MFMA result layout of
//    S^T is already the B-operand layout of P^T; V^T is read from the same
//    LDS tile with ds_read_b64_tr_b16, each fragment feeding four MFMAs.
//  * Pipeline: in step i the score waves work on block i while the value
//    waves apply block i - 1 (probabilities double-buffered by parity); one
//    s_barrier per step. LDS holds a ring of 4 one-block slots (32 KB ckv +
//    4 KB kpe); the value waves copy blocks in with global_load_lds_dwordx4
//    (16 B per lane, a quarter of each block per wave), one copy between
//    the MFMAs of each value fragment: a copy can hold its wave at issue for
//    its share of the CU's vector-memory rate, and meanwhile the score wave
//    on the same SIMD keeps the MFMA pipe busy.
//  * No rescaling inside the loop: every head's reference maximum is the
//    maximum over the row's first block, and probabilities relative to it
//    may grow up to 2^15 (finite in fp16 and bf16, exact to the format's
//    precision). Each score lane tracks the true maximum of its own scores;
//    if any ends more than 15 (base 2) above its head's reference, the
//    workgroup makes a second pass over the row with the exact maxima as
//    references. The accumulators only ever see MFMA updates.
//  * LDS fragment reads in the MFMA loops are issued several MFMAs ahead
//    (dev::lds_read_*), with explicit lgkmcnt waits.
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
constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr int NSC = 4;                          // score waves (0..3)
constexpr int DT_WAVE = LAT / 16 / 4;           // 8 output dim tiles per value wave
constexpr int HT_ALL = HPW / 16;                // 4 head tiles per workgroup
constexpr int OPS = BS + BS * KPE_ROW / 1024;   // 36 copy instructions per block
constexpr int OPW = OPS / 4;                    // 9 per value wave
constexpr int XP = NSLOT * SLOT;                // probabilities [parity][wave][lane] 16 B
constexpr int XM = XP + 2 * NSC * 64 * 16;      // per-head floats [wave][2][16]
constexpr int XFLAG = XM + NSC * 32 * 4;        // "second pass needed" flag
constexpr int LDS_BYTES = XFLAG + 16;
constexpr float HEADROOM_LOG2 = 15.0f;          // p <= 2^15 against the reference
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(OPS % 4 == 0 && 3 * OPW < 64, "copy split / vmcnt range");
static_assert(OPW == DT_WAVE + 1, "one copy per value fragment, plus one");

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
  const bool scorer = wave < NSC;
  const int sw = wave & 3;    // index within the role
  const int hp = sw & 1;      // score waves: my 32 heads are 32 hp .. +32
  const int tt = sw >> 1;     // score waves: my 16 tokens are 16 tt .. +16

  int b, x, hg;
  if (!slot_of(blockIdx.x, groups, rows_per_req, slots, &b, &x, &hg)) return;
  const int hwg = hg * HPW;   // first head of the workgroup

  RowInfo ri;
  if (!find_row(b, x, direct, total_rows, max_blocks, context_lens, row_indptr, partitions,
                splits, &ri))
    return;
  const int row = ri.row;
  const int nblocks = ri.nblocks;
  // Output of value-wave lane (ln, lg) for head tile ht (head hwg + 16 ht +
  // ln) and dim tile dt (dims 16 dt + 4 lg .. + 4).
  auto store = [&](int ht, int dt, f32x4 v) {
    const int64_t h = hwg + 16 * ht + ln;
    const int d0 = dt * 16 + lg * 4;
    if (direct) {
      vec4 hv;
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = static_cast<scalar>(v[e]);
      *reinterpret_cast<vec4*>(reinterpret_cast<uint16_t*>(a.out) +
                               ((int64_t)b * a.heads + h) * LAT + d0) = hv;
    } else {
      *reinterpret_cast<f32x4*>(a.partial_out + ((int64_t)row * a.heads + h) * LAT + d0) = v;
    }
  };
  auto store_lse = [&](int h_local, float v) {
    const int64_t i = (int64_t)(direct ? b : row) * a.heads + hwg + h_local;
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
    // No visible token: zero output, lse2 = -inf (value waves write it).
    if (scorer) return;
#pragma unroll
    for (int ht = 0; ht < HT_ALL; ++ht) {
#pragma unroll
      for (int d = 0; d < DT_WAVE; ++d) store(ht, sw * DT_WAVE + d, f32x4{0.f, 0.f, 0.f, 0.f});
      if (sw == 0 && lg == 0) store_lse(16 * ht + ln, -INFINITY);
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
  // Value wave sw's quarter of block k's copies into slot k % 4: copy i is
  // op 9 sw + i; ops 0..31 are ckv rows, 32..35 kpe rows 8 (op - 32) .. + 8.
  // Chunk c of an LDS row sits at position c ^ swizzle(row).
  auto issue_one = [&](int k, int64_t phys, int i) {
    const uint32_t base = lds0 + (k & (NSLOT - 1)) * SLOT;
    const int op = sw * OPW + i;
    if (op < BS) {
      const uint32_t voff = ((lane & ~15) | ((lane & 15) ^ swz_ckv(op))) * 16;
      dma16s(voff, ckv_base + phys * (BS * CKV_ROW) + op * CKV_ROW, base + op * CKV_ROW);
    } else {
      const int t8 = op - BS;
      const int r = t8 * 8 + (lane >> 3);
      const uint32_t voff = (lane >> 3) * KPE_ROW + ((lane & 7) ^ swz_kpe(r)) * 16;
      dma16s(voff, kpe_base + phys * (BS * KPE_ROW) + t8 * 1024, base + SLOT_KPE + t8 * 1024);
    }
  };

  // Loop-invariant LDS byte offsets inside a slot. Score fragment (K-step
  // ks): row 16 tt + ln, chunk 4 ks + lg; chunks 16 apart keep the same
  // swizzled low bits, so ks = 4 m + kk is offs_k[kk] + 256 m. Value
  // fragment d: dim tile 8 sw + d, rows r1 = 4 lg + ln / 4 and r1 + 16
  // (16 KB further, same swizzle), chunk 2 (8 sw + d) + (ln / 2) % 2.
  const int rk = 16 * tt + ln;
  uint32_t offs_k[4], offs_p[2], offs_v[DT_WAVE];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) offs_k[kk] = rk * CKV_ROW + (((4 * kk + lg) ^ swz_ckv(rk)) * 16);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    offs_p[kk] = SLOT_KPE + rk * KPE_ROW + (((4 * kk + lg) ^ swz_kpe(rk)) * 16);
  const int r1 = 4 * lg + (ln >> 2);
#pragma unroll
  for (int d = 0; d < DT_WAVE; ++d)
    offs_v[d] = r1 * CKV_ROW + ((((2 * d + ((ln >> 1) & 1)) ^ swz_ckv(r1)) + 16 * sw) * 16) +
                (ln & 1) * 8;
  MLA_LDS float* xm = (MLA_LDS float*)(smem + XM);   // [score wave][j][ln]
  MLA_LDS uint32_t* flag = (MLA_LDS uint32_t*)(smem + XFLAG);
  if (tid == 0) *flag = 0u;   // seen by all after the first meeting below

  const float c2 = a.scale_log2;
  const int ntok = ri.tok_hi - ri.tok_lo;

  // The two roles run separate copies of the pass / step loops (so Q and
  // the accumulators are never live in the same wave) that meet at the same
  // barriers in the same order:
  //   per step i:      M_step(i)  [+ M_ref in step 0 of the first pass]
  //   after a pass:    M_flag     [+ M_x1, M_x2 before a second pass]
  //   epilogue:        M_epi
  if (scorer) {
    // Q: lane (ln, lg) of head tile j holds head hwg + 32 hp + 16 j + ln,
    // dims 32 k + 8 lg .. + 8. Score waves issue no copies, so the
    // compiler's own wait for these loads is exact; the first block takes
    // longer to arrive than Q.
    vec8 q[2][KSTEPS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t qr = (int64_t)b * a.heads + hwg + 32 * hp + 16 * j + ln;
      const vec8* qa = reinterpret_cast<const vec8*>(a.q_absorbed + qr * LAT);
      const vec8* qp = reinterpret_cast<const vec8*>(a.q_pe + qr * ROPE);
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k)
        q[j][k] = (k < LAT / 32) ? qa[4 * k + lg] : qp[4 * (k - LAT / 32) + lg];
    }
    float m_ref[2] = {-INFINITY, -INFINITY};  // reference maxima of my heads
    float m_run[2] = {-INFINITY, -INFINITY};  // max of this lane's own scores
    float l_part[2] = {0.f, 0.f};             // this lane's share of the sums
    for (int pass = 0; pass < 2; ++pass) {
      l_part[0] = l_part[1] = 0.f;
      for (int i = 0; i <= nblocks; ++i) {
        meet();   // M_step(i): block i is in LDS; P(i - 2)'s buffer is free
        if (i >= nblocks) continue;
        // ---- scores: my 16 tokens x 32 heads of block i -----------------------
        const uint32_t sbase = lds0 + (i & (NSLOT - 1)) * SLOT;
        const int valid = min(BS, ntok - i * BS);
        auto kaddr = [&](int ks) {
          return sbase + ((ks < LAT / 32) ? offs_k[ks & 3] + 256 * (ks >> 2)
                                          : offs_p[ks - LAT / 32]);
        };
        constexpr int KD = 5;
        f32x4 acc[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        vec8 kf[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) kf[ks] = lds_read_b128<vec8>(kaddr(ks));
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          if (ks + KD <= KSTEPS) lds_wait<KD - 1>(kf[ks]);
          else lds_wait<0>(kf[ks]);   // tail: fewer than KD - 1 reads after ks
          acc[0][ks & 1] = E::mfma(kf[ks], q[0][ks], acc[0][ks & 1]);
          acc[1][ks & 1] = E::mfma(kf[ks], q[1][ks], acc[1][ks & 1]);
          if (ks + KD < KSTEPS) kf[ks + KD] = lds_read_b128<vec8>(kaddr(ks + KD));
        }
        // Lane (ln, lg) holds head 32 hp + 16 j + ln at tokens 16 tt + 4 lg + e.
        float sc[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x4 sv = acc[j][0] + acc[j][1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sc[j][e] = (16 * tt + 4 * lg + e < valid) ? sv[e] * c2 : -INFINITY;
            m_run[j] = fmaxf(m_run[j], sc[j][e]);
          }
        }
        if (pass == 0 && i == 0) {
          // Reference maxima over the whole first block: both token halves
          // (score waves s and s ^ 2 hold the same heads).
          float bm[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            bm[j] = fmaxf(fmaxf(sc[j][0], sc[j][1]), fmaxf(sc[j][2], sc[j][3]));
            bm[j] = fmaxf(bm[j], shfl_xor(bm[j], 16));
            bm[j] = fmaxf(bm[j], shfl_xor(bm[j], 32));
            if (lg == 0) xm[(sw * 2 + j) * 16 + ln] = bm[j];
          }
          meet();   // M_ref
#pragma unroll
          for (int j = 0; j < 2; ++j) m_ref[j] = fmaxf(bm[j], xm[((sw ^ 2) * 2 + j) * 16 + ln]);
        }
        u32x4 pme;   // 16-bit P: head tile 0 tokens e = 0..3, then head tile 1
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          scalar p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = static_cast<scalar>(__builtin_amdgcn_exp2f(sc[j][e] - m_ref[j]));
            l_part[j] += static_cast<float>(p[e]);
          }
          pme[2 * j] = (uint32_t)__builtin_bit_cast(uint16_t, p[0]) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, p[1]) << 16);
          pme[2 * j + 1] = (uint32_t)__builtin_bit_cast(uint16_t, p[2]) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, p[3]) << 16);
        }
        *(MLA_LDS u32x4*)(smem + XP + (((i & 1) * NSC + sw) * 64 + lane) * 16) = pme;
      }
      if (pass == 1) break;
      // Did any score outgrow its head's reference?
      if (__any(m_run[0] > m_ref[0] + HEADROOM_LOG2 || m_run[1] > m_ref[1] + HEADROOM_LOG2) &&
          lane == 0)
        *flag = 1u;
      meet();   // M_flag
      if (*(const volatile MLA_LDS uint32_t*)flag == 0u) break;
      // Second pass: references become the exact maxima of the row.
      float mr[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        mr[j] = fmaxf(m_run[j], shfl_xor(m_run[j], 16));
        mr[j] = fmaxf(mr[j], shfl_xor(mr[j], 32));
        if (lg == 0) xm[(sw * 2 + j) * 16 + ln] = mr[j];
      }
      meet();   // M_x1
#pragma unroll
      for (int j = 0; j < 2; ++j) m_ref[j] = fmaxf(mr[j], xm[((sw ^ 2) * 2 + j) * 16 + ln]);
      meet();   // M_x2: xm is free again
    }
    // ---- epilogue: publish my heads' sums; write the LSE -------------------
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float lt = l_part[j] + shfl_xor(l_part[j], 16);
      lt += shfl_xor(lt, 32);
      if (lg == 0) xm[(sw * 2 + j) * 16 + ln] = lt;
    }
    meet();   // M_epi
    if (tt == 0 && lg == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float l = xm[(sw * 2 + j) * 16 + ln] + xm[((sw + 2) * 2 + j) * 16 + ln];
        store_lse(32 * hp + 16 * j + ln, m_ref[j] + __builtin_amdgcn_logf(l));
      }
    }
    return;
  }

  // ---- value waves ----------------------------------------------------------
  // Their only vector-memory operations before the end are the copies
  // (counted by wait_blocks); the debug store above is wave 0's.
  f32x4 o[DT_WAVE][HT_ALL];
  for (int pass = 0; pass < 2; ++pass) {
    // An opaque zero: a literal one would be hoisted out of the pass loop
    // and kept alive next to the accumulators.
    float zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
#pragma unroll
    for (int d = 0; d < DT_WAVE; ++d)
#pragma unroll
      for (int ht = 0; ht < HT_ALL; ++ht) o[d][ht] = f32x4{zero, zero, zero, zero};
    for (int k = 0; k < NSLOT && k < nblocks; ++k) {
      const int64_t ph = phys_of(k);
#pragma unroll
      for (int c = 0; c < OPW; ++c) issue_one(k, ph, c);
    }
    int64_t phys_next = nblocks > NSLOT ? phys_of(NSLOT) : 0;

    // Step i: apply block i - 1 (i >= 1) while the score waves score block i.
    for (int i = 0; i <= nblocks; ++i) {
      if (i < nblocks) {
        // Block i must be in LDS when the step starts; copies of blocks up
        // to min(max(3, i + 1), nblocks - 1) were issued before this point.
        wait_blocks(min(max(NSLOT - 1, i + 1), nblocks - 1) - i);
        const int valid = min(BS, ntok - i * BS);
        if (valid < BS) {
          // Rows past the context end may hold anything (NaN included): zero
          // the ckv rows this wave brought in, so that 0-probability tokens
          // add exactly 0.
          for (int r = max(valid, sw * OPW); r < min(BS, (sw + 1) * OPW); ++r)
            *(MLA_LDS u32x4*)(smem + (i & (NSLOT - 1)) * SLOT + r * CKV_ROW + lane * 16) =
                u32x4{0u, 0u, 0u, 0u};
        }
      }
      meet();                                   // M_step(i)
      if (pass == 0 && i == 0) meet();          // M_ref
      if (i < 1) continue;
      // ---- values: block i - 1, dims 128 sw .. +128, all 64 heads -------------
      const int kb = i - 1;
      const uint32_t sbase = lds0 + (kb & (NSLOT - 1)) * SLOT;
      // Refill the slot of block i - 2 (free since this step's meeting) with
      // block i + 2, one copy per value fragment.
      const bool refill = i >= 2 && i + 2 < nblocks;
      const int64_t phys_fill = phys_next;
      if (refill && i + 3 < nblocks) phys_next = phys_of(i + 3);
      if (refill) issue_one(i + 2, phys_fill, 0);
      // P^T B operand of head tile ht (pair ht / 2, tile ht % 2): tokens
      // 4 lg + e from score wave ht / 2, 16 + 4 lg + e from score wave ht / 2 + 2.
      const uint32_t pbase = lds0 + XP + ((kb & 1) * NSC * 64 + lane) * 16;
      u32x4 pw[NSC];
#pragma unroll
      for (int v = 0; v < NSC; ++v) pw[v] = lds_read_b128<u32x4>(pbase + v * 64 * 16);
      constexpr int VD = 3;   // value fragments read ahead
      u32x2 vr[DT_WAVE][2];
#pragma unroll
      for (int d = 0; d < VD; ++d) {
        vr[d][0] = lds_read_tr_b16(sbase + offs_v[d]);
        vr[d][1] = lds_read_tr_b16(sbase + offs_v[d] + 16 * CKV_ROW);
      }
      lds_wait<2 * VD>(pw[3]);
      vec8 pv[HT_ALL];
#pragma unroll
      for (int ht = 0; ht < HT_ALL; ++ht) {
        const u32x4 lo = pw[ht >> 1], hi = pw[(ht >> 1) + 2];
        const int jj = 2 * (ht & 1);
        pv[ht] = __builtin_bit_cast(vec8, u32x4{lo[jj], lo[jj + 1], hi[jj], hi[jj + 1]});
      }
#pragma unroll
      for (int d = 0; d < DT_WAVE; ++d) {
        // Reads issued after fragment d: fragments d+1 .. min(d+VD-1, 7).
        if (d + VD <= DT_WAVE) lds_wait<2 * (VD - 1)>(vr[d][1]);
        else if (d + VD == DT_WAVE + 1) lds_wait<2 * (VD - 2)>(vr[d][1]);
        else lds_wait<0>(vr[d][1]);
        const vec8 va =
            __builtin_bit_cast(vec8, u32x4{vr[d][0][0], vr[d][0][1], vr[d][1][0], vr[d][1][1]});
#pragma unroll
        for (int ht = 0; ht < HT_ALL; ++ht) o[d][ht] = E::mfma(va, pv[ht], o[d][ht]);
        if (d + VD < DT_WAVE) {
          vr[d + VD][0] = lds_read_tr_b16(sbase + offs_v[d + VD]);
          vr[d + VD][1] = lds_read_tr_b16(sbase + offs_v[d + VD] + 16 * CKV_ROW);
        }
        if (refill) issue_one(i + 2, phys_fill, d + 1);
      }
    }
    if (pass == 1) break;
    meet();   // M_flag
    if (*(const volatile MLA_LDS uint32_t*)flag == 0u) break;
    meet();   // M_x1
    meet();   // M_x2
  }
  // ---- epilogue: normalise with both token halves' sums of each head ---------
  meet();     // M_epi
#pragma unroll
  for (int ht = 0; ht < HT_ALL; ++ht) {
    const int w0 = ht >> 1, j = ht & 1;   // score waves w0 and w0 + 2
    const float l = xm[(w0 * 2 + j) * 16 + ln] + xm[((w0 + 2) * 2 + j) * 16 + ln];
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < DT_WAVE; ++d) store(ht, sw * DT_WAVE + d, o[d][ht] * inv);
  }
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
