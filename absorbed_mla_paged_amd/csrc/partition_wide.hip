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
// matrix cores and LDS are about as busy as the memory path, so the layout
// keeps each SIMD's MFMA pipe fed from two waves with different jobs:
//  * 512 threads = 8 wave64, two per SIMD (256 registers each). Waves 0-3
//    score, waves 4-7 apply values. The big per-wave arrays live in AGPRs:
//    Q (the score MFMAs' B operand) in score waves, the accumulators in
//    value waves (each wave gets 128 VGPRs and 128 AGPRs).
//  * Score wave s scores tokens 16 (s / 2) .. +16 of a 32-token block for
//    heads 32 (s % 2) .. +32 of the workgroup, S^T[token, head] =
//    K[token, :] . Q^T[:, head] on v_mfma_f32_16x16x32 (18 K-steps); Q of
//    its 32 heads (the B operand) sits in registers (mostly AGPRs), so
//    each K fragment read from LDS feeds two MFMAs. It then turns its scores
//    into 16-bit probabilities (the scale folded into the exponent's fma,
//    row sums by dot2 against ones) and publishes them in LDS.
//  * Value wave v accumulates O^T[dim, head] for dims 128 v .. +128 and all
//    64 heads (128 AGPRs) on v_mfma_f32_16x16x32. The MFMA result layout of
//    S^T is already the B-operand layout of P^T; V^T is read from the same
//    LDS tile with ds_read_b64_tr_b16, each fragment feeding four MFMAs.
//  * Pipeline: in step i the score waves work on block i while the value
//    waves apply block i - 1 (probabilities double-buffered by parity); one
//    s_barrier per step. LDS holds a ring of 4 one-block slots (32 KB ckv +
//    4 KB kpe), filled by the value waves with global_load_lds_dwordx4 (16 B
//    per lane, a quarter of each block per wave): blocks 0 and 1 before the
//    first step, then block i + 2 right after the meeting of step i, into
//    the slot of block i - 2 that the meeting has just freed. Each block
//    thus has two steps to arrive; that lead, not the arithmetic, bounds the
//    kernel. Before step 0 all waves stage the workgroup's Q through slots 2
//    and 3, and the score waves read their fragments from there.
//  * No rescaling inside the loop: every head's reference maximum is the
//    maximum over the row's first block, and probabilities relative to it
//    may grow up to 2^15 (finite in fp16 and bf16, exact to the format's
//    precision). Each score lane tracks the true maximum of its own scores;
//    if any ends more than 15 (base 2) above its head's reference, the
//    workgroup makes a second pass over the row with the exact maxima as
//    references. The accumulators only ever see MFMA updates.
//  * LDS fragment reads in the MFMA loops are issued several MFMAs ahead
//    (dev::lds_read_*), with explicit lgkmcnt waits that name every register
//    they guard.
//  * Partials go out as device-scope write-through buffer stores.
#include "partition_common.h"

#include <cmath>
#include <type_traits>

namespace mla {
namespace part {
namespace {

using namespace dev;

constexpr int HPW = 64;                         // heads per workgroup
constexpr int SLOT = SEG * (CKV_ROW + KPE_ROW); // 36 KB per one-block slot
constexpr int SLOT_KPE = SEG * CKV_ROW;         // kpe rows after the ckv rows
constexpr int NSLOT = 4;
// The value waves copy blocks 0 and 1 before the first step and block
// i + 2 right after the meeting of step i, into the slot of block i - 2.
constexpr int NPRO = 2;
constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr int NSC = 4;                          // score waves (0..3)
constexpr int DT_WAVE = LAT / 16 / 4;           // 8 output dim tiles per value wave
constexpr int HT_ALL = HPW / 16;                // 4 head tiles per workgroup
constexpr int OPS = SEG + SEG * KPE_ROW / 1024; // 36 copy instructions per block
constexpr int OPW = OPS / 4;                    // 9 per value wave
// E4M3 caches: the ring holds the cache bytes as stored (18 KB per block)
// and the MFMA loops widen each fragment after reading it from LDS.
constexpr int CKV_ROW8 = LAT;                        // 512 bytes
constexpr int KPE_ROW8 = ROPE;                       // 64 bytes
constexpr int SLOT8 = SEG * (CKV_ROW8 + KPE_ROW8);   // 18 KB per one-block slot
constexpr int SLOT_KPE8 = SEG * CKV_ROW8;
constexpr int OPW8 = 5;   // per value wave: 4 ckv copies of 2 rows, 8 kpe rows on 32 lanes
constexpr int QBYTES = HPW * (CKV_ROW + KPE_ROW);    // the workgroup's Q, 72 KB
// LDS layout: the ring of NSLOT slots, the Q staging from slot 2 on (idle
// until step 0), then the probabilities [parity][wave][lane] 16 B, the
// per-head floats [wave][2][16] and the "second pass needed" flag.
template <bool KV8> struct Lds {
  static constexpr int slot = KV8 ? SLOT8 : SLOT;
  static constexpr int q = 2 * slot;
  static constexpr int xp = q + QBYTES > NSLOT * slot ? q + QBYTES : NSLOT * slot;
  static constexpr int xm = xp + 2 * NSC * 64 * 16;
  static constexpr int flag = xm + NSC * 32 * 4;
  static constexpr int bytes = flag + 16;
  static_assert(bytes <= 160 * 1024, "LDS budget");
};
constexpr float HEADROOM_LOG2 = 15.0f;          // p <= 2^15 against the reference
// LDS fragments read ahead in the score and value MFMA loops (at most 15
// LDS reads may be in flight: the lgkmcnt field has 4 bits).
constexpr int KD_SCORE = 8;
constexpr int VD_VALUE = 5;
static_assert(KD_SCORE <= 15 && 4 + 2 * VD_VALUE <= 15, "lgkmcnt range");
static_assert(OPS % 4 == 0 && 3 * OPW < 64 && 3 * OPW8 < 64, "copy split / vmcnt range");
static_assert(4 * 4 * 2 * CKV_ROW8 == SLOT_KPE8 && 4 * 8 * KPE_ROW8 == SEG * KPE_ROW8,
              "E4M3 copy split: 4 x 4 two-row ckv copies and 4 x 8 kpe rows per block");

// E4M3 rows: chunk c (16 bytes) of ckv row r sits at c ^ swz8_ckv(r) (32
// chunks, the low 4 bits permuted), of kpe row r at c ^ swz8_kpe(r) (4
// chunks). 16 consecutive rows of either 16-token half, and the rows
// {0..7, 16..23} or {8..15, 24..31}, each take 16 distinct bank groups.
__device__ __forceinline__ int swz8_ckv(int r) { return (r & 15) ^ (((r >> 4) & 1) << 3); }
__device__ __forceinline__ int swz8_kpe(int r) { return (r >> 2) & 3; }

// Two probabilities rounded (to nearest even) into the 16-bit type, packed
// low / high; and the sum of such a pair added to an fp32 total (one dot2
// against (1, 1): exact products, one fp32 accumulation).
template <int DT> struct Prob;
template <> struct Prob<0> {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
  }
  static __device__ __forceinline__ float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, p), h2{(_Float16)1.0f, (_Float16)1.0f},
                                  acc, false);
  }
};
template <> struct Prob<1> {
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, h2{(__bf16)a, (__bf16)b});
  }
  static __device__ __forceinline__ float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(h2, p),
                                           h2{(__bf16)1.0f, (__bf16)1.0f}, acc, false);
  }
};

// Physical cache blocks holding one 32-token segment (both entries equal
// when the cache block is 32 tokens).
struct Phys {
  int64_t p[2];
};

// Wait until at most `later` blocks' worth of this wave's copies are still
// in flight (copies complete in issue order).
// W is the number of copy instructions per block and wave.
template <int W>
__device__ __forceinline__ void wait_blocks(int later) {
  switch (later) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<W>(); break;
    case 2: wait_vmcnt<2 * W>(); break;
    default: wait_vmcnt<3 * W>(); break;
  }
}

// Make this wave's LDS writes visible, then meet the other waves. No memory
// fence: the in-flight LDS copies must not be waited for here.
__device__ __forceinline__ void meet() {
  wait_lgkmcnt0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A "block" below is one 32-token segment of the row: one cache block of
// PG = 32 tokens, or two of PG = 16 (looked up separately in the table).
// KV8: the cache holds E4M3 bytes (times the one scale folded into
// scale_log2 and out_scale).
template <int DT, int PG, bool KV8>
__global__ __launch_bounds__(THREADS, 1) void wide_kernel(
    int32_t groups, int32_t batch, int32_t slots, int32_t flags, int32_t total_rows,
    int32_t max_blocks, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ row_indptr, const int32_t* __restrict__ partitions,
    const int32_t* __restrict__ splits, const int32_t* __restrict__ block_table,
    PartitionArgs a) {
  typedef Elem<DT> E;
  typedef typename E::vec8 vec8;
  typedef typename E::vec4 vec4;
  typedef typename E::scalar scalar;
  typedef Prob<DT> P;
  typedef Lds<KV8> L;
  constexpr int OPWK = KV8 ? OPW8 : OPW;   // copy instructions per block and value wave

  __shared__ __attribute__((aligned(1024))) char smem_raw[L::bytes];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lane_id = lane;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15;   // MFMA row/column inside a 16-wide tile
  const int lg = lane >> 4;   // MFMA k-group (0..3)
  const bool scorer = wave < NSC;
  const int sw = wave & 3;    // index within the role
  const int hp = sw & 1;      // score waves: my 32 heads are 32 hp .. +32
  const int tt = sw >> 1;     // score waves: my 16 tokens are 16 tt .. +16

  int u, hg;
  if (!slot_of(blockIdx.x, groups, slots, &u, &hg)) return;
  const int hwg = hg * HPW;   // first head of the workgroup

  const int direct = flags & 1;
  RowInfo ri;
  if (!find_row<PG>(u, batch, direct, total_rows, hidden_tail(flags, hwg), max_blocks,
                    context_lens, row_indptr, partitions, splits, &ri))
    return;
  const int b = ri.b;
  const int row = ri.row;
  const int nblocks = ri.nseg;   // 32-token blocks of the row
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
      // Written through the L2, from this workgroup's 64-head region of the row.
      const WtRegion part(a.partial_out + ((int64_t)row * a.heads + hwg) * LAT, HPW * LAT * 4);
      part.store((uint32_t)((16 * ht + ln) * LAT + d0) * 4, v);
    }
  };
  auto store_lse = [&](int h_local, float v) {
    const int64_t i = (int64_t)(direct ? b : row) * a.heads + hwg + h_local;
    float* lp = direct ? a.lse2_out : a.partial_lse2;
    if (lp) __hip_atomic_store(lp + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (a.debug_ranges && hg == 0 && tid == 0) {
    a.debug_ranges[2 * row] = ri.tok_lo;
    a.debug_ranges[2 * row + 1] = ri.tok_end;
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

  const int ntok_all = ri.tok_hi - ri.tok_lo;
  const int64_t tbl0 = (int64_t)b * max_blocks + ri.blk_lo;
  const int last_phys = a.num_blocks - 1;
  const char* ckv_base = reinterpret_cast<const char*>(a.ckv);
  const char* kpe_base = reinterpret_cast<const char*>(a.kpe);
  const uint32_t lds0 = lds_addr(smem);
  // Physical cache blocks of 32-token block k: with PG = 16 its two
  // halves, the second clamped to the row's last cache block with a token
  // (a half-filled last block reads its first half twice; rows past the end
  // are zeroed before use). With PG = 32 both are the one block.
  const int last_page = cdiv(ntok_all, PG) - 1;
  auto phys_of = [&](int k) {
    Phys ph;
    const int c0 = k * (SEG / PG);
    const int v0 = __builtin_amdgcn_readfirstlane(load_const(block_table, tbl0 + c0));
    ph.p[0] = (int64_t)max(0, min(v0, last_phys));
    if constexpr (PG == SEG) {
      ph.p[1] = ph.p[0];
    } else {
      const int c1 = min(c0 + 1, last_page);
      const int v1 = __builtin_amdgcn_readfirstlane(load_const(block_table, tbl0 + c1));
      ph.p[1] = (int64_t)max(0, min(v1, last_phys));
    }
    return ph;
  };
  // Value wave sw's quarter of block k's copies into slot k % 4: copy i is
  // op 9 sw + i; ops 0..31 are ckv rows, 32..35 kpe rows 8 (op - 32) .. + 8.
  // Chunk c of an LDS row sits at position c ^ swizzle(row).
  auto issue_one = [&](int k, const Phys& ph, int i) {
    const uint32_t base = lds0 + (k & (NSLOT - 1)) * L::slot;
    const int op = sw * OPW + i;
    // The lane offsets are recomputed per copy from an opaque lane index:
    // hoisted out of the step loop they would hold registers throughout it.
    int lane;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane) : "v"(lane_id));
    if constexpr (KV8) {
      // E4M3: copies 0..3 of value wave sw are ckv rows 2 o and 2 o + 1
      // (o = 4 sw + i; 32 lanes of 16 bytes each), copy 4 its kpe rows
      // 8 sw .. + 8 on lanes 0..31.
      if (i < 4) {
        const int o = 4 * sw + i;
        const int r = 2 * o + (lane >> 5);
        const uint32_t voff = (lane >> 5) * CKV_ROW8 + ((lane & 31) ^ swz8_ckv(r)) * 16;
        const int64_t pj = (PG == SEG || 2 * o < PG) ? ph.p[0] : ph.p[1];   // wave-uniform
        dma16s(voff, ckv_base + pj * (PG * CKV_ROW8) + ((2 * o) % PG) * CKV_ROW8,
               base + o * 2 * CKV_ROW8);
      } else if (lane < 32) {
        const int r = 8 * sw + (lane >> 2);
        const uint32_t voff = (lane >> 2) * KPE_ROW8 + ((lane & 3) ^ swz8_kpe(r)) * 16;
        const int64_t pj = (PG == SEG || 8 * sw < PG) ? ph.p[0] : ph.p[1];
        dma16s(voff, kpe_base + pj * (PG * KPE_ROW8) + ((8 * sw) % PG) * KPE_ROW8,
               base + SLOT_KPE8 + 8 * sw * KPE_ROW8);
      }
    } else if (op < SEG) {
      // ckv row op: row op % PG of cache block op / PG of the segment.
      const uint32_t voff = ((lane & ~15) | ((lane & 15) ^ swz_ckv(op))) * 16;
      const int64_t pj = (PG == SEG || op < PG) ? ph.p[0] : ph.p[1];   // wave-uniform
      dma16s(voff, ckv_base + pj * (PG * CKV_ROW) + (op % PG) * CKV_ROW, base + op * CKV_ROW);
    } else {
      // kpe rows 8 t8 .. + 8, all in one cache block.
      const int t8 = op - SEG;
      const int r = t8 * 8 + (lane >> 3);
      const uint32_t voff = (lane >> 3) * KPE_ROW + ((lane & 7) ^ swz_kpe(r)) * 16;
      const int64_t pj = (PG == SEG || t8 * 8 < PG) ? ph.p[0] : ph.p[1];
      dma16s(voff, kpe_base + pj * (PG * KPE_ROW) + ((t8 * 8) % PG) * KPE_ROW,
             base + SLOT_KPE + t8 * 1024);
    }
  };

  // Rows past the context end may hold anything (NaN included): after its
  // own copies of the last block have landed, a wave zeroes the ckv rows it
  // brought in, so that 0-probability tokens add exactly 0.
  auto zero_tail = [&](int k) {
    const int valid = min(SEG, ntok_all - k * SEG);
    if (valid < SEG) {
      if constexpr (KV8) {
        for (int r = max(valid, 8 * sw); r < 8 * sw + 8; ++r)
          *(MLA_LDS u32x2*)(smem + (k & (NSLOT - 1)) * L::slot + r * CKV_ROW8 + lane * 8) =
              u32x2{0u, 0u};
      } else {
        for (int r = max(valid, sw * OPW); r < min(SEG, (sw + 1) * OPW); ++r)
          *(MLA_LDS u32x4*)(smem + (k & (NSLOT - 1)) * L::slot + r * CKV_ROW + lane * 16) =
              u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // During step i the value waves fetch block i + 2 into the slot of block
  // i - 2, free since the step's meeting. `next` holds the block table entry
  // of the following refill, read one step ahead.
  auto refill = [&](int i, Phys& next) {
    if (i + 2 >= NPRO && i + 2 < nblocks) {
      const Phys ph = next;
      if (i + 3 < nblocks) next = phys_of(i + 3);
#pragma unroll
      for (int c = 0; c < OPWK; ++c) issue_one(i + 2, ph, c);
    }
  };

  // Q of the workgroup's 64 heads (64 rows of 512 latent dims, then 64 rows
  // of 64 rope dims: 72 KB) goes through LDS once, into ring slots 2 and 3,
  // which stay idle until step 0; each of the 8 waves copies 9 KB of it.
  // Loaded per score wave straight from memory it would cost every CU
  // 144 KB (two waves share each head), twice the first two KV blocks.
  // Rows are swizzled like the KV rows.
  const uint32_t qlds = lds0 + L::q;
  static_assert(QBYTES == 2 * SLOT && 8 * OPW == HPW + HPW * KPE_ROW / 1024,
                "Q staging: 72 KB in 8 x 9 copies");
  auto issue_q = [&]() {
    const int64_t q0 = (int64_t)b * a.heads + hwg;
    const char* qa_base = reinterpret_cast<const char*>(a.q_absorbed + q0 * LAT);
    const char* qp_base = reinterpret_cast<const char*>(a.q_pe + q0 * ROPE);
    int lane;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane) : "v"(lane_id));
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int op = wave * OPW + i;   // 0..63 latent rows, 64..71 rope rows 8 (op - 64) .. + 8
      if (op < HPW) {
        const uint32_t voff = ((lane & ~15) | ((lane & 15) ^ swz_ckv(op))) * 16;
        dma16s(voff, qa_base + op * CKV_ROW, qlds + op * CKV_ROW);
      } else {
        const int t8 = op - HPW;
        const int r = t8 * 8 + (lane >> 3);
        const uint32_t voff = (lane >> 3) * KPE_ROW + ((lane & 7) ^ swz_kpe(r)) * 16;
        dma16s(voff, qp_base + t8 * 1024, qlds + HPW * CKV_ROW + t8 * 1024);
      }
    }
  };

  MLA_LDS float* xm = (MLA_LDS float*)(smem + L::xm);   // [score wave][j][ln]
  MLA_LDS uint32_t* flag = (MLA_LDS uint32_t*)(smem + L::flag);
  if (tid == 0) *flag = 0u;   // seen by all after the first meeting below

  const float c2 = a.scale_log2;
  const int ntok = ri.tok_hi - ri.tok_lo;

  // The two roles run separate copies of the pass / step loops (so Q and
  // the accumulators are never live in the same wave) that meet at the same
  // barriers in the same order:
  //   before step 0:   M_q (Q is in LDS)
  //   per step i:      M_step(i)  [+ M_ref in step 0 of the first pass]
  //   after a pass:    M_flag     [+ M_x1, M_x2 before a second pass]
  //   epilogue:        M_epi
  if (scorer) {
    // Q: lane (ln, lg) of head tile j holds head hwg + 32 hp + 16 j + ln,
    // dims 32 k + 8 lg .. + 8, read from the LDS copy of Q. With two waves
    // per SIMD the compiler gives each wave 128 VGPRs and 128 AGPRs, and it
    // puts every MFMA accumulator in AGPRs (here the four score chains, 16
    // registers). The first KA K-steps of Q (112 registers) are read
    // straight into AGPRs, which the score MFMAs use as their B operand; the
    // rest go to VGPRs.
    issue_q();
    wait_vmcnt<0>();
    meet();   // M_q: Q is in LDS
    constexpr int KA = 14;
    u32x4 q[2][KA];
    vec8 qv[2][KSTEPS - KA];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 32 * hp + 16 * j + ln;
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        const uint32_t addr =
            k < LAT / 32 ? qlds + r * CKV_ROW + (((4 * k + lg) ^ swz_ckv(r)) * 16)
                         : qlds + HPW * CKV_ROW + r * KPE_ROW +
                               (((4 * (k - LAT / 32) + lg) ^ swz_kpe(r)) * 16);
        if (k < KA)
          asm volatile("ds_read_b128 %0, %1" : "=a"(q[j][k]) : "v"(addr) : "memory");
        else
          qv[j][k - KA] = lds_read_b128<vec8>(addr);
      }
    }
    // The reads are asynchronous to the compiler: wait, then tie every value
    // to that wait (a use is safe only after an ordered asm statement).
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int k = 0; k < KA; ++k) asm volatile("" : "+a"(q[j][k]));
#pragma unroll
      for (int k = 0; k < KSTEPS - KA; ++k) asm volatile("" : "+v"(qv[j][k]));
    }
    auto qfrag = [&](int j, int ks) {
      return ks < KA ? __builtin_bit_cast(vec8, q[j][ks < KA ? ks : 0])
                     : qv[j][ks < KA ? 0 : ks - KA];
    };
    // Loop-invariant LDS byte offsets inside a slot. Score fragment (K-step
    // ks): row 16 tt + ln, chunk 4 ks + lg; chunks 16 apart keep the same
    // swizzled low bits, so ks = 4 m + kk is offs_k[kk] + 256 m.
    // E4M3 fragment (K-step ks): the 8 bytes of row 16 tt + ln at byte
    // 32 ks + 8 lg, i.e. half lg % 2 of chunk 2 ks + lg / 2; chunks 16 apart
    // keep the same swizzled low bits, so ks = 8 m + kk is offs_k[kk] + 256 m.
    const int rk = 16 * tt + ln;
    constexpr int NOFF = KV8 ? 8 : 4;
    uint32_t offs_k[NOFF], offs_p[2];
#pragma unroll
    for (int kk = 0; kk < NOFF; ++kk)
      offs_k[kk] = KV8 ? rk * CKV_ROW8 + (((2 * kk + (lg >> 1)) ^ swz8_ckv(rk)) * 16) + (lg & 1) * 8
                       : rk * CKV_ROW + (((4 * kk + lg) ^ swz_ckv(rk)) * 16);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      offs_p[kk] = KV8 ? SLOT_KPE8 + rk * KPE_ROW8 +
                             (((2 * kk + (lg >> 1)) ^ swz8_kpe(rk)) * 16) + (lg & 1) * 8
                       : SLOT_KPE + rk * KPE_ROW + (((4 * kk + lg) ^ swz_kpe(rk)) * 16);
    float m_ref[2] = {-INFINITY, -INFINITY};  // reference maxima of my heads (scaled)
    float m_run[2] = {-INFINITY, -INFINITY};  // max of this lane's own raw scores
    float l_part[2] = {0.f, 0.f};             // this lane's share of the sums
    for (int pass = 0; pass < 2; ++pass) {
      l_part[0] = l_part[1] = 0.f;
      for (int i = 0; i <= nblocks; ++i) {
        meet();   // M_step(i): block i is in LDS; P(i - 2)'s buffer is free
        if (i >= nblocks) continue;
        // ---- scores: my 16 tokens x 32 heads of block i -----------------------
        const uint32_t sbase = lds0 + (i & (NSLOT - 1)) * L::slot;
        const int valid = min(SEG, ntok - i * SEG);
        auto kaddr = [&](int ks) {
          return sbase + ((ks < LAT / 32) ? offs_k[ks % NOFF] + 256 * (ks / NOFF)
                                          : offs_p[ks - LAT / 32]);
        };
        // A K fragment as read from LDS (8 E4M3 bytes, or 8 16-bit values)
        // and as the MFMA takes it.
        using KRaw = std::conditional_t<KV8, u32x2, vec8>;
        auto kread = [&](int ks) -> KRaw {
          if constexpr (KV8) return lds_read_b64(kaddr(ks));
          else return lds_read_b128<vec8>(kaddr(ks));
        };
        auto kwide = [&](const KRaw& r) -> vec8 {
          if constexpr (KV8) return __builtin_bit_cast(vec8, widen8<DT>(r[0], r[1]));
          else return r;
        };
        constexpr int KD = KD_SCORE;
        f32x4 acc[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        KRaw kf[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) kf[ks] = kread(ks);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          lds_wait_n(min(KD - 1, KSTEPS - 1 - ks), kf[ks]);   // reads issued after ks
          const vec8 kv = kwide(kf[ks]);
          acc[0][ks & 1] = E::mfma(kv, qfrag(0, ks), acc[0][ks & 1]);
          acc[1][ks & 1] = E::mfma(kv, qfrag(1, ks), acc[1][ks & 1]);
          if (ks + KD < KSTEPS) kf[ks + KD] = kread(ks + KD);
          // Keep the MFMAs between their waits: sunk below later waits they
          // would stop overlapping the reads.
          __builtin_amdgcn_sched_barrier(0);
        }
        // Lane (ln, lg) holds head 32 hp + 16 j + ln at tokens 16 tt + 4 lg + e.
        // Raw dot products: the scale goes into the exponent's fma, and
        // maxima are tracked unscaled (the scale is positive).
        float sc[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x4 sv = acc[j][0] + acc[j][1];
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[j][e] = sv[e];
        }
        if (valid < SEG) {   // the row's last block: hide tokens past its end
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (16 * tt + 4 * lg + e >= valid) sc[j][e] = -INFINITY;
        }
        float bm[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bm[j] = fmaxf(fmaxf(sc[j][0], sc[j][1]), fmaxf(sc[j][2], sc[j][3]));
          m_run[j] = fmaxf(m_run[j], bm[j]);
        }
        if (pass == 0 && i == 0) {
          // Reference maxima over the whole first block: both token halves
          // (score waves s and s ^ 2 hold the same heads).
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            bm[j] = fmaxf(bm[j], shfl_xor(bm[j], 16));
            bm[j] = fmaxf(bm[j], shfl_xor(bm[j], 32));
            if (lg == 0) xm[(sw * 2 + j) * 16 + ln] = bm[j];
          }
          meet();   // M_ref
#pragma unroll
          for (int j = 0; j < 2; ++j)
            m_ref[j] = c2 * fmaxf(bm[j], xm[((sw ^ 2) * 2 + j) * 16 + ln]);
        }
        u32x4 pme;   // 16-bit P: head tile 0 tokens e = 0..3, then head tile 1
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float pf[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pf[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j][e], c2, -m_ref[j]));
          pme[2 * j] = P::pack2(pf[0], pf[1]);
          pme[2 * j + 1] = P::pack2(pf[2], pf[3]);
          l_part[j] = P::sum2(pme[2 * j + 1], P::sum2(pme[2 * j], l_part[j]));
        }
        *(MLA_LDS u32x4*)(smem + L::xp + (((i & 1) * NSC + sw) * 64 + lane) * 16) = pme;
      }
      if (pass == 1) break;
      // Did any score outgrow its head's reference?
      if (__any(c2 * m_run[0] > m_ref[0] + HEADROOM_LOG2 ||
                c2 * m_run[1] > m_ref[1] + HEADROOM_LOG2) &&
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
      for (int j = 0; j < 2; ++j) m_ref[j] = c2 * fmaxf(mr[j], xm[((sw ^ 2) * 2 + j) * 16 + ln]);
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
  // LDS byte offsets of the value fragments inside a slot. Fragment d: dim
  // tile 8 sw + d, rows r1 = 4 lg + ln / 4 and r1 + 16 (16 KB further, same
  // swizzle), chunk c = 2 (8 sw + d) + (ln / 2) % 2 stored at c ^ swz(r1),
  // i.e. at 16 sw + 2 (d ^ (swz / 2)) + ((ln / 2) ^ swz) % 2. They are
  // rebuilt each step from an opaque copy of swz (three VALU operations per
  // fragment) instead of being held in eight registers.
  //
  // E4M3: fragment d is one 8-bit transposing read. Lanes 2 k and 2 k + 1
  // of a 16-lane group address the two 8-byte halves of dims 16 (8 sw + d)
  // .. + 16 of token T_k (4 lg + k, then 16 + 4 lg + k - 4: the token order
  // of the P^T operand), so lane ln receives dim 16 (8 sw + d) + ln of
  // tokens T_0 .. T_7, the A-operand layout. Chunk 8 sw + d of row T sits at
  // ((8 sw) ^ (swz & 8)) + (d ^ (swz & 7)).
  const int r1 = 4 * lg + (ln >> 2);
  const int t8 = (ln >> 1) < 4 ? 4 * lg + (ln >> 1) : 12 + 4 * lg + (ln >> 1);
  const int swz_v = KV8 ? swz8_ckv(t8) : swz_ckv(r1);
  const uint32_t vrow =
      KV8 ? t8 * CKV_ROW8 + ((8 * sw) ^ (swz_v & 8)) * 16 + (ln & 1) * 8
          : r1 * CKV_ROW + (16 * sw + (((ln >> 1) ^ swz_v) & 1)) * 16 + (ln & 1) * 8;
  f32x4 o[DT_WAVE][HT_ALL];
  // Block kb's values into o. The first block of a pass starts the
  // accumulators from a zero C operand instead of a separate zeroing (which
  // the compiler would keep apart from the accumulators and copy around).
  auto apply = [&](int kb, auto first_block) {
    constexpr bool first = decltype(first_block)::value;
    const uint32_t sbase = lds0 + (kb & (NSLOT - 1)) * L::slot;
    int sh;
    if constexpr (KV8)
      asm volatile("v_and_b32 %0, 7, %1" : "=v"(sh) : "v"(swz_v));        // swz & 7, opaque
    else
      asm volatile("v_lshrrev_b32 %0, 1, %1" : "=v"(sh) : "v"(swz_v));   // swz / 2, opaque
    const uint32_t vbase = sbase + vrow;
    auto vaddr = [&](int d) { return vbase + (KV8 ? 16u : 32u) * (uint32_t)(d ^ sh); };
    // P^T B operand of head tile ht (pair ht / 2, tile ht % 2): tokens
    // 4 lg + e from score wave ht / 2, 16 + 4 lg + e from score wave ht / 2 + 2.
    const uint32_t pbase = lds0 + L::xp + ((kb & 1) * NSC * 64 + lane) * 16;
    u32x4 pw[NSC];
#pragma unroll
    for (int v = 0; v < NSC; ++v) pw[v] = lds_read_b128<u32x4>(pbase + v * 64 * 16);
    constexpr int VD = VD_VALUE;
    constexpr int RPF = KV8 ? 1 : 2;   // LDS reads per fragment
    u32x2 vr[DT_WAVE][2];
    auto vread = [&](int d) {
      if constexpr (KV8) {
        vr[d][0] = lds_read_tr_b8(vaddr(d));
      } else {
        vr[d][0] = lds_read_tr_b16(vaddr(d));
        vr[d][1] = lds_read_tr_b16(vaddr(d) + 16 * CKV_ROW);
      }
    };
#pragma unroll
    for (int d = 0; d < VD; ++d) vread(d);
    lds_wait<RPF * VD>(pw[0], pw[1]);
    lds_wait<RPF * VD>(pw[2], pw[3]);
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
      vec8 va;
      if constexpr (KV8) {
        lds_wait_n(min(VD - 1, DT_WAVE - 1 - d), vr[d][0]);
        va = __builtin_bit_cast(vec8, widen8<DT>(vr[d][0][0], vr[d][0][1]));
      } else {
        lds_wait_n(2 * min(VD - 1, DT_WAVE - 1 - d), vr[d][0], vr[d][1]);
        va = __builtin_bit_cast(vec8, u32x4{vr[d][0][0], vr[d][0][1], vr[d][1][0], vr[d][1][1]});
      }
#pragma unroll
      for (int ht = 0; ht < HT_ALL; ++ht)
        o[d][ht] = E::mfma(va, pv[ht], first ? f32x4{0.f, 0.f, 0.f, 0.f} : o[d][ht]);
      if (d + VD < DT_WAVE) vread(d + VD);
      __builtin_amdgcn_sched_barrier(0);   // as in the score loop
    }
  };
  issue_q();
  for (int pass = 0; pass < 2; ++pass) {
    // Blocks 0 and 1 before the first step (the rest during the steps).
    const int npro = min(NPRO, nblocks);
    for (int k = 0; k < npro; ++k) {
      const Phys ph = phys_of(k);
#pragma unroll
      for (int c = 0; c < OPWK; ++c) issue_one(k, ph, c);
    }
    if (pass == 0) {
      wait_blocks<OPWK>(npro);   // my part of Q has landed (the block copies may not have)
      meet();              // M_q
    }
    // Start of step i: block i must be in LDS (my later copies, of blocks
    // i + 1 .. last, may still be in flight), then M_step(i), then the copy
    // of block i + 2.
    Phys phys_next = nblocks > NPRO ? phys_of(NPRO) : Phys{{0, 0}};
    auto step_begin = [&](int i) {
      if (i < nblocks) {
        const int last = min(max(npro - 1, i + 1), nblocks - 1);
        wait_blocks<OPWK>(last - i);
        if (i == nblocks - 1) zero_tail(i);
      }
      meet();
      if (i < nblocks) refill(i, phys_next);
    };
    // Step i applies block i - 1 while the score waves score block i.
    step_begin(0);
    if (pass == 0) meet();   // M_ref
    step_begin(1);
    apply(0, std::true_type{});
    for (int i = 2; i <= nblocks; ++i) {
      step_begin(i);
      apply(i - 1, std::false_type{});
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
    float inv = 1.0f / l;
    if constexpr (KV8) inv *= a.out_scale;
#pragma unroll
    for (int d = 0; d < DT_WAVE; ++d) store(ht, sw * DT_WAVE + d, o[d][ht] * inv);
  }
}

}  // namespace

void launch_wide(int dtype, int block_size, bool kv8, unsigned wgs, hipStream_t stream,
                 int32_t groups, int32_t batch, int32_t slots, int32_t flags,
                 int32_t total_rows, int32_t max_blocks, const int32_t* context_lens,
                 const int32_t* row_indptr, const int32_t* partitions, const int32_t* splits,
                 const int32_t* block_table, const PartitionArgs& a) {
  decltype(&wide_kernel<0, 16, false>) kernel;
  if (kv8)
    kernel = dtype == MLA_F16
                 ? (block_size == 16 ? wide_kernel<0, 16, true> : wide_kernel<0, 32, true>)
                 : (block_size == 16 ? wide_kernel<1, 16, true> : wide_kernel<1, 32, true>);
  else
    kernel = dtype == MLA_F16
                 ? (block_size == 16 ? wide_kernel<0, 16, false> : wide_kernel<0, 32, false>)
                 : (block_size == 16 ? wide_kernel<1, 16, false> : wide_kernel<1, 32, false>);
  hipLaunchKernelGGL(kernel, dim3(wgs), dim3(THREADS), 0, stream, groups, batch, slots,
                     flags, total_rows, max_blocks, context_lens, row_indptr, partitions, splits,
                     block_table, a);
}

}  // namespace part
}  // namespace mla
