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
// Mapping onto one CU: 512 threads = 8 wave64, two per SIMD.
//  * Stages: the row is cut into stages of 64 tokens (two 32-token cache
//    blocks, or four of 16: 64 KB of ckv + 8 KB of kpe), held in two
//    alternating LDS slots. The cache block size PG is a template
//    parameter; it changes only the index math and the table lookups.
//  * Copy waves (4..7) move stages in with global_load_lds_dwordx4 (16 B per
//    lane, one 1 KB row per instruction, so whole 128 B lines). Once the
//    memory queue of the CU is full, issuing a copy blocks the issuing wave;
//    keeping copies on their own waves means that block never delays the
//    arithmetic. Copy waves 4,5 serve slot 0, waves 6,7 slot 1; each waits
//    for its own copies and then bumps the slot's "ready" counter in LDS.
//  * Compute waves (0..3) wait on those counters, never on memory, and bump
//    the slot's "free" counter when done with it.
//  * Within an LDS row the 16-byte chunk c sits at position c ^ swz(row),
//    which keeps the row-wise reads of the score product and the transposed
//    reads of the value product free of bank conflicts.
//  * Scores: S^T[token, head] = K[token, :] . Q^T[:, head] on
//    v_mfma_f32_16x16x32 (K = 576 = 18 steps); compute wave w scores the
//    stage's 16-token tile w. Q (16 x 576) sits in their registers.
//  * Online softmax in the base-2 domain: each compute wave writes its raw
//    score tile to LDS and, after one meeting point per stage, reads all four
//    back. The MFMA output layout is the same in every wave, so lane (ln, lg)
//    reads exactly the 16 scores it needs: head ln at tokens 16 t + 4 lg + j,
//    which is also the B-operand layout of the value product. Every compute
//    wave then takes the same maximum, probabilities and running sum itself.
//    The running maximum only moves when a stage beats it by more than 2^8,
//    so rescaling is rare. The compute waves meet through an LDS counter
//    (never s_barrier, which would also wait for the copy waves).
//  * Values: O^T[dim, head] += V^T[dim, token] . P^T[token, head] on
//    v_mfma_f32_16x16x32; V^T is read from the same LDS tile with
//    ds_read_b64_tr_b16. Compute wave w owns dims [128 w, 128 w + 128).
//  * LDS fragment reads in both MFMA loops are issued ahead from inline asm
//    (dev::lds_read_*) with explicit lgkmcnt waits; a wait names every
//    register it guards.
//  * Outputs go out as device-scope write-through buffer stores, so the
//    release at the end of the kernel has no dirty partial lines left to
//    write back before the reduce can start.
//  * Caches stored as E4M3 bytes (KV8): the copy waves load a stage's bytes
//    into registers (half the bytes of a 16-bit stage), widen them to the
//    16-bit type -- exactly, every E4M3 value is an fp16 and a bf16 value --
//    and write them into the same swizzled LDS tile, so the compute waves
//    run unchanged. The cache scale is folded into the score scale and into
//    the output's normalisation.
#include "fused_common.h"
#include "partition_common.h"

#include <cmath>
#include <type_traits>

namespace mla {
namespace {

using namespace dev;
using namespace part;

constexpr int ST_TOK = 2 * SEG;                 // tokens per stage
constexpr int ST_KPE = ST_TOK * CKV_ROW;        // kpe rows after the ckv rows
constexpr int STAGE = ST_TOK * (CKV_ROW + KPE_ROW);   // 72 KB
constexpr int CWAVES = 4;                       // compute waves
constexpr int THREADS = 64 * 2 * CWAVES;        // plus as many copy waves
constexpr int HG = 16;                          // heads per workgroup
constexpr int DT_PER_WAVE = LAT / 16 / CWAVES;  // 8 output dim tiles per wave
constexpr int OPS_PER_COPY = STAGE / 1024 / 2;  // 36 copies per copy wave
// After the two slots: counters ready[2], free[2], issued, scored; then the
// score tiles [2 parities][4 tiles][64 lanes][16 B].
constexpr int XCNT = 2 * STAGE;
constexpr int XS = XCNT + 64;
constexpr int LDS_BYTES = XS + 2 * CWAVES * 64 * 16;
static_assert(OPS_PER_COPY * 2 * 1024 == STAGE, "stage split");
static_assert(OPS_PER_COPY < 64, "vmcnt range");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// The leading scalar kernel arguments (16 dwords, up to block_table) are
// preloaded into SGPRs at wave launch on gfx950, so finding the row costs
// no argument fetch; the PartitionArgs block is fetched meanwhile.
template <int DT, bool FUSED, int PG, bool KV8>
__global__ __launch_bounds__(THREADS) void partition_kernel(
    int32_t groups, int32_t batch, int32_t slots, int32_t flags, int32_t total_rows,
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
  const bool copier = wave >= CWAVES;
  const int direct = flags & 1;

  // ---- which (request, row, head group) this workgroup owns -------------
  // Slot u is the global row of a split launch (its request found in
  // row_indptr) or the request of a single-pass one (slot_of).
  int u, hg;
  if (!slot_of(blockIdx.x, groups, slots, &u, &hg)) return;
  const int b = direct ? u : request_of_row(row_indptr, batch, u);

  const int head0 = hg * HG;
  const int64_t qrow0 = (int64_t)b * a.heads + head0;   // first (b, head) row
  const int my_head = head0 + ln;

  // Fused launches: the bases of the merge hand-off state, read first.
  uint64_t* fh = nullptr;
  uint64_t f_sbase = 0, f_abase = 0, f_seen = 0;
  if constexpr (FUSED) {
    fh = fused::header(a.sync, b, hg);
    if (tid == 0) {
      f_sbase = fused::ld(fh + fused::kSbase);
      f_abase = fused::ld(fh + fused::kAbase);
    }
  }

  // All row metadata in one round trip.
  int n = load_const(context_lens, b);
  int P = 1, S = 1, row = b, x = 0, nrows = 1;
  if (!direct) {
    const int r0 = load_const(row_indptr, b);
    const int r1 = load_const(row_indptr, b + 1);
    const int pv = load_const(partitions, b);
    const int sv = load_const(splits, b);
    nrows = r1 - r0;
    P = max(1, min(pv, 1 << 25));
    S = max(1, min(sv, 1 << 25));
    row = u;
    x = u - r0;
  }
  n = max(0, min(n, max_blocks * PG));
  if (x < 0 || x >= nrows || row < 0 || row >= total_rows) return;
  if constexpr (FUSED) {
    if (tid == 0)
      __hip_atomic_fetch_add(fh + fused::kStarted, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int p = x / S;
  const int s = x % S;
  // Index math of mla_partition_range (must agree bit for bit).
  const int nblk = cdiv(n, PG);
  const int bpp = cdiv(nblk, P);
  const int pb0 = min(p * bpp, nblk);
  const int pb1 = min((p + 1) * bpp, nblk);
  const int m = pb1 - pb0;
  const int bps = m > 0 ? cdiv(m, S) : 0;
  const int blk_lo = (p < P) ? pb0 + min(s * bps, m) : nblk;
  const int blk_hi = (p < P) ? pb0 + min((s + 1) * bps, m) : nblk;
  const int tok_lo = min(blk_lo * PG, n);
  const int tok_end = min(blk_hi * PG, n);   // the row's range
  // With several new tokens per request, this head group belongs to one new
  // token, which does not see the last hidden_tail() tokens of the context.
  const int n_vis = max(0, n - hidden_tail(flags, head0));
  const int tok_hi = max(tok_lo, min(tok_end, n_vis));
  constexpr int NPG = ST_TOK / PG;                 // cache blocks per stage
  const int nblocks = cdiv(tok_hi - tok_lo, PG);   // non-empty cache blocks
  const int nst = cdiv(nblocks, NPG);               // stages

  // LDS counters, zeroed behind one barrier (it waits for the scalar loads
  // above, never for Q or the table).
  MLA_LDS uint32_t* ready = (MLA_LDS uint32_t*)(smem + XCNT);
  MLA_LDS uint32_t* freed = ready + 2;
  MLA_LDS uint32_t* issued = ready + 4;
  MLA_LDS uint32_t* scored = ready + 5;  // compute waves: score tiles written
  MLA_LDS uint32_t* stored = ready + 6;  // compute waves: outputs stored (fused)
  MLA_LDS uint32_t* decided = ready + 7; // merge pieces known (fused)
  MLA_LDS int32_t* pieces = (MLA_LDS int32_t*)(ready + 8);   // first, count
  // Copy waves read their first stage's block-table entries before the
  // start-up barrier, so that round trip overlaps the other waves' arrival
  // (a stage with fewer cache blocks than NPG repeats its last block).
  int64_t first_phys[NPG] = {};
  if (copier) {
    const int slot0 = (wave - CWAVES) >> 1;
    if (slot0 < nst) {
      const int nb_here = min(NPG, nblocks - NPG * slot0);
#pragma unroll
      for (int j = 0; j < NPG; ++j) {
        const int blk = blk_lo + NPG * slot0 + min(j, nb_here - 1);
        const int v = __builtin_amdgcn_readfirstlane(
            load_const(block_table, (int64_t)b * max_blocks + blk));
        first_phys[j] = (int64_t)max(0, min(v, a.num_blocks - 1));
      }
    }
  }
  if (tid < 8) ready[tid] = 0u;
  __syncthreads();

  // Fused launches, every wave at its end (compute waves once their stores
  // are issued): hand this row over, then merge the pieces it is given,
  // reusing stage slot 0 of the LDS for the merge's exchange.
  auto tail = [&]() {
    if (!copier) {
      wait_vmcnt<0>();   // this wave's stores have completed
      bump_counter(stored, lane);
      if (tid == 0) {
        wait_counter(stored, CWAVES);
        const fused::Decision d = fused::arrive(fh, f_sbase, f_abase, f_seen, nrows);
        pieces[0] = d.first;
        pieces[1] = d.count;
        bump_counter(decided, lane);
      }
    }
    wait_counter(decided, 1);
    const int first = __builtin_amdgcn_readfirstlane(pieces[0]);
    const int count = __builtin_amdgcn_readfirstlane(pieces[1]);
    const fused::MergeArgs ma{a.partial_out, a.partial_lse2, a.out, a.lse2_out, a.heads};
    for (int i = 0; i < count; ++i)
      fused::merge_piece<DT, THREADS>(ma, first + i, nrows, (int64_t)(row - x), b, head0, HG, smem);
  };

  // Q (compute waves), loaded after the barrier: it is needed only once
  // the first stage has landed, and its kernel-argument fetch and loads
  // would otherwise hold the compute waves (and so the copy waves) at the
  // barrier. B operand of the score product: lane (ln, lg) holds head
  // head0 + ln, dims 32 k + 8 lg .. + 8. Compute waves issue no copies, so
  // the compiler's own wait for Q is exact.
  vec8 q[KSTEPS];
  if (!copier) {
    const vec8* qa = reinterpret_cast<const vec8*>(a.q_absorbed + (qrow0 + ln) * LAT);
    const vec8* qp = reinterpret_cast<const vec8*>(a.q_pe + (qrow0 + ln) * ROPE);
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k)
      q[k] = (k < LAT / 32) ? qa[4 * k + lg] : qp[4 * (k - LAT / 32) + lg];
  }


  if (nst <= 0) {
    // No visible token: zero output, lse2 = -inf.
    if (copier) {
      if constexpr (FUSED) tail();
      return;
    }
    if constexpr (FUSED) {
      if (tid == 0) f_seen = fused::ld(fh + fused::kStarted);
    }
#pragma unroll
    for (int dt = 0; dt < DT_PER_WAVE; ++dt) {
      const int d0 = (wave * DT_PER_WAVE + dt) * 16 + lg * 4;
      if (direct) {
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.heads + my_head) * LAT + d0;
        *reinterpret_cast<u32x2*>(o) = u32x2{0u, 0u};
      } else {
        float* o = a.partial_out + ((int64_t)row * a.heads + my_head) * LAT + d0;
        *reinterpret_cast<f32x4*>(o) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (wave == 0 && lg == 0) {
      if (direct) {
        if (a.lse2_out) a.lse2_out[(int64_t)b * a.heads + my_head] = -INFINITY;
      } else {
        a.partial_lse2[(int64_t)row * a.heads + my_head] = -INFINITY;
      }
    }
    if (a.debug_ranges && hg == 0 && tid == 0) {
      a.debug_ranges[2 * row] = tok_lo;
      a.debug_ranges[2 * row + 1] = tok_end;
    }
    if constexpr (FUSED) tail();
    return;
  }

  if (copier && KV8) {
    // ---- copy waves, E4M3 cache: pair `slot` serves stages slot, slot + 2,
    // ... Each wave loads its half of a stage's 36 KB of bytes into
    // registers (18 one-KB loads: ops 0..31 are ckv rows 2 op and 2 op + 1,
    // 32 lanes x 16 B each; ops 32..35 kpe rows 16 (op - 32) .. + 16, 4
    // lanes each), issued before the slot is free; then widens them into the
    // slot's 16-bit tile, zeros for rows past the range's end.
    constexpr int OPS8 = ST_TOK * (LAT + ROPE) / 1024 / 2;   // 18
    const int cw = wave - CWAVES;
    const int slot = cw >> 1;
    const int64_t tbl0 = (int64_t)b * max_blocks;
    const int last_blk = a.num_blocks - 1;
    const char* ckv8 = reinterpret_cast<const char*>(a.ckv);
    const char* kpe8 = reinterpret_cast<const char*>(a.kpe);
    MLA_LDS char* sb = smem + slot * STAGE;
    struct Blocks {
      int64_t p[NPG];
    };
    auto lookup = [&](int k) {
      Blocks r;
      const int nb_here = min(NPG, nblocks - NPG * k);
#pragma unroll
      for (int j = 0; j < NPG; ++j) {
        const int blk = blk_lo + NPG * k + min(j, nb_here - 1);
        const int v = __builtin_amdgcn_readfirstlane(load_const(block_table, tbl0 + blk));
        r.p[j] = (int64_t)max(0, min(v, last_blk));
      }
      return r;
    };
    // The wave's half is a compile-time constant inside `run`, so every
    // load's cache block is a fixed element of the lookup (no indexing).
    auto run = [&](auto half_c) {
      constexpr int half = decltype(half_c)::value;
      Blocks phys_next;
#pragma unroll
      for (int j = 0; j < NPG; ++j) phys_next.p[j] = first_phys[j];   // stage `slot`
      for (int k = slot, g = 0; k < nst; k += 2, ++g) {
        const Blocks phys = phys_next;
        if (k + 2 < nst) phys_next = lookup(k + 2);
        wait_counter(issued, 2 * k);
        u32x4 v[OPS8];
#pragma unroll
        for (int i = 0; i < OPS8; ++i) {
          const int op = half * OPS8 + i;
          const char* src;
          if (op < ST_TOK / 2) {
            const int r0 = 2 * op;   // both rows sit in one cache block
            src = ckv8 + phys.p[r0 / PG] * (PG * LAT) + (r0 % PG + (lane >> 5)) * LAT + (lane & 31) * 16;
          } else {
            const int r0 = 16 * (op - ST_TOK / 2);
            src = kpe8 + phys.p[r0 / PG] * (PG * ROPE) + (r0 % PG + (lane >> 2)) * ROPE +
                  (lane & 3) * 16;
          }
          v[i] = *reinterpret_cast<const u32x4*>(src);
        }
        if (lane == 0) __hip_atomic_fetch_add(issued, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        wait_counter(freed + slot, CWAVES * g);
        const int valid = min(ST_TOK, tok_hi - (tok_lo + k * ST_TOK));
#pragma unroll
        for (int i = 0; i < OPS8; ++i) {
          const int op = half * OPS8 + i;
          u32x4 e0 = widen8<DT>(v[i][0], v[i][1]);   // elements 0..7 of the lane's 16
          u32x4 e1 = widen8<DT>(v[i][2], v[i][3]);   // elements 8..15
          // Chunk c of a row sits at position c ^ swizzle(row).
          if (op < ST_TOK / 2) {
            const int r = 2 * op + (lane >> 5);
            const int c = 2 * (lane & 31);
            if (r >= valid) e0 = e1 = u32x4{0u, 0u, 0u, 0u};
            *(MLA_LDS u32x4*)(sb + r * CKV_ROW + ((c ^ swz_ckv(r)) * 16)) = e0;
            *(MLA_LDS u32x4*)(sb + r * CKV_ROW + (((c + 1) ^ swz_ckv(r)) * 16)) = e1;
          } else {
            const int r = 16 * (op - ST_TOK / 2) + (lane >> 2);
            const int c = 2 * (lane & 3);
            if (r >= valid) e0 = e1 = u32x4{0u, 0u, 0u, 0u};
            *(MLA_LDS u32x4*)(sb + ST_KPE + r * KPE_ROW + ((c ^ swz_kpe(r)) * 16)) = e0;
            *(MLA_LDS u32x4*)(sb + ST_KPE + r * KPE_ROW + (((c + 1) ^ swz_kpe(r)) * 16)) = e1;
          }
        }
        bump_counter(ready + slot, lane);
      }
    };
    if (cw & 1) run(std::integral_constant<int, 1>{});
    else run(std::integral_constant<int, 0>{});
    return;
  }

  if (copier) {
    // ---- copy waves: pair `slot` serves stages slot, slot + 2, ... ------
    const int cw = wave - CWAVES;
    const int slot = cw >> 1;
    const int half = cw & 1;            // ops [36 half, 36 half + 36)
    const int64_t tbl0 = (int64_t)b * max_blocks;
    const int last_blk = a.num_blocks - 1;
    const char* ckv_base = reinterpret_cast<const char*>(a.ckv);
    const char* kpe_base = reinterpret_cast<const char*>(a.kpe);
    const uint32_t base = lds_addr(smem) + slot * STAGE;
    // Physical blocks of stage k (a stage with fewer cache blocks than
    // NPG copies its last block again, an L2 hit; those rows are either
    // never read or zeroed below). Looked up one stage ahead, so the
    // block-table round trip overlaps the waits below; the first stage's
    // were read before the start-up barrier.
    auto lookup = [&](int k, int64_t* ph) {
      const int nb_here = min(NPG, nblocks - NPG * k);
#pragma unroll
      for (int j = 0; j < NPG; ++j) {
        const int blk = blk_lo + NPG * k + min(j, nb_here - 1);
        const int v = __builtin_amdgcn_readfirstlane(load_const(block_table, tbl0 + blk));
        ph[j] = (int64_t)max(0, min(v, last_blk));
      }
    };
    int64_t phys[NPG], phys_next[NPG];
#pragma unroll
    for (int j = 0; j < NPG; ++j) phys_next[j] = first_phys[j];   // stage `slot`
    for (int k = slot, g = 0; k < nst; k += 2, ++g) {
#pragma unroll
      for (int j = 0; j < NPG; ++j) phys[j] = phys_next[j];
      if (k + 2 < nst) lookup(k + 2, phys_next);
      wait_counter(freed + slot, CWAVES * g);
      // Stages are issued in order, so the memory queue returns them in
      // order and stage k can be computed while stage k + 1 is arriving.
      wait_counter(issued, 2 * k);
      // ops 0..63: ckv row op of the stage (cache block op / PG, row
      // op % PG); 64..71: kpe rows 8 (op - 64) .. + 8 of the stage.
#pragma unroll
      for (int i = 0; i < OPS_PER_COPY; ++i) {
        const int op = half * OPS_PER_COPY + i;
        if (op < ST_TOK) {
          const int j = op / PG, r = op % PG;
          const int chunk = (lane & ~15) | ((lane & 15) ^ swz_ckv(op));
          dma16(ckv_base + phys[j] * (PG * CKV_ROW) + r * CKV_ROW + chunk * 16,
                base + op * CKV_ROW);
        } else {
          const int t8 = op - ST_TOK;
          const int sr = t8 * 8 + (lane >> 3);   // row of the stage
          const int j = (t8 * 8) / PG;            // the 8 rows share a cache block
          const int chunk = (lane & 7) ^ swz_kpe(sr);
          dma16(kpe_base + phys[j] * (PG * KPE_ROW) + (sr % PG) * KPE_ROW + chunk * 16,
                base + ST_KPE + t8 * 1024);
        }
      }
      if (lane == 0) __hip_atomic_fetch_add(issued, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      wait_vmcnt<0>();
      const int valid = min(ST_TOK, tok_hi - (tok_lo + k * ST_TOK));
      if (valid < ST_TOK) {
        // Rows past the context end may hold anything (NaN included): zero
        // the latent values of the ones this wave brought in, so that
        // 0-probability tokens add exactly 0. A stage of at most 32 tokens
        // never reads rows 32..63.
        const int zend = min(valid <= SEG ? SEG : ST_TOK, half ? 64 : 36);
        const int zbeg = max(valid, half ? 36 : 0);
        for (int idx = lane; idx < (zend - zbeg) * (CKV_ROW / 16); idx += 64) {
          const int r = zbeg + idx / (CKV_ROW / 16);
          const int c = idx % (CKV_ROW / 16);
          *(MLA_LDS u32x4*)(smem + slot * STAGE + r * CKV_ROW + c * 16) = u32x4{0u, 0u, 0u, 0u};
        }
      }
      bump_counter(ready + slot, lane);
    }
    if constexpr (FUSED) tail();
    return;
  }

  // ---- compute waves ------------------------------------------------------
  f32x4 o[DT_PER_WAVE];
#pragma unroll
  for (int dt = 0; dt < DT_PER_WAVE; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference maximum of my head, base 2
  float l_part = 0.f;       // this lane's 16 token slots of the running sum
  const float c2 = a.scale_log2;
  const int tt = wave;      // my score tile: tokens 16 tt .. 16 tt + 15 of a stage

  // LDS byte offsets inside a stage. Score fragment (K-step ks): row
  // 16 tt + ln, chunk 4 ks + lg; chunks 16 apart keep the same swizzled low
  // bits, so ks = 4 m + kk sits at offs_k[kk] + 256 m. Value fragment
  // (K-step kb, dim tile 8 tt + dt): rows r1 = 32 kb + 4 lg + ln / 4 and
  // r1 + 16 (same swizzle), chunk 2 (8 tt + dt) + (ln / 2) % 2, i.e. at
  // voff + 32 KB kb + 32 (dt ^ (swz / 2)).
  const int rk = 16 * tt + ln;
  uint32_t offs_k[4], offs_p[2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) offs_k[kk] = rk * CKV_ROW + (((4 * kk + lg) ^ swz_ckv(rk)) * 16);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    offs_p[kk] = ST_KPE + rk * KPE_ROW + (((4 * kk + lg) ^ swz_kpe(rk)) * 16);
  const int rv = 4 * lg + (ln >> 2);
  const int swz_v = swz_ckv(rv);
  const uint32_t voff = rv * CKV_ROW + (ln & 1) * 8 + 16 * (16 * tt + (((ln >> 1) ^ swz_v) & 1));
  const int vsh = swz_v >> 1;

  // Normalise and write this workgroup's output: 16 heads x my 128 dims
  // (fp32 partial of row `row`, or the rounded output when the request is a
  // single row) and the base-2 LSE, all written through the L2 from
  // wave-uniform regions (32 KB of partials per workgroup: the stores are
  // bound by the CU's store rate).
  auto finish = [&]() {
    float l_tot = l_part + shfl_xor(l_part, 16);
    l_tot = l_tot + shfl_xor(l_tot, 32);
    float inv = 1.0f / l_tot;
    if constexpr (KV8) inv *= a.out_scale;
    const int dbase = wave * DT_PER_WAVE * 16 + lg * 4;
    const uint32_t e_off = (uint32_t)(ln * LAT + dbase);   // element offset in the region
    if (direct) {
      const WtRegion dst(reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.heads + head0) * LAT,
                         HG * LAT * 2);
#pragma unroll
      for (int dt = 0; dt < DT_PER_WAVE; ++dt) {
        vec4 hv;
#pragma unroll
        for (int j = 0; j < 4; ++j) hv[j] = static_cast<scalar>(o[dt][j] * inv);
        dst.store(e_off * 2 + dt * 32, __builtin_bit_cast(u32x2, hv));
      }
    } else {
      const WtRegion dst(a.partial_out + ((int64_t)row * a.heads + head0) * LAT,
                         HG * LAT * 4);
#pragma unroll
      for (int dt = 0; dt < DT_PER_WAVE; ++dt) dst.store(e_off * 4 + dt * 64, o[dt] * inv);
    }
    if (wave == 0) {
      // Lanes with the same head write the same value.
      float* lp = direct ? a.lse2_out : a.partial_lse2;
      const WtRegion lse(lp ? lp + (int64_t)(direct ? b : row) * a.heads + head0 : nullptr,
                         lp ? HG * 4 : 0);
      lse.store((uint32_t)ln * 4, m_ref + __builtin_amdgcn_logf(l_tot));
    }
  };

  for (int k = 0; k < nst; ++k) {
    const int slot = k & 1;
    const uint32_t sbase = lds_addr(smem) + slot * STAGE;
    const int valid = min(ST_TOK, tok_hi - (tok_lo + k * ST_TOK));
    wait_counter(ready + slot, 2 * (k / 2 + 1));

    // ---- scores of my tile: all 18 K fragments read ahead (14 in flight)
    float xs[4];
    if (16 * tt < valid) {
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      auto kaddr = [&](int ks) {
        return sbase + ((ks < LAT / 32) ? offs_k[ks & 3] + 256 * (ks >> 2) : offs_p[ks - LAT / 32]);
      };
      constexpr int KD = 14;
      vec8 kf[KSTEPS];
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) kf[ks] = lds_read_b128<vec8>(kaddr(ks));
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        lds_wait_n(min(KD - 1, KSTEPS - 1 - ks), kf[ks]);
        acc[ks & 1] = E::mfma(kf[ks], q[ks], acc[ks & 1]);
        if (ks + KD < KSTEPS) kf[ks + KD] = lds_read_b128<vec8>(kaddr(ks + KD));
        __builtin_amdgcn_sched_barrier(0);   // keep each MFMA between its waits
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tk = 16 * tt + 4 * lg + j;
        xs[j] = (tk < valid) ? (acc[0][j] + acc[1][j]) * c2 : -INFINITY;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) xs[j] = -INFINITY;
    }
    // Publish my tile, meet, read all four tiles (same lane, same layout).
    const uint32_t sbuf = lds_addr(smem) + XS + (k & 1) * (CWAVES * 64 * 16);
    *(MLA_LDS f32x4*)(smem + XS + (k & 1) * (CWAVES * 64 * 16) + (tt * 64 + lane) * 16) =
        f32x4{xs[0], xs[1], xs[2], xs[3]};
    bump_counter(scored, lane);
    wait_counter(scored, CWAVES * (k + 1));
    f32x4 tile[CWAVES];
#pragma unroll
    for (int t = 0; t < CWAVES; ++t) tile[t] = lds_read_b128<f32x4>(sbuf + (t * 64 + lane) * 16);

    lds_wait<0>(tile[0], tile[1]);
    lds_wait<0>(tile[2], tile[3]);
    float sc[16];
#pragma unroll
    for (int t = 0; t < CWAVES; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[4 * t + j] = tile[t][j];
    float bm = sc[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) bm = fmaxf(bm, sc[j]);
    bm = fmaxf(bm, shfl_xor(bm, 16));
    bm = fmaxf(bm, shfl_xor(bm, 32));
    // Consume the shuffled maximum here, so that the compiler's wait for
    // the shuffles (lgkmcnt(0)) comes before the value reads below.
    asm volatile("" : "+v"(bm));
    __builtin_amdgcn_sched_barrier(0);

    // Values, K-step kb = tokens 32 kb .. 32 kb + 31, dim tiles 8 tt + dt:
    // fragment f = 8 kb + dt. Their transposed reads do not depend on the
    // probabilities, so the first VD fragments are issued before the
    // exponentials (after the cross-lane maximum, whose LDS-routed shuffles
    // the compiler waits for with lgkmcnt(0)). A one-block stage has one
    // K-step (its second half is never read).
    constexpr int VD = 7;   // fragments in flight: 2 VD <= 15
    auto vaddr = [&](int f) {
      return sbase + voff + (f >> 3) * (SEG * CKV_ROW) + 32u * (uint32_t)((f & 7) ^ vsh);
    };
    u32x2 vr[2 * DT_PER_WAVE][2];
#pragma unroll
    for (int f = 0; f < VD; ++f) {
      vr[f][0] = lds_read_tr_b16(vaddr(f));
      vr[f][1] = lds_read_tr_b16(vaddr(f) + 16 * CKV_ROW);
    }
    const bool need = bm > m_ref + RESCALE_LOG2;
    if (__any(need)) {
      const float m_new = need ? bm : m_ref;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
#pragma unroll
      for (int dt = 0; dt < DT_PER_WAVE; ++dt) o[dt] *= alpha;
      l_part *= alpha;
      m_ref = m_new;
    }
    // The B operand of lane (ln, lg) at K-step kb is P of head ln at tokens
    // 32 kb + 4 lg + j and 32 kb + 16 + 4 lg + j (j < 4): scores sc[8 kb + j].
    // Masked tokens give p = 0 exactly.
    vec8 pv[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const scalar pj = static_cast<scalar>(__builtin_amdgcn_exp2f(sc[8 * kb + j] - m_ref));
        pv[kb][j] = pj;
        l_part += static_cast<float>(pj);
      }
    auto values = [&](auto nfrag_tag) {
      constexpr int NF = decltype(nfrag_tag)::value;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        lds_wait_n(2 * min(VD - 1, NF - 1 - f), vr[f][0], vr[f][1]);
        const vec8 va =
            __builtin_bit_cast(vec8, u32x4{vr[f][0][0], vr[f][0][1], vr[f][1][0], vr[f][1][1]});
        o[f & 7] = E::mfma(va, pv[f >> 3], o[f & 7]);
        if (f + VD < NF) {
          vr[f + VD][0] = lds_read_tr_b16(vaddr(f + VD));
          vr[f + VD][1] = lds_read_tr_b16(vaddr(f + VD) + 16 * CKV_ROW);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (valid > SEG) values(std::integral_constant<int, 2 * DT_PER_WAVE>{});
    else values(std::integral_constant<int, DT_PER_WAVE>{});
    bump_counter(freed + slot, lane);
  }
  if constexpr (FUSED) {
    // All N workgroups of the request have begun by now unless the launch
    // did not fit the device at once.
    if (tid == 0) f_seen = fused::ld(fh + fused::kStarted);
  }
  finish();
  if (a.debug_ranges && hg == 0 && tid == 0) {
    a.debug_ranges[2 * row] = tok_lo;
    a.debug_ranges[2 * row + 1] = tok_end;
  }
  if constexpr (FUSED) tail();
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

namespace {

// Checks and launch shared by mla_decode_partition and mla_decode_fused.
int partition_launch(bool fused, bool kv8, float kv_scale, const void* q_absorbed,
                     const void* q_pe, const void* ckv_cache,
                     const void* kpe_cache, int32_t num_blocks, int32_t block_size,
                     const int32_t* block_table,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                     int32_t num_heads, int32_t q_len, float scale, int32_t dtype,
                     const int32_t* partitions,
                     const int32_t* splits, const int32_t* row_indptr, int32_t total_rows,
                     int32_t max_rows_per_req, int32_t heads_per_wg, float* partial_out,
                     float* partial_lse2, void* out, float* lse2_out, uint64_t* sync,
                     int32_t* debug_ranges, hipStream_t stream) {
  clear_error();
  if (batch < 0) return fail(MLA_E_SHAPE, "batch %d < 0", batch);
  if (num_heads < MLA_MIN_HEADS || num_heads > MLA_MAX_HEADS || num_heads % 16)
    return fail(MLA_E_UNSUPPORTED, "num_heads %d (need a multiple of 16 in [16, 128])",
                num_heads);
  if (dtype != MLA_F16 && dtype != MLA_BF16) return fail(MLA_E_UNSUPPORTED, "dtype %d", dtype);
  if (q_len < 1 || q_len > MLA_MAX_QLEN)
    return fail(MLA_E_UNSUPPORTED, "q_len %d (need 1 .. %d)", q_len, MLA_MAX_QLEN);
  const int32_t hpw = heads_per_wg ? heads_per_wg : default_heads_per_wg(num_heads);
  if (!valid_heads_per_wg(num_heads, hpw))
    return fail(MLA_E_UNSUPPORTED, "heads_per_wg %d for %d heads (16 or 64 dividing it)",
                hpw, num_heads);
  if (kv8 && !(std::isfinite(kv_scale) && kv_scale > 0.0f))
    return fail(MLA_E_RANGE, "kv_scale must be finite and > 0");
  if (!valid_block_size(block_size))
    return fail(MLA_E_UNSUPPORTED, "block_size %d (16 or 32 are supported)", block_size);
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(MLA_E_RANGE, "scale must be finite and > 0");
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
    if (fused) {
      if (!out || !sync) return fail(MLA_E_NULL, "fused split plan needs `out` and `sync`");
      if (!aligned(out, 16) || !aligned(sync, 64))
        return fail(MLA_E_ALIGN, "out (16 bytes) or sync (64 bytes) misaligned");
    }
  }
  if (!aligned(q_absorbed, 16) || !aligned(q_pe, 16) || !aligned(ckv_cache, 16) ||
      !aligned(kpe_cache, 16))
    return fail(MLA_E_ALIGN, "16-bit tensors must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4) || (lse2_out && !aligned(lse2_out, 4)) ||
      (debug_ranges && !aligned(debug_ranges, 8)))
    return fail(MLA_E_ALIGN, "int32/fp32 arrays misaligned");
  const bool merge_here = fused && !direct;
  const int32_t qrows = q_len * num_heads;   // query rows per request
  if (merge_here && hpw != HG)
    return fail(MLA_E_UNSUPPORTED, "fused merge with %d heads per workgroup", hpw);
  if (merge_here && qrows / hpw > fused::kGroupsPerRequest)
    return fail(MLA_E_UNSUPPORTED, "fused merge with %d head groups per request (at most %d)",
                qrows / hpw, fused::kGroupsPerRequest);

  part::PartitionArgs a;
  a.q_absorbed = static_cast<const uint16_t*>(q_absorbed);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.ckv = static_cast<const uint16_t*>(ckv_cache);
  a.kpe = static_cast<const uint16_t*>(kpe_cache);
  a.partial_out = partial_out;
  a.partial_lse2 = partial_lse2;
  a.out = out;
  a.lse2_out = lse2_out;
  a.debug_ranges = debug_ranges;
  a.sync = merge_here ? sync : nullptr;
  a.num_blocks = num_blocks;
  a.heads = qrows;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_scale = 1.0f;
  if (kv8) {
    a.scale_log2 *= kv_scale;
    a.out_scale = kv_scale;
  }
  const int32_t groups = qrows / hpw;
  // One slot per request (single pass) or per row (split): see slot_of.
  const int64_t slots = direct ? batch : total_rows;
  const int64_t wgs = ((slots + 7) / 8) * 8 * groups;
  if (wgs > INT32_MAX || slots > INT32_MAX)
    return fail(MLA_E_SHAPE, "grid too large (%lld workgroups)", (long long)wgs);
  const dim3 grid((unsigned)wgs), block(THREADS);
  const int32_t dflag = part::pack_flags(direct, q_len, num_heads), sl = (int32_t)slots;
  if (hpw != HG)
    part::launch_wide(dtype, block_size, kv8, (unsigned)wgs, stream, groups, batch, sl, dflag,
                      total_rows, max_blocks_per_seq, context_lens, row_indptr, partitions,
                      splits, block_table, a);
#define MLA_LAUNCH(K)                                                                        \
  hipLaunchKernelGGL(K, grid, block, 0, stream, groups, batch, sl, dflag, total_rows, \
                     max_blocks_per_seq, context_lens, row_indptr, partitions, splits,       \
                     block_table, a)
  else if (kv8) {
    if (block_size == 16 && dtype == MLA_F16) MLA_LAUNCH((partition_kernel<0, false, 16, true>));
    else if (block_size == 16) MLA_LAUNCH((partition_kernel<1, false, 16, true>));
    else if (dtype == MLA_F16) MLA_LAUNCH((partition_kernel<0, false, 32, true>));
    else MLA_LAUNCH((partition_kernel<1, false, 32, true>));
  } else if (block_size == 16) {
    if (dtype == MLA_F16 && merge_here) MLA_LAUNCH((partition_kernel<0, true, 16, false>));
    else if (dtype == MLA_F16) MLA_LAUNCH((partition_kernel<0, false, 16, false>));
    else if (merge_here) MLA_LAUNCH((partition_kernel<1, true, 16, false>));
    else MLA_LAUNCH((partition_kernel<1, false, 16, false>));
  } else {
    if (dtype == MLA_F16 && merge_here) MLA_LAUNCH((partition_kernel<0, true, 32, false>));
    else if (dtype == MLA_F16) MLA_LAUNCH((partition_kernel<0, false, 32, false>));
    else if (merge_here) MLA_LAUNCH((partition_kernel<1, true, 32, false>));
    else MLA_LAUNCH((partition_kernel<1, false, 32, false>));
  }
#undef MLA_LAUNCH
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_E_HIP, "partition launch: %s", hipGetErrorString(e));
  count(direct ? 0 : 1, 1);
  count(3, (uint64_t)total_rows);
  return MLA_OK;
}

}  // namespace

extern "C" int mla_decode_partition(
    const void* q_absorbed, const void* q_pe, const void* ckv_cache, const void* kpe_cache,
    int32_t num_blocks, int32_t block_size, const int32_t* block_table,
    int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t batch, int32_t num_heads, int32_t q_len, float scale,
    int32_t dtype,
    const int32_t* partitions, const int32_t* splits, const int32_t* row_indptr,
    int32_t total_rows, int32_t max_rows_per_req, int32_t heads_per_wg, float* partial_out,
    float* partial_lse2, void* out, float* lse2_out, int32_t* debug_ranges,
    hipStream_t stream) {
  return partition_launch(false, false, 1.0f, q_absorbed, q_pe, ckv_cache, kpe_cache, num_blocks,
                          block_size,
                          block_table,
                          max_blocks_per_seq, context_lens, batch, num_heads, q_len, scale, dtype,
                          partitions, splits, row_indptr, total_rows, max_rows_per_req,
                          heads_per_wg, partial_out, partial_lse2, out, lse2_out, nullptr,
                          debug_ranges, stream);
}

extern "C" int mla_decode_fused(
    const void* q_absorbed, const void* q_pe, const void* ckv_cache, const void* kpe_cache,
    int32_t num_blocks, int32_t block_size, const int32_t* block_table,
    int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t batch, int32_t num_heads, int32_t q_len, float scale,
    int32_t dtype,
    const int32_t* partitions, const int32_t* splits, const int32_t* row_indptr,
    int32_t total_rows, int32_t max_rows_per_req, int32_t heads_per_wg, float* partial_out,
    float* partial_lse2, void* out, float* lse2_out, uint64_t* sync, int32_t* debug_ranges,
    hipStream_t stream) {
  return partition_launch(true, false, 1.0f, q_absorbed, q_pe, ckv_cache, kpe_cache, num_blocks,
                          block_size,
                          block_table,
                          max_blocks_per_seq, context_lens, batch, num_heads, q_len, scale, dtype,
                          partitions, splits, row_indptr, total_rows, max_rows_per_req,
                          heads_per_wg, partial_out, partial_lse2, out, lse2_out, sync,
                          debug_ranges, stream);
}

extern "C" int mla_decode_partition_fp8(
    const void* q_absorbed, const void* q_pe, const void* ckv_cache, const void* kpe_cache,
    float kv_scale, int32_t num_blocks, int32_t block_size, const int32_t* block_table,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch, int32_t num_heads,
    int32_t q_len, float scale, int32_t dtype, const int32_t* partitions, const int32_t* splits,
    const int32_t* row_indptr, int32_t total_rows, int32_t max_rows_per_req,
    int32_t heads_per_wg, float* partial_out, float* partial_lse2, void* out, float* lse2_out,
    int32_t* debug_ranges, hipStream_t stream) {
  return partition_launch(false, true, kv_scale, q_absorbed, q_pe, ckv_cache, kpe_cache,
                          num_blocks, block_size, block_table, max_blocks_per_seq, context_lens,
                          batch, num_heads, q_len, scale, dtype, partitions, splits, row_indptr,
                          total_rows, max_rows_per_req, heads_per_wg, partial_out, partial_lse2,
                          out, lse2_out, nullptr, debug_ranges, stream);
}
