// Pieces shared by the two partition kernels (16-head and wide workgroups):
// the argument block, the swizzles of the LDS tiles, the row lookup with the
// partition/tile index math, and the launch entry of the wide kernel.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace part {

// Arguments not needed before the row is known (fetched from the kernel
// argument segment while the row metadata is in flight).
struct PartitionArgs {
  const uint16_t* q_absorbed;
  const uint16_t* q_pe;
  const uint16_t* ckv;
  const uint16_t* kpe;
  float* partial_out;
  float* partial_lse2;
  void* out;
  float* lse2_out;
  int32_t* debug_ranges;
  uint64_t* sync;    // merge hand-off state (fused launches only)
  int32_t num_blocks;
  int32_t heads;     // query rows per request: q_len x heads of one new token
  float scale_log2;  // scale * log2(e) (times the cache scale for E4M3 caches)
  float out_scale;   // factor on the normalised output: the E4M3 cache scale, else 1
};

// The `flags` kernel argument (preloaded with the row lookup's arguments):
// bit 0 single pass (write `out` directly), bits 1..3 q_len - 1, bits 8..
// heads of one new token.
constexpr int32_t pack_flags(bool direct, int32_t q_len, int32_t heads_per_query) {
  return (direct ? 1 : 0) | ((q_len - 1) << 1) | (heads_per_query << 8);
}

#ifdef __HIPCC__
// Tokens at the end of the context hidden from the head group starting at
// query row `head0`: new token j = head0 / heads_per_query of a window of
// q_len sees all but the last q_len - 1 - j.
__device__ __forceinline__ int hidden_tail(int32_t flags, int head0) {
  const int qm1 = (flags >> 1) & 7;
  return qm1 ? qm1 - head0 / (flags >> 8) : 0;
}
#endif

// Tokens per segment: one K-step of the value product and one LDS ring slot
// of the wide kernel. A segment is one cache block of 32 tokens or two of
// 16; the kernels are templates on the cache block size PG (16 or 32),
// which enters only the index math and the block-table lookups.
constexpr int SEG = 32;
constexpr int LAT = MLA_KV_LORA_RANK;   // 512
constexpr int ROPE = MLA_ROPE_DIM;      // 64
constexpr int CKV_ROW = LAT * 2;        // bytes per ckv row
constexpr int KPE_ROW = ROPE * 2;       // bytes per kpe row
constexpr int KSTEPS = (LAT + ROPE) / 32;  // 18 score K-steps of 32
constexpr float RESCALE_LOG2 = 8.0f;    // lazy-rescale threshold (base 2)

#ifdef __HIPCC__
// XOR swizzles of the 16-byte chunk index inside an LDS row: ckv rows hold
// 64 chunks (the low 4 bits are permuted, by r % 16 only), kpe rows 8. Any
// 16 consecutive ckv rows (a score read) take all 16 values, and
// swz_ckv >> 1 is one-to-one on each of the row sets {0..7}, {8..15},
// {0..3, 8..11} and {4..7, 12..15}: the transposing value reads (rows
// 4 lg + ln / 4, two chunks of each) then fall in distinct banks whichever
// two 16-lane groups the LDS serves together. (The bank-conflict counter
// shows lane groups 0 and 2 served together: with rows r and r + 8 sharing
// a chunk pair, every transposing read conflicted.)
__device__ __forceinline__ int swz_ckv(int r) {
  return (((r & 7) ^ ((r >> 1) & 4)) << 1) | ((r >> 3) & 1);
}
__device__ __forceinline__ int swz_kpe(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// One workgroup's row: request b, its token range and blocks.
struct RowInfo {
  int b;        // request
  int row;      // partial row (request b when the launch is single pass)
  int hg;       // head group
  int tok_lo, tok_hi;   // tokens this head group sees in the row
  int tok_end;          // end of the row's range itself (for debug_ranges)
  int blk_lo;   // first cache block of the range (request-local)
  int nseg;     // 32-token segments holding at least one visible token
};

// Which row slot and head group workgroup L owns. Workgroups are dealt to
// the 8 XCDs round-robin by linear id. Slot u is the global row index of a
// split launch (request-major, so every XCD gets the same number of rows,
// within one, whatever the requests' row counts), or the request of a
// single-pass launch. The id layout L = ((u / 8) * G + hg) * 8 + u % 8
// keeps the G head groups of one row on one XCD, so they share its L2.
// Returns false for grid padding.
__device__ __forceinline__ bool slot_of(int L, int groups, int slots, int* u, int* hg) {
  const int sl = L >> 3;
  *hg = sl % groups;
  *u = (sl / groups) * 8 + (L & 7);
  return *u < slots;
}

// Request of global row r: the b in [0, batch) with row_indptr[b] <= r <
// row_indptr[b + 1], by binary search over the (non-decreasing) row_indptr
// with scalar loads; ceil(log2(batch)) dependent loads, none for one
// request. A malformed row_indptr still yields some b in range, and the
// caller's check of r against that request's rows then rejects the row.
__device__ __forceinline__ int request_of_row(const int32_t* row_indptr, int batch, int r) {
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (dev::load_const(row_indptr, mid) <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Row metadata in one round of scalar loads, then the index math of
// mla_partition_range for cache blocks of PG tokens (must agree with it bit
// for bit). The row's range is
// cut from the whole context; `hidden` more tokens at its end are masked for
// this head group (new token j of a window of q_len sees all but the last
// q_len - 1 - j).
// Slot u is request b (single pass) or global row u (split launch, request
// found by request_of_row).
template <int PG>
__device__ __forceinline__ bool find_row(int u, int batch, int direct, int total_rows, int hidden,
                                         int max_blocks, const int32_t* context_lens,
                                         const int32_t* row_indptr,
                                         const int32_t* partitions, const int32_t* splits,
                                         RowInfo* ri) {
  using dev::load_const;
  const int b = direct ? u : request_of_row(row_indptr, batch, u);
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
  if (x < 0 || x >= nrows || row < 0 || row >= total_rows) return false;
  const int p = x / S;
  const int s = x % S;
  const int nblk = cdiv(n, PG);
  const int bpp = cdiv(nblk, P);
  const int pb0 = min(p * bpp, nblk);
  const int pb1 = min((p + 1) * bpp, nblk);
  const int m = pb1 - pb0;
  const int bps = m > 0 ? cdiv(m, S) : 0;
  const int blk_lo = (p < P) ? pb0 + min(s * bps, m) : nblk;
  const int blk_hi = (p < P) ? pb0 + min((s + 1) * bps, m) : nblk;
  ri->b = b;
  ri->row = row;
  const int n_vis = max(0, n - hidden);
  ri->tok_lo = min(blk_lo * PG, n);
  ri->tok_end = min(blk_hi * PG, n);
  ri->tok_hi = max(ri->tok_lo, min(ri->tok_end, n_vis));
  ri->blk_lo = blk_lo;
  ri->nseg = cdiv(ri->tok_hi - ri->tok_lo, SEG);
  return true;
}

// Four E4M3 bytes of `w` -> four values of the 16-bit type DT, exactly,
// as two packed words (byte i becomes element i).
template <int DT> __device__ __forceinline__ dev::u32x2 widen4(uint32_t w);
template <> __device__ __forceinline__ dev::u32x2 widen4<0>(uint32_t w) {
  return dev::u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))};
}
template <> __device__ __forceinline__ dev::u32x2 widen4<1>(uint32_t w) {
  return dev::u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}
// Eight E4M3 bytes (w0 then w1) -> one 16-byte chunk of eight 16-bit values.
template <int DT> __device__ __forceinline__ dev::u32x4 widen8(uint32_t w0, uint32_t w1) {
  const dev::u32x2 a = widen4<DT>(w0), b = widen4<DT>(w1);
  return dev::u32x4{a[0], a[1], b[0], b[1]};
}

// Spin until the LDS counter reaches `target`. Every counter a wave waits on
// is bumped by waves of the same (resident) workgroup that do not first
// wait on this one, so the wait ends.
__device__ __forceinline__ void wait_counter(const MLA_LDS uint32_t* c, uint32_t target) {
  while (*(const volatile MLA_LDS uint32_t*)c < target) __builtin_amdgcn_s_sleep(1);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void bump_counter(MLA_LDS uint32_t* c, int lane) {
  dev::wait_lgkmcnt0();  // this wave's LDS reads / writes before the bump are done
  if (lane == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
#endif  // __HIPCC__

// Launch of the wide kernel (heads_per_wg 64); arguments as the 16-head
// kernel's, kv8 for E4M3 caches. Host side, after the launcher's checks.
void launch_wide(int dtype, int block_size, bool kv8, unsigned wgs, hipStream_t stream,
                 int32_t groups, int32_t batch, int32_t slots, int32_t flags,
                 int32_t total_rows, int32_t max_blocks, const int32_t* context_lens,
                 const int32_t* row_indptr, const int32_t* partitions, const int32_t* splits,
                 const int32_t* block_table, const PartitionArgs& a);

}  // namespace part
}  // namespace mla
