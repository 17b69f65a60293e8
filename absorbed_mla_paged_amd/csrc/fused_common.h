// The merge step run inside the partition launch (mla_decode_fused).
//
// The merge itself is the log2-LSE merge of the reduce kernel (vllm-metal
// pull request 601 "[kernel] Wire MLA split-KV decode", "What changed";
// base-2 LSEs and request-major rows per mlxcel pull request 995, "How
// #898's merge kernel is reused"; rows with no visible key weigh 0 and the
// result is rounded once, MTPLX pull request 639). What differs is who runs
// it: the workgroups of the partition launch, once every row of their
// request has been written, instead of a second launch.
//
// Hand-off, per (request, head group) with N rows (= N workgroups):
//  * Each workgroup adds 1 to `started` when it begins, and reads `started`
//    again just before its stores. If it then sees all N begun, every
//    workgroup it could wait for is already running, and it may wait
//    ("willing"); otherwise it must not hold its CU waiting for workgroups
//    that may not have been dispatched yet.
//  * After its partial stores it adds to `arrived`: 1, plus 2^40 if it is
//    not willing. The value returned says how many rows arrived before it
//    (low 40 bits) and how many of those were not willing (high bits).
//  * The merge work of the group (its heads x 16 slices of 32 dims) is cut
//    into N equal pieces. A willing workgroup that is not last takes piece
//    (arrivals before it - unwilling before it), waits until all N have
//    arrived and merges it. The last arrival never waits: it takes the last
//    piece plus one per unwilling workgroup. So every piece is merged
//    exactly once, every wait is on running workgroups that do not wait,
//    and no workgroup waits at all when the launch does not fit at once.
//  * The fields only grow. `started` and `arrived` equal the bases
//    `sbase` / `abase` when a launch begins; the last arrival moves the
//    bases on, after every workgroup of the launch has read them. Counts
//    are compared as differences modulo 2^64, so they may wrap.
//  * Every wait is bounded; running out adds 1 to `errors` and skips the
//    piece (the host can read the word; it stays 0 in correct use).
#pragma once

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace fused {

using dev::f32x4;

enum Field { kSbase = 0, kStarted = 1, kAbase = 2, kArrived = 3, kErrors = 4, kFields = 8 };
constexpr int kGroupsPerRequest = MLA_MAX_HEADS / 16;
static_assert(kGroupsPerRequest * kFields * 8 == MLA_FUSED_SYNC_BYTES_PER_REQUEST, "layout");
constexpr uint64_t kUnwilling = 1ull << 40;
constexpr uint64_t kArrivalMask = kUnwilling - 1;

#ifdef __HIPCC__
constexpr int kSpinLimit = 1 << 17;   // polls, each at least one L2 round trip

__device__ __forceinline__ uint64_t* header(uint64_t* sync, int b, int hg) {
  return sync + ((int64_t)b * kGroupsPerRequest + hg) * kFields;
}
__device__ __forceinline__ uint64_t ld(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// What the leader lane of a workgroup learns when it arrives: the pieces
// [first, first + count) to merge (count 0: none).
struct Decision {
  int first, count;
};

// Leader lane only (one lane of the workgroup), after every partial store
// of the workgroup has completed. sbase / abase: read at the workgroup's
// start; started_seen: `started` read before the stores; N: rows of the
// request.
__device__ __forceinline__ Decision arrive(uint64_t* h, uint64_t sbase, uint64_t abase,
                                           uint64_t started_seen, int N) {
  const bool willing = started_seen - sbase >= (uint64_t)N;
  const uint64_t add = 1 + (willing ? 0 : kUnwilling);
  // Release: the partials of this workgroup are visible before the count
  // moves; acquire: the last arrival reads everyone's partials.
  const uint64_t old = __hip_atomic_fetch_add(h + kArrived, add, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t rel = old - abase;
  const uint64_t before64 = rel & kArrivalMask;
  const uint64_t unwilling64 = rel >> 40;
  if (before64 >= (uint64_t)N || unwilling64 > before64) {
    // Only a record that was not left consistent gets here (a launch that
    // did not complete, or two launches sharing it at once).
    __hip_atomic_fetch_add(h + kErrors, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return Decision{0, 0};
  }
  const int before = (int)before64;
  const int unwilling = (int)unwilling64;
  if (before == N - 1) {
    // Last arrival: every workgroup of the launch has read the bases.
    __hip_atomic_store(h + kSbase, sbase + (uint64_t)N, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(h + kAbase, old + add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return Decision{N - 1 - unwilling, unwilling + 1};
  }
  if (!willing) return Decision{0, 0};
  int spins = 0;
  while (((ld(h + kArrived) - abase) & kArrivalMask) < (uint64_t)N) {
    if (++spins >= kSpinLimit) {
      __hip_atomic_fetch_add(h + kErrors, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return Decision{0, 0};
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return Decision{before - unwilling, 1};
}

// ---- the merge of one piece ----------------------------------------------
//
// A piece is a range of slices of the group; slice j is head head0 + j / 16,
// dims 32 (j % 16) .. + 32. Thread layout (NT threads, NT / 64 = 8 waves):
// tid = (sp * R + rl) * 8 + c4, with c4 the 4-dim quarter-line of a slice
// row (8 threads read one 128-byte line), rl one of R row lanes and sp one
// of SP = NT / (8 R) slice slots. Each thread holds 8 load slots: slot j is
// row rl + R (j % JP + JP k) (k-th batch) of slice slot sp + SP (j / JP), so
// a thread merges JP rows of each of its 8 / JP slices per batch. R grows
// with N until 64 (4 rows per lane), so a piece's loads are in flight
// together. The row lanes are then merged in a fixed order: lane shuffles
// inside a wave, then the waves through LDS. The order depends only on N and
// the piece, so results are bit-identical run to run.
struct MergeArgs {
  const float* partial_out;
  const float* partial_lse2;
  void* out;
  float* lse2_out;
  int heads;
};

template <int DT, int NT, int JP>
__device__ void merge_piece_jp(const MergeArgs& a, int R, int N, int64_t r0, int b, int head0,
                               int s_lo, int s_hi, MLA_LDS char* scratch) {
  typedef dev::Elem<DT> E;
  constexpr int SPT = 8 / JP;       // slices per thread
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c4 = tid & 7;
  const int rl = (tid >> 3) & (R - 1);
  const int SP = NT / 8 / R;
  const int sp = (tid >> 3) / R;
  const int per_pass = SP * SPT;
  const int nbatch = (N + R * JP - 1) / (R * JP);
  MLA_LDS f32x4* x_acc = (MLA_LDS f32x4*)scratch;                 // [NW][SPT][8]
  MLA_LDS float* x_m = (MLA_LDS float*)(scratch + NW * SPT * 8 * 16);
  MLA_LDS float* x_w = x_m + NW * SPT * 8;

  for (int pass0 = s_lo; pass0 < s_hi; pass0 += per_pass) {
    float m[SPT], w[SPT];
    f32x4 acc[SPT];
#pragma unroll
    for (int js = 0; js < SPT; ++js) {
      m[js] = -INFINITY;
      w[js] = 0.f;
      acc[js] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int kb = 0; kb < nbatch; ++kb) {
      f32x4 v[8];
      float lw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int slice = pass0 + (j / JP) * SP + sp;
        const int r = rl + R * (j % JP + JP * kb);
        const bool ok = slice < s_hi && r < N;
        const int64_t hrow = (r0 + (ok ? r : 0)) * a.heads + head0 + (ok ? slice : s_lo) / 16;
        lw[j] = ok ? a.partial_lse2[hrow] : -INFINITY;
        v[j] = ok ? *reinterpret_cast<const f32x4*>(a.partial_out + hrow * MLA_KV_LORA_RANK +
                                                     ((ok ? slice : s_lo) % 16) * 32 + c4 * 4)
                  : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int js = 0; js < SPT; ++js) {
        float bm = m[js];
#pragma unroll
        for (int jr = 0; jr < JP; ++jr) bm = fmaxf(bm, lw[js * JP + jr]);
        if (bm > m[js]) {   // bm is finite here
          const float alpha = __builtin_amdgcn_exp2f(m[js] - bm);   // 0 when m = -inf
          acc[js] *= alpha;
          w[js] *= alpha;
          m[js] = bm;
        }
        if (m[js] != -INFINITY) {
#pragma unroll
          for (int jr = 0; jr < JP; ++jr) {
            const float e = __builtin_amdgcn_exp2f(lw[js * JP + jr] - m[js]);   // 0 for -inf
            acc[js] += e * v[js * JP + jr];
            w[js] += e;
          }
        }
      }
    }
    auto merge = [&](int js, float m2, float w2, f32x4 acc2) {
      const float mn = fmaxf(m[js], m2);
      const float s1 = (m[js] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[js] - mn);
      const float s2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
      acc[js] = s1 * acc[js] + s2 * acc2;
      w[js] = s1 * w[js] + s2 * w2;
      m[js] = mn;
    };
    // Row lanes inside the wave: lane bits 3.. (as many as R has, up to 3).
    for (int x = 8; x < 64 && x < 8 * R; x <<= 1) {
#pragma unroll
      for (int js = 0; js < SPT; ++js) {
        f32x4 acc2;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc2[i] = dev::shfl_xor(acc[js][i], x);
        merge(js, dev::shfl_xor(m[js], x), dev::shfl_xor(w[js], x), acc2);
      }
    }
    bool holder = rl == 0;
    if (R > 8) {
      // R / 8 waves per slice slot: lanes 0..7 of each hold its merge.
      const int wr = R / 8;
      if (lane < 8) {
#pragma unroll
        for (int js = 0; js < SPT; ++js) {
          const int e = (wave * SPT + js) * 8 + c4;
          x_acc[e] = acc[js];
          x_m[e] = m[js];
          x_w[e] = w[js];
        }
      }
      __syncthreads();
      holder = (wave % wr == 0) && lane < 8;
      if (holder) {
        for (int k = 1; k < wr; ++k) {
#pragma unroll
          for (int js = 0; js < SPT; ++js) {
            const int e = ((wave + k) * SPT + js) * 8 + c4;
            merge(js, x_m[e], x_w[e], x_acc[e]);
          }
        }
      }
      __syncthreads();   // the exchange area is reused by the next pass
    }
    if (holder) {
#pragma unroll
      for (int js = 0; js < SPT; ++js) {
        const int slice = pass0 + js * SP + sp;
        if (slice >= s_hi) continue;
        const int h = head0 + slice / 16;
        const int64_t oidx = ((int64_t)b * a.heads + h) * MLA_KV_LORA_RANK + (slice % 16) * 32 + c4 * 4;
        typename E::vec4 o;
        const bool empty = m[js] == -INFINITY;   // nothing visible in any row
        const float inv = empty ? 0.f : 1.0f / w[js];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = static_cast<typename E::scalar>(empty ? 0.f : acc[js][i] * inv);
        *reinterpret_cast<typename E::vec4*>(reinterpret_cast<uint16_t*>(a.out) + oidx) = o;
        if (a.lse2_out && slice % 16 == 0 && c4 == 0)
          a.lse2_out[(int64_t)b * a.heads + h] = empty ? -INFINITY : m[js] + __builtin_amdgcn_logf(w[js]);
      }
    }
  }
}

// Merge piece `piece` of N of the group: its rows are r0 .. r0 + N - 1,
// heads head0 .. head0 + hg_heads - 1. Every thread of the workgroup calls
// it (it holds workgroup barriers); `scratch` needs 3 KB of LDS.
template <int DT, int NT>
__device__ void merge_piece(const MergeArgs& a, int piece, int N, int64_t r0, int b, int head0,
                            int hg_heads, MLA_LDS char* scratch) {
  if (piece < 0 || piece >= N) return;
  const int SL = hg_heads * (MLA_KV_LORA_RANK / 32);
  const int s_lo = (int)((int64_t)piece * SL / N);
  const int s_hi = (int)((int64_t)(piece + 1) * SL / N);
  if (s_lo >= s_hi) return;   // uniform over the workgroup
  int R = 1;
  while (R < NT / 8 && R * 4 < N) R <<= 1;
  const int jr = (N + R - 1) / R;
  if (jr > 4) merge_piece_jp<DT, NT, 8>(a, R, N, r0, b, head0, s_lo, s_hi, scratch);
  else if (jr > 2) merge_piece_jp<DT, NT, 4>(a, R, N, r0, b, head0, s_lo, s_hi, scratch);
  else if (jr > 1) merge_piece_jp<DT, NT, 2>(a, R, N, r0, b, head0, s_lo, s_hi, scratch);
  else merge_piece_jp<DT, NT, 1>(a, R, N, r0, b, head0, s_lo, s_hi, scratch);
}
#endif  // __HIPCC__

}  // namespace fused
}  // namespace mla
