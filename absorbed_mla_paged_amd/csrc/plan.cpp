// Host side of the split-KV absorbed-MLA decode library: the partition
// chooser, the partition/tile index math, status strings, the per-thread
// error message and the path counters. Plain C++17; nothing here touches the
// device except the one compute-unit query when the caller leaves num_cus 0.
//
// The chooser implements the gates of vllm-metal pull request 601 "[kernel]
// Wire MLA split-KV decode", "What changed" (pure decode, long enough
// context, small decode launch, 2 to 8 partitions, bounded temporary memory)
// and the 32K+ start of the split path stated above that page's wrapper
// grid; the rule and its constants are spelled out in include/mla_decode.h.
#include "internal.h"

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

namespace mla {

namespace {
thread_local std::string g_last_error;
std::atomic<uint64_t> g_counters[4];

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

void clear_error() { g_last_error.clear(); }

void count(int which, uint64_t v) { g_counters[which].fetch_add(v, std::memory_order_relaxed); }

int default_heads_per_wg(int32_t heads) {
  // 64 heads (two 32-head waves per token) wherever they divide H: the
  // cache rows staged in LDS then feed 64 heads instead of 16, and the
  // partial written per workgroup stays at a quarter of the 128-head one.
  // Other head counts use one 16-row MFMA tile of heads per workgroup.
  return heads % 64 == 0 ? 64 : 16;
}

bool valid_heads_per_wg(int32_t heads, int32_t hpw) {
  return (hpw == 16 || hpw == 64) && heads % hpw == 0;
}

bool valid_block_size(int32_t bs) { return bs == MLA_BLOCK_SIZE || bs == MLA_BLOCK_SIZE_SMALL; }

TileRange tile_range(int64_t n, int32_t bs, int32_t P, int32_t S, int32_t p, int32_t s) {
  const int64_t nblk = cdiv(n, bs);
  const int64_t bpp = cdiv(nblk, P);
  const int64_t pb0 = std::min<int64_t>(p * bpp, nblk);
  const int64_t pb1 = std::min<int64_t>((p + 1) * bpp, nblk);
  const int64_t m = pb1 - pb0;
  const int64_t bps = m > 0 ? cdiv(m, S) : 0;
  const int64_t lo = pb0 + std::min<int64_t>(s * bps, m);
  const int64_t hi = pb0 + std::min<int64_t>((s + 1) * bps, m);
  TileRange r;
  r.blk_lo = lo;
  r.blk_hi = hi;
  r.tok_lo = std::min<int64_t>(lo * bs, n);
  r.tok_hi = std::min<int64_t>(hi * bs, n);
  return r;
}

}  // namespace mla

using namespace mla;

extern "C" {

void mla_default_plan_params(mla_plan_params* p) {
  if (!p) return;
  p->min_split_ctx = 32768;
  p->tokens_per_partition = 16384;
  p->min_partitions = 2;
  p->max_partitions = MLA_MAX_PARTITIONS;
  p->num_cus = 0;
  p->heads_per_wg = 0;
  p->min_tile_blocks = 4;
  p->wgs_per_cu = 1;
  p->force_partitions = 0;
  p->force_splits = 0;
  p->workspace_limit_bytes = 0;
}

int mla_partition_range(int32_t ctx, int32_t block_size, int32_t P, int32_t S, int32_t p,
                        int32_t s, int32_t* tok_begin, int32_t* tok_end) {
  clear_error();
  if (!tok_begin || !tok_end) return fail(MLA_E_NULL, "mla_partition_range: null output");
  if (!valid_block_size(block_size))
    return fail(MLA_E_UNSUPPORTED, "block_size %d (16 or 32 are supported)", block_size);
  if (ctx < 0 || P < 1 || S < 1 || p < 0 || p >= P || s < 0 || s >= S)
    return fail(MLA_E_RANGE, "mla_partition_range: ctx=%d P=%d S=%d p=%d s=%d", ctx, P, S, p, s);
  const TileRange r = tile_range(ctx, block_size, P, S, p, s);
  *tok_begin = static_cast<int32_t>(r.tok_lo);
  *tok_end = static_cast<int32_t>(r.tok_hi);
  return MLA_OK;
}

int mla_choose_partitions(int32_t batch, int32_t num_heads, int32_t q_len,
                          const int32_t* ctx, int32_t block_size,
                          const mla_plan_params* params, int32_t* P_out, int32_t* S_out,
                          int32_t* indptr_out, mla_plan_info* info) {
  clear_error();
  mla_plan_params prm;
  if (params) prm = *params; else mla_default_plan_params(&prm);

  if (batch < 0) return fail(MLA_E_SHAPE, "batch %d < 0", batch);
  if (q_len < 1) return fail(MLA_E_SHAPE, "q_len %d < 1", q_len);
  if (q_len > MLA_MAX_QLEN)
    return fail(MLA_E_UNSUPPORTED, "q_len %d (at most %d)", q_len, MLA_MAX_QLEN);
  if (!valid_block_size(block_size))
    return fail(MLA_E_UNSUPPORTED, "block_size %d (16 or 32 are supported)", block_size);
  if (num_heads < MLA_MIN_HEADS || num_heads > MLA_MAX_HEADS || num_heads % 16)
    return fail(MLA_E_UNSUPPORTED, "num_heads %d (need a multiple of 16 in [16, 128])", num_heads);
  if (batch > 0 && (!ctx || !P_out || !S_out)) return fail(MLA_E_NULL, "null per-request array");
  if (!indptr_out) return fail(MLA_E_NULL, "null row_indptr");
  if (prm.min_partitions < 1 || prm.min_partitions > prm.max_partitions ||
      prm.max_partitions > MLA_MAX_PARTITIONS)
    return fail(MLA_E_RANGE, "partition bounds [%d, %d]", prm.min_partitions, prm.max_partitions);
  if (prm.tokens_per_partition < 1 || prm.min_tile_blocks < 1 || prm.wgs_per_cu < 1 ||
      prm.min_split_ctx < 0 || prm.num_cus < 0)
    return fail(MLA_E_RANGE, "chooser parameter out of range");
  if (prm.force_partitions < 0 || prm.force_partitions > MLA_MAX_PARTITIONS ||
      prm.force_splits < 0 || prm.force_splits > MLA_MAX_SPLITS)
    return fail(MLA_E_RANGE, "forced P=%d S=%d out of range", prm.force_partitions,
                prm.force_splits);
  if (prm.workspace_limit_bytes < 0) return fail(MLA_E_RANGE, "negative workspace limit");
  const int32_t hpw = prm.heads_per_wg ? prm.heads_per_wg : default_heads_per_wg(num_heads);
  if (!valid_heads_per_wg(num_heads, hpw))
    return fail(MLA_E_UNSUPPORTED, "heads_per_wg %d for %d heads", hpw, num_heads);
  int64_t num_cus = prm.num_cus;
  if (num_cus == 0) {
    int st = device_compute_units(&num_cus);
    if (st != MLA_OK) return st;
  }
  for (int32_t b = 0; b < batch; ++b)
    if (ctx[b] < 0) return fail(MLA_E_RANGE, "context_lens[%d] = %d < 0", b, ctx[b]);

  // Workgroups per row: every query row of the request (q_len x heads) is
  // covered by head groups of hpw rows.
  const int64_t qrows = int64_t(q_len) * num_heads;
  const int64_t G = qrows / hpw;
  std::vector<int64_t> nblk(batch), P(batch), S(batch);
  int64_t total_blocks = 0;
  for (int32_t b = 0; b < batch; ++b) {
    nblk[b] = cdiv(ctx[b], block_size);
    total_blocks += nblk[b];
  }
  const bool autoP = prm.force_partitions == 0;
  const bool autoS = prm.force_splits == 0;
  int64_t tile = prm.min_tile_blocks;
  auto splits_for = [&](int64_t nb, int64_t p) {
    return std::max<int64_t>(1, cdiv(cdiv(nb, p), tile));
  };
  {
    // The policy split is for pure decode only; several new tokens per
    // request keep P_b = 1 but are still tiled for the device.
    const bool eligible = q_len == 1 && int64_t(batch) * G < num_cus;
    for (int32_t b = 0; b < batch; ++b) {
      if (!autoP) P[b] = prm.force_partitions;
      else if (eligible && ctx[b] >= prm.min_split_ctx)
        P[b] = std::min<int64_t>(std::max<int64_t>(cdiv(ctx[b], prm.tokens_per_partition),
                                                   prm.min_partitions),
                                 prm.max_partitions);
      else P[b] = 1;
    }
    const int64_t cap = num_cus * int64_t(prm.wgs_per_cu);
    tile = std::max<int64_t>(prm.min_tile_blocks, cdiv(G * total_blocks, cap));
    // Rounding each request's tiles up can still overshoot one wave of
    // workgroups; then take the smallest larger tile whose grid fits (rows
    // only shrink as the tile grows), or the one giving S_b = 1 everywhere.
    auto grid_rows = [&](int64_t t) {
      int64_t r = 0;
      for (int32_t b = 0; b < batch; ++b)
        r += P[b] * std::max<int64_t>(1, cdiv(cdiv(nblk[b], P[b]), t));
      return r;
    };
    if (autoS && G * grid_rows(tile) > cap) {
      int64_t hi = tile;
      for (int32_t b = 0; b < batch; ++b) hi = std::max(hi, cdiv(nblk[b], P[b]));
      if (G * grid_rows(hi) > cap) {
        tile = hi;
      } else {
        int64_t lo = tile;  // grid_rows(lo) too many, grid_rows(hi) fits
        while (hi - lo > 1) {
          const int64_t mid = lo + (hi - lo) / 2;
          if (G * grid_rows(mid) > cap) lo = mid; else hi = mid;
        }
        tile = hi;
      }
    }
    for (int32_t b = 0; b < batch; ++b) S[b] = autoS ? splits_for(nblk[b], P[b]) : prm.force_splits;
  }

  auto workspace = [&]() -> int64_t {
    int64_t rows = 0;
    bool multi = false;
    for (int32_t b = 0; b < batch; ++b) {
      rows += P[b] * S[b];
      multi = multi || P[b] * S[b] > 1;
    }
    return multi ? rows * qrows * (MLA_KV_LORA_RANK + 1) * 4 : 0;
  };
  const int64_t limit = prm.workspace_limit_bytes;
  if (limit > 0 && workspace() > limit) {
    if (autoS) {
      auto maxS = [&]() { return batch ? *std::max_element(S.begin(), S.end()) : 0; };
      while (workspace() > limit && maxS() > 1) {
        tile = std::min<int64_t>(tile * 2, int64_t(1) << 30);
        for (int32_t b = 0; b < batch; ++b) S[b] = splits_for(nblk[b], P[b]);
      }
    }
    if (autoP) {
      while (workspace() > limit) {
        int32_t best = -1;
        for (int32_t b = 0; b < batch; ++b)
          if (P[b] > 2 && (best < 0 || P[b] > P[best])) best = b;
        if (best < 0) break;
        P[best] -= 1;
      }
      while (workspace() > limit) {
        int32_t best = -1;
        for (int32_t b = 0; b < batch; ++b)
          if (P[b] > 1 && (best < 0 || ctx[b] < ctx[best])) best = b;
        if (best < 0) break;
        P[best] = 1;
      }
    }
    if (workspace() > limit)
      return fail(MLA_E_WORKSPACE, "workspace %lld B exceeds the limit %lld B with forced values",
                  (long long)workspace(), (long long)limit);
  }

  int64_t rows = 0, max_rows = 0;
  indptr_out[0] = 0;
  for (int32_t b = 0; b < batch; ++b) {
    rows += P[b] * S[b];
    max_rows = std::max(max_rows, P[b] * S[b]);
    if (rows > INT32_MAX / 2) return fail(MLA_E_RANGE, "too many rows (%lld)", (long long)rows);
    P_out[b] = static_cast<int32_t>(P[b]);
    S_out[b] = static_cast<int32_t>(S[b]);
    indptr_out[b + 1] = static_cast<int32_t>(rows);
  }
  if (info) {
    const int64_t ws = workspace();
    info->total_rows = static_cast<int32_t>(rows);
    info->max_rows_per_req = static_cast<int32_t>(max_rows);
    info->heads_per_wg = hpw;
    info->groups = static_cast<int32_t>(G);
    info->tile_blocks = static_cast<int32_t>(tile);
    info->needs_reduce = ws > 0;
    info->partial_out_bytes = ws > 0 ? rows * qrows * MLA_KV_LORA_RANK * 4 : 0;
    info->partial_lse_bytes = ws > 0 ? rows * qrows * 4 : 0;
  }
  return MLA_OK;
}

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_E_NULL: return "null pointer";
    case MLA_E_SHAPE: return "inconsistent shape";
    case MLA_E_RANGE: return "value out of range";
    case MLA_E_ALIGN: return "misaligned pointer";
    case MLA_E_WORKSPACE: return "workspace limit cannot be met";
    case MLA_E_UNSUPPORTED: return "unsupported geometry";
    case MLA_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

void mla_get_counters(uint64_t out[4]) {
  if (!out) return;
  for (int i = 0; i < 4; ++i) out[i] = g_counters[i].load(std::memory_order_relaxed);
}

void mla_reset_counters(void) {
  for (int i = 0; i < 4; ++i) g_counters[i].store(0, std::memory_order_relaxed);
}

}  // extern "C"
