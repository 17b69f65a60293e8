// Host driver for the partition chooser and the index math, built with g++
// and the address and undefined-behaviour sanitizers by
// tests/test_host_sanitized.py (no GPU code is involved). It draws inputs
// from a fixed linear congruential sequence, calls the two host entry points
// and prints one line per call: the inputs, the status and the outputs. The
// test compares every line with the Python mirror of the chooser.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "mla_decode.h"

namespace mla {
// The chooser asks the device for its compute units only when num_cus = 0;
// this host-only build answers 256.
int device_compute_units(int64_t* cus) {
  *cus = 256;
  return MLA_OK;
}
}  // namespace mla

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32() {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return static_cast<uint32_t>(g_state >> 33);
}
static int32_t pick(std::initializer_list<int32_t> v) {
  return *(v.begin() + next_u32() % v.size());
}

int main(int argc, char** argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 2000;
  for (int it = 0; it < n; ++it) {
    const int32_t batch = pick({0, 1, 1, 2, 3, 4, 8, 9});
    const int32_t heads = pick({16, 32, 48, 64, 96, 112, 128, 128, 24, 0, 144});
    const int32_t q_len = pick({1, 1, 1, 2, 4, 8, 0, 9});
    const int32_t bs = pick({32, 32, 16, 16, 8});
    std::vector<int32_t> ctx(batch);
    for (auto& c : ctx) {
      switch (next_u32() % 6) {
        case 0: c = pick({0, 1, 15, 16, 17, 31, 32, 33}); break;
        case 1: c = static_cast<int32_t>(next_u32() % 4096); break;
        case 2: c = 32768 + static_cast<int32_t>(next_u32() % 3) - 1; break;
        case 3: c = static_cast<int32_t>(next_u32() % (1 << 20)); break;
        case 4: c = static_cast<int32_t>(next_u32() % 131073); break;
        default: c = (next_u32() % 40 == 0) ? -1 : static_cast<int32_t>(next_u32() % 200000);
      }
    }
    mla_plan_params p;
    mla_default_plan_params(&p);
    p.num_cus = pick({0, 8, 64, 256, 256, 1024});
    p.heads_per_wg = pick({0, 0, 16, 64, 32});
    p.min_tile_blocks = pick({1, 4, 4, 16});
    p.wgs_per_cu = pick({1, 1, 2, 3});
    p.force_partitions = pick({0, 0, 0, 1, 3, 8, 9});
    p.force_splits = pick({0, 0, 0, 1, 2, 7});
    p.workspace_limit_bytes = pick({0, 0, 1 << 16, 1 << 20, 64 << 20});
    std::vector<int32_t> P(batch + 1, -7), S(batch + 1, -7), ind(batch + 2, -7);
    mla_plan_info info{};
    const int st = mla_choose_partitions(batch, heads, q_len, ctx.data(), bs, &p, P.data(),
                                         S.data(), ind.data(), &info);
    std::printf("plan %d %d %d %d |", batch, heads, q_len, bs);
    for (auto c : ctx) std::printf(" %d", c);
    std::printf(" | %d %d %d %d %d %d %" PRId64 " | %d |", p.num_cus, p.heads_per_wg,
                p.min_tile_blocks, p.wgs_per_cu, p.force_partitions, p.force_splits,
                p.workspace_limit_bytes, st);
    if (st == MLA_OK) {
      for (int b = 0; b < batch; ++b) std::printf(" %d/%d", P[b], S[b]);
      std::printf(" |");
      for (int b = 0; b <= batch; ++b) std::printf(" %d", ind[b]);
      std::printf(" | %d %d %d %d %d %d %" PRId64 " %" PRId64, info.total_rows,
                  info.max_rows_per_req, info.heads_per_wg, info.groups, info.tile_blocks,
                  info.needs_reduce, info.partial_out_bytes, info.partial_lse_bytes);
    }
    std::printf("\n");
    // The index math over a random tile of a random context.
    const int32_t c = static_cast<int32_t>(next_u32() % 300000) - 10;
    const int32_t PP = static_cast<int32_t>(next_u32() % 10), SS = static_cast<int32_t>(next_u32() % 20);
    const int32_t pp = static_cast<int32_t>(next_u32() % 10), ss = static_cast<int32_t>(next_u32() % 20);
    int32_t lo = -7, hi = -7;
    const int rs = mla_partition_range(c, bs, PP, SS, pp, ss, &lo, &hi);
    std::printf("range %d %d %d %d %d %d | %d | %d %d\n", c, bs, PP, SS, pp, ss, rs, lo, hi);
  }
  return 0;
}
