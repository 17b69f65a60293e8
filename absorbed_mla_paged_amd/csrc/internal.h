// Internal declarations shared by the host planning code and the launchers.
#pragma once

#include <cstdint>

#include "../../include/mla_decode.h"

namespace mla {

// Record a formatted message for mla_last_error() and return `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Path counters: 0 single-pass launches, 1 split launches, 2 reduce
// launches, 3 partition rows launched.
void count(int which, uint64_t v);

int default_heads_per_wg(int32_t heads);
bool valid_heads_per_wg(int32_t heads, int32_t hpw);

// Compute units of the current device (defined with the kernels).
int device_compute_units(int64_t* cus);

struct TileRange {
  int64_t blk_lo, blk_hi;  // blocks [blk_lo, blk_hi) of the request
  int64_t tok_lo, tok_hi;  // tokens [tok_lo, tok_hi)
};
// Cache block sizes the kernels are built for: 32 and 16 tokens.
bool valid_block_size(int32_t bs);
// The index math of mla_partition_range (host copy; the kernel has its own),
// for a context of n tokens in blocks of bs tokens.
TileRange tile_range(int64_t n, int32_t bs, int32_t P, int32_t S, int32_t p, int32_t s);

}  // namespace mla
