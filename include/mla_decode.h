/*
 * mla_decode.h -- C ABI of the split-KV, matrix-absorbed MLA decode library
 * for MI355X (gfx950).
 *
 * One decode step of Multi-head Latent Attention over a paged latent KV
 * cache. Every head of a request shares one 512-wide latent row (ckv) and
 * one 64-wide rope row (kpe) per cached token. For request b, head h:
 *
 *   s_t      = scale * (q_absorbed[b,h] . ckv_t + q_pe[b,h] . kpe_t)
 *   out[b,h] = sum_t softmax(s)_t * ckv_t                       (512 wide)
 *   lse2     = log2 sum_t exp(s_t)
 *
 * (mlxcel pull request 995, "What changed", Stage 1: the rope half of the
 * score is additive next to the latent half, one scale over both, and the
 * values are the latent rows.) The context is cut into block-aligned rows
 * (KV partitions, each tiled for the device); each row yields a normalised
 * partial output and its base-2 LSE, and a reduce merges the rows of a
 * request into the single-pass answer (vllm-metal pull request 601 "[kernel]
 * Wire MLA split-KV decode", "What changed"; the log2 merge contract of
 * mlxcel pull request 995, "How #898's merge kernel is reused").
 *
 * Conventions for every entry point:
 *  - Return value: MLA_OK (0) or a negative status; mla_last_error() gives a
 *    message for the calling thread. No exception crosses the ABI.
 *  - All argument checks run on the host before anything is launched, so a
 *    failed call launches nothing and changes no device memory.
 *  - "dev" pointers are device memory (hipMalloc / torch CUDA tensors);
 *    "host" pointers are host memory. The caller owns every buffer; the
 *    library allocates nothing and keeps no pointer after a call returns.
 *  - Launches are asynchronous on the caller's stream. The caller keeps the
 *    buffers alive until that stream's work completes.
 *  - Tensors are dense row-major. 16-bit tensors hold IEEE fp16 or bfloat16
 *    bit patterns (mla_dtype) and must be 16-byte aligned.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Geometry fixed by the cache layout (vllm-metal pull request 601,
 * "Wrapper benchmark": kv_lora_rank 512, qk_rope_head_dim 64, block 32).
 * Blocks of 16 tokens are also accepted (the "block16" layout that pull
 * request's reviewer asks to see covered): block_size is 16 or 32 wherever
 * an entry point takes it. */
#define MLA_KV_LORA_RANK 512
#define MLA_ROPE_DIM 64
#define MLA_BLOCK_SIZE 32
#define MLA_BLOCK_SIZE_SMALL 16
#define MLA_MAX_PARTITIONS 8     /* "2 to 8 partitions" (same page, "What changed") */
#define MLA_MAX_SPLITS 4096
#define MLA_MIN_HEADS 16
#define MLA_MAX_HEADS 128
#define MLA_MAX_QLEN 8           /* new tokens per request in one decode call */
/* Bytes of mla_decode_fused's hand-off state per request (8 head groups of
 * 8 counters). */
#define MLA_FUSED_SYNC_BYTES_PER_REQUEST 512

typedef enum { MLA_F16 = 0, MLA_BF16 = 1 } mla_dtype;

enum {
  MLA_OK = 0,
  MLA_E_NULL = -1,        /* a required pointer is NULL */
  MLA_E_SHAPE = -2,       /* sizes inconsistent or out of range */
  MLA_E_RANGE = -3,       /* a value (context length, count) out of range */
  MLA_E_ALIGN = -4,       /* a pointer is not aligned as documented */
  MLA_E_WORKSPACE = -5,   /* the workspace limit cannot be met */
  MLA_E_UNSUPPORTED = -6, /* a geometry this library declines (e.g. H % 16) */
  MLA_E_HIP = -7          /* a HIP runtime call failed; see mla_last_error() */
};

/*
 * Partition-chooser parameters. The pages state the gates of the split
 * decision -- pure decode only, long enough context, small decode launch,
 * 2 to 8 partitions, bounded temporary memory -- and that the split path
 * starts at 32K+ context (vllm-metal pull request 601, "What changed" and the
 * note above the wrapper grid); the constants are ours. A reviewer asked for
 * the thresholds to sit behind a device-aware helper (same page, review),
 * hence num_cus.
 */
typedef struct {
  int32_t min_split_ctx;         /* split only at n_b >= this (default 32768) */
  int32_t tokens_per_partition;  /* P_b = ceil(n_b / this), clamped (16384) */
  int32_t min_partitions;        /* lower clamp of the policy count (2) */
  int32_t max_partitions;        /* upper clamp, <= MLA_MAX_PARTITIONS (8) */
  int32_t num_cus;               /* compute units; 0 = ask the current device */
  int32_t heads_per_wg;          /* heads per workgroup: 16 or 64, dividing H;
                                    0 = library default (64 if 64 divides H,
                                    else 16) */
  int32_t min_tile_blocks;       /* smallest device tile in cache blocks (4) */
  int32_t wgs_per_cu;            /* device tiling target: workgroups per CU (1) */
  int32_t force_partitions;      /* >0: every request gets P_b = this */
  int32_t force_splits;          /* >0: every request gets S_b = this */
  int64_t workspace_limit_bytes; /* >0: bound on the partial workspace */
} mla_plan_params;

/* What the chooser decided, beside the per-request arrays. */
typedef struct {
  int32_t total_rows;        /* sum_b P_b * S_b: rows of the partial workspace */
  int32_t max_rows_per_req;  /* max_b P_b * S_b: grid extent of the partition launch */
  int32_t heads_per_wg;      /* heads one partition workgroup covers */
  int32_t groups;            /* q_len * H / heads_per_wg workgroups per row */
  int32_t tile_blocks;       /* device tile size used for S_b, in blocks */
  int32_t needs_reduce;      /* 1 iff some request has more than one row */
  int64_t partial_out_bytes; /* total_rows * q_len * H * 512 * 4, or 0 when no reduce */
  int64_t partial_lse_bytes; /* total_rows * q_len * H * 4, or 0 when no reduce */
} mla_plan_info;

/* Fill *p with the defaults listed above. */
void mla_default_plan_params(mla_plan_params* p);

/*
 * mla_choose_partitions -- host partition chooser (no device work, never
 * synchronises; with num_cus = 0 it queries the current device once).
 *
 * For each request b: the policy partition count P_b in [1, 8] and the
 * device tiling S_b >= 1; rows of request b are row_indptr[b] ..
 * row_indptr[b+1]-1, request-major (the request-major o_indptr of the merge
 * contract, mlxcel pull request 995, "How #898's merge kernel is reused").
 * Rule (G = q_len * H / heads_per_wg, the head groups over all query rows):
 *   eligible = q_len == 1 && B * G < num_cus
 *   P_b = force_partitions, else clamp(ceil(n_b / tokens_per_partition),
 *         min_partitions, max_partitions) if eligible && n_b >= min_split_ctx,
 *         else 1
 *   cap  = num_cus * wgs_per_cu
 *   tile = max(min_tile_blocks, ceil(G * sum nblk_b / cap))
 *   S_b = force_splits, else max(1, ceil(ceil(nblk_b / P_b) / tile))
 *   (auto S only) if G * sum P_b S_b > cap, tile becomes the smallest larger
 *   value with G * sum P_b S_b <= cap, or max_b ceil(nblk_b / P_b) if none
 *   fits, so the grid never spills into a second, nearly empty wave.
 * With q_len > 1 (several new tokens per request) the policy split stays
 * P_b = 1, since it is for pure decode only (vllm-metal pull request 601,
 * "What changed"), and S_b tiles as above. If a workspace limit is
 * set and exceeded: double the tile until it fits or all S_b = 1 (auto S
 * only); then lower the largest P_b by one (lowest b first) down to 2; then
 * set P_b = 1 in ascending n_b order (auto P only). When every request has
 * one row the decode writes `out` directly and needs no workspace.
 *
 * batch >= 0; num_heads in [16, 128], a multiple of 16; 1 <= q_len <=
 * MLA_MAX_QLEN;
 * context_lens_host[b] >= 0; block_size 16 or 32 (nblk_b = ceil(n_b /
 * block_size); tiles count blocks of that size). params may be NULL
 * (defaults). partitions_host, splits_host [batch] and row_indptr_host
 * [batch+1] are written; info may be NULL.
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_RANGE, MLA_E_UNSUPPORTED,
 * MLA_E_WORKSPACE (limit unreachable with forced values), MLA_E_HIP (device
 * query failed).
 */
int mla_choose_partitions(int32_t batch, int32_t num_heads, int32_t q_len,
                          const int32_t* context_lens_host, int32_t block_size,
                          const mla_plan_params* params, int32_t* partitions_host,
                          int32_t* splits_host, int32_t* row_indptr_host,
                          mla_plan_info* info);

/*
 * mla_partition_range -- the index math, exported for tests (host only).
 * Tokens [*tok_begin, *tok_end) of tile s of partition p of a context of
 * `ctx` tokens in blocks of block_size (16 or 32) tokens, split into P
 * partitions of S tiles each (BS = block_size):
 *   nblk = ceil(ctx/BS); bpp = ceil(nblk/P);
 *   partition p = blocks [min(p*bpp, nblk), min((p+1)*bpp, nblk));
 *   with m blocks in it and bps = ceil(m/S), tile s = blocks
 *   [lo, hi) = [b0 + min(s*bps, m), b0 + min((s+1)*bps, m));
 *   tokens [min(lo*BS, ctx), min(hi*BS, ctx)).
 * The partition kernel computes exactly the same ranges on the device.
 * Errors: MLA_E_NULL, MLA_E_RANGE (ctx < 0, P/S/p/s out of range),
 * MLA_E_UNSUPPORTED (block_size not 16 or 32).
 */
int mla_partition_range(int32_t ctx, int32_t block_size, int32_t P, int32_t S,
                        int32_t p, int32_t s, int32_t* tok_begin, int32_t* tok_end);

/*
 * mla_decode_partition -- the partition kernel (one launch).
 *
 * For every row of the plan and every head: the online-softmax pass over
 * the row's token range of the paged latent cache, writing the normalised
 * partial output (fp32, 512 wide) and its base-2 LSE. A row with no token
 * writes zeros and lse2 = -inf (MTPLX pull request 639, commit giving rows
 * without a visible key weight 0). Partials stay fp32 and are rounded once,
 * in the reduce (same page, commit keeping per-segment outputs in float32).
 *
 * Single pass: when total_rows == batch every request is one row; the
 * kernel then writes round(O/l) straight into `out` (and lse2 into
 * lse2_out if given), the plan arrays are not read and the partial buffers
 * may be NULL (vllm-metal pull request 601, "What changed": partition 0
 * writes directly into the final output).
 *
 * Several new tokens per request (q_len > 1, e.g. a speculative window):
 * the cache already holds all of them, so new token j sits at position
 * n_b - q_len + j and attends to positions 0 .. n_b - q_len + j (causal
 * inside the window). Query rows are token-major: row j * num_heads + h is
 * head h of new token j, in q_absorbed, q_pe, out, lse2_out and the
 * partials alike. A new token that sees no position gets zeros and -inf.
 * (The pages decode one token; this generalisation is ours.)
 *
 * num_heads   heads per new token: a multiple of 16 in [16, 128]
 * q_len       new tokens per request, 1 .. MLA_MAX_QLEN (the chooser's q_len)
 * q_absorbed  dev [batch, q_len, num_heads, 512]  16-bit, 16-byte aligned
 * q_pe        dev [batch, q_len, num_heads, 64]   16-bit, 16-byte aligned
 * ckv_cache   dev [num_blocks, block_size, 512]  16-bit, 16-byte aligned
 * kpe_cache   dev [num_blocks, block_size, 64]   16-bit, 16-byte aligned
 * block_size  tokens per cache block: 32, or 16; it must be the block size
 *             the plan was chosen for
 * block_table dev int32 [batch, max_blocks_per_seq]; entries below
 *             ceil(n_b/block_size) must lie in [0, num_blocks) (others are
 *             never read). An entry outside that range is clamped into it,
 *             never dereferenced out of bounds; the result is then
 *             unspecified.
 * context_lens dev int32 [batch], 0 <= n_b <= block_size * max_blocks_per_seq
 *             (clamped into that range on the device). Rows of the last
 *             block at t >= n_b may hold anything, NaN included.
 * scale       softmax scale applied to both score halves (finite, > 0; MLA_E_RANGE
 *             otherwise)
 * partitions, splits dev int32 [batch]; row_indptr dev int32 [batch+1]:
 *             the chooser's arrays, copied to the device by the caller.
 * total_rows, max_rows_per_req: from mla_plan_info.
 * heads_per_wg: from mla_plan_info (0 = library default for num_heads).
 * partial_out dev fp32 [total_rows, q_len * num_heads, 512] (16-byte aligned),
 * partial_lse2 dev fp32 [total_rows, q_len * num_heads]
 * out         dev 16-bit [batch, q_len * num_heads, 512] (single pass only)
 * lse2_out    dev fp32 [batch, q_len * num_heads] or NULL (single pass only)
 * debug_ranges dev int32 [total_rows, 2] or NULL: each row's token range
 *             [begin, end) as the kernel computed it (for bit-exact tests).
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_RANGE, MLA_E_ALIGN,
 * MLA_E_UNSUPPORTED, MLA_E_HIP.
 */
int mla_decode_partition(const void* q_absorbed, const void* q_pe, const void* ckv_cache,
                         const void* kpe_cache, int32_t num_blocks, int32_t block_size,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t batch, int32_t num_heads,
                         int32_t q_len, float scale, int32_t dtype, const int32_t* partitions,
                         const int32_t* splits, const int32_t* row_indptr,
                         int32_t total_rows, int32_t max_rows_per_req, int32_t heads_per_wg,
                         float* partial_out, float* partial_lse2, void* out, float* lse2_out,
                         int32_t* debug_ranges, hipStream_t stream);

/*
 * mla_decode_partition_fp8 -- the partition kernel over a latent cache
 * stored as one byte per value.
 *
 * The same computation as mla_decode_partition, with every cached value
 * (ckv and kpe alike) equal to its byte, read as E4M3 (the OCP 8-bit
 * floating point format: exponent bias 7, 3 mantissa bits, largest value
 * 448, S.1111.111 is NaN, no infinities), times kv_scale. Queries, outputs
 * and partials are as in mla_decode_partition. The pages keep 16-bit caches
 * only (mlxcel pull request 995 declines other cache modes); this layout,
 * with one scale for the whole latent cache, is ours.
 *
 * Arguments as mla_decode_partition, except:
 * ckv_cache   dev uint8 [num_blocks, block_size, 512], 16-byte aligned
 * kpe_cache   dev uint8 [num_blocks, block_size, 64], 16-byte aligned
 * kv_scale    the cache scale (finite, > 0; MLA_E_RANGE otherwise)
 * dtype       the 16-bit type of q_absorbed, q_pe and out
 * heads_per_wg 16 or 64 (or 0: the default for num_heads), as for
 *             mla_decode_partition; both workgroup shapes take E4M3 caches.
 * Errors: as mla_decode_partition.
 */
int mla_decode_partition_fp8(const void* q_absorbed, const void* q_pe, const void* ckv_cache,
                             const void* kpe_cache, float kv_scale, int32_t num_blocks,
                             int32_t block_size, const int32_t* block_table,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t batch, int32_t num_heads, int32_t q_len, float scale,
                             int32_t dtype, const int32_t* partitions, const int32_t* splits,
                             const int32_t* row_indptr, int32_t total_rows,
                             int32_t max_rows_per_req, int32_t heads_per_wg, float* partial_out,
                             float* partial_lse2, void* out, float* lse2_out,
                             int32_t* debug_ranges, hipStream_t stream);

/*
 * mla_decode_reduce -- the LSE-weighted reduce kernel (one launch).
 *
 * For each request b and query row h over rows r in [row_indptr[b],
 * row_indptr[b+1]): M = max lse2_r; if M = -inf the output is 0 and lse2 is
 * -inf; else w_r = 2^(lse2_r - M), out = sum w_r O_r / sum w_r rounded once
 * to nearest-even in `dtype`, lse2_out = M + log2 sum w_r. The summation
 * order is fixed, so results are bit-identical run to run (vllm-metal pull
 * request 601, "What changed"; mlxcel pull request 995, "How #898's merge
 * kernel is reused", for base 2 and request-major rows).
 *
 * num_heads   query rows per request (q_len * heads for several new
 *             tokens): a multiple of 16 in [16, MLA_MAX_HEADS * MLA_MAX_QLEN]
 * partial_out dev fp32 [total_rows, num_heads, 512], 16-byte aligned
 * partial_lse2 dev fp32 [total_rows, num_heads]
 * row_indptr  dev int32 [batch+1], non-decreasing, row_indptr[0] = 0,
 *             row_indptr[batch] = total_rows
 * out         dev 16-bit [batch, num_heads, 512], 16-byte aligned
 * lse2_out    dev fp32 [batch, num_heads] or NULL
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_ALIGN, MLA_E_UNSUPPORTED, MLA_E_HIP.
 */
int mla_decode_reduce(const float* partial_out, const float* partial_lse2,
                      const int32_t* row_indptr, int32_t batch, int32_t num_heads,
                      int32_t total_rows, int32_t dtype, void* out, float* lse2_out,
                      hipStream_t stream);

/*
 * mla_decode_fused -- partition and merge in one launch.
 *
 * The same result as mla_decode_partition followed by mla_decode_reduce,
 * without the second launch and the gap between the two (the aim of the
 * pages' direct write of partition 0 into the output: vllm-metal pull
 * request 601, "What changed"). The workgroups of the launch write their
 * fp32 partials as before; once every row of a request has arrived, the
 * merge of that request (the reduce's log2-LSE merge, rounded once) is
 * shared out among them and written to `out` and `lse2_out`. A workgroup
 * only waits for the others when all of them have begun, so the launch
 * finishes whether or not it fits the device at once (it is slower when it
 * does not). A single-pass plan (total_rows == batch) is the same launch as
 * mla_decode_partition.
 *
 * Arguments as mla_decode_partition, plus:
 * out         dev 16-bit [batch, num_heads, 512], 16-byte aligned (always)
 * lse2_out    dev fp32 [batch, num_heads] or NULL
 * sync        dev, MLA_FUSED_SYNC_BYTES_PER_REQUEST * batch bytes, 64-byte
 *             aligned, zero-filled before its first use. Every completed
 *             call leaves it ready for the next one; calls that use the
 *             same sync buffer must not run concurrently, and after a
 *             launch that did not complete it must be zero-filled again.
 *             Word 4 of each 64-byte record counts waits that ran out
 *             (0 in correct use). A wait that runs out skips its share of
 *             the merge, and the call still returns MLA_OK: `out` and
 *             `lse2_out` are then unspecified for that request. Callers that
 *             cannot rule this out (e.g. a sync buffer shared by concurrent
 *             launches) read word 4 back after the launch completes (the
 *             Python binding's fused_sync_errors does).
 * Currently heads_per_wg must be 16 for split plans, with at most 8 head
 * groups per request (q_len * num_heads <= 128); MLA_E_UNSUPPORTED
 * otherwise.
 * Errors: as mla_decode_partition.
 */
int mla_decode_fused(const void* q_absorbed, const void* q_pe, const void* ckv_cache,
                     const void* kpe_cache, int32_t num_blocks, int32_t block_size,
                     const int32_t* block_table,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                     int32_t num_heads, int32_t q_len, float scale, int32_t dtype,
                     const int32_t* partitions,
                     const int32_t* splits, const int32_t* row_indptr, int32_t total_rows,
                     int32_t max_rows_per_req, int32_t heads_per_wg, float* partial_out,
                     float* partial_lse2, void* out, float* lse2_out, uint64_t* sync,
                     int32_t* debug_ranges, hipStream_t stream);

/*
 * mla_absorb_query / mla_unabsorb_output -- the per-head products on either
 * side of absorbed decode (mlxcel pull request 995, "What changed", the
 * absorb.rs bullet: kv_b_proj splits into W_UK [H, qk_nope, r], folded into
 * the query, and W_UV^T [H, r, v_head], applied to the latent output; with
 * qk_nope = v_head = 128 and r = 512):
 *   q_absorbed[i, h, :] = q_nope[i, h, :] . W_UK[h]      (128 -> 512)
 *   o[i, h, :]          = out_latent[i, h, :] . W_UV^T[h] (512 -> 128)
 * fp32 accumulation in a fixed order, one round-to-nearest-even into the
 * 16-bit type of the tensors (bit-identical run to run).
 *
 * rows        rows of each head: the batch, or batch * q_len for several
 *             new tokens (token-major rows flatten into the batch), >= 0
 * num_heads   1 .. MLA_MAX_HEADS * MLA_MAX_QLEN
 * q_nope      dev 16-bit [rows, num_heads, 128];  w_uk dev [num_heads, 128, 512]
 * q_absorbed  dev 16-bit [rows, num_heads, 512] (written)
 * out_latent  dev 16-bit [rows, num_heads, 512];  w_uv_t dev [num_heads, 512, 128]
 * o           dev 16-bit [rows, num_heads, 128] (written)
 * All 16-byte aligned; dtype MLA_F16 or MLA_BF16 for every tensor.
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_ALIGN, MLA_E_UNSUPPORTED, MLA_E_HIP.
 */
int mla_absorb_query(const void* q_nope, const void* w_uk, void* q_absorbed, int32_t rows,
                     int32_t num_heads, int32_t dtype, hipStream_t stream);
int mla_unabsorb_output(const void* out_latent, const void* w_uv_t, void* o, int32_t rows,
                        int32_t num_heads, int32_t dtype, hipStream_t stream);

/*
 * mla_decode_noalloc -- the split decode without caller workspace.
 *
 * For callers that cannot allocate device memory between calls: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same result as mla_decode_partition followed by mla_decode_reduce
 * (bit for bit, same plan), but the fp32 partials and their LSEs go to a
 * fixed array inside this library's code object: MLA_NOALLOC_SCRATCH_BYTES
 * on each GPU the library runs on, held until the process ends. Its device
 * address is looked up once per device (hipGetSymbolAddress, with that
 * device current). The call allocates and frees nothing.
 *
 * Every call on one GPU shares that GPU's array and leaves the last call's
 * partials in it: calls that overlap on one GPU (different streams or
 * threads) race and give unspecified results; serialise them. Nothing in
 * the array needs clearing: every row of the plan is written before the
 * reduce reads it.
 *
 * Arguments as mla_decode_partition, without partial_out, partial_lse2 and
 * debug_ranges; out (always) and lse2_out (or NULL) as for
 * mla_decode_reduce. A single-pass plan (total_rows == batch) needs no
 * scratch and writes `out` directly.
 * Errors: as mla_decode_partition; MLA_E_WORKSPACE when the plan's partials
 * (mla_noalloc_scratch_bytes) exceed MLA_NOALLOC_SCRATCH_BYTES -- choose the
 * plan with workspace_limit_bytes at most that size.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int mla_decode_noalloc(const void* q_absorbed, const void* q_pe, const void* ckv_cache,
                       const void* kpe_cache, int32_t num_blocks, int32_t block_size,
                       const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t batch, int32_t num_heads,
                       int32_t q_len, float scale, int32_t dtype, const int32_t* partitions,
                       const int32_t* splits, const int32_t* row_indptr, int32_t total_rows,
                       int32_t max_rows_per_req, int32_t heads_per_wg, void* out,
                       float* lse2_out, hipStream_t stream);

/* Scratch bytes mla_decode_noalloc uses for a plan: the partials
 * [total_rows, q_len * num_heads, 512] fp32 (rounded up to 256 bytes) plus
 * their LSEs (0 for negative arguments). */
size_t mla_noalloc_scratch_bytes(int32_t total_rows, int32_t num_heads, int32_t q_len);

/*
 * mla_stream_read -- measurement helper, not part of the decode: one launch
 * of a plain contiguous read of `bytes` bytes at `src` (4096 workgroups of
 * 256 threads, one 16-byte load per thread and iteration). It is the
 * reference a benchmark times over the same byte count as a partition
 * launch, for the rate a launch that only reads reaches on this device.
 * src         dev, 16-byte aligned; bytes a multiple of 16 (0: nothing)
 * sink        dev uint32 [1]: written only by a thread whose XOR fold of
 *             the 4-byte words it read equals `never` (pass a value no such
 *             fold can take, e.g. one with a bit set that no word of the
 *             data has), so the loads stay and nothing is written
 * Errors: MLA_E_NULL, MLA_E_ALIGN, MLA_E_HIP.
 */
int mla_stream_read(const void* src, size_t bytes, uint32_t* sink, uint32_t never,
                    hipStream_t stream);

/*
 * mla_copy_probe -- measurement helper, not part of the decode: one launch
 * that only copies the KV of paged rows into LDS, as the partition kernels'
 * copies do (global_load_lds_dwordx4, 1 KB per instruction: the 32 ckv rows
 * and 4 kpe pieces of each 32-token block), with `groups` workgroups per
 * row on one XCD (1: every block read by one CU; 2 or 4: by that many, as
 * the 64-head workgroups of a 128-head row read it), `waves` copying waves
 * (4 or 8) each keeping `inflight` copies (4, 8 or 16) in flight. It shows
 * the rate the memory path gives such copies apart from any arithmetic.
 * ckv_pool   dev 16-bit [num_blocks, 32, 512]; kpe_pool dev 16-bit
 *            [num_blocks, 32, 64]
 * table      dev int32 [rows, blocks_per_row]: block k of row u is
 *            table[u * blocks_per_row + k] (clamped into [0, num_blocks))
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_UNSUPPORTED, MLA_E_HIP.
 */
int mla_copy_probe(const void* ckv_pool, const void* kpe_pool, int32_t num_blocks,
                   const int32_t* table, int32_t rows, int32_t blocks_per_row, int32_t groups,
                   int32_t waves, int32_t inflight, hipStream_t stream);

/* Text for a status code (static storage). */
const char* mla_status_string(int status);

/* Message of the calling thread's last failed call ("" if none). */
const char* mla_last_error(void);

/*
 * Path counters (process-wide, atomic): [0] single-pass partition launches,
 * [1] split partition launches, [2] reduce launches, [3] partition rows
 * launched. They make the path a measurement took provable from its output
 * (mlxcel pull request 995, "How to run the benchmark, and how to prove
 * which path it took").
 */
void mla_get_counters(uint64_t out[4]);
void mla_reset_counters(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
