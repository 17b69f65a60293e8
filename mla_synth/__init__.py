"""Seeded synthetic inputs for paged, matrix-absorbed MLA decode.

This module only draws and encodes inputs. It holds none of the attention
arithmetic: the f64 oracle and the HIP library both take what it returns.

Shapes and value recipe follow the workloads the pages describe:
  * latent row of width 512 (kv_lora_rank) plus a rope row of width 64
    (qk_rope_head_dim), block size 32 -- vllm-metal pull request 601
    "[kernel] Wire MLA split-KV decode", section "Wrapper benchmark" (setup
    line);
  * values drawn as standard normals, stored as fp16 or bf16.

Recipe (one numpy PCG64 generator per case, draws in this order):
  1. context lengths, only when a range is given: integers(lo, hi, endpoint)
  2. a permutation of the block pool (pool = pool_factor x blocks needed,
     unless the pool size is given)
  3. ckv pool  [pool, 32, 512]  standard normal float32
  4. kpe pool  [pool, 32, 64]   standard normal float32
  5. q_absorbed [B, Q*H, 512]   standard normal float32
  6. q_pe       [B, Q*H, 64]    standard normal float32
Q (``q_len``, default 1) is the number of new tokens per request: row j*H + h
is head h of new token j, which sits at position n - Q + j of the context.
Every float32 draw is multiplied by ``value_scale`` (a power of two, so the
product is exact) and rounded to nearest-even into the 16-bit storage type.
Request b's block table is the next ceil(n_b/32) entries of the permutation,
so all requests share one pool. Table entries past a request's last block
point at a block no request uses.

With ``poison=True`` every unreferenced pool block and every row past the
context end in a request's last block is filled with NaN: a correct kernel
never lets those rows reach its output.

With ``kv_dtype="fp8_e4m3"`` the two cache pools are stored one byte per
value in the E4M3 format of the OCP 8-bit floating point specification
(exponent bias 7, 3 mantissa bits, max 448, NaN = S.1111.111, no
infinities): each drawn value v (times value_scale) is stored as the code
nearest to v / kv_scale, ties to the even code, saturating at 448. Queries
stay 16-bit. The pages keep 16-bit caches only; this layout is ours.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK_SIZE = 32
KV_LORA_RANK = 512
ROPE_DIM = 64
# 1/sqrt(qk_nope + qk_rope) with qk_nope = 128 and qk_rope = 64.
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)

NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}
FP8_NAN = 0x7F          # E4M3 NaN (S.1111.111)
FP8_MAX = 448.0         # largest finite E4M3 value


def _fp8_positive_table() -> np.ndarray:
    """Values of the E4M3 codes 0x00..0x7E (OCP 8-bit floating point, E4M3:
    exponent bias 7, three mantissa bits, subnormals at exponent field 0, no
    infinities), ascending. Used only to encode inputs."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.asarray(vals, dtype=np.float64)


_FP8_TABLE = _fp8_positive_table()


def f32_to_fp8_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round values to E4M3 (nearest, ties to the even code), saturating at
    +-448; return raw bytes. Inputs here are finite."""
    y = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(y), FP8_MAX)
    hi = np.clip(np.searchsorted(_FP8_TABLE, a, side="left"), 0, _FP8_TABLE.size - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _FP8_TABLE[lo]
    dhi = _FP8_TABLE[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (nearest-even); return raw bits."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even on the bit pattern).

    Inputs here are finite normals, so no NaN/Inf handling is needed.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def encode16(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def _draw16(rng: np.random.Generator, shape, dtype: str, value_scale: float,
            chunk_rows: int = 1 << 22) -> np.ndarray:
    """Draw standard normals in float32 and encode them, a chunk at a time."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    total = flat.size
    step = max(1, chunk_rows)
    pos = 0
    while pos < total:
        k = min(step, total - pos)
        v = rng.standard_normal(k, dtype=np.float32)
        if value_scale != 1.0:
            v *= np.float32(value_scale)
        flat[pos:pos + k] = encode16(v, dtype)
        pos += k
    return out


def _draw8(rng: np.random.Generator, shape, value_scale: float, kv_scale: float,
           chunk_rows: int = 1 << 22) -> np.ndarray:
    """Draw standard normals in float32 (times value_scale) and store each
    value v as the E4M3 code nearest to v / kv_scale, a chunk at a time."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint8)
    flat = out.reshape(-1)
    pos = 0
    while pos < flat.size:
        k = min(max(1, chunk_rows), flat.size - pos)
        v = rng.standard_normal(k, dtype=np.float32)
        if value_scale != 1.0:
            v *= np.float32(value_scale)
        flat[pos:pos + k] = f32_to_fp8_e4m3_bits(v.astype(np.float64) / kv_scale)
        pos += k
    return out


@dataclasses.dataclass
class Case:
    """One decode batch: raw 16-bit payloads plus int32 metadata."""
    dtype: str
    batch: int
    heads: int
    context_lens: np.ndarray   # int32 [B]
    block_table: np.ndarray    # int32 [B, max_blocks]
    ckv_pool: np.ndarray       # uint16 [nblk, 32, 512]
    kpe_pool: np.ndarray       # uint16 [nblk, 32, 64]
    q_absorbed: np.ndarray     # uint16 [B, H, 512]
    q_pe: np.ndarray           # uint16 [B, H, 64]
    scale: float
    seed: int
    poisoned: bool = False
    q_len: int = 1             # new tokens per request; q rows are [B, q_len * H]
    block_size: int = BLOCK_SIZE   # tokens per cache block (32, or 16)
    # Latent cache storage: None = the 16-bit dtype above; "fp8_e4m3" = one
    # E4M3 byte per value, the stored value times kv_scale (one scale for the
    # ckv and kpe pools).
    kv_dtype: str | None = None
    kv_scale: float = 1.0

    @property
    def num_blocks(self) -> int:
        return int(self.ckv_pool.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def kv_bytes(self) -> int:
        return int(self.context_lens.astype(np.int64).sum()) * (KV_LORA_RANK + ROPE_DIM) * 2


def blocks_for(n: int, block_size: int = BLOCK_SIZE) -> int:
    return (int(n) + block_size - 1) // block_size


def make_case(seed: int, batch: int, heads: int, contexts=None, context_range=None,
              dtype: str = "f16", value_scale: float = 1.0, pool_factor: int = 2,
              pool_blocks: int | None = None, poison: bool = False,
              scale: float = DEFAULT_SCALE, max_blocks: int | None = None,
              q_len: int = 1, block_size: int = BLOCK_SIZE, kv_dtype: str | None = None,
              kv_scale: float = 1.0) -> Case:
    rng = np.random.Generator(np.random.PCG64(seed))
    if context_range is not None:
        lo, hi = context_range
        ctx = rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)
    else:
        ctx = np.asarray(contexts, dtype=np.int32).reshape(batch)
    nblk = [blocks_for(n, block_size) for n in ctx]
    needed = int(sum(nblk))
    pool = int(pool_blocks) if pool_blocks is not None else max(1, pool_factor * needed)
    if pool < needed:
        raise ValueError("pool smaller than the blocks the batch needs")
    perm = rng.permutation(pool).astype(np.int32)
    if kv_dtype is None:
        ckv = _draw16(rng, (pool, block_size, KV_LORA_RANK), dtype, value_scale)
        kpe = _draw16(rng, (pool, block_size, ROPE_DIM), dtype, value_scale)
    elif kv_dtype == "fp8_e4m3":
        ckv = _draw8(rng, (pool, block_size, KV_LORA_RANK), value_scale, kv_scale)
        kpe = _draw8(rng, (pool, block_size, ROPE_DIM), value_scale, kv_scale)
    else:
        raise ValueError(f"unknown kv_dtype {kv_dtype!r}")
    qa = _draw16(rng, (batch, q_len * heads, KV_LORA_RANK), dtype, value_scale)
    qp = _draw16(rng, (batch, q_len * heads, ROPE_DIM), dtype, value_scale)

    width = max(1, max(nblk) if nblk else 1)
    if max_blocks is not None:
        width = max(width, int(max_blocks))
    unused = perm[needed:]
    table = np.empty((batch, width), dtype=np.int32)
    off = 0
    for b in range(batch):
        k = nblk[b]
        table[b, :k] = perm[off:off + k]
        off += k
        rest = width - k
        if rest:
            filler = unused if unused.size else perm[:1]
            table[b, k:] = filler[np.arange(rest) % filler.size]

    case = Case(dtype=dtype, batch=batch, heads=heads, context_lens=ctx,
                block_table=table, ckv_pool=ckv, kpe_pool=kpe, q_absorbed=qa,
                q_pe=qp, scale=float(scale), seed=seed, q_len=int(q_len),
                block_size=int(block_size), kv_dtype=kv_dtype, kv_scale=float(kv_scale))
    if poison:
        poison_case(case)
    return case


def poison_case(case: Case) -> None:
    """Fill unreferenced blocks and the rows past each context end with NaN."""
    nan = np.uint8(FP8_NAN) if case.kv_dtype else np.uint16(NAN_BITS[case.dtype])
    used = np.zeros(case.num_blocks, dtype=bool)
    for b in range(case.batch):
        k = blocks_for(case.context_lens[b], case.block_size)
        used[case.block_table[b, :k]] = True
    case.ckv_pool[~used] = nan
    case.kpe_pool[~used] = nan
    for b in range(case.batch):
        n = int(case.context_lens[b])
        bs = case.block_size
        if n % bs:
            last = case.block_table[b, blocks_for(n, bs) - 1]
            case.ckv_pool[last, n % bs:] = nan
            case.kpe_pool[last, n % bs:] = nan
    case.poisoned = True


# The five workloads, by name. Seeds are fixed so every run sees the same data.
WORKLOADS = {
    # B=1, H=16, 1024 tokens (32 blocks) over a 64-block pool, fp16, 2 partitions.
    "tiny": dict(seed=1001, batch=1, heads=16, contexts=[1024], dtype="f16",
                 pool_blocks=64),
    # DeepSeek-V2-Lite-shaped: B=1, H=16, 32768 tokens, fp16.
    "v2lite_32k": dict(seed=1002, batch=1, heads=16, contexts=[32768], dtype="f16"),
    # Two requests in one pool, fp16.
    "two_req_32k_32k": dict(seed=1003, batch=2, heads=16, contexts=[32768, 32768],
                            dtype="f16"),
    "two_req_32k_20k": dict(seed=1003, batch=2, heads=16, contexts=[32768, 20000],
                            dtype="f16"),
    # DeepSeek-V3-shaped long context: B=1, H=128, bf16, values x0.5.
    "v3_81k": dict(seed=1004, batch=1, heads=128, contexts=[81920], dtype="bf16",
                   value_scale=0.5),
    "v3_131k": dict(seed=1004, batch=1, heads=128, contexts=[131072], dtype="bf16",
                    value_scale=0.5),
    # Mixed batch: B=8, H=128, contexts uniform in [4096, 131072], bf16.
    "mixed_b8": dict(seed=1005, batch=8, heads=128, context_range=(4096, 131072),
                     dtype="bf16"),
    # Several new tokens per request (multi-token decode: MTP / speculative
    # verification windows) at the V2-Lite and V3 shapes.
    "v2lite_32k_q2": dict(seed=1006, batch=1, heads=16, contexts=[32768], dtype="f16",
                          q_len=2),
    "v2lite_32k_q4": dict(seed=1006, batch=1, heads=16, contexts=[32768], dtype="f16",
                          q_len=4),
    "v3_131k_q2": dict(seed=1007, batch=1, heads=128, contexts=[131072], dtype="bf16",
                       value_scale=0.5, q_len=2),
}


def make_workload(name: str, **overrides) -> Case:
    """A named workload; block_size=16 stores the same contexts in 16-token
    blocks (a fixed pool size is doubled to hold the same tokens)."""
    spec = dict(WORKLOADS[name])
    bs = int(overrides.get("block_size", BLOCK_SIZE))
    if "pool_blocks" in spec and bs != BLOCK_SIZE:
        spec["pool_blocks"] = spec["pool_blocks"] * BLOCK_SIZE // bs
    spec.update(overrides)
    return make_case(**spec)
