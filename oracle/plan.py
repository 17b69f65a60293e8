"""Independent mirror of the host partition chooser and the index math.

Test infrastructure only. Written in plain Python integers from the rule
below; it shares no code with the C++ chooser, and the tests require the
two to agree bit for bit.

The pages give the chooser's gates but not its constants (vllm-metal pull
request 601 "[kernel] Wire MLA split-KV decode", "What changed": split only
for pure decode, a long enough context, a small decode launch, 2 to 8
partitions and bounded temporary memory; "Serving sanity check" paragraph
before the grid: the split path starts at 32K+ context). The rule:

  G          = q_len * H / heads_per_wg       workgroups per row (every
               query row of the request: q_len new tokens x H heads)
  eligible   = q_len == 1 and B * G < num_cus  pure decode, small launch
  P_b        = force_P, else clamp(ceil(n_b / tokens_per_partition),
               min_P, max_P) if eligible and n_b >= min_split_ctx, else 1
  cap        = num_cus * wgs_per_cu              workgroups in one wave
  tile       = max(min_tile_blocks, ceil(G * sum_b nblk_b / cap))
  S_b        = force_S, else max(1, ceil(ceil(nblk_b / P_b) / tile))
  fit        = (auto S only) if G * sum_b P_b * S_b > cap, the tile becomes
               the smallest larger one with G * sum_b P_b * S_b <= cap, or,
               if none fits, max_b ceil(nblk_b / P_b) (every S_b = 1)
  rows       = sum_b P_b * S_b, request-major (row_indptr)
  workspace  = rows * q_len * H * (512 + 1) * 4 bytes if any P_b * S_b > 1,
               else 0
With q_len > 1 the policy keeps P_b = 1 (the split is for pure decode only),
and the device tiling S_b applies as for one token. q_len is at most 8.

Workspace shedding, when a limit is set and exceeded, in order:
  1. (auto S only) double the tile until the limit holds or every S_b = 1;
  2. (auto P only) lower the largest P_b by one (lowest b on ties), not
     below 2, until the limit holds;
  3. (auto P only) set P_b = 1 in ascending n_b order (lowest b on ties)
     until the limit holds;
  still over the limit -> error (possible only with forced values).

Index math. With cache blocks of BS tokens (32, the pages' block size, or
16, the "block16" layout the vllm-metal pull request's review asks to see
covered) and nblk = ceil(n/BS):
  partition p of P covers blocks [min(p*bpp, nblk), min((p+1)*bpp, nblk)),
  bpp = ceil(nblk / P); tile s of S inside a partition of m blocks covers
  [b0 + min(s*bps, m), b0 + min((s+1)*bps, m)), bps = ceil(m / S); its
  tokens are [min(lo*BS, n), min(hi*BS, n)). The chooser's nblk_b and tile
  count blocks of the same size.
"""
from __future__ import annotations

import dataclasses

BLOCK_SIZE = 32
BLOCK_SIZES = (16, 32)
LATENT = 512
MAX_PARTITIONS = 8
MAX_SPLITS = 4096
MAX_QLEN = 8


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def default_heads_per_wg(heads: int) -> int:
    """Heads one workgroup of the partition kernel covers (library default):
    64 when 64 divides the head count, else one 16-row MFMA tile."""
    return 64 if heads % 64 == 0 else 16


@dataclasses.dataclass
class PlanParams:
    min_split_ctx: int = 32768
    tokens_per_partition: int = 16384
    min_partitions: int = 2
    max_partitions: int = MAX_PARTITIONS
    num_cus: int = 256
    heads_per_wg: int = 0
    min_tile_blocks: int = 4
    wgs_per_cu: int = 1
    force_partitions: int = 0
    force_splits: int = 0
    workspace_limit_bytes: int = 0


def partition_range(n: int, P: int, S: int, p: int, s: int,
                    block_size: int = BLOCK_SIZE):
    """Token range [begin, end) of tile s of partition p (see module doc)."""
    nblk = _cdiv(n, block_size)
    bpp = _cdiv(nblk, P)
    pb0 = min(p * bpp, nblk)
    pb1 = min((p + 1) * bpp, nblk)
    m = pb1 - pb0
    bps = _cdiv(m, S) if m > 0 else 0
    lo = pb0 + min(s * bps, m)
    hi = pb0 + min((s + 1) * bps, m)
    return min(lo * block_size, n), min(hi * block_size, n)


def row_ranges(ctx, P, S, block_size: int = BLOCK_SIZE):
    """List of (b, begin, end) for every row, request-major."""
    out = []
    for b, n in enumerate(ctx):
        for p in range(P[b]):
            for s in range(S[b]):
                lo, hi = partition_range(int(n), P[b], S[b], p, s, block_size)
                out.append((b, lo, hi))
    return out


def _splits_for(nblk: int, P: int, tile: int) -> int:
    return max(1, _cdiv(_cdiv(nblk, P), tile))


def choose_partitions(batch: int, heads: int, q_len: int, ctx, params: PlanParams | None = None,
                      block_size: int = BLOCK_SIZE):
    """Mirror of mla_choose_partitions. Raises ValueError on invalid input."""
    prm = params or PlanParams()
    if batch < 0 or q_len < 1 or q_len > MAX_QLEN or block_size not in BLOCK_SIZES:
        raise ValueError("shape")
    if heads < 16 or heads > 128 or heads % 16:
        raise ValueError("unsupported heads")
    ctx = [int(c) for c in ctx]
    if len(ctx) != batch or any(c < 0 for c in ctx):
        raise ValueError("context")
    if not (1 <= prm.min_partitions <= prm.max_partitions <= MAX_PARTITIONS):
        raise ValueError("partition bounds")
    if (prm.tokens_per_partition < 1 or prm.num_cus < 1 or prm.min_tile_blocks < 1
            or prm.wgs_per_cu < 1 or prm.min_split_ctx < 0):
        raise ValueError("params")
    if not (0 <= prm.force_partitions <= MAX_PARTITIONS) or not (0 <= prm.force_splits <= MAX_SPLITS):
        raise ValueError("force")
    if prm.workspace_limit_bytes < 0:
        raise ValueError("limit")
    hpw = prm.heads_per_wg or default_heads_per_wg(heads)
    if hpw not in (16, 64) or heads % hpw:
        raise ValueError("heads per workgroup")
    G = q_len * heads // hpw
    nblk = [_cdiv(n, block_size) for n in ctx]
    total_blocks = sum(nblk)

    if True:
        eligible = q_len == 1 and batch * G < prm.num_cus
        autoP = prm.force_partitions == 0
        autoS = prm.force_splits == 0
        P = []
        for n in ctx:
            if not autoP:
                P.append(prm.force_partitions)
            elif eligible and n >= prm.min_split_ctx:
                P.append(min(max(_cdiv(n, prm.tokens_per_partition), prm.min_partitions),
                             prm.max_partitions))
            else:
                P.append(1)
        cap = prm.num_cus * prm.wgs_per_cu
        tile = max(prm.min_tile_blocks, _cdiv(G * total_blocks, cap))

        def wgs(t):
            return G * sum(p * _splits_for(nb, p, t) for nb, p in zip(nblk, P))

        if autoS and wgs(tile) > cap:
            biggest = max([tile] + [_cdiv(nb, p) for nb, p in zip(nblk, P)])
            if wgs(biggest) > cap:
                tile = biggest
            else:
                # wgs() never grows with the tile: bisect for the first fit.
                bad, good = tile, biggest
                while good - bad > 1:
                    mid = (bad + good) // 2
                    if wgs(mid) <= cap:
                        good = mid
                    else:
                        bad = mid
                tile = good
        S = [(_splits_for(nb, p, tile) if autoS else prm.force_splits)
             for nb, p in zip(nblk, P)]

    def workspace():
        rows = sum(p * s for p, s in zip(P, S))
        if any(p * s > 1 for p, s in zip(P, S)):
            return rows * q_len * heads * (LATENT + 1) * 4
        return 0

    limit = prm.workspace_limit_bytes
    if limit > 0 and workspace() > limit:
        if autoS:
            while workspace() > limit and max(S) > 1:
                tile = min(tile * 2, 1 << 30)
                S = [_splits_for(nb, p, tile) for nb, p in zip(nblk, P)]
        if autoP:
            while workspace() > limit and max(P) > 2:
                top = max(P)
                b = P.index(top)
                P[b] -= 1
            while workspace() > limit and max(P) > 1:
                cands = [(ctx[b], b) for b in range(batch) if P[b] > 1]
                _, b = min(cands)
                P[b] = 1
        if workspace() > limit:
            raise ValueError("workspace")

    row_indptr = [0]
    for p, s in zip(P, S):
        row_indptr.append(row_indptr[-1] + p * s)
    ws = workspace()
    return dict(P=P, S=S, row_indptr=row_indptr, total_rows=row_indptr[-1],
                max_rows_per_req=max([p * s for p, s in zip(P, S)], default=0),
                tile_blocks=tile, workspace_bytes=ws, needs_reduce=int(ws > 0),
                heads_per_wg=hpw, groups=G)
