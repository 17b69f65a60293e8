"""f64 reference arithmetic for paged, matrix-absorbed MLA decode.

Test infrastructure only (see the package docstring). Every quantity is
computed in float64 from the 16-bit input values, with numpy matmul as the
only library primitive. No blocking, fusion or reordering beyond what the
definitions state.
"""
from __future__ import annotations

import math

import numpy as np

LATENT = 512
ROPE = 64
# log2(e); the split path's LSE is in base 2 (mlxcel pull request 995, "How
# #898's merge kernel is reused": the merge contract takes log2 LSEs).
LOG2_E = 1.4426950408889634
LN_2 = math.log(2.0)


def decode16(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw fp16 / bf16 bit patterns -> float64 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def decode_fp8_e4m3(bits: np.ndarray) -> np.ndarray:
    """Raw E4M3 bytes -> float64 values (exact), by the E4M3 definition of
    the OCP 8-bit floating point specification: sign bit, 4-bit exponent
    with bias 7, 3-bit mantissa; exponent field 0 holds the subnormals
    m/8 * 2^-6; S.1111.111 is NaN; there are no infinities (so 448 is the
    largest value)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (b & 0x7 == 0x7), np.nan, mag)
    return sign * mag


def decode_cache(rows: np.ndarray, dtype: str, kv_dtype=None, kv_scale: float = 1.0):
    """Cache rows -> float64: 16-bit rows of `dtype`, or E4M3 bytes times
    kv_scale when kv_dtype is "fp8_e4m3" (one scale for the whole latent
    cache; our reading, since the pages keep 16-bit caches only)."""
    if kv_dtype is None:
        return decode16(rows, dtype)
    if kv_dtype == "fp8_e4m3":
        return decode_fp8_e4m3(rows) * float(kv_scale)
    raise ValueError(f"unknown kv_dtype {kv_dtype!r}")


def gather_request(ckv_pool, kpe_pool, table_row, n: int, dtype: str,
                   lo: int = 0, hi: int | None = None, kv_dtype=None, kv_scale: float = 1.0):
    """Tokens [lo, hi) of one request, read through its block table.

    Token t lives in physical block table_row[t // BS], slot t % BS, where
    BS = ckv_pool.shape[1] is the block size (vllm-metal pull request 601,
    "Wrapper benchmark": block size 32 paged cache with a block table; its
    review also asks for blocks of 16). Only t < n is ever read.
    Returns (C [k, 512], Kp [k, 64]) in float64.
    """
    hi = n if hi is None else min(hi, n)
    lo = max(0, lo)
    if hi <= lo:
        return np.zeros((0, LATENT)), np.zeros((0, ROPE))
    bs = int(ckv_pool.shape[1])
    t = np.arange(lo, hi)
    phys = np.asarray(table_row)[t // bs]
    slot = t % bs
    C = decode_cache(ckv_pool[phys, slot], dtype, kv_dtype, kv_scale)
    Kp = decode_cache(kpe_pool[phys, slot], dtype, kv_dtype, kv_scale)
    return C, Kp


def _attend(qa, qp, C, Kp, scale):
    """Softmax attention of latent queries over gathered latent rows.

    Score s_t = scale * (qa . C_t + qp . Kp_t); weights exp(s_t - max);
    output sum_t w_t C_t / sum_t w_t; lse2 = (max + ln sum w) / ln 2.
    (mlxcel pull request 995, "What changed", Stage 1.)
    qa [h, 512], qp [h, 64] float64.

    Also returns the first two moments of the weights, sum_t w_t and
    sum_t w_t^2 (w_t = exp(s_t - max), so the largest weight is 1): they
    say how many tokens carry the softmax, which sizes the rounding error a
    GPU sum of 16-bit weights can have.
    """
    h = qa.shape[0]
    if C.shape[0] == 0:
        # No visible token: zero output, lse2 = -inf, so the row carries
        # weight 0 in any merge (MTPLX pull request 639, commit on rows
        # without a visible key).
        return np.zeros((h, LATENT)), np.full(h, -np.inf), np.zeros(h), np.zeros(h)
    s = scale * (qa @ C.T + qp @ Kp.T)            # [h, k]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    z = w.sum(axis=1)
    out = (w @ C) / z[:, None]
    lse2 = (m[:, 0] + np.log(z)) / LN_2
    return out, lse2, z, (w * w).sum(axis=1)


def visible_len(n: int, q_len: int, j: int) -> int:
    """Tokens new token j of a window of q_len sees in a context of n.

    The cache write comes before attention (vllm-metal pull request 601,
    "Wrapper benchmark": the timed step writes the new token's KV, then
    attends), so n counts all q_len new tokens and token j sits at position
    n - q_len + j. Within the window attention is causal: token j sees
    positions 0 .. n - q_len + j. Our reading; the pages decode one token.
    """
    return max(0, n - q_len + 1 + j)


def latent_one(case, b: int, heads=None, lo: int = 0, hi: int | None = None,
               moments: bool = False):
    """Oracle output for request b (optionally a subset of query rows / a
    token range). Query row j * H + h is head h of new token j. With
    moments=True also the weight moments sum w and sum w^2 of each row."""
    n = int(case.context_lens[b])
    q_len = int(getattr(case, "q_len", 1))
    rows = np.arange(q_len * case.heads) if heads is None else np.asarray(heads)
    hi = n if hi is None else hi
    out = np.zeros((rows.size, LATENT))
    lse2 = np.zeros(rows.size)
    w1 = np.zeros(rows.size)
    w2 = np.zeros(rows.size)
    for j in sorted(set((rows // case.heads).tolist())):
        sel = rows // case.heads == j
        C, Kp = gather_request(case.ckv_pool, case.kpe_pool, case.block_table[b], n,
                               case.dtype, lo, min(hi, visible_len(n, q_len, j)),
                               getattr(case, "kv_dtype", None), getattr(case, "kv_scale", 1.0))
        qa = decode16(case.q_absorbed[b, rows[sel]], case.dtype)
        qp = decode16(case.q_pe[b, rows[sel]], case.dtype)
        out[sel], lse2[sel], w1[sel], w2[sel] = _attend(qa, qp, C, Kp, case.scale)
    if moments:
        return out, lse2, w1, w2
    return out, lse2


def latent_f64(case, requests=None, heads=None, moments: bool = False):
    """Single-pass absorbed decode for a whole batch (or a sample of it).

    Returns out [B, q_len * H, 512] and lse2 [B, q_len * H]; entries outside
    the requested sample are NaN. With moments=True, also the weight moments
    sum_t w_t and sum_t w_t^2 [B, q_len * H] (w_t = exp(s_t - max s)).
    """
    B, H = case.batch, int(getattr(case, "q_len", 1)) * case.heads
    out = np.full((B, H, LATENT), np.nan)
    lse2 = np.full((B, H), np.nan)
    w1 = np.full((B, H), np.nan)
    w2 = np.full((B, H), np.nan)
    reqs = range(B) if requests is None else requests
    hs = np.arange(H) if heads is None else np.asarray(heads)
    for b in reqs:
        out[b, hs], lse2[b, hs], w1[b, hs], w2[b, hs] = latent_one(case, b, hs, moments=True)
    if moments:
        return out, lse2, w1, w2
    return out, lse2


# --------------------------------------------------------------------------
# Pre-absorption (decompressed) attention.
# mlxcel pull request 995, "What changed", absorb.rs bullet: kv_b_proj folds
# into W_UK [H, qk_nope, r] on the query side and W_UV^T [H, r, v_head] on
# the output side.
# --------------------------------------------------------------------------

def decompressed_f64(case, q_nope, W_UK, W_UV_T, requests=None):
    """Ordinary attention over up-projected keys and values.

    q_nope [B, H, dn] float64; W_UK [H, dn, 512]; W_UV_T [H, 512, dv].
    Per head: key_t = [W_UK ckv_t ; kpe_t], value_t = ckv_t W_UV^T,
    score = scale * [q_nope ; q_pe] . key_t, output = softmax-weighted
    values. Returns o [B, H, dv], lse2 [B, H].
    """
    assert int(getattr(case, "q_len", 1)) == 1, "pre-absorption path: one new token"
    B, H = case.batch, case.heads
    dv = W_UV_T.shape[2]
    o = np.full((B, H, dv), np.nan)
    lse2 = np.full((B, H), np.nan)
    reqs = range(B) if requests is None else requests
    for b in reqs:
        n = int(case.context_lens[b])
        C, Kp = gather_request(case.ckv_pool, case.kpe_pool, case.block_table[b], n,
                               case.dtype, 0, None, getattr(case, "kv_dtype", None),
                               getattr(case, "kv_scale", 1.0))
        qp = decode16(case.q_pe[b], case.dtype)
        for h in range(H):
            if n == 0:
                o[b, h] = 0.0
                lse2[b, h] = -np.inf
                continue
            K_nope = C @ W_UK[h].T                 # [n, dn]
            V = C @ W_UV_T[h]                      # [n, dv]
            s = case.scale * (K_nope @ q_nope[b, h] + Kp @ qp[h])
            m = s.max()
            w = np.exp(s - m)
            z = w.sum()
            o[b, h] = (w @ V) / z
            lse2[b, h] = (m + math.log(z)) / LN_2
    return o, lse2


def absorb_query(q_nope, W_UK):
    """q_absorbed[b, h] = q_nope[b, h] @ W_UK[h]  (query-side fold)."""
    return np.einsum("bhd,hdr->bhr", q_nope, W_UK)


def unabsorb_output(out_latent, W_UV_T):
    """o[b, h] = out_latent[b, h] @ W_UV^T[h]  (output-side fold)."""
    return np.einsum("bhr,hrv->bhv", out_latent, W_UV_T)


def orthogonal_weights(seed: int, heads: int, dim: int = LATENT):
    """Per-head orthogonal W_UK, W_UV^T of shape [H, dim, dim] (QR of Gaussians).

    With square orthogonal folds, q_nope = q_absorbed W_UK^T reproduces the
    given q_absorbed exactly in real arithmetic, so pre-absorption can be run
    at the full latent shape and mapped back by a transpose.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    def one():
        q, r = np.linalg.qr(rng.standard_normal((dim, dim)))
        return q * np.sign(np.diag(r))[None, :]
    W_UK = np.stack([one() for _ in range(heads)])
    W_UV_T = np.stack([one() for _ in range(heads)])
    return W_UK, W_UV_T


# --------------------------------------------------------------------------
# Split-KV partials and the log2 merge.
# vllm-metal pull request 601, "What changed": slices of the context, each
# with its softmax summary (LSE), combined into the same final answer.
# mlxcel pull request 995, "What changed" (split_kv.rs bullet) and "How #898's
# merge kernel is reused": normalised partial + log2 LSE per chunk,
# request-major rows.
# --------------------------------------------------------------------------

def partials_f64(case, ranges, row_indptr):
    """Normalised partial outputs and log2 LSEs for explicit token ranges.

    ranges: list over rows of (b, lo, hi); row_indptr [B+1] request-major.
    Returns partial_out [rows, H, 512], partial_lse2 [rows, H].
    """
    rows = len(ranges)
    H = int(getattr(case, "q_len", 1)) * case.heads
    po = np.zeros((rows, H, LATENT))
    pl = np.full((rows, H), -np.inf)
    for r, (b, lo, hi) in enumerate(ranges):
        assert row_indptr[b] <= r < row_indptr[b + 1]
        o, l = latent_one(case, b, None, lo, hi)
        po[r] = o
        pl[r] = l
    return po, pl


def merge_log2_f64(partial_out, partial_lse2, row_indptr):
    """Merge partials of each request by their log2 LSEs.

    M = max_r lse2_r; w_r = 2^(lse2_r - M); out = sum w_r O_r / sum w_r;
    lse2 = M + log2(sum w_r). All rows at -inf (nothing visible) merge to a
    zero output with lse2 = -inf (MTPLX pull request 639, commit on rows
    without a visible key).
    """
    row_indptr = np.asarray(row_indptr)
    B = row_indptr.size - 1
    H, D = partial_out.shape[1], partial_out.shape[2]
    out = np.zeros((B, H, D))
    lse2 = np.full((B, H), -np.inf)
    for b in range(B):
        r0, r1 = int(row_indptr[b]), int(row_indptr[b + 1])
        if r1 <= r0:
            continue
        L = partial_lse2[r0:r1]                     # [k, H]
        M = L.max(axis=0)                            # [H]
        for h in range(H):
            if M[h] == -np.inf:
                continue
            w = np.exp2(L[:, h] - M[h])
            W = w.sum()
            out[b, h] = (w @ partial_out[r0:r1, h]) / W
            lse2[b, h] = M[h] + math.log2(W)
    return out, lse2


def merge_ln_wrong(partial_out, partial_lse2, row_indptr):
    """Negative control: natural-log LSEs fed to the base-2 merge.

    The log2 values are converted to natural-log units (times ln 2) and
    handed to the same merge, which then weights rows by 2^(ln-units). It
    still returns a plausible weighted average, just the wrong one (mlxcel
    pull request 995, "How #898's merge kernel is reused").
    """
    return merge_log2_f64(partial_out, partial_lse2 * LN_2, row_indptr)
