"""50-digit scalar brute force over the literal definitions (tiny inputs only).

Test infrastructure only. These loops share nothing with ``reference``: they
decode bits themselves, walk the block table themselves and never subtract a
running maximum, so a slip in the f64 oracle's gather, scaling, softmax or
LSE shows up as a disagreement.
"""
from __future__ import annotations

import struct

import mpmath

mpmath.mp.dps = 50


def _bits_to_mpf(bits: int, dtype: str):
    bits = int(bits)
    if dtype == "f16":
        sign = -1 if bits >> 15 else 1
        e = (bits >> 10) & 0x1F
        f = bits & 0x3FF
        if e == 0:
            return sign * mpmath.mpf(f) * mpmath.mpf(2) ** -24
        if e == 31:
            raise ValueError("non-finite input")
        return sign * (1 + mpmath.mpf(f) / 1024) * mpmath.mpf(2) ** (e - 15)
    if dtype == "bf16":
        val = struct.unpack("<f", struct.pack("<I", bits << 16))[0]
        return mpmath.mpf(val)
    raise ValueError(dtype)


def _row(pool, phys, slot, dtype):
    return [_bits_to_mpf(v, dtype) for v in pool[phys][slot]]


def _fp8_to_mpf(code: int):
    """One E4M3 byte by the OCP 8-bit floating point definition, case by
    case: exponent field 0 is subnormal (m * 2^-9), 15 with mantissa 7 is
    NaN, otherwise (8 + m) * 2^(e - 10)."""
    code = int(code)
    neg = code >= 128
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        raise ValueError("non-finite input")
    v = mpmath.mpf(m) * mpmath.mpf(2) ** -9 if e == 0 else \
        mpmath.mpf(8 + m) * mpmath.mpf(2) ** (e - 10)
    return -v if neg else v


def _cache_row(case, pool, phys: int, slot: int):
    """A cache row as mpf values: 16-bit rows, or E4M3 bytes times the
    cache scale."""
    if getattr(case, "kv_dtype", None) == "fp8_e4m3":
        sc = mpmath.mpf(float(case.kv_scale))
        return [_fp8_to_mpf(v) * sc for v in pool[phys][slot]]
    return _row(pool, phys, slot, case.dtype)


def latent_brute(case, b: int, h: int):
    """out[b, h] (list of 512 mpf) and lse2[b, h] (mpf) by the definition."""
    n = int(case.context_lens[b])
    bs = int(case.ckv_pool.shape[1])   # tokens per cache block
    qa = [_bits_to_mpf(v, case.dtype) for v in case.q_absorbed[b][h]]
    qp = [_bits_to_mpf(v, case.dtype) for v in case.q_pe[b][h]]
    scale = mpmath.mpf(case.scale)
    num = [mpmath.mpf(0)] * len(qa)
    den = mpmath.mpf(0)
    for t in range(n):
        phys = int(case.block_table[b][t // bs])
        c = _cache_row(case, case.ckv_pool, phys, t % bs)
        k = _cache_row(case, case.kpe_pool, phys, t % bs)
        s = scale * (mpmath.fsum(x * y for x, y in zip(qa, c))
                     + mpmath.fsum(x * y for x, y in zip(qp, k)))
        e = mpmath.exp(s)
        den += e
        for i in range(len(num)):
            num[i] += e * c[i]
    if n == 0:
        return [mpmath.mpf(0)] * len(qa), mpmath.mpf("-inf")
    return [x / den for x in num], mpmath.log(den) / mpmath.log(2)


def weight_moments_brute(case, b: int, h: int):
    """sum_t w_t and sum_t w_t^2 with w_t = exp(s_t - max_t s_t), by the
    definition (scores by plain sums, the maximum found first)."""
    n = int(case.context_lens[b])
    bs = int(case.ckv_pool.shape[1])
    qa = [_bits_to_mpf(v, case.dtype) for v in case.q_absorbed[b][h]]
    qp = [_bits_to_mpf(v, case.dtype) for v in case.q_pe[b][h]]
    scale = mpmath.mpf(case.scale)
    scores = []
    for t in range(n):
        phys = int(case.block_table[b][t // bs])
        c = _cache_row(case, case.ckv_pool, phys, t % bs)
        k = _cache_row(case, case.kpe_pool, phys, t % bs)
        scores.append(scale * (mpmath.fsum(x * y for x, y in zip(qa, c))
                               + mpmath.fsum(x * y for x, y in zip(qp, k))))
    if not scores:
        return mpmath.mpf(0), mpmath.mpf(0)
    top = max(scores)
    w = [mpmath.exp(s - top) for s in scores]
    return mpmath.fsum(w), mpmath.fsum(x * x for x in w)


def latent_brute_window(case, b: int, j: int, h: int):
    """Head h of new token j in a window of case.q_len new tokens, by the
    definition with an explicit causal mask: token j sits at position
    pos = n - q_len + j and every t > pos is skipped."""
    n = int(case.context_lens[b])
    bs = int(case.ckv_pool.shape[1])   # tokens per cache block
    pos = n - int(case.q_len) + j
    row = j * case.heads + h
    qa = [_bits_to_mpf(v, case.dtype) for v in case.q_absorbed[b][row]]
    qp = [_bits_to_mpf(v, case.dtype) for v in case.q_pe[b][row]]
    scale = mpmath.mpf(case.scale)
    num = [mpmath.mpf(0)] * len(qa)
    den = mpmath.mpf(0)
    for t in range(n):
        if t > pos:
            continue
        phys = int(case.block_table[b][t // bs])
        c = _cache_row(case, case.ckv_pool, phys, t % bs)
        k = _cache_row(case, case.kpe_pool, phys, t % bs)
        s = scale * (mpmath.fsum(x * y for x, y in zip(qa, c))
                     + mpmath.fsum(x * y for x, y in zip(qp, k)))
        e = mpmath.exp(s)
        den += e
        for i in range(len(num)):
            num[i] += e * c[i]
    if den == 0:
        return [mpmath.mpf(0)] * len(qa), mpmath.mpf("-inf")
    return [x / den for x in num], mpmath.log(den) / mpmath.log(2)


def decompressed_brute(case, b: int, h: int, q_nope, W_UK, W_UV_T):
    """Pre-absorption attention for one (b, h) by the definition.

    q_nope [dn] floats; W_UK [dn, 512]; W_UV_T [512, dv] (plain floats).
    """
    n = int(case.context_lens[b])
    bs = int(case.ckv_pool.shape[1])   # tokens per cache block
    qn = [mpmath.mpf(float(x)) for x in q_nope]
    qp = [_bits_to_mpf(v, case.dtype) for v in case.q_pe[b][h]]
    scale = mpmath.mpf(case.scale)
    dn = len(qn)
    dv = len(W_UV_T[0])
    num = [mpmath.mpf(0)] * dv
    den = mpmath.mpf(0)
    for t in range(n):
        phys = int(case.block_table[b][t // bs])
        c = _cache_row(case, case.ckv_pool, phys, t % bs)
        k = _cache_row(case, case.kpe_pool, phys, t % bs)
        key = [mpmath.fsum(mpmath.mpf(float(W_UK[d][i])) * c[i] for i in range(len(c)))
               for d in range(dn)]
        val = [mpmath.fsum(c[i] * mpmath.mpf(float(W_UV_T[i][j])) for i in range(len(c)))
               for j in range(dv)]
        s = scale * (mpmath.fsum(x * y for x, y in zip(qn, key))
                     + mpmath.fsum(x * y for x, y in zip(qp, k)))
        e = mpmath.exp(s)
        den += e
        for j in range(dv):
            num[j] += e * val[j]
    return [x / den for x in num], mpmath.log(den) / mpmath.log(2)
