"""GPU parity of the 64-head partition kernel over E4M3 byte caches
(mla_decode_partition_fp8 with heads_per_wg = 64) against the f64 oracle.

This kernel keeps the cache bytes as stored in its LDS ring and widens each
fragment after reading it: the score operand with an 8-byte read, the value
operand with the 8-bit transposing read. Every E4M3 value is exactly an
fp16 and a bf16 value, so at scale 1 the kernel must give, bit for bit, what
the 16-bit 64-head kernel gives on the widened cache: that pins the byte
layout, the swizzle, the transposing read's lane order and the token order
of both products at once. Also covered: every finite code through the value
path, the 128-head workloads in both block sizes, edge cases, needles at row
boundaries (which force the second pass), several new tokens per request.
"""
import dataclasses

import numpy as np
import pytest
import torch

import absorbed_mla_paged_amd as mla
import mla_synth
import oracle
from oracle import reference

from gpu_helpers import compare, log, rows_of_plan, run_case, to_device

pytestmark = pytest.mark.gpu

KV_SCALE = 2.0 ** -5


def fp8_case(seed, contexts, heads, dtype="bf16", kv_scale=KV_SCALE, **kw):
    return mla_synth.make_case(seed=seed, batch=len(contexts), heads=heads, contexts=contexts,
                               dtype=dtype, kv_dtype="fp8_e4m3", kv_scale=kv_scale, **kw)


def device_fp8(case):
    d = to_device(case)
    d["ckv_cache"] = torch.from_numpy(np.ascontiguousarray(case.ckv_pool)).cuda()
    d["kpe_cache"] = torch.from_numpy(np.ascontiguousarray(case.kpe_pool)).cuda()
    d["kv_scale"] = case.kv_scale
    return d


def run_wide(case, prm):
    prm = dict(prm)
    prm.setdefault("heads_per_wg", 64)
    out, lse2, plan, ranges = run_case(case, mla.PlanParams(**prm), dev=device_fp8(case),
                                       want_ranges=True)
    assert plan.info["heads_per_wg"] == 64
    return out, lse2, plan, ranges


def check(case, prm, what):
    out, lse2, plan, ranges = run_wide(case, prm)
    log(f"[plan] {what} P={plan.info['P']} S={plan.info['S']} rows={plan.total_rows}")
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, what, moments=mom)
    if plan.total_rows > case.batch:
        want = rows_of_plan(case, plan)
        got = [tuple(r) for r in ranges[:plan.total_rows]]
        assert got == [(lo, hi) for _, lo, hi in want]
    return out, lse2, plan


def widened(case):
    """The same cache as 16-bit values (exact: E4M3 fits both 16-bit types)."""
    ckv = mla_synth.encode16(reference.decode_fp8_e4m3(case.ckv_pool).astype(np.float32),
                             case.dtype)
    kpe = mla_synth.encode16(reference.decode_fp8_e4m3(case.kpe_pool).astype(np.float32),
                             case.dtype)
    return dataclasses.replace(case, ckv_pool=ckv, kpe_pool=kpe, kv_dtype=None, kv_scale=1.0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("block_size", [32, 16])
def test_fp8_wide_every_code_bit_exact(dtype, block_size):
    # One token: every head's output is the dequantized row, which holds
    # every finite code, so the widening and the dims of the transposing
    # read are checked exactly for all 64 heads.
    case = fp8_case(511, [1], 64, dtype, block_size=block_size)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    row = np.concatenate([codes, codes[::-1], codes[:4]])[:512]
    phys = case.block_table[0, 0]
    case.ckv_pool[phys, 0] = row
    case.kpe_pool[phys, 0] = codes[7:71]
    out, _, _, _ = run_wide(case, dict(force_partitions=1, force_splits=1))
    want = reference.decode_fp8_e4m3(row) * KV_SCALE
    for h in range(64):
        assert np.array_equal(out[0, h], want), (h, np.flatnonzero(out[0, h] != want)[:8])


IDENT = [
    (64, [1000], 32, "bf16", dict(force_partitions=2, force_splits=1)),
    (64, [77, 3001], 16, "f16", {}),
    (128, [5000, 33], 32, "f16", dict(force_partitions=3, force_splits=2)),
    (128, [32768], 16, "bf16", {}),
    (128, [1, 31, 32, 33], 32, "bf16", dict(force_partitions=1, force_splits=1)),
]


@pytest.mark.parametrize("heads,contexts,bs,dtype,prm", IDENT,
                         ids=[f"H{h}-{c}-bs{b}-{d}-{p}" for h, c, b, d, p in IDENT])
def test_fp8_wide_bit_identical_to_widened_16bit(heads, contexts, bs, dtype, prm):
    case = fp8_case(512 + len(contexts), contexts, heads, dtype, kv_scale=1.0, block_size=bs,
                    poison=True)
    log(f"[case] fp8 wide identity H={heads} {contexts} bs{bs} {dtype} {prm}")
    a = run_wide(case, prm)
    p16 = dict(prm, heads_per_wg=64)
    b = run_case(widened(case), mla.PlanParams(**p16))
    assert b[2].info["heads_per_wg"] == 64
    assert np.array_equal(a[0], b[0]), np.argwhere(a[0] != b[0])[:8]
    assert np.array_equal(a[1], b[1])


WORKLOADS = [
    ("v3_81k", {}, 32),
    ("v3_81k", {}, 16),
    ("v3_81k", dict(force_partitions=1, force_splits=1), 32),   # single pass
    ("mixed_b8", dict(workspace_limit_bytes=64 << 20), 32),
]


@pytest.mark.parametrize("name,prm,bs", WORKLOADS,
                         ids=[f"{n}-bs{b}-{'-'.join(f'{k}{v}' for k, v in p.items()) or 'chooser'}"
                              for n, p, b in WORKLOADS])
def test_fp8_wide_workloads(name, prm, bs):
    log(f"[case] fp8 wide workload {name} {prm} block {bs}")
    case = mla_synth.make_workload(name, kv_dtype="fp8_e4m3", kv_scale=KV_SCALE, poison=True,
                                   block_size=bs)
    check(case, prm, f"fp8 wide {name} {prm} bs{bs}")


EDGE = [
    ([1], 64, "f16", 32, {}),
    ([31, 32, 33], 128, "bf16", 32, {}),
    ([15, 16, 17, 47], 64, "f16", 16, dict(force_partitions=2)),
    ([0, 100, 0], 64, "f16", 32, dict(force_partitions=2)),
    ([33], 128, "bf16", 16, dict(force_partitions=8, force_splits=16)),   # many empty rows
    ([40, 5000], 128, "bf16", 32, dict(force_partitions=8, force_splits=3)),
    ([4097, 1, 300], 64, "bf16", 16, dict(num_cus=4096, min_tile_blocks=1)),
]


@pytest.mark.parametrize("contexts,heads,dtype,bs,prm", EDGE,
                         ids=[f"{c}-H{h}-{d}-bs{b}-{p}" for c, h, d, b, p in EDGE])
def test_fp8_wide_edge_cases(contexts, heads, dtype, bs, prm):
    log(f"[case] fp8 wide edge {contexts} H={heads} {dtype} bs{bs} {prm}")
    case = fp8_case(610 + sum(contexts) % 89, contexts, heads, dtype, block_size=bs, poison=True)
    check(case, prm, f"fp8 wide edge {contexts} H={heads} bs{bs} {prm}")


@pytest.mark.parametrize("bs,heads", [(32, 64), (16, 128)])
def test_fp8_wide_needles_at_row_boundaries(bs, heads):
    # A dominant token at the first and last position of every row: in a
    # row's later blocks it outgrows the first block's maximum by far more
    # than 2^15, so the workgroup takes the second pass.
    n = 3000
    prm = dict(force_partitions=3, force_splits=4)
    rows = oracle.row_ranges([n], [3], [4], block_size=bs)
    spots = sorted({lo for _, lo, hi in rows if hi > lo} | {hi - 1 for _, lo, hi in rows if hi > lo})
    for i, t in enumerate(spots):
        case = fp8_case(87, [n], heads, "bf16", block_size=bs, poison=True)
        h = (37 * i) % heads
        phys = case.block_table[0, t // bs]
        sign = np.sign(reference.decode16(case.q_absorbed[0, h], case.dtype))
        sign[sign == 0] = 1
        case.ckv_pool[phys, t % bs] = mla_synth.f32_to_fp8_e4m3_bits(6.0 * sign / KV_SCALE)
        case.kpe_pool[phys, t % bs] = 0
        needle = reference.decode_fp8_e4m3(case.ckv_pool[phys, t % bs]) * KV_SCALE
        out, _, _, _ = run_wide(case, prm)
        assert np.all(np.isfinite(out))
        assert np.max(np.abs(out[0, h] - needle)) < 1e-2, (t, h)


@pytest.mark.parametrize("heads,q_len,bs", [(64, 2, 32), (128, 2, 16)])
def test_fp8_wide_multitoken(heads, q_len, bs):
    case = mla_synth.make_case(seed=88, batch=2, heads=heads, contexts=[3000, 49], dtype="f16",
                               q_len=q_len, block_size=bs, kv_dtype="fp8_e4m3",
                               kv_scale=KV_SCALE, poison=True)
    check(case, {}, f"fp8 wide q_len={q_len} H={heads} bs{bs}")
    check(case, dict(force_partitions=2), f"fp8 wide q_len={q_len} H={heads} bs{bs} P=2")
