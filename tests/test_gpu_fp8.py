"""GPU parity of the partition kernel over latent caches stored as E4M3 bytes
with one scale (mla_decode_partition_fp8) against the f64 oracle, at the same
bounds as the 16-bit caches.

The byte format is E4M3 of the OCP 8-bit floating point specification; the
oracle decodes it from that definition (pinned on the CPU). Every E4M3 value
is exactly an fp16 and a bf16 value, so the kernel's widened tile holds the
cached values exactly and the scale is applied to the scores and the output.
Covered: every finite code through the kernel bit for bit (one token), the
workloads with 16-head workgroups (64-head ones are in test_gpu_fp8_wide.py),
16-token blocks, edge cases, needles, several new tokens per request, and the
host checks.
"""
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


def fp8_workload(name, **kw):
    return mla_synth.make_workload(name, kv_dtype="fp8_e4m3", kv_scale=KV_SCALE, **kw)


def fp8_small(seed, contexts, heads=16, dtype="f16", **kw):
    kw.setdefault("kv_scale", KV_SCALE)
    return mla_synth.make_case(seed=seed, batch=len(contexts), heads=heads, contexts=contexts,
                               dtype=dtype, kv_dtype="fp8_e4m3", **kw)


def run_fp8(case, prm):
    prm = dict(prm)
    prm.setdefault("heads_per_wg", 16)
    dev = to_device_fp8(case)
    out, lse2, plan, ranges = run_case(case, mla.PlanParams(**prm), dev=dev, want_ranges=True)
    return out, lse2, plan, ranges


def to_device_fp8(case):
    d = to_device(case)
    d["ckv_cache"] = torch.from_numpy(np.ascontiguousarray(case.ckv_pool)).cuda()
    d["kpe_cache"] = torch.from_numpy(np.ascontiguousarray(case.kpe_pool)).cuda()
    d["kv_scale"] = case.kv_scale
    return d


def check(case, prm, what):
    assert case.ckv_pool.dtype == np.uint8
    out, lse2, plan, ranges = run_fp8(case, prm)
    log(f"[plan] {what} P={plan.info['P']} S={plan.info['S']} rows={plan.total_rows}")
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, what, moments=mom)
    if plan.total_rows > case.batch:
        want = rows_of_plan(case, plan)
        got = [tuple(r) for r in ranges[:plan.total_rows]]
        assert got == [(lo, hi) for _, lo, hi in want]
    return out, lse2, plan


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("block_size", [32, 16])
def test_fp8_every_code_bit_exact(dtype, block_size):
    # One token: the output is its dequantized row. The row holds every
    # finite E4M3 code (and their order across the 16-byte loads), so the
    # byte format, the widening and the element order are checked exactly.
    case = fp8_small(501, [1], heads=16, dtype=dtype, block_size=block_size)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    row = np.concatenate([codes, codes[::-1], codes[:4]])[:512]
    phys = case.block_table[0, 0]
    case.ckv_pool[phys, 0] = row
    case.kpe_pool[phys, 0] = codes[100:164]
    out, lse2, plan, _ = run_fp8(case, dict(force_partitions=1, force_splits=1))
    want = reference.decode_fp8_e4m3(row) * KV_SCALE
    for h in range(16):
        assert np.array_equal(out[0, h], want), (h, np.flatnonzero(out[0, h] != want)[:8])


WORKLOADS = [
    ("tiny", dict(force_partitions=2, force_splits=1), 32),
    ("tiny", dict(force_partitions=2), 16),
    ("v2lite_32k", {}, 32),
    ("v2lite_32k", dict(force_partitions=1, force_splits=1), 32),
    ("v2lite_32k", {}, 16),
    ("two_req_32k_20k", {}, 32),
    ("v3_81k", {}, 32),                              # 128 heads as eight 16-head groups
    ("mixed_b8", dict(workspace_limit_bytes=64 << 20), 32),
]


@pytest.mark.parametrize("name,prm,bs", WORKLOADS,
                         ids=[f"{n}-bs{b}-{'-'.join(f'{k}{v}' for k, v in p.items()) or 'chooser'}"
                              for n, p, b in WORKLOADS])
def test_fp8_workloads(name, prm, bs):
    log(f"[case] fp8 workload {name} {prm} block {bs}")
    case = fp8_workload(name, poison=True, block_size=bs)
    _, _, plan = check(case, prm, f"fp8 {name} {prm} bs{bs}")
    if name == "v2lite_32k" and not prm:
        assert plan.info["P"] == [2]


EDGE = [
    ([1], 16, "f16", 32, {}),
    ([31, 32, 33], 16, "bf16", 32, {}),
    ([15, 16, 17, 47], 32, "f16", 16, dict(force_partitions=2)),
    ([0, 100, 0], 16, "f16", 32, dict(force_partitions=2)),
    ([33], 16, "bf16", 16, dict(force_partitions=8, force_splits=16)),
    ([40, 5000], 128, "bf16", 32, dict(force_partitions=8, force_splits=3)),
    ([4097, 1, 300], 64, "bf16", 16, dict(num_cus=4096, min_tile_blocks=1)),
]


@pytest.mark.parametrize("contexts,heads,dtype,bs,prm", EDGE,
                         ids=[f"{c}-H{h}-{d}-bs{b}-{p}" for c, h, d, b, p in EDGE])
def test_fp8_edge_cases(contexts, heads, dtype, bs, prm):
    log(f"[case] fp8 edge {contexts} H={heads} {dtype} bs{bs} {prm}")
    case = fp8_small(600 + sum(contexts) % 89, contexts, heads, dtype, block_size=bs,
                     poison=True)
    check(case, prm, f"fp8 edge {contexts} H={heads} bs{bs} {prm}")


@pytest.mark.parametrize("bs", [32, 16])
def test_fp8_needles_at_row_boundaries(bs):
    n = 3000
    prm = dict(force_partitions=3, force_splits=4)
    rows = oracle.row_ranges([n], [3], [4], block_size=bs)
    spots = sorted({lo for _, lo, hi in rows if hi > lo} | {hi - 1 for _, lo, hi in rows if hi > lo})
    for i, t in enumerate(spots):
        case = fp8_small(83, [n], 32, "bf16", block_size=bs, poison=True)
        h = (5 * i) % 32
        phys = case.block_table[0, t // bs]
        sign = np.sign(reference.decode16(case.q_absorbed[0, h], case.dtype))
        sign[sign == 0] = 1
        # 6.0 in the dequantized domain: code of 6 / scale = 192.
        case.ckv_pool[phys, t % bs] = mla_synth.f32_to_fp8_e4m3_bits(6.0 * sign / KV_SCALE)
        case.kpe_pool[phys, t % bs] = 0
        needle = reference.decode_fp8_e4m3(case.ckv_pool[phys, t % bs]) * KV_SCALE
        out, _, _, _ = run_fp8(case, prm)
        assert np.max(np.abs(out[0, h] - needle)) < 1e-2, (t, h)


@pytest.mark.parametrize("heads,q_len,bs", [(16, 2, 32), (32, 4, 16)])
def test_fp8_multitoken(heads, q_len, bs):
    case = mla_synth.make_case(seed=84, batch=2, heads=heads, contexts=[3000, 49], dtype="f16",
                               q_len=q_len, block_size=bs, kv_dtype="fp8_e4m3",
                               kv_scale=KV_SCALE, poison=True)
    check(case, {}, f"fp8 q_len={q_len} H={heads} bs{bs}")
    check(case, dict(force_partitions=2), f"fp8 q_len={q_len} H={heads} bs{bs} P=2")


def test_fp8_run_to_run_bit_identical():
    case = fp8_workload("two_req_32k_20k")
    a = run_fp8(case, {})
    b = run_fp8(case, {})
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fp8_host_checks():
    case = fp8_small(85, [100], heads=128)
    dev = to_device_fp8(case)
    out = torch.empty((1, 128, 512), dtype=torch.float16, device="cuda")
    plan16 = mla.DecodePlan(case.context_lens, 128, mla.PlanParams(force_partitions=2,
                                                                   heads_per_wg=16))
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(mla.MlaError) as e:
            mla.decode(plan16, dev["q_absorbed"], dev["q_pe"], dev["ckv_cache"],
                       dev["kpe_cache"], dev["block_table"], dev["context_lens"], case.scale,
                       out, kv_scale=bad)
        assert e.value.status == -3
    with pytest.raises(mla.MlaError):
        mla.decode(plan16, dev["q_absorbed"], dev["q_pe"], dev["ckv_cache"], dev["kpe_cache"],
                   dev["block_table"], dev["context_lens"], case.scale, out, fused=True,
                   kv_scale=KV_SCALE)
