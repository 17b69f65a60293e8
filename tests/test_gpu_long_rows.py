"""GPU checks that see every interior block of long rows, at full size.

The N(0,1) parity bounds cannot, on their own, see one dropped 32-token
block among 131072 tokens: it moves the output by about 1e-4 and the LSE by
3.5e-4. Two checks here can:

* Uniform scores. With q_absorbed = q_pe = 0 every score is exactly 0, so
  every weight is exactly 1 (exp2(0) in any precision). The answer then has
  a plain closed form (mlxcel pull request 995, "What changed", Stage 1: a
  softmax over all visible tokens with the latent rows as values): the
  output is the mean of the visible ckv rows and lse2 = log2(n). The mean
  is computed here directly, in f64, from the stored 16-bit rows; the only
  rounding left on the GPU side is the fp32 sums and one rounding of the
  output, so |out - mean| <= half an output ulp + 2e-6 and
  |lse2 - log2 n| <= 1e-5. A dropped block moves lse2 by 3.5e-4 at 131072
  tokens (35x the bound) and the output by several ulps.
* Interior needles. One dominant token per probed head (its ckv row is
  6 * sign(q_absorbed[h]), its kpe row 0), placed inside rows, inside
  ring slots / stages of every residue, and on the last token of rows, in
  one launch of the full-size workload: the probed head's output must be
  that row, and every head must match the oracle beyond output rounding.

Both checks also run at full size with 16-token cache blocks and with E4M3
byte caches (the mean is then of the decoded bytes times the cache scale),
in the 16-head and the 64-head kernel.
"""
import numpy as np
import pytest

import absorbed_mla_paged_amd as mla
import mla_synth
import oracle
from oracle import reference

from gpu_helpers import compare_beyond_rounding, half_ulp, log, run_case, to_device

pytestmark = pytest.mark.gpu


def visible_mean(case, b):
    """Mean of the visible ckv rows of request b, in f64, from the stored
    16-bit values or E4M3 bytes times the cache scale (chunks of 256
    blocks)."""
    n = int(case.context_lens[b])
    bs = int(case.ckv_pool.shape[1])
    total = np.zeros(512)
    for t0 in range(0, n, 256 * bs):
        t = np.arange(t0, min(n, t0 + 256 * bs))
        rows = case.ckv_pool[case.block_table[b][t // bs], t % bs]
        if case.kv_dtype == "fp8_e4m3":
            total += reference.decode_fp8_e4m3(rows).sum(axis=0) * case.kv_scale
        else:
            total += reference.decode16(rows, case.dtype).sum(axis=0)
    return total / n


def device_inputs(case):
    """Device tensors of a case; E4M3 caches go up as their bytes."""
    import torch
    dev = to_device(case)
    if case.kv_dtype == "fp8_e4m3":
        dev["ckv_cache"] = torch.from_numpy(np.ascontiguousarray(case.ckv_pool)).cuda()
        dev["kpe_cache"] = torch.from_numpy(np.ascontiguousarray(case.kpe_pool)).cuda()
        dev["kv_scale"] = case.kv_scale
    return dev


# (workload, plan parameters, cache layout): the 16-bit caches in 32-token
# blocks, and at full size also 16-token blocks and E4M3 bytes, in both
# kernels (16 heads at V2-Lite, 64-head workgroups at V3).
FP8 = dict(kv_dtype="fp8_e4m3", kv_scale=2.0 ** -5)
UNIFORM = [
    ("v2lite_32k", {}, {}),
    ("v2lite_32k", dict(force_partitions=1, force_splits=1), {}),   # single pass, direct write
    ("two_req_32k_20k", {}, {}),
    ("v3_81k", {}, {}),
    ("v3_131k", {}, {}),
    ("mixed_b8", dict(workspace_limit_bytes=64 << 20), {}),
    ("v3_131k", {}, dict(block_size=16)),
    ("v2lite_32k", {}, FP8),
    ("v3_131k", {}, FP8),
]


def case_id(name, prm, layout):
    parts = [f"{k}{v}" for k, v in prm.items()]
    if layout.get("block_size"):
        parts.append(f"bs{layout['block_size']}")
    if layout.get("kv_dtype"):
        parts.append("e4m3")
    return f"{name}-{'-'.join(parts) or 'chooser'}"


@pytest.mark.parametrize("name,prm,layout", UNIFORM, ids=[case_id(*u) for u in UNIFORM])
def test_uniform_scores_closed_form(name, prm, layout):
    log(f"[case] uniform scores {name} {prm} {layout}")
    case = mla_synth.make_workload(name, poison=True, **layout)
    case.q_absorbed[...] = 0
    case.q_pe[...] = 0
    out, lse2, plan, _ = run_case(case, mla.PlanParams(**prm), dev=device_inputs(case))
    log(f"[plan] P={plan.info['P']} S={plan.info['S']} rows={plan.total_rows}")
    assert np.all(np.isfinite(out))
    for b in range(case.batch):
        n = int(case.context_lens[b])
        mean = visible_mean(case, b)
        bound = half_ulp(np.maximum(np.abs(mean)[None, :], np.abs(out[b])), case.dtype) + 2e-6
        err = np.abs(out[b] - mean[None, :])
        dl = np.abs(lse2[b] - np.log2(n))
        log(f"[uniform] {case_id(name, prm, layout)} b={b} n={n}: out err max {err.max():.3e} "
            f"(over bound {np.max(err / bound):.3f}), lse2 err max {dl.max():.3e}")
        assert np.all(err <= bound), (b, float(np.max(err / bound)))
        assert np.all(dl <= 1e-5), (b, float(dl.max()))


def plant(case, b, t, h):
    """Token t of request b becomes a needle for head h: its ckv row is
    6 * sign(q_absorbed[h]), its kpe row 0 (E4M3 caches: the codes of those
    values over the cache scale, 192 being exact). Returns the row's value."""
    bs = int(case.ckv_pool.shape[1])
    phys = case.block_table[b, t // bs]
    sign = np.sign(reference.decode16(case.q_absorbed[b, h], case.dtype))
    sign[sign == 0] = 1
    row = (6.0 * sign).astype(np.float32)
    if case.kv_dtype == "fp8_e4m3":
        case.ckv_pool[phys, t % bs] = mla_synth.f32_to_fp8_e4m3_bits(row / case.kv_scale)
        case.kpe_pool[phys, t % bs] = mla_synth.f32_to_fp8_e4m3_bits(np.zeros(64))
        return reference.decode_fp8_e4m3(case.ckv_pool[phys, t % bs]) * case.kv_scale
    case.ckv_pool[phys, t % bs] = mla_synth.encode16(row, case.dtype)
    case.kpe_pool[phys, t % bs] = mla_synth.encode16(np.zeros(64, np.float32), case.dtype)
    return reference.decode16(case.ckv_pool[phys, t % bs], case.dtype)


def interior_spots(ranges, rng, per_row, seg):
    """Token positions inside rows: for a sample of rows, tokens in the
    row's first segments (every residue of a 4-slot ring / 2-segment stage),
    its middle, and its last token; plus random interior tokens."""
    spots = []
    rows = [r for r in ranges if r[2] > r[1]]
    pick = sorted(set([0, len(rows) // 3, len(rows) // 2, len(rows) - 1] +
                      list(rng.choice(len(rows), size=min(len(rows), per_row), replace=False))))
    for i in pick:
        b, lo, hi = rows[i]
        n_seg = (hi - lo + seg - 1) // seg
        for k, j in ((1, 5), (2, 17), (3, 31), (n_seg // 2, 9), (n_seg // 2 + 1, 30)):
            t = lo + k * seg + j
            if t < hi:
                spots.append((b, t))
        spots.append((b, hi - 1))
    return sorted(set(spots))


NEEDLES = [("v3_131k", {}, 48, {}), ("v3_81k", {}, 32, {}),
           ("mixed_b8", dict(workspace_limit_bytes=64 << 20), 48, {}),
           ("v2lite_32k", {}, 16, {}), ("two_req_32k_32k", {}, 16, {}),
           ("v3_131k", {}, 48, dict(block_size=16)), ("v3_131k", {}, 48, FP8),
           ("v2lite_32k", {}, 16, FP8)]


@pytest.mark.parametrize("name,prm,count,layout", NEEDLES,
                         ids=[case_id(n, {}, lay) for n, _, _, lay in NEEDLES])
def test_interior_needles_full_size(name, prm, count, layout):
    log(f"[case] interior needles {name} {prm} {layout}")
    case = mla_synth.make_workload(name, poison=True, **layout)
    bs = int(case.ckv_pool.shape[1])
    plan = mla.mla_choose_partitions(case.batch, case.heads, 1, case.context_lens,
                                     mla.PlanParams(**prm), block_size=bs)
    ranges = oracle.row_ranges(case.context_lens, plan["P"], plan["S"], block_size=bs)
    rng = np.random.default_rng(17)
    spots = interior_spots(ranges, rng, 8, 32)
    rng.shuffle(spots)
    # One needle per (request, head): heads are dealt round-robin per request.
    used = {}
    planted = []
    for b, t in spots:
        h = used.get(b, 0)
        if h >= case.heads or len(planted) >= count:
            continue
        used[b] = h + 1
        h = (h * 37) % case.heads
        planted.append((b, t, h, plant(case, b, t, h)))
    log(f"[needles] {len(planted)} planted, e.g. {[(b, t, h) for b, t, h, _ in planted[:6]]}")
    out, lse2, gplan, _ = run_case(case, mla.PlanParams(**prm), dev=device_inputs(case))
    assert gplan.info["P"] == plan["P"] and gplan.info["S"] == plan["S"]
    for b, t, h, row in planted:
        assert np.max(np.abs(out[b, h] - row)) < 1e-2, (b, t, h)
    ref, lref = oracle.latent_f64(case)
    compare_beyond_rounding(case, out, lse2, ref, lref, f"needles {name}")
