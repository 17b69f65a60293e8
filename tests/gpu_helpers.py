"""Shared helpers of the GPU parity tests: upload a case, run the library,
compare with the f64 oracle at the stated tolerances."""
from __future__ import annotations

import math
import sys

import numpy as np

import absorbed_mla_paged_amd as mla
import oracle

# Acceptance bounds on the latent output (fp16/bf16 inputs, fp32 accumulate).
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
# Relative L2 error of the whole output against the oracle's: bf16 output
# rounding alone is about 2^-9 / sqrt(3); a dropped 32-token block at
# 131072 tokens moves it past 1e-2.
REL_L2 = 1e-2
# Unit roundoff of the 16-bit types the weights are rounded to.
UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
LOG2E = 1.4426950408889634
# Worst-case LSE bound derived from the arithmetic: the weights are rounded
# to the 16-bit type before they are summed, a relative error of at most u
# per weight, so |d log2 l| <= log2(e) * u; plus fp32 slack.
LSE_SLACK = 2e-5
LSE_TOL = {k: LOG2E * u + LSE_SLACK for k, u in UNIT.items()}


def lse_bound(dtype: str, w1=None, w2=None):
    """Per-row LSE bound. With the oracle's weight moments (w1 = sum w,
    w2 = sum w^2, w = exp(s - max s)): the rounding errors of the weights
    are independent, each uniform within +-u relative, so the error of
    log(sum w) has standard deviation (u / sqrt 3) * sqrt(w2) / w1; six of
    those, never more than the worst case log2(e) * u, plus fp32 slack. At
    131072 near-uniform weights this is ~8e-5 for bf16, below the 3.5e-4 a
    dropped 32-token block moves the LSE by."""
    u = UNIT[dtype]
    if w1 is None:
        return LSE_TOL[dtype]
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        stat = LOG2E * 6.0 * (u / math.sqrt(3.0)) * np.sqrt(w2) / w1
    stat = np.where(np.isfinite(stat), stat, LOG2E * u)
    return np.minimum(stat, LOG2E * u) + LSE_SLACK


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def torch_dtype(dtype: str):
    import torch
    return torch.float16 if dtype == "f16" else torch.bfloat16


def to_device(case, device="cuda"):
    import torch
    td = torch_dtype(case.dtype)

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(td).to(device)
    return dict(
        q_absorbed=t16(case.q_absorbed), q_pe=t16(case.q_pe), ckv_cache=t16(case.ckv_pool),
        kpe_cache=t16(case.kpe_pool),
        block_table=torch.from_numpy(np.ascontiguousarray(case.block_table)).to(device),
        context_lens=torch.from_numpy(np.ascontiguousarray(case.context_lens)).to(device))


def run_case(case, params: mla.PlanParams | None = None, dev=None, want_ranges=False,
             fused=False):
    """Plan on the host, decode on the GPU; returns (out f64, lse2 f64, plan, ranges)."""
    import torch
    dev = dev or to_device(case)
    q_len = int(getattr(case, "q_len", 1))
    plan = mla.DecodePlan(case.context_lens, case.heads, params, q_len=q_len,
                          block_size=int(getattr(case, "block_size", 32)))
    rows = q_len * case.heads
    out = torch.empty((case.batch, rows, 512), dtype=torch_dtype(case.dtype), device="cuda")
    lse2 = torch.empty((case.batch, rows), dtype=torch.float32, device="cuda")
    ranges = None
    if want_ranges:
        ranges = torch.full((max(1, plan.total_rows), 2), -7, dtype=torch.int32, device="cuda")
    mla.decode(plan, dev["q_absorbed"], dev["q_pe"], dev["ckv_cache"], dev["kpe_cache"],
               dev["block_table"], dev["context_lens"], case.scale, out, lse2,
               debug_ranges=ranges, fused=fused, kv_scale=dev.get("kv_scale"))
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse2.cpu().numpy().astype(np.float64)
    r = ranges.cpu().numpy() if ranges is not None else None
    return o, l, plan, r


def compare(case, out, lse2, ref, lref, what="", moments=None):
    """Assert the acceptance bounds; return the error summary. `moments` is
    (w1, w2) from oracle.latent_f64(..., moments=True): with it the LSE bound
    shrinks with the number of tokens that carry the softmax (lse_bound)."""
    sel = ~np.isnan(lref)
    d = np.abs(out - ref)[sel]
    finite = np.isfinite(lref) & sel
    dl = np.abs(lse2[finite] - lref[finite])
    if moments is not None:
        tol = lse_bound(case.dtype, moments[0][finite], moments[1][finite])
    else:
        tol = np.full(dl.shape, LSE_TOL[case.dtype])
    rel = float(np.linalg.norm(d) / max(1e-30, np.linalg.norm(ref[sel])))
    summary = dict(max_abs=float(d.max()) if d.size else 0.0,
                   mean_abs=float(d.mean()) if d.size else 0.0,
                   rel_l2=rel, lse_max=float(dl.max()) if dl.size else 0.0,
                   lse_over_bound=float((dl / tol).max()) if dl.size else 0.0)
    log(f"[parity] {what} {summary}")
    assert np.all(np.isfinite(out[sel])), f"{what}: non-finite output"
    assert summary["max_abs"] <= MAX_ABS, (what, summary)
    assert summary["mean_abs"] <= MEAN_ABS, (what, summary)
    assert summary["rel_l2"] <= REL_L2, (what, summary)
    assert np.all(dl <= tol), (what, summary)
    # Requests with nothing visible: zeros and -inf exactly.
    for b in range(case.batch):
        if int(case.context_lens[b]) == 0:
            assert np.all(out[b] == 0) and np.all(lse2[b] == -np.inf)
    return summary


def half_ulp(x, dtype):
    """Half a unit in the last place of |x| in the 16-bit output type
    (normal range; fp16 subnormals and bf16 values below 2^-126 share the
    smallest normal's spacing)."""
    mant = 10 if dtype == "f16" else 7
    emin = -14 if dtype == "f16" else -126
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin)))
    return 0.5 * 2.0 ** (e - mant)


def compare_beyond_rounding(case, out, lse2, ref, lref, what):
    """Bounds for outputs that dominant tokens (needles with +-6 latent
    values) push far past N(0,1) size: rounding such an output to the
    16-bit type alone costs up to half an ulp (1.6e-2 at 6 in bf16), more
    than the 1e-2 meant for N(0,1)-sized outputs. The error beyond that
    rounding is held to the same thresholds."""
    sel = ~np.isnan(lref)
    excess = np.maximum(0.0, np.abs(out - ref) - half_ulp(ref, case.dtype))[sel]
    log(f"[parity] {what} excess max {excess.max():.3e} mean {excess.mean():.3e} "
        f"raw max {np.abs(out - ref)[sel].max():.3e}")
    assert np.all(np.isfinite(out)), what
    assert excess.max() <= 1e-2 and excess.mean() <= 1e-3, what
    finite = np.isfinite(lref) & sel
    assert np.max(np.abs(lse2 - lref)[finite]) <= LSE_TOL[case.dtype], what


def sync_records(plan):
    """The fused hand-off records of a plan: [batch, 8 head groups, 8] uint64."""
    return plan.sync.cpu().numpy().view(np.uint64).reshape(-1, 8, 8)


def check_sync_quiet(plan, what=""):
    """After a completed fused call: started == its base, arrived == its base,
    no wait ran out."""
    rec = sync_records(plan)
    assert np.all(rec[..., 1] == rec[..., 0]), (what, rec[..., :4])
    assert np.all(rec[..., 3] == rec[..., 2]), (what, rec[..., :4])
    assert np.all(rec[..., 4] == 0), (what, "waits ran out", rec[..., 4])


def rows_of_plan(case, plan):
    return oracle.row_ranges(case.context_lens, plan.info["P"], plan.info["S"],
                             block_size=int(getattr(case, "block_size", 32)))


def device_cus() -> int:
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def expected_lse_finite(case):
    return [int(n) > 0 for n in case.context_lens]


def fmt(x):
    return f"{x:.3e}" if isinstance(x, float) and not math.isnan(x) else str(x)
