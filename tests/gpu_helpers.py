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
# LSE bound derived from the arithmetic: the weights are rounded to the
# 16-bit type before they are summed, a relative error of at most u per
# weight, so |d log2 l| <= log2(e) * u; plus fp32 slack.
LSE_TOL = {"f16": 1.4427 * 2.0 ** -11 + 2e-5, "bf16": 1.4427 * 2.0 ** -8 + 2e-5}


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


def compare(case, out, lse2, ref, lref, what=""):
    """Assert the acceptance bounds; return the error summary."""
    sel = ~np.isnan(lref)
    d = np.abs(out - ref)[sel]
    finite = np.isfinite(lref) & sel
    dl = np.abs(lse2[finite] - lref[finite])
    rel = float(np.linalg.norm(d) / max(1e-30, np.linalg.norm(ref[sel])))
    summary = dict(max_abs=float(d.max()) if d.size else 0.0,
                   mean_abs=float(d.mean()) if d.size else 0.0,
                   rel_l2=rel, lse_max=float(dl.max()) if dl.size else 0.0)
    log(f"[parity] {what} {summary}")
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    assert summary["max_abs"] <= MAX_ABS, (what, summary)
    assert summary["mean_abs"] <= MEAN_ABS, (what, summary)
    assert summary["lse_max"] <= LSE_TOL[case.dtype], (what, summary)
    # Requests with nothing visible: zeros and -inf exactly.
    for b in range(case.batch):
        if int(case.context_lens[b]) == 0:
            assert np.all(out[b] == 0) and np.all(lse2[b] == -np.inf)
    return summary


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
