"""GPU parity of the per-head products on either side of absorbed decode
(mla_absorb_query, mla_unabsorb_output) against the oracle's f64 folds, and
of the three GPU steps together (fold, decode, unfold) against the
pre-absorption oracle (decompressed keys and values through W_UK / W_UV^T).

Bound for one product (derived from the arithmetic): the inputs are exact
16-bit values, the sum runs in fp32 (at most 512 terms, relative error well
under 1e-5 of sum |x w|), and the result is rounded once, so
|gpu - ref| <= u |ref| + 1e-4 with u the unit roundoff of the output type
(2^-11 fp16, 2^-8 bf16).
"""
import numpy as np
import pytest

import absorbed_mla_paged_amd as mla
import mla_synth
import oracle
from oracle import reference

from gpu_helpers import log, run_case, to_device, torch_dtype

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def draw(rng, shape, dtype, scale=1.0):
    bits = mla_synth.encode16((rng.standard_normal(shape) * scale).astype(np.float32), dtype)
    return bits, reference.decode16(bits, dtype)


def dev16(bits, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch_dtype(dtype)).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("rows,heads", [(1, 16), (3, 16), (8, 128), (13, 128), (2, 48), (17, 128), (40, 16)])
def test_fold_and_unfold_match_oracle(dtype, rows, heads):
    import torch
    rng = np.random.default_rng(rows * 1000 + heads)
    qn_b, qn = draw(rng, (rows, heads, 128), dtype)
    wk_b, wk = draw(rng, (heads, 128, 512), dtype, 1 / np.sqrt(128))
    ol_b, ol = draw(rng, (rows, heads, 512), dtype)
    wv_b, wv = draw(rng, (heads, 512, 128), dtype, 1 / np.sqrt(512))
    qa = torch.empty((rows, heads, 512), dtype=torch_dtype(dtype), device="cuda")
    o = torch.empty((rows, heads, 128), dtype=torch_dtype(dtype), device="cuda")
    mla.mla_absorb_query(dev16(qn_b, dtype), dev16(wk_b, dtype), qa)
    mla.mla_unabsorb_output(dev16(ol_b, dtype), dev16(wv_b, dtype), o)
    torch.cuda.synchronize()
    for name, got, ref in (("fold", host(qa), oracle.absorb_query(qn, wk)),
                           ("unfold", host(o), oracle.unabsorb_output(ol, wv))):
        err = np.abs(got - ref)
        log(f"[project] {name} rows={rows} H={heads} {dtype}: max {err.max():.3e} "
            f"mean {err.mean():.3e} (|ref| max {np.abs(ref).max():.2f})")
        assert np.all(err <= U[dtype] * np.abs(ref) + 1e-4), name
    # Fixed summation order: bit-identical when run again.
    qa2 = torch.empty_like(qa)
    mla.mla_absorb_query(dev16(qn_b, dtype), dev16(wk_b, dtype), qa2)
    torch.cuda.synchronize()
    assert torch.equal(qa, qa2)


def test_empty_rows_launch_nothing():
    import torch
    x = torch.empty((0, 16, 128), dtype=torch.float16, device="cuda")
    w = torch.zeros((16, 128, 512), dtype=torch.float16, device="cuda")
    y = torch.empty((0, 16, 512), dtype=torch.float16, device="cuda")
    mla.mla_absorb_query(x, w, y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,q_len", [("f16", 1), ("bf16", 2)])
def test_fold_decode_unfold_matches_pre_absorption(dtype, q_len):
    # q_nope -> q_absorbed (GPU fold) -> absorbed decode (GPU) -> o (GPU
    # unfold), against ordinary attention over decompressed keys W_UK ckv and
    # values W_UV^T ckv in f64 (mlxcel pull request 995, "Verified vs
    # unverified": a host f64 reference that performs the pre-absorption
    # computation). For q_len = 2 the pre-absorption reference runs once per
    # new token with its visible context.
    import torch
    H, n = 16, 3000
    case = mla_synth.make_case(seed=971, batch=1, heads=H, contexts=[n], dtype=dtype,
                               q_len=q_len)
    rng = np.random.default_rng(5)
    qn_b, qn = draw(rng, (q_len, H, 128), dtype)           # rows = new tokens
    wk_b, wk = draw(rng, (H, 128, 512), dtype, 1 / np.sqrt(128))
    wv_b, wv = draw(rng, (H, 512, 128), dtype, 4 / np.sqrt(512))
    qa = torch.empty((q_len, H, 512), dtype=torch_dtype(dtype), device="cuda")
    mla.mla_absorb_query(dev16(qn_b, dtype), dev16(wk_b, dtype), qa)
    torch.cuda.synchronize()
    case.q_absorbed = qa.cpu().view(torch.int16).numpy().view(np.uint16).reshape(1, q_len * H, 512)
    dev = to_device(case)
    plan = mla.DecodePlan(case.context_lens, H, mla.PlanParams(force_partitions=2), q_len=q_len)
    out = torch.empty((1, q_len * H, 512), dtype=torch_dtype(dtype), device="cuda")
    mla.decode(plan, dev["q_absorbed"], dev["q_pe"], dev["ckv_cache"], dev["kpe_cache"],
               dev["block_table"], dev["context_lens"], case.scale, out)
    o = torch.empty((q_len, H, 128), dtype=torch_dtype(dtype), device="cuda")
    mla.mla_unabsorb_output(out.view(q_len, H, 512), dev16(wv_b, dtype), o)
    torch.cuda.synchronize()
    got = host(o)
    ref = np.empty_like(got)
    for j in range(q_len):
        one = mla_synth.make_case(seed=971, batch=1, heads=H, contexts=[n], dtype=dtype,
                                  q_len=q_len)
        one.q_pe = one.q_pe[:, j * H:(j + 1) * H]
        one.q_len = 1
        one.context_lens = np.array([reference.visible_len(n, q_len, j)], dtype=np.int32)
        o_dec, _ = oracle.decompressed_f64(one, qn[j][None], wk, wv)
        ref[j] = o_dec[0]
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    log(f"[project] fold-decode-unfold {dtype} q_len={q_len}: rel L2 {rel:.3e}, "
        f"max {np.abs(got - ref).max():.3e} (|ref| max {np.abs(ref).max():.3f})")
    assert rel < 1e-2
