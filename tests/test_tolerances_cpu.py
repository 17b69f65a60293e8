"""The GPU acceptance check itself, on the CPU: at the 131072-token V3 shape
it must reject an answer that lost one interior 32-token block, and accept
the true answer rounded as the GPU rounds it (bf16 output, fp32 LSE).

The wrong answers are built with the oracle's own split and merge (vllm-metal
pull request 601, "What changed": partials over slices of the context merged
by their LSEs): the context minus block k, as the partials over [0, 32 k)
and [32 (k + 1), n) merged in base 2. Eight heads keep the f64 work short.
"""
import numpy as np
import pytest

import mla_synth
import oracle
from oracle import reference

from gpu_helpers import compare

HEADS = np.arange(0, 128, 16)


@pytest.fixture(scope="module")
def v3_case():
    case = mla_synth.make_workload("v3_131k")
    ref, lref, w1, w2 = oracle.latent_f64(case, heads=HEADS, moments=True)
    return case, ref, lref, (w1, w2)


def as_gpu(case, out, lse2):
    """Round as the library returns results: 16-bit output, fp32 LSE."""
    o = reference.decode16(mla_synth.encode16(np.nan_to_num(out).astype(np.float32), case.dtype),
                           case.dtype)
    o = np.where(np.isnan(out), np.nan, o)
    return o, lse2.astype(np.float32).astype(np.float64)


def without_block(case, k):
    n = int(case.context_lens[0])
    lo_o, lo_l = reference.latent_one(case, 0, HEADS, 0, 32 * k)
    hi_o, hi_l = reference.latent_one(case, 0, HEADS, 32 * (k + 1), n)
    o, l = reference.merge_log2_f64(np.stack([lo_o, hi_o]), np.stack([lo_l, hi_l]), [0, 2])
    out = np.full((1, 128, 512), np.nan)
    lse = np.full((1, 128), np.nan)
    out[0, HEADS] = o[0]
    lse[0, HEADS] = l[0]
    return out, lse


def test_true_answer_rounded_is_accepted(v3_case):
    case, ref, lref, mom = v3_case
    out, lse2 = as_gpu(case, ref, lref)
    compare(case, out, lse2, ref, lref, "true answer, rounded", moments=mom)


@pytest.mark.parametrize("k", [1000, 2048, 3500])
def test_dropped_interior_block_is_rejected(v3_case, k):
    case, ref, lref, mom = v3_case
    out, lse2 = as_gpu(case, *without_block(case, k))
    with pytest.raises(AssertionError):
        compare(case, out, lse2, ref, lref, f"block {k} dropped", moments=mom)
