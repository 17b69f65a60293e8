"""Pins of the f64 oracle against things other than itself (CPU only).

Each test names the passage it follows. Pins used: 50-digit brute force,
closed forms (one token, uniform scores), needles, layout invariance,
split/merge invariance, the absorption identity, the log2-vs-ln negative
control, and the pages' printed byte counts. A last test plants plausible
mistakes in a copy of the oracle and checks that some pin catches each.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest

import mla_synth
import oracle
from oracle import brute, reference

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_case(seed, contexts, heads=2, dtype="f16", **kw):
    return mla_synth.make_case(seed=seed, batch=len(contexts), heads=heads,
                               contexts=contexts, dtype=dtype, **kw)


def _brute_errors(case, b, h, out, lse2):
    bo, bl = brute.latent_brute(case, b, h)
    bo = np.array([float(x) for x in bo])
    return np.max(np.abs(out[b, h] - bo)), abs(lse2[b, h] - float(bl))


# --- P7: brute force on tiny inputs --------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("contexts", [[1], [31], [32, 33], [70, 5]])
def test_latent_matches_brute_force(dtype, contexts):
    # mlxcel pull request 995, "What changed", Stage 1: score
    # scale*(q_abs.ckv + q_pe.kpe), values ckv, softmax over the context.
    case = small_case(11 + len(contexts) + contexts[0], contexts, dtype=dtype,
                      poison=True)
    out, lse2 = oracle.latent_f64(case)
    for b in range(case.batch):
        for h in range(case.heads):
            eo, el = _brute_errors(case, b, h, out, lse2)
            assert eo < 1e-12 and el < 1e-12, (b, h, eo, el)


def test_decompressed_matches_brute_force():
    # mlxcel pull request 995, "Verified vs unverified": a host f64 reference
    # that performs the pre-absorption computation. Small nope/value widths
    # keep the 50-digit loops short; the identity does not depend on them.
    case = small_case(21, [37], heads=2, dtype="bf16")
    rng = np.random.default_rng(5)
    dn, dv = 8, 6
    q_nope = rng.standard_normal((1, 2, dn))
    W_UK = rng.standard_normal((2, dn, 512)) / 16
    W_UV_T = rng.standard_normal((2, 512, dv)) / 16
    o, l = oracle.decompressed_f64(case, q_nope, W_UK, W_UV_T)
    for h in range(2):
        bo, bl = brute.decompressed_brute(case, 0, h, q_nope[0, h], W_UK[h], W_UV_T[h])
        assert np.max(np.abs(o[0, h] - np.array([float(x) for x in bo]))) < 1e-12
        assert abs(l[0, h] - float(bl)) < 1e-12


# --- P8: the absorption identity ------------------------------------------

@pytest.mark.parametrize("contexts,heads", [([45], 2), ([300, 1], 4)])
def test_absorption_identity(contexts, heads):
    # mlxcel pull request 995, "What changed", absorb.rs: q_nope.(W_UK ckv) =
    # (q_nope W_UK).ckv and o = (sum p ckv) W_UV^T, so the latent path through
    # the folded weights equals the decompressed path (DeepSeek geometry:
    # qk_nope = v_head = 128).
    case = small_case(31 + heads, contexts, heads=heads, dtype="f16")
    rng = np.random.default_rng(7)
    q_nope = rng.standard_normal((case.batch, heads, 128))
    W_UK = rng.standard_normal((heads, 128, 512)) / 22
    W_UV_T = rng.standard_normal((heads, 512, 128)) / 22
    o_dec, l_dec = oracle.decompressed_f64(case, q_nope, W_UK, W_UV_T)
    qa = oracle.absorb_query(q_nope, W_UK)
    qp = reference.decode16(case.q_pe, case.dtype)
    for b in range(case.batch):
        C, Kp = oracle.gather_request(case.ckv_pool, case.kpe_pool, case.block_table[b],
                                      int(case.context_lens[b]), case.dtype)
        o_lat, l_lat = reference._attend(qa[b], qp[b], C, Kp, case.scale)[:2]
        o_back = oracle.unabsorb_output(o_lat[None], W_UV_T)[0]
        assert np.max(np.abs(o_back - o_dec[b])) < 1e-12
        assert np.max(np.abs(l_lat - l_dec[b])) < 1e-12


def test_square_orthogonal_pre_absorption_mode():
    # With square orthogonal folds the pre-absorption path runs at the full
    # 512-wide latent and maps back by a transpose; it must equal latent_f64.
    case = small_case(41, [777, 64], heads=3, dtype="bf16")
    W_UK, W_UV_T = oracle.orthogonal_weights(99, case.heads)
    qa = reference.decode16(case.q_absorbed, case.dtype)
    q_nope = np.einsum("bhr,hdr->bhd", qa, W_UK)          # q_abs W_UK^T
    o, l = oracle.decompressed_f64(case, q_nope, W_UK, W_UV_T)
    o_lat = np.einsum("bhv,hrv->bhr", o, W_UV_T)           # o (W_UV^T)^T
    ref, lref = oracle.latent_f64(case)
    assert np.max(np.abs(o_lat - ref)) < 1e-11
    assert np.max(np.abs(l - lref)) < 1e-11


# --- P1 / P2: closed forms ------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_single_token_closed_form(dtype):
    # One visible token: its weight is exactly 1, out = ckv_0, and
    # lse2 = s_0 / ln 2.
    case = small_case(51, [1, 1], heads=4, dtype=dtype, poison=True)
    out, lse2 = oracle.latent_f64(case)
    for b in range(2):
        phys = case.block_table[b, 0]
        c = reference.decode16(case.ckv_pool[phys, 0], dtype)
        k = reference.decode16(case.kpe_pool[phys, 0], dtype)
        for h in range(4):
            assert np.array_equal(out[b, h], c)
            qa = reference.decode16(case.q_absorbed[b, h], dtype)
            qp = reference.decode16(case.q_pe[b, h], dtype)
            s0 = case.scale * (math.fsum(qa * c) + math.fsum(qp * k))
            assert abs(lse2[b, h] - s0 * oracle.LOG2_E) < 1e-13


@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 64, 100, 1024])
def test_uniform_scores_closed_form(n):
    # q = 0 makes every score 0: out is the plain mean of the visible rows
    # and lse2 = log2 n. Exactly which rows are read shows in the mean.
    case = small_case(61 + n, [n], heads=2, dtype="bf16", poison=True)
    case.q_absorbed[:] = 0
    case.q_pe[:] = 0
    out, lse2 = oracle.latent_f64(case)
    rows = np.stack([reference.decode16(case.ckv_pool[case.block_table[0, t // 32], t % 32],
                                        "bf16") for t in range(n)])
    mean = rows.sum(axis=0) / n
    assert np.max(np.abs(out[0] - mean[None])) < 1e-13
    assert np.all(np.abs(lse2[0] - math.log2(n)) < 1e-13)
    if n & (n - 1) == 0:
        assert np.all(lse2[0] == math.log2(n))


def test_empty_context():
    # No visible token: zero output and lse2 = -inf, never NaN (MTPLX pull
    # request 639, commit on rows without a visible key).
    case = small_case(71, [0, 40], heads=2)
    out, lse2 = oracle.latent_f64(case)
    assert np.all(out[0] == 0) and np.all(lse2[0] == -np.inf)
    assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(lse2[1]))


# --- weight moments (they size the GPU acceptance's LSE bound) ----------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("contexts", [[1], [33], [70, 5]])
def test_weight_moments_match_brute_force(dtype, contexts):
    # sum_t w_t and sum_t w_t^2 with w_t = exp(s_t - max s), by 50-digit
    # scalar loops that find the maximum first.
    case = small_case(41 + contexts[0], contexts, dtype=dtype, poison=True)
    _, _, w1, w2 = oracle.latent_f64(case, moments=True)
    for b in range(case.batch):
        for h in range(case.heads):
            b1, b2 = brute.weight_moments_brute(case, b, h)
            assert abs(w1[b, h] - float(b1)) <= 1e-12 * float(b1)
            assert abs(w2[b, h] - float(b2)) <= 1e-12 * float(b2)
            assert 1.0 <= w2[b, h] <= w1[b, h] <= contexts[b]


def test_weight_moments_closed_forms():
    # q = 0: every weight is 1, so both moments equal n; one token: both 1;
    # no token: both 0.
    case = small_case(45, [100, 1, 0], heads=2, dtype="bf16", poison=True)
    case.q_absorbed[0] = 0
    case.q_pe[0] = 0
    _, _, w1, w2 = oracle.latent_f64(case, moments=True)
    assert np.all(w1[0] == 100) and np.all(w2[0] == 100)
    assert np.all(w1[1] == 1) and np.all(w2[1] == 1)
    assert np.all(w1[2] == 0) and np.all(w2[2] == 0)


# --- P3: needles ----------------------------------------------------------

def plant_needle(case, b, t, h):
    """Make token t of request b dominate head h's softmax (out ~= its row)."""
    phys = case.block_table[b, t // 32] if t // 32 < case.block_table.shape[1] else None
    sign = np.sign(reference.decode16(case.q_absorbed[b, h], case.dtype))
    sign[sign == 0] = 1
    row = (6.0 * sign).astype(np.float32)
    case.ckv_pool[phys, t % 32] = mla_synth.encode16(row, case.dtype)
    case.kpe_pool[phys, t % 32] = mla_synth.encode16(np.zeros(64, np.float32), case.dtype)
    return reference.decode16(case.ckv_pool[phys, t % 32], case.dtype)


@pytest.mark.parametrize("t", [0, 31, 32, 63, 64, 150, 199])
def test_needle_is_found(t):
    case = small_case(81, [200], heads=2)
    needle = plant_needle(case, 0, t, 1)
    out, _ = oracle.latent_f64(case)
    assert np.max(np.abs(out[0, 1] - needle)) < 1e-12


@pytest.mark.parametrize("t", [200, 223])
def test_needle_past_context_end_is_ignored(t):
    # Rows past the context end in the last block must not be read.
    case = small_case(82, [200], heads=2)
    before, _ = oracle.latent_f64(case)
    plant_needle(case, 0, t, 1)
    after, _ = oracle.latent_f64(case)
    assert np.array_equal(before, after)


# --- P4: layout invariance --------------------------------------------------

def test_block_permutation_invariance():
    # Only logical token order matters: permuting the physical pool and
    # rewriting the table leaves the answer bit-identical.
    case = small_case(91, [150, 65], heads=3, dtype="bf16")
    out, lse2 = oracle.latent_f64(case)
    rng = np.random.default_rng(3)
    perm = rng.permutation(case.num_blocks)          # new position of block i
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    case.ckv_pool = case.ckv_pool[inv]
    case.kpe_pool = case.kpe_pool[inv]
    case.block_table = perm[case.block_table].astype(np.int32)
    out2, lse22 = oracle.latent_f64(case)
    assert np.array_equal(out, out2) and np.array_equal(lse2, lse22)


# --- P5: split / merge invariance --------------------------------------------

@pytest.mark.parametrize("contexts", [[1000], [1024], [33, 97, 1]])
def test_split_merge_equals_single_pass(contexts):
    # vllm-metal pull request 601, "What changed": the LSE-weighted reduce of
    # slices gives the single-pass answer; mlxcel pull request 995, "How
    # #898's merge kernel is reused": the split matches at every chunk
    # length and the merge is associative across regroupings.
    case = small_case(101 + len(contexts), contexts, heads=2)
    ref, lref = oracle.latent_f64(case)
    for P in range(1, 9):
        for S in (1, 2, 3, 7):
            Ps = [P] * case.batch
            Ss = [S] * case.batch
            ranges = oracle.row_ranges(case.context_lens, Ps, Ss)
            indptr = np.concatenate([[0], np.cumsum([p * s for p, s in zip(Ps, Ss)])])
            po, pl = oracle.partials_f64(case, ranges, indptr)
            out, lse2 = oracle.merge_log2_f64(po, pl, indptr)
            assert np.max(np.abs(out - ref)) < 1e-13, (P, S)
            assert np.max(np.abs(lse2 - lref)) < 1e-12, (P, S)


def test_merge_regrouping_is_associative():
    # Merging rows in two stages (pairs first) equals merging all at once.
    case = small_case(111, [900], heads=2)
    ranges = oracle.row_ranges(case.context_lens, [8], [1])
    po, pl = oracle.partials_f64(case, ranges, [0, 8])
    one, l_one = oracle.merge_log2_f64(po, pl, [0, 8])
    pairs, l_pairs = oracle.merge_log2_f64(po, pl, [0, 2, 4, 6, 8])
    two, l_two = oracle.merge_log2_f64(pairs.reshape(4, 2, 512), l_pairs.reshape(4, 2), [0, 4])
    assert np.max(np.abs(one - two)) < 1e-14
    assert np.max(np.abs(l_one - l_two)) < 1e-13


def test_merge_of_empty_rows_gives_zero_not_nan():
    po = np.zeros((3, 2, 512))
    pl = np.full((3, 2), -np.inf)
    out, lse2 = oracle.merge_log2_f64(po, pl, [0, 3])
    assert np.all(out == 0) and np.all(lse2 == -np.inf)


# --- P6: negative control ----------------------------------------------------

def test_natural_log_lse_gives_wrong_answer():
    # mlxcel pull request 995, "How #898's merge kernel is reused": a
    # natural-log LSE fed to the log2 merge still returns a plausible but
    # wrong weighted average. The control needs partition LSEs a few units
    # apart (equal ones weight rows alike under both conventions; a dominant
    # needle makes both pick the same row), so partition 0's latent rows are
    # scaled by 1.5.
    case = small_case(121, [1024], heads=2)
    blocks = case.block_table[0, :8]
    hot = reference.decode16(case.ckv_pool[blocks], case.dtype) * 1.5
    case.ckv_pool[blocks] = mla_synth.encode16(hot.astype(np.float32), case.dtype)
    ref, _ = oracle.latent_f64(case)
    ranges = oracle.row_ranges(case.context_lens, [4], [1])
    po, pl = oracle.partials_f64(case, ranges, [0, 4])
    good, _ = oracle.merge_log2_f64(po, pl, [0, 4])
    bad, _ = oracle.merge_ln_wrong(po, pl, [0, 4])
    assert np.max(np.abs(good - ref)) < 1e-13
    assert np.max(np.abs(bad - ref)) > 10 * 1e-2
    assert np.all(np.isfinite(bad))


def test_negative_control_needs_unequal_lses():
    # With equal LSEs both conventions weight rows equally, which is why the
    # control above builds unequal ones.
    po = np.random.default_rng(0).standard_normal((4, 1, 512))
    pl = np.full((4, 1), 3.0)
    good, _ = oracle.merge_log2_f64(po, pl, [0, 4])
    bad, _ = oracle.merge_ln_wrong(po, pl, [0, 4])
    assert np.max(np.abs(good - bad)) < 1e-15


# --- P10: the pages' printed byte counts -------------------------------------

def test_byte_model_matches_printed_numbers():
    with open(os.path.join(GOLDEN, "kv_byte_model.json")) as f:
        g = json.load(f)
    geo, printed = g["geometry"], g["printed"]
    lat = oracle.latent_bytes_per_token(geo["elem_bytes"], geo["latent"], geo["rope"])
    dec = oracle.decompressed_bytes_per_token(geo["heads"], geo["qk_head_dim"],
                                              geo["v_head_dim"], geo["elem_bytes"])
    assert lat == 1152 and dec == 10240
    assert round(dec / lat, 2) == printed["ratio_rounded_2dp"]
    budget = printed["budget_bytes"]
    assert budget == 16 * 2 ** 30
    assert oracle.max_context_tokens(budget, dec, geo["layers"]) == printed["max_tokens_decompressed"]
    assert oracle.max_context_tokens(budget, lat, geo["layers"]) == printed["max_tokens_latent"]


# --- the generator's rounding ------------------------------------------------

def test_bf16_encoder_rounds_to_nearest_even():
    # Ties go to the even neighbour; everything else to the nearer one.
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                     -1.0 - 2 ** -8, 3.0e-39, 65504.0], dtype=np.float32)
    bits = mla_synth.f32_to_bf16_bits(vals)
    back = reference.decode16(bits, "bf16")
    expect = [1.0, 1.0, 1.0 + 2 * 2 ** -7, 1.0 + 2 ** -7, -1.0]
    assert list(back[:5]) == expect
    for v, r in zip(vals, back):
        # brute force: r is a nearest representable neighbour of v
        lo = reference.decode16(np.uint16(np.float32(v).view(np.uint32) >> 16), "bf16")
        hi_bits = (np.float32(v).view(np.uint32) >> 16) + 1
        hi = reference.decode16(np.uint16(hi_bits), "bf16")
        assert abs(r - v) <= min(abs(lo - v), abs(hi - v))


# --- planted mistakes: every one must trip a pin ------------------------------

def _pins_pass(case_b):
    """Run a quick brute-force + closed-form check; True if all agree."""
    out, lse2 = oracle.latent_f64(case_b)
    for b in range(case_b.batch):
        for h in range(case_b.heads):
            eo, el = _brute_errors(case_b, b, h, out, lse2)
            if not (eo < 1e-12 and el < 1e-12):
                return False
    return True


def _mutant_attend_no_rope(qa, qp, C, Kp, scale):
    return ORIG_ATTEND(qa, np.zeros_like(qp), C, Kp, scale)


def _mutant_attend_ln_lse(qa, qp, C, Kp, scale):
    o, l, w1, w2 = ORIG_ATTEND(qa, qp, C, Kp, scale)
    return o, l * reference.LN_2, w1, w2


def _mutant_attend_scale_twice(qa, qp, C, Kp, scale):
    return ORIG_ATTEND(qa, qp, C, Kp, scale * scale)


def _mutant_attend_sign(qa, qp, C, Kp, scale):
    return ORIG_ATTEND(-qa, -qp, C, Kp, scale)


def _mutant_gather_off_by_one(ckv_pool, kpe_pool, table_row, n, dtype, lo=0, hi=None, *rest):
    hi = n if hi is None else min(hi, n)
    t = np.arange(max(0, lo), hi)
    phys = np.asarray(table_row)[(t + 1) // 32]
    slot = (t + 1) % 32
    return (reference.decode16(ckv_pool[phys, slot], dtype),
            reference.decode16(kpe_pool[phys, slot], dtype))


def _mutant_gather_drop_last(ckv_pool, kpe_pool, table_row, n, dtype, lo=0, hi=None, *rest):
    return ORIG_GATHER(ckv_pool, kpe_pool, table_row, max(0, n - 1), dtype, lo, hi, *rest)


ORIG_ATTEND = reference._attend
ORIG_GATHER = reference.gather_request


@pytest.mark.parametrize("mutant", ["no_rope", "ln_lse", "scale_twice", "sign",
                                    "gather_off_by_one", "gather_drop_last"])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    case = small_case(131, [40], heads=1, dtype="f16")
    assert _pins_pass(case)
    if mutant.startswith("gather"):
        fn = {"gather_off_by_one": _mutant_gather_off_by_one,
              "gather_drop_last": _mutant_gather_drop_last}[mutant]
        monkeypatch.setattr(reference, "gather_request", fn)
    else:
        fn = {"no_rope": _mutant_attend_no_rope, "ln_lse": _mutant_attend_ln_lse,
              "scale_twice": _mutant_attend_scale_twice,
              "sign": _mutant_attend_sign}[mutant]
        monkeypatch.setattr(reference, "_attend", fn)
    assert not _pins_pass(case)


# --- several new tokens per request (the in-window causal mask) ---------------
# Our reading (no page decodes more than one token): the cache holds all
# q_len new tokens, token j sits at position n - q_len + j and sees positions
# 0 .. n - q_len + j.

@pytest.mark.parametrize("dtype,q_len,contexts", [("f16", 3, [40]), ("bf16", 2, [33, 5]),
                                                  ("f16", 4, [3])])
def test_window_matches_brute_force(dtype, q_len, contexts):
    # Each new token by the definition with an explicit causal mask, at 50
    # digits; [3] with four new tokens leaves the first one nothing to see.
    case = small_case(141 + q_len, contexts, heads=2, dtype=dtype, q_len=q_len)
    out, lse2 = oracle.latent_f64(case)
    assert out.shape == (len(contexts), 2 * q_len, 512)
    for b in range(len(contexts)):
        for j in range(q_len):
            for h in range(2):
                bo, bl = brute.latent_brute_window(case, b, j, h)
                r = j * 2 + h
                if bl == mpmath.mpf("-inf"):
                    assert lse2[b, r] == -np.inf and np.all(out[b, r] == 0)
                    continue
                eo = max(abs(float(x) - o) for x, o in zip(bo, out[b, r]))
                assert eo < 1e-12 and abs(float(bl) - lse2[b, r]) < 1e-12, (b, j, h)


def _window_counts_hold(case, n):
    out, lse2 = oracle.latent_f64(case)
    rows = np.stack([reference.decode16(case.ckv_pool[case.block_table[0, t // 32], t % 32],
                                        case.dtype) for t in range(n)])
    H = case.heads
    ok = True
    for j in range(case.q_len):
        cnt = n - case.q_len + j + 1          # positions 0 .. n - q_len + j
        mean = rows[:cnt].sum(axis=0) / cnt
        ok &= bool(np.max(np.abs(out[0, j * H:(j + 1) * H] - mean[None])) < 1e-13)
        ok &= bool(np.all(np.abs(lse2[0, j * H:(j + 1) * H] - math.log2(cnt)) < 1e-13))
    return ok


@pytest.mark.parametrize("q_len", [2, 5])
def test_window_uniform_scores_count(q_len):
    # q = 0: new token j's output is the plain mean of the rows it sees and
    # its lse2 is log2 of their number.
    n = 70
    case = small_case(151, [n], heads=2, dtype="bf16", poison=True, q_len=q_len)
    case.q_absorbed[:] = 0
    case.q_pe[:] = 0
    assert _window_counts_hold(case, n)


def test_window_off_by_one_is_caught(monkeypatch):
    n = 70
    case = small_case(152, [n], heads=2, dtype="bf16", q_len=3)
    case.q_absorbed[:] = 0
    case.q_pe[:] = 0
    assert _window_counts_hold(case, n)
    monkeypatch.setattr(reference, "visible_len", lambda n, q, j: max(0, n - q + j))
    assert not _window_counts_hold(case, n)


def test_window_needle_visibility():
    # A dominant token at position n - q_len + j is found by new token j and
    # left unseen by new token j - 1.
    n, q_len, H = 90, 3, 2
    for j in range(1, q_len):
        t = n - q_len + j
        for row, seen in ((j * H + 1, True), ((j - 1) * H + 1, False)):
            case = small_case(161, [n], heads=H, q_len=q_len)
            before, _ = oracle.latent_f64(case)
            needle = plant_needle(case, 0, t, row)
            after, _ = oracle.latent_f64(case)
            if seen:
                assert np.max(np.abs(after[0, row] - needle)) < 1e-12
            else:
                assert np.array_equal(before[0, row], after[0, row])


# --- Blocks of 16 tokens (the "block16" layout vllm-metal pull request 601's
# review asks to see covered) ------------------------------------------------

def relayout_16(case):
    """The same logical tokens stored as 16-token blocks: block k of 32
    tokens becomes blocks 2k and 2k + 1 of the new pool, in a fresh random
    order, and the table is rewritten to match."""
    pool32 = case.num_blocks
    ckv = case.ckv_pool.reshape(pool32 * 2, 16, 512)
    kpe = case.kpe_pool.reshape(pool32 * 2, 16, 64)
    perm = np.random.default_rng(7).permutation(pool32 * 2)   # new slot of old half i
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    table = np.empty((case.batch, case.max_blocks * 2), dtype=np.int32)
    table[:, 0::2] = perm[2 * case.block_table]
    table[:, 1::2] = perm[2 * case.block_table + 1]
    return mla_synth.Case(dtype=case.dtype, batch=case.batch, heads=case.heads,
                          context_lens=case.context_lens.copy(), block_table=table,
                          ckv_pool=ckv[inv].copy(), kpe_pool=kpe[inv].copy(),
                          q_absorbed=case.q_absorbed, q_pe=case.q_pe, scale=case.scale,
                          seed=case.seed, q_len=case.q_len, block_size=16)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("contexts", [[1], [15, 16], [17, 33], [70]])
def test_block16_latent_matches_brute_force(dtype, contexts):
    # Generated directly with 16-token blocks; the brute force walks the
    # table itself, slot t % 16 of block t // 16.
    case = small_case(401 + len(contexts) + contexts[0], contexts, dtype=dtype, poison=True,
                      block_size=16)
    assert case.ckv_pool.shape[1] == 16
    out, lse2 = oracle.latent_f64(case)
    for b in range(case.batch):
        for h in range(case.heads):
            eo, el = _brute_errors(case, b, h, out, lse2)
            assert eo < 1e-12 and el < 1e-12, (b, h, eo, el)


@pytest.mark.parametrize("contexts", [[200, 17], [1024], [16, 31, 32, 33]])
def test_block16_relayout_is_bit_identical(contexts):
    # The answer depends on the logical token sequence only, not on how the
    # cache cuts it into blocks.
    case = small_case(411 + len(contexts), contexts, heads=3, dtype="bf16")
    out, lse2 = oracle.latent_f64(case)
    c16 = relayout_16(case)
    out16, lse16 = oracle.latent_f64(c16)
    assert np.array_equal(out, out16) and np.array_equal(lse2, lse16)


@pytest.mark.parametrize("contexts", [[1000], [33, 97, 1, 16]])
def test_block16_split_merge_equals_single_pass(contexts):
    case = small_case(421 + len(contexts), contexts, heads=2, block_size=16)
    ref, lref = oracle.latent_f64(case)
    for P in (1, 2, 5, 8):
        for S in (1, 3, 7):
            Ps, Ss = [P] * case.batch, [S] * case.batch
            ranges = oracle.row_ranges(case.context_lens, Ps, Ss, block_size=16)
            assert all(lo % 16 == 0 for _, lo, hi in ranges if hi > lo)
            indptr = np.concatenate([[0], np.cumsum([p * s for p, s in zip(Ps, Ss)])])
            po, pl = oracle.partials_f64(case, ranges, indptr)
            out, lse2 = oracle.merge_log2_f64(po, pl, indptr)
            assert np.max(np.abs(out - ref)) < 1e-13, (P, S)
            assert np.max(np.abs(lse2 - lref)) < 1e-12, (P, S)


@pytest.mark.parametrize("t", [0, 15, 16, 31, 47, 199])
def test_block16_needle_is_found(t):
    case = small_case(431, [200], heads=2, block_size=16)
    phys = case.block_table[0, t // 16]
    sign = np.sign(reference.decode16(case.q_absorbed[0, 1], case.dtype))
    sign[sign == 0] = 1
    case.ckv_pool[phys, t % 16] = mla_synth.encode16((6.0 * sign).astype(np.float32), case.dtype)
    case.kpe_pool[phys, t % 16] = mla_synth.encode16(np.zeros(64, np.float32), case.dtype)
    needle = reference.decode16(case.ckv_pool[phys, t % 16], case.dtype)
    out, _ = oracle.latent_f64(case)
    assert np.max(np.abs(out[0, 1] - needle)) < 1e-12


# --- latent caches stored as E4M3 bytes with one scale --------------------------
# The pages keep 16-bit caches; the 8-bit layout is the next step beyond them.
# The byte format is the E4M3 format of the OCP 8-bit floating point
# specification (bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN).

def fp8_case(seed, contexts, heads=2, dtype="f16", kv_scale=0.0625, **kw):
    return small_case(seed, contexts, heads=heads, dtype=dtype, kv_dtype="fp8_e4m3",
                      kv_scale=kv_scale, **kw)


def test_fp8_decode_closed_forms():
    # Values fixed by the format definition: zero and negative zero, the
    # smallest subnormal 2^-9 and the largest 7 * 2^-9, the smallest normal
    # 2^-6, one, the largest finite value 1.75 * 2^8 = 448, and the two NaNs.
    codes = np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0xB8, 0x7E, 0xFE, 0x40, 0x3C])
    want = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, -1.0, 448.0, -448.0, 2.0, 1.5]
    got = reference.decode_fp8_e4m3(codes)
    assert list(got) == want
    assert np.signbit(got[1])
    assert np.all(np.isnan(reference.decode_fp8_e4m3(np.array([0x7F, 0xFF]))))
    # Finite positive codes are strictly increasing; the negative half mirrors them.
    pos = reference.decode_fp8_e4m3(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(reference.decode_fp8_e4m3(np.arange(0x80, 0xFF)), -pos)


def test_fp8_encoder_round_trips_every_finite_code():
    # The generator's encoder (its own table) and the oracle's decoder agree
    # on every finite code, and the encoder picks the nearest code.
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = reference.decode_fp8_e4m3(codes)
    assert np.array_equal(mla_synth.f32_to_fp8_e4m3_bits(vals)[1:], codes[1:])
    rng = np.random.default_rng(4)
    x = rng.standard_normal(2000) * 30
    enc = reference.decode_fp8_e4m3(mla_synth.f32_to_fp8_e4m3_bits(x))
    finite = reference.decode_fp8_e4m3(codes)
    nearest = np.min(np.abs(finite[None, :] - np.clip(x, -448, 448)[:, None]), axis=1)
    assert np.all(np.abs(enc - np.clip(x, -448, 448)) == nearest)


@pytest.mark.parametrize("contexts,block_size", [([1], 32), ([40], 32), ([33, 17], 16)])
def test_fp8_latent_matches_brute_force(contexts, block_size):
    # The 50-digit loops decode the bytes case by case, times the scale.
    case = fp8_case(451 + contexts[0], contexts, block_size=block_size, poison=True)
    assert case.ckv_pool.dtype == np.uint8
    out, lse2 = oracle.latent_f64(case)
    for b in range(case.batch):
        for h in range(case.heads):
            eo, el = _brute_errors(case, b, h, out, lse2)
            assert eo < 1e-12 and el < 1e-12, (b, h, eo, el)


def test_fp8_single_token_closed_form():
    # One token: the output is that token's dequantized row exactly, and
    # lse2 = scale * (qa . c + qp . k) * log2(e).
    case = fp8_case(461, [1], heads=3, kv_scale=0.125)
    out, lse2 = oracle.latent_f64(case)
    phys = case.block_table[0, 0]
    c = reference.decode_fp8_e4m3(case.ckv_pool[phys, 0]) * 0.125
    k = reference.decode_fp8_e4m3(case.kpe_pool[phys, 0]) * 0.125
    for h in range(3):
        assert np.array_equal(out[0, h], c)
        qa = reference.decode16(case.q_absorbed[0, h], case.dtype)
        qp = reference.decode16(case.q_pe[0, h], case.dtype)
        assert abs(lse2[0, h] - case.scale * (qa @ c + qp @ k) * reference.LOG2_E) < 1e-12


def test_fp8_scale_is_linear_in_the_values():
    # Doubling the scale doubles every dequantized value: the output doubles
    # exactly when the queries are zero (uniform weights).
    case = fp8_case(471, [70], heads=2)
    case.q_absorbed[:] = 0
    case.q_pe[:] = 0
    a, la = oracle.latent_f64(case)
    case.kv_scale *= 2
    b, lb = oracle.latent_f64(case)
    assert np.array_equal(b, 2 * a) and np.array_equal(la, lb)


def test_fp8_wrong_exponent_bias_is_caught(monkeypatch):
    # The other common E4M3 variant (bias 8, no negative zero) is a
    # plausible mistake; the closed forms reject it.
    def fnuz(bits):
        b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
        e, m = (b >> 3) & 0xF, (b & 7).astype(np.float64)
        mag = np.where(e == 0, m / 8.0 * 2.0 ** -7, (1.0 + m / 8.0) * np.exp2(e - 8.0))
        return np.where(b >> 7, -mag, mag)
    monkeypatch.setattr(reference, "decode_fp8_e4m3", fnuz)
    with pytest.raises(AssertionError):
        test_fp8_decode_closed_forms()
