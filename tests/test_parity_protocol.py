"""The GPU-versus-oracle comparison protocol on the CPU.

The oracle's own outputs stand in for the GPU's; planted deviations must be
reported as mismatches, and only the documented exceptions (a nucleus
boundary within the band, fp32 rounding of the residual mass, a final draw
that fp32 weights cannot resolve) excused.
"""
import copy

import numpy as np
import pytest

from oracle import parity

B, K, V = 24, 4, 64


@pytest.fixture(scope="module")
def run(oracle_lib):
    rng = np.random.default_rng(3)
    t = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    d = (t[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    top3 = np.argsort(-d, axis=2)[:, :, :3]  # draft tokens inside the draft nucleus
    g = np.take_along_axis(top3, rng.integers(0, 3, size=(B, K, 1)), axis=2)[..., 0]
    host = {"target": t, "draft": d, "draft_tokens": g.astype(np.int32),
            "draft_len": np.full(B, K, np.int32), "temperature": np.ones(B, np.float32)}
    ref = parity.oracle_on(host, 7, top_p=np.full(B, 0.9, np.float32))
    assert np.nanmin(ref["margin_nucleus"]) > 1e-6 and np.nanmin(ref["margin_accept"]) > 1e-6
    return host, ref


def _cmp(gpu, ref, host):
    return parity.compare(gpu, ref, host["draft_len"], host["temperature"], K)


def _ok_seq(ref, min_n=0, max_n=K):
    """A sequence that ended OK with min_n <= accepted <= max_n."""
    for b in range(B):
        n = int(ref["num_accepted"][b])
        if ref["seq_status"][b] == parity.SEQ_OK and min_n <= n <= max_n:
            return b
    pytest.skip("no such sequence in the batch")


def test_identical_outputs_pass(run):
    host, ref = run
    rep = _cmp(copy.deepcopy(ref), ref, host)
    assert rep.ok(), rep.summary()
    assert rep.flagged == 0 and rep.boundary_values == 0
    assert rep.sequences == B


def test_planted_token_is_reported(run):
    host, ref = run
    b = _ok_seq(ref, min_n=1)
    gpu = copy.deepcopy(ref)
    gpu["out_tokens"][b, 0] = (gpu["out_tokens"][b, 0] + 1) % V
    assert any("accepted token 0" in m for m in _cmp(gpu, ref, host).mismatches)


def test_planted_final_token_is_reported(run):
    host, ref = run
    b = _ok_seq(ref)
    n = int(ref["num_accepted"][b])
    gpu = copy.deepcopy(ref)
    gpu["out_tokens"][b, n] = (gpu["out_tokens"][b, n] + 1) % V
    assert any("final token" in m for m in _cmp(gpu, ref, host).mismatches)


def test_planted_count_is_reported(run):
    host, ref = run
    b = _ok_seq(ref, max_n=K - 1)
    gpu = copy.deepcopy(ref)
    gpu["num_accepted"][b] += 1
    assert not _cmp(gpu, ref, host).ok()


@pytest.mark.parametrize("key", ["p_g", "q_g"])
def test_value_error_is_reported(run, key):
    host, ref = run
    b = _ok_seq(ref)
    gpu = copy.deepcopy(ref)
    gpu[key][b, K - 1] *= 1 + 5e-5  # 5x the relative tolerance
    rep = _cmp(gpu, ref, host)
    assert any(f"{key}[{K - 1}]" in m for m in rep.mismatches), rep.summary()


def test_value_on_a_boundary_row_past_the_stop_is_skipped(run):
    """A row the round does not depend on, whose own nucleus boundary lies
    within the band, may keep a different set: its values are not compared."""
    host, ref = run
    b = _ok_seq(ref, max_n=K - 2)
    i = int(ref["num_accepted"][b]) + 1  # a draft row past the stop
    ref2 = copy.deepcopy(ref)
    ref2["margin_nucleus"][b, K + 1 + i] = 1e-9
    gpu = copy.deepcopy(ref)
    gpu["q_g"][b, i] *= 1.01
    rep = _cmp(gpu, ref2, host)
    assert rep.ok(), rep.summary()
    assert rep.boundary_values == 1
    # the same error without the boundary is reported
    assert not _cmp(gpu, ref, host).ok()
    # and a boundary on the target row does not excuse the draft value
    ref3 = copy.deepcopy(ref)
    ref3["margin_nucleus"][b, i + 1] = 1e-9
    assert not _cmp(gpu, ref3, host).ok()


def test_boundary_on_a_dependent_row_flags_the_sequence(run):
    host, ref = run
    b = _ok_seq(ref)
    ref2 = copy.deepcopy(ref)
    ref2["margin_nucleus"][b, 0] = 1e-9
    gpu = copy.deepcopy(ref)
    gpu["out_tokens"][b, int(ref["num_accepted"][b])] = -5  # would be a mismatch otherwise
    rep = _cmp(gpu, ref2, host)
    assert rep.ok(), rep.summary()
    assert rep.flagged == 1 and rep.flagged_disagree == 1


def test_residual_mass_tolerance(run):
    """S is compared within rel plus RESID_ABS: an error below the fp32
    rounding bound passes, one well above it does not."""
    host, ref = run
    b = next(x for x in range(B) if np.isfinite(ref["resid_mass"][x]))
    S = float(ref["resid_mass"][b])
    gpu = copy.deepcopy(ref)
    gpu["resid_mass"][b] = S + 0.9 * parity.RESID_ABS
    assert _cmp(gpu, ref, host).ok()
    gpu["resid_mass"][b] = S + 1e-5 * S + 4 * parity.RESID_ABS
    assert any("resid_mass" in m for m in _cmp(gpu, ref, host).mismatches)


def test_status_mismatch_is_reported(run):
    host, ref = run
    b = _ok_seq(ref)
    gpu = copy.deepcopy(ref)
    gpu["seq_status"][b] = 2
    assert any("status" in m for m in _cmp(gpu, ref, host).mismatches)


def test_flagged_final_draw_must_land_in_the_band_window(run):
    """A flagged final draw may differ from the oracle's token only within the
    oracle's band window; a token outside it is a mismatch even though the
    oracle's margin is below the band."""
    host, ref = run
    b = _ok_seq(ref)
    n = int(ref["num_accepted"][b])
    tok = int(ref["out_tokens"][b, n])
    ref2 = copy.deepcopy(ref)
    ref2["margin_draw"][b] = 1e-8  # as if v sat next to a CDF boundary
    ref2["draw_window"][b] = (tok, tok + 1)
    gpu = copy.deepcopy(ref)
    gpu["out_tokens"][b, n] = tok + 1  # the neighbour inside the window: allowed
    rep = _cmp(gpu, ref2, host)
    assert rep.ok(), rep.summary()
    assert rep.flagged_disagree == 1
    gpu["out_tokens"][b, n] = (tok + 7) % V  # outside the window: reported
    rep = _cmp(gpu, ref2, host)
    assert any("band window" in m for m in rep.mismatches), rep.summary()


def test_oracle_window_contains_its_own_token(run):
    host, ref = run
    for b in range(B):
        if ref["seq_status"][b] == parity.SEQ_OK and host["temperature"][b] > 0:
            lo, hi = ref["draw_window"][b]
            assert lo <= ref["out_tokens"][b, ref["num_accepted"][b]] <= hi


# ---------------------------------------------------------------------------
# A final draw's band widens with the fp32 resolution of its CDF.
# ---------------------------------------------------------------------------

def test_draw_band_closed_form(oracle_lib):
    import oracle
    eps = 2.0 ** -24
    # p = q uniform over n ids: sqrt(sum max(p, q)^2) = 1 / sqrt(n)
    for n, S in ((4, 0.5), (64, 1e-3), (1000, 1e-9)):
        p = np.full(n, 1.0 / n)
        want = max(1e-6, 8 * eps / np.sqrt(n) / S)
        assert oracle.draw_band(p, p.copy(), S, 1e-6) == pytest.approx(want, rel=1e-12)
    # without q the scale is p's alone; the larger of p and q counts per id
    p = np.array([0.5, 0.25, 0.25])
    q = np.array([0.25, 0.5, 0.25])
    m = np.array([0.5, 0.5, 0.25])
    assert oracle.draw_band(p, q, 1e-4, 1e-6) == pytest.approx(
        8 * eps * np.sqrt((m ** 2).sum()) / 1e-4, rel=1e-12)
    assert oracle.draw_band(p, None, 1e-4, 1e-6) == pytest.approx(
        8 * eps * np.sqrt((p ** 2).sum()) / 1e-4, rel=1e-12)
    # never below the base band, and the base band where there is no mass
    assert oracle.draw_band(p, q, 1.0, 1e-3) == 1e-3
    assert oracle.draw_band(p, q, 0.0, 1e-6) == 1e-6


def _dominant_case():
    """Target and draft nearly one-hot on the same id at a low temperature,
    and a drafted token from the far tail: a certain rejection whose
    residual mass (about 2.6e-10) is far below fp32's resolution of the
    dominant id's weight."""
    t = np.array([[-1.6796875, -4.0, -2.625, -2.375, 1.25, -0.67578125, 6.625],
                  [-7.4375, 6.1875, 2.140625, -0.80859375, 4.28125, 4.875, -5.71875]],
                 np.float32)[None]
    d = np.array([[-2.65625, -3.71875, -2.59375, -1.859375, 0.84765625, -0.78515625, 6.21875]],
                 np.float32)[None]
    host = {"target": t, "draft": d, "draft_tokens": np.array([[2]], np.int32),
            "draft_len": np.array([1], np.int32), "temperature": np.array([0.3], np.float32)}
    return host


def test_unresolved_residual_is_flagged_not_compared(oracle_lib):
    host = _dominant_case()
    seed = 2558530382594599338
    ref = parity.oracle_on(host, seed)
    assert ref["num_accepted"][0] == 0 and ref["draw_kind"][0] == parity.DRAW_RESIDUAL
    assert ref["resid_mass"][0] < 1e-9 and ref["band_draw"][0] > 1.0
    lo, hi = ref["draw_window"][0]
    assert (lo, hi) == (0, 6)  # a band of 1 or more covers every id with weight
    # another id with residual weight (p > q there): flagged, not a mismatch
    gpu = copy.deepcopy(ref)
    gpu["out_tokens"][0, 0] = 0
    gpu["resid_mass"][0] = 8.1e-13
    rep = parity.compare(gpu, ref, host["draft_len"], host["temperature"], 1)
    assert rep.ok(), rep.summary()
    assert rep.flagged == 1 and rep.flagged_wide == 1 and rep.flagged_disagree == 1
    # the fp32 residual rounded to nothing: drawn from p instead, still flagged
    gpu2 = copy.deepcopy(gpu)
    gpu2["draw_kind"][0] = parity.DRAW_RESIDUAL_AS_P
    gpu2["resid_mass"][0] = 1.0
    rep2 = parity.compare(gpu2, ref, host["draft_len"], host["temperature"], 1)
    assert rep2.ok() and rep2.flagged == 1, rep2.summary()


def test_resolved_draws_keep_the_base_band(run, oracle_lib):
    """Where the weights resolve the draw its band is the base band, and the
    same disagreement as above (a large margin) is a mismatch."""
    host, ref = run
    ok = [b for b in range(B) if ref["seq_status"][b] == parity.SEQ_OK
          and ref["band_draw"][b] == 1e-6 and ref["margin_draw"][b] > 1e-3]
    assert ok
    b = ok[0]
    n = int(ref["num_accepted"][b])
    gpu = copy.deepcopy(ref)
    gpu["out_tokens"][b, n] = (gpu["out_tokens"][b, n] + 1) % V
    assert any("final token" in m for m in _cmp(gpu, ref, host).mismatches)
