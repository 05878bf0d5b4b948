"""The GPU-versus-oracle comparison protocol on the CPU.

The oracle's own outputs stand in for the GPU's; planted deviations must be
reported as mismatches, and only the documented exceptions (a nucleus
boundary within the band, fp32 rounding of the residual mass) excused.
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
