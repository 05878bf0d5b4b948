"""Degenerate inputs of the plain step against the oracle: rows with masked
tokens (logit -inf, weight 0), logits quantised to a coarse grid so that the
row maximum is tied between several tokens, and temperatures from 1e-3
(the softmax nearly one-hot, or uniform over the tied maxima; most other
weights underflow fp32) to 100 (nearly uniform), next to greedy sequences.
Drafted tokens come from the draft's own distribution, so some are masked in
the target (p(g) = 0: a certain rejection) and the residual often keeps a
single token; a few are then masked in the draft as well (q(g) = 0: status
QZERO once the scan reaches them). Early exit must give the full step's
outputs bit for bit."""
import numpy as np
import pytest
import scipy.special
import torch

from conftest import bf16_bits, bf16_to_f32

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

import speculative_decoding_verification_11_amd as sv  # noqa: E402
from oracle import parity  # noqa: E402
from test_gpu_parity import DEV, batch_to, check, host, raw_batch, run_gpu, say  # noqa: E402

TAUS = (1e-3, 0.05, 1.0, 0.0, 30.0, 100.0)


def _edge_batch(rng, B, k, V, dtype, mask_frac):
    t = np.round(rng.standard_normal((B, k + 1, V)) * 3.0 * 2) / 2   # steps of 0.5: ties
    d = np.round((t[:, :k] + rng.standard_normal((B, k, V))) * 2) / 2
    t[rng.random(t.shape) < mask_frac] = -np.inf
    d[rng.random(d.shape) < mask_frac] = -np.inf
    t[:, :, 0] = np.maximum(t[:, :, 0], -5.0)  # every row keeps a finite logit
    d[:, :, 0] = np.maximum(d[:, :, 0], -5.0)
    t, d = t.astype(np.float32), d.astype(np.float32)
    if dtype == "bf16":
        t, d = bf16_bits(t), bf16_bits(d)
        dv = bf16_to_f32(d)
    else:
        dv = d
    tau = np.array([TAUS[b % len(TAUS)] for b in range(B)], np.float32)
    L = rng.integers(0, k + 1, size=B).astype(np.int32)
    g = np.full((B, k), -1, np.int32)
    for b in range(B):
        for i in range(L[b]):
            if tau[b] == 0:
                g[b, i] = int(np.argmax(dv[b, i]))
            else:
                q = scipy.special.softmax(dv[b, i].astype(np.float64) / float(tau[b]))
                g[b, i] = int(rng.choice(V, p=q))
    # A drafted token the draft row masks (q(g) = 0 exactly): status QZERO
    # once the scan reaches it, on both sides.
    for b in range(2, B, 9):
        if tau[b] > 0 and L[b] > 0 and g[b, 0] != 0:
            d[b, 0, g[b, 0]] = 0xFF80 if dtype == "bf16" else -np.inf
    return raw_batch(t, d, g, L, tau)


@pytest.mark.parametrize("V,dtype,mask_frac", [(20000, "bf16", 0.4), (9000, "f32", 0.4),
                                               (3000, "bf16", 0.97)])
def test_masked_tied_and_extreme_temperatures(V, dtype, mask_frac):
    rng = np.random.default_rng(V + int(mask_frac * 100))
    B, k = 48, 5
    cb = _edge_batch(rng, B, k, V, dtype, mask_frac)
    gb = batch_to(cb, DEV)
    h = host(cb)
    total = parity.Report()
    for seed in (5, 0xABCDEF):
        say(f"[case] edges V={V} {dtype} masked {mask_frac} seed={seed:#x}")
        g = run_gpu(gb, seed)
        r = parity.oracle_on(h, seed)
        total.merge(parity.compare(g, r, h["draft_len"], h["temperature"], k))
        ee = sv.spec_verify_early_exit(gb.target, gb.draft, gb.draft_tokens, gb.draft_len,
                                       gb.temperature, seed, aux=True)
        torch.cuda.synchronize()
        assert np.array_equal(ee[0].cpu().numpy(), g["out_tokens"])
        assert np.array_equal(ee[1].cpu().numpy(), g["num_accepted"])
        for key in ("seq_status", "draw_kind", "draw_row"):
            assert np.array_equal(ee[2][key].cpu().numpy(), g[key]), key
        kinds = set(g["draw_kind"].tolist())
        assert sv.DRAW_RESIDUAL in kinds and sv.DRAW_GREEDY in kinds, kinds
        assert (g["seq_status"] == sv.SEQ_QZERO).any()
    check(total, f"edges V={V} {dtype}")


def test_residual_below_fp32_resolution_is_flagged():
    """Target and draft one-hot on the same id at tau 0.3 and a drafted token
    from the far tail: the residual mass (about 2.6e-10) is below fp32's
    resolution of the dominant id's weight. The GPU's draw must still be a
    valid one (inside the oracle's window), reported as flagged by the
    draw's widened band rather than compared."""
    from test_parity_protocol import _dominant_case
    host_arrays = _dominant_case()
    seed = 2558530382594599338
    cb = raw_batch(host_arrays["target"], host_arrays["draft"], host_arrays["draft_tokens"],
                   host_arrays["draft_len"], host_arrays["temperature"])
    g = run_gpu(batch_to(cb, DEV), seed)
    r = parity.oracle_on(host(cb), seed)
    assert r["band_draw"][0] > 1.0
    rep = parity.compare(g, r, host_arrays["draft_len"], host_arrays["temperature"], 1)
    check(rep, "residual below fp32 resolution")
    assert rep.flagged == 1 and rep.flagged_wide == 1
