"""Vocabularies far beyond the workloads'. A row of 257 chunks is more than the
locate stages in LDS (128 chunks' masses), so it reads the chunk masses from
global memory, and the decision folds 257 chunk partials per row; a bf16 row
of 262,149 tokens goes through the top-p filter's counting pass. Every
sequence is checked against the oracle, with and without top-p, and the
early-exit schedule against the full step."""
import numpy as np
import pytest
import torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

import speculative_decoding_verification_11_amd as sv  # noqa: E402
import oracle  # noqa: E402
from oracle import parity  # noqa: E402
from test_gpu_parity import check, say  # noqa: E402

DEV = "cuda:0"
CHUNK_BYTES = 32 * 1024
MASS_STAGED_CHUNKS = 128  # the locate keeps a sequence's chunk masses in LDS up to this


def _batch(B, k, V, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    t = torch.randn((B, k + 1, V), generator=g, device=DEV) * 2.5
    d = t[:, :k] + torch.randn((B, k, V), generator=g, device=DEV) * 0.8
    tau = torch.tensor([(0.0, 0.8, 1.0, 1.4)[b % 4] for b in range(B)], dtype=torch.float32,
                       device=DEV)
    L = torch.tensor([(b % k) + 1 for b in range(B)], dtype=torch.int32, device=DEV)
    top = d.argmax(dim=2).to(torch.int32)
    rnd = torch.randint(0, V, (B, k), generator=g, device=DEV).to(torch.int32)
    tok = torch.where(torch.rand((B, k), generator=g, device=DEV) < 0.6, top, rnd)
    if dtype == "bf16":
        t, d = t.to(torch.bfloat16), d.to(torch.bfloat16)
    return t.contiguous(), d.contiguous(), tok.contiguous(), L.contiguous(), tau.contiguous()


def _host(x):
    x = x.cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def _np(res):
    out, n, aux = res
    g = {key: v.cpu().numpy() for key, v in aux.items()}
    g["out_tokens"] = out.cpu().numpy()
    g["num_accepted"] = n.cpu().numpy()
    return g


# (B, k, V, dtype)
CASES = [
    (8, 3, 16 * 16384 + 5, "bf16"),   # nc = 17: three fold batches; a long filtered row
    (3, 2, (1 << 21) + 3, "f32"),     # nc = 257: chunk masses read from global memory
]


@pytest.mark.parametrize("B,k,V,dtype", CASES)
def test_huge_vocabularies_match_the_oracle(B, k, V, dtype):
    nc = -(-V // (CHUNK_BYTES // (2 if dtype == "bf16" else 4)))
    assert nc > 16 and (dtype == "bf16" or nc > MASS_STAGED_CHUNKS)
    t, d, tok, L, tau = _batch(B, k, V, dtype, V % 1000)
    h = dict(target=_host(t), draft=_host(d), draft_tokens=_host(tok), draft_len=_host(L),
             temperature=_host(tau))
    top_p = np.array([(1.0, 0.9)[b % 2] for b in range(B)], np.float32)
    for seed in (17, 0xBADC0FFEE):
        say(f"[case] huge vocabulary B={B} k={k} V={V} {dtype} nc={nc} seed={seed:#x}")
        full = sv.spec_verify(t, d, tok, L, tau, seed, aux=True)
        ee = sv.spec_verify_early_exit(t, d, tok, L, tau, seed, aux=True)
        torch.cuda.synchronize()
        assert torch.equal(ee[0], full[0]) and torch.equal(ee[1], full[1])
        for key in ("seq_status", "draw_row", "draw_kind"):
            assert torch.equal(ee[2][key], full[2][key]), key
        assert torch.equal(ee[2]["resid_mass"].view(torch.int32),
                           full[2]["resid_mass"].view(torch.int32))
        ref = oracle.spec_verify_ref(h["target"], h["draft"], h["draft_tokens"], h["draft_len"],
                                     h["temperature"], seed)
        check(parity.compare(_np(full), ref, h["draft_len"], h["temperature"], k),
              f"huge V={V} {dtype}")
        kinds = set(_np(full)["draw_kind"].tolist())
        assert sv.DRAW_RESIDUAL in kinds or sv.DRAW_BONUS in kinds

        tp = torch.as_tensor(top_p, device=DEV)
        g = _np(sv.spec_verify_top_p(t, d, tok, L, tau, tp, seed, aux=True))
        ref_p = oracle.spec_verify_ref(h["target"], h["draft"], h["draft_tokens"],
                                       h["draft_len"], h["temperature"], seed, top_p=top_p)
        check(parity.compare(g, ref_p, h["draft_len"], h["temperature"], k),
              f"huge V={V} {dtype} top-p")
