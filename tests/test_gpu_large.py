"""Batches large enough that the library splits its launches into slices
(more than 2^22 workgroups): results on both sides of a slice boundary
must match the oracle, and the global sequence index must carry over
(Philox counters, seq_base)."""
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
SLICE_ITEMS = 1 << 22  # the library's largest grid per launch


def _big_batch(B, k, V, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    t = torch.randn((B, k + 1, V), generator=g, device=DEV) * 2
    d = t[:, :k] + torch.randn((B, k, V), generator=g, device=DEV) * 0.7
    tau = torch.where(torch.arange(B, device=DEV) % 5 == 0, 0.0, 0.9).to(torch.float32)
    L = torch.randint(0, k + 1, (B,), generator=g, device=DEV).to(torch.int32)
    tok = d.argmax(dim=2).to(torch.int32)  # the draft's top token: inside any nucleus
    return t.contiguous(), d.contiguous(), tok.contiguous(), L.contiguous(), tau.contiguous()


def _host(t, d, tok, L, tau, rows):
    idx = torch.as_tensor(rows, device=DEV)
    return dict(target=t[idx].cpu().numpy(), draft=d[idx].cpu().numpy(),
                draft_tokens=tok[idx].cpu().numpy(), draft_len=L[idx].cpu().numpy(),
                temperature=tau[idx].cpu().numpy())


def test_sliced_launches_match_the_oracle():
    B, k, V = 300_000, 7, 16
    per_slice = SLICE_ITEMS // ((2 * k + 1) * 1)
    assert B > per_slice
    t, d, tok, L, tau = _big_batch(B, k, V, 5)
    rows = sorted(set(list(range(per_slice - 40, per_slice + 40)) + list(range(0, 20))
                      + list(range(B - 20, B))))
    seed = 0xFEED
    base = 1000  # a nonzero seq_base shifts every global index
    full = sv.spec_verify(t, d, tok, L, tau, seed, seq_base=base, aux=True)
    ee = sv.spec_verify_early_exit(t, d, tok, L, tau, seed, seq_base=base, aux=True)
    tp = torch.full((B,), 0.9, dtype=torch.float32, device=DEV)
    top = sv.spec_verify_top_p(t, d, tok, L, tau, tp, seed, seq_base=base, aux=True)
    torch.cuda.synchronize()
    h = _host(t, d, tok, L, tau, rows)
    say(f"[case] sliced B={B} k={k} V={V}, {len(rows)} sequences checked")

    def pick(res):
        out, n, aux = res
        g = {key: v.cpu().numpy()[rows] for key, v in aux.items()}
        g["out_tokens"] = out.cpu().numpy()[rows]
        g["num_accepted"] = n.cpu().numpy()[rows]
        return g

    def oracle_rows(top_p=None):
        parts = []
        for j, b in enumerate(rows):
            one = {key: v[j:j + 1] for key, v in h.items()}
            parts.append(oracle.spec_verify_ref(one["target"], one["draft"], one["draft_tokens"],
                                                one["draft_len"], one["temperature"], seed,
                                                seq_base=base + b,
                                                top_p=None if top_p is None else [top_p]))
        return {key: np.concatenate([p[key] for p in parts]) for key in parts[0]}

    ref = oracle_rows()
    g_full = pick(full)
    check(parity.compare(g_full, ref, h["draft_len"], h["temperature"], k), "sliced full")
    g_ee = pick(ee)
    for key in ("out_tokens", "num_accepted", "seq_status", "draw_kind"):
        assert np.array_equal(g_ee[key], g_full[key]), key
    check(parity.compare(pick(top), oracle_rows(0.9), h["draft_len"], h["temperature"], k),
          "sliced top-p")


def test_sliced_tree_launches_match_the_oracle():
    B, N, V = 70_000, 64, 16
    assert B * N > SLICE_ITEMS
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    t = (torch.randn((B, N, V), generator=g, device=DEV) * 2).contiguous()
    amax = t.argmax(dim=2)
    par = torch.zeros((B, N), dtype=torch.int64, device=DEV)
    par[:, 1:] = (torch.rand((B, N - 1), generator=g, device=DEV)
                  * torch.arange(1, N, device=DEV)).long()
    hit = torch.rand((B, N), generator=g, device=DEV) < 0.8
    tok = torch.where(hit, torch.gather(amax, 1, par), torch.zeros_like(par))
    par[:, 0] = -1
    tok[:, 0] = 0
    par = par.to(torch.int32).contiguous()
    tok = tok.to(torch.int32).contiguous()
    nn = torch.full((B,), N, dtype=torch.int32, device=DEV)
    out, path, n, aux = sv.spec_verify_tree(t, par, tok, nn, aux=True)
    torch.cuda.synchronize()
    per_slice = SLICE_ITEMS // N
    rows = list(range(per_slice - 30, per_slice + 30)) + list(range(B - 10, B))
    idx = torch.as_tensor(rows, device=DEV)
    ref = oracle.spec_tree_ref(t[idx].cpu().numpy(), par[idx].cpu().numpy(),
                               tok[idx].cpu().numpy(), nn[idx].cpu().numpy())
    np.testing.assert_array_equal(out.cpu().numpy()[rows], ref["out_tokens"])
    np.testing.assert_array_equal(path.cpu().numpy()[rows], ref["path_nodes"])
    np.testing.assert_array_equal(n.cpu().numpy()[rows], ref["num_accepted"])
