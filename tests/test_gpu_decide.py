"""The decision's own launch (draw grids above 4096 workgroups) issues its
loads early: the drafted tokens, the first eight chunk partials of each row
and the drafted tokens' logits go out with the draft length, before the
inputs are validated. Small grids take the plain decision inside the draw
kernel. Every output of a large batch must equal, bit for bit, what the same
sequences give in small slices (each with its global index as seq_base), and
match the oracle on sampled sequences, also with rows of more than eight
chunks, k = 0, and invalid token ids, lengths and temperatures mixed in."""
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
FOLD_ITEMS = 4096  # draw grids up to this many workgroups decide inside the draw kernel
CHUNK_BYTES = 32 * 1024


def _batch(B, k, V, dtype, seed, broken):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    t = torch.randn((B, k + 1, V), generator=g, device=DEV) * 2
    d = t[:, :k] + torch.randn((B, k, V), generator=g, device=DEV) * 0.7
    tau = torch.tensor([(0.0, 0.7, 1.0, 1.3)[b % 4] for b in range(B)], dtype=torch.float32,
                       device=DEV)
    L = torch.randint(0, k + 1, (B,), generator=g, device=DEV).to(torch.int32)
    if k > 0:
        top = d.argmax(dim=2).to(torch.int32)
        rnd = torch.randint(0, V, (B, k), generator=g, device=DEV).to(torch.int32)
        pick = torch.rand((B, k), generator=g, device=DEV) < 0.7
        tok = torch.where(pick, top, rnd)
    else:
        tok = torch.zeros((B, 0), dtype=torch.int32, device=DEV)
    if broken:
        # Out-of-range ids (the early gathers must skip them), and lengths and
        # temperatures the decision rejects.
        bad_ids = (-1, V, 2**31 - 1, -2**31)
        for j, b in enumerate(range(3, B, 97)):
            if k > 0:
                tok[b, j % k] = bad_ids[j % len(bad_ids)]
                L[b] = k
        for b in range(5, B, 211):
            L[b] = k + 1 if b % 2 else -1
        for b in range(7, B, 263):
            tau[b] = float("nan") if b % 2 else -0.5
    if dtype == "bf16":
        t, d = t.to(torch.bfloat16), d.to(torch.bfloat16)
    return t.contiguous(), d.contiguous(), tok.contiguous(), L.contiguous(), tau.contiguous()


def _host_rows(t, d, tok, L, tau, rows):
    idx = torch.as_tensor(rows, device=DEV)

    def arr(x):
        x = x[idx].cpu()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16)
        return x.numpy()

    return dict(target=arr(t), draft=arr(d), draft_tokens=arr(tok), draft_len=arr(L),
                temperature=arr(tau))


def _np(res):
    out, n, aux = res
    g = {key: v.cpu().numpy() for key, v in aux.items()}
    g["out_tokens"] = out.cpu().numpy()
    g["num_accepted"] = n.cpu().numpy()
    return g


CASES = [
    (600, 3, 152064, "bf16", False),  # 10 chunks a row: a second fold batch, bonus reload
    (5000, 0, 1000, "f32", False),    # k = 0: every sequence draws a bonus token
    (4500, 7, 2000, "bf16", True),    # invalid ids, lengths and temperatures mixed in
]


@pytest.mark.parametrize("B,k,V,dtype,broken", CASES)
def test_decision_launch_equals_in_draw_decisions(B, k, V, dtype, broken):
    nc = -(-V // (CHUNK_BYTES // (2 if dtype == "bf16" else 4)))
    assert B * nc > FOLD_ITEMS
    t, d, tok, L, tau = _batch(B, k, V, dtype, B + k, broken)
    seed = 0xD15C0
    say(f"[case] decision launch B={B} k={k} V={V} {dtype} nc={nc} broken={broken}")
    big = _np(sv.spec_verify(t, d, tok, L, tau, seed, aux=True))
    step = max(1, FOLD_ITEMS // nc // 2)  # slices small enough to decide in the draw kernel
    for s in range(0, B, step):
        e = min(B, s + step)
        small = _np(sv.spec_verify(t[s:e], d[s:e], tok[s:e], L[s:e], tau[s:e], seed,
                                   seq_base=s, aux=True))
        for key, v in small.items():
            assert np.array_equal(v, big[key][s:e], equal_nan=True), (key, s)
    torch.cuda.synchronize()
    rows = sorted(set(list(range(0, 16)) + list(range(B // 2, B // 2 + 16))
                      + list(range(B - 16, B)) + list(range(3, B, 97))[:24]))
    h = _host_rows(t, d, tok, L, tau, rows)
    parts = []
    for j, b in enumerate(rows):
        one = {key: v[j:j + 1] for key, v in h.items()}
        parts.append(oracle.spec_verify_ref(one["target"], one["draft"], one["draft_tokens"],
                                            one["draft_len"], one["temperature"], seed,
                                            seq_base=b))
    ref = {key: np.concatenate([p[key] for p in parts]) for key in parts[0]}
    g = {key: v[rows] for key, v in big.items()}
    check(parity.compare(g, ref, h["draft_len"], h["temperature"], k), f"decision B={B} k={k}")
    if broken:
        st = big["seq_status"]
        assert (st == sv.SEQ_BAD_TOKEN).any() and (st == sv.SEQ_BAD_LEN).any()
        assert (st == sv.SEQ_BAD_TEMP).any()
