"""Row passes that stream two chunks per workgroup: the row statistics of
spec_verify and the early-exit schedule take chunk pairs on grids of at least
16384 chunks. Rows whose chunk count is odd (a pair holding one chunk), whose
last chunk is short, or that are not 16-byte aligned (each chunk then goes
through the general chunk pass) are checked against the oracle on sampled
sequences, and the two schedules against each other on every sequence."""
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
PAIR_CHUNKS = 16384  # grids of at least this many chunks take pairs
CHUNK_BYTES = 32 * 1024


def _batch(B, k, V, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    t = torch.randn((B, k + 1, V), generator=g, device=DEV) * 2
    d = t[:, :k] + torch.randn((B, k, V), generator=g, device=DEV) * 0.7
    tau = torch.where(torch.arange(B, device=DEV) % 5 == 0, 0.0, 0.9).to(torch.float32)
    L = torch.randint(0, k + 1, (B,), generator=g, device=DEV).to(torch.int32)
    top = d.argmax(dim=2).to(torch.int32)  # accepted often: later positions get read
    rnd = torch.randint(0, V, (B, k), generator=g, device=DEV).to(torch.int32)
    pick = torch.rand((B, k), generator=g, device=DEV) < 0.7
    tok = torch.where(pick, top, rnd)
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


def _pick(res, rows):
    out, n, aux = res
    g = {key: v.cpu().numpy()[rows] for key, v in aux.items()}
    g["out_tokens"] = out.cpu().numpy()[rows]
    g["num_accepted"] = n.cpu().numpy()[rows]
    return g


# (V, dtype): chunk count nc, and why the case is there.
CASES = [
    (3 * 16384 - 8, "bf16"),   # nc = 3: the last pair holds one short chunk; single blocks
    (2 * 16384 + 3, "bf16"),   # nc = 3, V not a multiple of 8: odd rows misaligned
    (3 * 8192 + 5, "f32"),     # nc = 4 fp32 chunks, the last of 5 elements
]


@pytest.mark.parametrize("V,dtype", CASES)
def test_pair_passes_match_the_oracle_and_each_other(V, dtype):
    k = 2
    elems = CHUNK_BYTES // (2 if dtype == "bf16" else 4)
    nc = -(-V // elems)
    B = -(-PAIR_CHUNKS // (2 * nc)) + 3  # position 0 alone fills a pair grid
    assert B * 2 * nc >= PAIR_CHUNKS and B * (2 * k + 1) * nc >= PAIR_CHUNKS
    t, d, tok, L, tau = _batch(B, k, V, dtype, V)
    rows = sorted(set(list(range(0, 24)) + list(range(B // 2 - 12, B // 2 + 12))
                      + list(range(B - 24, B))))
    h = _host_rows(t, d, tok, L, tau, rows)
    for seed in (3, 0xC0FFEE1234):
        say(f"[case] pairs V={V} {dtype} nc={nc} B={B} k={k} seed={seed:#x}")
        full = sv.spec_verify(t, d, tok, L, tau, seed, aux=True)
        ee = sv.spec_verify_early_exit(t, d, tok, L, tau, seed, aux=True)
        torch.cuda.synchronize()
        for key in ("seq_status", "draw_row", "draw_kind"):
            assert torch.equal(ee[2][key], full[2][key]), key
        assert torch.equal(ee[0], full[0]) and torch.equal(ee[1], full[1])
        assert torch.equal(ee[2]["resid_mass"].view(torch.int32),
                           full[2]["resid_mass"].view(torch.int32))
        parts = []
        for j, b in enumerate(rows):
            one = {key: v[j:j + 1] for key, v in h.items()}
            parts.append(oracle.spec_verify_ref(one["target"], one["draft"], one["draft_tokens"],
                                                one["draft_len"], one["temperature"], seed,
                                                seq_base=b))
        ref = {key: np.concatenate([p[key] for p in parts]) for key in parts[0]}
        check(parity.compare(_pick(full, rows), ref, h["draft_len"], h["temperature"], k),
              f"pairs V={V} {dtype}")
