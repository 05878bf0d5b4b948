"""Seeded synthetic inputs for the speculative-sampling verification step.

This module only *draws inputs*: target logits at k+1 positions, draft logits at
k positions, the drafted tokens, per-sequence draft lengths and temperatures.
It holds none of the verification arithmetic (no softmax, no acceptance test,
no residual, no inverse CDF), so both the fp64 oracle and the HIP path can
consume its output without sharing any of the method's code.

Recipe (one entry of ``WORKLOADS`` per shape; all draws come from one
``torch.Generator`` seeded with the workload's input seed, in the fixed order
written in :func:`generate`):

* target logits ~ N(0, sigma_t^2), optionally plus
  - ``boost`` added to ``boost_count`` distinct random tokens of every row, or
  - a Zipf-ranked bias ``-s * ln(rank(tok))`` where ``rank`` comes from one
    seeded permutation of 1..V shared by all rows (a stand-in for a vocabulary
    ordered by frequency);
* draft logits = target + N(0, sigma_d^2) noise, sigma_d fixed or drawn per
  sequence from U(lo, hi);
* both are rounded once to the storage dtype (bf16 round-to-nearest-even);
* temperature is fixed or drawn per sequence from a set; 0 selects greedy;
* draft length is k or drawn per sequence from U{1..k};
* drafted token g_i is drawn from the draft model's own distribution at the
  sequence's temperature (Gumbel-max on the *rounded* draft logits, so g really
  is a sample of what the verifier sees), or is the draft argmax when the
  temperature is 0; positions at or beyond the draft length hold -1 (they must
  be ignored by every consumer).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple, Union

import torch

DTYPE_F32 = 0
DTYPE_BF16 = 1

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_DTYPE_CODE = {"f32": DTYPE_F32, "bf16": DTYPE_BF16}
_ELEM_BYTES = {"f32": 4, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    """Shape and value distribution of one synthetic verification batch."""

    name: str
    B: int
    k: int
    V: int
    dtype: str  # "f32" | "bf16"
    target_sigma: float
    draft_sigma: Union[float, Tuple[float, float]]  # fixed, or per-sequence U(lo, hi)
    temperature: Union[float, Tuple[float, ...]]  # fixed, or per-sequence choice
    ragged: bool = False  # draft length ~ U{1..k} per sequence
    boost_count: int = 0  # tokens per row raised by `boost`
    boost: float = 0.0
    zipf_s: Optional[float] = None  # Zipf-ranked additive bias exponent
    seed: int = 0
    description: str = ""

    @property
    def dtype_code(self) -> int:
        return _DTYPE_CODE[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return _ELEM_BYTES[self.dtype]

    @property
    def positions(self) -> int:
        """Verified draft positions per call, B*(k+1)."""
        return self.B * (self.k + 1)

    def with_batch(self, B: int, name: Optional[str] = None) -> "Workload":
        d = dict(self.__dict__)
        d["B"] = B
        d["name"] = name or f"{self.name}[B={B}]"
        return Workload(**d)


def _c(i: int) -> int:
    return 1000 * i + 1


WORKLOADS = {
    "c1": Workload(
        "c1", B=4, k=4, V=1024, dtype="f32", target_sigma=2.0, draft_sigma=0.5,
        temperature=1.0, seed=_c(1),
        description="B=4 k=4 V=1024 fp32, target N(0,4), draft +N(0,0.25), tau 1",
    ),
    "c2": Workload(
        "c2", B=8, k=4, V=32000, dtype="f32", target_sigma=3.0, draft_sigma=0.7,
        temperature=1.0, boost_count=20, boost=8.0, seed=_c(2),
        description="B=8 k=4 V=32000 fp32, target N(0,9)+8 on 20 tokens/row, draft +N(0,0.49), tau 1",
    ),
    "c3": Workload(
        "c3", B=64, k=5, V=128256, dtype="bf16", target_sigma=3.0, draft_sigma=1.0,
        temperature=0.7, zipf_s=1.1, seed=_c(3),
        description="B=64 k=5 V=128256 bf16, target N(0,9)+Zipf(1.1) bias, draft +N(0,1), tau 0.7",
    ),
    "c4": Workload(
        "c4", B=256, k=4, V=152064, dtype="bf16", target_sigma=3.0, draft_sigma=1.0,
        temperature=(0.0, 0.6, 1.0), ragged=True, zipf_s=1.1, seed=_c(4),
        description="B=256 k=4 V=152064 bf16, Zipf target, draft +N(0,1), tau in {0,0.6,1}, L~U{1..4}",
    ),
    "c5": Workload(
        "c5", B=1024, k=7, V=128256, dtype="bf16", target_sigma=3.0, draft_sigma=(0.2, 2.0),
        temperature=0.8, ragged=True, zipf_s=1.1, seed=_c(5),
        description="B=1024 k=7 V=128256 bf16, Zipf target, draft +N(0,s_b^2) s_b~U(0.2,2), tau 0.8, L~U{1..7}",
    ),
}


def philox_seeds(name: str, count: int = 8) -> list:
    """Verification seeds used for a workload: 0xC0FFEE00 + index + 2^32 * r."""
    idx = int(name[1:]) if name[:1] == "c" and name[1:].isdigit() else 0
    return [0xC0FFEE00 + idx + (r << 32) for r in range(count)]


@dataclass
class Batch:
    """One verification batch. Tensors live on the device they were drawn on."""

    workload: Workload
    target: torch.Tensor  # [B, k+1, V] storage dtype
    draft: torch.Tensor  # [B, k, V] storage dtype
    draft_tokens: torch.Tensor  # [B, k] int32; -1 at positions >= draft_len
    draft_len: torch.Tensor  # [B] int32 in 1..k
    temperature: torch.Tensor  # [B] float32; 0 = greedy
    extras: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return self.target.shape[0]

    @property
    def k(self) -> int:
        return self.draft_tokens.shape[1]

    @property
    def V(self) -> int:
        return self.target.shape[2]

    def rows_read(self) -> Tuple[int, int]:
        """(target rows, draft rows) that one verification call must read once.

        Target rows 0..L_b of every sequence; draft rows 0..L_b-1 of sampling
        sequences only (greedy sequences never need the draft distribution).
        """
        L = self.draft_len.to("cpu", torch.int64)
        tau = self.temperature.to("cpu")
        t_rows = int((L + 1).sum())
        d_rows = int(L[tau > 0].sum())
        return t_rows, d_rows

    def algorithmic_bytes(self) -> int:
        """Bytes one verification call must read: each needed logit row once."""
        t_rows, d_rows = self.rows_read()
        return (t_rows + d_rows) * self.V * self.workload.elem_bytes

    def select(self, seqs: Sequence[int]) -> "Batch":
        """Host copy of a subset of sequences (same values, in the given order)."""
        idx = torch.as_tensor(list(seqs), dtype=torch.int64, device=self.target.device)
        return Batch(
            self.workload,
            self.target.index_select(0, idx).cpu(),
            self.draft.index_select(0, idx).cpu(),
            self.draft_tokens.index_select(0, idx).cpu(),
            self.draft_len.index_select(0, idx).cpu(),
            self.temperature.index_select(0, idx).cpu(),
            dict(self.extras),
        )


def _gumbel_like(shape, gen, device) -> torch.Tensor:
    u = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    # Map u in [0,1) to (0,1) before the double log.
    u = u.clamp_(min=float.fromhex("0x1p-30"), max=1.0 - float.fromhex("0x1p-24"))
    return -torch.log(-torch.log(u))


def generate(w: Workload, device: Union[str, torch.device] = "cpu", seq_block: int = 64) -> Batch:
    """Draw one batch for workload ``w`` on ``device``.

    The draw order is fixed: Zipf permutation, per-sequence draft sigma,
    temperatures, draft lengths, then per block of ``seq_block`` sequences:
    target noise, boosts, draft noise, Gumbel noise. The same seed on the same
    device type gives the same batch.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    B, k, V = w.B, w.k, w.V
    sdt = _TORCH_DTYPE[w.dtype]

    bias = None
    if w.zipf_s is not None:
        perm = torch.randperm(V, generator=gen, device=device)
        rank = (perm + 1).to(torch.float32)
        bias = -w.zipf_s * torch.log(rank)

    if isinstance(w.draft_sigma, tuple):
        lo, hi = w.draft_sigma
        dsig = lo + (hi - lo) * torch.rand(B, generator=gen, device=device)
    else:
        dsig = torch.full((B,), float(w.draft_sigma), device=device)

    if isinstance(w.temperature, tuple):
        choices = torch.tensor(w.temperature, dtype=torch.float32, device=device)
        tidx = torch.randint(len(w.temperature), (B,), generator=gen, device=device)
        tau = choices[tidx]
    else:
        tau = torch.full((B,), float(w.temperature), dtype=torch.float32, device=device)

    if w.ragged:
        L = torch.randint(1, k + 1, (B,), generator=gen, device=device, dtype=torch.int64)
    else:
        L = torch.full((B,), k, dtype=torch.int64, device=device)

    target = torch.empty((B, k + 1, V), dtype=sdt, device=device)
    draft = torch.empty((B, k, V), dtype=sdt, device=device)
    tokens = torch.empty((B, k), dtype=torch.int64, device=device)
    for b0 in range(0, B, seq_block):
        b1 = min(B, b0 + seq_block)
        nb = b1 - b0
        t = torch.randn((nb, k + 1, V), generator=gen, device=device) * w.target_sigma
        if w.boost_count:
            keys = torch.rand((nb, k + 1, V), generator=gen, device=device)
            hot = keys.topk(w.boost_count, dim=-1).indices
            t.scatter_add_(-1, hot, torch.full(hot.shape, w.boost, device=device))
            del keys, hot
        if bias is not None:
            t += bias
        d = t[:, :k, :] + torch.randn((nb, k, V), generator=gen, device=device) * dsig[b0:b1, None, None]
        target[b0:b1] = t.to(sdt)
        draft[b0:b1] = d.to(sdt)
        del t, d
        # Drafted tokens: a sample of the draft's own tempered distribution,
        # taken by Gumbel-max on the stored (rounded) draft logits.
        x = draft[b0:b1].to(torch.float32)
        g = _gumbel_like(x.shape, gen, device)
        tb = tau[b0:b1]
        safe = torch.where(tb > 0, tb, torch.ones_like(tb))[:, None, None]
        sampled = (x / safe + g).argmax(dim=-1)
        greedy = x.argmax(dim=-1)
        tokens[b0:b1] = torch.where((tb > 0)[:, None], sampled, greedy)
        del x, g, sampled, greedy

    pos = torch.arange(k, device=device)[None, :]
    tokens = torch.where(pos < L[:, None], tokens, torch.full_like(tokens, -1))
    return Batch(
        w,
        target.contiguous(),
        draft.contiguous(),
        tokens.to(torch.int32).contiguous(),
        L.to(torch.int32).contiguous(),
        tau.contiguous(),
        {"draft_sigma": dsig.cpu()},
    )


def to_host_arrays(batch: Batch) -> dict:
    """Numpy views for consumers that take raw host buffers.

    bf16 logits are returned as their raw uint16 bit patterns.
    """
    import numpy as np

    def logits(t: torch.Tensor):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    return {
        "target": logits(batch.target),
        "draft": logits(batch.draft),
        "dtype": batch.workload.dtype_code,
        "draft_tokens": batch.draft_tokens.detach().cpu().numpy().astype(np.int32),
        "draft_len": batch.draft_len.detach().cpu().numpy().astype(np.int32),
        "temperature": batch.temperature.detach().cpu().numpy().astype(np.float32),
    }


# ---------------------------------------------------------------------------
# Candidate trees (greedy tree verification).
#
# Recipe: level widths are fixed per workload (level d holds widths[d-1]
# nodes, numbered breadth first after the root); each node of level d picks
# its parent uniformly from level d-1. Target rows are drawn as for the
# linear workloads (N(0, sigma^2) plus the Zipf-ranked bias, rounded to the
# storage dtype). A node's children carry the best-ranked distinct tokens of
# a draft row at that node (target row + N(0, sigma_d^2), never stored): the
# first child the draft's top token, the second its runner-up, and so on, as
# a tree drafter expands its most likely candidates. The draft noise sets
# how often a child hits the target's argmax.
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class TreeWorkload:
    name: str
    B: int
    V: int
    dtype: str
    widths: Tuple[int, ...]  # nodes per level below the root
    target_sigma: float = 3.0
    draft_sigma: float = 1.0
    zipf_s: Optional[float] = 1.1
    seed: int = 0
    description: str = ""

    @property
    def N(self) -> int:
        return 1 + sum(self.widths)

    @property
    def dtype_code(self) -> int:
        return _DTYPE_CODE[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return _ELEM_BYTES[self.dtype]


TREE_WORKLOADS = {
    "t1": TreeWorkload("t1", B=4, V=1024, dtype="f32", widths=(3, 4, 4, 3, 1),
                       target_sigma=2.0, draft_sigma=0.7, zipf_s=None, seed=7001,
                       description="B=4 N=16 V=1024 fp32 trees, widths 3-4-4-3-1"),
    "t2": TreeWorkload("t2", B=16, V=32000, dtype="f32", widths=(4, 8, 12, 12, 10, 8, 6, 3),
                       draft_sigma=1.0, seed=7002,
                       description="B=16 N=64 V=32000 fp32 trees, 8 levels"),
    "t3": TreeWorkload("t3", B=128, V=128256, dtype="bf16", widths=(4, 8, 12, 12, 10, 8, 6, 3),
                       draft_sigma=1.0, seed=7003,
                       description="B=128 N=64 V=128256 bf16 trees, 8 levels (widths "
                                   "4-8-12-12-10-8-6-3)"),
}


@dataclass
class TreeBatch:
    workload: TreeWorkload
    target: torch.Tensor  # [B, N, V]
    parents: torch.Tensor  # [B, N] int32, -1 at the root
    tokens: torch.Tensor  # [B, N] int32, 0 at the root
    n_nodes: torch.Tensor  # [B] int32

    def bytes_read(self) -> int:
        """Each node row once."""
        return int(self.n_nodes.to(torch.int64).sum()) * self.workload.V * self.workload.elem_bytes


def generate_tree(w: TreeWorkload, device: Union[str, torch.device] = "cpu",
                  seq_block: int = 16) -> TreeBatch:
    """Draw one batch of candidate trees for ``w`` on ``device``. Draw order:
    Zipf permutation, parents (level by level), then per block of sequences
    target noise and draft noise."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    B, N, V = w.B, w.N, w.V
    sdt = _TORCH_DTYPE[w.dtype]
    bias = None
    if w.zipf_s is not None:
        perm = torch.randperm(V, generator=gen, device=device)
        bias = -w.zipf_s * torch.log((perm + 1).to(torch.float32))
    parents = torch.full((B, N), -1, dtype=torch.int64, device=device)
    first = [1]
    for d, width in enumerate(w.widths):
        first.append(first[-1] + width)
    for d, width in enumerate(w.widths):
        lo, hi = first[d], first[d + 1]
        plo, phi = (0, 1) if d == 0 else (first[d - 1], first[d])
        parents[:, lo:hi] = torch.randint(plo, phi, (B, width), generator=gen, device=device)
    par_cpu = parents.cpu()
    # rank of each node among its siblings (by node index)
    rank = torch.zeros((B, N), dtype=torch.int64)
    for b in range(B):
        seen = {}
        for n in range(1, N):
            pnode = int(par_cpu[b, n])
            rank[b, n] = seen.get(pnode, 0)
            seen[pnode] = int(rank[b, n]) + 1
    kmax = int(rank.max()) + 1 if N > 1 else 1
    rank = rank.to(device)
    target = torch.empty((B, N, V), dtype=sdt, device=device)
    tokens = torch.zeros((B, N), dtype=torch.int64, device=device)
    for b0 in range(0, B, seq_block):
        b1 = min(B, b0 + seq_block)
        nb = b1 - b0
        t = torch.randn((nb, N, V), generator=gen, device=device) * w.target_sigma
        if bias is not None:
            t += bias
        target[b0:b1] = t.to(sdt)
        d = target[b0:b1].to(torch.float32) + \
            torch.randn((nb, N, V), generator=gen, device=device) * w.draft_sigma
        top = d.topk(kmax, dim=-1).indices  # [nb, N, kmax]
        del t, d
        par = parents[b0:b1].clamp(min=0)
        cand = torch.gather(top, 1, par[:, :, None].expand(nb, N, kmax))  # parent's list
        tokens[b0:b1] = torch.gather(cand, 2, rank[b0:b1, :, None]).squeeze(2)
    tokens[:, 0] = 0
    return TreeBatch(w, target.contiguous(), parents.to(torch.int32).contiguous(),
                     tokens.to(torch.int32).contiguous(),
                     torch.full((B,), N, dtype=torch.int32, device=device))


def tree_to_host_arrays(batch: TreeBatch) -> dict:
    import numpy as np

    t = batch.target.detach().cpu().contiguous()
    target = t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
    return {"target": target,
            "parents": batch.parents.cpu().numpy().astype(np.int32),
            "tokens": batch.tokens.cpu().numpy().astype(np.int32),
            "n_nodes": batch.n_nodes.cpu().numpy().astype(np.int32)}


# ---------------------------------------------------------------------------
# Contexts for prompt lookup.
#
# Recipe (copy-heavy text, as in summarisation, code editing or RAG): a
# context is a run of segments; each is, with probability copy_p, a copy of
# an earlier stretch of the same context (start uniform, length geometric
# with mean copy_len), else fresh tokens uniform in [0, vocab) (length
# geometric with mean fresh_len). The context then ends part-way through one
# more copied stretch, so its last tokens have occurred before. Lengths are
# U{T_max/2..T_max} per sequence. numpy Generator seeded per workload.
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class LookupWorkload:
    name: str
    B: int
    T_max: int
    vocab: int
    n_min: int
    n_max: int
    k: int
    copy_p: float = 0.3
    copy_len: int = 32
    fresh_len: int = 64
    seed: int = 0
    description: str = ""


LOOKUP_WORKLOADS = {
    "p1": LookupWorkload("p1", B=8, T_max=256, vocab=50, n_min=1, n_max=3, k=5, copy_len=8,
                         fresh_len=16, seed=8001,
                         description="B=8 T<=256 vocab 50, n 1..3, k 5"),
    "p2": LookupWorkload("p2", B=64, T_max=4096, vocab=32000, n_min=1, n_max=4, k=7, seed=8002,
                         description="B=64 T<=4096 vocab 32000, n 1..4, k 7"),
    "p3": LookupWorkload("p3", B=1024, T_max=32768, vocab=128256, n_min=1, n_max=4, k=7,
                         seed=8003,
                         description="B=1024 T<=32768 vocab 128256, n 1..4, k 7, copy-heavy"),
}


def generate_contexts(w: LookupWorkload):
    """(contexts [B, T_max] int32, context_len [B] int32) as numpy arrays; the
    unused tail of a row holds -7 (never read)."""
    import numpy as np

    rng = np.random.default_rng(w.seed)
    ctx = np.full((w.B, w.T_max), -7, dtype=np.int32)
    lens = rng.integers(w.T_max // 2, w.T_max + 1, size=w.B).astype(np.int32)
    for b in range(w.B):
        T = int(lens[b])
        row = ctx[b]
        pos = 0
        while pos < T:
            if pos > 8 and rng.random() < w.copy_p:
                ln = min(int(rng.geometric(1.0 / w.copy_len)), T - pos)
                src = int(rng.integers(0, pos))
                for j in range(ln):  # may overlap itself: copy token by token
                    row[pos + j] = row[src + j]
            else:
                ln = min(int(rng.geometric(1.0 / w.fresh_len)), T - pos)
                row[pos:pos + ln] = rng.integers(0, w.vocab, size=ln)
            pos += ln
        # end inside a copied stretch: overwrite the last few tokens by a copy
        if T > 16:
            ln = int(rng.integers(2, min(12, T // 4) + 1))
            src = int(rng.integers(0, T - ln - 1))
            row[T - ln:T] = row[src:src + ln].copy()
    return ctx, lens


__all__ = [
    "LookupWorkload", "LOOKUP_WORKLOADS", "generate_contexts",
    "TreeWorkload", "TreeBatch", "TREE_WORKLOADS", "generate_tree", "tree_to_host_arrays",
    "Workload", "Batch", "WORKLOADS", "generate", "philox_seeds", "to_host_arrays",
    "DTYPE_F32", "DTYPE_BF16",
]
