"""GPU-versus-oracle parity protocol (test infrastructure).

Compares the outputs of the HIP library with the fp64 oracle on the same
inputs, sequence by sequence:

* status codes must match (a draft probability that underflows fp32 is the
  one documented exception: the GPU reports QZERO where the oracle's exact
  q(g) is positive but below FLT_MIN);
* greedy sequences: argmax rows, tokens and counts bit-exact;
* sampling sequences: p_i(g_i) and q_i(g_i) within ``rel`` (plus an absolute
  floor for fp32 underflow), and every accept decision and the final token
  bit-exact, except where the oracle's uniform lies within ``band`` of its
  decision threshold or CDF boundary. The first such draw of a sequence
  ends the comparison of that sequence (a flip there cascades) and is
  counted as flagged. A row whose own nucleus boundary lies within the
  band has its gathered values skipped (counted as ``boundary_values``).
  The residual mass S is compared wherever the final draw is compared,
  within ``rel`` plus the absolute ``RESID_ABS`` derived below.

A final draw's band is ``band`` or, where that is larger, the fp32
resolution of the CDF it scans (``band_draw`` from the oracle: 8 * 2^-24 *
sqrt(sum max(p, q)^2) / S). It exceeds ``band`` only when S is small against
the largest weights the kernel rounds, as when two nearly equal rows put
almost all their mass on one token; such draws are counted in
``flagged_wide``. Where it reaches 1 and one side's fp32 residual rounded to
nothing (kind RESIDUAL against RESIDUAL_AS_P), the draw is unresolved and
counted as one flagged draw.

A flagged final draw on which the two sides part must still land inside the
oracle's band window: the token ids that the oracle's own draw would pick
with its uniform moved by at most the draw's band. A disagreement outside
that window is a mismatch however small the oracle's margin, so a locate
error among low-weight tokens (whose margins are always below the band) is
caught.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from . import DRAW_GREEDY, DRAW_RESIDUAL, DRAW_RESIDUAL_AS_P, SEQ_OK, SEQ_QZERO, spec_verify_ref

FLT_MIN = float(np.finfo(np.float32).tiny)


def host_threads(cap: int = 16) -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def oracle_on(host: dict, seed: int, seqs=None, nthreads: int = 1, top_p=None,
              top_k=None) -> dict:
    """Run the oracle on all sequences, or on the listed ones (each with its
    own global index as the Philox sequence index). ``top_p`` / ``top_k``:
    None, or [B] filter parameters."""
    t, d, g, L, tau = (host["target"], host["draft"], host["draft_tokens"], host["draft_len"],
                       host["temperature"])
    tp = None if top_p is None else np.broadcast_to(np.asarray(top_p, np.float32), (len(L),))
    tk = None if top_k is None else np.broadcast_to(np.asarray(top_k, np.int32), (len(L),))
    if seqs is None:
        return spec_verify_ref(t, d, g, L, tau, seed, seq_base=0, nthreads=nthreads, top_p=tp,
                               top_k=tk)
    seqs = [int(b) for b in seqs]

    def one(b):
        return spec_verify_ref(t[b:b + 1], d[b:b + 1], g[b:b + 1], L[b:b + 1], tau[b:b + 1], seed,
                               seq_base=b, top_p=None if tp is None else tp[b:b + 1],
                               top_k=None if tk is None else tk[b:b + 1])

    if nthreads > 1:
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            parts = list(ex.map(one, seqs))
    else:
        parts = [one(b) for b in seqs]
    return {key: np.concatenate([p[key] for p in parts]) for key in parts[0]}


@dataclass
class Report:
    """Counts over compared draws. A draw is one acceptance test or one final
    (correction/bonus) draw. ``flagged`` counts draws whose oracle margin is
    below the band; ``flagged_disagree`` those of them where the GPU took the
    other branch/token (allowed); ``mismatches`` lists disagreements outside
    the band (never allowed) and value/status errors."""

    sequences: int = 0
    draws: int = 0
    flagged: int = 0
    flagged_disagree: int = 0
    flagged_wide: int = 0  # flagged only by a final draw's band wider than `band`
    boundary_status: int = 0
    boundary_values: int = 0
    compared_tokens: int = 0
    max_disagree_margin: float = 0.0
    resid_compared: int = 0
    max_abs_dS: float = 0.0
    max_rel_dS_large: float = 0.0  # over S > S_LARGE, where 1e-5 * S exceeds RESID_ABS
    band_counts: dict = field(default_factory=dict)
    mismatches: list = field(default_factory=list)

    def merge(self, other: "Report") -> "Report":
        self.sequences += other.sequences
        self.draws += other.draws
        self.flagged += other.flagged
        self.flagged_disagree += other.flagged_disagree
        self.flagged_wide += other.flagged_wide
        self.boundary_status += other.boundary_status
        self.boundary_values += other.boundary_values
        self.compared_tokens += other.compared_tokens
        self.max_disagree_margin = max(self.max_disagree_margin, other.max_disagree_margin)
        self.resid_compared += other.resid_compared
        self.max_abs_dS = max(self.max_abs_dS, other.max_abs_dS)
        self.max_rel_dS_large = max(self.max_rel_dS_large, other.max_rel_dS_large)
        for key, v in other.band_counts.items():
            self.band_counts[key] = self.band_counts.get(key, 0) + v
        self.mismatches += other.mismatches
        return self

    @property
    def flagged_fraction(self) -> float:
        return self.flagged / max(1, self.draws)

    def ok(self) -> bool:
        return not self.mismatches

    def summary(self) -> str:
        bands = " ".join(f"<{b:g}:{n}" for b, n in sorted(self.band_counts.items(), reverse=True))
        head = (f"sequences={self.sequences} draws={self.draws} flagged={self.flagged} "
                f"({self.flagged_fraction:.2e}) flagged_wide={self.flagged_wide} "
                f"flagged_disagree={self.flagged_disagree} "
                f"max_disagree_margin={self.max_disagree_margin:.2e} margins[{bands}] "
                f"boundary_status={self.boundary_status} boundary_values={self.boundary_values} "
                f"S_compared={self.resid_compared} max|dS|={self.max_abs_dS:.2e} "
                f"max_rel_dS(S>{S_LARGE:.2f})={self.max_rel_dS_large:.2e} "
                f"mismatches={len(self.mismatches)}")
        return head + ("" if not self.mismatches else "\n  " + "\n  ".join(self.mismatches[:20]))


BANDS = (1e-6, 1e-7, 1e-8, 1e-9)


def _close(a: float, b: float, rel: float, floor: float) -> bool:
    if np.isnan(a) and np.isnan(b):
        return True
    return abs(a - b) <= rel * abs(b) + floor


# Absolute part of the residual-mass tolerance. S = sum_v max(0, p(v) - q(v))
# is a difference of fp32 softmax values, so its rounding error scales with
# sum_v (p(v) + q(v)) = 2 (or the two kept masses), not with S: every p(v)
# carries a relative error of a few ulps from the normaliser and the exp2,
# plus ln2 * |t| ulps from rounding its exponent t = (x - m) * s; weighted by
# p that mean |t| is at most log2(V) + a few bits (the row's entropy), under
# 17 bits for V <= 131072. Two rows of (4 + 0.7 * 17) < 16 ulps each give
# 32 ulps of fp32 epsilon 2^-24, i.e. 2^-19.
RESID_ABS = 2.0 ** -19
# Above this S the relative part of the tolerance (1e-5 * S) is the larger.
S_LARGE = RESID_ABS / 1e-5


def compare(gpu: dict, ref: dict, draft_len, temperature, k: int, rows=None, rel: float = 1e-5,
            floor: float = 1e-30, band: float = 1e-6, label: str = "") -> Report:
    """Compare GPU outputs (numpy, for the sequences in ``rows`` of the GPU
    batch, or all) with oracle outputs for the same sequences."""
    rep = Report(band_counts={b: 0 for b in BANDS})
    n_ref = ref["num_accepted"].shape[0]
    rows = list(range(n_ref)) if rows is None else [int(r) for r in rows]

    def draw(margin: float, agree: bool, what: str, in_window: bool = True,
             band_here: float = band) -> bool:
        """Account one draw; returns False when the comparison must stop.
        ``in_window``: for a final draw, whether the GPU's token lies in the
        oracle's band window (a flagged disagreement must). ``band_here``:
        the draw's own flag band (a final draw's may be wider than ``band``
        where fp32 weights cannot resolve it)."""
        rep.draws += 1
        for b_ in BANDS:
            if margin < b_:
                rep.band_counts[b_] += 1
        if margin < band_here:
            rep.flagged += 1
            if not margin < band:
                rep.flagged_wide += 1
            if not agree:
                rep.flagged_disagree += 1
                rep.max_disagree_margin = max(rep.max_disagree_margin, margin)
                if not in_window:
                    rep.mismatches.append(what + f" (flagged, margin {margin:.3e}, but outside "
                                          "the oracle's band window)")
                return False
            return True
        if not agree:
            rep.max_disagree_margin = max(rep.max_disagree_margin, margin)
            rep.mismatches.append(what + f" (oracle margin {margin:.3e})")
            return False
        return True

    for j, b in enumerate(rows):
        rep.sequences += 1
        tag = f"{label}b={b}"
        L = int(draft_len[b])
        tau = float(temperature[b])
        gs, rs = int(gpu["seq_status"][b]), int(ref["seq_status"][j])
        g_out, r_out = gpu["out_tokens"][b], ref["out_tokens"][j]
        g_n, r_n = int(gpu["num_accepted"][b]), int(ref["num_accepted"][j])
        if gs != rs:
            qg = ref["q_g"][j]
            if gs == SEQ_QZERO and rs == SEQ_OK and np.nanmin(qg[:max(L, 1)]) < FLT_MIN:
                rep.boundary_status += 1
                continue
            if "margin_nucleus" in ref and SEQ_QZERO in (gs, rs):
                # a draft token on a nucleus boundary within the band: in on
                # one side, out (q = 0) on the other
                mn = ref["margin_nucleus"][j]
                near = [x for x in mn if not np.isnan(x) and x < band]
                if near:
                    draw(min(near), False, f"{tag}: nucleus boundary status")
                    continue
            rep.mismatches.append(f"{tag}: status gpu={gs} oracle={rs}")
            continue
        if gs != SEQ_OK:
            if not (np.all(g_out == -1) and g_n == 0):
                rep.mismatches.append(f"{tag}: error status {gs} but outputs not cleared")
            continue
        if tau == 0.0:
            rep.draws += 1
            if not np.array_equal(gpu["argmax"][b, :L + 1], ref["argmax"][j, :L + 1]):
                rep.mismatches.append(f"{tag}: greedy argmax {gpu['argmax'][b, :L + 1]} vs "
                                      f"{ref['argmax'][j, :L + 1]}")
            if g_n != r_n or not np.array_equal(g_out, r_out):
                rep.mismatches.append(f"{tag}: greedy tokens {g_out}/{g_n} vs {r_out}/{r_n}")
            if int(gpu["draw_kind"][b]) != DRAW_GREEDY:
                rep.mismatches.append(f"{tag}: greedy draw_kind {gpu['draw_kind'][b]}")
            rep.compared_tokens += r_n + 1
            continue
        # a nucleus boundary within the band on a row the round depends on
        # (target rows 0..n, draft rows 0..min(n, L-1)) may legitimately
        # differ: the whole sequence counts as one flagged draw
        mn = ref.get("margin_nucleus")
        if mn is not None:
            mn = mn[j]
            dep = list(range(min(r_n, L) + 1)) + [k + 1 + i for i in range(min(r_n + 1, L))]
            near = [mn[x] for x in dep if not np.isnan(mn[x]) and mn[x] < band]
            if near:
                agree = (g_n == r_n and np.array_equal(g_out, r_out))
                draw(min(near), agree, f"{tag}: nucleus boundary")
                continue
        # sampling: gathered probabilities at every valid position, except on
        # a row (past the stop) whose own nucleus boundary lies within the
        # band: its kept set, hence its renormalised values, may differ
        for i in range(L):
            for key, r_ in (("p_g", i), ("q_g", k + 1 + i)):
                if mn is not None and not np.isnan(mn[r_]) and mn[r_] < band:
                    rep.boundary_values += 1
                    continue
                a, o = float(gpu[key][b, i]), float(ref[key][j, i])
                if not _close(a, o, rel, floor):
                    rep.mismatches.append(f"{tag}: {key}[{i}] gpu={a!r} oracle={o!r} "
                                          f"rel={abs(a - o) / max(abs(o), 1e-300):.2e}")
        # acceptance tests, left to right, until the two sides part
        going = True
        for i in range(min(r_n + 1, L)):
            ref_acc = i < r_n
            gpu_acc = g_n > i
            if not draw(float(ref["margin_accept"][j, i]), ref_acc == gpu_acc,
                        f"{tag}: accept test {i}: gpu {gpu_acc} oracle {ref_acc}"):
                going = False
                break
            if ref_acc:
                rep.compared_tokens += 1
                if g_out[i] != r_out[i]:
                    rep.mismatches.append(f"{tag}: accepted token {i}: {g_out[i]} vs {r_out[i]}")
        if not going:
            continue
        if g_n != r_n:
            rep.mismatches.append(f"{tag}: accepted count {g_n} vs {r_n}")
            continue
        # the final draw's flag band: the oracle's (ref_draw_band), at least `band`
        bd = float(ref["band_draw"][j]) if "band_draw" in ref else float("nan")
        band_here = max(band, bd) if np.isfinite(bd) else band
        kinds = {int(gpu["draw_kind"][b]), int(ref["draw_kind"][j])}
        if band_here >= 1.0 and kinds == {DRAW_RESIDUAL, DRAW_RESIDUAL_AS_P}:
            # a residual that fp32 cannot tell from zero on one side: its
            # mass, kind and token are all unresolved; one flagged draw
            draw(0.0, False, f"{tag}: unresolved residual", True, band_here)
            continue
        if len(kinds) > 1:
            rep.mismatches.append(f"{tag}: draw kind {gpu['draw_kind'][b]} vs {ref['draw_kind'][j]}")
        S_g, S_r = float(gpu["resid_mass"][b]), float(ref["resid_mass"][j])
        rep.resid_compared += 1
        dS = abs(S_g - S_r)
        rep.max_abs_dS = max(rep.max_abs_dS, dS)
        if S_r > S_LARGE:
            rep.max_rel_dS_large = max(rep.max_rel_dS_large, dS / S_r)
        if not _close(S_g, S_r, rel, RESID_ABS):
            rep.mismatches.append(f"{tag}: resid_mass gpu={S_g!r} oracle={S_r!r}")
        if not np.array_equal(g_out[r_n + 1:], r_out[r_n + 1:]):
            rep.mismatches.append(f"{tag}: padding {g_out} vs {r_out}")
        lo, hi = (int(x) for x in ref["draw_window"][j]) if "draw_window" in ref else (-1, -1)
        in_window = "draw_window" in ref and lo <= int(g_out[r_n]) <= hi
        if draw(float(ref["margin_draw"][j]), g_out[r_n] == r_out[r_n],
                f"{tag}: final token {g_out[r_n]} vs {r_out[r_n]} (window {lo}..{hi})",
                in_window, band_here):
            rep.compared_tokens += 1
    return rep
