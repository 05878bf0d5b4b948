"""Host-side checks of the HIP library that need no GPU.

The library must load, export every function the header declares, size its
workspace, and reject bad arguments before it touches the device.
"""
import ctypes
import os
import re

import pytest

from conftest import ROOT

sv = pytest.importorskip("speculative_decoding_verification_11_amd")


def _header_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"typedef[^;]*;", "", text, flags=re.S)
        for m in re.finditer(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", text):
            name = m.group(1)
            if name.startswith("spec_"):
                names.add(name)
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.binding.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return sv.library()


def test_library_exports_every_declared_function(lib):
    declared = _header_functions()
    assert {"spec_verify", "spec_verify_workspace_size", "spec_verify_strerror",
            "spec_verify_version"} <= declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert set(sv.binding.EXPORTED) <= declared


def test_library_is_built_for_gfx950():
    data = open(sv.binding.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_workspace_size(lib):
    assert sv.workspace_size(0, 4, 1024, sv.F32) > 0
    assert sv.workspace_size(64, 5, 128256, sv.BF16) >= 64 * 11 * 8 * 8
    for bad in [(-1, 4, 10, 0), (1, -1, 10, 0), (1, 64, 10, 0), (1, 4, 0, 0), (1, 4, 10, 2)]:
        assert sv.workspace_size(*bad) == 0
    # grows with B, k and V
    assert sv.workspace_size(200, 4, 100000, 0) > sv.workspace_size(100, 4, 100000, 0)
    assert sv.workspace_size(100, 5, 100000, 0) > sv.workspace_size(100, 4, 100000, 0)
    assert sv.workspace_size(100, 4, 200000, 0) > sv.workspace_size(100, 4, 100000, 0)


def _call(lib, **kw):
    args = dict(target=0x1000, draft=0x2000, dtype=0, tokens=0x3000, lens=None, temp=0x4000,
                B=2, k=2, V=64, seed=0, seq_base=0, out=0x5000, nacc=0x6000, aux=None,
                ws=None, ws_bytes=1 << 20, stream=None)
    # ws defaults to NULL: a call that passes every other check still stops
    # at the workspace check, so nothing here can reach a kernel launch.
    args.update(kw)
    return lib.spec_verify(args["target"], args["draft"], args["dtype"], args["tokens"],
                           args["lens"], args["temp"], args["B"], args["k"], args["V"],
                           ctypes.c_uint64(args["seed"]), ctypes.c_uint32(args["seq_base"]),
                           args["out"], args["nacc"], args["aux"], args["ws"], args["ws_bytes"],
                           args["stream"])


def test_host_side_errors_are_reported_before_any_launch(lib):
    # every call below is rejected before the library touches the device
    assert _call(lib, B=0) == 0  # empty batch: nothing to do
    assert _call(lib, B=-1) == 1
    assert _call(lib, k=64) == 1
    assert _call(lib, V=0) == 1
    assert _call(lib, dtype=3) == 1
    assert _call(lib, target=None) == 1
    assert _call(lib, temp=None) == 1
    assert _call(lib, out=None) == 1
    assert _call(lib, nacc=None) == 1
    assert _call(lib, draft=None) == 1  # k > 0 needs the draft
    assert _call(lib, tokens=None) == 1
    assert _call(lib, target=0x1002) == 1  # fp32 logits must be 4-byte aligned
    assert _call(lib, dtype=1, target=0x1002, draft=0x2002) == 2  # bf16: 2-byte aligned is fine
    assert _call(lib, dtype=1, target=0x1001) == 1
    assert _call(lib, tokens=0x3002) == 1
    assert _call(lib) == 2  # valid arguments, no workspace
    assert _call(lib, ws=0x10010) == 2  # not 256-byte aligned
    assert _call(lib, ws=0x10000, ws_bytes=16) == 2  # too small
    for st in range(4):
        assert sv.strerror(st)


def test_binding_rejects_bad_tensors():
    import torch

    t = torch.zeros(2, 3, 8)
    with pytest.raises(ValueError):
        sv.spec_verify(t, torch.zeros(2, 2, 8), torch.zeros(2, 2, dtype=torch.int32))
    with pytest.raises(ValueError):
        sv.spec_verify(torch.zeros(2, 8), None, None)


def test_binding_checks_caller_outputs_and_workspace():
    """Output tensors the caller passes are checked before any launch: the C
    ABI sees only pointers, so a short, int64, strided or foreign-device
    buffer would be written past its end."""
    import torch

    from speculative_decoding_verification_11_amd.binding import check_out, check_workspace

    dev = torch.device("cpu")
    good = (torch.empty(4, 6, dtype=torch.int32), torch.empty(4, dtype=torch.int32))
    assert check_out(good, ((4, 6), (4,)), dev, "e") == good
    bad = [
        (torch.empty(4, 5, dtype=torch.int32), good[1]),            # too short
        (torch.empty(4, 6, dtype=torch.int64), good[1]),            # wrong dtype
        (torch.empty(6, 4, dtype=torch.int32).t(), good[1]),        # not contiguous
        (good[0],),                                                  # wrong count
        (good[0], torch.empty(4, dtype=torch.float32)),              # float counts
        (good[0], None),
    ]
    for out in bad:
        with pytest.raises(ValueError):
            check_out(out, ((4, 6), (4,)), dev, "e")
    with pytest.raises(ValueError):  # wrong device
        check_out(good, ((4, 6), (4,)), torch.device("meta"), "e")
    ws = torch.empty(64, dtype=torch.uint8)
    assert check_workspace(ws, 32, dev, "e") is ws
    assert check_workspace(ws, 128, dev, "e").numel() == 128  # too small: a new one
    with pytest.raises(ValueError):
        check_workspace(torch.empty(8, 16, dtype=torch.uint8).t(), 16, dev, "e")
    with pytest.raises(ValueError):
        check_workspace(ws, 16, torch.device("meta"), "e")


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(sv.binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        sv.binding.library(str(tmp_path / "missing.so"))


def test_other_entry_points_reject_bad_arguments_before_any_launch(lib):
    import speculative_decoding_verification_11_amd.binding as bd

    # spec_verify_top_p: a missing top_p is an argument error
    rc = lib.spec_verify_top_p(0x1000, 0x2000, 0, 0x3000, None, 0x4000, None, 2, 2, 64,
                               ctypes.c_uint64(0), ctypes.c_uint32(0), 0x5000, 0x6000, None, None,
                               1 << 20, None)
    assert rc == 1
    rc = lib.spec_verify_top_p(0x1000, 0x2000, 0, 0x3000, None, 0x4000, 0x7000, 2, 2, 64,
                               ctypes.c_uint64(0), ctypes.c_uint32(0), 0x5000, 0x6000, None, None,
                               1 << 20, None)
    assert rc == 2  # valid arguments, no workspace
    # spec_verify_top_k_top_p: at least one filter; a misaligned top_k
    def topk(tk, tp):
        return lib.spec_verify_top_k_top_p(0x1000, 0x2000, 0, 0x3000, None, 0x4000, tk, tp, 2, 2,
                                           64, ctypes.c_uint64(0), ctypes.c_uint32(0), 0x5000,
                                           0x6000, None, None, 1 << 20, None)
    assert topk(None, None) == 1
    assert topk(0x7002, None) == 1
    assert topk(0x7000, None) == 2  # valid arguments, no workspace
    assert topk(None, 0x7000) == 2
    assert topk(0x7000, 0x8000) == 2
    # spec_verify_tree: sizes, pointers, workspace
    def tree(**kw):
        a = dict(target=0x1000, dtype=1, par=0x2000, tok=0x3000, nn=0x4000, B=2, N=8, V=64,
                 out=0x5000, path=0x6000, nacc=0x7000, aux=None, ws=None, ws_bytes=1 << 20)
        a.update(kw)
        return lib.spec_verify_tree(a["target"], a["dtype"], a["par"], a["tok"], a["nn"], a["B"],
                                    a["N"], a["V"], a["out"], a["path"], a["nacc"], a["aux"],
                                    a["ws"], a["ws_bytes"], None)
    assert tree(B=0) == 0
    assert tree(N=0) == 1 and tree(N=bd.MAX_TREE + 1) == 1 and tree(V=0) == 1
    assert tree(dtype=2) == 1 and tree(par=None) == 1 and tree(out=None) == 1
    assert tree(target=0x1001) == 1
    assert tree() == 2 and tree(ws=0x10010) == 2 and tree(ws=0x10000, ws_bytes=8) == 2
    assert sv.tree_workspace_size(2, 8, 64, 1) > 0 and sv.tree_workspace_size(2, 65, 64, 1) == 0
    # spec_prompt_lookup: parameters are checked before any launch
    def lookup(**kw):
        a = dict(ctx=0x1000, lens=0x2000, B=2, T=16, n_min=1, n_max=3, k=4, draft=0x3000,
                 dlen=0x4000)
        a.update(kw)
        return lib.spec_prompt_lookup(a["ctx"], a["lens"], a["B"], a["T"], a["n_min"], a["n_max"],
                                      a["k"], a["draft"], a["dlen"], None, None, None)
    assert lookup(B=0) == 0
    for bad in (dict(n_min=0), dict(n_max=0), dict(n_max=bd.MAX_NGRAM + 1), dict(k=-1),
                dict(k=bd.MAX_K + 1), dict(T=-1), dict(lens=None), dict(dlen=None),
                dict(draft=None), dict(ctx=0x1002)):
        assert lookup(**bad) == 1, bad
