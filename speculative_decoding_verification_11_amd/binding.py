"""Python binding of libspecverify.so: argument marshalling only.

Every step of the verification runs in the HIP kernels behind the C ABI
declared in include/spec_verify.h. PyTorch supplies device memory and the
current stream; this module checks shapes and dtypes, allocates outputs and
workspace with torch, and calls the C entry point. There is no CPU fallback:
if the library is missing, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Union

import torch

from .build import LIB as LIB_PATH

F32 = 0
BF16 = 1
MAX_K = 63
MAX_TREE = 64
MAX_NGRAM = 16

SEQ_OK, SEQ_BAD_TOKEN, SEQ_BAD_LEN, SEQ_BAD_TEMP, SEQ_QZERO, SEQ_BAD_TREE, SEQ_BAD_TOP_P = range(7)
DRAW_NONE, DRAW_GREEDY, DRAW_RESIDUAL, DRAW_BONUS, DRAW_RESIDUAL_AS_P = range(5)

STATUS_NAMES = {0: "SPEC_OK", 1: "SPEC_EINVAL", 2: "SPEC_EWORKSPACE", 3: "SPEC_ELAUNCH",
                4: "SPEC_ESCRATCH"}
NOALLOC_SCRATCH_BYTES = 8 << 20  # SPEC_NOALLOC_SCRATCH_BYTES

EXPORTED = ("spec_verify", "spec_verify_early_exit", "spec_verify_top_p", "spec_verify_top_k_top_p",
            "spec_verify_workspace_size", "spec_verify_noalloc",
            "spec_verify_tree", "spec_verify_tree_workspace_size", "spec_prompt_lookup",
            "spec_verify_strerror", "spec_verify_version")


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Aux(ctypes.Structure):
    """Mirror of spec_verify_aux_t."""

    _fields_ = [
        ("p_g", ctypes.c_void_p),
        ("q_g", ctypes.c_void_p),
        ("resid_mass", ctypes.c_void_p),
        ("argmax", ctypes.c_void_p),
        ("seq_status", ctypes.c_void_p),
        ("draw_row", ctypes.c_void_p),
        ("draw_kind", ctypes.c_void_p),
        ("event_begin", ctypes.c_void_p),
        ("event_end", ctypes.c_void_p),
    ]


class TreeAux(ctypes.Structure):
    """Mirror of spec_tree_aux_t."""

    _fields_ = [
        ("seq_status", ctypes.c_void_p),
        ("argmax", ctypes.c_void_p),
        ("event_begin", ctypes.c_void_p),
        ("event_end", ctypes.c_void_p),
    ]


_lock = threading.Lock()
_lib = None


def library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library not built ({path} missing); run "
                "`python -m speculative_decoding_verification_11_amd.build` or "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, u32, u64 = ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64
        lib.spec_verify_workspace_size.argtypes = [i32, i32, i32, i32]
        lib.spec_verify_workspace_size.restype = ctypes.c_size_t
        for fn in (lib.spec_verify, lib.spec_verify_early_exit):
            fn.argtypes = [P, P, i32, P, P, P, i32, i32, i32, u64, u32, P, P,
                           ctypes.POINTER(Aux), P, ctypes.c_size_t, P]
            fn.restype = ctypes.c_int
        lib.spec_verify_noalloc.argtypes = [P, P, i32, P, P, P, i32, i32, i32, u64, u32, P, P,
                                            ctypes.POINTER(Aux), P]
        lib.spec_verify_noalloc.restype = ctypes.c_int
        lib.spec_verify_top_p.argtypes = [P, P, i32, P, P, P, P, i32, i32, i32, u64, u32, P, P,
                                          ctypes.POINTER(Aux), P, ctypes.c_size_t, P]
        lib.spec_verify_top_p.restype = ctypes.c_int
        lib.spec_verify_top_k_top_p.argtypes = [P, P, i32, P, P, P, P, P, i32, i32, i32, u64, u32,
                                                P, P, ctypes.POINTER(Aux), P, ctypes.c_size_t, P]
        lib.spec_verify_top_k_top_p.restype = ctypes.c_int
        lib.spec_verify_tree_workspace_size.argtypes = [i32, i32, i32, i32]
        lib.spec_verify_tree_workspace_size.restype = ctypes.c_size_t
        lib.spec_verify_tree.argtypes = [P, i32, P, P, P, i32, i32, i32, P, P, P,
                                         ctypes.POINTER(TreeAux), P, ctypes.c_size_t, P]
        lib.spec_verify_tree.restype = ctypes.c_int
        lib.spec_prompt_lookup.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, P, P, P]
        lib.spec_prompt_lookup.restype = ctypes.c_int
        lib.spec_verify_strerror.argtypes = [ctypes.c_int]
        lib.spec_verify_strerror.restype = ctypes.c_char_p
        lib.spec_verify_version.argtypes = []
        lib.spec_verify_version.restype = ctypes.c_int
        if path == LIB_PATH:
            _lib = lib
        return lib


def workspace_size(B: int, k: int, V: int, dtype: int) -> int:
    return int(library().spec_verify_workspace_size(B, k, V, dtype))


def strerror(status: int) -> str:
    return library().spec_verify_strerror(status).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def check_out(out, shapes, device, entry: str) -> tuple:
    """Validate caller-supplied output tensors before any launch: the C ABI
    sees only pointers, so a short, non-int32, foreign-device or strided
    buffer would be overwritten past its end. ``shapes``: one expected shape
    per tensor. Returns the tensors as a tuple."""
    if not isinstance(out, (tuple, list)) or len(out) != len(shapes):
        raise ValueError(f"{entry}: out must be a tuple of {len(shapes)} tensors")
    for i, (t, shape) in enumerate(zip(out, shapes)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{entry}: out[{i}] must be a tensor")
        if (tuple(t.shape) != tuple(shape) or t.dtype != torch.int32 or t.device != device
                or not t.is_contiguous()):
            raise ValueError(f"{entry}: out[{i}] must be contiguous {list(shape)} int32 on "
                             f"{device}, got {list(t.shape)} {t.dtype} on {t.device}"
                             f"{'' if t.is_contiguous() else ' (not contiguous)'}")
    return tuple(out)


def check_workspace(workspace, need: int, device, entry: str):
    """A caller's workspace must be a contiguous tensor on the call's device;
    None, or one smaller than ``need`` bytes, is replaced by a new one."""
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != device \
                or not workspace.is_contiguous():
            raise ValueError(f"{entry}: workspace must be a contiguous tensor on {device}")
        if workspace.numel() * workspace.element_size() >= need:
            return workspace
    return torch.empty(need, dtype=torch.uint8, device=device)


def spec_verify(target: torch.Tensor, draft: Optional[torch.Tensor],
                draft_tokens: Optional[torch.Tensor], draft_len: Optional[torch.Tensor] = None,
                temperature: Union[float, torch.Tensor] = 1.0, seed: int = 0, *,
                seq_base: int = 0, aux: bool = False, workspace: Optional[torch.Tensor] = None,
                out: Optional[tuple] = None, events: Optional[tuple] = None):
    """Verify B drafted continuations on the GPU (C entry point spec_verify).
    See _verify for the arguments."""
    return _verify("spec_verify", target, draft, draft_tokens, draft_len, temperature, seed,
                   seq_base, aux, workspace, out, events)


def spec_verify_noalloc(target: torch.Tensor, draft: Optional[torch.Tensor],
                        draft_tokens: Optional[torch.Tensor],
                        draft_len: Optional[torch.Tensor] = None,
                        temperature: Union[float, torch.Tensor] = 1.0, seed: int = 0, *,
                        seq_base: int = 0, aux: bool = False, out: Optional[tuple] = None,
                        events: Optional[tuple] = None):
    """spec_verify without a workspace (C entry point spec_verify_noalloc):
    the library's static per-GPU scratch is used and nothing is allocated by
    the call itself (pass ``out`` to allocate nothing here either). Raises
    SpecVerifyError with SPEC_ESCRATCH when the sizes need more scratch than
    NOALLOC_SCRATCH_BYTES."""
    return _verify("spec_verify_noalloc", target, draft, draft_tokens, draft_len, temperature,
                   seed, seq_base, aux, None, out, events, noalloc=True)


def spec_verify_early_exit(target: torch.Tensor, draft: Optional[torch.Tensor],
                           draft_tokens: Optional[torch.Tensor],
                           draft_len: Optional[torch.Tensor] = None,
                           temperature: Union[float, torch.Tensor] = 1.0, seed: int = 0, *,
                           seq_base: int = 0, aux: bool = False,
                           workspace: Optional[torch.Tensor] = None, out: Optional[tuple] = None,
                           events: Optional[tuple] = None):
    """Same outputs as spec_verify, reading only the rows up to each
    sequence's first rejection (C entry point spec_verify_early_exit). The
    p_g / q_g / argmax diagnostics past the stop are NaN / -1. ``events``
    bracket the per-position launches."""
    return _verify("spec_verify_early_exit", target, draft, draft_tokens, draft_len, temperature,
                   seed, seq_base, aux, workspace, out, events)


def spec_verify_top_p(target: torch.Tensor, draft: Optional[torch.Tensor],
                      draft_tokens: Optional[torch.Tensor], draft_len: Optional[torch.Tensor] = None,
                      temperature: Union[float, torch.Tensor] = 1.0,
                      top_p: Union[float, torch.Tensor] = 1.0, seed: int = 0, *,
                      seq_base: int = 0, aux: bool = False,
                      workspace: Optional[torch.Tensor] = None, out: Optional[tuple] = None,
                      events: Optional[tuple] = None):
    """spec_verify with top-p (nucleus) filtering of every target and draft
    row (C entry point spec_verify_top_p). top_p: float or [B] float32."""
    B = target.shape[0]
    if isinstance(top_p, torch.Tensor):
        tp = top_p
        if (tuple(tp.shape) != (B,) or tp.dtype != torch.float32 or tp.device != target.device
                or not tp.is_contiguous()):
            raise ValueError(f"top_p must be contiguous [{B}] float32 on {target.device}")
    else:
        tp = torch.full((B,), float(top_p), dtype=torch.float32, device=target.device)
    return _verify("spec_verify_top_p", target, draft, draft_tokens, draft_len, temperature, seed,
                   seq_base, aux, workspace, out, events, top_p=tp)


def _per_sequence(value, B, dtype, name, device):
    """A scalar broadcast to [B], or a checked contiguous [B] tensor."""
    if isinstance(value, torch.Tensor):
        if (tuple(value.shape) != (B,) or value.dtype != dtype or value.device != device
                or not value.is_contiguous()):
            raise ValueError(f"{name} must be contiguous [{B}] {dtype} on {device}")
        return value
    return torch.full((B,), value, dtype=dtype, device=device)


def spec_verify_top_k_top_p(target: torch.Tensor, draft: Optional[torch.Tensor],
                            draft_tokens: Optional[torch.Tensor],
                            draft_len: Optional[torch.Tensor] = None,
                            temperature: Union[float, torch.Tensor] = 1.0,
                            top_k: Union[int, torch.Tensor, None] = 0,
                            top_p: Union[float, torch.Tensor, None] = None, seed: int = 0, *,
                            seq_base: int = 0, aux: bool = False,
                            workspace: Optional[torch.Tensor] = None, out: Optional[tuple] = None,
                            events: Optional[tuple] = None):
    """spec_verify with top-k, then top-p, filtering of every target and
    draft row (C entry point spec_verify_top_k_top_p). top_k: int or [B]
    int32 (<= 0 or >= V: no top-k); top_p: None (no top-p), float or [B]
    float32."""
    B, dev = target.shape[0], target.device
    tk = None if top_k is None else _per_sequence(
        int(top_k) if not isinstance(top_k, torch.Tensor) else top_k, B, torch.int32, "top_k", dev)
    tp = None if top_p is None else _per_sequence(
        float(top_p) if not isinstance(top_p, torch.Tensor) else top_p, B, torch.float32, "top_p",
        dev)
    if tk is None and tp is None:
        raise ValueError("top_k and top_p cannot both be None")
    return _verify("spec_verify_top_k_top_p", target, draft, draft_tokens, draft_len, temperature,
                   seed, seq_base, aux, workspace, out, events, top_p=tp, top_k=tk,
                   filters=True)


def _verify(entry, target, draft, draft_tokens, draft_len, temperature, seed, seq_base, aux,
            workspace, out, events, top_p=None, top_k=None, filters=False, noalloc=False):
    """Verify B drafted continuations on the GPU.

    target [B, k+1, V] and draft [B, k, V]: float32 or bfloat16, contiguous,
    same device. draft_tokens [B, k] int32; draft_len [B] int32 or None (all
    k); temperature: float or [B] float32 tensor (0 = greedy).

    Returns (out_tokens [B, k+1] int32, num_accepted [B] int32), plus a dict
    of diagnostics when ``aux`` is true. ``events`` = (begin, end) raw
    hipEvent_t handles recorded around the row-statistics kernel.
    """
    if target.dim() != 3:
        raise ValueError("target must be [B, k+1, V]")
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("target must be a GPU tensor")
    dt = _dtype_code(target)
    if not target.is_contiguous():
        raise ValueError("target must be contiguous")
    if k > 0:
        if draft is None or draft_tokens is None:
            raise ValueError("draft logits and draft tokens are required when k > 0")
        if tuple(draft.shape) != (B, k, V) or draft.dtype != target.dtype or draft.device != dev:
            raise ValueError(f"draft must be [{B}, {k}, {V}] {target.dtype} on {dev}")
        if not draft.is_contiguous():
            raise ValueError("draft must be contiguous")
        if (tuple(draft_tokens.shape) != (B, k) or draft_tokens.dtype != torch.int32
                or draft_tokens.device != dev or not draft_tokens.is_contiguous()):
            raise ValueError(f"draft_tokens must be contiguous [{B}, {k}] int32 on {dev}")
    if draft_len is not None and (tuple(draft_len.shape) != (B,) or draft_len.dtype != torch.int32
                                  or draft_len.device != dev or not draft_len.is_contiguous()):
        raise ValueError(f"draft_len must be contiguous [{B}] int32 on {dev}")
    if isinstance(temperature, torch.Tensor):
        temp = temperature
        if (tuple(temp.shape) != (B,) or temp.dtype != torch.float32 or temp.device != dev
                or not temp.is_contiguous()):
            raise ValueError(f"temperature must be contiguous [{B}] float32 on {dev}")
    else:
        temp = torch.full((B,), float(temperature), dtype=torch.float32, device=dev)

    lib = library()
    if out is None:
        out_tokens = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
        num_acc = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        out_tokens, num_acc = check_out(out, ((B, k + 1), (B,)), dev, entry)
    need = int(lib.spec_verify_workspace_size(B, k, V, dt))
    if need == 0:
        raise SpecVerifyError(1, "invalid sizes for the workspace query")
    if not noalloc:
        workspace = check_workspace(workspace, need, dev, entry)

    aux_t = None
    aux_out = None
    if aux or events is not None:
        aux_t = Aux()
        if aux:
            aux_out = dict(
                p_g=torch.empty((B, k), dtype=torch.float32, device=dev),
                q_g=torch.empty((B, k), dtype=torch.float32, device=dev),
                resid_mass=torch.empty((B,), dtype=torch.float32, device=dev),
                argmax=torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                seq_status=torch.empty((B,), dtype=torch.int32, device=dev),
                draw_row=torch.empty((B,), dtype=torch.int32, device=dev),
                draw_kind=torch.empty((B,), dtype=torch.int32, device=dev),
            )
            for name, t in aux_out.items():
                setattr(aux_t, name, t.data_ptr())
        if events is not None:
            aux_t.event_begin, aux_t.event_end = events

    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        if filters:
            extra = (_ptr(top_k), _ptr(top_p))
        else:
            extra = (top_p.data_ptr(),) if top_p is not None else ()
        ws_args = () if noalloc else (workspace.data_ptr(), need)
        rc = getattr(lib, entry)(
            target.data_ptr(), _ptr(draft) if k > 0 else None, dt,
            _ptr(draft_tokens) if k > 0 else None, _ptr(draft_len), temp.data_ptr(), *extra,
            B, k, V, ctypes.c_uint64(seed & (2**64 - 1)), ctypes.c_uint32(seq_base & 0xFFFFFFFF),
            out_tokens.data_ptr(), num_acc.data_ptr(),
            ctypes.byref(aux_t) if aux_t is not None else None, *ws_args, stream)
    if rc != 0:
        raise SpecVerifyError(rc, strerror(rc))
    if aux:
        return out_tokens, num_acc, aux_out
    return out_tokens, num_acc


def tree_workspace_size(B: int, N: int, V: int, dtype: int) -> int:
    return int(library().spec_verify_tree_workspace_size(B, N, V, dtype))


def spec_verify_tree(target: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor,
                     n_nodes: torch.Tensor, *, aux: bool = False,
                     workspace: Optional[torch.Tensor] = None, out: Optional[tuple] = None,
                     events: Optional[tuple] = None):
    """Greedy verification of B candidate trees (C entry point spec_verify_tree).

    target [B, N, V] float32 or bfloat16 (row n scored at node n); parents,
    tokens [B, N] int32 (entry 0 ignored); n_nodes [B] int32. Returns
    (out_tokens [B, N], path_nodes [B, N], num_accepted [B]), plus a dict with
    seq_status and argmax when ``aux`` is true. ``events`` = (begin, end) raw
    hipEvent_t handles recorded around the row kernel.
    """
    if target.dim() != 3:
        raise ValueError("target must be [B, N, V]")
    B, N, V = target.shape
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("target must be a GPU tensor")
    dt = _dtype_code(target)
    if not target.is_contiguous():
        raise ValueError("target must be contiguous")
    for name, t, shape in (("parents", parents, (B, N)), ("tokens", tokens, (B, N)),
                           ("n_nodes", n_nodes, (B,))):
        if (tuple(t.shape) != shape or t.dtype != torch.int32 or t.device != dev
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous {list(shape)} int32 on {dev}")
    lib = library()
    if out is None:
        out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
        path_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
        num_acc = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        out_tokens, path_nodes, num_acc = check_out(out, ((B, N), (B, N), (B,)), dev,
                                                    "spec_verify_tree")
    need = int(lib.spec_verify_tree_workspace_size(B, N, V, dt))
    if need == 0:
        raise SpecVerifyError(1, "invalid sizes for the tree workspace query")
    workspace = check_workspace(workspace, need, dev, "spec_verify_tree")
    aux_t, aux_out = None, None
    if aux or events is not None:
        aux_t = TreeAux()
        if aux:
            aux_out = dict(seq_status=torch.empty((B,), dtype=torch.int32, device=dev),
                           argmax=torch.empty((B, N), dtype=torch.int32, device=dev))
            aux_t.seq_status = aux_out["seq_status"].data_ptr()
            aux_t.argmax = aux_out["argmax"].data_ptr()
        if events is not None:
            aux_t.event_begin, aux_t.event_end = events
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = lib.spec_verify_tree(target.data_ptr(), dt, parents.data_ptr(), tokens.data_ptr(),
                                  n_nodes.data_ptr(), B, N, V, out_tokens.data_ptr(),
                                  path_nodes.data_ptr(), num_acc.data_ptr(),
                                  ctypes.byref(aux_t) if aux_t is not None else None,
                                  workspace.data_ptr(), need, stream)
    if rc != 0:
        raise SpecVerifyError(rc, strerror(rc))
    if aux:
        return out_tokens, path_nodes, num_acc, aux_out
    return out_tokens, path_nodes, num_acc


def spec_prompt_lookup(contexts: torch.Tensor, context_len: torch.Tensor, n_min: int, n_max: int,
                       k: int, *, match: bool = False, out: Optional[tuple] = None):
    """Prompt-lookup drafting (C entry point spec_prompt_lookup).

    contexts [B, T_max] int32 (row b holds context_len[b] tokens), context_len
    [B] int32. Returns (draft_tokens [B, k], draft_len [B]), plus (match_n,
    match_start) when ``match`` is true.
    """
    if contexts.dim() != 2:
        raise ValueError("contexts must be [B, T_max]")
    B, T_max = contexts.shape
    dev = contexts.device
    if dev.type != "cuda":
        raise ValueError("contexts must be a GPU tensor")
    for name, t, shape in (("contexts", contexts, (B, T_max)), ("context_len", context_len, (B,))):
        if (tuple(t.shape) != shape or t.dtype != torch.int32 or t.device != dev
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous {list(shape)} int32 on {dev}")
    if out is None:
        draft = torch.empty((B, max(k, 0)), dtype=torch.int32, device=dev)
        dlen = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        draft, dlen = check_out(out, ((B, max(k, 0)), (B,)), dev, "spec_prompt_lookup")
    mn = ms = None
    if match:
        mn = torch.empty((B,), dtype=torch.int32, device=dev)
        ms = torch.empty((B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = library().spec_prompt_lookup(
            contexts.data_ptr(), context_len.data_ptr(), B, T_max, n_min, n_max, k,
            draft.data_ptr() if k > 0 else None, dlen.data_ptr(),
            _ptr(mn), _ptr(ms), stream)
    if rc != 0:
        raise SpecVerifyError(rc, strerror(rc))
    if match:
        return draft, dlen, mn, ms
    return draft, dlen
