"""Thin ctypes binding of libspecverify (the C ABI declared in include/spec_verify.h).

Argument marshalling only: every step of verification runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  The
library must be built (python -m draft_token_verification_07_amd._build);
calling any entry point without it raises.

    tokens, accept_len, p_tok, q_tok, status = spec_verify_sample(
        target_logits, draft_logits, draft_tokens, u_accept, u_sample,
        temperature, top_p, d2t=None)
    tokens, accept_len, p_tok, q_tok, status = spec_verify_sample_noalloc(..., out=outputs)
    tokens, accept_len, status = spec_verify_greedy(target_logits, draft_tokens)
    tokens, prob, status = spec_draft_sample(logits, u, temperature, top_p, top_k)
    spec_verify_count(accept_len, gamma, counters)
    path, tokens, accept_len, status = spec_verify_tree_greedy(target_logits, node_tokens, parents)

Tensors must live on the same GPU and be contiguous: logits float32 or
bfloat16, token ids / d2t / parents int32, uniforms float32.  Outputs are
new device tensors, written asynchronously on the current stream.  A
workspace (zeroed once at allocation, reused afterwards) is kept per
(device, stream) unless one is passed in.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
SV_SEQ_TOKEN_RANGE, SV_SEQ_D2T, SV_SEQ_NO_MASS, SV_SEQ_BAD_PARENT = 1, 2, 4, 8
SV_MAX_GAMMA, SV_MAX_TREE_NODES, SV_MAX_VOCAB = 255, 4096, 1 << 24

_STATUS = {0: "SV_OK", 1: "SV_ERR_INVALID_ARG", 2: "SV_ERR_UNSUPPORTED_DTYPE",
           3: "SV_ERR_WORKSPACE_TOO_SMALL", 4: "SV_ERR_HIP", 5: "SV_ERR_TOO_LARGE"}

_lib = None
_lock = threading.Lock()
_workspaces: dict = {}


class SpecVerifyError(RuntimeError):
    def __init__(self, fn: str, code: int):
        msg = lib().spec_verify_strerror(code).decode() if _lib is not None else ""
        super().__init__("%s failed: %s (%s)" % (fn, _STATUS.get(code, code), msg))
        self.code = code


def lib() -> C.CDLL:
    """Load libspecverify.so (built in-tree).  Raises if it is missing."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        "libspecverify.so is not built (%s); run "
                        "`python -m draft_token_verification_07_amd._build`" % LIB_PATH)
                L = C.CDLL(LIB_PATH)
                P, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
                L.spec_verify_strerror.restype = C.c_char_p
                L.spec_verify_strerror.argtypes = [C.c_int]
                L.sv_workspace_bytes_sample.restype = sz
                L.sv_workspace_bytes_sample.argtypes = [i32, i32, i32, i32, C.c_float]
                L.sv_workspace_bytes_greedy.restype = sz
                L.sv_workspace_bytes_greedy.argtypes = [i32, i32, i32]
                L.sv_workspace_bytes_tree.restype = sz
                L.sv_workspace_bytes_tree.argtypes = [i32, i32, i32]
                L.spec_verify_sample.restype = C.c_int
                L.spec_verify_sample.argtypes = [P, C.c_int, P, C.c_int, P, P, P, P, i32, i32, i32, i32,
                                                 C.c_float, C.c_float, P, P, P, P, P, P, sz, P]
                L.spec_verify_greedy.restype = C.c_int
                L.spec_verify_greedy.argtypes = [P, C.c_int, P, i32, i32, i32, P, P, P, P, sz, P]
                L.spec_verify_sample_noalloc.restype = C.c_int
                L.spec_verify_sample_noalloc.argtypes = [P, C.c_int, P, C.c_int, P, P, P, P, i32, i32, i32, i32,
                                                         C.c_float, C.c_float, P, P, P, P, P, P]
                L.sv_workspace_bytes_draft.restype = sz
                L.sv_workspace_bytes_draft.argtypes = [i32, i32]
                L.spec_draft_sample.restype = C.c_int
                L.spec_draft_sample.argtypes = [P, C.c_int, P, P, i32, i32, C.c_float, C.c_float, i32,
                                                P, P, P, P, sz, P]
                L.spec_verify_count.restype = C.c_int
                L.spec_verify_count.argtypes = [P, i32, i32, P, P]
                L.spec_fanout_lookup.restype = C.c_int
                L.spec_fanout_lookup.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, P, P]
                L.sv_workspace_bytes_vocab_trim.restype = sz
                L.sv_workspace_bytes_vocab_trim.argtypes = [i32]
                L.spec_vocab_trim.restype = C.c_int
                L.spec_vocab_trim.argtypes = [P, C.c_int64, i32, C.c_float, P, P, P, P, P, sz, P]
                L.sv_workspace_bytes_lmhead.restype = sz
                L.sv_workspace_bytes_lmhead.argtypes = [i32, i32]
                L.spec_lmhead_verify_greedy.restype = C.c_int
                L.spec_lmhead_verify_greedy.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P, P, P, P, sz, P]
                L.spec_lmhead_verify_tree.restype = C.c_int
                L.spec_lmhead_verify_tree.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, P, P, P, P, P, sz, P]
                L.spec_verify_tree_greedy.restype = C.c_int
                L.spec_verify_tree_greedy.argtypes = [P, C.c_int, P, P, i32, i32, i32, P, P, P, P, P, sz, P]
                _lib = L
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError("logits must be float32 or bfloat16, got %s" % t.dtype)


def _check(t: torch.Tensor, name: str, dev: torch.device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != dev:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def workspace(nbytes: int, dev: torch.device) -> torch.Tensor:
    """The cached workspace of the current (device, stream), grown to nbytes
    and zeroed when (re)allocated.  Calls on one stream are ordered, so they
    can share it; the kernels return it to zero."""
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def _raise(fn, code):
    if code != 0:
        raise SpecVerifyError(fn, code)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def sv_workspace_bytes_sample(B, gamma, Vt, Vd, top_p) -> int:
    return int(lib().sv_workspace_bytes_sample(B, gamma, Vt, Vd, float(top_p)))


def sv_workspace_bytes_greedy(B, gamma, V) -> int:
    return int(lib().sv_workspace_bytes_greedy(B, gamma, V))


def sv_workspace_bytes_tree(B, N, V) -> int:
    return int(lib().sv_workspace_bytes_tree(B, N, V))


def spec_verify_sample(target_logits, draft_logits, draft_tokens, u_accept, u_sample,
                       temperature: float, top_p: float, d2t=None, *, want_probs: bool = True,
                       ws: torch.Tensor | None = None, out=None):
    """Sampling verification.  Returns (tokens [B, g+1], accept_len [B],
    p_tok [B, g] | None, q_tok [B, g] | None, status [B]) as device tensors."""
    L = lib()
    dev = target_logits.device
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, gamma+1, Vt]")
    B, g1, Vt = target_logits.shape
    g = g1 - 1
    _check(target_logits, "target_logits", dev)
    tdt = _dtype_code(target_logits)
    if g > 0:
        _check(draft_logits, "draft_logits", dev)
        if draft_logits.dim() != 3 or tuple(draft_logits.shape[:2]) != (B, g):
            raise ValueError("draft_logits must be [B, gamma, Vd]")
        Vd = draft_logits.shape[2]
        ddt = _dtype_code(draft_logits)
        _check(draft_tokens, "draft_tokens", dev, torch.int32, (B, g))
        _check(u_accept, "u_accept", dev, torch.float32, (B, g))
    else:
        Vd = Vt if d2t is None else d2t.shape[0]
        ddt = tdt if draft_logits is None else _dtype_code(draft_logits)
    _check(u_sample, "u_sample", dev, torch.float32, (B,))
    if d2t is not None:
        _check(d2t, "d2t", dev, torch.int32, (Vd,))
    if out is None:
        out_tokens = torch.empty((B, g + 1), dtype=torch.int32, device=dev)
        out_len = torch.empty((B,), dtype=torch.int32, device=dev)
        out_p = torch.empty((B, g), dtype=torch.float32, device=dev) if want_probs else None
        out_q = torch.empty((B, g), dtype=torch.float32, device=dev) if want_probs else None
        out_status = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        out_tokens, out_len, out_p, out_q, out_status = out
    need = sv_workspace_bytes_sample(B, g, Vt, Vd, top_p)
    if ws is None:
        ws = workspace(need, dev)
    rc = L.spec_verify_sample(
        _ptr(target_logits), tdt, _ptr(draft_logits if g > 0 else None), ddt,
        _ptr(draft_tokens if g > 0 else None), _ptr(d2t), _ptr(u_accept if g > 0 else None), _ptr(u_sample),
        B, g, Vt, Vd, float(temperature), float(top_p),
        _ptr(out_tokens), _ptr(out_len), _ptr(out_p), _ptr(out_q), _ptr(out_status),
        _ptr(ws), ws.numel(), _stream(dev))
    _raise("spec_verify_sample", rc)
    return out_tokens, out_len, out_p, out_q, out_status


def spec_verify_sample_noalloc(target_logits, draft_logits, draft_tokens, u_accept, u_sample,
                               temperature: float, top_p: float, d2t=None, *, out):
    """spec_verify_sample without a workspace: the library's static per-GPU
    scratch is used and nothing is allocated.  The outputs are the caller's:
    out = (tokens [B, g+1] int32, accept_len [B] int32, p_tok [B, g] float32
    or None, q_tok [B, g] float32 or None, status [B] int32 or None)."""
    L = lib()
    dev = target_logits.device
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, gamma+1, Vt]")
    B, g1, Vt = target_logits.shape
    g = g1 - 1
    _check(target_logits, "target_logits", dev)
    tdt = _dtype_code(target_logits)
    if g > 0:
        _check(draft_logits, "draft_logits", dev)
        if draft_logits.dim() != 3 or tuple(draft_logits.shape[:2]) != (B, g):
            raise ValueError("draft_logits must be [B, gamma, Vd]")
        Vd = draft_logits.shape[2]
        ddt = _dtype_code(draft_logits)
        _check(draft_tokens, "draft_tokens", dev, torch.int32, (B, g))
        _check(u_accept, "u_accept", dev, torch.float32, (B, g))
    else:
        Vd = Vt if d2t is None else d2t.shape[0]
        ddt = tdt if draft_logits is None else _dtype_code(draft_logits)
    _check(u_sample, "u_sample", dev, torch.float32, (B,))
    if d2t is not None:
        _check(d2t, "d2t", dev, torch.int32, (Vd,))
    out_tokens, out_len, out_p, out_q, out_status = out
    _check(out_tokens, "out_tokens", dev, torch.int32, (B, g + 1))
    _check(out_len, "out_accept_len", dev, torch.int32, (B,))
    rc = L.spec_verify_sample_noalloc(
        _ptr(target_logits), tdt, _ptr(draft_logits if g > 0 else None), ddt,
        _ptr(draft_tokens if g > 0 else None), _ptr(d2t), _ptr(u_accept if g > 0 else None), _ptr(u_sample),
        B, g, Vt, Vd, float(temperature), float(top_p),
        _ptr(out_tokens), _ptr(out_len), _ptr(out_p), _ptr(out_q), _ptr(out_status), _stream(dev))
    _raise("spec_verify_sample_noalloc", rc)
    return out_tokens, out_len, out_p, out_q, out_status


def sv_workspace_bytes_draft(B, V) -> int:
    return int(lib().sv_workspace_bytes_draft(B, V))


def spec_draft_sample(logits, u, temperature: float, top_p: float = 1.0, top_k: int = 0, d2t=None, *,
                      ws: torch.Tensor | None = None, out=None):
    """Draft-side sampler: one token per row of logits [B, V].  Returns
    (tokens [B] int32, prob [B] float32, status [B] int32) device tensors."""
    L = lib()
    dev = logits.device
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    B, V = logits.shape
    _check(logits, "logits", dev)
    dt = _dtype_code(logits)
    _check(u, "u", dev, torch.float32, (B,))
    if d2t is not None:
        _check(d2t, "d2t", dev, torch.int32, (V,))
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.float32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    need = sv_workspace_bytes_draft(B, V)
    if ws is None:
        ws = workspace(need, dev)
    rc = L.spec_draft_sample(_ptr(logits), dt, _ptr(d2t), _ptr(u), B, V, float(temperature), float(top_p), int(top_k),
                             _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(ws), ws.numel(), _stream(dev))
    _raise("spec_draft_sample", rc)
    return out


def spec_verify_count(accept_len, gamma: int, counters):
    """Add one verification call's accept_len [B] to counters [5] (int64 device
    tensor: target calls, drafts proposed, accepted, emitted, invalid)."""
    L = lib()
    dev = accept_len.device
    _check(accept_len, "accept_len", dev, torch.int32)
    _check(counters, "counters", dev, torch.int64, (5,))
    rc = L.spec_verify_count(_ptr(accept_len), accept_len.numel(), int(gamma), _ptr(counters), _stream(dev))
    _raise("spec_verify_count", rc)
    return counters


def spec_fanout_lookup(out_tokens, accept_len, cand, branch_drafts=None, *, counters=None, want_next=True):
    """SSD fan-out lookup.  cand [B, g+1, f], branch_drafts [B, (g+1) f, L].
    Returns (branch [B] int32, next [B, L] int32 | None)."""
    L_ = lib()
    dev = out_tokens.device
    B, g1 = out_tokens.shape
    _check(out_tokens, "out_tokens", dev, torch.int32)
    _check(accept_len, "accept_len", dev, torch.int32, (B,))
    _check(cand, "cand", dev, torch.int32)
    if cand.dim() != 3 or tuple(cand.shape[:2]) != (B, g1):
        raise ValueError("cand must be [B, gamma+1, f]")
    f = cand.shape[2]
    Ln = 0
    if branch_drafts is not None:
        _check(branch_drafts, "branch_drafts", dev, torch.int32)
        if branch_drafts.dim() != 3 or tuple(branch_drafts.shape[:2]) != (B, g1 * f):
            raise ValueError("branch_drafts must be [B, (gamma+1) f, L]")
        Ln = branch_drafts.shape[2]
    if counters is not None:
        _check(counters, "counters", dev, torch.int64, (2,))
    br = torch.empty(B, dtype=torch.int32, device=dev)
    nx = torch.empty((B, Ln), dtype=torch.int32, device=dev) if (want_next and branch_drafts is not None) else None
    rc = L_.spec_fanout_lookup(_ptr(out_tokens), _ptr(accept_len), _ptr(cand), _ptr(branch_drafts), B, g1 - 1, f,
                               Ln, _ptr(br), _ptr(nx), _ptr(counters), _stream(dev))
    _raise("spec_fanout_lookup", rc)
    return br, nx


def sv_workspace_bytes_vocab_trim(Vt) -> int:
    return int(lib().sv_workspace_bytes_vocab_trim(Vt))


def spec_vocab_trim(tokens, Vt: int, P: float = 0.95, *, ws: torch.Tensor | None = None, out=None):
    """Vocabulary-trim d2t builder.  Returns (d2t [Vt] int32 -- the first vd
    entries valid --, t2d [Vt] int32, vd [1] int32, info [3] int64) device
    tensors (no host synchronization)."""
    L = lib()
    dev = tokens.device
    _check(tokens, "tokens", dev, torch.int32)
    if out is None:
        out = (torch.empty(Vt, dtype=torch.int32, device=dev), torch.empty(Vt, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev), torch.empty(3, dtype=torch.int64, device=dev))
    need = sv_workspace_bytes_vocab_trim(Vt)
    if ws is None:
        ws = workspace(need, dev)
    rc = L.spec_vocab_trim(_ptr(tokens), tokens.numel(), int(Vt), float(P), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
                           _ptr(out[3]), _ptr(ws), ws.numel(), _stream(dev))
    _raise("spec_vocab_trim", rc)
    return out


def sv_workspace_bytes_lmhead(M, V) -> int:
    return int(lib().sv_workspace_bytes_lmhead(M, V))


def _lmhead_common(hidden, W, what):
    dev = hidden.device
    _check(hidden, "hidden", dev, torch.bfloat16)
    _check(W, "W", dev, torch.bfloat16)
    if hidden.dim() != 3 or W.dim() != 2 or hidden.shape[2] != W.shape[1]:
        raise ValueError("%s: hidden must be [B, R, d] and W [V, d]" % what)
    return dev, hidden.shape[0], hidden.shape[1], hidden.shape[2], W.shape[0]


def spec_lmhead_verify_greedy(hidden, W, draft_tokens, *, want_rows: bool = True,
                              ws: torch.Tensor | None = None, out=None):
    """Fused lm_head -> greedy chain verification.  hidden [B, g+1, d] bf16,
    W [V, d] bf16.  Returns (tokens [B, g+1], accept_len [B], argmax [B, g+1]
    | None, maxlogit [B, g+1] | None, status [B])."""
    L = lib()
    dev, B, R, d, V = _lmhead_common(hidden, W, "spec_lmhead_verify_greedy")
    g = R - 1
    if g > 0:
        _check(draft_tokens, "draft_tokens", dev, torch.int32, (B, g))
    if out is None:
        out = (torch.empty((B, R), dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty((B, R), dtype=torch.int32, device=dev) if want_rows else None,
               torch.empty((B, R), dtype=torch.float32, device=dev) if want_rows else None,
               torch.empty(B, dtype=torch.int32, device=dev))
    need = sv_workspace_bytes_lmhead(B * R, V)
    if ws is None:
        ws = workspace(need, dev)
    rc = L.spec_lmhead_verify_greedy(_ptr(hidden), _ptr(W), _ptr(draft_tokens if g > 0 else None), B, g, d, V,
                                     _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(out[3]), _ptr(out[4]), _ptr(ws),
                                     ws.numel(), _stream(dev))
    _raise("spec_lmhead_verify_greedy", rc)
    return out


def spec_lmhead_verify_tree(hidden, W, node_tokens, parents, *, want_rows: bool = True,
                            ws: torch.Tensor | None = None, out=None):
    """Fused lm_head -> greedy tree verification.  hidden [B, N, d] bf16.
    Returns (path [B, N], tokens [B, N], accept_len [B], argmax [B, N] | None,
    maxlogit [B, N] | None, status [B])."""
    L = lib()
    dev, B, N, d, V = _lmhead_common(hidden, W, "spec_lmhead_verify_tree")
    _check(node_tokens, "node_tokens", dev, torch.int32, (B, N))
    _check(parents, "parents", dev, torch.int32, (B, N))
    if out is None:
        out = (torch.empty((B, N), dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty((B, N), dtype=torch.int32, device=dev) if want_rows else None,
               torch.empty((B, N), dtype=torch.float32, device=dev) if want_rows else None,
               torch.empty(B, dtype=torch.int32, device=dev))
    need = sv_workspace_bytes_lmhead(B * N, V)
    if ws is None:
        ws = workspace(need, dev)
    rc = L.spec_lmhead_verify_tree(_ptr(hidden), _ptr(W), _ptr(node_tokens), _ptr(parents), B, N, d, V, _ptr(out[0]),
                                   _ptr(out[1]), _ptr(out[2]), _ptr(out[3]), _ptr(out[4]), _ptr(out[5]), _ptr(ws),
                                   ws.numel(), _stream(dev))
    _raise("spec_lmhead_verify_tree", rc)
    return out


def spec_verify_greedy(target_logits, draft_tokens, *, ws: torch.Tensor | None = None, out=None):
    """Greedy verification.  Returns (tokens [B, g+1], accept_len [B], status [B])."""
    L = lib()
    dev = target_logits.device
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, gamma+1, V]")
    B, g1, V = target_logits.shape
    g = g1 - 1
    _check(target_logits, "target_logits", dev)
    dt = _dtype_code(target_logits)
    if g > 0:
        _check(draft_tokens, "draft_tokens", dev, torch.int32, (B, g))
    if out is None:
        out_tokens = torch.empty((B, g + 1), dtype=torch.int32, device=dev)
        out_len = torch.empty((B,), dtype=torch.int32, device=dev)
        out_status = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        out_tokens, out_len, out_status = out
    need = sv_workspace_bytes_greedy(B, g, V)
    if ws is None:
        ws = workspace(need, dev)
    rc = L.spec_verify_greedy(_ptr(target_logits), dt, _ptr(draft_tokens if g > 0 else None), B, g, V,
                              _ptr(out_tokens), _ptr(out_len), _ptr(out_status), _ptr(ws), ws.numel(),
                              _stream(dev))
    _raise("spec_verify_greedy", rc)
    return out_tokens, out_len, out_status


def spec_verify_tree_greedy(target_logits, node_tokens, parents, *, ws: torch.Tensor | None = None, out=None):
    """Greedy tree verification.  Returns (path [B, N], tokens [B, N], accept_len [B], status [B])."""
    L = lib()
    dev = target_logits.device
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, N, V]")
    B, N, V = target_logits.shape
    _check(target_logits, "target_logits", dev)
    dt = _dtype_code(target_logits)
    _check(node_tokens, "node_tokens", dev, torch.int32, (B, N))
    _check(parents, "parents", dev, torch.int32, (B, N))
    if out is None:
        out_path = torch.empty((B, N), dtype=torch.int32, device=dev)
        out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
        out_len = torch.empty((B,), dtype=torch.int32, device=dev)
        out_status = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        out_path, out_tokens, out_len, out_status = out
    need = sv_workspace_bytes_tree(B, N, V)
    if ws is None:
        ws = workspace(need, dev)
    rc = L.spec_verify_tree_greedy(_ptr(target_logits), dt, _ptr(node_tokens), _ptr(parents), B, N, V,
                                   _ptr(out_path), _ptr(out_tokens), _ptr(out_len), _ptr(out_status),
                                   _ptr(ws), ws.numel(), _stream(dev))
    _raise("spec_verify_tree_greedy", rc)
    return out_path, out_tokens, out_len, out_status
