"""CPU oracle for batched draft-token verification (TEST INFRASTRUCTURE ONLY).

The oracle is the plain float64 statement of what the verification path
computes, written from the pages (see the header of spec_oracle.c for the
sources and each function for the passage it follows).  Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import this package.
It shares no code with the GPU library and never imports it.

This module compiles spec_oracle.c with the host C compiler (plain -O2, no
fast-math) into liboracle.so next to it and wraps the entry points with ctypes
over NumPy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FLOAT32, BFLOAT16, FLOAT64 = 0, 1, 2

ST_TOKEN_RANGE, ST_D2T, ST_NO_MASS, ST_BAD_PARENT = 1, 2, 4, 8
FL_ACCEPT_EDGE, FL_CDF_EDGE, FL_ZERO_RESID = 1, 2, 4

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle.  Plain C, -O2, IEEE semantics (no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = C.CDLL(_LIB)
        P = C.c_void_p
        i32, f64 = C.c_int, C.c_double
        lib.oracle_verify_sample.argtypes = [P, i32, P, i32, P, P, P, P, i32, i32, i32, i32,
                                             f64, f64, f64, P, P, P, P, P, P, P, P, i32]
        lib.oracle_row_dist.argtypes = [P, i32, i32, f64, f64, i32, i32, P, P, P, P]
        lib.oracle_draft_sample.argtypes = [P, i32, P, P, i32, i32, f64, f64, i32, f64, P, P, P, P, P, P, P]
        lib.oracle_count.argtypes = [P, i32, i32, P]
        lib.oracle_fanout_lookup.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, P]
        lib.oracle_vocab_trim.argtypes = [P, C.c_int64, i32, f64, P, P, P, P]
        lib.oracle_greedy_from_argmax.argtypes = [P, P, i32, i32, i32, P, P, P]
        lib.oracle_tree_from_argmax.argtypes = [P, P, P, i32, i32, i32, P, P, P, P]
        lib.oracle_chain_from_dists.argtypes = [P, P, P, P, C.c_float, i32, i32, C.c_double, P, P]
        lib.oracle_verify_greedy.argtypes = [P, i32, P, i32, i32, i32, P, P, P]
        lib.oracle_verify_tree_greedy.argtypes = [P, i32, P, P, i32, i32, i32, P, P, P, P]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _logits(a):
    """Raw logits as (contiguous array, dtype code).  bfloat16 arrives as uint16 bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, FLOAT32
    if a.dtype == np.uint16:
        return a, BFLOAT16
    if a.dtype == np.float64:
        return a, FLOAT64
    raise TypeError("logits must be float32, float64 or uint16 (bfloat16 bits), got %s" % a.dtype)


def verify_sample(target_logits, draft_logits, tokens, u_accept, u_sample, temperature, top_p,
                  d2t=None, band=1e-5, k_delta=None, nthreads=1):
    """Sampling verification of a batch.  Returns a dict of NumPy arrays:
    tokens [B, g+1], accept_len [B], p_tok/q_tok [B, g] (float64), status [B],
    flags [B] (boundary diagnostics), margin [B, 2g+1, 2] (top-p margins, target
    rows then draft rows)."""
    tl, tdt = _logits(target_logits)
    B, g1, Vt = tl.shape
    g = g1 - 1
    if g > 0:
        dl, ddt = _logits(draft_logits)
        Vd = dl.shape[2]
        assert dl.shape[:2] == (B, g)
    else:
        dl, ddt, Vd = np.zeros(1, np.float32), FLOAT32, (Vt if d2t is None else len(d2t))
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, g)
    ua = np.ascontiguousarray(u_accept, dtype=np.float32).reshape(B, g)
    us = np.ascontiguousarray(u_sample, dtype=np.float32).reshape(B)
    dm = None if d2t is None else np.ascontiguousarray(d2t, dtype=np.int32)
    kd = None if k_delta is None else np.ascontiguousarray(k_delta, dtype=np.int8).reshape(B, 2 * g + 1)
    out = dict(tokens=np.empty((B, g + 1), np.int32), accept_len=np.empty(B, np.int32),
               p_tok=np.empty((B, g), np.float64), q_tok=np.empty((B, g), np.float64),
               status=np.empty(B, np.int32), flags=np.empty(B, np.int32),
               margin=np.empty((B, 2 * g + 1, 2), np.float64))
    rc = _load().oracle_verify_sample(
        _ptr(tl), tdt, _ptr(dl), ddt, _ptr(tok), _ptr(dm), _ptr(ua), _ptr(us),
        B, g, Vt, Vd, float(temperature), float(top_p), float(band), _ptr(kd),
        _ptr(out["tokens"]), _ptr(out["accept_len"]), _ptr(out["p_tok"]), _ptr(out["q_tok"]),
        _ptr(out["status"]), _ptr(out["flags"]), _ptr(out["margin"]), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_verify_sample: bad arguments (code %d)" % rc)
    return out


def row_dist(z, temperature, top_p, k_delta=0, top_k=0):
    """D1 on one row: returns (p [V] float64, status, k, margin_lo, margin_hi).
    top_k caps the kept count (the draft-side sampler's reading; 0 = off); k
    is the top-p count before the cap."""
    z, dt = _logits(np.asarray(z).reshape(-1))
    V = z.shape[0]
    p = np.empty(V, np.float64)
    k = np.zeros(1, np.int32)
    lo = np.zeros(1, np.float64)
    hi = np.zeros(1, np.float64)
    st = _load().oracle_row_dist(_ptr(z), dt, V, float(temperature), float(top_p), int(top_k), int(k_delta),
                                 _ptr(p), _ptr(k), _ptr(lo), _ptr(hi))
    if st < 0:
        raise ValueError("oracle_row_dist: bad arguments")
    return p, st, int(k[0]), float(lo[0]), float(hi[0])


def chain_from_dists(P, Q, tokens, u_accept, u_sample, band=0.0):
    """D3-D6 on given distributions P [g+1, V], Q [g, V] (float64).  Returns
    (n, tokens [g+1], flags): flags are the boundary diagnostics of
    verify_sample for the given band (0 with band = 0)."""
    P = np.ascontiguousarray(P, dtype=np.float64)
    g1, V = P.shape
    g = g1 - 1
    Q = np.ascontiguousarray(Q if g > 0 else np.zeros((1, V)), dtype=np.float64)
    tok = np.zeros(max(g, 1), np.int32)
    ua = np.zeros(max(g, 1), np.float32)
    if g > 0:
        tok[:] = np.asarray(tokens, dtype=np.int32).reshape(g)
        ua[:] = np.asarray(u_accept, dtype=np.float32).reshape(g)
    out = np.empty(g + 1, np.int32)
    fl = np.zeros(1, np.int32)
    n = _load().oracle_chain_from_dists(_ptr(P), _ptr(Q), _ptr(tok), _ptr(ua),
                                        C.c_float(float(u_sample)), g, V, C.c_double(float(band)),
                                        _ptr(out), _ptr(fl))
    if n < 0:
        raise MemoryError("oracle_chain_from_dists")
    return n, out, int(fl[0])


def draft_sample(logits, u, temperature, top_p, top_k=0, d2t=None, band=1e-5, k_delta=None):
    """D9: one draw per row of logits [B, V] with uniforms u [B].  Returns a
    dict: tokens [B] (target ids through d2t when given), prob [B] (p of the
    drawn id, float64), status [B], flags [B] (CDF-edge diagnostics), margin
    [B, 2] (top-p margins), k [B] (top-p count before the top-k cap)."""
    lg, dt = _logits(logits)
    B, V = lg.shape
    uu = np.ascontiguousarray(u, dtype=np.float32).reshape(B)
    dm = None if d2t is None else np.ascontiguousarray(d2t, dtype=np.int32)
    kd = None if k_delta is None else np.ascontiguousarray(k_delta, dtype=np.int8).reshape(B)
    out = dict(tokens=np.empty(B, np.int32), prob=np.empty(B, np.float64), status=np.empty(B, np.int32),
               flags=np.empty(B, np.int32), margin=np.empty((B, 2), np.float64), k=np.empty(B, np.int32))
    rc = _load().oracle_draft_sample(_ptr(lg), dt, _ptr(dm), _ptr(uu), B, V, float(temperature), float(top_p),
                                     int(top_k), float(band), _ptr(kd), _ptr(out["tokens"]), _ptr(out["prob"]),
                                     _ptr(out["status"]), _ptr(out["flags"]), _ptr(out["margin"]), _ptr(out["k"]))
    if rc != 0:
        raise ValueError("oracle_draft_sample: bad arguments (code %d)" % rc)
    return out


def count(accept_len, gamma, counters=None):
    """Acceptance counters (target calls, drafted, accepted, emitted, invalid)
    after adding one call's accept_len [B]."""
    a = np.ascontiguousarray(accept_len, dtype=np.int32).reshape(-1)
    c = np.zeros(5, np.uint64) if counters is None else np.ascontiguousarray(counters, dtype=np.uint64).copy()
    rc = _load().oracle_count(_ptr(a), a.shape[0], int(gamma), _ptr(c))
    if rc != 0:
        raise ValueError("oracle_count: bad arguments")
    return c


def fanout_lookup(out_tokens, accept_len, cand, drafts, counters=None):
    """D10: SSD fan-out lookup.  out_tokens [B, g+1], accept_len [B], cand
    [B, g+1, f], drafts [B, (g+1) f, L].  Returns (branch [B], next [B, L],
    counters [2] = lookups, hits)."""
    ot = np.ascontiguousarray(out_tokens, dtype=np.int32)
    B, g1 = ot.shape
    al = np.ascontiguousarray(accept_len, dtype=np.int32).reshape(B)
    cd = np.ascontiguousarray(cand, dtype=np.int32)
    f = cd.shape[2]
    dr = np.ascontiguousarray(drafts, dtype=np.int32)
    L = dr.shape[2]
    br = np.empty(B, np.int32)
    nx = np.empty((B, L), np.int32)
    c = np.zeros(2, np.uint64) if counters is None else np.ascontiguousarray(counters, dtype=np.uint64).copy()
    rc = _load().oracle_fanout_lookup(_ptr(ot), _ptr(al), _ptr(cd), _ptr(dr), B, g1 - 1, f, L, _ptr(br), _ptr(nx),
                                      _ptr(c))
    if rc != 0:
        raise ValueError("oracle_fanout_lookup: bad arguments")
    return br, nx, c


def vocab_trim(tokens, Vt, P):
    """D11: vocabulary trim.  Returns (d2t [Vd] ascending, t2d [Vt], info =
    (kept mass, valid tokens, invalid tokens))."""
    tk = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
    d2t = np.empty(Vt, np.int32)
    t2d = np.empty(Vt, np.int32)
    vd = np.zeros(1, np.int32)
    info = np.zeros(3, np.int64)
    rc = _load().oracle_vocab_trim(_ptr(tk), tk.shape[0], int(Vt), float(np.float32(P)), _ptr(d2t), _ptr(t2d),
                                   _ptr(vd), _ptr(info))
    if rc != 0:
        raise ValueError("oracle_vocab_trim: bad arguments")
    return d2t[:vd[0]].copy(), t2d, info


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def lmhead_logits(hidden_bits, W_bits):
    """D12: the lm_head's logits in float64: hidden [M, d] times W [V, d]^T from
    bfloat16 bit patterns (widened exactly; numpy's float64 matmul), and the
    same product of the absolute values, |hidden| |W|^T, which bounds the
    rounding of any float32 accumulation of the same terms."""
    h = _bf16_to_f64(hidden_bits)
    w = _bf16_to_f64(W_bits)
    return h @ w.T, np.abs(h) @ np.abs(w).T


def lmhead_admissible(z, zabs, eps):
    """Per row of float64 logits z [M, V]: the argmax (lowest id on ties) and
    a boolean mask of the ids a float32 accumulation with relative error
    eps (of |h||w|) may also report as the maximum: z_v >= z_max -
    eps (zabs_v + zabs_max)."""
    g = np.argmax(z, axis=1)
    rows = np.arange(z.shape[0])
    zm = z[rows, g]
    am = zabs[rows, g]
    return g.astype(np.int32), z >= zm[:, None] - eps * (zabs + am[:, None])


def greedy_from_argmax(g, tokens, V):
    """D7's chain on given row argmaxes g [B, g+1]."""
    gg = np.ascontiguousarray(g, dtype=np.int32)
    B, g1 = gg.shape
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, g1 - 1)
    out = dict(tokens=np.empty((B, g1), np.int32), accept_len=np.empty(B, np.int32), status=np.empty(B, np.int32))
    rc = _load().oracle_greedy_from_argmax(_ptr(gg), _ptr(tok), B, g1 - 1, int(V), _ptr(out["tokens"]),
                                           _ptr(out["accept_len"]), _ptr(out["status"]))
    if rc != 0:
        raise ValueError("oracle_greedy_from_argmax: bad arguments")
    return out


def tree_from_argmax(g, node_tokens, parents, V):
    """D8's walk on given row argmaxes g [B, N]."""
    gg = np.ascontiguousarray(g, dtype=np.int32)
    B, N = gg.shape
    nt = np.ascontiguousarray(node_tokens, dtype=np.int32).reshape(B, N)
    pa = np.ascontiguousarray(parents, dtype=np.int32).reshape(B, N)
    out = dict(path=np.empty((B, N), np.int32), tokens=np.empty((B, N), np.int32),
               accept_len=np.empty(B, np.int32), status=np.empty(B, np.int32))
    rc = _load().oracle_tree_from_argmax(_ptr(gg), _ptr(nt), _ptr(pa), B, N, int(V), _ptr(out["path"]),
                                         _ptr(out["tokens"]), _ptr(out["accept_len"]), _ptr(out["status"]))
    if rc != 0:
        raise ValueError("oracle_tree_from_argmax: bad arguments")
    return out


def verify_greedy(logits, tokens):
    """Greedy verification: returns dict(tokens [B, g+1], accept_len [B], status [B])."""
    lg, dt = _logits(logits)
    B, g1, V = lg.shape
    g = g1 - 1
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, g)
    out = dict(tokens=np.empty((B, g + 1), np.int32), accept_len=np.empty(B, np.int32),
               status=np.empty(B, np.int32))
    rc = _load().oracle_verify_greedy(_ptr(lg), dt, _ptr(tok), B, g, V, _ptr(out["tokens"]),
                                      _ptr(out["accept_len"]), _ptr(out["status"]))
    if rc != 0:
        raise ValueError("oracle_verify_greedy: bad arguments")
    return out


def verify_tree_greedy(logits, node_tokens, parents):
    """Greedy tree verification: returns dict(path [B, N], tokens [B, N], accept_len [B], status [B])."""
    lg, dt = _logits(logits)
    B, N, V = lg.shape
    nt = np.ascontiguousarray(node_tokens, dtype=np.int32).reshape(B, N)
    pa = np.ascontiguousarray(parents, dtype=np.int32).reshape(B, N)
    out = dict(path=np.empty((B, N), np.int32), tokens=np.empty((B, N), np.int32),
               accept_len=np.empty(B, np.int32), status=np.empty(B, np.int32))
    rc = _load().oracle_verify_tree_greedy(_ptr(lg), dt, _ptr(nt), _ptr(pa), B, N, V,
                                           _ptr(out["path"]), _ptr(out["tokens"]),
                                           _ptr(out["accept_len"]), _ptr(out["status"]))
    if rc != 0:
        raise ValueError("oracle_verify_tree_greedy: bad arguments")
    return out
