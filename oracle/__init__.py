"""fp64 CPU oracle for gated-delta-rule draft verification (ctypes binding).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and nothing here
imports the product path.

Every function takes numpy arrays holding the exact values handed to the GPU
(fp32, bf16 inputs widened exactly to fp32) and computes in fp64 by walking
each root-to-node path token by token (see oracle.c for the definition and its
citations).  ``Oracle(path)`` binds one compiled copy of oracle.c; the
module-level functions use the default build, oracle/liboracle.so.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

__all__ = ["Oracle", "default", "verify", "commit", "chain_decode", "log_decay", "verify_dfs",
           "gather", "read_states", "select", "BAD_PARENT", "BAD_ACCEPTED", "BAD_SLOT",
           "BAD_POSITION"]

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)

BAD_PARENT = 1
BAD_ACCEPTED = 2
BAD_SLOT = 4
BAD_POSITION = 8


def _threads(n):
    return int(n) if n else (os.cpu_count() or 1)


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _i32(x):
    return np.ascontiguousarray(x, dtype=np.int32)


def _p(x, t):
    return None if x is None else x.ctypes.data_as(t)


class Oracle:
    """One compiled copy of oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i = ctypes.c_int
        lib.oracle_verify.argtypes = [i, i, i, i, i, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p,
                                      _i32p, _f64p, _f64p, _f64p, i]
        lib.oracle_commit.argtypes = [i, i, i, i, i, _f32p, _f32p, _f32p, _f32p, _f32p, _i32p,
                                      _i32p, _f64p, i]
        lib.oracle_chain_decode.argtypes = [i, i, i, i, i, _f32p, _f32p, _f32p, _f32p, _f32p,
                                            _f32p, _f64p, i]
        lib.oracle_verify_dfs.argtypes = [i, i, i, i, i, _f32p, _f32p, _f32p, _f32p, _f32p,
                                          _f32p, _i32p, _f64p, i]
        lib.oracle_gather.argtypes = [i, i, i, i, i, i, i, _f32p, _i32p, _f32p, _f64p, _f32p, i]
        lib.oracle_read_states.argtypes = [i, i, i, i, i, i, i, _f32p, _f32p, _f32p, _f32p, _f32p,
                                           _i32p, _i32p, _f32p, _f64p, i]
        lib.oracle_select.argtypes = [i, i, ctypes.c_long, _f32p, _i32p, _i32p, _i32p, _i32p,
                                      _i32p, _i32p, i]
        lib.oracle_log_decay.argtypes = [i, i, i, _f32p, _i32p, _f64p]
        for f in ("oracle_verify", "oracle_commit", "oracle_chain_decode", "oracle_log_decay",
                  "oracle_verify_dfs", "oracle_gather", "oracle_read_states", "oracle_select"):
            getattr(lib, f).restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def verify(self, q, k, v, a, beta, S0, parent=None, want_states=False, want_u=False,
               nthreads=None):
        """All node outputs o[b, n, h, :] = S_n q_n (fp64), and optionally every
        node state S_n.  parent=None means a chain.  Returns (o, states, status),
        or (o, u, states, status) with ``want_u`` (u_n the node corrections)."""
        q, k, v, a, beta, S0 = map(_f32, (q, k, v, a, beta, S0))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        par = None if parent is None else _i32(parent)
        o = np.zeros((B, T, H, dv), dtype=np.float64)
        u = np.zeros((B, T, H, dv), dtype=np.float64) if want_u else None
        st = np.zeros((B, T, H, dv, dk), dtype=np.float64) if want_states else None
        status = self.lib.oracle_verify(B, T, H, dk, dv, _p(q, _f32p), _p(k, _f32p), _p(v, _f32p),
                                        _p(a, _f32p), _p(beta, _f32p), _p(S0, _f32p),
                                        _p(par, _i32p), _p(o, _f64p), _p(u, _f64p), _p(st, _f64p),
                                        _threads(nthreads))
        if want_u:
            return o, u, st, status
        return o, st, status

    def commit(self, k, v, a, beta, S0, accepted, parent=None, nthreads=None):
        """Committed state per (b, h): the state at accepted[b], S0 when -1.
        Returns (S_out fp64 [B, H, dv, dk], status)."""
        k, v, a, beta, S0 = map(_f32, (k, v, a, beta, S0))
        B, T, H, dk = k.shape
        dv = v.shape[-1]
        par = None if parent is None else _i32(parent)
        acc = _i32(accepted)
        S_out = np.zeros((B, H, dv, dk), dtype=np.float64)
        status = self.lib.oracle_commit(B, T, H, dk, dv, _p(k, _f32p), _p(v, _f32p), _p(a, _f32p),
                                        _p(beta, _f32p), _p(S0, _f32p), _p(par, _i32p),
                                        _p(acc, _i32p), _p(S_out, _f64p), _threads(nthreads))
        return S_out, status

    def log_decay(self, a, parent=None):
        """log P_n per (b, n, h): the log of the product of the decay gates on
        the root-to-n path, multiplied in fp64 along the walk.  parent=None
        means a chain.  Returns (logp fp64 [B, T, H], status)."""
        a = _f32(a)
        B, T, H = a.shape
        par = None if parent is None else _i32(parent)
        logp = np.zeros((B, T, H), dtype=np.float64)
        status = self.lib.oracle_log_decay(B, T, H, _p(a, _f32p), _p(par, _i32p), _p(logp, _f64p))
        return logp, status

    def chain_decode(self, q, k, v, a, beta, S0, nthreads=None):
        """Sequential decode with one running state: o_n read after token n."""
        q, k, v, a, beta, S0 = map(_f32, (q, k, v, a, beta, S0))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        o = np.zeros((B, T, H, dv), dtype=np.float64)
        self.lib.oracle_chain_decode(B, T, H, dk, dv, _p(q, _f32p), _p(k, _f32p), _p(v, _f32p),
                                     _p(a, _f32p), _p(beta, _f32p), _p(S0, _f32p), _p(o, _f64p),
                                     _threads(nthreads))
        return o

    def verify_dfs(self, q, k, v, a, beta, S0, parent, nthreads=None):
        """Branch-by-branch depth-first traversal, one state per tree edge."""
        q, k, v, a, beta, S0 = map(_f32, (q, k, v, a, beta, S0))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        par = _i32(parent)
        o = np.zeros((B, T, H, dv), dtype=np.float64)
        status = self.lib.oracle_verify_dfs(B, T, H, dk, dv, _p(q, _f32p), _p(k, _f32p),
                                            _p(v, _f32p), _p(a, _f32p), _p(beta, _f32p),
                                            _p(S0, _f32p), _p(par, _i32p), _p(o, _f64p),
                                            _threads(nthreads))
        return o, status

    def gather(self, pool, slot, queries=None, want_states=True, nthreads=None):
        """Reads at chosen pool slots: (o fp64 [B, P, H, Qn, dv] or None,
        states fp32 [B, P, H, dv, dk] or None, status)."""
        pool = _f32(pool)
        slot = _i32(slot)
        num_slots, H, dv, dk = pool.shape
        B, P = slot.shape
        qv = None if queries is None else _f32(queries)
        Qn = 0 if qv is None else qv.shape[3]
        o = None if qv is None else np.zeros((B, P, H, Qn, dv), dtype=np.float64)
        st = np.zeros((B, P, H, dv, dk), dtype=np.float32) if want_states else None
        status = self.lib.oracle_gather(B, P, H, dk, dv, num_slots, Qn, _p(pool, _f32p),
                                        _p(slot, _i32p), _p(qv, _f32p), _p(o, _f64p),
                                        _p(st, _f32p), _threads(nthreads))
        return o, st, status

    def read_states(self, k, v, a, beta, S0, pos, queries, parent=None, nthreads=None):
        """Reads of in-block states: o[b, p, h, i] = S_{pos[b, p]} q (S0 for
        position -1).  Returns (o fp64 [B, P, H, Qn, dv], status)."""
        k, v, a, beta, S0, qv = map(_f32, (k, v, a, beta, S0, queries))
        B, T, H, dk = k.shape
        dv = v.shape[-1]
        pos = _i32(pos)
        P, Qn = pos.shape[1], qv.shape[3]
        par = None if parent is None else _i32(parent)
        o = np.zeros((B, P, H, Qn, dv), dtype=np.float64)
        status = self.lib.oracle_read_states(B, T, H, dk, dv, P, Qn, _p(k, _f32p), _p(v, _f32p),
                                             _p(a, _f32p), _p(beta, _f32p), _p(S0, _f32p),
                                             _p(par, _i32p), _p(pos, _i32p), _p(qv, _f32p),
                                             _p(o, _f64p), _threads(nthreads))
        return o, status

    def select(self, logits, tokens, parent=None, nthreads=None):
        """Greedy accepted-node selection.  logits [B, T+1, V] (fp32 values),
        tokens [B, T].  Returns (target [B, T+1], accepted [B], acc_len [B],
        bonus [B], status); entries of a sequence with an invalid parent row
        are -2 in accepted, acc_len and bonus."""
        lg = _f32(logits)
        tok = _i32(tokens)
        B, T1, V = lg.shape
        T = T1 - 1
        par = None if parent is None else _i32(parent)
        target = np.zeros((B, T1), dtype=np.int32)
        acc = np.full(B, -2, dtype=np.int32)
        alen = np.full(B, -2, dtype=np.int32)
        bonus = np.full(B, -2, dtype=np.int32)
        status = self.lib.oracle_select(B, T, V, _p(lg, _f32p), _p(tok, _i32p), _p(par, _i32p),
                                        _p(target, _i32p), _p(acc, _i32p), _p(alen, _i32p),
                                        _p(bonus, _i32p), _threads(nthreads))
        return target, acc, alen, bonus, status


_DEFAULT = None


def default() -> Oracle:
    """The oracle built from oracle.c into oracle/liboracle.so (built on first use)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _DEFAULT = Oracle(_build.LIB)
    return _DEFAULT


def verify(*args, **kw):
    return default().verify(*args, **kw)


def commit(*args, **kw):
    return default().commit(*args, **kw)


def chain_decode(*args, **kw):
    return default().chain_decode(*args, **kw)


def log_decay(*args, **kw):
    return default().log_decay(*args, **kw)


def verify_dfs(*args, **kw):
    return default().verify_dfs(*args, **kw)


def gather(*args, **kw):
    return default().gather(*args, **kw)


def read_states(*args, **kw):
    return default().read_states(*args, **kw)


def select(*args, **kw):
    return default().select(*args, **kw)
