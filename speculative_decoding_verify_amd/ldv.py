"""Python binding of the ldv C ABI (include/ldv.h): argument marshalling only.

Every step of the verify / commit / gather path runs in the HIP kernels of
libldv.so.  This module checks tensor placement, dtype, shape and layout,
allocates outputs that the caller did not pass, and hands raw device pointers
and torch's current HIP stream to the library.  There is no fallback: if the
library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libldv.so")

LDV_OK, LDV_ERR_ARG, LDV_ERR_UNSUPPORTED, LDV_ERR_LAUNCH = 0, -1, -2, -3
LDV_BF16, LDV_F32 = 0, 1
STATUS_BAD_PARENT, STATUS_BAD_ACCEPTED, STATUS_BAD_SLOT, STATUS_BAD_POSITION = 1, 2, 4, 8
MAX_T = 64
MAX_LONG_T = 8192

_lib = None


class LdvError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__("%s failed: %d (%s)" % (fn, code, status_string(code)))
        self.code = code


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libldv.so (built by speculative_decoding_verify_amd/build.py)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError("libldv.so not found at %s: build it with "
                          "`python speculative_decoding_verify_amd/build.py`" % p)
    lib = ctypes.CDLL(p)
    i, vp, fp, ip = ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.ldv_verify_tree.argtypes = [i, i, i, i, i, i, vp, vp, vp, fp, fp, fp, ip, fp, fp, fp, ip, vp]
    lib.ldv_verify_chain.argtypes = [i, i, i, i, i, i, vp, vp, vp, fp, fp, fp, fp, fp, fp, ip, vp]
    lib.ldv_verify_chain_long.argtypes = [i, i, i, i, i, i, vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, ip, vp]
    lib.ldv_commit_state.argtypes = [i, i, i, i, i, i, vp, fp, fp, ip, ip, fp, fp, ip, vp]
    lib.ldv_gather_states.argtypes = [i, i, i, i, i, i, i, i, fp, ip, vp, fp, fp, ip, vp]
    lib.ldv_read_block_states.argtypes = [i, i, i, i, i, i, i, i, vp, fp, fp, ip, fp, ip, vp, fp, ip, vp]
    ll = ctypes.c_longlong
    lib.ldv_gather_states_packed.argtypes = [i, i, i, i, i, i, i, i, fp, ip, vp, vp, ll, ll, i, ip, vp]
    lib.ldv_read_block_states_packed.argtypes = [i, i, i, i, i, i, i, i, vp, fp, fp, ip, fp, ip, vp, vp, ll, ll, i,
                                                 ip, vp]
    lib.ldv_select_accepted.argtypes = [i, i, i, i, vp, ip, ip, ip, ip, ip, ip, ip, vp, ctypes.c_size_t, vp]
    lib.ldv_select_accepted_noalloc.argtypes = [i, i, i, i, vp, ip, ip, ip, ip, ip, ip, ip, vp]
    lib.ldv_select_workspace_bytes.argtypes = [i, i, i]
    lib.ldv_select_workspace_bytes.restype = ctypes.c_size_t
    for f in ("ldv_verify_tree", "ldv_verify_chain", "ldv_verify_chain_long", "ldv_commit_state", "ldv_gather_states",
              "ldv_read_block_states", "ldv_gather_states_packed", "ldv_read_block_states_packed",
              "ldv_select_accepted", "ldv_select_accepted_noalloc", "ldv_version"):
        getattr(lib, f).restype = ctypes.c_int
    lib.ldv_status_string.argtypes = [ctypes.c_int]
    lib.ldv_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().ldv_status_string(int(code)).decode()


# ------------------------------------------------------------- marshalling

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU (got %s)" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    return t


def _qkv_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LDV_BF16
    if t.dtype == torch.float32:
        return LDV_F32
    raise TypeError("q/k/v/queries must be bfloat16 or float32 (got %s)" % t.dtype)


def _stream(stream, dev: torch.device) -> ctypes.c_void_p:
    """The HIP stream to enqueue on: the given one, else torch's current
    stream of the tensors' device."""
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif stream.device != dev:
        raise ValueError("stream is on %s, the tensors on %s" % (stream.device, dev))
    return ctypes.c_void_p(stream.cuda_stream)


def _same_device(dev: torch.device, **tensors):
    """One call works on one GPU: every tensor it is given must be there."""
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError("%s is on %s, the call's other tensors on %s" % (name, t.device, dev))


def _check(fn: str, rc: int):
    if rc != LDV_OK:
        raise LdvError(fn, rc)


def _invoke(fn: str, dev: torch.device, *args):
    """Call the C entry point with ``dev`` current, so that the HIP runtime
    and the stream agree on the device."""
    with torch.cuda.device(dev):
        rc = getattr(load(), fn)(*args)
    _check(fn, rc)


def _alloc(shape, dtype, dev, stream):
    """A new device tensor for an output or scratch buffer of a call that
    enqueues on ``stream``.  torch's caching allocator ties a block to the
    stream current at allocation; when the call runs on another stream, the
    block is also recorded on that one, so that it is not handed out again
    (for instance once a dropped scratch tensor is freed) before the call's
    kernels are done with it."""
    t = torch.empty(shape, dtype=dtype, device=dev)
    if stream is not None and stream != torch.cuda.current_stream(dev):
        t.record_stream(stream)
    return t


def _opt(t, name, dtype, shape, dev, stream=None):
    if t is None:
        return _alloc(shape, dtype, dev, stream)
    return _dev(t, name, dtype, shape)


def _verify(fn, q, k, v, a, beta, S0, parent, o, u, logp, factors, status, stream):
    _dev(q, "q")
    B, T, H, dk = q.shape
    code = _qkv_code(q)
    _dev(k, "k", q.dtype, (B, T, H, dk))
    _dev(v, "v", q.dtype)
    if v.dim() != 4 or tuple(v.shape[:3]) != (B, T, H):
        raise ValueError("v must have shape [B, T, H, dv]")
    dv = v.shape[3]
    _dev(a, "a", torch.float32, (B, T, H))
    _dev(beta, "beta", torch.float32, (B, T, H))
    _dev(S0, "S0", torch.float32, (B, H, dv, dk))
    dev = q.device
    o = _opt(o, "o", torch.float32, (B, T, H, dv), dev, stream)
    if factors:
        u = _opt(u, "u", torch.float32, (B, T, H, dv), dev, stream)
        logp = _opt(logp, "logp", torch.float32, (B, T, H), dev, stream)
    else:
        u = logp = None
    if status is not None:
        _dev(status, "status", torch.int32)
    args = [B, T, H, dk, dv, code, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(S0)]
    if fn == "ldv_verify_tree":
        _dev(parent, "parent", torch.int32, (B, T))
        args.append(_ptr(parent))
    _same_device(dev, k=k, v=v, a=a, beta=beta, S0=S0, parent=parent, o=o, u=u, logp=logp, status=status)
    args += [_ptr(o), _ptr(u), _ptr(logp), _ptr(status), _stream(stream, dev)]
    _invoke(fn, dev, *args)
    return o, u, logp


def verify_chain(q, k, v, a, beta, S0, o=None, u=None, logp=None, factors=True,
                 status=None, stream=None):
    """Verify a chain of T drafts per sequence (parent[n] = n - 1).

    q, k [B, T, H, dk] and v [B, T, H, dv] (bf16 or fp32, same dtype);
    a, beta [B, T, H] fp32; S0 [B, H, dv, dk] fp32.  Returns (o, u, logp):
    o [B, T, H, dv] fp32 and, when ``factors``, the commit factors u
    [B, T, H, dv] and logp [B, T, H] (else None)."""
    return _verify("ldv_verify_chain", q, k, v, a, beta, S0, None, o, u, logp, factors, status, stream)


def verify_tree(q, k, v, a, beta, S0, parent, o=None, u=None, logp=None, factors=True,
                status=None, stream=None):
    """Verify a draft tree per sequence; parent [B, T] int32, parent[n] in [-1, n-1]."""
    return _verify("ldv_verify_tree", q, k, v, a, beta, S0, parent, o, u, logp, factors, status, stream)


def verify_chain_long(q, k, v, a, beta, S0, o=None, u=None, logp=None, S_work=None, status=None,
                      stream=None):
    """Verify a chain of any length (up to MAX_LONG_T) in chunks of MAX_T
    nodes, each from the state at the end of the previous chunk.  Same
    arguments and results as verify_chain (u and logp are always produced);
    S_work [B, H, dv, dk] fp32 is scratch, allocated here when not given and
    T > MAX_T.  Returns (o, u, logp)."""
    _dev(q, "q")
    B, T, H, dk = q.shape
    code = _qkv_code(q)
    _dev(k, "k", q.dtype, (B, T, H, dk))
    _dev(v, "v", q.dtype)
    if v.dim() != 4 or tuple(v.shape[:3]) != (B, T, H):
        raise ValueError("v must have shape [B, T, H, dv]")
    dv = v.shape[3]
    _dev(a, "a", torch.float32, (B, T, H))
    _dev(beta, "beta", torch.float32, (B, T, H))
    _dev(S0, "S0", torch.float32, (B, H, dv, dk))
    dev = q.device
    o = _opt(o, "o", torch.float32, (B, T, H, dv), dev, stream)
    u = _opt(u, "u", torch.float32, (B, T, H, dv), dev, stream)
    logp = _opt(logp, "logp", torch.float32, (B, T, H), dev, stream)
    if S_work is None and T > MAX_T:
        S_work = _alloc((B, H, dv, dk), torch.float32, dev, stream)
    elif S_work is not None:
        _dev(S_work, "S_work", torch.float32, (B, H, dv, dk))
    if status is not None:
        _dev(status, "status", torch.int32)
    _same_device(dev, k=k, v=v, a=a, beta=beta, S0=S0, o=o, u=u, logp=logp, S_work=S_work, status=status)
    _invoke("ldv_verify_chain_long", dev,
            B, T, H, dk, dv, code, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(S0), _ptr(o), _ptr(u),
            _ptr(logp), _ptr(S_work), _ptr(status), _stream(stream, dev))
    return o, u, logp


def commit_state(k, u, logp, accepted, S0, S_out=None, parent=None, status=None, stream=None):
    """Materialise the accepted node's state.  ``S_out=S0`` commits in place.

    k [B, T, H, dk] (bf16/fp32), u [B, T, H, dv] and logp [B, T, H] from the
    verify call, accepted [B] int32 in [-1, T-1], parent [B, T] int32 or None
    (chain).  Returns S_out [B, H, dv, dk] fp32."""
    _dev(k, "k")
    B, T, H, dk = k.shape
    code = _qkv_code(k)
    _dev(u, "u", torch.float32)
    if u.dim() != 4 or tuple(u.shape[:3]) != (B, T, H):
        raise ValueError("u must have shape [B, T, H, dv]")
    dv = u.shape[3]
    _dev(logp, "logp", torch.float32, (B, T, H))
    _dev(accepted, "accepted", torch.int32, (B,))
    _dev(S0, "S0", torch.float32, (B, H, dv, dk))
    if parent is not None:
        _dev(parent, "parent", torch.int32, (B, T))
    S_out = _opt(S_out, "S_out", torch.float32, (B, H, dv, dk), k.device, stream)
    if S_out.data_ptr() != S0.data_ptr():
        lo0, hi0 = S0.data_ptr(), S0.data_ptr() + S0.numel() * 4
        lo1, hi1 = S_out.data_ptr(), S_out.data_ptr() + S_out.numel() * 4
        if lo0 < hi1 and lo1 < hi0:
            raise ValueError("S_out overlaps S0 without being S0")
    if status is not None:
        _dev(status, "status", torch.int32)
    dev = k.device
    _same_device(dev, u=u, logp=logp, accepted=accepted, S0=S0, parent=parent, S_out=S_out, status=status)
    _invoke("ldv_commit_state", dev,
            B, T, H, dk, dv, code, _ptr(k), _ptr(u), _ptr(logp), _ptr(parent), _ptr(accepted),
            _ptr(S0), _ptr(S_out), _ptr(status), _stream(stream, dev))
    return S_out


def gather_states(pool, slot, queries=None, o=None, states_out=None, want_states=False,
                  status=None, stream=None):
    """Read pool states at slot[b, p]: o = pool[slot, h] q_i for each query and,
    when ``want_states`` (or states_out is given), a bit copy of the states.

    pool [num_slots, H, dv, dk] fp32; slot [B, P] int32; queries
    [B, P, H, Qn, dk] bf16/fp32 or None.  Returns (o, states_out)."""
    _dev(pool, "pool", torch.float32)
    num_slots, H, dv, dk = pool.shape
    _dev(slot, "slot", torch.int32)
    B, P = slot.shape
    dev = pool.device
    code, Qn = LDV_BF16, 0
    if queries is not None:
        _dev(queries, "queries")
        code = _qkv_code(queries)
        if queries.dim() != 5 or tuple(queries.shape[:3]) != (B, P, H) or queries.shape[4] != dk:
            raise ValueError("queries must have shape [B, P, H, Qn, dk]")
        Qn = queries.shape[3]
        o = _opt(o, "o", torch.float32, (B, P, H, Qn, dv), dev, stream)
    else:
        o = None
    if states_out is None and want_states:
        states_out = _alloc((B, P, H, dv, dk), torch.float32, dev, stream)
    elif states_out is not None:
        _dev(states_out, "states_out", torch.float32, (B, P, H, dv, dk))
    if status is not None:
        _dev(status, "status", torch.int32)
    _same_device(dev, slot=slot, queries=queries, o=o, states_out=states_out, status=status)
    _invoke("ldv_gather_states", dev,
            B, P, H, dk, dv, num_slots, Qn, code, _ptr(pool), _ptr(slot), _ptr(queries), _ptr(o),
            _ptr(states_out), _ptr(status), _stream(stream, dev))
    return o, states_out


def read_block_states(k, u, logp, S0, pos, queries, parent=None, o=None, status=None, stream=None):
    """Read states inside the verified block without forming them:
    o[b, p, h, i] = S_j q with j = pos[b, p] in [-1, T-1] (S0 for -1).

    k [B, T, H, dk] (bf16/fp32) and u [B, T, H, dv], logp [B, T, H] from the
    verify call on the same S0 [B, H, dv, dk]; pos [B, P] int32; queries
    [B, P, H, Qn, dk] with k's dtype; parent [B, T] int32 or None (chain).
    Returns o [B, P, H, Qn, dv] fp32."""
    _dev(k, "k")
    B, T, H, dk = k.shape
    code = _qkv_code(k)
    _dev(u, "u", torch.float32)
    if u.dim() != 4 or tuple(u.shape[:3]) != (B, T, H):
        raise ValueError("u must have shape [B, T, H, dv]")
    dv = u.shape[3]
    _dev(logp, "logp", torch.float32, (B, T, H))
    _dev(S0, "S0", torch.float32, (B, H, dv, dk))
    _dev(pos, "pos", torch.int32)
    if pos.dim() != 2 or pos.shape[0] != B:
        raise ValueError("pos must have shape [B, P]")
    P = pos.shape[1]
    _dev(queries, "queries", k.dtype)
    if queries.dim() != 5 or tuple(queries.shape[:3]) != (B, P, H) or queries.shape[4] != dk:
        raise ValueError("queries must have shape [B, P, H, Qn, dk]")
    Qn = queries.shape[3]
    if parent is not None:
        _dev(parent, "parent", torch.int32, (B, T))
    o = _opt(o, "o", torch.float32, (B, P, H, Qn, dv), k.device, stream)
    if status is not None:
        _dev(status, "status", torch.int32)
    dev = k.device
    _same_device(dev, u=u, logp=logp, S0=S0, pos=pos, queries=queries, parent=parent, o=o, status=status)
    _invoke("ldv_read_block_states", dev,
            B, T, H, dk, dv, P, Qn, code, _ptr(k), _ptr(u), _ptr(logp), _ptr(parent), _ptr(S0), _ptr(pos),
            _ptr(queries), _ptr(o), _ptr(status), _stream(stream, dev))
    return o


def _feat(feat, B, P, width, col):
    """A packed destination: a contiguous [B, P, W] or [B * P, W] tensor,
    fp32 or bf16, with columns col .. col + width - 1 to be written.
    Returns (dtype code, W)."""
    _dev(feat, "feat")
    if feat.dtype == torch.float32:
        code = LDV_F32
    elif feat.dtype == torch.bfloat16:
        code = LDV_BF16
    else:
        raise TypeError("feat must be float32 or bfloat16 (got %s)" % feat.dtype)
    if tuple(feat.shape[:-1]) not in ((B, P), (B * P,)):
        raise ValueError("feat must have shape [B, P, W] or [B * P, W] (got %s)" % (tuple(feat.shape),))
    W = feat.shape[-1]
    if col < 0 or col + width > W:
        raise ValueError("columns %d .. %d do not fit rows of %d" % (col, col + width - 1, W))
    return code, W


def gather_states_packed(pool, slot, queries, feat, col=0, status=None, stream=None):
    """The reads of gather_states written straight into packed drafter
    features: row b * P + p of ``feat`` gets o[b, p] (heads, queries, values
    in that order) at columns col .. col + H * Qn * dv - 1, as fp32 or as bf16
    (feat's dtype); every other element of feat is left as it is.  No state
    copies.  Returns feat."""
    _dev(pool, "pool", torch.float32)
    num_slots, H, dv, dk = pool.shape
    _dev(slot, "slot", torch.int32)
    B, P = slot.shape
    _dev(queries, "queries")
    code = _qkv_code(queries)
    if queries.dim() != 5 or tuple(queries.shape[:3]) != (B, P, H) or queries.shape[4] != dk:
        raise ValueError("queries must have shape [B, P, H, Qn, dk]")
    Qn = queries.shape[3]
    fcode, W = _feat(feat, B, P, H * Qn * dv, col)
    if status is not None:
        _dev(status, "status", torch.int32)
    dev = pool.device
    _same_device(dev, slot=slot, queries=queries, feat=feat, status=status)
    _invoke("ldv_gather_states_packed", dev,
            B, P, H, dk, dv, num_slots, Qn, code, _ptr(pool), _ptr(slot), _ptr(queries), _ptr(feat), W, col,
            fcode, _ptr(status), _stream(stream, dev))
    return feat


def read_block_states_packed(k, u, logp, S0, pos, queries, feat, col=0, parent=None, status=None, stream=None):
    """The reads of read_block_states written straight into packed drafter
    features, laid out as in gather_states_packed.  Returns feat."""
    _dev(k, "k")
    B, T, H, dk = k.shape
    code = _qkv_code(k)
    _dev(u, "u", torch.float32)
    if u.dim() != 4 or tuple(u.shape[:3]) != (B, T, H):
        raise ValueError("u must have shape [B, T, H, dv]")
    dv = u.shape[3]
    _dev(logp, "logp", torch.float32, (B, T, H))
    _dev(S0, "S0", torch.float32, (B, H, dv, dk))
    _dev(pos, "pos", torch.int32)
    if pos.dim() != 2 or pos.shape[0] != B:
        raise ValueError("pos must have shape [B, P]")
    P = pos.shape[1]
    _dev(queries, "queries", k.dtype)
    if queries.dim() != 5 or tuple(queries.shape[:3]) != (B, P, H) or queries.shape[4] != dk:
        raise ValueError("queries must have shape [B, P, H, Qn, dk]")
    Qn = queries.shape[3]
    if parent is not None:
        _dev(parent, "parent", torch.int32, (B, T))
    fcode, W = _feat(feat, B, P, H * Qn * dv, col)
    if status is not None:
        _dev(status, "status", torch.int32)
    dev = k.device
    _same_device(dev, u=u, logp=logp, S0=S0, pos=pos, queries=queries, parent=parent, feat=feat, status=status)
    _invoke("ldv_read_block_states_packed", dev,
            B, T, H, dk, dv, P, Qn, code, _ptr(k), _ptr(u), _ptr(logp), _ptr(parent), _ptr(S0), _ptr(pos),
            _ptr(queries), _ptr(feat), W, col, fcode, _ptr(status), _stream(stream, dev))
    return feat


def select_accepted(logits, tokens, parent=None, target=None, accepted=None, accepted_len=None,
                    bonus=None, status=None, workspace=None, split=True, stream=None):
    """Greedy accepted-node selection on the device.

    logits [B, T+1, V] bf16/fp32 (row 0: the committed position, row n+1:
    after node n); tokens [B, T] int32; parent [B, T] int32 or None (chain).
    With split=True the library may split few, long rows over several
    workgroups, through a workspace (uint8 device tensor of at least
    select_workspace_bytes(B, T, V) bytes; allocated here when not given).
    Returns (target [B, T+1], accepted [B], accepted_len [B], bonus [B]),
    all int32."""
    _dev(logits, "logits")
    if logits.dim() != 3:
        raise ValueError("logits must have shape [B, T+1, V]")
    B, T1, V = logits.shape
    T = T1 - 1
    code = _qkv_code(logits)
    _dev(tokens, "tokens", torch.int32, (B, T))
    if parent is not None:
        _dev(parent, "parent", torch.int32, (B, T))
    dev = logits.device
    target = _opt(target, "target", torch.int32, (B, T1), dev, stream)
    accepted = _opt(accepted, "accepted", torch.int32, (B,), dev, stream)
    accepted_len = _opt(accepted_len, "accepted_len", torch.int32, (B,), dev, stream)
    bonus = _opt(bonus, "bonus", torch.int32, (B,), dev, stream)
    if status is not None:
        _dev(status, "status", torch.int32)
    ws_bytes = 0
    if split:
        need = select_workspace_bytes(B, T, V)
        if workspace is None and need > 0:
            workspace = _alloc((need,), torch.uint8, dev, stream)
        if workspace is not None:
            _dev(workspace, "workspace", torch.uint8)
            ws_bytes = workspace.numel()
    else:
        workspace = None
    _same_device(dev, tokens=tokens, parent=parent, target=target, accepted=accepted,
                 accepted_len=accepted_len, bonus=bonus, status=status, workspace=workspace)
    _invoke("ldv_select_accepted", dev,
            B, T, V, code, _ptr(logits), _ptr(tokens), _ptr(parent), _ptr(target), _ptr(accepted),
            _ptr(accepted_len), _ptr(bonus), _ptr(status), _ptr(workspace), ctypes.c_size_t(ws_bytes),
            _stream(stream, dev))
    return target, accepted, accepted_len, bonus


def select_accepted_noalloc(logits, tokens, target, accepted, parent=None, accepted_len=None, bonus=None,
                            status=None, stream=None):
    """select_accepted through the entry point that allocates nothing: rows
    are split as select_accepted splits them with a workspace, the partial
    results in the library's own per-GPU array.  Every output is the
    caller's (target [B, T+1] and accepted [B] int32 required, accepted_len
    and bonus [B] int32 optional), so that the call allocates nothing; calls
    that overlap on one GPU race.  Returns (target, accepted, accepted_len,
    bonus)."""
    _dev(logits, "logits")
    if logits.dim() != 3:
        raise ValueError("logits must have shape [B, T+1, V]")
    B, T1, V = logits.shape
    T = T1 - 1
    code = _qkv_code(logits)
    _dev(tokens, "tokens", torch.int32, (B, T))
    if parent is not None:
        _dev(parent, "parent", torch.int32, (B, T))
    _dev(target, "target", torch.int32, (B, T1))
    _dev(accepted, "accepted", torch.int32, (B,))
    if accepted_len is not None:
        _dev(accepted_len, "accepted_len", torch.int32, (B,))
    if bonus is not None:
        _dev(bonus, "bonus", torch.int32, (B,))
    if status is not None:
        _dev(status, "status", torch.int32)
    dev = logits.device
    _same_device(dev, tokens=tokens, parent=parent, target=target, accepted=accepted,
                 accepted_len=accepted_len, bonus=bonus, status=status)
    _invoke("ldv_select_accepted_noalloc", dev,
            B, T, V, code, _ptr(logits), _ptr(tokens), _ptr(parent), _ptr(target), _ptr(accepted),
            _ptr(accepted_len), _ptr(bonus), _ptr(status), _stream(stream, dev))
    return target, accepted, accepted_len, bonus


def select_workspace_bytes(B: int, T: int, V: int) -> int:
    """Workspace bytes select_accepted uses for these sizes (0: none)."""
    return int(load().ldv_select_workspace_bytes(int(B), int(T), int(V)))


def version() -> int:
    return load().ldv_version()
