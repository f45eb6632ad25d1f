"""Python access to the CPU oracle (``ddtree_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers. The GPU package never
imports this module, and this module imports nothing from the GPU package.

Arrays are numpy (or CPU torch tensors, converted here). bfloat16 data is
handed to C as its raw 16-bit patterns with ``dtype=BF16``; float32 as is.
The C side documents each step and the page passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

BF16 = 0
F32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ddtree_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        L.oracle_exp_fixed.restype = ctypes.c_uint64
        L.oracle_exp_fixed.argtypes = [ctypes.c_float]
        L.oracle_log64.restype = ctypes.c_double
        L.oracle_log64.argtypes = [ctypes.c_double]
        L.oracle_row_topk.restype = ctypes.c_int
        L.oracle_tree.restype = ctypes.c_int
        for name in ("oracle_mask", "oracle_build", "oracle_attn_rows",
                     "oracle_argmax_rows", "oracle_walk", "oracle_accept",
                     "oracle_philox4x32_10", "oracle_accept_sample", "oracle_commit_kv"):
            getattr(L, name).restype = None
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_get_threads.restype = ctypes.c_int
        L.oracle_get_threads.argtypes = []
        L.oracle_sample_row.restype = ctypes.c_int
        L.oracle_sample_row.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int]
        L.oracle_accept_sample.argtypes = [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 3 + \
            [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64] + [ctypes.c_void_p] * 5
        L.oracle_commit_kv.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t] + \
            [ctypes.c_void_p] * 5 + [ctypes.c_int] * 3 + [ctypes.c_int64] + [ctypes.c_void_p] * 2
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Threads for the batch-level calls (1 by default; results do not
    depend on it)."""
    lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(lib().oracle_get_threads())


def host_cores() -> int:
    """CPU cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


class threads:
    """Context manager: run the enclosed oracle calls on n threads."""

    def __init__(self, n: int):
        self.n = int(n)

    def __enter__(self):
        self.prev = get_threads()
        set_threads(self.n)
        return self

    def __exit__(self, *exc):
        set_threads(self.prev)
        return False


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    return ctypes.c_void_p(a.ctypes.data)


def as_raw(x):
    """Return (contiguous numpy array, dtype code) for float32 or bfloat16 data."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            raise TypeError("oracle takes float32 or bfloat16 data, got %s" % x.dtype)
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("oracle takes float32 or raw bfloat16 (uint16) data, got %s" % x.dtype)


def _i32(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def exp_fixed(d: float) -> int:
    return int(lib().oracle_exp_fixed(ctypes.c_float(d)))


def log64(s: float) -> float:
    return float(lib().oracle_log64(ctypes.c_double(s)))


def row_topk(row, K: int, tau: float):
    """One drafter row -> dict(tok, lp, m, S, lse, flags)."""
    raw, dt = as_raw(row)
    V = raw.shape[-1]
    tok = np.zeros(K, np.int32)
    lp = np.zeros(K, np.float32)
    m = ctypes.c_float()
    S = ctypes.c_uint64()
    lse = ctypes.c_float()
    flags = lib().oracle_row_topk(_p(raw), dt, V, K, ctypes.c_float(tau), _p(tok), _p(lp),
                                  ctypes.byref(m), ctypes.byref(S), ctypes.byref(lse))
    return dict(tok=tok, lp=lp, m=m.value, S=S.value, lse=lse.value, flags=flags)


def tree(topk_tok, topk_lp, L: int, K: int, N: int, root_token: int):
    """Best-first tree of one request from its [L, K] candidate tables."""
    tt = _i32(topk_tok).reshape(L, K)
    tl = np.ascontiguousarray(np.asarray(topk_lp, dtype=np.float32)).reshape(L, K)
    T = N + 1
    tokens = np.zeros(T, np.int32)
    parents = np.zeros(T, np.int32)
    depths = np.zeros(T, np.int32)
    scores = np.zeros(T, np.float32)
    n = lib().oracle_tree(_p(tt), _p(tl), L, K, N, ctypes.c_int32(root_token), _p(tokens),
                          _p(parents), _p(depths), _p(scores))
    return dict(tokens=tokens, parents=parents, depths=depths, scores=scores, num_nodes=int(n))


def mask(parents, num_nodes: int, T: int):
    par = _i32(parents)
    W = (T + 63) // 64
    out = np.zeros((T, W), np.uint64)
    lib().oracle_mask(_p(par), int(num_nodes), T, _p(out))
    return out


def build_tree(logits, root_tokens, K: int, N: int, tau: float, want_mask: bool = True):
    """Steps 1-3 for logits [batch, L, V] -> dict of arrays."""
    raw, dt = as_raw(logits)
    B, L, V = raw.shape
    roots = _i32(root_tokens).reshape(B)
    T = N + 1
    W = (T + 63) // 64
    out = dict(
        tokens=np.zeros((B, T), np.int32), parents=np.zeros((B, T), np.int32),
        depths=np.zeros((B, T), np.int32), scores=np.zeros((B, T), np.float32),
        num_nodes=np.zeros(B, np.int32),
        mask=np.zeros((B, T, W), np.uint64) if want_mask else None,
        topk_tok=np.zeros((B, L, K), np.int32), topk_lp=np.zeros((B, L, K), np.float32),
        status=np.zeros(B, np.int32), row_m=np.zeros((B, L), np.float32),
        row_S=np.zeros((B, L), np.uint64), row_lse=np.zeros((B, L), np.float32))
    lib().oracle_build(_p(raw), dt, _p(roots), B, L, V, K, N, ctypes.c_float(tau),
                       _p(out["tokens"]), _p(out["parents"]), _p(out["depths"]),
                       _p(out["scores"]), _p(out["num_nodes"]), _p(out["mask"]),
                       _p(out["topk_tok"]), _p(out["topk_lp"]), _p(out["status"]),
                       _p(out["row_m"]), _p(out["row_S"]), _p(out["row_lse"]))
    return out


def attn_rows(q, k, v, kv_offsets, prefix_lens, num_nodes, mask_words, T: int, Hq: int,
              Hkv: int, D: int, scale: float, sel):
    """fp64 tree attention for the (b, i, h) triples in sel -> [len(sel), D].
    The caches' row count is k's first dimension."""
    qr, dq = as_raw(q)
    kr, dk = as_raw(k)
    vr, dv = as_raw(v)
    assert dq == dk == dv, "q, k, v must share a dtype"
    offs = np.ascontiguousarray(np.asarray(kv_offsets, dtype=np.int64))
    pl = _i32(prefix_lens)
    nn = _i32(num_nodes)
    mw = np.ascontiguousarray(np.asarray(mask_words, dtype=np.uint64))
    s = _i32(sel).reshape(-1, 3)
    out = np.zeros((s.shape[0], D), np.float64)
    lib().oracle_attn_rows(_p(qr), _p(kr), _p(vr), dq, _p(offs), _p(pl), _p(nn), _p(mw), T, Hq,
                           Hkv, D, ctypes.c_int64(kr.shape[0]), ctypes.c_double(scale), _p(s),
                           s.shape[0], _p(out))
    return out


def argmax_rows(logits):
    raw, dt = as_raw(logits)
    V = raw.shape[-1]
    rows = raw.size // V
    out = np.zeros(rows, np.int32)
    lib().oracle_argmax_rows(_p(raw), dt, ctypes.c_int64(rows), V, _p(out))
    return out.reshape(raw.shape[:-1])


def walk(tokens, parents, num_nodes: int, tgt, L: int):
    tk = _i32(tokens)
    pa = _i32(parents)
    tg = _i32(tgt)
    acc = np.zeros(L, np.int32)
    accn = np.zeros(L, np.int32)
    alen = ctypes.c_int32()
    bonus = ctypes.c_int32()
    lib().oracle_walk(_p(tk), _p(pa), int(num_nodes), _p(tg), L, _p(acc), _p(accn),
                      ctypes.byref(alen), ctypes.byref(bonus))
    return dict(accepted=acc, accepted_nodes=accn, accept_len=alen.value, bonus=bonus.value)


def accept(target_logits, target_ids, tokens, parents, num_nodes, L: int):
    """Steps 5a+5b for a batch. Give target_logits [batch, T, V] or target_ids [batch, T]."""
    tk = _i32(tokens)
    B, T = tk.shape
    pa = _i32(parents)
    nn = _i32(num_nodes)
    if target_logits is not None:
        raw, dt = as_raw(target_logits)
        V = raw.shape[-1]
        ids = None
    else:
        raw, dt, V = None, F32, 1
        ids = _i32(target_ids).reshape(B, T)
    out = dict(accepted=np.zeros((B, L), np.int32), accepted_nodes=np.zeros((B, L), np.int32),
               accept_len=np.zeros(B, np.int32), bonus=np.zeros(B, np.int32),
               target_argmax=np.zeros((B, T), np.int32))
    lib().oracle_accept(_p(raw), dt, _p(ids), _p(tk), _p(pa), _p(nn), B, T, V, L,
                        _p(out["accepted"]), _p(out["accepted_nodes"]), _p(out["accept_len"]),
                        _p(out["bonus"]), _p(out["target_argmax"]))
    return out


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds: four 32-bit counter words, two key words."""
    c = np.asarray(counter, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def sample_row(row, tau: float, seed: int, offset: int, b: int = 0, i: int = 0) -> int:
    """The sampled target token of one logit row (temperature tau > 0)."""
    raw, dt = as_raw(row)
    raw = np.ascontiguousarray(raw.reshape(-1))
    return int(lib().oracle_sample_row(_p(raw), dt, raw.size, float(tau), int(seed), int(offset),
                                       int(b), int(i)))


def accept_sample(target_logits, tokens, parents, num_nodes, L: int, tau: float, seed: int,
                  offset: int):
    """Acceptance at target temperature tau > 0: sampled tokens, then the walk."""
    tk = _i32(tokens)
    B, T = tk.shape
    pa = _i32(parents)
    nn = _i32(num_nodes)
    raw, dt = as_raw(target_logits)
    V = raw.shape[-1]
    out = dict(accepted=np.zeros((B, L), np.int32), accepted_nodes=np.zeros((B, L), np.int32),
               accept_len=np.zeros(B, np.int32), bonus=np.zeros(B, np.int32),
               target_tokens=np.zeros((B, T), np.int32))
    lib().oracle_accept_sample(_p(raw), dt, _p(tk), _p(pa), _p(nn), B, T, V, L, float(tau),
                               int(seed), int(offset), _p(out["accepted"]),
                               _p(out["accepted_nodes"]), _p(out["accept_len"]), _p(out["bonus"]),
                               _p(out["target_tokens"]))
    return out


def commit_kv(k_cache, v_cache, kv_offsets, prefix_lens, accept_len, accepted_nodes, bonus,
              T: int):
    """KV compaction of the accepted path and the bonus hand-off, on copies of
    the caches ([rows, Hkv, D], float32 or bfloat16). Returns the compacted
    caches (raw arrays of the same dtype code as the inputs), the new prefix
    lengths and the next roots."""
    kr, dt = as_raw(k_cache)
    vr, dt2 = as_raw(v_cache)
    assert dt == dt2 and kr.shape == vr.shape
    kr, vr = kr.copy(), vr.copy()
    rows = kr.shape[0]
    row_bytes = kr[0].nbytes if rows else 0
    offs = np.ascontiguousarray(np.asarray(
        kv_offsets.detach().cpu().numpy() if hasattr(kv_offsets, "detach") else kv_offsets,
        dtype=np.int64))
    P = _i32(prefix_lens)
    n = _i32(accept_len)
    a = _i32(accepted_nodes)
    bo = _i32(bonus)
    B, L = a.shape
    newp = np.zeros(B, np.int32)
    roots = np.zeros(B, np.int32)
    lib().oracle_commit_kv(_p(kr), _p(vr), row_bytes, _p(offs), _p(P), _p(n), _p(a), _p(bo), B,
                           L, int(T), rows, _p(newp), _p(roots))
    return dict(k=kr, v=vr, dtype=dt, new_prefix_lens=newp, next_roots=roots)
