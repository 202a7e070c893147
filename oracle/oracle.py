"""ctypes front of the plain C oracle (sla_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.  It shares nothing
with the GPU library; inputs are float32 numpy arrays, results fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sla_oracle.c")
LIB = os.path.join(HERE, "libsla_oracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math, no contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("SLA_ORACLE_LIB")   # a test may point at a planted-mistake build
        if path is None:
            path = build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_long
        L.sla_oracle_threads.restype = ctypes.c_int
        L.sla_oracle_counts.argtypes = [I64, ctypes.c_double, ctypes.c_double,
                                        ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
        L.sla_oracle_counts.restype = ctypes.c_int
        L.sla_oracle_pool.argtypes = [P, I64, I64, I64, I64, P]
        L.sla_oracle_classify.argtypes = [P, P, I64, I64, I64, ctypes.c_int, ctypes.c_int,
                                          P, P, P, P, P]
        L.sla_oracle_phi.argtypes = [P, I64, I64, P]
        L.sla_oracle_forward_rows.argtypes = [P, P, P, P, I64, I64, I64, I64, P, P, I64, P, P, P]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def threads() -> int:
    return lib().sla_oracle_threads()


def counts(Nb: int, rho_c: float, rho_n: float):
    kc, kn = ctypes.c_int(), ctypes.c_int()
    if lib().sla_oracle_counts(Nb, rho_c, rho_n, ctypes.byref(kc), ctypes.byref(kn)) != 0:
        raise ValueError("fractions out of range")
    return kc.value, kn.value


def pool(x: np.ndarray, blk: int = 64) -> np.ndarray:
    """x [..., N, d] -> block means [..., Nb, d] float32."""
    x = _f32(x)
    *lead, N, d = x.shape
    BH = int(np.prod(lead)) if lead else 1
    Nb = -(-N // blk)
    out = np.empty((*lead, Nb, d), np.float32)
    lib().sla_oracle_pool(_ptr(x), BH, N, d, blk, _ptr(out))
    return out


def classify(qp: np.ndarray, kp: np.ndarray, rho_c: float, rho_n: float,
             want_scores: bool = False, want_pc: bool = False) -> dict:
    """Pooled Q, K [..., Nb, d] -> mask, critical and negligible lists."""
    qp, kp = _f32(qp), _f32(kp)
    *lead, Nb, d = qp.shape
    BH = int(np.prod(lead)) if lead else 1
    kc, kn = counts(Nb, rho_c, rho_n)
    mask = np.empty((*lead, Nb, Nb), np.int8)
    crit = np.empty((*lead, Nb, kc), np.int32)
    negl = np.empty((*lead, Nb, kn), np.int32)
    scores = np.empty((*lead, Nb, Nb), np.float64) if want_scores else None
    pc = np.empty((*lead, Nb, Nb), np.float64) if want_pc else None
    lib().sla_oracle_classify(_ptr(qp), _ptr(kp), BH, Nb, d, kc, kn, _ptr(mask), _ptr(crit),
                              _ptr(negl), _ptr(scores), _ptr(pc))
    out = dict(mask=mask, crit=crit, negl=negl, k_c=kc, k_n=kn)
    if want_scores:
        out["scores"] = scores
    if want_pc:
        out["pc"] = pc
    return out


def phi(x: np.ndarray) -> np.ndarray:
    x = _f32(x)
    *lead, d = x.shape
    n = int(np.prod(lead)) if lead else 1
    out = np.empty(x.shape, np.float64)
    lib().sla_oracle_phi(_ptr(x), n, d, _ptr(out))
    return out


def forward(q, k, v, w, blk: int = 64, rho_c: float = 0.05, rho_n: float = 0.10,
            rows: Optional[np.ndarray] = None, cls: Optional[dict] = None) -> dict:
    """The whole forward pass.

    q, k, v [B, H, N, d]; w [d, d].  rows: optional [n, 2] int array of
    (b*H + h, query block) pairs (sorted) to evaluate; default every block.
    Returns dict with 'o', 'o_s', 'o_l' of shape [n, blk, d] (fp64) plus the
    classification ('mask', 'crit', 'negl', 'k_c', 'k_n') and pooled 'qp', 'kp'.
    """
    q, k, v, w = _f32(q), _f32(k), _f32(v), _f32(w)
    B, H, N, d = q.shape
    Nb = -(-N // blk)
    qp = pool(q, blk)
    kp = pool(k, blk)
    if cls is None:
        cls = classify(qp, kp, rho_c, rho_n)
    if rows is None:
        rows = np.array([(bh, i) for bh in range(B * H) for i in range(Nb)], np.int32).reshape(-1, 2)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    n = rows.shape[0]
    o = np.empty((n, blk, d), np.float64)
    o_s = np.empty_like(o)
    o_l = np.empty_like(o)
    mask = np.ascontiguousarray(cls["mask"], dtype=np.int8)
    lib().sla_oracle_forward_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(w), B * H, N, d, blk,
                                  _ptr(mask), _ptr(rows), n, _ptr(o), _ptr(o_s), _ptr(o_l))
    out = dict(cls)
    out.update(o=o, o_s=o_s, o_l=o_l, qp=qp, kp=kp, rows=rows)
    return out


def rows_to_dense(res: dict, B: int, H: int, N: int, key: str = "o") -> np.ndarray:
    """Scatter per-row results of a full evaluation back to [B, H, N, d]."""
    o = res[key]
    n, blk, d = o.shape
    Nb = -(-N // blk)
    dense = np.zeros((B * H, Nb * blk, d), np.float64)
    for r, (bh, i) in enumerate(res["rows"]):
        dense[bh, i * blk:(i + 1) * blk] = o[r]
    return dense[:, :N].reshape(B, H, N, d)
