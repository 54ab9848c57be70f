"""ctypes wrapper of the plain C reference (oracle/dsa_ref.c).

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: the tests, the smoke check and the
benchmark's CPU baseline use it; the GPU library never does. The shared object is compiled
with gcc (OpenMP when available) next to the source, on first use or when the source changed.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "dsa_ref.c")
LIB = os.path.join(_HERE, "libdsa_ref.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile dsa_ref.c into libdsa_ref.so (gcc -O2, with -fopenmp when gcc has it)."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    base = ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", tmp, SRC, "-lm"]
    res = subprocess.run(base[:1] + ["-fopenmp"] + base[1:], capture_output=True, text=True)
    if res.returncode != 0:
        res = subprocess.run(base, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed on {SRC}:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        l = C.CDLL(build())
        P, I, D = C.c_void_p, C.c_int, C.c_double
        l.dsa_ref_index_scores.argtypes = [P, P, I, P, I, I, P]
        l.dsa_ref_select_topk.argtypes = [P, I, I, P]
        l.dsa_ref_sparse_mla.argtypes = [P, I, P, I, D, D, P, P]
        for f in (l.dsa_ref_index_scores, l.dsa_ref_select_topk, l.dsa_ref_sparse_mla):
            f.restype = None
        _lib = l
    return _lib


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def index_scores(q_codes, w, key_rows, p: int, L_max: int) -> np.ndarray:
    """One query: q_codes [Hi, 128] uint8, w [Hi], key_rows [>= p+1, 128] uint8 (token order)."""
    q = np.ascontiguousarray(q_codes, dtype=np.uint8)
    ww = np.ascontiguousarray(w, dtype=np.float32)
    k = np.ascontiguousarray(key_rows, dtype=np.uint8)
    assert k.shape[0] >= p + 1 and k.shape[1] == 128 and q.shape[1] == 128
    out = np.empty(L_max, dtype=np.float64)
    lib().dsa_ref_index_scores(_p(q), _p(ww), q.shape[0], _p(k), int(p), int(L_max), _p(out))
    return out


def select_topk(scores32, p: int, k: int) -> np.ndarray:
    s = np.ascontiguousarray(scores32, dtype=np.float32)
    assert s.shape[0] >= p + 1
    out = np.empty(k, dtype=np.int32)
    lib().dsa_ref_select_topk(_p(s), int(p), int(k), _p(out))
    return out


def sparse_mla(q_bits, rows, scale: float, latent_scale: float = 0.0):
    """q_bits [H, 576] uint16; rows [m, 576] uint16 (bf16 bits) or uint8 (E4M3 codes, then
    values are latent_scale x code). Returns (o [H, 512], lse [H]) in float64."""
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    r = np.ascontiguousarray(rows)
    e4 = r.dtype == np.uint8
    if r.shape[0] == 0:
        r = np.zeros((1, 576), dtype=r.dtype)
        m = 0
    else:
        m = r.shape[0]
    H = q.shape[0]
    o = np.empty((H, 512), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    lib().dsa_ref_sparse_mla(_p(q), H, _p(r), m, float(scale), float(latent_scale) if e4 else 0.0, _p(o), _p(lse))
    return o, lse
