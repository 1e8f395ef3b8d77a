"""numpy front end of the RMM oracle (rmm_oracle.c).  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this module.  It marshals numpy arrays into the C oracle and back; every step
of the arithmetic is in rmm_oracle.c (plain fp64, single-threaded).  It imports
nothing from the GPU package.

Source of the method: "Reduced Matrix Multiplication: Input-Adaptive
Matrix-Product Reduction for LLM Inference", technical summary (gist.science),
section "Metodologia" (Mecanismo Central; Estratégia de Seleção; Escopo de
Aplicação).  The readings taken where the pages are silent (R1-R6, R9-R11) are
listed in the header of rmm_oracle.c.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librmm_oracle.so")

_lib = None

NEAR_TIE_REL = 1e-6  # band around the k-th score inside which sets may differ


def load(path=None):
    """Load (building it first if absent) the oracle library; returns the CDLL."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        from . import build as _build
        _build.build(out=p)
    lib = ctypes.CDLL(p)
    _declare(lib)
    if path is None:
        _lib = lib
    return lib


_D = ctypes.POINTER(ctypes.c_double)
_F = ctypes.POINTER(ctypes.c_float)
_I32 = ctypes.POINTER(ctypes.c_int32)
_I64 = ctypes.POINTER(ctypes.c_int64)
_I8 = ctypes.POINTER(ctypes.c_int8)
_L = ctypes.c_int64


def _declare(lib):
    lib.oracle_kk.restype = _L
    lib.oracle_kk.argtypes = [ctypes.c_double, _L]
    lib.oracle_rownorms.restype = None
    lib.oracle_rownorms.argtypes = [_D, _L, _L, _L, _D]
    lib.oracle_colnorms.restype = None
    lib.oracle_colnorms.argtypes = [_D, _L, _L, _L, _D]
    lib.oracle_scores.restype = None
    lib.oracle_scores.argtypes = [_D, _L, _L, _L, _D, _L, _D, _F]
    lib.oracle_topk.restype = ctypes.c_int
    lib.oracle_topk.argtypes = [_F, _L, _L, _I32]
    lib.oracle_reduced.restype = None
    lib.oracle_reduced.argtypes = [_D, _L, _D, _L, _L, _L, _I32, _L, _L, _L, _L, _D, _L]
    lib.oracle_reduced_entries.restype = None
    lib.oracle_reduced_entries.argtypes = [_D, _L, _D, _L, _L, _I32, _L, _L, _I64, _I64, _L, _D]
    lib.oracle_bound.restype = ctypes.c_double
    lib.oracle_bound.argtypes = [_D, _L, _I32, _L]
    lib.oracle_thresh.restype = ctypes.c_float
    lib.oracle_thresh.argtypes = [_F, _I32, _L]
    lib.oracle_near_ties.restype = _L
    lib.oracle_near_ties.argtypes = [_D, _F, _L, _I32, _L, ctypes.c_double, _I32]
    lib.oracle_pv_prefix.restype = _L
    lib.oracle_pv_prefix.argtypes = [_L, _L, _L, ctypes.c_int]
    lib.oracle_pv_scores.restype = None
    lib.oracle_pv_scores.argtypes = [_D, _L, _L, _D, _L, _L, _D, _F]
    lib.oracle_pv_block.restype = None
    lib.oracle_pv_block.argtypes = [_D, _L, _L, _D, _L, _I32, _L, _D]
    lib.oracle_pv_bound.restype = ctypes.c_double
    lib.oracle_pv_bound.argtypes = [_D, _L, _L, _D, _L, _L, _I32, _L]
    lib.oracle_quantize_q8.restype = None
    lib.oracle_quantize_q8.argtypes = [_F, _L, _L, _L, _I8, _L, _F]
    lib.oracle_dequant_q8.restype = None
    lib.oracle_dequant_q8.argtypes = [_I8, _L, _F, _L, _L, _D, _L]
    lib.oracle_rownorms_q8.restype = None
    lib.oracle_rownorms_q8.argtypes = [_I8, _L, _F, _L, _L, _D]
    lib.oracle_qk_scores.restype = None
    lib.oracle_qk_scores.argtypes = [_D, _D, _L, _L, _L, _L, ctypes.c_int, _D, _F]
    lib.oracle_attn_probs.restype = None
    lib.oracle_attn_probs.argtypes = [_D, _D, _L, _L, _L, _L, ctypes.c_int, _I32, _L, _D]


def _p(a, typ):
    return a.ctypes.data_as(typ)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


# ---------------------------------------------------------------- widening
def widen_bf16(bits):
    """bf16 bit patterns (uint16/int16 array) -> exact float64 values."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def widen_f32(x):
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- linear path
def kk(r, K, lib=None):
    """Retained count ceil(r*K) under reading R3; -1 for r outside (0, 1]."""
    lib = lib or load()
    return int(lib.oracle_kk(float(r), int(K)))


def rownorms(B, lib=None):
    lib = lib or load()
    B = _f64(B)
    K, N = B.shape
    out = np.empty(K, np.float64)
    lib.oracle_rownorms(_p(B, _D), K, N, N, _p(out, _D))
    return out


def colnorms(A, lib=None):
    lib = lib or load()
    A = _f64(A)
    rows, K = A.shape
    out = np.empty(K, np.float64)
    lib.oracle_colnorms(_p(A, _D), rows, K, K, _p(out, _D))
    return out


def scores(A, group_rows, b=None, lib=None):
    """(s64, s32), each [G, K]: per-group slice scores (readings R1, R2)."""
    lib = lib or load()
    A = _f64(A)
    M, K = A.shape
    G = -(-M // group_rows)
    s64 = np.empty((G, K), np.float64)
    s32 = np.empty((G, K), np.float32)
    bp = None
    if b is not None:
        b = _f64(b)
        bp = _p(b, _D)
    lib.oracle_scores(_p(A, _D), M, K, K, bp, group_rows, _p(s64, _D), _p(s32, _F))
    return s64, s32


def topk(s32, kk_, lib=None):
    """Kept indices (ascending) of the kk best binary32 scores, ties to the lower index."""
    lib = lib or load()
    s32 = np.ascontiguousarray(s32, dtype=np.float32)
    out = np.empty(kk_, np.int32)
    rc = lib.oracle_topk(_p(s32, _F), s32.shape[0], kk_, _p(out, _I32))
    if rc != 0:
        raise ValueError("kk out of range")
    return out


def thresh(s32_row, idx, lib=None):
    """The binary32 score of rank kk (the smallest key among the kept idx)."""
    lib = lib or load()
    s = np.ascontiguousarray(s32_row, dtype=np.float32)
    i = np.ascontiguousarray(idx, dtype=np.int32)
    return np.float32(lib.oracle_thresh(_p(s, _F), _p(i, _I32), len(i)))


def near_ties(s64_row, s32_row, idx, rel=NEAR_TIE_REL, lib=None):
    """Ascending indices whose unrounded score lies within `rel` (relative) of
    the unrounded score of the rank-kk element."""
    lib = lib or load()
    s64 = _f64(s64_row)
    s32 = np.ascontiguousarray(s32_row, dtype=np.float32)
    i = np.ascontiguousarray(idx, dtype=np.int32)
    out = np.empty(len(s64), np.int32)
    n = lib.oracle_near_ties(_p(s64, _D), _p(s32, _F), len(s64), _p(i, _I32), len(i), float(rel), _p(out, _I32))
    return out[:n].copy()


def select(A, r, group_rows, b=None, lib=None):
    """The whole selection step for a linear layer.

    Returns dict(kk, idx [G, kk] ascending, s64, s32, thresh [G] (binary32 k-th
    score), bound [G] (sum of dropped unrounded scores), near [list of arrays]:
    each group's near-tie band, logged by the GPU tests).
    """
    lib = lib or load()
    A = _f64(A)
    M, K = A.shape
    kk_ = kk(r, K, lib)
    if kk_ < 0:
        raise ValueError("r outside (0, 1]")
    s64, s32 = scores(A, group_rows, b, lib)
    G = s64.shape[0]
    idx = np.empty((G, kk_), np.int32)
    th = np.empty(G, np.float32)
    bound = np.empty(G, np.float64)
    near = []
    for g in range(G):
        idx[g] = topk(s32[g], kk_, lib)
        th[g] = thresh(s32[g], idx[g], lib)
        row = np.ascontiguousarray(s64[g])
        bound[g] = lib.oracle_bound(_p(row, _D), K, _p(idx[g], _I32), kk_)
        near.append(near_ties(s64[g], s32[g], idx[g], lib=lib))
    return dict(kk=kk_, idx=idx, s64=s64, s32=s32, thresh=th, bound=bound, near=near)


def reduced(A, B, idx, kk_, group_rows, m0=0, m1=None, lib=None):
    """Y[m0:m1] of the reduced product; idx is [G, >=kk] (row g = group g)."""
    lib = lib or load()
    A = _f64(A)
    B = _f64(B)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    M, K = A.shape
    N = B.shape[1]
    m1 = M if m1 is None else m1
    Y = np.empty((m1 - m0, N), np.float64)
    lib.oracle_reduced(_p(A, _D), K, _p(B, _D), N, N, group_rows, _p(idx, _I32), idx.shape[1],
                       kk_, m0, m1, _p(Y, _D), N)
    return Y


def reduced_entries(A, B, idx, kk_, group_rows, ms, ns, lib=None):
    lib = lib or load()
    A = _f64(A)
    B = _f64(B)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(len(ms), np.float64)
    lib.oracle_reduced_entries(_p(A, _D), A.shape[1], _p(B, _D), B.shape[1], group_rows,
                               _p(idx, _I32), idx.shape[1], kk_, _p(ms, _I64), _p(ns, _I64),
                               len(ms), _p(out, _D))
    return out


def dense(A, B, lib=None):
    """The unreduced product: the reduced product with every index kept."""
    A = _f64(A)
    K = A.shape[1]
    idx = np.arange(K, dtype=np.int32)[None, :]
    return reduced(A, B, idx, K, A.shape[0], lib=lib)


def bound(s64_row, idx, lib=None):
    lib = lib or load()
    s = _f64(s64_row)
    i = np.ascontiguousarray(idx, dtype=np.int32)
    return float(lib.oracle_bound(_p(s, _D), len(s), _p(i, _I32), len(i)))


# ---------------------------------------------------------------- P.V path
def pv_prefix(L, qblock, g, causal=True, lib=None):
    lib = lib or load()
    return int(lib.oracle_pv_prefix(L, qblock, g, int(bool(causal))))


def pv_block_inputs(Pt, q0, nq, Kg):
    """Slice of key-major P (Pt[k, q] = P[q, k]) seen by one query block, as float64."""
    return _f64(Pt[:Kg, q0:q0 + nq])


def pv_scores(Ptb, V, lib=None):
    """(s64, s32) over the block's candidate keys; Ptb is [Kg, nq] float64."""
    lib = lib or load()
    Ptb = _f64(Ptb)
    V = _f64(V)
    Kg, nq = Ptb.shape
    D = V.shape[1]
    s64 = np.empty(Kg, np.float64)
    s32 = np.empty(Kg, np.float32)
    lib.oracle_pv_scores(_p(Ptb, _D), nq, nq, _p(V, _D), D, Kg, _p(s64, _D), _p(s32, _F))
    return s64, s32


def pv_block(Ptb, V, idx, lib=None):
    """O [nq, D] of one query block over the kept keys idx."""
    lib = lib or load()
    Ptb = _f64(Ptb)
    V = _f64(V)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    Kg, nq = Ptb.shape
    D = V.shape[1]
    O = np.empty((nq, D), np.float64)
    lib.oracle_pv_block(_p(Ptb, _D), nq, nq, _p(V, _D), D, _p(idx, _I32), len(idx), _p(O, _D))
    return O


def pv_bound(Ptb, V, idx, lib=None):
    lib = lib or load()
    Ptb = _f64(Ptb)
    V = _f64(V)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    Kg, nq = Ptb.shape
    return float(lib.oracle_pv_bound(_p(Ptb, _D), nq, nq, _p(V, _D), V.shape[1], Kg,
                                     _p(idx, _I32), len(idx)))


def pv_select_block(Pt, V, L, qblock, g, r, causal=True, lib=None):
    """Selection for one (head, query block): dict(Kg, kk, idx, s64, s32, near)."""
    lib = lib or load()
    q0 = g * qblock
    nq = min(qblock, L - q0)
    Kg = pv_prefix(L, qblock, g, causal, lib)
    Ptb = pv_block_inputs(Pt, q0, nq, Kg)
    Vg = _f64(V[:Kg])
    s64, s32 = pv_scores(Ptb, Vg, lib)
    kk_ = kk(r, Kg, lib)
    idx = topk(s32, kk_, lib)
    return dict(Kg=Kg, kk=kk_, idx=idx, s64=s64, s32=s32, Ptb=Ptb, V=Vg,
                near=near_ties(s64, s32, idx, lib=lib))


# ---------------------------------------------------------------- QK^T and the probabilities
def qk_scores(Q, K, q0, nq, Kg, use_k=True, lib=None):
    """(s64, s32) of the D features for queries q0 .. q0+nq-1 of one head
    (Q, K: [L, D]) with candidate keys k < Kg, reading R10."""
    lib = lib or load()
    Q = _f64(Q)
    K = _f64(K)
    D = Q.shape[1]
    s64 = np.empty(D, np.float64)
    s32 = np.empty(D, np.float32)
    lib.oracle_qk_scores(_p(Q, _D), _p(K, _D), D, q0, nq, Kg, int(bool(use_k)), _p(s64, _D), _p(s32, _F))
    return s64, s32


def qk_select_block(Q, K, qblock, g, r, causal=True, use_k=True, lib=None):
    """Kept features of one (head, query block): dict(Kg, kk, idx, s64, s32, near)."""
    lib = lib or load()
    L, D = Q.shape
    q0 = g * qblock
    nq = min(qblock, L - q0)
    Kg = pv_prefix(L, qblock, g, causal, lib)
    s64, s32 = qk_scores(Q, K, q0, nq, Kg, use_k, lib)
    kk_ = kk(r, D, lib)
    idx = topk(s32, kk_, lib)
    return dict(Kg=Kg, kk=kk_, idx=idx, s64=s64, s32=s32, near=near_ties(s64, s32, idx, lib=lib))


def attn_probs(Q, K, q0, nq, causal=True, idx=None, lib=None):
    """P [nq, L] float64: rows q0 .. q0+nq-1 of one head's attention
    probabilities over the kept features idx (None: all), reading R11."""
    lib = lib or load()
    Q = _f64(Q)
    K = _f64(K)
    L, D = Q.shape
    P = np.empty((nq, L), np.float64)
    if idx is None:
        lib.oracle_attn_probs(_p(Q, _D), _p(K, _D), L, D, q0, nq, int(bool(causal)), None, D, _p(P, _D))
    else:
        i = np.ascontiguousarray(idx, dtype=np.int32)
        lib.oracle_attn_probs(_p(Q, _D), _p(K, _D), L, D, q0, nq, int(bool(causal)), _p(i, _I32), len(i),
                              _p(P, _D))
    return P


# ---------------------------------------------------------------- int8 weights
def quantize_q8(B, lib=None):
    """(q int8 [K, N], scale float32 [N]) of a weight given as binary32 values
    (bf16 weights widened exactly), reading R9."""
    lib = lib or load()
    B = np.ascontiguousarray(B, dtype=np.float32)
    K, N = B.shape
    q = np.empty((K, N), np.int8)
    s = np.empty(N, np.float32)
    lib.oracle_quantize_q8(_p(B, _F), K, N, N, _p(q, _I8), N, _p(s, _F))
    return q, s


def dequant_q8(q, scale, lib=None):
    """The dequantised weight scale[n] * q[k, n] as float64 (exact)."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    K, N = q.shape
    Bd = np.empty((K, N), np.float64)
    lib.oracle_dequant_q8(_p(q, _I8), N, _p(s, _F), K, N, _p(Bd, _D), N)
    return Bd


def rownorms_q8(q, scale, lib=None):
    """Row norms of the dequantised weight, float64 [K]."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    K, N = q.shape
    b = np.empty(K, np.float64)
    lib.oracle_rownorms_q8(_p(q, _I8), N, _p(s, _F), K, N, _p(b, _D))
    return b


__all__ = [
    "load", "widen_bf16", "widen_f32", "kk", "rownorms", "colnorms", "scores", "topk", "select",
    "reduced", "reduced_entries", "dense", "bound", "pv_prefix", "pv_block_inputs", "pv_scores",
    "pv_block", "pv_bound", "pv_select_block", "near_ties", "thresh", "NEAR_TIE_REL",
    "quantize_q8", "dequant_q8", "rownorms_q8", "qk_scores", "qk_select_block", "attn_probs",
]
