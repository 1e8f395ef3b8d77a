"""Pins of the oracle: checks against things other than the oracle itself.

Each function takes the oracle's ctypes library (`lib`) so the same battery can
run against the real oracle (tests/test_oracle_pins.py) and against copies with
a planted mistake (tests/test_oracle_mutants.py), which must fail at least one
pin.  Every check compares with one of:
  - a library routine (numpy norms, stable argsort, fancy-indexed matmul),
  - exact rational arithmetic (fractions.Fraction),
  - brute force over all subsets on tiny inputs,
  - a closed form or an invariant of the mathematics,
  - the hand-worked fixtures under tests/golden/.

Method source: "Reduced Matrix Multiplication: Input-Adaptive Matrix-Product
Reduction for LLM Inference", technical summary (gist.science), section
"Metodologia" -- Mecanismo Central (the reduced product), Estratégia de Seleção
(column-norm score, top ceil(rho d)), Escopo de Aplicação (XW, QK^T, PV).
"""
import ast
import itertools
import math
import os
from fractions import Fraction

import numpy as np

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse `key = python-literal` lines of a golden fixture (# starts a comment)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        text = "\n".join(line.split("#", 1)[0] for line in f)
    for stmt in ast.parse(text).body:
        out[stmt.targets[0].id] = ast.literal_eval(stmt.value)
    return out


def _rng(seed):
    return np.random.default_rng(seed)


def _ties_matrix(rng, M, K, N):
    """A, B with exactly repeated columns/rows, zero columns and a ragged spread."""
    A = rng.standard_normal((M, K))
    A[:, 3] = A[:, 1]          # equal score to column 1
    A[:, 5] = 0.0              # zero column: score 0
    A[:, 6] = 0.0
    A *= rng.lognormal(0, 1, K)[None, :]
    A[:, 3] = A[:, 1]
    B = rng.standard_normal((K, N))
    B[3] = B[1]
    return A, B


# ------------------------------------------------------------------ retained count
def pin_kk_exact_rational(lib):
    """kk(r, K) == ceil(Fraction(decimal r) * K), clamped to >= 1, on a grid."""
    for num in range(1, 1001):
        r_str = f"{num / 1000:.3f}"
        for K in (1, 7, 64, 100, 128, 256, 1000, 4096, 14336, 16384):
            want = max(1, math.ceil(Fraction(r_str) * K))
            got = O.kk(float(r_str), K, lib)
            assert got == want, (r_str, K, got, want)
    for r_str in ("0.07", "0.29", "0.57", "0.33", "0.1", "0.0001", "0.9999"):
        for K in (3, 10, 100, 333, 1000, 8191):
            want = max(1, math.ceil(Fraction(r_str) * K))
            assert O.kk(float(r_str), K, lib) == want, (r_str, K)


def pin_kk_golden(lib):
    g = read_golden("kk_table.txt")
    for r, K, want in g["rows"]:
        assert O.kk(r, K, lib) == want, (r, K)
    for r, K in g["invalid"]:
        assert O.kk(float(r), K, lib) == -1, (r, K)


# ------------------------------------------------------------------ scores
def pin_norms_numpy(lib):
    rng = _rng(1)
    B = rng.standard_normal((37, 53)) * rng.lognormal(0, 2, 37)[:, None]
    B[4] = 0.0
    want = np.linalg.norm(B, axis=1)
    got = O.rownorms(B, lib)
    assert np.allclose(got, want, rtol=1e-14, atol=0), np.max(np.abs(got - want) / np.maximum(want, 1e-300))
    A = rng.standard_normal((29, 41))
    A[:, 7] = 0.0
    want = np.linalg.norm(A, axis=0)
    got = O.colnorms(A, lib)
    assert np.allclose(got, want, rtol=1e-14, atol=0)


def pin_scores_numpy(lib):
    """Per-group product scores == numpy column norms x row norms, ragged last group."""
    rng = _rng(2)
    M, K, N, gr = 45, 33, 17, 16          # groups of 16, 16, 13 rows
    A, B = _ties_matrix(rng, M, K, N)
    b = np.linalg.norm(B, axis=1)
    s64, s32 = O.scores(A, gr, b, lib)
    assert s64.shape == (3, K)
    for g in range(3):
        want = np.linalg.norm(A[g * gr:(g + 1) * gr], axis=0) * b
        assert np.allclose(s64[g], want, rtol=1e-14, atol=0), g
    assert np.array_equal(s32, s64.astype(np.float32))
    # activation-only rule of the pages: no B norms
    s64a, _ = O.scores(A, gr, None, lib)
    for g in range(3):
        want = np.linalg.norm(A[g * gr:(g + 1) * gr], axis=0)
        assert np.allclose(s64a[g], want, rtol=1e-14, atol=0)


# ------------------------------------------------------------------ selection
def _argsort_topk(s32, kk):
    order = np.argsort(-s32.astype(np.float64), kind="stable")   # ties keep index order
    return np.sort(order[:kk]).astype(np.int32)


def pin_topk_argsort(lib):
    rng = _rng(3)
    for K in (1, 2, 9, 64, 257, 1000):
        for trial in range(3):
            s = rng.lognormal(0, 1, K).astype(np.float32)
            if K > 4:
                s[rng.integers(0, K, K // 3)] = s[0]           # many exact ties
                s[rng.integers(0, K, K // 5)] = 0.0            # ties at zero
            for kk in sorted({1, max(1, K // 3), max(1, K // 2), K}):
                got = O.topk(s, kk, lib)
                assert np.array_equal(got, _argsort_topk(s, kk)), (K, kk, trial)


def pin_topk_invariants(lib):
    rng = _rng(4)
    s = np.repeat(rng.lognormal(0, 1, 40).astype(np.float32), 3)
    rng.shuffle(s)
    K = len(s)
    for kk in (1, 17, 60, 119, 120):
        idx = O.topk(s, kk, lib)
        assert len(idx) == kk and np.all(np.diff(idx) > 0)
        kept = np.zeros(K, bool)
        kept[idx] = True
        if kk < K:
            assert s[kept].min() >= s[~kept].max()
            t = s[kept].min()
            eq_kept = np.nonzero(kept & (s == t))[0]
            eq_drop = np.nonzero(~kept & (s == t))[0]
            if len(eq_drop):
                assert eq_kept.max() < eq_drop.min()


def pin_topk_bruteforce(lib):
    """For K <= 11: the kept set minimises the dropped score sum and is the
    lexicographically smallest such set (i.e. ties go to the lower index)."""
    rng = _rng(5)
    for K in (3, 6, 9, 11):
        for trial in range(4):
            s = rng.integers(0, 4, K).astype(np.float32)    # small integers: many ties
            for kk in range(1, K + 1):
                best = None
                for sub in itertools.combinations(range(K), kk):
                    dropped = sum(float(s[k]) for k in range(K) if k not in sub)
                    key = (dropped, sub)
                    if best is None or key < best:
                        best = key
                got = tuple(int(i) for i in O.topk(s, kk, lib))
                assert got == best[1], (K, kk, s, got, best)


def pin_select_nesting(lib):
    """I(r1) is a subset of I(r2) for r1 <= r2, and the bound does not grow."""
    rng = _rng(6)
    A, B = _ties_matrix(rng, 40, 50, 8)
    b = np.linalg.norm(B, axis=1)
    prev = None
    for r in (0.1, 0.25, 0.5, 0.7, 0.9, 1.0):
        sel = O.select(A, r, 16, b, lib)
        if prev is not None:
            for g in range(sel["idx"].shape[0]):
                assert set(prev["idx"][g]).issubset(set(sel["idx"][g])), (r, g)
                assert sel["bound"][g] <= prev["bound"][g] * (1 + 1e-12) + 1e-300
        prev = sel
    assert np.all(prev["bound"] == 0.0)   # r = 1 drops nothing


# ------------------------------------------------------------------ reduced product
def pin_reduced_numpy(lib):
    """Y_g == A_g[:, I_g] @ B[I_g, :] (numpy fancy indexing + matmul), ragged groups."""
    rng = _rng(7)
    M, K, N, gr = 45, 70, 23, 16
    A, B = _ties_matrix(rng, M, K, N)
    b = np.linalg.norm(B, axis=1)
    sel = O.select(A, 0.4, gr, b, lib)
    Y = O.reduced(A, B, sel["idx"], sel["kk"], gr, lib=lib)
    for g in range(sel["idx"].shape[0]):
        I = sel["idx"][g]
        want = A[g * gr:(g + 1) * gr][:, I] @ B[I, :]
        got = Y[g * gr:(g + 1) * gr]
        err = np.abs(got - want)
        tol = 1e-13 * (np.abs(A[g * gr:(g + 1) * gr][:, I]) @ np.abs(B[I, :]))
        assert np.all(err <= tol + 1e-300), g
    # a row range gives the same rows
    part = O.reduced(A, B, sel["idx"], sel["kk"], gr, m0=17, m1=40, lib=lib)
    assert np.array_equal(part, Y[17:40])
    # single entries: same sum, same order -> identical bits
    ms = rng.integers(0, M, 50)
    ns = rng.integers(0, N, 50)
    ent = O.reduced_entries(A, B, sel["idx"], sel["kk"], gr, ms, ns, lib)
    assert np.array_equal(ent, Y[ms, ns])


def pin_dense_numpy(lib):
    """r = 1 keeps everything: the reduced product equals numpy's A @ B."""
    rng = _rng(8)
    A = rng.standard_normal((19, 31))
    B = rng.standard_normal((31, 12))
    sel = O.select(A, 1.0, 19, None, lib)
    assert sel["kk"] == 31 and np.array_equal(sel["idx"][0], np.arange(31))
    Y = O.reduced(A, B, sel["idx"], 31, 19, lib=lib)
    want = A @ B
    assert np.all(np.abs(Y - want) <= 1e-13 * (np.abs(A) @ np.abs(B)))
    assert np.array_equal(O.dense(A, B, lib), Y)


def pin_reduced_exact(lib):
    """Tiny inputs: the fp64 result is within fp64 rounding of the exact
    rational sum of the kept outer products."""
    rng = _rng(9)
    for trial in range(6):
        M, K, N = rng.integers(1, 6), rng.integers(2, 12), rng.integers(1, 6)
        A = rng.standard_normal((M, K))
        B = rng.standard_normal((K, N))
        kk = int(rng.integers(1, K + 1))
        idx = np.sort(rng.choice(K, kk, replace=False)).astype(np.int32)[None, :]
        Y = O.reduced(A, B, idx, kk, M, lib=lib)
        for m in range(M):
            for n in range(N):
                exact = sum(Fraction(float(A[m, k])) * Fraction(float(B[k, n])) for k in idx[0])
                mag = sum(abs(float(A[m, k]) * float(B[k, n])) for k in idx[0])
                assert abs(Fraction(float(Y[m, n])) - exact) <= Fraction(2 * kk * 2.0 ** -53 * mag), (m, n)


def pin_bound(lib):
    """||Y_dense - Y_rmm||_F <= beta_g, tight when one slice is dropped, and the
    top-k set minimises beta over all k-subsets."""
    rng = _rng(10)
    M, K, N, gr = 32, 24, 9, 16
    A = rng.standard_normal((M, K)) * rng.lognormal(0, 1, K)[None, :]
    B = rng.standard_normal((K, N))
    b = np.linalg.norm(B, axis=1)
    for r in (0.25, 0.5, 0.75):
        sel = O.select(A, r, gr, b, lib)
        Yr = O.reduced(A, B, sel["idx"], sel["kk"], gr, lib=lib)
        Yd = A @ B
        for g in range(2):
            err = np.linalg.norm((Yd - Yr)[g * gr:(g + 1) * gr])
            assert err <= sel["bound"][g] * (1 + 1e-12), (r, g)
            drop = np.setdiff1d(np.arange(K), sel["idx"][g])
            want = float(np.sum(np.linalg.norm(A[g * gr:(g + 1) * gr], axis=0)[drop] * b[drop]))
            assert math.isclose(sel["bound"][g], want, rel_tol=1e-12)
    # one dropped slice: the error is the rank-1 term, ||a|| ||b|| exactly
    sel = O.select(A, (K - 1) / K, gr, b, lib)
    assert sel["kk"] == K - 1
    Yr = O.reduced(A, B, sel["idx"], sel["kk"], gr, lib=lib)
    for g in range(2):
        err = np.linalg.norm((A @ B - Yr)[g * gr:(g + 1) * gr])
        assert math.isclose(err, sel["bound"][g], rel_tol=1e-9)
    # brute force: top-k minimises the bound
    A2 = rng.standard_normal((4, 9)) * rng.lognormal(0, 1, 9)[None, :]
    B2 = rng.standard_normal((9, 3))
    b2 = np.linalg.norm(B2, axis=1)
    s = np.linalg.norm(A2, axis=0) * b2
    for kk in range(1, 9):
        sel = O.select(A2, kk / 9, 4, b2, lib)
        best = min(sum(s[k] for k in range(9) if k not in sub)
                   for sub in itertools.combinations(range(9), kk))
        assert math.isclose(sel["bound"][0], best, rel_tol=1e-12), kk


def pin_closed_forms(lib):
    rng = _rng(11)
    M, K, N, gr = 24, 20, 7, 12
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    b = np.linalg.norm(B, axis=1)
    # a group with at most kk nonzero columns loses nothing
    A0 = A.copy()
    A0[:, 10:] = 0.0
    sel = O.select(A0, 0.5, gr, b, lib)
    Yr = O.reduced(A0, B, sel["idx"], sel["kk"], gr, lib=lib)
    assert np.array_equal(Yr, O.dense(A0, B, lib))
    assert np.all(np.abs(Yr - A0 @ B) <= 1e-13 * (np.abs(A0) @ np.abs(B)))
    assert np.all(sel["bound"] == 0.0)
    # positive power-of-two scaling: same sets, exactly scaled output
    sel1 = O.select(A, 0.4, gr, b, lib)
    Y1 = O.reduced(A, B, sel1["idx"], sel1["kk"], gr, lib=lib)
    for c in (4.0, 0.125):
        selc = O.select(A * c, 0.4, gr, b, lib)
        assert np.array_equal(selc["idx"], sel1["idx"])
        assert np.array_equal(O.reduced(A * c, B, selc["idx"], selc["kk"], gr, lib=lib), Y1 * c)
    # joint permutation of the contraction index permutes the sets, Y unchanged
    perm = rng.permutation(K)
    selp = O.select(A[:, perm], 0.4, gr, b[perm], lib)
    for g in range(2):
        assert set(perm[selp["idx"][g]]) == set(sel1["idx"][g])
    Yp = O.reduced(A[:, perm], B[perm], selp["idx"], selp["kk"], gr, lib=lib)
    assert np.allclose(Yp, Y1, rtol=0, atol=1e-12 * np.abs(Y1).max())


def pin_hand_examples(lib):
    g = read_golden("hand_linear.txt")
    A = np.array(g["A"], float)
    B = np.array(g["B"], float)
    b = O.rownorms(B, lib)
    assert np.allclose(b ** 2, g["b_squared"], rtol=1e-15)
    sel = O.select(A, g["r"], A.shape[0], b, lib)
    assert sel["kk"] == g["kk"]
    assert list(sel["idx"][0]) == g["I_product"]
    Y = O.reduced(A, B, sel["idx"], sel["kk"], A.shape[0], lib=lib)
    assert np.array_equal(Y, np.array(g["Y_product"], float))
    assert sel["bound"][0] == g["bound_product"]
    assert np.linalg.norm(O.dense(A, B, lib) - Y) == g["error_product"]
    sela = O.select(A, g["r"], A.shape[0], None, lib)
    assert list(sela["idx"][0]) == g["I_activation_only"]
    Ya = O.reduced(A, B, sela["idx"], sela["kk"], A.shape[0], lib=lib)
    assert np.array_equal(Ya, np.array(g["Y_activation_only"], float))
    t = read_golden("hand_ties.txt")
    selt = O.select(np.array(t["A"], float), t["r"], 1, O.rownorms(np.array(t["B"], float), lib), lib)
    assert list(selt["idx"][0]) == t["I"]


def pin_thresh_near_ties_hand(lib):
    """The threshold and the near-tie band against tests/golden/hand_near_ties.txt:
    scores at 0.9e-6 and 1.1e-6 relative of the rank-kk score, exact ties, a
    zero threshold, two scores sharing one binary32 key, and the band centred
    on the unrounded score; case 1 again at two power-of-two scales."""
    g = read_golden("hand_near_ties.txt")
    cases = [("s1", "1a"), ("s1", "1b"), ("s1", "1c"), ("s3", "3a"), ("s3", "3b"), ("s4", "4a"), ("s4", "4b"),
             ("s5", "5")]
    for c in ("1a", "1b", "1c"):
        for sc in g["scale2"]:
            cases.append((("s1", sc), c))
    for src, c in cases:
        scale = 1.0
        if isinstance(src, tuple):
            src, scale = src
        s64 = np.array(g[src], float) * scale
        s32 = s64.astype(np.float32)
        kk = g[f"kk{c}"]
        idx = O.topk(s32, kk, lib)
        assert list(idx) == g[f"I{c}"], (c, scale, list(idx))
        t = O.thresh(s32, idx, lib)
        assert t == np.float32(g[f"T{c}"] * scale), (c, scale, t)
        band = O.near_ties(s64, s32, idx, lib=lib)
        assert list(band) == g[f"band{c}"], (c, scale, list(band))


def pin_thresh_near_ties_sort(lib):
    """On random scores with repeats and zeros: T is the kk-th largest binary32
    key by numpy's sort; the band holds every slice whose unrounded score equals
    the rank-kk slice's (band width 0) and lies inside [T-, T+] of any wider
    band; every slice with a key strictly between the kept and dropped extremes
    is ordered as the band says."""
    rng = _rng(41)
    for trial in range(40):
        K = int(rng.integers(2, 300))
        s64 = rng.lognormal(0, 2, K)
        s64[rng.integers(0, K, K // 5)] = 0.0
        rep = rng.integers(0, K, K // 4)
        s64[rep] = s64[rng.integers(0, K)]
        s32 = s64.astype(np.float32)
        kk = int(rng.integers(1, K + 1))
        idx = O.topk(s32, kk, lib)
        t = O.thresh(s32, idx, lib)
        assert t == np.sort(s32)[::-1][kk - 1]
        # the rank-kk slice by the rank definition (stable argsort on (-key, index))
        order = np.lexsort((np.arange(K), -s32.astype(np.float64)))
        last = order[kk - 1]
        b0 = O.near_ties(s64, s32, idx, rel=0.0, lib=lib)
        assert list(b0) == list(np.nonzero(s64 == s64[last])[0])
        b = O.near_ties(s64, s32, idx, lib=lib)
        assert last in b and np.all(np.diff(b) > 0)
        assert set(b0) <= set(b)


# ------------------------------------------------------------------ P.V
def _causal_probs(rng, L):
    logits = rng.standard_normal((L, L))
    logits[np.triu_indices(L, 1)] = -np.inf
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)


def pin_pv_numpy(lib):
    """P.V at r = 1 over the causal prefix equals the masked dense product;
    scores equal numpy's block column mass times ||V_k||; bound holds."""
    rng = _rng(12)
    L, D, qb = 40, 6, 16               # blocks of 16, 16, 8 queries
    P = _causal_probs(rng, L)
    V = rng.standard_normal((L, D))
    Pt = np.ascontiguousarray(P.T)
    for g in range(3):
        q0 = g * qb
        nq = min(qb, L - q0)
        Kg = O.pv_prefix(L, qb, g, True, lib)
        assert Kg == min(L, qb * (g + 1))
        assert O.pv_prefix(L, qb, g, False, lib) == L
        Ptb = O.pv_block_inputs(Pt, q0, nq, Kg)
        s64, _ = O.pv_scores(Ptb, V[:Kg], lib)
        want = P[q0:q0 + nq, :Kg].sum(axis=0) * np.linalg.norm(V[:Kg], axis=1)
        assert np.allclose(s64, want, rtol=1e-13, atol=0)
        full = O.pv_block(Ptb, V[:Kg], np.arange(Kg, dtype=np.int32), lib)
        want_o = P[q0:q0 + nq] @ V
        assert np.all(np.abs(full - want_o) <= 1e-13 * (np.abs(P[q0:q0 + nq]) @ np.abs(V)) + 1e-300)
        for r in (0.3, 0.5):
            sel = O.pv_select_block(Pt, V, L, qb, g, r, True, lib)
            assert sel["kk"] == max(1, math.ceil(Fraction(str(r)) * Kg))
            assert np.array_equal(sel["idx"], _argsort_topk(sel["s32"], sel["kk"]))
            part = O.pv_block(sel["Ptb"], sel["V"], sel["idx"], lib)
            I = sel["idx"]
            assert np.allclose(part, P[q0:q0 + nq][:, I] @ V[I], rtol=0, atol=1e-13)
            beta = O.pv_bound(sel["Ptb"], sel["V"], sel["idx"], lib)
            assert np.linalg.norm(full - part) <= beta * (1 + 1e-12)
            drop = np.setdiff1d(np.arange(Kg), I)
            want_b = np.sum(np.linalg.norm(P[q0:q0 + nq][:, drop], axis=0) * np.linalg.norm(V[drop], axis=1))
            assert math.isclose(beta, want_b, rel_tol=1e-12) or (beta == 0 and want_b == 0)


def pin_pv_hand(lib):
    g = read_golden("hand_pv.txt")
    P = np.array(g["P"], float)
    V = np.array(g["V"], float)
    Pt = np.ascontiguousarray(P.T)
    L = P.shape[0]
    for blk in g["blocks"]:
        sel = O.pv_select_block(Pt, V, L, g["qblock"], blk["g"], g["r"], True, lib)
        assert sel["Kg"] == blk["Kg"] and sel["kk"] == blk["kk"]
        assert np.allclose(sel["s64"] ** 2, blk["scores_squared"], rtol=1e-15)
        assert list(sel["idx"]) == blk["I"]
        Ob = O.pv_block(sel["Ptb"], sel["V"], sel["idx"], lib)
        assert np.array_equal(Ob, np.array(blk["O"], float))


# ------------------------------------------------------------------ int8 weights
def pin_q8_hand(lib):
    """The hand-worked quantisation of tests/golden/hand_q8.txt; the dequantised
    values and row norms checked in exact rational arithmetic."""
    g = read_golden("hand_q8.txt")
    B = np.array(g["B"], np.float32)
    q, s = O.quantize_q8(B, lib)
    assert q.tolist() == g["q"], q
    assert s.view(np.uint32).tolist() == g["scale_bits"]
    Bd = O.dequant_q8(q, s, lib)
    b = O.rownorms_q8(q, s, lib)
    for k in range(B.shape[0]):
        ss = Fraction(0)
        for n in range(B.shape[1]):
            v = Fraction(float(s[n])) * int(q[k, n])
            assert Fraction(float(Bd[k, n])) == v
            ss += v * v
        assert abs(Fraction(float(b[k])) ** 2 - ss) <= ss * Fraction(1, 10 ** 15)


def pin_q8_rounding(lib):
    """Scales equal numpy's binary32 division of the column absmax by 127; every
    code is the integer nearest to B/s (exact halves to even), within [-127, 127],
    +-127 at each column's absmax; all-zero columns give s = 0, q = 0."""
    rng = _rng(21)
    K, N = 37, 29
    B = (rng.standard_normal((K, N)) * rng.lognormal(0, 1, N)[None, :] * 0.02).astype(np.float32)
    B[:, 4] = 0.0
    B[:, 7] = 0.0
    B[3, 7] = -2.5
    # a column whose scale is exactly 2^-4, with exact halves in B/s
    B[:, 10] = np.array([(k - 18) * 0.5 * 2.0 ** -4 for k in range(K)], np.float32)
    B[0, 10] = 127 * 2.0 ** -4
    q, s = O.quantize_q8(B, lib)
    amax = np.abs(B).max(axis=0)
    want_s = (amax / np.float32(127)).astype(np.float32)
    assert np.array_equal(s.view(np.uint32), want_s.view(np.uint32))
    assert s[10] == 2.0 ** -4
    assert np.all(q[:, 4] == 0) and s[4] == 0
    assert q[3, 7] == -127 and np.count_nonzero(q[:, 7]) == 1
    assert np.all(np.abs(q.astype(int)) <= 127)
    nz = s > 0
    x = B[:, nz].astype(np.float64) / s[nz].astype(np.float64)
    qn = q[:, nz].astype(np.float64)
    assert np.all(np.abs(x - qn) <= 0.5 + 1e-6)
    far = np.abs(np.abs(x - np.floor(x)) - 0.5) > 1e-5
    assert np.array_equal(qn[far], np.rint(x)[far])
    assert np.array_equal(q[:, 10].astype(np.float64), np.rint(B[:, 10] / 2.0 ** -4))
    am = np.argmax(np.abs(B), axis=0)
    assert np.all(np.abs(q[am[nz], np.flatnonzero(nz)].astype(int)) == 127)


def pin_q8_dequant_norms(lib):
    """Dequantised weight = numpy's float64 product scale[n] * q[k, n]; its
    error is at most half a step per element; row norms = numpy's norms."""
    rng = _rng(22)
    K, N = 45, 33
    B = (rng.standard_normal((K, N)) * rng.lognormal(0, 1, N)[None, :] * 0.02).astype(np.float32)
    q, s = O.quantize_q8(B, lib)
    Bd = O.dequant_q8(q, s, lib)
    want = s.astype(np.float64)[None, :] * q.astype(np.float64)
    assert np.array_equal(Bd, want)
    assert np.all(np.abs(B.astype(np.float64) - Bd) <= 0.5 * s.astype(np.float64)[None, :] * (1 + 1e-6))
    b = O.rownorms_q8(q, s, lib)
    assert np.allclose(b, np.linalg.norm(want, axis=1), rtol=1e-13, atol=0)


# ------------------------------------------------------------------ QK^T and probabilities
def pin_qk_hand(lib):
    """The hand-worked feature selection and probabilities of
    tests/golden/hand_qk.txt (causal, every key, activation-only)."""
    g = read_golden("hand_qk.txt")
    Q = np.array(g["Q"], float)
    K = np.array(g["K"], float)
    qb = g["qblock"]
    rows = []
    for blk in g["blocks"]:
        sel = O.qk_select_block(Q, K, qb, blk["g"], g["r"], True, True, lib)
        assert sel["Kg"] == blk["Kg"] and sel["kk"] == 2
        assert np.allclose(sel["s64"] ** 2, blk["scores_squared"], rtol=1e-15, atol=0)
        assert list(sel["idx"]) == blk["I"]
        nc = O.qk_select_block(Q, K, qb, blk["g"], g["r"], False, True, lib)
        assert np.allclose(nc["s64"] ** 2, blk["noncausal_scores_squared"], rtol=1e-15, atol=0)
        assert list(nc["idx"]) == blk["noncausal_I"]
        ao = O.qk_select_block(Q, K, qb, blk["g"], g["r"], True, False, lib)
        assert list(ao["idx"]) == blk["aonly_I"]
        q0 = blk["g"] * qb
        rows.append(O.attn_probs(Q, K, q0, qb, True, sel["idx"], lib))
    P = np.vstack(rows)
    want = np.array([[float(Fraction(str(x))) for x in row] for row in g["P_decimal"]])
    assert np.all(np.abs(P - want) <= 4e-16 * np.maximum(want, 1e-300)), P - want


def _qk_inputs(rng, L, D):
    Q = rng.standard_normal((L, D)) * rng.lognormal(0, 1, D)[None, :]
    K = rng.standard_normal((L, D))
    Q[:, 2] = 0.0                        # a dead feature: score 0
    K[:, 4] = K[:, 1]
    Q[:, 4] = Q[:, 1]                    # features 1 and 4 tie exactly
    return Q, K


def pin_qk_scores(lib):
    """Feature scores equal numpy's norms of the block's query columns times
    the norms of the candidate keys' columns; keys a block does not see change
    nothing; the dropped scores bound the error of the reduced logits; the kept
    set matches a stable argsort and nests in r."""
    rng = _rng(31)
    L, D, qb = 37, 8, 12                 # blocks of 12, 12, 12, 1 queries
    Q, K = _qk_inputs(rng, L, D)
    for causal in (True, False):
        for g in range(4):
            q0 = g * qb
            nq = min(qb, L - q0)
            Kg = O.pv_prefix(L, qb, g, causal, lib)
            s64, s32 = O.qk_scores(Q, K, q0, nq, Kg, True, lib)
            want = np.linalg.norm(Q[q0:q0 + nq], axis=0) * np.linalg.norm(K[:Kg], axis=0)
            assert np.allclose(s64, want, rtol=1e-14, atol=0)
            assert np.array_equal(s32, s64.astype(np.float32))
            a64, _ = O.qk_scores(Q, K, q0, nq, Kg, False, lib)
            assert np.allclose(a64, np.linalg.norm(Q[q0:q0 + nq], axis=0), rtol=1e-14, atol=0)
            # keys past the candidates and queries outside the block do not matter
            K2 = K.copy()
            K2[Kg:] *= 1e3
            Q2 = Q.copy()
            Q2[:q0] = 7.0
            Q2[q0 + nq:] = -3.0
            assert np.array_equal(O.qk_scores(Q2, K2, q0, nq, Kg, True, lib)[0], s64)
            prev = None
            for r in (0.25, 0.5, 0.75, 1.0):
                sel = O.qk_select_block(Q, K, qb, g, r, causal, True, lib)
                assert sel["kk"] == math.ceil(Fraction(str(r)) * D)
                assert np.array_equal(sel["idx"], _argsort_topk(sel["s32"], sel["kk"]))
                if prev is not None:
                    assert set(prev) <= set(sel["idx"])
                prev = sel["idx"]
                # bound on the unscaled logits over the block x candidate keys
                I = sel["idx"]
                full = Q[q0:q0 + nq] @ K[:Kg].T
                red = Q[q0:q0 + nq][:, I] @ K[:Kg][:, I].T
                drop = np.setdiff1d(np.arange(D), I)
                beta = float(np.sum(s64[drop]))
                assert np.linalg.norm(full - red) <= beta * (1 + 1e-12) + 1e-12
    # brute force: the kept set minimises the dropped score sum (D = 8, kk = 4)
    s64, s32 = O.qk_scores(Q, K, 0, qb, qb, True, lib)
    sel = O.qk_select_block(Q, K, qb, 0, 0.5, True, True, lib)
    best = min(itertools.combinations(range(D), 4),
               key=lambda c: (sum(float(s32[j]) for j in range(D) if j not in c), c))
    assert tuple(sel["idx"]) == best


def pin_attn_probs(lib):
    """Probabilities equal scipy's softmax of numpy's masked logits (the dropped
    features zeroed); rows sum to 1 and are 0 past the causal edge; identical
    keys give 1/(q+1); a common shift of every key leaves P unchanged."""
    import scipy.special as sps
    rng = _rng(32)
    L, D = 29, 8
    Q, K = _qk_inputs(rng, L, D)
    for causal in (True, False):
        for idx in (None, np.array([0, 1, 3, 6], np.int32), np.array([5], np.int32)):
            P = O.attn_probs(Q, K, 0, L, causal, idx, lib)
            Qm = Q.copy()
            if idx is not None:
                keep = np.zeros(D, bool)
                keep[idx] = True
                Qm[:, ~keep] = 0.0
            S = (Qm @ K.T) / math.sqrt(D)
            if causal:
                S = np.where(np.tril(np.ones((L, L), bool)), S, -np.inf)
            want = sps.softmax(S, axis=1)
            assert np.allclose(P, want, rtol=1e-12, atol=1e-300)
            assert np.all(np.abs(P.sum(axis=1) - 1.0) <= 1e-14 * L)
            if causal:
                assert np.all(P[np.triu_indices(L, 1)] == 0.0)
            # a block of rows in the middle equals the same rows of the whole
            part = O.attn_probs(Q, K, 9, 7, causal, idx, lib)
            assert np.array_equal(part, P[9:16])
            shift = rng.standard_normal(D)
            Ps = O.attn_probs(Q, K + shift[None, :], 0, L, causal, idx, lib)
            assert np.allclose(Ps, P, rtol=1e-11, atol=1e-300)
    Keq = np.tile(rng.standard_normal(D), (L, 1))
    P = O.attn_probs(Q, Keq, 0, L, True, None, lib)
    for q in range(L):
        assert np.all(P[q, :q + 1] == 1.0 / (q + 1))


ALL_PINS = [
    pin_kk_exact_rational, pin_kk_golden, pin_norms_numpy, pin_scores_numpy, pin_topk_argsort,
    pin_topk_invariants, pin_topk_bruteforce, pin_select_nesting, pin_reduced_numpy,
    pin_dense_numpy, pin_reduced_exact, pin_bound, pin_closed_forms, pin_hand_examples,
    pin_thresh_near_ties_hand, pin_thresh_near_ties_sort,
    pin_pv_numpy, pin_pv_hand, pin_q8_hand, pin_q8_rounding, pin_q8_dequant_norms,
    pin_qk_hand, pin_qk_scores, pin_attn_probs,
]
