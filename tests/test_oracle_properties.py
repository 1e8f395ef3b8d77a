"""Property-based checks of the oracle (CPU only), drawn by hypothesis over
small random inputs.  Each property is a fact of the mathematics or an
independent formulation, not the oracle's own code:

  - the kept set equals the rank definition (a slice is kept iff fewer than
    kk slices beat it, ties going to the lower index), ascending;
  - the retained count is ceil(r K) in exact rational arithmetic for decimal r;
  - kept sets nest as r grows;
  - at r = 1 the reduced product is numpy's A @ B;
  - the dropped scores bound the Frobenius error of the reduced product;
  - attention rows sum to 1, are 0 past the causal edge, and do not change
    when every key moves by the same vector.

Method source: "Reduced Matrix Multiplication: Input-Adaptive Matrix-Product
Reduction for LLM Inference", technical summary (gist.science), Metodologia
(Mecanismo Central; Estrategia de Selecao; Escopo de Aplicacao).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _matrix(seed, rows, cols, ties):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols))
    if ties:
        a = np.round(a * 2) / 2          # coarse values: many equal column norms
    return a


@SETTINGS
@given(st.integers(0, 2 ** 31), st.integers(1, 40), st.data())
def test_topk_is_the_rank_definition(seed, K, data):
    rng = np.random.default_rng(seed)
    s = rng.integers(0, 6, size=K).astype(np.float32) * np.float32(0.25)   # many ties, zeros
    kk = data.draw(st.integers(1, K))
    idx = O.topk(s, kk)
    rank = np.array([np.sum((s > s[k]) | ((s == s[k]) & (np.arange(K) < k))) for k in range(K)])
    assert list(idx) == sorted(np.flatnonzero(rank < kk).tolist())


@SETTINGS
@given(st.integers(1, 999), st.integers(1, 5000))
def test_kk_is_exact_ceiling(milli, K):
    r = milli / 1000
    want = max(1, math.ceil(Fraction(milli, 1000) * K))
    assert O.kk(r, K) == min(K, want)


@SETTINGS
@given(st.integers(0, 2 ** 31), st.integers(1, 9), st.integers(2, 24), st.booleans())
def test_selection_nests_in_r(seed, M, K, ties):
    A = _matrix(seed, M, K, ties)
    prev = set()
    for r in (0.1, 0.3, 0.5, 0.8, 1.0):
        sel = O.select(A, r, M, None)
        cur = set(sel["idx"][0].tolist())
        assert prev <= cur
        prev = cur


@SETTINGS
@given(st.integers(0, 2 ** 31), st.integers(1, 12), st.integers(1, 16), st.integers(1, 9), st.integers(1, 6))
def test_dense_at_r1_and_bound(seed, M, K, N, gr):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)) * rng.lognormal(0, 1, K)[None, :]
    B = rng.standard_normal((K, N))
    b = O.rownorms(B)
    full = O.select(A, 1.0, gr, b)
    Y1 = O.reduced(A, B, full["idx"], K, gr)
    assert np.allclose(Y1, A @ B, rtol=1e-12, atol=1e-12)
    sel = O.select(A, 0.5, gr, b)
    kk = sel["kk"]
    Y = O.reduced(A, B, sel["idx"], kk, gr)
    for g in range(-(-M // gr)):
        rows = slice(g * gr, min(M, (g + 1) * gr))
        beta = O.bound(sel["s64"][g], sel["idx"][g])
        assert np.linalg.norm((A @ B)[rows] - Y[rows]) <= beta * (1 + 1e-12) + 1e-12


@SETTINGS
@given(st.integers(0, 2 ** 31), st.integers(1, 20), st.integers(1, 8), st.booleans())
def test_attention_rows(seed, L, D, causal):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((L, D)) * 2
    K = rng.standard_normal((L, D))
    P = O.attn_probs(Q, K, 0, L, causal)
    assert np.all(np.abs(P.sum(axis=1) - 1.0) <= 1e-13)
    if causal:
        assert np.all(P[np.triu_indices(L, 1)] == 0.0)
    shift = rng.standard_normal(D)
    assert np.allclose(O.attn_probs(Q, K + shift[None, :], 0, L, causal), P, rtol=1e-10, atol=1e-300)


@SETTINGS
@given(st.integers(0, 2 ** 31), st.integers(2, 24), st.integers(2, 8), st.integers(1, 8))
def test_qk_scores_ignore_unseen_keys(seed, L, D, qb):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((L, D))
    K = rng.standard_normal((L, D))
    G = -(-L // qb)
    g = int(rng.integers(0, G))
    q0 = g * qb
    nq = min(qb, L - q0)
    Kg = O.pv_prefix(L, qb, g, True)
    s, _ = O.qk_scores(Q, K, q0, nq, Kg, True)
    K2 = K.copy()
    K2[Kg:] = rng.standard_normal((L - Kg, D)) * 100
    s2, _ = O.qk_scores(Q, K2, q0, nq, Kg, True)
    assert np.array_equal(s, s2)
