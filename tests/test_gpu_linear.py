"""GPU parity of the linear-layer hot path (score -> select -> gather -> reduced
GEMM, and the r = 1 dense baseline) against the oracle, through the C ABI.

Small cases span several tiles and ragged tails (short last group, N not a
multiple of the tile, kk not a multiple of 8 or 64) and are compared element by
element; the full workload sizes are compared on every group's scores and kept
set and on every output element.  Scores, B norms, kept sets and panels must be
bit-exact (both sides sum in binary64 in ascending order and round once to
binary32); outputs within the bound documented in tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (DEV, check_output, compare_sets, down, log, oracle_rows, up_bf16,
                      up_f32, widen)
from input_adaptive_reduced_02_amd import rmm, synth

pytestmark = pytest.mark.gpu


def make_case(workload, M, K, N, seed=0):
    d = synth.linear_inputs(workload, M, K, N, seed=seed)
    if d["dtype"] == "bf16":
        A64, B64 = O.widen_bf16(d["A"]), O.widen_bf16(d["B"])
        A, B = up_bf16(d["A"]), up_bf16(d["B"])
    else:
        A64, B64 = O.widen_f32(d["A"]), O.widen_f32(d["B"])
        A, B = up_f32(d["A"]), up_f32(d["B"])
    return dict(A=A, B=B, A64=A64, B64=B64, f32=d["dtype"] == "f32", raw=d)


def run_chain(c, r, gr, bnorm):
    """The hot path through the C ABI; returns (idx, scores, thresh, bound, Ap, Y)."""
    A, B = c["A"], c["B"]
    M, K = A.shape
    kk = rmm.rmm_kk(r, K)
    G = -(-M // gr)
    scores = torch.empty((G, K), dtype=torch.float32, device=DEV)
    thresh = torch.empty(G, dtype=torch.float32, device=DEV)
    bound = torch.empty(G, dtype=torch.float64, device=DEV)
    idx = torch.zeros((G, rmm.rmm_kk_pad(kk)), dtype=torch.int32, device=DEV)
    if c["f32"]:
        rmm.rmm_select(A, r, gr, bnorm=bnorm, idx=idx, scores=scores, thresh=thresh, bound=bound)
        check_index_range(idx, K)
        Ap, Bp = rmm.rmm_gather(A, idx, kk, gr, B=B)
        Y = rmm.rmm_gemm(Ap, Bp, None, kk, gr, ydt=torch.float32)
    else:
        # the launch sequence the benchmark times: select + gather in one call
        _, Ap = rmm.rmm_select_gather(A, r, gr, bnorm=bnorm, idx=idx, scores=scores, thresh=thresh,
                                      bound=bound)
        check_index_range(idx, K)
        Y = rmm.rmm_gemm(Ap, B, idx, kk, gr)
    torch.cuda.synchronize()
    return idx, scores, thresh, bound, Ap, Y


def check_index_range(idx, K):
    """Host check before any kernel reads rows by these indices."""
    torch.cuda.synchronize()
    ig = down(idx)
    assert ig.min() >= 0 and ig.max() < K, f"kept index out of range [{ig.min()}, {ig.max()}], K={K}"


def check_selection(c, r, gr, bnorm, idx, scores, thresh, bound, tag):
    sel = O.select(c["A64"], r, gr, O.rownorms(c["B64"]))
    kk = sel["kk"]
    assert np.array_equal(down(scores), sel["s32"]), f"{tag}: scores differ from the oracle"
    ig = down(idx)
    for g in range(ig.shape[0]):
        compare_sets(ig[g], sel, g, kk, tag)
        assert np.all(ig[g, kk:] == ig[g, kk - 1]), f"{tag}: padding of group {g}"
    assert np.array_equal(down(thresh), sel["thresh"]), f"{tag}: thresholds differ from the oracle"
    assert np.allclose(down(bound), sel["bound"], rtol=1e-6, atol=0)
    n_near = sum(len(x) for x in sel["near"])
    log(f"  {tag}: kk={kk} groups={ig.shape[0]} sets exact, near-tie indices={n_near}")
    return sel, ig


SMALL = [
    # (workload, M, K, N, group_rows, r)
    ("tiny", 64, 256, 128, 64, 0.5),                 # the full tiny workload
    ("attn_proj", 300, 1000, 264, 128, 0.3),         # groups 128,128,44; N tail 8; kk=300
    ("attn_proj", 300, 1000, 264, 128, 0.5),
    ("mlp_down", 256, 2048, 512, 128, 0.7),
    ("decode", 64, 4096, 1024, 64, 0.3),             # narrow tiles, kk=1229
    ("attn_proj", 200, 520, 72, 128, 0.37),          # kk=193: not a multiple of 8
    ("mlp_down", 96, 136, 40, 32, 0.9),              # group_rows 32, kk=123
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-g{c[4]}-r{c[5]}")
def test_chain_small(case):
    workload, M, K, N, gr, r = case
    tag = f"{workload} {M}x{K}x{N} gr={gr} r={r}"
    log(f"case {tag}")
    c = make_case(workload, M, K, N)
    bnorm = rmm.rmm_rownorms(c["B"])
    torch.cuda.synchronize()
    b_ref = O.rownorms(c["B64"])
    assert np.array_equal(down(bnorm), b_ref), "B row norms differ from the oracle"
    idx, scores, thresh, bound, Ap, Y = run_chain(c, r, gr, bnorm)
    sel, ig = check_selection(c, r, gr, bnorm, idx, scores, thresh, bound, tag)
    kk = sel["kk"]
    # panel: exact bf16 of the kept columns, zero padding
    ap = down(Ap)
    A_bits = c["raw"]["A"]
    for m in range(M):
        cols = ig[m // gr, :kk]
        if c["f32"]:
            want = torch.from_numpy(np.ascontiguousarray(A_bits[m, cols])).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        else:
            want = A_bits[m, cols]
        assert np.array_equal(ap[m, :kk], want), f"panel row {m}"
        assert np.all(ap[m, kk:] == 0)
    # output, computed by the oracle on the GPU's kept sets
    Yref = O.reduced(c["A64"], c["B64"], ig, kk, gr)
    Sabs = O.reduced(np.abs(c["A64"]), np.abs(c["B64"]), ig, kk, gr)
    check_output(widen(Y), Yref, Sabs, kk, tag, f32_inputs=c["f32"])


@pytest.mark.parametrize("shape", [(300, 1000, 264, 128), (64, 4096, 1024, 64), (200, 520, 72, 128),
                                   (130, 64, 8, 128)])
def test_dense_baseline_small(shape):
    """r = 1: the same GEMM kernel, A and B read in place, equals the oracle's dense product."""
    M, K, N, gr = shape
    c = make_case("attn_proj", M, K, N, seed=3)
    log(f"dense {shape}")
    Y = rmm.rmm_gemm(c["A"], c["B"], None, K, gr)
    Y32 = rmm.rmm_gemm(c["A"], c["B"], None, K, gr, ydt=torch.float32)
    torch.cuda.synchronize()
    Yref = O.dense(c["A64"], c["B64"])
    Sabs = O.dense(np.abs(c["A64"]), np.abs(c["B64"]))
    check_output(widen(Y), Yref, Sabs, K, f"dense bf16 {shape}")
    # fp32 output: no output rounding, only accumulation error
    err = np.abs(widen(Y32) - Yref)
    assert np.all(err <= 1.01 * K * 2.0 ** -24 * Sabs + 1e-30)


def test_determinism():
    c = make_case("attn_proj", 512, 2048, 1024)
    bnorm = rmm.rmm_rownorms(c["B"])
    out1 = run_chain(c, 0.5, 128, bnorm)
    out2 = run_chain(c, 0.5, 128, bnorm)
    for a, b in zip(out1, out2):
        assert torch.equal(a, b)


def test_edge_cases():
    # all-zero columns and columns of equal norm: ties everywhere, lower index wins
    rng = np.random.default_rng(5)
    M, K, N, gr = 128, 512, 256, 64
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:, 100:300] = 0.0                    # 200 zero columns (score 0)
    a[:, 300:400] = a[:, 7:8]              # 100 copies of column 7 (equal scores)
    b = np.full((K, N), 0.5, np.float32)   # equal B row norms
    A = up_bf16(synth.f32_to_bf16_bits(a))
    B = up_bf16(synth.f32_to_bf16_bits(b))
    A64, B64 = widen(A), widen(B)
    bnorm = rmm.rmm_rownorms(B)
    for r in (1e-6, 0.05, 0.2, 0.4, 0.5, 0.9, 1.0):
        idx = torch.zeros((M // gr, rmm.rmm_kk_pad(rmm.rmm_kk(r, K))), dtype=torch.int32, device=DEV)
        rmm.rmm_select(A, r, gr, bnorm=bnorm, idx=idx)
        check_index_range(idx, K)
        sel = O.select(A64, r, gr, O.rownorms(B64))
        ig = down(idx)
        assert np.array_equal(ig[:, :sel["kk"]], sel["idx"]), r
        kk = sel["kk"]
        Ap, _ = rmm.rmm_gather(A, idx, kk, gr)
        Y = rmm.rmm_gemm(Ap, B, idx, kk, gr)
        torch.cuda.synchronize()
        Yref = O.reduced(A64, B64, ig, kk, gr)
        check_output(widen(Y), Yref, O.reduced(np.abs(A64), B64, ig, kk, gr), kk, f"ties r={r}")
    # kk = 1, K tiny, a group larger than M, one-row groups, the activation-only rule
    for (M, K, N, gr, r, act) in [(64, 8, 8, 64, 0.1, False), (50, 64, 16, 1000, 0.5, False),
                                  (16, 96, 24, 1, 0.25, False), (160, 256, 64, 128, 0.5, True)]:
        c = make_case("attn_proj", M, K, N, seed=9)
        bn = None if act else rmm.rmm_rownorms(c["B"])
        idx = torch.zeros((-(-M // gr), rmm.rmm_kk_pad(rmm.rmm_kk(r, K))), dtype=torch.int32, device=DEV)
        rmm.rmm_select(c["A"], r, gr, bnorm=bn, idx=idx)
        check_index_range(idx, K)
        Y = rmm.linear(c["A"], c["B"], r, gr, bnorm=bn, activation_only=act)
        torch.cuda.synchronize()
        sel = O.select(c["A64"], r, gr, None if act else O.rownorms(c["B64"]))
        ig = down(idx)
        assert np.array_equal(ig[:, :sel["kk"]], sel["idx"])
        Yref = O.reduced(c["A64"], c["B64"], sel["idx"], sel["kk"], gr)
        Sabs = O.reduced(np.abs(c["A64"]), np.abs(c["B64"]), sel["idx"], sel["kk"], gr)
        check_output(widen(Y), Yref, Sabs, sel["kk"], f"edge M={M} K={K} N={N} gr={gr} r={r} act={act}")


def test_select_large_threshold_buckets():
    """Groups whose threshold bucket holds many keys: every score equal (all
    K keys in one bucket, the search shared by the whole workgroup), 1500
    columns of equal norm around the kk-th score, and a few hundred equal
    columns; kept sets against the oracle, through rmm_select and
    rmm_select_gather."""
    rng = np.random.default_rng(17)
    M, K, N, gr = 384, 4096, 64, 128
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[0:128] = 0.0                                     # group 0: every score 0
    a[128:256, 1000:2500] = a[128:256, 7:8]            # group 1: 1500 equal columns
    a[256:384, 3000:3300] = a[256:384, 5:6]            # group 2: 300 equal columns
    A = up_bf16(synth.f32_to_bf16_bits(a))
    B = up_bf16(synth.f32_to_bf16_bits(np.full((K, N), 0.25, np.float32)))
    A64, B64 = widen(A), widen(B)
    bnorm = rmm.rmm_rownorms(B)
    for r in (0.3, 0.5, 0.7):
        kk = rmm.rmm_kk(r, K)
        sel = O.select(A64, r, gr, O.rownorms(B64))
        idx = torch.zeros((3, rmm.rmm_kk_pad(kk)), dtype=torch.int32, device=DEV)
        rmm.rmm_select(A, r, gr, bnorm=bnorm, idx=idx)
        idx2, ap = rmm.rmm_select_gather(A, r, gr, bnorm=bnorm)
        torch.cuda.synchronize()
        ig = down(idx)
        assert np.array_equal(ig[:, :kk], sel["idx"]), r
        assert torch.equal(idx, idx2), r
        pan = down(ap)
        bits = synth.f32_to_bf16_bits(a)
        for m in (0, 127, 128, 200, 383):
            assert np.array_equal(pan[m, :kk], bits[m, ig[m // gr, :kk]]), (r, m)


@pytest.mark.parametrize("K", [32768, 32760], ids=lambda k: f"K{k}")
def test_max_contraction(K):
    """The largest K the selection takes (32 keys per thread), and a ragged one:
    rows of 64 KiB are past the LDS-staged gather, so the gather reads A by
    index; kept sets against the oracle, the panel exact, every output row
    within the bound."""
    M, N, gr, r = 200, 72, 128, 0.5
    tag = f"max K={K}"
    log(f"case {tag}")
    c = make_case("attn_proj", M, K, N, seed=23)
    bnorm = rmm.rmm_rownorms(c["B"])
    idx, scores, thresh, bound, Ap, Y = run_chain(c, r, gr, bnorm)
    sel, ig = check_selection(c, r, gr, bnorm, idx, scores, thresh, bound, tag)
    kk = sel["kk"]
    ap = down(Ap)
    for m in (0, 127, 128, 199):
        assert np.array_equal(ap[m, :kk], c["raw"]["A"][m, ig[m // gr, :kk]]), f"{tag}: panel row {m}"
        assert np.all(ap[m, kk:] == 0)
    Yref = O.reduced(c["A64"], c["B64"], ig, kk, gr)
    Sabs = O.reduced(np.abs(c["A64"]), np.abs(c["B64"]), ig, kk, gr)
    check_output(widen(Y), Yref, Sabs, kk, tag)


# ---------------------------------------------------------------- full sizes
FULL = [("attn_proj", 0.3), ("attn_proj", 0.5), ("attn_proj", 0.7), ("attn_proj", 1.0),
        ("mlp_down", 0.5), ("mlp_down", 0.7), ("mlp_down", 0.9), ("mlp_down", 1.0),
        ("decode", 0.3), ("decode", 0.5), ("decode", 0.7), ("decode", 1.0)]

_full_cache = {}


def _full(workload):
    if workload not in _full_cache:
        _full_cache.clear()
        M, K, N = synth.FULL_SHAPES[workload]
        c = make_case(workload, M, K, N)
        c["bnorm"] = rmm.rmm_rownorms(c["B"])
        c["b_ref"] = O.rownorms(c["B64"])
        c["A64abs"] = np.abs(c["A64"])
        c["B64abs"] = np.abs(c["B64"])
        _full_cache[workload] = c
    return _full_cache[workload]


@pytest.mark.parametrize("workload,r", FULL, ids=lambda x: str(x))
def test_full_size(workload, r):
    """Full workload shape, in the launch configuration the benchmark times:
    every group's scores and kept set exact; every output element against the
    oracle's product on the GPU's kept sets."""
    c = _full(workload)
    M, K = c["A"].shape
    N = c["B"].shape[1]
    gr = synth.GROUP_ROWS[workload]
    tag = f"{workload} {M}x{K}x{N} r={r}"
    log(f"full {tag}")
    assert np.array_equal(down(c["bnorm"]), c["b_ref"])
    G = -(-M // gr)
    rows = np.arange(M)
    if r == 1.0:
        Y = rmm.linear(c["A"], c["B"], r, gr, bnorm=c["bnorm"])
        torch.cuda.synchronize()
        ig = np.arange(K, dtype=np.int32)[None, :].repeat(G, 0)
        kk = K
    else:
        idx, scores, thresh, bound, Ap, Y = run_chain(c, r, gr, c["bnorm"])
        sel, ig = check_selection(c, r, gr, c["bnorm"], idx, scores, thresh, bound, tag)
        kk = sel["kk"]
    Yg = widen(Y)
    Yref, Sabs = oracle_rows(c["A64"], c["B64"], ig, kk, gr, rows, c["A64abs"], c["B64abs"])
    check_output(Yg, Yref, Sabs, kk, tag + f" (all {M} rows)")


@pytest.mark.parametrize("case", [("attn_proj", 4096, 1000, 8, 8, 0.3), ("decode", 2048, 3000, 8, 4, 0.5),
                                  ("mlp_down", 1024, 256, 8, 2, 0.7)],
                         ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-g{c[4]}-r{c[5]}")
def test_select_many_groups(case):
    """512 or more groups take the one-wave-per-group select: scores, kept sets,
    thresholds and bounds against the oracle, including groups of 2 rows whose
    scores repeat and groups where every key is equal (rows of zeros)."""
    workload, M, K, N, gr, r = case
    tag = f"many groups {workload} {M}x{K} gr={gr} r={r}"
    log(f"case {tag}")
    c = make_case(workload, M, K, N, seed=5)
    A = c["A"].clone()
    A[: 3 * gr] = 0   # three all-zero groups: every score 0, ties broken by index
    c = dict(c, A=A, A64=np.where(np.arange(M)[:, None] < 3 * gr, 0.0, c["A64"]))
    assert -(-M // gr) >= 512
    bnorm = rmm.rmm_rownorms(c["B"])
    kk = rmm.rmm_kk(r, K)
    G = -(-M // gr)
    scores = torch.empty((G, K), dtype=torch.float32, device=DEV)
    thresh = torch.empty(G, dtype=torch.float32, device=DEV)
    bound = torch.empty(G, dtype=torch.float64, device=DEV)
    idx = torch.zeros((G, rmm.rmm_kk_pad(kk)), dtype=torch.int32, device=DEV)
    rmm.rmm_select(A, r, gr, bnorm=bnorm, idx=idx, scores=scores, thresh=thresh, bound=bound)
    check_index_range(idx, K)
    check_selection(c, r, gr, bnorm, idx, scores, thresh, bound, tag)


@pytest.mark.parametrize("workload,r", [("attn_proj", 0.5), ("decode", 0.3)], ids=lambda x: str(x))
def test_full_size_activation_only(workload, r):
    """The pages' activation-only rule (score = ||A[rows_g, k]||_2, no B norms)
    at full size: every group's scores and kept set against the oracle's
    activation-only selection, every output element."""
    c = _full(workload)
    M, K = c["A"].shape
    N = c["B"].shape[1]
    gr = synth.GROUP_ROWS[workload]
    tag = f"{workload} activation-only r={r}"
    log(f"full {tag}")
    kk = rmm.rmm_kk(r, K)
    G = -(-M // gr)
    scores = torch.empty((G, K), dtype=torch.float32, device=DEV)
    idx = torch.zeros((G, rmm.rmm_kk_pad(kk)), dtype=torch.int32, device=DEV)
    rmm.rmm_select(c["A"], r, gr, idx=idx, scores=scores)
    check_index_range(idx, K)
    sel = O.select(c["A64"], r, gr, None)
    assert np.array_equal(down(scores), sel["s32"]), f"{tag}: scores differ from the oracle"
    ig = down(idx)
    for g in range(G):
        compare_sets(ig[g], sel, g, kk, tag)
    Ap, _ = rmm.rmm_gather(c["A"], idx, kk, gr)
    Y = rmm.rmm_gemm(Ap, c["B"], idx, kk, gr)
    torch.cuda.synchronize()
    Yref, Sabs = oracle_rows(c["A64"], c["B64"], ig, kk, gr, np.arange(M), c["A64abs"], c["B64abs"])
    check_output(widen(Y), Yref, Sabs, kk, tag + f" (all {M} rows)")


# ---------------------------------------------------------------- select + gather in one call
SG = [
    # (workload, M, K, N, group_rows, r, lda): the fused kernel's slicing and
    # staging sizes, ragged groups, a padded leading dimension, and shapes that
    # take the two-launch fallback (K > 8192, 512 or more groups)
    ("attn_proj", 2048, 4096, 8, 128, 0.5, 4096),   # 16 groups x 16 slices of 8 rows (64 KiB staged)
    ("attn_proj", 2048, 4096, 8, 128, 0.3, 4096),
    ("decode", 64, 8192, 8, 64, 0.3, 8192),         # one group, 64 slices of one 16 KiB row
    ("attn_proj", 300, 1000, 8, 128, 0.37, 1000),   # groups 128, 128, 44; rows of 2000 bytes
    ("attn_proj", 384, 8192, 8, 128, 0.5, 8200),    # 3 groups: 2 rows per slice, lda > K
    ("attn_proj", 100, 2050, 8, 16, 0.9, 2056),     # 7 groups, ragged last group, kk not a multiple of 8
    ("mlp_down", 200, 136, 8, 32, 0.25, 136),       # short rows, one row per slice
    ("attn_proj", 2048, 5120, 8, 128, 0.5, 5120),   # 80 KiB staged per workgroup (the largest staging)
    ("mlp_down", 512, 1500, 8, 64, 0.6, 1504),      # 2 keys per thread, lda > K
    ("mlp_down", 256, 14336, 8, 128, 0.5, 14336),   # K > 8192: two launches
    ("attn_proj", 4096, 1000, 8, 8, 0.3, 1000),     # 512 groups: two launches
]


@pytest.mark.parametrize("case", SG, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-g{c[4]}-r{c[5]}-ld{c[6]}")
def test_select_gather_equals_select_then_gather(case):
    """rmm_select_gather returns, bit for bit, what rmm_select followed by
    rmm_gather returns (indices with padding, scores, thresholds, bounds,
    panel); the kept sets and the panel are also checked against the oracle.
    Each case runs twice, the second time on a smaller input that reuses the
    output buffers, to catch state left over from a previous call."""
    workload, M, K, N, gr, r, lda = case
    tag = f"select+gather {workload} {M}x{K} gr={gr} r={r} lda={lda}"
    log(f"case {tag}")
    c = make_case(workload, M, K, N, seed=21)
    if lda > K:
        wide = torch.zeros((M, lda), dtype=c["A"].dtype, device=DEV)
        wide[:, :K] = c["A"]
        c["A"] = wide[:, :K]
    kk = rmm.rmm_kk(r, K)
    kpad = rmm.rmm_kk_pad(kk)
    bnorm = rmm.rmm_rownorms(c["B"])
    for MM in (M, max(1, M // 3 + 5)):
        A = c["A"][:MM]
        G = -(-MM // gr)
        outs = []
        for fused in (False, True):
            sc = torch.full((G, K), -1.0, dtype=torch.float32, device=DEV)
            th = torch.full((G,), -1.0, dtype=torch.float32, device=DEV)
            bd = torch.full((G,), -1.0, dtype=torch.float64, device=DEV)
            ix = torch.full((G, kpad), -7, dtype=torch.int32, device=DEV)
            ap = torch.full((MM, kpad), 3.0, dtype=torch.bfloat16, device=DEV)
            if fused:
                rmm.rmm_select_gather(A, r, gr, bnorm=bnorm, idx=ix, Apanel=ap, scores=sc, thresh=th, bound=bd)
            else:
                rmm.rmm_select(A, r, gr, bnorm=bnorm, idx=ix, scores=sc, thresh=th, bound=bd)
                check_index_range(ix, K)
                rmm.rmm_gather(A, ix, kk, gr, Apanel=ap)
            torch.cuda.synchronize()
            outs.append((ix, sc, th, bd, ap))
        for name, a, b in zip(("idx", "scores", "thresh", "bound", "panel"), *outs):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f"{tag} M={MM}: {name}"
        # the kept sets and the panel against the oracle
        A64 = c["A64"][:MM]
        sel = O.select(A64, r, gr, O.rownorms(c["B64"]))
        ig = down(outs[1][0])
        for g in range(G):
            compare_sets(ig[g], sel, g, kk, tag)
        pan = down(outs[1][4])
        A_bits = c["raw"]["A"]
        for m in np.unique(np.linspace(0, MM - 1, 17).astype(int)):
            assert np.array_equal(pan[m, :kk], A_bits[m, ig[m // gr, :kk]]), f"{tag}: panel row {m}"
            assert np.all(pan[m, kk:] == 0), f"{tag}: panel padding row {m}"


# ---------------------------------------------------------------- score and selection as separate calls
@pytest.mark.parametrize("case", [("attn_proj", 300, 1000, 64, 128, 0.37, "cache"),
                                  ("mlp_down", 256, 14336, 64, 128, 0.5, "from_B"),
                                  ("decode", 64, 8192, 64, 64, 0.3, "none"),
                                  ("attn_proj", 4096, 1000, 8, 8, 0.3, "cache")],
                         ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-g{c[4]}-r{c[5]}-{c[6]}")
def test_scores_then_select_scores(case):
    """rmm_scores followed by rmm_select_scores gives, bit for bit, the scores,
    kept indices (with padding), thresholds and bounds of rmm_select, and the
    scores and kept sets of the oracle: B norms cached, computed from B, and
    absent (the activation-only rule); one group per thread block and the
    one-wave-per-group selection (512 groups)."""
    workload, M, K, N, gr, r, norms = case
    tag = f"scores+select {workload} {M}x{K} gr={gr} r={r} {norms}"
    log(f"case {tag}")
    c = make_case(workload, M, K, N, seed=27)
    bnorm = rmm.rmm_rownorms(c["B"]) if norms == "cache" else None
    B = c["B"] if norms == "from_B" else None
    kk = rmm.rmm_kk(r, K)
    G = -(-M // gr)
    outs = []
    for split in (False, True):
        sc = torch.full((G, K), -1.0, dtype=torch.float32, device=DEV)
        th = torch.full((G,), -1.0, dtype=torch.float32, device=DEV)
        bd = torch.full((G,), -1.0, dtype=torch.float64, device=DEV)
        ix = torch.full((G, rmm.rmm_kk_pad(kk)), -7, dtype=torch.int32, device=DEV)
        if split:
            rmm.rmm_scores(c["A"], gr, bnorm=bnorm, B=B, scores=sc)
            rmm.rmm_select_scores(sc, r, idx=ix, thresh=th, bound=bd)
        else:
            rmm.rmm_select(c["A"], r, gr, bnorm=bnorm, B=B, idx=ix, scores=sc, thresh=th, bound=bd)
        torch.cuda.synchronize()
        outs.append((sc, ix, th, bd))
    for name, a, b in zip(("scores", "idx", "thresh", "bound"), *outs):
        assert torch.equal(a, b), f"{tag}: {name} differs from rmm_select"
    b64 = None if norms == "none" else O.rownorms(c["B64"])
    sel = O.select(c["A64"], r, gr, b64)
    assert np.array_equal(down(outs[1][0]), sel["s32"]), f"{tag}: scores differ from the oracle"
    ig = down(outs[1][1])
    for g in range(G):
        compare_sets(ig[g], sel, g, kk, tag)
    assert np.array_equal(down(outs[1][2]), sel["thresh"]), f"{tag}: thresholds differ from the oracle"


# ---------------------------------------------------------------- two workgroups per CU
WT = [
    # (M, K, N, group_rows, r): at least 512 tiles of 128 x 256, so bf16
    # outputs take the two-workgroups-per-CU kernel
    (4046, 1000, 4104, 128, 0.37),   # 32 groups, the last of 78 rows; N tail of 8; kk = 370
    (4046, 1000, 4104, 128, 1.0),    # the dense product, A and B in place
    (2048, 520, 8192, 256, 0.5),     # two row tiles per group; kk = 260 (ragged last slab)
    (4096, 40, 4096, 128, 0.5),      # kk = 20: one partial slab, no main loop
    (4096, 200, 4096, 128, 0.004),   # kk = 1
    (4096, 1096, 4096, 128, 0.61),   # kk = 669: three index chunks, an odd slab count (21)
]


@pytest.mark.parametrize("case", WT, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}-g{c[3]}-r{c[4]}")
def test_two_per_cu_gemm(case):
    """The prefill shapes with at least two tiles per CU: every output element
    against the oracle, and the bf16 output equal to the round-to-nearest-even
    bf16 of the binary32 output (which runs the eight-wave kernel, with the
    same accumulation order)."""
    M, K, N, gr, r = case
    tag = f"two-per-CU {M}x{K}x{N} gr={gr} r={r}"
    log(f"case {tag}")
    G = -(-M // gr)
    assert G * -(-min(gr, M) // 128) * -(-N // 256) >= 512
    c = make_case("mlp_down", M, K, N, seed=33)
    bnorm = rmm.rmm_rownorms(c["B"])
    if r < 1.0:
        idx, scores, thresh, bound, Ap, Y = run_chain(c, r, gr, bnorm)
        sel, ig = check_selection(c, r, gr, bnorm, idx, scores, thresh, bound, tag)
        kk = sel["kk"]
        Y32 = rmm.rmm_gemm(Ap, c["B"], idx, kk, gr, ydt=torch.float32)
    else:
        kk = K
        Y = rmm.rmm_gemm(c["A"], c["B"], None, K, gr)
        Y32 = rmm.rmm_gemm(c["A"], c["B"], None, K, gr, ydt=torch.float32)
        ig = np.arange(K, dtype=np.int32)[None, :].repeat(G, 0)
    torch.cuda.synchronize()
    assert np.array_equal(down(Y), synth.f32_to_bf16_bits(down(Y32))), f"{tag}: bf16 output is not RNE(fp32 output)"
    Yref, Sabs = oracle_rows(c["A64"], c["B64"], ig, kk, gr, np.arange(M))
    check_output(widen(Y), Yref, Sabs, kk, tag)


def test_two_per_cu_far_rows():
    """Kept B rows more than 2^32 bytes past B's start (a 2 MiB row stride, so
    rows from 2048 on): their 32-bit offsets do not hold, and the waves that
    meet them recompute their part with 64-bit addresses.  The output equals,
    bit for bit, that of the same product over a compact copy of B (the fast
    path), and every output element matches the oracle."""
    M, K, N, gr, r = 4096, 2304, 4096, 128, 0.5
    ldb = 1 << 20
    tag = f"far rows {M}x{K}x{N} ldb={ldb} r={r}"
    log(f"case {tag}")
    c = make_case("mlp_down", M, K, N, seed=35)
    bnorm = rmm.rmm_rownorms(c["B"])
    idx, scores, thresh, bound, Ap, Y = run_chain(c, r, gr, bnorm)
    kk = rmm.rmm_kk(r, K)
    far = ((1 << 32) - 1 - 2 * N) // (2 * ldb)
    assert int(idx[:, :kk].max()) > far, "no kept row past the 32-bit offsets"
    Bbig = torch.empty((K, ldb), dtype=torch.bfloat16, device=DEV)   # 4.8 GB, first N columns used
    Bbig[:, :N] = c["B"]
    Yfar = rmm.rmm_gemm(Ap, Bbig[:, :N], idx, kk, gr)
    torch.cuda.synchronize()
    assert torch.equal(Yfar, Y), f"{tag}: output differs from the compact-B product"
    del Bbig
    ig = down(idx)[:, :kk]
    Yref, Sabs = oracle_rows(c["A64"], c["B64"], ig, kk, gr, np.arange(M))
    check_output(widen(Yfar), Yref, Sabs, kk, tag + f" (all {M} rows)")
