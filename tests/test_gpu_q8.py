"""GPU parity of the int8-weight path against the oracle, through the C ABI:
the quantiser (codes and scales), the row norms of the dequantised weight,
and the score -> select -> gather -> reduced int8 GEMM chain.

Codes, scales and row norms must be bit-exact: both sides divide in binary32
with correct rounding and round half to even; the norms add the same exact
terms in the same order with the same binary64 roundings.  Kept sets follow
the rules of the bf16 path.  Outputs are compared with the oracle's reduced
product on the dequantised weight (exact in binary64) within the bound of
tests/gpu_util.py: each product of a bf16 activation and a code is exact in
fp32, the sum is accumulated in fp32 and the scale multiplies it once.

Method: "Reduced Matrix Multiplication (RMM) para Inferencia de LLM"
(gist.science), Resultados Experimentais > Compatibilidade (INT8 weights).
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, check_output, compare_sets, down, log, oracle_rows, up_bf16, widen
from input_adaptive_reduced_02_amd import rmm, synth

pytestmark = pytest.mark.gpu


def weight_bits(K, N, seed):
    """bf16 weight bits: N(0, 0.02) times lognormal column scales, with an
    all-zero column, a column whose scale is exactly 2^-4 and whose B/s are
    exact halves (ties), and a column whose absmax is negative."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((K, N)) * 0.02 * rng.lognormal(0, 1, N)[None, :]).astype(np.float32)
    if N > 3:
        w[:, 1] = 0.0
        j = (np.arange(K) % 201) - 100
        w[:, 2] = (2 * j + 1) * 2.0 ** -5          # (j + 0.5) * 2^-4: bf16-exact halves
        w[0, 2] = 127 * 2.0 ** -4
        w[K // 2, 3] = -4.0 * np.abs(w[:, 3]).max() - 0.5
    return synth.f32_to_bf16_bits(w)


def quantize_both(bits):
    B = up_bf16(bits)
    Bq, s = rmm.rmm_quantize_q8(B)
    torch.cuda.synchronize()
    q_ref, s_ref = O.quantize_q8(synth.bf16_bits_to_f32(bits))
    return B, Bq, s, q_ref, s_ref


@pytest.mark.parametrize("shape", [(300, 272), (64, 16), (1, 32), (1000, 4096)], ids=str)
def test_quantize(shape):
    K, N = shape
    log(f"quantize {K}x{N}")
    _, Bq, s, q_ref, s_ref = quantize_both(weight_bits(K, N, seed=K + N))
    assert np.array_equal(down(s).view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    qg = down(Bq)
    bad = np.argwhere(qg != q_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: {qg[tuple(bad[0])]} vs {q_ref[tuple(bad[0])]}"


@pytest.mark.parametrize("shape", [(300, 272), (1000, 4096)], ids=str)
def test_rownorms(shape):
    K, N = shape
    log(f"rownorms_q8 {K}x{N}")
    _, Bq, s, q_ref, s_ref = quantize_both(weight_bits(K, N, seed=7))
    b = rmm.rmm_rownorms_q8(Bq, s)
    torch.cuda.synchronize()
    assert np.array_equal(down(b), O.rownorms_q8(q_ref, s_ref))


def run_chain_q8(A, Bq, s, bnorm, r, gr):
    M, K = A.shape
    kk = rmm.rmm_kk(r, K)
    G = -(-M // gr)
    if kk == K:
        Y = rmm.rmm_gemm_q8(A, Bq, s, None, K, gr)
        torch.cuda.synchronize()
        return None, None, Y
    scores = torch.empty((G, K), dtype=torch.float32, device=DEV)
    idx = torch.zeros((G, rmm.rmm_kk_pad(kk)), dtype=torch.int32, device=DEV)
    rmm.rmm_select(A, r, gr, bnorm=bnorm, idx=idx, scores=scores)
    torch.cuda.synchronize()
    ig = down(idx)
    assert ig.min() >= 0 and ig.max() < K, "kept index out of range"
    Ap, _ = rmm.rmm_gather(A, idx, kk, gr)
    Y = rmm.rmm_gemm_q8(Ap, Bq, s, idx, kk, gr)
    torch.cuda.synchronize()
    return idx, scores, Y


def check_chain(A64, Bd, b_ref, idx, scores, Y, r, gr, tag, rows=None):
    M, K = A64.shape
    kk = O.kk(r, K)
    G = -(-M // gr)
    if idx is None:
        ig = np.arange(K, dtype=np.int32)[None, :].repeat(G, 0)
    else:
        sel = O.select(A64, r, gr, b_ref)
        assert np.array_equal(down(scores), sel["s32"]), f"{tag}: scores differ"
        ig = down(idx)
        for g in range(G):
            compare_sets(ig[g], sel, g, kk, tag)
    rows = np.arange(M) if rows is None else rows
    Yref, Sabs = oracle_rows(A64, Bd, ig, kk, gr, rows)
    check_output(widen(Y)[rows], Yref, Sabs, kk, tag)


SMALL = [
    # (M, K, N, group_rows, r); groups of at most 64 rows keeping at most 4096
    # rows run the shared-stream kernel (q8s), the others the split-tile one
    (64, 4096, 1024, 64, 0.3),       # q8s, decode-like: one group, kk = 1229
    (300, 1000, 272, 128, 0.5),      # split: groups 128,128,44 (3 row tiles each); N tail 16
    (200, 520, 80, 128, 0.37),       # split: kk = 193, N = 80 (one partial column tile)
    (96, 136, 48, 32, 0.9),          # q8s: groups of 32 rows (half-empty row tiles), kk = 123
    (128, 512, 256, 64, 1.0),        # q8s: the dense product, no index list, also binary32 out
    (256, 384, 272, 128, 1.0),       # split: the dense product, also binary32 out
    (64, 8, 16, 64, 0.1),            # q8s: kk = 1
    (16, 96, 32, 1, 0.25),           # q8s: one-row groups
    (130, 704, 400, 64, 0.6),        # q8s: ragged last group (2 rows), N = 400 (partial tile)
    (64, 8320, 272, 64, 0.5),        # split: kk = 4160, just past the q8s limit
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}-g{c[3]}-r{c[4]}")
def test_chain_small(case):
    M, K, N, gr, r = case
    tag = f"q8 chain {M}x{K}x{N} gr={gr} r={r}"
    log(f"case {tag}")
    d = synth.linear_inputs("decode", M, K, N, seed=3)
    A = up_bf16(d["A"])
    A64 = O.widen_bf16(d["A"])
    _, Bq, s, q_ref, s_ref = quantize_both(weight_bits(K, N, seed=M + K))
    assert np.array_equal(down(Bq), q_ref) and np.array_equal(down(s), s_ref)
    bnorm = rmm.rmm_rownorms_q8(Bq, s)
    b_ref = O.rownorms_q8(q_ref, s_ref)
    idx, scores, Y = run_chain_q8(A, Bq, s, bnorm, r, gr)
    check_chain(A64, O.dequant_q8(q_ref, s_ref), b_ref, idx, scores, Y, r, gr, tag)
    if r == 1.0:   # binary32 output of the same kernel
        Yf = rmm.rmm_gemm_q8(A, Bq, s, None, K, gr, ydt=torch.float32)
        torch.cuda.synchronize()
        check_chain(A64, O.dequant_q8(q_ref, s_ref), b_ref, None, None, Yf, r, gr, tag + " f32 out")


def test_determinism():
    d = synth.linear_inputs("decode", 64, 2048, 512, seed=4)
    A = up_bf16(d["A"])
    Bq, s = rmm.rmm_quantize_q8(up_bf16(weight_bits(2048, 512, seed=1)))
    bn = rmm.rmm_rownorms_q8(Bq, s)
    outs = [down(run_chain_q8(A, Bq, s, bn, 0.5, 64)[2]) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


# ---------------------------------------------------------------- full size
@pytest.fixture(scope="module")
def decode_q8():
    M, K, N = synth.FULL_SHAPES["decode"]
    d = synth.linear_inputs("decode", M, K, N)
    A = up_bf16(d["A"])
    Bq, s = rmm.rmm_quantize_q8(up_bf16(d["B"]))
    bnorm = rmm.rmm_rownorms_q8(Bq, s)
    torch.cuda.synchronize()
    q = down(Bq)
    sg = down(s)
    c = dict(A=A, A64=O.widen_bf16(d["A"]), Bq=Bq, s=s, bnorm=bnorm, q=q, sg=sg, Bbits=d["B"])
    yield c
    c.clear()


def test_full_decode_quantiser(decode_q8):
    """Decode weight 8192 x 28672: scales and codes of sampled columns (the
    quantisation is per column), row norms of sampled rows, bit-exact."""
    c = decode_q8
    K, N = c["q"].shape
    rng = np.random.default_rng(2)
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 62)]))
    w = synth.bf16_bits_to_f32(c["Bbits"][:, cols])
    q_ref, s_ref = O.quantize_q8(w)
    assert np.array_equal(c["sg"][cols].view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(c["q"][:, cols], q_ref)
    rows = np.unique(np.concatenate([[0, K - 1], rng.integers(0, K, 30)]))
    assert np.array_equal(down(c["bnorm"])[rows], O.rownorms_q8(c["q"][rows], c["sg"]))


@pytest.mark.parametrize("r", [0.3, 0.5, 0.7, 1.0])
def test_full_decode_chain(decode_q8, r):
    """Decode shape in the benchmark's launch configuration: the group's scores
    and kept set exact; every output row element by element."""
    c = decode_q8
    M, K = c["A64"].shape
    tag = f"q8 decode {M}x{K}x{c['q'].shape[1]} r={r}"
    log(f"full {tag}")
    b_ref = O.rownorms_q8(c["q"], c["sg"])
    assert np.array_equal(down(c["bnorm"]), b_ref)
    idx, scores, Y = run_chain_q8(c["A"], c["Bq"], c["s"], c["bnorm"], r, 64)
    check_chain(c["A64"], O.dequant_q8(c["q"], c["sg"]), b_ref, idx, scores, Y, r, 64, tag)


def test_workspace_reuse_and_graph_replay():
    """One zero-filled workspace serves consecutive calls of different sizes,
    and the chain captured in a HIP graph gives the eager result on every
    replay (eager work and synchronisations between the replays).  K = 8192:
    r = 0.7 and 1 keep more than 4096 rows, so they run the split tiles that
    meet through the workspace; r = 0.3 runs the shared-stream kernel."""
    M, K, N, gr = 64, 8192, 4096, 64
    d = synth.linear_inputs("decode", M, K, N, seed=8)
    A = up_bf16(d["A"])
    Bq, s = rmm.rmm_quantize_q8(up_bf16(weight_bits(K, N, seed=3)))
    bn = rmm.rmm_rownorms_q8(Bq, s)
    need = max(rmm.rmm_gemm_q8_workspace_bytes(M, N, rmm.rmm_kk(r, K), gr) for r in (0.3, 0.7, 1.0))
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    ref = {}
    for r in (0.7, 0.3, 1.0, 0.7):
        kk = rmm.rmm_kk(r, K)
        idx = rmm.rmm_select(A, r, gr, bnorm=bn) if r < 1 else None
        Ap = rmm.rmm_gather(A, idx, kk, gr)[0] if r < 1 else A
        Yw = rmm.rmm_gemm_q8(Ap, Bq, s, idx, kk, gr, ws=ws)
        Yf = rmm.rmm_gemm_q8(Ap, Bq, s, idx, kk, gr)   # fresh zero-filled workspace
        torch.cuda.synchronize()
        assert np.array_equal(down(Yw), down(Yf)), f"reused workspace differs at r={r}"
        ref[r] = down(Yf)
    # graph: select -> gather -> GEMM at r = 0.7 (split tiles) on fixed buffers
    r, kk = 0.7, rmm.rmm_kk(0.7, K)
    idx = torch.zeros((1, rmm.rmm_kk_pad(kk)), dtype=torch.int32, device=DEV)
    Ap = torch.empty((M, rmm.rmm_kk_pad(kk)), dtype=torch.bfloat16, device=DEV)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    sws = torch.empty(max(1, rmm.rmm_select_workspace_bytes(M, K, gr)), dtype=torch.uint8, device=DEV)

    def step():
        rmm.rmm_select(A, r, gr, bnorm=bn, idx=idx, ws=sws)
        rmm.rmm_gather(A, idx, kk, gr, Apanel=Ap)
        rmm.rmm_gemm_q8(Ap, Bq, s, idx, kk, gr, Y=Y, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        Y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(down(Y), ref[0.7]), f"graph replay {rep} differs"
        step()   # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(down(Y), ref[0.7])


def test_workspace_reuse_across_shapes():
    """One workspace, zero-filled once and sized for the largest shape, serves
    calls with different tile counts in any order (the arrival counters sit at
    the start of the workspace and are back at zero after every call, the
    partial sums at its end): each result equals the one from a fresh
    zero-filled workspace.  K = 10240: kk = 5120 at r = 0.5, past the
    shared-stream kernel's 4096, so every call runs split tiles."""
    M, K, gr = 64, 10240, 64
    d = synth.linear_inputs("decode", M, K, 4096, seed=12)
    A = up_bf16(d["A"])
    shapes = [4096, 2048, 4096, 1024, 2048]
    Bs = {}
    for N in set(shapes):
        Bq, s = rmm.rmm_quantize_q8(up_bf16(weight_bits(K, N, seed=N)))
        Bs[N] = (Bq, s, rmm.rmm_rownorms_q8(Bq, s))
    r = 0.5
    kk = rmm.rmm_kk(r, K)
    need = max(rmm.rmm_gemm_q8_workspace_bytes(M, N, kk, gr) for N in shapes)
    assert need > 0 and len({rmm.rmm_gemm_q8_workspace_bytes(M, N, kk, gr) for N in shapes}) > 1
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for N in shapes:
        Bq, s, bn = Bs[N]
        idx = rmm.rmm_select(A, r, gr, bnorm=bn)
        Ap = rmm.rmm_gather(A, idx, kk, gr)[0]
        Yw = rmm.rmm_gemm_q8(Ap, Bq, s, idx, kk, gr, ws=ws)
        Yf = rmm.rmm_gemm_q8(Ap, Bq, s, idx, kk, gr)   # fresh zero-filled workspace
        torch.cuda.synchronize()
        assert np.array_equal(down(Yw), down(Yf)), f"reused workspace differs at N={N}"
