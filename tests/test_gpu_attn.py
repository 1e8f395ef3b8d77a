"""GPU parity of the attention producer against the oracle, through the C ABI:
the QK^T feature reduction (feature scores and kept features per 128-query
block), the attention probabilities over the kept features stored key-major,
and the P.V key scores the producer forms from its own stored probabilities.

Inputs: Q, K, V bf16 N(0,1) [H, L, D = 128] (synth.pv_qkv).

Bars:
  - feature scores and P.V key scores within one binary32 ulp of the
    oracle's (the P.V scores against the oracle evaluated on the
    probabilities the GPU stored): the GPU sums in binary64 in a fixed order
    of its own (partial sums added pairwise), the oracle in ascending order,
    and the two binary64 sums differ by about n 2^-53 relative;
  - kept feature and key sets identical where the two sides' keys are
    bit-identical; elsewhere the GPU's set is the kk best of its own keys and
    differs from the oracle's only inside the near-tie band;
  - probabilities within the bound derived from the arithmetic, per element:
      |P_gpu - P_ref| <= 1.01 [ (2^-8 + e) P_ref ] + 2^-126
    2^-8: rounding to bf16; e: relative error of the binary32 value before
    it, from the logit (fp32 sum of kk exact products:
    kk 2^-24 sum_j |q_j k_j|, times log2(e)/sqrt(128) and ln 2), the row
    statistics (at most L + 64 fp32 additions: (L + 64) 2^-24) and exp2/log2
    (2^-20); 2^-126: exp2 results below the binary32 normal range may flush
    to zero;
  - entries past a block's candidate keys left untouched.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, check_output, compare_scores_ulp, compare_sets_keys, down, log, up_bf16
from input_adaptive_reduced_02_amd import rmm, synth

pytestmark = pytest.mark.gpu

QB = 128
D = 128
SENTINEL = 0x7FC1          # a NaN bf16 pattern the producer never writes


def make_qkv(H, L, seed):
    q, k, v = synth.pv_qkv(H, L, D, seed=seed)
    return q, k, v, up_bf16(q), up_bf16(k), up_bf16(v)


def run_producer(Qd, Kd, Vd, r_qk, causal, use_k=True, pv=True):
    """(idx_qk, qk_scores, Pt, pv_scores) from the GPU."""
    H, L, _ = Qd.shape
    G = -(-L // QB)
    idx = None
    qs = None
    if r_qk < 1.0:
        qs = torch.zeros((H, G, D), dtype=torch.float32, device=DEV)
        idx = rmm.rmm_qk_select(Qd, Kd, r_qk, QB, causal, use_k, scores_out=qs)
    Pt = torch.full((H, L, L), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    pvs = torch.zeros((H, G, L), dtype=torch.float32, device=DEV) if pv else None
    rmm.rmm_attn_probs(Qd, Kd, idx, r_qk, QB, causal, Pt=Pt, V=Vd if pv else None, pv_scores=pvs)
    torch.cuda.synchronize()
    return idx, qs, Pt, pvs


def prob_bound(Pref, Qh, Kh, rows, Kg, kept, L):
    """Per-element bound of the module docstring for one block's rows."""
    kk = len(kept)
    A = np.abs(Qh[rows][:, kept]) @ np.abs(Kh[:Kg][:, kept]).T
    e = (kk * 2.0 ** -24 * A) * (math.log2(math.e) / math.sqrt(D)) * math.log(2.0) \
        + (L + 64) * 2.0 ** -24 + 2.0 ** -20
    return 1.01 * (2.0 ** -8 + e) * Pref + 2.0 ** -126


def check_block(q, k, v, idx_np, qs_np, Pt_np, pvs_np, h, g, L, r_qk, causal, use_k, tag,
                check_probs=True):
    """One (head, block): feature scores and kept set, probabilities, P.V scores."""
    Qh, Kh = O.widen_bf16(q[h]), O.widen_bf16(k[h])
    q0 = g * QB
    nq = min(QB, L - q0)
    Kg = O.pv_prefix(L, QB, g, causal)
    kept = None
    if r_qk < 1.0:
        sel = O.qk_select_block(Qh, Kh, QB, g, r_qk, causal, use_k)
        compare_scores_ulp(qs_np[h, g], sel["s32"], f"{tag} h={h} g={g} feature scores")
        kk = sel["kk"]
        compare_sets_keys(idx_np[h * (-(-L // QB)) + g, :kk], qs_np[h, g], sel["idx"], sel["s32"], sel["near"], kk,
                          f"{tag} h={h} g={g} features")
        kept = idx_np[h * (-(-L // QB)) + g, :kk].astype(np.int32)
    feats = np.arange(D, dtype=np.int32) if kept is None else kept
    out = {}
    if check_probs:
        Pref = O.attn_probs(Qh, Kh, q0, nq, causal, kept)[:, :Kg]
        Pg = O.widen_bf16(np.ascontiguousarray(Pt_np[h, :Kg, q0:q0 + nq].T))
        bnd = prob_bound(Pref, Qh, Kh, np.arange(q0, q0 + nq), Kg, feats, L)
        err = np.abs(Pg - Pref)
        bad = err > bnd
        exact = np.mean(Pg == O.widen_bf16(synth.f32_to_bf16_bits(Pref.astype(np.float32))))
        out["exact"] = exact
        assert not bad.any(), f"{tag} h={h} g={g}: {bad.sum()} probabilities outside the bound, first {np.argwhere(bad)[0]}"
        if causal:
            ql = np.arange(nq)[:, None] + q0
            kl = np.arange(Kg)[None, :]
            assert np.all(Pg[kl > ql] == 0.0), f"{tag} h={h} g={g}: masked entries not zero"
        # past the candidates: untouched
        assert np.all(Pt_np[h, Kg:, q0:q0 + nq] == SENTINEL), f"{tag} h={h} g={g}: wrote past K_g"
    if pvs_np is not None:
        Ptb = O.widen_bf16(Pt_np[h, :Kg, q0:q0 + nq])
        _, s32 = O.pv_scores(Ptb, O.widen_bf16(v[h])[:Kg])
        compare_scores_ulp(pvs_np[h, g, :Kg], s32, f"{tag} h={h} g={g} P.V scores")
    return out


@pytest.mark.parametrize("H,L,causal", [(2, 384, True), (2, 328, True), (1, 256, False), (2, 200, False)])
@pytest.mark.parametrize("r_qk", [0.3, 0.5, 1.0])
def test_producer_small(H, L, causal, r_qk):
    tag = f"attn H={H} L={L} causal={causal} r_qk={r_qk}"
    log(tag)
    q, k, v, Qd, Kd, Vd = make_qkv(H, L, seed=3)
    idx, qs, Pt, pvs = run_producer(Qd, Kd, Vd, r_qk, causal)
    idx_np = down(idx) if idx is not None else None
    qs_np = down(qs) if qs is not None else None
    Pt_np, pvs_np = down(Pt), down(pvs)
    G = -(-L // QB)
    ex = []
    for h in range(H):
        for g in range(G):
            ex.append(check_block(q, k, v, idx_np, qs_np, Pt_np, pvs_np, h, g, L, r_qk, causal, True, tag)["exact"])
    log(f"  {tag}: P equal to the rounded exact value: {np.mean(ex):.5f}")
    assert np.mean(ex) >= 0.95


def test_activation_only_features():
    """use_k = 0: the pages' rule, feature scores from the queries alone."""
    H, L = 2, 256
    q, k, v, Qd, Kd, Vd = make_qkv(H, L, seed=4)
    idx, qs, Pt, pvs = run_producer(Qd, Kd, Vd, 0.5, True, use_k=False, pv=False)
    idx_np, qs_np, Pt_np = down(idx), down(qs), down(Pt)
    for h in range(H):
        for g in range(2):
            check_block(q, k, v, idx_np, qs_np, Pt_np, None, h, g, L, 0.5, True, False, "aonly")


def test_all_features_list_equals_dense():
    """A feature list holding every feature gives the dense probabilities bit
    for bit (the same products in the same order)."""
    H, L = 2, 264
    q, k, v, Qd, Kd, Vd = make_qkv(H, L, seed=5)
    G = -(-L // QB)
    allf = torch.arange(D, dtype=torch.int32, device=DEV).repeat(H * G, 1).contiguous()
    P1 = rmm.rmm_attn_probs(Qd, Kd, None, 1.0, QB, True)
    P2 = rmm.rmm_attn_probs(Qd, Kd, allf, 1.0, QB, True)
    torch.cuda.synchronize()
    for h in range(H):
        for g in range(G):
            Kg = O.pv_prefix(L, QB, g, True)
            a = down(P1)[h, :Kg, g * QB:g * QB + min(QB, L - g * QB)]
            b = down(P2)[h, :Kg, g * QB:g * QB + min(QB, L - g * QB)]
            assert np.array_equal(a, b)


def test_deterministic():
    H, L = 2, 384
    q, k, v, Qd, Kd, Vd = make_qkv(H, L, seed=6)
    a = run_producer(Qd, Kd, Vd, 0.5, True)
    b = run_producer(Qd, Kd, Vd, 0.5, True)
    kpad = rmm.rmm_kk_pad(rmm.rmm_kk(0.5, D))       # the written part of the feature lists
    assert torch.equal(a[0][:, :kpad], b[0][:, :kpad])
    for x, y in zip(a[1:], b[1:]):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16),
                           y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16))


def test_chain_small():
    """qk select -> probabilities with P.V scores -> key select -> reduced P.V:
    kept keys from the producer's scores equal the oracle's on the stored P,
    and the output matches the oracle's product over them."""
    H, L = 2, 384
    q, k, v, Qd, Kd, Vd = make_qkv(H, L, seed=7)
    idx, qs, Pt, pvs = run_producer(Qd, Kd, Vd, 0.5, True)
    G = -(-L // QB)
    # the producer's key scores and the P.V path's block scores over the same
    # stored P sum in the same order: equal bit for bit on every candidate key
    sc2 = torch.zeros((H, G, L), dtype=torch.float32, device=DEV)
    rmm.rmm_pv_select(Pt, Vd, 0.5, QB, True, scores_out=sc2)
    torch.cuda.synchronize()
    a, b = down(pvs), down(sc2)
    for g in range(G):
        Kg = O.pv_prefix(L, QB, g, True)
        assert np.array_equal(a[:, g, :Kg].view(np.uint32), b[:, g, :Kg].view(np.uint32)), f"block {g}"
    for r in (0.3, 0.5):
        kidx = rmm.rmm_pv_select_scores(pvs, r, QB, True)
        O_ = rmm.rmm_pv_gemm(Pt, Vd, r, kidx, QB, True)
        torch.cuda.synchronize()
        Pt_np, kidx_np, O_np, pvs_np = down(Pt), down(kidx), down(O_), down(pvs)
        for h in range(H):
            Vh = O.widen_bf16(v[h])
            for g in range(G):
                q0 = g * QB
                nq = min(QB, L - q0)
                Kg = O.pv_prefix(L, QB, g, True)
                Ptb = O.widen_bf16(Pt_np[h, :Kg, q0:q0 + nq])
                s64, s32 = O.pv_scores(Ptb, Vh[:Kg])
                compare_scores_ulp(pvs_np[h, g, :Kg], s32, f"chain r={r} h={h} g={g} P.V scores")
                kk = O.kk(r, Kg)
                ref = O.topk(s32, kk)
                compare_sets_keys(kidx_np[h * G + g, :kk], pvs_np[h, g, :Kg], ref, s32, O.near_ties(s64, s32, ref),
                                  kk, f"chain r={r} h={h} g={g} keys")
                kept = kidx_np[h * G + g, :kk].astype(np.int32)
                Ob = O.pv_block(Ptb, Vh[:Kg], kept)
                Sb = O.pv_block(np.abs(Ptb), np.abs(Vh[:Kg]), kept)
                check_output(O.widen_bf16(O_np[h, q0:q0 + nq]), Ob, Sb, kk, f"chain r={r} h={h} g={g}")


def test_full_size_sampled():
    """32 heads, L = 4096, r_qk = 0.5: every block's feature scores and kept
    features; probabilities and P.V scores of sampled blocks of heads 0 and 31."""
    H, L = 32, 4096
    log("attn full size H=32 L=4096 r_qk=0.5")
    q, k, v, Qd, Kd, Vd = make_qkv(H, L, seed=0)
    idx, qs, Pt, pvs = run_producer(Qd, Kd, Vd, 0.5, True)
    idx_np, qs_np, pvs_np = down(idx), down(qs), down(pvs)
    G = L // QB
    for h in range(H):
        Qh, Kh = O.widen_bf16(q[h]), O.widen_bf16(k[h])
        for g in range(G):
            sel = O.qk_select_block(Qh, Kh, QB, g, 0.5, True, True)
            compare_scores_ulp(qs_np[h, g], sel["s32"], f"full h={h} g={g} feature scores")
            compare_sets_keys(idx_np[h * G + g, :64], qs_np[h, g], sel["idx"], sel["s32"], sel["near"], 64,
                              f"full h={h} g={g} features")
    for h in (0, 31):
        Pt_h = down(Pt[h])
        Pt_np = Pt_h[None]
        for g in (0, 1, 15, 31):
            log(f"  full h={h} g={g}")
            check_block(q[h:h + 1], k[h:h + 1], v[h:h + 1], idx_np[h * G:(h + 1) * G], qs_np[h:h + 1], Pt_np,
                        pvs_np[h:h + 1], 0, g, L, 0.5, True, True, f"full h={h}")


def test_peaked_rows_key_sums():
    """Queries scaled up make peaked rows whose probabilities span many
    binary orders, down to underflow: the P.V key scores must still equal the
    oracle's ascending binary64 sums on the stored P, and P stays within its
    bound."""
    H, L = 2, 384
    q, k, v = synth.pv_qkv(H, L, D, seed=8)
    qf = synth.bf16_bits_to_f32(q)
    qf[:, 100:300] *= 9.0                      # logits with std ~9: P spans ~e^-60
    q = synth.f32_to_bf16_bits(qf)
    Qd, Kd, Vd = up_bf16(q), up_bf16(k), up_bf16(v)
    idx, qs, Pt, pvs = run_producer(Qd, Kd, Vd, 0.5, True)
    idx_np, qs_np, Pt_np, pvs_np = down(idx), down(qs), down(Pt), down(pvs)
    tiny = np.count_nonzero((Pt_np & 0x7FFF) > 0) - np.count_nonzero((Pt_np & 0x7FFF) >= (88 << 7))
    log(f"  peaked: {tiny} stored probabilities below 2^-39")
    for h in range(H):
        for g in range(3):
            check_block(q, k, v, idx_np, qs_np, Pt_np, pvs_np, h, g, L, 0.5, True, True, "peaked")


def test_long_sequence_sampled():
    """32 heads, L = 16384 (the longer P.V configuration), r = 0.5: feature
    scores and kept features of sampled blocks of heads 0 and 31, their
    probabilities and P.V key scores, and the kept keys from those scores."""
    H, L = 32, 16384
    log("attn long H=32 L=16384 r=0.5")
    q, k, v, Qd, Kd, Vd = make_qkv(H, L, seed=2)
    G = L // QB
    qs = torch.zeros((H, G, D), dtype=torch.float32, device=DEV)
    idx = rmm.rmm_qk_select(Qd, Kd, 0.5, QB, True, True, scores_out=qs)
    Pt = torch.full((H, L, L), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    pvs = torch.zeros((H, G, L), dtype=torch.float32, device=DEV)
    rmm.rmm_attn_probs(Qd, Kd, idx, 0.5, QB, True, Pt=Pt, V=Vd, pv_scores=pvs)
    kidx = rmm.rmm_pv_select_scores(pvs, 0.5, QB, True)
    torch.cuda.synchronize()
    idx_np, qs_np, pvs_np, kidx_np = down(idx), down(qs), down(pvs), down(kidx)
    for h in (0, 31):
        Pt_np = down(Pt[h])[None]
        for g in (0, 77, G - 1):
            log(f"  long h={h} g={g}")
            check_block(q[h:h + 1], k[h:h + 1], v[h:h + 1], idx_np[h * G:(h + 1) * G], qs_np[h:h + 1], Pt_np,
                        pvs_np[h:h + 1], 0, g, L, 0.5, True, True, f"long h={h}")
            Kg = O.pv_prefix(L, QB, g, True)
            kk = O.kk(0.5, Kg)
            Ptb = O.widen_bf16(Pt_np[0, :Kg, g * QB:(g + 1) * QB])
            s64, s32 = O.pv_scores(Ptb, O.widen_bf16(v[h])[:Kg])
            ref = O.topk(s32, kk)
            compare_sets_keys(kidx_np[h * G + g, :kk], pvs_np[h, g, :Kg], ref, s32, O.near_ties(s64, s32, ref), kk,
                              f"long keys h={h} g={g}")
        del Pt_np


@pytest.mark.parametrize("H,L,causal,r_qk", [(1, 8, True, 0.5), (1, 8, False, 0.001), (2, 136, True, 0.001),
                                             (1, 136, False, 1.0), (3, 64, True, 0.3)])
def test_edge_shapes(H, L, causal, r_qk):
    """Tiny and ragged sequences (one block of 8 queries; a last block of 8),
    a single kept feature (r small enough that kk = 1), several heads."""
    tag = f"edge H={H} L={L} causal={causal} r_qk={r_qk}"
    log(tag)
    q, k, v, Qd, Kd, Vd = make_qkv(H, L, seed=9)
    idx, qs, Pt, pvs = run_producer(Qd, Kd, Vd, r_qk, causal)
    idx_np = down(idx) if idx is not None else None
    qs_np = down(qs) if qs is not None else None
    Pt_np, pvs_np = down(Pt), down(pvs)
    for h in range(H):
        for g in range(-(-L // QB)):
            check_block(q, k, v, idx_np, qs_np, Pt_np, pvs_np, h, g, L, r_qk, causal, True, tag)


def test_graph_replay():
    """The whole attention chain (feature select, producer with key scores,
    key select, reduced P.V) captured in a HIP graph gives the eager result
    on every replay, with eager work and synchronisations between replays."""
    H, L, r = 2, 384, 0.5
    q, k, v, Qd, Kd, Vd = make_qkv(H, L, seed=10)
    G = L // QB
    fidx = torch.zeros((H * G, rmm.rmm_kk_pad(D)), dtype=torch.int32, device=DEV)
    qs = torch.zeros((H, G, D), dtype=torch.float32, device=DEV)
    Pt = torch.zeros((H, L, L), dtype=torch.bfloat16, device=DEV)
    pvs = torch.zeros((H, G, L), dtype=torch.float32, device=DEV)
    kidx = torch.zeros((H * G, rmm.rmm_kk_pad(L)), dtype=torch.int32, device=DEV)
    O_ = torch.zeros((H, L, D), dtype=torch.bfloat16, device=DEV)
    wsp = torch.empty(max(1, int(rmm.lib().rmm_attn_probs_workspace_bytes(H, L, D, 1))), dtype=torch.uint8,
                      device=DEV)

    def step():
        rmm.rmm_qk_select(Qd, Kd, r, QB, True, True, idx_out=fidx, scores_out=qs)
        rmm.rmm_attn_probs(Qd, Kd, fidx, r, QB, True, Pt=Pt, V=Vd, pv_scores=pvs, ws=wsp)
        rmm.rmm_pv_select_scores(pvs, r, QB, True, idx_out=kidx)
        rmm.rmm_pv_gemm(Pt, Vd, r, kidx, QB, True, O=O_)

    step()
    torch.cuda.synchronize()
    ref = [down(x).copy() for x in (Pt, pvs, O_)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for x in (Pt, pvs, O_):
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [down(x) for x in (Pt, pvs, O_)]
        for a, b, name in zip(got, ref, ("Pt", "pv scores", "O")):
            assert np.array_equal(a, b), f"replay {rep}: {name} differs from the eager result"
        rmm.rmm_pv_gemm(Pt, Vd, 1.0, None, QB, True)   # eager work between replays
        torch.cuda.synchronize()
