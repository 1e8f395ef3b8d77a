"""GPU parity of the P.V variant (key-dimension reduction per 128-query block)
against the oracle, through the C ABI.

P is the causal row-softmax of Q K^T / sqrt(128) made by synth.pv_probs_t on
the device, stored key-major; its bits are the input of both sides (the oracle
reads them back, it does not recompute the softmax).  Block scores within one
binary32 ulp of the oracle's (the GPU sums each key's probabilities in
binary64 as eight partial sums added pairwise, the oracle in ascending
order); kept sets identical where the keys are, otherwise the kk best of the
GPU's own keys and different only inside the near-tie band; outputs within
the bound of tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, check_output, compare_scores_ulp, compare_sets_keys, down, log, up_bf16, widen
from input_adaptive_reduced_02_amd import rmm, synth

pytestmark = pytest.mark.gpu

QB = 128


def make_pv(H, L, seed=0, causal=True):
    q, k, v = synth.pv_qkv(H, L, 128, seed=seed)
    Pt = synth.pv_probs_t(q, k, causal=causal, device=DEV)
    V = up_bf16(v)
    torch.cuda.synchronize()
    return Pt, V


def run_pv(Pt, V, r, causal=True):
    H, L, D = V.shape
    G = -(-L // QB)
    kpad_max = rmm.rmm_kk_pad(L)
    idx = torch.zeros((H * G, kpad_max), dtype=torch.int32, device=DEV)
    scores = torch.zeros((H, G, L), dtype=torch.float32, device=DEV)
    O_ = rmm.rmm_attn_pv(Pt, V, r, QB, causal, idx_out=idx if r < 1 else None,
                         scores_out=scores if r < 1 else None)
    torch.cuda.synchronize()
    ig = down(idx)
    assert ig.min() >= 0 and ig.max() < L
    return O_, idx, scores


def check_block(Pt_h, V_h, O_h, idx_h, scores_h, L, g, r, causal, tag, q_sample=None):
    """One (head, block): scores and kept set exact, output rows within bound."""
    Vh64 = O.widen_bf16(V_h)
    q0 = g * QB
    nq = min(QB, L - q0)
    Kg = O.pv_prefix(L, QB, g, causal)
    Ptb = O.widen_bf16(Pt_h[:Kg, q0:q0 + nq])
    if r < 1:
        s64, s32 = O.pv_scores(Ptb, Vh64[:Kg])
        compare_scores_ulp(scores_h[g, :Kg], s32, f"{tag} block {g} scores")
        kk = O.kk(r, Kg)
        ref_idx = O.topk(s32, kk)
        compare_sets_keys(idx_h[g, :kk], scores_h[g, :Kg], ref_idx, s32, O.near_ties(s64, s32, ref_idx), kk,
                          f"{tag} block {g}")
        kpad = -(-kk // 64) * 64
        assert np.all(idx_h[g, kk:kpad] == idx_h[g, kk - 1]), f"{tag} block {g}: padding"

        kept = idx_h[g, :kk].astype(np.int32)
    else:
        kk = Kg
        kept = np.arange(Kg, dtype=np.int32)
    rows = np.arange(nq) if q_sample is None else q_sample[q_sample < nq]
    Ob = O.pv_block(np.ascontiguousarray(Ptb[:, rows]), Vh64[:Kg], kept)
    Sb = O.pv_block(np.abs(np.ascontiguousarray(Ptb[:, rows])), np.abs(Vh64[:Kg]), kept)
    Og = O.widen_bf16(O_h[q0 + rows])
    return Og, Ob, Sb, kk


@pytest.mark.parametrize("H,L,causal", [(2, 512, True), (2, 520, True), (1, 384, False), (3, 1024, True)])
@pytest.mark.parametrize("r", [0.3, 0.5, 1.0])
def test_pv_small(H, L, causal, r):
    tag = f"pv H={H} L={L} causal={causal} r={r}"
    log(tag)
    Pt, V = make_pv(H, L, seed=1, causal=causal)
    O_, idx, scores = run_pv(Pt, V, r, causal)
    G = -(-L // QB)
    Pt_np, V_np, O_np = down(Pt), down(V), down(O_)
    idx_np = down(idx).reshape(H, G, -1)
    sc_np = down(scores)
    for h in range(H):
        outs = [check_block(Pt_np[h], V_np[h], O_np[h], idx_np[h], sc_np[h], L, g, r, causal, f"{tag} h={h}")
                for g in range(G)]
        Og = np.concatenate([o[0] for o in outs])
        Ob = np.concatenate([o[1] for o in outs])
        Sb = np.concatenate([o[2] for o in outs])
        kk_max = max(o[3] for o in outs)
        check_output(Og, Ob, Sb, kk_max, f"{tag} h={h}")


@pytest.mark.parametrize("L,r", [(4096, 0.3), (4096, 0.5), (4096, 1.0),
                                 (16384, 0.3), (16384, 0.5), (16384, 1.0)])
def test_pv_full(L, r):
    """The full P.V workload (32 heads, head dim 128); heads 0 and 31 checked:
    at L=4096 every block's scores, kept set and output rows, at L=16384 every
    8th block and the last, 16 sampled output rows of each."""
    H = 32
    key = ("pv", L)
    if getattr(test_pv_full, "_key", None) != key:
        test_pv_full._data = None
        torch.cuda.empty_cache()
        test_pv_full._data = make_pv(H, L, seed=0)
        test_pv_full._key = key
    Pt, V = test_pv_full._data
    tag = f"pv full L={L} r={r}"
    log(tag)
    O_, idx, scores = run_pv(Pt, V, r)
    G = L // QB
    blocks = list(range(G)) if L <= 4096 else sorted(set(range(0, G, 8)) | {G - 1})
    rng = np.random.default_rng(3)
    q_sample = None if L <= 4096 else np.unique(np.concatenate([[0, QB - 1], rng.integers(0, QB, 14)]))
    for h in (0, H - 1):
        Pt_h = down(Pt[h])
        V_h, O_h = down(V[h]), down(O_[h])
        idx_h = down(idx.view(H, G, -1)[h])
        sc_h = down(scores[h])
        outs = [check_block(Pt_h, V_h, O_h, idx_h, sc_h, L, g, r, True, f"{tag} h={h}", q_sample)
                for g in blocks]
        check_output(np.concatenate([o[0] for o in outs]), np.concatenate([o[1] for o in outs]),
                     np.concatenate([o[2] for o in outs]), max(o[3] for o in outs), f"{tag} h={h}")
    del O_, idx, scores


@pytest.mark.parametrize("L,r", [(520, 0.3), (1024, 0.5)])
def test_split_entry_points_match(L, r):
    """rmm_pv_select then rmm_pv_gemm give the kept lists, scores and output of
    rmm_attn_pv bit for bit (the same kernels), and rmm_pv_gemm without a list
    equals the r = 1 product."""
    H = 3
    Pt, V = make_pv(H, L, seed=11)
    O1, idx1, sc1 = run_pv(Pt, V, r)
    G = -(-L // QB)
    idx2 = torch.zeros_like(idx1)
    sc2 = torch.zeros_like(sc1)
    rmm.rmm_pv_select(Pt, V, r, QB, True, idx_out=idx2, scores_out=sc2)
    O2 = rmm.rmm_pv_gemm(Pt, V, r, idx2, QB, True)
    Od = rmm.rmm_pv_gemm(Pt, V, 1.0, None, QB, True)
    Od_ref = rmm.rmm_attn_pv(Pt, V, 1.0, QB, True)
    torch.cuda.synchronize()
    assert torch.equal(sc1, sc2) and torch.equal(idx1, idx2)
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
    assert torch.equal(Od.view(torch.int16), Od_ref.view(torch.int16))
    log(f"split entry points H={H} L={L} r={r}: identical ({H * G} blocks)")
