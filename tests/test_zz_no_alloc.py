"""rmm_select_gather_noalloc (the entry point for callers that cannot allocate)
against rmm_select_gather with a workspace, through the C ABI.

Each case makes two calls in a row, the second on a smaller input, so the
second call runs on the scratch the first one left behind.  Kept indices (with
their padding), the bf16 panel, the thresholds, the bounds and, where asked
for, the scores must equal the workspace entry point's bit for bit; the kept
sets are also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, compare_sets, down, log, up_bf16
from input_adaptive_reduced_02_amd import rmm, synth

pytestmark = pytest.mark.gpu

# (workload, [(M, K), (M', K')], group_rows, r, norms): norms "cache" passes the
# per-weight B norms, "from_B" lets the call compute them into the scratch,
# "none" is the activation-only rule.  K <= 8192 with fewer than 512 groups runs
# the fused select + gather launch, K > 8192 the two launches.
CASES = [
    ("attn_proj", [(2048, 4096), (300, 1000)], 128, 0.5, "cache"),
    ("mlp_down", [(512, 2048), (130, 520)], 128, 0.37, "from_B"),
    ("mlp_down", [(256, 14336), (128, 9000)], 128, 0.5, "none"),
    ("decode", [(64, 8192), (64, 4096)], 64, 0.3, "cache"),
]


def _call(fn, A, r, gr, bnorm, B, want_scores):
    M, K = A.shape
    kk = rmm.rmm_kk(r, K)
    G = -(-M // gr)
    kpad = rmm.rmm_kk_pad(kk)
    idx = torch.full((G, kpad), -7, dtype=torch.int32, device=DEV)
    ap = torch.full((M, kpad), 3.0, dtype=torch.bfloat16, device=DEV)
    th = torch.full((G,), -1.0, dtype=torch.float32, device=DEV)
    bd = torch.full((G,), -1.0, dtype=torch.float64, device=DEV)
    sc = torch.full((G, K), -1.0, dtype=torch.float32, device=DEV) if want_scores else None
    fn(A, r, gr, idx=idx, Apanel=ap, bnorm=bnorm, B=B, scores=sc, thresh=th, bound=bd)
    return idx, ap, th, bd, sc


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1][0][0]}x{c[1][0][1]}-r{c[3]}-{c[4]}")
def test_noalloc_equals_workspace_entry_point(case):
    workload, shapes, gr, r, norms = case
    for want_scores in (False, True):
        for M, K in shapes:
            tag = f"noalloc {workload} {M}x{K} gr={gr} r={r} norms={norms} scores={want_scores}"
            log(f"case {tag}")
            d = synth.linear_inputs(workload, M, K, 64, seed=31)
            A, B = up_bf16(d["A"]), up_bf16(d["B"])
            bnorm = rmm.rmm_rownorms(B) if norms == "cache" else None
            Bx = B if norms == "from_B" else None
            ref = _call(rmm.rmm_select_gather, A, r, gr, bnorm, Bx, want_scores)
            got = _call(rmm.rmm_select_gather_noalloc, A, r, gr, bnorm, Bx, want_scores)
            torch.cuda.synchronize()
            for name, a, b in zip(("idx", "panel", "thresh", "bound", "scores"), ref, got):
                if a is None:
                    continue
                if a.dtype == torch.bfloat16:
                    a, b = a.view(torch.int16), b.view(torch.int16)
                assert torch.equal(a, b), f"{tag}: {name} differs from rmm_select_gather"
            # the kept sets against the oracle
            A64 = O.widen_bf16(d["A"])
            b64 = None if norms == "none" else O.rownorms(O.widen_bf16(d["B"]))
            sel = O.select(A64, r, gr, b64)
            ig = down(got[0])
            for g in range(ig.shape[0]):
                compare_sets(ig[g], sel, g, sel["kk"], tag)
            assert np.array_equal(down(got[2]), sel["thresh"]), f"{tag}: thresholds"


def test_noalloc_rejects_a_call_past_its_scratch():
    """65 groups of 32768 binary32 scores need 8.5 MB, past the 8 MiB scratch:
    RMM_ESCRATCH, and the outputs are untouched."""
    M, K, gr = 16 * 65, 32768, 16
    A = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    kk = rmm.rmm_kk(0.5, K)
    idx = torch.full((65, rmm.rmm_kk_pad(kk)), -7, dtype=torch.int32, device=DEV)
    ap = torch.full((M, rmm.rmm_kk_pad(kk)), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rmm.RMMError) as e:
        rmm.rmm_select_gather_noalloc(A, 0.5, gr, idx, ap)
    assert e.value.code == rmm.RMM_ESCRATCH
    torch.cuda.synchronize()
    assert bool((idx == -7).all()) and bool((ap == 3.0).all())
