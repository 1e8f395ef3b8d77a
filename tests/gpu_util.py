"""Helpers of the GPU parity tests: moving seeded inputs to the device and
comparing the HIP path's outputs with the oracle's.

Output tolerance (per element), derived from the arithmetic of the path:
  |y_gpu - y_ref| <= 2^-8 |y_ref|                (bf16 output, round to nearest)
                   + kk * 2^-24 * S              (fp32 accumulation of kk terms)
                   + [fp32 inputs] 2^-7 * S      (inputs rounded to bf16 panels)
with S = sum_k |a_k| |b_k| over the kept slices, times 1.01 for the roundings of
the bound itself.  On top of that, every output matrix must be within the
relative Frobenius error 5e-3 of the oracle.
"""
import concurrent.futures as cf
import os

import numpy as np
import torch

import oracle as O

DEV = "cuda:0"
FROB_TOL = 5e-3


# host threads the oracle runs on (each call is single-threaded C; ctypes
# releases the GIL, so calls on different rows run on different cores)
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def oracle_rows(A64, B64, idx, kk, gr, rows, A64abs=None, B64abs=None):
    """(Y, S) of the oracle's reduced product for the given rows, every column:
    Y the product, S the same sum over |a_k b_k| (the scale of the element
    bound); one single-threaded oracle call per row, on a thread pool."""
    A64abs = np.abs(A64) if A64abs is None else A64abs
    B64abs = np.abs(B64) if B64abs is None else B64abs

    def one(m):
        return (O.reduced(A64, B64, idx, kk, gr, m0=m, m1=m + 1)[0],
                O.reduced(A64abs, B64abs, idx, kk, gr, m0=m, m1=m + 1)[0])

    with cf.ThreadPoolExecutor(ORACLE_THREADS) as ex:
        out = list(ex.map(one, [int(m) for m in rows]))
    return np.stack([y for y, _ in out]), np.stack([a for _, a in out])


def log(*a):
    print(*a, flush=True)


def up_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def up_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def down(t):
    """Device tensor -> numpy: bf16 as uint16 bits, others as they are."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen(t):
    """Device tensor (bf16 or fp32) -> exact float64 numpy values."""
    if t.dtype == torch.bfloat16:
        return O.widen_bf16(down(t))
    return down(t).astype(np.float64)


def elementwise_bound(y_ref, s_abs, kk, f32_inputs=False):
    b = 2.0 ** -8 * np.abs(y_ref) + kk * 2.0 ** -24 * s_abs
    if f32_inputs:
        b = b + 2.0 ** -7 * s_abs
    return 1.01 * b + 1e-30


def check_output(y_gpu, y_ref, s_abs, kk, tag, f32_inputs=False):
    err = np.abs(y_gpu - y_ref)
    bnd = elementwise_bound(y_ref, s_abs, kk, f32_inputs)
    bad = err > bnd
    nref = np.linalg.norm(y_ref)
    rel = np.linalg.norm(y_gpu - y_ref) / nref if nref > 0 else np.linalg.norm(y_gpu)
    log(f"  {tag}: rel_frob={rel:.3e} max_err/bound={np.max(err / bnd):.3f} n={y_ref.size}")
    assert not bad.any(), f"{tag}: {bad.sum()} elements outside the bound, first at {np.argwhere(bad)[0]}"
    assert rel <= FROB_TOL, f"{tag}: relative Frobenius error {rel:.3e} > {FROB_TOL}"
    return rel


def compare_sets(idx_gpu, sel, g, kk, tag):
    """Kept sets must match the oracle's exactly.  Every caller first asserts
    that the GPU's binary32 keys equal the oracle's bit for bit, and the
    selection is a deterministic function of those keys (score descending,
    ties to the lower index), so any difference is a selection bug, inside the
    near-tie band or not.  The oracle's near-tie band is only logged, as the
    acceptance rule asks."""
    a = np.asarray(idx_gpu[:kk])
    b = sel["idx"][g]
    near = sel["near"][g]
    if len(near) > 1:
        log(f"  {tag} group {g}: {len(near)} indices in the near-tie band {near[:8].tolist()}")
    if not np.array_equal(a, b):
        diff = np.setxor1d(a, b)
        raise AssertionError(f"{tag} group {g}: kept set differs from the oracle at {diff[:10].tolist()} "
                             f"(near-tie band {near[:10].tolist()})")
    return True


def compare_scores_ulp(s32_gpu, s32_ref, tag):
    """Scores the GPU sums in binary64 in another fixed order than the
    oracle's ascending one: the two binary64 sums differ by about n 2^-53
    relative, so the binary32 scores must agree to within one unit in the
    last place (and mostly exactly).  Returns the number of differing keys."""
    a = np.ascontiguousarray(s32_gpu, dtype=np.float32)
    b = np.ascontiguousarray(s32_ref, dtype=np.float32)
    diff = np.abs(a.astype(np.float64) - b.astype(np.float64))
    ulp = np.spacing(np.abs(b)).astype(np.float64)
    bad = diff > ulp
    assert not bad.any(), f"{tag}: {bad.sum()} scores more than one binary32 ulp from the oracle's, first at " \
                          f"{np.argwhere(bad)[0]}"
    n = int((a.view(np.uint32) != b.view(np.uint32)).sum())
    if n:
        log(f"  {tag}: {n} of {a.size} scores one ulp from the oracle's")
    return n


def top_kk(keys, kk):
    """Ascending indices of the kk best binary32 keys, ties to the lower index:
    the selection rule, applied to a given key row (numpy lexsort)."""
    order = np.lexsort((np.arange(len(keys)), -np.asarray(keys, dtype=np.float64)))
    return np.sort(order[:kk]).astype(np.int32)


def compare_sets_keys(idx_gpu, keys_gpu, ref_idx, keys_ref, near, kk, tag):
    """Kept sets when the two sides' keys may differ by one ulp: with
    bit-identical keys the sets must be identical; otherwise the GPU's set must
    be the kk best of its own keys under the selection rule, and may differ
    from the oracle's only inside the oracle's near-tie band."""
    a = np.asarray(idx_gpu[:kk])
    kg = np.ascontiguousarray(keys_gpu, dtype=np.float32)
    kr = np.ascontiguousarray(keys_ref, dtype=np.float32)
    if np.array_equal(kg.view(np.uint32), kr.view(np.uint32)):
        assert np.array_equal(a, ref_idx), f"{tag}: kept set differs from the oracle's with identical keys"
        return True
    assert np.array_equal(a, top_kk(kg, kk)), f"{tag}: kept set is not the top-kk of the GPU's own keys"
    if not np.array_equal(a, ref_idx):
        diff = np.setxor1d(a, ref_idx)
        log(f"  {tag}: {len(diff)} kept indices differ from the oracle's, near-tie band {list(near)[:10]}")
        assert set(diff.tolist()) <= set(np.asarray(near).tolist()), \
            f"{tag}: kept set differs outside the near-tie band"
    return False
