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
import numpy as np
import torch

import oracle as O

DEV = "cuda:0"
FROB_TOL = 5e-3


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
    """Kept sets must match exactly; a difference is only tolerated inside the
    near-tie band of the oracle (then it is logged)."""
    a = np.asarray(idx_gpu[:kk])
    b = sel["idx"][g]
    if np.array_equal(a, b):
        return True
    diff = np.setxor1d(a, b)
    near = set(sel["near"][g].tolist())
    log(f"  {tag} group {g}: {len(diff)} indices differ: {diff[:10]} (near-tie band {sorted(near)[:10]})")
    assert set(diff.tolist()) <= near, f"{tag} group {g}: set differs outside the near-tie band"
    return False
