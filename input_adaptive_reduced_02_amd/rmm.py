"""Python binding of librmm.so (include/rmm.h): argument marshalling only.

Every function has the name of the C entry point it calls and forwards torch
tensors as device pointers with their leading dimensions, on the current HIP
stream of the tensors' device.  All arithmetic runs in the library's HIP
kernels; there is no CPU or PyTorch fallback: if librmm.so has not been built,
the first call raises.

Method: "Reduced Matrix Multiplication: Input-Adaptive Matrix-Product Reduction
for LLM Inference", technical summary (gist.science), Metodologia (score each
contraction slice, keep ceil(rho d), multiply only the kept slices).
"""
import ctypes
import os

import torch

# the library built in-tree; RMM_LIB selects another build of it
LIB_PATH = os.environ.get("RMM_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "librmm.so")

RMM_OK, RMM_EINVAL, RMM_EUNSUPPORTED, RMM_EHIP, RMM_ESCRATCH = 0, -1, -2, -3, -4
RMM_NOALLOC_SCRATCH_BYTES = 8 << 20
RMM_F32, RMM_BF16 = 0, 1
KPAD = 64

_lib = None


class RMMError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {code} ({rmm_strerror(code)})")


def lib():
    """The loaded librmm.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m input_adaptive_reduced_02_amd.build`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


_P = ctypes.c_void_p
_L = ctypes.c_int64
_I = ctypes.c_int
_S = ctypes.c_size_t
_Dbl = ctypes.c_double


def _declare(L):
    L.rmm_kk.restype = _L
    L.rmm_kk.argtypes = [_Dbl, _L]
    L.rmm_kk_pad.restype = _L
    L.rmm_kk_pad.argtypes = [_L]
    L.rmm_strerror.restype = ctypes.c_char_p
    L.rmm_strerror.argtypes = [_I]
    L.rmm_rownorms.restype = _I
    L.rmm_rownorms.argtypes = [_P, _I, _L, _L, _L, _P, _P]
    L.rmm_select_workspace_bytes.restype = _S
    L.rmm_select_workspace_bytes.argtypes = [_L, _L, _L, _I, _I]
    L.rmm_select.restype = _I
    L.rmm_select.argtypes = [_P, _I, _L, _L, _L, _P, _P, _L, _L, _Dbl, _L, _P, _L, _P, _P, _P, _P, _S, _P]
    L.rmm_gather.restype = _I
    L.rmm_select_gather.restype = _I
    L.rmm_select_gather.argtypes = [_P, _I, _L, _L, _L, _P, _P, _L, _L, _Dbl, _L, _P, _L, _P, _L, _P, _P, _P,
                                    _P, _S, _P]
    L.rmm_gather.argtypes = [_P, _I, _L, _L, _L, _P, _L, _L, _L, _P, _L, _P, _L, _L, _P, _L, _P]
    L.rmm_scores.restype = _I
    L.rmm_scores.argtypes = [_P, _I, _L, _L, _L, _P, _P, _L, _L, _L, _P, _P, _S, _P]
    L.rmm_select_scores.restype = _I
    L.rmm_select_scores.argtypes = [_P, _L, _L, _L, _Dbl, _P, _L, _P, _P, _P]
    L.rmm_select_gather_noalloc.restype = _I
    L.rmm_select_gather_noalloc.argtypes = [_P, _I, _L, _L, _L, _P, _P, _L, _L, _Dbl, _L, _P, _L, _P, _L, _P, _P,
                                            _P, _P]
    L.rmm_gemm_workspace_bytes.restype = _S
    L.rmm_gemm_workspace_bytes.argtypes = [_L, _L, _L, _L]
    L.rmm_gemm.restype = _I
    L.rmm_gemm.argtypes = [_P, _L, _P, _L, _P, _L, _L, _L, _L, _L, _P, _I, _L, _P, _S, _P]
    L.rmm_attn_pv_workspace_bytes.restype = _S
    L.rmm_attn_pv_workspace_bytes.argtypes = [_L, _L, _L, _Dbl, _L, _I, _I, _I]
    L.rmm_attn_pv.restype = _I
    L.rmm_attn_pv.argtypes = [_P, _P, _L, _L, _L, _Dbl, _L, _I, _P, _I, _P, _L, _P, _P, _S, _P]
    L.rmm_pv_select.restype = _I
    L.rmm_pv_select.argtypes = [_P, _P, _L, _L, _L, _Dbl, _L, _I, _P, _L, _P, _P, _S, _P]
    L.rmm_pv_gemm.restype = _I
    L.rmm_pv_gemm.argtypes = [_P, _P, _L, _L, _L, _Dbl, _L, _I, _P, _L, _P, _I, _P]
    L.rmm_quantize_q8.restype = _I
    L.rmm_quantize_q8.argtypes = [_P, _L, _L, _L, _P, _L, _P, _P]
    L.rmm_rownorms_q8.restype = _I
    L.rmm_rownorms_q8.argtypes = [_P, _L, _P, _L, _L, _P, _P]
    L.rmm_gemm_q8_workspace_bytes.restype = _S
    L.rmm_gemm_q8_workspace_bytes.argtypes = [_L, _L, _L, _L]
    L.rmm_gemm_q8.restype = _I
    L.rmm_gemm_q8.argtypes = [_P, _L, _P, _L, _P, _P, _L, _L, _L, _L, _L, _P, _I, _L, _P, _S, _P]
    L.rmm_qk_select_workspace_bytes.restype = _S
    L.rmm_qk_select_workspace_bytes.argtypes = [_L, _L, _L, _L, _I]
    L.rmm_qk_select.restype = _I
    L.rmm_qk_select.argtypes = [_P, _P, _L, _L, _L, _Dbl, _L, _I, _I, _P, _L, _P, _P, _S, _P]
    L.rmm_attn_probs_workspace_bytes.restype = _S
    L.rmm_attn_probs_workspace_bytes.argtypes = [_L, _L, _L, _I]
    L.rmm_attn_probs.restype = _I
    L.rmm_attn_probs.argtypes = [_P, _P, _L, _L, _L, _L, _I, _P, _L, _Dbl, _P, _P, _P, _P, _S, _P]
    L.rmm_pv_select_scores.restype = _I
    L.rmm_pv_select_scores.argtypes = [_P, _L, _L, _Dbl, _L, _I, _P, _L, _P]
    return L


# ------------------------------------------------------------------ helpers
def _dt(t):
    if t.dtype == torch.bfloat16:
        return RMM_BF16
    if t.dtype == torch.float32:
        return RMM_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(fn, code):
    if code != RMM_OK:
        raise RMMError(fn, code)


def _ws(nbytes, device, ws):
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points
def rmm_kk(r, K):
    return int(lib().rmm_kk(float(r), int(K)))


def rmm_kk_pad(kk):
    return int(lib().rmm_kk_pad(int(kk)))


def rmm_strerror(code):
    return lib().rmm_strerror(int(code)).decode()


def rmm_rownorms(B, bnorm=None):
    """||B[k, :]||_2 for every row k, binary64 [K] (computed once per weight)."""
    K, N = B.shape
    if bnorm is None:
        bnorm = torch.empty(K, dtype=torch.float64, device=B.device)
    _check("rmm_rownorms", lib().rmm_rownorms(_ptr(B), _dt(B), K, N, _ld(B), _ptr(bnorm), _stream(B)))
    return bnorm


def rmm_select_workspace_bytes(M, K, group_rows, have_scores=False, norms_from_B=False):
    return int(lib().rmm_select_workspace_bytes(M, K, group_rows, int(bool(have_scores)),
                                                int(bool(norms_from_B))))


def rmm_select(A, r, group_rows, bnorm=None, B=None, idx=None, scores=None, thresh=None, bound=None,
               ws=None):
    """Per-group top-kk slice indices [G, kk_pad] int32 (ascending, padded)."""
    M, K = A.shape
    kk = rmm_kk(r, K)
    if kk < 1:
        raise ValueError("r must lie in (0, 1]")
    G = -(-M // group_rows)
    if idx is None:
        idx = torch.empty((G, rmm_kk_pad(kk)), dtype=torch.int32, device=A.device)
    from_B = bnorm is None and B is not None
    need = rmm_select_workspace_bytes(M, K, group_rows, scores is not None, from_B)
    w = _ws(need, A.device, ws)
    N, ldb = (B.shape[1], _ld(B)) if from_B else (0, 0)
    _check("rmm_select", lib().rmm_select(
        _ptr(A), _dt(A), M, K, _ld(A), _ptr(bnorm), _ptr(B) if from_B else None, N, ldb, float(r),
        group_rows, _ptr(idx), _ld(idx), _ptr(scores), _ptr(thresh), _ptr(bound), _ptr(w), need,
        _stream(A)))
    return idx


def rmm_select_gather(A, r, group_rows, bnorm=None, B=None, idx=None, Apanel=None, scores=None, thresh=None,
                      bound=None, ws=None):
    """rmm_select and rmm_gather of its indices in one call: (idx [G, kk_pad]
    int32, bf16 panel [M, kk_pad])."""
    M, K = A.shape
    kk = rmm_kk(r, K)
    if kk < 1:
        raise ValueError("r must lie in (0, 1]")
    G = -(-M // group_rows)
    kpad = rmm_kk_pad(kk)
    if idx is None:
        idx = torch.empty((G, kpad), dtype=torch.int32, device=A.device)
    if Apanel is None:
        Apanel = torch.empty((M, kpad), dtype=torch.bfloat16, device=A.device)
    from_B = bnorm is None and B is not None
    need = rmm_select_workspace_bytes(M, K, group_rows, scores is not None, from_B)
    w = _ws(need, A.device, ws)
    N, ldb = (B.shape[1], _ld(B)) if from_B else (0, 0)
    _check("rmm_select_gather", lib().rmm_select_gather(
        _ptr(A), _dt(A), M, K, _ld(A), _ptr(bnorm), _ptr(B) if from_B else None, N, ldb, float(r),
        group_rows, _ptr(idx), _ld(idx), _ptr(Apanel), _ld(Apanel), _ptr(scores), _ptr(thresh), _ptr(bound),
        _ptr(w), need, _stream(A)))
    return idx, Apanel


def rmm_scores(A, group_rows, bnorm=None, B=None, scores=None, ws=None):
    """Per-group slice scores [G, K] binary32 (the score half of rmm_select)."""
    M, K = A.shape
    G = -(-M // group_rows)
    if scores is None:
        scores = torch.empty((G, K), dtype=torch.float32, device=A.device)
    from_B = bnorm is None and B is not None
    need = rmm_select_workspace_bytes(M, K, group_rows, True, from_B)
    w = _ws(need, A.device, ws)
    N, ldb = (B.shape[1], _ld(B)) if from_B else (0, 0)
    _check("rmm_scores", lib().rmm_scores(
        _ptr(A), _dt(A), M, K, _ld(A), _ptr(bnorm), _ptr(B) if from_B else None, N, ldb, group_rows,
        _ptr(scores), _ptr(w), need, _stream(A)))
    return scores


def rmm_select_scores(scores, r, idx=None, thresh=None, bound=None):
    """Kept indices [G, kk_pad] from given scores [G, K] (the selection half of rmm_select)."""
    G, K = scores.shape
    kk = rmm_kk(r, K)
    if kk < 1:
        raise ValueError("r must lie in (0, 1]")
    if idx is None:
        idx = torch.empty((G, rmm_kk_pad(kk)), dtype=torch.int32, device=scores.device)
    _check("rmm_select_scores", lib().rmm_select_scores(
        _ptr(scores), G, K, _ld(scores), float(r), _ptr(idx), _ld(idx), _ptr(thresh), _ptr(bound),
        _stream(scores)))
    return idx


def rmm_select_gather_noalloc(A, r, group_rows, idx, Apanel, bnorm=None, B=None, scores=None, thresh=None,
                              bound=None):
    """rmm_select_gather with the library's fixed per-GPU scratch instead of a
    workspace: the caller passes every output (idx [G, >= kk_pad] int32, Apanel
    [M, >= kk_pad] bf16), so the call allocates nothing.  Returns (idx, Apanel)."""
    M, K = A.shape
    from_B = bnorm is None and B is not None
    N, ldb = (B.shape[1], _ld(B)) if from_B else (0, 0)
    _check("rmm_select_gather_noalloc", lib().rmm_select_gather_noalloc(
        _ptr(A), _dt(A), M, K, _ld(A), _ptr(bnorm), _ptr(B) if from_B else None, N, ldb, float(r),
        group_rows, _ptr(idx), _ld(idx), _ptr(Apanel), _ld(Apanel), _ptr(scores), _ptr(thresh), _ptr(bound),
        _stream(A)))
    return idx, Apanel


def rmm_gather(A, idx, kk, group_rows, Apanel=None, B=None, Bpanel=None):
    """bf16 panel of the kept columns of A [M, kk_pad] (and of the kept rows of B)."""
    M, K = A.shape
    kpad = rmm_kk_pad(kk)
    if Apanel is None:
        Apanel = torch.empty((M, kpad), dtype=torch.bfloat16, device=A.device)
    N, ldb, ldbp = 0, 0, 0
    if B is not None:
        N = B.shape[1]
        ldb = _ld(B)
        if Bpanel is None:
            Bpanel = torch.empty((kpad, N), dtype=torch.bfloat16, device=A.device)
        ldbp = _ld(Bpanel)
    _check("rmm_gather", lib().rmm_gather(
        _ptr(A), _dt(A), M, K, _ld(A), _ptr(idx), _ld(idx), kk, group_rows, _ptr(Apanel), _ld(Apanel),
        _ptr(B), N, ldb, _ptr(Bpanel), ldbp, _stream(A)))
    return Apanel, Bpanel


def rmm_gemm(A, B, idx, kk, group_rows, Y=None, ydt=torch.bfloat16, M=None, ws=None):
    """Y = A[:, :kk] * B[rows, :] per group; rows = idx[g] (or 0..kk-1 when idx is None)."""
    M = A.shape[0] if M is None else M
    N = B.shape[1]
    if Y is None:
        Y = torch.empty((M, N), dtype=ydt, device=A.device)
    need = int(lib().rmm_gemm_workspace_bytes(M, N, kk, group_rows))
    w = _ws(need, A.device, ws)
    _check("rmm_gemm", lib().rmm_gemm(
        _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(idx), _ld(idx) if idx is not None else 0, M, N, kk,
        group_rows, _ptr(Y), _dt(Y), _ld(Y), _ptr(w), need, _stream(A)))
    return Y


def rmm_attn_pv_workspace_bytes(H, L, D, r, qblock=128, causal=True, have_idx_out=False,
                                have_scores_out=False):
    return int(lib().rmm_attn_pv_workspace_bytes(H, L, D, float(r), qblock, int(bool(causal)),
                                                 int(bool(have_idx_out)), int(bool(have_scores_out))))


def rmm_attn_pv(Pt, V, r, qblock=128, causal=True, O=None, odt=torch.bfloat16, idx_out=None,
                scores_out=None, ws=None):
    """O [H, L, D] of P.V reduced along keys; Pt is key-major [H, L, L] bf16."""
    H, L, D = V.shape
    if O is None:
        O = torch.empty((H, L, D), dtype=odt, device=V.device)
    need = rmm_attn_pv_workspace_bytes(H, L, D, r, qblock, causal, idx_out is not None,
                                       scores_out is not None)
    w = _ws(need, V.device, ws)
    ldix = idx_out.stride(0) if idx_out is not None else 0
    _check("rmm_attn_pv", lib().rmm_attn_pv(
        _ptr(Pt), _ptr(V), H, L, D, float(r), qblock, int(bool(causal)), _ptr(O), _dt(O), _ptr(idx_out),
        ldix, _ptr(scores_out), _ptr(w), need, _stream(V)))
    return O


def rmm_pv_select(Pt, V, r, qblock=128, causal=True, idx_out=None, scores_out=None, ws=None):
    """Kept-key lists [H*G, pad(L)] int32 of P.V (the scoring and selection of
    rmm_attn_pv without the product)."""
    H, L, D = V.shape
    G = -(-L // qblock)
    if idx_out is None:
        idx_out = torch.empty((H * G, rmm_kk_pad(L)), dtype=torch.int32, device=V.device)
    need = rmm_attn_pv_workspace_bytes(H, L, D, r, qblock, causal, True, scores_out is not None)
    w = _ws(need, V.device, ws)
    _check("rmm_pv_select", lib().rmm_pv_select(
        _ptr(Pt), _ptr(V), H, L, D, float(r), qblock, int(bool(causal)), _ptr(idx_out), idx_out.stride(0),
        _ptr(scores_out), _ptr(w), need, _stream(V)))
    return idx_out


def rmm_pv_gemm(Pt, V, r, idx=None, qblock=128, causal=True, O=None, odt=torch.bfloat16):
    """O [H, L, D] = P.V over the kept keys idx (rmm_pv_select's lists); idx
    None: the dense causal product."""
    H, L, D = V.shape
    if O is None:
        O = torch.empty((H, L, D), dtype=odt, device=V.device)
    ldix = idx.stride(0) if idx is not None else 0
    _check("rmm_pv_gemm", lib().rmm_pv_gemm(
        _ptr(Pt), _ptr(V), H, L, D, float(r), qblock, int(bool(causal)), _ptr(idx), ldix, _ptr(O), _dt(O),
        _stream(V)))
    return O


def rmm_qk_select(Q, K, r, qblock=128, causal=True, use_k=True, idx_out=None, scores_out=None, ws=None):
    """Kept features [H*G, pad(D)] int32 of QK^T per (head, query block);
    Q, K are [H, L, D] bf16."""
    H, L, D = Q.shape
    G = -(-L // qblock)
    if idx_out is None:
        idx_out = torch.empty((H * G, rmm_kk_pad(D)), dtype=torch.int32, device=Q.device)
    need = int(lib().rmm_qk_select_workspace_bytes(H, L, D, qblock, int(scores_out is not None)))
    w = _ws(need, Q.device, ws)
    _check("rmm_qk_select", lib().rmm_qk_select(
        _ptr(Q), _ptr(K), H, L, D, float(r), qblock, int(bool(causal)), int(bool(use_k)), _ptr(idx_out),
        idx_out.stride(0), _ptr(scores_out), _ptr(w), need, _stream(Q)))
    return idx_out


def rmm_attn_probs(Q, K, idx_qk=None, r_qk=1.0, qblock=128, causal=True, Pt=None, V=None, pv_scores=None,
                   ws=None):
    """Key-major attention probabilities Pt [H, L, L] bf16 over the kept
    features idx_qk (None: all); with V and pv_scores [H, G, L] float32 also
    the P.V key scores."""
    H, L, D = Q.shape
    if Pt is None:
        Pt = torch.empty((H, L, L), dtype=torch.bfloat16, device=Q.device)
    need = int(lib().rmm_attn_probs_workspace_bytes(H, L, D, int(pv_scores is not None)))
    w = _ws(need, Q.device, ws)
    ldix = idx_qk.stride(0) if idx_qk is not None else 0
    _check("rmm_attn_probs", lib().rmm_attn_probs(
        _ptr(Q), _ptr(K), H, L, D, qblock, int(bool(causal)), _ptr(idx_qk), ldix, float(r_qk), _ptr(Pt),
        _ptr(V), _ptr(pv_scores), _ptr(w), need, _stream(Q)))
    return Pt


def rmm_pv_select_scores(scores, r, qblock=128, causal=True, idx_out=None):
    """Kept-key lists [H*G, pad(L)] int32 from rmm_attn_probs' P.V scores [H, G, L]."""
    H, G, L = scores.shape
    if idx_out is None:
        idx_out = torch.empty((H * G, rmm_kk_pad(L)), dtype=torch.int32, device=scores.device)
    _check("rmm_pv_select_scores", lib().rmm_pv_select_scores(
        _ptr(scores), H, L, float(r), qblock, int(bool(causal)), _ptr(idx_out), idx_out.stride(0),
        _stream(scores)))
    return idx_out


def rmm_quantize_q8(B, Bq=None, scale=None):
    """(Bq int8 [K, N], scale float32 [N]) of a bf16 weight B [K, N]."""
    K, N = B.shape
    if Bq is None:
        Bq = torch.empty((K, N), dtype=torch.int8, device=B.device)
    if scale is None:
        scale = torch.empty(N, dtype=torch.float32, device=B.device)
    _check("rmm_quantize_q8", lib().rmm_quantize_q8(_ptr(B), K, N, _ld(B), _ptr(Bq), _ld(Bq), _ptr(scale),
                                                     _stream(B)))
    return Bq, scale


def rmm_rownorms_q8(Bq, scale, bnorm=None):
    """Row norms of the dequantised int8 weight, binary64 [K]."""
    K, N = Bq.shape
    if bnorm is None:
        bnorm = torch.empty(K, dtype=torch.float64, device=Bq.device)
    _check("rmm_rownorms_q8", lib().rmm_rownorms_q8(_ptr(Bq), _ld(Bq), _ptr(scale), K, N, _ptr(bnorm),
                                                     _stream(Bq)))
    return bnorm


def rmm_gemm_q8_workspace_bytes(M, N, kk, group_rows):
    return int(lib().rmm_gemm_q8_workspace_bytes(M, N, kk, group_rows))


def rmm_gemm_q8(A, Bq, scale, idx, kk, group_rows, Y=None, ydt=torch.bfloat16, M=None, ws=None):
    """Y = scale * (A[:, :kk] * Bq[rows, :]) per group, rows as rmm_gemm.  A
    caller's `ws` must be zero-filled before its first use (it stays reusable)."""
    M = A.shape[0] if M is None else M
    N = Bq.shape[1]
    if Y is None:
        Y = torch.empty((M, N), dtype=ydt, device=A.device)
    need = rmm_gemm_q8_workspace_bytes(M, N, kk, group_rows)
    if ws is None and need:
        ws = torch.zeros(need, dtype=torch.uint8, device=A.device)   # zero-filled before first use
    w = _ws(need, A.device, ws)
    _check("rmm_gemm_q8", lib().rmm_gemm_q8(
        _ptr(A), _ld(A), _ptr(Bq), _ld(Bq), _ptr(scale), _ptr(idx), _ld(idx) if idx is not None else 0, M, N,
        kk, group_rows, _ptr(Y), _dt(Y), _ld(Y), _ptr(w), 0 if w is None else w.numel() * w.element_size(),
        _stream(A)))
    return Y


def linear_q8(A, Bq, scale, r, group_rows, bnorm, ydt=torch.bfloat16):
    """The linear-layer chain on an int8 weight: select (with the dequantised
    weight's row norms `bnorm`) -> gather -> reduced int8 GEMM; r == 1 runs
    the same GEMM on A in place."""
    M, K = A.shape
    kk = rmm_kk(r, K)
    if kk == K:
        return rmm_gemm_q8(A, Bq, scale, None, K, group_rows, ydt=ydt)
    idx, Ap = rmm_select_gather(A, r, group_rows, bnorm=bnorm)
    return rmm_gemm_q8(Ap, Bq, scale, idx, kk, group_rows, ydt=ydt)


def linear(A, B, r, group_rows, bnorm=None, ydt=torch.bfloat16, activation_only=False):
    """The whole linear-layer chain: select -> gather -> reduced GEMM.

    Scores use the B row norms `bnorm` (computed from B on the fly when not
    given), or the activation column norms alone when activation_only is set.
    r == 1 runs the same GEMM kernel on A and B in place (the dense baseline).
    B is [K, N] row-major (the transpose of torch.nn.Linear's weight layout).
    """
    M, K = A.shape
    kk = rmm_kk(r, K)
    if kk == K and A.dtype == torch.bfloat16 and B.dtype == torch.bfloat16 and K % 8 == 0:
        return rmm_gemm(A, B, None, K, group_rows, ydt=ydt)
    sel_B = None if activation_only or bnorm is not None else B
    if B.dtype != torch.bfloat16:
        idx = rmm_select(A, r, group_rows, bnorm=bnorm, B=sel_B)
        if idx.shape[0] != 1:
            raise ValueError("binary32 B needs a single selection group (packed B panel)")
        Ap, Bp = rmm_gather(A, idx, kk, group_rows, B=B)
        return rmm_gemm(Ap, Bp, None, kk, group_rows, ydt=ydt)
    idx, Ap = rmm_select_gather(A, r, group_rows, bnorm=bnorm, B=sel_B)
    return rmm_gemm(Ap, B, idx, kk, group_rows, ydt=ydt)
