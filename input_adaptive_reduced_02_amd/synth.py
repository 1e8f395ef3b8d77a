"""Seeded synthetic inputs for the RMM hot path.

The one module that both the GPU path's tests/bench and the oracle's tests draw
their inputs from.  It holds input construction only: seeded random draws, the
rounding of binary32 draws to the bf16 bit patterns that are then stored, and
the attention-probability recipe of the P.V workload.  None of the method's
arithmetic (scores, selection, reduced product) is here.

Every tensor has its own PCG64 stream, keyed by (seed, workload id, tensor id),
so a smaller instance of a workload draws the same kind of values and any
tensor can be regenerated alone.

Workloads (matrix shapes of the pages' evaluation, which used LLaMA 3.1/3.2 and
Qwen models on QA, reasoning, summarisation and long-context tasks -- none of
which are available here, so these seeded stand-ins take their place):
  tiny       A fp32 [M,K] = N(0,1) * column scale ~ lognormal(0,1); B fp32 N(0,1)
  attn_proj  X bf16 = N(0,1) * channel scale ~ lognormal(0,1), with
             round(0.01*K) outlier channels (drawn without replacement) x20;
             W bf16 N(0, 0.02)
  mlp_down   X bf16 = silu(g) * u, g, u ~ N(0,1); W bf16 N(0, 0.02)
  decode     X bf16 = N(0,1) * channel scale ~ lognormal(0,1) (no outliers);
             W bf16 N(0, 0.02)
  pv         Q, K, V bf16 N(0,1), [H, L, D]; P = causal row-softmax of
             Q K^T / sqrt(D) in fp32 from the bf16 values, rounded to bf16 and
             stored key-major (Pt[h, k, q] = P[h, q, k]).
"""
import numpy as np

WORKLOAD_IDS = {"tiny": 1, "attn_proj": 2, "mlp_down": 3, "pv": 4, "decode": 5}

# full sizes of each workload: (M, K, N) for the linear ones, (H, L, D) for pv
FULL_SHAPES = {
    "tiny": (64, 256, 128),
    "attn_proj": (2048, 4096, 4096),
    "mlp_down": (4096, 14336, 4096),
    "decode": (64, 8192, 28672),
    "pv": (32, 16384, 128),
}
GROUP_ROWS = {"tiny": 64, "attn_proj": 128, "mlp_down": 128, "decode": 64, "pv": 128}
RATIOS = {
    "tiny": (0.5,),
    "attn_proj": (0.3, 0.5, 0.7, 1.0),
    "mlp_down": (0.5, 0.7, 0.9, 1.0),
    "pv": (0.3, 0.5, 1.0),
    "decode": (0.3, 0.5, 0.7, 1.0),
}


def generator(workload, tensor, seed=0):
    wid = WORKLOAD_IDS[workload]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, tensor])))


def f32_to_bf16_bits(x):
    """Round binary32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _normal(g, shape, std=1.0):
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def linear_inputs(workload, M=None, K=None, N=None, seed=0):
    """A [M,K] and B [K,N] of a linear-layer workload.

    bf16 workloads return uint16 bit arrays, `tiny` returns float32 arrays.
    Returns dict(A=..., B=..., dtype='bf16'|'f32').
    """
    M0, K0, N0 = FULL_SHAPES[workload]
    M = M0 if M is None else M
    K = K0 if K is None else K
    N = N0 if N is None else N
    if workload == "tiny":
        a = _normal(generator(workload, 0, seed), (M, K))
        scale = generator(workload, 2, seed).lognormal(0.0, 1.0, K).astype(np.float32)
        a *= scale[None, :]
        b = _normal(generator(workload, 1, seed), (K, N))
        return dict(A=a, B=b, dtype="f32")
    if workload in ("attn_proj", "decode"):
        a = _normal(generator(workload, 0, seed), (M, K))
        scale = generator(workload, 2, seed).lognormal(0.0, 1.0, K)
        if workload == "attn_proj":
            n_out = int(round(0.01 * K))
            out = generator(workload, 3, seed).choice(K, size=n_out, replace=False)
            scale[out] *= 20.0
        a *= scale.astype(np.float32)[None, :]
    elif workload == "mlp_down":
        gate = _normal(generator(workload, 0, seed), (M, K))
        up = _normal(generator(workload, 4, seed), (M, K))
        a = gate / (np.float32(1.0) + np.exp(-gate)) * up
    else:
        raise ValueError(workload)
    b = _normal(generator(workload, 1, seed), (K, N), std=0.02)
    return dict(A=f32_to_bf16_bits(a), B=f32_to_bf16_bits(b), dtype="bf16")


def pv_qkv(H=None, L=None, D=None, seed=0):
    """Q, K, V bf16 bit arrays [H, L, D] of the P.V workload."""
    H0, L0, D0 = FULL_SHAPES["pv"]
    H = H0 if H is None else H
    L = L0 if L is None else L
    D = D0 if D is None else D
    q = f32_to_bf16_bits(_normal(generator("pv", 0, seed), (H, L, D)))
    k = f32_to_bf16_bits(_normal(generator("pv", 1, seed), (H, L, D)))
    v = f32_to_bf16_bits(_normal(generator("pv", 2, seed), (H, L, D)))
    return q, k, v


def pv_probs_t(q_bits, k_bits, causal=True, device="cpu", out=None):
    """Key-major attention probabilities Pt [H, L, L] (torch.bfloat16 on `device`).

    Per head: logits = Q K^T / sqrt(D) in fp32 from the bf16 values, keys after
    the query masked out when causal, row softmax in fp32, rounded to bf16,
    stored transposed so that Pt[h, k, :] is key k's row of probabilities.  The
    stored bits are the input of both the GPU path and the oracle.
    """
    import torch

    H, L, D = q_bits.shape
    if out is None:
        out = torch.empty((H, L, L), dtype=torch.bfloat16, device=device)
    mask = None
    if causal:
        mask = torch.ones((L, L), dtype=torch.bool, device=device).triu_(1)
    for h in range(H):
        qf = torch.from_numpy(bf16_bits_to_f32(q_bits[h])).to(device)
        kf = torch.from_numpy(bf16_bits_to_f32(k_bits[h])).to(device)
        logits = torch.matmul(qf, kf.t().contiguous()) * (1.0 / float(np.sqrt(D)))
        if mask is not None:
            logits.masked_fill_(mask, float("-inf"))
        p = torch.softmax(logits, dim=-1)
        del logits
        out[h].copy_(p.t().to(torch.bfloat16))
        del p
    return out
