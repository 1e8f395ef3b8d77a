#!/usr/bin/env python3
"""Benchmark of the Reduced Matrix Multiplication hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: score -> select -> gather -> reduced bf16 MFMA GEMM
(for r = 1 the dense baseline: the same GEMM kernel on A and B in place).  The
B row norms depend only on the weight and are computed once, before timing.

Headline workload: the MLP down-projection, X 4096x14336 bf16 (silu(g) * u,
g, u ~ N(0,1)) times W 14336x4096 bf16 (N(0, 0.02)), one selection per
128-token block, r in {0.5, 0.7, 0.9, 1.0}: the largest linear configuration
(481 GFLOP at r = 1).  `value` is the retained-K TFLOP/s of the whole step at
r = 0.5 (2*M*kk*N / step time); per-r stage times, GEMM-only TFLOP/s and the
speed-ups over r = 1.0 are reported beside it, the step both warm (the same
inputs every step) and cold (inputs rotated over copies larger than the
256 MB last-level cache).  The same line carries, under "configs", every other
configuration (attention projection, decode, P.V at L = 4096 and 16384, the
tiny case), each with its own MFMA or HBM roofline, and under "stages" the
achieved HBM GB/s of the score, select and gather steps.  Other workloads
(--workload attn_proj, decode, decode_q8, pv4k, pv16k, attn4k, attn16k, tiny)
use the same contract; decode_q8 is the decode shape on the int8 weight path;
attn4k and attn16k the attention chain (feature scores and selection,
probabilities producer with the P.V key scores, key selection, reduced P.V).

Every timed pass (whole steps, the per-stage pass, the GEMM back to back, the
cold step) first runs its own work untimed for --settle-ms (30 ms) of GPU time,
then its --warmup steps, then exactly --steps timed steps: after any idle spell
the clocks need about 10 ms of work to reach their steady state.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
_ORACLE_PASS = None
np = None
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "reduced-GEMM TFLOP/s on retained K + speedup vs r=1.0 dense, per r"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--settle-ms", type=float, default=30.0,
                   help="untimed GPU work (ms) each timed pass runs first, so it sees steady-state clocks")
    p.add_argument("--workload", default="mlp_down",
                   choices=["attn_proj", "mlp_down", "decode", "decode_q8", "pv4k", "pv16k", "attn4k", "attn16k",
                            "tiny"])
    p.add_argument("--ratios", type=str, default=None, help="comma-separated r values")
    p.add_argument("--headline-r", type=float, default=0.5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-groups", type=int, default=None, help="row groups the oracle baseline runs")
    p.add_argument("--error-study", action="store_true",
                   help="instead of timing: relative Frobenius error of the reduced product against the r = 1 "
                        "product, for the product score, the activation-only score and random retention")
    p.add_argument("--configs", type=str, default=None,
                   help="comma-separated other workloads measured into the same line (default with the headline "
                        "mlp_down: attn_proj,decode,pv4k,pv16k,tiny; none otherwise); 'none' for none")
    p.add_argument("--no-cold", action="store_true", help="skip the cold-input step timing of the prefill configs")
    p.add_argument("--oracle-pass", type=str, default=None, help=argparse.SUPPRESS)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="before the workload, copy a MIB-MiB buffer 5 times (reference kernel for HBM counters)")
    return p.parse_args()


# ------------------------------------------------------------------ workloads
class Linear:
    """X [M,K] times W [K,N] with per-group selection (attn_proj, mlp_down, decode, tiny;
    decode_q8: the decode inputs with the weight quantised to int8)."""

    # copies of (X, W) the cold step rotates over: more than the 256 MB
    # last-level cache passes between two reads of one copy
    COLD_COPIES = {"attn_proj": 8, "mlp_down": 3}

    def __init__(self, name, dev):
        import numpy as np
        import torch
        from input_adaptive_reduced_02_amd import rmm, synth
        self.rmm, self.torch, self.np = rmm, torch, np
        self.name = name
        self.q8 = name == "decode_q8"
        base = "decode" if self.q8 else name
        self.M, self.K, self.N = synth.FULL_SHAPES[base]
        self.gr = synth.GROUP_ROWS[base]
        self.ratios = synth.RATIOS[base]
        t0 = time.time()
        d = synth.linear_inputs(base)
        self.host = d
        if d["dtype"] == "bf16":
            self.A = torch.from_numpy(d["A"].view(np.int16)).view(torch.bfloat16).to(dev)
            self.B = torch.from_numpy(d["B"].view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            self.A = torch.from_numpy(d["A"]).to(dev)
            self.B = torch.from_numpy(d["B"]).to(dev)
        self.f32 = d["dtype"] == "f32"
        # per-weight work, outside the timed step: B row norms (and for int8
        # weights the quantisation and the norms of the dequantised weight)
        if self.q8:
            self.B, self.scale = rmm.rmm_quantize_q8(self.B)
            self.bnorm = rmm.rmm_rownorms_q8(self.B, self.scale)
        else:
            self.bnorm = rmm.rmm_rownorms(self.B)
        # The decode weight's kept rows (70-470 MB) are the size of the 256 MB
        # last-level cache; steps rotate over copies of the weight (3 of the
        # bf16 weight, 8 of the int8 one) so that between two reads of one copy
        # at least 280 MB of other weight rows stream by, and every step reads
        # its weight from HBM, as a real decode step would.
        copies = {"decode": 3, "decode_q8": 8}.get(name, 1)
        self.decode = copies > 1
        self.As = [self.A]
        self.Bs = [self.B] + [self.B.clone() for _ in range(copies - 1)]
        self._rot = 0
        torch.cuda.synchronize()
        log(f"[bench] {name}: inputs {self.M}x{self.K} @ {self.K}x{self.N} ready in {time.time() - t0:.1f}s")
        self.G = -(-self.M // self.gr)
        self.dev = dev

    def make_cold(self):
        """Copies of X and W for the cold step (the B norms are those of W)."""
        n = self.COLD_COPIES.get(self.name, 1)
        if len(self.As) < n:
            self.As = [self.A] + [self.A.clone() for _ in range(n - 1)]
            self.Bs = [self.B] + [self.B.clone() for _ in range(n - 1)]
            self.torch.cuda.synchronize()
        return n > 1

    def drop_cold(self):
        self.As, self.Bs = [self.A], [self.B] + self.Bs[1:] if self.decode else [self.B]

    def describe(self, r):
        dt = "fp32" if self.f32 else "bf16"
        wdt = "int8 (one binary32 scale per column)" if self.q8 else dt
        return (f"{self.name}: X {self.M}x{self.K} {dt} @ W {self.K}x{self.N} {wdt}, "
                f"{self.gr}-row selection groups, r={r}")

    def stages(self, r, cold=False):
        """([(name, fn)] of one step at ratio r, kk, fn of one GEMM launch for the
        back-to-back pass); buffers are allocated once here.  The first stage
        moves to the next copy of the inputs when they rotate (cold steps:
        X and W; decode: W, also in the back-to-back GEMM launches)."""
        rmm, torch = self.rmm, self.torch
        kk = rmm.rmm_kk(r, self.K)
        self.kk = kk
        rot_a = cold and len(self.As) > 1
        rot_b = (cold and len(self.Bs) > 1) or self.decode

        def adv():
            if rot_a or rot_b:
                self._rot += 1

        A_ = lambda: self.As[self._rot % len(self.As)] if rot_a else self.A
        B_ = lambda: self.Bs[self._rot % len(self.Bs)] if rot_b else self.B
        Y = torch.empty((self.M, self.N), dtype=torch.float32 if self.f32 else torch.bfloat16, device=self.dev)
        if self.q8:
            wq = torch.zeros(max(1, rmm.rmm_gemm_q8_workspace_bytes(self.M, self.N, kk, self.gr)),
                             dtype=torch.uint8, device=self.dev)
        if kk == self.K and not self.f32:
            if self.q8:
                g = lambda: rmm.rmm_gemm_q8(A_(), B_(), self.scale, None, kk, self.gr, Y=Y, ws=wq)
            else:
                g = lambda: rmm.rmm_gemm(A_(), B_(), None, kk, self.gr, Y=Y)
            step = lambda: (adv(), g())
            b2b = lambda: (adv() if self.decode else None, g())
            return [("gemm", step)], kk, b2b
        kpad = rmm.rmm_kk_pad(kk)
        idx = torch.empty((self.G, kpad), dtype=torch.int32, device=self.dev)
        self.idx = idx
        Ap = torch.empty((self.M, kpad), dtype=torch.bfloat16, device=self.dev)
        ws = torch.empty(max(1, rmm.rmm_select_workspace_bytes(self.M, self.K, self.gr)), dtype=torch.uint8,
                         device=self.dev)
        if self.f32:
            Bp = torch.empty((kpad, self.N), dtype=torch.bfloat16, device=self.dev)
            g = lambda: rmm.rmm_gemm(Ap, Bp, None, kk, self.gr, Y=Y)
            return [("select", lambda: (adv(), rmm.rmm_select(A_(), r, self.gr, bnorm=self.bnorm, idx=idx, ws=ws))),
                    ("gather", lambda: rmm.rmm_gather(A_(), idx, kk, self.gr, Apanel=Ap, B=B_(), Bpanel=Bp)),
                    ("gemm", g)], kk, g
        # bf16 activations: selection and gather in one call (one launch after
        # the scores where the shape allows, else the two launches)
        selg = ("select+gather", lambda: (adv(), rmm.rmm_select_gather(A_(), r, self.gr, bnorm=self.bnorm, idx=idx,
                                                                       Apanel=Ap, ws=ws)))
        if self.q8:
            g = lambda: rmm.rmm_gemm_q8(Ap, B_(), self.scale, idx, kk, self.gr, Y=Y, ws=wq)
        else:
            g = lambda: rmm.rmm_gemm(Ap, B_(), idx, kk, self.gr, Y=Y)
        b2b = lambda: (adv() if self.decode else None, g())
        return [selg, ("gemm", g)], kk, b2b

    def anatomy(self, r, steps, warmup):
        """The score, select and gather steps as separate launches (rmm_scores,
        rmm_select_scores, rmm_gather), and the select + gather call of the
        step (scores included), each timed back to back; achieved GB/s on the
        algorithmic bytes of each, against the HBM peak."""
        rmm, torch = self.rmm, self.torch
        if self.f32:
            return None
        kk = rmm.rmm_kk(r, self.K)
        kpad = rmm.rmm_kk_pad(kk)
        M, K, G = self.M, self.K, self.G
        scores = torch.empty((G, K), dtype=torch.float32, device=self.dev)
        idx = torch.empty((G, kpad), dtype=torch.int32, device=self.dev)
        Ap = torch.empty((M, kpad), dtype=torch.bfloat16, device=self.dev)
        ws = torch.empty(max(1, rmm.rmm_select_workspace_bytes(M, K, self.gr)), dtype=torch.uint8, device=self.dev)
        es = 2
        nbytes = {
            "score": M * K * es + K * 8 + G * K * 4,            # X once, the B norms, the scores
            "select": G * K * 4 + G * kpad * 4,                 # the scores, the kept indices
            "gather": M * K * es + G * kpad * 4 + M * kpad * 2,  # whole X rows, the indices, the panel
        }
        nbytes["select+gather"] = nbytes["score"] + G * K * 4 + G * kpad * 4 + M * K * es + M * kpad * 2
        fns = [("score", lambda: rmm.rmm_scores(self.A, self.gr, bnorm=self.bnorm, scores=scores)),
               ("select", lambda: rmm.rmm_select_scores(scores, r, idx=idx)),
               ("gather", lambda: rmm.rmm_gather(self.A, idx, kk, self.gr, Apanel=Ap)),
               ("select+gather", lambda: rmm.rmm_select_gather(self.A, r, self.gr, bnorm=self.bnorm, idx=idx,
                                                                Apanel=Ap, ws=ws))]
        out = {}
        for name, fn in fns:
            ms = back_to_back(torch, fn, steps, warmup)
            gbs = nbytes[name] / (ms * 1e-3) / 1e9
            out[name] = dict(us=round(ms * 1e3, 2), bytes=nbytes[name], gbs=round(gbs, 1),
                             frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
        return out

    def flops(self, r):
        return 2.0 * self.M * self.rmm.rmm_kk(r, self.K) * self.N

    def kept_rows(self, r):
        """B rows kept by at least one group (each is read from HBM at least
        once): kk for one group, up to K for many; from the last selection run."""
        kk = self.rmm.rmm_kk(r, self.K)
        cache = self.__dict__.setdefault("_rows", {})
        if r not in cache:
            if kk == self.K or self.G == 1 or getattr(self, "idx", None) is None or self.idx.shape[1] < kk:
                cache[r] = kk
            else:
                cache[r] = int(self.torch.unique(self.idx[:, :kk]).numel())
        return cache[r]

    def gemm_bytes(self, r):
        """Algorithmic HBM bytes of one reduced-GEMM launch: every B row some
        group keeps, once (int8: one byte per weight, plus the column scales),
        the A panel (or A), and Y."""
        kk = self.rmm.rmm_kk(r, self.K)
        rows = self.kept_rows(r)
        yb = 4 if self.f32 else 2
        brow = (1.0 * rows * self.N + 4.0 * self.N) if self.q8 else 2.0 * rows * self.N
        return brow + 2.0 * self.M * kk + yb * self.M * self.N

    bound = property(lambda self: "hbm" if self.name in ("decode", "decode_q8") else "mfma")

    @property
    def kernel(self):
        return self.kernel_for(0.5)

    def kernel_for(self, r):
        """The kernel the reduced GEMM runs on at ratio r: int8 weights the
        shared-stream kernel for groups of at most 64 rows keeping at most 4096
        rows, else the split-tile one; groups of at most 64 rows the decode
        kernel; prefill shapes with at least 512 tiles of 128 x 256 and bf16
        output two workgroups per CU, other prefill shapes eight waves."""
        if self.q8:
            kk = self.rmm.rmm_kk(r, self.K)
            return "rmm::k_gemm_q8s" if self.gr <= 64 and kk <= 4096 else "rmm::k_gemm_q8"
        if self.gr <= 64:
            return "rmm::k_gemm_sk"
        tiles = self.G * -(-min(self.gr, self.M) // 128) * -(-self.N // 256)
        return "rmm::k_gemm_wb" if tiles >= 512 and not self.f32 else "rmm::k_gemm_dl"

    def cpu_baseline(self, r, groups):
        """The oracle (single-threaded fp64 C) on `groups` row groups at ratio r:
        scores of those groups, selection, reduced product."""
        import oracle as O
        np = self.np
        d = self.host
        widen = O.widen_f32 if self.f32 else O.widen_bf16
        rows = min(self.M, groups * self.gr)
        A64 = widen(d["A"][:rows])
        # per-weight work outside the timed part (as on the GPU)
        if self.q8:
            from input_adaptive_reduced_02_amd import synth
            q, s = O.quantize_q8(synth.bf16_bits_to_f32(d["B"]))
            B64 = O.dequant_q8(q, s)
            b = O.rownorms_q8(q, s)
        else:
            B64 = widen(d["B"])
            b = O.rownorms(B64)
        t0 = time.perf_counter()
        sel = O.select(A64, r, self.gr, b)
        Y = O.reduced(A64, B64, sel["idx"], sel["kk"], self.gr)
        dt = time.perf_counter() - t0
        del Y
        fl = 2.0 * rows * sel["kk"] * self.N
        return dict(value=fl / dt / 1e12, unit="TFLOP/s", cores=1, kind="oracle",
                    sample=f"{rows // self.gr} of {self.G} row groups ({rows} of {self.M} rows) at r={r}: "
                           f"score + select + reduced product, {fl / 1e9:.2f} GFLOP in {dt:.1f} s on one core",
                    seconds=round(dt, 2))


class PV:
    """P.V reduced along keys: 32 heads, head dim 128, 128-query blocks, causal."""

    def __init__(self, L, dev):
        import torch
        from input_adaptive_reduced_02_amd import rmm, synth
        self.rmm, self.torch = rmm, torch
        self.H, self.L, self.D = 32, L, 128
        self.copies = 1
        self.name = f"pv{L // 1024}k"
        self.ratios = synth.RATIOS["pv"]
        self.dev = dev
        t0 = time.time()
        q, k, v = synth.pv_qkv(self.H, L, self.D)
        self.Pt = synth.pv_probs_t(q, k, causal=True, device=dev)
        self.V = torch.from_numpy(v.view("int16")).view(torch.bfloat16).to(dev)
        torch.cuda.synchronize()
        self.G = L // 128
        log(f"[bench] {self.name}: P ({self.H}x{L}x{L} bf16, key-major) ready in {time.time() - t0:.1f}s")

    def describe(self, r):
        return (f"{self.name}: P.V, {self.H} heads, L={self.L}, head dim {self.D}, bf16, causal, "
                f"128-query blocks, r={r}")

    def _kks(self, r):
        return [self.rmm.rmm_kk(r, min(self.L, 128 * (g + 1))) for g in range(self.G)]

    def stages(self, r, cold=False):
        rmm, torch = self.rmm, self.torch
        O_ = torch.empty((self.H, self.L, self.D), dtype=torch.bfloat16, device=self.dev)
        self.kk = max(self._kks(r))
        if r >= 1.0:
            g = lambda: rmm.rmm_pv_gemm(self.Pt, self.V, 1.0, None, O=O_)
            return [("gemm", g)], self.kk, g
        idx = torch.empty((self.H * self.G, rmm.rmm_kk_pad(self.L)), dtype=torch.int32, device=self.dev)
        need = rmm.rmm_attn_pv_workspace_bytes(self.H, self.L, self.D, r, have_idx_out=True)
        ws = torch.empty(max(1, need), dtype=torch.uint8, device=self.dev)
        g = lambda: rmm.rmm_pv_gemm(self.Pt, self.V, r, idx, O=O_)
        return [("select", lambda: rmm.rmm_pv_select(self.Pt, self.V, r, idx_out=idx, ws=ws)),
                ("gemm", g)], self.kk, g

    def select_bytes(self, r):
        """Algorithmic HBM bytes of the P.V scoring and selection: the causal
        part of Pt and V read once, the block scores written and read once,
        the kept-key lists written."""
        pt = sum(128 * min(self.L, 128 * (g + 1)) * 2.0 for g in range(self.G)) * self.H
        sc = sum(min(self.L, 128 * (g + 1)) * 4.0 * 2 for g in range(self.G)) * self.H
        return pt + 2.0 * self.H * self.L * self.D + sc + 4.0 * sum(self._kks(r)) * self.H

    def flops(self, r):
        return sum(2.0 * 128 * kk * self.D for kk in self._kks(r)) * self.H

    def gemm_bytes(self, r):
        kept_p = sum(kk * 128 * 2.0 for kk in self._kks(r)) * self.H
        return kept_p + 2.0 * 2 * self.H * self.L * self.D   # + V once, + O once

    bound = property(lambda self: "hbm")
    kernel = "rmm::k_pv_gemm"

    def cpu_baseline(self, r, groups):
        import numpy as np

        import oracle as O
        # `groups` (head 0, block) pairs from the end of the sequence (the heaviest)
        Pt0 = self.Pt[0].cpu().view(torch_int16(self.torch)).numpy().view(np.uint16)
        V0 = self.V[0].cpu().view(torch_int16(self.torch)).numpy().view(np.uint16)
        fl = 0.0
        t0 = time.perf_counter()
        for g in range(self.G - 1, max(-1, self.G - 1 - groups), -1):
            sel = O.pv_select_block(Pt0, V0, self.L, 128, g, r, True)
            O.pv_block(sel["Ptb"], sel["V"], sel["idx"])
            fl += 2.0 * 128 * sel["kk"] * self.D
        dt = time.perf_counter() - t0
        return dict(value=fl / dt / 1e12, unit="TFLOP/s", cores=1, kind="oracle",
                    sample=f"{groups} query blocks of head 0 (the last ones) at r={r}: score + select + "
                           f"reduced P.V, {fl / 1e9:.2f} GFLOP in {dt:.1f} s", seconds=round(dt, 2))


class Attn:
    """Causal attention with both attention-side reductions: QK^T over the kept
    features of each 128-query block (the probabilities producer), then P.V
    over the kept keys chosen from the scores the producer emits.  32 heads,
    head dim 128.  One r for both reductions; r = 1 is the dense producer and
    the dense causal P.V."""

    def __init__(self, L, dev):
        import torch
        from input_adaptive_reduced_02_amd import rmm, synth
        self.rmm, self.torch = rmm, torch
        self.H, self.L, self.D = 32, L, 128
        self.copies = 1
        self.name = f"attn{L // 1024}k"
        self.ratios = synth.RATIOS["pv"]
        self.dev = dev
        self.G = L // 128
        q, k, v = synth.pv_qkv(self.H, L, self.D)
        self.q_bits, self.k_bits, self.v_bits = q, k, v
        up = lambda b: torch.from_numpy(b.view("int16")).view(torch.bfloat16).to(dev)
        self.Q, self.K, self.V = up(q), up(k), up(v)
        self.Pt = torch.empty((self.H, L, L), dtype=torch.bfloat16, device=dev)
        self.pvs = torch.empty((self.H, self.G, L), dtype=torch.float32, device=dev)
        self.idx_qk = torch.empty((self.H * self.G, rmm.rmm_kk_pad(self.D)), dtype=torch.int32, device=dev)
        self.idx_pv = torch.empty((self.H * self.G, rmm.rmm_kk_pad(L)), dtype=torch.int32, device=dev)
        self.O = torch.empty((self.H, L, self.D), dtype=torch.bfloat16, device=dev)
        self.qs = torch.empty((self.H, self.G, self.D), dtype=torch.float32, device=dev)
        self.wsq = torch.empty(int(rmm.lib().rmm_qk_select_workspace_bytes(self.H, L, self.D, 128, 1)),
                               dtype=torch.uint8, device=dev)
        need = int(rmm.lib().rmm_attn_probs_workspace_bytes(self.H, L, self.D, 1))
        self.wsp = torch.empty(need, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def describe(self, r):
        return (f"{self.name}: causal attention producer (QK^T over kept features, softmax, key-major P, "
                f"P.V key scores) + P.V over kept keys, {self.H} heads, L={self.L}, head dim {self.D}, bf16, "
                f"128-query blocks, r={r} for both")

    def _kks(self, r):
        return [self.rmm.rmm_kk(r, min(self.L, 128 * (g + 1))) for g in range(self.G)]

    def stages(self, r, cold=False):
        rmm = self.rmm
        if r >= 1.0:
            probs = lambda: rmm.rmm_attn_probs(self.Q, self.K, None, 1.0, Pt=self.Pt)
            return [("probs", probs),
                    ("gemm", lambda: rmm.rmm_pv_gemm(self.Pt, self.V, 1.0, None, O=self.O))], self.D, probs
        probs = lambda: rmm.rmm_attn_probs(self.Q, self.K, self.idx_qk, r, Pt=self.Pt, V=self.V,
                                           pv_scores=self.pvs, ws=self.wsp)
        return [("score", lambda: rmm.rmm_qk_select(self.Q, self.K, r, idx_out=self.idx_qk, scores_out=self.qs,
                                                          ws=self.wsq)),
                ("probs", probs),
                ("select", lambda: rmm.rmm_pv_select_scores(self.pvs, r, idx_out=self.idx_pv)),
                ("gemm", lambda: rmm.rmm_pv_gemm(self.Pt, self.V, r, self.idx_pv, O=self.O))], \
            self.rmm.rmm_kk(r, self.D), probs

    roof_stage = "probs"

    def flops(self, r):
        """The method's retained work, each product counted once: QK^T over
        the kept features on the causal prefixes, P.V over the kept keys."""
        kq = self.rmm.rmm_kk(r, self.D)
        qk = sum(2.0 * 128 * min(self.L, 128 * (g + 1)) * kq for g in range(self.G)) * self.H
        pv = sum(2.0 * 128 * kk * self.D for kk in self._kks(r)) * self.H
        return qk + pv

    def gemm_bytes(self, r):
        """Algorithmic HBM bytes of one producer launch: Q and K read once, the
        causal half of Pt written, and (r < 1) the P.V scores written and the
        V norms read once."""
        pt = sum(128 * min(self.L, 128 * (g + 1)) * 2.0 for g in range(self.G)) * self.H
        qk = 2.0 * 2 * self.H * self.L * self.D
        extra = 0.0
        if r < 1.0:
            extra = sum(min(self.L, 128 * (g + 1)) * 4.0 for g in range(self.G)) * self.H + 8.0 * self.H * self.L
        return pt + qk + extra

    bound = property(lambda self: "hbm")
    kernel = "rmm::k_attn_probs<1>"
    profile_prefix = "k_attn_probs"

    def cpu_baseline(self, r, groups):
        import numpy as np

        import oracle as O
        groups = min(groups, self.H * self.G)
        heads = {}
        fl = 0.0
        t0 = time.perf_counter()
        for i in range(groups):
            # the query blocks of head 0, heaviest first, then those of head 1, ...
            h, g = i // self.G, self.G - 1 - i % self.G
            if h not in heads:
                heads.clear()
                heads[h] = tuple(O.widen_bf16(x[h]) for x in (self.q_bits, self.k_bits, self.v_bits))
            Q0, K0, V0 = heads[h]
            sel = O.qk_select_block(Q0, K0, 128, g, r, True, True)
            P = O.attn_probs(Q0, K0, g * 128, 128, True, sel["idx"])
            Kg = min(self.L, 128 * (g + 1))
            Ptb = np.ascontiguousarray(P[:, :Kg].T)
            s64, s32 = O.pv_scores(Ptb, V0[:Kg])
            kk = O.kk(r, Kg)
            O.pv_block(Ptb, V0[:Kg], O.topk(s32, kk))
            fl += 2.0 * 128 * Kg * sel["kk"] + 2.0 * 128 * kk * self.D
        dt = time.perf_counter() - t0
        return dict(value=fl / dt / 1e12, unit="TFLOP/s", cores=1, kind="oracle",
                    sample=f"{groups} query blocks (per head from the last, heads in order) at r={r}: "
                           f"feature scores + select + probabilities + key scores + select + reduced P.V, "
                           f"{fl / 1e9:.2f} GFLOP in {dt:.1f} s",
                    seconds=round(dt, 2))


def torch_int16(torch):
    return torch.int16


# ------------------------------------------------------------------ timing
SETTLE_MS = 30.0   # --settle-ms


def settle(torch, fn):
    """Run `fn` untimed until the GPU has been busy with it for SETTLE_MS.
    After an idle spell (input generation, a CPU baseline, another pass's
    synchronisation) the clocks take about 10 ms of work to ramp up: the
    mlp_down r = 0.5 step measured 362 us over its first 20 steps, 328 over
    the next 20 and 302-311 from then on, and 352 again after 0.5 s idle.  So
    every timed pass first settles on its own work, then runs its warmup
    steps, then its timed steps."""
    if SETTLE_MS <= 0:
        return
    s = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    a.record(s)
    while True:
        for _ in range(4):
            fn()
        b = torch.cuda.Event(enable_timing=True)
        b.record(s)
        b.synchronize()
        if a.elapsed_time(b) >= SETTLE_MS:
            return


def back_to_back(torch, fn, steps, warmup):
    """ms per launch of `fn` run `steps` times back to back between two events
    on the launch stream, after the settling runs and `warmup` untimed runs:
    the kernel's duration plus the small gap between queued launches."""
    settle(torch, fn)
    for _ in range(warmup):
        fn()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_stages(torch, stages, steps, warmup, b2b):
    """Warm up, then time `steps` whole steps (no events inside); in a second
    pass, each stage with events on the launch stream around it; in a third,
    `steps` launches of the roofline kernel's call `b2b` back to back (events
    around a single launch would add its launch latency).  Returns
    (ms_per_step, {stage: mean ms}, ms per back-to-back launch)."""
    def one():
        for _, fn in stages:
            fn()
    settle(torch, one)
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(steps):
        for _, fn in stages:
            fn()
    e1.record(s)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        for j, (_, fn) in enumerate(stages):
            evs[i][j].record(s)
            fn()
        evs[i][-1].record(s)
    torch.cuda.synchronize()
    per = {}
    for j, (name, _) in enumerate(stages):
        per[name] = sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)) / steps
    return ms_step, per, back_to_back(torch, b2b, steps, 0)


def step_time(torch, stages, steps, warmup):
    """ms per whole step, `steps` steps between two events after `warmup`."""
    def one():
        for _, fn in stages:
            fn()
    return back_to_back(torch, one, steps, warmup)


# ------------------------------------------------------------------ HBM traffic
# sources of the kernel the roofline is taken on, per workload family
GEMM_SOURCES = {
    "linear": ["rmm_gemm.hip", "rmm_gemm_dl.h", "rmm_gemm_sk.h", "rmm_gemm_wt.h", "rmm_gemm_wb.h", "rmm_tile.h",
               "rmm_internal.h"],
    "pv": ["rmm_pv.hip", "rmm_tile.h", "rmm_internal.h"],
    "q8": ["rmm_q8.hip", "rmm_gemm_dl.h", "rmm_tile.h", "rmm_internal.h"],
    "attn": ["rmm_attn.hip", "rmm_tile.h", "rmm_internal.h"],
}


def source_family(workload):
    if workload.startswith("attn") and workload != "attn_proj":
        return "attn"
    return "pv" if workload.startswith("pv") else "q8" if workload.endswith("_q8") else "linear"


def gemm_source_hash(family="linear"):
    """sha256 over the GEMM kernel sources of a workload family, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES[family]:
        with open(os.path.join(ROOT, "input_adaptive_reduced_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, r, prefix="k_gemm"):
    """HBM bytes per launch of the roofline kernel from the committed counter
    summary of this workload and ratio (profiles/<prefix>_<workload>_r<r>_traffic.txt,
    prefix the kernel's name), or None when there is none or the kernel's
    sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{prefix}_{workload}_r{r}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != gemm_source_hash(source_family(workload)):
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, mib, dev):
    """A plain device-to-device copy of known size, run before the workload so
    that a counter profile of this command holds a reference dispatch."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
        torch.cuda.synchronize()
    log(f"[bench] copy calibration: 5 copies of {mib} MiB")
    del src, dst


def error_study(torch, dev):
    """Selection quality on the synthetic linear workloads: for every r < 1,
    ||Y_r - Y_1||_F / ||Y_1||_F with Y_1 the r = 1 product, for the product score
    (with B norms), the pages' activation-only score, and a seeded uniformly
    random kept set of the same size (the pages' random-pruning baseline).
    Every product runs through the hot-path kernels with binary32 outputs; the
    product rule also reports its Frobenius bound sqrt(sum_g beta_g^2) relative
    to ||Y_1||_F."""
    import numpy as np
    rows = []
    for name in ("attn_proj", "mlp_down", "decode"):
        W = Linear(name, dev)
        rmm = W.rmm
        M, K, gr = W.M, W.K, W.gr
        G = -(-M // gr)
        Y1 = rmm.rmm_gemm(W.A, W.B, None, K, gr, ydt=torch.float32).double()
        n1 = torch.linalg.norm(Y1).item()
        rng = np.random.default_rng(0)
        for r in [x for x in W.ratios if x < 1.0]:
            kk = rmm.rmm_kk(r, K)
            kpad = rmm.rmm_kk_pad(kk)
            for rule in ("product", "activation_only", "random"):
                bound = None
                if rule == "product":
                    bound = torch.empty(G, dtype=torch.float64, device=dev)
                    idx = rmm.rmm_select(W.A, r, gr, bnorm=W.bnorm, bound=bound)
                elif rule == "activation_only":
                    idx = rmm.rmm_select(W.A, r, gr)
                else:
                    ix = np.empty((G, kpad), np.int32)
                    for g in range(G):
                        ix[g, :kk] = np.sort(rng.choice(K, kk, replace=False))
                        ix[g, kk:] = ix[g, kk - 1]
                    idx = torch.from_numpy(ix).to(dev)
                Ap, _ = rmm.rmm_gather(W.A, idx, kk, gr)
                Y = rmm.rmm_gemm(Ap, W.B, idx, kk, gr, ydt=torch.float32).double()
                row = dict(workload=name, r=r, kk=kk, rule=rule,
                           rel_frob=round(torch.linalg.norm(Y - Y1).item() / n1, 6))
                if bound is not None:
                    row["rel_bound"] = round(torch.sqrt((bound ** 2).sum()).item() / n1, 6)
                rows.append(row)
                log(f"[study] {name} r={r} {rule}: {row['rel_frob']}" +
                    (f" (bound {row['rel_bound']})" if bound is not None else ""))
        del W
        torch.cuda.empty_cache()
    print(json.dumps({"study": "selection_error", "data": "synthetic",
                      "unit": "relative Frobenius error against the r = 1 product", "rows": rows}), flush=True)


def make_workload(name, dev):
    if name in ("pv4k", "pv16k"):
        return PV(4096 if name == "pv4k" else 16384, dev)
    if name in ("attn4k", "attn16k"):
        return Attn(4096 if name == "attn4k" else 16384, dev)
    return Linear(name, dev)


def roofline(W, r, gemm_ms):
    """The GEMM's (the attention chain: the producer's) roofline at ratio r on
    its back-to-back launch time: MFMA-bound prefill GEMMs on retained FLOP,
    the rest on algorithmic HBM bytes."""
    if W.bound == "mfma":
        achieved = W.flops(r) / (gemm_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4))
    else:
        achieved = W.gemm_bytes(r) / (gemm_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4))
    roof["traffic"] = measured_traffic(W.name, r, getattr(W, "profile_prefix", "k_gemm"))
    roof["kernel"] = W.kernel_for(r) if hasattr(W, "kernel_for") else W.kernel
    roof["kernel_ms"] = round(gemm_ms, 5)
    return roof


def rounded(v):
    if isinstance(v, float):
        return round(v, 5)
    if isinstance(v, dict):
        return {k: rounded(x) for k, x in v.items()}
    return v


def measure(torch, W, ratios, steps, warmup, headline, cold):
    """Every r of one workload: the warm step, its stages, the GEMM back to
    back, the speed-ups over r = 1, and (prefill configurations) the cold step
    on rotated inputs; the roofline at the headline r."""
    per_r = {}
    for r in ratios:
        stages, kk, b2b = W.stages(r)
        ms_step, per, gemm_ms = time_stages(torch, stages, steps, warmup, b2b)
        fl = W.flops(r)
        rec = dict(kk=kk, ms_per_step=ms_step, stage_ms=per, gemm_ms=gemm_ms,
                   step_tflops=fl / (ms_step * 1e-3) / 1e12,
                   gemm_tflops=fl / (gemm_ms * 1e-3) / 1e12,
                   gemm_gbs=W.gemm_bytes(r) / (gemm_ms * 1e-3) / 1e9)
        if hasattr(W, "select_bytes") and "select" in per:
            rec["select_gbs"] = W.select_bytes(r) / (per["select"] * 1e-3) / 1e9
        del stages
        if cold and isinstance(W, Linear) and W.make_cold():
            cstages, _, _ = W.stages(r, cold=True)
            rec["ms_per_step_cold"] = step_time(torch, cstages, steps, warmup)
            rec["step_tflops_cold"] = fl / (rec["ms_per_step_cold"] * 1e-3) / 1e12
            del cstages
        per_r[r] = rec
        log(f"[bench] {W.name} r={r}: kk={kk} step {ms_step * 1e3:.1f} us"
            + (f" (cold {rec['ms_per_step_cold'] * 1e3:.1f} us)" if "ms_per_step_cold" in rec else "")
            + ", stages " + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in per.items())
            + f"; {getattr(W, 'roof_stage', 'gemm')} back to back {gemm_ms * 1e3:.1f} us, "
            f"{rec['gemm_tflops']:.1f} TFLOP/s {rec['gemm_gbs']:.0f} GB/s")
    if isinstance(W, Linear):
        W.drop_cold()
        torch.cuda.empty_cache()
    base = per_r[1.0]
    for r, v in per_r.items():
        v["speedup_step_vs_r1"] = base["ms_per_step"] / v["ms_per_step"]
        v["speedup_gemm_vs_r1"] = base["gemm_ms"] / v["gemm_ms"]
        if "ms_per_step_cold" in v and "ms_per_step_cold" in base:
            v["speedup_step_cold_vs_r1"] = base["ms_per_step_cold"] / v["ms_per_step_cold"]
    return per_r, roofline(W, headline, per_r[headline]["gemm_ms"])


def host_description():
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def _oracle_group(g):
    """One row group of the parallel oracle pass (runs in a forked worker)."""
    import oracle as O
    A64, B64, b, r, gr = _ORACLE_PASS
    rows = A64[g * gr:(g + 1) * gr]
    sel = O.select(rows, r, gr, b)
    Y = O.reduced(rows, B64, sel["idx"], sel["kk"], gr)
    return 2.0 * rows.shape[0] * sel["kk"] * B64.shape[1], float(np.abs(Y).sum())


def oracle_pass(spec):
    """The oracle over every row group of a linear workload at ratio r, groups
    in parallel over `workers` processes, each group one single-threaded oracle
    call (score, select, reduced product).  Runs in a child process that never
    touches the GPU; prints one JSON line."""
    global _ORACLE_PASS, np
    import multiprocessing as mp

    import numpy as np

    import oracle as O
    from input_adaptive_reduced_02_amd import synth
    name, r, workers = spec.split(":")
    r, workers = float(r), int(workers)
    d = synth.linear_inputs(name)
    widen = O.widen_f32 if d["dtype"] == "f32" else O.widen_bf16
    A64, B64 = widen(d["A"]), widen(d["B"])
    b = O.rownorms(B64)   # per weight, outside the timed part (as on the GPU)
    gr = synth.GROUP_ROWS[name]
    G = -(-A64.shape[0] // gr)
    _ORACLE_PASS = (A64, B64, b, r, gr)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.map(_oracle_group, range(G), chunksize=1)
    wall = time.perf_counter() - t0
    fl = sum(x for x, _ in res)
    print(json.dumps(dict(workload=name, r=r, groups=G, workers=workers, wall_s=round(wall, 2),
                          gflop=round(fl / 1e9, 2), tflops=fl / wall / 1e12)), flush=True)


def run_oracle_pass(name, r, workers):
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--oracle-pass", f"{name}:{r}:{workers}"]
    t0 = time.time()
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if p.returncode != 0:
        log(f"[bench] parallel oracle pass failed ({p.returncode}): {p.stderr[-500:]}")
        return None
    out = json.loads(p.stdout.strip().splitlines()[-1])
    log(f"[bench] parallel oracle pass: {out['groups']} groups on {out['workers']} processes, "
        f"{out['gflop']} GFLOP in {out['wall_s']} s ({time.time() - t0:.1f} s with input generation)")
    return out


def main():
    global SETTLE_MS
    args = parse()
    SETTLE_MS = args.settle_ms
    if args.oracle_pass:
        oracle_pass(args.oracle_pass)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): this build has no "
              "multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    linear = args.workload in ("attn_proj", "mlp_down", "decode", "decode_q8", "tiny")
    # the oracle over the whole headline workload, in parallel over the host's
    # cores (at most 16 processes), before the GPU is touched
    par = None
    if not args.no_cpu_baseline and linear and not args.error_study:
        workers = max(1, min(16, os.cpu_count() or 1))
        par = run_oracle_pass("decode" if args.workload == "decode_q8" else args.workload, args.headline_r,
                              workers)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    if args.error_study:
        error_study(torch, dev)
        return
    if args.copy_calibration > 0:
        copy_calibration(torch, args.copy_calibration, dev)
    W = make_workload(args.workload, dev)
    ratios = [float(x) for x in args.ratios.split(",")] if args.ratios else list(W.ratios)
    if 1.0 not in ratios:
        ratios.append(1.0)
    headline = args.headline_r if args.headline_r in ratios else ratios[0]
    cold = not args.no_cold
    per_r, roof = measure(torch, W, ratios, args.steps, args.warmup, headline, cold)
    h = per_r[headline]
    stages = W.anatomy(headline, args.steps, args.warmup) if isinstance(W, Linear) else None
    if stages:
        log("[bench] stages at r=%s: " % headline + ", ".join(
            f"{k} {v['us']:.1f} us {v['gbs']:.0f} GB/s ({v['frac_hbm']:.2f} of HBM)" for k, v in stages.items()))

    cpu = None
    if not args.no_cpu_baseline:
        groups = args.cpu_groups
        if groups is None:
            groups = {"attn_proj": 24, "mlp_down": 8, "decode": 1, "decode_q8": 1, "tiny": 1, "pv4k": 32,
                      "pv16k": 128, "attn4k": 512, "attn16k": 96}[W.name]
        log(f"[bench] oracle baseline on {groups} groups ...")
        cpu = W.cpu_baseline(headline, groups)
        host_cores, model = host_description()
        cpu["host_cores"] = host_cores
        cpu["cpu_model"] = model
        if par is not None:
            cpu["parallel"] = dict(groups=par["groups"], workers=par["workers"], wall_s=par["wall_s"],
                                   gflop=par["gflop"], value=par["tflops"], unit="TFLOP/s",
                                   sample=f"every row group of {par['workload']} at r={par['r']}, one "
                                          f"single-threaded oracle process per group, {par['workers']} at once")
        log(f"[bench] oracle: {cpu['value'] * 1e3:.3f} GFLOP/s on one core ({cpu['seconds']} s); host has "
            f"{host_cores} cores ({model})")

    # the other configurations, each with its own roofline
    if args.configs is None:
        extra = ["attn_proj", "decode", "pv4k", "pv16k", "tiny"] if args.workload == "mlp_down" else []
    elif args.configs == "none":
        extra = []
    else:
        extra = [x for x in args.configs.split(",") if x and x != args.workload]
    configs = {}
    del W
    torch.cuda.empty_cache()
    for name in extra:
        X = make_workload(name, dev)
        xr = list(X.ratios) + ([1.0] if 1.0 not in X.ratios else [])
        xh = 0.5 if 0.5 in xr else xr[0]
        xper, xroof = measure(torch, X, xr, args.steps, args.warmup, xh, cold)
        rec = dict(workload=X.describe(xh), per_r={str(r): rounded(v) for r, v in xper.items()}, roofline=xroof)
        if isinstance(X, Linear) and not X.f32:
            rec["stages"] = X.anatomy(xh, args.steps, args.warmup)
        configs[name] = rec
        del X
        torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": round(h["step_tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(h["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded stand-in for the pages' model activations and weights)",
        "config": {"workload": make_description(args.workload, headline), "r": headline,
                   "parallelism": "single GPU",
                   **({"weights": "int8"} if args.workload == "decode_q8" else {})},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_r": {str(r): rounded(v) for r, v in per_r.items()},
        "stages": stages,
        "configs": configs,
    }
    print(json.dumps(out), flush=True)


def make_description(name, r):
    from input_adaptive_reduced_02_amd import synth
    if name in ("pv4k", "pv16k", "attn4k", "attn16k"):
        L = 4096 if name.endswith("4k") else 16384
        kind = "P.V" if name.startswith("pv") else "causal attention producer + P.V"
        return f"{name}: {kind}, 32 heads, L={L}, head dim 128, bf16, causal, 128-query blocks, r={r}"
    base = "decode" if name == "decode_q8" else name
    M, K, N = synth.FULL_SHAPES[base]
    dt = "fp32" if name == "tiny" else "bf16"
    wdt = "int8 (one binary32 scale per column)" if name == "decode_q8" else dt
    return f"{name}: X {M}x{K} {dt} @ W {K}x{N} {wdt}, {synth.GROUP_ROWS[base]}-row selection groups, r={r}"


if __name__ == "__main__":
    main()
