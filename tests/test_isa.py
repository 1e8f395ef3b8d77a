"""Static checks of the gfx950 code hipcc generates for csrc/*.hip (CPU only).

* no kernel uses scratch (private segment) memory: a staged array that fails
  to stay in registers turns every access into a slow memory round trip;
* no packed-fp32 arithmetic (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32): the
  build disables it, this makes sure it stays disabled;
* m0 is written only by the DMA sequences (s_mov_b32 m0, sN directly followed
  by a global_load_lds_*), so nothing else relies on its value;
* every kernel's static LDS fits one CU (160 KiB);
* the streams a launch touches once keep their non-temporal policy (the `nt`
  modifier): the attention producer's P stores, the P.V kernel's P loads, the
  decode GEMMs' kept-row loads, the prefill GEMM's Y stores and the fused
  select+gather's panel stores.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from input_adaptive_reduced_02_amd import build as B

HIPCC = B.HIPCC
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

LDS_LIMIT = 160 * 1024


@pytest.fixture(scope="module")
def device_asm():
    tmp = tempfile.mkdtemp(prefix="rmm_isa_")

    def one(src):
        out = os.path.join(tmp, os.path.splitext(src)[0] + ".s")
        cmd = [HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, open(out).read()

    try:
        with cf.ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as ex:
            yield dict(ex.map(one, B.SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def kernels(asm):
    """(name, metadata dict) for every kernel in the metadata block."""
    meta = asm[asm.find("amdhsa.kernels:"):]
    out = []
    for blk in re.split(r"\n  - ", meta)[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk)
        if not name:
            continue
        fields = dict(re.findall(r"\.(private_segment_fixed_size|group_segment_fixed_size):\s+(\d+)", blk))
        out.append((name.group(1), {k: int(v) for k, v in fields.items()}))
    return out


def test_every_source_has_kernels(device_asm):
    with_kernels = [src for src, asm in device_asm.items() if kernels(asm)]
    assert "rmm_gemm.hip" in with_kernels and "rmm_select.hip" in with_kernels


def test_no_scratch(device_asm):
    bad = [(src, n, m["private_segment_fixed_size"]) for src, asm in device_asm.items()
           for n, m in kernels(asm) if m.get("private_segment_fixed_size", 0) != 0]
    assert not bad, bad


def test_lds_fits_a_cu(device_asm):
    bad = [(src, n, m["group_segment_fixed_size"]) for src, asm in device_asm.items()
           for n, m in kernels(asm) if m.get("group_segment_fixed_size", 0) > LDS_LIMIT]
    assert not bad, bad


def test_no_packed_fp32(device_asm):
    pat = re.compile(r"^\s*v_pk_(add|mul|fma)_f32\b", re.M)
    bad = [src for src, asm in device_asm.items() if pat.search(asm)]
    assert not bad, bad


def test_m0_only_feeds_dma(device_asm):
    for src, asm in device_asm.items():
        lines = [ln.strip() for ln in asm.splitlines() if ln.strip() and not ln.strip().startswith(";")]
        for i, ln in enumerate(lines):
            if re.search(r"\bm0\b", ln) and not ln.startswith("global_load_lds"):
                assert re.match(r"s_mov_b32 m0, s\d+$", ln), (src, ln)
                assert lines[i + 1].startswith("global_load_lds"), (src, ln, lines[i + 1])


def kernel_bodies(asm, part):
    """{mangled name: body} for every kernel whose mangled name contains `part`."""
    out = {}
    for m in re.finditer(r"^(_Z\S*" + part + r"\S*):[^\n]*$", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        out[m.group(1)] = asm[m.end():end]
    return out


# (source, kernel, instruction, every instantiation or at least one): the
# prefill GEMM's non-bf16 epilogue and the select kernels without a fused
# gather have no such stream
NT_STREAMS = [
    ("rmm_attn.hip", "k_attn_probs", "buffer_store_dwordx4", True),
    ("rmm_pv.hip", "k_pv_gemm", "global_load_lds_dwordx4", True),
    ("rmm_score.hip", "k_pv_mass", "global_load_dwordx4", True),
    ("rmm_gemm.hip", "k_gemm_sk", "global_load_lds_dwordx4", True),
    ("rmm_gemm.hip", "k_gemm_sk", "global_store_dwordx4", True),
    ("rmm_q8.hip", "k_gemm_q8", "global_load_lds_dwordx4", True),
    ("rmm_gemm.hip", "k_gemm_dl", "global_store_dwordx4", False),
    ("rmm_gemm.hip", "k_gemm_wt", "global_store_dwordx4", True),
    ("rmm_gemm.hip", "k_gemm_wb", "global_store_dwordx4", True),
    ("rmm_gather.hip", "k_gather_rows", "global_store_dwordx4", True),
    ("rmm_select.hip", "k_select", "global_store_dwordx4", False),
]


@pytest.mark.parametrize("src,kernel,insn,every", NT_STREAMS, ids=[f"{k}-{i}" for _, k, i, _ in NT_STREAMS])
def test_nontemporal_streams(device_asm, src, kernel, insn, every):
    bodies = kernel_bodies(device_asm[src], kernel)
    assert bodies, f"no {kernel} in {src}"
    has = {name: bool(re.search(r"^\s*" + insn + r"\b[^\n]*\bnt\b", body, re.M)) for name, body in bodies.items()}
    if every:
        assert all(has.values()), [n for n, v in has.items() if not v]
    else:
        assert any(has.values()), list(has)
