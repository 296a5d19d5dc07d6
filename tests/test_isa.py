"""Instruction-level checks on the gfx950 code of this library (CPU only).

The forward and grad_radial must add separately rounded fp32 products (no
fused multiply-add), so the fp32 kernels may contain no v_fma_f32 /
v_fmac_f32 / v_fma_mix and no packed fp32 VALU instructions; the hot kernels
must not spill to scratch.  The assembly is produced from the sources with the
library's own flags (hipcc --cuda-device-only -S).
"""
import os
import re

import pytest

from edge_node_scatter_amd import build as zs_build

@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm")
    texts = {}
    for path in zs_build.device_asm(str(out)):
        texts[os.path.basename(path)] = open(path).read()
    return texts


def _kernels(text):
    """{symbol: body} for every kernel in an assembly file."""
    bodies = {}
    for m in re.finditer(r"^(_Z\S+):[^\n]*\n(.*?)^\s*s_endpgm", text, flags=re.M | re.S):
        bodies[m.group(1)] = m.group(2)
    return bodies


def _meta(text, sym):
    m = re.search(r"\.name:\s+" + re.escape(sym) + r"\s*\n(.*?)(?=\n\s+- \.|\n\s*\.\.\.|\Z)",
                  text, flags=re.S)
    return m.group(1) if m else ""


# The normalised forward computes 1/sqrt(deg) once per node with the correctly
# rounded fp32 square root (v_sqrt_f32 and an fma residual test) followed by
# the IEEE division sequence (div_scale, rcp, fma Newton steps, div_fmas,
# div_fixup).  Those fp32 FMAs are exact-residual steps of the two operations,
# not accumulation; they are cut out (one short block per kernel) before the
# check below.
_SQRT_DIV = re.compile(r"^\s*v_sqrt_f32(?:_e32)?\s.*?^\s*v_div_fixup_f32\b[^\n]*\n", flags=re.M | re.S)


def _strip_sqrt_div(body):
    blocks = _SQRT_DIV.findall(body)
    for b in blocks:
        assert b.count("\n") < 60, "square-root/division block unexpectedly long"
    return _SQRT_DIV.sub("", body), len(blocks)


def test_no_fp32_fma_or_packed_ops(asm):
    seen = norm_blocks = 0
    for name in ("zs_fwd-gfx950.s", "zs_bwd-gfx950.s"):
        for sym, body in _kernels(asm[name]).items():
            seen += 1
            body, nb = _strip_sqrt_div(body)
            normalised = "zs_fwd" in sym and sym.split("NS_8InLayout")[0].endswith("Lb1EEEvPKfS3_")
            # the staged kernel's 4-edge instantiations at <= 4 channels per lane
            # also hold the 8-edge path for heavy nodes: one block per path
            m = re.search(r"zs_fwd_staged_kernelILi(\d+)ELi(\d+)E", sym)
            paths = 2 if m and int(m.group(1)) <= 4 and int(m.group(2)) == 4 else 1
            assert nb == (paths if normalised else 0), sym
            norm_blocks += nb
            bad = re.findall(r"\b(v_fmac?_f32|v_fma_mix\w*|v_pk_(?:fma|mul|add)_f32|v_mad_f32)\b",
                             body)
            assert not bad, f"{sym}: {sorted(set(bad))}"
    assert seen >= 4
    assert norm_blocks >= 2   # every normalised forward instantiation has its block


def test_fp64_channel_sums_use_fma(asm):
    body = "".join(b for s, b in _kernels(asm["zs_bwd-gfx950.s"]).items()
                   if "zs_bwd_staged_kernel" in s)
    assert "v_fma_f64" in body or "v_fmac_f64" in body


def test_kernels_do_not_spill(asm):
    seen = 0
    for name in ("zs_fwd-gfx950.s", "zs_bwd-gfx950.s", "zs_csr-gfx950.s", "zs_norm-gfx950.s"):
        text = asm[name]
        for sym in _kernels(text):
            seen += 1
            meta = _meta(text, sym)
            spill = re.search(r"\.vgpr_spill_count:\s+(\d+)", meta)
            priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", meta)
            assert spill and int(spill.group(1)) == 0, f"{sym} spills VGPRs"
            assert priv and int(priv.group(1)) == 0, f"{sym} uses scratch"
    assert seen >= 10
