"""The kernels that accumulate matrix products in AGPRs through inline
assembly must wait out each product's write latency themselves, since the
compiler does not: the compiled assembly is checked for any instruction that
touches such an AGPR too early, along every control-flow path.  CPU only
(hipcc cross-compiles gfx950)."""
import os
import shutil

import pytest

from exact_io_aware_73_amd import asm_hazards as H
from exact_io_aware_73_amd import build as B

needs_hipcc = pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                                 reason="hipcc not available")

_SNIPPET = """\
kern:
; %bb.0:
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
{between}\tv_accvgpr_read_b32 v8, a3
\ts_endpgm
.Lfunc_end0:
"""


def test_checker_flags_an_early_read():
    bad = H.agpr_hazards(_SNIPPET.format(between=""))["kern"]
    assert len(bad) == 1 and "a3" in bad[0][1]


def test_checker_counts_nops_as_wait_states():
    ok = _SNIPPET.format(between="\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n")
    assert H.agpr_hazards(ok)["kern"] == []
    short = _SNIPPET.format(between="\ts_nop 7\n")
    assert len(H.agpr_hazards(short)["kern"]) == 1


def test_checker_follows_branches():
    asm = """\
kern:
; %bb.0:
\tv_mfma_f32_32x32x16_bf16 a[16:31], v[0:3], v[4:7], a[16:31]
\ts_cbranch_scc1 .LBB0_2
; %bb.1:
\ts_nop 7
\ts_nop 7
\ts_nop 7
\ts_branch .LBB0_3
.LBB0_2:
\tv_accvgpr_mov_b32 a40, a20
.LBB0_3:
\ts_endpgm
.Lfunc_end0:
"""
    bad = H.agpr_hazards(asm)["kern"]
    assert len(bad) == 1 and bad[0][0] == ".LBB0_2"


def test_dependent_products_are_not_violations():
    asm = """\
kern:
; %bb.0:
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[8:11], v[12:15], a[0:15]
\ts_endpgm
.Lfunc_end0:
"""
    assert H.agpr_hazards(asm)["kern"] == []


@needs_hipcc
@pytest.mark.parametrize("source", H.SOURCES)
def test_kernels_wait_out_inline_products(source):
    found = H.agpr_hazards(H.device_asm(source))
    assert found, f"{source}: no kernel with AGPR-accumulating inline products"
    for kernel, bad in found.items():
        assert bad == [], (kernel, bad[:3])
