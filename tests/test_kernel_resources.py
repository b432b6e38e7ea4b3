"""Register and LDS budgets of the kernels in the built library (CPU: the code objects' metadata notes).

Each kernel's speed rests on an occupancy plan: the 64-key dK/dV kernel and the wide-head kernels run one
wave per SIMD (at most 512 registers, arch and accumulation together), the dQ kernels, the 128-key dK/dV
layouts and the stored-dS pass two (at most 256), and the LDS of the workgroups a CU holds must fit its
160 KB. A change that breaks a plan, or makes a hot loop spill, would otherwise show only as a slower
bench line; here it fails by name. Spills the code carries on purpose are listed with their reason.
"""
import os
import re
import subprocess
import tempfile

import pytest

from attention_backward_fa_amd import binding as B
from tests import asm_hazards as A

LDS_PER_CU = 160 * 1024


def _notes(lib):
    """{mangled kernel name: (template arguments, vgpr_count, vgpr spills, LDS bytes)} over every
    code object of the library (kernels instantiated in several units appear once)."""
    out = {}
    for obj in A.code_objects(lib):
        with tempfile.NamedTemporaryFile(suffix=".o") as f:
            f.write(obj)
            f.flush()
            text = subprocess.run([f"{A.LLVM}/llvm-readobj", "--notes", f.name], check=True, capture_output=True,
                                  text=True).stdout
        for blk in text.split(".args:")[1:]:
            name = re.search(r"\.name:\s+(\S+)", blk)
            if not name:
                continue

            def num(key):
                m = re.search(r"\.%s:\s+(\d+)" % re.escape(key), blk)
                return int(m.group(1)) if m else 0

            mangled = name.group(1)
            args = [int(v) for _, v in re.findall(r"L([ib])(\d+)E", mangled.split("I", 1)[1])] if "I" in mangled else []
            out[mangled] = (args, num("vgpr_count"), num("vgpr_spill_count"), num("group_segment_fixed_size"))
    return out


@pytest.fixture(scope="module")
def notes():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("library not built")
    return _notes(B.LIB_PATH)


def _kernels(notes, prefix):
    found = {k: v for k, v in notes.items() if k.startswith(prefix)}
    assert found, f"no kernel {prefix} in the library"
    return found


def test_64key_dkdv_kernel_one_wave_per_simd(notes):
    # <causal, stores dS, window>: 512 registers, one workgroup per CU; the non-causal instances keep one
    # register in scratch, stored once before the step loop and loaded once after it
    for name, (args, vgpr, spill, lds) in _kernels(notes, "_ZN2fa13fa_bwd_dkdv64I").items():
        causal = args[0] == 1
        assert vgpr <= 512 and lds <= LDS_PER_CU, name
        assert spill == 0 if causal else spill <= 1, name


def test_stored_ds_pass_two_waves_per_simd(notes):
    # <DQ, exact, pieces, causal, window, waves>: two workgroups of four waves per CU, or one of eight
    for name, (args, vgpr, spill, lds) in _kernels(notes, "_ZN2fa12fa_bwd_dq_dsI").items():
        waves = args[5]
        assert waves in (4, 8), name
        assert vgpr <= 256 and spill == 0 and (8 // waves) * lds <= LDS_PER_CU, name


def test_dq_kernel_budgets(notes):
    # <DQ, DV, causal, window, exact, key groups>: heads up to 128 two waves per SIMD (two workgroups of
    # four waves per CU, or one of two key groups), wider heads one
    for name, (args, vgpr, spill, lds) in _kernels(notes, "_ZN2fa9fa_bwd_dqI").items():
        dq, dv, groups = args[0], args[1], args[5]
        if max(dq, dv) <= 128:
            assert vgpr <= 256 and spill == 0, name
            assert (2 // groups) * lds <= LDS_PER_CU, name
        else:
            assert vgpr <= 512 and spill == 0 and lds <= LDS_PER_CU, name


def test_128key_and_wide_dkdv_budgets(notes):
    # <DQ, DV, causal, window, exact, M-tiles>: heads up to 128 two waves per SIMD (eight-wave workgroups,
    # or two four-wave workgroups per CU), wider heads one (four-wave workgroups with two M-tiles, or
    # two two-wave workgroups per CU with one); no VGPR spills
    for name, (args, vgpr, spill, lds) in _kernels(notes, "_ZN2fa11fa_bwd_dkdvI").items():
        dq, dv, nmt = args[0], args[1], args[5]
        assert spill == 0, name
        if max(dq, dv) <= 128:
            assert vgpr <= 256 and (2 if nmt == 1 else 1) * lds <= LDS_PER_CU, name
        else:
            assert vgpr <= 512 and (2 if nmt == 1 else 1) * lds <= LDS_PER_CU, name
            assert nmt == 2 or dq + dv <= 320, name  # one M-tile only where both outputs' sums fit


def test_row_kernels_do_not_spill(notes):
    for prefix in ("_ZN2fa10fa_bwd_preI", "_ZN2fa14fa_bwd_dq_castI", "_ZN2fa19fa_bwd_split_reduceI"):
        for name, (args, vgpr, spill, lds) in _kernels(notes, prefix).items():
            assert spill == 0, name
