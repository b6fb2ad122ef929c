"""The decode kernels' K loads are inline assembly waited for by explicit
vmcnt counts, so the compiler does not know when their registers fill.  A
compiler copy, spill or reuse of such a register before its wait would read
or clobber data silently and non-deterministically.  These tests check the
scanner on hand-written sequences, then compile the kernels to gfx950
assembly and require that no instruction touches a register with an
outstanding load into it.
"""
import os
import shutil
import subprocess

import pytest

from tests.asm_scan import kernel_bodies, scan_function


def _fn(lines):
    return "\n".join(lines)


def test_copy_before_wait_is_found():
    hits = scan_function(_fn([
        "global_load_dwordx4 v[4:7], v1, s[2:3]",
        "v_mov_b64_e32 v[10:11], v[6:7]",
        "s_waitcnt vmcnt(0)",
        "v_mov_b64_e32 v[12:13], v[6:7]",
    ]))
    assert [h[0] for h in hits] == [1]
    assert hits[0][3] == [0]


def test_partial_wait_counts_in_issue_order():
    body = _fn([
        "global_load_dwordx4 v[4:7], v1, s[2:3]",   # oldest
        "global_load_lds_dwordx4 v2, s[2:3]",        # into LDS: no registers
        "global_load_dwordx4 v[8:11], v1, s[2:3]",
        "s_waitcnt vmcnt(1)",                        # the first two are done
        "v_add_f32_e32 v20, v4, v5",
        "v_add_f32_e32 v21, v8, v9",                 # still outstanding
    ])
    assert [h[0] for h in scan_function(body)] == [5]


def test_clobber_and_load_reuse():
    body = _fn([
        "global_load_dwordx4 v[4:7], v1, s[2:3]",
        "global_load_dwordx4 v[4:7], v1, s[2:3] offset:64",  # in order: allowed
        "v_mov_b32_e32 v5, 0",                                   # clobbered by the loads
        "s_waitcnt vmcnt(0)",
    ])
    assert [h[0] for h in scan_function(body)] == [2]


def test_jump_target_starts_clean():
    body = _fn([
        "global_load_dwordx4 v[4:7], v1, s[2:3]",
        "s_branch .LBB0_2",
        ".LBB0_1:",
        "v_mov_b32_e32 v4, 0",          # reached by a jump only
        ".LBB0_2:",
        "s_waitcnt vmcnt(0)",
    ])
    assert scan_function(body) == []


def test_kernel_bodies_split():
    asm = "\n_ZN3art1fEv: ; @f\n  v_mov_b32 v0, 0\n.Lfunc_end0:\n_ZN3art1gEv:\n  s_endpgm\n.Lfunc_end1:\n"
    assert set(kernel_bodies(asm, "_ZN3art")) == {"_ZN3art1fEv", "_ZN3art1gEv"}


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="no hipcc")
@pytest.mark.parametrize("src", ["art_kernels.hip", "select_kernels.hip"])
def test_generated_kernels_have_no_access_to_outstanding_loads(tmp_path, src):
    from kv_cache_early_amd import build as B
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / "k.s"
    cmd = [_hipcc(), *flags, "-I" + B.INCLUDE, "-I" + B.CSRC, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    bodies = kernel_bodies(out.read_text(), "_ZN3art")
    assert bodies, "no kernels found in the assembly"
    bad = {name: hits[:3] for name, body in bodies.items() if (hits := scan_function(body))}
    assert not bad, bad
