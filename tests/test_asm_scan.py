"""The decode kernels' K loads are inline assembly waited for by explicit
vmcnt counts, so the compiler does not know when their registers fill.  A
compiler copy, spill or reuse of such a register before its wait would read
or clobber data silently and non-deterministically.  These tests check the
scanner on hand-written sequences, then compile the kernels to gfx950
assembly and require that no instruction touches a register with an
outstanding load into it.
"""
import os
import re
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


def test_hazard_reached_only_through_a_branch():
    """The load is outstanding only on the path that jumps over the wait."""
    body = _fn([
        "global_load_dwordx4 v[4:7], v1, s[2:3]",
        "s_cbranch_scc1 .LBB0_2",
        "s_waitcnt vmcnt(0)",
        ".LBB0_2:",
        "v_mov_b32_e32 v8, v5",          # reached with the load in flight via the branch
        "s_endpgm",
    ])
    assert [h[0] for h in scan_function(body)] == [3]


def test_hazard_reached_only_through_a_back_edge():
    """A load issued at the bottom of a loop for the next iteration, and a
    copy at the loop head before its wait: in layout order the head comes
    first, so only the back-edge carries the load there."""
    body = _fn([
        "s_mov_b32 s0, 0",
        ".LBB0_1:",
        "v_mov_b32_e32 v8, v4",          # loop head: v4 may still be loading
        "s_waitcnt vmcnt(0)",
        "v_add_f32_e32 v9, v4, v5",
        "global_load_dwordx4 v[4:7], v1, s[2:3]",
        "s_add_i32 s0, s0, 1",
        "s_cmp_lg_u32 s0, 8",
        "s_cbranch_scc1 .LBB0_1",
        "s_waitcnt vmcnt(0)",
        "s_endpgm",
    ])
    assert [h[0] for h in scan_function(body)] == [1]


def test_jump_over_the_only_use_is_clean():
    body = _fn([
        "global_load_dwordx4 v[4:7], v1, s[2:3]",
        "s_branch .LBB0_2",
        ".LBB0_1:",
        "v_mov_b32_e32 v4, 0",          # no path reaches it
        ".LBB0_2:",
        "s_waitcnt vmcnt(0)",
        "v_mov_b32_e32 v8, v4",
        "s_endpgm",
    ])
    assert scan_function(body) == []


def test_flag_steered_paths_are_kept_apart():
    """The compiler's flag pattern: one path loads and sets s[4:5] = 0, the
    other sets it to -1; the join branches on it, so the block that writes
    v18 is reached only from the path without the load."""
    body = _fn([
        "s_cbranch_scc0 .LBB0_2",
        "global_load_dwordx4 v[18:21], v[30:31], off",
        "s_mov_b64 s[4:5], 0",
        "s_branch .LBB0_3",
        ".LBB0_2:",
        "s_mov_b64 s[4:5], -1",
        ".LBB0_3:",
        "s_andn2_b64 vcc, exec, s[4:5]",
        "s_cbranch_vccnz .LBB0_4",
        "v_mov_b32_e32 v18, 0",          # only the s[4:5] = -1 path gets here
        ".LBB0_4:",
        "s_waitcnt vmcnt(0)",
        "s_endpgm",
    ])
    assert scan_function(body) == []
    # the same shape with the flag overwritten before the branch is flagged
    body2 = body.replace("s_andn2_b64 vcc, exec, s[4:5]", "s_and_b64 s[4:5], s[4:5], s[6:7]\n"
                         "s_andn2_b64 vcc, exec, s[4:5]")
    assert [h[1] for h in scan_function(body2)] == ["v_mov_b32_e32 v18, 0"]


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
    from concurrent.futures import ProcessPoolExecutor
    names = sorted(bodies)
    with ProcessPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        results = list(pool.map(scan_function, [bodies[n] for n in names]))
    bad = {n: hits[:3] for n, hits in zip(names, results) if hits}
    assert not bad, bad
    # No flat (generic address) memory instruction: a flat load is counted
    # on the vector-memory counter as well, so waiting for one waits for
    # every K/V load in flight.  Accesses to LDS words shared between waves
    # must be LDS instructions.
    flat = {name: re.findall(r"^\s*(flat_\w+.*)$", body, re.M)[:3] for name, body in bodies.items()}
    flat = {k: v for k, v in flat.items() if v}
    assert not flat, flat
