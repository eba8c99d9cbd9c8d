"""Checks the build applies to its own compiled code (CPU only)."""
import os

import pytest

from int4_weight_only_linear_amd import build as B

OBJ = os.path.join(B.BUILD, "w4a16_gemm.hip.o")
NAME = "_ZN5w4a1612_GLOBAL__N_111gemm_kernelILi1ELi128ELb1ELi1ELi1ELb0EEEvNS0_10GemmParamsE"


def _listing(ops):
    return "\n".join([f"0000000000001000 <{NAME}>:"] + [f"\t{op} v0, v1   // 000000001000: 00000000" for op in ops]
                     + ["0000000000002000 <_ZN5other>:"])


def test_thin_tile_waits_in_this_build():
    if not os.path.exists(OBJ):
        pytest.skip("not built")
    # every partial-wait step barrier of every 32-token instance is preceded
    # by exactly the step after next's weight and x loads
    assert B.check_thin_tile_waits(OBJ) >= 48


def test_thin_tile_wait_check_catches_a_wrong_order():
    # a well-formed step: metadata, two weight loads, two x loads, vmcnt(4)
    good = ["global_load_ushort", "global_load_dword", "global_load_dwordx4", "global_load_dwordx4",
            "global_load_lds_dwordx4", "global_load_lds_dwordx4", "s_waitcnt vmcnt(4) lgkmcnt(0)", "s_barrier"]
    assert B.thin_tile_waits_in(_listing(good)) == 1
    # the weights after the x loads, a dropped weight load, a count that
    # would not cover the next step, no metadata before the group
    for bad in (good[:2] + good[4:6] + good[2:4] + good[6:],
                good[:3] + good[4:],
                good[:6] + ["s_waitcnt vmcnt(5) lgkmcnt(0)", "s_barrier"],
                good[2:]):
        with pytest.raises(RuntimeError):
            B.thin_tile_waits_in(_listing(bad))
    # a full wait is always fine
    assert B.thin_tile_waits_in(_listing(["global_load_lds_dwordx4", "s_waitcnt vmcnt(0) lgkmcnt(0)", "s_barrier"])) == 0
