"""The ISA checker finds each kind of planted dependency mistake in small gfx950 listings, passes
correct ones, and passes the built kernels (CPU only)."""
import glob
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _mod():
    spec = importlib.util.spec_from_file_location(
        "fa_isa_check", os.path.join(ROOT, "exact_attention_125_amd", "isa_check.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


IC = _mod()


def listing(*lines):
    return "_Zk:\n" + "\n".join("\t" + l if not l.startswith(".") else l for l in lines) + "\n.Lfunc_end0:\n"


MFMA = "v_mfma_f32_32x32x16_bf16"


def test_clean_chain_passes():
    asm = listing("v_mov_b32 v16, 0", "s_nop 7",
                  f"{MFMA} a[0:15], v[16:19], v[20:23], a[0:15]",
                  f"{MFMA} a[0:15], v[16:19], v[20:23], a[0:15]",   # accumulation in place
                  "s_nop 15", "s_nop 7",
                  "v_accvgpr_read_b32 v0, a0", "s_endpgm")
    assert IC.mfma_hazards(asm, "_Zk") == []


@pytest.mark.parametrize("lines,kind", [
    (["v_mov_b32 v17, 1.0", f"{MFMA} a[0:15], v[16:19], v[20:23], a[0:15]"], "operand written before"),
    ([f"{MFMA} v[0:15], v[16:19], a[0:3], v[20:35]", "v_add_f32 v40, v3, v4"], "result accessed"),
    ([f"{MFMA} v[0:15], v[16:19], a[0:3], v[20:35]", "v_mov_b32 v22, 1.0"], "accumulator input overwritten"),
    ([f"{MFMA} v[0:15], v[16:19], a[0:3], 0", f"{MFMA} v[32:47], v[0:3], a[0:3], 0"], "result used by a product"),
    ([f"{MFMA} v[0:15], v[16:19], a[0:3], 0", "ds_read_b128 v[4:7], v50"], "result accessed"),
])
def test_planted_mfma_hazards(lines, kind):
    found = IC.mfma_hazards(listing(*lines, "s_endpgm"), "_Zk")
    assert [f[2] for f in found] == [kind]


def test_hazard_across_a_branch():
    # the VALU read sits on the taken path only
    asm = listing(f"{MFMA} v[0:15], v[16:19], a[0:3], 0", "s_cbranch_scc1 .LBB0_2",
                  "s_nop 15", "s_nop 15", "s_endpgm",
                  ".LBB0_2:", "v_add_f32 v40, v1, v2", "s_endpgm")
    assert [f[2] for f in IC.mfma_hazards(asm, "_Zk")] == ["result accessed"]


def test_enough_wait_states_pass():
    asm = listing(f"{MFMA} v[0:15], v[16:19], a[0:3], 0", "s_nop 15", "s_nop 3",
                  "v_add_f32 v40, v3, v4", "s_endpgm")
    assert IC.mfma_hazards(asm, "_Zk") == []


def test_untracked_lds_reads():
    early = listing("ds_read_b128 v[0:3], v10", "v_add_f32 v20, v1, v1", "s_endpgm")
    assert len(IC.early_lds_uses(early, "_Zk")) == 1
    covered = listing("ds_read_b128 v[0:3], v10", "ds_read_b128 v[4:7], v11",
                      "s_waitcnt lgkmcnt(1)", "v_add_f32 v20, v1, v1", "s_endpgm")
    assert IC.early_lds_uses(covered, "_Zk") == []
    # lgkmcnt(1) does not cover the younger read
    uncovered = listing("ds_read_b128 v[0:3], v10", "ds_read_b128 v[4:7], v11",
                        "s_waitcnt lgkmcnt(1)", "v_add_f32 v20, v5, v5", "s_endpgm")
    assert len(IC.early_lds_uses(uncovered, "_Zk")) == 1
    # a copy of the result before the wait is an early use too
    copied = listing("ds_read_b64_tr_b16 v[0:1], v10", "v_mov_b32 v30, v0",
                     "s_waitcnt lgkmcnt(0)", "s_endpgm")
    assert len(IC.early_lds_uses(copied, "_Zk")) == 1


def test_built_kernels_are_clean():
    """The assembly the build checked (present once the library has been built)."""
    files = sorted(glob.glob(os.path.join(ROOT, "_build", "*.hip.s")))
    if not files:
        pytest.skip("library not built")
    for path in files:
        mfma = not os.path.basename(path).startswith("fwd_main")
        bad = IC.check_asm(open(path).read(), mfma=mfma)
        assert bad == {}, (path, {k: v[:2] for k, v in bad.items()})
