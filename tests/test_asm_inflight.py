"""No register written by an in-flight inline-asm load is touched before its
wait, in any kernel that streams its loads that way (the per-head prefill
kernels, the segment combine and the tiled channel-gate recurrence; see tests/asm_inflight.py),
and the analysis itself finds a planted copy of such a register."""
import os

import pytest

from asm_inflight import check_kernel, compile_asm, kernels

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_115_amd", "csrc")


def _compile(tmp_path_factory, name):
    from gated_delta_rule_115_amd.build import CFLAGS
    flags = [f for f in CFLAGS if f not in ("-Wall",)]
    return compile_asm(os.path.join(CSRC, name), str(tmp_path_factory.mktemp("asm") / "k.s"),
                       flags)


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return _compile(tmp_path_factory, "gdn_prefill_head.hip")


def test_tiled_chgate_recurrence_has_no_inflight_hazard(tmp_path_factory):
    text = _compile(tmp_path_factory, "gdn_chgate.hip")
    names = [k for k in kernels(text) if "chgate_recur_tile_kernel" in k]
    assert len(names) == 2  # bf16 and f32 output
    for k in names:
        rep = check_kernel(text, k)
        assert rep == [], (k, rep[:5])


def test_per_head_kernels_have_no_inflight_hazard(asm):
    names = [k for k in kernels(asm) if "prefill_" in k]
    assert len(names) == 8  # lead and output kernels x {bf16, f32 out} x {fused conv, not}
    names += [k for k in kernels(asm) if "segment_combine_kernel" in k]
    assert len(names) == 10  # + the combine with and without prefetch
    for k in names:
        rep = check_kernel(asm, k)
        assert rep == [], (k, rep[:5])


def test_planted_copy_of_inflight_register_is_found(asm):
    k = next(k for k in kernels(asm) if "prefill_out_kernel" in k)
    lines = asm.split("\n")
    start = next(i for i, l in enumerate(lines) if l.startswith(k + ":"))
    at = next(i for i in range(start, len(lines))
              if "global_load_dwordx4 v[" in lines[i] and "ASM" not in lines[i])
    reg = lines[at].split("v[")[1].split(":")[0]
    lines.insert(at + 1, f"\tv_mov_b32_e32 v0, v{reg}")
    rep = check_kernel("\n".join(lines), k)
    assert any(r[0] == at + 2 for r in rep)
