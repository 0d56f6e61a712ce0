"""gdn_prefill_chunked_noalloc: the prefill entry point that allocates nothing
(for callers under graph capture or in loops that cannot call hipMalloc),
whose scratch is the library's static device array.  Checked through the C
ABI against gdn_prefill_chunked with a caller workspace on the same inputs,
two calls in a row with the second smaller (the scratch keeps the first
call's contents), and against the oracle."""
import pytest
import torch

import gated_delta_rule_115_amd as gdn
import oracle
import synthetic
from common import TOL, dev, err, f64, say

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "alpha", "beta")


def _both(x, chunk, out_dtype):
    ins = [dev(x[n]) for n in NAMES]
    s0 = dev(x["state0"])
    o_ref, s_ref = gdn.gdn_prefill_chunked(*ins, s0, chunk=chunk, out_dtype=out_dtype)
    o = torch.full_like(o_ref, float("nan"))
    s = torch.full_like(s_ref, float("nan"))
    gdn.gdn_prefill_chunked_noalloc(*ins, s0, o, s, chunk=chunk)
    torch.cuda.synchronize()
    return o, s, o_ref, s_ref


# (dtype, B, T, H, D, chunk): the per-head kernels with the segment split
# (scratch holds the segment maps; 46.5 MiB, then a smaller call), and the
# two-kernel form (scratch holds per-chunk records), each first large then
# small.
@pytest.mark.parametrize("calls", [
    [("bf16", 1, 16384, 8, 128, 64), ("bf16", 1, 3000, 2, 128, 64)],
    [("f32", 2, 1000, 4, 64, 32), ("f32", 1, 100, 2, 64, 32)],
    [("bf16", 2, 700, 3, 64, 64), ("bf16", 1, 65, 1, 64, 16)],
])
def test_noalloc_matches_workspace_entry_point(calls):
    for i, (dtype, B, T, H, D, chunk) in enumerate(calls):
        need = gdn.gdn_prefill_workspace_bytes(B, T, H, D, D, chunk,
                                               gdn.GDN_BF16 if dtype == "bf16" else gdn.GDN_F32)
        assert 0 < need <= gdn.GDN_NOALLOC_SCRATCH_BYTES
        x = synthetic.gdn_inputs(B, T, H, D, D, dtype=dtype, seed=100 + i, state0="randn")
        o, s, o_ref, s_ref = _both(x, chunk, torch.float32)
        eo, es = err(o, f64(o_ref)), err(s, f64(s_ref))
        say(f"noalloc {dtype} B{B} T{T} H{H} d{D} C{chunk} (scratch {need} B): "
            f"vs workspace call {eo:.1e} {es:.1e}")
        assert eo <= TOL[dtype] and es <= TOL[dtype]
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
        if T <= 3000:
            ro, rs = oracle.gdn_recurrence(*(f64(x[n]) for n in NAMES), f64(x["state0"]))
            assert err(o, ro) <= TOL[dtype] and err(s, rs) <= TOL[dtype]


def test_noalloc_bf16_output_and_no_state():
    x = synthetic.gdn_inputs(1, 3000, 2, 128, 128, dtype="bf16", seed=7)
    ins = [dev(x[n]) for n in NAMES]
    o_ref, _ = gdn.gdn_prefill_chunked(*ins, None, chunk=64, want_state=False)
    o = torch.empty_like(o_ref)
    gdn.gdn_prefill_chunked_noalloc(*ins, None, o, None, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    B, T, H, D = 1, 8192, 32, 64
    need = gdn.gdn_prefill_workspace_bytes(B, T, H, D, D, 64, gdn.GDN_F32)
    assert need > gdn.GDN_NOALLOC_SCRATCH_BYTES
    x = synthetic.gdn_inputs(B, T, H, D, D, dtype="f32", seed=3)
    o = torch.zeros(B, T, H, D, device="cuda")
    with pytest.raises(gdn.GdnError, match="static scratch"):
        gdn.gdn_prefill_chunked_noalloc(*(dev(x[n]) for n in NAMES), None, o, None, chunk=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0
