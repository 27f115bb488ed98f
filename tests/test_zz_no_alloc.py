"""The allocation-free prefill (kda_chunk_fwd_no_alloc) against kda_chunk_fwd.

kda_chunk_fwd_no_alloc runs the same kernels with the same plan as kda_chunk_fwd
but takes its workspace from the library's per-GPU buffer, which keeps the
previous call's contents; so each call here is compared bit for bit with the
allocating entry point on the same inputs, calls follow each other on one
stream, and later calls are smaller than earlier ones (the buffer then holds
stale data past what the call uses).
"""
import pytest
import torch

import kda_inputs as ki
from kda_testutil import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_10_amd as m
    m.library()
    return m


def both(kda, inp, varlen, **kw):
    N = len(inp["lengths"])
    T, H, D = inp["q"].shape
    common = dict(cu_seqlens=inp["cu_seqlens"] if varlen else None,
                  cu_seqlens_host=inp["cu_seqlens_host"] if varlen else None,
                  initial_state=inp["initial_state"], num_seqs=N, **kw)
    o_ref, s_ref = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], **common)
    o = torch.full_like(inp["q"], float("nan"))
    sf = torch.full((N, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    kda.chunk_fwd_no_alloc(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o, sf, **common)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(sf).all()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(sf.view(torch.int32), s_ref.view(torch.int32))


def test_no_alloc_equals_chunk_fwd_on_consecutive_calls(kda):
    announce("no-alloc prefill: three-segment split, then smaller calls")
    # 1: one 8,192-token sequence of 96 heads: the automatic three-segment split,
    #    56.6 MiB of segment states in the buffer
    big = ki.make_prefill(ki.PrefillConfig("t", (8192,), 96, "bf16", init_std=0.02),
                          device="cuda", seed=81)
    assert kda.chunk_fwd_workspace_size(big["q"], num_seqs=1, segments=0) > (32 << 20)
    both(kda, big, varlen=False, segments=0)
    del big
    # 2: a smaller ragged pack with explicit segments (sequence order + segment states)
    small = ki.make_prefill(ki.PrefillConfig("t", (1000, 37, 0, 513), 8, "bf16", init_std=0.1,
                                             varlen=True), device="cuda", seed=82)
    both(kda, small, varlen=True, segments=3)
    # 3: a fixed batch whose chains are cut between workgroups (hand-over flags
    #    in the buffer, cleared by each call), twice in a row
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        ho = ki.make_prefill(ki.PrefillConfig("t", (1000, 1000, 1000), 96, "bf16", init_std=0.02),
                             device="cuda", seed=83)
        assert kda.chunk_fwd_workspace_size(ho["q"], num_seqs=3, segments=0) > 0
        both(kda, ho, varlen=False, segments=0)
        both(kda, ho, varlen=False, segments=0)


def test_no_alloc_rejects_a_plan_beyond_the_buffer(kda):
    announce("no-alloc prefill: oversize plan")
    x = ki.make_prefill(ki.PrefillConfig("t", (8192,), 96, "bf16"), device="cuda", seed=84)
    need = kda.chunk_fwd_workspace_size(x["q"], num_seqs=1, segments=64)
    assert need > kda.no_alloc_max_workspace()
    o = torch.zeros_like(x["q"])
    sf = torch.zeros((1, 96, 128, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(kda.KDAError) as err:
        kda.chunk_fwd_no_alloc(x["q"], x["k"], x["v"], x["g"], x["beta"], o, sf, num_seqs=1,
                               segments=64)
    assert err.value.status == 3  # KDA_ERROR_WORKSPACE
    torch.cuda.synchronize()
    assert not o.any() and not sf.any()  # nothing written
