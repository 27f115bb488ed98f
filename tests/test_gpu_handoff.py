"""The failure path of the balanced schedule's state hand-over, forced from the host.

A workgroup that finishes a chain another workgroup began waits for that
state's flag a bounded number of times.  With the poll limit set to 0 every such
workgroup gives up at once, without touching the flag or the state: it must set
KDA_DEVICE_HANDOFF_TIMEOUT in the GPU's status word and write NaN to exactly its
own o rows and its chain's final state, leaving every other output as a normal
call writes it.  Every kernel still runs to completion.
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


def run(kda, inp, N):
    o = torch.full_like(inp["q"], 3.0)
    T, H, D = inp["q"].shape
    sf = torch.full((N, H, D, D), 3.0, dtype=torch.float32, device="cuda")
    kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                  initial_state=inp["initial_state"], num_seqs=N, out=o, final_state=sf)
    torch.cuda.synchronize()
    return o, sf


def test_handoff_give_up_reports_and_poisons(kda):
    N, T, H = 3, 1000, 96
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sched = kda.balanced_schedule(N, T, H, cus)
    if sched is None:
        pytest.skip(f"no balanced schedule for {N} x {T} x {H} on {cus} units")
    tails = [(c, c0, c1) for c, c0, c1, role, _ in sched if role == 2]
    assert tails
    announce(f"hand-over give-up b{N} t{T} h{H}, {len(tails)} tails")
    inp = ki.make_prefill(ki.PrefillConfig("t", (T,) * N, H, "bf16", init_std=0.02),
                          device="cuda", seed=21)
    inp["g"].mul_(0.02)
    kda.device_status(clear=True)
    o_ref, sf_ref = run(kda, inp, N)
    assert kda.device_status(clear=True) == 0
    assert torch.isfinite(o_ref.float()).all() and torch.isfinite(sf_ref).all()

    old = kda.handoff_poll_limit()
    try:
        kda.set_handoff_poll_limit(0)
        o, sf = run(kda, inp, N)
    finally:
        kda.set_handoff_poll_limit(old)
    status = kda.device_status(clear=True)
    assert status & kda.DEVICE_HANDOFF_TIMEOUT, f"status {status:#x}"
    assert kda.device_status(clear=False) == 0, "the clear reset the word"

    poisoned_o = torch.zeros(o.shape[:2], dtype=torch.bool, device="cuda")
    poisoned_sf = torch.zeros(sf.shape[:2], dtype=torch.bool, device="cuda")
    for chain, c0, c1 in tails:
        n, h = divmod(chain, H)
        t0, t1 = n * T + c0 * 64, n * T + min(c1 * 64, T)
        poisoned_o[t0:t1, h] = True
        poisoned_sf[n, h] = True
    assert torch.isnan(o.float()[poisoned_o]).all(), "a tail's o rows are not NaN"
    assert torch.isnan(sf[poisoned_sf]).all(), "a cut chain's final state is not NaN"
    keep_o, keep_sf = ~poisoned_o, ~poisoned_sf
    assert torch.equal(o[keep_o].view(torch.int16), o_ref[keep_o].view(torch.int16)), \
        "rows outside the tails changed"
    assert torch.equal(sf[keep_sf].view(torch.int32), sf_ref[keep_sf].view(torch.int32)), \
        "final states of uncut chains changed"

    # back to the default limit: a normal call, nothing reported, same bits
    o2, sf2 = run(kda, inp, N)
    assert kda.device_status(clear=True) == 0
    assert torch.equal(o2.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(sf2.view(torch.int32), sf_ref.view(torch.int32))

