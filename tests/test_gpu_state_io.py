"""GPU checks of kda_state_io: zero / copy / gather / scatter with fp32 <-> bf16
conversion.  Copies are exact; fp32 -> bf16 rounds to nearest even, the same
rounding as torch's conversion, so every case is compared bit for bit."""
import pytest
import torch

from kda_testutil import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_10_amd as m
    m.library()
    return m


@pytest.mark.parametrize("sdt,ddt", [(torch.float32, torch.float32),
                                     (torch.float32, torch.bfloat16),
                                     (torch.bfloat16, torch.float32),
                                     (torch.bfloat16, torch.bfloat16)])
def test_gather_scatter_copy_zero(kda, sdt, ddt):
    announce(f"state_io {sdt}->{ddt}")
    H = 5
    src = torch.randn((7, H, 128, 128), device="cuda").to(sdt)
    dst0 = torch.randn((6, H, 128, 128), device="cuda").to(ddt)
    # gather: dst[i] = src[idx[i]], negative / out-of-range skip
    idx = torch.tensor([6, 0, -1, 3, 9, 2], dtype=torch.int32, device="cuda")
    dst = dst0.clone()
    kda.state_io(kda.STATE_GATHER, dst, src, idx)
    exp = dst0.clone()
    for i, s in enumerate(idx.tolist()):
        if 0 <= s < 7:
            exp[i] = src[s].to(ddt)
    torch.cuda.synchronize()
    assert torch.equal(dst, exp)
    # scatter: dst[idx[i]] = src[i]
    idx2 = torch.tensor([5, -4, 1, 0], dtype=torch.int32, device="cuda")
    dst = dst0.clone()
    kda.state_io(kda.STATE_SCATTER, dst, src, idx2)
    exp = dst0.clone()
    for i, d in enumerate(idx2.tolist()):
        if 0 <= d < 6:
            exp[d] = src[i].to(ddt)
    torch.cuda.synchronize()
    assert torch.equal(dst, exp)
    # copy of the first 4 slots
    dst = dst0.clone()
    kda.state_io(kda.STATE_COPY, dst, src, count=4)
    exp = dst0.clone()
    exp[:4] = src[:4].to(ddt)
    torch.cuda.synchronize()
    assert torch.equal(dst, exp)
    # zero selected slots
    dst = dst0.clone()
    kda.state_io(kda.STATE_ZERO, dst, None, torch.tensor([1, 4], dtype=torch.int32,
                                                         device="cuda"))
    exp = dst0.clone()
    exp[1] = 0
    exp[4] = 0
    torch.cuda.synchronize()
    assert torch.equal(dst, exp)
