"""moe_verify_step_static (the verify step with its workspace in the
library's static device scratch, for callers that cannot allocate) against
moe_verify_step on the same context and inputs, through the C ABI: two or
more calls in a row with the second smaller, and a second context of other
sizes in between (it lays the shared array out differently).  Outputs are
committed tokens and counts: equal bit for bit to moe_verify_step's and to
the oracle's."""
import numpy as np
import pytest

from moe_decoder_speculative_amd import binding
from moe_decoder_speculative_amd.model import VerifyModel, to_device
import parity
import workloads

pytestmark = pytest.mark.gpu


def _both(model, hidden_np, drafts_np, B, K):
    import torch
    hidden = to_device(np.ascontiguousarray(hidden_np))
    drafts = to_device(np.ascontiguousarray(drafts_np.astype(np.int32))) if K > 0 else None
    c0, n0 = model.alloc_outputs(B, K)
    c1, n1 = model.alloc_outputs(B, K)
    c1.fill_(-7)
    n1.fill_(-7)
    model.step(hidden, drafts, B, K, c0, n0)
    binding.moe_verify_step_static(model.ctx, hidden, drafts, B, K, c1, n1)
    torch.cuda.synchronize()
    return (c0.cpu().numpy(), n0.cpu().numpy()), (c1.cpu().numpy(), n1.cpu().numpy())


def _check(model, case, nseq, tag):
    w = case.w
    K = w.K
    T = nseq * (K + 1)
    parity.say(f"[no-alloc] {tag}: workload={w.name} B={nseq} K={K} T={T} entry=moe_verify_step_static")
    (c0, n0), (c1, n1) = _both(model, case.hidden[:T], case.drafts[:nseq], nseq, K)
    assert np.array_equal(c1, c0) and np.array_equal(n1, n0), f"{tag}: static step differs from moe_verify_step"
    # sequences are independent: the oracle's step on the whole batch gives these sequences' results
    assert np.array_equal(n1, case.ref.counts[:nseq]), f"{tag}: counts differ from the oracle"
    assert np.array_equal(c1, case.ref.committed[:nseq]), f"{tag}: committed tokens differ from the oracle"
    parity.say(f"[no-alloc] {tag} ok: counts {n1[:8].tolist()}")


def test_static_step_matches_context_step():
    big = workloads.cached_case("decode_b32_zipf")
    small = workloads.build_case(workloads.small_bf16(B=5, K=3, L=2, seed_id=61))
    mb = VerifyModel(big.w, big.weights, max_tokens=big.w.T)
    ms = VerifyModel(small.w, small.weights, max_tokens=small.w.T)
    try:
        _check(mb, big, 32, "full batch")            # 128 rows: the largest step the scratch takes
        _check(mb, big, 3, "smaller batch")          # the next call, smaller
        _check(ms, small, 5, "other context")        # other sizes lay the array out differently
        _check(mb, big, 1, "back to the first")
        # beyond the limit: rejected before any launch
        import torch
        h = torch.zeros((33 * 4, big.w.H), dtype=torch.bfloat16, device="cuda")
        d = torch.zeros((33, 3), dtype=torch.int32, device="cuda")
        c, n = mb.alloc_outputs(33, 3)
        with pytest.raises(binding.MoeVerifyError) as e:
            binding.moe_verify_step_static(mb.ctx, h, d, 33, 3, c, n)
        assert e.value.code == binding.MOE_EINVAL
    finally:
        mb.close()
        ms.close()
