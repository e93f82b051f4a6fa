"""The dense bf16 MFMA loop behind the bench's measured peak (a measurement
utility, not part of the method): the flops it reports are the products it
runs, every work-group computes the same, and its result scales with the
number of rounds -- so a timed launch really does that many products."""
import pytest
import torch

import gated_deltanet_amd as fk

pytestmark = pytest.mark.gpu


def test_peak_loop_counts_what_it_runs():
    n_wg = 8
    print("[peak] n_wg 8, iters 16 and 32", flush=True)
    sums = {}
    for iters in (16, 32):
        sink = torch.full((n_wg,), float("nan"), dtype=torch.float32, device="cuda")
        flops = fk.fk_peak_mfma_bf16(n_wg, iters, sink=sink)
        torch.cuda.synchronize()
        # 4 waves per work-group, 8 chains per wave, 2*32*32*16 flop per product
        assert flops == n_wg * 4 * iters * 8 * 2 * 32 * 32 * 16
        s = sink.cpu()
        assert torch.isfinite(s).all() and (s > 0).all()
        assert torch.equal(s, s[:1].expand_as(s))   # same operands in every work-group
        sums[iters] = float(s[0])
    assert sums[32] == pytest.approx(2 * sums[16], rel=1e-5)
    with pytest.raises(fk._lib.FkError):
        fk.fk_peak_mfma_bf16(0, 16)
