"""The fixed-order projection (fk_proj_gemm; Flide section 3.5: every matrix
product sums each output element in one order whatever the number of rows;
section 3.3.3: the last layer's products only at the readout rows) against
the fp64 oracle (bf16 bar: max-abs 2e-2, mean-abs 2e-3), and batch
invariance: a row's bits are the same alone, inside any batch, at any
position, and gathered through an index buffer.

Inputs: x ~ N(0, 1) and w ~ N(0, 1/K) (a linear layer's usual scale, so
outputs are ~N(0, 1)), rounded to bf16; seeded."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
import oracle
from tests.harness import to_f64
from workloads.tensors import bf16_to_f64, to_bf16

pytestmark = pytest.mark.gpu
MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def _draw(seed, M, K, N):
    rng = np.random.default_rng(seed)
    x = to_bf16(rng.standard_normal((M, K), dtype=np.float32))
    w = to_bf16(rng.standard_normal((N, K), dtype=np.float32) / np.sqrt(K))
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    return x, w, xt, wt


def _err(o, ref):
    assert np.isfinite(o).all()
    d = np.abs(o - ref)
    return d.max(), d.mean()


@pytest.mark.parametrize("M,K,N", [(1, 64, 128), (300, 256, 384), (129, 1024, 256), (1000, 4096, 128),
                                   (1, 64, 256), (257, 192, 512), (600, 320, 768)])
def test_proj_matches_oracle(M, K, N):
    x, w, xt, wt = _draw(M + K + N, M, K, N)
    print(f"[proj] M={M} K={K} N={N}", flush=True)
    y = to_f64(fk.fk_proj_gemm(xt, wt))
    ref = oracle.proj(bf16_to_f64(x), bf16_to_f64(w))
    mx, mean = _err(y, ref)
    print(f"  max-abs {mx:.3e} mean-abs {mean:.3e}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS


def test_proj_index_buffer():
    """Gathered rows equal the oracle's gathered product; unused entries (-1)
    leave their rows untouched; each gathered row has the bits of that row of
    the plain product."""
    M, K, N = 200, 512, 256
    x, w, xt, wt = _draw(5, M, K, N)
    rng = np.random.default_rng(5)
    rows = rng.integers(0, M, 77).astype(np.int32)
    rows[[3, 40, 76]] = -1
    rows[10] = rows[11]
    rt = torch.from_numpy(rows).cuda()
    y = torch.full((len(rows), N), 7.0, dtype=torch.bfloat16, device="cuda")
    fk.fk_proj_gemm(xt, wt, rows=rt, out=y)
    full = fk.fk_proj_gemm(xt, wt)
    used = torch.from_numpy(rows >= 0).cuda()
    assert torch.equal(y[used], full[rt[used].long()])
    assert torch.all(y[~used] == 7.0)
    ref = oracle.proj(bf16_to_f64(x), bf16_to_f64(w), rows=rows)
    mx, mean = _err(to_f64(y)[rows >= 0], ref[rows >= 0])
    assert mx <= MAX_ABS and mean <= MEAN_ABS


def test_proj_batch_invariance():
    """A row alone, in a small batch, in a large batch, at another position
    of a permuted batch, and through an index buffer: the same bits."""
    M, K, N = 1500, 2048, 256
    _, _, xt, wt = _draw(9, M, K, N)
    full = fk.fk_proj_gemm(xt, wt)
    for m in (0, 127, 128, 777, M - 1):
        alone = fk.fk_proj_gemm(xt[m:m + 1].contiguous(), wt)
        assert torch.equal(alone[0], full[m]), m
    few = fk.fk_proj_gemm(xt[100:105].contiguous(), wt)
    assert torch.equal(few, full[100:105])
    perm = torch.randperm(M, generator=torch.Generator().manual_seed(3)).cuda()
    yp = fk.fk_proj_gemm(xt[perm].contiguous(), wt)
    assert torch.equal(yp, full[perm])
    rows = perm[:333].to(torch.int32).contiguous()
    yr = fk.fk_proj_gemm(xt, wt, rows=rows)
    assert torch.equal(yr, full[perm[:333]])
    again = fk.fk_proj_gemm(xt, wt)
    assert torch.equal(again, full)


def test_proj_model_size():
    """An output projection of the long-context attention's width (32 heads x
    128 = 4096 -> 4096) over the mixture's 24,526 stream rows, in the bench's
    launch configuration; 64 seeded rows against the oracle, all features."""
    M, K, N = 24526, 4096, 4096
    x, w, xt, wt = _draw(1001, M, K, N)
    y = fk.fk_proj_gemm(xt, wt)
    torch.cuda.synchronize()
    sel = np.sort(np.random.default_rng(1).choice(M, 64, replace=False))
    sel[-1] = M - 1
    ref = oracle.proj(bf16_to_f64(x), bf16_to_f64(w), rows=sel.astype(np.int32))
    mx, mean = _err(to_f64(y)[sel], ref)
    print(f"[proj model size] max-abs {mx:.3e} mean-abs {mean:.3e} on {len(sel)} rows x {N}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS
