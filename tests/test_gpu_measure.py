"""The on-device peak measurements (dsa_bench_mfma, dsa_bench_stream) through the C ABI (GPU).

They are measurement helpers, not the indexer's method: the checks are that they run, that
the MFMA stream leaves finite sums that differ between lanes (so the work was done on the
operands), and that the stream copy is a byte-exact copy while the read-only sweep leaves its
destination alone.
"""

import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


@pytest.mark.parametrize("precision", ["bf16", "fp8", "mxfp8"])
def test_mfma_stream(precision):
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    blocks, iters = 8, 16
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flops = dsa.bench_mfma(precision, blocks, iters, out)
    torch.cuda.synchronize()
    per = 32 * 32 * (16 if precision == "bf16" else 64) * 2
    assert flops == blocks * 4 * iters * 4 * per
    assert bool(torch.isfinite(out).all())
    assert out.unique().numel() > 1


def test_mfma_rejects_short_output():
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    out = torch.empty(100, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        dsa.bench_mfma("fp8", 8, 4, out)


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 22) + 16 * 7])
def test_stream_copy_and_read(nbytes):
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    assert dsa.bench_stream(src, dst, copy=True) == 2 * nbytes
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].count_nonzero()) == 0
    dst2 = torch.zeros(64, dtype=torch.uint8, device="cuda")
    assert dsa.bench_stream(src, dst2, copy=False) == nbytes
    torch.cuda.synchronize()
    assert int(dst2.count_nonzero()) == 0
