"""The allocation-free split-K entry point (svdq_w4a4_linear_splitk_noalloc,
for callers that cannot allocate device memory): called through the C ABI,
its output equals svdq_w4a4_linear_splitk's (same kernels, same summation
order) bit for bit on two calls in a row, the second with a smaller input
that still splits, so the shared static scratch holds the first call's
larger contents when the second runs.  A shape whose split needs more than
the static buffer is refused with SVDQ_ERR_SCRATCH before anything runs."""
import sys

import numpy as np
import pytest

import w4a4_rank_corrected_quantize_amd as svdq
from w4a4_rank_corrected_quantize_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MX = svdq.MXFP4


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    svdq.check_device()


def _inputs(M, K, N, seed):
    L = synth.make_layer(synth.SPECS["qkv"], M=M, K=K, N=N)
    p = svdq.pack_weights(L["W"], L["act_absmax"], prec=MX)
    d = svdq.to_device(p)
    xq, xs, h = svdq.quantize_act(svdq.bf16_tensor(L["X"]), d["smooth"], d["down"], MX)
    return (xq, xs, h, d["wq"], d["wscale"], d["up"], svdq.bf16_tensor(L["bias"]))


def test_noalloc_matches_splitk_twice_second_smaller():
    cases = [(1024, 12288, 3072, True), (300, 4096, 520, False)]      # the second is smaller
    for M, K, N, gelu in cases:
        need = svdq.linear_splitk_workspace_bytes(M, N, K, MX)
        assert 0 < need <= svdq.NOALLOC_SCRATCH_BYTES, (M, K, N, need)
    outs = []
    for M, K, N, gelu in cases:
        _say(f"noalloc split-K M={M} K={K} N={N}")
        args = _inputs(M, K, N, 0)
        epi = svdq.EPI_GELU_TANH if gelu else svdq.EPI_NONE
        Yn = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        svdq.w4a4_linear_splitk_noalloc(*args, MX, epi, Y=Yn)
        Ys = svdq.w4a4_linear_splitk(*args, MX, epi)
        torch.cuda.synchronize()
        assert torch.equal(Yn.view(torch.int16), Ys.view(torch.int16)), (M, K, N)
        outs.append((args, epi, Ys))
    # the first shape again, after the smaller call left its partial sums in
    # the scratch: still the same result
    args, epi, Ys = outs[0]
    Yn = svdq.w4a4_linear_splitk_noalloc(*args, MX, epi)
    torch.cuda.synchronize()
    assert torch.equal(Yn.view(torch.int16), Ys.view(torch.int16))


def test_noalloc_unsplit_shapes_pass_through():
    """INT4, and an MXFP4 shape whose tiles fill the chip: no scratch used,
    the output is svdq_w4a4_linear's."""
    for prec, M, K, N in [(svdq.INT4, 130, 2048, 264), (MX, 2000, 512, 9000)]:
        L = synth.make_layer(synth.SPECS["qkv"], M=M, K=K, N=N)
        p = svdq.pack_weights(L["W"], L["act_absmax"], prec=prec)
        d = svdq.to_device(p)
        xq, xs, h = svdq.quantize_act(svdq.bf16_tensor(L["X"]), d["smooth"], d["down"], prec)
        args = (xq, xs, h, d["wq"], d["wscale"], d["up"], svdq.bf16_tensor(L["bias"]))
        Yn = svdq.w4a4_linear_splitk_noalloc(*args, prec, svdq.EPI_GELU_TANH)
        Y = svdq.w4a4_linear(*args, prec, svdq.EPI_GELU_TANH)
        torch.cuda.synchronize()
        assert torch.equal(Yn.view(torch.int16), Y.view(torch.int16)), (prec, M, K, N)


def test_scratch_holds_every_split_on_this_device():
    """A split uses S slices of `tiles` 256 x 256 tiles with S * tiles at most
    the compute-unit count, so its slice sums need at most CUs * 256 * 256 *
    4 bytes: 64 MiB on a 256-CU MI355X, the size of the static buffer.  Every
    shape therefore fits here (a device with more compute units would get
    SVDQ_ERR_SCRATCH for the largest splits)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    worst = 0
    for M in list(range(1, 4097, 97)) + [256, 512, 1024, 2048, 4096]:
        for N in list(range(64, 16385, 264)) + [3072, 9216, 12288]:
            worst = max(worst, svdq.linear_splitk_workspace_bytes(M, N, 12288, MX))
    assert 0 < worst <= cus * 256 * 256 * 4
    if cus <= 256:
        assert worst <= svdq.NOALLOC_SCRATCH_BYTES
