"""HIP path vs the fp64 oracle on the GPU, through the C ABI.

Bar: codes and scales bit-exact; h within the blocked fp32-summation bound;
the bf16 output within |y - y_ref| <= 8e-3 |y_ref| + 1e-3 rms(y_ref), where
y_ref is the oracle's fp64 output on the same codes (those are bit-exact, so
both sides take every integer decision in the same precision).
"""
import os
import sys

import numpy as np
import pytest

import w4a4_rank_corrected_quantize_amd as svdq
from oracle import oracle as O
from w4a4_rank_corrected_quantize_amd import synth
from w4a4_rank_corrected_quantize_amd.synth import bf16_bits_to_f32

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL, ABS_RMS = 8e-3, 1e-3


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    svdq.check_device()


def _t(a):
    """numpy -> device tensor (uint16 arrays become bf16)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return svdq.bf16_tensor(a)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _np(t):
    if t.dtype == torch.bfloat16:
        return svdq.bf16_bits(t)
    return t.cpu().numpy()


def _h_bound(X, down):
    """(K/16 + 64) 2^-24 sum_k |X_mk down_jk|: fp32 accumulation of exact bf16
    products in chunks of at most 16 partial sums plus the wave reduction."""
    K = X.shape[1]
    a = np.abs(bf16_bits_to_f32(X).astype(np.float64)) @ np.abs(bf16_bits_to_f32(down).astype(np.float64)).T
    return (K / 16 + 64) * 2.0 ** -24 * a + 1e-30


def _quant_act_check(X, s, down, prec):
    xq, xs, h = svdq.quantize_act(_t(X), _t(s), _t(down), prec)
    torch.cuda.synchronize()
    oq, os_, oh = O.quant_act(X, s, down, prec)
    gq, gs, gh = _np(xq), _np(xs), _np(h)
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    assert np.array_equal(gs.view(np.uint8), os_.view(np.uint8)), \
        f"scales differ at {np.argwhere(gs.view(np.uint8).reshape(gs.shape[0], -1) != os_.view(np.uint8).reshape(os_.shape[0], -1))[:5]}"
    assert np.all(np.abs(gh.astype(np.float64) - oh) <= _h_bound(X, down))
    return xq, xs, h, oh


def _y_check(Y, y_ref, what=""):
    y = bf16_bits_to_f32(_np(Y)).astype(np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2)) if y_ref.size else 0.0
    bad = np.abs(y - y_ref) > REL * np.abs(y_ref) + ABS_RMS * rms
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst "
                           f"{np.max(np.abs(y - y_ref) / (REL * np.abs(y_ref) + ABS_RMS * rms)):.3f}")


def _layer(spec_name, M, K, N, prec, bias=True):
    spec = synth.SPECS[spec_name]
    if spec.x_dist == "external":
        spec = synth.SPECS["qkv"]
    L = synth.make_layer(spec, M=M, K=K, N=N)
    if not bias:
        L["bias"] = None
    p = svdq.pack_weights(L["W"], L["act_absmax"], prec=prec)
    return L, p


# ------------------------------------------------------------ activation step

PRECS = [svdq.INT4, svdq.MXFP4]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("M,K", [(128, 256), (1, 64), (15, 128), (17, 320), (100, 3072), (33, 12288)])
def test_quantize_act_synthetic(prec, M, K):
    if prec == svdq.INT4 and K % 64:
        pytest.skip("INT4 needs K % 64 == 0")
    _say(f"quantize_act prec={prec} M={M} K={K}")
    L, p = _layer("qkv", M, K, 64, prec)
    _quant_act_check(L["X"], p["smooth"], p["down"], prec)


def test_quantize_act_mx_half_step():
    """K = 32 * odd (MXFP4 only; INT4 groups are 64 wide): the MXFP4 kernel
    ends on half a 64-channel step."""
    prec = svdq.MXFP4
    _say("quantize_act mx K=96/160")
    for M, K in [(20, 96), (3, 160)]:
        L, p = _layer("qkv", M, K, 16, prec)
        _quant_act_check(L["X"], p["smooth"], p["down"], prec)


@pytest.mark.parametrize("prec", PRECS)
def test_quantize_act_near_ties(prec):
    """X = +-1 and s = the target values: xhat = s exactly, so every element can
    sit on or next to a rounding boundary of its group."""
    _say(f"quantize_act near ties prec={prec}")
    rng = np.random.default_rng(77 + prec)
    M, K = 64, 1024
    g = 64 if prec == svdq.INT4 else 32
    t = np.zeros(K, np.float32)
    for b in range(K // g):
        a = np.float32(rng.uniform(0.5, 2.0) * 2.0 ** rng.integers(-20, 20))
        if prec == svdq.INT4:
            sc = np.float32(np.float64(a) / 7)
            v = ((rng.integers(0, 7, g) + 0.5) * np.float64(sc)).astype(np.float32)
        else:
            mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
            v = (mids[rng.integers(0, 8, g)] * 2.0 ** (np.floor(np.log2(a)) - 2)).astype(np.float32)
        nudge = rng.integers(-1, 2, g)
        v = np.where(nudge < 0, np.nextafter(v, np.float32(0)), np.where(nudge > 0, np.nextafter(v, np.float32(np.inf)), v))
        v[0] = a
        t[b * g:(b + 1) * g] = v
    X = np.where(rng.random((M, K)) < 0.5, 0x3F80, 0xBF80).astype(np.uint16)
    down = synth.f64_to_bf16_bits(rng.normal(0, 0.1, (32, K)))
    _quant_act_check(X, t, down, prec)


@pytest.mark.parametrize("prec", PRECS)
def test_quantize_act_subnormal_and_zero_groups(prec):
    _say(f"quantize_act subnormal prec={prec}")
    rng = np.random.default_rng(91)
    M, K = 32, 512
    t = (rng.standard_normal(K) * 2.0 ** rng.integers(-149, -110, K).astype(np.float64)).astype(np.float32)
    t[:64] = 0.0                                   # an all-zero group
    t[64:128] = np.float32(2.0 ** -149) * rng.integers(-12, 13, 64).astype(np.float32)
    X = np.where(rng.random((M, K)) < 0.5, 0x3F80, 0xBF80).astype(np.uint16)
    X[5] = 0                                       # an all-zero row
    down = synth.f64_to_bf16_bits(rng.normal(0, 0.1, (32, K)))
    _quant_act_check(X, t, down, prec)


def test_quantize_act_deterministic_and_empty():
    _say("quantize_act determinism")
    L, p = _layer("qkv", 200, 1024, 16, svdq.INT4)
    X, s, d = _t(L["X"]), _t(p["smooth"]), _t(p["down"])
    a = [svdq.quantize_act(X, s, d) for _ in range(3)]
    torch.cuda.synchronize()
    for r in a[1:]:
        for u, v in zip(a[0], r):
            assert torch.equal(u, v)
    e = svdq.quantize_act(X[:0], s, d)
    assert e[0].shape == (0, 512)


# ------------------------------------------------------------------- linear

@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("M,K,N,bias,gelu", [
    (128, 256, 256, False, False),       # the small configuration
    (1, 64, 8, True, False),
    (50, 128, 40, True, True),           # a single 128-channel step
    (37, 192, 24, True, True),
    (130, 320, 136, True, False),
    (257, 512, 264, False, True),
    (300, 1024, 512, True, True),
])
def test_linear_synthetic(prec, M, K, N, bias, gelu):
    _linear_case(prec, M, K, N, bias, gelu)


@pytest.mark.parametrize("M,K,N,bias,gelu", [
    (45, 96, 40, True, True),
    (130, 160, 264, True, False),
    (77, 2080, 136, False, True),
])
def test_linear_mx_odd_blocks(M, K, N, bias, gelu):
    """MXFP4 only (INT4 groups are 64 wide): an odd number of 32-channel blocks
    per row, so the register-staged kernel's last 64-channel slice is half
    zero-filled."""
    _linear_case(svdq.MXFP4, M, K, N, bias, gelu)


def _linear_case(prec, M, K, N, bias, gelu):
    _say(f"linear prec={prec} M={M} K={K} N={N} bias={bias} gelu={gelu}")
    spec = "small" if (M, K, N) == (128, 256, 256) else "qkv"
    L, p = _layer(spec, M, K, N, prec, bias=bias)
    xq, xs, h, oh = _quant_act_check(L["X"], p["smooth"], p["down"], prec)
    Y = svdq.w4a4_linear(xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]), prec,
                         svdq.EPI_GELU_TANH if gelu else svdq.EPI_NONE)
    torch.cuda.synchronize()
    y_ref = O.linear(_np(xq), _np(xs), oh, p["wq"], p["wscale"], p["up"], L["bias"], prec, gelu=gelu)
    _y_check(Y, y_ref, f"M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,gelu", [
    (130, 2048, 264, True),      # 2 tiles, 8 steps: 2 slices
    (300, 4096, 520, False),     # 6 tiles: 4 slices of 4 steps
    (1, 3072, 64, True),         # one token: 3 slices of 4 steps
    (257, 3328, 40, False),      # 13 steps: slices of 5, 5 and 3
])
def test_linear_splitk_synthetic(M, K, N, gelu):
    """The split-K MXFP4 linear: every output against the oracle (the unsplit
    call sums in another order, so the two may differ in low bf16 places);
    the workspace is used (S > 1) and its stale contents do not matter."""
    prec = svdq.MXFP4
    _say(f"linear split-K M={M} K={K} N={N} gelu={gelu}")
    need = svdq.linear_splitk_workspace_bytes(M, N, K, prec)
    assert need > 0 and need % (4 * M * N) == 0 and need // (4 * M * N) >= 2
    L, p = _layer("qkv", M, K, N, prec)
    xq, xs, h, oh = _quant_act_check(L["X"], p["smooth"], p["down"], prec)
    epi = svdq.EPI_GELU_TANH if gelu else svdq.EPI_NONE
    args = (xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]), prec, epi)
    work = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")   # stale contents
    Ys = svdq.w4a4_linear_splitk(*args, work=work)
    Ys2 = svdq.w4a4_linear_splitk(*args, work=work)
    Y = svdq.w4a4_linear(*args)
    torch.cuda.synchronize()
    assert torch.equal(Ys, Ys2), "split-K result not deterministic"
    y_ref = O.linear(_np(xq), _np(xs), oh, p["wq"], p["wscale"], p["up"], L["bias"], prec, gelu=gelu)
    _y_check(Ys, y_ref, f"split-K M={M} K={K} N={N}")
    _y_check(Y, y_ref, f"unsplit M={M} K={K} N={N}")


def test_linear_splitk_passthrough():
    """Shapes that are not split (INT4; tiles that fill the chip; K % 256)
    need no workspace and give exactly svdq_w4a4_linear's output."""
    _say("linear split-K pass-through")
    for prec, M, K, N in [(svdq.INT4, 130, 2048, 264), (svdq.MXFP4, 2000, 512, 9000), (svdq.MXFP4, 50, 2080, 40)]:
        assert svdq.linear_splitk_workspace_bytes(M, N, K, prec) == 0
        L, p = _layer("qkv", M, K, N, prec)
        xq, xs, h = svdq.quantize_act(_t(L["X"]), _t(p["smooth"]), _t(p["down"]), prec)
        args = (xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]), prec, svdq.EPI_GELU_TANH)
        Ys = svdq.w4a4_linear_splitk(*args)
        Y = svdq.w4a4_linear(*args)
        torch.cuda.synchronize()
        assert torch.equal(Ys, Y), (prec, M, K, N)


def test_linear_splitk_full_size_fc2_1024():
    """The MXFP4 fc2 of a 512 x 512 image (1024 x 12288 -> 3072, fc1's GELU
    output re-quantized): every output against the oracle."""
    _say("linear split-K 1024 x 12288 -> 3072")
    prec = svdq.MXFP4
    f1 = synth.make_layer(synth.SPECS["mx1k_fc1"])
    p1 = svdq.pack_weights(f1["W"], f1["act_absmax"], prec=prec)
    xq, xs, h = svdq.quantize_act(_t(f1["X"]), _t(p1["smooth"]), _t(p1["down"]), prec)
    Y1 = svdq.w4a4_linear(xq, xs, h, _t(p1["wq"]), _t(p1["wscale"]), _t(p1["up"]), _t(f1["bias"]), prec,
                          svdq.EPI_GELU_TANH)
    torch.cuda.synchronize()
    f2 = synth.make_layer(synth.SPECS["mx1k_fc2"], X_bits=_np(Y1))
    p2 = svdq.pack_weights(f2["W"], f2["act_absmax"], prec=prec)
    xq, xs, h, oh = _quant_act_check(_np(Y1), p2["smooth"], p2["down"], prec)
    assert svdq.linear_splitk_workspace_bytes(1024, 3072, 12288, prec) > 0
    Y2 = svdq.w4a4_linear_splitk(xq, xs, h, _t(p2["wq"]), _t(p2["wscale"]), _t(p2["up"]), _t(f2["bias"]), prec)
    torch.cuda.synchronize()
    y_ref = O.linear(_np(xq), _np(xs), oh, p2["wq"], p2["wscale"], p2["up"], f2["bias"], prec)
    _y_check(Y2, y_ref, "split-K fc2 1024 (all rows)")


@pytest.mark.parametrize("prec", PRECS)
def test_layer_graph_replay(prec):
    """The activation step and the linear captured in a HIP graph (as a
    serving loop would): every replay, with eager work and synchronizations
    in between, equals the eager launches bit for bit."""
    _say(f"graph replay prec={prec}")
    M, K, N = 300, 1024, 520
    L, p = _layer("qkv", M, K, N, prec)
    X = _t(L["X"])
    args = dict(smooth=_t(p["smooth"]), down=_t(p["down"]), wq=_t(p["wq"]), ws=_t(p["wscale"]), up=_t(p["up"]),
                b=_t(L["bias"]))
    g = svdq.group_of(prec)
    sdt = torch.float32 if prec == svdq.INT4 else torch.uint8
    xq = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M, K // g), dtype=sdt, device="cuda")
    h = torch.empty((M, svdq.RANK), dtype=torch.float32, device="cuda")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        svdq.quantize_act(X, args["smooth"], args["down"], prec, xq=xq, xscale=xs, h=h)
        svdq.w4a4_linear(xq, xs, h, args["wq"], args["ws"], args["up"], args["b"], prec, svdq.EPI_GELU_TANH, Y=Y)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (xq, xs, h, Y)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        for t in (xq, h, Y):
            t.zero_()
        xs.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((xq, xs, h, Y), ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("prec", PRECS)
def test_linear_invariants(prec):
    """up = 0 => the 4-bit product alone; residual codes 0 => the low-rank
    product alone (+ bias)."""
    _say(f"linear invariants prec={prec}")
    M, K, N = 96, 512, 128
    L, p = _layer("qkv", M, K, N, prec)
    xq, xs, h, oh = _quant_act_check(L["X"], p["smooth"], p["down"], prec)
    y_ref, yq, ylr = O.linear(_np(xq), _np(xs), oh, p["wq"], p["wscale"], p["up"], L["bias"], prec,
                              parts=True)
    zero_up = np.zeros_like(p["up"])
    Y = svdq.w4a4_linear(xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(zero_up), None, prec)
    _y_check(Y, yq, "up = 0")
    Y2 = svdq.w4a4_linear(xq, xs, h, _t(np.zeros_like(p["wq"])), _t(p["wscale"]), _t(p["up"]),
                          _t(L["bias"]), prec)
    _y_check(Y2, ylr + bf16_bits_to_f32(L["bias"]).astype(np.float64)[None, :], "residual = 0")
    torch.cuda.synchronize()


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("M,K,N", [(96, 512, 128), (133, 512, 200)])
def test_linear_bias_alone_is_exact(prec, M, K, N):
    """Zero residual codes and zero `up` leave y = b exactly: the 4-bit and
    low-rank terms are exact zeros and the bias is a bf16 value, so every
    output row must equal the bias (no GELU), whichever unit adds it."""
    _say(f"bias alone prec={prec} M={M} K={K} N={N}")
    L, p = _layer("qkv", M, K, N, prec)
    xq, xs, h = svdq.quantize_act(_t(L["X"]), _t(p["smooth"]), _t(p["down"]), prec)
    Y = svdq.w4a4_linear(xq, xs, h, _t(np.zeros_like(p["wq"])), _t(p["wscale"]), _t(np.zeros_like(p["up"])),
                         _t(L["bias"]), prec)
    got = bf16_bits_to_f32(_np(Y))
    want = np.broadcast_to(bf16_bits_to_f32(L["bias"])[None, :], (M, N))
    assert np.array_equal(got, want)
    torch.cuda.synchronize()


def test_linear_deterministic_and_empty():
    _say("linear determinism")
    L, p = _layer("qkv", 160, 512, 256, svdq.INT4)
    xq, xs, h = svdq.quantize_act(_t(L["X"]), _t(p["smooth"]), _t(p["down"]))
    args = (xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]))
    Ys = [svdq.w4a4_linear(*args, svdq.INT4, svdq.EPI_GELU_TANH) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(Ys[0], y) for y in Ys[1:])
    e = svdq.w4a4_linear(xq[:0], xs[:0], h[:0], *args[3:], svdq.INT4)
    assert e.shape == (0, 256)


# --------------------------------------------- fused next-layer requantization

def _requant_case(M, K, N, bias, gelu, prec, rows=None):
    """fc1 -> fc2 with fc2's activation step fused into fc1's epilogue: the
    codes and scales must equal the separate activation step on the Y the
    plain kernel stores (bit-exact), and the oracle's on that Y; h2 within the
    blocked-summation bound."""
    L, p = _layer("qkv", M, K, N, prec, bias=bias)
    xq, xs, h = svdq.quantize_act(_t(L["X"]), _t(p["smooth"]), _t(p["down"]), prec)
    epi = svdq.EPI_GELU_TANH if gelu else svdq.EPI_NONE
    args = (xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]))
    Y = svdq.w4a4_linear(*args, prec, epi)
    torch.cuda.synchronize()
    Yb = _np(Y)
    f2 = synth.make_layer(synth.SPECS["fc2"], M=M, K=N, N=64, X_bits=Yb)
    p2 = svdq.pack_weights(f2["W"], f2["act_absmax"], prec=prec)
    s2, d2 = _t(p2["smooth"]), _t(p2["down"])
    uq, us, uh = svdq.quantize_act(Y, s2, d2, prec)
    fq, fs, fh = svdq.w4a4_linear_requant(*args, s2, d2, prec, epi)
    torch.cuda.synchronize()
    assert torch.equal(fq, uq), f"codes differ at {torch.nonzero(fq != uq)[:5].tolist()}"
    assert torch.equal(fs.view(torch.uint8), us.view(torch.uint8)), "scales differ"
    rows = np.arange(M) if rows is None else rows
    oq, os_, oh = O.quant_act(Yb[rows], p2["smooth"], p2["down"], prec)
    assert np.array_equal(_np(fq)[rows], oq)
    assert np.array_equal(_np(fs)[rows].view(np.uint8), os_.view(np.uint8))
    assert np.all(np.abs(_np(fh)[rows].astype(np.float64) - oh) <= _h_bound(Yb[rows], p2["down"]))
    # the fused h2 is deterministic
    fq2, fs2, fh2 = svdq.w4a4_linear_requant(*args, s2, d2, prec, epi)
    torch.cuda.synchronize()
    assert torch.equal(fh2, fh) and torch.equal(fq2, fq)


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("M,K,N,bias,gelu", [
    (130, 256, 512, True, True),       # ragged M, two 256-channel tiles
    (64, 512, 320, False, False),      # last channel tile 64 wide
    (1, 256, 64, True, True),
    (300, 512, 1024, True, True),
    (600, 768, 768, True, True),       # three tiles of N, M over two MX token tiles
])
def test_requant_matches_unfused(prec, M, K, N, bias, gelu):
    _say(f"requant prec={prec} M={M} K={K} N={N} bias={bias} gelu={gelu}")
    _requant_case(M, K, N, bias, gelu, prec)


@pytest.mark.parametrize("prec", PRECS)
def test_requant_mlp_full_size(prec):
    """fc1 (4608 x 3072 -> 12288, GELU) feeding fc2's activation step at the
    bench's size: every row's codes, scales and h2 against the separate step
    and against the oracle."""
    _say(f"requant full-size fc1 -> fc2 prec={prec}")
    _requant_case(4608, 3072, 12288, True, True, prec)


# ------------------------------------------------- full sizes, bench launches

@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("K", [256, 768])
def test_linear_many_tiles_ragged(prec, K):
    """More output tiles than CUs (the persistent kernels take several each),
    ragged in both M and N, one and an odd number of 256-channel steps per
    tile; every output against the oracle."""
    M, N = 2000, 9000
    _say(f"linear many tiles prec={prec} M={M} K={K} N={N}")
    L, p = _layer("qkv", M, K, N, prec)
    xq, xs, h, oh = _quant_act_check(L["X"], p["smooth"], p["down"], prec)
    Y = svdq.w4a4_linear(xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]), prec,
                         svdq.EPI_GELU_TANH)
    torch.cuda.synchronize()
    y_ref = O.linear(_np(xq), _np(xs), oh, p["wq"], p["wscale"], p["up"], L["bias"], prec, gelu=True)
    _y_check(Y, y_ref, "many tiles")


@pytest.mark.parametrize("M,K,N", [(2100, 64, 4000), (2100, 192, 4000), (2100, 704, 4000), (2100, 3072, 4000),
                                   (1500, 704, 5880)])
def test_linear_int4_tail_pieces(M, K, N):
    """INT4 shapes whose tiles fill whole rounds of one block per CU plus a
    few: 2100 x 4000 has 17 x 16 = 272 tiles on 256 CUs, 16 left over, which
    run as 16 pieces of 64 x 32 each; 1500 x 5880 has 12 x 23 = 276, 20 left
    over, as 8 pieces of 64 x 64 each.  K is split over the block's waves
    (one group: only the last wave has any; three, so some waves have none;
    eleven, uneven; 48).  Every output against the oracle, and a second call
    gives the same bits."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the split into whole rounds below assumes 256 CUs")
    prec = svdq.INT4
    _say(f"linear INT4 tail pieces M={M} K={K} N={N}")
    L, p = _layer("qkv", M, K, N, prec)
    xq, xs, h, oh = _quant_act_check(L["X"], p["smooth"], p["down"], prec)
    w = (_t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]))
    Y = svdq.w4a4_linear(xq, xs, h, *w, prec, svdq.EPI_GELU_TANH)
    Y2 = svdq.w4a4_linear(xq, xs, h, *w, prec, svdq.EPI_GELU_TANH)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))
    y_ref = O.linear(_np(xq), _np(xs), oh, p["wq"], p["wscale"], p["up"], L["bias"], prec, gelu=True)
    _y_check(Y, y_ref, "tail pieces")


@pytest.mark.parametrize("prec", PRECS)
def test_largest_accepted_activation(prec):
    """The largest activation the calls accept: 65535 x 16384, one row short
    of SVDQ_MAX_ELEMENTS (2^30) elements, so the last token tile is ragged
    too.  The activation step's codes and scales bit-exact and h within the
    bound, and the linear's output within tolerance, on 48 rows: the first
    and last rows of the matrix and of several tiles, and random ones."""
    M, K, N = 65535, 16384, 256
    assert M * K < (1 << 30) <= (M + 1) * K
    _say(f"largest activation prec={prec} M={M} K={K} N={N}")
    rng = np.random.default_rng(2026)
    X = np.empty((M, K), np.uint16)
    for r0 in range(0, M, 4096):
        b = min(4096, M - r0)
        X[r0:r0 + b] = synth.f32_to_bf16_bits(rng.standard_normal((b, K), dtype=np.float32))
    X[:, 7] = synth.f32_to_bf16_bits(np.full(M, 40.0, np.float32) * rng.standard_normal(M, dtype=np.float32))
    W = synth.f32_to_bf16_bits(rng.normal(0.0, 0.02, (N, K)).astype(np.float32))
    bias = synth.f32_to_bf16_bits(rng.normal(0.0, 0.01, N).astype(np.float32))
    Xt = _t(X)
    act = Xt.abs().amax(dim=0).float().cpu().numpy()
    p = svdq.pack_weights(W, act, prec=prec)
    xq, xs, h = svdq.quantize_act(Xt, _t(p["smooth"]), _t(p["down"]), prec)
    Y = svdq.w4a4_linear(xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(bias), prec, svdq.EPI_NONE)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 4607, 4608, M - 257, M - 256, M - 129, M - 128,
                                      M - 2, M - 1], rng.choice(M, 34, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    gq, gs, gh = _np(xq[ridx]), _np(xs[ridx]), _np(h[ridx])
    oq, os_, oh = O.quant_act(X[rows], p["smooth"], p["down"], prec)
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    assert np.array_equal(gs.view(np.uint8), os_.view(np.uint8))
    assert np.all(np.abs(gh.astype(np.float64) - oh) <= _h_bound(X[rows], p["down"]))
    y_ref = O.linear(gq, gs, oh, p["wq"], p["wscale"], p["up"], bias, prec)
    _y_check(Y[ridx], y_ref, "largest activation")


@pytest.mark.parametrize("prec,tokens", [(svdq.INT4, 4608), (svdq.MXFP4, 4608), (svdq.MXFP4, 1024)])
def test_full_size_dit_block(prec, tokens):
    """QKV and the fc1 -> fc2 MLP pair at 4608 tokens (1024 for the MXFP4
    512 x 512 image), hidden 3072, in the launch configuration the benchmark
    times: codes, scales and h of every row bit-exact / bounded, and every
    output of every row against the oracle."""
    _say(f"full-size DiT block prec={prec} tokens={tokens}")
    if prec == svdq.INT4:
        names = ("qkv", "fc1", "fc2")
    else:
        names = ("mx_qkv", "mx_fc1", "mx_fc2") if tokens == 4608 else ("mx1k_qkv", "mx1k_fc1", "mx1k_fc2")
    q = synth.make_layer(synth.SPECS[names[0]])
    pq = svdq.pack_weights(q["W"], q["act_absmax"], prec=prec)
    xq, xs, h, oh = _quant_act_check(q["X"], pq["smooth"], pq["down"], prec)
    Y = svdq.w4a4_linear(xq, xs, h, _t(pq["wq"]), _t(pq["wscale"]), _t(pq["up"]), _t(q["bias"]), prec)
    torch.cuda.synchronize()
    y_ref = O.linear(_np(xq), _np(xs), oh, pq["wq"], pq["wscale"], pq["up"], q["bias"], prec)
    _y_check(Y, y_ref, names[0])
    del y_ref
    _say("  fc1")
    f1 = synth.make_layer(synth.SPECS[names[1]])
    p1 = svdq.pack_weights(f1["W"], f1["act_absmax"], prec=prec)
    xq, xs, h, oh = _quant_act_check(f1["X"], p1["smooth"], p1["down"], prec)
    Y1 = svdq.w4a4_linear(xq, xs, h, _t(p1["wq"]), _t(p1["wscale"]), _t(p1["up"]), _t(f1["bias"]), prec,
                          svdq.EPI_GELU_TANH)
    torch.cuda.synchronize()
    y_ref = O.linear(_np(xq), _np(xs), oh, p1["wq"], p1["wscale"], p1["up"], f1["bias"], prec, gelu=True)
    _y_check(Y1, y_ref, names[1])
    del y_ref
    _say("  fc2 (fc1 output re-quantized)")
    Y1b = _np(Y1)
    f2 = synth.make_layer(synth.SPECS[names[2]], X_bits=Y1b)
    p2 = svdq.pack_weights(f2["W"], f2["act_absmax"], prec=prec)
    xq, xs, h, oh = _quant_act_check(Y1b, p2["smooth"], p2["down"], prec)
    Y2 = svdq.w4a4_linear(xq, xs, h, _t(p2["wq"]), _t(p2["wscale"]), _t(p2["up"]), _t(f2["bias"]), prec)
    torch.cuda.synchronize()
    y_ref = O.linear(_np(xq), _np(xs), oh, p2["wq"], p2["wscale"], p2["up"], f2["bias"], prec)
    _y_check(Y2, y_ref, names[2])


# ------------------------------------------------------- AWQ W4A16 (INT4 g64)

def _awq_case(M, K, N, bias=True, seed=0):
    rng = np.random.default_rng(seed + 17 * M + K + N)
    X = synth.f64_to_bf16_bits(rng.standard_normal((M, K)))
    w = rng.normal(0, 0.02, (N, K))
    w[:, rng.choice(K, 4, replace=False)] *= 30.0
    W = synth.f64_to_bf16_bits(w)
    b = synth.f64_to_bf16_bits(rng.normal(0, 0.01, N)) if bias else None
    return X, W, b


def _awq_run(X, W, b):
    wq, ws = svdq.awq_pack_weights(W)
    owq, ows = O.awq_pack(W)
    assert np.array_equal(wq, owq) and np.array_equal(ws.view(np.uint32), ows.view(np.uint32))
    Y = svdq.awq_w4a16_linear(_t(X), _t(wq), _t(ws), _t(b))
    torch.cuda.synchronize()
    return Y, wq, ws


@pytest.mark.parametrize("M,K,N", [(1, 256, 16), (3, 768, 40), (16, 512, 33), (17, 256, 64), (40, 1024, 130)])
def test_awq_exact_small_integers(M, K, N):
    """Every step exact: X in {-1, 0, 1} (8 non-zeros per row), W = q 2^-4 with
    a +-7 in every group (scale 2^-4), so y = (sum x q) / 16 is a bf16 number
    and the kernel must return it bit for bit -- a check of the storage order,
    the operand layout and the offset removal."""
    rng = np.random.default_rng(M * 1000 + N)
    x = np.zeros((M, K))
    for m in range(M):
        ks = rng.choice(K, 8, replace=False)
        x[m, ks] = rng.choice([-1.0, 1.0], 8)
    q = rng.integers(-7, 8, (N, K)).astype(np.float64)
    q[:, ::64] = np.where(rng.random((N, K // 64)) < 0.5, 7.0, -7.0)
    X = synth.f64_to_bf16_bits(x)
    W = synth.f64_to_bf16_bits(q / 16.0)
    Y, wq, ws = _awq_run(X, W, None)
    assert np.all(ws == np.float32(1 / 16))
    y_ref = O.awq_linear(X, wq, ws, None)
    assert np.array_equal(bf16_bits_to_f32(_np(Y)).astype(np.float64), y_ref)


@pytest.mark.parametrize("M,K,N,bias", [(1, 256, 48, True), (2, 3072, 9216, True), (5, 512, 130, False),
                                        (16, 1024, 64, True), (33, 768, 96, True)])
def test_awq_synthetic(M, K, N, bias):
    X, W, b = _awq_case(M, K, N, bias)
    _say(f"awq M={M} K={K} N={N} bias={bias}")
    Y, wq, ws = _awq_run(X, W, b)
    _y_check(Y, O.awq_linear(X, wq, ws, b), f"awq {M}x{K}x{N}")


def test_awq_full_size_modulation():
    """The modulation shape the benchmark times: 1 x 3072 -> 18432."""
    lay = synth.make_layer(synth.SPECS["awq_mod"])
    _say("awq full size 1 x 3072 -> 18432")
    Y, wq, ws = _awq_run(lay["X"], lay["W"], lay["bias"])
    _y_check(Y, O.awq_linear(lay["X"], wq, ws, lay["bias"]), "awq modulation")


def test_awq_deterministic_and_empty():
    X, W, b = _awq_case(4, 512, 64)
    wq, ws = svdq.awq_pack_weights(W)
    Y1 = svdq.awq_w4a16_linear(_t(X), _t(wq), _t(ws), _t(b))
    Y2 = svdq.awq_w4a16_linear(_t(X), _t(wq), _t(ws), _t(b))
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    Y0 = svdq.awq_w4a16_linear(_t(X[:0]), _t(wq), _t(ws), _t(b))
    torch.cuda.synchronize()
    assert Y0.shape == (0, 64)


# ------------------------------- QKV projection + Q/K RMS-norm + rotary (INT4)

def _qkvnorm_case(M, K, N, bias=True, rows=None, eps=1e-6, prec=svdq.INT4):
    L, p = _layer("qkv", M, K, N, prec, bias=bias)
    nq, nk = synth.gen_qk_norm(2, 10), synth.gen_qk_norm(2, 11)
    c, s = synth.gen_rope(M)
    xq, xs, h, oh = _quant_act_check(L["X"], p["smooth"], p["down"], prec)
    Y = svdq.w4a4_linear_qkv_norm_rope(xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]),
                                       _t(nq), _t(nk), eps, _t(c), _t(s), prec)
    Yp = svdq.w4a4_linear(xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]), prec)
    torch.cuda.synchronize()
    ylin = O.linear(_np(xq), _np(xs), oh, p["wq"], p["wscale"], p["up"], L["bias"], prec, rows=rows)
    sel = slice(None) if rows is None else rows
    pick = (lambda t: t) if rows is None else (lambda t: t[torch.from_numpy(rows).long().cuda()])
    # the projection itself, as the plain kernel stores it, against the oracle
    _y_check(pick(Yp), ylin, f"qkv projection {M}x{K}->{N}")
    # the norm and rotation consume that bf16 projection on both sides (the
    # bf16 rounding is a decision taken once, in fp32, by the GPU; a 1-ulp
    # difference there can exceed the tolerance after a rotation cancels)
    yb = bf16_bits_to_f32(_np(pick(Yp))).astype(np.float64)
    y_ref = O.qkv_norm_rope(yb, nq, nk, eps, c[sel], s[sel])
    _y_check(pick(Y), y_ref, f"qkv norm rope {M}x{K}->{N}")
    # V heads are exactly what the plain linear stores
    H = N // 384
    yv = _np(Y)[:, 256 * H:]
    assert np.array_equal(yv, _np(Yp)[:, 256 * H:])
    return Y


@pytest.mark.parametrize("M,K,N,bias", [(64, 256, 384, True), (130, 512, 768, False), (257, 320, 1152, True),
                                        (1, 128, 384, True)])
def test_qkv_norm_rope_synthetic(M, K, N, bias):
    _say(f"qkv norm rope M={M} K={K} N={N} bias={bias}")
    _qkvnorm_case(M, K, N, bias)


@pytest.mark.parametrize("M,K,N,bias", [(64, 256, 384, True), (130, 512, 768, False), (300, 1024, 1152, True),
                                        (1, 256, 384, True), (600, 768, 3072, True)])
def test_qkv_norm_rope_mx_synthetic(M, K, N, bias):
    """The MXFP4 form (the persistent LDS-DMA kernel, K % 256 == 0): a head is
    one wave's 128 channels; odd head counts leave half of the last 256-wide
    channel tile empty."""
    _say(f"qkv norm rope mx M={M} K={K} N={N} bias={bias}")
    _qkvnorm_case(M, K, N, bias, prec=svdq.MXFP4)


def test_qkv_norm_rope_mx_needs_whole_steps():
    L, p = _layer("qkv", 16, 320, 384, svdq.MXFP4)
    xq, xs, h = svdq.quantize_act(_t(L["X"]), _t(p["smooth"]), _t(p["down"]), svdq.MXFP4)
    c, s = synth.gen_rope(16)
    with pytest.raises(svdq.SvdqError) as e:
        svdq.w4a4_linear_qkv_norm_rope(xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), None,
                                       _t(synth.gen_qk_norm(2, 10)), _t(synth.gen_qk_norm(2, 11)), 1e-6, _t(c), _t(s),
                                       svdq.MXFP4)
    assert e.value.status == -4


@pytest.mark.parametrize("eps_factor", [1.0, 4.0])
def test_qkv_norm_rope_eps_comparable_to_mean_square(eps_factor):
    """eps set to a multiple of the Q/K heads' mean square, so that eps decides
    a large part of every output: agreement with the oracle then pins where
    eps enters (the same outputs checked against the oracle without eps must
    fail the tolerance, which shows the check can see it)."""
    M, K, N = 130, 512, 768
    _say(f"qkv norm rope eps = {eps_factor} x mean square")
    L, p = _layer("qkv", M, K, N, svdq.INT4)
    nq, nk = synth.gen_qk_norm(2, 10), synth.gen_qk_norm(2, 11)
    c, s = synth.gen_rope(M)
    xq, xs, h = svdq.quantize_act(_t(L["X"]), _t(p["smooth"]), _t(p["down"]), svdq.INT4)
    lin = (xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]))
    Yp = svdq.w4a4_linear(*lin, svdq.INT4)
    torch.cuda.synchronize()
    yb = bf16_bits_to_f32(_np(Yp)).astype(np.float64)
    H = N // 384
    eps = float(eps_factor * np.mean(yb[:, :256 * H] ** 2))
    Y = svdq.w4a4_linear_qkv_norm_rope(*lin, _t(nq), _t(nk), eps, _t(c), _t(s))
    torch.cuda.synchronize()
    _y_check(Y, O.qkv_norm_rope(yb, nq, nk, eps, c, s), f"qkv norm rope eps={eps:.4g}")
    with pytest.raises(AssertionError):
        _y_check(Y, O.qkv_norm_rope(yb, nq, nk, 0.0, c, s), "eps left out")


@pytest.mark.parametrize("K", [256, 704])
def test_qkv_norm_rope_int4_tail_pieces(K):
    """2800 tokens x 3072 channels (8 heads each of Q, K, V): 22 x 12 = 264
    INT4 tiles on 256 CUs, the 8 left over computed in pieces of 32 tokens x
    one head with K split over a block's waves.  Every output against the
    oracle, V heads bit-equal to the plain linear's (whose leftover tiles
    take the same pieces' sums)."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the split into whole rounds below assumes 256 CUs")
    _say(f"qkv norm rope INT4 tail pieces K={K}")
    _qkvnorm_case(2800, K, 3072)


@pytest.mark.parametrize("prec", PRECS)
def test_qkv_norm_rope_full_size(prec):
    """4608 tokens x 3072 -> 9216 (24 heads each of Q, K, V) with the
    FLUX-like rotary table; every output of every token (text and image)."""
    _say(f"qkv norm rope full size prec={prec}")
    _qkvnorm_case(4608, 3072, 9216, prec=prec)


def test_qkv_norm_rope_deterministic_and_empty():
    L, p = _layer("qkv", 40, 256, 384, svdq.INT4)
    nq, nk = synth.gen_qk_norm(2, 10), synth.gen_qk_norm(2, 11)
    c, s = synth.gen_rope(40)
    xq, xs, h, _ = _quant_act_check(L["X"], p["smooth"], p["down"], svdq.INT4)
    args = (xq, xs, h, _t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]), _t(nq), _t(nk), 1e-6, _t(c), _t(s))
    Y1 = svdq.w4a4_linear_qkv_norm_rope(*args)
    Y2 = svdq.w4a4_linear_qkv_norm_rope(*args)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    Y0 = svdq.w4a4_linear_qkv_norm_rope(xq[:0], xs[:0], h[:0], *args[3:10], _t(c[:0]), _t(s[:0]))
    torch.cuda.synchronize()
    assert Y0.shape == (0, 384)


# -------------------------------------------- NF4 W4A16 (weight-only, bf16 X)

def _nf4_case(M, K, N, bias=True, seed=0):
    rng = np.random.default_rng(seed + 31 * M + K + N)
    X = synth.f64_to_bf16_bits(rng.standard_normal((M, K)))
    W = synth.f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    b = synth.f64_to_bf16_bits(rng.normal(0, 0.01, N)) if bias else None
    return X, W, b


def _nf4_run(X, W, b, rows=None):
    """The library packs (its own storage order) and runs on the GPU; the
    oracle packs W itself (codes checked bit-exact against the library's in
    the CPU tests) and computes the fp64 reference."""
    lq, la, lc = svdq.nf4_pack_weights(W)
    oq, oa, oc = O.nf4_pack(W)
    Y = svdq.nf4_w4a16_linear(_t(X), _t(lq), _t(la), _t(lc), _t(b))
    torch.cuda.synchronize()
    return Y, O.nf4_linear(X, oq, oa, oc, b, rows=rows), (lq, la, lc), (oq, oa, oc)


@pytest.mark.parametrize("N,K", [(8, 64), (40, 128), (264, 3072), (1000, 640), (136, 12288)])
def test_nf4_dequantize_bit_exact(N, K):
    """The GPU's decoded weights (the values the linear multiplies) equal the
    oracle's w' = bf16(fl32(level * fl32(q d))) bit for bit."""
    _say(f"nf4 dequantize N={N} K={K}")
    _, W, _ = _nf4_case(4, K, N)
    W[0, :64] = 0                                     # a zero block
    lq, la, lc = svdq.nf4_pack_weights(W)
    oq, oa, oc = O.nf4_pack(W)
    Wd = svdq.nf4_dequantize(_t(lq), _t(la), _t(lc))
    torch.cuda.synchronize()
    want = O.nf4_dequant(oq, oa, oc, N, K)
    got = _np(Wd)
    assert np.array_equal(got, want), f"dequantized weights differ at {np.argwhere(got != want)[:5]}"


@pytest.mark.parametrize("M,K,N,bias", [(1, 64, 8, True), (37, 192, 24, False), (256, 256, 256, True),
                                        (300, 1024, 520, True), (257, 3072, 264, False), (513, 640, 1000, True),
                                        (64, 12288, 136, True)])
def test_nf4_linear_synthetic(M, K, N, bias):
    _say(f"nf4 linear M={M} K={K} N={N} bias={bias}")
    X, W, b = _nf4_case(M, K, N, bias)
    Y, y_ref, _, _ = _nf4_run(X, W, b)
    _y_check(Y, y_ref, f"nf4 {M}x{K}->{N}")


@pytest.mark.parametrize("name", ["nf4_qkv", "nf4_fc1"])
def test_nf4_full_size(name):
    """The comparison path's two workloads (4608 tokens, 3072 -> 9216 and
    3072 -> 12288, activations N(0, 1)): every output against the oracle."""
    lay = synth.make_layer(synth.SPECS[name])
    _say(f"nf4 full size {name}")
    Y, y_ref, _, _ = _nf4_run(lay["X"], lay["W"], lay["bias"])
    _y_check(Y, y_ref, name)


def test_nf4_deterministic_and_empty():
    X, W, b = _nf4_case(300, 512, 264)
    lq, la, lc = (_t(a) for a in svdq.nf4_pack_weights(W))
    Y1 = svdq.nf4_w4a16_linear(_t(X), lq, la, lc, _t(b))
    Y2 = svdq.nf4_w4a16_linear(_t(X), lq, la, lc, _t(b))
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    Y0 = svdq.nf4_w4a16_linear(_t(X[:0]), lq, la, lc, _t(b))
    torch.cuda.synchronize()
    assert Y0.shape == (0, 264)
