"""Every device call captured in a HIP graph (as a serving loop or a HIP-graph
runtime would): each replay, with eager work, output clearing and
synchronizations in between, equals the eager launch bit for bit.  None of
the calls records a memset (outputs are cleared here by fill kernels,
outside the graph), and workspaces and the allocation-free call's static
buffer keep their addresses across replays.  Last, the calls from several
host threads at once, each on its own stream (default priority)."""
import numpy as np
import pytest

import w4a4_rank_corrected_quantize_amd as svdq
from w4a4_rank_corrected_quantize_amd import synth
from tests.test_gpu_parity import _layer, _nf4_case, _awq_case, _say, _t

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PRECS = [svdq.INT4, svdq.MXFP4]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    svdq.check_device()


def _replays_match(call, outs, replays=3):
    """Run `call` eagerly, capture it, then replay it `replays` times after
    clearing `outs`, with an unrelated eager kernel in between; every replay
    must reproduce the eager outputs exactly."""
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for _ in range(replays):
        for o in outs:
            o.zero_()
        scratch.normal_()                       # other work on the stream between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8) if o.dtype == torch.bfloat16 else o,
                               r.view(torch.uint8) if r.dtype == torch.bfloat16 else r)


def _acts(prec, M, K, N, bias=True):
    L, p = _layer("qkv", M, K, N, prec, bias=bias)
    xq, xs, h = svdq.quantize_act(_t(L["X"]), _t(p["smooth"]), _t(p["down"]), prec)
    torch.cuda.synchronize()
    w = (_t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]))
    return L, p, (xq, xs, h), w


@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_splitk(noalloc):
    _say(f"graph split-K noalloc={noalloc}")
    prec, M, K, N = svdq.MXFP4, 130, 2048, 264
    _, _, a, w = _acts(prec, M, K, N)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    need = svdq.linear_splitk_workspace_bytes(M, N, K, prec)
    assert need > 0
    work = torch.empty((need // 4,), dtype=torch.float32, device="cuda")
    if noalloc:
        call = lambda: svdq.w4a4_linear_splitk_noalloc(*a, *w, prec, svdq.EPI_GELU_TANH, Y=Y)  # noqa: E731
    else:
        call = lambda: svdq.w4a4_linear_splitk(*a, *w, prec, svdq.EPI_GELU_TANH, Y=Y, work=work)  # noqa: E731
    _replays_match(call, [Y])


@pytest.mark.parametrize("prec", PRECS)
def test_graph_requant(prec):
    _say(f"graph requant prec={prec}")
    M, K, N = 300, 512, 512
    _, _, a, w = _acts(prec, M, K, N)
    f2 = synth.make_layer(synth.SPECS["fc2"], M=M, K=N, N=64,
                          X_bits=synth.f64_to_bf16_bits(np.random.default_rng(3).standard_normal((M, N))))
    p2 = svdq.pack_weights(f2["W"], f2["act_absmax"], prec=prec)
    s2, d2 = _t(p2["smooth"]), _t(p2["down"])
    g = svdq.group_of(prec)
    sdt = torch.float32 if prec == svdq.INT4 else torch.uint8
    out = (torch.empty((M, N // 2), dtype=torch.uint8, device="cuda"),
           torch.empty((M, N // g), dtype=sdt, device="cuda"),
           torch.empty((M, svdq.RANK), dtype=torch.float32, device="cuda"))
    work = torch.empty((svdq.requant_workspace_bytes(M, N, prec=prec),), dtype=torch.uint8, device="cuda")
    _replays_match(lambda: svdq.w4a4_linear_requant(*a, *w, s2, d2, prec, svdq.EPI_GELU_TANH, out=out, work=work),
                   list(out))


@pytest.mark.parametrize("prec", PRECS)
def test_graph_qkv_norm_rope(prec):
    _say(f"graph qkv norm rope prec={prec}")
    M, K, N = 257, 512, 768
    _, _, a, w = _acts(prec, M, K, N)
    nq, nk = _t(synth.gen_qk_norm(2, 10)), _t(synth.gen_qk_norm(2, 11))
    c, s = synth.gen_rope(M)
    c, s = _t(c), _t(s)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _replays_match(lambda: svdq.w4a4_linear_qkv_norm_rope(*a, *w, nq, nk, 1e-6, c, s, prec, Y=Y), [Y])


def test_graph_int4_tail_pieces():
    """The INT4 linear and its Q/K-norm form at shapes whose leftover tiles
    run in pieces (two launches per call): both captured and replayed."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the split into whole rounds assumes 256 CUs")
    _say("graph INT4 tail pieces")
    prec = svdq.INT4
    M, K, N = 2100, 192, 4000           # 272 tiles: 16 left over
    _, _, a, w = _acts(prec, M, K, N)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _replays_match(lambda: svdq.w4a4_linear(*a, *w, prec, svdq.EPI_GELU_TANH, Y=Y), [Y])
    M, K, N = 2800, 256, 3072           # 264 tiles: 8 left over, 8 heads each of Q, K, V
    _, _, a, w = _acts(prec, M, K, N)
    nq, nk = _t(synth.gen_qk_norm(2, 10)), _t(synth.gen_qk_norm(2, 11))
    c, s = synth.gen_rope(M)
    c, s = _t(c), _t(s)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _replays_match(lambda: svdq.w4a4_linear_qkv_norm_rope(*a, *w, nq, nk, 1e-6, c, s, prec, Y=Y), [Y])


def test_graph_awq():
    _say("graph awq")
    M, K, N = 3, 1024, 264
    X, W, b = _awq_case(M, K, N)
    wq, ws = svdq.awq_pack_weights(W)
    Xt, wqt, wst, bt = _t(X), _t(wq), _t(ws), _t(b)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _replays_match(lambda: svdq.awq_w4a16_linear(Xt, wqt, wst, bt, Y=Y), [Y])


def test_graph_nf4():
    _say("graph nf4")
    M, K, N = 300, 640, 264
    X, W, b = _nf4_case(M, K, N)
    q, qa, ch = svdq.nf4_pack_weights(W)
    Xt, qt, qat, cht, bt = _t(X), _t(q), _t(qa), _t(ch), _t(b)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Wd = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    _replays_match(lambda: svdq.nf4_w4a16_linear(Xt, qt, qat, cht, bt, Y=Y), [Y])
    _replays_match(lambda: svdq.nf4_dequantize(qt, qat, cht, Wd=Wd), [Wd])


@pytest.mark.parametrize("prec", PRECS)
def test_concurrent_host_threads(prec):
    """The calls are thread-safe: four host threads, each on its own stream
    with its own buffers, run the activation step and the linear together
    (ctypes releases the GIL during the calls); every result equals the
    single-threaded one bit for bit."""
    import threading
    _say(f"host threads prec={prec}")
    M, K, N = 200, 768, 264
    L, p = _layer("qkv", M, K, N, prec)
    X, s, d = _t(L["X"]), _t(p["smooth"]), _t(p["down"])
    w = (_t(p["wq"]), _t(p["wscale"]), _t(p["up"]), _t(L["bias"]))
    xq, xs, h = svdq.quantize_act(X, s, d, prec)
    ref = svdq.w4a4_linear(xq, xs, h, *w, prec, svdq.EPI_GELU_TANH)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(t):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for i in range(5):
                    q, sc, hh = svdq.quantize_act(X, s, d, prec)
                    y = svdq.w4a4_linear(q, sc, hh, *w, prec, svdq.EPI_GELU_TANH)
                    results[(t, i)] = (q, y)
            st.synchronize()
        except Exception as e:      # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    assert len(results) == 20
    for (q, y) in results.values():
        assert torch.equal(q, xq)
        assert torch.equal(y.view(torch.uint8), ref.view(torch.uint8))
