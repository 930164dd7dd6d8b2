"""Lifetime of the library-owned workspace under graph capture (C ABI rules
in include/wqbmm.h, "Workspace").

  * A call whose stream's workspace would have to grow while the stream is
    being captured returns WQBMM_ERR_CAPTURE and launches nothing.
  * A graph captured on a stream keeps working after an eager call of a
    larger shape has grown that stream's workspace: the buffer the graph
    uses is retired, not freed, and every replay reproduces the eager bits.

Shapes: the decode contraction at M = 16 (operands passed through the
workspace), the fused decode kernel at M = 1 with K = 8192 (its K-splits
meet in the workspace's accumulators), and a prefill call that needs a much
larger workspace.
"""
import numpy as np
import pytest

from weight_only_quantized_msd_amd import datagen

pytestmark = pytest.mark.gpu

DECODE, PREFILL, AUTO = 1, 2, 0


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_msd_amd as W
    W.lib()
    return torch


def announce(msg):
    print(f"\n[gpu case] {msg}", flush=True)


def case(torch, M, K, N, gs, seed):
    import weight_only_quantized_msd_amd as W
    d = datagen.random_case(M, K, N, gs, seed=seed)
    w = W.wqbmm_a16w4_tile_weights(torch.from_numpy(d["w_packed"]).cuda())
    return dict(x=torch.from_numpy(d["x"]).cuda(), w=w, s=torch.from_numpy(d["scale"]).cuda(),
                gs=gs, M=M, K=K, N=N)


def raw_call(W, c, y, path, stream):
    return W._lib.wqbmm_a16w4_msd_path_raw(c["x"].data_ptr(), c["w"].data_ptr(), c["s"].data_ptr(),
                                           c["gs"], c["M"], c["K"], c["N"], y.data_ptr(), path,
                                           int(stream.cuda_stream))


def test_growth_during_capture_is_refused(torch_dev):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    c = case(torch, 16, 1024, 256, 128, seed=11)
    s = torch.cuda.Stream()                       # a new stream: no workspace yet
    y = torch.full((c["M"], c["N"]), 3.0, dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    announce("capture on a stream without workspace")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rc = raw_call(W, c, y, DECODE, s)
    assert rc == W.WQBMM_ERR_CAPTURE, W.status_string(rc)
    g.replay()
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()), "a refused call launched work"
    # after one eager call the same capture succeeds and replays the eager bits
    with torch.cuda.stream(s):
        ref = W.wqbmm_a16w4_msd_path(c["x"], c["w"], c["s"], c["gs"], DECODE, stream=s)
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    y.fill_(3.0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g2, stream=s):
        rc = raw_call(W, c, y, DECODE, s)
    assert rc == W.WQBMM_OK, W.status_string(rc)
    for _ in range(3):
        y.fill_(3.0)
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


def test_graph_survives_growth_by_a_larger_eager_call(torch_dev):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    small = [case(torch, 16, 4096, 512, 128, seed=21),       # decode contraction: operands
             case(torch, 1, 8192, 1024, 128, seed=22)]       # fused decode, K split: accumulators
    big = case(torch, 2048, 4096, 1024, 128, seed=23)        # prefill: a far larger workspace
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        refs = [W.wqbmm_a16w4_msd_path(c["x"], c["w"], c["s"], c["gs"], DECODE, stream=s) for c in small]
    torch.cuda.synchronize()
    ys = [torch.empty_like(r) for r in refs]
    announce("capture the small calls")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c, y in zip(small, ys):
            assert raw_call(W, c, y, DECODE, s) == W.WQBMM_OK
    announce("grow the stream's workspace with an eager prefill call")
    with torch.cuda.stream(s):
        big_ref = W.wqbmm_a16w4_msd_path(big["x"], big["w"], big["s"], big["gs"], PREFILL, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        for y in ys:
            y.fill_(5.0)
        with torch.cuda.stream(s):
            g.replay()
            # eager work on the grown workspace between replays
            again = [W.wqbmm_a16w4_msd_path(c["x"], c["w"], c["s"], c["gs"], DECODE, stream=s)
                     for c in small]
            big_again = W.wqbmm_a16w4_msd_path(big["x"], big["w"], big["s"], big["gs"], PREFILL,
                                               stream=s)
        torch.cuda.synchronize()
        for y, r, a in zip(ys, refs, again):
            assert torch.equal(y.view(torch.int16), r.view(torch.int16)), rep
            assert torch.equal(a.view(torch.int16), r.view(torch.int16)), rep
        assert torch.equal(big_again.view(torch.int16), big_ref.view(torch.int16)), rep
    assert np.isfinite(big_ref.float().cpu().numpy()).all()
