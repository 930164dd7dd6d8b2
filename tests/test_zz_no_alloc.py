"""The allocation-free entry point wqbmm_a16w4_msd_noalloc (include/wqbmm.h)
against wqbmm_a16w4_msd, through the C ABI.

Both run the same kernels, so the outputs must be bit-identical.  Each case
makes two calls in a row on the entry point's one scratch array, the second
with a smaller input (fewer rows, and for the two-kernel paths a smaller K),
so that stale operands or accumulators from the first call would show.
Shapes cover every path: the fused decode kernel with K split over
workgroups (accumulators), the decode contraction (operands; one and several
column tiles per workgroup), and the prefill GEMMs at group sizes 128 and 64.
"""
import pytest

from weight_only_quantized_msd_amd import datagen

pytestmark = pytest.mark.gpu


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


def inputs(torch, M, K, N, gs, seed):
    import weight_only_quantized_msd_amd as W
    d = datagen.random_case(M, K, N, gs, seed=seed)
    w = W.wqbmm_a16w4_tile_weights(torch.from_numpy(d["w_packed"]).cuda())
    return torch.from_numpy(d["x"]).cuda(), w, torch.from_numpy(d["scale"]).cuda()


PAIRS = [  # (first call (M, K, N, gs), second, smaller call)
    ((4, 8192, 1024, 128), (1, 6272, 512, 64)),       # fused decode, K split: accumulators
    ((16, 4096, 1024, 128), (5, 1024, 512, 64)),      # decode contraction: operands
    ((16, 4096, 8192, 128), (9, 2048, 4608, 64)),     # decode contraction, several tiles per workgroup
    ((2048, 4096, 1024, 128), (130, 1024, 288, 128)),  # prefill, group size 128
    ((256, 2048, 2048, 64), (17, 512, 160, 64)),      # prefill, group size 64
]


@pytest.mark.parametrize("first,second", PAIRS, ids=[f"M{a[0]}K{a[1]}g{a[3]}-M{b[0]}" for a, b in PAIRS])
def test_noalloc_matches_msd_on_two_calls(torch_dev, first, second):
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    for i, (M, K, N, gs) in enumerate((first, second)):
        x, w, s = inputs(torch, M, K, N, gs, seed=M + K + N + i)
        announce(f"noalloc call {i} M={M} K={K} N={N} gs={gs}")
        ref = W.wqbmm_a16w4_msd(x, w, s, gs)
        y = torch.full((M, N), 9.0, dtype=torch.float16, device="cuda")
        W.wqbmm_a16w4_msd_noalloc(x, w, s, gs, y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), (i, M, K, N, gs)


def test_noalloc_back_to_back_and_repeat(torch_dev):
    """Queued back to back with no host sync in between, alternating shapes:
    every output equals the allocating entry point's."""
    import weight_only_quantized_msd_amd as W
    torch = torch_dev
    cases = [inputs(torch, *shape, seed=7 + j) + (shape,) for j, shape in
             enumerate([(1, 8192, 1024, 128), (12, 2048, 512, 128), (3, 4096, 256, 64)])]
    refs = [W.wqbmm_a16w4_msd(x, w, s, sh[3]) for (x, w, s, sh) in cases]
    torch.cuda.synchronize()
    announce("noalloc back to back")
    outs = []
    for rep in range(8):
        for (x, w, s, sh) in cases:
            y = torch.empty((sh[0], sh[2]), dtype=torch.float16, device="cuda")
            outs.append(W.wqbmm_a16w4_msd_noalloc(x, w, s, sh[3], y))
    torch.cuda.synchronize()
    for i, y in enumerate(outs):
        assert torch.equal(y.view(torch.int16), refs[i % len(cases)].view(torch.int16)), i


def test_noalloc_rejects_too_large_before_launch(torch_dev):
    """Real device buffers of the stated shapes (uninitialised: nothing reads
    them when the size check works), so that no call can reach a kernel with
    an invalid pointer."""
    import weight_only_quantized_msd_amd as W
    from weight_only_quantized_msd_amd import _lib as L
    torch = torch_dev
    announce("noalloc too large")

    def bufs(M, K, N, gs):
        x = torch.empty((M, K), dtype=torch.float16, device="cuda")
        w = torch.empty((N // 16, (K + 127) // 128 * 1024), dtype=torch.uint8, device="cuda")
        s = torch.empty((K // gs, N), dtype=torch.float16, device="cuda")
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        return x, w, s, y

    def call(M, K, N, gs, null_x=False):
        x, w, s, y = bufs(M, K, N, gs)
        rc = L.wqbmm_a16w4_msd_noalloc_raw(0 if null_x else x.data_ptr(), w.data_ptr(), s.data_ptr(), gs,
                                           M, K, N, y.data_ptr(), None)
        torch.cuda.synchronize()
        return rc

    # prefill operands beyond 62 MiB
    assert call(16384, 4096, 4096, 128) == W.WQBMM_ERR_TOO_LARGE
    # split-K accumulators beyond 2 MiB (M = 4, K > 4096, N = 131072)
    assert call(4, 8192, 131072, 128) == W.WQBMM_ERR_TOO_LARGE
    # the usual validation still comes first
    assert call(4, 256, 256, 128, null_x=True) == W.WQBMM_ERR_NULLPTR
