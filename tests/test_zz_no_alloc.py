"""w8a16_gemm_noalloc (split-K scratch in a static device array, no
allocation) against w8a16_gemm, through the C ABI: identical bits for the
same default plan, on two calls in a row (the second smaller), for plans
that split K in the stream kernel and in the tile kernel and for one that
does not; a plan beyond the scratch is refused with C untouched."""

import numpy as np
import pytest

import datagen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def w8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp8_w8a16_amd as mod
    mod.library()
    return mod


def _bufs(p):
    dev = torch.device("cuda")
    return (torch.from_numpy(p.a).view(torch.int16).to(dev), torch.from_numpy(p.w).to(dev),
            torch.from_numpy(p.scale).to(dev), torch.from_numpy(p.c).view(torch.int16).to(dev))


def _call(w8, fn, p, bufs, stream):
    a, w, s, c = bufs
    st = fn(a.data_ptr(), p.a_row_stride, w.data_ptr(), s.data_ptr(), c.data_ptr(),
            p.c_row_stride, p.m, p.n, p.k, stream)
    assert st == 0, w8.last_error()


# (larger, smaller) pairs: stream-kernel K splits (narrow N), tile-kernel
# splits added by the reduction kernel, tile splits followed by stream splits,
# and a plan without splits.
PAIRS = [((16, 1024, 8192), (4, 512, 4096)),
         ((128, 4096, 8192), (72, 3072, 6144)),
         ((128, 4096, 8192), (16, 1024, 8192)),
         ((8, 4096, 4096), (3, 1000, 1024))]


@pytest.mark.parametrize("big,small", PAIRS)
def test_noalloc_matches_gemm_on_two_calls(w8, big, small):
    stream = torch.cuda.Stream()
    for i, (m, n, k) in enumerate((big, small)):
        plan = w8.plan(m, n, k)
        assert plan.workspace_bytes <= w8.NOALLOC_WORKSPACE_BYTES
        p = datagen.make_problem(m, n, k, seed=4400 + 10 * i + m, a_row_stride=k + 8,
                                 c_row_stride=n + 3, c_extra_rows=1)
        ref, got = _bufs(p), _bufs(p)
        torch.cuda.synchronize()
        _call(w8, w8.gemm_raw, p, ref, stream.cuda_stream)
        _call(w8, w8.gemm_noalloc_raw, p, got, stream.cuda_stream)
        torch.cuda.synchronize()
        r = ref[3].cpu().numpy().view(np.uint16)
        g = got[3].cpu().numpy().view(np.uint16)
        assert np.array_equal(r, g), "noalloc differs from w8a16_gemm at %s (plan %s)" % (
            (m, n, k), plan.as_dict())
        # pitch pad and the extra row keep their sentinel
        assert (g.reshape(p.c.shape)[:, p.n:] == p.c[:, p.n:]).all()
        assert (g.reshape(p.c.shape)[p.m:] == p.c[p.m:]).all()


def test_noalloc_refuses_a_plan_beyond_the_scratch(w8):
    # 384 x 8192 x 16384: 128-row tiles, 2 K splits of 64 steps -> 24 MiB of
    # partials, more than the 16 MiB scratch
    m, n, k = 384, 8192, 16384
    plan = w8.plan(m, n, k)
    assert plan.splits > 1 and plan.workspace_bytes > w8.NOALLOC_WORKSPACE_BYTES
    dev = torch.device("cuda")
    a = torch.zeros((m, k), dtype=torch.int16, device=dev)
    w = torch.zeros((n, k), dtype=torch.uint8, device=dev)
    s = torch.ones(((n + 127) // 128, k // 128), dtype=torch.float32, device=dev)
    c = torch.full((m, n), 0x1234, dtype=torch.int16, device=dev)
    torch.cuda.synchronize()
    st = w8.gemm_noalloc_raw(a.data_ptr(), k, w.data_ptr(), s.data_ptr(), c.data_ptr(), n,
                             m, n, k, 0)
    assert st == w8.ERR_WORKSPACE
    assert "scratch" in w8.last_error()
    torch.cuda.synchronize()
    assert bool((c == 0x1234).all())
    # argument checks come first, as in w8a16_gemm
    assert w8.gemm_noalloc_raw(a.data_ptr(), k, w.data_ptr(), s.data_ptr(), c.data_ptr(), n,
                               0, n, k, 0) == w8.ERR_M_ZERO
