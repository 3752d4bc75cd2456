"""GPU parity of the W4A4 MX GEMV (page "w4a4_proj/mx_plan.rs", read as OCP
MXFP4) against the CPU oracle, through the C ABI.

Bar: every output within 2^-8 * sum|a*w*sa*sw| + ulp_bf16(oracle) (the same
form as the W8A16 GEMM's: the hardware takes exact FP4 products, applies the
two power-of-two block scales exactly and sums in FP32, whose error over K
terms stays far below 2^-8 of the absolute sum), and no NaN or Inf.  Data
whose FP32 sums are exact must match the oracle bit for bit: that pins the
nibble order, the per-lane scale layout and the block scales.
"""

import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def w8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp8_w8a16_amd as mod
    mod.library()
    return mod


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_mx(w8, p, plan=None, stream=None):
    a, asc, w, wsc = _dev(p.a), _dev(p.a_scale), _dev(p.w), _dev(p.w_scale)
    c = torch.from_numpy(p.c).view(torch.int16).cuda()
    st = w8.gemm_w4a4_raw(a.data_ptr(), p.a_row_stride, asc.data_ptr(), w.data_ptr(),
                          wsc.data_ptr(), c.data_ptr(), p.c_row_stride, p.m, p.n, p.k,
                          0 if stream is None else stream.cuda_stream, plan)
    assert st == 0, w8.last_error()
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16).reshape(p.c.shape)


def check_mx(p, g, exact=False):
    oc, tot, bound = oracle.gemm_w4a4(p.a, p.a_scale, p.w, p.w_scale, p.m, p.n, p.k,
                                      a_row_stride=p.a_row_stride)
    got = g[:p.m, :p.n]
    if exact:
        bad = np.argwhere(got != oc[:, :p.n])
        assert bad.size == 0, "first mismatches %s: gpu %s oracle %s" % (
            bad[:5].tolist(), got[tuple(bad[:5].T)], oc[tuple(bad[:5].T)])
    ok = oracle.within_tolerance(got, oc[:, :p.n], bound)
    assert ok.all(), np.argwhere(~ok)[:5]
    assert (g[:p.m, p.n:] == p.c[:p.m, p.n:]).all()
    assert (g[p.m:, :] == p.c[p.m:, :]).all()


def exact_mx(m, n, k, seed, a_row_stride=None, c_row_stride=None, c_extra_rows=1):
    """Random E2M1 codes (all 16) with scale exponents in {-1, 0, 1}: every
    product is a multiple of 2^-4 after scaling and |sum| <= 36 * 4 * K stays
    below 2^24 such units for K <= 2048, so FP32 sums are exact."""
    assert k <= 2048
    p = datagen.make_mx_problem(m, n, k, seed, a_row_stride, c_row_stride,
                                c_extra_rows=c_extra_rows)
    rng = np.random.default_rng(seed + 1)
    p.a[:, :k // 2] = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    p.w[...] = rng.integers(0, 256, size=p.w.shape, dtype=np.uint8)
    p.a_scale[...] = rng.integers(126, 129, size=p.a_scale.shape, dtype=np.uint8)
    p.w_scale[...] = rng.integers(126, 129, size=p.w_scale.shape, dtype=np.uint8)
    return p


W4A4_SHAPES = [(1, 1), (1, 2), (1, 4), (2, 1), (2, 2), (2, 4), (4, 1), (4, 2)]
# the built variants: two groups of 4 K steps of mb + nb blocks per wave
W4A4_VARIANTS = [(mb, nb, w) for mb, nb in W4A4_SHAPES for w in (4, 8, 16)
                 if w == 4 or (w == 8 and mb + nb <= 4) or (w == 16 and mb + nb <= 2)]


@pytest.mark.parametrize("mb,nb,waves", W4A4_VARIANTS)
def test_exact_data_every_w4a4_variant(w8, mb, nb, waves):
    """Ragged rows and columns, A pitch padding, K steps that leave a
    partial group of 4 and fewer groups than waves, whole groups of 4
    (16-byte scale loads), two and more row tiles."""
    for m, n, k in [(16 * mb - 3, 16 * nb * 3 + 5, 128 * 11), (16 * mb + 1, 16 * nb + 1, 256),
                    (16 * mb, 16 * nb * 2 - 1, 128 * 12)]:
        if m > 64 or m < 1:
            continue
        p = exact_mx(m, n, k, seed=100 * mb + 10 * nb + waves + m, a_row_stride=k + 64,
                     c_row_stride=n + 3)
        plan = w8.make_plan(m, n, k, w8.KERNEL_W4A4, mb, nb, 1, waves=waves)
        check_mx(p, run_mx(w8, p, plan), exact=True)


# 16 waves' partial tiles of four row blocks alone take 128 KiB of LDS
PS_CASES = [(m, w) for m in (1, 9, 16, 17, 32, 33, 48) for w in (4, 8, 16) if m <= 32 or w < 16]


@pytest.mark.parametrize("m,waves", PS_CASES)
def test_exact_data_persistent_w4a4(w8, m, waves):
    """Persistent kernel: equal contiguous tile ranges per workgroup, K
    split over the waves.  Many tiles per wave with whole tiles stored by
    one wave (4 workgroups), tiles split across several waves (one
    workgroup, long K), fewer tiles than workgroups, K with a partial group
    of 4 steps and K of whole groups; calls back to back on one stream."""
    mb = 1 if m <= 16 else (2 if m <= 32 else 4)
    stream = torch.cuda.Stream()
    cases = [(16 * 97 + 7, 128 * 9, 4), (16 * 97 + 7, 128 * 16, 4), (40, 128 * 15, 1),
             (16 * 3, 128 * 8, 16)]
    for seed, (n, k, cus) in enumerate(cases):
        lds = mb * 16 * (k // 2 + 16) + -(-(mb * 16 * (k // 32)) // 256) * 256 + waves * 2 * mb * 1024
        if lds > 160 * 1024 - 256:
            continue                       # A and the waves' partial tiles exceed LDS
        p = exact_mx(m, n, k, seed=500 + 7 * m + waves + seed, a_row_stride=k + 32,
                     c_row_stride=n + 1)
        plan = w8.make_plan(m, n, k, w8.KERNEL_W4A4_PS, mb, 1, 1, waves=waves, cu_count=cus)
        assert plan.grid == min(cus, -(-n // 16)) and plan.counter_count == 0
        check_mx(p, run_mx(w8, p, plan, stream), exact=True)


def test_every_e2m1_code_and_scale_lane(w8):
    """C[i][j] picks one weight element times one activation element: A row
    i is one-hot (1.0) at K position 37 i + 5 (every 32-element block and
    both nibbles over the rows), weight row j holds code (j + t) mod 16 at
    position t, and every row/block has its own scale exponent; the result is
    exactly w * 2^(ea + ew)."""
    m, n, k = 48, 64, 2048
    p = datagen.make_mx_problem(m, n, k, seed=3)
    codes = (np.arange(n)[:, None] + np.arange(k)[None, :]) % 16
    p.w[...] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    p.a[...] = 0
    pos = (37 * np.arange(m) + 5) % k
    for i, t in enumerate(pos):
        p.a[i, t // 2] = 0x02 << (4 * (t % 2))
    rng = np.random.default_rng(4)
    p.a_scale[...] = rng.integers(120, 135, size=p.a_scale.shape, dtype=np.uint8)
    p.w_scale[...] = rng.integers(120, 135, size=p.w_scale.shape, dtype=np.uint8)
    g = run_mx(w8, p)
    check_mx(p, g, exact=True)
    seen = set(codes[np.arange(n)[None, :], pos[:, None]].reshape(-1).tolist())
    assert seen == set(range(16))


@pytest.mark.parametrize("m,n,k,pitch", [(8, 4096, 4096, 4096), (16, 12288, 5120, 5120),
                                         (32, 6144, 2048, 2560), (3, 1000, 512, 640),
                                         (64, 2048, 4096, 4096), (16, 32768, 4096, 4096),
                                         (24, 33000, 2048, 2048), (40, 3000, 1152, 1152),
                                         (32, 2048, 16384, 16384), (1, 16, 128, 128)])
def test_w4a4_default_plans_full_parity(w8, m, n, k, pitch):
    """MXFP4-quantized N(0,1) activations and N(0,0.02) weights, default
    plans (tiled and persistent), every output against the oracle."""
    p = datagen.make_mx_problem(m, n, k, seed=m + n + k, a_row_stride=pitch,
                                c_row_stride=n + 8, c_extra_rows=1)
    plan = w8.plan_w4a4(m, n, k)
    check_mx(p, run_mx(w8, p))
    assert plan.kernel in (w8.KERNEL_W4A4, w8.KERNEL_W4A4_PS)


def test_w4a4_determinism_and_graph_replay(w8):
    m, n, k = 16, 32768, 2048                      # persistent plan
    assert w8.plan_w4a4(m, n, k).kernel == w8.KERNEL_W4A4_PS
    p = datagen.make_mx_problem(m, n, k, seed=9)
    a, asc, w, wsc = _dev(p.a), _dev(p.a_scale), _dev(p.w), _dev(p.w_scale)
    c = torch.zeros((m, n), dtype=torch.int16, device="cuda")
    stream = torch.cuda.Stream()

    def call():
        st = w8.gemm_w4a4_raw(a.data_ptr(), k, asc.data_ptr(), w.data_ptr(), wsc.data_ptr(),
                              c.data_ptr(), n, m, n, k, stream.cuda_stream)
        assert st == 0, w8.last_error()

    with torch.cuda.stream(stream):
        call()
        torch.cuda.synchronize()
        want = c.cpu().numpy().copy()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            call()
        for _ in range(3):
            c.fill_(0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(c.cpu().numpy(), want)
            call()
            torch.cuda.synchronize()
            assert np.array_equal(c.cpu().numpy(), want)


@pytest.mark.parametrize("m,n,k", [(8, 69632, 131072), (16, 540672, 16384)])
def test_w4a4_weight_above_4_gib_sampled(w8, m, n, k):
    """A packed FP4 weight of more than 4 GiB under the default plan (tiled,
    then persistent): row j holds E2M1 code 1 + j % 7 in both nibbles and
    its K blocks' scales cycle through 2^-1, 2^0, 2^1, so a row or K offset
    that wraps at 2^32 bytes reads other values; sampled outputs, including
    the rows just past 2^32 bytes and the last rows, against the oracle."""
    rng = np.random.default_rng(4444 + m)
    code = (1 + np.arange(n) % 7).astype(np.uint8)
    w = np.empty((n, k // 2), dtype=np.uint8)
    w[:] = (code | (code << 4))[:, None]
    assert w.nbytes > 1 << 32
    wsc = np.empty((n, k // 32), dtype=np.uint8)
    wsc[:] = (126 + np.arange(k // 32) % 3).astype(np.uint8)[None, :]
    a = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    asc = rng.integers(125, 130, size=(m, k // 32), dtype=np.uint8)
    print("W4A4 weight above 4 GiB: m=%d n=%d k=%d plan=%s"
          % (m, n, k, w8.plan_w4a4(m, n, k).as_dict()), flush=True)
    ad, ascd, wd, wscd = _dev(a), _dev(asc), _dev(w), _dev(wsc)
    c = torch.full((m + 1, n), 0x7777, dtype=torch.int16, device="cuda")
    st = w8.gemm_w4a4_raw(ad.data_ptr(), k, ascd.data_ptr(), wd.data_ptr(), wscd.data_ptr(),
                          c.data_ptr(), n, m, n, k)
    assert st == 0, w8.last_error()
    torch.cuda.synchronize()
    g = c.cpu().numpy().view(np.uint16)
    del ad, ascd, wd, wscd, c
    torch.cuda.empty_cache()
    rows, cols = datagen.sample_indices(m, n, 300, seed=12)
    wrap = (1 << 32) // (k // 2)               # first weight row past 2^32 bytes
    extra = np.array([n - 1, n - 2, wrap - 1, wrap, wrap + 1], dtype=np.uint32)
    rows = np.concatenate([rows, np.repeat(np.uint32(m - 1), 5), np.zeros(5, np.uint32)])
    cols = np.concatenate([cols, extra, extra])
    oc, _, bound = oracle.gemm_w4a4_at(a, asc, w, wsc, m, n, k, rows, cols)
    assert oracle.within_tolerance(g[rows, cols], oc, bound).all()
    assert (g[m, :] == 0x7777).all()


def test_w4a4_argument_errors_leave_c_untouched(w8):
    m, n, k = 8, 256, 512
    p = datagen.make_mx_problem(m, n, k, seed=5)
    a, asc, w, wsc = _dev(p.a), _dev(p.a_scale), _dev(p.w), _dev(p.w_scale)
    c = torch.full((m, n), 0x1234, dtype=torch.int16, device="cuda")
    ptrs = (a.data_ptr(), asc.data_ptr(), w.data_ptr(), wsc.data_ptr(), c.data_ptr())

    def call(ars, crs, mm, nn, kk, nullify=None):
        q = list(ptrs)
        if nullify is not None:
            q[nullify] = 0
        return w8.gemm_w4a4_raw(q[0], ars, q[1], q[2], q[3], q[4], crs, mm, nn, kk, 0)

    assert call(k, n, 0, n, k) == w8.ERR_M_ZERO
    assert call(k, n, m, n, 100) == w8.ERR_K_NOT_MULT_128
    assert call(k - 32, n, m, n, k) == w8.ERR_PITCH_TOO_SHORT
    assert call(k, n - 1, m, n, k) == w8.ERR_PITCH_TOO_SHORT
    assert call(k + 16, n, m, n, k) == w8.ERR_A_STRIDE_ALIGN
    assert call(k, n, m, 0, k) == w8.ERR_N_ZERO
    for i in range(5):
        assert call(k, n, m, n, k, nullify=i) == w8.ERR_NULL_PTR
    assert call(k, n, 65, n, k) == w8.ERR_BAD_PLAN
    assert call((1 << 24) + 32, n, m, n, k) == w8.ERR_BAD_PLAN     # A pitch past 2^24
    torch.cuda.synchronize()
    assert bool((c == 0x1234).all())


def test_w4a4_torch_wrapper(w8):
    m, n, k = 5, 300, 1024
    p = datagen.make_mx_problem(m, n, k, seed=6, a_row_stride=1056)
    a, asc, w, wsc = _dev(p.a), _dev(p.a_scale), _dev(p.w), _dev(p.w_scale)
    c = w8.gemm_w4a4(a, asc, w, wsc, k)
    torch.cuda.synchronize()
    got = c.view(torch.int16).cpu().numpy().view(np.uint16)
    oc, _, bound = oracle.gemm_w4a4(p.a, p.a_scale, p.w, p.w_scale, m, n, k,
                                    a_row_stride=1056)
    assert oracle.within_tolerance(got, oc, bound).all()
