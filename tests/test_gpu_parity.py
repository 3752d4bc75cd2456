"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar (written out in ``oracle.within_tolerance``): every output satisfies
|gpu - oracle| <= 2^-8 * sum|a*w*s| + ulp_bf16(oracle), and no GPU output is
NaN or infinite.  Data whose FP32 accumulation is exact must match the
oracle bit for bit, which the graded tolerance alone would not force.
"""

import warnings

import numpy as np
import pytest

import datagen
import oracle
from variants import plan_ok, tile_variants

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def w8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_fp8_w8a16_amd as mod
    mod.library()          # raises if the HIP library is not built
    return mod


def dev_u16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).view(torch.int16).cuda()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_gpu(w8, prob, plan=None, stream=None):
    """Run the GEMM on device copies of a datagen.Problem; returns the whole
    C buffer (BF16 bits, including pitch pad and extra rows)."""
    a = dev_u16(prob.a)
    w = dev(prob.w)
    s = dev(prob.scale)
    c = dev_u16(prob.c)
    st = w8.gemm_raw(a.data_ptr(), prob.a_row_stride, w.data_ptr(), s.data_ptr(),
                     c.data_ptr(), prob.c_row_stride, prob.m, prob.n, prob.k,
                     0 if stream is None else stream.cuda_stream, plan)
    assert st == 0, w8.last_error()
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16).reshape(prob.c.shape)


def check_full(prob, gpu_c, exact=False):
    m, n = prob.m, prob.n
    oc, tot, bound = oracle.gemm(prob.a, prob.w, prob.scale, m, n, prob.k,
                                 a_row_stride=prob.a_row_stride)
    g = gpu_c[:m, :n]
    if exact:
        bad = np.argwhere(g != oc)
        assert bad.size == 0, "first mismatches %s: gpu %s oracle %s" % (
            bad[:5].tolist(), g[tuple(bad[:5].T)], oc[tuple(bad[:5].T)])
    ok = oracle.within_tolerance(g, oc, bound)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        raise AssertionError("out of tolerance at %s: gpu %s oracle %s bound %s" % (
            bad.tolist(), oracle.bf16_bits_to_f64(g[tuple(bad.T)]),
            oracle.bf16_bits_to_f64(oc[tuple(bad.T)]), bound[tuple(bad.T)]))
    # everything outside [m, n] keeps the sentinel
    assert (gpu_c[:m, n:] == prob.c[:m, n:]).all()
    assert (gpu_c[m:, :] == prob.c[m:, :]).all()
    return oc, bound


# Largest weight code magnitude (exclusive) of exact_problem: exponent field
# e <= 8 (values up to 3.75) for K <= 1024, e <= 5 (up to 0.46875) above.
def _exact_code_top(k):
    return 0x48 if k <= 1024 else 0x30


def exact_problem(m, n, k, seed, a_row_stride=None, c_row_stride=None, c_extra_rows=1):
    """Operands whose products and FP32 sums are exact: A in {-2..2}, weight
    codes with |value| < 4 for K <= 1024 and < 1/2 for K <= 8192 (all
    subnormals included), scales in {1/2, 1, 2}.  Every product a*w is a
    multiple of 2^-9 and every scaled one a multiple of 2^-10; the largest
    possible |sum| over all of K, 2 * wmax * 2 * K, stays below 2^14, i.e.
    below 2^24 units of 2^-10, so every FP32 partial sum, in any order and
    with any split, is exact (asserted below)."""
    assert k <= 8192
    top = _exact_code_top(k)
    wmax = max(abs(oracle.e4m3_value(c)) for c in range(top))
    assert 2.0 * wmax * 2.0 * k < 2.0 ** 14, "exact_problem bound does not hold"
    rng = np.random.default_rng(seed)
    p = datagen.make_problem(m, n, k, seed, a_row_stride, c_row_stride,
                             c_extra_rows=c_extra_rows)
    a_int = rng.integers(-2, 3, size=(m, k)).astype(np.float32)
    p.a[:, :k] = datagen.to_bf16_bits(a_int)
    mag = rng.integers(0, top, size=(n, k), dtype=np.uint8)
    sign = rng.integers(0, 2, size=(n, k), dtype=np.uint8) << 7
    p.w[...] = mag | sign
    p.scale[...] = rng.choice(np.float32([0.5, 1.0, 2.0]), size=p.scale.shape)
    return p


# ----------------------------------------------------------- dequant exactness

def test_every_finite_e4m3_code_dequantizes_exactly(w8):
    """C[i, j] = W[j, pi(i)] * 1.0: one-hot rows of A pick single weights,
    and weight row j holds the codes (j + k) mod 256 (NaN codes -> 0)."""
    m, n, k = 16, 256, 256
    p = datagen.make_problem(m, n, k, seed=1, c_extra_rows=0)
    codes = (np.arange(n)[:, None] + np.arange(k)[None, :]) % 256
    codes[(codes == 0x7F) | (codes == 0xFF)] = 0
    p.w[...] = codes.astype(np.uint8)
    p.scale[...] = 1.0
    pick = np.arange(m) * 16 + 3          # 16 different columns, all residues
    a = np.zeros((m, k), np.float32)
    a[np.arange(m), pick] = 1.0
    p.a[:, :k] = datagen.to_bf16_bits(a)
    g = run_gpu(w8, p)
    want = np.empty((m, n), np.uint16)
    for i in range(m):
        for j in range(n):
            want[i, j] = oracle.bf16_rne(oracle.e4m3_value(int(codes[j, pick[i]])))
    got = g[:m, :n]
    # -0.0 (code 0x80) times +1 accumulates to +0 from a zero start: compare
    # values, then bits for everything nonzero
    gv, wv = oracle.bf16_bits_to_f64(got), oracle.bf16_bits_to_f64(want)
    assert np.array_equal(gv, wv)
    nz = wv != 0
    assert np.array_equal(got[nz], want[nz])
    # all 254 finite codes were exercised
    seen = set(codes[np.arange(n)[None, :], pick[:, None]].reshape(-1).tolist())
    assert seen == set(range(256)) - {0x7F, 0xFF}


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (5, 130, 512), (16, 256, 1024),
                                   (17, 100, 384), (32, 96, 256), (40, 200, 640),
                                   (64, 64, 128), (33, 1000, 1024)])
def test_exact_data_bit_exact_default_plan(w8, m, n, k):
    p = exact_problem(m, n, k, seed=m * 7 + n + k)
    g = run_gpu(w8, p)
    check_full(p, g, exact=True)


STREAM_SHAPES = [(1, 1), (1, 2), (1, 3), (1, 4), (1, 8), (2, 1), (2, 2), (2, 4),
                 (4, 1), (4, 2)]


# The collection-time filters below pass the plan's kernel and flag codes as
# numbers (kernel 1 stream, 2 tile, 3 ring; flag 4 XCD-local grouping): the
# package is imported inside plan_ok only.
def _stream_case(mb, nb, splits):
    return 16 * mb - 3, 16 * nb * 3 + 5, 1024 if splits == 1 else 128 * 7


# every (shape, depth, A staging, splits, waves) the stream kernel's planner
# accepts (the rest need more LDS than a CU has)
STREAM_VARIANTS = [(mb, nb, depth, direct, splits, waves)
                   for mb, nb in STREAM_SHAPES for depth in (1, 2, 4) for direct in (0, 1)
                   for splits in (1, 3) for waves in (4, 8, 16)
                   if plan_ok(*_stream_case(mb, nb, splits), 1, mb, nb, splits, depth=depth,
                              flags=direct, waves=waves)]


@pytest.mark.parametrize("mb,nb,depth,direct,splits,waves", STREAM_VARIANTS)
def test_exact_data_every_stream_variant(w8, mb, nb, depth, direct, splits, waves):
    m, n, k = _stream_case(mb, nb, splits)
    p = exact_problem(m, n, k, seed=100 * mb + 10 * nb + splits + 1000 * depth + waves)
    plan = w8.make_plan(m, n, k, w8.KERNEL_STREAM, mb, nb, splits, depth=depth,
                        flags=direct, waves=waves)
    g = run_gpu(w8, p, plan)
    check_full(p, g, exact=True)


def run_gpu_pair(w8, p1, p2, plan, stream):
    """Both problems enqueued back to back on `stream` with one plan (one
    split workspace), then one synchronisation; returns both C buffers."""
    bufs = []
    for prob in (p1, p2):
        a, w, s, c = dev_u16(prob.a), dev(prob.w), dev(prob.scale), dev_u16(prob.c)
        bufs.append((a, w, s, c))
    torch.cuda.synchronize()
    for prob, (a, w, s, c) in zip((p1, p2), bufs):
        st = w8.gemm_raw(a.data_ptr(), prob.a_row_stride, w.data_ptr(), s.data_ptr(),
                         c.data_ptr(), prob.c_row_stride, prob.m, prob.n, prob.k,
                         stream.cuda_stream, plan)
        assert st == 0, w8.last_error()
    torch.cuda.synchronize()
    return [c.cpu().numpy().view(np.uint16).reshape(prob.c.shape)
            for prob, (_, _, _, c) in zip((p1, p2), bufs)]


XCD_SHAPES = STREAM_SHAPES + [(2, 8)]


def _xcd_case(mb, nb, ksteps):
    return 16 * mb - 3, 16 * nb * 8 - 5, 128 * ksteps


XCD_VARIANTS = [(mb, nb, splits, ksteps, waves)
                for mb, nb in XCD_SHAPES for splits, ksteps in ((2, 16), (4, 13), (8, 64))
                for waves in (4, 8, 16)
                if plan_ok(*_xcd_case(mb, nb, ksteps), 1, mb, nb, splits, depth=1, flags=4,
                           waves=waves)]


@pytest.mark.parametrize("mb,nb,splits,ksteps,waves", XCD_VARIANTS)
def test_exact_data_xcd_local_splits(w8, mb, nb, splits, ksteps, waves):
    """Split plans grouped per XCD: 8 tiles (one per XCD range), two
    different problems back to back on one stream, so a partial read
    before its writer's stores completed (or a stale one from the previous
    call) breaks bit exactness."""
    m, n, k = _xcd_case(mb, nb, ksteps)
    p1 = exact_problem(m, n, k, seed=7000 + 100 * mb + 10 * nb + splits + waves)
    p2 = exact_problem(m, n, k, seed=9000 + 100 * mb + 10 * nb + splits + waves)
    plan = w8.make_plan(m, n, k, w8.KERNEL_STREAM, mb, nb, splits, depth=1,
                        flags=w8.FLAG_XCD_LOCAL, waves=waves)
    assert plan.grid == 8 * plan.splits and plan.flags == w8.FLAG_XCD_LOCAL
    g1, g2 = run_gpu_pair(w8, p1, p2, plan, torch.cuda.Stream())
    check_full(p1, g1, exact=True)
    check_full(p2, g2, exact=True)


def test_xcd_local_splits_on_concurrent_streams(w8):
    """Split plans on two streams at once (each stream has its own split
    split workspace and counters): four calls per stream, interleaved, with no
    synchronisation between them; every result bit-exact."""
    m, n, k = 13, 16 * 4 * 8 - 3, 128 * 32
    plan = w8.make_plan(m, n, k, w8.KERNEL_STREAM, 1, 4, 4, depth=1,
                        flags=w8.FLAG_XCD_LOCAL, waves=8)
    assert plan.splits == 4 and plan.grid == 32
    probs = [exact_problem(m, n, k, seed=8400 + i) for i in range(8)]
    bufs = [(dev_u16(p.a), dev(p.w), dev(p.scale), dev_u16(p.c)) for p in probs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for i, (p, (a, w, s, c)) in enumerate(zip(probs, bufs)):
        st = w8.gemm_raw(a.data_ptr(), p.a_row_stride, w.data_ptr(), s.data_ptr(),
                         c.data_ptr(), p.c_row_stride, m, n, k, streams[i % 2].cuda_stream,
                         plan)
        assert st == 0, w8.last_error()
    torch.cuda.synchronize()
    for p, (_, _, _, c) in zip(probs, bufs):
        check_full(p, c.cpu().numpy().view(np.uint16).reshape(p.c.shape), exact=True)


@pytest.mark.parametrize("mb,nb", [(1, 1), (1, 4), (2, 2), (4, 1)])
@pytest.mark.parametrize("tiles,splits,ksteps", [(1, 8, 64), (2, 4, 16), (3, 8, 24),
                                                 (5, 3, 13)])
def test_exact_data_splits_across_xcds(w8, mb, nb, tiles, splits, ksteps):
    """Split plans without the XCD grouping: the logical id map spreads a
    tile's splits over several XCDs (one tile of 8 splits: one split per
    XCD), so partials cross L2s.  Two different problems back to back on
    one stream: a partial read before it was published, or a stale one from
    the previous call, breaks bit exactness."""
    m, n, k = 16 * mb - 1, 16 * nb * tiles - 3, 128 * ksteps
    p1 = exact_problem(m, n, k, seed=8100 + 100 * mb + 10 * nb + splits + tiles)
    p2 = exact_problem(m, n, k, seed=8200 + 100 * mb + 10 * nb + splits + tiles)
    plan = w8.make_plan(m, n, k, w8.KERNEL_STREAM, mb, nb, splits, depth=1, waves=4)
    assert plan.grid == tiles * splits and plan.flags == 0
    g1, g2 = run_gpu_pair(w8, p1, p2, plan, torch.cuda.Stream())
    check_full(p1, g1, exact=True)
    check_full(p2, g2, exact=True)


@pytest.mark.parametrize("m,n,k", [(1, 1024, 8192), (16, 1024, 8192), (4, 2048, 14336),
                                   (8, 512, 8192), (16, 1536, 5120), (32, 768, 2048),
                                   (1, 128, 65536)])
def test_default_split_plans_at_size_sampled(w8, m, n, k):
    """Default plans that split K (narrow N, splits grouped per XCD): two
    problems back to back on one stream, sampled parity of both."""
    plan = w8.plan(m, n, k)
    assert plan.splits > 1 and plan.flags & w8.FLAG_XCD_LOCAL
    p1 = datagen.make_problem(m, n, k, seed=m + n + k, c_extra_rows=1)
    p2 = datagen.make_problem(m, n, k, seed=m + n + k + 1, c_extra_rows=1)
    g1, g2 = run_gpu_pair(w8, p1, p2, None, torch.cuda.Stream())
    rows, cols = datagen.sample_indices(m, n, 300, seed=6)
    for p, g in ((p1, g1), (p2, g2)):
        oc, _, bound = oracle.gemm_at(p.a, p.w, p.scale, m, n, k, rows, cols,
                                      a_row_stride=p.a_row_stride)
        assert oracle.within_tolerance(g[rows, cols], oc, bound).all()
        assert (g[m:, :] == p.c[m:, :]).all()


def _big_weight(n, k):
    """[n, k] E4M3 codes 0x30 + j % 7 + b % 5 for row j, K block b: rows
    32768 apart and neighbouring K blocks hold different values."""
    w = np.empty((n, k), dtype=np.uint8)
    np.add((0x30 + np.arange(n) % 7).astype(np.uint8)[:, None],
           np.repeat((np.arange(k // 128) % 5).astype(np.uint8), 128)[None, :], out=w)
    return w


def _big_samples(m, n, k):
    rows, cols = datagen.sample_indices(m, n, 300, seed=11)
    wrap = (1 << 32) // k                      # first weight row past 2^32 bytes
    extra_c = np.array([n - 1, n - 2, wrap - 1, wrap, wrap + 1], dtype=np.uint32)
    rows = np.concatenate([rows, np.repeat(np.uint32(m - 1), 5), np.zeros(5, np.uint32)])
    return rows, np.concatenate([cols, extra_c, extra_c])


@pytest.mark.parametrize("m,n,k", [(3, 34816, 131072), (24, 36864, 131072),
                                   (128, 36864, 131072)])
def test_weight_above_4_gib_sampled(w8, m, n, k):
    """A weight of more than 4 GiB under the default plan (a stream plan, a
    ring plan and a tile plan with 16 K splits): W's code in row j, K block b is
    0x30 + j % 7 + b % 5, so a row or K offset that wraps at 2^32 bytes
    (rows 32768 apart differ in j % 7) reads other values; sampled outputs,
    including the last rows and those just past 2^32 bytes, against the
    oracle, and C's extra row untouched."""
    rng = np.random.default_rng(4242 + m)
    w = _big_weight(n, k)
    assert w.nbytes > 1 << 32
    scale = rng.uniform(0.5, 2.0, size=(-(-n // 128), k // 128)).astype(np.float32)
    a = datagen.to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    c = np.full((m + 1, n), datagen.C_SENTINEL, dtype=np.uint16)
    print("weight above 4 GiB: m=%d n=%d k=%d plan=%s" % (m, n, k, w8.plan(m, n, k).as_dict()),
          flush=True)
    ad, wd, sd, cd = dev_u16(a), dev(w), dev(scale), dev_u16(c)
    st = w8.gemm_raw(ad.data_ptr(), k, wd.data_ptr(), sd.data_ptr(), cd.data_ptr(), n, m, n, k)
    assert st == 0, w8.last_error()
    torch.cuda.synchronize()
    g = cd.cpu().numpy().view(np.uint16).reshape(c.shape)
    del ad, wd, sd, cd
    torch.cuda.empty_cache()
    rows, cols = _big_samples(m, n, k)
    oc, _, bound = oracle.gemm_at(a, w, scale, m, n, k, rows, cols)
    assert oracle.within_tolerance(g[rows, cols], oc, bound).all()
    assert (g[m, :] == datagen.C_SENTINEL).all()


RING_SHAPES = [(1, 1), (1, 2), (1, 4), (2, 1), (2, 2), (2, 4)]


def _ring_case(mb, nb, sk, depth, msmall):
    return 5 if msmall else 16 * mb - 3, 16 * nb * 3 + 5, 128 * (sk * (depth + 1) + 3)


# the 8-row A staging (msmall) applies to one M block; ring variants that
# are not built are not collected
RING_VARIANTS = [(mb, nb, sk, depth, wv, msmall)
                 for mb, nb in RING_SHAPES for sk in (4, 8) for depth in (2, 3, 4)
                 for wv in (8, 16) for msmall in (False, True)
                 if (not msmall or mb == 1) and
                 plan_ok(*_ring_case(mb, nb, sk, depth, msmall), 3, mb, nb, 1, depth=depth,
                         flags=0, waves=wv, stage_steps=sk)]


@pytest.mark.parametrize("mb,nb,sk,depth,wv,msmall", RING_VARIANTS)
def test_exact_data_every_ring_variant(w8, mb, nb, sk, depth, wv, msmall):
    """More stages than ring slots, a ragged last stage, ragged m and n."""
    m, n, k = _ring_case(mb, nb, sk, depth, msmall)
    plan = w8.make_plan(m, n, k, w8.KERNEL_RING, mb, nb, 1, depth=depth, flags=0,
                        waves=wv, stage_steps=sk)
    assert plan.flags == (w8.FLAG_A8 if msmall else 0)
    p = exact_problem(m, n, k, seed=mb * 1000 + nb * 100 + sk * 10 + depth + wv)
    check_full(p, run_gpu(w8, p, plan), exact=True)


def test_ring_kernel_strides_and_short_k(w8):
    """Pitched A and C, and K shorter than one stage (the whole ring is
    clamped loads but the first slot)."""
    for (m, n, k) in [(7, 300, 128 * 20), (16, 200, 128), (30, 100, 128 * 3)]:
        p = datagen.make_problem(m, n, k, seed=m + n + k, a_row_stride=k + 24,
                                 c_row_stride=n + 11, c_extra_rows=2)
        mb = 1 if m <= 16 else 2
        ran = 0
        for sk, depth, wv, nb in [(8, 4, 16, 1), (8, 3, 16, 1), (4, 3, 8, 2), (4, 2, 16, 1),
                                  (4, 3, 16, 2)]:
            try:
                plan = w8.make_plan(m, n, k, w8.KERNEL_RING, mb, nb, 1, depth=depth,
                                    flags=0, waves=wv, stage_steps=sk)
            except w8.W8A16Error:
                continue
            g = run_gpu(w8, p, plan)
            check_full(p, g)
            assert np.array_equal(g, run_gpu(w8, p, plan))
            ran += 1
        assert ran >= 2


TILE_VARIANTS = tile_variants()


# producer-wave layouts (6 and 10 waves) that are not built for a ring
# size are not collected
TILE_CASES = [(mb, nb, depth, a_depth, splits, m, waves)
              for mb, nb, depth, a_depth in TILE_VARIANTS for splits in (1, 3)
              for m in (40, 128, 200) for waves in (4, 6, 8, 10)
              if plan_ok(m, 16 * nb * 3 + 7, 128 * 23, 2, mb, nb, splits, depth=depth,
                         a_depth=a_depth, waves=waves)]


@pytest.mark.parametrize("mb,nb,depth,a_depth,splits,m,waves", TILE_CASES)
def test_exact_data_every_tile_variant(w8, mb, nb, depth, a_depth, splits, m, waves):
    """K long enough for both rings to wrap, in every split; 8 waves split
    every K step between two groups; 6 and 10 add two producer waves."""
    n, k = 16 * nb * 3 + 7, 128 * 23
    p = exact_problem(m, n, k, seed=7 * m + nb + 10 * depth + 100 * splits + a_depth + waves + mb)
    plan = w8.make_plan(m, n, k, w8.KERNEL_TILE, mb, nb, splits, depth=depth,
                        a_depth=a_depth, waves=waves)
    assert plan.block == 64 * waves
    g = run_gpu(w8, p, plan)
    check_full(p, g, exact=True)


@pytest.mark.parametrize("m,splits,n,ksteps",
                         [(m, sp, n, ks) for m in (1, 65, 128, 200) for sp in (1, 2, 3)
                          for n, ks in ((507, 8), (300, 7), (256, 1), (1031, 5)) if sp <= ks])
def test_exact_data_wide_tile(w8, m, splits, n, ksteps):
    """128 x 256 tiles (32x32x16 MFMAs, weight ring of 3 steps, A ring of 3
    half steps): ragged rows and columns, one and several row tiles, K
    splits including uneven ones, one-step splits, bit-exact."""
    k = 128 * ksteps
    p = exact_problem(m, n, k, seed=31 * m + n + 7 * splits + ksteps, a_row_stride=k + 40,
                      c_row_stride=n + 9, c_extra_rows=2)
    plan = w8.make_plan(m, n, k, w8.KERNEL_TILE, 8, 16, splits, depth=3, a_depth=3)
    assert plan.block == 256 and plan.lds_bytes == 147968
    g = run_gpu(w8, p, plan)
    check_full(p, g, exact=True)
    assert np.array_equal(g, run_gpu(w8, p, plan))


def test_wide_tile_long_k_and_strides(w8):
    """Rings that wrap many times (40 and 64 steps per split), pitches."""
    for m, n, ksteps, splits in [(130, 300, 40, 1), (128, 512, 128, 2), (97, 769, 40, 3)]:
        k = 128 * ksteps
        p = datagen.make_problem(m, n, k, seed=m + n + k, a_row_stride=k + 24,
                                 c_row_stride=n + 11, c_extra_rows=2)
        plan = w8.make_plan(m, n, k, w8.KERNEL_TILE, 8, 16, splits, depth=3, a_depth=3)
        g = run_gpu(w8, p, plan)
        check_full(p, g)
        assert np.array_equal(g, run_gpu(w8, p, plan))


def test_tile_kernel_long_k_and_strides(w8):
    p = datagen.make_problem(130, 300, 128 * 40, seed=21, a_row_stride=128 * 40 + 24,
                             c_row_stride=311, c_extra_rows=2)
    for mb, nb, depth, splits, a_depth, waves in [
            (8, 8, 5, 1, 2, 4), (8, 8, 3, 4, 3, 8), (8, 4, 6, 5, 2, 8), (8, 4, 4, 2, 3, 4),
            (8, 8, 4, 3, 2, 6), (8, 4, 6, 2, 3, 10), (4, 8, 6, 1, 2, 8), (4, 8, 4, 2, 3, 10),
            (4, 4, 8, 3, 3, 6), (4, 4, 6, 1, 2, 4), (4, 8, 3, 2, 6, 8), (4, 8, 4, 3, 5, 4),
            (4, 4, 6, 1, 6, 8), (4, 4, 8, 2, 4, 10)]:
        plan = w8.make_plan(p.m, p.n, p.k, w8.KERNEL_TILE, mb, nb, splits, depth=depth,
                            a_depth=a_depth, waves=waves)
        g = run_gpu(w8, p, plan)
        check_full(p, g)
        assert np.array_equal(g, run_gpu(w8, p, plan))


# ------------------------------------------------------------- workloads

@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_workload_full_parity(w8, idx):
    wl = datagen.workload(idx)
    p = datagen.make_workload(wl)
    g = run_gpu(w8, p)
    oc, bound = check_full(p, g)
    # the A pitch pad holds NaN: had it been read, outputs would be NaN
    assert np.isfinite(oracle.bf16_bits_to_f64(g[:p.m, :p.n])).all()


def test_largest_workload_full_parity(w8):
    """M=128, N=K=8192 (zero blocks, log-uniform scales): every one of the
    1 048 576 outputs against the whole FP64 oracle (about 8.6 G
    multiply-adds on the host cores)."""
    wl = datagen.workload(4)
    p = datagen.make_workload(wl)
    g = run_gpu(w8, p)
    check_full(p, g)
    assert np.isfinite(oracle.bf16_bits_to_f64(g[:p.m, :p.n])).all()


def test_determinism_and_plans_agree_within_tolerance(w8):
    p = datagen.make_problem(24, 3000, 2048, seed=77, a_row_stride=2056,
                             c_row_stride=3001, c_extra_rows=1)
    g1 = run_gpu(w8, p)
    g2 = run_gpu(w8, p)
    assert np.array_equal(g1, g2)
    check_full(p, g1)
    for mb, nb, splits, depth, direct, waves in [(2, 1, 1, 1, 0, 4), (2, 4, 4, 2, 1, 8),
                                                 (2, 2, 16, 4, 0, 4), (4, 2, 2, 2, 1, 16),
                                                 (2, 1, 3, 4, 1, 16), (2, 2, 1, 1, 1, 16)]:
        plan = w8.make_plan(p.m, p.n, p.k, w8.KERNEL_STREAM, mb, nb, splits, depth, direct,
                            waves)
        g = run_gpu(w8, p, plan)
        check_full(p, g)
        assert np.array_equal(g, run_gpu(w8, p, plan))


def test_m_sweep(w8):
    """Every row count the planner treats differently, 1..256."""
    for m in list(range(1, 41)) + [47, 63, 64, 65, 100, 127, 128, 129, 160, 192, 255, 256]:
        p = datagen.make_problem(m, 272, 384, seed=300 + m, c_extra_rows=1)
        g = run_gpu(w8, p)
        check_full(p, g)


@pytest.mark.parametrize("m,n,k", [(96, 4096, 4096), (192, 2048, 8192), (24, 8192, 8192),
                                   (48, 4096, 4096), (48, 8192, 8192), (40, 6144, 4096),
                                   (8, 12288, 5120), (65, 8192, 8192), (40, 6144, 2048),
                                   (48, 2048, 4096), (128, 4096, 4096), (96, 2048, 4096),
                                   (96, 4096, 6144)])
def test_default_plans_at_size_sampled(w8, m, n, k):
    """Default plans of the M sweep's larger shapes (three or four 32 x 64
    stream row tiles up to 128 rows over small weights, two 128-row tiles,
    ring with two row blocks, two 32-row stream tiles, one 64-row tile for
    33..64 rows over a large weight, two for 65 rows, 48-column stream
    tiles, 64-column tiles with 2 splits), sampled parity."""
    p = datagen.make_problem(m, n, k, seed=m + n + k, c_extra_rows=1)
    g = run_gpu(w8, p)
    rows, cols = datagen.sample_indices(m, n, 300, seed=5)
    oc, _, bound = oracle.gemm_at(p.a, p.w, p.scale, m, n, k, rows, cols,
                                  a_row_stride=p.a_row_stride)
    assert oracle.within_tolerance(g[rows, cols], oc, bound).all()
    assert (g[m:, :] == p.c[m:, :]).all()


def test_ragged_n_and_single_step(w8):
    for n in [1, 7, 16, 17, 127, 128, 129, 1000]:
        p = datagen.make_problem(3, n, 128, seed=400 + n, c_extra_rows=1)
        check_full(p, run_gpu(w8, p))


def test_scale_doubling_doubles_only_that_block(w8):
    p = exact_problem(8, 256, 512, seed=9)
    g0 = run_gpu(w8, p)
    p.scale[1, 2] *= 2
    g1 = run_gpu(w8, p)
    check_full(p, g1, exact=True)
    assert np.array_equal(g0[:, :128], g1[:, :128])   # other scale row untouched


def test_zero_weights_give_zero(w8):
    p = datagen.make_problem(8, 300, 256, seed=10)
    p.w[...] = 0
    g = run_gpu(w8, p)
    assert (oracle.bf16_bits_to_f64(g[:8, :300]) == 0).all()


def test_non_default_stream_and_torch_wrapper(w8):
    p = datagen.make_problem(12, 512, 1024, seed=11)
    a = dev_u16(p.a).view(torch.bfloat16)
    w = dev(p.w).view(torch.float8_e4m3fn)
    s = dev(p.scale)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        c = w8.gemm(a, w, s)
    st.synchronize()
    got = c.view(torch.int16).cpu().numpy().view(np.uint16)
    oc, _, bound = oracle.gemm(p.a, p.w, p.scale, p.m, p.n, p.k)
    assert oracle.within_tolerance(got, oc, bound).all()
    # strided views of A and C
    abig = torch.zeros((12, 1032), dtype=torch.bfloat16, device="cuda")
    abig[:, :1024] = a
    cbig = torch.zeros((12, 520), dtype=torch.bfloat16, device="cuda")
    w8.gemm(abig[:, :1024], w, s, cbig[:, :512])
    torch.cuda.synchronize()
    got2 = cbig[:, :512].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, got2)


@pytest.mark.parametrize("m,n,k", [(1, 1024, 8192), (32, 768, 2048), (8, 4096, 4096),
                                   (96, 4096, 6144)])
def test_graph_replays_match_eager(w8, m, n, k):
    """Calls captured into a HIP graph after a warm-up call (split workspace
    set up outside the capture), then
    replayed three times with eager calls and synchronisations between the
    replays: every replay gives the eager call's bits.  Covers stream K
    splits (narrow N), an unsplit stream plan and the tile kernel with its
    split-reduction kernel."""
    probs = [datagen.make_problem(m, n, k, seed=900 + i + m) for i in range(3)]
    bufs = [(dev_u16(p.a), dev(p.w), dev(p.scale), dev_u16(p.c)) for p in probs]
    stream = torch.cuda.Stream()

    def call(i):
        p, (a, w, s, c) = probs[i], bufs[i]
        st = w8.gemm_raw(a.data_ptr(), p.a_row_stride, w.data_ptr(), s.data_ptr(),
                         c.data_ptr(), p.c_row_stride, m, n, k, stream.cuda_stream)
        assert st == 0, w8.last_error()

    def outputs():
        return [c.cpu().numpy().view(np.uint16).reshape(p.c.shape)
                for p, (_, _, _, c) in zip(probs, bufs)]

    with torch.cuda.stream(stream):
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        eager = outputs()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(3):
                call(i)
        for rep in range(3):
            for _, _, _, c in bufs:
                c.fill_(0)
            call(rep % 3)                       # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for want, got in zip(eager, outputs()):
                assert np.array_equal(want, got), "replay %d differs from eager" % rep
    rows, cols = datagen.sample_indices(m, n, 200, seed=3)
    for p, g in zip(probs, eager):
        oc, _, bound = oracle.gemm_at(p.a, p.w, p.scale, m, n, k, rows, cols,
                                      a_row_stride=p.a_row_stride)
        assert oracle.within_tolerance(g[rows, cols], oc, bound).all()


def _bufs(p):
    return dev_u16(p.a), dev(p.w), dev(p.scale), dev_u16(p.c)


def _call_on(w8, p, bufs, stream):
    a, w, s, c = bufs
    return w8.gemm_raw(a.data_ptr(), p.a_row_stride, w.data_ptr(), s.data_ptr(), c.data_ptr(),
                       p.c_row_stride, p.m, p.n, p.k, stream.cuda_stream)


def test_graph_survives_workspace_growth(w8):
    """A graph captured with a small split plan keeps working after a larger
    plan has grown that stream's workspace (the old buffer stays alive), and
    a call that would have to grow the workspace during capture is refused
    with W8A16_ERR_WORKSPACE and enqueues nothing."""
    small = datagen.make_problem(8, 512, 4096, seed=61)        # stream kernel, 4 K splits
    big = datagen.make_problem(16, 1024, 8192, seed=62)        # 4 K splits, twice the slots
    assert w8.plan(8, 512, 4096).splits > 1
    assert w8.plan(16, 1024, 8192).workspace_bytes > w8.plan(8, 512, 4096).workspace_bytes
    sb, bb = _bufs(small), _bufs(big)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        assert _call_on(w8, small, sb, stream) == 0, w8.last_error()
        torch.cuda.synchronize()
        want = sb[3].cpu().numpy()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            assert _call_on(w8, small, sb, stream) == 0, w8.last_error()
        assert _call_on(w8, big, bb, stream) == 0, w8.last_error()     # grows the workspace
        torch.cuda.synchronize()
        big_first = bb[3].cpu().numpy()
        for rep in range(3):
            sb[3].fill_(0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(sb[3].cpu().numpy(), want), "replay %d" % rep
            assert _call_on(w8, big, bb, stream) == 0, w8.last_error()
            torch.cuda.synchronize()
            assert np.array_equal(bb[3].cpu().numpy(), big_first)
    check_full(small, want.view(np.uint16).reshape(small.c.shape))
    # a fresh stream has no workspace: capturing a split call there is refused
    fresh = torch.cuda.Stream()
    c_before = bb[3].clone()
    g2 = torch.cuda.CUDAGraph()
    with warnings.catch_warnings():
        warnings.filterwarnings("ignore", message="The CUDA Graph is empty")
        with torch.cuda.graph(g2, stream=fresh):
            st = _call_on(w8, big, bb, fresh)
    assert st == w8.ERR_WORKSPACE, (st, w8.last_error())
    assert "capturing" in w8.last_error()
    torch.cuda.synchronize()
    assert torch.equal(bb[3], c_before)


def test_tile_splits_then_stream_splits_on_one_stream(w8):
    """Tile and stream split plans alternating on one stream share its split
    workspace (partials, then the stream kernel's counters): every result
    exact."""
    t = exact_problem(128, 4096, 1024, seed=63)
    sp = exact_problem(8, 512, 1024, seed=64)
    tplan = w8.make_plan(128, 4096, 1024, w8.KERNEL_TILE, 4, 8, 2, depth=4, a_depth=4, waves=10)
    splan = w8.make_plan(8, 512, 1024, w8.KERNEL_STREAM, 1, 1, 4, depth=1, waves=8)
    stream = torch.cuda.Stream()
    tb, sbuf = _bufs(t), _bufs(sp)
    for _ in range(2):
        for prob, bufs, plan in ((t, tb, tplan), (sp, sbuf, splan)):
            a, w, s, c = bufs
            st = w8.gemm_raw(a.data_ptr(), prob.a_row_stride, w.data_ptr(), s.data_ptr(),
                             c.data_ptr(), prob.c_row_stride, prob.m, prob.n, prob.k,
                             stream.cuda_stream, plan)
            assert st == 0, w8.last_error()
    torch.cuda.synchronize()
    check_full(t, tb[3].cpu().numpy().view(np.uint16).reshape(t.c.shape), exact=True)
    check_full(sp, sbuf[3].cpu().numpy().view(np.uint16).reshape(sp.c.shape), exact=True)


def test_argument_errors_with_device_pointers(w8):
    p = datagen.make_problem(4, 64, 256, seed=12)
    a, w, s, c = dev_u16(p.a), dev(p.w), dev(p.scale), dev_u16(p.c)
    before = c.clone()
    args = (a.data_ptr(), 256, w.data_ptr(), s.data_ptr(), c.data_ptr(), 64)
    assert w8.gemm_raw(*args, 0, 64, 256) == w8.ERR_M_ZERO
    assert w8.gemm_raw(*args, 4, 64, 200) == w8.ERR_K_NOT_MULT_128
    assert w8.gemm_raw(a.data_ptr(), 128, w.data_ptr(), s.data_ptr(), c.data_ptr(),
                       64, 4, 64, 256) == w8.ERR_PITCH_TOO_SHORT
    assert w8.gemm_raw(a.data_ptr(), 260, w.data_ptr(), s.data_ptr(), c.data_ptr(),
                       64, 4, 64, 256) == w8.ERR_A_STRIDE_ALIGN
    torch.cuda.synchronize()
    assert torch.equal(before, c)


# ------------------------------------------------------------ batched tier

def run_gpu_batched(w8, probs, stream=None):
    """Run every problem in one w8a16_gemm_batched call; returns each whole C
    buffer (BF16 bits, pads and extra rows included)."""
    keep, descs = [], []
    for p in probs:
        a, w, s, c = dev_u16(p.a), dev(p.w), dev(p.scale), dev_u16(p.c)
        keep.append((a, w, s, c))
        descs.append(dict(a=a.data_ptr(), w_fp8=w.data_ptr(), block_scale=s.data_ptr(),
                          c=c.data_ptr(), a_row_stride=p.a_row_stride,
                          c_row_stride=p.c_row_stride, m=p.m, n=p.n, k=p.k))
    st = w8.gemm_batched_raw(descs, 0 if stream is None else stream.cuda_stream)
    assert st == 0, w8.last_error()
    torch.cuda.synchronize()
    return [t[3].cpu().numpy().view(np.uint16).reshape(p.c.shape) for t, p in zip(keep, probs)]


BATCHES = [
    # (m, n, k, a_row_stride, c_row_stride) per arm
    [(8, 640, 1024, 1040, 700), (8, 128, 1024, 1024, 136), (8, 130, 1024, 1032, 130)],
    [(1, 300, 256, 264, 301)],
    [(24, 256, 384, None, None), (3, 520, 512, 520, 530), (17, 64, 128, None, 70),
     (40, 200, 640, 648, 200)],
    [(64, 96, 256, None, None)] * 8,
]


@pytest.mark.parametrize("arms", BATCHES)
def test_batched_exact_data_bit_exact(w8, arms):
    """Each arm of a batched call equals the oracle bit for bit on exact data
    and leaves its pads and extra rows untouched."""
    probs = [exact_problem(m, n, k, seed=50 + i, a_row_stride=ars, c_row_stride=crs,
                           c_extra_rows=2)
             for i, (m, n, k, ars, crs) in enumerate(arms)]
    outs = run_gpu_batched(w8, probs)
    for p, g in zip(probs, outs):
        check_full(p, g, exact=True)


def test_batched_equals_single_calls_with_the_same_variant(w8):
    """The batched grid runs the single-GEMM kernel body: each arm is bitwise
    the single call with the batched plan's variant (random data)."""
    arms = [(16, 1000, 2048), (16, 256, 2048), (5, 384, 1024)]
    probs = [datagen.make_problem(m, n, k, seed=90 + i, c_extra_rows=1)
             for i, (m, n, k) in enumerate(arms)]
    bp = w8.plan_batched(arms)
    outs = run_gpu_batched(w8, probs)
    for p, g in zip(probs, outs):
        single = w8.make_plan(p.m, p.n, p.k, w8.KERNEL_STREAM, bp.m_blocks, bp.n_blocks, 1,
                              bp.depth, 0, bp.waves)
        assert np.array_equal(g, run_gpu(w8, p, single))
        check_full(p, g)


def test_batched_qkv_at_size_sampled(w8):
    """Decode-size Q/K/V arms (8 rows, hidden 4096, K and V with 1024
    columns), sampled parity."""
    probs = [datagen.make_problem(8, n, 4096, seed=7 + n, c_extra_rows=1)
             for n in (4096, 1024, 1024)]
    outs = run_gpu_batched(w8, probs, stream=torch.cuda.Stream())
    for p, g in zip(probs, outs):
        rows, cols = datagen.sample_indices(p.m, p.n, 400, seed=3)
        oc, _, bound = oracle.gemm_at(p.a, p.w, p.scale, p.m, p.n, p.k, rows, cols,
                                      a_row_stride=p.a_row_stride)
        assert oracle.within_tolerance(g[rows, cols], oc, bound).all()
        assert (g[p.m:, :] == p.c[p.m:, :]).all()


def test_batched_torch_wrapper(w8):
    p1 = datagen.make_problem(4, 256, 512, seed=1)
    p2 = datagen.make_problem(4, 128, 512, seed=2)
    ts = []
    for p in (p1, p2):
        a = dev_u16(p.a).view(torch.bfloat16)[:, :p.k]
        w = dev(p.w)
        s = dev(p.scale)
        c = torch.empty((p.m, p.n), dtype=torch.bfloat16, device="cuda")
        ts.append((a, w, s, c))
    outs = w8.gemm_batched(ts)
    torch.cuda.synchronize()
    for p, c in zip((p1, p2), outs):
        g = c.view(torch.int16).cpu().numpy().view(np.uint16)
        oc, _, bound = oracle.gemm(p.a, p.w, p.scale, p.m, p.n, p.k,
                                   a_row_stride=p.a_row_stride)
        assert oracle.within_tolerance(g, oc, bound).all()


# ------------------------------------------------- FP8 activations, W8A8

def run_act_quant(w8, a_bits, m, k, a_row_stride, q_row_stride):
    a = dev_u16(a_bits)
    q = torch.full((m, q_row_stride), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((m, k // 128), -1.0, dtype=torch.float32, device="cuda")
    st = w8.act_quant_fp8_raw(a.data_ptr(), a_row_stride, q.data_ptr(), q_row_stride,
                              s.data_ptr(), m, k)
    assert st == 0, w8.last_error()
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("m,k,a_pad,q_pad", [(1, 128, 0, 0), (5, 384, 8, 16), (33, 4096, 0, 0),
                                             (300, 1024, 24, 32), (2, 128 * 200, 0, 0)])
def test_act_quant_bit_exact(w8, m, k, a_pad, q_pad):
    """Codes and scales equal the oracle's bit for bit (both divide in
    binary32); code pads are untouched."""
    p = datagen.make_problem(m, 1, k, seed=m + k, a_row_stride=k + a_pad)
    if m >= 3:
        p.a[1, :128] = 0                          # zero group
        p.a[2, 128 * (k // 256):128 * (k // 256) + 128] = 0x8000   # -0 group
        tiny = np.float32(np.linspace(-1e-30, 1e-30, 128))
        p.a[0, :128] = datagen.to_bf16_bits(tiny)
    q, s = run_act_quant(w8, p.a, m, k, k + a_pad, k + q_pad)
    oq, os_ = oracle.act_quant(p.a, m, k, a_row_stride=k + a_pad, q_row_stride=k + q_pad)
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))
    bad = np.argwhere(q[:, :k] != oq[:, :k])
    assert bad.size == 0, (bad[:5].tolist(), q[tuple(bad[:5].T)], oq[tuple(bad[:5].T)])
    assert (q[:, k:] == 0xAB).all()


def test_act_quant_rounding_ties_and_subnormals(w8):
    """With the group maximum 448 the scale is exactly 1 and the codes are
    the E4M3 rounding of the inputs themselves: every midpoint between two
    adjacent E4M3 values (ties to even), and values around the subnormal
    range, against the oracle's encoder."""
    pos = [oracle.e4m3_value(c) for c in range(0x7F)]
    mids = [(x + y) / 2 for x, y in zip(pos, pos[1:])]
    extra = [2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 2.0 ** -9 * 7.5, 2.0 ** -6 * 0.96875]
    vals = np.array([448.0] + mids + [-v for v in mids] + extra + [-v for v in extra],
                    dtype=np.float32)
    k = 128 * (-(-vals.size // 127))
    rows = []
    for g in range(k // 128):
        chunk = vals[127 * g:127 * (g + 1)]
        row = np.zeros(128, np.float32)
        row[0] = 448.0
        row[1:1 + chunk.size] = chunk
        rows.append(row)
    x = np.concatenate(rows)[None, :]
    bits = datagen.to_bf16_bits(x)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), x)   # exact in BF16
    q, s = run_act_quant(w8, bits, 1, k, k, k)
    oq, os_ = oracle.act_quant(bits, 1, k)
    assert (s == 1.0).all() and (os_ == 1.0).all()
    assert np.array_equal(q[:, :k], oq)


def exact_w8a8_problem(m, n, k, seed, qa_pad=0, c_row_stride=None):
    """W8A8 operands whose products and FP32 sums are exact: activation
    values in {0, +-1/8, ..., +-1}, weight codes below 0x38 (|w| < 1,
    subnormals included), scales in {1, 2}, K <= 512."""
    assert k <= 512
    rng = np.random.default_rng(seed)
    act_vals = np.array([j / 8.0 for j in range(-8, 9)], np.float32)
    qa = np.zeros((m, k + qa_pad), np.uint8)
    qa[:, :k] = np.vectorize(oracle.e4m3_rne)(rng.choice(act_vals, size=(m, k)))
    mag = rng.integers(0, 0x38, size=(n, k), dtype=np.uint8)
    w = mag | (rng.integers(0, 2, size=(n, k), dtype=np.uint8) << 7)
    sa = rng.choice(np.float32([1.0, 2.0]), size=(m, k // 128))
    sw = rng.choice(np.float32([1.0, 2.0]), size=((n + 127) // 128, k // 128))
    return qa, sa, w, sw


def run_w8a8(w8, qa, sa, w, sw, m, n, k, qa_row_stride, c_row_stride, c_rows, plan=None):
    dq, dsa, dw, dsw = dev(qa), dev(sa), dev(w), dev(sw)
    c = torch.full((c_rows, c_row_stride), 0x7777, dtype=torch.int16, device="cuda")
    st = w8.gemm_w8a8_raw(dq.data_ptr(), qa_row_stride, dsa.data_ptr(), dw.data_ptr(),
                          dsw.data_ptr(), c.data_ptr(), c_row_stride, m, n, k, 0, plan)
    assert st == 0, w8.last_error()
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)


W8A8_VARIANTS = [(1, 1, 4), (1, 1, 8), (1, 1, 16), (1, 2, 8), (1, 2, 16), (1, 3, 8), (1, 4, 4),
                 (1, 4, 8), (2, 1, 8), (2, 1, 16), (2, 2, 8), (2, 4, 4), (2, 4, 8),
                 (4, 1, 4), (4, 1, 8), (4, 2, 4), (4, 2, 8)]


@pytest.mark.parametrize("mb,nb,waves", W8A8_VARIANTS)
@pytest.mark.parametrize("m", [3, 40])
def test_w8a8_exact_data_every_variant(w8, mb, nb, waves, m):
    n, k = 16 * nb * 2 + 5, 384
    qa, sa, w, sw = exact_w8a8_problem(m, n, k, seed=mb * 100 + nb * 10 + waves + m, qa_pad=16)
    plan = w8.make_plan(m, n, k, w8.KERNEL_W8A8, mb, nb, 1, waves=waves)
    c = run_w8a8(w8, qa, sa, w, sw, m, n, k, k + 16, n + 3, m + 1, plan)
    oc, _, _ = oracle.gemm_w8a8(qa, sa, w, sw, m, n, k, qa_row_stride=k + 16)
    bad = np.argwhere(c[:m, :n] != oc)
    assert bad.size == 0, (bad[:5].tolist(), c[tuple(bad[:5].T)], oc[tuple(bad[:5].T)])
    assert (c[:m, n:] == 0x7777).all() and (c[m:, :] == 0x7777).all()


@pytest.mark.parametrize("m,n,k", [(1, 256, 256), (8, 4096, 4096), (16, 12288, 5120),
                                   (32, 6144, 2048), (100, 700, 1280), (48, 4096, 4096),
                                   (40, 6144, 2048), (24, 4096, 4096)])
def test_w8a8_default_plan_within_tolerance(w8, m, n, k):
    """Random codes and log-uniform scales, default plan, sampled against
    the oracle with the W8A16 tolerance form."""
    rng = np.random.default_rng(m + n)
    qa = rng.choice(np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8),
                    size=(m, k))
    w = datagen.make_problem(1, n, k, seed=n + k).w
    sa = np.exp2(rng.uniform(-10, 2, size=(m, k // 128))).astype(np.float32)
    sw = np.exp2(rng.uniform(-12, -4, size=((n + 127) // 128, k // 128))).astype(np.float32)
    c = run_w8a8(w8, qa, sa, w, sw, m, n, k, k, n, m)
    rows, cols = datagen.sample_indices(m, n, 2000, seed=9)
    oc, _, bound = oracle.gemm_w8a8_at(qa, sa, w, sw, m, n, k, rows, cols)
    assert oracle.within_tolerance(c[rows, cols], oc, bound).all()


def test_w8a8_weight_above_4_gib_sampled(w8):
    """The W8A8 GEMM over a weight of more than 4 GiB (default plan): codes
    as in the W8A16 case, random finite FP8 activations and scales; sampled
    outputs, including rows past 2^32 bytes, against the oracle."""
    m, n, k = 16, 34816, 131072
    rng = np.random.default_rng(4343)
    w = _big_weight(n, k)
    qa = (rng.integers(0, 0x7F, size=(m, k), dtype=np.uint8) |
          (rng.integers(0, 2, size=(m, k), dtype=np.uint8) << 7))
    sa = rng.uniform(0.01, 0.1, size=(m, k // 128)).astype(np.float32)
    sw = rng.uniform(0.5, 2.0, size=(-(-n // 128), k // 128)).astype(np.float32)
    print("W8A8 weight above 4 GiB: plan=%s" % w8.plan_w8a8(m, n, k).as_dict(), flush=True)
    c = run_w8a8(w8, qa, sa, w, sw, m, n, k, k, n, m + 1)
    torch.cuda.empty_cache()
    rows, cols = _big_samples(m, n, k)
    oc, _, bound = oracle.gemm_w8a8_at(qa, sa, w, sw, m, n, k, rows, cols)
    assert oracle.within_tolerance(c[rows, cols], oc, bound).all()
    assert (c[m, :] == 0x7777).all()


def test_graph_replays_quantizer_w8a8_and_batched(w8):
    """The FP8 quantizer, the W8A8 GEMM it feeds and a batched call,
    captured in one HIP graph, replayed three times with eager work and
    synchronisations between the replays: every replay equals the eager
    results bit for bit (outputs cleared before each replay)."""
    m, n, k = 16, 2048, 1024
    p = datagen.make_problem(m, n, k, seed=77)
    a, ww, sw = dev_u16(p.a), dev(p.w), dev(p.scale)
    q = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sa = torch.empty((m, k // 128), dtype=torch.float32, device="cuda")
    c8 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    arms = [datagen.make_problem(8, nn, 512, seed=78 + nn) for nn in (512, 256)]
    abufs = [(dev_u16(x.a), dev(x.w), dev(x.scale), dev_u16(x.c)) for x in arms]
    descs = [dict(a=t[0].data_ptr(), w_fp8=t[1].data_ptr(), block_scale=t[2].data_ptr(),
                  c=t[3].data_ptr(), a_row_stride=x.a_row_stride, c_row_stride=x.c_row_stride,
                  m=x.m, n=x.n, k=x.k) for x, t in zip(arms, abufs)]
    stream = torch.cuda.Stream()

    def work():
        assert w8.act_quant_fp8_raw(a.data_ptr(), k, q.data_ptr(), k, sa.data_ptr(), m, k,
                                    stream.cuda_stream) == 0, w8.last_error()
        assert w8.gemm_w8a8_raw(q.data_ptr(), k, sa.data_ptr(), ww.data_ptr(), sw.data_ptr(),
                                c8.data_ptr(), n, m, n, k, stream.cuda_stream) == 0, \
            w8.last_error()
        assert w8.gemm_batched_raw(descs, stream.cuda_stream) == 0, w8.last_error()

    def outputs():
        return [t.clone() for t in (q, sa, c8)] + [t[3].clone() for t in abufs]

    with torch.cuda.stream(stream):
        work()
        torch.cuda.synchronize()
        eager = outputs()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            work()
        for rep in range(3):
            for t in [q, sa, c8] + [t[3] for t in abufs]:
                t.zero_()
            work()                              # eager work between replays
            torch.cuda.synchronize()
            for t in [q, sa, c8] + [t[3] for t in abufs]:
                t.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for want, got in zip(eager, outputs()):
                assert torch.equal(want, got), "replay %d differs from eager" % rep
    oq, os_ = oracle.act_quant(p.a, m, k)
    assert np.array_equal(eager[0].cpu().numpy(), oq)


def test_quantize_then_w8a8_pipeline(w8):
    """BF16 activations -> GPU quantizer -> GPU W8A8 GEMM, against the
    oracle's quantizer and W8A8 GEMM: identical codes and scales, outputs
    within tolerance."""
    m, n, k = 24, 3000, 2048
    p = datagen.make_problem(m, n, k, seed=41)
    a = dev_u16(p.a)
    q = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    s = torch.empty((m, k // 128), dtype=torch.float32, device="cuda")
    assert w8.act_quant_fp8_raw(a.data_ptr(), k, q.data_ptr(), k, s.data_ptr(), m, k) == 0
    ww, sw = dev(p.w), dev(p.scale)
    c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    w8.gemm_w8a8(q, s, ww, sw, c)
    torch.cuda.synchronize()
    oq, os_ = oracle.act_quant(p.a, m, k)
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)
    oc, _, bound = oracle.gemm_w8a8(oq, os_, p.w, p.scale, m, n, k)
    g = c.view(torch.int16).cpu().numpy().view(np.uint16)
    assert oracle.within_tolerance(g, oc, bound).all()
    # and the torch wrappers agree with the raw entry points
    q2, s2 = w8.act_quant_fp8(dev_u16(p.a).view(torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(q2, q) and torch.equal(s2, s)
