"""Pins for the CPU oracle (CPU only).

The oracle is checked against things other than itself:
  * library witnesses: torch's float8_e4m3fn decode and its float32->bfloat16
    rounding (independent code);
  * the OCP FP8 specification's anchor values (tests/golden/e4m3_anchors.txt);
  * exact rational arithmetic (fractions.Fraction) on tiny GEMMs, rounded to
    BF16 by a brute-force nearest search over every finite BF16 value;
  * invariants of the block-scaled GEMM (zero weights, block-scale doubling,
    sign symmetry, row independence, permutations of whole K blocks, a
    permutation-matrix weight, one scaled dot product).
"""

import bisect
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

FINITE_CODES = [c for c in range(256) if c not in (0x7F, 0xFF)]


def torch_e4m3(codes):
    t = torch.tensor(list(codes), dtype=torch.uint8).view(torch.float8_e4m3fn)
    return t.float().double().tolist()


def torch_bf16_bits(x32):
    t = torch.from_numpy(np.asarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------- E4M3

def test_e4m3_matches_torch_on_all_finite_codes():
    ref = torch_e4m3(FINITE_CODES)
    got = [oracle.e4m3_value(c) for c in FINITE_CODES]
    for c, r, g in zip(FINITE_CODES, ref, got):
        assert math.copysign(1.0, r) == math.copysign(1.0, g), hex(c)
        assert r == g, (hex(c), r, g)


def test_e4m3_nan_codes():
    assert math.isnan(oracle.e4m3_value(0x7F))
    assert math.isnan(oracle.e4m3_value(0xFF))


def test_e4m3_spec_anchors():
    # tests/golden/e4m3_anchors.txt: code -> value pairs taken from the OCP
    # 8-bit floating point specification (OFP8), E4M3 column.
    path = os.path.join(GOLDEN, "e4m3_anchors.txt")
    n = 0
    with open(path) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            code, value = line.split()
            got = oracle.e4m3_value(int(code, 16))
            assert got == float(Fraction(value)), (code, value, got)
            n += 1
    assert n >= 10


def test_e4m3_order_and_symmetry():
    pos = [oracle.e4m3_value(c) for c in range(0x00, 0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:])), "codes 0..0x7E increase"
    for c in range(0x00, 0x7F):
        assert oracle.e4m3_value(c | 0x80) == -oracle.e4m3_value(c)
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0
    # 126 distinct positive values plus zero; every one is a BF16 value.
    assert len(set(pos)) == 127
    for v in pos:
        assert oracle.bf16_value(oracle.bf16_rne(v)) == v


# --------------------------------------------------------------------- BF16

def test_bf16_value_is_top_half_of_float32():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, 4000, dtype=np.uint32).astype(np.uint16)
    for b in bits[:500]:
        f = np.array([np.uint32(b) << np.uint32(16)], np.uint32).view(np.float32)[0]
        v = oracle.bf16_value(int(b))
        if np.isnan(f):
            assert math.isnan(v)
        else:
            assert v == float(f)


def test_bf16_rne_matches_torch_on_float_inputs():
    rng = np.random.default_rng(6)
    xs = np.concatenate([
        rng.standard_normal(3000).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        (rng.standard_normal(1000) * 1e-38).astype(np.float32),   # subnormals
        (rng.standard_normal(500) * 1e-44).astype(np.float32),
        # exact BF16 midpoints (ties) in several binades
        (np.arange(1, 500, dtype=np.float32) * 2.0 + 1.0) * np.float32(2.0 ** -9),
        np.float32([3.3895314e38, -3.3895314e38, 3.4e38, 1.17549435e-38]),
    ]).astype(np.float32)
    ref = torch_bf16_bits(xs)
    got = np.array([oracle.bf16_rne(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(ref, got)


def test_bf16_rne_constructed_cases():
    assert oracle.bf16_rne(1 + 2 ** -8) == 0x3F80          # tie -> even (down)
    assert oracle.bf16_rne(1 + 3 * 2 ** -8) == 0x3F82      # tie -> even (up)
    # the double-rounding trap: via float this would become 1.0
    assert oracle.bf16_rne(1 + 2 ** -8 + 2 ** -40) == 0x3F81
    assert oracle.bf16_rne(-(1 + 2 ** -8 + 2 ** -40)) == 0xBF81
    assert oracle.bf16_rne(0.0) == 0x0000
    assert oracle.bf16_rne(-0.0) == 0x8000
    assert oracle.bf16_rne(2.0 ** -133) == 0x0001          # smallest subnormal
    assert oracle.bf16_rne(2.0 ** -134) == 0x0000          # tie to even zero
    assert oracle.bf16_rne(3 * 2.0 ** -134) == 0x0002
    maxf = (2 - 2 ** -7) * 2.0 ** 127
    assert oracle.bf16_rne(maxf) == 0x7F7F
    assert oracle.bf16_rne((2 - 2 ** -8) * 2.0 ** 127) == 0x7F80  # midpoint -> inf
    assert oracle.bf16_rne(-(2 - 2 ** -8 - 2 ** -30) * 2.0 ** 127) == 0xFF7F
    assert oracle.bf16_rne(float("inf")) == 0x7F80
    assert oracle.bf16_rne(float("nan")) & 0x7FC0 == 0x7FC0


# ------------------------------------------------- brute force with rationals

_BF16_POS = None


def _bf16_positive_table():
    """Every finite positive BF16 value, as (Fraction, bits), ascending."""
    global _BF16_POS
    if _BF16_POS is None:
        bits = np.arange(1, 0x7F80, dtype=np.uint32)
        vals = (bits << 16).astype(np.uint32).view(np.float32)
        _BF16_POS = ([Fraction(float(v)) for v in vals], bits.tolist())
    return _BF16_POS


def brute_bf16_rne(x: Fraction) -> int:
    """Nearest BF16 to an exact rational, ties to the even bit pattern,
    found by search over the sorted list of all finite BF16 values."""
    if x == 0:
        return 0
    vals, bits = _bf16_positive_table()
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    maxv = vals[-1]
    half_ulp_max = Fraction(2) ** 119          # half the spacing at the top
    if a >= maxv + half_ulp_max:
        return sign | 0x7F80
    i = bisect.bisect_left(vals, a)
    cands = []
    if i < len(vals):
        cands.append((vals[i], bits[i]))
    if i > 0:
        cands.append((vals[i - 1], bits[i - 1]))
    else:
        cands.append((Fraction(0), 0))
    best = min(cands, key=lambda vb: (abs(vb[0] - a), vb[1] & 1))
    return sign | best[1]


def _rand_codes(rng, shape):
    return rng.choice(np.array(FINITE_CODES, dtype=np.uint8), size=shape)


def _exact_gemm(a_bits, a_stride, w_codes, scale, m, n, k):
    """Exact rational C (list of lists) and the bound; written from the
    definition with torch as the E4M3 decoder."""
    wv = np.array(torch_e4m3(w_codes.reshape(-1).tolist())).reshape(n, k)
    av = (a_bits.reshape(-1).astype(np.uint32) << 16).view(np.float32)
    kb = k // 128
    out = []
    for i in range(m):
        row = []
        for j in range(n):
            tot = Fraction(0)
            for b in range(kb):
                p = Fraction(0)
                for t in range(128):
                    kk = 128 * b + t
                    p += Fraction(float(av[i * a_stride + kk])) * Fraction(float(wv[j, kk]))
                tot += Fraction(float(scale[j // 128, b])) * p
            row.append(tot)
        out.append(row)
    return out


@pytest.mark.parametrize("m,n,k,a_pad", [(1, 1, 128, 0), (2, 5, 256, 8),
                                          (3, 130, 128, 16), (1, 129, 256, 0)])
def test_gemm_equals_exact_rational_then_rne(m, n, k, a_pad):
    rng = np.random.default_rng(100 + m * 1000 + n + k)
    a_stride = k + a_pad
    a = np.full((m, a_stride), datagen.A_PAD_BITS, dtype=np.uint16)
    af = rng.standard_normal((m, k)).astype(np.float32)
    af[:, ::17] *= np.float32(2.0 ** -60)        # tiny activations
    af[:, 5::31] *= np.float32(2.0 ** 40)        # huge activations
    a[:, :k] = torch_bf16_bits(af)
    w = _rand_codes(rng, (n, k))
    nb = (n + 127) // 128
    scale = np.exp2(rng.uniform(-20, 5, size=(nb, k // 128))).astype(np.float32)
    scale[0, 0] = np.float32(0.75)               # not a power of two
    c, tot, bound = oracle.gemm(a, w, scale, m, n, k, a_row_stride=a_stride)
    exact = _exact_gemm(a, a_stride, w, scale, m, n, k)
    skipped = 0
    for i in range(m):
        for j in range(n):
            x = exact[i][j]
            # the double total differs from the exact one by rounding only
            assert abs(Fraction(tot[i, j]) - x) <= Fraction(bound[i, j]) * Fraction(2) ** -48
            want = brute_bf16_rne(x)
            if want != c[i, j]:
                # only acceptable when the exact value sits on a rounding
                # boundary closer than the double total can resolve
                lo = Fraction(oracle.bf16_value(int(want)))
                hi = Fraction(oracle.bf16_value(int(c[i, j])))
                mid = (lo + hi) / 2
                assert abs(x - mid) <= Fraction(bound[i, j]) * Fraction(2) ** -48, (i, j)
                skipped += 1
    assert skipped <= 1


def test_c_pitch_and_pad_untouched():
    p = datagen.make_problem(3, 130, 256, seed=7, a_row_stride=264,
                             c_row_stride=141, c_extra_rows=0)
    init = np.full((3, 141), 0xFFFF, dtype=np.uint16)
    c, _, _ = oracle.gemm(p.a, p.w, p.scale, 3, 130, 256, a_row_stride=264,
                          c_row_stride=141, c_init=init)
    assert (c[:, 130:] == 0xFFFF).all()
    c2, _, _ = oracle.gemm(np.ascontiguousarray(p.a[:, :256]), p.w, p.scale,
                           3, 130, 256)
    assert np.array_equal(c[:, :130], c2)


def test_gemm_at_matches_full():
    p = datagen.make_problem(4, 300, 384, seed=8)
    c, tot, bound = oracle.gemm(p.a, p.w, p.scale, 4, 300, 384)
    rows, cols = datagen.sample_indices(4, 300, 50, seed=1)
    cs, ts, bs = oracle.gemm_at(p.a, p.w, p.scale, 4, 300, 384, rows, cols)
    assert np.array_equal(cs, c[rows, cols])
    assert np.array_equal(ts, tot[rows, cols])
    assert np.array_equal(bs, bound[rows, cols])


def test_rejects_invalid_shapes():
    a = np.zeros(256, np.uint16)
    w = np.zeros(256, np.uint8)
    s = np.zeros(2, np.float32)
    with pytest.raises(ValueError):
        oracle.gemm(a, w, s, 1, 1, 200)


# --------------------------------------------------------------- invariants

def _prob(m=3, n=256, k=512, seed=11):
    return datagen.make_problem(m, n, k, seed)


def test_zero_weights_give_zero():
    p = _prob()
    c, tot, _ = oracle.gemm(p.a, np.zeros_like(p.w), p.scale, p.m, p.n, p.k)
    assert (tot == 0).all()
    assert ((c == 0) | (c == 0x8000)).all()


def test_doubling_one_block_scale_adds_that_block():
    p = _prob()
    _, tot0, bnd = oracle.gemm(p.a, p.w, p.scale, p.m, p.n, p.k)
    nb, kb = 1, 2
    s2 = p.scale.copy()
    s2[nb, kb] *= 2
    _, tot1, _ = oracle.gemm(p.a, p.w, s2, p.m, p.n, p.k)
    # the block's own contribution, from a separate call with only that block
    w_only = np.zeros_like(p.w)
    w_only[128 * nb:128 * (nb + 1), 128 * kb:128 * (kb + 1)] = \
        p.w[128 * nb:128 * (nb + 1), 128 * kb:128 * (kb + 1)]
    _, tblk, _ = oracle.gemm(p.a, w_only, p.scale, p.m, p.n, p.k)
    diff = tot1 - tot0
    assert np.all(np.abs(diff - tblk) <= bnd * 2.0 ** -48)
    others = np.ones(p.n, bool)
    others[128 * nb:128 * (nb + 1)] = False
    assert np.array_equal(tot1[:, others], tot0[:, others])


def test_negating_a_negates_c():
    p = _prob()
    c0, _, _ = oracle.gemm(p.a, p.w, p.scale, p.m, p.n, p.k)
    c1, _, _ = oracle.gemm(p.a ^ np.uint16(0x8000), p.w, p.scale, p.m, p.n, p.k)
    assert np.array_equal(c1, c0 ^ np.uint16(0x8000))


def test_rows_are_independent():
    p = _prob(m=4)
    c0, _, _ = oracle.gemm(p.a, p.w, p.scale, 4, p.n, p.k)
    for i in range(4):
        ci, _, _ = oracle.gemm(np.ascontiguousarray(p.a[i]), p.w, p.scale, 1, p.n, p.k)
        assert np.array_equal(ci[0], c0[i])


def test_permuting_k_blocks_with_scales():
    p = _prob(k=512)
    perm = [2, 0, 3, 1]
    cols = np.concatenate([np.arange(128 * b, 128 * (b + 1)) for b in perm])
    a2 = np.ascontiguousarray(p.a[:, cols])
    w2 = np.ascontiguousarray(p.w[:, cols])
    s2 = np.ascontiguousarray(p.scale[:, perm])
    _, t0, bnd = oracle.gemm(p.a, p.w, p.scale, p.m, p.n, p.k)
    _, t1, _ = oracle.gemm(a2, w2, s2, p.m, p.n, p.k)
    assert np.all(np.abs(t1 - t0) <= bnd * 2.0 ** -48)


def test_permutation_matrix_weight_selects_columns():
    m, n, k = 5, 256, 256
    rng = np.random.default_rng(12)
    pi = rng.permutation(k)
    w = np.zeros((n, k), np.uint8)
    w[np.arange(n), pi] = 0x38                    # E4M3 1.0
    scale = np.ones((2, 2), np.float32)
    a = torch_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    c, _, _ = oracle.gemm(a, w, scale, m, n, k)
    assert np.array_equal(c, a[:, pi])


def test_single_block_is_scaled_dot_product():
    rng = np.random.default_rng(13)
    a = torch_bf16_bits(rng.standard_normal((1, 128)).astype(np.float32))
    w = _rand_codes(rng, (1, 128))
    s = np.array([[0.3]], np.float32)
    _, tot, _ = oracle.gemm(a, w, s, 1, 1, 128)
    av = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[0]
    wv = np.array(torch_e4m3(w[0].tolist()))
    ref = float(np.float32(0.3)) * float(np.dot(av, wv))
    assert abs(tot[0, 0] - ref) <= 2.0 ** -45 * float(np.abs(av * wv).sum())


def test_golden_regression_small_workload():
    """Stored output of the smallest workload, written by
    tests/golden/make_golden.py from the oracle alone; guards against
    unintended changes to the oracle's arithmetic."""
    path = os.path.join(GOLDEN, "m1_n256_k256.c_bits.txt")
    want = np.loadtxt(path, dtype=np.int64).astype(np.uint16)
    p = datagen.make_workload(datagen.workload("m1_n256_k256"))
    c, _, _ = oracle.gemm(p.a, p.w, p.scale, p.m, p.n, p.k)
    assert np.array_equal(c.reshape(-1), want.reshape(-1))


# ----------------------------------------------- FP8 activation quantizer

def _e4m3_positive_values():
    """(value, code) of every finite non-negative E4M3FN code, ascending,
    decoded by torch (independent of the oracle)."""
    codes = list(range(0, 0x7F))
    return list(zip(torch_e4m3(codes), codes))


def brute_e4m3_rne(x: float) -> int:
    """Nearest E4M3FN code to x by search over all finite values, ties to the
    even code, saturating at 448, sign kept (also for zero)."""
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = Fraction(abs(float(x)))
    best = None
    for v, c in _e4m3_positive_values():
        d = abs(Fraction(v) - a)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return sign | best[1]


def test_e4m3_rne_round_trips_every_finite_code():
    for c in FINITE_CODES:
        v = oracle.e4m3_value(c)
        assert oracle.e4m3_rne(v) == c, hex(c)


def test_e4m3_rne_ties_go_to_the_even_code():
    vals = _e4m3_positive_values()
    for (v0, c0), (v1, c1) in zip(vals, vals[1:]):
        mid = (v0 + v1) / 2                       # exact in binary32
        want = c0 if c0 % 2 == 0 else c1
        assert oracle.e4m3_rne(mid) == want, (v0, v1)
        assert oracle.e4m3_rne(-mid) == 0x80 | want


def test_e4m3_rne_matches_brute_force_and_torch():
    rng = np.random.default_rng(5)
    xs = np.concatenate([
        rng.uniform(-448, 448, 3000),
        np.exp2(rng.uniform(-12, 9, 3000)) * rng.choice([-1.0, 1.0], 3000),
    ]).astype(np.float32)
    xs = np.clip(xs, -448, 448)
    t = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, tc in zip(xs[:800], t[:800]):
        assert oracle.e4m3_rne(x) == brute_e4m3_rne(float(x)), float(x)
    got = np.array([oracle.e4m3_rne(x) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, t)


def test_e4m3_rne_saturates_and_flushes():
    assert oracle.e4m3_rne(448.0) == 0x7E
    assert oracle.e4m3_rne(463.9) == 0x7E
    assert oracle.e4m3_rne(1e30) == 0x7E and oracle.e4m3_rne(-1e30) == 0xFE
    assert oracle.e4m3_rne(2.0 ** -10) == 0x00           # tie at half the least subnormal
    assert oracle.e4m3_rne(2.0 ** -10 * 1.0001) == 0x01
    assert oracle.e4m3_rne(-(2.0 ** -11)) == 0x80        # rounds to zero, keeps the sign
    assert oracle.e4m3_rne(-0.0) == 0x80 and oracle.e4m3_rne(0.0) == 0x00


def _act(m, k, seed, pitch=None):
    rng = np.random.default_rng(seed)
    pitch = k if pitch is None else pitch
    a = np.full((m, pitch), datagen.A_PAD_BITS, dtype=np.uint16)
    a[:, :k] = torch_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    return a


def test_act_quant_codes_are_torch_e4m3_of_x_over_s():
    """Each code is the E4M3 cast (torch) of x / s in binary32, the group
    maximum lands on +-448, and s is the largest |x| over 448."""
    m, k = 3, 512
    a = _act(m, k, 1, pitch=520)
    q, s = oracle.act_quant(a, m, k, a_row_stride=520, q_row_stride=528)
    x = (a[:, :k].astype(np.uint32) << 16).view(np.float32)
    for i in range(m):
        for g in range(k // 128):
            xs = x[i, 128 * g:128 * g + 128]
            assert s[i, g] > 0
            y = np.clip(xs / s[i, g], -448, 448).astype(np.float32)
            want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[i, 128 * g:128 * g + 128], want)
            j = int(np.argmax(np.abs(xs)))
            assert q[i, 128 * g + j] in (0x7E, 0xFE)
            assert abs(float(s[i, g]) * 448 - float(np.abs(xs).max())) <= \
                float(np.abs(xs).max()) * 2.0 ** -23
    assert (q[:, k:] == 0).all()


def test_act_quant_dequantization_error_bound():
    """|e4m3(q) * s - x| <= 2^-4 |x| (normal range) + 2^-10 s (subnormal
    half-spacing): three fraction bits, round to nearest."""
    m, k = 4, 1024
    a = _act(m, k, 2)
    a[1, :128] = torch_bf16_bits(np.float32(np.linspace(-1e-3, 1e-3, 128)))  # small group
    q, s = oracle.act_quant(a, m, k)
    x = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dec = np.array(torch_e4m3(q.reshape(-1).tolist())).reshape(m, k)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(dec * srep - x)
    assert (err <= np.abs(x) * 2.0 ** -4 + srep * 2.0 ** -10 + 1e-300).all()


def test_act_quant_zero_group_and_power_of_two_scaling():
    m, k = 2, 384
    a = _act(m, k, 3)
    a[0, 128:256] = 0
    a[1, 256:384] = 0x8000                       # -0.0
    q, s = oracle.act_quant(a, m, k)
    assert s[0, 1] == 0 and (q[0, 128:256] == 0).all()
    assert s[1, 2] == 0 and (q[1, 256:384] == 0).all()
    # scaling a group by 2^e scales s by 2^e and keeps every code
    x = (a.astype(np.uint32) << 16).view(np.float32)
    a4 = torch_bf16_bits(x * np.float32(4.0))
    q4, s4 = oracle.act_quant(a4, m, k)
    assert np.array_equal(q4, q) and np.array_equal(s4, s * np.float32(4.0))


# --------------------------------------------------------------- W8A8 GEMM

def _exact_w8a8(qa, sa, w, sw, m, n, k):
    av = np.array(torch_e4m3(qa.reshape(-1).tolist())).reshape(m, k)
    wv = np.array(torch_e4m3(w.reshape(-1).tolist())).reshape(n, k)
    out = []
    for i in range(m):
        row = []
        for j in range(n):
            tot = Fraction(0)
            for b in range(k // 128):
                p = sum(Fraction(av[i, kk]) * Fraction(wv[j, kk])
                        for kk in range(128 * b, 128 * b + 128))
                tot += Fraction(float(sa[i, b])) * Fraction(float(sw[j // 128, b])) * p
            row.append(tot)
        out.append(row)
    return out


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (2, 5, 256), (3, 130, 128)])
def test_w8a8_equals_exact_rational_then_rne(m, n, k):
    rng = np.random.default_rng(m * 7 + n + k)
    qa = _rand_codes(rng, (m, k))
    w = _rand_codes(rng, (n, k))
    sa = np.exp2(rng.uniform(-10, 3, size=(m, k // 128))).astype(np.float32)
    sw = np.exp2(rng.uniform(-12, -4, size=((n + 127) // 128, k // 128))).astype(np.float32)
    sa[0, 0] = np.float32(0.3)
    c, tot, bound = oracle.gemm_w8a8(qa, sa, w, sw, m, n, k)
    exact = _exact_w8a8(qa, sa, w, sw, m, n, k)
    for i in range(m):
        for j in range(n):
            x = exact[i][j]
            assert abs(Fraction(tot[i, j]) - x) <= Fraction(bound[i, j]) * Fraction(2) ** -48
            assert brute_bf16_rne(x) == c[i, j] or \
                abs(x - (Fraction(oracle.bf16_value(int(c[i, j]))) +
                         Fraction(oracle.bf16_value(brute_bf16_rne(x)))) / 2) <= \
                Fraction(bound[i, j]) * Fraction(2) ** -48


def test_w8a8_with_unit_a_scales_is_the_w8a16_gemm_of_the_decoded_codes():
    """Every E4M3 value is a BF16 value: with all A scales 1 the W8A8 GEMM
    of codes qa equals the (separately pinned) W8A16 GEMM of their BF16
    decodings, bit for bit."""
    m, n, k = 3, 260, 512
    rng = np.random.default_rng(9)
    qa = _rand_codes(rng, (m, k))
    w = _rand_codes(rng, (n, k))
    sw = np.exp2(rng.uniform(-12, -4, size=((n + 127) // 128, k // 128))).astype(np.float32)
    a_bits = torch_bf16_bits(np.array(torch_e4m3(qa.reshape(-1).tolist()),
                                      dtype=np.float32)).reshape(m, k)
    c8, tot8, b8 = oracle.gemm_w8a8(qa, np.ones((m, k // 128), np.float32), w, sw, m, n, k)
    c16, tot16, b16 = oracle.gemm(a_bits, w, sw, m, n, k)
    assert np.array_equal(c8, c16) and np.array_equal(tot8, tot16)
    rows = np.array([0, 2, 1]); cols = np.array([0, 259, 128])
    ca, ta, _ = oracle.gemm_w8a8_at(qa, np.ones((m, k // 128), np.float32), w, sw, m, n, k,
                                    rows, cols)
    assert np.array_equal(ca, c8[rows, cols])


def test_w8a8_pipeline_close_to_w8a16():
    """Quantize-then-W8A8 stays within the quantization error of the W8A16
    result: |C8 - C16| <= 2^-4 * B (three fraction bits per activation)."""
    m, n, k = 2, 128, 512
    a = _act(m, k, 4)
    rng = np.random.default_rng(4)
    w = _rand_codes(rng, (n, k))
    sw = np.full((1, k // 128), 2.0 ** -6, np.float32)
    q, s = oracle.act_quant(a, m, k)
    _, t8, _ = oracle.gemm_w8a8(q, s, w, sw, m, n, k)
    _, t16, b16 = oracle.gemm(a, w, sw, m, n, k)
    assert (np.abs(t8 - t16) <= b16 * 2.0 ** -4 + 1e-30).all()


# ------------------------------------------------------ the parity tolerance
#
# The bar every non-exact GPU test is graded with:
#     |gpu - oracle| <= 2^-8 * B + ulp_bf16(oracle),   no NaN / Inf from the GPU,
# with ulp(v) the BF16 spacing at v (2^(max(floor(log2|v|), -126) - 7)) and
# ulp(0) = 2^-133.  The helpers are pinned against torch's BF16 decoding and
# against hand-built values at the edge of the bar.

def _torch_bf16_to_f64(bits):
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).double().numpy()


ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_bf16_bits_to_f64_equals_torch_and_scalar_decode_on_all_patterns():
    got = oracle.bf16_bits_to_f64(ALL_BF16)
    ref = _torch_bf16_to_f64(ALL_BF16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    for b in range(0, 1 << 16, 257):
        v = oracle.bf16_value(b)
        assert (math.isnan(v) and math.isnan(got[b])) or v == got[b]


def test_bf16_ulp_is_the_gap_to_the_next_bf16_value():
    # every finite positive pattern except the largest: the gap to the next
    # pattern (torch decode) is the ulp of the value, for both signs
    pos = np.arange(0, 0x7F7F, dtype=np.uint32).astype(np.uint16)
    v = _torch_bf16_to_f64(pos)
    gap = _torch_bf16_to_f64(pos + 1) - v
    assert np.array_equal(oracle.bf16_ulp(v), gap)
    assert np.array_equal(oracle.bf16_ulp(-v), gap)
    # the largest finite value: the gap below it (same binade)
    top = _torch_bf16_to_f64(np.uint16([0x7F7F, 0x7F7E]))
    assert oracle.bf16_ulp(top[0]) == top[0] - top[1] == 2.0 ** 120


def test_bf16_ulp_anchors():
    assert oracle.bf16_ulp(0.0) == 2.0 ** -133
    assert oracle.bf16_ulp(-0.0) == 2.0 ** -133
    assert oracle.bf16_ulp(2.0 ** -133) == 2.0 ** -133          # smallest subnormal
    assert oracle.bf16_ulp(2.0 ** -127) == 2.0 ** -133          # subnormal
    assert oracle.bf16_ulp(2.0 ** -126) == 2.0 ** -133          # smallest normal
    assert oracle.bf16_ulp(1.0) == 2.0 ** -7
    assert oracle.bf16_ulp(-1.0) == 2.0 ** -7
    assert oracle.bf16_ulp(1.9921875) == 2.0 ** -7               # top of [1, 2)
    assert oracle.bf16_ulp(2.0) == 2.0 ** -6
    assert oracle.bf16_ulp(448.0) == 2.0 ** 1


def _bits(x):
    """BF16 bits of a float that is exactly a BF16 value."""
    b = oracle.bf16_rne(x)
    assert oracle.bf16_value(b) == x
    return b


def _passes(gpu, orc, bound):
    return bool(oracle.within_tolerance(np.uint16([gpu]), np.uint16([orc]),
                                        np.float64([bound]))[0])


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_within_tolerance_at_the_edge_of_the_bar(sign):
    one = _bits(sign * 1.0)
    # B = 6: 2^-8 B = 3 * 2^-7, plus ulp(1) = 2^-7 -> lim = 2^-5 exactly
    assert _passes(_bits(sign * (1 + 2 ** -5)), one, 6.0)
    assert not _passes(_bits(sign * (1 + 2 ** -5 + 2 ** -7)), one, 6.0)
    assert _passes(_bits(sign * (1 - 2 ** -5)), one, 6.0)
    assert not _passes(_bits(sign * (1 - 2 ** -5 - 2 ** -8)), one, 6.0)
    # 2^-8, not 2^-7: B = 2 gives lim = 2^-7 + 2^-7; one more ulp fails
    assert _passes(_bits(sign * (1 + 2 ** -6)), one, 2.0)
    assert not _passes(_bits(sign * (1 + 2 ** -6 + 2 ** -7)), one, 2.0)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_within_tolerance_takes_the_ulp_of_the_oracle_value(sign):
    two = _bits(sign * 2.0)
    # ulp(2) = 2^-6; ulp of the GPU value 2 - 2^-6 would be 2^-7
    assert _passes(_bits(sign * (2 - 2 ** -6)), two, 0.0)
    assert not _passes(_bits(sign * (2 - 2 ** -6 - 2 ** -7)), two, 0.0)
    # and an oracle value just below the binade: ulp 2^-7, not 2^-6
    below = _bits(sign * (2 - 2 ** -7))
    assert _passes(_bits(sign * 2.0), below, 0.0)
    assert not _passes(_bits(sign * (2 + 2 ** -6)), below, 0.0)


def test_within_tolerance_at_zero_and_subnormals():
    assert _passes(0x0001, 0x0000, 0.0)                  # 2^-133 off zero
    assert _passes(0x8001, 0x0000, 0.0)
    assert not _passes(0x0002, 0x0000, 0.0)
    assert _passes(0x8000, 0x0000, 0.0)                  # -0 vs +0
    assert _passes(0x0003, 0x0002, 0.0)
    assert not _passes(0x0004, 0x0002, 0.0)


def test_within_tolerance_rejects_nan_and_inf():
    one = _bits(1.0)
    for bad in (0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80):
        assert not _passes(bad, one, 1e30)
    # an infinite oracle value is never produced by finite data; a GPU
    # infinity against it still fails
    assert not _passes(0x7F80, 0x7F80, 0.0)


def test_within_tolerance_is_elementwise():
    g = np.uint16([_bits(1.0), _bits(1.5), 0x7FC0, _bits(-3.0)])
    o = np.uint16([_bits(1.0), _bits(1.0), _bits(1.0), _bits(-3.0 - 2 ** -6)])
    b = np.float64([0.0, 1e3, 1e3, 0.0])
    assert oracle.within_tolerance(g, o, b).tolist() == [True, True, False, True]


# ------------------------------------------------------------- W4A4 MX GEMV
#
# Reading of page "w4a4_proj/mx_plan.rs": OCP MXFP4 (E2M1 elements, two per
# byte with the even element in the low nibble, one E8M0 scale per 32 K
# elements).  Pins: the format table (tests/golden/e2m1_anchors.txt), torch's
# float8_e8m0fnu decode, exact rationals rounded by brute force, invariants.

def _e2m1_golden():
    out = {}
    for line in open(os.path.join(GOLDEN, "e2m1_anchors.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        out[int(code, 16)] = float(val)
    return out


def test_e2m1_decode_equals_the_format_table():
    table = _e2m1_golden()
    assert sorted(table) == list(range(16))
    for code, val in table.items():
        got = oracle.e2m1_value(code)
        assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), code
    # only the low 4 bits are read
    assert oracle.e2m1_value(0xF2) == 1.0


def test_e8m0_decode_equals_torch_on_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().tolist()
    for e in range(256):
        got = oracle.e8m0_value(e)
        if e == 255:
            assert math.isnan(got) and math.isnan(ref[e])
        else:
            assert got == ref[e] == math.ldexp(1.0, e - 127), e


def _mx_rand(rng, m, n, k, a_pitch=None):
    a_pitch = k if a_pitch is None else a_pitch
    a = rng.integers(0, 256, size=(m, a_pitch // 2), dtype=np.uint8)
    w = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    asc = rng.integers(118, 136, size=(m, k // 32), dtype=np.uint8)
    wsc = rng.integers(118, 136, size=(n, k // 32), dtype=np.uint8)
    return a, asc, w, wsc


def _exact_w4a4(a, asc, w, wsc, m, n, k):
    vals = [Fraction(v) for v in _e2m1_golden_list()]
    out = np.empty((m, n), dtype=object)
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for b in range(k // 32):
                s = Fraction(2) ** (int(asc[i, b]) - 127) * Fraction(2) ** (int(wsc[j, b]) - 127)
                p = Fraction(0)
                for t in range(32 * b, 32 * b + 32):
                    ai = (int(a[i, t // 2]) >> (4 * (t % 2))) & 15
                    wj = (int(w[j, t // 2]) >> (4 * (t % 2))) & 15
                    p += vals[ai] * vals[wj]
                tot += s * p
            out[i, j] = tot
    return out


def _e2m1_golden_list():
    t = _e2m1_golden()
    return [t[c] for c in range(16)]


@pytest.mark.parametrize("m,n,k,pad", [(1, 1, 32, 0), (2, 5, 64, 32), (3, 17, 128, 64),
                                       (1, 3, 256, 0)])
def test_w4a4_gemm_equals_exact_rational_then_rne(m, n, k, pad):
    rng = np.random.default_rng(700 + m + n + k)
    a, asc, w, wsc = _mx_rand(rng, m, n, k, k + pad)
    c, tot, bound = oracle.gemm_w4a4(a, asc, w, wsc, m, n, k, a_row_stride=k + pad)
    exact = _exact_w4a4(a, asc, w, wsc, m, n, k)
    for i in range(m):
        for j in range(n):
            assert int(c[i, j]) == brute_bf16_rne(exact[i, j]), (i, j)
            assert tot[i, j] == float(exact[i, j])


def test_w4a4_gemm_at_equals_exact_rational_then_rne():
    """The sampled W4A4 entry: selected outputs (repeats and any order)
    against brute force with exact rationals, and every index checked
    before any read."""
    rng = np.random.default_rng(733)
    m, n, k, pad = 3, 7, 128, 64
    a, asc, w, wsc = _mx_rand(rng, m, n, k, k + pad)
    exact = _exact_w4a4(a, asc, w, wsc, m, n, k)
    rows = np.array([2, 0, 1, 2, 2, 0], np.uint32)
    cols = np.array([6, 0, 3, 6, 1, 5], np.uint32)
    c, tot, bound = oracle.gemm_w4a4_at(a, asc, w, wsc, m, n, k, rows, cols,
                                        a_row_stride=k + pad)
    for s_, (i, j) in enumerate(zip(rows, cols)):
        assert int(c[s_]) == brute_bf16_rne(exact[i, j]), (i, j)
        assert tot[s_] == float(exact[i, j])
    _, _, full_bound = oracle.gemm_w4a4(a, asc, w, wsc, m, n, k, a_row_stride=k + pad)
    assert np.array_equal(bound, full_bound[rows, cols])
    for bad_r, bad_c in [(m, 0), (0, n)]:
        with pytest.raises(ValueError):
            oracle.gemm_w4a4_at(a, asc, w, wsc, m, n, k, np.array([bad_r], np.uint32),
                                np.array([bad_c], np.uint32), a_row_stride=k + pad)


def test_w4a4_pad_is_not_read():
    rng = np.random.default_rng(11)
    a, asc, w, wsc = _mx_rand(rng, 2, 4, 128, 192)
    c1, t1, _ = oracle.gemm_w4a4(a, asc, w, wsc, 2, 4, 128, a_row_stride=192)
    a[:, 64:] ^= 0xFF
    c2, t2, _ = oracle.gemm_w4a4(a, asc, w, wsc, 2, 4, 128, a_row_stride=192)
    assert np.array_equal(c1, c2) and np.array_equal(t1, t2)


def test_w4a4_even_element_is_the_low_nibble():
    k = 128
    a = np.zeros((1, k // 2), np.uint8)
    w = np.zeros((1, k // 2), np.uint8)
    asc = np.full((1, k // 32), 127, np.uint8)
    wsc = np.full((1, k // 32), 127, np.uint8)
    a[0, 0] = 0x02                       # element 0 = 1.0, element 1 = 0
    w[0, 0] = 0x20                       # element 0 = 0, element 1 = 1.0
    _, tot, _ = oracle.gemm_w4a4(a, asc, w, wsc, 1, 1, k)
    assert tot[0, 0] == 0.0
    w[0, 0] = 0x07                       # element 0 = 6.0
    _, tot, _ = oracle.gemm_w4a4(a, asc, w, wsc, 1, 1, k)
    assert tot[0, 0] == 6.0
    a[0, 1] = 0x50                       # element 3 = 3.0; w element 3 = 0
    _, tot, _ = oracle.gemm_w4a4(a, asc, w, wsc, 1, 1, k)
    assert tot[0, 0] == 6.0


def test_w4a4_invariants():
    rng = np.random.default_rng(12)
    m, n, k = 3, 6, 256
    a, asc, w, wsc = _mx_rand(rng, m, n, k)
    c, tot, bound = oracle.gemm_w4a4(a, asc, w, wsc, m, n, k)
    # zero weights
    _, t0, b0 = oracle.gemm_w4a4(a, asc, np.zeros_like(w), wsc, m, n, k)
    assert (t0 == 0).all() and (b0 == 0).all()
    # negating every activation (sign bit of each nibble) negates the result
    cn, tn, _ = oracle.gemm_w4a4(a ^ 0x88, asc, w, wsc, m, n, k)
    assert np.array_equal(tn, -tot)
    nz = tot != 0
    assert np.array_equal(cn[nz] ^ 0x8000, c[nz])
    # one block alone, then its weight scale exponent + 1: exactly twice
    wb = np.zeros_like(w)
    wb[:, 32:48] = w[:, 32:48]           # K block 2 (elements 64..95)
    _, t1, _ = oracle.gemm_w4a4(a, asc, wb, wsc, m, n, k)
    wsc2 = wsc.copy()
    wsc2[:, 2] += 1
    _, t2, _ = oracle.gemm_w4a4(a, asc, wb, wsc2, m, n, k)
    assert np.array_equal(t2, 2 * t1)
    # raising another block's scale does not change it
    wsc3 = wsc.copy()
    wsc3[:, 5] += 3
    _, t3, _ = oracle.gemm_w4a4(a, asc, wb, wsc3, m, n, k)
    assert np.array_equal(t3, t1)
    # permuting whole 32-element blocks of A and W together with their
    # scales leaves the total unchanged (up to the order of the block sums)
    perm = rng.permutation(k // 32)
    ap = a.reshape(m, k // 32, 16)[:, perm].reshape(m, k // 2)
    wp = w.reshape(n, k // 32, 16)[:, perm].reshape(n, k // 2)
    _, tp, _ = oracle.gemm_w4a4(ap, asc[:, perm], wp, wsc[:, perm], m, n, k)
    assert (np.abs(tp - tot) <= bound * 2.0 ** -50).all()
    # rows are independent
    _, tr, _ = oracle.gemm_w4a4(a[1:2], asc[1:2], w, wsc, 1, n, k)
    assert np.array_equal(tr[0], tot[1])
