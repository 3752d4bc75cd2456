"""C ABI checks that need no GPU: the library loads, exports every symbol
include/w8a16.h declares, rejects bad arguments in the documented order
before touching the GPU, and plans that cover the problem exactly."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import block_scaled_fp8_w8a16_amd as w8
from block_scaled_fp8_w8a16_amd import Plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a16.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a16_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = w8.library()
    declared = _declared_functions()
    assert set(declared) == set(w8.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", w8.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(w8a16_\w+)", out))
    for name in declared:
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings():
    for code in range(0, 9):
        assert w8.status_string(code)
    assert w8.status_string(1234) == "unknown status"


@pytest.mark.parametrize("args,want", [
    ((0, 16, 128, 128, 16), w8.ERR_M_ZERO),
    ((0, 0, 100, 0, 0), w8.ERR_M_ZERO),            # m first
    ((1, 16, 0, 128, 16), w8.ERR_K_NOT_MULT_128),
    ((1, 16, 100, 128, 16), w8.ERR_K_NOT_MULT_128),
    ((1, 16, 100, 4, 0), w8.ERR_K_NOT_MULT_128),   # k before pitches
    ((1, 16, 256, 128, 16), w8.ERR_PITCH_TOO_SHORT),
    ((1, 16, 256, 256, 15), w8.ERR_PITCH_TOO_SHORT),
    ((1, 16, 256, 260, 15), w8.ERR_PITCH_TOO_SHORT),  # pitches before alignment
    ((1, 16, 256, 260, 16), w8.ERR_A_STRIDE_ALIGN),
    ((1, 0, 256, 260, 0), w8.ERR_A_STRIDE_ALIGN),  # alignment before n == 0
    ((1, 0, 256, 256, 0), w8.ERR_N_ZERO),
    ((1, 16, 256, 264, 17), w8.OK),
    ((32, 6144, 2048, 2560, 8192), w8.OK),
])
def test_check_args_order(args, want):
    assert w8.check_args(*args) == want


def test_gemm_rejects_before_any_gpu_call():
    # Argument errors return before HIP is touched, so they work on a host
    # without a GPU; the message follows the page's wording.
    st = w8.gemm_raw(0, 128, 0, 0, 0, 16, 0, 16, 128)
    assert st == w8.ERR_M_ZERO
    assert "m=0 has no rows" in w8.last_error()
    st = w8.gemm_raw(0, 128, 0, 0, 0, 16, 1, 16, 130)
    assert st == w8.ERR_K_NOT_MULT_128
    assert "K=130 must be a positive multiple of 128" in w8.last_error()
    st = w8.gemm_raw(0, 100, 0, 0, 0, 16, 1, 16, 128)
    assert st == w8.ERR_PITCH_TOO_SHORT
    st = w8.gemm_raw(0, 132, 0, 0, 0, 16, 1, 16, 128)
    assert st == w8.ERR_A_STRIDE_ALIGN
    st = w8.gemm_raw(0, 128, 0, 0, 0, 16, 1, 16, 128)
    assert st == w8.ERR_NULL_PTR
    p = w8.plan(1, 16, 128)
    st = w8.gemm_raw(0, 128, 0, 0, 0, 16, 1, 16, 128, plan_=p)
    assert st == w8.ERR_NULL_PTR


def _covers(p: Plan, m, n, k):
    """Every (m block, n block, K step) is owned by exactly one workgroup."""
    ksteps = k // 128
    assert p.splits * p.steps_per_split >= ksteps
    assert (p.splits - 1) * p.steps_per_split < ksteps
    assert p.m_tiles * 16 * p.m_blocks >= m > (p.m_tiles - 1) * 16 * p.m_blocks
    assert p.n_tiles * 16 * p.n_blocks >= n > (p.n_tiles - 1) * 16 * p.n_blocks
    assert p.grid == p.m_tiles * p.n_tiles * p.splits
    owned = {}
    for s in range(p.splits):
        for t in range(s * p.steps_per_split, min(ksteps, (s + 1) * p.steps_per_split)):
            owned[t] = owned.get(t, 0) + 1
    assert sorted(owned) == list(range(ksteps))
    assert set(owned.values()) == {1}


@pytest.mark.parametrize("m,n,k", [(1, 256, 256), (8, 4096, 4096), (16, 12288, 5120),
                                   (32, 6144, 2048), (128, 8192, 8192), (1, 1, 128),
                                   (40, 1000, 384), (64, 17, 128 * 37),
                                   (65, 300, 1024), (3, 70000, 128)])
def test_default_plans_cover_the_problem(m, n, k):
    p = w8.plan(m, n, k)
    _covers(p, m, n, k)
    assert p.block in (256, 384, 512, 640, 1024)
    assert p.lds_bytes <= 160 * 1024
    if p.splits > 1 and p.kernel == w8.KERNEL_TILE:
        # whole FP32 tiles per split; no arrival counters (second kernel)
        assert p.workspace_bytes == (p.splits * p.m_tiles * 16 * p.m_blocks * p.n_tiles *
                                     16 * p.n_blocks * 4)
        assert p.counter_count == 0
    elif p.splits > 1:
        assert p.workspace_bytes == p.grid * p.m_blocks * p.n_blocks * 1024
        assert p.counter_count == p.m_tiles * p.n_tiles * 64
    else:
        assert p.workspace_bytes == 0


def test_small_m_plans_fill_the_chip():
    # weights under 48 MiB stream; 8..32 rows over a larger weight take the
    # ring kernel, unless 48-column stream tiles fill the CUs better
    p = w8.plan(16, 12288, 5120)
    assert (p.kernel, p.n_blocks, p.grid) == (w8.KERNEL_STREAM, 3, 256)
    for m, n, k, kern in [(8, 4096, 4096, w8.KERNEL_STREAM), (16, 12288, 5120, w8.KERNEL_STREAM),
                          (32, 6144, 2048, w8.KERNEL_STREAM), (4, 14336, 4096, w8.KERNEL_STREAM),
                          (16, 16384, 5120, w8.KERNEL_RING), (32, 8192, 8192, w8.KERNEL_RING)]:
        p = w8.plan(m, n, k)
        assert p.kernel == kern, (m, n, k)
        # 17..32 rows stream as two 16-row tiles when that asks each CU for
        # fewer bytes (32 x 6144 x 2048: 16 x 48 tiles); the ring keeps one
        assert p.m_blocks == (1 if m <= 16 or kern == w8.KERNEL_STREAM else 2)
        assert p.grid >= 192          # at least three quarters of the 256 CUs
        assert p.splits == 1
        if kern == w8.KERNEL_RING:
            assert p.stage_steps == 4 and p.depth in (2, 3)
            assert p.flags == (w8.FLAG_A8 if m <= 8 else 0)
            assert p.lds_bytes <= 160 * 1024 - 256
        else:
            assert p.stage_steps == 0


def test_ring_plans():
    p = w8.make_plan(16, 12288, 5120, w8.KERNEL_RING, 1, 4, 1, depth=3, waves=16, stage_steps=4)
    _covers(p, 16, 12288, 5120)
    stage = 4 * (64 * 128 + 16 * 256)
    assert p.lds_bytes == 3 * stage + (40 + 63) // 64 * 256
    assert p.block == 1024 and p.flags == 0 and p.workspace_bytes == 0
    # the 8-row A staging is derived from m
    p = w8.make_plan(5, 300, 1024, w8.KERNEL_RING, 1, 1, 1, depth=4, waves=16, stage_steps=8,
                     flags=0)
    assert p.flags == w8.FLAG_A8
    bad = [dict(splits=2),                                   # no K split
           dict(stage_steps=6),                              # 4 or 8 steps per stage
           dict(depth=5),                                    # 2..4 stages
           dict(waves=4),                                    # 8 or 16 waves
           dict(n_blocks=4, stage_steps=8, depth=4)]         # ring exceeds LDS
    for b in bad:
        args = dict(m_blocks=1, n_blocks=1, splits=1, depth=3, waves=16, stage_steps=4)
        args.update(b)
        with pytest.raises(w8.W8A16Error) as e:
            w8.make_plan(16, 4096, 4096, w8.KERNEL_RING, args["m_blocks"], args["n_blocks"],
                         args["splits"], depth=args["depth"], waves=args["waves"],
                         stage_steps=args["stage_steps"])
        assert e.value.status == w8.ERR_BAD_PLAN, b
    # K/128 must not exceed the threads (one scale per thread)
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(16, 256, 128 * 513, w8.KERNEL_RING, 1, 1, 1, depth=3, waves=8,
                     stage_steps=4)


def test_large_m_plans_tile_kernel():
    p = w8.plan(128, 8192, 8192)
    assert p.kernel == w8.KERNEL_TILE
    # one 128-row tile x 64 128-column tiles x 4 splits of 16 K steps: one
    # workgroup per CU, the weight read once
    assert (p.m_blocks, p.n_blocks, p.splits, p.steps_per_split) == (8, 8, 4, 16)
    assert (p.depth, p.a_depth, p.waves) == (3, 3, 8)
    assert (p.m_tiles, p.grid, p.counter_count) == (1, 256, 0)
    assert p.workspace_bytes == 4 * 128 * 8192 * 4
    assert p.lds_bytes == p.a_depth * 128 * 256 + p.depth * 128 * 128 + 256
    assert p.lds_bytes <= 160 * 1024 - 256
    assert (w8.plan(65, 8192, 8192).m_blocks, w8.plan(96, 8192, 8192).m_blocks) == (8, 8)
    # splits of 8 K steps keep two 64-row tiles
    for n, k in ((8192, 4096), (4096, 8192)):
        p = w8.plan(128, n, k)
        assert (p.kernel, p.m_blocks, p.n_blocks, p.m_tiles) == (w8.KERNEL_TILE, 4, 8, 2), (n, k)
        assert p.grid == 256 and p.lds_bytes == p.a_depth * 64 * 256 + p.depth * 128 * 128 + 256
    p3 = w8.make_plan(128, 8192, 8192, w8.KERNEL_TILE, 8, 8, 4, depth=3, a_depth=3,
                      waves=4)
    assert p3.lds_bytes == 3 * 128 * 256 + 3 * 128 * 128 + 256
    # a split may not exceed 64 K steps (one scale per lane)
    p = w8.plan(200, 256, 128 * 200)
    assert p.kernel == w8.KERNEL_TILE and p.steps_per_split <= 64
    _covers(p, 200, 256, 128 * 200)
    # up to 128 rows over a weight of at most 16 MiB stream when one round
    # of stream tiles covers C; two rounds go to the tile kernel
    p = w8.plan(100, 256, 128 * 200)
    assert p.kernel == w8.KERNEL_STREAM and p.m_tiles * p.n_tiles <= 256
    assert (w8.plan(128, 4096, 4096).kernel, w8.plan(128, 6144, 2048).kernel,
            w8.plan(129, 4096, 4096).kernel) == (w8.KERNEL_STREAM, w8.KERNEL_TILE,
                                                 w8.KERNEL_TILE)
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(100, 256, 128 * 200, w8.KERNEL_TILE, 8, 8, 1, depth=3, waves=4)
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(128, 256, 1024, w8.KERNEL_TILE, 8, 8, 1, depth=6, waves=4)
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(128, 256, 1024, w8.KERNEL_TILE, 8, 4, 1, depth=5, waves=4)
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(128, 256, 1024, w8.KERNEL_TILE, 2, 8, 1, depth=3, waves=4)
    with pytest.raises(w8.W8A16Error):      # 64-row tiles: weight buffers 4 or 6
        w8.make_plan(128, 256, 1024, w8.KERNEL_TILE, 4, 8, 1, depth=3, waves=4)
    with pytest.raises(w8.W8A16Error):      # a producer wave's vmcnt holds 4 x 16 loads at most
        w8.make_plan(128, 256, 1024, w8.KERNEL_TILE, 4, 8, 1, depth=6, waves=6)
    with pytest.raises(w8.W8A16Error):      # three A buffers leave room for 3 weight buffers
        w8.make_plan(128, 256, 1024, w8.KERNEL_TILE, 8, 8, 1, depth=4, a_depth=3,
                     waves=4)
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(128, 256, 1024, w8.KERNEL_TILE, 8, 8, 1, depth=3, flags=w8.FLAG_A8,
                     waves=4)


def test_64_row_tiles():
    p = w8.make_plan(128, 8192, 8192, w8.KERNEL_TILE, 4, 8, 2, depth=6, a_depth=3,
                     waves=8)
    assert (p.m_tiles, p.n_tiles, p.grid, p.steps_per_split) == (2, 64, 256, 32)
    assert p.lds_bytes == 3 * 64 * 256 + 6 * 128 * 128 + 256
    assert p.workspace_bytes == 2 * 128 * 8192 * 4
    p = w8.make_plan(40, 1000, 1024, w8.KERNEL_TILE, 4, 4, 1, depth=8, waves=10)
    assert (p.m_tiles, p.n_tiles, p.block) == (1, 16, 640)
    assert p.lds_bytes == 2 * 64 * 256 + 8 * 64 * 128 + 256
    _covers(p, 40, 1000, 1024)


def test_tile_plans_fill_the_cus_with_long_splits():
    # 128-column tiles would need 4 splits of 12 K steps; 64-column tiles
    # fill the chip with 2 splits of 24 steps
    p = w8.plan(96, 4096, 6144)
    assert (p.kernel, p.m_blocks, p.n_blocks, p.splits, p.steps_per_split, p.grid) == \
        (w8.KERNEL_TILE, 4, 4, 2, 24, 256)
    _covers(p, 96, 4096, 6144)
    # 128-column tiles with 16-step splits
    p = w8.plan(48, 8192, 8192)
    assert (p.kernel, p.m_blocks, p.n_blocks, p.splits, p.grid) == (w8.KERNEL_TILE, 4, 8, 4, 256)
    # above 128 rows, 128-row tiles
    p = w8.plan(256, 4096, 4096)
    assert (p.m_blocks, p.m_tiles, p.n_blocks, p.splits, p.grid) == (8, 2, 4, 2, 256)
    # 33..64 rows over a weight of at most 16 MiB stream
    assert w8.plan(48, 4096, 4096).kernel == w8.KERNEL_STREAM
    assert w8.plan(64, 6144, 2048).kernel == w8.KERNEL_STREAM
    assert w8.plan(33, 8192, 4096).kernel == w8.KERNEL_TILE


@pytest.mark.parametrize("m,n,k,mb,nb", [
    (32, 6144, 2048, 1, 3),     # 256 tiles of 16 x 48: 80 units per CU vs 96 for 32 x 32
    (24, 4096, 4096, 1, 2),     # 256 tiles of 16 x 32: 64 vs 80 for 32 x 16
    (17, 2048, 2048, 1, 1),     # 256 tiles of 16 x 16
    (16, 6144, 2048, 1, 2),     # 16 rows: unchanged
    (48, 4096, 4096, 2, 2),     # two 32 x 32 row tiles: 96 vs 144 for 64 x 16
    (64, 4096, 4096, 2, 2),
    (40, 6144, 2048, 2, 4),     # two 32 x 64 row tiles: 128 vs 160 for 64 x 32
    (48, 2048, 4096, 1, 2),     # three 16 x 32 row tiles: 64 vs 144
])
def test_stream_tile_cost_model_17_to_64_rows(m, n, k, mb, nb):
    p = w8.plan(m, n, k)
    _covers(p, m, n, k)
    assert (p.kernel, p.m_blocks, p.n_blocks) == (w8.KERNEL_STREAM, mb, nb)
    assert p.m_tiles == -(-m // (16 * mb))
    if (mb, nb) == (2, 4):
        assert p.waves == 8


STREAM_TILES = [(1, 1), (1, 2), (1, 3), (1, 4), (1, 8), (2, 1), (2, 2), (2, 4), (4, 1), (4, 2)]


def _stream_cost(m, n, mb, nb, cus=256):
    """Bytes per 128 of K one CU requests: the tile's BF16 A rows plus FP8
    weight rows, times its rounds of tiles."""
    tiles = -(-m // (16 * mb)) * -(-((n + 15) // 16) // nb)
    return -(-tiles // cus) * (32 * mb + 16 * nb)


def test_stream_tile_minimises_bytes_per_cu():
    """Property of the planner over a sweep of shapes: above 16 rows, a
    stream plan's tile costs no more than any built stream tile (32 x 128
    left out), by the bytes-per-CU model."""
    rng = np.random.default_rng(17)
    checked = 0
    for _ in range(400):
        m = int(rng.integers(17, 129))
        n = int(rng.integers(1, 12289))
        k = 128 * int(rng.integers(1, 41))
        p = w8.plan(m, n, k)
        if p.kernel != w8.KERNEL_STREAM:
            continue
        best = min(_stream_cost(m, n, mb, nb) for mb, nb in STREAM_TILES)
        assert _stream_cost(m, n, p.m_blocks, p.n_blocks) == best, (m, n, k, p.as_dict())
        checked += 1
    assert checked > 200


def test_split_k_only_when_tiles_leave_cus_idle():
    p = w8.plan(1, 128, 65536)
    assert p.splits > 1 and p.grid <= 256
    _covers(p, 1, 128, 65536)
    # default splits are grouped per XCD: 8 equal ranges of whole tiles
    assert p.flags & w8.FLAG_XCD_LOCAL
    assert p.grid % 8 == 0 and (p.grid // 8) % p.splits == 0
    # tiles that fill the CUs are not split
    p = w8.plan(8, 4096, 4096)
    assert p.splits == 1 and p.flags == 0


@pytest.mark.parametrize("m,n,k,splits,waves", [
    (1, 1024, 8192, 4, 8),      # 64 tiles x 4 splits of 16 steps
    (16, 1024, 8192, 4, 8),
    (4, 2048, 14336, 2, 16),    # 128 tiles x 2 splits of 56 steps
    (8, 512, 8192, 8, 8),       # 32 tiles x 8 splits of 8 steps
    (8, 512, 4096, 4, 8),       # 32 tiles x 4 splits of 8 steps
    (16, 1536, 5120, 2, 8),     # 96 tiles x 2 splits of 20 steps
    (32, 768, 2048, 2, 8),      # 48 tiles x 2 splits of 8 steps
    (1, 100, 8192, 1, 16),      # 7 tiles: no split keeps XCD ranges whole
])
def test_split_rule_narrow_n(m, n, k, splits, waves):
    p = w8.plan(m, n, k)
    _covers(p, m, n, k)
    assert (p.kernel, p.splits, p.waves) == (w8.KERNEL_STREAM, splits, waves)
    assert bool(p.flags & w8.FLAG_XCD_LOCAL) == (splits > 1)
    assert p.steps_per_split >= 8 or splits == 1


def test_xcd_local_plans_need_whole_tiles_per_xcd():
    # 48 tiles x 2 splits: 12 ids per XCD, 6 whole tiles each
    p = w8.make_plan(32, 768, 2048, w8.KERNEL_STREAM, 2, 1, 2, depth=1,
                     flags=w8.FLAG_XCD_LOCAL, waves=8)
    assert p.grid == 96 and p.flags == w8.FLAG_XCD_LOCAL
    bad = [(32, 768, 2048, 2, 1, 1),      # no split
           (8, 100, 4096, 1, 1, 2),       # 7 tiles x 2 = 14: not a multiple of 8
           (8, 192, 4096, 1, 1, 4)]       # 12 tiles x 4 = 48: 6 ids per XCD, 1.5 tiles
    for m, n, k, mb, nb, sp in bad:
        with pytest.raises(w8.W8A16Error) as e:
            w8.make_plan(m, n, k, w8.KERNEL_STREAM, mb, nb, sp, depth=1,
                         flags=w8.FLAG_XCD_LOCAL, waves=8)
        assert e.value.status == w8.ERR_BAD_PLAN and "XCD" in str(e.value)
    # without the flag any split count is a valid stream plan (the splits of
    # a tile may then run on several XCDs)
    for m, n, k, mb, nb, sp in bad[1:]:
        p = w8.make_plan(m, n, k, w8.KERNEL_STREAM, mb, nb, sp, depth=1, waves=8)
        assert p.splits == sp and p.flags == 0
    # an unknown flag bit is rejected
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(32, 768, 2048, w8.KERNEL_STREAM, 2, 1, 2, depth=1,
                     flags=w8.FLAG_XCD_LOCAL | 8, waves=8)
    # other kernels take no XCD grouping flag
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(128, 8192, 8192, w8.KERNEL_TILE, 4, 8, 2, depth=4,
                     flags=w8.FLAG_XCD_LOCAL, waves=8)


def test_wide_tile_plans():
    # 128 x 256 tiles: 32 column tiles x 8 splits of 8 steps at 128 x 8192 x 8192
    p = w8.make_plan(128, 8192, 8192, w8.KERNEL_TILE, 8, 16, 8, depth=3, a_depth=3)
    assert (p.grid, p.block, p.lds_bytes, p.waves) == (256, 256, 147968, 4)
    assert (p.m_tiles, p.n_tiles, p.steps_per_split) == (1, 32, 8)
    assert p.workspace_bytes == 8 * 128 * 8192 * 4
    # ragged: 200 rows, 1031 columns -> 2 x 5 tiles
    p = w8.make_plan(200, 1031, 1024, w8.KERNEL_TILE, 8, 16, 3, depth=0, a_depth=0, waves=0)
    assert (p.m_tiles, p.n_tiles, p.splits, p.depth, p.a_depth, p.waves) == (2, 5, 3, 3, 3, 4)
    assert p.workspace_bytes == 3 * 256 * 1280 * 4
    for depth, a_depth, waves, flags in [(4, 3, 4, 0), (3, 2, 4, 0), (3, 3, 8, 0), (3, 3, 4, 1)]:
        with pytest.raises(w8.W8A16Error) as e:
            w8.make_plan(128, 8192, 8192, w8.KERNEL_TILE, 8, 16, 8, depth=depth,
                         a_depth=a_depth, waves=waves, flags=flags)
        assert e.value.status == w8.ERR_BAD_PLAN
    # at most 64 K steps per split
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(128, 8192, 8192 * 2, w8.KERNEL_TILE, 8, 16, 1, depth=3, a_depth=3)


def test_explicit_plans():
    p = w8.make_plan(16, 4096, 4096, w8.KERNEL_STREAM, 1, 4, 8)
    _covers(p, 16, 4096, 4096)
    assert p.splits == 8 and p.steps_per_split == 4
    p = w8.make_plan(16, 4096, 128 * 33, w8.KERNEL_STREAM, 1, 2, 5)
    _covers(p, 16, 4096, 128 * 33)
    assert (p.splits, p.steps_per_split) == (5, 7)
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(16, 4096, 4096, w8.KERNEL_STREAM, 1, 4, 1, depth=3)
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(16, 4096, 4096, w8.KERNEL_STREAM, 1, 4, 1, flags=2)
    p = w8.make_plan(16, 4096, 4096, w8.KERNEL_STREAM, 1, 4, 1, depth=4, flags=w8.FLAG_DIRECT)
    assert (p.depth, p.flags) == (4, w8.FLAG_DIRECT)
    with pytest.raises(w8.W8A16Error) as e:
        w8.make_plan(16, 4096, 4096, w8.KERNEL_STREAM, 3, 4, 1)
    assert e.value.status == w8.ERR_BAD_PLAN
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(16, 4096, 4096, w8.KERNEL_STREAM, 1, 4, 33)
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(16, 4096, 4096, 99, 1, 4, 1)
    with pytest.raises(w8.W8A16Error) as e:
        w8.make_plan(0, 4096, 4096, w8.KERNEL_STREAM, 1, 4, 1)
    assert e.value.status == w8.ERR_M_ZERO


# ------------------------------------------------------------ batched tier

def test_batched_plan_one_variant_for_all_problems():
    # decode-style Q/K/V arms: 8 rows, hidden 4096, grouped K/V heads
    p = w8.plan_batched([(8, 4096, 4096), (8, 1024, 4096), (8, 1024, 4096)])
    assert (p.kernel, p.m_blocks, p.splits, p.flags, p.depth) == (w8.KERNEL_STREAM, 1, 1, 0, 1)
    nb = p.n_blocks
    tiles = [-(-n // (16 * nb)) for n in (4096, 1024, 1024)]
    assert p.grid == sum(tiles) and p.n_tiles == sum(tiles) and p.m_tiles == 1
    assert p.grid >= 3 * 256 // 4          # fills about three quarters of the CUs
    assert p.block == 64 * p.waves and p.lds_bytes <= 160 * 1024
    # above 16 rows the tile with the fewest bytes per CU over all arms'
    # tiles (small arms: 16-row tiles, several per tall arm); the shortest K
    # sets the waves
    p = w8.plan_batched([(40, 512, 1024), (3, 256, 256)])
    assert p.m_blocks == 1 and p.m_tiles == 3
    assert p.waves == 4                    # K = 256: two steps
    assert w8.plan_batched([(17, 64, 128)]).m_blocks == 1
    # Q/K/V arms of 48 rows: two 32 x 64 row tiles per arm, eight waves
    p = w8.plan_batched([(48, 4096, 4096), (48, 1024, 4096), (48, 1024, 4096)])
    assert (p.m_blocks, p.n_blocks, p.m_tiles, p.waves) == (2, 4, 2, 8)
    assert p.grid == 2 * (64 + 16 + 16)


def test_batched_tile_minimises_bytes_per_cu():
    """Property of the batched planner: above 16 rows the variant costs no
    more, over all arms' tiles, than any built stream tile (32 x 128 left
    out) by the bytes-per-CU model."""
    rng = np.random.default_rng(23)
    for _ in range(200):
        arms = [(int(rng.integers(1, 65)), int(rng.integers(1, 8193)),
                 128 * int(rng.integers(2, 41))) for _ in range(int(rng.integers(1, 5)))]
        if max(m for m, _, _ in arms) <= 16:
            continue
        p = w8.plan_batched(arms)

        def cost(mb, nb):
            tiles = sum(-(-m // (16 * mb)) * -(-((n + 15) // 16) // nb) for m, n, _ in arms)
            return -(-tiles // 256) * (32 * mb + 16 * nb)
        assert cost(p.m_blocks, p.n_blocks) == min(cost(mb, nb) for mb, nb in STREAM_TILES), arms


def test_batched_rejections_name_the_descriptor():
    with pytest.raises(w8.W8A16Error) as e:
        w8.plan_batched([])
    assert e.value.status == w8.ERR_BAD_PLAN
    with pytest.raises(w8.W8A16Error) as e:
        w8.plan_batched([(8, 64, 128)] * 9)
    assert e.value.status == w8.ERR_BAD_PLAN
    with pytest.raises(w8.W8A16Error) as e:
        w8.plan_batched([(8, 64, 128), (65, 64, 128)])
    assert e.value.status == w8.ERR_BAD_PLAN and "descriptor 1" in str(e.value)
    with pytest.raises(w8.W8A16Error) as e:
        w8.plan_batched([(8, 64, 128), (8, 64, 128), (8, 64, 100)])
    assert e.value.status == w8.ERR_K_NOT_MULT_128
    assert "descriptor 2: K=100" in str(e.value)


def test_batched_gemm_rejects_before_any_gpu_call():
    ok = dict(a=1 << 20, w_fp8=1 << 21, block_scale=1 << 22, c=1 << 23,
              a_row_stride=128, c_row_stride=64, m=4, n=64, k=128)
    assert w8.gemm_batched_raw([]) == w8.ERR_BAD_PLAN
    bad = dict(ok, m=0)
    assert w8.gemm_batched_raw([ok, bad]) == w8.ERR_M_ZERO
    assert w8.last_error().startswith("w8a16_gemm_batched: descriptor 1: m=0")
    bad = dict(ok, a_row_stride=100)
    assert w8.gemm_batched_raw([bad, ok]) == w8.ERR_PITCH_TOO_SHORT
    assert "descriptor 0" in w8.last_error()
    bad = dict(ok, c=0)
    assert w8.gemm_batched_raw([ok, ok, bad]) == w8.ERR_NULL_PTR
    assert "descriptor 2" in w8.last_error()
    bad = dict(ok, a_row_stride=132)
    assert w8.gemm_batched_raw([ok, bad]) == w8.ERR_A_STRIDE_ALIGN


# ------------------------------------------------- FP8 activations, W8A8

def test_act_quant_rejects_in_order_before_any_gpu_call():
    f = w8.act_quant_fp8_raw
    assert f(1, 128, 2, 128, 3, 0, 128) == w8.ERR_M_ZERO
    assert "w8a16_act_quant_fp8: m=0" in w8.last_error()
    assert f(1, 128, 2, 128, 3, 1, 100) == w8.ERR_K_NOT_MULT_128
    assert f(1, 120, 2, 128, 3, 1, 128) == w8.ERR_PITCH_TOO_SHORT
    assert f(1, 128, 2, 112, 3, 1, 128) == w8.ERR_PITCH_TOO_SHORT
    assert f(1, 132, 2, 128, 3, 1, 128) == w8.ERR_A_STRIDE_ALIGN
    assert f(1, 136, 2, 136, 3, 1, 128) == w8.ERR_A_STRIDE_ALIGN   # codes need 16-byte rows
    assert "q_row_stride=136" in w8.last_error()
    assert f(0, 128, 2, 128, 3, 1, 128) == w8.ERR_NULL_PTR
    assert f(1, 128, 2, 128, 0, 1, 128) == w8.ERR_NULL_PTR


def test_w8a8_rejects_before_any_gpu_call():
    f = w8.gemm_w8a8_raw
    assert f(1, 128, 2, 3, 4, 5, 16, 0, 16, 128) == w8.ERR_M_ZERO
    assert f(1, 136, 2, 3, 4, 5, 16, 1, 16, 128) == w8.ERR_A_STRIDE_ALIGN
    assert "qa_row_stride=136" in w8.last_error()
    assert f(1, 128, 0, 3, 4, 5, 16, 1, 16, 128) == w8.ERR_NULL_PTR
    p = w8.plan(4, 64, 256)
    assert f(1, 256, 2, 3, 4, 5, 64, 4, 64, 256, plan_=p) == w8.ERR_BAD_PLAN
    p8 = w8.plan_w8a8(4, 64, 256)
    assert w8.gemm_raw(1, 256, 3, 4, 5, 64, 4, 64, 256, plan_=p8) == w8.ERR_BAD_PLAN
    assert "W8A8" in w8.last_error()


@pytest.mark.parametrize("m,n,k,mb,nb", [
    (48, 4096, 4096, 2, 2),     # two 32 x 32 row tiles: 64 units per CU vs 80
    (32, 6144, 2048, 1, 3),     # tie with 32 x 32 (64): fewer rows win
    (40, 6144, 2048, 2, 4),     # tie with 64 x 32 (96): fewer rows win
    (24, 4096, 4096, 1, 2),
    (16, 12288, 5120, 1, 3),    # 16 rows: the fill rule
])
def test_w8a8_tile_cost_model(m, n, k, mb, nb):
    p = w8.plan_w8a8(m, n, k)
    _covers(p, m, n, k)
    assert (p.kernel, p.m_blocks, p.n_blocks) == (w8.KERNEL_W8A8, mb, nb)


def test_w8a8_plans():
    p = w8.plan_w8a8(8, 4096, 4096)
    assert (p.kernel, p.splits, p.depth, p.m_blocks) == (w8.KERNEL_W8A8, 1, 2, 1)
    assert p.grid == p.m_tiles * p.n_tiles >= 192
    assert p.lds_bytes == max(p.waves * (p.n_blocks + p.m_blocks) * 2048,
                              p.waves * p.n_blocks * p.m_blocks * 1024)
    for m, n, k in [(1, 256, 256), (16, 12288, 5120), (32, 6144, 2048), (48, 1000, 384),
                    (200, 300, 1024)]:
        p = w8.plan_w8a8(m, n, k)
        _covers(p, m, n, k)
        assert p.waves * 2 <= max(8, k // 128) or p.waves == 4
        assert p.waves != 16 or p.m_blocks * p.n_blocks <= 2
    with pytest.raises(w8.W8A16Error):          # 16 waves only with <= 2 blocks
        w8.make_plan(32, 256, 4096, w8.KERNEL_W8A8, 2, 2, 1, waves=16)
    with pytest.raises(w8.W8A16Error):          # no K split
        w8.make_plan(32, 256, 4096, w8.KERNEL_W8A8, 2, 2, 2, waves=8)
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(32, 256, 4096, w8.KERNEL_W8A8, 4, 4, 1, waves=8)


# --------------------------------------------------------------- W4A4 MX GEMV

def _w4a4_cost(m, n, mb, nb, cus=256):
    tiles = -(-m // (16 * mb)) * -(-n // (16 * nb))
    return -(-tiles // cus) * (mb + nb)


W4A4_TILES = [(1, 1), (1, 2), (1, 4), (2, 1), (2, 2), (2, 4), (4, 1), (4, 2)]


def _w4a4_ps_lds(mb, k, waves):
    a = mb * 16 * (k // 2 + 16)
    sc = -(-(mb * 16 * (k // 32)) // 256) * 256
    return a + sc + waves * 2 * mb * 1024


def test_w4a4_plans_cover_and_take_the_cheapest_tile():
    rng = np.random.default_rng(21)
    kinds = set()
    for _ in range(300):
        m = int(rng.integers(1, 65))
        n = int(rng.integers(1, 40000))
        k = 128 * int(rng.integers(1, 129))
        p = w8.plan_w4a4(m, n, k)
        kinds.add(p.kernel)
        mb = 1 if m <= 16 else (2 if m <= 32 else 4)
        n16 = -(-n // 16)
        fits = [w for w in (8, 4) if _w4a4_ps_lds(mb, k, w) <= 160 * 1024 - 256]
        grid = min(256, n16)
        items = -(-n16 // grid) * -(-(k // 128) // 4)
        if p.kernel == w8.KERNEL_W4A4_PS:
            # two or more tiles per CU and A fits in LDS: 8 waves, 4 for few
            # items or little LDS room
            assert fits and n16 >= 2 * 256 and p.m_blocks == mb and p.n_blocks == 1
            want = 8 if 8 in fits and items >= 8 else 4
            assert p.waves == want and p.grid == grid, (m, n, k)
            assert p.counter_count == 0 and p.lds_bytes == _w4a4_ps_lds(mb, k, p.waves)
            continue
        assert not fits or n16 < 2 * 256, (m, n, k)
        assert p.kernel == w8.KERNEL_W4A4 and p.splits == 1
        assert p.m_tiles * 16 * p.m_blocks >= m and p.n_tiles * 16 * p.n_blocks >= n
        assert p.grid == p.m_tiles * p.n_tiles
        best = min(_w4a4_cost(m, n, mb, nb) for mb, nb in W4A4_TILES)
        assert _w4a4_cost(m, n, p.m_blocks, p.n_blocks) == best, (m, n, k)
        assert p.lds_bytes == p.waves * p.m_blocks * p.n_blocks * 1024
        assert w4a4_variant_ok(p.m_blocks, p.n_blocks, p.waves)
        bigger = [w for w in (8, 16) if w > p.waves and w4a4_variant_ok(p.m_blocks, p.n_blocks, w)]
        assert not bigger or -(-k // 512) < 2 * bigger[0], (m, n, k, p.waves)
    assert kinds == {w8.KERNEL_W4A4, w8.KERNEL_W4A4_PS}


def w4a4_variant_ok(mb, nb, waves):
    """Register rule of the built tiled W4A4 variants: two groups of 4 K
    steps of mb + nb operand blocks in flight per wave."""
    return waves == 4 or (waves == 8 and mb + nb <= 4) or (waves == 16 and mb + nb <= 2)


def test_w4a4_explicit_plans_take_exactly_the_built_variants():
    for mb, nb in W4A4_TILES:
        for waves in (4, 8, 16):
            m = 16 * mb
            if w4a4_variant_ok(mb, nb, waves):
                p = w8.make_plan(m, 4096, 4096, w8.KERNEL_W4A4, mb, nb, 1, waves=waves)
                assert (p.block, p.lds_bytes) == (64 * waves, waves * mb * nb * 1024)
            else:
                with pytest.raises(w8.W8A16Error) as e:
                    w8.make_plan(m, 4096, 4096, w8.KERNEL_W4A4, mb, nb, 1, waves=waves)
                assert e.value.status == w8.ERR_BAD_PLAN


def test_w4a4_persistent_rule():
    # persistent with two or more 16-row tiles per CU and A in LDS
    for m, n, k in [(16, 32768, 4096), (16, 12288, 5120), (1, 8192, 4096), (33, 8192, 1024),
                    (24, 33000, 2048)]:
        assert w8.plan_w4a4(m, n, k).kernel == w8.KERNEL_W4A4_PS, (m, n, k)
    # one tile per CU or so: tiled
    for m, n, k in [(8, 4096, 4096), (32, 6144, 2048), (3, 1000, 512), (16, 8176, 4096)]:
        assert w8.plan_w4a4(m, n, k).kernel == w8.KERNEL_W4A4, (m, n, k)
    # A does not fit: 32 rows x 16384 K, 64 rows x 4096 K
    for m, n, k in [(32, 65536, 16384), (64, 32768, 4096), (16, 65536, 1 << 16)]:
        assert w8.plan_w4a4(m, n, k).kernel == w8.KERNEL_W4A4, (m, n, k)
    p = w8.plan_w4a4(12, 40000, 2048, cu_count=100)
    assert p.kernel == w8.KERNEL_W4A4_PS and p.grid == 100 and p.waves == 8
    p = w8.plan_w4a4(16, 32768, 4096)
    assert (p.waves, p.grid) == (8, 256)
    assert p.lds_bytes == 16 * 2064 + 16 * 128 + 8 * 2 * 1024
    # few items per workgroup: 4 waves
    p = w8.plan_w4a4(16, 8192, 512)
    assert (p.kernel, p.waves) == (w8.KERNEL_W4A4_PS, 4)
    # the tiled kernel gives each wave two groups of 4 K steps
    p = w8.plan_w4a4(8, 4096, 4096)
    assert (p.m_blocks, p.n_blocks, p.waves) == (1, 1, 4)


def test_w4a4_plan_errors():
    with pytest.raises(w8.W8A16Error) as e:
        w8.plan_w4a4(65, 4096, 4096)
    assert e.value.status == w8.ERR_BAD_PLAN
    for args, status in [((0, 16, 128), w8.ERR_M_ZERO), ((1, 16, 100), w8.ERR_K_NOT_MULT_128),
                         ((1, 0, 128), w8.ERR_N_ZERO)]:
        with pytest.raises(w8.W8A16Error) as e:
            w8.plan_w4a4(*args)
        assert e.value.status == status
    # K and the A pitch stay within the kernels' 32-bit buffer ranges
    for m, n, k in [(1, 16, (1 << 24) + 128), (16, 4096, 1 << 25)]:
        with pytest.raises(w8.W8A16Error) as e:
            w8.plan_w4a4(m, n, k)
        assert e.value.status == w8.ERR_BAD_PLAN
    assert w8.plan_w4a4(1, 16, 1 << 24).kernel == w8.KERNEL_W4A4
    # explicit plans: unsupported tile, waves, persistent rows not covered
    for kern, mb, nb, waves, m in [(w8.KERNEL_W4A4, 4, 4, 8, 64), (w8.KERNEL_W4A4, 1, 8, 8, 16),
                                   (w8.KERNEL_W4A4, 1, 1, 6, 16),
                                   (w8.KERNEL_W4A4_PS, 1, 1, 16, 17),
                                   (w8.KERNEL_W4A4_PS, 3, 1, 8, 40),
                                   (w8.KERNEL_W4A4_PS, 2, 1, 6, 32)]:
        with pytest.raises(w8.W8A16Error):
            w8.make_plan(m, 4096, 4096, kern, mb, nb, 1, waves=waves)
    p = w8.make_plan(17, 4096, 4096, w8.KERNEL_W4A4_PS, 2, 1, 1, waves=8, cu_count=4)
    assert (p.grid, p.block, p.counter_count) == (4, 512, 0)
    # fewer workgroups than CUs when the weight has fewer 16-row tiles
    p = w8.make_plan(17, 100 * 16, 4096, w8.KERNEL_W4A4_PS, 2, 1, 1, waves=16)
    assert p.grid == 100
    # A and the partial tiles must fit in LDS: 64 rows x 4096 K at 16 waves do not
    with pytest.raises(w8.W8A16Error):
        w8.make_plan(64, 4096, 4096, w8.KERNEL_W4A4_PS, 4, 1, 1, waves=16)


def test_torch_bindings_reject_host_tensors():
    """The tensor-level entry points refuse host tensors before any library
    call (a host pointer handed to a kernel would fault the GPU)."""
    import torch
    a = torch.zeros((4, 256), dtype=torch.bfloat16)
    w = torch.zeros((64, 256), dtype=torch.uint8)
    s = torch.ones((1, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensors"):
        w8.gemm(a, w, s)
    qa = torch.zeros((4, 256), dtype=torch.uint8)
    sa = torch.ones((4, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensors"):
        w8.gemm_w8a8(qa, sa, w, s)
    with pytest.raises(ValueError, match="a_scales must hold"):
        w8.gemm_w8a8(qa, sa[:2], w, s)
    with pytest.raises(ValueError, match="CUDA tensor"):
        w8.act_quant_fp8(a)
