"""Collection-time helpers for the variant tests: the tile kernel's built
ring sizes, read from the table the launcher is generated from
(``W8A16_TILE_VARIANTS`` in csrc/plan.h), and a filter that keeps only the
parameter combinations the library's planner accepts (a pure host call), so
the tests cover exactly the variants the library dispatches and collect no
combination that could only be skipped."""

import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PLAN_H = os.path.join(ROOT, "block_scaled_fp8_w8a16_amd", "csrc", "plan.h")


def tile_variants():
    """[(m_blocks, n_blocks, depth, a_depth), ...] in table order."""
    text = open(PLAN_H).read()
    start = text.index("#define W8A16_TILE_VARIANTS(X)")
    end = text.index("\n\n", start)
    table = text[start:end].split("\n", 1)[1]
    return [tuple(int(v) for v in t) for t in
            re.findall(r"X\((\d+),\s*(\d+),\s*(\d+),\s*(\d+)\)", table)]


def plan_ok(m, n, k, kernel, m_blocks, n_blocks, splits, **kw):
    """True if w8a16_plan_finalize accepts the plan.  Runs on the host
    without a GPU; if the library is not built, every combination is kept
    (the tests then fail loudly when they load it)."""
    try:
        import block_scaled_fp8_w8a16_amd as w8
        w8.make_plan(m, n, k, kernel, m_blocks, n_blocks, splits, **kw)
        return True
    except ImportError:
        return True
    except Exception as e:              # W8A16Error: a plan the library rejects
        if type(e).__name__ == "W8A16Error":
            return False
        raise
