"""The tile kernel's built ring sizes, read from the table the launcher is
generated from (``W8A16_TILE_VARIANTS`` in csrc/plan.h), so the tests cover
exactly the variants the library dispatches."""

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
