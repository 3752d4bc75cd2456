"""Calls of every enqueuing entry point on small seeded problems, for the
diagnostics tests: run once in a child process with W8A16_LOG=1 and
W8A16_DEBUG_SYNC=1 (``python tests/diag_calls.py OUT.npz``) and once in the
test process without them; the outputs must agree bit for bit (the same
plans give the same bits)."""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import datagen  # noqa: E402


def run_all():
    import torch
    import block_scaled_fp8_w8a16_amd as w8
    out = {}

    def t16(x):
        return torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16).cuda()

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    def bits(c):
        torch.cuda.synchronize()
        return c.cpu().view(torch.int16).numpy().view(np.uint16).copy()

    # default plans: stream kernel (called twice: logged once), a K split,
    # the tile kernel
    for name, (m, n, k) in (("stream", (16, 4096, 1024)), ("split", (1, 1024, 8192)),
                            ("tile", (40, 2304, 8192))):
        p = datagen.make_problem(m, n, k, seed=11)
        a, wq, s = t16(p.a), t(p.w), t(p.scale)
        c = w8.gemm(a, wq, s)
        if name == "stream":
            c = w8.gemm(a, wq, s, c)
        out[name] = bits(c)
    # an explicit plan
    p = datagen.make_problem(16, 4096, 1024, seed=12)
    plan = w8.make_plan(16, 4096, 1024, w8.KERNEL_STREAM, 1, 2, 1, depth=1, waves=8)
    out["planned"] = bits(w8.gemm(t16(p.a), t(p.w), t(p.scale), plan_=plan))
    # quantizer and W8A8
    p = datagen.make_problem(8, 2048, 1024, seed=13)
    qa, sa = w8.act_quant_fp8(t16(p.a))
    out["w8a8"] = bits(w8.gemm_w8a8(qa, sa, t(p.w), t(p.scale)))
    # W4A4
    mx = datagen.make_mx_problem(8, 4096, 2048, seed=14)
    out["w4a4"] = bits(w8.gemm_w4a4(t(mx.a), t(mx.a_scale), t(mx.w), t(mx.w_scale), mx.k))
    # batched
    probs = [datagen.make_problem(4, 1024, 512, seed=15), datagen.make_problem(8, 512, 1024, seed=16)]
    args = [(t16(q.a), t(q.w), t(q.scale),
             torch.empty((q.m, q.n), dtype=torch.bfloat16, device="cuda")) for q in probs]
    cs = w8.gemm_batched(args)
    out["batched0"], out["batched1"] = bits(cs[0]), bits(cs[1])
    # captured into a graph on a side stream (the debug wait is skipped
    # while capturing), then replayed
    p = datagen.make_problem(16, 4096, 1024, seed=17)
    a, wq, s = t16(p.a), t(p.w), t(p.scale)
    c = torch.zeros((16, 4096), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        g.capture_begin()
        w8.gemm(a, wq, s, c, stream=side)
        g.capture_end()
    g.replay()
    out["graph"] = bits(c)
    return out


if __name__ == "__main__":
    res = run_all()
    np.savez(sys.argv[1], **res)
    print("diag calls done", flush=True)
