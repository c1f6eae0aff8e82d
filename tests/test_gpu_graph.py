"""The decode entry points under HIP graph capture.

A decode loop replays the same layer calls every token, so it can capture
them once into a graph instead of paying the host launch path per call.
The compute entry points enqueue kernels only (no memset, copy or
synchronization), so a captured sequence of them must reproduce the eager
results bit for bit on every replay (all kernels reduce in a fixed order).
The replays are separated by eager work that overwrites the outputs and by
synchronizations, as a real loop would interleave them."""
import numpy as np
import pytest

import synth
from tests.gpu_util import dev, say, torch

pytestmark = pytest.mark.gpu

q = pytest.importorskip("gemm_unpack_bit_amd")


def test_decode_sequence_replays_bitwise_in_a_graph():
    t = torch()
    N, K = 1024, 2048
    uc = synth.uniform_case(501, 16, N, K, 4)
    wq, s, zq = q.pack(dev(uc["codes"]), 4), dev(uc["scales"]), q.pack_zeros(dev(uc["zeros"]), 4)
    x1, x4 = dev(uc["x"][:1]), dev(uc["x"][:4])
    lc = synth.lut4_case(502, 1, N, K)
    lwq, la, llut = q.pack(dev(lc["codes"]), 4), dev(lc["absmax"]), dev(lc["lut"])
    oc = synth.outlier_case(503, 1, N, K)
    ptr, rec = q.tilecoo_encode(N, K, oc["o_rows"], oc["o_cols"], oc["o_vals"])
    owq, os_, ozq = q.pack(dev(oc["codes"]), 4), dev(oc["scales"]), q.pack_zeros(dev(oc["zeros"]), 4)
    tp, tr = dev(ptr.view(np.int32)), dev(rec.view(np.int32))
    cc = synth.codebook_case(504, 4, N, K)
    ccodes, ccb, cs = q.pack(dev(cc["codes"]), 8, q.LAYOUT_ROWS64), dev(cc["codebook"]), dev(cc["scales"])
    cws = t.zeros(max(q.codebook_workspace_bytes(4, N, K), 4), dtype=t.uint8, device="cuda")
    ws8 = t.zeros(q.w4a8_workspace_bytes(1, K), dtype=t.uint8, device="cuda")
    x4c = dev(cc["x"][:4])
    xg = dev(synth.activations(505, 96, K))  # prefill rows: the matrix-core GEMM

    shapes = [(1, N), (4, N), (1, N), (1, N), (4, N), (1, N), (96, N)]
    outs = [t.empty(m, n, dtype=t.float16, device="cuda") for m, n in shapes]

    def sequence():
        q.w4a16(x1, wq, s, zq, out=outs[0])
        q.uniform(x4, wq, s, zq, 4, q.PATH_MFMA, out=outs[1])
        q.lut4(x1, lwq, la, llut, out=outs[2])
        q.outlier(x1, owq, os_, ozq, tp, tr, out=outs[3])
        q.codebook(x4c, ccodes, ccb, cs, ws=cws, out=outs[4])
        q.w4a8(x1, wq, s, zq, ws8, out=outs[5])
        q.gemm_uniform(xg, wq, s, zq, 4, out=outs[6])

    say("graph: eager sequence")
    sequence()
    t.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for o in eager:
        assert bool(t.isfinite(o.float()).all())

    g = t.cuda.CUDAGraph()
    say("graph: capture")
    with t.cuda.graph(g):
        sequence()
    t.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))  # eager work between replays
        t.cuda.synchronize()
        say("graph: replay", rep)
        g.replay()
        t.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert t.equal(o.view(t.int16), e.view(t.int16)), f"replay {rep}: call {i} differs from the eager result"
