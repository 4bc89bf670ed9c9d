"""GPU: products captured into a HIP graph replay to the eager results, every time.

A decode step is a chain of short launches, so callers capture it into a graph
(the bench times the batch-1 step that way).  Captured here, in one graph: a
batch-1 product (GEMV), a batch-16 product (streaming MFMA kernel), two
batch-256 products (one that splits k through the binding's workspace, i.e.
a GEMM launch and a reduction launch, and one that does not) and a grouped
batch-1 dispatch.  The graph is replayed four times; before each replay the
outputs are poisoned eagerly and other eager products run, and after it every
output must equal its eager result bit for bit (all these paths add in a fixed
order) and stay within the design bound of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DESIGN_BOUND = 1e-4


@pytest.fixture(scope="module")
def nbw():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nested_bit_weight_amd as m
    m.library()
    return m


def rel_err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    return float((np.abs(y - ref).max(axis=1) / den).max())


def _problem(nbw, n, k, batch, r, seed):
    case = synth.random_case(n, k, batch, seed=seed, recipe="gptq_like", outliers=batch > 16)
    w = nbw.pack_bitplanes(torch.from_numpy(case["codes"]).cuda())
    x = torch.from_numpy(case["x"]).view(torch.bfloat16).cuda()
    s = torch.from_numpy(case["scales"]).view(torch.bfloat16).cuda()
    return case, w.slice_view(r), x, s, r


def test_graph_replays_match_eager(nbw):
    specs = [(1000, 2048, 1, 3), (512, 1024, 16, 4), (512, 4096, 256, 4), (2304, 768, 256, 2)]
    probs = [_problem(nbw, *sp, seed=90 + i) for i, sp in enumerate(specs)]
    assert nbw.workspace_bytes(256, 512, 4096, 4) > 0, "the third product must split k"
    assert nbw.workspace_bytes(256, 2304, 768, 2) == 0, "the fourth must not (6 groups: no split)"
    calls = [nbw.QgemmCall(x, w, s, r) for _, w, x, s, r in probs]
    gprobs = [_problem(nbw, 300 + 16 * i, 1024, 1, 2 + i, seed=100 + i) for i in range(3)]
    gitems = [(x, w, s, r) for _, w, x, s, r in gprobs]
    gouts = [torch.empty((1, w.n), dtype=torch.float32, device="cuda") for _, w, _, _, _ in gprobs]

    for c in calls:
        c()
    nbw.qgemm_grouped(gitems, outs=gouts)
    torch.cuda.synchronize()
    eager = [c.out.clone() for c in calls] + [o.clone() for o in gouts]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one warm-up on a side stream before capture
        for c in calls:
            c()
        nbw.qgemm_grouped(gitems, outs=gouts)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
        nbw.qgemm_grouped(gitems, outs=gouts)
    torch.cuda.synchronize()

    outs = [c.out for c in calls] + gouts
    other = _problem(nbw, 256, 1024, 64, 4, seed=120)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        nbw.qgemm(other[2], other[1], other[3], other[4])  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"replay {rep}: output {i} differs from the eager result"
    for (case, w, x, s, r), y in zip(probs + gprobs, outs):
        ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], w.n, w.k, r)
        assert rel_err(y.cpu().numpy(), ref) <= DESIGN_BOUND
