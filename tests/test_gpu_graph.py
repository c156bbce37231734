"""A whole forward + backward step captured in a HIP graph (torch.cuda.graph)
and replayed: the library's calls enqueue only kernels (no allocation, no
memset node, no host synchronisation), so short launch-bound steps can be
replayed without host overhead. Every replay must give the eager bits."""
import math

import pytest
import torch

import exact_attention_71_amd as ea
from workloads import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _step(g, causal, det, opts, plan=None, varlen=None):
    if varlen is None:
        o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=causal)
        grads = ea.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, causal=causal,
                       deterministic=det, options=opts)
    else:
        mx = varlen
        cq, ck = g["cu_seqlens_q"], g["cu_seqlens_k"]
        o, lse = ea.fwd_varlen(g["q"], g["k"], g["v"], cq, ck, mx, mx, causal=causal, plan=plan)
        grads = ea.bwd_varlen(g["q"], g["k"], g["v"], o, g["do"], lse, cq, ck, mx, mx,
                              causal=causal, deterministic=det, options=opts, plan=plan)
    return (o, lse) + tuple(grads)


@pytest.mark.parametrize("d,design,det", [(64, ea.BWD_AUTO, False), (128, ea.BWD_AUTO, False),
                                          (128, ea.BWD_FUSED_DQ, True),
                                          (256, ea.BWD_RECOMPUTE, False)])
@pytest.mark.parametrize("varlen", [False, True])
def test_captured_step_replays_match_eager(d, design, det, varlen):
    torch.manual_seed(0)
    if varlen:
        lengths = [700, 3, 0, 1300, 257]
        inp = make_inputs(0, 0, 0, 4, 2, d, seed=61, lengths=lengths)
        g = {k: v.to(DEV) for k, v in inp.items()}
        mx = max(lengths)
        plan = ea.varlen_plan(g["cu_seqlens_q"], g["cu_seqlens_k"], mx, mx, sum(lengths),
                              sum(lengths), 4, 2, d, True)
    else:
        inp = make_inputs(2, 600, 600, 4, 2, d, seed=61)
        g = {k: v.to(DEV) for k, v in inp.items()}
        mx, plan = None, None
    opts = dict(bwd_design=design)
    eager = _step(g, True, det, opts, plan, mx)   # also warms every lazily set-up launch path
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = _step(g, True, det, opts, plan, mx)
    for r in range(3):
        graph.replay()
        # eager work of the program between replays
        other = _step(g, True, det, opts, plan, mx)
        torch.cuda.synchronize()
        for i, (x, y, z) in enumerate(zip(eager, captured, other)):
            assert torch.equal(x, y), (r, i)
            assert torch.equal(x, z), (r, i)
