"""Decode steps captured in a HIP graph and replayed give the same bits as the same steps run
eagerly.

One window of L lock-step decode steps (L - 1 replays and the fused fold) is captured from a fresh
state, where the host's count bounds start and end at zero, and replayed several times with
eager work and synchronizations between the replays. A second state runs the same steps eagerly;
after every replay all L outputs and, at the end, the exported checkpoints must be identical.
"""
import pytest
import torch

from harness import to_dev
from ssm_decode_state_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
bd = pytest.importorskip("ssm_decode_state_amd.binding")
DEV = torch.device("cuda:0")


def _state(shape, seed, rc):
    A, D = synth.head_constants(shape, seed)
    h0 = synth.initial_state(shape, seed, 0.3)
    cfg = bd.make_config(shape.kind, shape.batch, shape.heads, shape.groups, shape.dim_p,
                         shape.dim_n, shape.window, 1, bd.SSM_IN_BF16, rc)
    return bd.State(cfg, h0.to(DEV), None if A is None else A.to(DEV),
                    None if D is None else D.to(DEV))


@pytest.mark.parametrize("kind,rc", [(synth.MAMBA2, 0), (synth.MAMBA2, bd.SSM_RC_FP8_ROW),
                                     (synth.GDN, 0), (synth.KDA, 0), (synth.GDN, bd.SSM_RC_FP4_B16),
                                     (synth.KDA, bd.SSM_RC_FP8_ROW)])
def test_graph_window_replays_match_eager(kind, rc):
    L, R = 8, 3
    if kind == synth.MAMBA2:
        shape = synth.Shape(kind, 4, 8, 8, 64, 128, L, 1)
    else:
        shape = synth.Shape(kind, 3, 4, 4, 128, 128, L, 1)
    seed = 400 + kind + 3 * rc
    inputs = [to_dev(synth.token_inputs(shape, seed, "graph", i), DEV) for i in range(L)]
    eager, graphed = _state(shape, seed, rc), _state(shape, seed, rc)
    ye = [torch.empty(shape.batch, shape.heads, shape.dim_p, device=DEV) for _ in range(L)]
    yg = [torch.zeros_like(t) for t in ye]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(L):
            bd.ssm_replay_decode(graphed, inputs[i], yg[i])
    assert (graphed.st.count_lo, graphed.st.count_hi) == (0, 0)
    scratch = torch.randn(1 << 20, device=DEV)
    for r in range(R):
        for i in range(L):
            bd.ssm_replay_decode(eager, inputs[i], ye[i])
        scratch.mul_(0.5).add_(1.0)  # unrelated eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(L):
            assert torch.equal(yg[i], ye[i]), "replay %d, step %d" % (r, i)
    sh = shape
    ne = torch.empty(sh.batch, sh.heads, sh.dim_p, sh.dim_n, device=DEV)
    ng = torch.empty_like(ne)
    bd.ssm_ckpt_export(eager, ne)
    bd.ssm_ckpt_export(graphed, ng)
    torch.cuda.synchronize()
    assert torch.equal(ne, ng)
