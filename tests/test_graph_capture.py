"""The library's calls inside a captured HIP graph.

The library allocates nothing and issues no memset or synchronisation (the
fused backward clears its workspace with a kernel), so a forward and a
backward can be captured into one graph (outputs and workspaces come from
torch's graph pool) and replayed.  Each replay must give the eager results
bit for bit where the kernels are deterministic -- everything except the
fused backward's query gradients, whose atomic fp32 additions come in a
varying order; those must agree to bf16 rounding.  The library's choices
(partitions, form, workspace) depend on the sizes only.  Eager work and
synchronisations run between the replays.
"""
import pytest
import torch

from attention_distillation_kl_amd import make_inputs, ops
from attention_distillation_kl_amd.inputs import upstream_grad
from parity_util import log

pytestmark = pytest.mark.gpu

DEV = "cuda"


# B, H, NQ, NK, d, causal: a shape that fills the GPU with the plain kernels;
# a short query block that takes the split-K forward and the key-partitioned
# backward (both with workspace); one query tile per head, which takes the
# split-K forward and the fused backward.
CASES = [(1, 32, 4096, 4096, 128, False), (1, 4, 128, 8192, 128, True), (1, 4, 64, 8192, 128, True)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_forward_and_backward_replay_from_a_captured_graph(case):
    B, H, NQ, NK, d, causal = case
    log(f"graph capture {case}")
    from attention_distillation_kl_amd import _lib
    plain = _lib.fwd_splits(B, H, NQ, NK, d, int(causal), _lib.BF16) == 1
    assert plain == (_lib.bwd_workspace_size(B, H, NQ, NK, d, int(causal), _lib.BF16, 3) == 0)
    fused = _lib.bwd_fused_selected(B, H, NQ, NK, d, int(causal), _lib.BF16, 3) == 1
    assert fused == (NQ <= 64)
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, torch.bfloat16, "student", 0.3, seed=NQ + 3, device=DEV)
    g = upstream_grad(B, H, NQ, seed=9, device=DEV)
    scale = d ** -0.5

    def step():
        kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, scale, causal)
        return (kl, l1, l2) + tuple(ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal))

    want = step()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream's side, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got = step()
    for rep in range(3):
        other = step()  # eager work between replays, on the same allocator
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, y, z in zip(("kl", "lse1", "lse2", "dq1", "dk1", "dq2", "dk2"), got, want, other):
            if fused and name.startswith("dq"):
                for v, tag in ((x, "replay"), (z, "eager")):
                    rel = ((v.double() - y.double()).norm() / y.double().norm()).item()
                    assert rel < 4e-3, (rep, name, tag, rel)
                continue
            assert torch.equal(x, y), (rep, name)
            assert torch.equal(z, y), (rep, name, "eager")
