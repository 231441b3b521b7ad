"""The attention forward captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

The library allocates nothing, never synchronises and issues no memset: one call is one kernel
launch on the caller's stream, so it can be captured and replayed.  Each replay runs after eager
work on the same buffers and must reproduce the eager result bit for bit (the kernels are
deterministic), for every replay, not only the first.
"""
import pytest
import torch

from attention_forward_06_amd import binding

from gpu_util import gpu_qkv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode,D,dtype,bs", [("causal", 128, "bf16", 0), ("none", 64, "f16", 0),
                                             ("block_diag", 128, "f16", 64),
                                             ("causal", 256, "bf16_v_e5m2", 0)])
def test_graph_replays_match_eager(mode, D, dtype, bs):
    q, k, v = gpu_qkv(2, 4, 512, D, dtype, seed=31)
    ref, ref_lse = binding.attn_fwd(q, k, v, mask=mode, block_size=bs, return_lse=True)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    # warm-up call on a side stream before capture (default priority)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        binding.attn_fwd(q, k, v, mask=mode, block_size=bs, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _, lse = binding.attn_fwd(q, k, v, mask=mode, block_size=bs, out=out, return_lse=True)
    for _ in range(3):
        out.fill_(float("nan"))          # eager work on the graph's buffers between replays
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(lse, ref_lse)


def test_graph_of_several_calls_on_fresh_inputs():
    """Three calls in one graph; new input values copied into the captured buffers before each
    replay are picked up (the graph holds pointers, not values)."""
    shapes = [("causal", 128, "bf16", 0), ("none", 64, "f16", 0), ("block_diag", 64, "bf16", 32)]
    bufs = [gpu_qkv(1, 3, 384, D, dt, seed=5) for _, D, dt, _ in shapes]
    outs = [torch.empty_like(q) for q, _, _ in bufs]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for (mode, _, _, bs), (q, k, v), o in zip(shapes, bufs, outs):
            binding.attn_fwd(q, k, v, mask=mode, block_size=bs, out=o)
    for seed in (11, 12):
        for (mode, D, dt, bs), (q, k, v) in zip(shapes, bufs):
            nq, nk, nv = gpu_qkv(1, 3, 384, D, dt, seed=seed)
            q.copy_(nq)
            k.copy_(nk)
            v.copy_(nv)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (mode, _, _, bs), (q, k, v), o in zip(shapes, bufs, outs):
            ref = binding.attn_fwd(q, k, v, mask=mode, block_size=bs)
            torch.cuda.synchronize()
            assert torch.equal(o, ref), (mode, seed)
