"""The quantize / dequantize entry points enqueue only kernel launches on the
caller's stream (no allocation, memset or host synchronization), so a caller can
capture them in a HIP graph. Each replay is checked against the eager result,
with eager work and synchronizations between replays."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hadamard", [False, True])
def test_graph_replays_match_eager(gpu, hadamard):
    x = to_dev(workloads.workload(5 if hadamard else 4, (64, 1024) if hadamard else (96, 28672)))
    offs = (-8, 8) if hadamard else (-2, 6)
    c_ref, s_ref, g_ref = gpu.quantize(x, offs, hadamard=hadamard)
    y_ref = gpu.dequantize(c_ref, s_ref, g_ref, torch.float32)
    torch.cuda.synchronize()

    ws = torch.empty(gpu.workspace_bytes(*x.shape), dtype=torch.uint8, device=x.device)
    codes = torch.empty_like(c_ref)
    scales = torch.empty_like(s_ref)
    y = torch.empty_like(y_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        c, s, g = gpu.quantize(x, offs, hadamard=hadamard, workspace=ws)  # warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        c, s, g = gpu.quantize(x, offs, hadamard=hadamard, workspace=ws)
        gpu.dequantize(c, s, g, torch.float32, out=y)
        codes.copy_(c)
        scales.copy_(s)
    for rep in range(4):
        codes.zero_()
        scales.zero_()
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, c_ref), rep
        assert torch.equal(scales, s_ref), rep
        assert torch.equal(g, g_ref), rep
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), rep
        # unrelated eager work between replays
        gpu.quantize(x, (0, 0), hadamard=hadamard)
        torch.cuda.synchronize()
