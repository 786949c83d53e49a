"""HIP graph capture of mpgemm_w4a16 (decode and prefill kernels).

A caller that captures the GEMM into a graph must get, on every replay, what the eager
call gives.  The kernels allocate nothing and clear nothing with memset, so capture adds
no graph nodes besides the kernel launches.  Each graph is replayed several times, with
eager work (another GEMM, torch ops) and synchronizations between replays, and every
replay is compared bit-for-bit with the eager result (same kernel, deterministic order).
"""
import numpy as np
import pytest
import torch

import weight_only_quantized_mpgemm_amd as mp
import workloads

pytestmark = pytest.mark.gpu


def _packed(K, N, g, seed):
    codes, scales, zeros = workloads.weights(K, N, g, False, 0.005, 0.02, seed)
    dev = torch.device("cuda")
    return mp.pack_weights(torch.from_numpy(codes).to(dev),
                           torch.from_numpy(scales.view(np.int16)).to(dev).view(torch.float16),
                           torch.from_numpy(zeros).to(dev), g)


@pytest.mark.parametrize("M,K,N", [(1, 1024, 512), (16, 2048, 768), (200, 512, 528), (256, 1024, 1024)])
def test_graph_replays_match_eager(M, K, N):
    print(f"[case] graph M={M} K={K} N={N}", flush=True)
    dev = torch.device("cuda")
    packed = _packed(K, N, 128, 11)
    other = _packed(K, N, 128, 12)
    x = torch.from_numpy(workloads.activations(M, K, "f16", 13).view(np.int16)).to(dev).view(torch.float16)
    eager = mp.w4a16(x, packed)
    torch.cuda.synchronize()

    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        mp.w4a16(x, packed, out=y)            # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        mp.w4a16(x, packed, out=y)

    for r in range(4):
        y.fill_(float("nan"))
        z = mp.w4a16(x, other)                # eager work between replays
        z.add_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
