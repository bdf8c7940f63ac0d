"""The quant + GEMM step captured in a HIP graph (as the benchmark times launch-bound decode
rows) replays to the eager result, bit for bit, on every replay, with eager work and device
synchronisations between the replays.  No kernel of the library records a memset."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import w4a4_outlier_split_amd as osc  # noqa: E402
from gpu_util import dev_bits16, pack, quant  # noqa: E402


@pytest.mark.parametrize("S", [16, 300])
def test_graph_replays_match_eager(S):
    N, H, G = 512, 1024, 32
    X = dev_bits16(synth.random_bf16((S, H), seed=S, scale=3.0))
    W = dev_bits16(synth.random_bf16((N, H), seed=N, scale=0.05))
    L = np.random.default_rng(S).integers(-1, G, H // G).astype(np.int32)
    QW, SW, WL = pack(W, N, H, G, L, osc.OSC_MXFP4)
    QX, SX, B = quant(X, S, H, G, L, osc.OSC_MXFP4)
    Y = torch.empty((S, N), dtype=torch.bfloat16, device="cuda:0")

    def step(stream):
        osc.osc_quant_act(X, S, H, G, L, osc.OSC_MXFP4, QX, SX, B, stream)
        osc.osc_gemm(QX, SX, B, QW, SW, WL, S, N, H, G, Y, osc.OSC_Y_BF16, stream)

    step(None)
    torch.cuda.synchronize()
    ref = Y.clone()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        Y.fill_(0)
        QX.fill_(0)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
