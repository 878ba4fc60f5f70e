"""The layer forward captured as a HIP graph and replayed.

Each replay, with the program's own eager work and synchronisations between
replays, gives the same bits as an eager forward of the same batch (the
library launches kernels only: no memset nodes, no allocation in the
captured region).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_common import bf16_dev, bf16_values_host, host, log
from test_gpu_layer import build_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T", [("mid", 200), ("mid", 2048)])
def test_forward_graph_replays(name, T):
    cfg = synth.CONFIGS[name].with_(T=T)
    layer, C, b = build_layer(cfg)
    xs = [synth.gen_x(cfg, seed=s) for s in (11, 12, 13)]
    log(f"[graph] {name} T={T}: eager forwards")
    eager = []
    for xb in xs:
        eager.append((bf16_values_host(layer.forward(bf16_dev(xb))),
                      host(layer.buffers(T).topk_idx).copy()))
    x_in = bf16_dev(xs[0])
    g = layer.capture(x_in)
    bufs = layer.buffers(T)
    for rep in range(2):
        for i, xb in enumerate(xs):
            x_in.copy_(bf16_dev(xb))
            g.replay()
            torch.cuda.synchronize()
            y = bf16_values_host(bufs.y)
            assert np.array_equal(y, eager[i][0]), (rep, i)
            assert np.array_equal(host(bufs.topk_idx), eager[i][1]), (rep, i)
            # eager work of the program's own between replays
            other = layer.forward(bf16_dev(xs[(i + 1) % 3]))
            torch.cuda.synchronize()
            assert np.array_equal(bf16_values_host(other), eager[(i + 1) % 3][0])
    log(f"[graph] {name} T={T}: 6 replays equal the eager forwards")
