"""HIP-graph capture of the forward: it only enqueues kernels (no allocation,
sync or memset), so a captured graph must replay to the eager result, bit
for bit, every time -- with the program's own eager work and syncs between
replays."""
import numpy as np
import pytest
import torch

import bit_rank_post_amd as tq
import synth
from bit_rank_post_amd import io as tqio
from tests.gpu_util import need_gpu
from tests.test_gpu_parity import small_swiglu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    need_gpu()


@pytest.mark.parametrize("which,T,path", [("tiny", 64, 1), ("tiny", 64, 2),
                                          ("swiglu", 24, 1), ("swiglu", 300, 2),
                                          ("shared", 24, 1), ("shared", 300, 2)])
def test_graph_replay_matches_eager(which, T, path):
    if which == "tiny":
        cfg = synth.CONFIG_BY_NAME["tiny"]
        layer = synth.make_layer(cfg)
        x, ids, g = synth.make_tokens(cfg, T)
        act, d_out = cfg.act, cfg.d_ff
    else:
        layer = small_swiglu("f16", 3)
        if which == "shared":
            # the shared expert runs on the layer's second stream: the capture
            # must follow the fork and the join
            layer["shared"] = synth.make_shared(256, 384, np.random.SeedSequence(11))
        x, ids, g = synth.make_custom_tokens(256, 8, 2, T, "f16", seed=5)
        act, d_out = "f16", 256
    L = tqio.upload_layer(layer)
    L.set_path(path)
    xd, idd, gd = tqio.tokens_to_device(x, ids, g, act)
    k = ids.shape[1]
    ws = tqio.workspace(L, T, k)
    y_eager = torch.empty((T, d_out), dtype=torch.float32, device="cuda")
    L.forward(xd, T, idd, gd, k, y_eager, tq.TQ_F32, ws)
    torch.cuda.synchronize()
    ref = y_eager.clone()
    y = torch.full((T, d_out), float("nan"), dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.forward(xd, T, idd, gd, k, y, tq.TQ_F32, ws)
    for rep in range(4):
        y.fill_(float("nan"))
        scratch = torch.randn(1 << 16, device="cuda")      # eager work between replays
        (scratch * 2).sum().item()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep} differs from eager"
