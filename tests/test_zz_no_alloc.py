"""The allocation-free forward (tq_forward_noalloc, static scratch array)
against tq_forward with a caller workspace: the same kernels on the same
inputs, so the outputs must agree bit for bit (at least within the parity
bar), on two calls in a row with the second one smaller, at both execution
paths; requests beyond the scratch size are rejected before any launch."""
import numpy as np
import pytest
import torch

import bit_rank_post_amd as tq
import synth
from bit_rank_post_amd import io as tqio
from tests.gpu_util import TORCH_DT, Y_DT, assert_parity, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    need_gpu()


def both(L, x, ids, g, act, y_dtype):
    T, k = ids.shape
    xd, idd, gd = tqio.tokens_to_device(x, ids, g, act)
    d_out = L.d_ff if L.kind == tq.TQ_SINGLE else L.d_model
    y_ws = torch.empty((T, d_out), dtype=TORCH_DT[y_dtype], device="cuda")
    y_na = torch.full((T, d_out), float("nan"), dtype=TORCH_DT[y_dtype], device="cuda")
    ws = tqio.workspace(L, T, k)
    L.forward(xd, T, idd, gd, k, y_ws, Y_DT[y_dtype], ws)
    L.forward_noalloc(xd, T, idd, gd, k, y_na, Y_DT[y_dtype])
    torch.cuda.synchronize()
    return y_ws.double().cpu().numpy(), y_na.double().cpu().numpy()


@pytest.mark.parametrize("name,Ts", [("mixtral8x7b_decode", (32, 8)),
                                     ("qwen15_moe_prefill512", (512, 100)),
                                     ("tiny", (64, 3))])
def test_noalloc_matches_workspace_forward(name, Ts):
    cfg = synth.CONFIG_BY_NAME[name]
    layer = synth.make_layer(cfg)
    L = tqio.upload_layer(layer)
    for T in Ts:                       # second call smaller than the first
        need = L.workspace_size(T, cfg.topk)
        say(f"  {name} T={T}: path {L.forward_path(T, cfg.topk)}, workspace {need} bytes "
            f"(scratch {64 << 20})")
        x, ids, g = synth.make_tokens(cfg, T)
        y_ws, y_na = both(L, x, ids, g, cfg.act, "f16")
        assert np.all(np.isfinite(y_na))
        assert_parity(y_na, y_ws, "f16", what=f"noalloc vs workspace {name} T={T}")
        assert np.array_equal(y_na, y_ws), f"{name} T={T}: outputs differ"
    L.close()


def test_noalloc_rejects_beyond_scratch():
    cfg = synth.CONFIG_BY_NAME["tiny"]
    L = tqio.upload_layer(synth.make_layer(cfg))
    T = 65536
    assert L.workspace_size(T, 2) > (64 << 20)
    x = torch.zeros((T, cfg.d_model), dtype=torch.float16, device="cuda")
    ids = torch.zeros((T, 2), dtype=torch.int32, device="cuda")
    g = torch.zeros((T, 2), dtype=torch.float32, device="cuda")
    y = torch.zeros((T, cfg.d_ff), dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TileQError, match="static scratch"):
        L.forward_noalloc(x, T, ids, g, 2, y, tq.TQ_F32)
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0            # nothing ran
    L.close()
