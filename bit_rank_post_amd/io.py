"""Marshalling helpers: host arrays (the stored format of a layer) to device
tensors and uploads through the C ABI.  No arithmetic of the method here."""
from __future__ import annotations

import numpy as np
import torch

from . import TQ_BF16, TQ_F16, TQ_F32, TQ_SINGLE, TQ_SWIGLU, Layer

ACT = {"f16": TQ_F16, "bf16": TQ_BF16}
PROJ_INDEX = {"single": 0, "gate": 0, "up": 1, "down": 2}


def to_device(a: np.ndarray, act: str | None = None, device="cuda"):
    """Copy a host array to the GPU.  bf16 data (uint16 bit patterns) becomes a
    torch.bfloat16 tensor; uint32/uint16 become int32/int16 views."""
    a = np.ascontiguousarray(a)
    if act == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


def upload_proj(L: Layer, which: int, p: dict, stream=None):
    """sigma goes up as stored: float16 arrays as TQ_F16, anything else as f32."""
    act = p["act"]
    sig = np.asarray(p["sigma"])
    sig16 = sig.dtype == np.float16
    sig = sig if sig16 else sig.astype(np.float32)
    dev = dict(U=to_device(p["U"], act) if p["rank"] else None,
               V=to_device(p["V"], act) if p["rank"] else None,
               sigma=to_device(sig.view(np.uint16) if sig16 else sig) if p["rank"] else None,
               codes=to_device(p["codes"]),
               scales=to_device(p["scales"].view(np.uint16)),
               zeros=to_device(p["zeros"].view(np.uint16)))
    L.upload_proj(which, K=p["K"], M=p["M"], N=p["N"], d_in=p["d_in"], d_out=p["d_out"],
                  rank=p["rank"], group=p["group"], tile_of_expert=p["tile_of_expert"],
                  bits=p.get("bits", 2), sigma_dtype=TQ_F16 if sig16 else TQ_F32,
                  stream=stream, **dev)


def upload_layer(layer: dict, stream=None) -> Layer:
    """Upload a layer dict {kind, act, K, d_model, d_ff, proj: {...}, shared}."""
    kind = TQ_SINGLE if layer["kind"] == "single" else TQ_SWIGLU
    L = Layer(kind, ACT[layer["act"]], layer["d_model"], layer["d_ff"], layer["K"])
    for name, p in layer["proj"].items():
        upload_proj(L, PROJ_INDEX[name], p, stream)
    sh = layer.get("shared")
    if sh is not None:
        L.upload_shared_expert(sh["d_ff"], to_device(sh["wg"]), to_device(sh["wu"]),
                               to_device(sh["wd"]), stream)
    return L


def tokens_to_device(x, ids, gates, act):
    return (to_device(x, act), torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
            torch.from_numpy(np.ascontiguousarray(gates, np.float32)).cuda())


def workspace(L: Layer, T: int, topk: int):
    n = L.workspace_size(T, topk)
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
