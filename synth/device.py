"""Placement of generated inputs in device memory (torch is plumbing here).

bf16 values travel as their bit patterns and are viewed as torch.bfloat16 on
the device; fp32 values are copied as they are.
"""
import numpy as np


def tensor(x, dtype, device):
    import torch
    if x is None:
        return None
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device)


def weights_to_device(inp, device):
    wd = inp.cfg.weight_dtype
    out = {k: tensor(getattr(inp, k), wd, device) for k in ("wq", "u", "v", "w1", "w2")}
    for src, dst in (("gamma", "h_gamma"), ("b1", "b1"), ("b2", "b2")):
        if getattr(inp, src) is not None:
            out[dst] = tensor(getattr(inp, src), wd, device)
    return out


def to_device(inp, device):
    """All inputs of one call as device tensors (dict)."""
    import torch
    c = inp.cfg
    w = weights_to_device(inp, device)
    return {
        "states": tensor(inp.buf, c.state_dtype, device),
        "accept_idx": torch.from_numpy(np.ascontiguousarray(inp.accept_idx, dtype=np.int32)).to(device),
        "h": tensor(inp.h, c.act_dtype, device),
        "weights": w,
    }


def torch_dtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_numpy_bits(t, dtype):
    """Device tensor -> numpy (bf16 as uint16 bit patterns, fp32 as float32)."""
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().astype(np.float32, copy=False)
