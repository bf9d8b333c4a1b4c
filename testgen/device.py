"""Copy generated inputs to the GPU as torch tensors (plumbing only).

bf16 tensors keep their exact bit patterns (uint16 -> torch.bfloat16 view).
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np


def tensor(a, bf16: bool, device="cuda"):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if bf16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def upload(inp, device="cuda") -> SimpleNamespace:
    import torch
    cfg = inp.cfg
    bf = cfg.bf16
    ns = SimpleNamespace(cfg=cfg)
    ns.parent = torch.from_numpy(np.ascontiguousarray(inp.parent, np.int32)).to(device)
    ns.path = torch.from_numpy(np.ascontiguousarray(inp.path, np.int32)).to(device)
    ns.path_len = torch.from_numpy(np.ascontiguousarray(inp.path_len, np.int32)).to(device)
    for k in ("x", "B", "C", "dt_raw", "window", "z"):
        setattr(ns, k, tensor(getattr(inp, k), bf, device))
    ns.state = tensor(inp.state, bool(getattr(cfg, "state_bf16", False)), device)
    for k in ("A", "D", "dt_bias", "conv_w", "conv_b"):
        setattr(ns, k, tensor(getattr(inp, k), False, device))
    return ns
