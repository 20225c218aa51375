"""Copy a ``workloads.Inputs`` instance to torch device tensors (plumbing only)."""

import numpy as np


def to_torch(inp, device):
    """Returns a dict with q, k, v (bfloat16 or float32 [B, H, n, d]), global_idx (int32),
    key_pad (uint8) and layout (int32), the last three None when absent."""
    import torch

    def mat(a):
        if inp.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    def opt(a, dt):
        if a is None:
            return None
        h = np.ascontiguousarray(a, dtype=dt)
        return torch.from_numpy(h if h.flags.writeable else h.copy()).to(device)

    return dict(
        q=mat(inp.q), k=mat(inp.k), v=mat(inp.v),
        global_idx=opt(inp.global_idx, np.int32),
        key_pad=opt(inp.key_pad, np.uint8),
        layout=opt(inp.layout, np.int32),
    )
