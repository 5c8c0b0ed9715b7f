"""A small owner object for one layer shape: a library handle plus a
device workspace sized for ``moe_forward`` (and every stage call)."""
from __future__ import annotations

import torch

from . import binding as B


class MoELayer:
    def __init__(self, desc: B.moe_desc, device: int = 0):
        self.desc = desc
        self.device = device
        self.handle = B.moe_create(device)
        nbytes = B.moe_workspace_size(desc)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=f"cuda:{device}")

    def forward(self, x, W_r, bias, W1, b1, W2, b2, Wsh_gu=None, Wsh_dn=None, y=None,
                stream=None, aux_stream=None):
        if y is None:
            y = torch.empty(x.shape, dtype=B._odt(self.desc), device=x.device)
        B.moe_forward(self.handle, self.desc, x, W_r, bias, W1, b1, W2, b2, Wsh_gu, Wsh_dn, y,
                      self.ws, stream=stream, aux_stream=aux_stream)
        return y

    def close(self):
        if self.handle is not None:
            B.moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
