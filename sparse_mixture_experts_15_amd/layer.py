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
        """y = the layer on x, enqueued on `stream` (default: the current
        stream), the shared expert on `aux_stream` when given.

        The library needs every buffer ready on `stream`.  The workspace and
        a new y come from torch's caching allocator on the current stream,
        and the inputs are normally produced there, so a different `stream`
        first waits for the current one; the workspace and y are then marked
        as used by `stream` and `aux_stream`, so the allocator does not hand
        their memory out again while that work is pending."""
        cur = torch.cuda.current_stream(x.device)
        if y is None:
            y = torch.empty(x.shape, dtype=B._odt(self.desc), device=x.device)
        s = cur if stream is None else stream
        if s != cur:
            s.wait_stream(cur)
        B.moe_forward(self.handle, self.desc, x, W_r, bias, W1, b1, W2, b2, Wsh_gu, Wsh_dn, y,
                      self.ws, stream=s, aux_stream=aux_stream)
        if torch.cuda.is_current_stream_capturing():
            return y   # a captured graph keeps its memory for its own lifetime
        for st in (s, aux_stream):
            if st is not None and st != cur:
                self.ws.record_stream(st)
                y.record_stream(st)
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
