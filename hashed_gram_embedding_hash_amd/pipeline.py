"""One Engram layer forward pass as a sequence of C-ABI calls.

"Conditional Memory via Scalable Lookup", Figure 1 and sections 2.2-2.4:
compress the raw ids, hash every suffix n-gram into its tables, gather and
concatenate the rows, then gate the memory against each branch's hidden
state and add it to the residual.  This class only owns the parameters and
the intermediate device buffers and issues the calls on one stream
(compression, hashing and the gather as one fused call, then the gate); the
arithmetic is in the HIP kernels.  Passing one W_V tensor for every branch
(section 2.4, Eq. (6)) lets the gate compute W_V e once for all of them.
With fused=True the whole pass is one call, engram_lookup_gate, whose gate kernel
loads the table rows itself (no memory-vector buffer).  Its key tiles are feature-major,
so its results equal the two calls' bit for bit where those take feature-major key tiles
too (decode-sized batches; engram_debug_gate_key_form); for larger batches the two calls
take memory-major key tiles and the logits differ in fp32 rounding order only.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

from . import KEY_NORM_MEMORY, engram_gate_forward, engram_lookup, engram_lookup_gate


class EngramLayer:
    def __init__(self, cmap: torch.Tensor, orders: Sequence[int], heads: int, mult: np.ndarray,
                 tables: Sequence[torch.Tensor], wk: Sequence[torch.Tensor], wv: Sequence[torch.Tensor],
                 gq: Sequence[torch.Tensor], gk: Sequence[torch.Tensor], eps: float = 1e-6,
                 pad_id: Optional[int] = None, key_norm: int = KEY_NORM_MEMORY):
        self.cmap = cmap
        self.orders = tuple(orders)
        self.heads = heads
        self.mult = np.ascontiguousarray(mult, dtype=np.uint64)
        self.tables = list(tables)
        self.rows = np.array([t.shape[0] for t in tables], dtype=np.uint32)
        self.wk, self.wv, self.gq, self.gk = list(wk), list(wv), list(gq), list(gk)
        self.eps = eps
        self.key_norm = key_norm
        # default padding id: one past the largest canonical id
        self.pad_id = int(cmap.max().item()) + 1 if pad_id is None else pad_id
        self._bufs = {}

    @property
    def n_tables(self) -> int:
        return len(self.orders) * self.heads

    def buffers(self, batch: int, seq: int):
        key = (batch, seq)
        if key not in self._bufs:
            dev = self.cmap.device
            n = batch * seq
            w = self.tables[0].shape[1]
            self._bufs[key] = dict(
                ids=torch.empty((batch, seq), dtype=torch.int32, device=dev),
                idx=torch.empty((n, self.n_tables), dtype=torch.int32, device=dev),
                mem=torch.empty((n, self.n_tables * w), dtype=self.tables[0].dtype, device=dev),
            )
        return self._bufs[key]

    def __call__(self, raw: torch.Tensor, h: Sequence[torch.Tensor], out: Optional[Sequence[torch.Tensor]] = None,
                 gate_out: Optional[torch.Tensor] = None, stream=None, fused: bool = False) -> List[torch.Tensor]:
        """raw: int32 [batch, seq]; h: per-branch [batch*seq, d_model]; returns per-branch outputs.
        fused: one engram_lookup_gate call (bf16 tables; nothing but the outputs is stored, so
        the layer's buffers are neither used nor allocated)."""
        batch, seq = raw.shape
        if fused:
            return engram_lookup_gate(raw, self.cmap, self.orders, self.heads, self.mult, self.tables, self.pad_id,
                                      h, self.wk, self.wv, self.gq, self.gk, self.eps, out=out, gate_out=gate_out,
                                      key_norm=self.key_norm, stream=stream)
        b = self.buffers(batch, seq)
        engram_lookup(raw, self.cmap, self.orders, self.heads, self.mult, self.tables, self.pad_id,
                      out=b["mem"], ids_out=b["ids"], idx_out=b["idx"], stream=stream)
        return engram_gate_forward(b["mem"], h, self.wk, self.wv, self.gq, self.gk, self.eps, out=out,
                                   gate_out=gate_out, key_norm=self.key_norm, stream=stream)
