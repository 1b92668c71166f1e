"""Caller-side buffers for an offloaded MoE stack: pinned host rows per
layer, device slot banks, per-layer shared experts, and the C cache over
them.  Allocation and marshalling only (torch owns the memory); every step
of the layer runs in the HIP library."""
from __future__ import annotations

import numpy as np
import torch

from . import (MOE_FMT_BF16, make_pool, make_shared, moe_bank_row_bytes, moe_cache_create,
               moe_cache_destroy, moe_layer_decode, moe_layer_decode_hybrid)


def pinned(a: np.ndarray) -> torch.Tensor:
    t = torch.empty(a.shape, dtype=torch.uint8, pin_memory=True)
    t.numpy()[...] = a
    return t


class SlotCacheLayers:
    """host_rows[l]: list over banks of uint8 arrays [E, row_bytes] (numpy,
    copied into pinned memory) or pinned uint8 tensors (used as given).
    shared[l]: (w13 [2F*H] u16, w2 [H*F] u16, gate [H] u16) numpy or None."""

    def __init__(self, *, layers, experts, slots, hidden, ffn, fmt=MOE_FMT_BF16, host_rows,
                 shared=None, max_tokens=1, max_top_k=8, overlap=1, one_call_width=256,
                 query_width=128, max_routes=None, gather_workgroups=0, device="cuda"):
        self.L, self.E, self.S, self.H, self.F, self.fmt = layers, experts, slots, hidden, ffn, fmt
        self.device = torch.device(device)
        self.row_bytes = moe_bank_row_bytes(fmt, hidden, ffn)
        self.host = []
        for l in range(layers):
            banks = []
            for b, a in enumerate(host_rows[l]):
                t = a if isinstance(a, torch.Tensor) else pinned(np.ascontiguousarray(a))
                assert t.is_pinned() and t.shape == (experts, self.row_bytes[b])
                banks.append(t)
            self.host.append(banks)
        self.slot_banks = [torch.zeros((slots, r), dtype=torch.uint8, device=self.device)
                           for r in self.row_bytes]
        self.shared = None
        if shared is not None:
            self.shared = []
            for l in range(layers):
                if shared[l] is None:
                    self.shared.append(None)
                    continue
                w13, w2, gate = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.device)
                                 for a in shared[l])
                self.shared.append(make_shared(w13, w2, gate, ffn=w2.numel() // hidden))
        if max_routes is None:
            max_routes = max(max_tokens * max_top_k, 1)
        self.cache = moe_cache_create(
            num_layers=layers, num_experts=experts, num_slots=slots, hidden=hidden, ffn=ffn,
            weight_format=fmt, one_call_width=one_call_width, query_width=query_width,
            max_routes=max_routes, max_tokens=max_tokens, max_top_k=max_top_k, overlap=overlap,
            gather_workgroups=gather_workgroups, host_banks=self.host, slot_banks=self.slot_banks)

    def _shared(self, layer):
        # the library checks the layer; an out-of-range one gets no shared expert here
        if self.shared is None or not 0 <= layer < len(self.shared):
            return None
        return self.shared[layer]

    def decode(self, layer, x, logits, K, out, ids_out=None, w_out=None, max_fetch=-1, stream=None):
        sh = self._shared(layer)
        moe_layer_decode(self.cache, layer, x, logits, K, out, shared=sh, max_fetch=max_fetch,
                         ids_out=ids_out, w_out=w_out, stream=stream)

    def decode_hybrid(self, layer, x, logits, K, out, ids_out=None, w_out=None, max_fetch=-1,
                      stream=None):
        sh = self._shared(layer)
        moe_layer_decode_hybrid(self.cache, layer, x, logits, K, out, shared=sh, max_fetch=max_fetch,
                                ids_out=ids_out, w_out=w_out, stream=stream)

    def streamed_pool(self, layer):
        """The whole layer's experts copied to device memory, rows = expert
        ids: the non-cached reference layer for the routed kernels."""
        banks = [h.to(self.device) for h in self.host[layer]]
        return make_pool(self.fmt, self.H, self.F, self.E, banks)

    def close(self):
        if self.cache is not None:
            moe_cache_destroy(self.cache)
        self.cache = None
        # drop the pinned host store and the slot banks with the cache
        self.host = []
        self.slot_banks = []
        self.shared = None
