"""Device and pinned-host buffers for calling the C ABI from PyTorch.

Allocation only: caller-owned classify outputs as torch device tensors, and
pinned host banks from ft_host_alloc exposed as NumPy views.
"""
import numpy as np
import torch

from . import (FtClassifyOut, ft_cache_create, ft_cache_create_layers, ft_cache_destroy, ft_host_alloc,
               ft_host_free, host_array, profile, shape)


class ClassifyBuffers:
    """Caller-owned device arrays of one ft_cache_classify call."""

    def __init__(self, capacity: int, device="cuda"):
        kw = dict(device=device)
        self.capacity = capacity
        self.counts = torch.zeros(4, dtype=torch.int32, **kw)
        self.uniq = torch.full((capacity,), -7, dtype=torch.int32, **kw)
        self.cls = torch.full((capacity,), 255, dtype=torch.uint8, **kw)
        self.slot = torch.full((capacity,), -7, dtype=torch.int32, **kw)
        self.ev_slot = torch.full((capacity,), -7, dtype=torch.int32, **kw)
        self.ev_old = torch.full((capacity,), -7, dtype=torch.int32, **kw)
        self.ev_new = torch.full((capacity,), -7, dtype=torch.int32, **kw)
        self.cpu_ids = torch.full((capacity,), -7, dtype=torch.int32, **kw)
        self.struct = FtClassifyOut(self.counts.data_ptr(), self.uniq.data_ptr(), self.cls.data_ptr(),
                                    self.slot.data_ptr(), self.ev_slot.data_ptr(), self.ev_old.data_ptr(),
                                    self.ev_new.data_ptr(), self.cpu_ids.data_ptr(), capacity)

    def host(self):
        """Valid entries as Python lists (synchronises)."""
        n_uniq, hits, m, q = (int(v) for v in self.counts.cpu())
        return {
            "n_uniq": n_uniq, "hits": hits, "m": m, "q": q,
            "uniq": self.uniq[:n_uniq].cpu().tolist(),
            "cls": self.cls[:n_uniq].cpu().tolist(),
            "slot": self.slot[:n_uniq].cpu().tolist(),
            "ev_slot": self.ev_slot[:q].cpu().tolist(),
            "ev_old": self.ev_old[:q].cpu().tolist(),
            "ev_new": self.ev_new[:q].cpu().tolist(),
            "cpu_ids": self.cpu_ids[:m - q].cpu().tolist(),
        }


class PinnedBank:
    """Pinned, device-mapped host memory holding layer-expert records."""

    def __init__(self, nbytes: int):
        self.nbytes = nbytes
        self.ptr = ft_host_alloc(nbytes)
        self.array = host_array(self.ptr, nbytes)

    def records(self, S: int) -> np.ndarray:
        return self.array[: (self.nbytes // S) * S].reshape(-1, S)

    def close(self):
        if self.ptr:
            ft_host_free(self.ptr)
            self.ptr = 0
            self.array = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class SlotCache:
    """An ft_cache handle with its shape and profile (closed on close()).
    `bank_ptr` is one pinned bank of all layers, or a list of per-layer bank
    addresses (ft_cache_create_layers)."""

    def __init__(self, layers, experts, top_k, d_model, d_ff, fmt, bank_ptr, num_slots, max_tokens,
                 bp_mbps, bh_mbps, max_fetch=-1):
        self.shape = shape(layers, experts, top_k, d_model, d_ff, fmt)
        self.profile = profile(bp_mbps, bh_mbps, max_fetch)
        if isinstance(bank_ptr, (list, tuple)):
            self.handle = ft_cache_create_layers(self.shape, self.profile, list(bank_ptr), num_slots, max_tokens)
        else:
            self.handle = ft_cache_create(self.shape, self.profile, bank_ptr, num_slots, max_tokens)
        self.num_slots = num_slots

    def close(self):
        if self.handle:
            ft_cache_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
