"""Paged KV-cache buffers for the megakernel (device memory via torch).

Pool layouts (bf16): keys [n_layers][n_pages][n_kv_heads][16][head_dim],
values [n_layers][n_pages][n_kv_heads][head_dim][16] (transposed within a
page); the page table (int32 [max_batch][max_pages_per_seq]) maps (slot,
position // 16) to a pool page.  Pages are handed out from a seeded random permutation of the pool
("shuffled page tables").
"""
from __future__ import annotations

import torch

PAGE = 16


class PagedKV:
    def __init__(self, model: dict, max_batch: int, max_pages_per_seq: int,
                 n_pages: int | None = None, device="cuda", seed: int = 2,
                 shuffle: bool = True):
        L, nkv, hd = model["n_layers"], model["n_kv_heads"], model["head_dim"]
        self.model, self.B, self.maxp = model, max_batch, max_pages_per_seq
        self.n_pages = n_pages if n_pages is not None else max_batch * max_pages_per_seq
        self.k_pool = torch.zeros((L, self.n_pages, nkv, PAGE, hd), dtype=torch.bfloat16,
                                  device=device)
        self.v_pool = torch.zeros((L, self.n_pages, nkv, hd, PAGE), dtype=torch.bfloat16,
                                  device=device)
        g = torch.Generator()
        g.manual_seed(int(seed))
        order = (torch.randperm(self.n_pages, generator=g) if shuffle
                 else torch.arange(self.n_pages))
        self.free_pages = [int(p) for p in order]
        self.table_host = torch.full((max_batch, max_pages_per_seq), -1, dtype=torch.int32)
        self.page_table = self.table_host.to(device)
        self.device = device

    def assign(self, slot: int, n_tokens: int, upload: bool = True) -> bool:
        """Give slot enough pages for n_tokens positions (keeps existing ones).
        Returns whether a page was added; `upload=False` leaves the device
        copy of the table to a later `upload()`."""
        need = (n_tokens + PAGE - 1) // PAGE
        if need > self.maxp:
            raise ValueError("sequence longer than max_pages_per_seq * 16")
        row = self.table_host[slot]
        added = False
        for j in range(need):
            if int(row[j]) < 0:
                if not self.free_pages:
                    raise RuntimeError("page pool exhausted")
                row[j] = self.free_pages.pop()
                added = True
        if upload and added:
            self.upload()
        return added

    def release(self, slot: int, upload: bool = True):
        """Return the slot's pages to the pool (the slot retires)."""
        row = self.table_host[slot]
        for j in range(self.maxp):
            if int(row[j]) >= 0:
                self.free_pages.append(int(row[j]))
                row[j] = -1
        if upload:
            self.upload()

    def upload(self):
        self.page_table.copy_(self.table_host)

    def write_tokens(self, slot: int, K, V, start: int = 0):
        """Copy keys/values [L, n, nkv, hd] (bf16) of positions start..start+n
        into the slot's pages."""
        n = K.shape[1]
        self.assign(slot, start + n)
        pos = torch.arange(start, start + n)
        pages = self.table_host[slot, pos // PAGE].long().to(self.k_pool.device)
        slots = (pos % PAGE).to(self.k_pool.device)
        # advanced indices (pages, slots) put the token axis first
        self.k_pool[:, pages, :, slots, :] = K.to(self.k_pool.device).permute(1, 0, 2, 3)
        self.v_pool[:, pages, :, :, slots] = V.to(self.v_pool.device).permute(1, 0, 2, 3)

    def read_tokens(self, slot: int, n: int):
        """Keys/values of positions 0..n-1 of a slot: bf16 [L, n, nkv, hd]."""
        pos = torch.arange(n)
        pages = self.table_host[slot, pos // PAGE].long().to(self.k_pool.device)
        slots = (pos % PAGE).to(self.k_pool.device)
        k = self.k_pool[:, pages, :, slots, :].permute(1, 0, 2, 3)
        v = self.v_pool[:, pages, :, :, slots].permute(1, 0, 2, 3)
        return k, v
