"""Device buffers for one layer's decode step and the decode step itself.

``DecodeStep`` owns (as torch tensors) the page statistics, the selection rows, the
workspaces and the output for a fixed batch geometry, and issues

    decode_step = page_meta_update (tail page) + select_pages + sparse_decode

as one call on one stream; ``step_separate`` issues the three calls one by one. ``dense()`` runs the dense baseline on the same inputs. Nothing here computes:
it sizes buffers and forwards pointers to the C-ABI.
"""
from __future__ import annotations

import numpy as np
import torch

from . import api


def _to_device_bits(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype == "bf16":
        return t.view(torch.int16).to(device).view(torch.bfloat16)
    return t.to(device)


class DecodeStep:
    def __init__(self, q: torch.Tensor, cache: torch.Tensor, block_table: torch.Tensor,
                 seq_lens: torch.Tensor, budgets: torch.Tensor, head_dim_v: int,
                 latent: bool, b_max: int | None = None, v_host: bool = False,
                 kv_host: bool = False):
        """q [B, H_q, D]; cache [2, NB, 16, H_kv, D] (or [1, ...] when ``latent``: V is the
        first ``head_dim_v`` dims of K); block_table [B, max_pages] int32; seq_lens and
        budgets [B] int32. All on the same HIP device. ``v_host`` moves V to pinned host
        memory (the value tier in host DRAM): the attention then reads only the kept
        pages' V rows over the host link. ``kv_host`` moves K as well (the page statistics
        stay in device memory)."""
        self.q, self.cache = q, cache
        self.block_table, self.seq_lens, self.budgets = block_table, seq_lens, budgets
        self.k = cache[0]
        self.v = cache[0][..., :head_dim_v] if latent else cache[1]
        if v_host or kv_host:
            if latent:
                raise ValueError("a latent cache holds V inside K: V cannot move alone")
            host = torch.empty(self.v.shape, dtype=self.v.dtype, pin_memory=True)
            host.copy_(self.v)
            self.v = host
        if kv_host:
            host = torch.empty(self.k.shape, dtype=self.k.dtype, pin_memory=True)
            host.copy_(self.k)
            self.k = host
        self.shape = api.make_shape(q, self.k, self.v, block_table, head_dim_v)
        B, Hq, D = q.shape
        NB, _, Hkv, _ = self.k.shape
        dev = q.device
        if b_max is None:
            b_max = int(budgets.max().item())
        self.b_max = max(2, int(b_max))
        self.scale = 1.0 / float(D) ** 0.5
        cd = 32 if q.dtype == torch.bfloat16 else 16  # dims per 64-byte statistics chunk
        self.meta = torch.empty((NB, Hkv, D // cd, 2, cd), dtype=q.dtype, device=dev)
        self.sel_pages = torch.empty((B, Hkv, self.b_max), dtype=torch.int32, device=dev)
        self.sel_count = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, Hq, head_dim_v), dtype=torch.float32, device=dev)
        self.out_dense = torch.empty_like(self.out)
        sel_ws = api.select_workspace_bytes(self.shape, self.b_max)
        dec_ws = api.decode_workspace_bytes(self.shape, self.b_max)
        den_ws = api.decode_workspace_bytes(self.shape, self.shape.max_pages_per_seq)
        if sel_ws == 0 or dec_ws == 0 or den_ws == 0:
            raise api.PsdError(-2, "workspace query")
        self.ws_select = torch.empty(sel_ws, dtype=torch.uint8, device=dev)
        self.ws_decode = torch.empty(dec_ws, dtype=torch.uint8, device=dev)
        self.ws_dense = torch.empty(den_ws, dtype=torch.uint8, device=dev)
        fused_ws = api.select_sparse_decode_workspace_bytes(self.shape, self.b_max)
        if fused_ws == 0:
            raise api.PsdError(-2, "workspace query")
        self.ws_fused = torch.empty(fused_ws, dtype=torch.uint8, device=dev)
        self.first_page_zero = torch.zeros(B, dtype=torch.int32, device=dev)
        self.ws_coverage = None  # sized on first use of select_coverage

    @classmethod
    def from_arrays(cls, q: np.ndarray, cache: np.ndarray, block_table: np.ndarray,
                    seq_lens: np.ndarray, budgets: np.ndarray, dtype: str, head_dim_v: int,
                    latent: bool, device="cuda", b_max: int | None = None, v_host: bool = False,
                    kv_host: bool = False):
        dev = torch.device(device)
        return cls(_to_device_bits(q, dtype, dev), _to_device_bits(cache, dtype, dev),
                   torch.from_numpy(np.ascontiguousarray(block_table, dtype=np.int32)).to(dev),
                   torch.from_numpy(np.ascontiguousarray(seq_lens, dtype=np.int32)).to(dev),
                   torch.from_numpy(np.ascontiguousarray(budgets, dtype=np.int32)).to(dev),
                   head_dim_v, latent, b_max, v_host, kv_host)

    # -- the calls ------------------------------------------------------------------------
    def build_meta(self, stream=None):
        """Rebuild the statistics of every page (prefill)."""
        api.page_meta_update(self.shape, self.k, self.meta, self.block_table, self.seq_lens,
                             self.first_page_zero, stream)

    def refresh_tail(self, stream=None):
        api.page_meta_update(self.shape, self.k, self.meta, self.block_table, self.seq_lens,
                             None, stream)

    def select(self, stream=None):
        api.select_pages(self.shape, self.q, self.meta, self.block_table, self.seq_lens,
                         self.budgets, self.b_max, self.sel_pages, self.sel_count, self.ws_select,
                         stream)

    def select_score(self, stream=None):
        """First stage of ``select``: page scores and per-chunk candidates."""
        api.select_score(self.shape, self.q, self.meta, self.block_table, self.seq_lens,
                         self.budgets, self.b_max, self.sel_pages, self.sel_count, self.ws_select,
                         stream)

    def select_merge(self, stream=None):
        """Second stage of ``select``: the winners of every unit from the candidates."""
        api.select_merge(self.shape, self.q, self.meta, self.block_table, self.seq_lens,
                         self.budgets, self.b_max, self.sel_pages, self.ws_select, stream)

    def select_coverage(self, coverage: float, stream=None):
        """Adaptive coverage selection into ``sel_pages`` / ``sel_count`` (reads every
        valid K row; the statistics are not used)."""
        if self.ws_coverage is None:
            nbytes = api.select_coverage_workspace_bytes(self.shape)
            if nbytes == 0:
                raise api.PsdError(-2, "psd_select_coverage_workspace_bytes")
            self.ws_coverage = torch.empty(nbytes, dtype=torch.uint8, device=self.q.device)
        api.select_pages_coverage(self.shape, self.q, self.k, self.block_table, self.seq_lens,
                                  coverage, self.scale, self.b_max, self.sel_pages,
                                  self.sel_count, self.ws_coverage, stream)

    def sparse(self, stream=None):
        api.sparse_decode(self.shape, self.q, self.k, self.v, self.block_table, self.seq_lens,
                          self.sel_pages, self.sel_count, self.b_max, self.scale, self.out,
                          self.ws_decode, stream)

    def select_sparse(self, stream=None):
        """``select`` then ``sparse`` as one call (one launch where a workgroup holds a unit)."""
        api.select_sparse_decode(self.shape, self.q, self.meta, self.k, self.v, self.block_table,
                                 self.seq_lens, self.budgets, self.b_max, self.scale,
                                 self.sel_pages, self.sel_count, self.out, self.ws_fused, stream)

    def dense(self, stream=None):
        api.dense_decode(self.shape, self.q, self.k, self.v, self.block_table, self.seq_lens,
                         self.scale, self.out_dense, self.ws_dense, stream)

    def step(self, stream=None):
        """One sparse decode step in one call: tail refresh, selection, attention over the
        kept pages."""
        api.decode_step(self.shape, self.q, self.meta, self.k, self.v, self.block_table,
                        self.seq_lens, self.budgets, self.b_max, self.scale, self.sel_pages,
                        self.sel_count, self.out, self.ws_fused, stream)

    def step_noalloc(self, stream=None):
        """The same step with the library's static scratch instead of a workspace."""
        api.decode_step_noalloc(self.shape, self.q, self.meta, self.k, self.v, self.block_table,
                                self.seq_lens, self.budgets, self.b_max, self.scale,
                                self.sel_pages, self.sel_count, self.out, stream)

    def walk(self, kind: int, stream=None):
        """Diagnostic: the step's reads with no arithmetic (0: the kept pages' K and V rows
        of the last selection; 1: every candidate page's statistics record); the XOR of
        each unit's words lands in ``walk_checksum`` [B * H_kv]."""
        if getattr(self, "walk_checksum", None) is None:
            self.walk_checksum = torch.zeros(self.sel_count.numel(), dtype=torch.int32,
                                             device=self.q.device)
        api.diag_walk(self.shape, kind, self.k, self.v, self.meta, self.block_table,
                      self.seq_lens, self.sel_pages, self.sel_count, self.b_max,
                      self.walk_checksum, stream)

    # -- value tier: V in (pinned host) memory, a resident hot buffer in device memory ------
    def enable_tier(self, slots: int, kv: bool = False):
        """Keep up to ``slots`` (block, KV head) V slices resident in a device hot buffer;
        each tiered step copies only the kept slices that are not resident (from ``v``,
        pinned host memory when the step was built with ``v_host``). With ``kv`` (the KV
        tier) each resident slice holds its K rows too, in ``tier_hot_k``."""
        dev = self.q.device
        B, Hkv = self.sel_count.shape
        dv = self.v.shape[-1]
        self.tier_kv = bool(kv)
        self.tier_hot_k = (torch.empty((slots, 16, self.k.shape[-1]), dtype=self.q.dtype,
                                       device=dev) if kv and slots > 0 else None)
        st_bytes = api.value_tier_state_bytes(self.shape, slots)
        ws_bytes = api.value_tier_workspace_bytes(self.shape, self.b_max, slots)
        if st_bytes == 0 or ws_bytes == 0:
            raise api.PsdError(-2, "value tier (GQA shapes with D == D_v in {64, 128})")
        self.tier_slots = int(slots)
        self.tier_hot = (torch.empty((slots, 16, dv), dtype=self.q.dtype, device=dev)
                         if slots > 0 else None)
        self.tier_state = torch.empty(st_bytes, dtype=torch.uint8, device=dev)
        self.tier_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        self.tier_vslot = torch.empty((B, Hkv, self.b_max), dtype=torch.int32, device=dev)
        self.tier_stats = torch.zeros(4, dtype=torch.int64, device=dev)
        self.tier_step = 0
        api.value_tier_reset(self.shape, self.tier_slots, self.tier_state)

    def tier_stage(self, stream=None):
        """Slots for this step's kept V slices (after ``select``); copies the missed ones."""
        self.tier_step += 1
        if self.tier_kv:
            api.kv_tier_stage(self.shape, self.k, self.v, self.tier_hot_k, self.tier_hot,
                              self.tier_state, self.tier_slots, self.tier_step, self.block_table,
                              self.seq_lens, self.sel_pages, self.sel_count, self.b_max,
                              self.tier_vslot, self.tier_stats, self.tier_ws, stream)
            return
        api.value_tier_stage(self.shape, self.v, self.tier_hot, self.tier_state, self.tier_slots,
                             self.tier_step, self.block_table, self.seq_lens, self.sel_pages,
                             self.sel_count, self.b_max, self.tier_vslot, self.tier_stats,
                             self.tier_ws, stream)

    def sparse_tiered(self, stream=None):
        if self.tier_kv:
            api.sparse_decode_kv_tiered(self.shape, self.q, self.k, self.v, self.tier_hot_k,
                                        self.tier_hot, self.tier_vslot, self.block_table,
                                        self.seq_lens, self.sel_pages, self.sel_count,
                                        self.b_max, self.scale, self.out, self.ws_decode, stream)
            return
        api.sparse_decode_tiered(self.shape, self.q, self.k, self.v, self.tier_hot,
                                 self.tier_vslot, self.block_table, self.seq_lens,
                                 self.sel_pages, self.sel_count, self.b_max, self.scale,
                                 self.out, self.ws_decode, stream)

    def step_tiered(self, stream=None):
        """One decode step with V in the value tier: tail refresh, selection, staging of the
        kept slices, attention."""
        self.refresh_tail(stream)
        self.select(stream)
        self.tier_stage(stream)
        self.sparse_tiered(stream)

    def tier_counts(self) -> dict:
        """The last stage's counts (synchronises): hits, misses (entries), slices copied,
        entries read from the host pool."""
        h, m, c, o = (int(x) for x in self.tier_stats.cpu().tolist())
        return {"hits": h, "misses": m, "copied": c, "from_host": o}

    def step_separate(self, stream=None):
        """The same step as three calls: tail refresh, selection, attention."""
        self.refresh_tail(stream)
        self.select(stream)
        self.sparse(stream)
