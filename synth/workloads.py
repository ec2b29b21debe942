"""Seeded synthetic paged-KV decode workloads.

This module only builds inputs: queries, a paged KV cache in the vLLM block layout
``[2, num_blocks, 16, H_kv, D]`` with a block table, sequence lengths and page budgets.
It holds none of the method's arithmetic (no page statistics, no page scores, no
selection, no attention). Both the fp64 oracle side and the GPU side receive the same
arrays from here.

Recipe (the pages describe the cache layout and the 16-token page on the EntmaxKV
README, introduction; the page-clustered key distribution, the needles and the sizes
are the workload definitions this library is measured on):

* keys of page p, KV head g, dim d = mu[p, g, d] + eps[p, t, g, d] with
  mu ~ N(0, mean_std^2) shared by the page's 16 tokens and eps ~ N(0, noise_std^2);
* values and queries ~ N(0, 1);
* "needle" pages: for each (sequence, KV head) ``needles`` distinct logical pages are
  drawn uniformly from 1..n-2; needle j adds 3 * q_h / |q_h| to every valid key of
  that page, where h = g * G + (j mod G) cycles over the GQA group;
* values are drawn in fp32 and rounded to bf16 with round-to-nearest-even (fp32
  workloads keep them as drawn);
* slots of the tail page past the sequence length hold NaN in K and V, so any use of
  an unwritten slot shows up;
* the physical block pool has sum(n_s) blocks; the block table is a seeded random
  permutation of it; table entries past a sequence's last page are 0;
* budgets are either an absolute page count or floor(n * percent / 100), clamped
  to [min(n, 2), n], always counting the sink and the tail page.

Random streams are addressed, not sequential: every purpose (lengths, permutation,
queries, needles, and each (sequence, page-chunk) of the cache) draws from its own
``numpy.random.SeedSequence(seed, spawn_key=...)`` child, so the arrays do not depend
on thread scheduling.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

PAGE = 16
_CHUNK_PAGES = 256  # pages drawn per random stream (fixes the draw order)

_K_LENS, _K_PERM, _K_Q, _K_NEEDLE, _K_CACHE = 1, 2, 3, 4, 5


@dataclass(frozen=True)
class WorkloadSpec:
    """Shape and distribution of one synthetic decode step."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    head_dim_v: int
    dtype: str  # "f32" or "bf16"; q, K and V share it
    seq_lens: tuple = ()  # fixed lengths (len == batch), or empty with len_range
    len_range: tuple = ()  # (lo, hi) inclusive, uniform integers
    budget_pages: int = 0  # absolute budget (pages, incl. sink + tail) when > 0
    budget_percent: int = 0  # otherwise floor(n * percent / 100)
    needles: int = 0  # needle pages per (sequence, KV head)
    mean_std: float = 0.5
    noise_std: float = 0.5
    latent: bool = False  # one latent head; V = first head_dim_v dims of K
    max_len: int = 0  # block-table width in tokens (0: the largest length)
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


# The five measured workloads.
SPECS = {
    "tiny": WorkloadSpec(
        name="tiny", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64, head_dim_v=64,
        dtype="f32", seq_lens=(1024,), budget_pages=8, needles=2),
    "gqa8b_32k": WorkloadSpec(
        name="gqa8b_32k", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        head_dim_v=128, dtype="bf16", seq_lens=(32768,), budget_percent=5, needles=8),
    "ragged_b32_32k": WorkloadSpec(
        name="ragged_b32_32k", batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
        head_dim_v=128, dtype="bf16", len_range=(16384, 32768), budget_percent=5,
        needles=8, max_len=32768),
    "long_1m": WorkloadSpec(
        name="long_1m", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        head_dim_v=128, dtype="bf16", seq_lens=(1048576,), budget_pages=128, needles=16),
    "mla_64k": WorkloadSpec(
        name="mla_64k", batch=16, num_q_heads=128, num_kv_heads=1, head_dim=576,
        head_dim_v=512, dtype="bf16", seq_lens=(65536,) * 16, budget_percent=5,
        needles=8, mean_std=math.sqrt(0.5), noise_std=math.sqrt(0.5), latent=True),
}

CONFIG_ORDER = ["tiny", "gqa8b_32k", "ragged_b32_32k", "long_1m", "mla_64k"]


def num_pages(length: int) -> int:
    return (int(length) + PAGE - 1) // PAGE


def budget_for(spec: WorkloadSpec, n: int) -> int:
    """Pages attended for a sequence of n pages (sink and tail included)."""
    if spec.budget_pages > 0:
        b = spec.budget_pages
    else:
        b = (n * spec.budget_percent) // 100
    return max(min(n, 2), min(b, n))


@dataclass
class Workload:
    """One decode step's inputs, as raw arrays in the dtype they are stored in.

    ``q``: [B, H_q, D] (uint16 bf16 bits, or float32); ``cache``: [P, NB, 16, H_kv, D]
    with P = 2 planes (K, V) or P = 1 for a latent cache whose V is the first
    ``head_dim_v`` dims of K; ``block_table``: [B, max_pages] int32; ``seq_lens``,
    ``budgets``: [B] int32; ``needle_pages``: [B, H_kv, needles] int32 logical pages.
    """

    spec: WorkloadSpec
    q: np.ndarray
    cache: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    budgets: np.ndarray
    needle_pages: np.ndarray
    scale: float
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return self.cache.shape[1]

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]

    @property
    def k_raw(self) -> np.ndarray:
        return self.cache[0]

    @property
    def v_raw(self) -> np.ndarray:
        """V as stored: [NB, 16, H_kv, D_v] (a view; strided for a latent cache)."""
        if self.spec.latent:
            return self.cache[0][..., : self.spec.head_dim_v]
        return self.cache[1]


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of an array stored as bf16 bits or float32."""
    if dtype == "bf16":
        return bf16_bits_to_f32(raw).astype(np.float64)
    return raw.astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bits, nearest-even; NaN maps to the quiet NaN 0x7FC0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).copy()
    nan = np.isnan(x)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (u >> np.uint32(16)).astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(key)))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_workload(spec: WorkloadSpec | str, seed: int | None = None) -> Workload:
    """Build the seeded synthetic inputs of ``spec`` (name or spec object)."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    if seed is not None:
        spec = replace(spec, seed=seed)
    s0 = spec.seed
    B, Hq, Hkv, D, Dv = (spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                         spec.head_dim_v)
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv

    if spec.seq_lens:
        lens = np.asarray(spec.seq_lens, dtype=np.int64)
        assert lens.shape == (B,)
    else:
        lo, hi = spec.len_range
        lens = _rng(s0, _K_LENS).integers(lo, hi, endpoint=True, size=B)
    n_pages = np.array([num_pages(x) for x in lens], dtype=np.int64)
    max_len = spec.max_len or int(lens.max())
    max_pages = num_pages(max_len)
    if int(n_pages.max()) > max_pages:
        raise ValueError("a sequence exceeds max_len")

    NB = int(n_pages.sum())
    perm = _rng(s0, _K_PERM).permutation(NB).astype(np.int32)
    block_table = np.zeros((B, max_pages), dtype=np.int32)
    starts = np.concatenate([[0], np.cumsum(n_pages)[:-1]])
    for s in range(B):
        block_table[s, : n_pages[s]] = perm[starts[s]: starts[s] + n_pages[s]]

    # Queries, drawn in fp32 and stored in the workload dtype.
    q32 = _rng(s0, _K_Q).standard_normal((B, Hq, D), dtype=np.float32)
    if spec.dtype == "bf16":
        q_raw = f32_to_bf16_bits(q32)
    else:
        q_raw = q32
    q64 = to_f64(q_raw, spec.dtype)
    qn = (3.0 * q64 / np.linalg.norm(q64, axis=-1, keepdims=True)).astype(np.float32)

    # Needle pages per (sequence, KV head): distinct, uniform over 1..n-2.
    needle_pages = np.full((B, Hkv, spec.needles), -1, dtype=np.int32)
    nrng = _rng(s0, _K_NEEDLE)
    for s in range(B):
        inner = int(n_pages[s]) - 2
        for g in range(Hkv):
            if spec.needles and inner > 0:
                k = min(spec.needles, inner)
                needle_pages[s, g, :k] = 1 + nrng.choice(inner, size=k, replace=False)

    planes = 1 if spec.latent else 2
    if spec.latent and Hkv != 1:
        raise ValueError("a latent cache has one KV head")
    store_dtype = np.uint16 if spec.dtype == "bf16" else np.float32
    cache = np.empty((planes, NB, PAGE, Hkv, D), dtype=store_dtype)

    # Needle offsets as a dense per-page add: (s, page) -> list of (g, vector).
    needle_add = {}
    for s in range(B):
        for g in range(Hkv):
            for j, p in enumerate(needle_pages[s, g]):
                if p < 0:
                    continue
                h = g * G + (j % G)
                needle_add.setdefault((s, int(p)), []).append((g, qn[s, h]))

    def fill(job):
        s, c = job
        L = int(lens[s])
        n = int(n_pages[s])
        p0 = c * _CHUNK_PAGES
        p1 = min(n, p0 + _CHUNK_PAGES)
        P = p1 - p0
        rng = _rng(s0, _K_CACHE, s, c)
        mean = rng.standard_normal((P, 1, Hkv, D), dtype=np.float32)
        mean *= np.float32(spec.mean_std)
        k = rng.standard_normal((P, PAGE, Hkv, D), dtype=np.float32)
        k *= np.float32(spec.noise_std)
        k += mean
        del mean
        for p in range(p0, p1):
            for g, vec in needle_add.get((s, p), ()):
                k[p - p0, :, g, :] += vec
        v = None
        if not spec.latent:
            v = rng.standard_normal((P, PAGE, Hkv, Dv), dtype=np.float32)
        # Slots past the sequence length are never written by a real decoder.
        if p1 == n and L % PAGE:
            k[P - 1, L % PAGE:] = np.nan
            if v is not None:
                v[P - 1, L % PAGE:] = np.nan
        blocks = block_table[s, p0:p1]
        if spec.dtype == "bf16":
            cache[0, blocks] = f32_to_bf16_bits(k)
            if v is not None:
                cache[1, blocks] = f32_to_bf16_bits(v)
        else:
            cache[0, blocks] = k
            if v is not None:
                cache[1, blocks] = v

    jobs = [(s, c) for s in range(B)
            for c in range((int(n_pages[s]) + _CHUNK_PAGES - 1) // _CHUNK_PAGES)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, jobs))

    budgets = np.array([budget_for(spec, int(n)) for n in n_pages], dtype=np.int32)
    return Workload(spec=spec, q=q_raw, cache=cache, block_table=block_table,
                    seq_lens=lens.astype(np.int32), budgets=budgets,
                    needle_pages=needle_pages, scale=1.0 / math.sqrt(D))


def small_spec(name: str = "small", **kw) -> WorkloadSpec:
    """A small GQA workload for parity tests; keyword arguments override fields."""
    base = WorkloadSpec(name=name, batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        head_dim_v=128, dtype="bf16", seq_lens=(1000, 37, 4096),
                        budget_percent=5, needles=4, max_len=4096)
    return replace(base, **kw)


class F64View:
    """Lazily decoded float64 view of a raw cache plane, indexable by block ids."""

    def __init__(self, raw: np.ndarray, dtype: str):
        self.raw = raw
        self.dtype = dtype

    def __getitem__(self, idx):
        return to_f64(self.raw[idx], self.dtype)


def oracle_inputs(w: Workload) -> dict:
    """The workload as float64 arrays / lazy views, in the form the oracle takes."""
    return dict(q=to_f64(w.q, w.spec.dtype), k_cache=F64View(w.k_raw, w.spec.dtype),
                v_cache=F64View(w.v_raw, w.spec.dtype), block_table=w.block_table,
                seq_lens=w.seq_lens, budgets=w.budgets, scale=w.scale,
                head_dim_v=w.spec.head_dim_v, num_kv_heads=w.spec.num_kv_heads)
