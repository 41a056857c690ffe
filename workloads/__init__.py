"""Seeded synthetic inputs for paged-decode attention.

This module only draws numbers and lays them out in memory: it holds none of
the attention arithmetic, so the FP64 oracle (``oracle/``) and the HIP path
(``paged_decode_attention_splitk_amd``) can both be fed from it without
sharing any code with each other.

Recipe (the same for every workload):

1. ``rng = numpy.random.default_rng(seed)``.
2. Sequence lengths: a fixed list, or ``rng.integers(lo, hi, n, endpoint=True)``
   (inclusive integer uniform), then any forced lengths are written in.
3. Block placement: every sequence needs ``ceil(L / block_size)`` blocks; the
   pool holds their sum (or a fixed count); ``rng.permutation(pool_blocks)``
   hands them out in sequence order, so block tables are a shuffle of the pool.
4. Queries: ``rng.standard_normal((num_seqs, num_q_heads, head_dim), float32)``.
5. K and V of sequence ``s`` come from ``default_rng([seed, s])``: one
   ``standard_normal`` draw of shape ``(blocks, block_size, num_kv_heads,
   head_dim)`` for K, then one for V.  A sequence can therefore be regenerated
   on its own.
6. FP32 -> BF16 by round-to-nearest-even on the bit pattern (NaN kept NaN).
7. Token slots past the end of a sequence, and pool blocks no sequence owns,
   hold a quiet-NaN canary in correctness runs (``canary=True``) and zeros
   otherwise, so a kernel that reads masked memory into its arithmetic shows
   up as NaN.  Block-table entries past a sequence's last block are -1.

All arrays are numpy; BF16 data is held as ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 values to BF16 (nearest, ties to even) and return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = BF16_QNAN
    return out


E4M3_QNAN = np.uint8(0x7F)


def _e4m3_magnitudes() -> np.ndarray:
    """The 127 non-negative finite values of the OCP FP8 E4M3 ("fn") format,
    indexed by their 7-bit code (sign clear): exponent bias 7, 3 mantissa bits,
    subnormals at exponent field 0, code 0x7F reserved for NaN."""
    codes = np.arange(127)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7))


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round values to OCP FP8 E4M3 (nearest, ties to the even code), with
    magnitudes past the largest finite value (448) saturating to it; NaN
    becomes the NaN code.  An input-generation helper (quantising synthetic
    data); it decodes nothing for either side."""
    x = np.asarray(x, dtype=np.float64)
    mags = _e4m3_magnitudes()
    a = np.minimum(np.abs(x), mags[-1])
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - mags[lo], mags[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code |= np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))
    code[np.isnan(x)] = E4M3_QNAN
    return code


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to FP32 (exact).  A convenience for callers
    that want to look at generated data; the oracle decodes on its own."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------
# Workload definitions (shapes, length mixes, seeds)
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    seq_lens: tuple | None = None          # fixed lengths, or None to draw
    len_range: tuple | None = None         # (lo, hi) inclusive
    forced: tuple = ()                     # ((index, length), ...)
    pool_blocks: int | None = None         # fixed pool size (else = total needed)
    layout: str = "paged"                  # "paged", "scratch" or "prefill"
    tile_capacity: int = 0                 # tiled API only
    q_len: int = 0                         # prefill only: query rows
    q_offset: int = 0                      # prefill only: position of query row 0
    description: str = ""


WORKLOADS = {
    "tiny": Workload(
        name="tiny", seed=0, num_seqs=2, num_q_heads=8, num_kv_heads=2,
        head_dim=128, block_size=16, seq_lens=(37, 100), pool_blocks=32,
        description="2 seqs, lengths 37 and 100, 8 q / 2 kv heads, D 128, "
                    "block 16, pool of 32 blocks, num_splits 1 and pinned 4"),
    "batch": Workload(
        name="batch", seed=1, num_seqs=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, len_range=(512, 4096),
        description="32 seqs, lengths U[512, 4096], 32 q / 8 kv heads, D 128, "
                    "block 16, shuffled pool sized to the context, Auto on 256 CUs"),
    "long": Workload(
        name="long", seed=2, num_seqs=1, num_q_heads=24, num_kv_heads=4,
        head_dim=128, block_size=16, seq_lens=(131072,),
        description="1 seq of 131072 tokens, 24 q / 4 kv heads, D 128, block 16, "
                    "Auto clamped to the split ceiling"),
    "packed": Workload(
        name="packed", seed=3, num_seqs=64, num_q_heads=32, num_kv_heads=4,
        head_dim=256, block_size=16, len_range=(1024, 8192),
        description="64 seqs, lengths U[1024, 8192], 32 q / 4 kv heads (pack "
                    "width 8), D 256, block 16"),
    "tiled": Workload(
        name="tiled", seed=4, num_seqs=128, num_q_heads=16, num_kv_heads=4,
        head_dim=256, block_size=32, len_range=(0, 16384),
        forced=((0, 0), (1, 1), (2, 31), (3, 32), (4, 2048), (5, 16384), (127, 0)),
        layout="scratch", tile_capacity=64,
        description="128 seqs, lengths U[0, 16384] plus forced edge lengths, "
                    "16 q / 4 kv heads, D 256, block 32, scratch-pool layout, "
                    "64 blocks per tile"),
    # causal prefill of one sequence (the prefill page's 128-row kernel shape:
    # head dim 256, GQA, paged BF16 cache)
    "prefill": Workload(
        name="prefill", seed=5, num_seqs=1, num_q_heads=32, num_kv_heads=4,
        head_dim=256, block_size=16, seq_lens=(4096,), layout="prefill",
        q_len=4096, q_offset=0,
        description="causal prefill of one 4096-token sequence, 32 q / 4 kv heads, "
                    "D 256, block 16, shuffled pool"),
    "prefill_chunk": Workload(
        name="prefill_chunk", seed=6, num_seqs=1, num_q_heads=32, num_kv_heads=4,
        head_dim=256, block_size=16, seq_lens=(8192,), layout="prefill",
        q_len=2048, q_offset=6144,
        description="chunked causal prefill: the last 2048 of 8192 tokens, 32 q / "
                    "4 kv heads, D 256, block 16, shuffled pool"),
}


def draw_seq_lens(w: Workload) -> np.ndarray:
    rng = np.random.default_rng(w.seed)
    return _draw_lens(w, rng)


def _draw_lens(w: Workload, rng) -> np.ndarray:
    if w.seq_lens is not None:
        lens = np.array(w.seq_lens, dtype=np.int64)
    else:
        lo, hi = w.len_range
        lens = rng.integers(lo, hi, w.num_seqs, endpoint=True).astype(np.int64)
    for idx, L in w.forced:
        lens[idx] = L
    assert lens.shape == (w.num_seqs,)
    return lens


# --------------------------------------------------------------------------
# Generated inputs
# --------------------------------------------------------------------------

@dataclasses.dataclass
class PagedInputs:
    """One batch of paged-decode inputs (all host numpy arrays).

    q            uint16 [num_seqs, num_q_heads, head_dim]            (BF16 bits)
    k_cache      uint16 [num_blocks, block_size, num_kv_heads, head_dim]
    v_cache      uint16 [num_blocks, block_size, num_kv_heads, head_dim]
    block_tables int32  [num_seqs, max_blocks_per_seq]  (-1 = unused)
    seq_lens     int32  [num_seqs]
    scale        float  (an FP32 value)
    """
    workload: Workload
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    seq_lens: np.ndarray
    scale: float

    @property
    def num_seqs(self): return self.q.shape[0]
    @property
    def num_q_heads(self): return self.q.shape[1]
    @property
    def head_dim(self): return self.q.shape[2]
    @property
    def num_kv_heads(self): return self.k_cache.shape[2]
    @property
    def block_size(self): return self.k_cache.shape[1]
    @property
    def num_blocks(self): return self.k_cache.shape[0]


@dataclasses.dataclass
class ScratchInputs:
    """Inputs for the tiled step API with the scratch-pool slot layout
    ``[slot, K|V, kv_head, block_size, head_dim]``.

    q            uint16 [num_seqs, num_q_heads, head_dim]
    pool         uint16 [num_slots, 2, num_kv_heads, block_size, head_dim]
    slot_tables  int32  [num_seqs, max_blocks_per_seq]  (-1 = unused)
    seq_lens     int32  [num_seqs]
    """
    workload: Workload
    q: np.ndarray
    pool: np.ndarray
    slot_tables: np.ndarray
    seq_lens: np.ndarray

    @property
    def num_seqs(self): return self.q.shape[0]
    @property
    def num_q_heads(self): return self.q.shape[1]
    @property
    def head_dim(self): return self.q.shape[2]
    @property
    def num_kv_heads(self): return self.pool.shape[2]
    @property
    def block_size(self): return self.pool.shape[3]
    @property
    def num_slots(self): return self.pool.shape[0]


def _seq_kv(seed: int, s: int, nblk: int, bs: int, nkv: int, D: int):
    r = np.random.default_rng([seed, s])
    k = r.standard_normal((nblk, bs, nkv, D), dtype=np.float32)
    v = r.standard_normal((nblk, bs, nkv, D), dtype=np.float32)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def _layout(w: Workload, rng, lens: np.ndarray, bs: int):
    nblk = (lens + bs - 1) // bs
    total = int(nblk.sum())
    pool_blocks = total if w.pool_blocks is None else w.pool_blocks
    if pool_blocks < total:
        raise ValueError(f"pool of {pool_blocks} blocks cannot hold {total}")
    perm = rng.permutation(pool_blocks)
    max_blocks = max(1, int(nblk.max()) if len(nblk) else 1)
    tables = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    off = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = perm[off:off + n]
        off += n
    return nblk, pool_blocks, tables


def make_paged(w: Workload | str, canary: bool = True, scale: float | None = None,
               seq_lens=None) -> PagedInputs:
    """Generate one paged-decode batch for workload ``w``.

    ``seq_lens`` overrides the drawn lengths (the rest of the recipe is
    unchanged) so edge cases can reuse a workload's shapes.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    assert w.layout == "paged"
    rng = np.random.default_rng(w.seed)
    lens = _draw_lens(w, rng)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int64)
        w = dataclasses.replace(w, num_seqs=len(lens), seq_lens=tuple(int(x) for x in lens),
                                len_range=None, forced=())
    bs, nkv, D, nq = w.block_size, w.num_kv_heads, w.head_dim, w.num_q_heads
    nblk, pool_blocks, tables = _layout(w, rng, lens, bs)
    q = f32_to_bf16_bits(rng.standard_normal((len(lens), nq, D), dtype=np.float32))
    fill = BF16_QNAN if canary else np.uint16(0)
    k_cache = np.full((pool_blocks, bs, nkv, D), fill, dtype=np.uint16)
    v_cache = np.full((pool_blocks, bs, nkv, D), fill, dtype=np.uint16)

    def one(s):
        n = int(nblk[s])
        if n == 0:
            return
        k, v = _seq_kv(w.seed, s, n, bs, nkv, D)
        tail = int(lens[s]) - (n - 1) * bs          # valid slots of the last block
        if canary and tail < bs:
            k[n - 1, tail:] = BF16_QNAN
            v[n - 1, tail:] = BF16_QNAN
        ids = tables[s, :n]
        k_cache[ids] = k
        v_cache[ids] = v

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(len(lens))))
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    return PagedInputs(w, q, k_cache, v_cache, tables, lens.astype(np.int32), float(np.float32(scale)))


def make_scratch(w: Workload | str, canary: bool = True, seq_lens=None) -> ScratchInputs:
    """Generate inputs for the tiled API in the scratch-pool slot layout."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    assert w.layout == "scratch"
    rng = np.random.default_rng(w.seed)
    lens = _draw_lens(w, rng)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int64)
        w = dataclasses.replace(w, num_seqs=len(lens), seq_lens=tuple(int(x) for x in lens),
                                len_range=None, forced=())
    bs, nkv, D, nq = w.block_size, w.num_kv_heads, w.head_dim, w.num_q_heads
    nblk, pool_blocks, tables = _layout(w, rng, lens, bs)
    q = f32_to_bf16_bits(rng.standard_normal((len(lens), nq, D), dtype=np.float32))
    fill = BF16_QNAN if canary else np.uint16(0)
    pool = np.full((max(pool_blocks, 1), 2, nkv, bs, D), fill, dtype=np.uint16)

    def one(s):
        n = int(nblk[s])
        if n == 0:
            return
        k, v = _seq_kv(w.seed, s, n, bs, nkv, D)     # [n, bs, nkv, D]
        tail = int(lens[s]) - (n - 1) * bs
        if canary and tail < bs:
            k[n - 1, tail:] = BF16_QNAN
            v[n - 1, tail:] = BF16_QNAN
        ids = tables[s, :n]
        pool[ids, 0] = k.transpose(0, 2, 1, 3)
        pool[ids, 1] = v.transpose(0, 2, 1, 3)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(len(lens))))
    return ScratchInputs(w, q, pool, tables, lens.astype(np.int32))


def subset_paged(inp: PagedInputs, seqs) -> PagedInputs:
    """The same pool with only the rows ``seqs`` of q / block_tables / seq_lens
    (used to run a sequence alone against the very same memory)."""
    seqs = np.asarray(seqs, dtype=np.int64)
    return PagedInputs(inp.workload, np.ascontiguousarray(inp.q[seqs]), inp.k_cache, inp.v_cache,
                       np.ascontiguousarray(inp.block_tables[seqs]),
                       np.ascontiguousarray(inp.seq_lens[seqs]), inp.scale)


@dataclasses.dataclass
class PrefillInputs:
    """Causal prefill inputs for one sequence (host numpy arrays).

    q            uint16 [q_len, num_q_heads, head_dim]   (BF16 bits); row i
                 is the token at position q_offset + i
    k_cache      uint16 [num_blocks, block_size, num_kv_heads, head_dim]
    v_cache      uint16 [num_blocks, block_size, num_kv_heads, head_dim]
    block_table  int32  [max_blocks]   (-1 = unused)
    kv_len       tokens of K / V in the cache for this sequence
    scale        float  (an FP32 value, 1/sqrt(head_dim))
    """
    workload: Workload
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray
    kv_len: int
    q_offset: int
    scale: float

    @property
    def q_len(self): return self.q.shape[0]
    @property
    def num_q_heads(self): return self.q.shape[1]
    @property
    def head_dim(self): return self.q.shape[2]
    @property
    def num_kv_heads(self): return self.k_cache.shape[2]
    @property
    def block_size(self): return self.k_cache.shape[1]
    @property
    def num_blocks(self): return self.k_cache.shape[0]


def make_prefill(w: Workload | str, canary: bool = True, q_len: int | None = None,
                 kv_len: int | None = None, q_offset: int | None = None) -> PrefillInputs:
    """Generate causal-prefill inputs: the sequence's K / V follow the paged
    recipe above (steps 1-3, 5-7) with ``kv_len`` tokens; then the queries,
    ``rng.standard_normal((q_len, num_q_heads, head_dim), float32)``, are
    drawn after the block permutation.  ``q_len`` / ``kv_len`` / ``q_offset``
    override the workload's values."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    assert w.layout == "prefill"
    kv = int(w.seq_lens[0] if kv_len is None else kv_len)
    ql = int(w.q_len if q_len is None else q_len)
    qo = int(w.q_offset if q_offset is None else q_offset)
    w = dataclasses.replace(w, seq_lens=(kv,), q_len=ql, q_offset=qo)
    rng = np.random.default_rng(w.seed)
    lens = _draw_lens(w, rng)
    bs, nkv, D, nq = w.block_size, w.num_kv_heads, w.head_dim, w.num_q_heads
    nblk, pool_blocks, tables = _layout(w, rng, lens, bs)
    q = f32_to_bf16_bits(rng.standard_normal((ql, nq, D), dtype=np.float32))
    fill = BF16_QNAN if canary else np.uint16(0)
    k_cache = np.full((max(pool_blocks, 1), bs, nkv, D), fill, dtype=np.uint16)
    v_cache = np.full((max(pool_blocks, 1), bs, nkv, D), fill, dtype=np.uint16)
    n = int(nblk[0])
    if n:
        k, v = _seq_kv(w.seed, 0, n, bs, nkv, D)
        tail = kv - (n - 1) * bs
        if canary and tail < bs:
            k[n - 1, tail:] = BF16_QNAN
            v[n - 1, tail:] = BF16_QNAN
        k_cache[tables[0, :n]] = k
        v_cache[tables[0, :n]] = v
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    return PrefillInputs(w, q, k_cache, v_cache, tables[0].copy(), kv, qo, scale)


@dataclasses.dataclass
class PagedFP8Inputs:
    """A paged-decode batch with an FP8 (OCP E4M3) KV cache and per-tensor
    FP32 scales: K = decode(k8) * k_scale, V = decode(v8) * v_scale.

    q            uint16 [num_seqs, num_q_heads, head_dim]   (BF16 bits)
    k8, v8       uint8  [num_blocks, block_size, num_kv_heads, head_dim]
    block_tables int32  [num_seqs, max_blocks_per_seq]  (-1 = unused)
    seq_lens     int32  [num_seqs]
    """
    workload: Workload
    q: np.ndarray
    k8: np.ndarray
    v8: np.ndarray
    block_tables: np.ndarray
    seq_lens: np.ndarray
    scale: float
    k_scale: float
    v_scale: float

    @property
    def num_seqs(self): return self.q.shape[0]
    @property
    def num_q_heads(self): return self.q.shape[1]
    @property
    def head_dim(self): return self.q.shape[2]
    @property
    def num_kv_heads(self): return self.k8.shape[2]
    @property
    def block_size(self): return self.k8.shape[1]
    @property
    def num_blocks(self): return self.k8.shape[0]


def make_paged_fp8(w: Workload | str, canary: bool = True, seq_lens=None,
                   k_scale: float | None = None, v_scale: float | None = None) -> PagedFP8Inputs:
    """The paged recipe above with the K / V draws (FP32 N(0, 1), step 5)
    quantised to E4M3 instead of BF16: each tensor is divided by its scale
    and rounded (``f32_to_e4m3_bits``).  The scales default to a fixed
    ``4.0 / 448`` (so |x| up to 4 is representable, larger values saturate);
    they are FP32 values.  Canaries are the E4M3 NaN code."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    assert w.layout == "paged"
    rng = np.random.default_rng(w.seed)
    lens = _draw_lens(w, rng)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int64)
        w = dataclasses.replace(w, num_seqs=len(lens), seq_lens=tuple(int(x) for x in lens),
                                len_range=None, forced=())
    bs, nkv, D, nq = w.block_size, w.num_kv_heads, w.head_dim, w.num_q_heads
    nblk, pool_blocks, tables = _layout(w, rng, lens, bs)
    q = f32_to_bf16_bits(rng.standard_normal((len(lens), nq, D), dtype=np.float32))
    ks = float(np.float32(4.0 / 448.0 if k_scale is None else k_scale))
    vs = float(np.float32(4.0 / 448.0 if v_scale is None else v_scale))
    fill = E4M3_QNAN if canary else np.uint8(0)
    k8 = np.full((max(pool_blocks, 1), bs, nkv, D), fill, dtype=np.uint8)
    v8 = np.full((max(pool_blocks, 1), bs, nkv, D), fill, dtype=np.uint8)

    def one(s):
        n = int(nblk[s])
        if n == 0:
            return
        r = np.random.default_rng([w.seed, s])
        k = r.standard_normal((n, bs, nkv, D), dtype=np.float32)
        v = r.standard_normal((n, bs, nkv, D), dtype=np.float32)
        kq = f32_to_e4m3_bits(k.astype(np.float64) / ks)
        vq = f32_to_e4m3_bits(v.astype(np.float64) / vs)
        tail = int(lens[s]) - (n - 1) * bs
        if canary and tail < bs:
            kq[n - 1, tail:] = E4M3_QNAN
            vq[n - 1, tail:] = E4M3_QNAN
        ids = tables[s, :n]
        k8[ids] = kq
        v8[ids] = vq

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(len(lens))))
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    return PagedFP8Inputs(w, q, k8, v8, tables, lens.astype(np.int32), scale, ks, vs)


def plan_tiles(block_lists, seq_lens, block_size, tile_capacity):
    """Schedule whole-sequence KV folding as step_tile calls.

    ``block_lists[s]`` holds sequence s's block ids in token order.  Each
    call carries, per sequence, up to ``tile_capacity`` of its next blocks
    and one ``last_block_valid_slots`` value for all of them, so a sequence
    whose last block is partial gets that block in a call of its own,
    grouped with the other sequences that end with the same number of valid
    slots.  Returns a list of (tile_blocks [S][cap] lists, counts [S],
    last_block_valid_slots).  Pure host logic; nothing is launched.

    This is the caller's side of the tiled API ("metrale_storage/
    tiled_attention.rs", step_tile: one valid-slot count per call, read as
    the count of every sequence's last block in that call), so it lives with
    the harness that drives the calls, not in the library binding.  Only
    block ids are moved: no attention arithmetic.
    """
    S = len(seq_lens)
    full = []      # per sequence: list of blocks that are entirely valid
    tail = []      # per sequence: (block, valid) of a partial last block, or None
    for s in range(S):
        L = int(seq_lens[s])
        n = -(-L // block_size)
        blocks = [int(b) for b in block_lists[s][:n]]
        r = L - (n - 1) * block_size if n else 0
        if n and r < block_size:
            full.append(blocks[:-1])
            tail.append((blocks[-1], r))
        else:
            full.append(blocks)
            tail.append(None)
    calls = []
    # tiles of a sequence: its full blocks cut every tile_capacity blocks from
    # the start (the same cut alone or in any batch)
    tiles = [[f[i:i + tile_capacity] for i in range(0, len(f), tile_capacity)] for f in full]
    rounds = max((len(t) for t in tiles), default=0)
    # each sequence's tiles go, in order, to the rounds that hold the fewest
    # blocks so far (sequences with more tiles placed first), so every round
    # carries about the same work; a sequence's tiles and their order do not
    # depend on the rest of the batch, only the round numbers do
    load = [0] * rounds
    slot = [[] for _ in range(S)]
    for s in sorted(range(S), key=lambda s: (-len(tiles[s]), -len(full[s]), s)):
        k = len(tiles[s])
        pick = sorted(sorted(range(rounds), key=lambda r: (load[r], r))[:k])
        for r, t in zip(pick, tiles[s]):
            load[r] += len(t)
        slot[s] = pick
    for i in range(rounds):
        tb = [[0] * tile_capacity for _ in range(S)]
        cnt = [0] * S
        for s in range(S):
            if i in slot[s]:
                part = tiles[s][slot[s].index(i)]
                tb[s][:len(part)] = part
                cnt[s] = len(part)
        calls.append((tb, cnt, block_size))
    for r in sorted({t[1] for t in tail if t is not None}):
        tb = [[0] * tile_capacity for _ in range(S)]
        cnt = [0] * S
        for s in range(S):
            if tail[s] is not None and tail[s][1] == r:
                tb[s][0] = tail[s][0]
                cnt[s] = 1
        calls.append((tb, cnt, r))
    return calls
