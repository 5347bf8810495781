"""Seeded synthetic inputs for the TurboQuant store / decode workloads.

This module only draws random inputs (K, V, queries, sign vectors, block
tables, sequence lengths, slot mappings) with NumPy's PCG64; it holds none of
the quantization or attention arithmetic.  Both the CPU oracle (tests,
cpu_baseline) and the GPU path (tests, bench, smoke) take their inputs from
here, so the two sides always see identical bytes.

16-bit float inputs are returned as uint16 bit patterns plus a dtype tag
("bf16" or "f16").

Workloads (head_dim 128 except hd256; synthetic stand-ins for model
activations, shaped like the models they are named after):

  tiny       4bit_nc, 1 seq x 256 tokens, Hq=2/Hk=1, bs=16, fp16 N(0,1) with
             4 outlier channels x8 (shared by K and V), sequential blocks.
  llama8b    k8v4, 32 seqs x 4096 tokens, Hq=32/Hk=8, bs=16, bf16
             N(0,1)*sigma_c with sigma_c log-uniform in [0.5, 4] per (KV head,
             channel), drawn separately for K and V; block tables = first
             8192 entries of a permutation of a 16384-block pool.
  qwen32b    3bit_nc, 64 seqs, lengths uniform in [1024, 16384], Hq=64/Hk=8,
             bs=64, bf16 Student-t (nu=5) i.i.d.; pool = 2x the blocks needed,
             random permutation.
  store      all four presets, 65536 tokens x 8 KV heads, bs=32, bf16 N(0,1)
             with ceil(2% of 128) = 3 channels per KV head scaled x16 (same
             channels for K and V); slot mapping = random permutation of the
             65536 pool slots.
  longctx    k3v4_nc, 4 seqs x 131072 tokens, Hq=40/Hk=8, bs=128, 32 KV
             splits, bf16 N(0,1)*sigma_c with sigma_c log-uniform in
             [0.25, 8]; 4096 blocks, random permutation.
  hd256      k8v4 at head_dim 256 (the 256-dim heads of the pages' Bench F),
             64 seqs x 4096 tokens, Hq=16/Hk=2, bs=16, bf16 N(0,1)*sigma_c
             with sigma_c log-uniform in [0.5, 4]; pool = 2x the blocks
             needed, random permutation (203 MB of k8v4 cache per step).
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    preset: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    block_size: int
    dtype: str  # "bf16" | "f16"
    dist: str  # "normal_outliers" | "normal_chscale" | "student_t"
    seed: int
    seq_len: int = 0  # fixed context length (0 -> drawn, see len_range)
    lens: tuple = ()  # explicit per-sequence lengths (overrides seq_len / len_range)
    len_range: tuple = (0, 0)
    num_kv_splits: int = 0  # 0 -> caller's choice
    pool_factor: float = 1.0  # pool blocks = factor * needed
    sequential_table: bool = False
    outliers: int = 0
    outlier_scale: float = 1.0
    chscale_range: tuple = (1.0, 1.0)
    head_dim: int = HEAD_DIM
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", "turboquant_4bit_nc", 1, 2, 1, 16, "f16", "normal_outliers", seed=0, seq_len=256,
                     sequential_table=True, outliers=4, outlier_scale=8.0),
    "llama8b": Workload("llama8b", "turboquant_k8v4", 32, 32, 8, 16, "bf16", "normal_chscale", seed=2, seq_len=4096,
                        pool_factor=2.0, chscale_range=(0.5, 4.0)),
    "qwen32b": Workload("qwen32b", "turboquant_3bit_nc", 64, 64, 8, 64, "bf16", "student_t", seed=3,
                        len_range=(1024, 16384), pool_factor=2.0),
    "hd256": Workload("hd256", "turboquant_k8v4", 64, 16, 2, 16, "bf16", "normal_chscale", seed=6, seq_len=4096,
                      pool_factor=2.0, chscale_range=(0.5, 4.0), head_dim=256),
    "longctx": Workload("longctx", "turboquant_k3v4_nc", 4, 40, 8, 128, "bf16", "normal_chscale", seed=5,
                        seq_len=131072, num_kv_splits=32, pool_factor=1.0, chscale_range=(0.25, 8.0)),
}

#: store sweep: tokens, KV heads, block size, presets
STORE_WORKLOAD = dict(name="store", num_tokens=65536, num_kv_heads=8, block_size=32, dtype="bf16", seed=4,
                      outlier_frac=0.02, outlier_scale=16.0,
                      presets=("turboquant_k8v4", "turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"))


def scaled(w: Workload, **kw) -> Workload:
    """A smaller copy of a workload (same distributions), for parity tests."""
    return replace(w, **kw)


# --------------------------------------------------------------------------
# 16-bit encodings of the generated values (input rounding only)
# --------------------------------------------------------------------------


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        # round to nearest even in uint32 (finite inputs: no carry out of 32 bits)
        u = x.view(np.uint32)
        return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) & 0xFFFFFFFF for k in key])


# --------------------------------------------------------------------------
# Per-workload draws
# --------------------------------------------------------------------------


def seq_lens(w: Workload) -> np.ndarray:
    if w.lens:
        return np.array(w.lens, dtype=np.int32)
    if w.seq_len:
        return np.full(w.batch, w.seq_len, dtype=np.int32)
    lo, hi = w.len_range
    return _rng(w.seed, 11).integers(lo, hi + 1, size=w.batch).astype(np.int32)


def blocks_needed(w: Workload, lens=None) -> np.ndarray:
    lens = seq_lens(w) if lens is None else lens
    return (lens.astype(np.int64) + w.block_size - 1) // w.block_size


def num_blocks(w: Workload) -> int:
    need = int(blocks_needed(w).sum())
    return max(1, int(math.ceil(need * w.pool_factor)))


def block_table(w: Workload) -> np.ndarray:
    """(B, max_blocks) int32; rows padded with -1 past each sequence's blocks
    (those entries are never read)."""
    need = blocks_needed(w)
    nb = num_blocks(w)
    width = max(1, int(need.max()))
    if w.sequential_table:
        ids = np.arange(nb, dtype=np.int64)
    else:
        ids = _rng(w.seed, 12).permutation(nb)
    tab = np.full((w.batch, width), -1, dtype=np.int32)
    pos = 0
    for b in range(w.batch):
        tab[b, : need[b]] = ids[pos : pos + need[b]]
        pos += need[b]
    return tab


def signs(w_or_seed, d: int = HEAD_DIM) -> np.ndarray:
    """Rademacher +-1 signs for the rotation, float32 (D,): D = the workload's
    head_dim, or d for a plain seed."""
    if isinstance(w_or_seed, Workload):
        seed, d = w_or_seed.seed, w_or_seed.head_dim
    else:
        seed = int(w_or_seed)
    return np.where(_rng(seed, 13).integers(0, 2, size=d) == 1, -1.0, 1.0).astype(np.float32)


def _channel_scales(w: Workload, which: int) -> np.ndarray:
    lo, hi = w.chscale_range
    r = _rng(w.seed, 14, which)
    return np.exp(r.uniform(math.log(lo), math.log(hi), size=(w.num_kv_heads, w.head_dim))).astype(np.float32)


def _outlier_channels(w: Workload) -> np.ndarray:
    return _rng(w.seed, 15).choice(w.head_dim, size=w.outliers, replace=False)


CHUNK = 8192  # tokens per independently seeded piece of a sequence


def _kv_chunk(w: Workload, b: int, c: int, L: int):
    """Tokens [c*CHUNK, min(L, (c+1)*CHUNK)) of sequence b: (K, V) uint16 bits."""
    n = min(L, (c + 1) * CHUNK) - c * CHUNK
    shape = (n, w.num_kv_heads, w.head_dim)
    out = []
    for which in (0, 1):
        r = _rng(w.seed, 16, b, which, c)
        if w.dist == "student_t":
            z = r.standard_normal(shape, dtype=np.float32)
            g = r.standard_gamma(2.5, shape, dtype=np.float32) * np.float32(2.0 / 5.0)
            x = z / np.sqrt(g)
        else:
            x = r.standard_normal(shape, dtype=np.float32)
            if w.dist == "normal_chscale":
                x *= _channel_scales(w, which)[None]
            elif w.dist == "normal_outliers":
                x[..., _outlier_channels(w)] *= np.float32(w.outlier_scale)
        out.append(to_bits(x, w.dtype))
    return out[0], out[1]


def kv_sequence(w: Workload, b: int, lens=None, threads: int = 1):
    """(K, V) of sequence b: uint16 bits of shape (L_b, Hk, D) each."""
    L = int((seq_lens(w) if lens is None else lens)[b])
    K = np.empty((L, w.num_kv_heads, w.head_dim), np.uint16)
    V = np.empty_like(K)

    def fill(c):
        k, v = _kv_chunk(w, b, c, L)
        K[c * CHUNK : c * CHUNK + k.shape[0]] = k
        V[c * CHUNK : c * CHUNK + v.shape[0]] = v

    nchunks = -(-L // CHUNK)
    if threads > 1 and nchunks > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nchunks)))
    else:
        for c in range(nchunks):
            fill(c)
    return K, V


def kv_all(w: Workload, threads: int = 8):
    """K, V for every sequence (lists), generated chunk-parallel."""
    lens = seq_lens(w)
    Ks = [np.empty((int(L), w.num_kv_heads, w.head_dim), np.uint16) for L in lens]
    Vs = [np.empty_like(k) for k in Ks]
    jobs = [(b, c) for b in range(w.batch) for c in range(-(-int(lens[b]) // CHUNK))]

    def fill(job):
        b, c = job
        k, v = _kv_chunk(w, b, c, int(lens[b]))
        Ks[b][c * CHUNK : c * CHUNK + k.shape[0]] = k
        Vs[b][c * CHUNK : c * CHUNK + v.shape[0]] = v

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, jobs))
    return Ks, Vs


def slot_mapping_for_sequence(w: Workload, b: int, table=None, lens=None) -> np.ndarray:
    """Slot ids of tokens [0, L_b) of sequence b under its block table."""
    table = block_table(w) if table is None else table
    L = int((seq_lens(w) if lens is None else lens)[b])
    t = np.arange(L, dtype=np.int64)
    return table[b, t // w.block_size].astype(np.int64) * w.block_size + t % w.block_size


def queries(w: Workload) -> np.ndarray:
    """(B, Hq, D) uint16 bits, N(0,1) in the workload's dtype."""
    x = _rng(w.seed, 17).standard_normal((w.batch, w.num_q_heads, w.head_dim), dtype=np.float32)
    return to_bits(x, w.dtype)


# --------------------------------------------------------------------------
# Store sweep inputs
# --------------------------------------------------------------------------


def store_inputs(num_tokens=None, num_kv_heads=None, block_size=None, seed=None, dtype=None, head_dim=HEAD_DIM):
    """(K, V, slot_mapping, num_blocks) for the store sweep (defaults = the
    full sweep).  K, V: uint16 bits (N, Hk, D)."""
    s = STORE_WORKLOAD
    N = s["num_tokens"] if num_tokens is None else num_tokens
    Hk = s["num_kv_heads"] if num_kv_heads is None else num_kv_heads
    bs = s["block_size"] if block_size is None else block_size
    seed = s["seed"] if seed is None else seed
    dtype = s["dtype"] if dtype is None else dtype
    r = _rng(seed, 21)
    n_out = int(math.ceil(s["outlier_frac"] * head_dim))
    ch = np.stack([r.choice(head_dim, size=n_out, replace=False) for _ in range(Hk)])
    out = []
    for which in (0, 1):
        x = _rng(seed, 22, which).standard_normal((N, Hk, head_dim), dtype=np.float32)
        for h in range(Hk):
            x[:, h, ch[h]] *= np.float32(s["outlier_scale"])
        out.append(to_bits(x, dtype))
    nblocks = -(-N // bs)
    slots = _rng(seed, 23).permutation(nblocks * bs)[:N].astype(np.int64)
    return out[0], out[1], slots, nblocks
