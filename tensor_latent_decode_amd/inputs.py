"""Seeded synthetic inputs for TPLA decode (shared by tests, bench and smoke).

This module only draws random numbers and lays them out; it holds none of the
attention, transform or paging arithmetic.  Both the HIP path and the CPU
oracle consume exactly the arrays produced here.

Recipe (all workloads):
  * numpy ``Generator(PCG64)`` streams from ``SeedSequence(seed).spawn(8)``
    (lengths, block permutation, history latent, history rope, new latent,
    new rope, query latent, query rope).
  * Samples are standard normal float32.  For bf16 workloads they are rounded
    to bf16 once, here, and handed out as uint16 bit patterns.
  * History latent rows stand for rows the prefill already wrote into the
    cache in the rotated basis.  An orthonormal rotation of an iid N(0, 1)
    row is again iid N(0, 1), so those rows are drawn directly as N(0, 1);
    where the workload asks for RMS-normalised rows each row is then scaled
    to unit root-mean-square (eps 1e-6) before the bf16 rounding.
  * The new token's latent and the absorbed query are drawn in the
    unrotated basis (the decode step rotates them).  Scaling the new latent
    to unit RMS commutes with the rotation, so it is done here too.
  * Physical cache blocks are a random permutation of all blocks in use; one
    extra physical block (the last id) is reserved as a poison block that
    unused block-table entries point at, so a kernel that reads past a
    sequence end reads NaN instead of another sequence's data.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple, Union

import numpy as np

__all__ = ["TplaConfig", "CONFIGS", "Case", "make_case", "bf16_bits", "BF16_NAN",
           "PrefillConfig", "PREFILL_CONFIGS", "PrefillCase", "make_prefill_case"]

BF16_NAN = np.uint16(0xFFFF)


@dataclass(frozen=True)
class TplaConfig:
    name: str
    batch: int
    heads: int
    d_c: int
    tp: int
    d_r: int
    ctx: Union[int, Tuple[int, int]]   # fixed length, or (lo, hi) uniform per sequence
    scale: float
    dtype: str                         # "fp32" or "bf16"
    block_size: int
    seed: int
    rms_rows: bool                     # history/new latent rows scaled to unit RMS
    desc: str = ""

    @property
    def d_s(self) -> int:
        return self.d_c // self.tp


CONFIGS = {
    "tiny_fp32": TplaConfig(
        "tiny_fp32", batch=1, heads=4, d_c=64, tp=2, d_r=16, ctx=128,
        scale=1.0 / math.sqrt(48.0), dtype="fp32", block_size=64, seed=1,
        rms_rows=False,
        desc="tiny TPLA decode, fp32: B=1, H=4, d_c=64 (TP=2, 32 per shard), "
             "d_r=16, context 128"),
    "dsv3_4k": TplaConfig(
        "dsv3_4k", batch=1, heads=128, d_c=512, tp=2, d_r=64, ctx=4096,
        scale=1.0 / math.sqrt(192.0), dtype="bf16", block_size=64, seed=2,
        rms_rows=True,
        desc="DeepSeek-V3-shaped shard, bf16: B=1, H=128, d_c=512 (TP=2), "
             "d_r=64, context 4096, block 64"),
    "dsv3_32k": TplaConfig(
        "dsv3_32k", batch=16, heads=128, d_c=512, tp=2, d_r=64, ctx=32768,
        scale=1.0 / math.sqrt(192.0), dtype="bf16", block_size=64, seed=3,
        rms_rows=True,
        desc="DeepSeek-V3-shaped shard, bf16, long context: B=16, H=128, "
             "d_c=512 (TP=2, 256 per shard), d_r=64, context 32768, block 64"),
    "kimi_k2_32k": TplaConfig(
        "kimi_k2_32k", batch=16, heads=64, d_c=512, tp=4, d_r=64, ctx=32768,
        scale=1.0 / math.sqrt(192.0), dtype="bf16", block_size=64, seed=4,
        rms_rows=False,
        desc="Kimi-K2-shaped shard, bf16: B=16, H=64, d_c=512 (TP=4, 128 per "
             "shard), d_r=64, context 32768, block 64"),
    "mla_tp2_32k": TplaConfig(
        "mla_tp2_32k", batch=16, heads=64, d_c=512, tp=1, d_r=64, ctx=32768,
        scale=1.0 / math.sqrt(192.0), dtype="bf16", block_size=64, seed=6,
        rms_rows=True,
        desc="plain MLA under TP=2 on one device (the comparison TPLA is measured "
             "against), bf16: B=16, 64 of DeepSeek-V3's 128 heads, the whole "
             "512-wide latent, d_r=64, context 32768, block 64"),
    "mla_tp4_32k": TplaConfig(
        "mla_tp4_32k", batch=16, heads=16, d_c=512, tp=1, d_r=64, ctx=32768,
        scale=1.0 / math.sqrt(192.0), dtype="bf16", block_size=64, seed=7,
        rms_rows=False,
        desc="plain MLA under TP=4 on one device (the comparison TPLA is measured "
             "against), bf16: B=16, 16 of Kimi-K2's 64 heads, the whole 512-wide "
             "latent, d_r=64, context 32768, block 64"),
    "ragged_tp2": TplaConfig(
        "ragged_tp2", batch=32, heads=128, d_c=512, tp=2, d_r=64,
        ctx=(1024, 32768), scale=1.0 / math.sqrt(192.0), dtype="bf16",
        block_size=64, seed=5, rms_rows=True,
        desc="ragged TP=2 step on one GPU, bf16: B=32, H=128, d_c=512, d_r=64, "
             "lengths uniform in [1024, 32768], block 64, both shards"),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), nearest-even, in chunks."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    step = 1 << 22
    for i in range(0, flat_in.size, step):
        u = flat_in[i:i + step].view(np.uint32).copy()
        u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        flat_out[i:i + step] = (u >> np.uint32(16)).astype(np.uint16)
    return out


@dataclass
class Case:
    cfg: TplaConfig
    seq_lens: np.ndarray        # [B] int32, final lengths (history + 1 new token)
    hist_latent: np.ndarray     # [N, d_c] rotated-basis rows already in the cache
    hist_rope: np.ndarray       # [N, d_r]
    hist_seq: np.ndarray        # [N] int32
    hist_pos: np.ndarray        # [N] int32
    new_latent: np.ndarray      # [B, d_c] unrotated latent of the new token
    new_rope: np.ndarray        # [B, d_r]
    new_pos: np.ndarray         # [B] int32 (= seq_lens - 1)
    q_latent: np.ndarray        # [B, H, d_c] unrotated absorbed query
    q_rope: np.ndarray          # [B, H, d_r]
    block_table: np.ndarray     # [B, max_blocks] int32
    num_blocks: int             # physical blocks incl. the poison block (last id)
    max_blocks: int
    extra: dict = field(default_factory=dict)

    @property
    def poison_block(self) -> int:
        return self.num_blocks - 1


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _unit_rms(x: np.ndarray) -> np.ndarray:
    ms = np.einsum("ij,ij->i", x, x, dtype=np.float64) / x.shape[1]
    return (x / np.sqrt(ms + 1e-6)[:, None]).astype(np.float32)


def make_case(cfg: TplaConfig, *, batch: Optional[int] = None,
              ctx: Optional[Union[int, Tuple[int, int], List[int]]] = None,
              seed: Optional[int] = None, block_size: Optional[int] = None,
              heads: Optional[int] = None) -> Case:
    """Draw one decode step's inputs for `cfg` (fields may be overridden)."""
    over = {}
    if batch is not None:
        over["batch"] = batch
    if ctx is not None:
        over["ctx"] = ctx
    if seed is not None:
        over["seed"] = seed
    if block_size is not None:
        over["block_size"] = block_size
    if heads is not None:
        over["heads"] = heads
    if over:
        cfg = replace(cfg, **over)
    B, H, d_c, d_r, bs = cfg.batch, cfg.heads, cfg.d_c, cfg.d_r, cfg.block_size
    ss = np.random.SeedSequence(cfg.seed).spawn(8)
    rngs = [np.random.Generator(np.random.PCG64(s)) for s in ss]

    if isinstance(cfg.ctx, tuple):
        lo, hi = cfg.ctx
        seq_lens = rngs[0].integers(lo, hi + 1, size=B).astype(np.int32)
    elif isinstance(cfg.ctx, list):          # one length per sequence
        if len(cfg.ctx) != B:
            raise ValueError("a list of lengths needs one per sequence")
        seq_lens = np.array(cfg.ctx, dtype=np.int32)
    else:
        seq_lens = np.full(B, int(cfg.ctx), dtype=np.int32)
    if np.any(seq_lens < 1):
        raise ValueError("every sequence needs at least the new token")

    blocks_per_seq = (seq_lens + bs - 1) // bs
    max_blocks = int(blocks_per_seq.max())
    used = int(blocks_per_seq.sum())
    num_blocks = used + 1
    poison = num_blocks - 1
    perm = rngs[1].permutation(used).astype(np.int32)
    block_table = np.full((B, max_blocks), poison, dtype=np.int32)
    k = 0
    for b in range(B):
        nb = int(blocks_per_seq[b])
        block_table[b, :nb] = perm[k:k + nb]
        k += nb

    hist_lens = seq_lens - 1
    N = int(hist_lens.sum())
    bf16 = cfg.dtype == "bf16"
    store_dt = np.uint16 if bf16 else np.float32
    hist_latent = np.empty((N, d_c), dtype=store_dt)
    hist_rope = np.empty((N, d_r), dtype=store_dt)
    hist_seq = np.empty(N, dtype=np.int32)
    hist_pos = np.empty(N, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(hist_lens[b])
        if n == 0:
            continue
        lat = _normal(rngs[2], (n, d_c))
        if cfg.rms_rows:
            lat = _unit_rms(lat)
        rope = _normal(rngs[3], (n, d_r))
        hist_latent[off:off + n] = bf16_bits(lat) if bf16 else lat
        hist_rope[off:off + n] = bf16_bits(rope) if bf16 else rope
        hist_seq[off:off + n] = b
        hist_pos[off:off + n] = np.arange(n, dtype=np.int32)
        off += n

    new_lat = _normal(rngs[4], (B, d_c))
    if cfg.rms_rows:
        new_lat = _unit_rms(new_lat)
    new_rope = _normal(rngs[5], (B, d_r))
    q_lat = _normal(rngs[6], (B, H, d_c))
    q_rope = _normal(rngs[7], (B, H, d_r))
    conv = bf16_bits if bf16 else (lambda a: a)
    return Case(cfg=cfg, seq_lens=seq_lens,
                hist_latent=hist_latent, hist_rope=hist_rope,
                hist_seq=hist_seq, hist_pos=hist_pos,
                new_latent=conv(new_lat), new_rope=conv(new_rope),
                new_pos=(seq_lens - 1).astype(np.int32),
                q_latent=conv(q_lat), q_rope=conv(q_rope),
                block_table=block_table, num_blocks=num_blocks,
                max_blocks=max_blocks)


# ---------------------------------------------------------------------------
# MLA-form prefill inputs: prompts of latent rows [c || k_rope] and their
# absorbed queries, with the decode cases' value distributions (unit-RMS
# latent rows, standard normal rope keys and queries).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class PrefillConfig:
    name: str
    batch: int
    heads: int
    d_c: int
    d_r: int
    lens: Union[int, Tuple[int, int]]   # prompt length, or (lo, hi) uniform per prompt
    max_len: int                        # positions in the buffers
    scale: float
    seed: int
    desc: str = ""


PREFILL_CONFIGS = {
    "prefill_small": PrefillConfig(
        "prefill_small", batch=2, heads=16, d_c=512, d_r=64, lens=(1, 200), max_len=200,
        scale=1.0 / math.sqrt(192.0), seed=21,
        desc="small MLA-form prefill: B=2 prompts of 1..200 tokens, 16 heads"),
    "mla_prefill_4k": PrefillConfig(
        "mla_prefill_4k", batch=2, heads=64, d_c=512, d_r=64, lens=4096, max_len=4096,
        scale=1.0 / math.sqrt(192.0), seed=22,
        desc="MLA-form prefill on one device of DeepSeek-V3 under TP=2: B=2 prompts of 4096 "
             "tokens, 64 of the 128 heads, latent 512, rope 64"),
}


@dataclass
class PrefillCase:
    cfg: PrefillConfig
    seq_lens: np.ndarray        # [B] int32
    q_latent: np.ndarray        # [B, S, H, d_c] bf16 bits
    q_rope: np.ndarray          # [B, S, H, d_r] bf16 bits
    kv: np.ndarray              # [B, S, d_c + d_r] bf16 bits: [latent || rope key]


def make_prefill_case(cfg: PrefillConfig, *, batch: Optional[int] = None,
                      heads: Optional[int] = None,
                      lens: Optional[Union[int, Tuple[int, int]]] = None,
                      max_len: Optional[int] = None, seed: Optional[int] = None) -> PrefillCase:
    """Draw a batch of prompts for `cfg` (fields may be overridden)."""
    over = {k: v for k, v in (("batch", batch), ("heads", heads), ("lens", lens),
                              ("max_len", max_len), ("seed", seed)) if v is not None}
    if over:
        cfg = replace(cfg, **over)
    B, H, d_c, d_r, S = cfg.batch, cfg.heads, cfg.d_c, cfg.d_r, cfg.max_len
    ss = np.random.SeedSequence(cfg.seed).spawn(5)
    rngs = [np.random.Generator(np.random.PCG64(x)) for x in ss]
    if isinstance(cfg.lens, tuple):
        seq_lens = rngs[0].integers(cfg.lens[0], cfg.lens[1] + 1, size=B).astype(np.int32)
    else:
        seq_lens = np.full(B, int(cfg.lens), dtype=np.int32)
    if np.any(seq_lens > S) or np.any(seq_lens < 0):
        raise ValueError("prompt lengths must lie in [0, max_len]")
    kv = np.empty((B, S, d_c + d_r), dtype=np.uint16)
    q_lat = np.empty((B, S, H, d_c), dtype=np.uint16)
    q_rope = np.empty((B, S, H, d_r), dtype=np.uint16)
    for b in range(B):
        kv[b, :, :d_c] = bf16_bits(_unit_rms(_normal(rngs[1], (S, d_c))))
        kv[b, :, d_c:] = bf16_bits(_normal(rngs[2], (S, d_r)))
        for t0 in range(0, S, 256):
            t1 = min(S, t0 + 256)
            q_lat[b, t0:t1] = bf16_bits(_normal(rngs[3], (t1 - t0, H, d_c)))
            q_rope[b, t0:t1] = bf16_bits(_normal(rngs[4], (t1 - t0, H, d_r)))
    return PrefillCase(cfg=cfg, seq_lens=seq_lens, q_latent=q_lat, q_rope=q_rope, kv=kv)
