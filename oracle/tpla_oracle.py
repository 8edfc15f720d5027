"""Plain fp64 CPU oracle for TPLA decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Sources (web pages about arXiv 2508.15881, "TPLA: Tensor Parallel Latent
Attention for Efficient Disaggregated Prefill & Decode Inference"):

* [ABS]  The English abstract, as shown on the chatpaper.ai, fugumt.com and
  searcharxiv.org pages.  In our words: the per-token cache is MLA's one
  compressed latent; TPLA cuts it, and every head's input width with it,
  into T slices held on T devices; each device runs the attention of all
  heads over its own slice and the T results are added by an all-reduce;
  an orthogonal transform (Hadamard, or PCA) is applied to the latent first
  so the slices disagree less; no head loses access to any latent column.
* [ABS-R] The revised English abstract on the paperbot-e5f.pages.dev page: it
  names the cached latent ``cKV``, calls the transforms orthogonal
  reparameterisations of RMSNorm and softmax, and keeps MLA for prefill and
  TPLA for the memory-bound decode.
* [BLOG] The blogs.edgentiq.com article, sections "Introducing
  Tensor-Parallel Latent Attention (TPLA)" and "How TPLA Works: Smart Slicing
  and Reparameterization" (orthogonal transform before the split so that
  local computations approximate the global score).

The pages print no equations.  Where they leave a step open the plain reading
is taken:

* The rope key/query are not part of the latent: every shard carries them
  whole and adds their score term (reading R1).
* The softmax scale is the model's scale on every shard (reading R2).
* Shard outputs live in disjoint latent columns, so the all-reduce sum is the
  sum of zero-padded partials, i.e. placement (reading R3).
* The Hadamard matrix is Sylvester's, in natural order, scaled by 1/sqrt(n),
  applied to query and latent over the whole latent width, never to the rope
  (reading R4).
* RMSNorm slicing ([BLOG] "How TPLA Works"): a device that holds one slice of
  the rotated latent normalises that slice by the root mean square of the
  slice alone (eps inside the root); the model's norm uses the whole vector.
  The norm's gain is taken as folded into the weights that read the latent,
  so both norms here are gain-free (reading R10).
* The all-reduce sums real arithmetic once each device applies its slice of
  the value up-projection: device g holds rows g*d_s .. of every head's
  transposed W_UV (latent index first), rotated like the latent, and its
  up-projected output is summed over devices (reading R11).
* Prefill keeps the MLA form ([ABS-R]; [BLOG] "Prefill-Decode Separation for
  Optimal Performance"): no slicing and no rotation; prompt position t of
  every head attends causally to the prompt's own positions 0..t, with the
  decode step's score (latent dot product plus rope dot product, times the
  scale) and the whole latent row as the value (reading R12).

Every function works in float64.  bf16 data enter as their exact values.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "sylvester_hadamard",
    "fwht",
    "bf16_bits_to_f64",
    "f32_to_bf16_bits",
    "page_slot",
    "paged_append",
    "gather_sequence",
    "shard_attention",
    "merge_partials",
    "shard_slice",
    "tpla_shards",
    "combine_shards",
    "tpla_decode",
    "tpla_decode_paged",
    "mla_decode",
    "mla_decode_unabsorbed",
    "mla_prefill",
    "rms_normalize",
    "slice_rms_normalize",
    "rotate_normalize_latent",
    "up_project_shard",
    "up_project_combine",
    "rotate_weight_rows",
]


# ---------------------------------------------------------------------------
# Orthogonal transform applied before slicing  ([ABS]; [BLOG] "How TPLA
# Works"; [ABS-R] reparameterisation of softmax and RMSNorm)
# ---------------------------------------------------------------------------

def sylvester_hadamard(n: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix H_n (entries +-1), n = 2**k.

    H_1 = [1]; H_2m is the 2x2 block matrix [[H_m, H_m], [H_m, -H_m]].
    """
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError(f"n must be a power of two, got {n}")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht(x: np.ndarray) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform along the last axis: x @ H_n / sqrt(n).

    Written as the textbook in-place butterfly: for each stride
    h = 1, 2, 4, ..., n/2 the pair (a, b) = (x[i], x[i+h]) becomes (a+b, a-b).
    H_n is symmetric, so x @ H_n and H_n @ x agree row-wise.
    """
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError(f"last dimension must be a power of two, got {n}")
    lead = y.shape[:-1]
    y = y.reshape(-1, n)
    h = 1
    while h < n:
        blocks = y.reshape(y.shape[0], n // (2 * h), 2, h)
        a = blocks[:, :, 0, :].copy()
        b = blocks[:, :, 1, :].copy()
        blocks[:, :, 0, :] = a + b
        blocks[:, :, 1, :] = a - b
        h *= 2
    y /= math.sqrt(n)
    return y.reshape(*lead, n)


# ---------------------------------------------------------------------------
# bf16 storage (the cache and the MFMA operands are bf16)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns, to nearest, ties to even.

    Keep the top 16 bits of the float32 pattern; the dropped 16 bits decide:
    above half an ulp rounds up, below rounds down, exactly half rounds to
    the even result.  NaN stays NaN.
    """
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = x32.view(np.uint32).astype(np.uint64)
    hi = bits >> np.uint64(16)
    lo = bits & np.uint64(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint64(1)) == 1))
    out = (hi + up.astype(np.uint64)).astype(np.uint16)
    nan = np.isnan(x32)
    out[nan] = np.uint16(0x7FC0)
    return out


# ---------------------------------------------------------------------------
# Paged latent cache ([ABS-R]: only cKV is cached; paging is the layout the
# caches use here, block table -> physical block of block_size rows)
# ---------------------------------------------------------------------------

def page_slot(block_table: np.ndarray, b: int, pos: int, block_size: int) -> int:
    """Physical row of logical token `pos` of sequence `b`."""
    return int(block_table[b, pos // block_size]) * block_size + pos % block_size


def paged_append(cache: np.ndarray, block_table: np.ndarray, block_size: int,
                 row_seq: np.ndarray, row_pos: np.ndarray,
                 latent: np.ndarray, rope: np.ndarray) -> None:
    """Write rows [latent_t || rope_t] at their paged slots, in place.

    `cache` is [num_blocks, block_size, d_s + d_r].  For a uint16 (bf16) cache,
    uint16 sources are copied bit for bit and float32 sources are rounded to
    bf16 (nearest even).  For a float32 cache the source is stored as float32.
    """
    d_s = latent.shape[1]
    flat = cache.reshape(-1, cache.shape[-1])
    for t in range(len(row_seq)):
        slot = page_slot(block_table, int(row_seq[t]), int(row_pos[t]), block_size)
        for part, lo in ((latent[t], 0), (rope[t], d_s)):
            if cache.dtype == np.uint16:
                if part.dtype == np.uint16:
                    val = part
                else:
                    val = f32_to_bf16_bits(part)
            else:
                val = np.asarray(part, dtype=cache.dtype)
            flat[slot, lo:lo + len(part)] = val


def gather_sequence(cache: np.ndarray, block_table: np.ndarray, b: int,
                    length: int, block_size: int) -> np.ndarray:
    """Logical rows 0..length-1 of sequence b, as float64 [length, d_s + d_r]."""
    flat = cache.reshape(-1, cache.shape[-1])
    slots = [page_slot(block_table, b, j, block_size) for j in range(length)]
    rows = flat[np.asarray(slots, dtype=np.int64)] if slots else flat[:0]
    if cache.dtype == np.uint16:
        return bf16_bits_to_f64(rows)
    return rows.astype(np.float64)


# ---------------------------------------------------------------------------
# Per-shard attention ([ABS]: each shard runs attention on its own slice;
# [BLOG] "How TPLA Works": the global score is approximated by local ones)
# ---------------------------------------------------------------------------

def shard_attention(q_lat: np.ndarray, q_rope: np.ndarray, c_lat: np.ndarray,
                    k_rope: np.ndarray, scale: float):
    """One sequence, one shard, all heads.

    q_lat [H, d_s], q_rope [H, d_r], c_lat [L, d_s], k_rope [L, d_r].
    Score s[h, j] = scale * (q_lat[h] . c_lat[j] + q_rope[h] . k_rope[j]);
    softmax over j; the value of token j is its latent slice c_lat[j].
    Returns (o [H, d_s], lse [H]); L = 0 gives o = 0 and lse = -inf.
    """
    q_lat = np.asarray(q_lat, np.float64)
    q_rope = np.asarray(q_rope, np.float64)
    c_lat = np.asarray(c_lat, np.float64)
    k_rope = np.asarray(k_rope, np.float64)
    H = q_lat.shape[0]
    if c_lat.shape[0] == 0:
        return np.zeros((H, c_lat.shape[1])), np.full(H, -np.inf)
    s = scale * (q_lat @ c_lat.T + q_rope @ k_rope.T)          # [H, L]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    o = (w @ c_lat) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine attention over disjoint token sets given each set's (o, lse).

    LSE = log sum_s exp(lse_s); o = sum_s exp(lse_s - LSE) * o_s.  Parts with
    lse = -inf (no tokens) carry no weight.
    """
    lse_parts = np.asarray(lse_parts, np.float64)          # [S, H]
    o_parts = np.asarray(o_parts, np.float64)              # [S, H, d]
    m = lse_parts.max(axis=0)                              # [H]
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - safe_m), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(tot > 0, safe_m + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    o = np.einsum("sh,shd->hd", w, o_parts) / np.where(tot > 0, tot, 1.0)[:, None]
    return o, lse


# ---------------------------------------------------------------------------
# TPLA: rotate, slice, attend per shard, combine  ([ABS], [ABS-R], [BLOG])
# ---------------------------------------------------------------------------

def shard_slice(x: np.ndarray, g: int, tp: int) -> np.ndarray:
    """Columns g*d_s .. (g+1)*d_s of the last axis, d_s = d_c / tp."""
    d_c = x.shape[-1]
    if d_c % tp:
        raise ValueError("latent width not divisible by tp")
    d_s = d_c // tp
    return x[..., g * d_s:(g + 1) * d_s]


def tpla_shards(q_lat, q_rope, c_lat, k_rope, tp: int, scale: float, hadamard: bool,
                rope_split: bool = False, latent_mult: float = 1.0):
    """Per-shard outputs of TPLA for one sequence.

    q_lat [H, d_c] (absorbed query, latent space), q_rope [H, d_r],
    c_lat [L, d_c] (cached latent cKV), k_rope [L, d_r].
    Step 1 (optional): rotate query and latent by the orthonormal Hadamard
    over the full latent width.  Step 2: slice both along the latent into tp
    shards; every head keeps all its shards.  Step 3: each shard attends on
    its own (own softmax).  Returns a list of (o_g [H, d_s], lse_g [H]).

    Two other readings of the pages, for diagnostics only (the defaults are
    readings R1 and R2): rope_split gives each shard its d_r / tp slice of
    the rope query and key instead of the whole rope; latent_mult multiplies
    each shard's latent score term (latent_mult = tp makes a shard's partial
    score an estimate of the whole latent score).
    """
    if hadamard:
        q_lat = fwht(q_lat)
        c_lat = fwht(c_lat)
    out = []
    for g in range(tp):
        qr, kr = ((shard_slice(q_rope, g, tp), shard_slice(k_rope, g, tp)) if rope_split
                  else (q_rope, k_rope))
        out.append(shard_attention(latent_mult * shard_slice(q_lat, g, tp), qr,
                                   shard_slice(c_lat, g, tp), kr, scale))
    return out


def combine_shards(o_shards) -> np.ndarray:
    """The all-reduce: sum over shards of each output zero-padded to d_c.

    o_shards is a sequence of arrays [..., d_s]; shard g occupies columns
    g*d_s .. (g+1)*d_s of the result.
    """
    tp = len(o_shards)
    d_s = o_shards[0].shape[-1]
    out = np.zeros(o_shards[0].shape[:-1] + (tp * d_s,))
    for g, o in enumerate(o_shards):
        padded = np.zeros_like(out)
        padded[..., g * d_s:(g + 1) * d_s] = o
        out += padded
    return out


def tpla_decode(q_lat, q_rope, c_lat, k_rope, tp: int, scale: float,
                hadamard: bool, unrotate: bool = False) -> np.ndarray:
    """Full TPLA decode for one sequence: [H, d_c] output.

    With hadamard=True the result is in the rotated basis unless
    unrotate=True, which applies the (self-inverse) transform once more.
    """
    parts = tpla_shards(q_lat, q_rope, c_lat, k_rope, tp, scale, hadamard)
    out = combine_shards([o for o, _ in parts])
    if hadamard and unrotate:
        out = fwht(out)
    return out


def tpla_decode_paged(q_lat_shard, q_rope, cache, block_table, seq_lens,
                      block_size: int, d_s: int, scale: float):
    """One shard over a paged cache, every sequence of the batch.

    q_lat_shard [B, H, d_s] (already rotated and sliced), q_rope [B, H, d_r],
    cache [num_blocks, block_size, d_s + d_r].  Returns (o [B, H, d_s],
    lse [B, H]).
    """
    q_lat_shard = np.asarray(q_lat_shard, np.float64)
    q_rope = np.asarray(q_rope, np.float64)
    B, H, _ = q_lat_shard.shape
    o = np.zeros((B, H, d_s))
    lse = np.zeros((B, H))
    for b in range(B):
        rows = gather_sequence(cache, block_table, b, int(seq_lens[b]), block_size)
        o[b], lse[b] = shard_attention(q_lat_shard[b], q_rope[b], rows[:, :d_s],
                                       rows[:, d_s:], scale)
    return o, lse


# ---------------------------------------------------------------------------
# Plain MLA decode (the T = 1 case, and the un-absorbed textbook form)
# ---------------------------------------------------------------------------

def mla_decode(q_lat, q_rope, c_lat, k_rope, scale: float):
    """Absorbed MLA decode for one sequence: every head attends over the
    whole latent (no slicing, no rotation).  Returns (o [H, d_c], lse [H])."""
    return shard_attention(q_lat, q_rope, c_lat, k_rope, scale)


def mla_decode_unabsorbed(q_nope, q_rope, c_lat, k_rope, w_uk, w_uv, scale: float):
    """MLA with explicit per-head keys and values up-projected from the latent.

    q_nope [H, d_n], q_rope [H, d_r], c_lat [L, d_c], k_rope [L, d_r],
    w_uk [H, d_n, d_c], w_uv [H, d_v, d_c].  Head h: key_j = w_uk[h] @ c_j
    (plus the shared rope key), value_j = w_uv[h] @ c_j.  Returns [H, d_v].
    """
    H = q_nope.shape[0]
    c_lat = np.asarray(c_lat, np.float64)
    out = np.zeros((H, w_uv.shape[1]))
    for h in range(H):
        keys = c_lat @ np.asarray(w_uk[h], np.float64).T         # [L, d_n]
        vals = c_lat @ np.asarray(w_uv[h], np.float64).T         # [L, d_v]
        s = scale * (keys @ q_nope[h] + k_rope @ q_rope[h])
        w = np.exp(s - s.max())
        out[h] = (w / w.sum()) @ vals
    return out


# ---------------------------------------------------------------------------
# MLA-form prefill ([ABS-R]: MLA kept for the compute-bound prefill; [BLOG]
# "Prefill-Decode Separation for Optimal Performance")
# ---------------------------------------------------------------------------

def mla_prefill(q_lat, q_rope, c_lat, k_rope, scale: float):
    """Causal attention of one prompt in the MLA form.

    q_lat [S, H, d_c], q_rope [S, H, d_r], c_lat [S, d_c], k_rope [S, d_r].
    Position t, head h: s[t, h, j] = scale * (q_lat[t, h] . c_lat[j] +
    q_rope[t, h] . k_rope[j]) for j <= t (later positions are not seen);
    softmax over j; the value of position j is its whole latent row.
    Returns (o [S, H, d_c], lse [S, H]).
    """
    q_lat = np.asarray(q_lat, np.float64)
    q_rope = np.asarray(q_rope, np.float64)
    c_lat = np.asarray(c_lat, np.float64)
    k_rope = np.asarray(k_rope, np.float64)
    S = c_lat.shape[0]
    s = scale * (np.einsum("thk,jk->thj", q_lat, c_lat) +
                 np.einsum("thk,jk->thj", q_rope, k_rope))          # [S, H, S]
    later = np.arange(S)[None, :] > np.arange(S)[:, None]           # [t, j]: j > t
    s = np.where(later[:, None, :], -np.inf, s)
    m = s.max(axis=2, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=2, keepdims=True)
    o = np.einsum("thj,jk->thk", w, c_lat) / l
    lse = (m + np.log(l))[:, :, 0]
    return o, lse


# ---------------------------------------------------------------------------
# RMSNorm slicing ([BLOG] "How TPLA Works: Smart Slicing and
# Reparameterization": a latent split across devices would be normalised
# with only part of the data; an orthogonal transform applied before the
# split makes those local statistics approximate the global ones.  [ABS-R]:
# the reparameterisation of RMSNorm.)
# ---------------------------------------------------------------------------

def rms_normalize(y: np.ndarray, eps: float) -> np.ndarray:
    """Global RMS norm over the last axis: y / sqrt(mean(y**2) + eps)."""
    y = np.asarray(y, dtype=np.float64)
    ms = np.mean(y * y, axis=-1, keepdims=True)
    return y / np.sqrt(ms + eps)


def slice_rms_normalize(y: np.ndarray, d_s: int, eps: float) -> np.ndarray:
    """RMSNorm slicing: every block of d_s consecutive columns of the last
    axis is divided by the RMS of that block alone (reading R10)."""
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[-1]
    if d_s < 1 or n % d_s != 0:
        raise ValueError(f"slice width {d_s} must divide {n}")
    blocks = y.reshape(*y.shape[:-1], n // d_s, d_s)
    ms = np.mean(blocks * blocks, axis=-1, keepdims=True)
    return (blocks / np.sqrt(ms + eps)).reshape(y.shape)


def rotate_normalize_latent(x: np.ndarray, mode: str, d_s: int, eps: float,
                            hadamard: bool = True) -> np.ndarray:
    """The cached latent from the down-projected one: rotate (or not), then
    normalise globally ("global"), per d_s slice ("slice") or not ("none")."""
    y = fwht(x) if hadamard else np.asarray(x, dtype=np.float64)
    if mode == "none":
        return y
    if mode == "global":
        return rms_normalize(y, eps)
    if mode == "slice":
        return slice_rms_normalize(y, d_s, eps)
    raise ValueError(f"unknown mode {mode!r}")


# ---------------------------------------------------------------------------
# Value up-projection per shard and the all-reduce sum ([ABS]: each shard's
# attention runs on its own and the results are combined with an
# all-reduce; [ABS-R]: the orthogonal reparameterisation keeps MLA's
# weights usable).  In MLA the head-h value of token t is W_UV[h] @ c_t, so
# head h's output is W_UV[h] @ (sum_t p_t c_t): the latent-space output
# times the head's W_UV.
# ---------------------------------------------------------------------------

def up_project_shard(o_shard: np.ndarray, w_shard: np.ndarray) -> np.ndarray:
    """One device's up-projected output: y[b, h, :] = o[b, h, :] @ w[h].

    o_shard [B, H, d_s] (this device's latent-space attention output),
    w_shard [H, d_s, d_v] (its rows of every head's transposed W_UV).
    """
    o = np.asarray(o_shard, dtype=np.float64)
    w = np.asarray(w_shard, dtype=np.float64)
    # per head: [B, d_s] @ [d_s, d_v]
    return np.matmul(o.transpose(1, 0, 2), w).transpose(1, 0, 2)


def up_project_combine(o_shards, w_shards) -> np.ndarray:
    """The all-reduce: sum over devices of up_project_shard (reading R11)."""
    parts = [up_project_shard(o, w) for o, w in zip(o_shards, w_shards)]
    out = np.zeros_like(parts[0])
    for y in parts:
        out = out + y
    return out


def rotate_weight_rows(w_t: np.ndarray) -> np.ndarray:
    """Transposed W_UV [H, d_c, d_v] for a latent rotated by Hn: Hn @ w_t[h].

    With c~ = c @ Hn the latent-space output is o~ = o @ Hn, and
    o @ w_t = o~ @ (Hn^T @ w_t) = o~ @ (Hn @ w_t) since Hn is symmetric and
    orthonormal.  Hn @ w_t[h] is the transform applied along the d_c axis.
    """
    w = np.asarray(w_t, dtype=np.float64)
    return fwht(w.transpose(0, 2, 1)).transpose(0, 2, 1)
