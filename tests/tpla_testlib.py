"""Helpers shared by the GPU tests: upload seeded inputs, run the library's
pipeline, and build the oracle's reference for the same inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from tensor_latent_decode_amd import tpla
from tensor_latent_decode_amd.inputs import Case

# max|gpu - ref| / max|ref| for bf16 inputs with float32 accumulation
TOL_BF16 = 5e-3
TOL_FP32 = 1e-5


def dev(a: np.ndarray) -> torch.Tensor:
    """Host array -> device tensor (uint16 arrays are bf16 bit patterns)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array of its exact bits (uint16 for bf16)."""
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    denom = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (denom if denom > 0 else 1.0)


def torch_dtype(case: Case):
    return torch.bfloat16 if case.cfg.dtype == "bf16" else torch.float32


def empty_cache(case: Case, d_s: int) -> torch.Tensor:
    """Paged cache filled with NaN, so a read of a never-written row shows."""
    shape = (case.num_blocks, case.cfg.block_size, d_s + case.cfg.d_r)
    if case.cfg.dtype == "bf16":
        return torch.full(shape, -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


class GpuCase:
    """The case's inputs on the device."""

    def __init__(self, case: Case):
        self.case = case
        self.bt = dev(case.block_table)
        self.hist_seq = dev(case.hist_seq)
        self.hist_pos = dev(case.hist_pos)
        self.hist_latent = dev(case.hist_latent)
        self.hist_rope = dev(case.hist_rope)
        self.new_latent = dev(case.new_latent)
        self.new_rope = dev(case.new_rope)
        self.new_seq = torch.arange(case.cfg.batch, dtype=torch.int32, device="cuda")
        self.new_pos = dev(case.new_pos)
        self.q_latent = dev(case.q_latent)
        self.q_rope = dev(case.q_rope)
        self.seq_lens = dev(case.seq_lens)
        self.hist_lens = dev((case.seq_lens - 1).astype(np.int32))

    def prefill(self, g: int, d_s: int) -> torch.Tensor:
        """Shard g's cache holding the history rows (written by tpla_append_kv)."""
        cache = empty_cache(self.case, d_s)
        if self.hist_latent.shape[0] > 0:
            tpla.append_kv(cache, self.bt, self.hist_seq, self.hist_pos,
                           self.hist_latent[:, g * d_s:(g + 1) * d_s], self.hist_rope)
        return cache


def oracle_rows(case: Case, b: int):
    """History rows of sequence b in float64 (rotated basis), and rope."""
    start = int(np.sum(case.seq_lens[:b] - 1))
    n = int(case.seq_lens[b] - 1)
    return as_f64(case.hist_latent[start:start + n]), as_f64(case.hist_rope[start:start + n])


def oracle_step(case: Case, b: int, tp: int, hadamard: bool, with_new: bool = True,
                q_is_rotated: bool = False):
    """Reference for one sequence of a decode step, every shard.

    The query and the new token's latent are rotated by the oracle's own
    transform (unless q_is_rotated), the history rows are taken as stored;
    then slice, attend per shard and combine (TPLA abstract).  Returns
    (combined [H, d_c], [(o_g, lse_g)]).
    """
    lat, rope = oracle_rows(case, b)
    q = as_f64(case.q_latent[b])
    if hadamard and not q_is_rotated:
        q = oracle.fwht(q)
    if with_new:
        new = as_f64(case.new_latent[b])[None]
        if hadamard:
            new = oracle.fwht(new)
        lat = np.concatenate([lat, new])
        rope = np.concatenate([rope, as_f64(case.new_rope[b])[None]])
    qr = as_f64(case.q_rope[b])
    parts = [oracle.shard_attention(oracle.shard_slice(q, g, tp), qr,
                                    oracle.shard_slice(lat, g, tp), rope, case.cfg.scale)
             for g in range(tp)]
    return oracle.combine_shards([o for o, _ in parts]), parts
