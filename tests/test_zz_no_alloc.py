"""tpla_decode_shard_noalloc, the decode entry point that allocates nothing.

It runs the kernels of tpla_decode_shard with the split outputs in the
library's static device scratch instead of a caller's workspace, so on the
same inputs and split count both give the same bits.  Each test makes two
calls in a row through the C ABI, the second one smaller than the first
(the scratch then holds the first call's leftovers), and checks both
against tpla_decode_shard and, on sampled sequences, against the oracle.
"""
import numpy as np
import pytest
import torch

from tensor_latent_decode_amd import tpla
from tensor_latent_decode_amd.inputs import CONFIGS, make_case
from tpla_testlib import TOL_BF16, GpuCase, host_f64, oracle_step, rel_err

pytestmark = pytest.mark.gpu


def _shard(case, g, hadamard):
    """Shard g's cache with the history and the new token, and its query slice
    (rotated if hadamard; a latent width that is no power of two is not)."""
    gc = GpuCase(case)
    d_s = case.cfg.d_s
    q = tpla.hadamard_latent(gc.q_latent) if hadamard else gc.q_latent
    new = tpla.hadamard_latent(gc.new_latent) if hadamard else gc.new_latent
    cache = gc.prefill(g, d_s)
    tpla.append_kv(cache, gc.bt, gc.new_seq, gc.new_pos, new[:, g * d_s:(g + 1) * d_s], gc.new_rope)
    return gc, q[:, :, g * d_s:(g + 1) * d_s].contiguous(), cache


def _both(case, g, num_splits, hadamard):
    """(noalloc out, noalloc lse, workspace out, workspace lse) of shard g."""
    gc, q, cache = _shard(case, g, hadamard)
    cfg = case.cfg
    B, H, d_s = cfg.batch, cfg.heads, cfg.d_s
    maxlen = int(case.seq_lens.max())
    res = []
    for noalloc in (True, False):
        # poisoned outputs: every element must be written
        out = torch.full((B, H, d_s), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            tpla.decode_shard_noalloc(q, gc.q_rope, cache, gc.bt, gc.seq_lens, cfg.scale, maxlen,
                                      out, lse, num_splits)
        else:
            tpla.decode_shard(q, gc.q_rope, cache, gc.bt, gc.seq_lens, cfg.scale, maxlen,
                              out=out, lse=lse, num_splits=num_splits)
        torch.cuda.synchronize()
        res += [out.cpu().numpy(), lse.cpu().numpy()]
    return res


def _check(case, g, sample, num_splits=0, hadamard=True):
    print(f"noalloc: {case.cfg.name} batch {case.cfg.batch} shard {g} splits {num_splits}", flush=True)
    o_n, l_n, o_w, l_w = _both(case, g, num_splits, hadamard)
    assert np.array_equal(o_n.view(np.uint32), o_w.view(np.uint32))
    assert np.array_equal(l_n.view(np.uint32), l_w.view(np.uint32))
    for b in sample:
        _, parts = oracle_step(case, b, case.cfg.tp, hadamard=hadamard)
        assert rel_err(o_n[b].astype(np.float64), parts[g][0]) <= TOL_BF16, b
        assert np.max(np.abs(l_n[b] - parts[g][1])) <= 2e-2, b


def test_noalloc_matches_workspace_call_large_then_small():
    """The bench's shard shape at full size, then a small ragged batch."""
    big = make_case(CONFIGS["dsv3_32k"])
    _check(big, 0, sample=(0, big.cfg.batch - 1))
    small = make_case(CONFIGS["dsv3_4k"], batch=3, ctx=(1, 3000), seed=91)
    _check(small, 1, sample=range(3), num_splits=3)


def test_noalloc_other_kernels_large_then_small():
    """A 64-head shard (its own streaming kernel), then a float32-kernel shape."""
    from dataclasses import replace
    kimi = make_case(CONFIGS["kimi_k2_32k"], batch=4, ctx=(9000, 20000), seed=92)
    _check(kimi, 2, sample=(0, 3))
    odd = replace(CONFIGS["dsv3_4k"], heads=5, d_c=80, tp=2, d_r=8, scale=0.2)
    small = make_case(odd, batch=2, ctx=(1, 300), seed=93)
    _check(small, 0, sample=range(2), num_splits=2, hadamard=False)
