"""Pins of the fp64 oracle against things other than itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped rope
term, a wrong sign or index, a transposed operand, a wrong Hadamard order or
normalisation, a wrong slice offset, a broken merge) makes at least one fail:

* library routines: scipy.linalg.hadamard, torch scaled_dot_product_attention
  (float64, CPU), torch's float32 -> bfloat16 cast;
* closed forms and hand-worked examples (tests/golden/worked_examples.json);
* invariants the method states or implies (T = 1 equals MLA; a shared
  orthogonal transform leaves scores unchanged; absorbed = un-absorbed MLA);
* brute force with scalar Python loops on tiny inputs.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from tensor_latent_decode_amd.inputs import CONFIGS, make_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# Hadamard
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 128, 512, 1024])
def test_hadamard_matrix_is_sylvester_and_orthogonal(n):
    h = oracle.sylvester_hadamard(n)
    np.testing.assert_array_equal(h, scipy.linalg.hadamard(n))
    np.testing.assert_array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


@pytest.mark.parametrize("n", [2, 4, 16, 64, 256, 512])
def test_fwht_equals_dense_library_product(n):
    x = _rng(n).standard_normal((7, n))
    dense = x @ scipy.linalg.hadamard(n).astype(np.float64) / math.sqrt(n)
    y = oracle.fwht(x)
    assert np.max(np.abs(y - dense)) <= 1e-12 * max(1.0, np.max(np.abs(dense)))


def test_fwht_self_inverse_norm_preserving_and_batched():
    x = _rng(3).standard_normal((2, 3, 512))
    y = oracle.fwht(x)
    np.testing.assert_allclose(oracle.fwht(y), x, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-13)
    for i in range(2):
        for j in range(3):
            np.testing.assert_array_equal(y[i, j], oracle.fwht(x[i, j]))


def test_fwht_golden():
    for ex in json.load(open(GOLDEN))["fwht"]:
        np.testing.assert_allclose(oracle.fwht(np.array(ex["x"], float)), ex["y"],
                                   rtol=0, atol=1e-15)


def test_fwht_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.fwht(np.zeros(12))


# --------------------------------------------------------------------------
# bf16 storage
# --------------------------------------------------------------------------

def test_bf16_round_matches_torch_cast():
    rng = _rng(11)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
    ])
    # exact ties: low 16 bits == 0x8000, with even and odd kept parts
    tie_bits = (rng.integers(0, 1 << 15, 4000, dtype=np.uint32) << 16) | 0x8000
    tie_bits = tie_bits[(tie_bits >> 23) & 0xFF != 0xFF]      # finite values only
    x = np.concatenate([x, tie_bits.astype(np.uint32).view(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 65504.0], np.float32)])
    ours = oracle.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_bits_to_f64_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # drop inf/nan patterns
    ours = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


# --------------------------------------------------------------------------
# Shard attention
# --------------------------------------------------------------------------

def _sdpa(q_lat, q_rope, c_lat, k_rope, scale):
    """Library attention: q = [q_lat || q_rope], k = [c || r], v = c."""
    q = torch.from_numpy(np.concatenate([q_lat, q_rope], axis=1))[None, :, None, :]
    k = torch.from_numpy(np.concatenate([c_lat, k_rope], axis=1))[None, None]
    v = torch.from_numpy(np.ascontiguousarray(c_lat))[None, None]
    H = q.shape[1]
    k = k.expand(1, H, -1, -1).contiguous()
    v = v.expand(1, H, -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("H,d_s,d_r,L", [(4, 32, 16, 128), (3, 8, 4, 1), (5, 16, 0, 37),
                                         (2, 64, 64, 300)])
def test_shard_attention_matches_library_sdpa(H, d_s, d_r, L):
    rng = _rng(H * 1000 + L)
    ql, qr = rng.standard_normal((H, d_s)), rng.standard_normal((H, d_r))
    c, r = rng.standard_normal((L, d_s)), rng.standard_normal((L, d_r))
    scale = 1.0 / math.sqrt(d_s + d_r)
    o, _ = oracle.shard_attention(ql, qr, c, r, scale)
    np.testing.assert_allclose(o, _sdpa(ql, qr, c, r, scale), rtol=0, atol=1e-12)


def test_shard_attention_brute_force_loops():
    rng = _rng(5)
    H, d_s, d_r, L = 2, 3, 2, 5
    ql, qr = rng.standard_normal((H, d_s)), rng.standard_normal((H, d_r))
    c, r = rng.standard_normal((L, d_s)), rng.standard_normal((L, d_r))
    scale = 0.37
    o, lse = oracle.shard_attention(ql, qr, c, r, scale)
    for h in range(H):
        s = []
        for j in range(L):
            acc = math.fsum(ql[h][k] * c[j][k] for k in range(d_s))
            acc += math.fsum(qr[h][k] * r[j][k] for k in range(d_r))
            s.append(scale * acc)
        z = math.fsum(math.exp(v) for v in s)
        assert abs(lse[h] - math.log(z)) < 1e-13
        for k in range(d_s):
            ref = math.fsum(math.exp(s[j]) * c[j][k] for j in range(L)) / z
            assert abs(o[h][k] - ref) < 1e-13


def test_shard_attention_golden():
    for ex in json.load(open(GOLDEN))["attention"]:
        o, lse = oracle.shard_attention(np.array(ex["q_lat"]), np.array(ex["q_rope"]),
                                        np.array(ex["c_lat"]), np.array(ex["k_rope"]),
                                        ex["scale"])
        np.testing.assert_allclose(o, ex["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, ex["lse"], rtol=0, atol=1e-14)


def test_single_token_closed_form():
    rng = _rng(6)
    ql, qr = rng.standard_normal((4, 8)), rng.standard_normal((4, 3))
    c, r = rng.standard_normal((1, 8)), rng.standard_normal((1, 3))
    o, lse = oracle.shard_attention(ql, qr, c, r, 0.5)
    np.testing.assert_allclose(o, np.repeat(c, 4, axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * (ql @ c[0] + qr @ r[0]), rtol=0, atol=1e-15)


def test_zero_query_gives_mean_and_log_length():
    rng = _rng(7)
    L = 97
    c, r = rng.standard_normal((L, 16)), rng.standard_normal((L, 4))
    o, lse = oracle.shard_attention(np.zeros((3, 16)), np.zeros((3, 4)), c, r, 0.3)
    np.testing.assert_allclose(o, np.repeat(c.mean(axis=0, keepdims=True), 3, 0),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.full(3, math.log(L)), rtol=0, atol=1e-13)


def test_empty_sequence():
    o, lse = oracle.shard_attention(np.ones((2, 4)), np.ones((2, 2)), np.zeros((0, 4)),
                                    np.zeros((0, 2)), 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_constant_rope_key_only_shifts_lse():
    rng = _rng(8)
    L, H = 50, 3
    ql, qr = rng.standard_normal((H, 8)), rng.standard_normal((H, 4))
    c = rng.standard_normal((L, 8))
    r_row = rng.standard_normal(4)
    r = np.repeat(r_row[None], L, axis=0)
    o1, lse1 = oracle.shard_attention(ql, qr, c, r, 0.4)
    o0, lse0 = oracle.shard_attention(ql, np.zeros_like(qr), c, r, 0.4)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse1 - lse0, 0.4 * (qr @ r_row), rtol=0, atol=1e-13)


def test_rope_term_is_not_dropped():
    rng = _rng(9)
    ql, qr = rng.standard_normal((2, 8)), rng.standard_normal((2, 4)) * 3
    c, r = rng.standard_normal((20, 8)), rng.standard_normal((20, 4))
    o1, _ = oracle.shard_attention(ql, qr, c, r, 0.5)
    o0, _ = oracle.shard_attention(ql, np.zeros_like(qr), c, r, 0.5)
    assert np.max(np.abs(o1 - o0)) > 1e-2


# --------------------------------------------------------------------------
# Split-K merge
# --------------------------------------------------------------------------

def test_merge_over_any_partition_equals_unsplit():
    rng = _rng(10)
    L, H = 200, 4
    ql, qr = rng.standard_normal((H, 16)), rng.standard_normal((H, 4))
    c, r = rng.standard_normal((L, 16)), rng.standard_normal((L, 4))
    o_ref, lse_ref = oracle.shard_attention(ql, qr, c, r, 0.25)
    for cuts in ([0, 200], [0, 64, 128, 200], [0, 1, 2, 3, 199, 200], [0, 0, 70, 70, 200]):
        os_, ls_ = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            o, l = oracle.shard_attention(ql, qr, c[a:b], r[a:b], 0.25)
            os_.append(o)
            ls_.append(l)
        o, lse = oracle.merge_partials(os_, ls_)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)


def test_merge_all_empty():
    o, lse = oracle.merge_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(lse == -np.inf)


# --------------------------------------------------------------------------
# TPLA slicing and combine
# --------------------------------------------------------------------------

def test_tp1_equals_mla():
    rng = _rng(12)
    ql, qr = rng.standard_normal((4, 64)), rng.standard_normal((4, 16))
    c, r = rng.standard_normal((128, 64)), rng.standard_normal((128, 16))
    ref, _ = oracle.mla_decode(ql, qr, c, r, 0.2)
    out = oracle.tpla_decode(ql, qr, c, r, tp=1, scale=0.2, hadamard=False)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out, _sdpa(ql, qr, c, r, 0.2), rtol=0, atol=1e-12)


def test_tp1_orthogonal_invariance():
    rng = _rng(13)
    ql, qr = rng.standard_normal((4, 64)), rng.standard_normal((4, 16))
    c, r = rng.standard_normal((128, 64)), rng.standard_normal((128, 16))
    ref, lse_ref = oracle.mla_decode(ql, qr, c, r, 0.2)
    rotated = oracle.tpla_decode(ql, qr, c, r, tp=1, scale=0.2, hadamard=True)
    back = oracle.tpla_decode(ql, qr, c, r, tp=1, scale=0.2, hadamard=True, unrotate=True)
    np.testing.assert_allclose(back, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(rotated @ scipy.linalg.hadamard(64) / 8.0, ref, rtol=0, atol=1e-12)
    (_, lse_rot), = oracle.tpla_shards(ql, qr, c, r, 1, 0.2, True)
    np.testing.assert_allclose(lse_rot, lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("tp,g0", [(2, 0), (2, 1), (4, 2)])
def test_query_on_one_shard_reduces_to_library_attention(tp, g0, hadamard):
    """If the (rotated) latent query lives in shard g0's columns only, shard
    g0 sees the full MLA score and its output is library attention on its
    slice; every other shard sees only the rope score."""
    rng = _rng(100 * tp + g0)
    H, d_c, d_r, L = 3, 64, 8, 90
    d_s = d_c // tp
    q_rot = np.zeros((H, d_c))
    q_rot[:, g0 * d_s:(g0 + 1) * d_s] = rng.standard_normal((H, d_s))
    c_rot = rng.standard_normal((L, d_c))
    qr, r = rng.standard_normal((H, d_r)), rng.standard_normal((L, d_r))
    hd = scipy.linalg.hadamard(d_c).astype(float) / math.sqrt(d_c)
    # inputs in the unrotated basis when the method rotates them itself
    q_in, c_in = (q_rot @ hd, c_rot @ hd) if hadamard else (q_rot, c_rot)
    scale = 0.3
    parts = oracle.tpla_shards(q_in, qr, c_in, r, tp, scale, hadamard)
    full = _sdpa(q_rot, qr, c_rot, r, scale)     # MLA in the rotated basis
    for g, (o, _) in enumerate(parts):
        sl = slice(g * d_s, (g + 1) * d_s)
        if g == g0:
            np.testing.assert_allclose(o, full[:, sl], rtol=0, atol=1e-11)
        else:
            ref = _sdpa(np.zeros((H, d_s)), qr, c_rot[:, sl], r, scale)
            np.testing.assert_allclose(o, ref, rtol=0, atol=1e-11)
    combined = oracle.tpla_decode(q_in, qr, c_in, r, tp, scale, hadamard)
    np.testing.assert_allclose(combined[:, g0 * d_s:(g0 + 1) * d_s], full[:, g0 * d_s:(g0 + 1) * d_s],
                               rtol=0, atol=1e-11)


def test_two_shard_golden():
    ex = json.load(open(GOLDEN))["tpla_two_shards"]
    parts = oracle.tpla_shards(np.array(ex["q_lat"]), np.array(ex["q_rope"]),
                               np.array(ex["c_lat"]), np.array(ex["k_rope"]),
                               ex["tp"], ex["scale"], False)
    np.testing.assert_allclose(parts[0][0], ex["shard0_o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(parts[0][1], ex["shard0_lse"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(parts[1][0], ex["shard1_o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(parts[1][1], ex["shard1_lse"], rtol=0, atol=1e-15)
    combined = oracle.combine_shards([p[0] for p in parts])
    assert combined.shape == (1, 4)
    np.testing.assert_allclose(combined, ex["combined"], rtol=0, atol=1e-15)


def test_combine_is_concatenation():
    rng = _rng(14)
    parts = [rng.standard_normal((2, 3, 8)) for _ in range(4)]
    np.testing.assert_array_equal(oracle.combine_shards(parts), np.concatenate(parts, axis=-1))


def test_absorbed_mla_equals_unabsorbed():
    rng = _rng(15)
    H, d_n, d_c, d_r, d_v, L = 3, 16, 32, 8, 12, 40
    q_nope, q_rope = rng.standard_normal((H, d_n)), rng.standard_normal((H, d_r))
    c, r = rng.standard_normal((L, d_c)), rng.standard_normal((L, d_r))
    w_uk = rng.standard_normal((H, d_n, d_c)) / 4
    w_uv = rng.standard_normal((H, d_v, d_c)) / 4
    scale = 1 / math.sqrt(d_n + d_r)
    ref = oracle.mla_decode_unabsorbed(q_nope, q_rope, c, r, w_uk, w_uv, scale)
    q_lat = np.einsum("hn,hnc->hc", q_nope, w_uk)               # absorb W_UK into the query
    o_lat, _ = oracle.mla_decode(q_lat, q_rope, c, r, scale)
    out = np.einsum("hc,hvc->hv", o_lat, w_uv)                    # W_UV after attention
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# Paged cache
# --------------------------------------------------------------------------

def _fill(case, dtype):
    d_s = case.cfg.d_s
    width = d_s + case.cfg.d_r
    cache = np.full((case.num_blocks, case.cfg.block_size, width),
                    0xFFFF if dtype == np.uint16 else np.nan, dtype=dtype)
    return cache


def test_paged_append_and_gather_roundtrip_and_permutation_invariance():
    case = make_case(CONFIGS["tiny_fp32"], block_size=16, batch=3, ctx=(20, 70), seed=21)
    d_s = case.cfg.d_s
    for g in range(case.cfg.tp):
        lat = case.hist_latent[:, g * d_s:(g + 1) * d_s]
        cache = _fill(case, np.float32)
        oracle.paged_append(cache, case.block_table, 16, case.hist_seq, case.hist_pos,
                            lat, case.hist_rope)
        # a different physical placement of the same logical rows
        perm = np.random.default_rng(3).permutation(case.num_blocks - 1)
        bt2 = np.where(case.block_table == case.num_blocks - 1, case.num_blocks - 1,
                       perm[np.minimum(case.block_table, case.num_blocks - 2)])
        cache2 = _fill(case, np.float32)
        oracle.paged_append(cache2, bt2, 16, case.hist_seq, case.hist_pos, lat, case.hist_rope)
        off = 0
        for b in range(case.cfg.batch):
            n = int(case.seq_lens[b]) - 1
            rows = oracle.gather_sequence(cache, case.block_table, b, n, 16)
            rows2 = oracle.gather_sequence(cache2, bt2, b, n, 16)
            np.testing.assert_array_equal(rows[:, :d_s], lat[off:off + n])
            np.testing.assert_array_equal(rows[:, d_s:], case.hist_rope[off:off + n])
            np.testing.assert_array_equal(rows, rows2)
            off += n
        # unused slots were never written
        used = set()
        for b in range(case.cfg.batch):
            for j in range(int(case.seq_lens[b]) - 1):
                used.add(oracle.page_slot(case.block_table, b, j, 16))
        flat = cache.reshape(-1, cache.shape[-1])
        unused = [s for s in range(flat.shape[0]) if s not in used]
        assert np.all(np.isnan(flat[unused]))


def test_paged_append_bf16_bits_and_fp32_source_rounding():
    case = make_case(CONFIGS["dsv3_4k"], ctx=100, seed=22, heads=4)
    cache = np.full((case.num_blocks, 64, 320), 0xFFFF, np.uint16)
    lat = case.hist_latent[:, :256]
    oracle.paged_append(cache, case.block_table, 64, case.hist_seq, case.hist_pos,
                        lat, case.hist_rope)
    rows = cache.reshape(-1, 320)[[oracle.page_slot(case.block_table, 0, j, 64)
                                   for j in range(99)]]
    np.testing.assert_array_equal(rows[:, :256], lat)
    src = np.random.default_rng(1).standard_normal((1, 256)).astype(np.float32)
    oracle.paged_append(cache, case.block_table, 64, np.array([0]), np.array([99]),
                        src, np.zeros((1, 64), np.float32))
    got = cache.reshape(-1, 320)[oracle.page_slot(case.block_table, 0, 99, 64), :256]
    ref = torch.from_numpy(src[0]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_paged_decode_matches_logical_decode():
    case = make_case(CONFIGS["tiny_fp32"], batch=2, ctx=(60, 130), seed=23, block_size=16)
    cfg = case.cfg
    d_s = cfg.d_s
    for g in range(cfg.tp):
        cache = _fill(case, np.float32)
        oracle.paged_append(cache, case.block_table, 16, case.hist_seq, case.hist_pos,
                            case.hist_latent[:, g * d_s:(g + 1) * d_s], case.hist_rope)
        lens = case.seq_lens - 1
        ql = case.q_latent[..., g * d_s:(g + 1) * d_s]
        o, lse = oracle.tpla_decode_paged(ql, case.q_rope, cache, case.block_table, lens,
                                          16, d_s, cfg.scale)
        off = 0
        for b in range(cfg.batch):
            n = int(lens[b])
            ref_o, ref_l = oracle.shard_attention(
                ql[b], case.q_rope[b], case.hist_latent[off:off + n, g * d_s:(g + 1) * d_s],
                case.hist_rope[off:off + n], cfg.scale)
            np.testing.assert_array_equal(o[b], ref_o)
            np.testing.assert_array_equal(lse[b], ref_l)
            off += n


# --------------------------------------------------------------------------
# RMSNorm slicing (global RMS norm vs per-slice RMS norm of the rotated latent)
# --------------------------------------------------------------------------

def test_rms_norm_closed_form_two_levels():
    # slices of constant magnitude 1 and 3: the global RMS is sqrt(5), each
    # slice's own RMS is its constant
    x = np.array([1.0] * 256 + [-3.0] * 256)
    g = oracle.rms_normalize(x, 0.0)
    np.testing.assert_allclose(g[:256], 1 / math.sqrt(5), rtol=0, atol=1e-15)
    np.testing.assert_allclose(g[256:], -3 / math.sqrt(5), rtol=0, atol=1e-15)
    s = oracle.slice_rms_normalize(x, 256, 0.0)
    np.testing.assert_allclose(s, np.sign(x), rtol=0, atol=1e-15)
    eps = 0.5
    np.testing.assert_allclose(oracle.slice_rms_normalize(x, 256, eps)[:2], 1 / math.sqrt(1.5), rtol=1e-15)
    np.testing.assert_allclose(oracle.slice_rms_normalize(x, 256, eps)[-1], -3 / math.sqrt(9.5), rtol=1e-15)


@pytest.mark.parametrize("d_s", [512, 256, 128, 64])
def test_rms_norm_matches_library(d_s):
    x = _rng(d_s).standard_normal((5, 512)) * _rng(7).uniform(0.1, 10, size=(5, 1))
    eps = 1e-6
    ref_g = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,), eps=eps).numpy()
    np.testing.assert_allclose(oracle.rms_normalize(x, eps), ref_g, rtol=1e-13, atol=0)
    ref_s = torch.nn.functional.rms_norm(torch.from_numpy(x).reshape(5, 512 // d_s, d_s), (d_s,),
                                         eps=eps).reshape(5, 512).numpy()
    np.testing.assert_allclose(oracle.slice_rms_normalize(x, d_s, eps), ref_s, rtol=1e-13, atol=0)


def test_slice_rms_norm_brute_force_loops():
    x = _rng(3).standard_normal((2, 16))
    got = oracle.slice_rms_normalize(x, 4, 0.01)
    for r in range(2):
        for blk in range(4):
            ss = 0.0
            for k in range(4):
                ss += x[r, 4 * blk + k] ** 2
            den = math.sqrt(ss / 4 + 0.01)
            for k in range(4):
                assert abs(got[r, 4 * blk + k] - x[r, 4 * blk + k] / den) < 1e-14


def test_rms_norm_invariants():
    x = _rng(5).standard_normal((4, 512)) * 7.0
    s = oracle.slice_rms_normalize(x, 128, 0.0)
    np.testing.assert_allclose(np.mean(s.reshape(4, 4, 128) ** 2, axis=-1), 1.0, rtol=1e-13)
    # the global norm commutes with the orthonormal transform; the per-slice
    # norm in general does not
    np.testing.assert_allclose(oracle.rms_normalize(oracle.fwht(x), 1e-6),
                               oracle.fwht(oracle.rms_normalize(x, 1e-6)), rtol=1e-12, atol=1e-13)
    assert not np.allclose(oracle.slice_rms_normalize(oracle.fwht(x), 128, 0.0),
                           oracle.fwht(oracle.slice_rms_normalize(x, 128, 0.0)))
    # the transform of a one-hot vector is flat, so every slice already has
    # the global RMS: slice norm = global norm exactly
    e = np.zeros(512)
    e[37] = -4.0
    y = oracle.fwht(e)
    np.testing.assert_array_equal(oracle.slice_rms_normalize(y, 64, 0.0), oracle.rms_normalize(y, 0.0))
    np.testing.assert_array_equal(oracle.rotate_normalize_latent(e, "slice", 64, 0.0),
                                  oracle.rotate_normalize_latent(e, "global", 64, 0.0))
    with pytest.raises(ValueError):
        oracle.slice_rms_normalize(x, 100, 0.0)


def test_rotation_before_slicing_shrinks_the_norm_gap():
    # The transform spreads a few large channels over every slice, so the
    # slice statistics approach the global one (the blog's argument for
    # rotating before the split).  Latents with 4 outlier channels, all in
    # the first 256-column slice.
    rng = _rng(11)
    x = rng.standard_normal((64, 512))
    x[:, [3, 40, 100, 200]] *= 25.0
    eps = 1e-6

    def gap(hadamard):
        g = oracle.rotate_normalize_latent(x, "global", 256, eps, hadamard=hadamard)
        s = oracle.rotate_normalize_latent(x, "slice", 256, eps, hadamard=hadamard)
        return np.linalg.norm(s - g, axis=-1) / np.linalg.norm(g, axis=-1)

    plain, rotated = gap(False), gap(True)
    assert np.median(plain) > 0.3
    assert np.median(rotated) < 0.03
    assert np.all(rotated < plain)


# --------------------------------------------------------------------------
# Value up-projection per shard and the summing all-reduce
# --------------------------------------------------------------------------

def test_up_project_at_one_shard_equals_unabsorbed_mla():
    # T = 1, no rotation: the up-projected latent-space output is exactly
    # MLA with explicit per-head values (W_UV applied to every cached row)
    rng = _rng(41)
    H, d_n, d_c, d_r, d_v, L = 3, 16, 32, 8, 12, 40
    q_nope, q_rope = rng.standard_normal((H, d_n)), rng.standard_normal((H, d_r))
    c, r = rng.standard_normal((L, d_c)), rng.standard_normal((L, d_r))
    w_uk = rng.standard_normal((H, d_n, d_c)) / 4
    w_uv = rng.standard_normal((H, d_v, d_c)) / 4
    scale = 1 / math.sqrt(d_n + d_r)
    ref = oracle.mla_decode_unabsorbed(q_nope, q_rope, c, r, w_uk, w_uv, scale)
    q_lat = np.stack([w_uk[h].T @ q_nope[h] for h in range(H)])
    (o, _), = oracle.tpla_shards(q_lat, q_rope, c, r, 1, scale, hadamard=False)
    y = oracle.up_project_shard(o[None], w_uv.transpose(0, 2, 1))[0]
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_up_project_brute_force_and_shard_sum():
    rng = _rng(43)
    B, H, d_c, d_v, T = 2, 3, 8, 5, 2
    o = rng.standard_normal((B, H, d_c))
    w = rng.standard_normal((H, d_c, d_v))
    got = oracle.up_project_shard(o, w)
    for b in range(B):
        for h in range(H):
            for v in range(d_v):
                acc = 0.0
                for k in range(d_c):
                    acc += o[b, h, k] * w[h, k, v]
                assert abs(got[b, h, v] - acc) < 1e-12
    # the sum over devices of slice products is the product over the whole
    # latent: the all-reduce reassembles the un-split contraction
    d_s = d_c // T
    parts_o = [o[..., g * d_s:(g + 1) * d_s] for g in range(T)]
    parts_w = [w[:, g * d_s:(g + 1) * d_s, :] for g in range(T)]
    np.testing.assert_allclose(oracle.up_project_combine(parts_o, parts_w), got, rtol=1e-13, atol=1e-13)


def test_rotated_weights_undo_the_latent_rotation():
    # o @ w == (o @ Hn) @ (Hn @ w): the rotation applied to latent and query
    # is absorbed into W_UV's latent rows
    rng = _rng(47)
    o = rng.standard_normal((4, 3, 64))
    w = rng.standard_normal((3, 64, 7))
    y = oracle.up_project_shard(o, w)
    y_rot = oracle.up_project_shard(oracle.fwht(o), oracle.rotate_weight_rows(w))
    np.testing.assert_allclose(y_rot, y, rtol=1e-12, atol=1e-12)
    # rotate_weight_rows is Hn @ w[h] with the dense library matrix
    Hn = scipy.linalg.hadamard(64) / 8.0
    np.testing.assert_allclose(oracle.rotate_weight_rows(w)[1], Hn @ w[1], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# MLA-form prefill (causal attention of a prompt over its own latent rows)
# --------------------------------------------------------------------------

def _prefill_inputs(seed, S=23, H=3, d_c=16, d_r=4):
    rng = _rng(seed)
    return (rng.standard_normal((S, H, d_c)), rng.standard_normal((S, H, d_r)),
            rng.standard_normal((S, d_c)), rng.standard_normal((S, d_r)))


def test_prefill_matches_torch_causal_sdpa():
    # library routine: torch's causal scaled-dot-product attention in float64,
    # keys = [latent || rope], values = latent, heads as the batch
    ql, qr, c, r = _prefill_inputs(60)
    scale = 0.31
    o, _ = oracle.mla_prefill(ql, qr, c, r, scale)
    q = torch.from_numpy(np.concatenate([ql, qr], axis=2)).permute(1, 0, 2)      # [H, S, d]
    k = torch.from_numpy(np.concatenate([c, r], axis=1))[None].expand(q.shape[0], -1, -1)
    v = torch.from_numpy(c)[None].expand(q.shape[0], -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_prefill_brute_force_loops():
    ql, qr, c, r = _prefill_inputs(61, S=6, H=2, d_c=3, d_r=2)
    scale = 0.7
    o, lse = oracle.mla_prefill(ql, qr, c, r, scale)
    for t in range(6):
        for h in range(2):
            sc = []
            for j in range(t + 1):
                acc = 0.0
                for k in range(3):
                    acc += ql[t, h, k] * c[j, k]
                for k in range(2):
                    acc += qr[t, h, k] * r[j, k]
                sc.append(scale * acc)
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            assert abs(lse[t, h] - (mx + math.log(tot))) < 1e-12
            for k in range(3):
                assert abs(o[t, h, k] - sum(w[j] * c[j, k] for j in range(t + 1)) / tot) < 1e-12


def test_prefill_rows_are_decode_steps_over_the_prefix():
    # position t of the prefill is the decode of t's query over positions 0..t
    ql, qr, c, r = _prefill_inputs(62)
    o, lse = oracle.mla_prefill(ql, qr, c, r, 0.2)
    for t in range(c.shape[0]):
        ref, ref_l = oracle.mla_decode(ql[t], qr[t], c[:t + 1], r[:t + 1], 0.2)
        np.testing.assert_allclose(o[t], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[t], ref_l, rtol=1e-12, atol=1e-12)


def test_prefill_first_position_and_causality():
    ql, qr, c, r = _prefill_inputs(63)
    o, lse = oracle.mla_prefill(ql, qr, c, r, 0.45)
    # one visible key: its own row exactly, lse = its score
    for h in range(ql.shape[1]):
        np.testing.assert_array_equal(o[0, h], c[0])
        assert abs(lse[0, h] - 0.45 * (ql[0, h] @ c[0] + qr[0, h] @ r[0])) < 1e-12
    # later rows change nothing at earlier positions
    c2, r2 = c.copy(), r.copy()
    c2[10:] += 5.0
    r2[10:] -= 3.0
    o2, lse2 = oracle.mla_prefill(ql, qr, c2, r2, 0.45)
    np.testing.assert_array_equal(o2[:10], o[:10])
    np.testing.assert_array_equal(lse2[:10], lse[:10])
    assert np.max(np.abs(o2[10:] - o[10:])) > 1e-3


def test_prefill_identical_rows_closed_form():
    # every row the same: the output is that row and lse = score + log(t + 1)
    ql, qr, _, _ = _prefill_inputs(64)
    S = ql.shape[0]
    row = np.linspace(-1.0, 1.0, 16)
    rope = np.array([0.5, -0.25, 1.0, 2.0])
    o, lse = oracle.mla_prefill(ql, qr, np.tile(row, (S, 1)), np.tile(rope, (S, 1)), 0.3)
    for t in range(S):
        np.testing.assert_allclose(o[t], np.tile(row, (ql.shape[1], 1)), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[t], 0.3 * (ql[t] @ row + qr[t] @ rope) + math.log(t + 1),
                                   rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Other readings of the pages (diagnostic flags) and the TPLA-vs-MLA gap
# --------------------------------------------------------------------------

def test_alternative_readings_reduce_to_the_default():
    rng = _rng(70)
    ql, qr = rng.standard_normal((3, 32)), rng.standard_normal((3, 8))
    c, r = rng.standard_normal((40, 32)), rng.standard_normal((40, 8))
    base = oracle.tpla_shards(ql, qr, c, r, 2, 0.3, True)
    same = oracle.tpla_shards(ql, qr, c, r, 2, 0.3, True, rope_split=False, latent_mult=1.0)
    for (o1, l1), (o2, l2) in zip(base, same):
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)
    # one shard: the rope "slice" is the whole rope
    one = oracle.tpla_shards(ql, qr, c, r, 1, 0.3, False, rope_split=True)
    ref, _ = oracle.mla_decode(ql, qr, c, r, 0.3)
    np.testing.assert_allclose(one[0][0], ref, rtol=1e-13, atol=1e-13)


def test_alternative_readings_brute_force():
    # shard g's score with both flags: scale * (m * q_g . c_g + qr_g . r_g),
    # written out with loops on a tiny case
    rng = _rng(71)
    H, L, d_c, d_r, tp, m, sc = 2, 5, 8, 4, 2, 2.0, 0.4
    ql, qr = rng.standard_normal((H, d_c)), rng.standard_normal((H, d_r))
    c, r = rng.standard_normal((L, d_c)), rng.standard_normal((L, d_r))
    parts = oracle.tpla_shards(ql, qr, c, r, tp, sc, False, rope_split=True, latent_mult=m)
    d_s, d_rs = d_c // tp, d_r // tp
    for g in range(tp):
        for h in range(H):
            s = [sc * (m * sum(ql[h, g * d_s + k] * c[j, g * d_s + k] for k in range(d_s)) +
                       sum(qr[h, g * d_rs + k] * r[j, g * d_rs + k] for k in range(d_rs)))
                 for j in range(L)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            for k in range(d_s):
                want = sum(w[j] * c[j, g * d_s + k] for j in range(L)) / sum(w)
                assert abs(parts[g][0][h, k] - want) < 1e-12


def _cos_to_mla(q, qr, c, r, tp, scale, hadamard, **kw):
    ref, _ = oracle.mla_decode(q, qr, c, r, scale)
    parts = oracle.tpla_shards(q, qr, c, r, tp, scale, hadamard, **kw)
    out = oracle.combine_shards([o for o, _ in parts])
    if hadamard:
        out = oracle.fwht(out)
    return float(np.mean([ref[h] @ out[h] / np.linalg.norm(ref[h]) / np.linalg.norm(out[h])
                          for h in range(q.shape[0])]))


def test_tpla_vs_mla_gap_diagnostic():
    """Parity unpinned: TPLA with T > 1 approximates MLA and the pages give no
    closed form for the gap.  What the mathematics fixes: T = 1 is MLA
    exactly; on iid Gaussian data the rotation changes nothing in
    distribution.  The values (cosine of TPLA's head outputs to MLA's,
    H = 16, L = 2048, d_c = 512, d_r = 64) are printed for the record."""
    rng = _rng(72)
    H, L, d_c, d_r, scale = 16, 2048, 512, 64, 1 / math.sqrt(192.0)
    q, qr = rng.standard_normal((H, d_c)), rng.standard_normal((H, d_r))
    c, r = rng.standard_normal((L, d_c)), rng.standard_normal((L, d_r))
    assert abs(_cos_to_mla(q, qr, c, r, 1, scale, True) - 1.0) < 1e-12
    iid = {h: _cos_to_mla(q, qr, c, r, 2, scale, h) for h in (False, True)}
    assert abs(iid[False] - iid[True]) < 0.02, iid
    q2, c2 = q.copy(), c.copy()
    q2[:, :8] *= 10.0                 # 8 outlier channels in query and latent
    c2[:, :8] *= 10.0
    out = {h: _cos_to_mla(q2, qr, c2, r, 2, scale, h) for h in (False, True)}
    print(f"cosine to MLA, T=2: iid {iid}, outlier channels {out}")
    assert all(0.5 < v < 1.0 for v in list(iid.values()) + list(out.values()))
