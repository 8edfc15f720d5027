"""GPU parity of every libtpla entry point against the fp64 oracle.

Bars: integer/index work (append, combine placement) bit-exact; floating
point max|gpu - oracle| / max|oracle| <= 5e-3 for bf16 inputs with float32
accumulation (1e-5 for float32 inputs).  Caches start NaN-filled, so a
kernel that reads a row it was not given produces NaN and fails.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from tensor_latent_decode_amd import tpla
from tensor_latent_decode_amd.inputs import CONFIGS, make_case
from tpla_testlib import (TOL_BF16, TOL_FP32, GpuCase, as_f64, dev, host_bits, host_f64,
                          oracle_rows, oracle_step, rel_err)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# --------------------------------------------------------------------------
# Hadamard
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 4, 16, 64, 128, 512, 1024, 4096])
@pytest.mark.parametrize("dts", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16")])
def test_hadamard_parity(n, dts):
    rng = np.random.default_rng(n)
    rows = 37
    x32 = rng.standard_normal((rows, n)).astype(np.float32)
    tin = torch.bfloat16 if dts[0] == "bf16" else torch.float32
    tout = torch.bfloat16 if dts[1] == "bf16" else torch.float32
    x = torch.from_numpy(x32).cuda().to(tin)
    y = tpla.hadamard_latent(x, out_dtype=tout)
    ref = oracle.fwht(host_f64(x))
    tol = TOL_BF16 if "bf16" in dts[1] else TOL_FP32
    assert rel_err(host_f64(y), ref) <= tol


def test_hadamard_inplace_strided_rows_and_self_inverse():
    rng = np.random.default_rng(2)
    base = torch.from_numpy(rng.standard_normal((5, 7, 512)).astype(np.float32)).cuda()
    x = base[:, :, :]                       # [5, 7, 512] rows of a larger buffer
    big = torch.zeros((35, 1024), device="cuda")
    big[:, :512] = x.reshape(35, 512)
    view = big[:, :512]                     # row stride 1024
    ref = oracle.fwht(host_f64(view))
    tpla.hadamard_latent(view, out=view)
    assert rel_err(host_f64(view), ref) <= TOL_FP32
    assert torch.all(big[:, 512:] == 0)
    tpla.hadamard_latent(view, out=view)
    assert rel_err(host_f64(view), host_f64(x.reshape(35, 512))) <= 1e-5


@pytest.mark.parametrize("n", [16, 64, 512, 4096])
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_hadamard_unaligned_rows_match_aligned(n, dt):
    # rows that start one element off a 16-byte boundary take the element-wise
    # path; its results equal the vector path's bit for bit
    rng = np.random.default_rng(n + 7)
    x = torch.from_numpy(rng.standard_normal((23, n)).astype(np.float32)).cuda().to(dt)
    big = torch.zeros((23, n + 1), dtype=dt, device="cuda")
    big[:, 1:] = x
    odd = big[:, 1:]                         # odd row stride, odd start
    y_al = tpla.hadamard_latent(x)
    y_odd = torch.empty((23, n + 1), dtype=dt, device="cuda")[:, 1:]
    tpla.hadamard_latent(odd, out=y_odd)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y_odd.contiguous()), _bits(y_al))
    tol = TOL_BF16 if dt == torch.bfloat16 else TOL_FP32
    assert rel_err(host_f64(y_al), oracle.fwht(host_f64(x))) <= tol


# --------------------------------------------------------------------------
# Paged append (bit-exact)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,bs", [("tiny_fp32", 16), ("tiny_fp32", 64), ("dsv3_4k", 64),
                                    ("dsv3_4k", 16), ("kimi_k2_32k", 64)])
def test_append_bit_exact(cfg, bs):
    case = make_case(CONFIGS[cfg], batch=3, ctx=(30, 200), block_size=bs, seed=7,
                     heads=min(CONFIGS[cfg].heads, 32))
    g_case = GpuCase(case)
    d_s = case.cfg.d_s
    for g in range(case.cfg.tp):
        cache = g_case.prefill(g, d_s)
        tpla.append_kv(cache, g_case.bt, g_case.new_seq, g_case.new_pos,
                       g_case.new_latent[:, g * d_s:(g + 1) * d_s], g_case.new_rope)
        torch.cuda.synchronize()
        ref = np.full(tuple(cache.shape), 0xFFFF if case.cfg.dtype == "bf16" else np.nan,
                      dtype=np.uint16 if case.cfg.dtype == "bf16" else np.float32)
        oracle.paged_append(ref, case.block_table, bs, case.hist_seq, case.hist_pos,
                            case.hist_latent[:, g * d_s:(g + 1) * d_s], case.hist_rope)
        oracle.paged_append(ref, case.block_table, bs, np.arange(3), case.new_pos,
                            case.new_latent[:, g * d_s:(g + 1) * d_s], case.new_rope)
        got = host_bits(cache)
        np.testing.assert_array_equal(got.view(np.uint32 if got.dtype == np.float32 else np.uint16),
                                      ref.view(np.uint32 if ref.dtype == np.float32 else np.uint16))


def test_append_fp32_source_rounds_to_bf16_nearest_even():
    case = make_case(CONFIGS["dsv3_4k"], batch=2, ctx=(10, 80), seed=8, heads=32)
    g_case = GpuCase(case)
    rng = np.random.default_rng(9)
    src = rng.standard_normal((2, 256)).astype(np.float32)
    src[0, :8] = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0, 3e38,
                           1e-40, 2 ** -8], np.float32)     # ties, signed zero, big, subnormal
    rope = rng.standard_normal((2, 64)).astype(np.float32)
    cache = g_case.prefill(0, 256)
    tpla.append_kv(cache, g_case.bt, g_case.new_seq, g_case.new_pos, dev(src), dev(rope))
    ref = np.full(tuple(cache.shape), 0xFFFF, np.uint16)
    oracle.paged_append(ref, case.block_table, 64, case.hist_seq, case.hist_pos,
                        case.hist_latent[:, :256], case.hist_rope)
    oracle.paged_append(ref, case.block_table, 64, np.arange(2), case.new_pos, src, rope)
    np.testing.assert_array_equal(host_bits(cache), ref)


def test_append_skips_out_of_range_rows():
    case = make_case(CONFIGS["dsv3_4k"], batch=2, ctx=(10, 80), seed=10, heads=32)
    g_case = GpuCase(case)
    cache = g_case.prefill(0, 256)
    before = host_bits(cache).copy()
    bad_seq = torch.tensor([-1, 2, 0, 1], dtype=torch.int32, device="cuda")
    bad_pos = torch.tensor([0, 0, -5, case.max_blocks * 64], dtype=torch.int32, device="cuda")
    lat = torch.ones((4, 256), dtype=torch.bfloat16, device="cuda")
    rope = torch.ones((4, 64), dtype=torch.bfloat16, device="cuda")
    tpla.append_kv(cache, g_case.bt, bad_seq, bad_pos, lat, rope)
    bt = g_case.bt.clone()
    bt[0, 0] = case.num_blocks + 5           # invalid block id
    tpla.append_kv(cache, bt, torch.tensor([0], dtype=torch.int32, device="cuda"),
                   torch.tensor([0], dtype=torch.int32, device="cuda"), lat[:1], rope[:1])
    np.testing.assert_array_equal(host_bits(cache), before)


# --------------------------------------------------------------------------
# Fused rotation + append (one launch) against the separate calls and the oracle
# --------------------------------------------------------------------------

def _bits(t):
    h = host_bits(t)
    return h.view(np.uint32) if h.dtype == np.float32 else h


@pytest.mark.parametrize("cfg,bs,first,count", [("tiny_fp32", 16, 0, 2), ("dsv3_4k", 64, 0, 2),
                                                ("dsv3_4k", 16, 1, 1), ("kimi_k2_32k", 64, 0, 4),
                                                ("kimi_k2_32k", 64, 2, 2)])
def test_rotate_append_matches_separate_calls(cfg, bs, first, count):
    case = make_case(CONFIGS[cfg], batch=3, ctx=(30, 200), block_size=bs, seed=17,
                     heads=min(CONFIGS[cfg].heads, 32))
    gc = GpuCase(case)
    d_s = case.cfg.d_s
    shards = list(range(first, first + count))
    # separate calls: rotate query, rotate new latent, append per shard
    q_ref = tpla.hadamard_latent(gc.q_latent)
    new_ref = tpla.hadamard_latent(gc.new_latent)
    ref_caches = []
    for g in shards:
        c = gc.prefill(g, d_s)
        tpla.append_kv(c, gc.bt, gc.new_seq, gc.new_pos, new_ref[:, g * d_s:(g + 1) * d_s],
                       gc.new_rope)
        ref_caches.append(c)
    # one launch
    q_out = torch.empty_like(gc.q_latent)
    new_out = torch.empty_like(gc.new_latent)
    caches = [gc.prefill(g, d_s) for g in shards]
    tpla.rotate_append(gc.q_latent, q_out, gc.new_latent, gc.new_rope, gc.new_seq, gc.new_pos,
                       caches, gc.bt, first_shard=first, latent_out=new_out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(q_out), _bits(q_ref))
    assert np.array_equal(_bits(new_out), _bits(new_ref))
    for c, r in zip(caches, ref_caches):
        assert np.array_equal(_bits(c), _bits(r))
    # and the oracle: rotated query and the appended rows
    q64 = as_f64(case.q_latent)
    tol = TOL_BF16 if case.cfg.dtype == "bf16" else TOL_FP32
    assert rel_err(host_f64(q_out), oracle.fwht(q64)) <= tol
    new64 = oracle.fwht(as_f64(case.new_latent))
    for g, c in zip(shards, caches):
        got = host_f64(c)
        for b in range(3):
            p = int(case.new_pos[b])
            row = got[int(case.block_table[b, p // bs]), p % bs]
            assert rel_err(row[:d_s], new64[b, g * d_s:(g + 1) * d_s]) <= tol
            want = case.new_rope[b] if case.cfg.dtype == "bf16" else case.new_rope[b].view(np.uint32)
            assert np.array_equal(_bits(c)[int(case.block_table[b, p // bs]), p % bs, d_s:], want)


def test_rotate_append_unaligned_rows_match_aligned():
    # query and new-latent rows off a 16-byte boundary (element-wise path)
    case = make_case(CONFIGS["dsv3_4k"], batch=3, ctx=(30, 200), seed=23, heads=32)
    gc = GpuCase(case)
    n = case.cfg.d_c
    q = gc.q_latent.reshape(-1, n)
    qbig = torch.zeros((q.shape[0], n + 1), dtype=q.dtype, device="cuda")
    qbig[:, 1:] = q
    nbig = torch.zeros((3, n + 1), dtype=q.dtype, device="cuda")
    nbig[:, 1:] = gc.new_latent
    q_out = torch.empty((q.shape[0], n + 1), dtype=q.dtype, device="cuda")[:, 1:]
    new_out = torch.empty((3, n + 1), dtype=q.dtype, device="cuda")[:, 1:]
    caches = [gc.prefill(g, 256) for g in range(2)]
    tpla.rotate_append(qbig[:, 1:], q_out, nbig[:, 1:], gc.new_rope, gc.new_seq, gc.new_pos,
                       caches, gc.bt, latent_out=new_out)
    q_ref = torch.empty_like(q)
    new_ref = torch.empty_like(gc.new_latent)
    ref_caches = [gc.prefill(g, 256) for g in range(2)]
    tpla.rotate_append(q, q_ref, gc.new_latent, gc.new_rope, gc.new_seq, gc.new_pos,
                       ref_caches, gc.bt, latent_out=new_ref)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(q_out.contiguous()), _bits(q_ref))
    assert np.array_equal(_bits(new_out.contiguous()), _bits(new_ref))
    for c, r in zip(caches, ref_caches):
        assert np.array_equal(_bits(c), _bits(r))


@pytest.mark.parametrize("cfg", ["dsv3_4k", "kimi_k2_32k"])
@pytest.mark.parametrize("mode", ["global", "slice"])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_rotate_append_latent_norm(cfg, mode, dt):
    # new latent rows with outlier channels, RMS-normalised after the rotation
    # over the whole row or per shard slice (RMSNorm slicing), against the
    # oracle; the caches get exactly the stored slices; the query is
    # untouched by the norm
    case = make_case(CONFIGS[cfg], batch=4, ctx=(30, 200), seed=29, heads=32)
    gc = GpuCase(case)
    d_s, tp, n = case.cfg.d_s, case.cfg.tp, case.cfg.d_c
    rng = np.random.default_rng(31)
    x = rng.standard_normal((4, n)).astype(np.float32) * 3.0
    x[:, [5, 77, 130, 300]] *= 20.0
    x[1] *= 1e-3                                           # small row: eps matters little
    lat = torch.from_numpy(x).cuda().to(dt)
    rope = gc.new_rope.to(dt)
    eps = 1e-6
    lat_out = torch.empty_like(lat)
    caches = [gc.prefill(g, d_s) if dt == torch.bfloat16 else None for g in range(tp)]
    caches = [c for c in caches if c is not None]
    q_out = torch.empty_like(gc.q_latent)
    tpla.rotate_append(gc.q_latent, q_out, lat, rope, gc.new_seq, gc.new_pos, caches, gc.bt,
                       latent_out=lat_out, latent_norm=mode, norm_eps=eps,
                       slice_width=None if caches else d_s)
    q_ref = torch.empty_like(gc.q_latent)
    tpla.rotate_append(gc.q_latent, q_ref, None, None)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(q_out), _bits(q_ref))
    ref = oracle.rotate_normalize_latent(host_f64(lat), mode, d_s, eps)
    got = host_f64(lat_out)
    if dt == torch.bfloat16:   # one rounding of a float32 result: within one bf16 ulp
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30), float(np.max(np.abs(got - ref)))
    else:
        assert rel_err(got, ref) <= TOL_FP32
    if mode == "slice":   # rows where eps is negligible: every slice has unit mean square
        ms = np.mean(got.reshape(4, tp, d_s)[[0, 2, 3]] ** 2, axis=-1)
        np.testing.assert_allclose(ms, 1.0, rtol=1e-2)
    bits = _bits(lat_out)
    for g, c in enumerate(caches):
        cb = _bits(c)
        for b in range(4):
            p = int(case.new_pos[b])
            row = cb[int(case.block_table[b, p // 64]), p % 64]
            assert np.array_equal(row[:d_s], bits[b, g * d_s:(g + 1) * d_s])


def test_rotate_append_slice_norm_without_caches_and_checks():
    lat = torch.randn(3, 512, device="cuda")
    out = torch.empty_like(lat)
    tpla.rotate_append(None, None, lat, None, latent_out=out, latent_norm="slice", slice_width=128)
    torch.cuda.synchronize()
    ref = oracle.rotate_normalize_latent(host_f64(lat), "slice", 128, 1e-6)
    assert rel_err(host_f64(out), ref) <= TOL_FP32
    with pytest.raises(tpla.TplaError):
        tpla.rotate_append(None, None, lat, None, latent_out=out, latent_norm="slice", slice_width=4)
    with pytest.raises(tpla.TplaError):
        tpla.rotate_append(None, None, lat, None, latent_out=out, latent_norm="global", norm_eps=0.0)


def test_rotate_append_fp32_sources_and_skipped_rows():
    case = make_case(CONFIGS["dsv3_4k"], batch=4, ctx=(10, 80), seed=19, heads=32)
    gc = GpuCase(case)
    q32, new32, rope32 = gc.q_latent.float(), gc.new_latent.float(), gc.new_rope.float()
    q_out = torch.empty_like(gc.q_latent)                      # fp32 in, bf16 out
    seq = torch.tensor([0, -1, 2, 3], dtype=torch.int32, device="cuda")
    pos = gc.new_pos.clone()
    pos[3] = case.max_blocks * 64                               # past the table: skipped
    caches = [gc.prefill(g, 256) for g in range(2)]
    before = [_bits(c).copy() for c in caches]
    tpla.rotate_append(q32, q_out, new32, rope32, seq, pos, caches, gc.bt)
    ref_q = tpla.hadamard_latent(q32, out_dtype=torch.bfloat16)
    new_rot = tpla.hadamard_latent(new32)                      # fp32
    ref = [c.clone() for c in [gc.prefill(g, 256) for g in range(2)]]
    for g in range(2):
        tpla.append_kv(ref[g], gc.bt, seq[[0, 2]], pos[[0, 2]], new_rot[[0, 2], g * 256:(g + 1) * 256],
                       rope32[[0, 2]])
    torch.cuda.synchronize()
    assert np.array_equal(_bits(q_out), _bits(ref_q))
    for g in range(2):
        got = _bits(caches[g])
        assert np.array_equal(got, _bits(ref[g]))
        assert int(np.sum(got != before[g])) > 0


# --------------------------------------------------------------------------
# Combine (bit-exact placement)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("tp", [1, 2, 4])
@pytest.mark.parametrize("out_dt", [torch.float32, torch.bfloat16])
def test_combine_bit_exact(tp, out_dt):
    rng = np.random.default_rng(tp)
    parts = [rng.standard_normal((3, 5, 64)).astype(np.float32) for _ in range(tp)]
    parts[0][0, 0, :3] = [-0.0, 0.0, 1 + 2 ** -8]
    out = tpla.combine_shards([dev(p) for p in parts], out_dtype=out_dt)
    ref = oracle.combine_shards([p.astype(np.float64) for p in parts]).astype(np.float32)
    if out_dt == torch.float32:
        want = np.concatenate(parts, axis=-1)
        np.testing.assert_array_equal(host_bits(out).view(np.uint32), want.view(np.uint32))
        np.testing.assert_array_equal(host_bits(out), ref)
    else:
        # values, not bits: the oracle's zero-padded sum turns -0.0 into +0.0
        np.testing.assert_array_equal(oracle.bf16_bits_to_f64(host_bits(out)),
                                      oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(ref)))


def test_combine_accumulate():
    rng = np.random.default_rng(3)
    parts = [rng.standard_normal((2, 3, 32)).astype(np.float32) for _ in range(2)]
    base = rng.standard_normal((2, 3, 64)).astype(np.float32)
    out = dev(base)
    tpla.combine_shards([dev(p) for p in parts], out=out, accumulate=True)
    ref = base.astype(np.float64) + oracle.combine_shards([p.astype(np.float64) for p in parts])
    assert rel_err(host_f64(out), ref) <= 1e-6


# --------------------------------------------------------------------------
# Decode: tiny float32 TPLA, both shards, Hadamard on and off (full step)
# --------------------------------------------------------------------------

def run_step(gc: GpuCase, hadamard: bool, num_splits: int = 0, out_dtype=torch.float32):
    """The library's whole decode step on one GPU: rotate query and new latent,
    then for every shard append the new row and decode; combine."""
    case = gc.case
    cfg = case.cfg
    d_s = cfg.d_s
    q = tpla.hadamard_latent(gc.q_latent) if hadamard else gc.q_latent
    new = tpla.hadamard_latent(gc.new_latent) if hadamard else gc.new_latent
    outs, lses, caches = [], [], []
    for g in range(cfg.tp):
        cache = gc.prefill(g, d_s)
        tpla.append_kv(cache, gc.bt, gc.new_seq, gc.new_pos, new[:, g * d_s:(g + 1) * d_s],
                       gc.new_rope)
        lse = torch.empty((cfg.batch, cfg.heads), dtype=torch.float32, device="cuda")
        o, _ = tpla.decode_shard(q[:, :, g * d_s:(g + 1) * d_s], gc.q_rope, cache, gc.bt,
                                 gc.seq_lens, cfg.scale, int(case.seq_lens.max()), lse=lse,
                                 num_splits=num_splits, out_dtype=out_dtype)
        outs.append(o)
        lses.append(lse)
        caches.append(cache)
    combined = tpla.combine_shards([o.float() for o in outs])
    torch.cuda.synchronize()
    return combined, outs, lses


@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("bs", [64, 16])
def test_tiny_fp32_full_step(hadamard, bs):
    case = make_case(CONFIGS["tiny_fp32"], block_size=bs)
    gc = GpuCase(case)
    combined, outs, lses = run_step(gc, hadamard)
    ref, parts = oracle_step(case, 0, case.cfg.tp, hadamard)
    assert rel_err(host_f64(combined)[0], ref) <= TOL_FP32
    for g, (o, l) in enumerate(parts):
        assert rel_err(host_f64(outs[g])[0], o) <= TOL_FP32
        assert np.max(np.abs(host_f64(lses[g])[0] - l)) <= 1e-4


def test_tiny_fp32_hadamard_unrotate_matches_oracle():
    case = make_case(CONFIGS["tiny_fp32"])
    gc = GpuCase(case)
    combined, _, _ = run_step(gc, True)
    back = tpla.hadamard_latent(combined)
    ref, _ = oracle_step(case, 0, 2, True)
    assert rel_err(host_f64(back)[0], oracle.fwht(ref)) <= TOL_FP32


# --------------------------------------------------------------------------
# Decode: bf16 matrix-core kernel over shapes, tails, block sizes and splits
# --------------------------------------------------------------------------

SHAPES = [  # (heads, d_c, tp, d_r)
    (128, 512, 2, 64),      # DeepSeek-V3 shard
    (64, 512, 4, 64),       # Kimi-K2 shard
    (32, 128, 2, 64),
    (128, 256, 2, 0),
    (64, 512, 1, 64),       # plain MLA under TP=2: 64 heads, whole latent
    (128, 512, 1, 64),      # plain MLA, one device
    (48, 512, 1, 64),       # plain MLA in 16-head groups (Kimi-K2 under TP=4 has 16)
    (96, 512, 1, 64),       # plain MLA in 32-head groups
    (128, 512, 4, 64),      # two 64-head groups per unit (d_s = 128)
    (256, 512, 2, 64),      # two 128-head groups per unit (d_s = 256)
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bs", [64, 16, 128])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_bf16_ragged_parity(shape, bs, splits):
    H, d_c, tp, d_r = shape
    cfg = CONFIGS["dsv3_4k"]
    from dataclasses import replace
    cfg = replace(cfg, heads=H, d_c=d_c, tp=tp, d_r=d_r, scale=1 / math.sqrt(192.0))
    case = make_case(cfg, batch=6, ctx=(1, 700), block_size=bs, seed=31 + H + bs)
    gc = GpuCase(case)
    if d_c // tp == 512 and bs % 32 != 0:
        # the 512-wide kernel copies 32-token runs of one block; nothing else
        # takes a 512-wide latent in bf16
        with pytest.raises(tpla.TplaError, match="(?i)unsupported"):
            run_step(gc, hadamard=False, num_splits=splits)
        return
    combined, outs, lses = run_step(gc, hadamard=False, num_splits=splits)
    got = host_f64(combined)
    for b in range(cfg.batch):
        ref, parts = oracle_step(case, b, tp, hadamard=False)
        assert rel_err(got[b], ref) <= TOL_BF16, (b, int(case.seq_lens[b]))
        for g, (o, l) in enumerate(parts):
            assert np.max(np.abs(host_f64(lses[g])[b] - l)) <= 2e-2


@pytest.mark.parametrize("shape,bs", [(sh, bs) for sh in SHAPES[:3] for bs in (64, 16)] +
                         [(SHAPES[4], 64), (SHAPES[4], 32)])
def test_decode_bf16_late_score_spike(shape, bs):
    """A token deep inside the first split scores far above everything before
    it (head 0: about 2500 raw, ~260 in base-2 exponent units), so a softmax
    that kept the first tile's max as its reference would overflow.  Every
    head must still match the oracle on its own scale."""
    H, d_c, tp, d_r = shape
    from dataclasses import replace
    cfg = replace(CONFIGS["dsv3_4k"], heads=H, d_c=d_c, tp=tp, d_r=d_r, scale=1 / math.sqrt(192.0))
    case = make_case(cfg, batch=2, ctx=1500, block_size=bs, seed=70 + H + bs)
    d_s = d_c // tp
    q0 = as_f64(case.q_latent[0, 0])                      # head 0's query, whole latent
    k = 2500.0 / (cfg.scale * float(np.mean([q0[g * d_s:(g + 1) * d_s] @ q0[g * d_s:(g + 1) * d_s]
                                               for g in range(tp)])))
    from tensor_latent_decode_amd.inputs import bf16_bits
    case.hist_latent[700] = bf16_bits((k * q0).astype(np.float32))   # sequence 0, position 700
    gc = GpuCase(case)
    combined, outs, _ = run_step(gc, hadamard=False, num_splits=1)
    got = host_f64(combined)
    for b in range(2):
        ref, _ = oracle_step(case, b, tp, hadamard=False)
        for h in range(H):
            assert rel_err(got[b, h], ref[h]) <= TOL_BF16, (b, h)


@pytest.mark.parametrize("shape", [(128, 512, 2, 64), (64, 512, 4, 64), (32, 128, 2, 64), (5, 80, 2, 8)])
@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_decode_zero_and_negative_scale(shape, scale):
    """Every decode kernel (the two streaming shapes, the register-staged one,
    the float32 one) takes any finite scale: a zero scale averages the rows,
    a negative one favours the lowest scores."""
    H, d_c, tp, d_r = shape
    from dataclasses import replace
    cfg = replace(CONFIGS["dsv3_4k"], heads=H, d_c=d_c, tp=tp, d_r=d_r, scale=scale)
    case = make_case(cfg, batch=3, ctx=(1, 400), seed=88 + H)
    gc = GpuCase(case)
    rot = (d_c & (d_c - 1)) == 0              # the rotation needs a power-of-two width
    combined, outs, lses = run_step(gc, hadamard=rot, num_splits=2)
    got = host_f64(combined)
    for b in range(cfg.batch):
        ref, parts = oracle_step(case, b, tp, hadamard=rot)
        assert rel_err(got[b], ref) <= TOL_BF16, (b, int(case.seq_lens[b]))
        for g, (o, l) in enumerate(parts):
            assert np.max(np.abs(host_f64(lses[g])[b] - l)) <= 2e-2


def test_suggested_splits_uniform_and_ragged():
    """The host-side split suggestion keeps the automatic plan for uniform
    32K lengths (DeepSeek-V3 and Kimi-K2 shards): both kernels balance units
    over the lengths themselves, so the suggestion is 0; a ragged batch
    decoded with it matches the oracle on both shapes."""
    for heads, d_s in ((128, 256), (64, 128)):
        a = tpla.DecodeArgs()          # sizes only: the call reads no device memory
        a.batch, a.heads, a.d_s, a.d_r = 16, heads, d_s, 64
        a.block_size, a.num_blocks, a.max_blocks_per_seq, a.max_seq_len = 64, 8193, 512, 32768
        a.dtype, a.scale, a.out_dtype = 1, 0.07, 0
        fake = 0x10000
        a.q_latent, a.q_latent_stride_b, a.q_latent_stride_h = fake, heads * 512, 512
        a.q_rope, a.q_rope_stride_b, a.q_rope_stride_h = fake, heads * 64, 64
        a.cache, a.block_table, a.seq_lens = fake, fake, fake
        a.out, a.out_stride_b, a.out_stride_h = fake, heads * d_s, d_s
        auto = tpla.decode_workspace_size(a)
        a.num_splits = tpla.decode_suggest_splits(a, np.full(16, 32768, np.int32))
        assert tpla.decode_workspace_size(a) == auto, (heads, a.num_splits)
    for name in ("ragged_tp2", "kimi_k2_32k"):
        case = make_case(CONFIGS[name], batch=8, ctx=(64, 6000), seed=33)
        gc = GpuCase(case)
        d_s = case.cfg.d_s
        cache = gc.prefill(0, d_s)
        maxlen = int(case.seq_lens.max())
        out = torch.empty((case.cfg.batch, case.cfg.heads, d_s), dtype=torch.float32, device="cuda")
        args = tpla.make_decode_args(gc.q_latent[:, :, :d_s], gc.q_rope, cache, gc.bt, gc.hist_lens,
                                     case.cfg.scale, maxlen, out)
        sugg = tpla.decode_suggest_splits(args, case.seq_lens - 1)
        assert sugg == 0            # both shapes: units balanced on the device
        o, _ = tpla.decode_shard(gc.q_latent[:, :, :d_s], gc.q_rope, cache, gc.bt, gc.hist_lens,
                                 case.cfg.scale, maxlen, num_splits=sugg)
        torch.cuda.synchronize()
        for b in range(case.cfg.batch):
            _, parts = oracle_step(case, b, case.cfg.tp, hadamard=False, with_new=False,
                                   q_is_rotated=True)
            assert rel_err(host_f64(o)[b], parts[0][0]) <= TOL_BF16, (name, b)


def unit_map_reference(lens, n_target, max_tiles, cap):
    """The work units the balanced plan specifies, by brute force: T_b tiles
    per sequence, the smallest chunk c (tiles) with sum ceil(T_b / c) <= n_target
    (else the largest unit), and (first unit, unit count) per sequence."""
    tiles = [(min(max(int(L), 0), cap) + 63) // 64 for L in lens]
    nonempty = sum(t > 0 for t in tiles)
    if sum(tiles) == 0:
        c = 1
    elif nonempty >= n_target:
        c = max_tiles
    else:
        c = next((c for c in range(1, max_tiles + 1)
                  if sum(-(-t // c) for t in tiles) <= n_target), max_tiles)
    counts = [-(-t // c) for t in tiles]
    firsts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
    return c, np.stack([firsts, np.array(counts, dtype=np.int64)], axis=1)


def balanced_shard_decode(case, g=0):
    """Shard g's decode with the automatic (balanced-unit) plan; returns
    (out, lse, unit table read back from the workspace's tail)."""
    gc = GpuCase(case)
    cfg = case.cfg
    B, H, d_s = cfg.batch, cfg.heads, cfg.d_s
    q = tpla.hadamard_latent(gc.q_latent)
    new = tpla.hadamard_latent(gc.new_latent)
    cache = gc.prefill(g, d_s)
    tpla.append_kv(cache, gc.bt, gc.new_seq, gc.new_pos, new[:, g * d_s:(g + 1) * d_s], gc.new_rope)
    qs = q[:, :, g * d_s:(g + 1) * d_s]
    out = torch.full((B, H, d_s), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    maxlen = int(case.seq_lens.max())
    args = tpla.make_decode_args(qs, gc.q_rope, cache, gc.bt, gc.seq_lens, cfg.scale, maxlen, out,
                                 lse, 0)
    ws = tpla.decode_workspace(args)
    tpla.decode_shard(qs, gc.q_rope, cache, gc.bt, gc.seq_lens, cfg.scale, maxlen, out=out, lse=lse,
                      workspace=ws)
    torch.cuda.synchronize()
    tail = (B * 8 + 255) // 256 * 256
    table = ws[ws.numel() - tail:ws.numel() - tail + B * 8].cpu().numpy().view(np.int32).reshape(B, 2)
    return out.cpu().numpy(), lse.cpu().numpy(), table


def _balanced_lens(kind):
    rng = np.random.default_rng(123)
    if kind == "c5_mix":
        return rng.integers(1024, 32769, size=32).tolist()
    if kind == "min_max":
        # one token, tile edges, and one sequence past the largest unit (1024 tiles)
        return [1, 64, 65, 70001, 2049, 1]
    if kind == "more_than_cus":
        # more sequences than CUs: one unit each, the long one two
        return [70001] + rng.integers(1, 300, size=299).tolist()
    raise ValueError(kind)


@pytest.mark.parametrize("cfg_name", ["ragged_tp2", "kimi_k2_32k"])
@pytest.mark.parametrize("kind", ["c5_mix", "min_max", "more_than_cus"])
def test_balanced_units_table_and_parity(kind, cfg_name):
    """The automatic plan of the 128-head d_s = 256 and 64-head d_s = 128
    kernels (one head group per workgroup, so about one unit per CU): the
    unit table against the brute-force unit map, and every sequence against
    the oracle."""
    lens = _balanced_lens(kind)
    case = make_case(CONFIGS[cfg_name], batch=len(lens), ctx=lens, seed=77)
    tp = case.cfg.tp
    print(f"balanced units: {cfg_name} {kind}, batch {len(lens)}, max len {max(lens)}", flush=True)
    o, l, table = balanced_shard_decode(case, g=1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _, want = unit_map_reference(case.seq_lens, cus, 1024, int(case.seq_lens.max()))
    assert np.array_equal(table.astype(np.int64), want)
    worst = 0.0
    for b in range(case.cfg.batch):
        _, parts = oracle_step(case, b, tp, hadamard=True)
        err = rel_err(o[b].astype(np.float64), parts[1][0])
        worst = max(worst, err)
        assert err <= TOL_BF16, (b, int(case.seq_lens[b]))
        assert np.max(np.abs(l[b] - parts[1][1])) <= 2e-2, b
    print(f"  worst max|err|/max|ref| {worst:.3e}", flush=True)


@pytest.mark.parametrize("cfg_name", ["dsv3_4k", "kimi_k2_32k"])
@pytest.mark.parametrize("lens", [[1, 2, 63, 64], [65, 127, 128, 129], [4096, 1, 1000, 3]])
def test_decode_bf16_edge_lengths(lens, cfg_name):
    """Lengths at and around the 64-token tile, one sequence per call (a
    single unit), on the 128-head and the 64-head kernels."""
    cases = [make_case(CONFIGS[cfg_name], batch=1, ctx=L, seed=41 + i)
             for i, L in enumerate(lens)]
    for c in cases:
        gc = GpuCase(c)
        combined, _, _ = run_step(gc, hadamard=True)
        ref, _ = oracle_step(c, 0, c.cfg.tp, hadamard=True)
        assert rel_err(host_f64(combined)[0], ref) <= TOL_BF16, int(c.seq_lens[0])


def test_decode_generic_bf16_odd_shape():
    from dataclasses import replace
    cfg = replace(CONFIGS["dsv3_4k"], heads=5, d_c=80, tp=2, d_r=8, scale=0.2)
    case = make_case(cfg, batch=3, ctx=(1, 300), seed=50, block_size=32)
    gc = GpuCase(case)
    combined, _, _ = run_step(gc, hadamard=False, num_splits=2)
    for b in range(3):
        ref, _ = oracle_step(case, b, 2, hadamard=False)
        assert rel_err(host_f64(combined)[b], ref) <= TOL_BF16


def test_decode_empty_sequence_gives_zero_and_minus_inf():
    case = make_case(CONFIGS["dsv3_4k"], batch=2, ctx=100, seed=60)
    gc = GpuCase(case)
    cache = gc.prefill(0, 256)
    lens = torch.tensor([0, 99], dtype=torch.int32, device="cuda")
    lse = torch.empty((2, 128), dtype=torch.float32, device="cuda")
    o, _ = tpla.decode_shard(gc.q_latent[:, :, :256], gc.q_rope, cache, gc.bt, lens,
                             case.cfg.scale, 100, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    ref, parts = oracle_step(case, 1, 2, hadamard=False, with_new=False, q_is_rotated=True)
    assert rel_err(host_f64(o)[1], parts[0][0]) <= TOL_BF16


def test_decode_bf16_output_and_determinism():
    case = make_case(CONFIGS["dsv3_4k"], batch=2, ctx=(500, 3000), seed=61)
    gc = GpuCase(case)
    cache = gc.prefill(0, 256)
    lens = gc.hist_lens
    maxlen = int(case.seq_lens.max())
    a, _ = tpla.decode_shard(gc.q_latent[:, :, :256], gc.q_rope, cache, gc.bt, lens,
                             case.cfg.scale, maxlen, out_dtype=torch.bfloat16)
    b, _ = tpla.decode_shard(gc.q_latent[:, :, :256], gc.q_rope, cache, gc.bt, lens,
                             case.cfg.scale, maxlen, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for s in range(2):
        _, parts = oracle_step(case, s, 2, hadamard=False, with_new=False, q_is_rotated=True)
        assert rel_err(host_f64(a)[s], parts[0][0]) <= TOL_BF16


# --------------------------------------------------------------------------
# Plain MLA under tensor parallelism (whole 512-wide latent, 64-head groups)
# --------------------------------------------------------------------------

def mla_case(heads=64, batch=3, ctx=(1, 900), bs=64, seed=80, scale=None):
    from dataclasses import replace
    cfg = CONFIGS["mla_tp2_32k"]
    cfg = replace(cfg, heads=heads, scale=cfg.scale if scale is None else scale)
    return make_case(cfg, batch=batch, ctx=ctx, block_size=bs, seed=seed)


def mla_decode(gc: GpuCase, lens=None, **kw):
    case = gc.case
    cache = gc.prefill(0, 512)
    lens = gc.hist_lens if lens is None else lens
    lse = torch.empty((case.cfg.batch, case.cfg.heads), dtype=torch.float32, device="cuda")
    o, _ = tpla.decode_shard(gc.q_latent, gc.q_rope, cache, gc.bt, lens, case.cfg.scale,
                             int(case.seq_lens.max()), lse=lse, **kw)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(lse)


def mla_reference(case, b: int, n: int):
    """The oracle's plain MLA decode over the first n history rows of sequence b."""
    lat, rope = oracle_rows(case, b)
    return oracle.mla_decode(as_f64(case.q_latent[b]), as_f64(case.q_rope[b]), lat[:n], rope[:n],
                             case.cfg.scale)


@pytest.mark.parametrize("heads", [64, 16])
@pytest.mark.parametrize("scale", [-0.07, 0.0, 0.3])
def test_mla_decode_any_scale(scale, heads):
    """Zero and negative scales are valid softmax scales (a zero scale is the
    plain mean of the rows)."""
    case = mla_case(heads=heads, batch=2, ctx=(200, 700), seed=81, scale=scale)
    gc = GpuCase(case)
    o, lse = mla_decode(gc, num_splits=2)
    for b in range(2):
        n = int(case.seq_lens[b]) - 1
        ref_o, ref_l = mla_reference(case, b, n)
        assert rel_err(o[b], ref_o) <= TOL_BF16, b
        assert np.max(np.abs(lse[b] - ref_l)) <= 2e-2


@pytest.mark.parametrize("heads", [128, 16, 32])
@pytest.mark.parametrize("lens", [[1, 31, 32, 33], [63, 64, 65, 95], [96, 97, 2047, 2049]])
def test_mla_decode_tile_edges(lens, heads):
    """Lengths at and around the 32-token tile and the 64-token block, for
    64-, 16- and 32-head groups."""
    case = mla_case(heads=heads, batch=4, ctx=max(lens) + 1, seed=82)
    gc = GpuCase(case)
    L = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for splits in (0, 1, 5):
        o, lse = mla_decode(gc, lens=L, num_splits=splits)
        for b, n in enumerate(lens):
            ref_o, ref_l = mla_reference(case, b, n)
            assert rel_err(o[b], ref_o) <= TOL_BF16, (splits, b, n)
            assert np.max(np.abs(lse[b] - ref_l)) <= 2e-2, (splits, b, n)


def test_mla_decode_deterministic_and_strided_query():
    """Same bits on a second call; a query read through strides (heads of a
    wider buffer) gives the same bits as a packed one."""
    case = mla_case(batch=2, ctx=(900, 1500), seed=83)
    gc = GpuCase(case)
    a, _ = mla_decode(gc)
    b, _ = mla_decode(gc)
    assert np.array_equal(a, b)
    wide = torch.zeros((2, 64, 640), dtype=torch.bfloat16, device="cuda")
    wide[:, :, 64:576] = gc.q_latent
    cache = gc.prefill(0, 512)
    o, _ = tpla.decode_shard(wide[:, :, 64:576], gc.q_rope, cache, gc.bt, gc.hist_lens,
                             case.cfg.scale, int(case.seq_lens.max()))
    torch.cuda.synchronize()
    assert np.array_equal(host_f64(o), a)


# --------------------------------------------------------------------------
# The workloads at their real sizes (sampled sequences)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("heads,d_c,tp", [(128, 512, 2), (64, 512, 4), (64, 512, 1), (16, 512, 1)])
def test_decode_split_longer_than_tile_table(heads, d_c, tp):
    """A single requested split longer than the streaming kernel's tile
    table (65536 tokens) is planned as more splits and stays exact."""
    from dataclasses import replace
    cfg = replace(CONFIGS["dsv3_4k"], heads=heads, d_c=d_c, tp=tp)
    case = make_case(cfg, batch=1, ctx=70001, seed=72)
    gc = GpuCase(case)
    d_s = cfg.d_s
    cache = gc.prefill(0, d_s)
    o, _ = tpla.decode_shard(gc.q_latent[:, :, :d_s], gc.q_rope, cache, gc.bt, gc.hist_lens,
                             cfg.scale, int(case.seq_lens.max()), num_splits=1)
    torch.cuda.synchronize()
    _, parts = oracle_step(case, 0, tp, hadamard=False, with_new=False, q_is_rotated=True)
    assert rel_err(host_f64(o)[0], parts[0][0]) <= TOL_BF16


def test_decode_into_combined_columns_equals_combine():
    """Each shard's decode writing its latent columns of the combined output
    (strided out) gives the bits tpla_combine_shards gives from separate
    outputs."""
    case = make_case(CONFIGS["dsv3_4k"], batch=3, ctx=(100, 900), seed=71)
    gc = GpuCase(case)
    cfg = case.cfg
    d_s = cfg.d_s
    q = tpla.hadamard_latent(gc.q_latent)
    maxlen = int(case.seq_lens.max())
    combined = torch.empty((cfg.batch, cfg.heads, cfg.tp * d_s), dtype=torch.float32, device="cuda")
    outs = []
    for g in range(cfg.tp):
        cache = gc.prefill(g, d_s)
        o, _ = tpla.decode_shard(q[:, :, g * d_s:(g + 1) * d_s], gc.q_rope, cache, gc.bt,
                                 gc.hist_lens, cfg.scale, maxlen)
        tpla.decode_shard(q[:, :, g * d_s:(g + 1) * d_s], gc.q_rope, cache, gc.bt, gc.hist_lens,
                          cfg.scale, maxlen, out=combined[:, :, g * d_s:(g + 1) * d_s])
        outs.append(o)
    ref = tpla.combine_shards(outs)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(combined).view(np.uint32), host_bits(ref).view(np.uint32))


def test_dsv3_4k_full():
    case = make_case(CONFIGS["dsv3_4k"])
    gc = GpuCase(case)
    combined, outs, _ = run_step(gc, hadamard=True)
    ref, parts = oracle_step(case, 0, 2, hadamard=True)
    assert rel_err(host_f64(combined)[0], ref) <= TOL_BF16
    for g in range(2):
        assert rel_err(host_f64(outs[g])[0], parts[g][0]) <= TOL_BF16


# Real-size configurations decode long sequences, where the bf16 rounding of
# the softmax weights averages out: their worst error is watched against a
# tighter bound than the general one, so that a change eating into the
# margin shows before it crosses TOL_BF16.
TOL_BF16_WATCH = 4.5e-3


@pytest.mark.parametrize("name", ["dsv3_32k", "kimi_k2_32k", "mla_tp2_32k", "mla_tp4_32k"])
def test_32k_every_shard_every_sequence(name):
    """Every shard at its real shape with the split count the bench uses
    (the host-side suggestion from the lengths), every sequence and head
    against the oracle: output and lse."""
    case = make_case(CONFIGS[name])
    gc = GpuCase(case)
    cfg = case.cfg
    B, H, d_s = cfg.batch, cfg.heads, cfg.d_s
    maxlen = int(case.seq_lens.max())
    q = tpla.hadamard_latent(gc.q_latent)
    new = tpla.hadamard_latent(gc.new_latent)
    refs = [oracle_step(case, b, cfg.tp, hadamard=True)[1] for b in range(B)]
    for g in range(cfg.tp):
        cache = gc.prefill(g, d_s)
        tpla.append_kv(cache, gc.bt, gc.new_seq, gc.new_pos, new[:, g * d_s:(g + 1) * d_s],
                       gc.new_rope)
        qs = q[:, :, g * d_s:(g + 1) * d_s]
        out = torch.full((B, H, d_s), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
        args = tpla.make_decode_args(qs, gc.q_rope, cache, gc.bt, gc.seq_lens, cfg.scale, maxlen,
                                     out, lse, 0)
        splits = tpla.decode_suggest_splits(args, case.seq_lens)
        tpla.decode_shard(qs, gc.q_rope, cache, gc.bt, gc.seq_lens, cfg.scale, maxlen, out=out,
                          lse=lse, num_splits=splits)
        torch.cuda.synchronize()
        got, got_lse = host_f64(out), host_f64(lse)
        del cache
        worst = max(rel_err(got[b], refs[b][g][0]) for b in range(B))
        worst_lse = max(float(np.max(np.abs(got_lse[b] - refs[b][g][1]))) for b in range(B))
        print(f"{name} shard {g} splits {splits}: worst max|err|/max|ref| {worst:.3e}, "
              f"worst |lse err| {worst_lse:.3e}", flush=True)
        assert worst <= TOL_BF16_WATCH, (name, g, worst)
        assert worst_lse <= 2e-2, (name, g, worst_lse)


def test_ragged_tp2_full_step_every_sequence():
    """The ragged TP = 2 step as the bench runs it (both shards, automatic
    plan, combined output), every sequence against the oracle."""
    case = make_case(CONFIGS["ragged_tp2"])
    gc = GpuCase(case)
    combined, _, _ = run_step(gc, hadamard=True)
    got = host_f64(combined)
    worst = 0.0
    for b in range(case.cfg.batch):
        ref, _ = oracle_step(case, b, 2, hadamard=True)
        err = rel_err(got[b], ref)
        worst = max(worst, err)
        assert err <= TOL_BF16_WATCH, (b, int(case.seq_lens[b]), err)
    print(f"ragged_tp2: worst max|err|/max|ref| {worst:.3e}", flush=True)


# --------------------------------------------------------------------------
# Value up-projection per shard and the summing all-reduce
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,H,d_s,d_v", [(16, 128, 256, 128), (20, 8, 200, 100), (1, 3, 1024, 70),
                                         (33, 2, 64, 257), (5, 4, 37, 33), (40, 2, 12, 8)])
@pytest.mark.parametrize("dts", [("f32", "bf16", "f32"), ("bf16", "bf16", "bf16"), ("f32", "f32", "f32")])
def test_up_project_parity(B, H, d_s, d_v, dts):
    # several batch tiles (B > 32), partial row tiles of v, d_s with a partial
    # k-step or not a multiple of 8 (element reads), o misaligned (a column
    # slice of a wider output) or contiguous (16-byte reads)
    rng = np.random.default_rng(B * 1000 + d_s)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    wide = torch.from_numpy(rng.standard_normal((B, H, d_s + 7)).astype(np.float32)).cuda()
    o = wide[:, :, 3:3 + d_s].to(tdt[dts[0]]) if dts[0] == "bf16" else wide[:, :, 3:3 + d_s]
    w = torch.from_numpy((rng.standard_normal((H, d_v, d_s)) / 16).astype(np.float32)).cuda().to(tdt[dts[1]])
    y = tpla.up_project(o, w, out_dtype=tdt[dts[2]])
    torch.cuda.synchronize()
    ref = oracle.up_project_shard(host_f64(o), host_f64(w).transpose(0, 2, 1))
    tol = TOL_BF16 if dts[2] == "bf16" else TOL_FP32
    assert rel_err(host_f64(y), ref) <= tol


def test_up_project_accumulates_shards():
    # two devices' terms summed into one output equal the oracle's all-reduce
    rng = np.random.default_rng(5)
    B, H, d_s, d_v, T = 16, 16, 256, 128, 2
    os_ = [torch.from_numpy(rng.standard_normal((B, H, d_s)).astype(np.float32)).cuda() for _ in range(T)]
    ws = [torch.from_numpy((rng.standard_normal((H, d_v, d_s)) / 16).astype(np.float32)).cuda()
          .to(torch.bfloat16) for _ in range(T)]
    y = tpla.up_project(os_[0], ws[0])
    tpla.up_project(os_[1], ws[1], out=y, accumulate=True)
    y1 = tpla.up_project(os_[1], ws[1])
    torch.cuda.synchronize()
    ref = oracle.up_project_combine([host_f64(o) for o in os_], [host_f64(w).transpose(0, 2, 1) for w in ws])
    assert rel_err(host_f64(y), ref) <= TOL_FP32
    # the second call added its own result to the first one's, in float32
    y0 = tpla.up_project(os_[0], ws[0])
    torch.cuda.synchronize()
    assert torch.equal(y, y0 + y1)


@pytest.mark.parametrize("hadamard", [False, True])
def test_full_step_with_up_projection(hadamard):
    # decode both shards, up-project each with its rows of the (rotated)
    # transposed W_UV and sum: against the oracle's TPLA step followed by
    # its up-projection and all-reduce
    case = make_case(CONFIGS["dsv3_4k"], batch=3, ctx=(200, 900), seed=83, heads=32)
    gc = GpuCase(case)
    cfg = case.cfg
    d_s, d_v = cfg.d_s, 128
    rng = np.random.default_rng(89)
    w_t = rng.standard_normal((cfg.heads, cfg.d_c, d_v)) / 16          # [H, d_c, d_v]
    w_dev = oracle.rotate_weight_rows(w_t) if hadamard else w_t
    w_dev = np.ascontiguousarray(w_dev.transpose(0, 2, 1))          # W_UV layout [H, d_v, d_c]
    _, outs, _ = run_step(gc, hadamard)
    w_gpu = torch.from_numpy(w_dev.astype(np.float32)).cuda().to(torch.bfloat16)
    y = None
    for g in range(cfg.tp):
        wg = w_gpu[:, :, g * d_s:(g + 1) * d_s]                     # column slice
        y = tpla.up_project(outs[g], wg, out=y, accumulate=g > 0)
    torch.cuda.synchronize()
    w_used = host_f64(w_gpu).transpose(0, 2, 1)    # bf16 weights as the kernel saw them, [H, d_c, d_v]
    for b in range(cfg.batch):
        _, parts = oracle_step(case, b, cfg.tp, hadamard=hadamard)
        o_sh = [p[0][None] for p in parts]
        w_sh = [w_used[:, g * d_s:(g + 1) * d_s, :] for g in range(cfg.tp)]
        ref = oracle.up_project_combine(o_sh, w_sh)[0]
        assert rel_err(host_f64(y)[b], ref) <= TOL_BF16, b


@pytest.mark.parametrize("d_s", [100, 12, 264])
def test_up_project_aligned_float32_partial_kstep(d_s):
    # contiguous float32 o and w with d_s % 8 == 4: 16-byte reads whose last
    # window is shifted back into the row
    rng = np.random.default_rng(d_s)
    o = torch.from_numpy(rng.standard_normal((9, 3, d_s)).astype(np.float32)).cuda()
    w = torch.from_numpy(rng.standard_normal((3, 40, d_s)).astype(np.float32)).cuda()
    y = tpla.up_project(o, w)
    torch.cuda.synchronize()
    ref = oracle.up_project_shard(host_f64(o), host_f64(w).transpose(0, 2, 1))
    assert rel_err(host_f64(y), ref) <= TOL_FP32


# --------------------------------------------------------------------------
# MLA-form prefill (tpla_mla_prefill)
# --------------------------------------------------------------------------

from tensor_latent_decode_amd.inputs import PREFILL_CONFIGS, make_prefill_case  # noqa: E402

SENTINEL = 7.0


def prefill_ref(pc, b):
    """The oracle's causal MLA attention over prompt b."""
    L = int(pc.seq_lens[b])
    kv = as_f64(pc.kv[b, :L])
    d_c = pc.cfg.d_c
    return oracle.mla_prefill(as_f64(pc.q_latent[b, :L]), as_f64(pc.q_rope[b, :L]), kv[:, :d_c],
                              kv[:, d_c:], pc.cfg.scale)


def run_prefill(pc, out_dtype=torch.float32, lens=None):
    B, S, H, d_c = pc.q_latent.shape
    out = torch.full((B, S, H, d_c), SENTINEL, dtype=out_dtype, device="cuda")
    lse = torch.full((B, S, H), SENTINEL, dtype=torch.float32, device="cuda")
    lens = dev(pc.seq_lens) if lens is None else lens
    tpla.mla_prefill(dev(pc.q_latent), dev(pc.q_rope), dev(pc.kv), lens, pc.cfg.scale, out=out,
                     lse=lse)
    torch.cuda.synchronize()
    return host_f64(out), host_f64(lse)


@pytest.mark.parametrize("heads", [16, 64, 128, 3, 40])
@pytest.mark.parametrize("out_dt", [torch.float32, torch.bfloat16])
def test_prefill_parity(heads, out_dt):
    """Every position of ragged prompts against the oracle; heads that are not
    a multiple of 64 put several positions into one workgroup's rows."""
    pc = make_prefill_case(PREFILL_CONFIGS["prefill_small"], heads=heads, seed=90 + heads)
    out, lse = run_prefill(pc, out_dt)
    for b in range(pc.cfg.batch):
        L = int(pc.seq_lens[b])
        ref_o, ref_l = prefill_ref(pc, b)
        assert rel_err(out[b, :L], ref_o) <= TOL_BF16, (b, L)
        assert np.max(np.abs(lse[b, :L] - ref_l)) <= 2e-2, (b, L)
        assert np.all(out[b, L:] == SENTINEL) and np.all(lse[b, L:] == SENTINEL)


def test_prefill_tile_edge_lengths_and_empty_prompt():
    pc = make_prefill_case(PREFILL_CONFIGS["prefill_small"], batch=6, heads=64, lens=97,
                           max_len=97, seed=95)
    lens_host = np.array([0, 1, 31, 32, 33, 97], dtype=np.int32)
    pc.seq_lens = lens_host
    out, lse = run_prefill(pc)
    assert np.all(out[0] == SENTINEL) and np.all(lse[0] == SENTINEL)
    for b in range(1, 6):
        L = int(lens_host[b])
        ref_o, ref_l = prefill_ref(pc, b)
        assert rel_err(out[b, :L], ref_o) <= TOL_BF16, L
        assert np.max(np.abs(lse[b, :L] - ref_l)) <= 2e-2, L
        assert np.all(out[b, L:] == SENTINEL)


def test_prefill_late_score_spike():
    """A key far inside the prompt scores ~260 (base-2 units) above everything
    before it for one row: a softmax that kept the first tile's max would
    overflow; every row must still match the oracle."""
    pc = make_prefill_case(PREFILL_CONFIGS["prefill_small"], batch=1, heads=64, lens=180,
                           max_len=180, seed=96)
    q0 = as_f64(pc.q_latent[0, 170, 5])
    k = 2500.0 / (pc.cfg.scale * float(q0 @ q0))
    from tensor_latent_decode_amd.inputs import bf16_bits
    pc.kv[0, 130, :512] = bf16_bits((k * q0).astype(np.float32))
    out, lse = run_prefill(pc)
    ref_o, ref_l = prefill_ref(pc, 0)
    for t in (129, 130, 170, 179):
        for h in (0, 5, 63):
            assert rel_err(out[0, t, h], ref_o[t, h]) <= TOL_BF16, (t, h)
    assert rel_err(out[0], ref_o) <= TOL_BF16
    assert np.max(np.abs(lse[0] - ref_l)) <= 2e-2


@pytest.mark.parametrize("heads", [16, 64])
def test_prefill_strided_buffers_give_the_same_bits(heads):
    pc = make_prefill_case(PREFILL_CONFIGS["prefill_small"], heads=heads, seed=97)
    B, S, H, d_c = pc.q_latent.shape
    base, _ = run_prefill(pc)
    wq = torch.zeros((B, S, H, 640), dtype=torch.bfloat16, device="cuda")
    wq[..., 64:576] = dev(pc.q_latent)
    wr = torch.zeros((B, S, H, 72), dtype=torch.bfloat16, device="cuda")
    wr[..., 8:72] = dev(pc.q_rope)
    wkv = torch.zeros((B, S, 640), dtype=torch.bfloat16, device="cuda")
    wkv[..., :576] = dev(pc.kv)
    wout = torch.full((B, S, H, 520), SENTINEL, dtype=torch.float32, device="cuda")
    tpla.mla_prefill(wq[..., 64:576], wr[..., 8:72], wkv[..., :576], dev(pc.seq_lens), pc.cfg.scale,
                     out=wout[..., :512])
    torch.cuda.synchronize()
    got = host_f64(wout)
    assert np.array_equal(got[..., :512], base)
    assert np.all(got[..., 512:] == SENTINEL)


@pytest.mark.parametrize("out_dt,width", [(torch.float32, 516), (torch.bfloat16, 520), (torch.bfloat16, 516)])
def test_prefill_output_rows_aligned_or_not_give_the_same_bits(out_dt, width):
    """Output rows whose byte stride is a multiple of 16 (float 516, bf16 520
    wide) go out as whole 16-byte chunks, a bf16 stride of 516 (8-byte
    aligned, which the call accepts) as 8-byte pieces; both give the bits of
    the packed output and leave the row padding alone."""
    pc = make_prefill_case(PREFILL_CONFIGS["prefill_small"], heads=64, seed=98)
    B, S, H, d_c = pc.q_latent.shape
    base, _ = run_prefill(pc, out_dtype=out_dt)
    wout = torch.full((B, S, H, width), SENTINEL, dtype=out_dt, device="cuda")
    tpla.mla_prefill(dev(pc.q_latent), dev(pc.q_rope), dev(pc.kv), dev(pc.seq_lens), pc.cfg.scale,
                     out=wout[..., :512])
    torch.cuda.synchronize()
    got = host_f64(wout)
    assert np.array_equal(got[..., :512], base)
    assert np.all(got[..., 512:] == host_f64(torch.full((1,), SENTINEL, dtype=out_dt))[0])


@pytest.mark.parametrize("scale", [0.0, -0.06])
def test_prefill_zero_and_negative_scale(scale):
    """A zero scale weighs every visible key equally; a negative one flips the
    scores (64 heads: the role-split kernel's sign and zero handling)."""
    from dataclasses import replace
    pc = make_prefill_case(PREFILL_CONFIGS["prefill_small"], batch=2, heads=64, lens=140,
                           max_len=140, seed=99)
    pc.cfg = replace(pc.cfg, scale=scale)
    out, lse = run_prefill(pc)
    for b in range(2):
        L = int(pc.seq_lens[b])
        ref_o, ref_l = prefill_ref(pc, b)
        assert rel_err(out[b, :L], ref_o) <= TOL_BF16, (b, scale)
        assert np.max(np.abs(lse[b, :L] - ref_l)) <= 2e-2, (b, scale)


def test_prefill_4k_sampled():
    """The benchmarked shape (64 heads, 4096-token prompts), one prompt;
    sampled positions against the oracle's decode over the prefix (the
    prefill row identity pinned in the oracle tests)."""
    pc = make_prefill_case(PREFILL_CONFIGS["mla_prefill_4k"], batch=1)
    out, lse = run_prefill(pc)
    kv = as_f64(pc.kv[0])
    for t in (0, 1, 31, 32, 33, 1000, 2047, 4095):
        ref_o, ref_l = oracle.mla_decode(as_f64(pc.q_latent[0, t]), as_f64(pc.q_rope[0, t]),
                                         kv[:t + 1, :512], kv[:t + 1, 512:], pc.cfg.scale)
        assert rel_err(out[0, t], ref_o) <= TOL_BF16, t
        assert np.max(np.abs(lse[0, t] - ref_l)) <= 2e-2, t


def test_prefill_then_tpla_decode():
    """The hand-off: the prompt's rows go into the two shard caches through
    tpla_rotate_append, the next token's row is appended, and the TPLA decode
    of the next query over the whole prompt matches the oracle's TPLA decode."""
    pc = make_prefill_case(PREFILL_CONFIGS["prefill_small"], batch=2, heads=64, lens=150,
                           max_len=151, seed=98)
    B, S, H, d_c = pc.q_latent.shape
    tp, d_s, bs = 2, 256, 64
    L = 150                                     # prompt; position 150 is the next token
    _, _ = run_prefill(pc)
    nb = (S + bs - 1) // bs
    bt = torch.arange(B * nb, dtype=torch.int32, device="cuda").view(B, nb)
    caches = [torch.zeros((B * nb, bs, d_s + 64), dtype=torch.bfloat16, device="cuda")
              for _ in range(tp)]
    kv = dev(pc.kv)
    rows = kv[:, :L + 1].reshape(B * (L + 1), 576)
    seq = torch.arange(B, dtype=torch.int32, device="cuda").repeat_interleave(L + 1)
    pos = torch.arange(L + 1, dtype=torch.int32, device="cuda").repeat(B)
    tpla.rotate_append(None, None, rows[:, :512], rows[:, 512:], seq, pos, caches, bt)
    q_next = dev(np.ascontiguousarray(pc.q_latent[:, L]))
    qr_next = dev(np.ascontiguousarray(pc.q_rope[:, L]))
    q_rot = tpla.hadamard_latent(q_next)
    lens = torch.full((B,), L + 1, dtype=torch.int32, device="cuda")
    outs = [tpla.decode_shard(q_rot[:, :, g * d_s:(g + 1) * d_s], qr_next, caches[g], bt, lens,
                              pc.cfg.scale, L + 1)[0] for g in range(tp)]
    got = host_f64(tpla.combine_shards(outs))
    for b in range(B):
        kvb = as_f64(pc.kv[b, :L + 1])
        ref = oracle.tpla_decode(as_f64(pc.q_latent[b, L]), as_f64(pc.q_rope[b, L]), kvb[:, :512],
                                 kvb[:, 512:], tp, pc.cfg.scale, hadamard=True)
        assert rel_err(got[b], ref) <= TOL_BF16, b
