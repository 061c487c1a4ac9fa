"""GPU parity of the K=1 pointwise paths (RoPE cos/sin table, fp32 outer)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from layout_aware_gemm_amd import tgemm
from parity_util import K1_F32_ABS_TOL, TRIG_ABS_TOL, bf16_to_f64, bits, dev

pytestmark = pytest.mark.gpu


def check_tables(cos, sin, pos, inv_freq, rows=None):
    pos_np = pos.cpu().numpy() if rows is None else pos.cpu().numpy()[rows]
    _, rc, rs = oracle.rope_tables(pos_np, inv_freq.cpu().numpy())
    c = bits(cos) if rows is None else bits(cos[torch.as_tensor(rows, device=cos.device)])
    s = bits(sin) if rows is None else bits(sin[torch.as_tensor(rows, device=sin.device)])
    dc = np.abs(oracle.bf16_bits_to_f64(c) - oracle.bf16_bits_to_f64(rc)).max()
    ds = np.abs(oracle.bf16_bits_to_f64(s) - oracle.bf16_bits_to_f64(rs)).max()
    assert dc <= TRIG_ABS_TOL and ds <= TRIG_ABS_TOL
    return float(np.mean(c == rc)), float(np.mean(s == rs))


def test_rope_table_4096x64():
    w = workloads.rope()
    pos, inv = w["pos"].to(dev()), w["inv_freq"].to(dev())
    cos, sin = tgemm.rope_cos_sin(pos, inv)
    torch.cuda.synchronize()
    assert cos.shape == (4096, 128) and sin.shape == (4096, 128)
    fc, fs = check_tables(cos, sin, w["pos"], w["inv_freq"])
    assert fc > 0.99 and fs > 0.99            # nearly all bits equal
    assert torch.equal(cos[:, :64], cos[:, 64:]) and torch.equal(sin[:, :64], sin[:, 64:])
    assert (bits(cos[0]) == 0x3F80).all() and (bits(sin[0]) == 0).all()


@pytest.mark.parametrize("F", [64, 5])
def test_rope_positions_across_the_reduction_range(F):
    """Positions on both sides of the range the short argument reduction
    serves (|t| <= 65536), negative positions and positions up to 2^24:
    rows whose arguments all lie inside take the reduced path, the others
    the library sincosf; every row must match the oracle."""
    rng = np.random.default_rng(7)
    special = [0, 1, -1, 4095, 65535, 65536, 65537, -65536, -65537, 100000, 2 ** 20,
               2 ** 24 - 1, -(2 ** 24 - 1)]
    pos = np.concatenate([special, rng.integers(-2 ** 24 + 1, 2 ** 24, 200),
                          rng.integers(-70000, 70000, 300)]).astype(np.int64)
    inv = workloads.inv_freq(2 * F) if F == 64 else torch.tensor(
        [1.0, 0.5, 3.0e-3, 1.7, 0.25], dtype=torch.float32)
    P = pos.size
    pos_t = torch.from_numpy(pos)
    cos, sin = tgemm.rope_cos_sin(pos_t.to(dev()), inv.to(dev()))
    torch.cuda.synchronize()
    fc, fs = check_tables(cos, sin, pos_t, inv)
    assert fc > 0.97 and fs > 0.97
    assert cos.shape == (P, 2 * F)


def test_rope_product_is_exact_fp32():
    """The K=1 product itself (fp32 outer, positions cast to fp32) must equal
    the oracle bit for bit (max abs error 0 <= 1e-5)."""
    w = workloads.rope()
    posf = w["pos"].to(torch.float32).to(dev())
    inv = w["inv_freq"].to(dev())
    t = tgemm.outer_f32(posf, inv)                      # [4096, 64]
    torch.cuda.synchronize()
    ang, _, _ = oracle.rope_tables(w["pos"].numpy(), w["inv_freq"].numpy())
    got = t.cpu().numpy()
    assert np.array_equal(got, ang)
    assert np.abs(got.astype(np.float64) - ang.astype(np.float64)).max() <= K1_F32_ABS_TOL


def test_rope_batched_256x4096():
    w = workloads.rope_batched(256)
    pos, inv = w["pos"].to(dev()), w["inv_freq"].to(dev())
    cos, sin = tgemm.rope_cos_sin(pos, inv)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([np.arange(0, pos.numel(), 4099),
                                     rng.integers(0, pos.numel(), 2000)]))
    check_tables(cos, sin, w["pos"], w["inv_freq"], rows=rows)
    # sequence b repeats sequence 0 exactly
    assert torch.equal(cos[:4096], cos[4096 * 255:]) and torch.equal(sin[:4096], sin[-4096:])


@pytest.mark.parametrize("P,F,ldc_pad", [(1, 1, 0), (37, 5, 3), (1000, 64, 8), (333, 12, 0)])
def test_rope_ragged_and_strided(P, F, ldc_pad):
    g = torch.Generator().manual_seed(P * F)
    pos = torch.randint(-5000, 5000, (P,), generator=g, dtype=torch.int64)
    inv = workloads.inv_freq(2 * F) if F > 1 else torch.tensor([1.0])
    ldc = 2 * F + ldc_pad
    cos = torch.full((P, ldc), float("nan"), dtype=torch.bfloat16, device=dev())
    sin = torch.full((P, ldc), float("nan"), dtype=torch.bfloat16, device=dev())
    # positions with an element stride of 2 and frequencies stored as an [F, 1] column
    pos2 = torch.stack([pos, pos], 1).reshape(-1).to(dev())
    inv2 = torch.stack([inv, inv], 1).reshape(-1).to(dev())
    tgemm.run("N", "T", P, F, 1, pos2, 2, inv2, 2, cos, ldc, tgemm.EPI_ROPE_COSSIN, out_grad=sin)
    torch.cuda.synchronize()
    check_tables(cos[:, :2 * F], sin[:, :2 * F], pos, inv)
    if ldc_pad:
        assert torch.isnan(cos[:, 2 * F:].float()).all() and torch.isnan(sin[:, 2 * F:].float()).all()


def test_outer_f32_random_exact():
    rng = np.random.default_rng(3)
    a = (rng.normal(size=513) * 100).astype(np.float32)
    b = rng.normal(size=129).astype(np.float32)
    c = tgemm.outer_f32(torch.from_numpy(a).to(dev()), torch.from_numpy(b).to(dev()))
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), oracle.k1_outer(a, b))


def test_rope_region_page_size():
    """The region at the listing's sizes in one launch: the query
    [4096, 32*128] widened and permuted to fp32 [32, 4096, 128] must equal
    the oracle bit for bit (a bf16 -> fp32 widening is exact), and the
    tables must match the oracle as the K = 1 path's do."""
    w = workloads.rope_region()
    q, pos, inv = w["q"].to(dev()), w["pos"].to(dev()), w["inv_freq"].to(dev())
    H = w["heads"]
    q_heads, cos, sin = tgemm.rope_region(q, pos, inv, H)
    torch.cuda.synchronize()
    P, HD = w["q"].shape
    D = HD // H
    ref_q, _, rc, rs = oracle.rope_region(bits(w["q"]).reshape(-1), HD, P, H, D,
                                          w["pos"].numpy(), w["inv_freq"].numpy())
    assert q_heads.shape == (H, P, D)
    assert np.array_equal(q_heads.cpu().numpy().astype(np.float64), ref_q)
    fc, fs = check_tables(cos, sin, w["pos"], w["inv_freq"])
    assert fc > 0.99 and fs > 0.99
    # the same tables as the K = 1 entry point, bit for bit
    c1, s1 = tgemm.rope_cos_sin(pos, inv)
    torch.cuda.synchronize()
    assert torch.equal(c1, cos) and torch.equal(s1, sin)


@pytest.mark.parametrize("P,H,D,qpad,cpad,spos", [(1, 1, 2, 0, 0, 1), (37, 3, 10, 3, 1, 2),
                                                  (333, 5, 16, 0, 8, 1), (70, 2, 128, 5, 0, 3)])
def test_rope_region_ragged_and_strided(P, H, D, qpad, cpad, spos):
    """Odd head widths (the scalar path), padded query rows and table rows,
    strided positions; nothing is written past each table row's D columns."""
    g = torch.Generator().manual_seed(P * H + D)
    ldq = H * D + qpad
    q = torch.randn(P, ldq, generator=g).to(torch.bfloat16)
    pos = torch.randint(-3000, 3000, (P * spos,), generator=g, dtype=torch.int64)
    inv = workloads.inv_freq(D)
    ldc = D + cpad
    cos = torch.full((P, ldc), float("nan"), dtype=torch.bfloat16, device=dev())
    sin = torch.full((P, ldc), float("nan"), dtype=torch.bfloat16, device=dev())
    q_out = torch.full((H * P * D,), float("nan"), dtype=torch.float32, device=dev())
    tgemm.run_rope_region(q.to(dev()), ldq, P, H, D, pos.to(dev()), spos, inv.to(dev()), cos, sin,
                          ldc, q_out)
    torch.cuda.synchronize()
    ref_q, _, rc, rs = oracle.rope_region(bits(q).reshape(-1), ldq, P, H, D,
                                          pos.numpy()[::spos], inv.numpy())
    assert np.array_equal(q_out.cpu().numpy().reshape(H, P, D).astype(np.float64), ref_q)
    check_tables(cos[:, :D], sin[:, :D], pos[::spos], inv)
    if cpad:
        assert torch.isnan(cos[:, D:].float()).all() and torch.isnan(sin[:, D:].float()).all()
