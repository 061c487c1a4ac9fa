"""Pins for the CPU oracle: each check comes from outside the oracle itself.

Brute force (pure-Python loops with exact decoding via ``struct``), closed
forms, identities, special cases that reduce to a library routine, and the
shapes the pages print (tests/golden/page_shapes.json).  Chosen so that a
dropped term, a wrong sign or index, or a transposed operand fails at least
one of them.  CPU only.
"""

import json
import math
import os
import random
import struct

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers
def py_bf16_to_float(bits):
    """Independent bf16 decode: 16 bits into the top of a big-endian binary32."""
    return struct.unpack(">f", struct.pack(">I", (int(bits) & 0xFFFF) << 16))[0]


def stored_elem(flat, ld, r, c):
    return py_bf16_to_float(flat[r * ld + c])


def brute_gemm(transA, transB, M, N, K, A, lda, B, ldb):
    """Triple loop straight from the definition of op(X) and the product."""
    out = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            terms = []
            for k in range(K):
                a = stored_elem(A, lda, m, k) if transA == "N" else stored_elem(A, lda, k, m)
                b = stored_elem(B, ldb, k, n) if transB == "N" else stored_elem(B, ldb, n, k)
                terms.append(a * b)
            out[m][n] = math.fsum(terms)
    return np.array(out, dtype=np.float64)


def case(M, N, K, ta, tb, seed, **kw):
    d = workloads.random_operands(M, N, K, ta, tb, seed, **kw)
    return (workloads.bf16_bits(d["A"]).reshape(-1), d["lda"],
            workloads.bf16_bits(d["B"]).reshape(-1), d["ldb"], d)


LAYOUTS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


# ------------------------------------------------------------------- bf16
@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
    (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just above the tie
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),    # rounds past the largest -> inf
    (2.0 ** -133, 0x0001),                     # smallest subnormal
    (2.0 ** -134, 0x0000),                     # tie -> even (zero)
    (3 * 2.0 ** -134, 0x0002),                 # tie -> even (2)
    (2.0 ** -126, 0x0080),                     # smallest normal
])
def test_bf16_encode_known(value, bits):
    assert int(oracle.f64_to_bf16_bits(np.array([value]))[0]) == bits


def test_bf16_nan():
    assert int(oracle.f64_to_bf16_bits(np.array([np.nan]))[0]) & 0x7FFF > 0x7F80


def test_bf16_matches_torch_on_fp32_values():
    # for values that are exact fp32, one rounding from fp64 equals torch's
    # fp32 -> bf16 round-to-nearest-even (library cross-check)
    g = torch.Generator().manual_seed(7)
    x = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 20)
    ours = oracle.f64_to_bf16_bits(x.double().numpy())
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode_exact():
    bits = np.arange(0, 65536, 37, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    for b, v in zip(bits[::50], got[::50]):
        ref = py_bf16_to_float(b)
        assert (math.isnan(ref) and math.isnan(v)) or ref == v


# ------------------------------------------------------------------- GEMM
TINY = [(1, 1, 1), (3, 5, 7), (7, 3, 13), (13, 17, 2), (5, 9, 16), (17, 1, 9), (2, 16, 1),
        (9, 4, 9), (6, 6, 6),  # square cases catch a transpose swapped for a no-op
        (1, 11, 14), (1, 1, 17)]  # a row vector times a matrix, a dot product


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", TINY)
def test_gemm_brute_force(ta, tb, M, N, K):
    A, lda, B, ldb, _ = case(M, N, K, ta, tb, seed=M * 1000 + N * 10 + K, pad=3)
    got = oracle.gemm(ta, tb, M, N, K, A, lda, B, ldb)
    ref = brute_gemm(ta, tb, M, N, K, A, lda, B, ldb)
    assert got.shape == (M, N)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_gemm_nt_equals_nn_on_explicit_transpose():
    M, N, K = 33, 47, 61
    A, lda, B, ldb, d = case(M, N, K, "N", "T", seed=11)
    nt = oracle.gemm("N", "T", M, N, K, A, lda, B, ldb)
    w = d["B"]                                   # stored [N, K]
    wt = workloads.bf16_bits(w.t().contiguous()).reshape(-1)
    nn = oracle.gemm("N", "N", M, N, K, A, lda, wt, N)
    assert np.array_equal(nt, nn)


def test_gemm_all_layouts_agree_bitwise():
    M, N, K = 40, 24, 72
    outs = []
    for ta, tb in LAYOUTS:
        A, lda, B, ldb, _ = case(M, N, K, ta, tb, seed=5)      # same logical matrices
        outs.append(oracle.gemm(ta, tb, M, N, K, A, lda, B, ldb))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_gemm_integer_exact(ta, tb):
    M, N, K = 29, 31, 1024
    A, lda, B, ldb, d = case(M, N, K, ta, tb, seed=3, int_range=4)
    got = oracle.gemm(ta, tb, M, N, K, A, lda, B, ldb)
    ref = d["opA"].to(torch.int64) @ d["opB"].to(torch.int64)
    assert np.array_equal(got, ref.numpy().astype(np.float64))


@pytest.mark.parametrize("tb", ["N", "T"])
def test_gemm_identity_left(tb):
    K = N = 19
    eye = torch.eye(K, dtype=torch.bfloat16)
    d = workloads.random_operands(K, N, K, "N", tb, seed=9)
    A = workloads.bf16_bits(eye).reshape(-1)
    B = workloads.bf16_bits(d["B"]).reshape(-1)
    got = oracle.gemm("N", tb, K, N, K, A, K, B, d["ldb"])
    assert np.array_equal(got, d["opB"].double().numpy())


def test_gemm_k1_is_outer_product():
    M, N = 37, 53
    A, lda, B, ldb, d = case(M, N, 1, "N", "N", seed=4)
    got = oracle.gemm("N", "N", M, N, 1, A, lda, B, ldb)
    ref = np.multiply.outer(d["opA"].double().numpy()[:, 0], d["opB"].double().numpy()[0])
    assert np.array_equal(got, ref)


def test_gemm_torch_fp64_crosscheck():
    M, N, K = 64, 80, 96
    A, lda, B, ldb, d = case(M, N, K, "T", "T", seed=8)
    got = oracle.gemm("T", "T", M, N, K, A, lda, B, ldb)
    ref = torch.matmul(d["opA"].double(), d["opB"].double()).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_gemm_rows_subset():
    M, N, K = 50, 30, 20
    A, lda, B, ldb, _ = case(M, N, K, "T", "N", seed=10)
    full = oracle.gemm("T", "N", M, N, K, A, lda, B, ldb)
    rows = [0, 7, 49]
    sub = oracle.gemm("T", "N", M, N, K, A, lda, B, ldb, rows=rows)
    assert np.array_equal(sub, full[rows])


def test_gemm_rejects_short_buffer():
    with pytest.raises(ValueError):
        oracle.gemm("N", "N", 4, 4, 4, np.zeros(10, np.uint16), 4, np.zeros(16, np.uint16), 4)


# ---------------------------------------------------------- cross-entropy
def brute_ce_row(y, label):
    """Unshifted textbook form: log(sum exp(y_j)) - y_label, exact sums."""
    lse = math.log(math.fsum(math.exp(v) for v in y))
    return lse - y[label]


def test_ce_zero_logits_closed_form():
    for N in (1, 2, 256, 32000):
        y = np.zeros((3, N))
        labels = np.array([0, N - 1, N // 2])
        loss, grad, lse = oracle.cross_entropy(y, labels)
        assert np.all(np.abs(loss - math.log(N)) <= 1e-15 * max(1.0, math.log(N)))
        onehot = np.zeros((3, N))
        onehot[np.arange(3), labels] = 1
        np.testing.assert_allclose(grad, 1.0 / N - onehot, rtol=0, atol=1e-16)


def test_ce_constant_rows_give_ln_n():
    y = np.full((4, 1000), 3.25)
    loss, _, _ = oracle.cross_entropy(y, np.array([1, 2, 3, 999]))
    np.testing.assert_allclose(loss, math.log(1000), rtol=1e-14)


def test_ce_brute_force_and_invariants():
    rng = np.random.default_rng(0)
    M, N = 12, 77
    y = rng.normal(size=(M, N)) * 3
    labels = rng.integers(0, N, M)
    loss, grad, lse = oracle.cross_entropy(y, labels)
    for i in range(M):
        assert abs(loss[i] - brute_ce_row(list(y[i]), labels[i])) <= 1e-12 * max(1, abs(loss[i]))
    assert np.all(loss >= 0)
    assert np.all(np.abs(grad.sum(axis=1)) <= 1e-12)
    # grad is softmax minus one-hot: label entry negative, the rest positive
    assert np.all(grad[np.arange(M), labels] < 0)
    mask = np.ones_like(grad, bool)
    mask[np.arange(M), labels] = False
    assert np.all(grad[mask] > 0)


def test_ce_single_column():
    loss, grad, _ = oracle.cross_entropy(np.array([[5.0], [-7.0]]), np.array([0, 0]))
    assert np.all(loss == 0) and np.all(grad == 0)


def test_ce_large_logits_need_the_max_shift():
    y = np.array([[1000.0, 1001.0, 999.0], [-2000.0, -2001.0, -2003.0]])
    loss, grad, _ = oracle.cross_entropy(y, np.array([1, 2]))
    assert np.all(np.isfinite(loss)) and np.all(np.isfinite(grad))
    ref0 = brute_ce_row([-1.0, 0.0, -2.0], 1)          # shift-invariance by hand
    ref1 = brute_ce_row([1.0, 0.0, -2.0], 2)
    # the logits are ~1e3, so the loss carries ~1e3 * eps of cancellation error
    np.testing.assert_allclose(loss, [ref0, ref1], rtol=0, atol=1e-12)


def test_ce_torch_crosscheck():
    g = torch.Generator().manual_seed(3)
    y = torch.randn(32, 300, generator=g, dtype=torch.float64) * 4
    labels = torch.randint(0, 300, (32,), generator=g)
    loss, grad, lse = oracle.cross_entropy(y.numpy(), labels.numpy())
    ref_loss = torch.nn.functional.cross_entropy(y, labels, reduction="none")
    ref_grad = torch.softmax(y, 1) - torch.nn.functional.one_hot(labels, 300).double()
    np.testing.assert_allclose(loss, ref_loss.numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(grad, ref_grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, torch.logsumexp(y, 1).numpy(), rtol=1e-14)


def test_ce_out_of_range_label_is_nan():
    y = np.random.default_rng(1).normal(size=(3, 10))
    loss, grad, _ = oracle.cross_entropy(y, np.array([3, 10, -1]))
    assert np.isfinite(loss[0]) and np.isnan(loss[1]) and np.isnan(loss[2])
    np.testing.assert_allclose(grad[1].sum(), 1.0, rtol=1e-14)   # plain softmax


# --------------------------------------------------------------- merge
def test_merge_any_split_any_order():
    rng = np.random.default_rng(2)
    M, N = 9, 1000
    y = rng.normal(size=(M, N)) * 10
    _, _, lse = oracle.cross_entropy(y, np.zeros(M, int))
    splits = [list(range(0, N + 1, 256)) + [N], sorted(set([0, N] + list(rng.integers(0, N, 13))))]
    for edges in splits:
        edges = sorted(set(edges))
        ms, ss = oracle.tile_partials(y, edges)
        for order in (None, list(reversed(range(len(edges) - 1))),
                      list(rng.permutation(len(edges) - 1))):
            m, s, l2 = oracle.merge_partials(ms, ss, order)
            np.testing.assert_allclose(l2, lse, rtol=1e-13)
            assert np.array_equal(m, y.max(axis=1))
            np.testing.assert_allclose(s, np.exp(y - m[:, None]).sum(1), rtol=1e-12)


def test_merge_identity_and_empty_tiles():
    y = np.array([[1.0, 2.0, 3.0]])
    ms, ss = oracle.tile_partials(y, [0, 0, 2, 2, 3, 3])
    assert np.isneginf(ms[0][0]) and ss[0][0] == 0
    m, s, lse = oracle.merge_partials(ms, ss)
    assert m[0] == 3.0
    np.testing.assert_allclose(lse[0], math.log(math.exp(1) + math.exp(2) + math.exp(3)), rtol=1e-14)
    mm, s2 = oracle.merge_pair(-np.inf, 0.0, -np.inf, 0.0)
    assert np.isneginf(mm) and s2 == 0


# ---------------------------------------------------------------- K = 1
def test_k1_outer_is_fp32_product():
    rng = np.random.default_rng(5)
    a = rng.normal(size=100).astype(np.float32)
    b = (rng.normal(size=70) * 1e3).astype(np.float32)
    t = oracle.k1_outer(a, b)
    assert t.dtype == np.float32
    assert np.array_equal(t, np.float32(a)[:, None] * np.float32(b)[None, :])


def test_rope_tables_structure_and_special_cases():
    w = workloads.rope()
    ang, cos, sin = oracle.rope_tables(w["pos"].numpy(), w["inv_freq"].numpy())
    pos = w["pos"].numpy()
    inv = w["inv_freq"].numpy()
    assert ang.shape == (4096, 64) and ang.dtype == np.float32
    assert cos.shape == (4096, 128) and sin.shape == (4096, 128)
    # the angles are the fp32 products (NumPy's own fp32 multiply)
    assert np.array_equal(ang, pos.astype(np.float32)[:, None] * inv[None, :])
    # the page's order ([frequencies] x [positions], then a permute) gives the
    # same bits: an fp32 product is exactly rounded and commutes
    assert np.array_equal(oracle.k1_outer(inv, pos.astype(np.float32)).T, ang)
    assert np.array_equal(cos[:, :64], cos[:, 64:]) and np.array_equal(sin[:, :64], sin[:, 64:])
    assert np.all(cos[0] == 0x3F80) and np.all(sin[0] == 0)          # position 0
    assert inv[0] == 1.0 and np.array_equal(ang[:, 0], pos.astype(np.float32))
    c = oracle.bf16_bits_to_f64(cos)
    s = oracle.bf16_bits_to_f64(sin)
    assert np.max(np.abs(c * c + s * s - 1)) <= 2 * 2.0 ** -7
    rng = random.Random(0)
    for _ in range(300):
        p, d = rng.randrange(4096), rng.randrange(128)
        x = float(np.float32(float(pos[p])) * np.float32(inv[d % 64]))   # python-side fp32 angle
        assert x == float(ang[p, d % 64])
        assert abs(py_bf16_to_float(cos[p, d]) - math.cos(x)) <= 2.0 ** -9
        assert abs(py_bf16_to_float(sin[p, d]) - math.sin(x)) <= 2.0 ** -9


def test_rope_inv_freq_input():
    inv = workloads.inv_freq().numpy()
    for i in (0, 1, 31, 63):
        assert inv[i] == np.float32(10000.0 ** (-(2 * i) / 128.0))


def test_rope_region_query_steps_brute_force():
    """View [P, H, D], permute to [H, P, D], widen: element by element with
    Python loops and the struct decode, on a strided tiny case."""
    rng = np.random.default_rng(9)
    P, H, D, ldq = 5, 3, 4, 14
    bits = rng.integers(0, 2 ** 16, size=(P - 1) * ldq + H * D).astype(np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] = 0x3F80          # no NaN / inf patterns
    pos = np.array([0, 3, 7, 100, 4095])
    q_heads, ang, cos, sin = oracle.rope_region(bits, ldq, P, H, D, pos, workloads.inv_freq(D).numpy())
    assert q_heads.shape == (H, P, D)
    for h in range(H):
        for p in range(P):
            for d in range(D):
                assert q_heads[h, p, d] == py_bf16_to_float(int(bits[p * ldq + h * D + d]))
    ang2, cos2, sin2 = oracle.rope_tables(pos, workloads.inv_freq(D).numpy())
    assert np.array_equal(ang, ang2) and np.array_equal(cos, cos2) and np.array_equal(sin, sin2)


def test_rope_region_matches_torch_view_permute():
    """Library cross-check: torch's view / permute / float of the same bf16
    tensor, at the page's shapes ([1, 4096, 4096] -> [1, 4096, 32, 128] ->
    [1, 32, 4096, 128])."""
    w = workloads.rope_region()
    q = w["q"]
    P, HD = q.shape
    H, D = w["heads"], HD // w["heads"]
    q_heads, _, _, _ = oracle.rope_region(workloads.bf16_bits(q), HD, P, H, D, w["pos"].numpy(),
                                          w["inv_freq"].numpy())
    ref = q.view(1, P, H, D).permute(0, 2, 1, 3).float()
    assert np.array_equal(q_heads, ref[0].double().numpy())


# -------------------------------------------------------------- golden
def test_golden_page_shapes():
    with open(os.path.join(GOLDEN, "page_shapes.json")) as f:
        g = json.load(f)
    nt = g["nt_down_projection"]
    w = workloads.nt_mlp(batch=nt["input"]["shape"][0], pairs=nt["input"]["shape"][1],
                         hidden=64, out=40)          # shrunk K/N, same leading dims
    x = w["X"]
    assert list(x.shape[:2]) == nt["input"]["shape"][:2]
    flat = x.reshape(-1, x.shape[-1])
    assert list(flat.shape[:1]) == nt["flattened_input"]["shape"][:1]
    assert flat.data_ptr() == x.data_ptr()            # flattening is a view
    r = g["rope_region"]
    ang, cos, sin = oracle.rope_tables(workloads.rope()["pos"].numpy(),
                                       workloads.rope()["inv_freq"].numpy())
    assert [1] + list(ang.T.shape) == r["matmul_T19"]["shape"]
    assert [1] + list(ang.shape) == r["permute_T20"]["shape"]
    assert [1] + list(cos.shape) == r["cat_T23"]["shape"]
    assert [1, 1] + list(cos.shape) == r["outputs_T29_T31"]["shape"]
    assert [1, 1] + list(sin.shape) == r["outputs_T29_T31"]["shape"]
    assert list(workloads.rope()["inv_freq"].shape) == r["inv_freq_T3"]["shape"]
    rr = workloads.rope_region()
    assert [1] + list(rr["q"].shape) == r["query_T0"]["shape"]
    H = rr["heads"]
    D = rr["q"].shape[1] // H
    assert [1, rr["q"].shape[0], H, D] == r["view_T5"]["shape"]
    assert [1, H, rr["q"].shape[0], D] == r["permute_T6"]["shape"] == r["cast_T34"]["shape"]


# --------------------------------------------------------------- fp8 (e4m3fn)
def torch_e4m3(y_f32):
    """Library routine: torch's CPU cast to float8_e4m3fn and back."""
    return torch.from_numpy(np.asarray(y_f32, dtype=np.float32)).to(torch.float8_e4m3fn).double().numpy()


def all_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_grid_is_fixed_and_complete():
    """Every finite e4m3fn value (decoded by torch from all 256 codes) is a
    fixed point of the rounding; the set has 253 distinct finite values from
    -448 to 448 and exactly two NaN codes."""
    v = all_e4m3_values()
    fin = v[np.isfinite(v)]
    assert np.isnan(v).sum() == 2 and np.isinf(v).sum() == 0
    assert len(np.unique(fin)) == 253 and fin.max() == 448.0 and fin.min() == -448.0
    assert oracle.E4M3_MAX == 448.0
    assert np.array_equal(oracle.e4m3_round(fin), fin)


def test_e4m3_round_matches_library_cast_on_ties_and_random():
    """Midpoints between neighbouring e4m3fn values (the ties), their fp32
    neighbours, and random values in range: the oracle's rounding equals
    torch's cast bit for bit (as values)."""
    fin = np.unique(all_e4m3_values()[np.isfinite(all_e4m3_values())])
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)  # exact in fp32
    ys = [fin.astype(np.float32), mids,
          np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))]
    rng = np.random.default_rng(5)
    ys += [(rng.standard_normal(20000) * 40).astype(np.float32),
           (rng.standard_normal(5000) * 0.004).astype(np.float32)]
    y = np.concatenate(ys)
    y = y[np.abs(y) <= 448]
    assert np.array_equal(oracle.e4m3_round(y), torch_e4m3(y))


@pytest.mark.parametrize("x,expect", [
    (1.0625, 1.0),            # halfway between 1 and 1.125: even fraction 000
    (1.1875, 1.25),           # halfway between 1.125 and 1.25: even fraction 010
    (2.0 ** -10, 0.0),        # half the smallest subnormal: ties to zero
    (3 * 2.0 ** -10, 2.0 ** -8),  # 1.5 subnormal steps: ties to 2 steps
    (2.0 ** -9, 2.0 ** -9),   # smallest subnormal
    (0.0146484375, 0.015625),  # 7.5 * 2^-9: ties to 8 * 2^-9 = 2^-6, the smallest normal
    (440.0, 448.0),           # 13.75 steps of 32 above 0: to 14
    (-0.0, -0.0),
])
def test_e4m3_round_closed_forms(x, expect):
    got = float(oracle.e4m3_round(np.float32(x)))
    assert got == expect and math.copysign(1.0, got) == math.copysign(1.0, expect)


def test_quantize_scale_clamp_nan():
    """The page's cast: fp32 multiply, clamp to the largest finite value, round."""
    x = np.array([1.0, 30.0, -50.0, 44.8, 0.3, np.nan, np.inf, -np.inf], dtype=np.float32)
    q = oracle.quantize(x, 10.0)
    # 300 rounds to 288 (spacing 32 above 256), -500 clamps, 44.8 * 10 rounds to 448
    assert list(q[:5]) == [10.0, 288.0, -448.0, 448.0, 3.0]
    assert np.isnan(q[5]) and q[6] == 448.0 and q[7] == -448.0
    # the multiply rounds once in fp32 before the cast (0.1f * 3 is not 0.3)
    s = np.float32(0.1)
    y = np.float32(np.float32(3.0) * s)
    assert oracle.quantize(np.float32(3.0), s) == torch_e4m3(y)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (9, 4, 9), (1, 6, 11), (5, 1, 4)])
def test_gemm_fp8_brute_force(ta, tb, M, N, K):
    """Triple loop with each operand element cast by torch (the library
    routine), against the oracle; scales and an output scale included."""
    A, lda, B, ldb, _ = case(M, N, K, ta, tb, seed=M * 77 + N * 7 + K, pad=2, std=100.0)
    sa, sb, so = 0.7, 3.0, 0.125
    got = oracle.gemm_fp8(ta, tb, M, N, K, A, lda, B, ldb, sa, sb, so)

    def qv(v, s):
        y = np.clip(np.float32(v) * np.float32(s), -448, 448).astype(np.float32)
        return float(torch_e4m3(np.array([y]))[0])

    ref = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            terms = []
            for k in range(K):
                a = stored_elem(A, lda, m, k) if ta == "N" else stored_elem(A, lda, k, m)
                b = stored_elem(B, ldb, k, n) if tb == "N" else stored_elem(B, ldb, n, k)
                terms.append(qv(a, sa) * qv(b, sb))
            ref[m, n] = math.fsum(terms) * so
    assert np.array_equal(got, ref)


def test_gemm_fp8_reduces_to_gemm_on_small_integers():
    """Integers in [-8, 8] are e4m3fn values: with unit scales the fp8 GEMM is
    the bf16 GEMM exactly (a special case that reduces to the plain oracle)."""
    for ta, tb in LAYOUTS:
        A, lda, B, ldb, _ = case(40, 24, 70, ta, tb, seed=3, int_range=8)
        assert np.array_equal(oracle.gemm_fp8(ta, tb, 40, 24, 70, A, lda, B, ldb, 1.0, 1.0),
                              oracle.gemm(ta, tb, 40, 24, 70, A, lda, B, ldb))
