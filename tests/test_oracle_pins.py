"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

None of these retypes the oracle's formula: the expected values come from
format definitions checked against independent library decoders, closed
forms (all-ones, identity, permutation), exact rational arithmetic on tiny
integer inputs, numpy's float64 matmul, and invariants of the epilogue.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import acceptance
import synthetic as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = ("row", "col")


# ---------------------------------------------------------------- decoders

def test_decode_f16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    got = oracle.decode("f16", bits)
    want = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_decode_bf16_all_patterns():
    # bfloat16 is by definition the upper 16 bits of an IEEE binary32
    bits = np.arange(65536, dtype=np.uint32)
    got = oracle.decode("bf16", bits)
    with np.errstate(invalid="ignore"):
        want = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_decode_e4m3_table():
    bits = np.arange(256, dtype=np.uint32)
    got = oracle.decode("f8e4m3", bits)
    want = torch.from_numpy(bits.astype(np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    fin = got[np.isfinite(got)]
    assert fin.size == 254                      # only S.1111.111 is NaN
    assert fin.max() == 448.0 and fin.min() == -448.0
    assert np.min(fin[fin > 0]) == 2.0 ** -9    # smallest subnormal
    assert not np.isinf(got).any()


def test_decode_f32_random_patterns():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    got = oracle.decode("f32", bits)
    with np.errstate(invalid="ignore"):
        want = bits.view(np.float32).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


# ---------------------------------------------------------------- encoder

def _finite_table(dtype):
    bits = np.arange(65536, dtype=np.uint32)
    vals = oracle.decode(dtype, bits)
    keep = np.isfinite(vals) & ~((vals == 0) & (bits >= 0x8000))  # drop -0
    return vals[keep], bits[keep]


def _brute_rne(dtype, x, table):
    """Nearest finite value by exhaustive search; ties to even bit pattern."""
    vals, bits = table
    order = np.argsort(vals)
    vals, bits = vals[order], bits[order]
    out = []
    for v in x:
        if v > vals[-1] or v < vals[0]:
            # beyond the largest finite: RNE overflows to infinity only past
            # the halfway point to the next (unrepresentable) binade step
            top = vals[-1]
            step = top - vals[-2]
            if abs(v) >= abs(top) + step / 2:
                inf = {"f16": 0x7C00, "bf16": 0x7F80}[dtype]
                out.append(np.uint32(inf | (0x8000 if v < 0 else 0)))
                continue
            out.append(bits[-1] if v > 0 else bits[0])
            continue
        i = np.searchsorted(vals, v)
        cands = [j for j in (i - 1, i) if 0 <= j < len(vals)]
        d = [abs(Fraction(float(vals[j])) - Fraction(float(v))) for j in cands]
        m = min(d)
        best = [cands[t] for t in range(len(cands)) if d[t] == m]
        if len(best) > 1:
            best = [j for j in best if bits[j] % 2 == 0]
        b = bits[best[0]]
        if v == 0 or (vals[best[0]] == 0 and np.signbit(v)):
            b = np.uint32(0x8000) if np.signbit(v) else np.uint32(0)
        out.append(b)
    return np.array(out, dtype=np.uint32)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_encode_matches_exhaustive_nearest(dtype):
    rng = np.random.default_rng(2)
    table = _finite_table(dtype)
    vals = table[0]
    # random values, exact ties between neighbours, subnormals, overflow edge
    x = list(rng.standard_normal(300) * np.exp2(rng.integers(-30, 30, 300)))
    fin = np.sort(vals[vals > 0])
    for t in rng.integers(0, fin.size - 1, 200):
        x.append((fin[t] + fin[t + 1]) / 2)          # exact tie in fp64
        x.append(-(fin[t] + fin[t + 1]) / 2)
    x += [fin[0] / 2, fin[0] * 0.75, fin[-1] * 1.001, 1025.0, 1027.0, 1028.0]
    x = np.array(x, dtype=np.float64)
    got = oracle.encode(dtype, x)
    want = _brute_rne(dtype, x, table)
    assert (got == want).all(), np.where(got != want)


def test_encode_f16_matches_numpy():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(50000) * np.exp2(rng.integers(-28, 18, 50000))
    got = oracle.encode("f16", x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16).astype(np.uint32)
    assert (got == want).all()


def test_encode_f32_matches_c_cast():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(50000) * np.exp2(rng.integers(-140, 120, 50000))
    got = oracle.encode("f32", x)
    want = x.astype(np.float32).view(np.uint32)
    assert (got == want).all()


def test_bf16_rounds_1025_to_1024():
    # K + 1 = 1025 is a tie between 1024 and 1032 in bf16; even wins
    assert oracle.decode("bf16", oracle.encode("bf16", [1025.0]))[0] == 1024.0


# ---------------------------------------------------------------- GEMM pins

def _read_golden(name):
    kv = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


def _golden_problem(kv):
    M, N, K = int(kv["M"]), int(kv["N"]), int(kv["K"])
    fill = lambda key, shape: np.full(shape, float(kv[key]), dtype=np.float32)
    dt = kv["dtype"]
    return syn.Problem(M, N, K, syn.cast(fill("fill_a", (M, K)), dt),
                       syn.cast(fill("fill_b", (K, N)), dt),
                       syn.cast(fill("fill_c", (M, N)), dt),
                       float(kv["alpha"]), float(kv["beta"]), None, None,
                       dt, dt, kv["layout"], kv["layout"], kv["layout"])


@pytest.mark.parametrize("name,rows", [("ones_fp16_128.txt", None),
                                       ("ones_fp16_1024.txt", [0, 517, 1023])])
def test_golden_ones(name, rows):
    kv = _read_golden(name)
    p = _golden_problem(kv)
    r = oracle.gemm(p, rows=rows)
    assert (r.ref == float(kv["expect_all"])).all()
    assert (r.d_exact == float(kv["expect_all"])).all()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_ones_closed_form_all_dtypes(dtype):
    K = 256
    p = syn.make_problem(64, 48, K, dtype_ab=dtype, dtype_cd=dtype,
                         dist_a="ones", dist_b="ones", dist_c="ones", beta=1.0)
    r = oracle.gemm(p)
    assert (r.ref == K + 1).all()
    assert (r.d_exact == oracle.decode(dtype, oracle.encode(dtype, [K + 1.0]))[0]).all()


def _with_operand(p, which, logical, dtype):
    layout = {"A": p.la, "B": p.lb, "C": p.lc}[which]
    t = syn.cast(syn.to_storage(logical.astype(np.float32), layout), dtype)
    setattr(p, which, t)
    return p


def _logical(p, which):
    """Logical fp64 values of an operand, via torch's decoder (independent)."""
    t = getattr(p, which).to(torch.float64).numpy()
    layout = {"A": p.la, "B": p.lb, "C": p.lc, "aux": p.lc}[which]
    return t if layout == "row" else t.T


@pytest.mark.parametrize("la,lb,lc", list(itertools.product(LAYOUTS, repeat=3)))
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_identity_and_permutation(la, lb, lc, dtype):
    rng = np.random.default_rng(5)
    M = K = 24
    N = 17
    p = syn.make_problem(M, N, K, dtype_ab=dtype, dtype_cd=dtype, la=la, lb=lb,
                         lc=lc, dist_c="normal", alpha=1.0, beta=1.0, seed=6)
    # A = I: D = B + C, each sum a single rounding of two exact values
    _with_operand(p, "A", np.eye(M, dtype=np.float32), dtype)
    r = oracle.gemm(p)
    want = _logical(p, "B") + _logical(p, "C")
    assert np.array_equal(r.ref, want)
    # A = P (permutation), beta = 0: rows of B permuted, exactly
    perm = rng.permutation(M)
    P = np.zeros((M, K), dtype=np.float32)
    P[np.arange(M), perm] = 1.0
    _with_operand(p, "A", P, dtype)
    p.beta = 0.0
    r = oracle.gemm(p)
    assert np.array_equal(r.ref, _logical(p, "B")[perm])
    assert np.array_equal(r.d_exact, _logical(p, "B")[perm])


def test_permutation_pin_catches_layout_mixup():
    """A planted mistake (B read with the other layout) fails the pin."""
    rng = np.random.default_rng(7)
    M = K = N = 8
    p = syn.make_problem(M, N, K, dtype_ab="f16", dtype_cd="f16", lb="row")
    perm = rng.permutation(M)
    P = np.zeros((M, K), dtype=np.float32)
    P[np.arange(M), perm] = 1.0
    _with_operand(p, "A", P, "f16")
    good = oracle.gemm(p).ref
    p.lb = "col"                                # the planted transposition
    bad = oracle.gemm(p).ref
    p.lb = "row"
    want = _logical(p, "B")[perm]
    assert np.array_equal(good, want) and not np.array_equal(bad, want)


def _fraction_gemm(p, relu):
    A = _logical(p, "A")
    B = _logical(p, "B")
    C = _logical(p, "C") if p.C is not None else None
    al, be = Fraction(float(np.float32(p.alpha))), Fraction(float(np.float32(p.beta)))
    sa = Fraction(float(np.float32(p.scale_a or 1.0)))
    sb = Fraction(float(np.float32(p.scale_b or 1.0)))
    out = []
    for i in range(p.M):
        row = []
        for j in range(p.N):
            acc = sum((Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
                       for k in range(p.K)), Fraction(0))
            v = al * acc * sa * sb
            if be != 0:
                v += be * Fraction(float(C[i, j]))
            if relu and v <= 0:
                v = Fraction(0)
            row.append(v)
        out.append(row)
    return out


@pytest.mark.parametrize("dtype_ab,dtype_cd", [("f32", "f32"), ("f16", "f16"),
                                               ("bf16", "bf16"), ("f8e4m3", "bf16")])
@pytest.mark.parametrize("relu", [False, True])
def test_brute_force_fraction_tiny(dtype_ab, dtype_cd, relu):
    rng = np.random.default_rng(8)
    for trial in range(6):
        M, N, K = (int(v) for v in rng.integers(1, 7, 3))
        la, lb, lc = (LAYOUTS[int(v)] for v in rng.integers(0, 2, 3))
        p = syn.integer_problem(M, N, K, dtype_ab=dtype_ab, dtype_cd=dtype_cd,
                                la=la, lb=lb, lc=lc, lo=-5, hi=5,
                                alpha=float(rng.choice([1.0, 0.75, -1.5])),
                                beta=float(rng.choice([0.0, 1.0, -0.5])),
                                seed=100 + trial)
        if dtype_ab == "f8e4m3":
            p.scale_a, p.scale_b = 0.5, 4.0
        r = oracle.gemm(p, relu=relu)
        exact = _fraction_gemm(p, relu)
        for i in range(M):
            for j in range(N):
                assert Fraction(float(r.ref[i, j])) == exact[i][j]
        want_bits = oracle.encode(dtype_cd, [[float(v) for v in row] for row in exact])
        assert np.array_equal(r.d_bits, want_bits)


@pytest.mark.parametrize("dtype_ab,dtype_cd", [("f32", "f32"), ("f16", "f16"),
                                               ("bf16", "bf16"), ("f8e4m3", "bf16")])
def test_matches_numpy_float64_matmul(dtype_ab, dtype_cd):
    for (M, N, K, la, lb, lc) in [(33, 65, 130, "row", "row", "row"),
                                  (64, 31, 257, "col", "col", "col"),
                                  (50, 70, 96, "row", "col", "col")]:
        p = syn.make_problem(M, N, K, dtype_ab=dtype_ab, dtype_cd=dtype_cd,
                             la=la, lb=lb, lc=lc, dist_c="normal",
                             alpha=0.5, beta=-2.0, seed=9)
        r = oracle.gemm(p)
        A, B, C = _logical(p, "A"), _logical(p, "B"), _logical(p, "C")
        sab = (p.scale_a or 1.0) * (p.scale_b or 1.0)
        want = 0.5 * (A @ B) * sab - 2.0 * C
        S = 0.5 * sab * (np.abs(A) @ np.abs(B))
        assert np.all(np.abs(r.ref - want) <= 4 * K * 2.0 ** -52 * (S + 2 * np.abs(C)))
        assert np.allclose(r.S, S, rtol=1e-12, atol=0)


def test_relu_invariant_and_fused_equals_unfused():
    p = syn.make_problem(40, 52, 77, dtype_ab="f16", dtype_cd="f16",
                         dist_c="normal", alpha=1.0, beta=1.0, seed=10)
    lin = oracle.gemm(p, relu=False)
    fused = oracle.gemm(p, relu=True)
    assert (fused.ref >= 0).all()
    assert np.array_equal(fused.ref, np.maximum(lin.ref, 0.0))
    assert np.array_equal(fused.d_exact, np.maximum(lin.d_exact, 0.0))
    assert (fused.ref == 0).sum() > 0 and (fused.ref > 0).sum() > 0


def test_alpha_power_of_two_doubles_exactly():
    p = syn.make_problem(20, 30, 40, dtype_ab="bf16", dtype_cd="bf16", seed=11)
    r1 = oracle.gemm(p)
    p.alpha = 2.0
    r2 = oracle.gemm(p)
    assert np.array_equal(r2.ref, 2 * r1.ref)
    assert np.array_equal(r2.d_exact, 2 * r1.d_exact)


def test_beta_zero_ignores_c():
    p = syn.make_problem(8, 9, 10, dtype_ab="f16", dtype_cd="f16", dist_c="normal",
                         beta=0.0, seed=12)
    r1 = oracle.gemm(p)
    p.C = torch.full_like(p.C, float("nan"))
    r2 = oracle.gemm(p)
    assert np.array_equal(r1.ref, r2.ref) and np.isfinite(r2.ref).all()


def test_fp8_scales_multiply_exactly():
    p = syn.integer_problem(16, 24, 32, dtype_ab="f8e4m3", dtype_cd="bf16",
                            with_c=False, seed=13)
    r1 = oracle.gemm(p)
    p.scale_a, p.scale_b = 0.25, 8.0
    r2 = oracle.gemm(p)
    assert np.array_equal(r2.ref, 2.0 * r1.ref)


def test_entries_equal_rows():
    p = syn.make_problem(30, 40, 50, dtype_ab="bf16", dtype_cd="bf16", la="col",
                         lb="row", lc="col", dist_c="normal", beta=0.5, seed=14)
    rows = oracle.gemm(p, relu=True)
    rng = np.random.default_rng(15)
    ii, jj = rng.integers(0, 30, 100), rng.integers(0, 40, 100)
    ent = oracle.gemm_entries(p, ii, jj, relu=True)
    assert np.array_equal(ent.ref, rows.ref[ii, jj])
    assert np.array_equal(ent.d_bits, rows.d_bits[ii, jj])


def test_grouped_equals_loop_of_singles():
    probs = syn.config3(seed=3, count=4,
                        shapes=[(32, 128, 128), (64, 256, 128), (96, 128, 256),
                                (32, 512, 128)])
    g = oracle.grouped(probs)
    for p, r in zip(probs, g):
        s = oracle.gemm(p)
        assert np.array_equal(r.ref, s.ref) and np.array_equal(r.d_bits, s.d_bits)


def test_degenerate_sizes():
    p = syn.make_problem(5, 6, 0, dtype_ab="f16", dtype_cd="f16", dist_c="normal",
                         beta=2.0, seed=16)
    r = oracle.gemm(p, relu=True)           # K = 0: D = relu(beta * C)
    assert np.array_equal(r.ref, np.maximum(2.0 * _logical(p, "C"), 0))
    p0 = syn.make_problem(0, 6, 3, dtype_ab="f16", dtype_cd="f16")
    assert oracle.gemm(p0).ref.shape == (0, 6)


def test_acceptance_rules():
    # ulp: one unit in the last place of the output format
    assert acceptance.ulp("f16", 1025.0) == 1.0
    assert acceptance.ulp("bf16", 1.0) == 2.0 ** -7
    assert acceptance.ulp("f32", 0.0) == 2.0 ** -149
    assert acceptance.ulp("f16", 2.0 ** -20) == 2.0 ** -24      # subnormal quantum
    tol = acceptance.tolerance("f16", "f16", np.array([1.0]), np.array([10.0]))
    assert tol[0] == 2 * 2.0 ** -10 + 2e-3 * 10
    with pytest.raises(AssertionError):
        acceptance.check_close([1.1], [1.0], [1.0], "f16", "f16")
    acceptance.check_exact([0.0, 1.0], [-0.0, 1.0])


# ---------------------------------------------------------------- bias + activations

def _k0_problem(dtype, values, bias_values, beta=1.0):
    """K = 0 makes D = act(beta * C + bias) with no products involved."""
    M, N = len(values), len(values[0])
    p = syn.make_problem(M, N, 0, dtype_ab=dtype, dtype_cd=dtype, dist_c="zeros",
                         beta=beta, seed=20)
    _with_operand(p, "C", np.array(values, dtype=np.float32), dtype)
    p.bias = syn.cast(np.array(bias_values, dtype=np.float32), dtype)
    return p


def test_sigmoid_tanh_closed_forms():
    ln3, ln2 = float(np.float32(np.log(3.0))), float(np.float32(np.log(2.0)))
    p = _k0_problem("f32", [[0.0, ln3, -ln3, ln2]], [0.0, 0.0, 0.0, 0.0])
    s = oracle.gemm(p, act="sigmoid").ref[0]
    assert s[0] == 0.5                                   # sigma(0) = 1/2
    assert abs(s[1] - 0.75) < 1e-8 and abs(s[2] - 0.25) < 1e-8   # sigma(ln 3) = 3/4
    t = oracle.gemm(p, act="tanh").ref[0]
    assert t[0] == 0.0                                   # tanh(0) = 0
    assert abs(t[3] - 0.6) < 1e-8                        # tanh(ln 2) = 3/5
    assert t[2] == -t[1]                                 # odd
    # saturation: sigma(40) rounds to 1 in fp64, tanh(40) too
    q = _k0_problem("f32", [[40.0, -40.0]], [0.0, 0.0])
    assert oracle.gemm(q, act="sigmoid").ref[0][0] == 1.0
    assert oracle.gemm(q, act="tanh").ref[0][0] == 1.0
    assert 0.0 < oracle.gemm(q, act="sigmoid").ref[0][1] < 1e-17


def test_sigmoid_is_half_shifted_tanh():
    """sigma(x) = (1 + tanh(x/2)) / 2 ties the two activations together, so a
    sign or scale slip in either one fails."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((6, 20)) * 4).astype(np.float32)
    p = _k0_problem("f32", x, np.zeros(20, dtype=np.float32))
    s = oracle.gemm(p, act="sigmoid").ref
    p.beta = 0.5                                         # v = x / 2 exactly
    t = oracle.gemm(p, act="tanh").ref
    assert np.allclose(s, (1.0 + t) / 2.0, rtol=0, atol=4e-16)
    assert ((s > 0) & (s < 1)).all()


@pytest.mark.parametrize("dtype_ab,dtype_cd", [("f32", "f32"), ("f16", "f16"),
                                               ("bf16", "bf16"), ("f8e4m3", "bf16")])
@pytest.mark.parametrize("act", ["identity", "relu"])
def test_bias_brute_force_fraction_tiny(dtype_ab, dtype_cd, act):
    rng = np.random.default_rng(22)
    for trial in range(5):
        M, N, K = (int(v) for v in rng.integers(1, 7, 3))
        la, lb, lc = (LAYOUTS[int(v)] for v in rng.integers(0, 2, 3))
        p = syn.integer_problem(M, N, K, dtype_ab=dtype_ab, dtype_cd=dtype_cd,
                                la=la, lb=lb, lc=lc, lo=-5, hi=5,
                                alpha=float(rng.choice([1.0, -0.5])),
                                beta=float(rng.choice([0.0, 1.0])),
                                with_bias=True, seed=200 + trial)
        r = oracle.gemm(p, act=act)
        exact = _fraction_gemm(p, False)
        bias = p.bias.to(torch.float64).numpy()
        for i in range(M):
            for j in range(N):
                v = exact[i][j] + Fraction(float(bias[j]))
                if act == "relu" and v <= 0:
                    v = Fraction(0)
                assert Fraction(float(r.ref[i, j])) == v


def test_bias_is_per_column():
    """A planted mistake (the bias indexed by row) fails: with M != N and a
    bias that differs per column, D - D(no bias) must equal bias[j] in every
    row."""
    p = syn.integer_problem(5, 7, 9, dtype_ab="bf16", dtype_cd="bf16", lo=-2, hi=2,
                            with_bias=True, seed=23)
    with_b = oracle.gemm(p).ref
    bias = p.bias.to(torch.float64).numpy()
    p.bias = None
    without = oracle.gemm(p).ref
    diff = with_b - without
    assert np.array_equal(diff, np.tile(bias, (5, 1)))
    assert not np.array_equal(diff, np.tile(bias[:5, None], (1, 7)))


def test_bias_activation_rows_equal_entries():
    p = syn.make_problem(12, 40, 33, dtype_ab="f16", dtype_cd="f16", lc="col",
                         dist_c="normal", beta=0.5, dist_bias="normal", seed=24)
    for act in ("sigmoid", "tanh"):
        rows = oracle.gemm(p, act=act)
        rng = np.random.default_rng(25)
        ii, jj = rng.integers(0, 12, 60), rng.integers(0, 40, 60)
        ent = oracle.gemm_entries(p, ii, jj, act=act)
        assert np.array_equal(ent.ref, rows.ref[ii, jj])
        assert np.array_equal(ent.d_bits, rows.d_bits[ii, jj])


# ---------------------------------------------------------------- MX block scales
# The pages name MXFP8 among the scaled GEMMs ("Generating State-of-the-Art
# GEMMs with TorchInductor's CuteDSL backend", sections 5.1 and 5.2); the
# format (32-element blocks along K, E8M0 scales) is the OCP MX v1.0 one.

def test_decode_e8m0_definition():
    codes = np.arange(256, dtype=np.uint32)
    got = oracle.decode("e8m0", codes)
    # an unsigned biased exponent: code c is 2^(c-127) computed with
    # torch's ldexp; 0xFF is NaN
    want = torch.ldexp(torch.ones(255, dtype=torch.float64),
                       torch.arange(255, dtype=torch.int64) - 127).numpy()
    assert np.array_equal(got[:255], want)
    assert np.isnan(got[255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def _with_mx(p, fa, fb):
    nb = p.K // 32
    xa = torch.tensor([[fa(i, b) for b in range(nb)] for i in range(p.M)], dtype=torch.uint8)
    xb = torch.tensor([[fb(j, b) for b in range(nb)] for j in range(p.N)], dtype=torch.uint8)
    import dataclasses
    return dataclasses.replace(p, mx_a=xa, mx_b=xb, scale_a=None, scale_b=None)


def test_mx_unit_scales_equal_plain_fp8():
    p = syn.make_problem(24, 40, 96, dtype_ab="f8e4m3", dtype_cd="bf16", la="row", lb="col",
                         dist_c="normal", beta=0.5, seed=80)
    import dataclasses
    plain = dataclasses.replace(p, scale_a=None, scale_b=None)
    mx = _with_mx(p, lambda i, b: 127, lambda j, b: 127)
    r0, r1 = oracle.gemm(plain), oracle.gemm(mx)
    assert np.array_equal(r0.ref, r1.ref) and np.array_equal(r0.d_bits, r1.d_bits)
    assert np.array_equal(r0.S, r1.S)


def test_mx_all_ones_closed_form():
    # A = B = 1, four blocks; A's block b of row i scaled 2^(b - i%3), B's
    # column j scaled 2^(j%2): D = 32 * (1+2+4+8) * 2^(j%2 - i%3)
    M, N, K = 9, 6, 128
    p = syn.integer_problem(M, N, K, dtype_ab="f8e4m3", dtype_cd="bf16", lo=1, hi=1,
                            with_c=False)                       # e4m3 ones
    p = _with_mx(p, lambda i, b: 127 + b - i % 3, lambda j, b: 127 + j % 2)
    r = oracle.gemm(p)
    want = np.array([[480.0 * 2.0 ** (j % 2 - i % 3) for j in range(N)] for i in range(M)])
    assert np.array_equal(r.ref, want)


@pytest.mark.parametrize("la,lb", list(itertools.product(LAYOUTS, LAYOUTS)))
def test_mx_equals_prescaled_plain_gemm(la, lb):
    # Scaling a block by 2^e is multiplying its elements by 2^e: with
    # integer elements in [-2, 2] and |e| <= 2 the premultiplied elements are
    # exact e4m3 values, so the plain (already pinned) GEMM of the
    # premultiplied operands must give the same values bit for bit. Scales
    # differ per row and per block, so a transposed or shifted scale index
    # changes the result.
    q = syn.mx_integer_problem(20, 28, 160, la=la, lb=lb, lc="row", seed=81)
    xa = 2.0 ** (q.mx_a.numpy().astype(np.float64) - 127)       # [M, K/32]
    xb = 2.0 ** (q.mx_b.numpy().astype(np.float64) - 127)       # [N, K/32]
    a = oracle.decode("f8e4m3", syn.raw(q.A)).reshape(q.A.shape)
    b = oracle.decode("f8e4m3", syn.raw(q.B)).reshape(q.B.shape)
    a_log = a if la == "row" else a.T                            # [M, K]
    b_log = b if lb == "row" else b.T                            # [K, N]
    a2 = a_log * np.repeat(xa, 32, axis=1)
    b2 = b_log * np.repeat(xb, 32, axis=1).T
    import dataclasses
    plain = dataclasses.replace(
        q, A=syn.cast(syn.to_storage(a2.astype(np.float32), la), "f8e4m3"),
        B=syn.cast(syn.to_storage(b2.astype(np.float32), lb), "f8e4m3"), mx_a=None, mx_b=None,
        scale_a=1.0, scale_b=1.0)
    assert np.array_equal(oracle.decode("f8e4m3", syn.raw(plain.A)).reshape(q.A.shape),
                          syn.to_storage(a2, la))                # premultiplied exactly
    r_mx, r_plain = oracle.gemm(q), oracle.gemm(plain)
    assert np.array_equal(r_mx.ref, r_plain.ref)
    assert np.array_equal(r_mx.S, r_plain.S)
    assert np.array_equal(r_mx.d_bits, r_plain.d_bits)


def test_mx_nan_scale_poisons_one_row_or_column():
    p = syn.mx_integer_problem(6, 5, 64, seed=82, with_c=False)
    p.mx_a[2, 1] = 255
    p.mx_b[4, 0] = 255
    r = oracle.gemm(p)
    nan = np.isnan(r.ref)
    assert nan[2, :].all() and nan[:, 4].all()
    assert nan.sum() == 5 + 6 - 1


def test_mx_rejects_partial_blocks_and_half_scales():
    p = syn.mx_integer_problem(4, 4, 64, seed=83)
    import dataclasses
    with pytest.raises(ValueError):      # K not a multiple of 32
        oracle.gemm(dataclasses.replace(p, K=48))
    with pytest.raises(ValueError):      # one operand scaled, the other not
        oracle.gemm(dataclasses.replace(p, mx_b=None))
    with pytest.raises(ValueError):      # MX elements must be e4m3
        q = syn.integer_problem(4, 4, 64, dtype_ab="bf16", dtype_cd="bf16")
        oracle.gemm(dataclasses.replace(q, mx_a=p.mx_a, mx_b=p.mx_b))


def test_mx_quantizer_round_trips_within_e4m3_precision():
    # the input generator's MX conversion: every block's largest element
    # lands in e4m3's top binade [256, 448]; dequantized values sit within
    # half an e4m3 ulp (2^-4 relative) of the fp32 draw, except those above
    # 448 * 2^e, which saturate to +-448 * 2^e (the MX conversion clamps)
    rng = np.random.default_rng(84)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    q, codes = syn.mx_quantize(x)
    e = codes.numpy().astype(np.float64) - 127
    qe = syn.cast(q, "f8e4m3").float().numpy().astype(np.float64)
    top = np.abs(qe).reshape(8, 8, 32).max(axis=2)
    assert ((top >= 256) & (top <= 448)).all()
    X = np.repeat(2.0 ** e, 32, axis=1)
    deq = qe * X
    sat = np.abs(x) > 448.0 * X
    assert sat.any() and (np.abs(deq[sat]) == 448.0 * X[sat]).all()
    ok = np.abs(deq - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * X
    assert ok[~sat].all()


# ---------------------------------------------------------------- MXFP4
# "Generating State-of-the-Art GEMMs with TorchInductor's CuteDSL backend",
# section 5.1, lists MXF4 beside MXFP8 in the scaled mm family; the element
# format is OCP FP4 E2M1 (OCP MX v1.0), packed two per byte along K with
# element 2t in the low nibble of byte t, under the same E8M0 block scales.

OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]     # OCP MX v1.0 FP4 magnitudes


def test_decode_e2m1_ocp_table():
    got = oracle.decode("f4e2m1", np.arange(16, dtype=np.uint32))
    assert list(got[:8]) == OCP_E2M1
    assert list(-got[8:]) == OCP_E2M1 and np.signbit(got[8:]).all()
    # every FP4 value is an FP8 E4M3 value: torch's e4m3 cast keeps each one
    # exactly and the (already pinned) e4m3 decoder reads it back unchanged
    e4 = torch.tensor(got, dtype=torch.float32).to(torch.float8_e4m3fn)
    assert np.array_equal(oracle.decode("f8e4m3", syn.raw(e4)), got)


def test_e2m1_storage_cast_is_nearest_even():
    # the generator's RNE cast against exhaustive nearest-value search over
    # the decoded table (ties to the code with a zero fraction bit, beyond 6
    # saturating), on a grid holding every midpoint
    vals = oracle.decode("f4e2m1", np.arange(16, dtype=np.uint32))
    x = np.concatenate([np.arange(-7.0, 7.0001, 0.125), [0.3, -2.9, 5.01, -100.0]])
    codes = syn.e2m1_codes(x)
    for xv, c in zip(x, codes):
        d = np.abs(vals - min(max(xv, -6.0), 6.0))
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:                           # a tie: the even code (or +-0)
            best = [b for b in best if b % 2 == 0]
        assert vals[c] == vals[best[0]], (xv, c, best)


def test_e2m1_pack_round_trip_and_nibble_order():
    rng = np.random.default_rng(85)
    codes = rng.integers(0, 16, size=(3, 64)).astype(np.uint8)
    packed = syn.pack_e2m1(codes).numpy()
    assert packed.shape == (3, 32)
    assert np.array_equal(syn.unpack_e2m1(packed), codes)
    assert packed[1, 5] == codes[1, 10] | (codes[1, 11] << 4)   # element 2t low


def _mx4_logical(q):
    """Logical fp64 [M, K] / [K, N] element values of an MXFP4 problem, read
    with the generator's unpacking and the OCP table (not the oracle's)."""
    grid = np.array(OCP_E2M1)
    def val(codes):
        return np.where(codes & 8, -1.0, 1.0) * grid[codes & 7]
    a = val(syn.unpack_e2m1(syn.raw(q.A)))            # [M, K]
    b = val(syn.unpack_e2m1(syn.raw(q.B))).T          # B stored [N, K]
    return a, b


def test_mxfp4_equals_mxfp8_of_the_same_values():
    # every e2m1 value is an e4m3 value, so an MXFP4 problem and the MXFP8
    # problem holding the same element values and block scales must give the
    # same outputs bit for bit (ties the FP4 path to the pinned FP8 one)
    import dataclasses
    q4 = syn.mx_integer_problem(20, 28, 192, lo=-4, hi=4, seed=86, elem="f4e2m1")
    a, b = _mx4_logical(q4)
    q8 = dataclasses.replace(q4, A=syn.cast(a.astype(np.float32), "f8e4m3"),
                             B=syn.cast(np.ascontiguousarray(b.T).astype(np.float32), "f8e4m3"),
                             dtype_ab="f8e4m3")
    r4, r8 = oracle.gemm(q4), oracle.gemm(q8)
    assert np.array_equal(r4.ref, r8.ref) and np.array_equal(r4.S, r8.S)
    assert np.array_equal(r4.d_bits, r8.d_bits)
    # and the half-precision values in between: 0.5 and 1.5 elements
    q4b = syn.make_mx_problem(12, 16, 128, seed=87, elem="f4e2m1")
    a, b = _mx4_logical(q4b)
    assert (np.abs(a) % 1 == 0.5).any()
    q8b = dataclasses.replace(q4b, A=syn.cast(a.astype(np.float32), "f8e4m3"),
                              B=syn.cast(np.ascontiguousarray(b.T).astype(np.float32), "f8e4m3"),
                              dtype_ab="f8e4m3")
    assert np.array_equal(oracle.gemm(q4b).ref, oracle.gemm(q8b).ref)


@pytest.mark.parametrize("k0", [0, 1, 30, 31, 32, 63])
def test_mxfp4_one_hot_finds_its_element(k0):
    # A holds one nonzero element, 3 at (2, k0); B is the K x K identity
    # (N = K): D is 3 * X_A(2, k0/32) * X_B(k0, k0/32) at (2, k0) and zero
    # elsewhere, so a swapped nibble order or a shifted index moves it
    import dataclasses
    M, K = 4, 64
    a = np.zeros((M, K))
    a[2, k0] = 3.0
    b = np.eye(K)                                       # logical [K, N]
    q = syn.mx_integer_problem(M, K, K, lo=0, hi=0, seed=88, elem="f4e2m1", with_c=False)
    q = dataclasses.replace(q, A=syn.pack_e2m1(syn.e2m1_codes(a)),
                            B=syn.pack_e2m1(syn.e2m1_codes(np.ascontiguousarray(b.T))))
    r = oracle.gemm(q)
    xa = 2.0 ** (q.mx_a.numpy().astype(np.float64) - 127)
    xb = 2.0 ** (q.mx_b.numpy().astype(np.float64) - 127)
    want = np.zeros((M, K))
    want[2, k0] = 3.0 * xa[2, k0 // 32] * xb[k0, k0 // 32]
    assert np.array_equal(r.ref, want)


def test_mxfp4_exact_rational_brute_force():
    for seed, (M, N, K) in enumerate([(3, 5, 32), (6, 4, 64), (2, 3, 96)]):
        q = syn.mx_integer_problem(M, N, K, lo=-4, hi=4, seed=90 + seed, elem="f4e2m1",
                                   with_bias=True)
        a, b = _mx4_logical(q)
        xa = 2.0 ** (q.mx_a.numpy().astype(np.float64) - 127)
        xb = 2.0 ** (q.mx_b.numpy().astype(np.float64) - 127)
        c = q.C.float().numpy().astype(np.float64)
        bias = q.bias.float().numpy().astype(np.float64)
        r = oracle.gemm(q, relu=True)
        for i in range(M):
            for j in range(N):
                acc = sum((Fraction(a[i, k]) * Fraction(xa[i, k // 32])) *
                          (Fraction(b[k, j]) * Fraction(xb[j, k // 32])) for k in range(K))
                v = acc + Fraction(q.beta) * Fraction(c[i, j]) + Fraction(bias[j])
                v = v if v > 0 else Fraction(0)
                assert Fraction(float(r.ref[i, j])) == v, (i, j)


def test_mxfp4_needs_block_scales():
    import dataclasses
    q = syn.mx_integer_problem(4, 4, 64, seed=89, elem="f4e2m1")
    with pytest.raises(ValueError):      # FP4 elements exist only under MX scales
        oracle.gemm(dataclasses.replace(q, mx_a=None, mx_b=None))
    with pytest.raises(ValueError):      # whole 32-element blocks
        oracle.gemm(dataclasses.replace(q, K=48))


def test_mxfp4_quantizer_round_trips_within_e2m1_precision():
    # the generator's MXFP4 conversion: every block's largest magnitude lands
    # in e2m1's top binade [4, 6]; dequantized values sit within half an
    # e2m1 step of the draw (steps of 2^(e-1) in binade [2^e, 2^(e+1)),
    # 1/2 below 1), or saturate at 6 * 2^x
    rng = np.random.default_rng(91)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    q, codes = syn.mx_quantize(x, syn.E2M1_EMAX)
    vals = oracle.decode("f4e2m1", np.arange(16, dtype=np.uint32))
    qe = vals[syn.e2m1_codes(q)]
    top = np.abs(qe).reshape(8, 8, 32).max(axis=2)
    assert ((top >= 4) & (top <= 6)).all()
    X = np.repeat(2.0 ** (codes.numpy().astype(np.float64) - 127), 32, axis=1)
    s = np.abs(q.astype(np.float64))
    step = np.where(s < 2, 0.5, np.where(s < 4, 1.0, 2.0))
    sat = s > 6
    assert (np.abs(qe[sat]) == 6).all()
    assert (np.abs(qe - q)[~sat] <= step[~sat] / 2).all()


# ---------------------------------------------------------------- auxiliary tensor
# The epilogue-fusion kernels load and store auxiliary tensors and combine
# them by elementwise add, subtract, multiply or divide ("Generating
# State-of-the-Art GEMMs with TorchInductor's CuteDSL backend", section 7).

AUX_OPS = ("add", "sub", "mul", "div")


def _fraction_aux(p, act):
    """Exact D and Z of an aux problem: the rational GEMM + bias, the op on
    its side of the activation (relu or identity)."""
    exact = _fraction_gemm(p, False)
    bias = p.bias.to(torch.float64).numpy() if p.bias is not None else None
    X = _logical(p, "aux")
    ops = {"add": lambda y, x: y + x, "sub": lambda y, x: y - x,
           "mul": lambda y, x: y * x, "div": lambda y, x: y / x}
    op = ops[p.aux_op]
    relu = (lambda v: v if v > 0 else Fraction(0)) if act == "relu" else (lambda v: v)
    D, Z = [], []
    for i in range(p.M):
        drow, zrow = [], []
        for j in range(p.N):
            v = exact[i][j] + (Fraction(float(bias[j])) if bias is not None else 0)
            x = Fraction(float(X[i, j]))
            if p.aux_pos == "before":
                z = op(v, x)
                d = relu(z)
            else:
                z = v
                d = op(relu(v), x)
            drow.append(d)
            zrow.append(z)
        D.append(drow)
        Z.append(zrow)
    return D, Z


@pytest.mark.parametrize("dtype_ab,dtype_cd", [("f32", "f32"), ("f16", "f16"),
                                               ("bf16", "bf16"), ("f8e4m3", "bf16")])
@pytest.mark.parametrize("op", AUX_OPS)
@pytest.mark.parametrize("pos", ["before", "after"])
def test_aux_brute_force_fraction_tiny(dtype_ab, dtype_cd, op, pos):
    """Exact rational brute force: every op on both sides of ReLU / identity,
    random layouts, with and without bias and beta*C, one K = 0 case. A
    division is one correctly rounded fp64 quotient of exact values, which is
    what float(Fraction) gives."""
    rng = np.random.default_rng(31)
    for trial in range(5):
        M, N = (int(v) for v in rng.integers(1, 7, 2))
        K = 0 if trial == 4 else int(rng.integers(1, 7))
        la, lb, lc = (LAYOUTS[int(v)] for v in rng.integers(0, 2, 3))
        p = syn.integer_problem(M, N, K, dtype_ab=dtype_ab, dtype_cd=dtype_cd,
                                la=la, lb=lb, lc=lc, lo=-5, hi=5,
                                alpha=float(rng.choice([1.0, -0.5])),
                                beta=float(rng.choice([0.0, 1.0])),
                                with_bias=bool(trial % 2), seed=300 + trial)
        syn.add_aux(p, op, pos, dist="int_nz" if op == "div" else "int", seed=400 + trial)
        for act in ("identity", "relu"):
            r = oracle.gemm(p, act=act)
            D, Z = _fraction_aux(p, act)
            for i in range(M):
                for j in range(N):
                    assert float(r.ref[i, j]) == float(D[i][j]), (trial, act, i, j)
                    assert float(r.z_ref[i, j]) == float(Z[i][j]), (trial, act, i, j)
            # by value: a product or quotient of 0 keeps the sign IEEE gives it,
            # and +0 and -0 are the same result
            for got, want in ((r.d_bits, D), (r.z_bits, Z)):
                want_bits = oracle.encode(dtype_cd, [[float(v) for v in row] for row in want])
                assert np.array_equal(oracle.decode(dtype_cd, got),
                                      oracle.decode(dtype_cd, want_bits))


@pytest.mark.parametrize("lc", LAYOUTS)
def test_aux_add_and_sub_equal_beta_c(lc):
    """X + v with beta = 0 is beta = 1 with C = X; v - X is beta = -1."""
    p = syn.make_problem(9, 13, 20, dtype_ab="f16", dtype_cd="f32", lc=lc,
                         dist_c="normal", beta=1.0, seed=32)
    with_c = oracle.gemm(p).ref
    p.beta = -1.0
    minus_c = oracle.gemm(p).ref
    p.aux, p.beta = p.C, 0.0
    p.aux_op, p.aux_pos = "add", "before"
    assert np.array_equal(oracle.gemm(p).ref, with_c)
    p.aux_op = "sub"
    assert np.array_equal(oracle.gemm(p).ref, minus_c)


def test_aux_mul_by_two_and_div_by_half_double_exactly():
    p = syn.make_problem(7, 11, 40, dtype_ab="bf16", dtype_cd="bf16", dist_c="normal",
                         beta=0.5, dist_bias="normal", seed=33)
    base = oracle.gemm(p, act="tanh")
    for op, val in (("mul", 2.0), ("div", 0.5)):
        for pos in ("before", "after"):
            syn.add_aux(p, op, pos, dist="ones")
            p.aux = p.aux * val
            r = oracle.gemm(p, act="identity" if pos == "before" else "tanh")
            want = oracle.gemm(p.__class__(**{**p.__dict__, "aux": None}),
                               act="identity" if pos == "before" else "tanh").ref * 2.0
            assert np.array_equal(r.ref, want)
    p.aux = None
    assert np.array_equal(oracle.gemm(p, act="tanh").ref, base.ref)


def test_aux_store_is_the_activation_input():
    """Before the activation Z = v op X and D = act(Z); after it, Z is the
    plain linear result and D = act(Z) op X."""
    p = syn.make_problem(6, 10, 24, dtype_ab="f16", dtype_cd="f16", dist_c="normal",
                         beta=1.0, seed=34)
    plain = oracle.gemm(p).ref
    syn.add_aux(p, "mul", "before", dist="away", seed=35)
    r = oracle.gemm(p, act="sigmoid")
    assert np.allclose(r.ref, 1.0 / (1.0 + np.exp(-r.z_ref)), rtol=1e-15, atol=0)
    assert np.array_equal(r.z_ref, oracle.gemm(p, act="identity").ref)
    p.aux_pos = "after"
    r = oracle.gemm(p, act="relu")
    assert np.array_equal(r.z_ref, plain)
    X = _logical(p, "aux")
    assert np.array_equal(r.ref, np.maximum(plain, 0.0) * X)


def test_aux_position_decides_with_negative_factors():
    """relu(v * X) and relu(v) * X differ where X < 0: the two readings are
    told apart (a planted swap of the side fails)."""
    p = syn.integer_problem(6, 6, 5, dtype_ab="f16", dtype_cd="f16", lo=-3, hi=3, seed=36)
    syn.add_aux(p, "mul", "before", dist="int_nz", seed=37)
    before = oracle.gemm(p, act="relu").ref
    p.aux_pos = "after"
    after = oracle.gemm(p, act="relu").ref
    assert (before >= 0).all() and (after < 0).any()
    assert not np.array_equal(before, after)


def test_aux_pin_catches_transposed_aux():
    """A planted mistake (X read with the other layout) fails the rational pin."""
    p = syn.integer_problem(5, 5, 4, dtype_ab="f32", dtype_cd="f32", lo=-3, hi=3, seed=38)
    syn.add_aux(p, "sub", "before", dist="int", seed=39)
    D, _ = _fraction_aux(p, "identity")
    want = np.array([[float(v) for v in row] for row in D])
    assert np.array_equal(oracle.gemm(p).ref, want)
    p.aux = p.aux.T.contiguous()                # the planted transposition
    assert not np.array_equal(oracle.gemm(p).ref, want)


def test_aux_rows_equal_entries():
    p = syn.make_problem(12, 40, 33, dtype_ab="f16", dtype_cd="f16", lc="col",
                         dist_c="normal", beta=0.5, dist_bias="normal", seed=40)
    syn.add_aux(p, "div", "after", dist="away", seed=41)
    rows = oracle.gemm(p, act="tanh")
    rng = np.random.default_rng(42)
    ii, jj = rng.integers(0, 12, 60), rng.integers(0, 40, 60)
    ent = oracle.gemm_entries(p, ii, jj, act="tanh")
    for name in ("ref", "S", "d_bits", "z_ref", "z_S", "z_bits"):
        assert np.array_equal(getattr(ent, name), getattr(rows, name)[ii, jj]), name


def test_aux_tolerance_scale_follows_the_op():
    """The error of v (scale S) is multiplied by |X| through a mul and divided
    by it through a div; add and sub leave it; Z keeps the plain S when the op
    comes after the activation."""
    p = syn.make_problem(5, 8, 16, dtype_ab="f16", dtype_cd="f16", seed=43)
    S0 = oracle.gemm(p).S
    for op in AUX_OPS:
        for pos in ("before", "after"):
            syn.add_aux(p, op, pos, dist="away", seed=44)
            X = np.abs(_logical(p, "aux"))
            r = oracle.gemm(p, act="relu")
            f = {"add": 1.0, "sub": 1.0, "mul": X, "div": 1.0 / X}[op]
            assert np.allclose(r.S, S0 * f, rtol=1e-15)
            assert np.allclose(r.z_S, S0 * (f if pos == "before" else 1.0), rtol=1e-15)
