"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test pins one part of the oracle to something it does not compute
itself: values the paper prints for a worked example, closed forms,
library routines (torch / numpy in float64 or exact integers), exact
rational arithmetic on tiny inputs, and invariants of the method.

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from memory_bounded_weight_amd import synth
from tests import golden

f = oracle.bf16_to_float
EQ5 = golden.values("eq5_write_boundary.txt")  # [PSI] sec. II-C eq. (5)


def torch_bf16_bits(a64) -> np.ndarray:
    """Library rounding: float64 -> float32 (exact here) -> bfloat16 via torch."""
    t = torch.as_tensor(np.asarray(a64, dtype=np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def exact_bf16_round(q: Fraction) -> Fraction:
    """Round an exact rational to the nearest bfloat16 value, ties to even
    (normal range only).  Brute-force definition for tiny cases."""
    if q == 0:
        return Fraction(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128  # 8 significant bits: 128 <= scaled < 256
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * Fraction(fl) * Fraction(2) ** (e - 7)


def frac_of_bits(u) -> Fraction:
    return Fraction(float(f(np.uint16(u))))


# ----------------------------------------------------------------- rounding

def test_eq5_write_boundary_scalars():
    """[PSI] sec. II-C eq. (5), the worked example in tests/golden: B(B(z) + b)
    and B(z + b) for z = 257/256, b = 1/256."""
    z, b = float(EQ5["z"]), float(EQ5["b"])
    once = oracle.bf16_from_float_scalar(z + b)
    twice = oracle.bf16_from_float_scalar(float(f(oracle.bf16_from_float_scalar(z))) + b)
    assert Fraction(float(f(np.uint16(once)))) == EQ5["B(z + b)"]
    assert Fraction(float(f(np.uint16(twice)))) == EQ5["B(B(z) + b)"]


def test_eq5_linear_bias_variants():
    """Pin P1: x = [1, 2^-8], W = [[1, 1]], b = [2^-8].  The accumulator is
    257/256 exactly; modified (fp32 bias) gives 129/128, baseline (product
    rounded to BF16 first) gives 1 -- the sec. III-A distinction."""
    x = synth.f32_to_bf16_bits(np.array([[1.0, 2.0 ** -8]], np.float32))
    W = synth.f32_to_bf16_bits(np.array([[1.0, 1.0]], np.float32))
    b = synth.f32_to_bf16_bits(np.array([2.0 ** -8], np.float32))
    y_mod, acc = oracle.linear(x, W, b, variant=0, want_acc=True)
    y_base = oracle.linear(x, W, b, variant=1)
    assert Fraction(float(acc[0, 0])) == EQ5["z"]
    assert Fraction(float(f(y_mod)[0, 0])) == EQ5["B(z + b)"]
    assert Fraction(float(f(y_base)[0, 0])) == EQ5["B(B(z) + b)"]


def test_bf16_from_float_matches_torch_rounding():
    """B() on binary32 equals torch's float32 -> bfloat16 conversion (a
    library routine) on random bit patterns, every tie pattern and
    boundary values."""
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, size=20_000).astype(np.uint32) << 16) | 0x8000
    edge = np.array([0, 0x80000000, 0x7F7FFFFF, 0x7F7F8000, 0x00000001, 0x00008000,
                     0x3F808000, 0x3F818000, 0x7F800000, 0xFF800000], dtype=np.uint32)
    allb = np.concatenate([bits, ties.astype(np.uint32), edge])
    vals = allb.view(np.float32)
    finite = np.isfinite(vals) | np.isinf(vals)
    vals = vals[finite & ~np.isnan(vals)]
    ours = np.array([oracle.bf16_from_float_scalar(float(v)) for v in vals[:30000]], dtype=np.uint16)
    ref = torch.from_numpy(vals[:30000].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # vectorised path through linear's epilogue is covered by the other pins;
    # here also the NaN convention:
    assert oracle.bf16_from_float_scalar(float("nan")) == 0x7FC0


def test_bf16_from_double_rounds_once():
    """B() of a double rounds ONCE: compare with exact rational rounding on
    values chosen next to bf16 midpoints, where rounding through binary32
    first would give a different answer."""
    rng = np.random.default_rng(7)
    for _ in range(3000):
        m = int(rng.integers(128, 256))
        e = int(rng.integers(-100, 100))
        # midpoint between m and m+1 (in units of 2^(e-7)), nudged by a tiny
        # amount that binary32 cannot hold
        nudge = Fraction(int(rng.integers(-3, 4)), 2 ** 40)
        q = (Fraction(m) + Fraction(1, 2) + nudge) * Fraction(2) ** (e - 7)
        if rng.random() < 0.5:
            q = -q
        got = oracle.bf16_from_double_scalar(float(q))
        assert Fraction(float(q)) == q  # the test value is exactly a double
        assert frac_of_bits(got) == exact_bf16_round(q)


def test_eq6_round_once_sign_and_value():
    """[PSI] sec. IV-B eq. (6): the exact value -46489387/2^39 rounds to the
    nearest BF16 value -177/2^21 (the paper's native result), not -175/2^21.
    Pin P2: a Linear whose operands sum exactly to that value (the paper's
    own operands are not published) returns -177/2^21."""
    q = Fraction(-46489387, 2 ** 39)
    assert exact_bf16_round(q) == Fraction(-177, 2 ** 21)
    assert frac_of_bits(oracle.bf16_from_double_scalar(float(q))) == Fraction(-177, 2 ** 21)
    pieces = [46399488, 89600, 298]  # each has <= 8 significant bits
    x = synth.f32_to_bf16_bits(np.array([[-p * 2.0 ** -39 for p in pieces]], np.float32))
    assert [Fraction(float(v)) for v in f(x)[0]] == [Fraction(-p, 2 ** 39) for p in pieces]
    W = synth.f32_to_bf16_bits(np.ones((1, 3), np.float32))
    b = synth.f32_to_bf16_bits(np.array([-1 * 2.0 ** -39], np.float32))
    y = oracle.linear(x, W, b)
    assert Fraction(float(f(y)[0, 0])) == Fraction(-177, 2 ** 21)
    assert Fraction(float(f(y)[0, 0])) != Fraction(-175, 2 ** 21)


# ------------------------------------------------------------------ linear

@pytest.mark.parametrize("seed,M,K,N", [(0, 3, 5, 4), (1, 7, 16, 9), (2, 4, 64, 6), (3, 1, 33, 1)])
def test_linear_brute_force_exact(seed, M, K, N):
    """Pin P5: exact rational sum of the BF16 products plus bias, rounded
    once, equals the oracle except where the fp32 accumulation error bound
    straddles a rounding boundary (every mismatch must lie inside it)."""
    rng = np.random.default_rng(seed)
    x = synth.normal_bf16(rng, (M, K), 1.0)
    W = synth.normal_bf16(rng, (N, K), 1.0 / K)
    b = synth.normal_bf16(rng, (N,), 0.02)
    y = oracle.linear(x, W, b)
    xf, Wf, bf = f(x), f(W), f(b)
    mism = 0
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(xf[m, k])) * Fraction(float(Wf[n, k])) for k in range(K)]
            exact = sum(terms, Fraction(0)) + Fraction(float(bf[n]))
            r = exact_bf16_round(exact)
            got = Fraction(float(f(y)[m, n]))
            if got != r:
                mism += 1
                bound = (K + 1) * 2.0 ** -24 * (sum(abs(float(t)) for t in terms) + abs(float(bf[n])))
                ulp = float(abs(r)) * 2.0 ** -7
                # the oracle's value must be one of the two bf16 neighbours of
                # a value within the fp32 error bound of the exact sum
                assert abs(float(got) - float(exact)) <= ulp + bound
    assert mism <= max(1, (M * N) // 20)


def test_linear_integer_lattice_bitwise():
    """Pin P7: with operands in {-2..2} and small integer biases every fp32
    partial sum is exact, so the oracle must equal the exact integer result
    (numpy int64 matmul) rounded once by torch's conversion, bitwise."""
    rng = np.random.default_rng(11)
    M, K, N = 37, 4096, 29
    xi = rng.integers(-2, 3, size=(M, K))
    Wi = rng.integers(-2, 3, size=(N, K))
    bi = rng.integers(-8, 9, size=(N,))
    x = synth.f32_to_bf16_bits(xi.astype(np.float32))
    W = synth.f32_to_bf16_bits(Wi.astype(np.float32))
    b = synth.f32_to_bf16_bits(bi.astype(np.float32))
    y, acc = oracle.linear(x, W, b, want_acc=True)
    exact = xi @ Wi.T
    assert np.array_equal(acc.astype(np.int64), exact)
    assert np.array_equal(y, torch_bf16_bits(exact + bi[None, :]))


def test_linear_vs_float64_library_matmul():
    """Pin P9: the fp32 accumulator agrees with numpy's float64 matmul of the
    widened operands to within the fp32 accumulation bound, on a
    non-square case (a transposed operand or dropped term would fail)."""
    c = synth.linear_case(seed=5, M=48, K=320, N=72)
    y, acc = oracle.linear(c["x"], c["W"], c["b"], want_acc=True)
    ref = f(c["x"]).astype(np.float64) @ f(c["W"]).astype(np.float64).T
    absref = np.abs(f(c["x"]).astype(np.float64)) @ np.abs(f(c["W"]).astype(np.float64)).T
    assert np.all(np.abs(acc - ref) <= 320 * 2.0 ** -24 * absref + 1e-30)
    yref = ref + f(c["b"]).astype(np.float64)[None, :]
    assert np.all(np.abs(f(y) - yref) <= 2.0 ** -8 * np.abs(yref) + 320 * 2.0 ** -23 * absref + 1e-30)


def test_linear_partitions_bitwise():
    """Pin P3 on the oracle ([PSI] sec. II-B, sec. IV-B): an output-column
    partition concatenates to the dense result bitwise, and a K-split with
    the fp32 accumulator carried in page order reproduces the dense chain
    bitwise (bias added once, after the last page)."""
    c = synth.linear_case(seed=9, M=40, K=384, N=96)
    dense, dacc = oracle.linear(c["x"], c["W"], c["b"], want_acc=True)
    parts = [oracle.linear(c["x"], np.ascontiguousarray(c["W"][i:i + 32]), c["b"][i:i + 32].copy())
             for i in range(0, 96, 32)]
    assert np.array_equal(np.concatenate(parts, axis=1), dense)
    acc = None
    for k0 in range(0, 384, 128):
        xs = np.ascontiguousarray(c["x"][:, k0:k0 + 128])
        Ws = np.ascontiguousarray(c["W"][:, k0:k0 + 128])
        last = k0 + 128 == 384
        y, acc = oracle.linear(xs, Ws, c["b"] if last else None, acc_in=acc, want_acc=True)
    assert np.array_equal(acc, dacc)
    assert np.array_equal(y, dense)


# -------------------------------------------------------------------- GELU

def gelu_decimal(v: float, digits: int = 50) -> Fraction:
    """phi(v) = v/2 (1 + tanh z), z = sqrt(2/pi)(v + 0.044715 v^3), with
    1 + tanh z = 2 e^(2z) / (1 + e^(2z)), evaluated in 50-digit decimal
    arithmetic (an independent high-precision evaluation of the closed
    form)."""
    import decimal
    ctx = decimal.Context(prec=digits, Emin=-999999, Emax=999999)
    D = lambda t: ctx.create_decimal(t)
    pi = D("3.14159265358979323846264338327950288419716939937510582097494459")
    vv = D(repr(v))
    c = ctx.sqrt(ctx.divide(D(2), pi))
    z = ctx.multiply(c, ctx.add(vv, ctx.multiply(D("0.044715"), ctx.power(vv, 3))))
    e = ctx.exp(ctx.multiply(D(2), z)) if z < 0 else None
    if e is None:
        onep = ctx.divide(D(2), ctx.add(D(1), ctx.exp(ctx.multiply(D(-2), z))))
    else:
        onep = ctx.divide(ctx.multiply(D(2), e), ctx.add(D(1), e))
    return Fraction(ctx.multiply(ctx.multiply(D("0.5"), vv), onep))


def test_gelu_exhaustive_vs_high_precision():
    """Pin P6: phi on every finite bf16 input against a 50-digit decimal
    evaluation of the tanh-GELU closed form, rounded once to bf16 by exact
    rational rounding: bitwise except where the double result lies within
    1e-13 (relative) of a rounding midpoint."""
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v32 = f(u)
    fin = np.isfinite(v32)
    u, v = u[fin], v32[fin].astype(np.float64)
    h = oracle.gelu_bf16(u)
    bad = []
    for i in range(u.size):
        ref = gelu_decimal(float(v[i]))
        if ref == 0:
            ok = f(h[i:i + 1])[0] == 0
        else:
            r = exact_bf16_round(ref) if abs(ref) >= Fraction(2) ** -126 else None
            got = Fraction(float(f(h[i:i + 1])[0]))
            if r is None:  # bf16 subnormal range: spacing 2^-133
                q = ref / Fraction(2) ** -133
                fl = q.numerator // q.denominator
                rem = q - fl
                fl = fl + 1 if (rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2)) else fl
                r = Fraction(fl) * Fraction(2) ** -133
            ok = got == r
            if not ok:
                # allowed only next to a midpoint, within the double evaluation error
                ulp = Fraction(2) ** -133  # bf16 spacing at |ref|
                while ulp * 256 <= abs(ref):
                    ulp *= 2
                mid_dist = abs(abs(ref - got) - ulp / 2)
                ok = mid_dist <= abs(ref) * Fraction(1, 10 ** 13)
        if not ok:
            bad.append(int(u[i]))
    assert not bad, [hex(b) for b in bad[:10]]
    assert oracle.gelu_bf16(np.array([0x0000], np.uint16))[0] == 0
    big = synth.f32_to_bf16_bits(np.array([30.0, -30.0], np.float32))
    hb = f(oracle.gelu_bf16(big))
    assert hb[0] == np.float32(30.0) and hb[1] == 0.0


def test_gelu_double_vs_torch_where_torch_is_accurate():
    """Cross-check with torch's float64 tanh-GELU (a library routine) where
    its literal 1 + tanh(z) does not cancel (z >= -2)."""
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v32 = f(u)
    v = v32[np.isfinite(v32)].astype(np.float64)
    z = np.sqrt(2 / np.pi) * (v + 0.044715 * v ** 3)
    v = v[z >= -2]
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    ours = np.array([oracle.gelu_tanh_double(float(t)) for t in v])
    assert np.allclose(ours, ref, rtol=1e-12, atol=0)


# --------------------------------------------------------------------- FFN

def _torch_ffn(x, U, a, V, b, residual=False):
    """Library composition in float64 with the declared bf16 writes done by
    torch conversions (tolerance check, not bitwise)."""
    xd = torch.from_numpy(f(x).astype(np.float64))
    pre = xd @ torch.from_numpy(f(U).astype(np.float64)).T + torch.from_numpy(f(a).astype(np.float64))
    pre = pre.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    H = torch.nn.functional.gelu(pre, approximate="tanh").to(torch.float32).to(torch.bfloat16).to(torch.float64)
    y = H @ torch.from_numpy(f(V).astype(np.float64)).T + torch.from_numpy(f(b).astype(np.float64))
    if residual:
        y = y.to(torch.float32).to(torch.bfloat16).to(torch.float64) + xd
    return y.numpy()


@pytest.mark.parametrize("residual", [False, True])
def test_ffn_vs_library_composition(residual):
    c = synth.ffn_case(seed=3, M=24, d=96, hidden=160)
    y = oracle.ffn(c["x"], c["U"], c["a"], c["V"], c["b"], residual=residual)
    ref = _torch_ffn(c["x"], c["U"], c["a"], c["V"], c["b"], residual)
    rel = np.abs(f(y) - ref) / np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
    assert rel.max() < 2e-2
    assert np.mean(rel) < 2e-3


def test_ffn_hidden_partition_bitwise():
    """[PSI] sec. II-B eq. (2) on the oracle: hidden tiles H_J computed
    separately concatenate to the dense H, and the down-projection summed
    tile by tile with a carried fp32 accumulator equals the dense FFN
    bitwise (output bias once)."""
    c = synth.ffn_case(seed=4, M=16, d=64, hidden=192)
    y, H, acc = oracle.ffn(c["x"], c["U"], c["a"], c["V"], c["b"], want_hidden=True, want_acc=True)
    carry = None
    for j in range(0, 192, 64):
        pre = oracle.linear(c["x"], np.ascontiguousarray(c["U"][j:j + 64]), c["a"][j:j + 64].copy())
        HJ = oracle.gelu_bf16(pre)
        assert np.array_equal(HJ, H[:, j:j + 64])
        last = j + 64 == 192
        yJ, carry = oracle.linear(HJ, np.ascontiguousarray(c["V"][:, j:j + 64]),
                                  c["b"] if last else None, acc_in=carry, want_acc=True)
    assert np.array_equal(carry, acc)
    assert np.array_equal(yJ, y)


def test_ffn_integer_lattice_bitwise():
    """Pin P7 extended to the FFN: the up-projection pre-activations are
    integers in a small range, GELU is then a per-value table (checked
    against torch), and the down-projection uses V in {-1,0,1} with values
    whose sums stay exact in fp32, so the oracle equals exact arithmetic."""
    rng = np.random.default_rng(21)
    M, d, h = 9, 64, 48
    # two ones per row of x, U in {-1,0,1}, a in {0,1,2}: pre-activations lie
    # in [-2, 4], where every bf16 GELU output is a multiple of 2^-12, so the
    # down-projection sums (<= 48 terms, |.| <= 192) stay exact in fp32
    xi = np.zeros((M, d), dtype=np.int64)
    for m in range(M):
        xi[m, rng.choice(d, size=2, replace=False)] = 1
    Ui = rng.integers(-1, 2, size=(h, d))
    ai = rng.integers(0, 3, size=(h,))
    Vi = rng.integers(-1, 2, size=(d, h))
    bi = rng.integers(-4, 5, size=(d,))
    bits = lambda a: synth.f32_to_bf16_bits(a.astype(np.float32))
    y, H, acc = oracle.ffn(bits(xi), bits(Ui), bits(ai), bits(Vi), bits(bi), want_hidden=True, want_acc=True)
    pre = xi @ Ui.T + ai[None, :]
    assert pre.min() >= -2 and pre.max() <= 4
    Hd = torch.nn.functional.gelu(torch.from_numpy(pre.astype(np.float64)), approximate="tanh").numpy()
    Hbits = np.array([oracle.bf16_from_double_scalar(float(t)) for t in Hd.ravel()], np.uint16).reshape(Hd.shape)
    assert np.array_equal(H, Hbits)
    # exact down-projection in rationals (all bf16 values are dyadic)
    Hq = f(Hbits).astype(np.float64)
    assert np.all(Hq * 2 ** 12 == np.round(Hq * 2 ** 12))
    exact = Hq @ Vi.T.astype(np.float64)  # exact in float64 (and in fp32)
    assert np.array_equal(acc.astype(np.float64), exact)
    assert np.array_equal(y, torch_bf16_bits(exact + bi[None, :]))


# --------------------------------------------------------------- attention

def test_attention_single_key_is_v():
    """Pin P8, eq. (3) with one key: p = 1, l = 1, z = v, so o = v bitwise."""
    rng = np.random.default_rng(0)
    q = synth.normal_bf16(rng, (5, 256), 1.0)
    k = synth.normal_bf16(rng, (1, 256), 1.0)
    v = synth.normal_bf16(rng, (1, 256), 1.0)
    o = oracle.attention(q, k, v, heads=2, dh=128)
    assert np.array_equal(o, np.repeat(v, 5, axis=0))


def test_attention_dominant_key():
    """Pin P8: a score gap larger than the float exponent range makes every
    other weight underflow to zero, so o equals the dominant key's value."""
    rng = np.random.default_rng(1)
    dh = 64
    q = synth.f32_to_bf16_bits(np.full((3, dh), 1.0, np.float32))
    kf = np.zeros((7, dh), np.float32)
    kf[4] = 16.0  # score 16*64/8 = 128 above the others (exp(-128) != 0 in fp32...)
    kf[4] = 64.0  # score 512: exp(-512) underflows to 0 in binary32
    k = synth.f32_to_bf16_bits(kf)
    v = synth.normal_bf16(rng, (7, dh), 1.0)
    o = oracle.attention(q, k, v, heads=1, dh=dh)
    assert np.array_equal(o, np.repeat(v[4:5], 3, axis=0))


def test_attention_constant_power_of_two_values():
    """Pin P8: when every key carries the same power-of-two value per
    column, z is that value times l exactly, so o = v bitwise."""
    rng = np.random.default_rng(2)
    q = synth.normal_bf16(rng, (11, 128), 1.0)
    k = synth.normal_bf16(rng, (37, 128), 1.0)
    col = 2.0 ** rng.integers(-4, 5, size=128) * rng.choice([-1.0, 1.0], size=128)
    v = synth.f32_to_bf16_bits(np.repeat(col[None, :].astype(np.float32), 37, axis=0))
    o = oracle.attention(q, k, v, heads=1, dh=128)
    assert np.array_equal(o, np.repeat(v[:1], 11, axis=0))


def test_attention_vs_torch_sdpa_float64():
    """Pin P8: dense oracle against torch's math scaled-dot-product attention
    in float64 on the same bf16 operands (scale 1/sqrt(dh), several heads,
    ragged sizes)."""
    rng = np.random.default_rng(3)
    heads, dh, Mq, Mk = 3, 64, 29, 45
    q = synth.normal_bf16(rng, (Mq, heads * dh), 1.0)
    k = synth.normal_bf16(rng, (Mk, heads * dh), 1.0)
    v = synth.normal_bf16(rng, (Mk, heads * dh), 1.0)
    o = oracle.attention(q, k, v, heads, dh)
    t = lambda a, M: torch.from_numpy(f(a).astype(np.float64)).view(M, heads, dh).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q, Mq), t(k, Mk), t(v, Mk))
    ref = ref.transpose(0, 1).reshape(Mq, heads * dh).numpy()
    rel = np.abs(f(o) - ref) / np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
    assert rel.max() < 1e-2
    assert np.mean(o != torch_bf16_bits(ref)) < 0.05


def test_attention_online_partition_equals_dense_in_float64():
    """[PSI] eqs. (3)-(4): the online update over a random disjoint key
    partition equals dense softmax in float64 (to 1e-12), checking the
    identity the paged kernel relies on against the oracle's dense form."""
    rng = np.random.default_rng(4)
    dh, Mk = 32, 50
    q = rng.standard_normal(dh)
    K = rng.standard_normal((Mk, dh))
    V = rng.standard_normal((Mk, dh))
    s = K @ q / np.sqrt(dh)
    dense = np.exp(s - s.max()) @ V / np.exp(s - s.max()).sum()
    cuts = np.sort(rng.choice(np.arange(1, Mk), size=6, replace=False))
    m, l, z = -np.inf, 0.0, np.zeros(dh)
    for T in np.split(np.arange(Mk), cuts):
        m2 = max(m, s[T].max())
        eta = np.exp(m - m2)
        l = eta * l + np.exp(s[T] - m2).sum()
        z = eta * z + np.exp(s[T] - m2) @ V[T]
        m = m2
    assert np.allclose(z / l, dense, rtol=1e-12, atol=1e-12)
    # and the oracle on bf16 versions of the same operands agrees in tolerance
    qb = synth.f32_to_bf16_bits(q[None, :].astype(np.float32))
    Kb = synth.f32_to_bf16_bits(K.astype(np.float32))
    Vb = synth.f32_to_bf16_bits(V.astype(np.float32))
    o = f(oracle.attention(qb, Kb, Vb, 1, dh))[0]
    sb = f(Kb).astype(np.float64) @ f(qb)[0].astype(np.float64) / np.sqrt(dh)
    ref = np.exp(sb - sb.max()) @ f(Vb).astype(np.float64) / np.exp(sb - sb.max()).sum()
    assert np.allclose(o, ref, rtol=1e-2, atol=1e-2 * np.abs(ref).max())


def test_attn_sublayer_vs_library_composition():
    """Attention sub-block (projections, attention, output projection,
    residual) against a torch float64 composition with the same bf16
    writes; self- and cross-attention."""
    rng = np.random.default_rng(5)
    d, heads, dh, M, Mc = 128, 2, 64, 20, 13
    x = synth.normal_bf16(rng, (M, d), 1.0)
    ctx = synth.normal_bf16(rng, (Mc, d), 1.0)
    w = synth.attn_weights(rng, d)
    D = lambda a: torch.from_numpy(f(a).astype(np.float64))
    R = lambda t: t.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    for use_ctx in (None, ctx):
        y = oracle.attn_sublayer(x, w["Wq"], w["bq"], w["Wk"], w["bk"], w["Wv"], w["bv"],
                                 w["Wo"], w["bo"], heads, dh, ctx=use_ctx)
        src = D(x if use_ctx is None else use_ctx)
        Q = R(D(x) @ D(w["Wq"]).T + D(w["bq"]))
        K = R(src @ D(w["Wk"]).T + D(w["bk"]))
        V = R(src @ D(w["Wv"]).T + D(w["bv"]))
        sp = lambda t: t.view(t.shape[0], heads, dh).transpose(0, 1)
        O = torch.nn.functional.scaled_dot_product_attention(sp(Q), sp(K), sp(V))
        O = R(O.transpose(0, 1).reshape(M, d))
        Y = R(O @ D(w["Wo"]).T + D(w["bo"]))
        ref = (Y + D(x)).numpy()
        rel = np.abs(f(y) - ref) / np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
        assert rel.max() < 2e-2


def test_block_is_composition_of_sublayers():
    """The block is the self-attention sub-block followed by the FFN
    sub-block, each with its residual write (oracle-internal consistency)."""
    rng = np.random.default_rng(6)
    d, heads, dh, M, hid = 128, 2, 64, 12, 256
    x = synth.normal_bf16(rng, (M, d), 1.0)
    w = synth.attn_weights(rng, d)
    w["U"], w["a"] = synth.linear_weights(rng, hid, d)
    w["V"], w["b"] = synth.linear_weights(rng, d, hid)
    y = oracle.block(x, w, heads, dh)
    t = oracle.attn_sublayer(x, w["Wq"], w["bq"], w["Wk"], w["bk"], w["Wv"], w["bv"],
                             w["Wo"], w["bo"], heads, dh)
    y2 = oracle.ffn(t, w["U"], w["a"], w["V"], w["b"], residual=True)
    assert np.array_equal(y, y2)


# ------------------------------------------------------------- residual

def test_residual_is_sum_rounded_once():
    """The residual write y = B(f(x) + f(Y)) (reading R7: the sub-block
    output is a declared BF16 value, then the sum is rounded once, [PSI]
    sec. III-A).  Every output equals the exact rational sum of its two
    BF16 operands rounded to the nearest BF16 value, ties to even, on random
    pairs, pairs with a large exponent gap, cancellations and hand-built
    ties; and the special cases: x + 0 = x, x + (-x) = +0, commutativity."""
    rng = np.random.default_rng(31)
    n = 4000
    x = synth.normal_bf16(rng, (n,), 1.0)
    y = synth.normal_bf16(rng, (n,), 1.0)
    # exponent gaps up to 2^30: the smaller operand falls below every BF16
    # half-ulp of the larger one, or just touches it
    scale = synth.f32_to_bf16_bits(np.float32(2.0) ** rng.integers(-30, 31, size=n).astype(np.float32))
    y = synth.f32_to_bf16_bits(f(y) * f(scale))
    # cancellations: y = -x nudged by a few BF16 ulps
    k = n // 8
    y[:k] = (x[:k] ^ 0x8000) + rng.integers(-3, 4, size=k).astype(np.uint16)
    # ties: x = 1 + m 2^-7, y = 2^-8 puts x + y on a BF16 midpoint
    m = np.arange(64, dtype=np.float32)
    xt = synth.f32_to_bf16_bits(1.0 + m * 2.0 ** -7)
    yt = synth.f32_to_bf16_bits(np.full(64, 2.0 ** -8, np.float32))
    x = np.concatenate([x, xt])
    y = np.concatenate([y, yt])
    got = oracle.residual(x, y)
    exact = [exact_bf16_round(frac_of_bits(a) + frac_of_bits(b)) for a, b in zip(x, y)]
    assert [frac_of_bits(g) for g in got] == exact
    # the midpoint cases round to the even neighbour: up for odd m, down for even m
    tie = f(got[-64:]).astype(np.float64)
    assert np.array_equal(tie, 1.0 + (m + (m % 2)) * 2.0 ** -7)
    assert np.array_equal(oracle.residual(x, np.zeros_like(x)), np.where(x == 0x8000, 0, x).astype(np.uint16))
    cancel = oracle.residual(x, x ^ 0x8000)
    assert np.all(cancel == 0)  # exactly +0 under round-to-nearest
    assert np.array_equal(got, oracle.residual(y, x))


def test_residual_vs_library_bf16_add():
    """Library cross-check: torch's BF16 tensor addition (widen, add in
    fp32, round to nearest even) gives the oracle's residual bits on a
    full-size row block of the block-output distribution."""
    rng = np.random.default_rng(32)
    x = synth.normal_bf16(rng, (64, 4096), 1.0)
    y = synth.normal_bf16(rng, (64, 4096), 0.3)
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    ty = torch.from_numpy(y.view(np.int16)).view(torch.bfloat16)
    ref = (tx + ty).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.residual(x, y), ref)


# --------------------------------------------- RMS normalisation and RoPE

def _bits(vals) -> np.ndarray:
    return synth.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def _rms_exact(xrow, grow, eps, digits=60):
    """y_i = B(g_i x_i / sqrt(s/d + eps)) with s = sum x^2 exact (rationals) and
    the square root in 60-digit decimal arithmetic."""
    from decimal import Decimal, getcontext
    getcontext().prec = digits
    xs = [frac_of_bits(u) for u in xrow]
    gs = [frac_of_bits(u) for u in grow]
    d = len(xs)
    s = sum(v * v for v in xs)
    q = s / d + Fraction(eps)
    den = (Decimal(q.numerator) / Decimal(q.denominator)).sqrt()
    out = []
    for xv, gv in zip(xs, gs):
        y = Decimal((gv * xv).numerator) / Decimal((gv * xv).denominator) / den
        out.append(exact_bf16_round(Fraction(y)))
    return out


def test_rmsnorm_hand_example_and_brute_force():
    """[PSI] sec. II-B full-row RMS: y = g x / sqrt(s/d + eps), s = sum x^2.
    [3, 4] gives 3/sqrt(12.5), 4/sqrt(12.5); random 8-wide rows agree with an
    exact-rational / 60-digit evaluation rounded to nearest-even BF16."""
    y = oracle.rmsnorm(_bits([[3.0, 4.0]]), _bits([1.0, 1.0]), eps=0.0)
    assert [frac_of_bits(u) for u in y[0]] == _rms_exact(_bits([3.0, 4.0]), _bits([1.0, 1.0]), 0.0)
    assert f(y[0]).tolist() == [0.84765625, 1.1328125]
    rng = np.random.default_rng(11)
    x = _bits(rng.standard_normal((6, 8)) * 3)
    g = _bits(1 + 0.3 * rng.standard_normal(8))
    for eps in (0.0, 1e-6, 0.25):
        y = oracle.rmsnorm(x, g, eps=eps, tile=3)
        for r in range(6):
            assert [frac_of_bits(u) for u in y[r]] == _rms_exact(x[r], g, eps), (eps, r)


def test_rmsnorm_closed_forms_and_invariants():
    """Constant rows normalise to +-g; scaling x by 2^k leaves y unchanged
    (eps = 0); scaling g by 2^k scales y by 2^k; a zero row with eps > 0 is
    zero; when every partial sum is exact, the tile width does not matter."""
    one = _bits(np.ones(16))
    c = _bits(np.full((2, 16), [[2.5], [-0.75]]))
    y = oracle.rmsnorm(c, one, eps=0.0)
    assert np.array_equal(f(y[0]), np.ones(16)) and np.array_equal(f(y[1]), -np.ones(16))
    rng = np.random.default_rng(12)
    x = _bits(rng.standard_normal((5, 64)))
    g = _bits(rng.standard_normal(64))
    y0 = oracle.rmsnorm(x, g, eps=0.0, tile=16)
    assert np.array_equal(oracle.rmsnorm(_bits(f(x) * 8.0), g, eps=0.0, tile=16), y0)
    assert np.array_equal(f(oracle.rmsnorm(x, _bits(f(g) * 0.25), eps=0.0, tile=16)), f(y0) * 0.25)
    z = oracle.rmsnorm(_bits(np.zeros((1, 8))), one[:8], eps=1e-6)
    assert np.array_equal(f(z), np.zeros((1, 8)))
    xi = _bits(rng.integers(-3, 4, size=(4, 48)).astype(np.float32))  # squares and sums exact
    gi = _bits(rng.standard_normal(48))
    ref = oracle.rmsnorm(xi, gi, eps=1e-6, tile=0)
    for tile in (1, 5, 16, 47):
        assert np.array_equal(oracle.rmsnorm(xi, gi, eps=1e-6, tile=tile), ref), tile


def test_rope_split_pairs_and_exact_angles():
    """[PSI] sec. II-B split RoPE: inside each head the pair (x_j, x_{j+dh/2})
    becomes (c a - s b, s a + c b).  cos 0 / sin 0 is the identity; a
    quarter turn maps (a, b) to (-b, a) exactly; a single nonzero element
    only touches its own pair in its own head; a rational rotation agrees
    with exact arithmetic."""
    heads, dh, M = 3, 8, 4
    rng = np.random.default_rng(13)
    x = _bits(rng.standard_normal((M, heads * dh)))
    z = np.zeros((M, dh // 2), np.float32)
    o = np.ones((M, dh // 2), np.float32)
    assert np.array_equal(oracle.rope_split(x, heads, dh, o, z), x)
    q = oracle.rope_split(x, heads, dh, z, o)
    fx, fq = f(x).reshape(M, heads, dh), f(q).reshape(M, heads, dh)
    assert np.array_equal(fq[..., :dh // 2], -fx[..., dh // 2:])
    assert np.array_equal(fq[..., dh // 2:], fx[..., :dh // 2])
    e = np.zeros((1, heads * dh), np.float32)
    e[0, 1 * dh + 1] = 1.0  # head 1, j = 1
    cs = np.full((1, dh // 2), 0.6, np.float32)
    sn = np.full((1, dh // 2), 0.8, np.float32)
    r = f(oracle.rope_split(_bits(e), heads, dh, cs, sn))[0]
    nz = np.nonzero(r)[0].tolist()
    assert nz == [1 * dh + 1, 1 * dh + 1 + dh // 2]
    # per-token, per-pair tables (rows and pair indices taken from the table)
    tab_c = rng.choice(np.array([1.0, 0.0, 0.6, -0.8, 0.28], np.float32), size=(M, dh // 2))
    tab_s = rng.choice(np.array([0.0, 1.0, 0.8, 0.6, -0.96], np.float32), size=(M, dh // 2))
    got = oracle.rope_split(x, heads, dh, tab_c, tab_s)
    for t in range(M):
        for h in range(heads):
            for j in range(dh // 2):
                cj, sj = Fraction(float(tab_c[t, j])), Fraction(float(tab_s[t, j]))
                a, b = frac_of_bits(x[t, h * dh + j]), frac_of_bits(x[t, h * dh + j + dh // 2])
                assert frac_of_bits(got[t, h * dh + j]) == exact_bf16_round(cj * a - sj * b)
                assert frac_of_bits(got[t, h * dh + j + dh // 2]) == exact_bf16_round(sj * a + cj * b)


def test_attention_bf16_numerator_two_keys():
    """Baseline PSI's BF16 numerator: with two keys whose scores differ by a
    gap g and one-hot values, the outputs are B(1 / l) and B(B(p) / l), with
    p = exp(-g) and l = 1 + p in fp32 (the normaliser keeps the fp32
    weight) -- versus B(p / l) for the fp32 weights of modified PSI.  A gap
    is chosen where rounding the numerator, or the normaliser, would change
    the BF16 output.  Equal scores give identical results."""
    dh = 4
    alpha = np.float32(0.5)  # 1 / sqrt(4)
    B = lambda v: f(synth.f32_to_bf16_bits(np.array([v], np.float32)))[0]  # noqa: E731
    chosen = None
    for kb in synth.f32_to_bf16_bits(-np.linspace(0.2, 4.0, 400, dtype=np.float32)):
        g = -np.float32(alpha * f(kb))
        p = np.float32(np.exp(np.float64(-g)))
        pb = np.float32(B(p))
        l, lb = np.float32(np.float32(1.0) + p), np.float32(np.float32(1.0) + pb)
        if B(pb / l) != B(p / l) and (B(np.float32(1.0) / lb) != B(np.float32(1.0) / l) or B(pb / lb) != B(pb / l)):
            chosen = (kb, p, pb, l)
            break
    assert chosen is not None
    kb, p, pb, l = chosen
    q = _bits([[1.0, 0.0, 0.0, 0.0]])
    k = np.array([_bits([0.0, 0, 0, 0]), np.array([kb, 0, 0, 0], np.uint16)])
    v = _bits([[1.0, 0, 0, 0], [0.0, 1.0, 0, 0]])
    o_b = f(oracle.attention_ex(q, k, v, 1, dh, bf16_p=True))[0]
    o_f = f(oracle.attention_ex(q, k, v, 1, dh, bf16_p=False))[0]
    assert o_b[1] == B(pb / l) and o_f[1] == B(p / l) and o_b[1] != o_f[1]
    assert o_b[0] == o_f[0] == B(np.float32(1.0) / l)
    qz = _bits(np.zeros((3, 8)))
    kz = _bits(np.random.default_rng(14).standard_normal((5, 8)))
    vz = _bits(np.random.default_rng(15).standard_normal((5, 8)))
    assert np.array_equal(oracle.attention_ex(qz, kz, vz, 2, 4, bf16_p=True), oracle.attention(qz, kz, vz, 2, 4))


def test_attn_sublayer_ext_reduces_to_plain_and_composes():
    """Without normalisation or rotary tables the extended sub-block is the
    pinned plain one; with them it is the plain sub-block on the projections
    normalised and rotated by the pinned pieces (checked through the
    attention core on those pieces)."""
    rng = np.random.default_rng(16)
    M, d, heads, dh = 12, 32, 2, 16
    x = _bits(rng.standard_normal((M, d)))
    w = {}
    for n in ("q", "k", "v", "o"):
        w["W" + n] = _bits(rng.standard_normal((d, d)) / np.sqrt(d))
        w["b" + n] = _bits(0.1 * rng.standard_normal(d))
    plain = oracle.attn_sublayer(x, w["Wq"], w["bq"], w["Wk"], w["bk"], w["Wv"], w["bv"], w["Wo"], w["bo"],
                                 heads, dh)
    assert np.array_equal(oracle.attn_sublayer_ext(x, w, heads, dh), plain)
    gq, gk = _bits(1 + 0.2 * rng.standard_normal(d)), _bits(1 + 0.2 * rng.standard_normal(d))
    ang = rng.uniform(0, 6.3, size=(M, dh // 2))
    cs, sn = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    y = oracle.attn_sublayer_ext(x, w, heads, dh, gq=gq, gk=gk, eps=1e-6, norm_tile=8, cos_q=cs, sin_q=sn,
                                 residual=False)
    Q = oracle.rope_split(oracle.rmsnorm(oracle.linear(x, w["Wq"], w["bq"]), gq, 1e-6, 8), heads, dh, cs, sn)
    K = oracle.rope_split(oracle.rmsnorm(oracle.linear(x, w["Wk"], w["bk"]), gk, 1e-6, 8), heads, dh, cs, sn)
    V = oracle.linear(x, w["Wv"], w["bv"])
    ref = oracle.linear(oracle.attention(Q, K, V, heads, dh), w["Wo"], w["bo"])
    assert np.array_equal(y, ref)
