"""Pins for the CPU oracle: each checks it against something other than itself.

Every pin is a plain function that raises AssertionError on failure, so the same
pins can be re-run with a mistake planted in the oracle (test_oracle_mutations).
Kinds of pin used: a published format table (OCP MX v1.0 E2M1 values), a worked
example written out by hand, exact rational arithmetic (fractions.Fraction),
closed forms, special cases that reduce to a textbook routine, and invariants.
"""
from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

import numpy as np

import oracle.moe as om
import oracle.mx as omx
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ fixtures

def golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return [vals[c] for c in range(16)]


def golden_worked_example():
    rows = []
    cur = {}
    with open(os.path.join(GOLDEN, "mxfp4_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(":", 1)
            cur[key] = rest.split()
            if key == "values":
                rows.append(cur)
                cur = {}
    scales = np.array([[int(s) for s in r["scales"]] for r in rows], np.uint8)
    packed = np.array([[int(b, 16) for b in r["bytes"]] for r in rows], np.uint8)
    values = np.array([[float(v) for v in r["values"]] for r in rows], np.float64)
    return packed, scales, values


def frac_bf16(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0])


def brute_weight(codes, scales, n, k, table):
    """Element (n, k) of an MXFP4 matrix by the storage rule, one element at a time."""
    byte = int(codes[n][k >> 1])
    nib = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
    return Fraction(table[nib]) * Fraction(2) ** (int(scales[n][k // 32]) - 127)


def sigmoid_ref(z: float) -> float:
    # the logistic function through tanh, a formula independent of the oracle's
    return 0.5 * (1.0 + math.tanh(0.5 * z))


# ------------------------------------------------------------------ MXFP4

def pin_e2m1_table():
    """The oracle's E2M1 decode equals the OCP MX v1.0 value table, signed zero included."""
    gold = golden_e2m1()
    for c in range(16):
        v = omx.E2M1[c]
        assert v == gold[c], (c, v, gold[c])
        assert math.copysign(1.0, v) == math.copysign(1.0, gold[c]), c


def pin_e8m0_bits():
    """E8M0 byte s equals the float64 whose exponent field is s-127+1023 (built from
    bits, not from a power function); 255 is NaN."""
    for s in range(255):
        ref = struct.unpack("<d", struct.pack("<Q", (s - 127 + 1023) << 52))[0]
        assert omx.E8M0[s] == ref, s
    assert math.isnan(omx.E8M0[255])
    assert omx.E8M0[127] == 1.0 and omx.E8M0[128] == 2.0 and omx.E8M0[126] == 0.5


def pin_dequant_worked_example():
    """Dequantising the hand-worked example reproduces its hand-written values."""
    packed, scales, values = golden_worked_example()
    got = omx.dequant(packed, scales)
    assert got.shape == values.shape
    assert np.array_equal(got, values), np.argwhere(got != values)[:5]
    assert np.array_equal(np.signbit(got), np.signbit(values))


def pin_dequant_exhaustive():
    """All 16 codes x 255 finite scales: value == ldexp(table value, s - 127)."""
    gold = golden_e2m1()
    codes = np.repeat(np.arange(16, dtype=np.uint8), 255)
    sc = np.tile(np.arange(255, dtype=np.uint8), 16)
    packed = np.repeat((codes | (codes << 4)).astype(np.uint8)[:, None], 16, axis=1)
    got = omx.dequant(packed, sc[:, None])
    for i in range(codes.size):
        ref = math.ldexp(gold[codes[i]], int(sc[i]) - 127)
        assert np.all(got[i] == ref), (codes[i], sc[i], got[i][0], ref)


def pin_one_hot_layout():
    """x = e_i picks column i of the dequantised gate matrix (plus the bias), for i on
    both nibbles and on both sides of a 32-element scale block; checked element by
    element against the storage rule."""
    gold = golden_e2m1()
    w = synth.tiny_workload(T=1, d=64, F=32, E=2, k=1, seed=11, scale_lo=120, scale_hi=130)
    L = w.layers[0]
    wg = omx.dequant(L.gate.codes[1], L.gate.scales[1])
    wu = omx.dequant(L.up.codes[1], L.up.scales[1])
    bg = om.bf16_to_f64(L.b_gate[1])
    bu = om.bf16_to_f64(L.b_up[1])
    for i in (0, 1, 30, 31, 32, 33, 62, 63):
        x = np.zeros((1, 64))
        x[0, i] = 1.0
        g, u = om.gate_up(x, wg, wu, bg, bu)
        for n in range(32):
            ref_g = brute_weight(L.gate.codes[1], L.gate.scales[1], n, i, gold) + frac_bf16(L.b_gate[1][n])
            ref_u = brute_weight(L.up.codes[1], L.up.scales[1], n, i, gold) + frac_bf16(L.b_up[1][n])
            assert Fraction(g[0, n]) == ref_g, (i, n)
            assert Fraction(u[0, n]) == ref_u, (i, n)


# ------------------------------------------------------------------ routing

def pin_router_exact():
    """Router logits against exact rational dot products (bf16 x, fp32 W_r, fp32 b_r)."""
    w = synth.tiny_workload(T=5, d=96, F=32, E=6, k=2, seed=3, zipf=True)
    L = w.layers[0]
    x = om.bf16_to_f64(w.x)
    got = om.router_logits(x, L.w_router, L.b_router)
    for t in range(w.T):
        for e in range(w.E):
            acc = Fraction(0)
            mag = 0.0
            for kk in range(w.d):
                p = frac_bf16(w.x[t, kk]) * Fraction(float(L.w_router[kk, e]))
                acc += p
                mag += abs(float(p))
            acc += Fraction(float(L.b_router[e]))
            mag += abs(float(L.b_router[e]))
            bound = (w.d + 2) * 2.0 ** -53 * mag
            assert abs(Fraction(got[t, e]) - acc) <= Fraction(bound), (t, e)


def pin_topk_vs_sorted():
    """Top-k (with many exact ties) equals Python's sorted() by (-logit, index)."""
    rng = np.random.default_rng(5)
    for E, k in ((8, 4), (32, 4), (128, 4), (7, 7), (5, 1), (16, 8)):
        l = rng.integers(-3, 4, size=(50, E)).astype(np.float64)  # lots of ties
        got = om.topk_select(l, k)
        for t in range(l.shape[0]):
            ref = sorted(range(E), key=lambda e: (-l[t, e], e))[:k]
            assert list(got[t]) == ref, (E, k, t)


def pin_zero_router():
    """W_r = 0, b_r = 0: every logit ties, so experts 0..k-1 win with weight 1/k exactly."""
    d, E, k = 32, 16, 4
    x = np.ones((3, d))
    idx, w, _ = om.route(x, np.zeros((d, E), np.float32), None, k)
    assert np.array_equal(idx, np.tile(np.arange(k), (3, 1)))
    assert np.all(w == 0.25)


def pin_ordered_bias():
    """W_r = 0 and a bias fixes the routing; the weights are the closed-form softmax
    of the four biggest biases."""
    d, E, k = 32, 12, 4
    b = np.zeros(E, np.float32)
    b[[2, 4, 3, 1]] = [40.0, 30.0, 20.0, 10.0]
    idx, w, _ = om.route(np.ones((2, d)), np.zeros((d, E), np.float32), b, k)
    assert np.array_equal(idx, np.array([[2, 4, 3, 1]] * 2))
    den = 1.0 + math.exp(-10.0) + math.exp(-20.0) + math.exp(-30.0)
    ref = [1.0 / den, math.exp(-10.0) / den, math.exp(-20.0) / den, math.exp(-30.0) / den]
    assert np.allclose(w, np.array([ref] * 2), rtol=1e-15, atol=0)


def pin_two_way_sigmoid():
    """k = 2: the first weight is the logistic function of the logit gap, the second
    its complement (the closed form of a 2-way softmax)."""
    rng = np.random.default_rng(6)
    l = rng.standard_normal((40, 9)) * 3
    idx = om.topk_select(l, 2)
    w = om.softmax_selected(l, idx)
    for t in range(40):
        gap = l[t, idx[t, 0]] - l[t, idx[t, 1]]
        assert abs(w[t, 0] - sigmoid_ref(gap)) <= 1e-15
        assert abs(w[t, 1] - sigmoid_ref(-gap)) <= 1e-15


def pin_softmax_after_topk_not_before():
    """Weights renormalise over the selected experts only: on a case where the other
    experts carry most of the probability mass the two readings differ a lot."""
    l = np.array([[5.0, 4.9, 4.8, 4.7, 4.6, 4.5, 4.4, 4.3]])
    idx = om.topk_select(l, 2)
    w = om.softmax_selected(l, idx)
    assert np.array_equal(idx[0], [0, 1])
    assert abs(w[0, 0] - sigmoid_ref(0.1)) <= 1e-15
    assert abs(w.sum() - 1.0) <= 1e-15


def pin_switch_k1():
    """k = 1 (switch routing): the single weight is exactly 1."""
    rng = np.random.default_rng(7)
    l = rng.standard_normal((30, 10))
    idx = om.topk_select(l, 1)
    w = om.softmax_selected(l, idx)
    assert np.all(w == 1.0)
    assert np.array_equal(idx[:, 0], np.argmax(l, axis=1))


def pin_dense_gating_e_eq_k():
    """E = k: softmax after top-k is the textbook softmax over all experts
    (scipy.special.softmax), just reordered."""
    from scipy.special import softmax as sp_softmax
    rng = np.random.default_rng(8)
    l = rng.standard_normal((25, 6)) * 2
    idx = om.topk_select(l, 6)
    w = om.softmax_selected(l, idx)
    ref = sp_softmax(l, axis=1)
    assert np.allclose(w, np.take_along_axis(ref, idx.astype(np.int64), 1), rtol=1e-14, atol=1e-16)


def pin_weights_sum_to_one():
    rng = np.random.default_rng(9)
    l = rng.standard_normal((500, 128)) * 4
    idx = om.topk_select(l, 4)
    w = om.softmax_selected(l, idx)
    assert np.max(np.abs(w.sum(1) - 1.0)) <= 1e-15
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)


# ------------------------------------------------------------------ dispatch

def _brute_permute(idx, E):
    T, k = idx.shape
    sorted_pair, counts = [], [0] * E
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t][j] == e:
                    sorted_pair.append(t * k + j)
                    counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    pair_row = [0] * (T * k)
    for p, q in enumerate(sorted_pair):
        pair_row[q] = p
    return counts, offsets, sorted_pair, pair_row


def pin_permute_brute():
    """Counts, offsets, order and inverse against a literal loop over experts/tokens."""
    rng = np.random.default_rng(10)
    for T, E, k in ((1, 4, 4), (13, 8, 3), (64, 32, 4), (50, 128, 4), (9, 5, 1)):
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        c, o, s, r = om.permute(idx, E)
        bc, bo, bs, br = _brute_permute(idx, E)
        assert list(c) == bc and list(o) == bo and list(s) == bs and list(r) == br, (T, E, k)


def pin_permute_invariants():
    """Bijection, per-expert blocks, ascending tokens inside a block, empty experts."""
    rng = np.random.default_rng(12)
    T, E, k = 3000, 64, 4
    # only 20 of 64 experts are ever used: the rest must come out empty
    used = rng.permutation(E)[:20]
    idx = np.stack([used[rng.permutation(20)[:k]] for _ in range(T)]).astype(np.int32)
    c, o, s, r = om.permute(idx, E)
    P = T * k
    assert o[0] == 0 and o[-1] == P and int(c.sum()) == P
    assert np.array_equal(np.diff(o), c)
    assert np.array_equal(np.sort(s), np.arange(P))
    assert np.array_equal(r[s], np.arange(P)) and np.array_equal(s[r], np.arange(P))
    flat = idx.reshape(-1)
    for e in range(E):
        blk = s[o[e]:o[e + 1]]
        assert np.all(flat[blk] == e)
        assert np.all(np.diff(blk // k) > 0)
        if e not in used:
            assert c[e] == 0


# ------------------------------------------------------------------ expert FFN

def pin_gate_up_exact():
    """g and u on a tiny expert (d = 64 != F = 32, two scale blocks) against exact
    rational GEMMs built element by element from the storage rule."""
    gold = golden_e2m1()
    w = synth.tiny_workload(T=3, d=64, F=32, E=1, k=1, seed=13)
    L = w.layers[0]
    x = om.bf16_to_f64(w.x)
    wg = omx.dequant(L.gate.codes[0], L.gate.scales[0])
    wu = omx.dequant(L.up.codes[0], L.up.scales[0])
    g, u = om.gate_up(x, wg, wu, om.bf16_to_f64(L.b_gate[0]), om.bf16_to_f64(L.b_up[0]))
    for t in range(3):
        xf = [frac_bf16(b) for b in w.x[t]]
        for n in range(32):
            eg = sum(xf[i] * brute_weight(L.gate.codes[0], L.gate.scales[0], n, i, gold) for i in range(64))
            eu = sum(xf[i] * brute_weight(L.up.codes[0], L.up.scales[0], n, i, gold) for i in range(64))
            eg += frac_bf16(L.b_gate[0][n])
            eu += frac_bf16(L.b_up[0][n])
            tol = Fraction(2.0 ** -45)
            assert abs(Fraction(g[t, n]) - eg) <= tol * (1 + abs(eg)), (t, n)
            assert abs(Fraction(u[t, n]) - eu) <= tol * (1 + abs(eu)), (t, n)


def pin_down_exact():
    """The down projection (K = F = 32, N = d = 64) against an exact rational GEMM."""
    gold = golden_e2m1()
    w = synth.tiny_workload(T=2, d=64, F=32, E=1, k=1, seed=14)
    L = w.layers[0]
    rng = np.random.default_rng(15)
    h = rng.standard_normal((2, 32)) * 10
    wd = omx.dequant(L.down.codes[0], L.down.scales[0])
    y = om.down(h, wd, om.bf16_to_f64(L.b_down[0]))
    assert y.shape == (2, 64)
    for t in range(2):
        for n in range(64):
            ey = sum(Fraction(h[t, i]) * brute_weight(L.down.codes[0], L.down.scales[0], n, i, gold)
                     for i in range(32)) + frac_bf16(L.b_down[0][n])
            assert abs(Fraction(y[t, n]) - ey) <= Fraction(2.0 ** -45) * (1 + abs(ey)), (t, n)


def pin_silu_identity():
    """silu(z) = (z/2)(1 + tanh(z/2)), including 0 and very large |z| (no overflow)."""
    z = np.concatenate([np.linspace(-40, 40, 801), [0.0, -800.0, 800.0, -1e4, 1e4]])
    s = om.silu(z)
    for zi, si in zip(z, s):
        ref = 0.5 * zi * (1.0 + math.tanh(0.5 * zi))
        # the tanh form cancels for z << 0, so its own error is ~|z| * 2^-53
        assert abs(si - ref) <= 4e-16 * max(1.0, abs(zi)), (zi, si, ref)
    assert om.silu(np.array([0.0]))[0] == 0.0
    g = np.array([1.5, -2.0]); u = np.array([3.0, 0.5])
    assert np.allclose(om.swiglu(g, u), [1.5 * sigmoid_ref(1.5) * 3.0, -2.0 * sigmoid_ref(-2.0) * 0.5],
                       rtol=1e-15)


def _identity_layer(d: int, E: int):
    """Every expert is W_gate = W_up = W_down = I (code 2 = 1.0 at scale byte 127), zero biases."""
    codes = np.zeros((E, d, d), np.uint8)
    for i in range(d):
        codes[:, i, i] = 2
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    sc = np.full((E, d, d // 32), 127, np.uint8)
    zb = np.zeros((E, d), np.uint16)
    mx = synth.MX4(packed, sc)
    rng = np.random.default_rng(16)
    wr = (rng.standard_normal((d, E)) * 0.3).astype(np.float32)
    return synth.LayerParams(wr, None, mx, synth.MX4(packed.copy(), sc.copy()),
                             synth.MX4(packed.copy(), sc.copy()), zb, zb.copy(), zb.copy())


def pin_identity_experts():
    """Identity experts: y = silu(x) * x for every expert, so out = silu(x) * x
    whatever the routing (the weights sum to 1)."""
    d, E, k = 64, 8, 4
    L = _identity_layer(d, E)
    rng = np.random.default_rng(17)
    xb = synth.bf16_bits(rng.standard_normal((20, d)) * 2)
    out = om.moe_layer(xb, L, k)["out"]
    x = om.bf16_to_f64(xb)
    for t in range(20):
        for i in range(d):
            xi = x[t, i]
            ref = xi * sigmoid_ref(xi) * xi
            assert abs(out[t, i] - ref) <= 1e-13 * max(1.0, abs(ref)), (t, i)


def pin_dense_equals_staged():
    """The dispatch/grouped path equals the dense masked formula over all experts."""
    for T, d, F, E, k, seed, z in ((9, 64, 32, 8, 4, 18, False), (6, 32, 64, 5, 2, 19, True),
                                   (4, 32, 32, 4, 4, 20, False)):
        w = synth.tiny_workload(T=T, d=d, F=F, E=E, k=k, seed=seed, zipf=z)
        a = om.moe_layer(w.x, w.layers[0], k)["out"]
        b = om.dense_moe(w.x, w.layers[0], k)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12 * np.abs(b).max()), (T, d, F, E, k)


def pin_identical_experts():
    """With all experts equal the layer is one FFN, independent of the routing."""
    w = synth.tiny_workload(T=7, d=64, F=64, E=6, k=3, seed=21)
    L = w.layers[0]
    for m in (L.gate, L.up, L.down):
        m.codes[:] = m.codes[0]
        m.scales[:] = m.scales[0]
    for b in (L.b_gate, L.b_up, L.b_down):
        b[:] = b[0]
    out = om.moe_layer(w.x, L, 3)["out"]
    x = om.bf16_to_f64(w.x)
    wg = omx.dequant(L.gate.codes[0], L.gate.scales[0])
    wu = omx.dequant(L.up.codes[0], L.up.scales[0])
    wd = omx.dequant(L.down.codes[0], L.down.scales[0])
    # one FFN written out with sigmoid through tanh
    g = x @ wg.T + om.bf16_to_f64(L.b_gate[0])
    u = x @ wu.T + om.bf16_to_f64(L.b_up[0])
    h = g * (0.5 * (1 + np.tanh(0.5 * g))) * u
    ref = h @ wd.T + om.bf16_to_f64(L.b_down[0])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def pin_combine_weights_follow_slots():
    """Combine pairs w[t, j] with the expert chosen in slot j: with one-hot expert
    outputs (expert e returns its bias e_e in a unit vector) out[t] = sum_j w[t,j] e_{idx[t,j]}."""
    T, E, k, d = 11, 6, 3, 32
    rng = np.random.default_rng(22)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k))
    c, o, s, r = om.permute(idx, E)
    y = np.zeros((T * k, d))
    flat = idx.reshape(-1)
    for p in range(T * k):
        y[p, flat[s[p]]] = 1.0
    out = om.combine(y, r, w)
    for t in range(T):
        ref = np.zeros(d)
        for j in range(k):
            ref[idx[t, j]] += w[t, j]
        assert np.array_equal(out[t], ref), t


# ------------------------------------------------------------------ RMSNorm

def pin_rmsnorm_constant_row():
    """A constant row c gives gain * c / sqrt(c^2 + eps)."""
    d = 2880
    gain = 1.0 + 0.01 * np.arange(d) / d
    for c in (1.0, -3.0, 1e-3, 250.0):
        n = om.rmsnorm(np.full((1, d), c), gain, 1e-5)
        ref = gain * c / math.sqrt(c * c + 1e-5)
        assert np.allclose(n[0], ref, rtol=1e-15, atol=0), c


def pin_rmsnorm_scale_invariance():
    """With eps = 0, scaling a row by 2^j leaves the normalised row unchanged; with
    eps = 1e-5 rows of RMS 1 and 1000 normalise to the same result within eps."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((4, 96))
    g = 1 + 0.02 * rng.standard_normal(96)
    a = om.rmsnorm(x, g, 0.0)
    for j in (-5, 3, 20):
        assert np.allclose(om.rmsnorm(x * 2.0 ** j, g, 0.0), a, rtol=1e-15, atol=0)
    assert np.allclose(om.rmsnorm(x * 1000, g, 1e-5), a, rtol=1e-11)
    rms = np.sqrt(np.mean((a / g) ** 2, axis=1))
    assert np.allclose(rms, 1.0, rtol=1e-15)




# ------------------------------------------------------------------ FP8 block-scaled weights

import oracle.fp8 as of8  # noqa: E402


def golden_e4m3():
    vals = {}
    with open(os.path.join(GOLDEN, "e4m3_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c, 16)] = float(v)
    return vals


def pin_e4m3_table():
    """The OCP E4M3 values of selected codes (golden file), sign symmetry over all
    256 codes, exactly two NaN codes, and strictly increasing finite magnitudes
    0x00 .. 0x7E (each step a fixed fraction of its binade)."""
    for c, v in golden_e4m3().items():
        got = of8.e4m3_value(c)
        assert (math.isnan(v) and math.isnan(got)) or got == v, (hex(c), got, v)
        assert (math.isnan(v) and math.isnan(of8.E4M3[c])) or of8.E4M3[c] == v
    t = of8.E4M3
    assert np.isnan(t).sum() == 2 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0
    for c in range(0x7F):
        assert t[c | 0x80] == -t[c]
        if c >= 8:
            _, e = math.frexp(t[c])   # within a binade [2^(e-1), 2^e) the step is 2^(e-1)/8
            assert t[c + 1] - t[c] == math.ldexp(1.0, e - 1 - 3) if c + 1 < 0x7F else True


def pin_fp8_block_dequant():
    """Element (n, k) of a block-scaled FP8 matrix is E4M3[code] times the scale
    of block (n // 128, k // 128), including partial edge blocks: checked one
    element at a time against a loop, on a non-square shape with partial blocks
    in both directions."""
    rng = np.random.default_rng(60)
    N, K = 200, 300
    codes = rng.integers(0, 0x7F, (N, K), dtype=np.uint8)
    codes[rng.random((N, K)) < 0.5] |= 0x80
    scales = (2.0 ** rng.integers(-9, 3, (2, 3)) * (1 + rng.random((2, 3)))).astype(np.float32)
    got = of8.dequant_fp8(codes, scales)
    for _ in range(400):
        n, k = int(rng.integers(N)), int(rng.integers(K))
        want = of8.e4m3_value(int(codes[n, k])) * float(scales[n // 128][k // 128])
        assert got[n, k] == want, (n, k)
    assert got.shape == (N, K)


def _mx4_to_fp8_bruteforce(packed, scales):
    """Convert one MXFP4 matrix [N][K] to FP8 with 128x128 block scales by brute
    force: block scale = 2^(largest E8M0 exponent in the block), and each element's
    code is the E4M3 code whose value equals element / block scale exactly
    (searched in the table); returns (codes, scales)."""
    vals = omx.dequant(packed, scales)
    N, K = vals.shape
    nb, kb = (N + 127) // 128, (K + 127) // 128
    bs = np.zeros((nb, kb), np.float32)
    codes = np.zeros((N, K), np.uint8)
    lookup = {}
    for c in range(256):
        v = of8.E4M3[c]
        if not np.isnan(v) and v not in lookup and not (v == 0 and c == 0x80):
            lookup[v] = c
    for i in range(nb):
        for j in range(kb):
            smax = int(scales[128 * i:128 * (i + 1), 4 * j:4 * (j + 1)].max())
            bs[i, j] = np.float32(math.ldexp(1.0, smax - 127))
            blk = vals[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)] / float(bs[i, j])
            codes[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)] = np.vectorize(lookup.__getitem__)(blk)
    return codes, bs


def pin_mxfp4_to_fp8_exact():
    """MXFP4 weights whose E8M0 exponents within a 128x128 block differ by at most
    8 are exactly FP8 block-scaled weights (the conversion the pages' Hopper
    engine made once): the brute-force conversion exists and its FP8 dequant
    equals the MXFP4 dequant exactly. Shape with partial blocks."""
    rng = np.random.default_rng(61)
    N, K = 160, 192
    packed = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(121, 125, (N, K // 32), dtype=np.uint8)
    codes, bs = _mx4_to_fp8_bruteforce(packed, scales)
    assert np.array_equal(of8.dequant_fp8(codes, bs), omx.dequant(packed, scales))


def pin_ffn_fp8_matches_mxfp4():
    """The FP8 expert FFN on exactly converted weights is the MXFP4 expert FFN
    (the same float64 values give the same result bit for bit), and on weights
    scaled by 2 in one block the output changes (the block scale is used)."""
    w = synth.tiny_workload(T=24, d=128, F=192, E=3, k=2, seed=62)
    L = w.layers[0]
    conv = {}
    for name in ("gate", "up", "down"):
        m = getattr(L, name)
        cs = [_mx4_to_fp8_bruteforce(m.codes[e], m.scales[e]) for e in range(3)]
        conv[name] = (np.stack([c for c, _ in cs]), np.stack([s for _, s in cs]))
    x = om.bf16_to_f64(w.x)
    idx, _, _ = om.route(x, L.w_router, L.b_router, 2)
    _, off, sp, _ = om.permute(idx, 3)
    y4 = om.ffn_sorted(x, sp, off, 2, L)
    y8 = om.ffn_sorted_fp8(x, sp, off, 2, conv, L.b_gate, L.b_up, L.b_down)
    assert np.array_equal(y4, y8)
    conv["down"][1][0, 0, 0] *= 2
    y8b = om.ffn_sorted_fp8(x, sp, off, 2, conv, L.b_gate, L.b_up, L.b_down)
    assert not np.array_equal(y4, y8b)


def pin_round_bf16():
    """Routing weights rounded to bf16: ties to even at 1 + 2^-8 and 1 + 3 2^-8,
    and equal to torch's float32 -> bfloat16 cast on random weights."""
    import torch
    r = om.round_bf16(np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 0.3]))
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1 + 2.0 ** -6
    w = np.random.default_rng(63).random(1000)
    want = torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(om.round_bf16(w), want)


# ------------------------------------------------------------------ attention with sinks

import oracle.attention as oat  # noqa: E402


def _attn_inputs(seed, B, Tq, S, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Tq, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    s = rng.standard_normal(Hq)
    return q, k, v, s


def pin_attention_without_sink_is_sdpa():
    """A sink of -inf takes no part: the result is torch's scaled dot-product
    attention (float64, CPU) with the same causal and sliding-window mask and the
    KV heads repeated for grouped queries."""
    import torch
    q, k, v, _ = _attn_inputs(70, 2, 6, 11, 4, 2, 8)
    for window in (0, 4):
        got = oat.attention_sink(q, k, v, np.full(4, -np.inf), 0.35, window)
        mask = torch.from_numpy(oat.visible(6, 11, window))
        for b in range(2):
            Q = torch.from_numpy(q[b]).permute(1, 0, 2)            # [H][Tq][D]
            K = torch.from_numpy(k[b]).permute(1, 0, 2).repeat_interleave(2, dim=0)
            V = torch.from_numpy(v[b]).permute(1, 0, 2).repeat_interleave(2, dim=0)
            want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=0.35)
            assert np.allclose(got[b], want.permute(1, 0, 2).numpy(), rtol=0, atol=1e-13)


def pin_attention_single_key():
    """One visible key: out = v * sigmoid(z - s), z = scale <q, k> (a two-way
    softmax with the sink); a window of 1 reduces every query to that case."""
    q, k, v, s = _attn_inputs(71, 1, 3, 3, 2, 1, 4)
    out = oat.attention_sink(q, k, v, s, 0.5, window=1)
    for i in range(3):
        for h in range(2):
            z = 0.5 * float(q[0, i, h] @ k[0, i, 0])
            assert np.allclose(out[0, i, h], v[0, i, 0] / (1 + math.exp(s[h] - z)), rtol=1e-14, atol=0)


def pin_attention_brute_force():
    """Every output element against a plain loop over keys with math.exp, on a
    ragged shape (Tq < S, grouped heads, a window)."""
    q, k, v, s = _attn_inputs(72, 1, 3, 7, 4, 2, 3)
    out = oat.attention_sink(q, k, v, s, 0.7, window=5)
    for i in range(3):
        pos = 7 - 3 + i
        for h in range(4):
            g = h // 2
            keys = [j for j in range(7) if j <= pos and j > pos - 5]
            w = [math.exp(0.7 * sum(q[0, i, h, c] * k[0, j, g, c] for c in range(3))) for j in keys]
            den = math.exp(s[h]) + sum(w)
            for c in range(3):
                want = sum(wj * v[0, j, g, c] for wj, j in zip(w, keys)) / den
                assert abs(out[0, i, h, c] - want) <= 1e-13 * (1 + abs(want))


def pin_attention_chunks_take_the_sink_once():
    """The split-KV form (online-softmax partials merged in chunk order, the sink
    in the first chunk only) equals the direct form; counting the sink in every
    chunk instead does not."""
    q, k, v, s = _attn_inputs(73, 2, 4, 13, 4, 1, 8)
    direct = oat.attention_sink(q, k, v, s, 0.3, 0)
    for chunk in (1, 4, 5, 13):
        assert np.allclose(oat.attention_sink_chunked(q, k, v, s, 0.3, 0, chunk), direct, rtol=1e-12, atol=1e-14)
    # the sink counted once per chunk: a larger denominator, outputs shrink
    K = 13
    twice = oat.attention_sink(q, k, v, s + math.log(math.ceil(K / 4)), 0.3, 0)
    assert not np.allclose(twice, direct)


def pin_attention_sink_limits():
    """A very large sink absorbs the softmax (outputs -> 0); the output is a
    convex combination of the visible values scaled by 1 - p_sink."""
    q, k, v, s = _attn_inputs(74, 1, 4, 6, 2, 2, 4)
    big = oat.attention_sink(q, k, v, np.full(2, 80.0), 0.2, 0)
    assert np.abs(big).max() < 1e-20
    out = oat.attention_sink(q, k, v, s, 0.2, 0)
    for i in range(4):
        pos = 6 - 4 + i
        for h in range(2):
            vis = v[0, :pos + 1, h, :]
            assert np.all(out[0, i, h] <= np.maximum(vis.max(axis=0), 0) + 1e-12)
            assert np.all(out[0, i, h] >= np.minimum(vis.min(axis=0), 0) - 1e-12)


ALL_PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}
