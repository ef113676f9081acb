"""Pins of the CPU oracle against things other than itself: brute force in
exact rational arithmetic, closed forms, invariants and library routines.
Each test names the step it pins (C1..C8, see oracle/__init__.py)."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from synth import recipes


def _f16(bits):
    return np.array(bits, np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------- generator
def test_generator_is_counter_based_and_deterministic():
    a = synth.normal_f32(7, 3, 1, 1000)
    b = synth.normal_f32(7, 3, 1, 1000)
    assert np.array_equal(a, b)
    # any slice regenerates on its own
    c = synth.normal_f32(7, 3, 1, 100, start=450)
    assert np.array_equal(a[450:550], c)
    # row slices of a weight matrix regenerate the same fields
    full = synth.q4k_fields(5, 9, 40, 512)
    part = synth.q4k_fields(5, 9, 40, 512, 17, 29)
    for k in ("d", "dmin", "sc", "m", "q"):
        assert np.array_equal(full[k][17:29], part[k])
    # different streams differ
    assert not np.array_equal(a, synth.normal_f32(7, 3, 2, 1000))


def test_generator_fp16_rounding_matches_numpy():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(20000) * np.logspace(-9, 5, 20000)
    # exact half-way cases between adjacent fp16 values, incl. subnormals
    hw = (np.arange(1, 2000, dtype=np.float64) + 0.5) * 2.0 ** -24
    hw2 = (1024 + np.arange(0, 1000) + 0.5) * 2.0 ** -10
    allv = np.concatenate([v, -v, hw, hw2, [0.0, 65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -25, 2.0 ** -24]])
    got = np.array([synth.f64_to_f16_bits(x) for x in allv], np.uint16)
    with np.errstate(over="ignore"):
        ref = allv.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_generator_field_ranges_and_distribution():
    W = synth.q4k_fields(0, 1, 256, 2048)
    assert W["q"].max() == 15 and W["q"].min() == 0
    assert W["sc"].max() == 63 and W["m"].max() == 63 and W["sc"].min() == 0
    d = _f16(W["d"])
    assert (d >= 0).all()
    # E|N(0, 0.01)| = 0.01*sqrt(2/pi)
    assert abs(d.mean() - 0.01 * np.sqrt(2 / np.pi)) < 3e-4
    # some d are fp16 subnormal (< 2^-14): about 0.49% of |N(0, 0.01)|
    frac_sub = np.mean(d < 2.0 ** -14)
    assert 0.002 < frac_sub < 0.009
    # codes uniform on 0..15
    counts = np.bincount(W["q"].ravel(), minlength=16) / W["q"].size
    assert np.abs(counts - 1 / 16).max() < 0.003
    x = synth.normal_f32(0, 2, 0, 200000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


# ----------------------------------------------------------------- C1 fp16
def test_f16_to_f32_all_bit_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32)
    got = np.array([orc.f16_to_f32(b) for b in bits], np.float32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


# ----------------------------------------------------------------- C2 quantizer
def test_quantizer_closed_form_properties(orc):
    x = synth.normal_f32(11, 1, 0, 7 * 4096).reshape(7, 4096)
    x[3, 64:96] = 0.0  # one all-zero group
    a8, s, gs = orc.quantize_rows(x)
    assert np.abs(a8.astype(int)).max() <= 127
    g = a8.reshape(7, -1, 32).astype(np.int64)
    assert np.array_equal(g.sum(-1), gs)
    nz = s > 0
    assert np.all(np.abs(g).max(-1)[nz] == 127)  # every non-zero group attains +-127
    assert np.all(g[~nz] == 0) and (~nz).sum() == 1
    err = np.abs(x.reshape(7, -1, 32).astype(np.float64) - s[..., None].astype(np.float64) * g)
    assert np.all(err <= s[..., None] / 2 * (1 + 2.0 ** -22))
    # power-of-two scaling is exact
    a8b, sb, _ = orc.quantize_rows(x * 4)
    assert np.array_equal(a8, a8b) and np.array_equal(sb, s * 4)


def test_quantizer_identity_and_round_half_even(orc):
    rng = np.random.default_rng(3)
    xi = rng.integers(-127, 128, size=(3, 256)).astype(np.float32)
    xi.reshape(3, -1, 32)[:, :, 0] = 127.0  # every group contains 127 -> s = 1 exactly
    a8, s, gs = orc.quantize_rows(xi)
    assert np.all(s == 1.0) and np.array_equal(a8.astype(np.float32), xi)
    # half-way values with s = 1 round to even
    h = np.zeros((1, 32), np.float32)
    h[0, 0] = 127
    h[0, 1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 126.5]
    a8, s, _ = orc.quantize_rows(h)
    assert s[0, 0] == 1.0
    assert list(a8[0, 1:9]) == [0, 2, 2, 0, -2, -2, 4, 126]


def test_quantizer_underflowing_scale_nan_and_inf(orc):
    """Groups with no usable scale and non-finite elements, from the reading:
    s = fl32(amax / 127) over the non-NaN elements; s == 0 (amax at most
    63 * 2^-149, where amax / 127 rounds to zero) or an all-NaN group gives
    s = 0 and zero codes; a NaN quotient codes as 0."""
    tiny = np.float32(2.0 ** -149)
    x = np.zeros((6, 32), np.float32)
    k = np.arange(32) - 16
    x[0] = (k % 4) * tiny                              # amax 3 * 2^-149
    x[1] = np.where(k == 0, 63, -(k % 7)) * tiny       # amax 63 * 2^-149: 63/127 * 2^-149 rounds to 0
    x[2] = np.clip(k * 4, -64, 64) * tiny              # amax 64 * 2^-149: s = 2^-149 exactly
    x[3] = synth.normal_f32(11, 2, 0, 32)
    x[3, 5] = np.nan
    x[4] = np.nan
    x[5] = synth.normal_f32(11, 3, 0, 32)
    x[5, 7] = np.inf
    x[5, 9] = -np.inf
    a8, s, gs = orc.quantize_rows(x)
    assert np.array_equal(s[:2, 0], [0.0, 0.0]) and not a8[:2].any() and not gs[:2].any()
    assert s[2, 0] == tiny and np.array_equal(a8[2], np.clip(k * 4, -64, 64))
    # a NaN element: amax and the other codes as if it were 0, its code 0
    x3 = x[3:4].copy()
    x3[0, 5] = 0.0
    a8z, sz, _ = orc.quantize_rows(x3)
    assert s[3, 0] == sz[0, 0] and np.array_equal(a8[3], a8z[0]) and a8[3, 5] == 0
    assert s[4, 0] == 0.0 and not a8[4].any()
    # infinite amax: every finite element codes as 0 and inf / inf is NaN -> 0
    assert np.isinf(s[5, 0]) and not a8[5].any() and gs[5, 0] == 0
    assert np.array_equal(gs[:, 0], a8.astype(np.int64).sum(1))


# ----------------------------------------------------------------- C1 + C3 GEMV
def _brute_gemv(W, a8, s):
    """Exact rational y[t][o] = sum_k (d*sc*q - dmin*m) * s * a8 from the definition."""
    N, K = W["q"].shape
    T = a8.shape[0]
    d = [[Fraction(float(v)) for v in row] for row in _f16(W["d"])]
    dm = [[Fraction(float(v)) for v in row] for row in _f16(W["dmin"])]
    out = np.zeros((T, N))
    for t in range(T):
        for o in range(N):
            acc = Fraction(0)
            for k in range(K):
                b, j = k // 256, (k % 256) // 32
                w = d[o][b] * int(W["sc"][o, b, j]) * int(W["q"][o, k]) - dm[o][b] * int(W["m"][o, b, j])
                acc += w * Fraction(float(s[t, k // 32])) * int(a8[t, k])
            out[t, o] = float(acc)
    return out


@pytest.mark.parametrize("N,K,T", [(3, 256, 1), (2, 512, 5), (4, 256, 12)])
def test_gemv_vs_exact_rational_brute_force(orc, N, K, T):
    W = synth.q4k_fields(21, N * 100 + T, N, K)
    x = synth.normal_f32(21, 7, T, T * K).reshape(T, K)
    a8, s, _ = orc.quantize_rows(x)
    y = orc.qgemv(W, x)
    ref = _brute_gemv(W, a8, s)
    scale = np.abs(ref).max()
    assert np.abs(y - ref).max() <= 1e-6 * scale
    # integer partial sums are exact
    P = orc.q4k_partials(W, a8)
    for t in range(T):
        for o in range(N):
            for g in range(K // 32):
                exp = sum(int(W["q"][o, g * 32 + i]) * int(a8[t, g * 32 + i]) for i in range(32))
                assert P[t, o, g] == exp


def _family(N, K, d_bits, dmin_bits, sc, m, seed):
    rng = np.random.default_rng(seed)
    nsb = K // 256
    return {"d": np.full((N, nsb), d_bits, np.uint16), "dmin": np.full((N, nsb), dmin_bits, np.uint16),
            "sc": np.broadcast_to(np.asarray(sc, np.uint8), (N, nsb, 8)).copy() if np.ndim(sc) < 3 else sc,
            "m": np.broadcast_to(np.asarray(m, np.uint8), (N, nsb, 8)).copy() if np.ndim(m) < 3 else m,
            "q": rng.integers(0, 16, size=(N, K)).astype(np.uint8)}


def _int_rows(T, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.integers(-127, 128, size=(T, K)).astype(np.float32)
    x.reshape(T, -1, 32)[:, :, 5] = -127.0  # |x| max 127 in every group -> s = 1
    return x


def test_gemv_exact_integer_families(orc):
    N, K, T = 24, 1024, 3
    x = _int_rows(T, K, 5)
    one, zero = 0x3C00, 0x0000
    # E1: d = 1, dmin = 0, sc = 1 -> y = sum q*x
    W = _family(N, K, one, zero, 1, 0, 1)
    assert np.array_equal(orc.qgemv(W, x), (x.astype(np.int64) @ W["q"].T.astype(np.int64)).astype(np.float32))
    # E2: d = 0, dmin = 1, m = 1 -> y = -sum x
    W = _family(N, K, zero, one, 0, 1, 2)
    assert np.array_equal(orc.qgemv(W, x), np.repeat(-x.sum(1, keepdims=True), N, 1).astype(np.float32))
    # E3: random sc, m per sub-block, d = dmin = 1 -> exact int64 combination
    rng = np.random.default_rng(9)
    sc = rng.integers(0, 64, size=(N, K // 256, 8)).astype(np.uint8)
    m = rng.integers(0, 64, size=(N, K // 256, 8)).astype(np.uint8)
    W = _family(N, K, one, one, sc, m, 3)
    xi = x.astype(np.int64).reshape(T, K // 32, 32)
    qi = W["q"].astype(np.int64).reshape(N, K // 32, 32)
    P = np.einsum("tgi,ogi->tog", xi, qi)
    scg, mg = sc.reshape(N, -1).astype(np.int64), m.reshape(N, -1).astype(np.int64)
    exp = (P * scg[None]).sum(-1) - (xi.sum(-1)[:, None, :] * mg[None]).sum(-1)
    assert np.abs(exp).max() < 2 ** 24
    assert np.array_equal(orc.qgemv(W, x), exp.astype(np.float32))
    # power-of-two scaling of d and dmin scales y exactly (0x4400 = 4.0)
    W4 = dict(W, d=np.full_like(W["d"], 0x4400), dmin=np.full_like(W["dmin"], 0x4400))
    assert np.array_equal(orc.qgemv(W4, x), 4 * exp.astype(np.float32))


def test_gemv_rows_are_independent(orc):
    W = synth.q4k_fields(4, 4, 64, 768)
    x = synth.normal_f32(4, 5, 0, 6 * 768).reshape(6, 768)
    y = orc.qgemv(W, x)
    for t in range(6):
        assert np.array_equal(y[t], orc.qgemv(W, x[t:t + 1])[0])


# ----------------------------------------------------------------- C4 FFN
def test_silu_closed_forms(orc):
    z = np.linspace(-30, 30, 2001).astype(np.float32)
    one = np.ones_like(z)
    h = orc.silu_mul(z, one).astype(np.float64)
    hn = orc.silu_mul(-z, one).astype(np.float64)
    assert orc.silu_mul(np.zeros(3, np.float32), np.ones(3, np.float32)).tolist() == [0, 0, 0]
    assert np.all(np.abs(h - hn - z) <= 4 * np.spacing(np.abs(z).astype(np.float32)) + 1e-30)
    assert np.all(np.abs(h[z > 20] - z[z > 20]) <= 1e-6 * z[z > 20])
    assert np.all(np.abs(h[z < -20]) < 1e-6)


def test_ffn_vs_independent_float64_evaluation(orc):
    # C4 against the float64 numpy evaluation of its definition (see the C5
    # helpers below): SiLU on the gate, times up, then down
    H, F, T = 512, 768, 3
    Wg, Wu, Wd = (synth.q4k_fields(8, 1, F, H), synth.q4k_fields(8, 2, F, H), synth.q4k_fields(8, 3, H, F))
    x = synth.normal_f32(8, 4, 0, T * H).reshape(T, H)
    y, h = orc.ffn(Wg, Wu, Wd, x, return_h=True)
    h_ref = _np_silu_mul(_np_gemv(Wg, x), _np_gemv(Wu, x))
    assert _z6(h, h_ref) <= 1e-5
    assert _z6(y, _np_gemv(Wd, h_ref)) <= 1e-5
    # SiLU applied to up instead of the gate is far outside that bound
    assert _z6(h, _np_silu_mul(_np_gemv(Wu, x), _np_gemv(Wg, x))) > 1e-2


def test_rmsnorm_closed_form(orc):
    x = synth.normal_f32(9, 1, 0, 4 * 5120, 0.0, 3.0).reshape(4, 5120)
    a = orc.rmsnorm(x).astype(np.float64)
    ms = np.mean(x.astype(np.float64) ** 2, 1)
    assert np.allclose(np.mean(a ** 2, 1), ms / (ms + 1e-6), rtol=1e-6)
    # direction preserved
    assert np.allclose(a / np.linalg.norm(a, axis=1, keepdims=True),
                       x / np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True), atol=1e-6)


# ----------------------------------------------------------------- C5 layer glue
# An independent float64 evaluation of the layer's definition in numpy: the
# quantizer written from its definition (fp32 division, round half to even,
# clamp), weights dequantized exactly in float64, library matmuls, and every
# stage output rounded to fp32 where the definition stores fp32.
def _np_q8(x32):
    T, K = x32.shape
    g = x32.reshape(T, K // 32, 32)
    s = (np.abs(g).max(-1) / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.where(s[..., None] > 0, np.rint(g / s[..., None]), 0.0)
    c = np.clip(c, -127, 127)
    return (c * s[..., None].astype(np.float64)).reshape(T, K)


def _np_deq(W):
    nsb = W["q"].shape[1] // 256
    d = np.repeat(_f16(W["d"]), 256, 1)
    dm = np.repeat(_f16(W["dmin"]), 256, 1)
    sc = np.repeat(W["sc"].reshape(W["q"].shape[0], nsb * 8).astype(np.float64), 32, 1)
    m = np.repeat(W["m"].reshape(W["q"].shape[0], nsb * 8).astype(np.float64), 32, 1)
    return d * sc * W["q"].astype(np.float64) - dm * m


def _np_gemv(W, x32):
    return (_np_q8(x32) @ _np_deq(W).T).astype(np.float32)


def _np_rms(x32):
    x = x32.astype(np.float64)
    return (x / np.sqrt(np.mean(x * x, 1, keepdims=True) + 1e-6)).astype(np.float32)


def _np_silu_mul(g32, u32):
    g = g32.astype(np.float64)
    return (g * u32.astype(np.float64) / (1.0 + np.exp(-g))).astype(np.float32)


def _np_layer(x32, W, variant="ok"):
    add = lambda a, b: (a.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    norm = _np_rms if variant != "no_norm" else (lambda v: v)
    u = _np_gemv(W["p_in"], norm(x32))
    y1 = _np_gemv(W["p_out"], u)
    x1 = add(x32, y1) if variant != "no_residual" else y1
    if variant == "post_norm":
        x1 = _np_rms(x1)
    a2 = norm(x1)
    g, uu = _np_gemv(W["gate"], a2), _np_gemv(W["up"], a2)
    h = _np_silu_mul(g, uu) if variant != "silu_on_up" else _np_silu_mul(uu, g)
    return add(x1, _np_gemv(W["down"], h))


def _small_layer(seed, H=512, P=768, F=1024):
    shp = {"p_in": (P, H), "p_out": (H, P), "gate": (F, H), "up": (F, H), "down": (H, F)}
    return {m: synth.q4k_fields(seed, 300 + i, *shp[m]) for i, m in enumerate(shp)}


def _zero_scales(W):
    return dict(W, d=np.zeros_like(W["d"]), dmin=np.zeros_like(W["dmin"]))


def test_layer_identity_when_output_projections_are_zero(orc):
    # P_out and W_down with d = dmin = 0 add exactly zero: the residual passes through bit for bit
    W = _small_layer(31)
    W["p_out"], W["down"] = _zero_scales(W["p_out"]), _zero_scales(W["down"])
    x = synth.normal_f32(31, 1, 0, 4 * 512, 0.0, 3.0).reshape(4, 512)
    assert np.array_equal(orc.layer(x, W), x)


def _z6(y, ref):
    y, ref = np.asarray(y, np.float64), np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1e-2 * rms)))


def test_layer_vs_independent_float64_evaluation(orc):
    W = _small_layer(32)
    x = synth.normal_f32(32, 2, 0, 3 * 512).reshape(3, 512)
    got = orc.layer(x, W)
    assert _z6(got, _np_layer(x, W)) <= 1e-5
    # each plausible mistake in the glue moves the layer far outside that bound
    # (a dropped residual is caught by the identity pin above: with N(0, 1)
    # rows the blocks' outputs are ~1e6 times larger than the residual here)
    for bad in ("post_norm", "no_norm", "silu_on_up"):
        assert _z6(got, _np_layer(x, W, bad)) > 1e-2, bad


# ----------------------------------------------------------------- C8 step composition
def test_decode_step_composition_with_planted_drafts(orc):
    H, P, F, V, L, T = 256, 512, 512, 300, 2, 6
    gs = [0, 3, 6]
    shp = {"p_in": (P, H), "p_out": (H, P), "gate": (F, H), "up": (F, H), "down": (H, F)}
    layers = [{m: synth.q4k_fields(33, 400 + 8 * l + i, *shp[m]) for i, m in enumerate(shp)} for l in range(L)]
    W16 = synth.normal_f16(33, 500, 0, V * H, 0.0, 0.02).reshape(V, H)
    x = synth.normal_f32(33, 501, 0, T * H).reshape(T, H)
    nh, d = 3, 16
    gdn = dict(synth.gdn_step_inputs(33, 502, T, nh, d, d))
    gdn["S"] = [synth.normal_f32(33, 503 + a, 0, nh * d * d, 0.0, 0.01).reshape(nh, d, d) for a in range(2)]
    # the argmax does not depend on the drafts: read it once, then plant drafts
    am = orc.decode_step(x, layers, W16, gs, np.zeros(4, np.int32))["argmax"]
    drafts = np.array([am[0], am[1], am[3], (am[4] + 1) % V], np.int32)  # agent 0: both; agent 1: first only
    out = orc.decode_step(x, layers, W16, gs, drafts, gdn=gdn)
    # layers: the independent float64 evaluation, layer after layer
    ref = x
    for l in range(L):
        ref = _np_layer(ref, layers[l])
        assert _z6(out["trace"][l], ref) <= 1e-5
    # lm_head input is the final RMSNorm; the argmax is numpy's float64 argmax
    logits = _np_rms(out["trace"][-1]).astype(np.float64) @ _f16(W16).T
    assert np.array_equal(out["argmax"], np.argmax(logits, 1))
    assert list(out["n_acc"]) == [2, 1]
    assert list(out["tokens"]) == [am[0], am[1], am[2], am[3], am[4], -1]
    # each agent's state absorbs exactly its rows 0..n_acc; outputs follow every row
    for a, (r0, r1) in enumerate(((0, 3), (3, 6))):
        for h in range(nh):
            R = gdn["S"][a][h].astype(np.float64)
            for t in range(r0, r1):
                R = _full_matrix_update(R, gdn["k"][t, h], gdn["v"][t, h], float(gdn["g"][t, h]),
                                        float(gdn["beta"][t, h]))
                assert np.allclose(out["gdn_o"][t, h], R.T @ gdn["q"][t, h].astype(np.float64), rtol=1e-5, atol=1e-7)
                if t - r0 == out["n_acc"][a]:
                    assert np.allclose(out["S"][a][h], R, rtol=1e-6, atol=1e-9)


# ----------------------------------------------------------------- C6 lm_head + verify
def test_lmhead_vs_numpy_and_planted_cases(orc):
    V, H, T = 1500, 384, 5
    W = synth.normal_f16(3, 50, 0, V * H, 0.0, 0.02).reshape(V, H)
    hid = synth.normal_f32(3, 51, 0, T * H).reshape(T, H)
    r = orc.lmhead(W, hid, return_logits=True)
    ref = hid.astype(np.float64) @ _f16(W).T  # library matmul in float64
    assert np.allclose(r["logits"], ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["top1"], np.argmax(ref, 1))
    # planted maximum: row 977 points along hid[2]
    W2 = W.copy()
    W2[977] = np.sign(hid[2]).astype(np.float16).view(np.uint16)
    assert orc.lmhead(W2, hid)["top1"][2] == 977
    # planted exact tie: rows 311 and 1200 identical and maximal for row 0 -> lowest index
    W3 = W.copy()
    W3[311] = np.sign(hid[0]).astype(np.float16).view(np.uint16)
    W3[1200] = W3[311]
    r3 = orc.lmhead(W3, hid)
    assert r3["top1"][0] == 311 and r3["top2"][0] == 1200 and r3["top1_val"][0] == r3["top2_val"][0]
    # NaN never wins
    W4 = W3.copy()
    W4[5] = 0x7E00
    assert orc.lmhead(W4, hid)["top1"][0] == 311


def test_all_nan_row_has_no_argmax_and_accepts_nothing(orc):
    # A hidden row of NaN makes every logit NaN (numpy agrees); NaN never wins,
    # so the row has no argmax (-1), and -1 matches no draft, not even a draft
    # of -1 (an id outside [0, V) is a mismatch).
    V, H = 40, 64
    W = synth.normal_f16(3, 70, 0, V * H, 0.0, 0.02).reshape(V, H)
    hid = synth.normal_f32(3, 71, 0, 3 * H).reshape(3, H)
    hid[1] = np.nan
    logits = hid.astype(np.float64) @ _f16(W).T
    assert np.isnan(logits[1]).all()
    r = orc.lmhead(W, hid)
    assert r["top1"][1] == -1
    assert r["top1"][0] == np.argmax(logits[0]) and r["top1"][2] == np.argmax(logits[2])
    # worked examples: (argmax, drafts) -> (n_acc, tokens)
    cases = [([5, -1, 7], [5, -1], 1, [5, -1, -1]),
             ([-1, 4], [-1], 0, [-1, -1]),
             ([2, 3, -1], [2, 3], 2, [2, 3, -1])]
    for am, dr, n_exp, tok_exp in cases:
        n_acc, tok = orc.verify(np.array(am, np.int32), [0, len(am)], np.array(dr, np.int32))
        assert n_acc[0] == n_exp and list(tok) == tok_exp, (am, dr)


def test_verify_exhaustive_match_patterns(orc):
    for n in range(1, 7):
        for pat in range(1 << (n - 1)):
            argmax = np.arange(100, 100 + n, dtype=np.int32)
            drafts = np.array([argmax[i] if (pat >> i) & 1 else 7 for i in range(n - 1)], np.int32)
            n_acc, tok = orc.verify(argmax, [0, n], drafts)
            lead = 0
            while lead < n - 1 and (pat >> lead) & 1:
                lead += 1
            assert n_acc[0] == lead
            assert list(tok[:lead + 1]) == list(drafts[:lead]) + [argmax[lead]]


def test_verify_groups_and_drafter_statistics(orc):
    # 4 groups of 3 rows (4 agents x [token + 2 drafts])
    argmax = np.arange(12, dtype=np.int32) * 3
    gs = [0, 3, 6, 9, 12]
    drafts = np.array([0, 3, 9, 99, 18, 21, 27, 30], np.int32)  # g0: 2 ok; g1: 1; g2: 2; g3: 2
    n_acc, tok = orc.verify(argmax, gs, drafts)
    assert list(n_acc) == [2, 1, 2, 2]
    assert list(tok[:3]) == [0, 3, 6] and list(tok[3:5]) == [9, 12]
    # drafter of the lm_head workload: P(n_acc = k) = .7^k .3 (k < 4), .7^4 (k = 4); mean 1.7731
    trials = 3000
    counts = np.zeros(5)
    for tr in range(trials):
        am = synth.uniform_i32(3, 77, tr, 5, 0, 151935)
        dr = recipes.drafts_from_argmax(am[:4], 151936, trial=tr)
        counts[orc.verify(am, [0, 5], dr)[0][0]] += 1
    p = np.array([0.3, 0.21, 0.147, 0.1029, 0.2401])
    chi2 = ((counts - trials * p) ** 2 / (trials * p)).sum()
    assert chi2 < 18.5  # 4 dof, p = 0.001
    assert abs((counts * np.arange(5)).sum() / trials - 1.7731) < 0.08


# ----------------------------------------------------------------- C7 Gated DeltaNet
def _full_matrix_update(S, k, v, g, b):
    k = k.astype(np.float64)
    v = v.astype(np.float64)
    A = np.eye(len(k)) - b * np.outer(k, k)
    return g * (A @ S) + b * np.outer(k, v)


@pytest.mark.parametrize("d", [2, 4, 8, 128])
def test_gdn_rank1_vs_full_matrix(orc, d):
    inp = synth.gdn_step_inputs(4, 900 + d, 6, 1, d, d)
    S0 = synth.normal_f32(4, 901, d, d * d, 0.0, 0.01).reshape(d, d).astype(np.float64)
    S = S0.copy()
    o = orc.gdn_rows(S, inp["q"][:, 0], inp["k"][:, 0], inp["v"][:, 0], inp["g"][:, 0], inp["beta"][:, 0])
    R = S0.copy()
    for t in range(6):
        R = _full_matrix_update(R, inp["k"][t, 0], inp["v"][t, 0], float(inp["g"][t, 0]), float(inp["beta"][t, 0]))
        assert np.allclose(o[t], (R.T @ inp["q"][t, 0].astype(np.float64)).astype(np.float32), rtol=1e-5,
                           atol=1e-7)
    assert np.allclose(S, R, rtol=1e-12, atol=1e-14)


def test_gdn_closed_forms(orc):
    d = 16
    rng = np.random.default_rng(2)
    S0 = rng.standard_normal((d, d))
    ks = rng.standard_normal((5, d)).astype(np.float32)
    vs = rng.standard_normal((5, d)).astype(np.float32)
    gs = np.array([0.9, 0.5, 0.75, 0.8, 0.95], np.float32)
    # beta = 0: pure decay
    S = S0.copy()
    orc.gdn_rows(S, None, ks, vs, gs, np.zeros(5, np.float32))
    assert np.allclose(S, np.prod(gs.astype(np.float64)) * S0, rtol=1e-12)
    # g = beta = 1 with a unit key: retrieval S^T k = v after the update
    k = ks[0] / np.linalg.norm(ks[0])
    S = S0.copy()
    orc.gdn_rows(S, None, k[None].astype(np.float32), vs[:1], np.ones(1, np.float32), np.ones(1, np.float32))
    kk = k.astype(np.float32).astype(np.float64)
    # k is fp32-rounded, so |k| = 1 only to ~1e-7
    assert np.allclose(S.T @ kk, vs[0], atol=1e-6)
    # the printed right-multiplied form does not retrieve v
    S = S0.copy()
    orc.gdn_rows(S, None, k[None].astype(np.float32), vs[:1], np.ones(1, np.float32), np.ones(1, np.float32),
                 literal=True)
    assert not np.allclose(S.T @ kk, vs[0], atol=1e-3)
    # orthonormal keys, g = beta = 1: S = (I - sum k k^T) S0 + sum k v^T
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    K4 = Q[:, :4].T.astype(np.float32)
    S = S0.copy()
    orc.gdn_rows(S, None, K4, vs[:4], np.ones(4, np.float32), np.ones(4, np.float32))
    Kd = K4.astype(np.float64)
    exp = (np.eye(d) - Kd.T @ Kd) @ S0 + Kd.T @ vs[:4].astype(np.float64)
    assert np.allclose(S, exp, atol=1e-5)


def test_gdn_step_commits_through_accepted_row(orc):
    nh, d, T = 3, 32, 5
    S0 = synth.normal_f32(4, 950, 0, nh * d * d, 0.0, 0.01).reshape(nh, d, d)
    inp = synth.gdn_step_inputs(4, 951, T, nh, d, d)
    for a in range(T):
        S1, o = orc.gdn_step(S0, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], a)
        for h in range(nh):
            R = S0[h].astype(np.float64)
            for t in range(a + 1):
                R = _full_matrix_update(R, inp["k"][t, h], inp["v"][t, h], float(inp["g"][t, h]),
                                        float(inp["beta"][t, h]))
            assert np.allclose(S1[h], R.astype(np.float32), rtol=1e-6, atol=1e-9)
        # outputs do not depend on the accept length
        _, o0 = orc.gdn_step(S0, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], 0)
        assert np.array_equal(o, o0)


def test_gdn_chain_equivalence_and_contraction(orc):
    nh, d, T = 2, 16, 4
    S = synth.normal_f32(4, 960, 0, nh * d * d, 0.0, 0.01).reshape(nh, d, d)
    S_one = S.copy()
    for step in range(20):
        inp = synth.gdn_step_inputs(4, 961 + step, T, nh, d, d)
        S, o = orc.gdn_step(S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], T - 1)
        for t in range(T):
            S_one, o1 = orc.gdn_step(S_one, inp["q"][t:t + 1], inp["k"][t:t + 1], inp["v"][t:t + 1],
                                     inp["g"][t:t + 1], inp["beta"][t:t + 1], 0)
            assert np.allclose(o1[0], o[t], rtol=1e-5, atol=1e-6)
        assert np.allclose(S, S_one, rtol=1e-5, atol=1e-7)
    # g < 1, beta in (0, 1), unit keys: the state stays bounded
    assert np.abs(S).max() < 10.0


# ----------------------------------------------------------------- byte accounting
def test_stack_bytes_match_the_pages_arithmetic():
    import json
    import os
    fig = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
    shapes = recipes.stack_shapes()
    per_layer = sum(n * k // 256 * 144 for n, k in shapes.values())
    assert per_layer == 209_387_520
    assert per_layer * fig["layers_total"]["value"] == 13_400_801_280
    # the page's own arithmetic: ~17 GB at 936 GB/s is about 18 ms
    ms = fig["weights_per_step_gb"]["value"] / fig["rtx3090_bandwidth_gb_s"]["value"] * 1e3
    assert abs(ms - fig["weight_read_ms"]["value"]) < 0.5
    assert len(recipes.gdn_layers()) == fig["layers_gdn"]["value"]


# ----------------------------------------------------------------- A1 attention
def _attn_small(ctx, sizes, Hq=4, Hkv=2, d=8, gate=True, fill=recipes.F16_NAN):
    return recipes.attn_inputs(ctx, sizes, Hq=Hq, Hkv=Hkv, d=d, gate=gate, fill=fill, seed=11)


def _run_attn(orc, a):
    return orc.attn_decode(a["q"], a["gate"], a["k"], a["v"], a["ctx"], a["group_start"])


def test_attn_brute_force_decimal(orc):
    """A1 against a 50-digit decimal evaluation of softmax(q K^T / sqrt(d)) V
    with the output gate, on two agents of unequal context and group size
    (every fp16 and fp32 input converts to Decimal exactly)."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    a = _attn_small([5, 0], [2, 3])
    o = _run_attn(orc, a)
    q, gt, K, V, ctx, gs = a["q"], a["gate"], a["k"], a["v"], a["ctx"], a["group_start"]
    T, Hq, d = q.shape
    Hkv = K.shape[1]
    Kf = _f16(K)
    Vf = _f16(V)
    sd = Decimal(d).sqrt()
    worst = 0.0
    for g in range(len(ctx)):
        for i in range(gs[g + 1] - gs[g]):
            t = gs[g] + i
            for hq in range(Hq):
                h = hq // (Hq // Hkv)
                n = ctx[g] + i + 1
                s = [sum(Decimal(float(q[t, hq, k])) * Decimal(float(Kf[g, h, j, k])) for k in range(d)) / sd
                     for j in range(n)]
                m = max(s)
                w = [(x - m).exp() for x in s]
                den = sum(w)
                for k in range(d):
                    y = sum(w[j] * Decimal(float(Vf[g, h, k, j])) for j in range(n)) / den
                    y = y / (1 + (-Decimal(float(gt[t, hq, k]))).exp())
                    worst = max(worst, abs(float(y) - float(o[t, hq, k])) / max(abs(float(y)), 1e-30))
    assert worst < 1e-6, worst


def test_attn_equal_keys_give_the_mean_of_visible_values(orc):
    """A1 closed form: when every key of a head is the same vector, all
    visible positions weigh the same, so row i of a group returns the plain
    mean of V over positions 0..ctx+i (no gate)."""
    a = _attn_small([7, 3], [3, 2], gate=False)
    a["k"][:] = a["k"][:, :, :1, :]  # position 0's key everywhere (also the unused slots)
    o = _run_attn(orc, a)
    Vf = _f16(a["v"])
    for g in range(2):
        for i in range(a["group_start"][g + 1] - a["group_start"][g]):
            n = a["ctx"][g] + i + 1
            t = a["group_start"][g] + i
            for hq in range(4):
                ref = Vf[g, hq // 2, :, :n].mean(axis=1)
                np.testing.assert_allclose(o[t, hq], ref, rtol=1e-6, atol=1e-7)


def test_attn_causal_bound_is_inclusive_of_own_row_only(orc):
    """A1 causal mask: a key planted at position ctx+i dominates row i of the
    group, while the same key at position ctx+i+1 (the group's next row) is
    invisible to row i."""
    d = 8
    for offset, visible in ((0, True), (1, False)):
        a = _attn_small([4, 9], [3, 3], d=d, gate=False)
        a["k"][:] = 0
        a["q"][:] = 0
        a["q"][:, :, 0] = 1.0
        t, g, i = 4, 1, 1  # group 1, row 1
        p = a["ctx"][g] + i + offset
        a["k"][g, :, p, 0] = synth.f64_to_f16_bits(64.0)
        o = _run_attn(orc, a)
        Vf = _f16(a["v"])
        n = a["ctx"][g] + i + 1
        for hq in range(4):
            h = hq // 2
            if visible:
                np.testing.assert_allclose(o[t, hq], Vf[g, h, :, p], rtol=1e-6, atol=1e-6)
            else:
                np.testing.assert_allclose(o[t, hq], Vf[g, h, :, :n].mean(axis=1), rtol=1e-6, atol=1e-7)


def test_attn_query_heads_share_kv_heads_in_groups(orc):
    """A1 grouped queries: query head hq reads KV head hq // (Hq / Hkv).  With
    V of KV head h equal to h + 1 everywhere the output is exactly that."""
    a = _attn_small([6], [2], Hq=8, Hkv=2, gate=False)
    for h in range(2):
        a["v"][:, h] = synth.f64_to_f16_bits(h + 1.0)
    o = _run_attn(orc, a)
    for hq in range(8):
        assert np.all(o[:, hq] == hq // 4 + 1.0)


def test_attn_value_cache_is_dimension_major(orc):
    """A1 layout: V [G][Hkv][d][cap].  With V[..][k][j] = k the output is k
    for every row and head."""
    a = _attn_small([10, 2], [2, 1], gate=False)
    for k in range(8):
        a["v"][:, :, k, :] = synth.f64_to_f16_bits(float(k))
    o = _run_attn(orc, a)
    assert np.all(o == np.arange(8, dtype=np.float32)[None, None, :])


def test_attn_zero_gate_halves_the_output(orc):
    """A1 gate: sigmoid(0) = 1/2, so a zero gate halves the ungated output
    exactly."""
    a = _attn_small([5, 1], [2, 2], gate=False)
    o0 = _run_attn(orc, a)
    a["gate"] = np.zeros_like(a["q"])
    o1 = _run_attn(orc, a)
    assert np.array_equal(o1, o0 * np.float32(0.5))


def test_attn_ignores_slots_past_the_last_position(orc):
    """A1 reads nothing past position ctx+n-1: NaN-filled and zero-filled
    unused slots give the same result."""
    a = _attn_small([3, 8], [3, 2], fill=recipes.F16_NAN)
    b = _attn_small([3, 8], [3, 2], fill=0)
    assert np.array_equal(_run_attn(orc, a), _run_attn(orc, b))
    assert np.isfinite(_run_attn(orc, a)).all()


def test_attn_large_scores_stay_finite(orc):
    """A1 is shift invariant: scores of about 2e6 (where exp alone overflows)
    still give the closed-form mean when all keys are equal."""
    a = _attn_small([5, 2], [2, 2], gate=False)
    a["k"][:] = 0
    a["k"][:, :, :, 0] = synth.f64_to_f16_bits(60000.0)
    a["q"][:] = 0
    a["q"][:, :, 0] = 100.0
    o = _run_attn(orc, a)
    Vf = _f16(a["v"])
    for g in range(2):
        for i in range(2):
            n = a["ctx"][g] + i + 1
            t = a["group_start"][g] + i
            for hq in range(4):
                np.testing.assert_allclose(o[t, hq], Vf[g, hq // 2, :, :n].mean(axis=1), rtol=1e-6, atol=1e-7)


def test_attn_q8_equals_fp16_path_on_exact_values(orc):
    """A2 against the pinned A1: with power-of-two scales every scale * code is
    an exact fp16 value, so the q8_0 result must equal, bit for bit, the fp16
    result on the dequantized caches.  Scales differ per (position, 32-dim
    block) for K and per (32-position block, dimension) for V, which pins
    which values each scale multiplies."""
    a = recipes.attn_inputs_q8([45, 7], [2, 3], Hq=4, Hkv=2, d=64, gate=True, seed=13)  # V codes tile-major
    G, Hkv, cap, d = a["k8"].shape
    e_k = synth.uniform_i32(13, 1, 0, G * Hkv * cap * (d // 32), -4, 3).reshape(G, Hkv, cap, d // 32)
    e_v = synth.uniform_i32(13, 2, 0, G * Hkv * (cap // 32) * d, -4, 3).reshape(G, Hkv, cap // 32, d)
    a["ks"] = np.vectorize(lambda e: synth.f64_to_f16_bits(2.0 ** e))(e_k).astype(np.uint16)
    a["vs"] = np.vectorize(lambda e: synth.f64_to_f16_bits(2.0 ** e))(e_v).astype(np.uint16)
    k8 = a["k8"].astype(np.float64)
    v8 = a["v8"].transpose(0, 1, 3, 2, 4).reshape(G, Hkv, d, cap).astype(np.float64)  # back to [d][cap]
    kval = k8 * np.repeat(2.0 ** e_k, 32, axis=3)
    vval = v8 * np.transpose(np.repeat(2.0 ** e_v, 32, axis=2), (0, 1, 3, 2))
    to16 = np.vectorize(synth.f64_to_f16_bits)
    k16 = to16(kval).astype(np.uint16)
    v16 = to16(vval).astype(np.uint16)
    assert np.array_equal(_f16(k16), kval) and np.array_equal(_f16(v16), vval)
    o8 = orc.attn_decode_q8(a["q"], a["gate"], a["k8"], a["ks"], a["v8"], a["vs"], a["ctx"], a["group_start"])
    o16 = orc.attn_decode(a["q"], a["gate"], k16, v16, a["ctx"], a["group_start"])
    assert np.array_equal(o8, o16)


# ----------------------------------------------------------------- F1-F3 sampling-mode verification
def test_topk_rows_vs_brute_force_with_ties_and_nan(orc):
    rng = np.random.default_rng(40)
    lg = np.round(rng.standard_normal((4, 300)) * 3, 1)  # rounding plants many exact ties
    lg[1, 17] = np.nan
    lg[1, 200] = np.nan
    lg[2, :] = 0.0  # every logit tied
    for k in (1, 5, 32):
        idx, val = orc.topk_rows(lg, k)
        for t in range(4):
            cand = [v for v in range(300) if not np.isnan(lg[t, v])]
            best = sorted(cand, key=lambda v: (-lg[t, v], v))[:k]
            assert list(idx[t]) == sorted(best)
            assert np.array_equal(val[t], lg[t, sorted(best)])
    assert list(orc.topk_rows(lg, 3)[0][2]) == [0, 1, 2]  # all tied: lowest indices
    # a row with fewer non-NaN logits than k is padded; an all-NaN row has no candidate
    lg2 = np.full((2, 10), np.nan)
    lg2[0, [3, 7]] = [1.0, 2.0]
    idx, val = orc.topk_rows(lg2, 4)
    assert list(idx[0]) == [3, 7, -1, -1] and list(idx[1]) == [-1] * 4
    assert np.isneginf(val[1]).all()
    n, tok, _ = orc.sample_verify(idx, val, [0, 1, 2], [], 0.6, np.zeros(2), np.full(2, 0.99))
    assert list(tok) == [7, -1] and list(n) == [0, 0]
    n, tok, _ = orc.sample_verify(idx[::-1].copy(), val[::-1].copy(), [0, 2], [3], 0.6, np.zeros(2), np.zeros(2))
    assert list(tok) == [-1, -1] and n[0] == 0  # the all-NaN row accepts nothing and emits nothing


def _row(seed, k=6):
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(1000, size=k, replace=False)).astype(np.int32)
    val = rng.standard_normal(k) * 2.0
    return idx, val


def test_sample_verify_keeps_the_target_distribution_exactly(orc):
    # One row with a draft: integrate over u_acc and u_samp.  P(emit d) =
    # p(d); for x != d, P(emit x) = (1 - p(d)) * (length of the u_samp
    # interval that picks x with d removed); that must equal p(x).
    idx, val = _row(41)
    tau = 0.6
    w = orc.sample_weights(val, tau)
    p = w / w.sum()
    grid = (np.arange(40000) + 0.5) / 40000
    for d in (int(idx[np.argmax(p)]), int(idx[np.argmin(p)]), 999999, -3):
        j = np.flatnonzero(idx == d)
        pd = p[j[0]] if len(j) else 0.0
        picks = np.zeros(len(idx))
        for u in grid:
            picks[orc._inverse_cdf(w, u, skip=j[0] if len(j) else None)[0]] += 1
        emit = (1 - pd) * picks / len(grid)
        if len(j):
            assert picks[j[0]] == 0
            emit[j[0]] += pd
        assert np.abs(emit - p).max() < 1e-4, d
        # the decision itself: accept exactly when u_acc < p(d)
        for ua in (0.0, pd * 0.999, pd, min(pd * 1.001 + 1e-9, 0.999)):
            n, tok, _ = orc.sample_verify(idx[None].repeat(2, 0), val[None].repeat(2, 0), [0, 2], [d], tau,
                                          np.array([ua, 0.5]), np.array([0.3, 0.3]))
            assert (n[0] == 1) == (ua < pd)


def test_sample_verify_chi_square_over_a_group(orc):
    # T = 3 rows, 2 drafts from a proposal that differs from the target; the
    # first emitted token follows p_0, and the second (when d_0 was accepted)
    # follows p_1.  A sampler that does not remove the rejected draft fails.
    rows = [_row(50 + i, k=8) for i in range(3)]
    idx = np.stack([r[0] for r in rows])
    val = np.stack([r[1] for r in rows])
    tau = 0.6
    p = [orc.sample_weights(val[i], tau) / orc.sample_weights(val[i], tau).sum() for i in range(3)]
    rng = np.random.default_rng(51)
    trials = 6000
    first, second = {}, {}
    n_first_acc = 0
    bad_first = {}
    for tr in range(trials):
        # drafts: the most likely token of the row with probability 0.5, else a uniform candidate
        dr = [int(idx[i][np.argmax(p[i])]) if rng.random() < 0.5 else int(rng.choice(idx[i])) for i in range(2)]
        ua, us = rng.random(3), rng.random(3)
        n, tok, _ = orc.sample_verify(idx, val, [0, 3], dr, tau, ua, us)
        first[tok[0]] = first.get(tok[0], 0) + 1
        if n[0] >= 1:
            n_first_acc += 1
            second[tok[1]] = second.get(tok[1], 0) + 1
        # planted mistake: on rejection sample p without removing the draft
        pd = p[0][list(idx[0]).index(dr[0])]
        if ua[0] < pd:
            b = dr[0]
        else:
            b = int(idx[0][orc._inverse_cdf(orc.sample_weights(val[0], tau), us[0])[0]])
        bad_first[b] = bad_first.get(b, 0) + 1

    def chi2(counts, i, n):
        obs = np.array([counts.get(int(v), 0) for v in idx[i]], np.float64)
        return float((((obs - n * p[i]) ** 2) / (n * p[i])).sum())

    crit = 24.3  # 7 dof, p = 0.001
    assert chi2(first, 0, trials) < crit
    assert chi2(second, 1, n_first_acc) < crit
    assert chi2(bad_first, 0, trials) > 3 * crit


def test_sample_verify_reduces_to_greedy(orc):
    # top_k = 1, or a temperature near 0, makes every target one-hot on the
    # argmax: the outcome is exactly the greedy verification (C6)
    rng = np.random.default_rng(52)
    lg = rng.standard_normal((6, 400)) * 3
    am = np.argmax(lg, 1).astype(np.int32)
    gs = [0, 3, 6]
    drafts = np.array([am[0], am[1], am[3], (am[4] + 1) % 400], np.int32)
    n_ref, t_ref = orc.verify(am, gs, drafts)
    for k, tau in ((1, 0.6), (32, 1e-4)):
        idx, val = orc.topk_rows(lg, k)
        for trial in range(20):
            n, tok, _ = orc.sample_verify(idx, val, gs, drafts, tau, rng.random(6), rng.random(6))
            assert np.array_equal(n, n_ref) and np.array_equal(tok, t_ref), (k, tau)


# ----------------------------------------------------------------- M1-M2 MTP draft loop
def _small_mtp(seed, H=256, F=512):
    return {"fc": synth.q4k_fields(seed, 600, H, 2 * H), "gate": synth.q4k_fields(seed, 601, F, H),
            "up": synth.q4k_fields(seed, 602, F, H), "down": synth.q4k_fields(seed, 603, H, F)}


def _np_mtp_block(m, E16, toks, h32, variant="ok"):
    V, H = E16.shape
    e = np.zeros((len(toks), H), np.float32)
    for i, t in enumerate(toks):
        if 0 <= t < V:
            e[i] = _f16(E16[t]).astype(np.float32)
    hn = _np_rms(h32) if variant != "no_hnorm" else h32
    z = np.concatenate([_np_rms(e), hn] if variant != "swapped" else [hn, _np_rms(e)], axis=1)
    u = _np_gemv(m["fc"], z)
    a = _np_rms(u)
    y = _np_gemv(m["down"], _np_silu_mul(_np_gemv(m["gate"], a), _np_gemv(m["up"], a)))
    if variant == "no_residual":
        return y
    return (u.astype(np.float64) + y.astype(np.float64)).astype(np.float32)


def test_mtp_block_vs_independent_float64_evaluation(orc):
    H, V = 256, 300
    m = _small_mtp(70)
    E16 = synth.normal_f16(70, 604, 0, V * H, 0.0, 0.02).reshape(V, H)
    h = synth.normal_f32(70, 605, 0, 4 * H, 0.0, 3.0).reshape(4, H)
    toks = [5, 299, -1, 300]  # the last two contribute zero embeddings
    got = orc.mtp_block(m, E16, toks, h)
    assert _z6(got, _np_mtp_block(m, E16, toks, h)) <= 1e-5
    for bad in ("swapped", "no_hnorm"):
        assert _z6(got, _np_mtp_block(m, E16, toks, h, bad)) > 1e-2, bad
    # with W_down at d = dmin = 0 the block is u itself, so a dropped residual is caught
    m0 = dict(m, down=_zero_scales(m["down"]))
    got0 = orc.mtp_block(m0, E16, toks, h)
    assert _z6(got0, _np_mtp_block(m0, E16, toks, h)) <= 1e-5
    assert np.abs(got0).max() > 0 and np.abs(_np_mtp_block(m0, E16, toks, h, "no_residual")).max() == 0


def test_mtp_draft_catch_up_rows_chain_and_vocabulary(orc):
    H, V, Vd, T, nd = 256, 500, 200, 6, 3
    m = _small_mtp(71)
    E16 = synth.normal_f16(71, 606, 0, V * H, 0.0, 0.02).reshape(V, H)
    hidden = synth.normal_f32(71, 607, 0, T * H, 0.0, 2.0).reshape(T, H)
    gs = [0, 3, 6]
    tokens = np.array([11, 250, -1, 40, 41, 499], np.int32)
    n_acc = [1, 2]
    out = orc.mtp_draft(m, E16, Vd, hidden, tokens, gs, n_acc, nd)
    d = out["drafts"]
    assert d.shape == (nd, 2) and (d >= 0).all() and (d < Vd).all()
    assert sorted(out["catchup"]) == [0, 1, 3, 4, 5]  # rows 0..n_acc of each group
    # catch-up rows and the chain against the independent evaluation; each draft is
    # numpy's float64 argmax over the draft-vocabulary prefix
    for g, rows in enumerate(([0, 1], [3, 4, 5])):
        ref = _np_mtp_block(m, E16, [tokens[r] for r in rows], hidden[rows])
        for j, r in enumerate(rows):
            assert _z6(out["catchup"][r], ref[j]) <= 1e-5
        prev = ref[-1]
        for k in range(nd):
            if k:
                prev = _np_mtp_block(m, E16, [d[k - 1, g]], prev[None])[0]
            assert _z6(out["chain"][k, g], prev) <= 1e-5
            lg = _np_rms(out["chain"][k, g][None]).astype(np.float64) @ _f16(E16[:Vd]).T
            assert d[k, g] == np.argmax(lg[0])
    # rows after n_acc (drafts that were rejected) do not matter; row n_acc does
    t2, h2 = tokens.copy(), hidden.copy()
    t2[2], h2[2] = 7, 0.0
    assert np.array_equal(orc.mtp_draft(m, E16, Vd, h2, t2, gs, n_acc, nd)["drafts"], d)
    t3 = tokens.copy()
    t3[1] = 12
    assert not np.array_equal(orc.mtp_draft(m, E16, Vd, hidden, t3, gs, n_acc, nd)["chain"][0, 0],
                              out["chain"][0, 0])


def test_mtp_draft_of_an_all_zero_head_is_token_zero(orc):
    # fc and W_down at zero: x' = 0, RMSNorm(0) = 0, every logit is 0 and the
    # tie goes to the lowest index at every draft step
    H, V = 256, 300
    m = _small_mtp(72)
    m["fc"], m["down"] = _zero_scales(m["fc"]), _zero_scales(m["down"])
    E16 = synth.normal_f16(72, 606, 0, V * H, 0.0, 0.02).reshape(V, H)
    hidden = synth.normal_f32(72, 607, 0, 2 * H).reshape(2, H)
    out = orc.mtp_draft(m, E16, 100, hidden, [3, 4], [0, 2], [1], 3)
    assert (out["drafts"] == 0).all() and (out["chain"] == 0).all()
