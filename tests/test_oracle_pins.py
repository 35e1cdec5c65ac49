"""Pins for the CPU oracle: each check ties an oracle function to something other
than its own formula -- a library routine, a closed form, an invariant, a
special case, or brute force on a tiny model written as scalar loops."""

import math

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle as orc
from synth_inputs import TINY, make_prompt, make_weights

# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------


def test_bf16_widen_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    got = orc.bf16_to_f32(bits)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, math.inf, -math.inf, 0.0, -0.0, 3.140625]
    for g, w in zip(got, want):
        assert g == np.float32(w)
    assert np.signbit(got[7])


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        (rng.standard_normal(10000) * 1e-39).astype(np.float32),            # subnormals
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),      # exact ties
                  3.3895e38, 3.4e38, np.finfo(np.float32).max, -np.finfo(np.float32).max,
                  np.inf, -np.inf, 0.0, -0.0, 2 ** -149], dtype=np.float32),
    ])
    got = orc.f32_to_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_bf16_ties_to_even_and_overflow():
    # 1 + 2^-8 lies halfway between bf16 1.0 (0x3F80) and 1.0078125 (0x3F81): even wins.
    assert orc.f32_to_bf16(np.array([1.0 + 2 ** -8], np.float32))[0] == 0x3F80
    assert orc.f32_to_bf16(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 0x3F82
    assert orc.f32_to_bf16(np.array([np.finfo(np.float32).max], np.float32))[0] == 0x7F80
    nan = orc.f32_to_bf16(np.array([np.nan], np.float32))[0]
    assert (int(nan) & 0x7F80) == 0x7F80 and (int(nan) & 0x7F) != 0


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------


def test_rmsnorm_unit_rms_before_gain():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(2048) * 3.7
    y = orc.rmsnorm(x, np.ones(2048), 1e-5)
    rms = math.sqrt(float(np.mean(y * y)))
    # exact value: sqrt(m / (m + eps)) with m = mean(x^2)
    m = float(np.mean(x * x))
    assert abs(rms - math.sqrt(m / (m + 1e-5))) < 1e-12
    assert abs(rms - 1.0) < 1e-6


def test_rmsnorm_scale_invariance_and_gain():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(256)
    g = rng.uniform(0.5, 1.5, 256)
    a = orc.rmsnorm(x, g, 0.0)
    b = orc.rmsnorm(17.0 * x, g, 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    # constant vector c: closed form c / sqrt(c^2 + eps) * g
    c = 0.01
    y = orc.rmsnorm(np.full(8, c), np.full(8, 2.0), 1e-5)
    np.testing.assert_allclose(y, 2.0 * c / math.sqrt(c * c + 1e-5), rtol=1e-12)
    assert np.all(orc.rmsnorm(np.zeros(8), np.ones(8), 1e-5) == 0)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------


def test_rope_two_dims_closed_form():
    # d_h = 2: one pair with frequency theta^0 = 1, so the angle is the position.
    for p in (0, 1, 7, 1000):
        y = orc.apply_rope(np.array([[1.0, 0.0]]), p, 500000.0)[0]
        np.testing.assert_allclose(y, [math.cos(p), math.sin(p)], atol=1e-12)
        y = orc.apply_rope(np.array([[0.0, 1.0]]), p, 500000.0)[0]
        np.testing.assert_allclose(y, [-math.sin(p), math.cos(p)], atol=1e-12)


def test_rope_pairing_and_frequency():
    # d_h = 4: pair (2, 3) rotates with frequency theta^(-2/4).
    theta, p = 10000.0, 5
    y = orc.apply_rope(np.array([[0.0, 0.0, 1.0, 0.0]]), p, theta)[0]
    ang = p * theta ** -0.5
    np.testing.assert_allclose(y, [0.0, 0.0, math.cos(ang), math.sin(ang)], atol=1e-12)
    y = orc.apply_rope(np.array([[1.0, 0.0, 0.0, 0.0]]), p, theta)[0]
    np.testing.assert_allclose(y, [math.cos(p), math.sin(p), 0.0, 0.0], atol=1e-12)


def test_rope_norm_identity_relative():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 64))
    k = rng.standard_normal((4, 64))
    np.testing.assert_allclose(orc.apply_rope(q, 0, 1e4), q, atol=0)
    for p in (1, 255, 8191):
        r = orc.apply_rope(q, p, 5e5)
        np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-12)
    # <R_m q, R_n k> = <q, R_{n-m} k>
    for m, n in ((3, 10), (100, 4000), (7, 7)):
        lhs = np.sum(orc.apply_rope(q, m, 1e4) * orc.apply_rope(k, n, 1e4), axis=-1)
        rhs = np.sum(q * orc.apply_rope(k, n - m, 1e4), axis=-1)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------------------
# Softmax, attention
# ---------------------------------------------------------------------------


def test_softmax_sum_shift_closed_form():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((3, 100)) * 20
    a = orc.softmax(s)
    np.testing.assert_allclose(a.sum(-1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(orc.softmax(s + 1234.5), a, rtol=1e-9)
    for x0, x1 in ((0.0, 1.0), (3.0, -2.0), (700.0, 701.0)):
        np.testing.assert_allclose(orc.softmax(np.array([x0, x1]))[1], expit(x1 - x0), rtol=1e-12)


def test_attention_single_position_returns_v():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((8, 64)).astype(np.float32)
    k = rng.standard_normal((2, 1, 64)).astype(np.float32)
    v = rng.standard_normal((2, 1, 64)).astype(np.float32)
    o = orc.gqa_attention(q, k, v)
    for j in range(8):
        np.testing.assert_array_equal(o[j], v[j // 4, 0])


def test_attention_zero_query_is_mean_and_two_positions():
    rng = np.random.default_rng(7)
    k = rng.standard_normal((1, 50, 16))
    v = rng.standard_normal((1, 50, 16))
    o = orc.gqa_attention(np.zeros((2, 16)), k, v)
    np.testing.assert_allclose(o[0], v[0].mean(0), rtol=1e-12)
    # two positions: weight of position 1 is logistic((s1 - s0) / sqrt(d))
    d = 16
    q = rng.standard_normal((1, d))
    k2 = rng.standard_normal((1, 2, d))
    v2 = np.zeros((1, 2, d)); v2[0, 1, 0] = 1.0
    s0, s1 = float(k2[0, 0] @ q[0]), float(k2[0, 1] @ q[0])
    o = orc.gqa_attention(q, k2, v2)
    np.testing.assert_allclose(o[0, 0], expit((s1 - s0) / math.sqrt(d)), rtol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((32, 64))
    k = rng.standard_normal((8, 20, 64))
    v = rng.standard_normal((8, 20, 64))
    a = orc.gqa_attention(q, k, v)
    b = orc.gqa_attention(q, np.repeat(k, 4, axis=0), np.repeat(v, 4, axis=0))
    np.testing.assert_allclose(a, b, rtol=1e-12)


# ---------------------------------------------------------------------------
# SiLU, SwiGLU
# ---------------------------------------------------------------------------


def test_silu_identities():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(orc.silu(z), z * expit(z), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(orc.silu(z) - orc.silu(-z), z, atol=1e-12)
    assert orc.silu(np.array([0.0]))[0] == 0.0


def test_swiglu_gate_role():
    rng = np.random.default_rng(9)
    H, F = 16, 32
    xn = rng.standard_normal(H)
    wu = rng.standard_normal((F, H))
    wd = rng.standard_normal((H, F))
    direction = xn / np.dot(xn, xn)
    # gate strongly negative: silu(gate) ~ 0, so the block outputs ~0 whatever "up" is
    wg_neg = np.tile(-200.0 * direction, (F, 1))
    assert np.max(np.abs(orc.swiglu_ffn(xn, wg_neg, wu, wd))) < 1e-50
    # gate strongly positive: silu(gate) ~ gate
    wg_pos = np.tile(50.0 * direction, (F, 1))
    np.testing.assert_allclose(orc.swiglu_ffn(xn, wg_pos, wu, wd), wd @ (50.0 * (wu @ xn)), rtol=1e-12)


# ---------------------------------------------------------------------------
# Brute force: a tiny decoder written as scalar loops in float64
# ---------------------------------------------------------------------------

def _brute_step(sh, W, token, pos, kc, vc):
    """Scalar-loop decode step (row-major [out][in] matrices, python floats)."""
    H, NQ, NK, D, F = sh.hidden, sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.ffn
    f = lambda name: orc.bf16_to_f32(W[name]).astype(np.float64)

    def mv(M, x):
        return [sum(M[i][j] * x[j] for j in range(len(x))) for i in range(len(M))]

    def norm(x, g):
        ms = sum(t * t for t in x) / len(x)
        r = 1.0 / math.sqrt(ms + sh.rms_eps)
        return [x[i] * r * g[i] for i in range(len(x))]

    def rot(vec, p):
        out = list(vec)
        for i in range(D // 2):
            a = p * sh.rope_theta ** (-2.0 * i / D)
            x0, x1 = vec[2 * i], vec[2 * i + 1]
            out[2 * i] = x0 * math.cos(a) - x1 * math.sin(a)
            out[2 * i + 1] = x0 * math.sin(a) + x1 * math.cos(a)
        return out

    x = list(f("embed")[token])
    for l in range(sh.n_layers):
        p = f"layers.{l}."
        xn = norm(x, f(p + "attn_norm"))
        q, k, v = mv(f(p + "wq"), xn), mv(f(p + "wk"), xn), mv(f(p + "wv"), xn)
        for h in range(NK):
            kr = rot(k[h * D:(h + 1) * D], pos)
            kc[l, h, pos] = orc.f32_to_bf16(np.array(kr, np.float32))
            vc[l, h, pos] = orc.f32_to_bf16(np.array(v[h * D:(h + 1) * D], np.float32))
        o = []
        for j in range(NQ):
            h = j // (NQ // NK)
            qj = rot(q[j * D:(j + 1) * D], pos)
            Kf = orc.bf16_to_f32(kc[l, h, :pos + 1]).astype(np.float64)
            Vf = orc.bf16_to_f32(vc[l, h, :pos + 1]).astype(np.float64)
            s = [sum(qj[d] * Kf[t][d] for d in range(D)) / math.sqrt(D) for t in range(pos + 1)]
            m = max(s)
            e = [math.exp(si - m) for si in s]
            z = sum(e)
            o += [sum(e[t] / z * Vf[t][d] for t in range(pos + 1)) for d in range(D)]
        att = mv(f(p + "wo"), o)
        x = [x[i] + att[i] for i in range(H)]
        xn = norm(x, f(p + "ffn_norm"))
        g, u = mv(f(p + "w_gate"), xn), mv(f(p + "w_up"), xn)
        hid = [g[i] / (1.0 + math.exp(-g[i])) * u[i] for i in range(F)]
        dn = mv(f(p + "w_down"), hid)
        x = [x[i] + dn[i] for i in range(H)]
    xf = norm(x, f("final_norm"))
    lm = f("embed") if sh.tie_embeddings else f("lm_head")
    return np.array(mv(lm, xf))


@pytest.mark.parametrize("tied", [True, False])
def test_brute_force_tiny_decoder(tied):
    sh = TINY.with_(name="micro", n_layers=2, hidden=8, n_heads=4, n_kv_heads=2, head_dim=4,
                    ffn=12, vocab=20, tie_embeddings=tied)
    W = make_weights(sh, master=11, gain_jitter=0.1)
    # make the weights large enough that every term matters
    for name in W:
        if not name.endswith("norm"):
            W[name] = orc.f32_to_bf16(orc.bf16_to_f32(W[name]) * 20)
    o = orc.Oracle(sh, W, dtype=np.float64)
    kc_o, vc_o = o.new_cache(6)
    kc_b, vc_b = kc_o.copy(), vc_o.copy()
    for pos, tok in enumerate([3, 17, 0, 9, 9]):
        lo = o.decode_step(tok, pos, kc_o, vc_o)
        lb = _brute_step(sh, W, tok, pos, kc_b, vc_b)
        np.testing.assert_allclose(lo, lb, rtol=1e-9, atol=1e-9)
        np.testing.assert_array_equal(kc_o, kc_b)
        np.testing.assert_array_equal(vc_o, vc_b)


# ---------------------------------------------------------------------------
# Whole-step properties on the tiny workload shape
# ---------------------------------------------------------------------------


@pytest.fixture(scope="module")
def tiny_weights():
    return make_weights(TINY, master=0, gain_jitter=0.1)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_incremental_equals_full_recompute(tiny_weights, dtype):
    o = orc.Oracle(TINY, tiny_weights, dtype=dtype)
    toks = make_prompt(TINY, 12)
    kc, vc = o.new_cache(16)
    inc = np.stack([o.decode_step(int(t), i, kc, vc) for i, t in enumerate(toks)])
    full = o.forward_full(toks)
    tol = 1e-9 if dtype == np.float64 else 2e-3
    np.testing.assert_allclose(inc, full, rtol=tol, atol=tol * np.abs(full).max())


def test_zero_layer_identity_all_ids():
    sh = TINY.with_(n_layers=0)
    W = make_weights(sh, master=0)
    o = orc.Oracle(sh, W, dtype=np.float64)
    ids = np.arange(sh.vocab)
    logits = o.forward_full(ids)                      # [V, V]; no attention with 0 layers
    E = orc.bf16_to_f32(W["embed"]).astype(np.float64)
    norms = np.linalg.norm(E, axis=1)
    # logit_t(t) = e_t . e_t / rms(e_t) = sqrt(H) * |e_t|   (eps negligible)
    diag = logits[ids, ids]
    want = math.sqrt(sh.hidden) * norms * np.sqrt(norms ** 2 / sh.hidden / (norms ** 2 / sh.hidden + sh.rms_eps))
    np.testing.assert_allclose(diag, want, rtol=1e-12)
    assert np.all(np.argmax(logits, axis=1) == ids)


def test_zero_residual_branches_is_identity(tiny_weights):
    W = make_weights(TINY, master=0, zero=("wo", "w_down"))
    sh0 = TINY.with_(n_layers=0)
    W0 = {k: v for k, v in W.items() if not k.startswith("layers.")}
    o = orc.Oracle(TINY, W, dtype=np.float64)
    o0 = orc.Oracle(sh0, W0, dtype=np.float64)
    kc, vc = o.new_cache(8)
    kc0, vc0 = o0.new_cache(8)
    for pos, tok in enumerate([5, 4000, 77]):
        np.testing.assert_array_equal(o.decode_step(tok, pos, kc, vc), o0.decode_step(tok, pos, kc0, vc0))


def test_float32_tracks_float64(tiny_weights):
    o32 = orc.Oracle(TINY, tiny_weights, dtype=np.float32)
    o64 = orc.Oracle(TINY, tiny_weights, dtype=np.float64)
    toks = make_prompt(TINY, 16)
    k32, v32 = o32.new_cache(20)
    k64, v64 = o64.new_cache(20)
    for i, t in enumerate(toks):
        a = o32.decode_step(int(t), i, k32, v32)
        b = o64.decode_step(int(t), i, k64, v64)
        assert np.max(np.abs(a - b)) <= 1e-4 * np.max(np.abs(b))


def test_cache_written_only_at_pos(tiny_weights):
    o = orc.Oracle(TINY, tiny_weights)
    kc, vc = o.new_cache(10)
    rng = np.random.default_rng(12)
    kc[:] = rng.integers(0, 0x7F00, kc.shape, dtype=np.uint16)
    vc[:] = rng.integers(0, 0x7F00, vc.shape, dtype=np.uint16)
    k0, v0 = kc.copy(), vc.copy()
    o.decode_step(7, 4, kc, vc)
    mask = np.ones(kc.shape, bool); mask[:, :, 4, :] = False
    np.testing.assert_array_equal(kc[mask], k0[mask])
    np.testing.assert_array_equal(vc[mask], v0[mask])


# ---------------------------------------------------------------------------
# Greedy token: first index of the maximum
# ---------------------------------------------------------------------------


def _first_max_scan(x):
    """Left-to-right scan that replaces the best only on a strictly larger value."""
    best, idx = x[0], 0
    for i in range(1, len(x)):
        if x[i] > best:
            best, idx = x[i], i
    return idx


def test_argmax_first_ties_and_ends():
    assert orc.argmax_first(np.array([1.0, 3.0, 3.0, 2.0], np.float32)) == 1
    assert orc.argmax_first(np.array([1.0, 3.0, 3.0, 0.0], np.float32)) == 1
    assert orc.argmax_first(np.full(17, -2.5, np.float32)) == 0          # all equal: the first
    assert orc.argmax_first(np.array([5.0, 1.0, 5.0], np.float32)) == 0  # tie of the first and the last
    assert orc.argmax_first(np.array([0.0, 1.0, 7.0], np.float32)) == 2  # maximum at the last index
    assert orc.argmax_first(np.array([9.0, 1.0, 7.0], np.float32)) == 0  # maximum at the first index
    # a signed value, not its magnitude, decides
    assert orc.argmax_first(np.array([-10.0, 2.0, -3.0], np.float32)) == 1
    # -0.0 and +0.0 compare equal: the first of them wins
    assert orc.argmax_first(np.array([-1.0, -0.0, 0.0], np.float32)) == 1
    assert orc.argmax_first(np.array([-1.0, 0.0, -0.0], np.float32)) == 1


def test_argmax_first_matches_scan_on_random_ties():
    # values from a small set, so many ties at the maximum, checked against a scalar scan
    rng = np.random.default_rng(13)
    for _ in range(200):
        n = int(rng.integers(1, 64))
        x = rng.integers(-3, 4, n).astype(np.float32)
        assert orc.argmax_first(x) == _first_max_scan(x)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_argmax_first_rejects_non_finite(bad):
    x = np.array([0.0, 1.0, bad, 2.0], np.float32)
    with pytest.raises(AssertionError):
        orc.argmax_first(x)
