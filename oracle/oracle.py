"""CPU oracle for one batch-1 decode step of a Llama-style decoder.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run anything under ``oracle/``.
The GPU library never calls it, and it shares no code with the GPU path: the
two only consume the same seeded bytes from ``synth_inputs``.

What is computed.  The subject pages ("Revolution der KI-Beschleunigung: Wie
ein Low-Latency Megakernel den Llama-1B Turbo zuendet", dasgeld.co; glossary
"Megakernel", synthszr.com) describe the megakernel as a faster organisation
of the *unchanged* Llama-1B forward pass in bfloat16 (glossary "Kernel-Tuning",
section on FlashAttention: the tuned kernel computes the same thing, only
with less memory traffic).  The pages print no formulas, so the forward pass
is the textbook pre-norm Llama-style decoder, read plainly:

  x  = E[token]
  per layer:  xn = rmsnorm(x, g_attn); q,k,v = Wq xn, Wk xn, Wv xn
              rotate q, k at position p (RoPE, consecutive pairs (2i, 2i+1),
              angle p * theta^(-2i/d_h), angle and trig in float64)
              append bf16(k), bf16(v) to the cache at slot p
              o_j = softmax_tau(q_j . K_h[tau] / sqrt(d_h)) V_h,  h = j // (n_q/n_kv)
              x += Wo o
              xn = rmsnorm(x, g_ffn);  x += Wd (silu(Wg xn) * (Wu xn))
  logits = W_lm rmsnorm(x, g_final)  (W_lm = E when tied)
  token  = first index of max(logits)

Precision: activations and arithmetic in float32 (``dtype=np.float64`` is
available for pins), weights widened exactly from bf16, K/V rounded to bf16
on append because the cache is bf16 state.

Parity pins live in ``tests/test_oracle_pins.py``; every function here is
pinned there by a closed form, an invariant, a special case or a brute-force
tiny-input check.
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# bfloat16 <-> float32 (bit-exact definitions)
# ---------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns: the bf16 word is the high half of the float32 word."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Narrow float32 to bf16 bit patterns with round-to-nearest, ties to even.

    Adding 0x7FFF plus the lowest kept bit and truncating implements RNE;
    overflow carries into the exponent and yields infinity, as IEEE requires.
    NaN inputs keep their sign and become a quiet NaN.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = ((u + (((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF))) >> np.uint32(16)).astype(np.uint16)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    quiet = ((u >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return np.where(is_nan, quiet, rounded)


# ---------------------------------------------------------------------------
# Building blocks
# ---------------------------------------------------------------------------


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x * (mean(x^2) + eps)^(-1/2) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * (1.0 / np.sqrt(ms + x.dtype.type(eps))) * g


def rope_angles(pos: int, head_dim: int, theta: float) -> np.ndarray:
    """Rotation angles p * theta^(-2i/d_h) for i in [0, d_h/2), in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return float(pos) * np.power(float(theta), -2.0 * i / head_dim)


def apply_rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate consecutive pairs (2i, 2i+1) of every head (last axis) by rope_angles."""
    d = x.shape[-1]
    ang = rope_angles(pos, d, theta)
    c = np.cos(ang).astype(x.dtype)
    s = np.sin(ang).astype(x.dtype)
    a = x[..., 0::2]
    b = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def softmax(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, with the maximum subtracted first."""
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Decode attention of one position.

    q: [n_q, d]; k, v: [n_kv, T, d] (positions 0..T-1, already widened).
    Query head j reads KV head j // (n_q / n_kv).
    """
    n_q, d = q.shape
    n_kv = k.shape[0]
    group = n_q // n_kv
    out = np.empty_like(q)
    scale = q.dtype.type(1.0 / math.sqrt(d))
    for j in range(n_q):
        h = j // group
        s = (k[h] @ q[j]) * scale          # [T]
        a = softmax(s)
        out[j] = a @ v[h]
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """z * logistic(z)."""
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(xn: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    return w_down @ (silu(w_gate @ xn) * (w_up @ xn))


def argmax_first(logits: np.ndarray) -> int:
    """Index of the maximum; the lowest index wins a tie (np.argmax returns the first)."""
    assert np.all(np.isfinite(logits)), "non-finite logits"
    return int(np.argmax(logits))


# ---------------------------------------------------------------------------
# The model
# ---------------------------------------------------------------------------


class Oracle:
    """Reference decoder over bf16 weights given as uint16 bit arrays.

    ``weights`` is the dict produced by ``synth_inputs.make_weights`` (or any
    dict with the same keys).  ``lazy=True`` widens each matrix when it is
    used instead of holding a widened copy of the whole model.
    """

    def __init__(self, shape, weights: dict, dtype=np.float32, lazy: bool = False):
        self.shape = shape
        self.dtype = np.dtype(dtype)
        self.lazy = lazy
        self._raw = weights
        self._wide: dict[str, np.ndarray] = {}
        if not lazy:
            for name in weights:
                self._wide[name] = bf16_to_f32(weights[name]).astype(self.dtype)

    def w(self, name: str) -> np.ndarray:
        if name in self._wide:
            return self._wide[name]
        return bf16_to_f32(self._raw[name]).astype(self.dtype)

    def lm_head(self) -> np.ndarray:
        return self.w("embed") if self.shape.tie_embeddings else self.w("lm_head")

    # -- one decode step ----------------------------------------------------
    def decode_step(self, token: int, pos: int, kcache: np.ndarray, vcache: np.ndarray) -> np.ndarray:
        """Run token at position pos; append K/V at slot pos; return logits.

        kcache, vcache: uint16 bf16 arrays [layers][n_kv][max_seq][head_dim]
        of one sequence, modified in place at slot ``pos`` only.
        """
        sh = self.shape
        dt = self.dtype
        assert 0 <= token < sh.vocab and 0 <= pos < kcache.shape[2]
        D, NQ, NK = sh.head_dim, sh.n_heads, sh.n_kv_heads
        x = bf16_to_f32(self._raw["embed"][token]).astype(dt)
        for l in range(sh.n_layers):
            p = f"layers.{l}."
            xn = rmsnorm(x, self.w(p + "attn_norm"), sh.rms_eps)
            q = (self.w(p + "wq") @ xn).reshape(NQ, D)
            k = (self.w(p + "wk") @ xn).reshape(NK, D)
            v = (self.w(p + "wv") @ xn).reshape(NK, D)
            q = apply_rope(q, pos, sh.rope_theta)
            k = apply_rope(k, pos, sh.rope_theta)
            kcache[l, :, pos, :] = f32_to_bf16(k.astype(np.float32))
            vcache[l, :, pos, :] = f32_to_bf16(v.astype(np.float32))
            K = bf16_to_f32(kcache[l, :, : pos + 1, :]).astype(dt)
            V = bf16_to_f32(vcache[l, :, : pos + 1, :]).astype(dt)
            o = gqa_attention(q, K, V).reshape(NQ * D)
            x = x + self.w(p + "wo") @ o
            xn = rmsnorm(x, self.w(p + "ffn_norm"), sh.rms_eps)
            x = x + swiglu_ffn(xn, self.w(p + "w_gate"), self.w(p + "w_up"), self.w(p + "w_down"))
        xf = rmsnorm(x, self.w("final_norm"), sh.rms_eps)
        return self.lm_head() @ xf

    # -- whole-sequence recompute (independent formulation, for pins) --------
    def forward_full(self, tokens) -> np.ndarray:
        """Logits at every position of ``tokens`` with causal attention over the
        whole sequence at once (K/V rounded to bf16 as the cache stores them)."""
        sh = self.shape
        dt = self.dtype
        T = len(tokens)
        D, NQ, NK = sh.head_dim, sh.n_heads, sh.n_kv_heads
        group = NQ // NK
        X = bf16_to_f32(self._raw["embed"][np.asarray(tokens)]).astype(dt)    # [T, H]
        for l in range(sh.n_layers):
            p = f"layers.{l}."
            Xn = rmsnorm(X, self.w(p + "attn_norm"), sh.rms_eps)
            Q = (Xn @ self.w(p + "wq").T).reshape(T, NQ, D)
            K = (Xn @ self.w(p + "wk").T).reshape(T, NK, D)
            Vv = (Xn @ self.w(p + "wv").T).reshape(T, NK, D)
            for t in range(T):
                Q[t] = apply_rope(Q[t], t, sh.rope_theta)
                K[t] = apply_rope(K[t], t, sh.rope_theta)
            K = bf16_to_f32(f32_to_bf16(K.astype(np.float32))).astype(dt)
            Vv = bf16_to_f32(f32_to_bf16(Vv.astype(np.float32))).astype(dt)
            mask = np.tril(np.ones((T, T), dtype=bool))
            O = np.empty((T, NQ, D), dtype=dt)
            for j in range(NQ):
                h = j // group
                S = (Q[:, j, :] @ K[:, h, :].T) / dt.type(math.sqrt(D))      # [T, T]
                S = np.where(mask, S, -np.inf)
                O[:, j, :] = softmax(S) @ Vv[:, h, :]
            X = X + O.reshape(T, NQ * D) @ self.w(p + "wo").T
            Xn = rmsnorm(X, self.w(p + "ffn_norm"), sh.rms_eps)
            G = Xn @ self.w(p + "w_gate").T
            U = Xn @ self.w(p + "w_up").T
            X = X + (silu(G) * U) @ self.w(p + "w_down").T
        Xf = rmsnorm(X, self.w("final_norm"), sh.rms_eps)
        return Xf @ self.lm_head().T

    # -- drivers ------------------------------------------------------------
    def new_cache(self, max_seq: int) -> tuple[np.ndarray, np.ndarray]:
        sh = self.shape
        z = np.zeros((sh.n_layers, sh.n_kv_heads, max_seq, sh.head_dim), dtype=np.uint16)
        return z, z.copy()

    def prefill(self, tokens, kcache, vcache, start: int = 0) -> np.ndarray:
        """Run tokens at positions start.. ; returns the last position's logits."""
        logits = None
        for i, t in enumerate(tokens):
            logits = self.decode_step(int(t), start + i, kcache, vcache)
        return logits

    def greedy(self, first_token: int, start_pos: int, steps: int, kcache, vcache):
        """Feed first_token at start_pos, then each argmax; returns (tokens, logits list)."""
        toks, all_logits = [], []
        t = first_token
        for i in range(steps):
            lg = self.decode_step(t, start_pos + i, kcache, vcache)
            all_logits.append(lg)
            t = argmax_first(lg)
            toks.append(t)
        return toks, all_logits
