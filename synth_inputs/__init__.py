"""Seeded synthetic inputs for the batch-1 decode step of a Llama-style decoder.

This module only *generates data*: model shapes, seeded bf16 weights, prompt
token ids, seeded KV caches and start tokens. It contains none of the
forward-pass arithmetic, so the CPU oracle (``oracle/``) and the GPU path
(``persistent_megakernel_cu_amd``) can both consume the same bytes without
sharing any code that computes the method.

The subject pages ("Revolution der KI-Beschleunigung: Wie ein Low-Latency
Megakernel den Llama-1B Turbo zuendet", dasgeld.co) measure the trained
Llama-1B in bfloat16; no trained weights are available here, so weights are
drawn at random with the shapes of that model family.

Recipe (every stream is a NumPy PCG64 generator seeded from a SeedSequence):

* weights: tensor ``i`` in the order embed, per layer [attn_norm, wq, wk, wv,
  wo, ffn_norm, w_gate, w_up, w_down], final_norm, lm_head (if untied), is
  drawn in chunks of ``CHUNK`` elements; chunk ``c`` uses
  ``SeedSequence([master, i, c])``.  Values are N(0, 0.02) (standard
  deviation 0.02) drawn in float32 and rounded to bfloat16 with
  round-to-nearest-even.  Norm gains are exactly 1.0 unless a test asks for
  ``gain_jitter`` (then 1 + N(0, gain_jitter), also bf16).
* prompt ids: ``SeedSequence([master, 10000])``, uniform in [0, vocab).
* KV cache of sequence b: ``SeedSequence([master, 20000 + b])``, N(0, 1),
  bf16; generated per (layer, kv head) block in that order.
* start token of sequence b: ``SeedSequence([master, 30000 + b])``, uniform.
* W2A8 matrix-vector cases (``make_w2a8_case``): ``SeedSequence([master,
  40000, rows, cols])``; ternary codes drawn directly (a uniform float32
  u per weight: -1 below 0.345, +1 from 0.655, else 0), so -1 / 0 / +1 with
  probabilities 0.345 / 0.31 / 0.345 (the shares that absmean coding gives a
  Gaussian matrix); row scales 0.02 * U(0.8, 1.2) (the mean |w| of a trained
  projection's row); activations N(0, 1) with one element in 512 scaled by
  U(10, 40) (the outlier channels of decoder activations).

Matrices are row-major ``[out][in]`` arrays of uint16 bf16 bit patterns.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded chunk of a weight tensor
WEIGHT_STD = 0.02

LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Shape of a Llama-style decoder (pre-norm, GQA, SwiGLU, RoPE)."""

    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    tie_embeddings: bool = True

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)

    def param_count(self) -> int:
        H, QD, KVD, F, V, L = self.hidden, self.q_dim, self.kv_dim, self.ffn, self.vocab, self.n_layers
        per_layer = 2 * H + QD * H + 2 * KVD * H + H * QD + 3 * F * H
        return V * H + L * per_layer + H + (0 if self.tie_embeddings else V * H)


# The workloads: a tiny decoder, the Llama-1B shape and the Llama-8B shape.
TINY = ModelShape("tiny-2L-256", 2, 256, 4, 2, 64, 1024, 4096, 1e-5, 10000.0, True)
LLAMA_1B = ModelShape("llama-1b", 16, 2048, 32, 8, 64, 8192, 128256, 1e-5, 500000.0, True)
LLAMA_8B = ModelShape("llama-8b", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, False)

SHAPES = {s.name: s for s in (TINY, LLAMA_1B, LLAMA_8B)}


def _rng(*stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(stream))))


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def _normal_bf16(out: np.ndarray, master: int, tensor_index: int, std: float, mean: float = 0.0) -> None:
    flat = out.reshape(-1)
    n = flat.size

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = _rng(master, tensor_index, c)
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        flat[lo:hi] = _to_bf16_bits(v)

    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(fill, range(nchunks)))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def weight_shapes(shape: ModelShape) -> list[tuple[str, int, tuple[int, ...]]]:
    """(name, stream index, array shape) for every tensor, in stream order."""
    H, QD, KVD, F, V = shape.hidden, shape.q_dim, shape.kv_dim, shape.ffn, shape.vocab
    out = [("embed", 0, (V, H))]
    per = {
        "attn_norm": (H,), "wq": (QD, H), "wk": (KVD, H), "wv": (KVD, H), "wo": (H, QD),
        "ffn_norm": (H,), "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F),
    }
    for l in range(shape.n_layers):
        for j, t in enumerate(LAYER_TENSORS):
            out.append((f"layers.{l}.{t}", 1 + 9 * l + j, per[t]))
    out.append(("final_norm", 1 + 9 * shape.n_layers, (H,)))
    if not shape.tie_embeddings:
        out.append(("lm_head", 2 + 9 * shape.n_layers, (V, H)))
    return out


def make_weights(shape: ModelShape, master: int = 0, gain_jitter: float = 0.0,
                 zero: tuple[str, ...] = ()) -> dict[str, np.ndarray]:
    """Seeded bf16 weights as uint16 arrays keyed by tensor name.

    ``gain_jitter`` > 0 draws norm gains as 1 + N(0, gain_jitter) (a test-only
    variant); ``zero`` lists per-layer tensor kinds (e.g. "wo") set to zero.
    """
    out: dict[str, np.ndarray] = {}
    for name, idx, shp in weight_shapes(shape):
        kind = name.rsplit(".", 1)[-1]
        a = np.empty(shp, dtype=np.uint16)
        if kind in ("attn_norm", "ffn_norm", "final_norm"):
            if gain_jitter > 0:
                _normal_bf16(a, master, idx, gain_jitter, 1.0)
            else:
                a.fill(0x3F80)  # bf16 1.0
        elif kind in zero:
            a.fill(0)
        else:
            _normal_bf16(a, master, idx, WEIGHT_STD)
        out[name] = a
    return out


def make_prompt(shape: ModelShape, n: int, master: int = 0) -> np.ndarray:
    return _rng(master, 10000).integers(0, shape.vocab, size=n, dtype=np.int64).astype(np.int32)


def make_start_token(shape: ModelShape, b: int, master: int = 0) -> int:
    return int(_rng(master, 30000 + b).integers(0, shape.vocab))


def make_kv_cache(shape: ModelShape, batch: int, max_seq: int, filled: int, master: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """bf16 K and V caches ``[batch][layers][kv_heads][max_seq][head_dim]``.

    Slots ``[0, filled)`` hold N(0,1) values from the sequence's stream; later
    slots are zero. K is drawn before V for each (layer, kv head) block.
    """
    L, NK, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
    k = np.zeros((batch, L, NK, max_seq, D), dtype=np.uint16)
    v = np.zeros_like(k)
    if filled <= 0:
        return k, v
    for b in range(batch):
        g = _rng(master, 20000 + b)
        for l in range(L):
            for h in range(NK):
                k[b, l, h, :filled] = _to_bf16_bits(g.standard_normal((filled, D), dtype=np.float32))
                v[b, l, h, :filled] = _to_bf16_bits(g.standard_normal((filled, D), dtype=np.float32))
    return k, v


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode workload: a model shape plus batch, cache and step counts."""

    name: str
    shape: ModelShape
    batch: int
    max_seq: int
    prompt_len: int      # tokens prefilled through the model (0: seeded cache instead)
    cache_filled: int    # seeded N(0,1) cache slots (0: none)
    steps: int           # greedy decode steps
    start_pos: int       # position of the first decode step


WORKLOADS = {
    "tiny": Workload("tiny", TINY, 1, 48, 16, 0, 32, 16),
    "llama1b": Workload("llama1b", LLAMA_1B, 1, 256, 128, 0, 128, 128),
    "llama1b-long": Workload("llama1b-long", LLAMA_1B, 1, 8192, 0, 8192, 1, 4096),
    "llama1b-b8": Workload("llama1b-b8", LLAMA_1B, 8, 1088, 0, 1024, 64, 1024),
    "llama8b": Workload("llama8b", LLAMA_8B, 1, 2112, 0, 2048, 64, 2048),
}


def make_w2a8_case(rows: int, cols: int, master: int = 0) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(codes int8 [rows][cols] in {-1, 0, 1}, row scales float32 [rows],
    activations float32 [cols]) for a W2A8 matrix-vector product."""
    g = _rng(master, 40000, rows, cols)
    u = g.random((rows, cols), dtype=np.float32)
    codes = (u >= np.float32(0.345)).astype(np.int8) + (u >= np.float32(0.655)).astype(np.int8) - np.int8(1)
    gamma = (0.02 * g.uniform(0.8, 1.2, size=rows)).astype(np.float32)
    x = g.standard_normal(cols, dtype=np.float32)
    if cols:
        n_out = max(1, cols // 512)
        idx = g.choice(cols, size=n_out, replace=False)
        x[idx] *= g.uniform(10.0, 40.0, size=n_out).astype(np.float32)
    return codes.astype(np.int8), gamma, x
