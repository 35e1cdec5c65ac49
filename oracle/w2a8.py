"""CPU oracle of the W2A8 matrix-vector product (ternary weights stored in two
bits, int8 activations).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use
it, and it shares no code with the GPU path.

What is computed.  The page "BitNet 1.58bit GPU Inference Kernel:
Revolutionaere Effizienz fuer KI-Modelle mit W2A8-Quantisierung"
(dasgeld.co, body) describes a GEMV whose weights take three values stored in
two bits and whose activations are 8-bit integers, the products formed as
4-wide int8 dot products.  It does not print the quantisers.  The plainest
reading, and the one the page's "1.58 bit" names, is the BitNet b1.58 scheme:

  weights (offline, per output row r):
      gamma_r = mean_k |W[r, k]|
      Q[r, k] = clip(round(W[r, k] / (gamma_r + eps_w)), -1, 1)      in {-1, 0, 1}
  activations (per vector, on the path):
      s       = 127 / max(max_k |x[k]|, eps_x)                         (float32)
      q[k]    = clip(round_half_even(x[k] * s), -128, 127)              (float32 product)
  product:
      acc[r]  = sum_k Q[r, k] * q[k]                                    (exact integer)
      y[r]    = (float32(acc[r]) * gamma_r) / s                         (float32)

so that y approximates W x with W ~ gamma * Q and x ~ q / s.  One scale per
row is the general case; a per-tensor scale is every row's gamma equal.

Precision: the activation codes are decided in float32, the precision the GPU
kernel uses (a code is an integer decided by floating point, so both sides
take that decision in the same precision); the integer sum is exact (int64);
the two scalings are single float32 roundings in the order written above.
Pinned in ``tests/test_oracle_w2a8.py``.
"""

from __future__ import annotations

import numpy as np

EPS_W = 1e-5   # added to gamma before dividing (an all-zero row quantises to zeros)
EPS_X = 1e-5   # floor of the activation range (an all-zero vector quantises to zeros)


def quantize_weights_absmean(w: np.ndarray, eps: float = EPS_W) -> tuple[np.ndarray, np.ndarray]:
    """Ternary codes and per-row scales of a [rows][cols] matrix: gamma_r is
    the mean absolute value of row r, the codes are W / (gamma_r + eps)
    rounded to the nearest integer (half to even) and clipped to [-1, 1]."""
    w = np.asarray(w, dtype=np.float64)
    gamma = np.mean(np.abs(w), axis=1)
    q = np.clip(np.rint(w / (gamma[:, None] + eps)), -1, 1).astype(np.int8)
    return q, gamma.astype(np.float32)


def quantize_activations_absmax(x: np.ndarray, eps: float = EPS_X) -> tuple[np.ndarray, np.float32]:
    """int8 codes and the scale s of one activation vector: s = 127 / max|x|
    (floored at eps), code = x * s rounded half to even, clipped to int8.
    Every step in float32."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    s = np.float32(127.0) / np.maximum(amax, np.float32(eps))
    q = np.clip(np.rint(x * s), -128, 127).astype(np.int8)
    return q, np.float32(s)


def w2a8_gemv(codes: np.ndarray, gamma: np.ndarray, xq: np.ndarray, s: np.float32) -> np.ndarray:
    """y[r] = (float32(sum_k codes[r, k] * xq[k]) * gamma[r]) / s: the integer
    dot product exactly, then two float32 roundings."""
    acc = np.asarray(codes, dtype=np.int64) @ np.asarray(xq, dtype=np.int64)
    y = acc.astype(np.float32) * np.asarray(gamma, dtype=np.float32)
    return (y / np.float32(s)).astype(np.float32)


def w2a8_linear(codes: np.ndarray, gamma: np.ndarray, x: np.ndarray) -> np.ndarray:
    """The whole product on a float32 input: quantise x, then the GEMV."""
    xq, s = quantize_activations_absmax(x)
    return w2a8_gemv(codes, gamma, xq, s)
