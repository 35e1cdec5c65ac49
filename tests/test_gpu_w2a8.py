"""GPU parity of the W2A8 matrix-vector product (mk_w2a8_quantize +
mk_w2a8_gemv, and the one-launch mk_w2a8_linear, through the C ABI) against
the oracle (oracle/w2a8.py).

The activation codes are integers decided in float32 on both sides, and the
weight sums are exact integers, so the bar is bit-exact: the codes, the
scale and every output element must equal the oracle's."""

import numpy as np
import pytest

from oracle import w2a8 as ow
from synth_inputs import make_w2a8_case
from tests.parity import log

pytestmark = pytest.mark.gpu


def run_gpu(codes, gamma, x, stream=None):
    import torch

    from persistent_megakernel_cu_amd import binding as mkb

    rows, cols = codes.shape
    packed = torch.from_numpy(mkb.w2a8_pack(codes).view(np.int32)).cuda()
    g = torch.from_numpy(gamma).cuda()
    xd = torch.from_numpy(x).cuda()
    xq = torch.zeros(max(cols, 64), dtype=torch.int8, device="cuda")
    s = torch.zeros(1, dtype=torch.float32, device="cuda")
    y = torch.full((max(rows, 1),), float("nan"), dtype=torch.float32, device="cuda")
    mkb.w2a8_quantize(xd, xq, s, stream)
    mkb.w2a8_gemv(packed, g, rows, cols, xq, s, y, stream)
    # the one-launch product from the float input gives the same bits
    y1 = torch.full((max(rows, 1),), float("nan"), dtype=torch.float32, device="cuda")
    mkb.w2a8_linear(packed, g, rows, cols, xd, y1, stream)
    torch.cuda.synchronize()
    y_np, y1_np = y.cpu().numpy()[:rows], y1.cpu().numpy()[:rows]
    assert np.array_equal(y_np.view(np.uint32), y1_np.view(np.uint32)), "mk_w2a8_linear differs from quantize + gemv"
    return xq.cpu().numpy()[:cols], np.float32(s.cpu().item()), y_np


def check_case(rows, cols, master=0, label=""):
    codes, gamma, x = make_w2a8_case(rows, cols, master=master)
    log(f"[w2a8] {label} rows={rows} cols={cols} master={master}")
    xq, s, y = run_gpu(codes, gamma, x)
    xq_ref, s_ref = ow.quantize_activations_absmax(x)
    assert s == s_ref
    assert np.array_equal(xq, xq_ref)
    y_ref = ow.w2a8_gemv(codes, gamma, xq_ref, s_ref)
    bad = np.flatnonzero(y.view(np.uint32) != y_ref.view(np.uint32))
    assert bad.size == 0, f"{bad.size} outputs differ, first row {bad[:5]}: {y[bad[:5]]} vs {y_ref[bad[:5]]}"
    return y


@pytest.mark.parametrize("rows,cols", [
    (1, 64), (4, 64), (37, 192),        # ragged row counts, one partial chunk
    (1000, 4096),                       # one full 4096-column chunk
    (513, 4160),                        # a second chunk with a single 64-column lane group
    (129, 8192 + 2048),                 # three chunks, the last half full
    (300, 16384),                       # the widest: four full chunks
])
def test_w2a8_parity(rows, cols):
    check_case(rows, cols, master=1, label="parity")


@pytest.mark.parametrize("name,rows,cols", [
    ("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336),
    ("lm_head", 128256, 4096),
])
def test_w2a8_llama8b_projection_shapes(name, rows, cols):
    # the projections of the Llama-8B shape at full size, every output checked
    check_case(rows, cols, master=2, label=name)


def test_w2a8_degenerate_inputs():
    # zero columns: every output is 0; an all-zero activation vector: codes 0, outputs 0
    y = check_case(5, 0, label="no columns")
    assert np.all(y == 0)
    codes, gamma, _ = make_w2a8_case(16, 128, master=4)
    xq, s, y = run_gpu(codes, gamma, np.zeros(128, dtype=np.float32))
    assert np.all(xq == 0) and s == np.float32(127.0) / np.float32(1e-5) and np.all(y == 0)
    # all-ones codes against the extreme activation -128 (x = -max): exact integer sums
    cols = 4096
    codes = np.ones((3, cols), dtype=np.int8)
    codes[1] = -1
    codes[2, ::2] = 0
    x = np.full(cols, -1.0, dtype=np.float32)
    xq, s, y = run_gpu(codes, np.ones(3, dtype=np.float32), x)
    assert np.all(xq == -127) and s == np.float32(127.0)
    assert y.tolist() == [np.float32(-127.0 * cols / 127.0), np.float32(127.0 * cols / 127.0),
                          np.float32(-127.0 * cols / 2 / 127.0)]


def test_w2a8_no_rows_is_a_no_op():
    import torch

    from persistent_megakernel_cu_amd import binding as mkb

    y = torch.full((4,), 7.0, device="cuda")
    mkb.w2a8_gemv(None, None, 0, 64, None, None, y)
    torch.cuda.synchronize()
    assert y.cpu().tolist() == [7.0] * 4


def test_w2a8_consecutive_calls_carry_no_state():
    # a large call, then a small one on the same stream: each matches the oracle
    check_case(4096, 14336, master=5, label="first")
    check_case(3, 64, master=6, label="second")
