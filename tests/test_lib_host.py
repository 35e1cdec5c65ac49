"""Host-only checks of libmk.so: it loads without a GPU, exports every function
include/mk.h declares, and its planner builds and validates the task tape."""

import ctypes

import pytest

from persistent_megakernel_cu_amd import binding as mkb
from synth_inputs import LLAMA_1B, LLAMA_8B, TINY


def test_exports_every_declared_function():
    names = mkb.header_functions()
    assert set(names) == {"mk_load", "mk_decode_step", "mk_decode_steps", "mk_reset", "mk_free", "mk_status",
                          "mk_error_string",
                          "mk_plan_describe", "mk_trace_copy", "mk_conv_workspace_size", "mk_conv_decode_step",
                          "mk_conv_decode_step_static", "mk_w2a8_pack", "mk_w2a8_quantize", "mk_w2a8_gemv", "mk_w2a8_linear"}
    L = mkb.lib()
    for n in names:
        assert getattr(L, n) is not None


def test_error_strings():
    for code in range(0, -11, -1):
        assert mkb.error_string(code) and mkb.error_string(code) != "unknown error"
    assert mkb.error_string(-99) == "unknown error"


@pytest.mark.parametrize("shape,max_seq,chunks", [
    (TINY, 48, 1), (LLAMA_1B, 256, 1), (LLAMA_1B, 8192, 32), (LLAMA_1B, 1088, 5), (LLAMA_8B, 2112, 9)])
def test_plan_validates(shape, max_seq, chunks):
    info = mkb.plan_describe(shape, max_seq, 256)
    assert info.num_stages == 5 * shape.n_layers + 1
    assert info.attn_chunks == chunks
    assert info.lds_bytes <= 160 * 1024
    # every byte of every matrix is in the packed arena once (LM head borrowed when rows need no padding)
    H, QD, KVD, F = shape.hidden, shape.q_dim, shape.kv_dim, shape.ffn
    per_layer = 2 * (QD * H + 2 * KVD * H + H * QD + 2 * F * H + H * F)
    if H % 512 == 0 and QD % 512 == 0 and F % 512 == 0:
        assert info.weight_bytes >= shape.n_layers * per_layer
        assert info.weight_bytes <= shape.n_layers * per_layer + 5 * shape.n_layers * 4096


def test_ring_depth_follows_the_lds_budget():
    # batch-1 plans keep 14 weight units per wave in flight; a plan whose LDS
    # does not fit beside that ring (the 8B shape's 14336-wide FFN
    # activation) is laid out with 8 for its description and address walk,
    # and mk_load refuses it; batched plans keep 10
    info = mkb.plan_describe(LLAMA_1B, 1088, 256)
    assert info.ring_units == 14 and info.lds_bytes <= 160 * 1024
    info = mkb.plan_describe(LLAMA_8B, 2112, 256)
    assert info.ring_units == 8 and info.lds_bytes <= 160 * 1024
    assert mkb.plan_describe(LLAMA_1B, 1088, 256, batch=8).ring_units == 10
    assert mkb.plan_describe(TINY, 48, 256).ring_units == 14


@pytest.mark.parametrize("shape,max_seq,batch,chunks", [
    (TINY, 48, 4, 1), (TINY, 48, 8, 1), (LLAMA_1B, 1088, 8, 4), (LLAMA_1B, 256, 2, 1)])
def test_plan_batched_validates(shape, max_seq, batch, chunks):
    # tiled plans: every (sequence, kv head, chunk) has a task, the LM head is repacked
    info = mkb.plan_describe(shape, max_seq, 256, batch=batch)
    assert info.attn_chunks == chunks
    assert info.num_stages == 5 * shape.n_layers + 1
    assert info.lds_bytes <= 160 * 1024
    H, QD, KVD, F, V = shape.hidden, shape.q_dim, shape.kv_dim, shape.ffn, shape.vocab
    per_layer = 2 * (QD * H + 2 * KVD * H + H * QD + 2 * F * H + H * F)
    assert info.weight_bytes >= shape.n_layers * per_layer + 2 * V * H


@pytest.mark.parametrize("wgs", [2, 7, 64, 255, 256])
def test_plan_any_workgroup_count(wgs):
    info = mkb.plan_describe(TINY, 48, wgs)
    assert info.num_wgs == wgs


def test_plan_needs_a_workgroup_per_kv_head():
    # one task per (stage, workgroup): attention needs at least n_kv_heads workgroups
    with pytest.raises(mkb.MkError) as e:
        mkb.plan_describe(TINY, 48, 1)
    assert e.value.code == mkb.MK_E_UNSUPPORTED


def test_plan_rejects_bad_configs():
    bad = [
        dict(n_heads=3),            # not a multiple of n_kv_heads
        dict(head_dim=96),          # the attention executor is built for 64 and 128
        dict(hidden=255),           # odd
    ]
    for kw in bad:
        sh = TINY.with_(**kw)
        with pytest.raises(mkb.MkError):
            mkb.plan_describe(sh, 48, 256)
    for kw in (dict(batch=9), dict(batch=2, head_dim=128)):  # batches of 2..8, head_dim 64
        sh = TINY.with_(**{k: v for k, v in kw.items() if k != "batch"})
        with pytest.raises(mkb.MkError) as e:
            mkb.plan_describe(sh, 48, 256, batch=kw["batch"])
        assert e.value.code == mkb.MK_E_UNSUPPORTED
    c = mkb.make_config(TINY, 48)
    info = mkb.MkPlanInfo()
    assert mkb.lib().mk_plan_describe(None, 256, ctypes.byref(info)) == mkb.MK_E_INVAL
    assert mkb.lib().mk_plan_describe(ctypes.byref(c), 256, None) == mkb.MK_E_INVAL


def test_null_arguments_are_rejected():
    L = mkb.lib()
    h = ctypes.c_void_p()
    assert L.mk_load(None, None, ctypes.byref(h)) == mkb.MK_E_INVAL
    assert L.mk_decode_step(None, None, 0, None, None, None, None) == mkb.MK_E_INVAL
    assert L.mk_reset(None) == mkb.MK_E_INVAL
    assert L.mk_status(None, None) == mkb.MK_E_INVAL
    L.mk_free(None)


def _batched_task_count(shape, max_seq, B, W=256):
    """Tasks of a batched plan from the planner's rules: a GEMM stage of `blocks`
    16-row blocks over nw workgroups has min(blocks, nw) tasks; an O- or down
    projection with 2 * blocks <= W whose row (kt 32-column tiles) splits into an
    even number of chunks of a multiple of 8 tiles (64-tile chunks, or two halves
    of a single-chunk row) has two tasks per block; attention has one task per
    (sequence, kv head, chunk); gate/up skips the attention workgroups when those
    are at most an eighth of all."""
    H, QD, KVD, F, V = shape.hidden, shape.q_dim, shape.kv_dim, shape.ffn, shape.vocab
    pad = lambda x: (x + 511) // 512 * 512
    C = min(-(-max_seq // 256), W // (B * shape.n_kv_heads))
    seqs_kv = B * shape.n_kv_heads

    def gemm(rows, kt, nw, splittable=False):
        blocks = rows // 16
        sch = 64 if kt > 64 else kt // 2
        if splittable and 2 * blocks <= W and kt % sch == 0 and (kt // sch) % 2 == 0 and sch % 8 == 0:
            return 2 * blocks
        return min(blocks, nw)

    gu_b0 = seqs_kv * C if seqs_kv * C * 8 <= W else 0
    per_layer = (gemm(QD + 2 * KVD, pad(H) // 32, W) + seqs_kv * C + gemm(H, pad(QD) // 32, W, True)
                 + gemm(2 * F, pad(H) // 32, W - gu_b0) + gemm(H, pad(F) // 32, W, True))
    return shape.n_layers * per_layer + gemm(V, pad(H) // 32, W)


@pytest.mark.parametrize("shape,max_seq,batch", [
    (TINY, 48, 4), (TINY, 48, 8), (LLAMA_1B, 1088, 8), (LLAMA_1B, 256, 2)])
def test_plan_batched_split_blocks(shape, max_seq, batch):
    # O-proj and down blocks split over workgroup pairs where the rule allows
    # (Llama-1B: 128 blocks each -> 256 tasks; tiny: 16 blocks -> 32 tasks)
    info = mkb.plan_describe(shape, max_seq, 256, batch=batch)
    assert info.num_tasks == _batched_task_count(shape, max_seq, batch)


def test_stage_timeline_summary():
    # two layers (10 stages + LM head) on 4 workgroups with known stamps (kHz 1000 -> 1 tick = 1 us)
    import numpy as np

    from persistent_megakernel_cu_amd.timeline import stage_table

    W, S = 4, 11
    st = np.zeros((W, S, 20), dtype=np.uint64)
    t = 100
    for s in range(S):
        for b in range(W):
            # entered, ready = +2, done = +5 (+b for the stragglers), left = done
            st[b, s, 0] = t
            st[b, s, 1] = t + 2
            st[b, s, 2] = t + 5 + b
            st[b, s, 3] = t + 5 + b
        t += 5 + W  # next stage starts after the slowest one
    out = stage_table(st, 1000)
    h, c, tl = out["per_kind"]["gate/up"]
    # stage s starts at 100 + 9 s: ready +2, done +5..+8 over the workgroups (median +6.5)
    assert abs(c - 4.5) < 1e-9                # median done - median ready
    assert abs(tl - 1.5) < 1e-9               # latest done - median done
    assert abs(h - 3.0) < 1e-9                # ready (+2) - previous stage's latest done (-9 + 8)
    assert out["layers"] == 2 and out["rows"][0]["tasks"] == W


def test_conv_workspace_size():
    # fp32 activations (x, xn, q, k, v, attention out, gate, up, hid), split-KV
    # partials of 256-position chunks and the argmax keys, 256-byte aligned pieces
    sh = TINY
    H, QD, KVD, F = sh.hidden, sh.q_dim, sh.kv_dim, sh.ffn
    up = lambda n: (n + 255) // 256 * 256
    for B, S in ((1, 48), (3, 600)):
        C = -(-S // 256)
        want = (up(B * H * 4) * 2 + up(B * QD * 4) * 2 + up(B * KVD * 4) * 2 + up(B * F * 4) * 3
                + up(B * sh.n_heads * C * (sh.head_dim + 2) * 4) + up(B * 256 * 8) + up(B * 4))
        assert mkb.conv_workspace_size(sh, S, B) == want


def test_conv_rejects_bad_configs():
    for kw, code in ((dict(head_dim=24), mkb.MK_E_UNSUPPORTED), (dict(head_dim=256), mkb.MK_E_UNSUPPORTED),
                     (dict(hidden=260), mkb.MK_E_INVAL), (dict(n_heads=3), mkb.MK_E_INVAL)):
        with pytest.raises(mkb.MkError) as e:
            mkb.conv_workspace_size(TINY.with_(**kw), 48)
        assert e.value.code == code
    with pytest.raises(mkb.MkError) as e:
        mkb.conv_workspace_size(TINY, 48, 9)
    assert e.value.code == mkb.MK_E_UNSUPPORTED
    n = ctypes.c_size_t()
    assert mkb.lib().mk_conv_workspace_size(None, ctypes.byref(n)) == mkb.MK_E_INVAL
    assert mkb.lib().mk_conv_decode_step(None, None, None, None, None, None, None, None, 0, None) == mkb.MK_E_INVAL


def test_partial_input_plans():
    # partial-input down projection: batch 1 and head_dim 64 only; the plan validates
    info = mkb.plan_describe(LLAMA_1B, 256, 256, partial_input=True)
    assert info.num_stages == 5 * LLAMA_1B.n_layers + 1
    mkb.plan_describe(TINY.with_(ffn=2048), 48, 256, partial_input=True)
    for kw in (dict(batch=2), ):
        with pytest.raises(mkb.MkError) as e:
            mkb.plan_describe(TINY, 48, 256, partial_input=True, **kw)
        assert e.value.code == mkb.MK_E_UNSUPPORTED
    with pytest.raises(mkb.MkError) as e:
        mkb.plan_describe(LLAMA_8B, 2112, 256, partial_input=True)
    assert e.value.code == mkb.MK_E_UNSUPPORTED


def test_prefill_plans():
    # prefill runs on the batched (MFMA) executors: 2..8 tokens per call, megakernel modes only
    info = mkb.plan_describe(LLAMA_1B, 256, 256, batch=8, prefill=True)
    assert info.num_stages == 5 * LLAMA_1B.n_layers + 1 and info.lds_bytes <= 160 * 1024
    for kw in ({"batch": 1}, {"batch": 4, "mode": "conv"}):
        with pytest.raises(mkb.MkError) as e:
            mkb.plan_describe(TINY, 48, 256, prefill=True, **kw)
        assert e.value.code in (mkb.MK_E_UNSUPPORTED, mkb.MK_E_INVAL)
