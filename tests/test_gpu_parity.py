"""GPU parity of the megakernel (and the launch-per-stage baselines) against
the CPU oracle, through the C ABI.  Run on an MI355X: pytest -m gpu."""

import numpy as np
import pytest

import oracle as orc
from synth_inputs import LLAMA_1B, TINY, make_kv_cache, make_prompt, make_start_token, make_weights
from tests.parity import GpuDecoder, check_step, log, logit_tol, run_batched_teacher_forced, run_teacher_forced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny_w():
    return make_weights(TINY, master=0, gain_jitter=0.1)


@pytest.mark.parametrize("mode", ["mega", "multi", "graph"])
def test_tiny_prompt_and_greedy(tiny_w, mode):
    # tiny decoder: 16-token prompt, then 32 greedy steps (positions 0..47)
    prompt = make_prompt(TINY, 16)
    run_teacher_forced(TINY, tiny_w, 48, prompt, 0, 32, mode=mode, label="tiny")


def test_tiny_unit_gains_untied():
    sh = TINY.with_(tie_embeddings=False)
    w = make_weights(sh, master=3)
    run_teacher_forced(sh, w, 48, make_prompt(sh, 8, master=3), 0, 8, mode="mega", label="tiny-untied")


def test_tiny_chunked_attention(tiny_w):
    # split-KV partials merged by the last chunk of each kv head
    run_teacher_forced(TINY, tiny_w, 48, make_prompt(TINY, 12), 0, 8, mode="mega", attn_chunks=4,
                       label="tiny-chunks4")


@pytest.mark.parametrize("wgs", [7, 64])
def test_tiny_other_grid_sizes(tiny_w, wgs):
    # plans over 7 and 64 workgroups: every stage's row items spread over
    # fewer waves, the gate/up ranges' one-workgroup offset wraps around a
    # grid that is not a multiple of the XCD count
    run_teacher_forced(TINY, tiny_w, 48, make_prompt(TINY, 8), 0, 8, mode="mega", num_wgs=wgs,
                       label=f"tiny-{wgs}wgs")


def test_tiny_zero_layers_identity():
    sh = TINY.with_(n_layers=0)
    w = make_weights(sh, master=0)
    gpu = GpuDecoder(sh, w, 8, mode="mega")
    try:
        rng = np.random.default_rng(5)
        for tok in rng.integers(0, sh.vocab, 64):
            lg, out = gpu.step(int(tok), 0)
            assert out == int(tok)
    finally:
        gpu.close()


@pytest.fixture(scope="module")
def llama1b():
    w = make_weights(LLAMA_1B, master=0)
    return w, orc.Oracle(LLAMA_1B, w)


@pytest.mark.parametrize("mode", ["mega", "graph", "multi"])
def test_llama1b_shape_short(llama1b, mode):
    # Llama-1B shape: a 4-token prompt and 4 greedy steps
    w, o = llama1b
    run_teacher_forced(LLAMA_1B, w, 256, make_prompt(LLAMA_1B, 4), 0, 4, mode=mode, oracle_obj=o,
                       label="llama1b")


@pytest.mark.parametrize("mode", ["mega", "graph"])
def test_llama1b_bench_workload_full(llama1b, mode):
    # The workload the benchmark times, whole: max_seq 256, the seeded 128-token
    # prompt teacher-forced at positions 0..127, then 128 greedy steps at
    # 128..255 (the oracle's token fed to both sides).  Every step checks the
    # logits, out_token, the KV slot written and the rest of the cache
    # unchanged.  Positions past 64 reach the later register passes of the
    # one-head-per-task attention.
    w, o = llama1b
    reps = run_teacher_forced(LLAMA_1B, w, 256, make_prompt(LLAMA_1B, 128), 0, 128, mode=mode, oracle_obj=o,
                              label="llama1b-bench-full")
    assert len(reps) == 256 and reps[-1].pos == 255


def test_llama1b_repeat_bit_identical(llama1b):
    # the same steps from the same cache give bit-identical logits and tokens, every time
    w, _ = llama1b
    gpu = GpuDecoder(LLAMA_1B, w, 256, mode="mega")
    toks = [int(t) for t in make_prompt(LLAMA_1B, 6, master=7)]
    try:
        first = None
        for rep in range(6):
            gpu.k.zero_()
            gpu.v.zero_()
            run = [gpu.step(t, p) for p, t in enumerate(toks)]
            if first is None:
                first = run
            for (a, ta), (b, tb) in zip(first, run):
                assert ta == tb and np.array_equal(a, b), f"repeat {rep} differs"
    finally:
        gpu.close()


def test_llama1b_long_context_positions(llama1b):
    # seeded N(0,1) cache of 8192 slots; single steps at 4096 and 8191 with 32
    # attention chunks; logits, out_token, the slot written and the rest of
    # the cache unchanged are checked at both positions
    sh = LLAMA_1B
    w, o = llama1b
    kv = make_kv_cache(sh, 1, 8192, 8192, master=0)
    tok = make_start_token(sh, 0)
    gpu = GpuDecoder(sh, w, 8192, mode="mega", kv_init=kv)
    kc, vc = kv[0][0].copy(), kv[1][0].copy()   # both sides carry the slot written at 4096 into 8191
    try:
        for pos in (4096, 8191):
            before = gpu.cache_np()
            lg, out = gpu.step(tok, pos)
            after = gpu.cache_np()
            lg_ref = o.decode_step(tok, pos, kc, vc)
            rep = check_step(pos, lg, out, lg_ref, before, after, (kc, vc))
            log(f"[parity] long pos={pos} err/tol={rep.max_abs_err / rep.tol:.3g} kv err/tol={rep.kv_err:.3g}")
            assert out == rep.oracle_token or rep.margin < rep.tol
    finally:
        gpu.close()


def test_determinism_and_nan_poison(tiny_w):
    # the same step twice is bit-identical; slots above pos are never read
    gpu = GpuDecoder(TINY, tiny_w, 48, mode="mega")
    try:
        for p, t in enumerate(make_prompt(TINY, 10)):
            gpu.step(int(t), p)
        k0, v0 = gpu.k.clone(), gpu.v.clone()
        a, ta = gpu.step(77, 10)
        gpu.k.copy_(k0)
        gpu.v.copy_(v0)
        b, tb = gpu.step(77, 10)
        assert np.array_equal(a, b) and ta == tb
        gpu.k.copy_(k0)
        gpu.v.copy_(v0)
        gpu.k[:, :, :, 11:, :] = 0x7FC0   # bf16 NaN
        gpu.v[:, :, :, 11:, :] = 0x7FC0
        c, tc = gpu.step(77, 10)
        assert np.array_equal(a, c) and ta == tc
    finally:
        gpu.close()


def test_error_paths(tiny_w):
    from persistent_megakernel_cu_amd import binding as mkb
    gpu = GpuDecoder(TINY, tiny_w, 48, mode="mega")
    try:
        with pytest.raises(mkb.MkError) as e:
            gpu.eng.decode_step(gpu.tok, 48, gpu.k, gpu.v, gpu.logits, gpu.out_tok)
        assert e.value.code == mkb.MK_E_RANGE
        with pytest.raises(mkb.MkError) as e:
            gpu.eng.decode_step(gpu.tok, -1, gpu.k, gpu.v, gpu.logits, gpu.out_tok)
        assert e.value.code == mkb.MK_E_RANGE
        # a bad token id is caught on the device: out_token = -1 and MK_E_TOKEN latched
        lg, out = gpu.step(TINY.vocab + 5, 0)
        assert out == -1
        st = gpu.eng.status()
        assert st.code == mkb.MK_E_TOKEN and st.detail == TINY.vocab + 5
        with pytest.raises(mkb.MkError) as e:
            gpu.step(1, 1)
        assert e.value.code == mkb.MK_E_STATE
        gpu.eng.reset()
        assert gpu.eng.status().code == 0
        lg, out = gpu.step(1, 0)
        assert out == int(np.argmax(lg))
    finally:
        gpu.close()


@pytest.mark.skip(reason="the first run of the Llama-8B shape (head_dim 128, hidden 4096) faulted the GPU; the "
                         "cause is not found yet (the host-side address walk of its plan finds every index in "
                         "bounds) and mk_load refuses head_dim 128 / hidden > 2048 until it is")
def test_llama8b_seeded_cache():
    # Llama-8B shape (head_dim 128, untied LM head) over a seeded 2048-slot
    # cache: two teacher-forced steps at positions 2048 and 2049
    import time

    from synth_inputs import LLAMA_8B

    sh = LLAMA_8B
    t0 = time.time()
    w = make_weights(sh, master=0)
    log(f"[8b] weights generated in {time.time() - t0:.0f}s")
    kv = make_kv_cache(sh, 1, 2112, 2048, master=0)
    o = orc.Oracle(sh, w, lazy=True)
    gpu = GpuDecoder(sh, w, 2112, mode="mega", kv_init=kv)
    log(f"[8b] engine loaded at {time.time() - t0:.0f}s")
    kc, vc = kv[0][0].copy(), kv[1][0].copy()
    tok = make_start_token(sh, 0)
    try:
        for pos in (2048, 2049):
            lg, out = gpu.step(tok, pos)
            lg_ref = o.decode_step(tok, pos, kc, vc)
            err = float(np.max(np.abs(lg.astype(np.float64) - lg_ref)))
            log(f"[parity] llama8b pos={pos} err/tol={err / logit_tol(lg_ref):.3g} at {time.time() - t0:.0f}s")
            assert err <= logit_tol(lg_ref)
            assert out == int(np.argmax(lg))
            ref_tok = orc.argmax_first(lg_ref)
            srt = np.sort(lg_ref)
            assert out == ref_tok or srt[-1] - srt[-2] < logit_tol(lg_ref)
            tok = ref_tok
    finally:
        gpu.close()


def test_llama8b_shape_refused():
    # mk_load refuses head_dim 128 / hidden > 2048 before touching any weight:
    # placeholder device buffers stand in for the 16 GB of weights
    import torch

    from persistent_megakernel_cu_amd import binding as mkb
    from synth_inputs import LLAMA_8B, weight_shapes

    dummy = torch.zeros(16, dtype=torch.int16, device="cuda")
    w = {name: dummy for name, _, _ in weight_shapes(LLAMA_8B)}
    with pytest.raises(mkb.MkError) as e:
        mkb.Engine(LLAMA_8B, w, 2112)
    assert e.value.code == mkb.MK_E_UNSUPPORTED


def test_large_arena_refused():
    # packed weights of 4 GiB or more are outside the envelope that has run
    # on the GPU (36 layers at Llama-1B widths pack 4.4 GB): refused before
    # any weight is read
    import torch

    from persistent_megakernel_cu_amd import binding as mkb
    from synth_inputs import weight_shapes

    sh = LLAMA_1B.with_(n_layers=36)
    assert mkb.plan_describe(sh, 256).weight_bytes >= 4 << 30
    dummy = torch.zeros(16, dtype=torch.int16, device="cuda")
    w = {name: dummy for name, _, _ in weight_shapes(sh)}
    with pytest.raises(mkb.MkError) as e:
        mkb.Engine(sh, w, 256)
    assert e.value.code == mkb.MK_E_UNSUPPORTED


def test_shallow_ring_plan_refused():
    # a batch-1 plan whose LDS does not fit beside the 14-unit weight ring (a
    # 14336-wide FFN activation) is described with 8 units and refused by
    # mk_load before any weight is read: the kernels carry the 14-unit ring
    import torch

    from persistent_megakernel_cu_amd import binding as mkb
    from synth_inputs import weight_shapes

    sh = TINY.with_(ffn=14336)
    assert mkb.plan_describe(sh, 48).ring_units == 8
    dummy = torch.zeros(16, dtype=torch.int16, device="cuda")
    w = {name: dummy for name, _, _ in weight_shapes(sh)}
    with pytest.raises(mkb.MkError) as e:
        mkb.Engine(sh, w, 48)
    assert e.value.code == mkb.MK_E_UNSUPPORTED


@pytest.mark.parametrize("mode", ["mega", "multi", "graph"])
def test_tiny_batched(tiny_w, mode):
    # 4 sequences with their own prompts, tiled weights and MFMA
    prompts = [make_prompt(TINY, 6, master=10 + n) for n in range(4)]
    run_batched_teacher_forced(TINY, tiny_w, 48, prompts, 0, 6, mode=mode, label="tiny-b4")


def test_tiny_batched_untied_chunked():
    # untied LM head, 3 sequences, attention split in 4 chunks per (sequence, kv head)
    sh = TINY.with_(tie_embeddings=False)
    w = make_weights(sh, master=4, gain_jitter=0.1)
    prompts = [make_prompt(sh, 5, master=20 + n) for n in range(3)]
    run_batched_teacher_forced(sh, w, 48, prompts, 0, 4, mode="mega", attn_chunks=4, label="tiny-b3-untied")


def test_tiny_batched_long_chunks(tiny_w):
    # 2 sequences over seeded 4000-slot caches, attention in 2 chunks of ~2000
    # positions: every wave walks about eight 32-position blocks, carrying its
    # softmax maximum, sum and P.V from block to block
    kv = make_kv_cache(TINY, 2, 4100, 4000, master=6)
    starts = [[make_start_token(TINY, n)] for n in range(2)]
    run_batched_teacher_forced(TINY, tiny_w, 4100, starts, 4000, 3, mode="mega", kv_init=kv, attn_chunks=2,
                               label="tiny-b2-long")


def test_llama1b_batch8_seeded_cache(llama1b):
    # batch 8 over seeded 1024-slot caches (attention chunks walked in blocks):
    # the start tokens at position 1024, then 8 greedy steps, every sequence
    # checked against its own oracle cache at every step
    w, o = llama1b
    kv = make_kv_cache(LLAMA_1B, 8, 1088, 1024, master=0)
    starts = [[make_start_token(LLAMA_1B, n)] for n in range(8)]
    run_batched_teacher_forced(LLAMA_1B, w, 1088, starts, 1024, 8, mode="mega", oracle_obj=o, kv_init=kv,
                               label="llama1b-b8")


@pytest.mark.parametrize("mode", ["mega", "multi"])
def test_tiny_mha_one_query_head_per_kv_head(mode):
    # n_heads == n_kv_heads (no grouping): the G = 1 kernel instance, batch 1
    sh = TINY.with_(n_kv_heads=4)
    w = make_weights(sh, master=5, gain_jitter=0.1)
    run_teacher_forced(sh, w, 48, make_prompt(sh, 10, master=5), 0, 8, mode=mode, label="tiny-mha")


def test_tiny_mha_batched():
    # n_heads == n_kv_heads with 2 sequences: the batched G = 1 instance
    sh = TINY.with_(n_kv_heads=4)
    w = make_weights(sh, master=6, gain_jitter=0.1)
    prompts = [make_prompt(sh, 5, master=30 + n) for n in range(2)]
    run_batched_teacher_forced(sh, w, 48, prompts, 0, 5, mode="mega", label="tiny-mha-b2")


def test_tiny_free_running_matches_golden():
    # Free-running greedy decode (each out_token is the next input) against the
    # oracle's stored run (tests/golden/tiny_greedy.json): tokens must agree up
    # to the first step whose top-2 margin is below the logit tolerance, where
    # either token is acceptable and the runs may part.
    import json
    import os

    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_greedy.json")) as f:
        gold = json.load(f)
    w = make_weights(TINY, master=0, gain_jitter=0.1)
    prompt = gold["prompt"]
    gpu = GpuDecoder(TINY, w, len(prompt) + len(gold["steps"]) + 1, mode="mega")
    try:
        for p, t in enumerate(prompt):
            lg, out = gpu.step(t, p)
        pos = len(prompt)
        compared = 0
        for i, st in enumerate(gold["steps"]):
            tol = 1e-2 * st["max_abs"]
            for idx, val in st["top"]:
                assert abs(float(lg[idx]) - val) <= tol, (i, idx, float(lg[idx]), val)
            margin = st["top"][0][1] - st["top"][1][1]
            if margin < tol:
                break
            assert out == gold["greedy_tokens"][i], (i, out, gold["greedy_tokens"][i])
            compared += 1
            if i + 1 < len(gold["steps"]):
                lg, out = gpu.step(out, pos)
                pos += 1
        log(f"[golden] tiny free-running: {compared} tokens equal to the stored oracle run")
        assert compared >= 4
    finally:
        gpu.close()


def test_watchdog_timeout_path(tiny_w):
    # A one-tick wait budget (negative watchdog_ms counts device clock ticks)
    # makes the first dependency wait that needs a second poll round give up:
    # the step latches MK_E_TIMEOUT with its stage and workgroup, raises the
    # abort flag, and every workgroup leaves its stage loop, so the kernel ends
    # normally.  Later steps are refused until mk_reset.
    from persistent_megakernel_cu_amd import binding as mkb

    gpu = GpuDecoder(TINY, tiny_w, 48, mode="mega", watchdog_ms=-1)
    try:
        st = None
        for p, t in enumerate(make_prompt(TINY, 4)):
            gpu.step(int(t), p)
            st = gpu.eng.status()
            if st.code != 0:
                break
        assert st.code == mkb.MK_E_TIMEOUT, st.code
        assert 0 <= st.stage < 5 * TINY.n_layers + 1 and 0 <= st.wg < 256
        log(f"[watchdog] timeout latched at stage {st.stage}, workgroup {st.wg}, last tag seen {st.detail}")
        with pytest.raises(mkb.MkError) as e:
            gpu.step(1, 0)
        assert e.value.code == mkb.MK_E_STATE
        gpu.eng.reset()
        assert gpu.eng.status().code == 0
    finally:
        gpu.close()
    # the device is unaffected: a handle with the normal budget decodes to parity
    run_teacher_forced(TINY, tiny_w, 48, make_prompt(TINY, 4), 0, 2, mode="mega", label="after-timeout")


def test_tiny_partial_input_down():
    # partial-input down projection (ffn 2048: rows of 4 units, 8 items per pair,
    # each wave staging a quarter of h); 16-token prompt and 8 greedy steps
    sh = TINY.with_(ffn=2048)
    w = make_weights(sh, master=12, gain_jitter=0.1)
    for mode in ("mega", "multi"):
        run_teacher_forced(sh, w, 48, make_prompt(sh, 16, master=12), 0, 8, mode=mode, partial_input=True,
                           label="tiny-partial")


def test_llama1b_partial_input_bench_workload(llama1b):
    # the benchmarked workload, whole, with the partial-input down projection
    w, o = llama1b
    reps = run_teacher_forced(LLAMA_1B, w, 256, make_prompt(LLAMA_1B, 128), 0, 128, mode="mega", oracle_obj=o,
                              partial_input=True, label="llama1b-partial-full")
    assert len(reps) == 256
