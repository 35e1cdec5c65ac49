"""GPU parity of the conventional one-kernel-per-operation path (an
independent second GPU implementation: eager launches, and the same launches
captured in a hipGraph) against the CPU oracle, through the C ABI."""

import numpy as np
import pytest

import oracle as orc
from synth_inputs import LLAMA_1B, TINY, make_kv_cache, make_prompt, make_start_token, make_weights
from tests.parity import GpuDecoder, check_step, log, run_batched_teacher_forced, run_teacher_forced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny_w():
    return make_weights(TINY, master=0, gain_jitter=0.1)


@pytest.mark.parametrize("mode", ["conv", "conv-graph"])
def test_conv_tiny_prompt_and_greedy(tiny_w, mode):
    run_teacher_forced(TINY, tiny_w, 48, make_prompt(TINY, 16), 0, 16, mode=mode, label="conv-tiny")


def test_conv_tiny_untied_mha():
    sh = TINY.with_(tie_embeddings=False, n_kv_heads=4)
    w = make_weights(sh, master=8, gain_jitter=0.1)
    run_teacher_forced(sh, w, 48, make_prompt(sh, 6, master=8), 0, 6, mode="conv", label="conv-tiny-untied-mha")


def test_conv_tiny_long_chunks():
    # 600 slots: attention runs 3 chunks of 256 positions and merges them
    sh = TINY
    w = make_weights(sh, master=9, gain_jitter=0.1)
    kv = make_kv_cache(sh, 1, 600, 540, master=9)
    run_teacher_forced(sh, w, 600, [make_start_token(sh, 0, master=9)], 540, 6, mode="conv-graph", kv_init=kv,
                       label="conv-tiny-3chunks")


@pytest.mark.parametrize("mode", ["conv", "conv-graph"])
def test_conv_tiny_batched(tiny_w, mode):
    prompts = [make_prompt(TINY, 6, master=40 + n) for n in range(4)]
    run_batched_teacher_forced(TINY, tiny_w, 48, prompts, 0, 6, mode=mode, label="conv-tiny-b4")


@pytest.fixture(scope="module")
def llama1b():
    w = make_weights(LLAMA_1B, master=0)
    return w, orc.Oracle(LLAMA_1B, w)


def test_conv_llama1b_bench_workload_full(llama1b):
    # the benchmarked workload, whole: 128-token prompt then 128 greedy steps
    w, o = llama1b
    reps = run_teacher_forced(LLAMA_1B, w, 256, make_prompt(LLAMA_1B, 128), 0, 128, mode="conv-graph", oracle_obj=o,
                              label="conv-llama1b-bench-full")
    assert len(reps) == 256


def test_conv_llama1b_long_context(llama1b):
    sh = LLAMA_1B
    w, o = llama1b
    kv = make_kv_cache(sh, 1, 8192, 8192, master=0)
    tok = make_start_token(sh, 0)
    gpu = GpuDecoder(sh, w, 8192, mode="conv", kv_init=kv)
    kc, vc = kv[0][0].copy(), kv[1][0].copy()
    try:
        for pos in (4096, 8191):
            before = gpu.cache_np()
            lg, out = gpu.step(tok, pos)
            after = gpu.cache_np()
            lg_ref = o.decode_step(tok, pos, kc, vc)
            rep = check_step(pos, lg, out, lg_ref, before, after, (kc, vc))
            log(f"[parity] conv long pos={pos} err/tol={rep.max_abs_err / rep.tol:.3g}")
            assert out == rep.oracle_token or rep.margin < rep.tol
    finally:
        gpu.close()


def test_conv_llama1b_batch8(llama1b):
    w, o = llama1b
    kv = make_kv_cache(LLAMA_1B, 8, 1088, 1024, master=0)
    starts = [[make_start_token(LLAMA_1B, n)] for n in range(8)]
    run_batched_teacher_forced(LLAMA_1B, w, 1088, starts, 1024, 3, mode="conv-graph", oracle_obj=o, kv_init=kv,
                               label="conv-llama1b-b8")


@pytest.mark.parametrize("mode", ["conv", "conv-graph"])
def test_conv_tiny_head_dim_128(mode):
    # head_dim 128 (16 threads per K/V row in attention), untied
    sh = TINY.with_(head_dim=128, tie_embeddings=False)
    w = make_weights(sh, master=11, gain_jitter=0.1)
    run_teacher_forced(sh, w, 48, make_prompt(sh, 8, master=11), 0, 8, mode=mode, label="conv-tiny-d128")


def test_conv_llama8b_seeded_cache():
    # the Llama-8B shape (head_dim 128, hidden 4096, untied LM head) on the
    # conventional path: two teacher-forced steps at positions 2048 and 2049
    # over a seeded 2048-slot cache, logits, tokens and cache slots checked
    import time

    from synth_inputs import LLAMA_8B

    sh = LLAMA_8B
    t0 = time.time()
    w = make_weights(sh, master=0)
    log(f"[conv-8b] weights generated in {time.time() - t0:.0f}s")
    kv = make_kv_cache(sh, 1, 2112, 2048, master=0)
    o = orc.Oracle(sh, w, lazy=True)
    gpu = GpuDecoder(sh, w, 2112, mode="conv", kv_init=kv)
    log(f"[conv-8b] engine loaded at {time.time() - t0:.0f}s")
    kc, vc = kv[0][0].copy(), kv[1][0].copy()
    tok = make_start_token(sh, 0)
    try:
        for pos in (2048, 2049):
            before = gpu.cache_np()
            lg, out = gpu.step(tok, pos)
            after = gpu.cache_np()
            log(f"[conv-8b] gpu step at {pos} done at {time.time() - t0:.0f}s")
            lg_ref = o.decode_step(tok, pos, kc, vc)
            rep = check_step(pos, lg, out, lg_ref, before, after, (kc, vc))
            log(f"[parity] conv llama8b pos={pos} err/tol={rep.max_abs_err / rep.tol:.3g} at {time.time() - t0:.0f}s")
            assert out == rep.oracle_token or rep.margin < rep.tol
            tok = rep.oracle_token
    finally:
        gpu.close()


def test_conv_bad_token(tiny_w):
    gpu = GpuDecoder(TINY, tiny_w, 48, mode="conv")
    try:
        lg, out = gpu.step(TINY.vocab + 3, 0)
        assert out == -1
        lg, out = gpu.step(5, 1)
        assert out == int(np.argmax(lg))
    finally:
        gpu.close()


def test_conv_stateless_call_matches_handle(tiny_w):
    # mk_conv_decode_step called directly with a caller workspace gives the
    # same bits as the handle's MK_MODE_CONV on the same inputs
    import torch

    from persistent_megakernel_cu_amd import binding as mkb

    sh = TINY
    wd = mkb.to_device(tiny_w)
    kv = make_kv_cache(sh, 2, 64, 20, master=2)
    toks = [17, 900]
    gpu = GpuDecoder(sh, tiny_w, 64, mode="conv", kv_init=kv, batch=2)
    try:
        gpu.tok = torch.tensor(toks, dtype=torch.int32, device="cuda")
        gpu.logits = torch.empty((2, sh.vocab), dtype=torch.float32, device="cuda")
        gpu.out_tok = torch.empty(2, dtype=torch.int32, device="cuda")
        gpu.eng.decode_step(gpu.tok, 20, gpu.k, gpu.v, gpu.logits, gpu.out_tok)
        torch.cuda.synchronize()
        ref_lg, ref_tok = gpu.logits.cpu().numpy(), gpu.out_tok.cpu().numpy()
        ref_k, ref_v = gpu.k.cpu().numpy(), gpu.v.cpu().numpy()
    finally:
        gpu.close()
    k = torch.from_numpy(kv[0].view(np.int16)).cuda()
    v = torch.from_numpy(kv[1].view(np.int16)).cuda()
    ws = torch.empty(mkb.conv_workspace_size(sh, 64, 2) // 4, dtype=torch.float32, device="cuda")
    d_pos = torch.tensor([20], dtype=torch.int32, device="cuda")
    tok = torch.tensor(toks, dtype=torch.int32, device="cuda")
    lg = torch.empty((2, sh.vocab), dtype=torch.float32, device="cuda")
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    mkb.conv_decode_step(sh, wd, 64, tok, d_pos, k, v, lg, out, ws, batch=2)
    torch.cuda.synchronize()
    assert np.array_equal(lg.cpu().numpy(), ref_lg) and np.array_equal(out.cpu().numpy(), ref_tok)
    assert np.array_equal(k.cpu().numpy(), ref_k) and np.array_equal(v.cpu().numpy(), ref_v)
