"""Multi-token resident decode (mk_decode_steps): one persistent launch runs N
greedy steps, the on-device argmax feeding the next embedding gather."""

import json
import os

import numpy as np
import pytest

import oracle as orc
from synth_inputs import LLAMA_1B, TINY, make_kv_cache, make_prompt, make_start_token, make_weights
from tests.parity import GpuDecoder, log, logit_tol, top2_margin

pytestmark = pytest.mark.gpu


def _chained_single_steps(gpu, first_tok, pos, n):
    """n greedy steps, one launch each, the token chained on the device."""
    import torch

    B = gpu.tok.numel()
    toks = torch.empty((n, B), dtype=torch.int32, device="cuda")
    lgs = torch.empty((n, B, gpu.shape.vocab), dtype=torch.float32, device="cuda")
    gpu.tok.copy_(first_tok)
    for i in range(n):
        gpu.eng.decode_step(gpu.tok if i == 0 else toks[i - 1], pos + i, gpu.k, gpu.v, lgs[i], toks[i])
    torch.cuda.synchronize()
    return lgs.cpu().numpy(), toks.cpu().numpy()


def _multi_steps(gpu, first_tok, pos, n, with_logits=True):
    import torch

    B = gpu.tok.numel()
    toks = torch.empty((n, B), dtype=torch.int32, device="cuda")
    lgs = torch.empty((n, B, gpu.shape.vocab), dtype=torch.float32, device="cuda") if with_logits else None
    gpu.tok.copy_(first_tok)
    gpu.eng.decode_steps(gpu.tok, pos, n, gpu.k, gpu.v, toks, lgs)
    torch.cuda.synchronize()
    return (lgs.cpu().numpy() if with_logits else None), toks.cpu().numpy()


def _decoder(shape, w, max_seq, batch, kv, mode="mega"):
    import torch

    gpu = GpuDecoder(shape, w, max_seq, mode=mode, kv_init=kv, batch=batch)
    gpu.tok = torch.zeros(batch, dtype=torch.int32, device="cuda")
    return gpu


@pytest.mark.parametrize("batch", [1, 4])
def test_tiny_steps_bit_identical_to_chained_launches(batch):
    import torch

    sh = TINY
    w = make_weights(sh, master=0, gain_jitter=0.1)
    kv = make_kv_cache(sh, batch, 64, 20, master=1)
    first = torch.tensor([make_start_token(sh, b, master=1) for b in range(batch)], dtype=torch.int32,
                         device="cuda")
    a = _decoder(sh, w, 64, batch, kv)
    b = _decoder(sh, w, 64, batch, kv)
    try:
        lg1, tk1 = _chained_single_steps(a, first, 20, 24)
        lg2, tk2 = _multi_steps(b, first, 20, 24)
        assert np.array_equal(tk1, tk2) and np.array_equal(lg1, lg2)
        assert np.array_equal(a.k.cpu().numpy(), b.k.cpu().numpy())
        assert np.array_equal(a.v.cpu().numpy(), b.v.cpu().numpy())
        # no logits requested: the same tokens
        c = _decoder(sh, w, 64, batch, kv)
        try:
            _, tk3 = _multi_steps(c, first, 20, 24, with_logits=False)
            assert np.array_equal(tk1, tk3)
        finally:
            c.close()
    finally:
        a.close()
        b.close()
    log(f"[steps] tiny batch {batch}: 24 steps in one launch bit-identical to 24 chained launches")


def test_tiny_steps_free_running_matches_golden():
    # the oracle's stored greedy run (tests/golden/tiny_greedy.json) from one multi-step launch
    import torch

    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_greedy.json")) as f:
        gold = json.load(f)
    w = make_weights(TINY, master=0, gain_jitter=0.1)
    prompt = gold["prompt"]
    n = len(gold["steps"])
    gpu = GpuDecoder(TINY, w, len(prompt) + n + 1, mode="mega")
    try:
        for p, t in enumerate(prompt[:-1]):
            gpu.step(t, p)
        lg, tk = _multi_steps(gpu, torch.tensor([prompt[-1]], dtype=torch.int32, device="cuda"), len(prompt) - 1, n)
        compared = 0
        for i, st in enumerate(gold["steps"]):
            tol = 1e-2 * st["max_abs"]
            for idx, val in st["top"]:
                assert abs(float(lg[i, 0, idx]) - val) <= tol, (i, idx)
            if st["top"][0][1] - st["top"][1][1] < tol:
                break
            assert int(tk[i, 0]) == gold["greedy_tokens"][i], (i, int(tk[i, 0]))
            compared += 1
        log(f"[steps] tiny free-running in one launch: {compared} tokens equal to the stored oracle run")
        assert compared >= 4
    finally:
        gpu.close()


def test_llama1b_steps_free_running_against_oracle():
    # Llama-1B shape: the 128-token prompt prefilled step by step, then 32
    # greedy steps in one launch; every step's logits against the oracle's
    # free-running run (same tokens until the first step whose top-2 margin is
    # below the tolerance, where the runs may part), and bit-identical to 32
    # chained single-step launches from the same state
    import torch

    sh = LLAMA_1B
    w = make_weights(sh, master=0)
    o = orc.Oracle(sh, w)
    prompt = make_prompt(sh, 128)
    a = GpuDecoder(sh, w, 256, mode="mega")
    kc, vc = o.new_cache(256)
    try:
        for p, t in enumerate(prompt[:-1]):
            a.step(int(t), p)
            o.decode_step(int(t), p, kc, vc)
        k0, v0 = a.k.clone(), a.v.clone()
        first = torch.tensor([int(prompt[-1])], dtype=torch.int32, device="cuda")
        lg, tk = _multi_steps(a, first, 127, 32)
        tok = int(prompt[-1])
        agree = 0
        for i in range(32):
            ref = o.decode_step(tok, 127 + i, kc, vc)
            err = float(np.max(np.abs(lg[i, 0].astype(np.float64) - ref)))
            assert err <= logit_tol(ref), (i, err, logit_tol(ref))
            gt = orc.argmax_first(ref)
            if int(tk[i, 0]) != gt:
                assert top2_margin(ref) < logit_tol(ref), (i, int(tk[i, 0]), gt)
                break
            agree += 1
            tok = gt
        log(f"[steps] llama1b: {agree} greedy tokens of one 32-step launch equal to the oracle's free-running run")
        a.k.copy_(k0)
        a.v.copy_(v0)
        lg2, tk2 = _chained_single_steps(a, first, 127, 32)
        assert np.array_equal(tk, tk2) and np.array_equal(lg, lg2)
    finally:
        a.close()


@pytest.mark.parametrize("mode", ["graph", "conv"])
def test_tiny_steps_other_modes(mode):
    # the other modes issue the steps one by one: same greedy tokens as the megakernel's single launch
    import torch

    sh = TINY
    w = make_weights(sh, master=0, gain_jitter=0.1)
    kv = make_kv_cache(sh, 1, 64, 20, master=1)
    first = torch.tensor([make_start_token(sh, 0, master=1)], dtype=torch.int32, device="cuda")
    a = _decoder(sh, w, 64, 1, kv)
    b = _decoder(sh, w, 64, 1, kv, mode=mode)
    try:
        lg1, tk1 = _multi_steps(a, first, 20, 12)
        lg2, tk2 = _multi_steps(b, first, 20, 12)
        for i in range(12):
            assert np.max(np.abs(lg1[i, 0] - lg2[i, 0])) <= 2 * logit_tol(lg1[i, 0])
            if tk1[i, 0] != tk2[i, 0]:
                assert top2_margin(lg1[i, 0]) < 2 * logit_tol(lg1[i, 0])
                break
    finally:
        a.close()
        b.close()


def test_steps_bad_token_and_range():
    import torch

    from persistent_megakernel_cu_amd import binding as mkb

    sh = TINY
    w = make_weights(sh, master=0)
    gpu = _decoder(sh, w, 32, 1, None)
    try:
        toks = torch.empty((4, 1), dtype=torch.int32, device="cuda")
        with pytest.raises(mkb.MkError) as e:
            gpu.eng.decode_steps(gpu.tok, 30, 4, gpu.k, gpu.v, toks)
        assert e.value.code == mkb.MK_E_RANGE
        gpu.tok.fill_(sh.vocab + 1)
        gpu.eng.decode_steps(gpu.tok, 0, 4, gpu.k, gpu.v, toks)
        torch.cuda.synchronize()
        assert int(toks[0, 0]) == -1
        assert gpu.eng.status().code == mkb.MK_E_TOKEN
        gpu.eng.reset()
        gpu.tok.fill_(7)
        gpu.eng.decode_steps(gpu.tok, 0, 4, gpu.k, gpu.v, toks)
        torch.cuda.synchronize()
        assert gpu.eng.status().code == 0 and int(toks[0, 0]) >= 0
    finally:
        gpu.close()
