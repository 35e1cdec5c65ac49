"""GPU parity of prefill inside the megakernel (mk_config.prefill: the batch
is the next B prompt tokens of one sequence, run as the batched MFMA GEMM
tasks with causal attention over the cache and the step's own tokens)
against the oracle, which runs the same tokens one decode step at a time.

Per token: logits within the decode tolerance, out_token == the first argmax
of its own logits; per call: the cache changes only at slots pos .. pos+B-1,
and those slots match the oracle's within the decode tolerance."""

import numpy as np
import pytest

import oracle as orc
from synth_inputs import LLAMA_1B, TINY, make_kv_cache, make_prompt, make_weights
from tests.parity import LOGIT_RTOL, GpuDecoder, log, logit_tol

pytestmark = pytest.mark.gpu


class Prefiller:
    """A prefill handle (batch = chunk tokens of one sequence) and that sequence's cache."""

    def __init__(self, shape, weights_np, max_seq, chunk, mode="mega", kv_init=None, wd=None, attn_chunks=0):
        import torch

        from persistent_megakernel_cu_amd import binding as mkb

        self.torch = torch
        self.T = chunk
        self.wd = wd if wd is not None else mkb.to_device(weights_np)
        self.eng = mkb.Engine(shape, self.wd, max_seq, mode=mode, batch=chunk, prefill=True, attn_chunks=attn_chunks)
        dims = (1, shape.n_layers, shape.n_kv_heads, max_seq, shape.head_dim)
        if kv_init is None:
            self.k = torch.zeros(dims, dtype=torch.int16, device="cuda")
            self.v = torch.zeros(dims, dtype=torch.int16, device="cuda")
        else:
            self.k = torch.from_numpy(kv_init[0][:1].view(np.int16)).cuda()
            self.v = torch.from_numpy(kv_init[1][:1].view(np.int16)).cuda()
        self.logits = torch.empty((chunk, shape.vocab), dtype=torch.float32, device="cuda")
        self.out = torch.empty(chunk, dtype=torch.int32, device="cuda")
        self.tok = torch.empty(chunk, dtype=torch.int32, device="cuda")

    def run(self, tokens, pos):
        self.tok.copy_(self.torch.tensor([int(t) for t in tokens], dtype=self.torch.int32))
        self.eng.decode_step(self.tok, pos, self.k, self.v, self.logits, self.out)
        self.torch.cuda.synchronize()
        return self.logits.cpu().numpy().copy(), [int(x) for x in self.out.cpu().tolist()]

    def cache_np(self):
        return (self.k.cpu().numpy().view(np.uint16)[0].copy(), self.v.cpu().numpy().view(np.uint16)[0].copy())

    def close(self):
        self.eng.close()


def check_chunk(pos, T, lg, out, lg_refs, before, after, ref_cache):
    worst = 0.0
    for i in range(T):
        err = float(np.max(np.abs(lg[i].astype(np.float64) - lg_refs[i])))
        tol = logit_tol(lg_refs[i])
        assert np.all(np.isfinite(lg[i])), f"pos {pos + i}: non-finite logits"
        assert err <= tol, f"pos {pos + i}: max|dlogit| {err:.4g} > tol {tol:.4g}"
        assert out[i] == int(np.argmax(lg[i])), f"pos {pos + i}: out_token is not the argmax of its logits"
        worst = max(worst, err / tol)
    for which in (0, 1):
        b, a, r = before[which], after[which], ref_cache[which]
        mask = np.ones(a.shape, dtype=bool)
        mask[:, :, pos:pos + T, :] = False
        assert np.array_equal(a[mask], b[mask]), f"chunk at {pos}: cache changed outside its slots"
        ga = orc.bf16_to_f32(a[:, :, pos:pos + T, :]).astype(np.float64)
        ra = orc.bf16_to_f32(r[:, :, pos:pos + T, :]).astype(np.float64)
        e = float(np.max(np.abs(ga - ra)))
        assert e <= LOGIT_RTOL * float(np.max(np.abs(ra))), f"chunk at {pos}: {'KV'[which]} slots differ by {e:.4g}"
    return worst


def run_prefill(shape, w, max_seq, prompt, start, chunk, mode="mega", o=None, kv_init=None, label="", attn_chunks=0):
    """Prefill ``prompt`` from ``start`` in calls of ``chunk`` tokens, each
    compared with the oracle's step-by-step run; returns the prefiller (open)
    and the oracle's cache after the prompt."""
    o = o or orc.Oracle(shape, w)
    if kv_init is None:
        kc, vc = o.new_cache(max_seq)
    else:
        kc, vc = kv_init[0][0].copy(), kv_init[1][0].copy()
    pf = Prefiller(shape, w, max_seq, chunk, mode=mode, kv_init=kv_init, attn_chunks=attn_chunks)
    worst = 0.0
    assert len(prompt) % chunk == 0
    lg_refs = []
    for c0 in range(0, len(prompt), chunk):
        toks = prompt[c0:c0 + chunk]
        pos = start + c0
        before = pf.cache_np()
        lg, out = pf.run(toks, pos)
        after = pf.cache_np()
        lg_refs = [o.decode_step(int(t), pos + i, kc, vc) for i, t in enumerate(toks)]
        worst = max(worst, check_chunk(pos, chunk, lg, out, lg_refs, before, after, (kc, vc)))
    log(f"[prefill] {label} mode={mode} tokens={len(prompt)} chunk={chunk} worst err/tol={worst:.3g}")
    return pf, (kc, vc), lg_refs[-1]


@pytest.fixture(scope="module")
def tiny_w():
    return make_weights(TINY, master=0, gain_jitter=0.1)


@pytest.mark.parametrize("mode", ["mega", "graph", "multi"])
def test_tiny_prefill_from_zero(tiny_w, mode):
    pf, _, _ = run_prefill(TINY, tiny_w, 48, list(make_prompt(TINY, 16, master=3)), 0, 4, mode=mode, label="tiny")
    pf.close()


@pytest.mark.parametrize("chunk", [2, 8])
def test_tiny_prefill_chunk_sizes_over_a_seeded_cache(tiny_w, chunk):
    # a seeded 20-slot cache, the prompt from position 20; 600 slots: three
    # attention chunks per kv head, merged
    kv = make_kv_cache(TINY, 1, 600, 20, master=4)
    pf, _, _ = run_prefill(TINY, tiny_w, 600, list(make_prompt(TINY, 16, master=4)), 20, chunk, kv_init=kv,
                           label=f"tiny-seeded-c{chunk}")
    pf.close()


def test_tiny_prefill_over_a_long_cache(tiny_w):
    # a seeded 4000-slot cache, 8-token prefill calls from position 4000, 2
    # attention chunks of ~2000 positions: every wave walks several 32-position
    # blocks, and the last block mixes cached slots with the call's own rows
    kv = make_kv_cache(TINY, 1, 4100, 4000, master=9)
    pf, _, _ = run_prefill(TINY, tiny_w, 4100, list(make_prompt(TINY, 16, master=9)), 4000, 8, kv_init=kv,
                           label="tiny-long-c8", attn_chunks=2)
    pf.close()


def test_tiny_prefill_mha_untied():
    sh = TINY.with_(tie_embeddings=False, n_kv_heads=4)
    w = make_weights(sh, master=8, gain_jitter=0.1)
    pf, _, _ = run_prefill(sh, w, 48, list(make_prompt(sh, 8, master=8)), 0, 4, label="tiny-mha-untied")
    pf.close()


def test_llama1b_prompt_then_decode():
    # the benchmarked workload's 128-token prompt in 16 calls of 8 tokens,
    # then greedy decode steps on the batch-1 megakernel from the prefilled cache
    w = make_weights(LLAMA_1B, master=0)
    o = orc.Oracle(LLAMA_1B, w)
    prompt = list(make_prompt(LLAMA_1B, 128))
    pf, (kc, vc), last_ref = run_prefill(LLAMA_1B, w, 256, prompt, 0, 8, o=o, label="llama1b-128")
    try:
        kv = pf.cache_np()
    finally:
        pf.close()
    kv_init = (kv[0][None], kv[1][None])
    dec = GpuDecoder(LLAMA_1B, w, 256, mode="mega", kv_init=kv_init)
    try:
        tok = orc.argmax_first(last_ref)   # teacher forced: the oracle's greedy token after the prompt
        for pos in range(128, 136):
            lg, out = dec.step(tok, pos)
            lg_ref = o.decode_step(tok, pos, kc, vc)
            assert float(np.max(np.abs(lg - lg_ref))) <= logit_tol(lg_ref)
            assert out == int(np.argmax(lg))
            tok = orc.argmax_first(lg_ref)
    finally:
        dec.close()


def test_prefill_refusals(tiny_w):
    import torch

    from persistent_megakernel_cu_amd import binding as mkb

    wd = mkb.to_device(tiny_w)
    for kw in ({"batch": 1}, {"batch": 4, "mode": "conv"}, {"batch": 9}):
        with pytest.raises(mkb.MkError) as e:
            mkb.Engine(TINY, wd, 48, prefill=True, **kw)
        assert e.value.code in (mkb.MK_E_UNSUPPORTED, mkb.MK_E_INVAL)
    pf = Prefiller(TINY, tiny_w, 48, 4, wd=wd)
    try:
        with pytest.raises(mkb.MkError) as e:      # positions 45..48 do not fit 48 slots
            pf.eng.decode_step(pf.tok, 45, pf.k, pf.v, pf.logits, pf.out)
        assert e.value.code == mkb.MK_E_RANGE
        out = torch.empty((2, 4), dtype=torch.int32, device="cuda")
        with pytest.raises(mkb.MkError) as e:      # multi-step launches are for decode handles
            pf.eng.decode_steps(pf.tok, 0, 2, pf.k, pf.v, out)
        assert e.value.code == mkb.MK_E_UNSUPPORTED
        lg, outs = pf.run([1, 2, 3, 4], 44)       # the last positions that fit
        assert outs == [int(np.argmax(x)) for x in lg]
    finally:
        pf.close()
