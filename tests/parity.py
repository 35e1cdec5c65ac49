"""GPU-vs-oracle parity harness (test infrastructure).

Acceptance per decode step (teacher forced: the oracle's token is fed to both
sides, so every step compares identical inputs):
  * logits: max|gpu - oracle| <= 1e-2 * max|oracle|;
  * out_token equals the first index of the maximum of the GPU's own logits;
  * the KV cache changes only at slot pos of every (layer, kv head), and
    those slots are within 1e-2 * max|K_oracle| (resp. V) of the oracle's;
  * the greedy token equals the oracle's argmax unless the oracle's top-2
    margin is below the logit tolerance.
"""

from __future__ import annotations

import dataclasses
import sys

import numpy as np

import oracle as orc

LOGIT_RTOL = 1e-2


def logit_tol(ref: np.ndarray) -> float:
    return LOGIT_RTOL * float(np.max(np.abs(ref)))


def top2_margin(x: np.ndarray) -> float:
    a = np.partition(x, -2)[-2:]
    return float(a[1] - a[0])


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class GpuDecoder:
    """A mk Engine plus device buffers for one sequence."""

    def __init__(self, shape, weights_np: dict, max_seq: int, mode: str = "mega", kv_init=None, **kw):
        import torch
        from persistent_megakernel_cu_amd import binding as mkb

        self.torch = torch
        self.shape = shape
        self.max_seq = max_seq
        self.wd = mkb.to_device(weights_np)
        self.eng = mkb.Engine(shape, self.wd, max_seq, mode=mode, **kw)
        dims = (1, shape.n_layers, shape.n_kv_heads, max_seq, shape.head_dim)
        if kv_init is None:
            self.k = torch.zeros(dims, dtype=torch.int16, device="cuda")
            self.v = torch.zeros(dims, dtype=torch.int16, device="cuda")
        else:
            self.k = torch.from_numpy(kv_init[0].view(np.int16)).cuda()
            self.v = torch.from_numpy(kv_init[1].view(np.int16)).cuda()
        self.logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
        self.out_tok = torch.empty(1, dtype=torch.int32, device="cuda")
        self.tok = torch.empty(1, dtype=torch.int32, device="cuda")

    def step(self, token: int, pos: int):
        self.tok.fill_(int(token))
        self.eng.decode_step(self.tok, pos, self.k, self.v, self.logits, self.out_tok)
        self.torch.cuda.synchronize()
        return self.logits.cpu().numpy()[0].copy(), int(self.out_tok.cpu().item())

    def cache_np(self):
        return (self.k.cpu().numpy().view(np.uint16)[0].copy(), self.v.cpu().numpy().view(np.uint16)[0].copy())

    def close(self):
        self.eng.close()


@dataclasses.dataclass
class StepReport:
    pos: int
    max_abs_err: float
    tol: float
    gpu_token: int
    oracle_token: int
    margin: float
    cache_ok: bool
    kv_err: float


def check_step(pos, lg_gpu, tok_gpu, lg_ref, before, after, ref_cache, check_cache=True) -> StepReport:
    err = float(np.max(np.abs(lg_gpu.astype(np.float64) - lg_ref.astype(np.float64))))
    tol = logit_tol(lg_ref)
    assert np.all(np.isfinite(lg_gpu)), f"pos {pos}: non-finite GPU logits"
    assert err <= tol, f"pos {pos}: max|dlogit| {err:.4g} > tol {tol:.4g}"
    # out_token is the first argmax of the GPU's own logits, bit-exact
    assert tok_gpu == int(np.argmax(lg_gpu)), f"pos {pos}: out_token {tok_gpu} != argmax {int(np.argmax(lg_gpu))}"
    kv_err = 0.0
    cache_ok = True
    if check_cache:
        for which in (0, 1):
            b, a, r = before[which], after[which], ref_cache[which]
            mask = np.ones(a.shape, dtype=bool)
            mask[:, :, pos, :] = False
            same = np.array_equal(a[mask], b[mask])
            assert same, f"pos {pos}: cache changed outside slot pos ({'KV'[which]})"
            ga = orc.bf16_to_f32(a[:, :, pos, :]).astype(np.float64)
            ra = orc.bf16_to_f32(r[:, :, pos, :]).astype(np.float64)
            e = float(np.max(np.abs(ga - ra)))
            t = LOGIT_RTOL * float(np.max(np.abs(ra)))
            assert e <= t, f"pos {pos}: {'KV'[which]} slot error {e:.4g} > {t:.4g}"
            kv_err = max(kv_err, e / max(t, 1e-30))
    ref_tok = orc.argmax_first(lg_ref)
    return StepReport(pos, err, tol, tok_gpu, ref_tok, top2_margin(lg_ref), cache_ok, kv_err)


def run_teacher_forced(shape, weights_np, max_seq, tokens_in, start_pos, n_steps, mode="mega", oracle_obj=None,
                       kv_init=None, check_cache=True, label="", **kw):
    """Feed ``tokens_in`` (prompt) then the oracle's greedy tokens for n_steps.

    Returns the list of StepReports for every position run.
    """
    o = oracle_obj or orc.Oracle(shape, weights_np)
    if kv_init is None:
        kc, vc = o.new_cache(max_seq)
    else:
        kc, vc = kv_init[0][0].copy(), kv_init[1][0].copy()
    gpu = GpuDecoder(shape, weights_np, max_seq, mode=mode, kv_init=kv_init, **kw)
    reports = []
    try:
        seq = list(tokens_in)
        pos = start_pos
        i = 0
        while i < len(seq):
            t = seq[i]
            before = gpu.cache_np() if check_cache else None
            lg_gpu, tok_gpu = gpu.step(t, pos)
            after = gpu.cache_np() if check_cache else None
            lg_ref = o.decode_step(int(t), pos, kc, vc)
            rep = check_step(pos, lg_gpu, tok_gpu, lg_ref, before, after, (kc, vc), check_cache)
            reports.append(rep)
            if i == len(seq) - 1 and len(seq) < len(tokens_in) + n_steps:
                seq.append(rep.oracle_token)
            pos += 1
            i += 1
        mism = [r for r in reports[len(tokens_in) - 1:] if r.gpu_token != r.oracle_token]
        for r in mism:
            assert r.margin < r.tol, f"pos {r.pos}: greedy token {r.gpu_token} != oracle {r.oracle_token} " \
                                     f"with margin {r.margin:.4g} >= tol {r.tol:.4g}"
        worst = max(r.max_abs_err / r.tol for r in reports)
        log(f"[parity] {label} mode={mode} steps={len(reports)} worst err/tol={worst:.3g} "
            f"token mismatches (all below margin)={len(mism)}")
    finally:
        gpu.close()
    return reports


class BatchDecoder:
    """A batched mk Engine: B sequences share the position, each with its own cache slice."""

    def __init__(self, shape, weights_np: dict, max_seq: int, batch: int, mode: str = "mega", kv_init=None, **kw):
        import torch
        from persistent_megakernel_cu_amd import binding as mkb

        self.torch = torch
        self.shape = shape
        self.B = batch
        self.wd = mkb.to_device(weights_np)
        self.eng = mkb.Engine(shape, self.wd, max_seq, mode=mode, batch=batch, **kw)
        dims = (batch, shape.n_layers, shape.n_kv_heads, max_seq, shape.head_dim)
        if kv_init is None:
            self.k = torch.zeros(dims, dtype=torch.int16, device="cuda")
            self.v = torch.zeros(dims, dtype=torch.int16, device="cuda")
        else:
            self.k = torch.from_numpy(kv_init[0].view(np.int16)).cuda()
            self.v = torch.from_numpy(kv_init[1].view(np.int16)).cuda()
        self.logits = torch.empty((batch, shape.vocab), dtype=torch.float32, device="cuda")
        self.out_tok = torch.empty(batch, dtype=torch.int32, device="cuda")
        self.tok = torch.empty(batch, dtype=torch.int32, device="cuda")

    def step(self, tokens, pos: int):
        self.tok.copy_(self.torch.tensor([int(t) for t in tokens], dtype=self.torch.int32))
        self.eng.decode_step(self.tok, pos, self.k, self.v, self.logits, self.out_tok)
        self.torch.cuda.synchronize()
        return self.logits.cpu().numpy().copy(), [int(x) for x in self.out_tok.cpu().tolist()]

    def cache_np(self):
        return (self.k.cpu().numpy().view(np.uint16).copy(), self.v.cpu().numpy().view(np.uint16).copy())

    def close(self):
        self.eng.close()


def run_batched_teacher_forced(shape, weights_np, max_seq, prompts, start_pos, n_steps, mode="mega", oracle_obj=None,
                               kv_init=None, label="", **kw):
    """B sequences at one shared position: feed each sequence's prompt, then the
    oracle's greedy tokens; every step checks every sequence against its own
    oracle cache (logit tolerance, out_token == own argmax, cache slots)."""
    o = oracle_obj or orc.Oracle(shape, weights_np)
    B = len(prompts)
    if kv_init is None:
        caches = [o.new_cache(max_seq) for _ in range(B)]
    else:
        caches = [(kv_init[0][n].copy(), kv_init[1][n].copy()) for n in range(B)]
    gpu = BatchDecoder(shape, weights_np, max_seq, B, mode=mode, kv_init=kv_init, **kw)
    worst = 0.0
    mism = 0
    try:
        seqs = [list(p) for p in prompts]
        plen = len(seqs[0])
        pos = start_pos
        for i in range(plen + n_steps):
            toks = [s[i] for s in seqs]
            before = gpu.cache_np()
            lg, outs = gpu.step(toks, pos)
            after = gpu.cache_np()
            for n in range(B):
                kc, vc = caches[n]
                lg_ref = o.decode_step(int(toks[n]), pos, kc, vc)
                rep = check_step(pos, lg[n], outs[n], lg_ref, (before[0][n], before[1][n]),
                                 (after[0][n], after[1][n]), (kc, vc))
                worst = max(worst, rep.max_abs_err / rep.tol)
                if i >= plen - 1:
                    if rep.gpu_token != rep.oracle_token:
                        assert rep.margin < rep.tol, (f"seq {n} pos {pos}: greedy token {rep.gpu_token} != oracle "
                                                      f"{rep.oracle_token} with margin {rep.margin:.4g}")
                        mism += 1
                    if i >= plen - 1 and len(seqs[n]) <= i + 1:
                        seqs[n].append(rep.oracle_token)
            pos += 1
        log(f"[parity] {label} mode={mode} batch={B} steps={plen + n_steps} worst err/tol={worst:.3g} "
            f"token mismatches (all below margin)={mism}")
    finally:
        gpu.close()
    return worst
