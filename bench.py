#!/usr/bin/env python3
"""Decode benchmark: us/token of greedy decode on one MI355X, with the
achieved HBM bandwidth of the megakernel against the 8 TB/s peak, the
baselines (the conventional one-kernel-per-operation path, eager and captured
in a hipGraph; the megakernel's own executors launched once per stage, eager
and captured) and the CPU oracle.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (llama1b): 16 layers, hidden 2048, 32 query / 8 KV heads of
64, SwiGLU 8192, vocab 128256, tied embedding, RoPE theta 5e5, bf16 weights
~N(0, 0.02) from seed 0.  A 128-token seeded prompt is run through the
model (untimed), W warm-up steps run, then K greedy steps are timed from
position 128 with the token chained on the device (out_token of step i is
d_token of step i+1).  The headline mode (mega-steps) runs the K timed steps
in one persistent launch; mega runs one launch per step.  Other workloads:
llama1b-long (single steps at positions 4096 and 8191 over a seeded
8192-slot cache, each repeated K times; headline: one launch per step),
llama1b-b8 (8 sequences) and llama8b (refused by the library for now).
Extra legs: the prompt as prefill calls against decode steps, and the W2A8
matrix-vector executor.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/token batch-1 decode (Llama-1B shape) + achieved HBM GB/s vs 8 TB/s peak"
HBM_PEAK_GBPS = 8000.0

# HBM bytes per decode step of the megakernel, per workload and execution
# mode, from rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a 1 GiB copy
# (summaries and commands: profiles/mk_persistent_llama1b_hbm_bytes.md for
# the batch-1 workloads, profiles/mk_persistent_steps_llama1b.md for all
# steps in one launch, profiles/mk_persistent_llama1b_b8_kernel_trace.md for
# 8 sequences; a multi-step launch's counters are divided by its steps, the
# long-context figure is the mean of its two positions).  They describe the
# kernel sources whose hash is recorded; any other source gives null.
MEASURED_TRAFFIC = {
    "sources_sha256_prefix": "5ba39d7953320f47",
    "fetch_factor": 2.000,
    "write_factor": 1.000,
    "per_step": {
        "llama1b": {
            "mega": {"fetch_bytes": 2.5058e9, "write_bytes": 2.319e6},
            "mega-steps": {"fetch_bytes": 2.5097e9, "write_bytes": 2.323e6},
        },
        "llama1b-long": {
            "mega": {"fetch_bytes": 2.6962e9, "write_bytes": 7.694e6},
        },
        "llama1b-b8": {
            "mega": {"fetch_bytes": 2.8192e9, "write_bytes": 2.241e7},
            "mega-steps": {"fetch_bytes": 2.8189e9, "write_bytes": 2.241e7},
        },
    },
}
KERNEL_SOURCES = ("csrc/mk_device.h", "csrc/mk_inst.hip", "csrc/mk_kernels.hip", "csrc/mk_internal.h",
                  "csrc/mk_addr.h", "csrc/mk_plan.cpp")


def kernel_sources_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "persistent_megakernel_cu_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, mode: str, steps_per_launch: int):
    """HBM bytes per launch from the committed counters, or None when the kernel changed since."""
    per = MEASURED_TRAFFIC["per_step"].get(workload, {}).get(mode)
    if per is None or kernel_sources_hash() != MEASURED_TRAFFIC["sources_sha256_prefix"]:
        return None
    return (per["fetch_bytes"] + per["write_bytes"]) * steps_per_launch


def algorithmic_bytes(shape, pos: int, batch: int = 1) -> int:
    """Bytes one decode step must move: every weight once, the norm gains, the
    embedding row(s), K/V reads of [0, pos] and the K/V writes of slot pos."""
    H, QD, KVD, F, V, L = shape.hidden, shape.q_dim, shape.kv_dim, shape.ffn, shape.vocab, shape.n_layers
    w = L * (QD * H + 2 * KVD * H + H * QD + 3 * F * H) * 2      # layer matrices
    w += V * H * 2                                                # LM head (== embedding when tied)
    w += (2 * L + 1) * H * 2                                      # norm gains
    w += batch * H * 2                                            # embedding rows
    kv_read = batch * (pos + 1) * L * 2 * KVD * 2
    kv_write = batch * L * 2 * KVD * 2
    return w + kv_read + kv_write


def cpu_model() -> str:
    """Model name of the host CPU (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_cores() -> int:
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
        v = os.environ.get(var)
        if v and v.isdigit():
            return int(v)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def device_cache(torch, shape, batch, max_seq, seeded_filled):
    """K and V caches on the device: zeros, or seeded N(0,1) bf16 in [0, filled)."""
    import numpy as np

    from synth_inputs import make_kv_cache

    dims = (batch, shape.n_layers, shape.n_kv_heads, max_seq, shape.head_dim)
    if seeded_filled <= 0:
        z = torch.zeros(dims, dtype=torch.int16, device="cuda")
        return z, torch.zeros_like(z)
    kc, vc = make_kv_cache(shape, batch, max_seq, seeded_filled, master=0)
    return (torch.from_numpy(kc.view(np.int16)).cuda(), torch.from_numpy(vc.view(np.int16)).cuda())


def time_mode(mk, torch, wl, wdev, mode, warmup, steps, max_seq, attn_chunks=0):
    """One engine in `mode` on workload `wl`.

    Chained workloads (a prompt, or a seeded cache and a start token) run
    `warmup` greedy steps, then `steps` timed greedy steps whose input token is
    the previous step's out_token on the device.  The long-context workload
    times `steps` repeats of one step at each of its positions (the step is
    idempotent: same token, same slot written).  Returns (ms per step, tokens
    of an untimed replay, per-position ms).
    """
    from synth_inputs import make_prompt, make_start_token

    shape, B = wl.shape, wl.batch
    steps_launch = mode == "mega-steps"  # all timed steps in one persistent launch (mk_decode_steps)
    if steps_launch:
        mode = "mega"
    exec_mode, partial = (mode[: -len("-partial")], True) if mode.endswith("-partial") else (mode, False)
    eng = mk.Engine(shape, wdev, max_seq, mode=exec_mode, batch=B, attn_chunks=attn_chunks, partial_input=partial)
    k, v = device_cache(torch, shape, B, max_seq, wl.cache_filled)
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    per_pos = {}
    if wl.prompt_len > 0:
        for p, t in enumerate(make_prompt(shape, wl.prompt_len, master=0)):
            tok.fill_(int(t))
            eng.decode_step(tok, p, k, v, logits, tok, stream)
    else:
        tok.copy_(torch.tensor([make_start_token(shape, b) for b in range(B)], dtype=torch.int32))
    torch.cuda.synchronize()
    first = tok.clone()
    if wl.name == "llama1b-long":
        out = torch.empty_like(tok)
        for pos in (wl.start_pos, wl.max_seq - 1):
            for _ in range(warmup):
                eng.decode_step(first, pos, k, v, logits, out, stream)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(steps):
                eng.decode_step(first, pos, k, v, logits, out, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            per_pos[pos] = e0.elapsed_time(e1) / steps
        toks = [int(x) for x in out.cpu().tolist()]
        ms = sum(per_pos.values()) / len(per_pos)
    elif steps_launch:
        start = wl.start_pos
        out = torch.empty((max(steps, warmup), B), dtype=torch.int32, device="cuda")
        if warmup > 0:
            eng.decode_steps(tok, start, warmup, k, v, out[:warmup], None, stream)
        torch.cuda.synchronize()
        e0.record(stream)
        eng.decode_steps(first, start, steps, k, v, out[:steps], None, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        toks = out[:steps].cpu().tolist()
    else:
        start = wl.start_pos
        for i in range(warmup):
            eng.decode_step(tok, start + i, k, v, logits, tok, stream)
        torch.cuda.synchronize()
        tok.copy_(first)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            eng.decode_step(tok, start + i, k, v, logits, tok, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        # replay once more, recording tokens, to compare modes (untimed)
        tok.copy_(first)
        rec = torch.empty((steps, B), dtype=torch.int32, device="cuda")
        for i in range(steps):
            eng.decode_step(tok, start + i, k, v, logits, tok, stream)
            rec[i].copy_(tok)
        torch.cuda.synchronize()
        toks = rec.cpu().tolist()
    st = eng.status()
    eng.close()
    if st.code != 0:
        raise RuntimeError(f"{mode}: device status {st.code} (stage {st.stage}, wg {st.wg})")
    return ms, toks, per_pos


def prefill_bench(mk, torch, wl, wdev, max_seq, chunk: int = 8, reps: int = 3) -> dict:
    """The workload's prompt run two ways on one GPU: as prefill calls of
    `chunk` tokens (mk_config.prefill: each call the batched MFMA executors
    over `chunk` consecutive tokens, reading the weights once) and as one
    batch-1 megakernel decode step per token.  Each way `reps` times, every
    time into a fresh cache; wall time from HIP events on the stream."""
    from synth_inputs import make_prompt

    shape = wl.shape
    T = wl.prompt_len - wl.prompt_len % chunk
    prompt = [int(t) for t in make_prompt(shape, wl.prompt_len, master=0)][:T]
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(eng, B, calls):
        k, v = device_cache(torch, shape, 1, max_seq, 0)
        logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
        out = torch.empty(B, dtype=torch.int32, device="cuda")
        toks = [torch.tensor(c, dtype=torch.int32, device="cuda") for c, _ in calls]
        for (c, pos), t in zip(calls, toks):  # warm-up pass
            eng.decode_step(t, pos, k, v, logits, out, stream)
        torch.cuda.synchronize()
        total = 0.0
        for _ in range(reps):
            k.zero_()
            v.zero_()
            torch.cuda.synchronize()
            e0.record(stream)
            for (c, pos), t in zip(calls, toks):
                eng.decode_step(t, pos, k, v, logits, out, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
        return total / reps * 1e3  # us

    eng = mk.Engine(shape, wdev, max_seq, mode="mega", batch=chunk, prefill=True)
    pf_us = timed(eng, chunk, [(prompt[i:i + chunk], i) for i in range(0, T, chunk)])
    eng.close()
    eng = mk.Engine(shape, wdev, max_seq, mode="mega", batch=1)
    dec_us = timed(eng, 1, [([t], i) for i, t in enumerate(prompt)])
    eng.close()
    return {
        "prompt_tokens": T,
        "chunk": chunk,
        "prefill_us": round(pf_us, 1),
        "prefill_tokens_per_s": round(T / (pf_us * 1e-6), 1),
        "decode_steps_us": round(dec_us, 1),
        "speedup": round(dec_us / pf_us, 3),
    }


def cpu_baseline(wl, weights, budget_s: float = 12.0):
    """Time the oracle on a bounded sample of the same workload (sequence 0)."""
    import numpy as np

    import oracle as orc
    from synth_inputs import make_kv_cache, make_start_token

    shape = wl.shape
    start_pos = wl.start_pos
    o = orc.Oracle(shape, weights, lazy=shape.n_layers * shape.hidden > 16 * 2048)
    cap = 1024 if wl.prompt_len > 0 else 64
    filled = wl.cache_filled if wl.cache_filled > 0 else start_pos
    kc, vc = make_kv_cache(shape, 1, max(wl.max_seq, start_pos + cap), filled, master=0)
    kc, vc = kc[0], vc[0]
    tok = make_start_token(shape, 0)
    n = 0
    t0 = time.perf_counter()
    while True:
        lg = o.decode_step(tok, start_pos + n, kc, vc)
        tok = int(np.argmax(lg))
        n += 1
        if time.perf_counter() - t0 > budget_s or n >= cap or start_pos + n >= kc.shape[2]:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(dt / n * 1e6, 1),
        "unit": "µs/token",
        "cores": cpu_cores(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{n} greedy decode step(s) of sequence 0 at positions {start_pos}..{start_pos + n - 1} over a "
                  f"cache whose first {filled} slots are seeded N(0,1) bf16 (for a prefilled prompt: the same "
                  f"cost as the prompt's own K/V); NumPy fp32"
                  + (", each matrix widened to fp32 inside the step" if o.lazy else ", weights widened before timing"),
    }


W2A8_LAYER = (("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336))
W2A8_LAYERS = 32


def w2a8_bench(mk, torch, passes: int = 10, warmup: int = 2) -> dict:
    """The W2A8 matrix-vector product over a model's worth of projections:
    the Llama-8B shape's four projections (QKV, O, gate/up, down) of 32
    layers, each layer's matrices in their own buffers (1.75 GB of packed
    weights, beyond the 256 MB last-level cache, so every pass streams them
    from HBM).  Packed words are drawn on the device with every two-bit field
    in {0, 1, 2} (timing only; parity is tested elsewhere).  A pass runs the
    128 one-launch products from float32 inputs (mk_w2a8_linear: codes formed
    in the kernel); the GEMV-only pass runs the 128 GEMVs on codes quantised
    once (mk_w2a8_gemv)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    mats = []
    for _ in range(W2A8_LAYERS):
        for name, rows, cols in W2A8_LAYER:
            w = torch.randint(0, 1 << 32, (rows, cols // 16), dtype=torch.int64, device="cuda", generator=gen)
            w = w ^ (((w >> 1) & w & 0x55555555) << 1)  # a field holding 3 becomes 1
            w = torch.where(w >= 1 << 31, w - (1 << 32), w)  # the same 32 bits as int32
            mats.append((name, rows, cols, w.to(torch.int32).contiguous()))
    xs = {c: torch.randn(c, device="cuda", generator=gen) for c in (4096, 14336)}
    xq = {c: torch.empty(c, dtype=torch.int8, device="cuda") for c in xs}
    sc = {c: torch.empty(1, dtype=torch.float32, device="cuda") for c in xs}
    gam = torch.ones(max(r for _, r, _ in W2A8_LAYER), device="cuda")
    y = torch.empty(max(r for _, r, _ in W2A8_LAYER), device="cuda")

    def one_pass(quantize: bool):
        for name, rows, cols, w in mats:
            if quantize:
                mk.w2a8_linear(w, gam, rows, cols, xs[cols], y)
            else:
                mk.w2a8_gemv(w, gam, rows, cols, xq[cols], sc[cols], y)

    def timed(quantize: bool) -> float:
        for _ in range(warmup):
            one_pass(quantize)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(passes):
            one_pass(quantize)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / passes  # us per pass

    for c in xs:
        mk.w2a8_quantize(xs[c], xq[c], sc[c])
    gemv_us = timed(False)
    pass_us = timed(True)
    # the kernel's streaming rate, launch overhead amortised: one launch over
    # the 32 layers' gate/up rows as one tall matrix (940 MB)
    tall_rows = W2A8_LAYERS * 28672
    tall = torch.randint(0, 1 << 32, (tall_rows, 4096 // 16), dtype=torch.int64, device="cuda", generator=gen)
    tall = tall ^ (((tall >> 1) & tall & 0x55555555) << 1)
    tall = torch.where(tall >= 1 << 31, tall - (1 << 32), tall).to(torch.int32).contiguous()
    tgam = torch.ones(tall_rows, device="cuda")
    ty = torch.empty(tall_rows, device="cuda")
    for _ in range(warmup):
        mk.w2a8_gemv(tall, tgam, tall_rows, 4096, xq[4096], sc[4096], ty)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(passes):
        mk.w2a8_gemv(tall, tgam, tall_rows, 4096, xq[4096], sc[4096], ty)
    e1.record()
    torch.cuda.synchronize()
    tall_us = e0.elapsed_time(e1) * 1e3 / passes
    tall_bytes = tall_rows * 4096 // 4 + 4096 + 8 * tall_rows
    tall_gbps = tall_bytes / (tall_us * 1e-6) / 1e9
    del tall, tgam, ty
    wbytes = sum(r * c // 4 for _, r, c, _ in mats)
    io_bytes = sum(c + 8 * r for _, r, c, _ in mats)  # codes in, scale + output per row
    achieved = (wbytes + io_bytes) / (gemv_us * 1e-6) / 1e9
    bf16_bytes = sum(2 * r * c for _, r, c, _ in mats)
    del mats
    torch.cuda.empty_cache()
    return {
        "workload": "Llama-8B projections (QKV 6144x4096, O 4096x4096, gate/up 28672x4096, down 4096x14336) "
                    f"x {W2A8_LAYERS} layers, batch 1, ternary weights in 2 bits, int8 activations",
        "launches_per_pass": len(W2A8_LAYER) * W2A8_LAYERS,
        "pass_us": round(pass_us, 1),
        "gemv_only_pass_us": round(gemv_us, 1),
        "weight_bytes_per_pass": wbytes,
        "bf16_weight_bytes_equivalent": bf16_bytes,
        "gemv_only_pass_GBps": round(achieved, 1),
        "tall_matrix": {"rows": tall_rows, "cols": 4096, "us_per_launch": round(tall_us, 1),
                        "bytes_per_launch": tall_bytes},
        "roofline": {"bound": "hbm", "achieved": round(tall_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(tall_gbps / HBM_PEAK_GBPS, 4),
                     "note": "mk_w2a8_gemv over the tall matrix: algorithmic bytes (packed weights, codes, "
                             "scales, outputs) per launch / average launch time (HIP events)"},
    }


def copy_probe(mib: int) -> int:
    """Plain copies of known size: their FETCH_SIZE / WRITE_SIZE per dispatch
    against mib MiB give the factor that turns those counters into bytes."""
    import torch

    a = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "dispatches": 4}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama1b")
    ap.add_argument("--modes", default="mega-steps,mega,graph,multi,conv,conv-graph",
                    help="mega-steps: the persistent megakernel running every timed step in one launch "
                         "(mk_decode_steps); mega: one launch per step; graph / multi: its executors one launch per stage, "
                         "captured or not; conv / conv-graph: the conventional one-kernel-per-operation path, "
                         "eager or captured in a hipGraph; mega-partial: the megakernel with the partial-input "
                         "down projection")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-w2a8", action="store_true", help="skip the W2A8 matrix-vector leg")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prompt-prefill leg")
    ap.add_argument("--w2a8-only", action="store_true", help="only run the W2A8 matrix-vector leg")
    ap.add_argument("--attn-chunks", type=int, default=0, help="KV split per head (0: automatic)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run 4 device-to-device copies of this many MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the decode path runs on one GPU; multi-GPU runs are not supported, "
                                   "use --gpus 1"}))
        return 2
    if args.copy_mib > 0:
        return copy_probe(args.copy_mib)

    import torch

    import persistent_megakernel_cu_amd.binding as mk
    from synth_inputs import WORKLOADS, make_weights

    if args.w2a8_only:
        print(json.dumps({"w2a8": w2a8_bench(mk, torch)}), flush=True)
        return 0
    wl = WORKLOADS[args.workload]
    shape = wl.shape
    if wl.steps <= 0:
        print(json.dumps({"error": f"workload {wl.name} has no decode steps to time"}))
        return 2
    steps = args.steps
    max_seq = wl.max_seq if wl.name == "llama1b-long" else max(wl.max_seq, wl.start_pos + max(steps, args.warmup))
    t0 = time.time()
    weights = make_weights(shape, master=0)
    wdev = mk.to_device(weights)
    print(f"[bench] {wl.name}: weights ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    results, tokens, per_pos = {}, {}, {}
    refused = {}
    for mode in args.modes.split(","):
        try:
            ms, toks, pp = time_mode(mk, torch, wl, wdev, mode, args.warmup, steps, max_seq, args.attn_chunks)
        except mk.MkError as e:
            if e.code != mk.MK_E_UNSUPPORTED:
                raise
            refused[mode] = mk.error_string(e.code)  # e.g. the megakernel modes at the Llama-8B shape
            print(f"[bench] {mode}: refused by the library ({refused[mode]})", file=sys.stderr, flush=True)
            continue
        results[mode], tokens[mode], per_pos[mode] = ms, toks, pp
        print(f"[bench] {mode}: {ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    if not results:
        print(json.dumps({"error": f"every mode was refused for workload {wl.name}", "refused": refused}))
        return 2

    # the headline: every timed step in one persistent launch where the
    # workload chains its steps, else one launch per step
    if "mega-steps" in results and wl.name != "llama1b-long":
        main_mode = "mega-steps"
    else:
        main_mode = "mega" if "mega" in results else next(iter(results))
    steps_per_launch = steps if main_mode == "mega-steps" else 1
    ms = results[main_mode]
    B = wl.batch
    us_tok = ms * 1e3 / B
    if wl.name == "llama1b-long":
        positions = sorted(per_pos[main_mode])
        avg_bytes = sum(algorithmic_bytes(shape, p, B) for p in positions) / len(positions)
        where = (f"single steps at positions {', '.join(map(str, positions))} over a seeded {wl.max_seq}-slot "
                 f"N(0,1) bf16 cache, each repeated {steps} times (same token, idempotent)")
    else:
        positions = list(range(wl.start_pos, wl.start_pos + steps))
        avg_bytes = sum(algorithmic_bytes(shape, p, B) for p in positions) / steps
        where = (f"positions {wl.start_pos}..{wl.start_pos + steps - 1} "
                 + (f"after a {wl.prompt_len}-token prefill" if wl.prompt_len > 0
                    else f"over a seeded {wl.cache_filled}-slot N(0,1) bf16 cache"))
    achieved = avg_bytes / (ms * 1e-3) / 1e9
    sh = shape
    model = (f"{sh.n_layers}L, H{sh.hidden}, {sh.n_heads}q/{sh.n_kv_heads}kv x{sh.head_dim}, SwiGLU {sh.ffn}, "
             f"V{sh.vocab}, {'tied' if sh.tie_embeddings else 'untied'}")
    out = {
        "metric": METRIC,
        "value": round(us_tok, 2),
        "unit": "µs/token",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 math, bf16 weights/KV, 24-bit activation words",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: batch-{B} greedy decode, {sh.name} shape ({model}), bf16 weights and KV "
                        f"cache, fp32 arithmetic and accumulation, activations handed between workgroups as 24-bit "
                        f"words (the fp32 value rounded to 16 significant bits), {where}",
            "batch": B,
            "weights": "bf16 ~N(0,0.02) seed 0",
            "tokens_per_s": round(1e6 / us_tok, 1),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(args.workload, main_mode, steps_per_launch),
            "bytes_per_step": int(avg_bytes),
            "steps_per_launch": steps_per_launch,
            "bytes_per_launch": int(avg_bytes * steps_per_launch),
            "traffic_unit": f"HBM bytes per launch ({main_mode}: {steps_per_launch} decode step(s) per launch)",
        },
        "main_mode": main_mode,
        "refused_modes": refused,
        "baselines": {m: {"us_per_token": round(v * 1e3 / B, 2), "tokens_per_s": round(B * 1e3 / v, 1)}
                      for m, v in results.items()},
        "modes_agree": all(t == tokens[main_mode] for t in tokens.values()),
    }
    if per_pos[main_mode]:
        out["per_position_us"] = {str(p): round(t * 1e3, 2) for p, t in sorted(per_pos[main_mode].items())}
    if "graph" in results and "mega" in results:
        out["speedup_vs_graph"] = round(results["graph"] / results[main_mode], 3)
    if "conv-graph" in results and "mega" in results:
        out["speedup_vs_conv_graph"] = round(results["conv-graph"] / results[main_mode], 3)
    if not args.no_prefill and wl.prompt_len >= 8 and B == 1:
        out["prefill"] = prefill_bench(mk, torch, wl, wdev, max_seq)
        print(f"[bench] prefill: {out['prefill']['prefill_us']} us for {out['prefill']['prompt_tokens']} tokens "
              f"(decode steps: {out['prefill']['decode_steps_us']} us)", file=sys.stderr, flush=True)
    if not args.no_w2a8:
        del wdev
        torch.cuda.empty_cache()
        out["w2a8"] = w2a8_bench(mk, torch)
        print(f"[bench] w2a8: {out['w2a8']['pass_us']} us per pass, GEMV-only {out['w2a8']['gemv_only_pass_us']} us",
              file=sys.stderr, flush=True)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, weights)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
