"""Stage timeline of one traced decode step: where the time between weight
streams goes (handoffs between dependent stages, stragglers, the LM head).

    python -m persistent_megakernel_cu_amd.timeline [--workload llama1b] [--pos P]

The library records, per (workgroup, stage), the device wall clock when the
stage was entered, when its inputs were ready, when its compute was done and
when it was left (``mk_trace_copy``; the handle is loaded with tracing on,
which costs ~3 % of the step).  For every stage this prints, over the
workgroups that had work there, the median ready and done times and the
latest done time; per stage kind, averaged over the layers:

- handoff: median inputs-ready minus the previous stage's latest done, i.e.
  the gap from the last producer to the typical consumer (store visibility,
  the consumer's poll round trip, staging and norm);
- compute: median done minus median ready;
- tail: latest done minus median done (the slowest workgroup).

The workload runs on seeded synthetic inputs as in bench.py; the step traced
is the last of a few greedy steps ending at position --pos.
"""

from __future__ import annotations

import argparse
import os
import sys

import numpy as np

KINDS = ("QKV", "attention", "O-proj", "gate/up", "down")


def stage_table(stamps: np.ndarray, khz: int) -> dict:
    """Summaries of a [workgroups][stages][20] stamp array (device clock at khz)."""
    tr = stamps.astype(np.int64)
    valid = tr[:, :, 0] > 0
    t0 = tr[:, :, 0][valid].min()
    us = lambda x: (x - t0) * 1e3 / khz
    rows = []
    for s in range(tr.shape[1]):
        m = valid[:, s]
        if not m.any():
            rows.append(None)
            continue
        rd, dn = us(tr[m, s, 1]), us(tr[m, s, 2])
        rows.append({"stage": s, "tasks": int(m.sum()), "ready_med": float(np.median(rd)),
                     "done_med": float(np.median(dn)), "done_max": float(dn.max())})
    per_kind = {}
    S = tr.shape[1]
    n_layers = (S - 1) // 5
    for k, name in enumerate(KINDS):
        h, c, t = [], [], []
        for l in range(n_layers):
            s = 5 * l + k
            r = rows[s]
            if r is None:
                continue
            prev = next((rows[q] for q in range(s - 1, -1, -1) if rows[q] is not None), None)
            h.append(r["ready_med"] - (prev["done_max"] if prev else 0.0))
            c.append(r["done_med"] - r["ready_med"])
            t.append(r["done_max"] - r["done_med"])
        if h:
            per_kind[name] = (float(np.mean(h)), float(np.mean(c)), float(np.mean(t)))
    lm, prev = rows[S - 1], rows[S - 2]
    return {"rows": rows, "per_kind": per_kind,
            "lm": (lm["ready_med"] - prev["done_max"], lm["done_med"] - lm["ready_med"], lm["done_max"] - lm["done_med"]),
            "step_us": max(r["done_max"] for r in rows if r is not None), "layers": n_layers}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama1b")
    ap.add_argument("--pos", type=int, default=0, help="position of the traced step (default: the workload's first)")
    ap.add_argument("--steps", type=int, default=4, help="greedy steps before and including the traced one")
    ap.add_argument("--save", default="", help="also write the raw stamps and clock rate to this .npz file")
    args = ap.parse_args()

    import torch

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    from persistent_megakernel_cu_amd import binding as mk
    from synth_inputs import WORKLOADS, make_kv_cache, make_prompt, make_start_token, make_weights

    wl = WORKLOADS[args.workload]
    sh, B = wl.shape, wl.batch
    last = args.pos if args.pos > 0 else wl.start_pos + args.steps - 1
    first = last - args.steps + 1
    max_seq = max(wl.max_seq, last + 1)
    wdev = mk.to_device(make_weights(sh, master=0))
    eng = mk.Engine(sh, wdev, max_seq, mode="mega", batch=B, trace=True)
    dims = (B, sh.n_layers, sh.n_kv_heads, max_seq, sh.head_dim)
    if wl.cache_filled > 0:
        kc, vc = make_kv_cache(sh, B, max_seq, wl.cache_filled, master=0)
        k = torch.from_numpy(kc.view(np.int16)).cuda()
        v = torch.from_numpy(vc.view(np.int16)).cuda()
    else:
        k = torch.zeros(dims, dtype=torch.int16, device="cuda")
        v = torch.zeros_like(k)
    logits = torch.empty((B, sh.vocab), dtype=torch.float32, device="cuda")
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    if wl.prompt_len > 0:
        prompt = make_prompt(sh, first, master=0) if first <= wl.prompt_len else None
        if prompt is None:
            raise SystemExit(f"--pos must leave the first traced step inside the {wl.prompt_len}-token prompt range")
        for p, t in enumerate(prompt):
            tok.fill_(int(t))
            eng.decode_step(tok, p, k, v, logits, tok)
    else:
        tok.copy_(torch.tensor([make_start_token(sh, b) for b in range(B)], dtype=torch.int32))
    for p in range(first, last + 1):
        eng.decode_step(tok, p, k, v, logits, tok)
    torch.cuda.synchronize()
    stamps, khz = eng.trace()
    st = eng.status()
    eng.close()
    if st.code != 0:
        raise SystemExit(f"device status {st.code}")

    if args.save:
        np.savez(args.save, stamps=stamps, khz=khz)
    t = stage_table(stamps, khz)
    print(f"workload {wl.name}, traced step at position {last}: {t['step_us']:.1f} us "
          f"(traced build), {t['layers']} layers\n")
    print("| stage kind | handoff into it | compute | tail |")
    print("|---|---|---|---|")
    for name, (h, c, tl) in t["per_kind"].items():
        print(f"| {name} | {h:.2f} us | {c:.2f} us | {tl:.2f} us |")
    h, c, tl = t["lm"]
    print(f"| LM head (once) | {h:.2f} us | {c:.2f} us | {tl:.2f} us |")
    idle = sum(v[0] for v in t["per_kind"].values()) * t["layers"] + h
    tails = sum(v[2] for v in t["per_kind"].values()) * t["layers"] + tl
    print(f"\nhandoffs per step: {idle:.1f} us; tails per step: {tails:.1f} us")
    return 0


if __name__ == "__main__":
    sys.exit(main())
