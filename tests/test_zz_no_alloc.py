"""mk_conv_decode_step_static (the allocation-free entry point: a fixed
per-GPU scratch buffer in place of the caller's workspace) against
mk_conv_decode_step on identical inputs, through the C ABI."""

import numpy as np
import pytest

from synth_inputs import LLAMA_1B, TINY, make_kv_cache, make_start_token, make_weights

pytestmark = pytest.mark.gpu


def _inputs(torch, shape, B, max_seq, filled, master):
    kv = make_kv_cache(shape, B, max_seq, filled, master=master)
    toks = [make_start_token(shape, b, master=master) for b in range(B)]
    return kv, torch.tensor(toks, dtype=torch.int32, device="cuda")


def _device_cache(torch, kv):
    return (torch.from_numpy(kv[0].view(np.int16)).cuda(), torch.from_numpy(kv[1].view(np.int16)).cuda())


def test_static_scratch_matches_workspace_variant():
    import torch

    from persistent_megakernel_cu_amd import binding as mkb

    cases = [  # (shape, batch, max_seq, position, master): the second call is the smaller one
        (LLAMA_1B, 2, 512, 300, 0),
        (TINY, 1, 48, 10, 3),
    ]
    refs, runs = [], []
    for shape, B, S, pos, master in cases:
        w = mkb.to_device(make_weights(shape, master=master, gain_jitter=0.1))
        kv, tok = _inputs(torch, shape, B, S, pos, master)
        d_pos = torch.tensor([pos], dtype=torch.int32, device="cuda")
        k, v = _device_cache(torch, kv)
        lg = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
        out = torch.empty(B, dtype=torch.int32, device="cuda")
        ws = torch.empty(mkb.conv_workspace_size(shape, S, B) // 4, dtype=torch.float32, device="cuda")
        mkb.conv_decode_step(shape, w, S, tok, d_pos, k, v, lg, out, ws, batch=B)
        torch.cuda.synchronize()
        refs.append((lg.cpu().numpy(), out.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()))
        k2, v2 = _device_cache(torch, kv)
        lg2 = torch.full((B, shape.vocab), float("nan"), dtype=torch.float32, device="cuda")
        out2 = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        runs.append((shape, w, S, tok, d_pos, k2, v2, lg2, out2, B))
        torch.cuda.synchronize()
    # the two static calls back to back, the second with the smaller input
    for shape, w, S, tok, d_pos, k2, v2, lg2, out2, B in runs:
        mkb.conv_decode_step_static(shape, w, S, tok, d_pos, k2, v2, lg2, out2, batch=B)
    torch.cuda.synchronize()
    for (ref_lg, ref_out, ref_k, ref_v), (shape, w, S, tok, d_pos, k2, v2, lg2, out2, B) in zip(refs, runs):
        assert np.array_equal(lg2.cpu().numpy(), ref_lg), shape.name
        assert np.array_equal(out2.cpu().numpy(), ref_out), shape.name
        assert np.array_equal(k2.cpu().numpy(), ref_k) and np.array_equal(v2.cpu().numpy(), ref_v), shape.name
        print(f"[no-alloc] {shape.name} batch {B}: static-scratch step bit-identical to the workspace step", flush=True)


def test_static_scratch_rejects_oversize():
    # 65536 positions at batch 8 need more than the 8 MiB buffer: refused before any launch
    import torch

    from persistent_megakernel_cu_amd import binding as mkb

    shape, B, S = LLAMA_1B, 8, 65536
    assert mkb.conv_workspace_size(shape, S, B) > 8 << 20
    dummy = torch.zeros(64, dtype=torch.int16, device="cuda")
    w = {name: dummy for name in ["embed", "final_norm"] + [f"layers.{l}.{t}" for l in range(shape.n_layers)
                                                            for t in ("attn_norm", "wq", "wk", "wv", "wo",
                                                                      "ffn_norm", "w_gate", "w_up", "w_down")]}
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    d_pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.empty(16, dtype=torch.float32, device="cuda")
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    with pytest.raises(mkb.MkError) as e:
        mkb.conv_decode_step_static(shape, w, S, tok, d_pos, dummy, dummy, lg, out, batch=B)
    assert e.value.code == mkb.MK_E_TOOBIG
