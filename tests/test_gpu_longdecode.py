"""Long decode: 4 layers, context grown to 262,144 slots, 64 append+decode steps.

Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq":
section "Konfiguracja" fixes the context at 262,144 tokens; section "4.
Poprawność w długich sesjach" asks for correct long sessions.  Workload: batch
1, 8 KV / 64 query heads, K/V Student-t (nu = 3) plus a per-(layer, tensor,
head, channel) Gaussian random-walk mean, prefix 262,080 slots, then 64 steps
that each append one token per layer and decode it (one decode-step call per
layer, the path bench.py times; the plain decode call at the checked steps).
Checked: for every KV
head of every layer the whole packed cache row (prefix and the 64 appended
tokens) is byte-identical to the oracle's, and the decode outputs of every
query head at steps 0, 31 and 63 of every layer are within max-abs 2e-3 and
relative L2 1e-3 of the oracle, with fp32 output, and with fp16 output (plus
half an fp16 ulp of the reference).
"""

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from workloads import WORKLOADS, K, V, kv_tensor, q_decode
from _rows import decode_row, pool_map
from _util import check_attn

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CHECK_STEPS = (0, 31, 63)


@pytest.mark.timeout(900)
def test_longdecode_262k_four_layers():
    w = WORKLOADS["longdecode"]
    T = w.n_ctx + w.steps                      # 262,144
    H, G = w.n_kv_heads, w.n_q_heads // w.n_kv_heads
    caches, new_k, new_v = [], [], []
    for layer in range(w.layers):
        cache = tb.KVCache(1, H, T)
        xk = kv_tensor(w, layer, K, 0, T)                  # [1][T][H][128], drift carried
        xv = kv_tensor(w, layer, V, 0, T)
        new_k.append(torch.from_numpy(xk[:, w.n_ctx:].copy()).cuda())
        new_v.append(torch.from_numpy(xv[:, w.n_ctx:].copy()).cuda())
        for t0 in range(0, w.n_ctx, 32768):
            t1 = min(w.n_ctx, t0 + 32768)
            tb.quantize_append(cache, torch.from_numpy(np.ascontiguousarray(xk[:, t0:t1])).cuda(),
                               torch.from_numpy(np.ascontiguousarray(xv[:, t0:t1])).cuda(), t0)
        del xk, xv
        caches.append(cache)
    torch.cuda.synchronize()

    # the 64 steps: per layer, one decode-step call (append the token at pos
    # and attend over pos + 1 slots, as bench.py times it); at the checked
    # steps the plain decode call once more, with fp32 output
    outs = {}
    ws = torch.empty(tb.decode_step_workspace_bytes(1, H, w.n_q_heads, T, 0), dtype=torch.uint8,
                     device="cuda")
    for step in range(w.steps):
        pos = w.n_ctx + step
        for layer in range(w.layers):
            q = torch.from_numpy(q_decode(w, layer, step)).cuda()
            out = tb.decode_step(caches[layer], new_k[layer][:, step:step + 1].contiguous(),
                                 new_v[layer][:, step:step + 1].contiguous(), q, pos,
                                 w.softmax_scale, workspace=ws)
            if step in CHECK_STEPS:
                outs[(layer, step, torch.float16)] = out.float().cpu().numpy()
                outs[(layer, step, torch.float32)] = tb.attn_decode(
                    caches[layer], q, pos + 1, w.softmax_scale, workspace=ws,
                    out_dtype=torch.float32).cpu().numpy()
    torch.cuda.synchronize()
    kg = [c.k.cpu().numpy() for c in caches]
    vg = [c.v.cpu().numpy() for c in caches]
    del caches, new_k, new_v
    torch.cuda.empty_cache()

    # oracle: every (layer, KV head) row, quantised in worker processes
    jobs = [("longdecode", layer, 0, g, T,
             [(step, q_decode(w, layer, step)[0, g * G:(g + 1) * G], w.n_ctx + step + 1,
               w.softmax_scale) for step in CHECK_STEPS])
            for layer in range(w.layers) for g in range(H)]
    for (_, layer, _, g, _, _), (kc, vc, refs) in zip(jobs, pool_map(decode_row, jobs)):
        assert np.array_equal(kg[layer][0, g], kc), f"layer {layer} head {g} K bytes"
        assert np.array_equal(vg[layer][0, g], vc), f"layer {layer} head {g} V bytes"
        for step in CHECK_STEPS:
            for od in (torch.float16, torch.float32):
                check_attn(outs[(layer, step, od)][0, g * G:(g + 1) * G], refs[step],
                           od == torch.float16, f"layer {layer} head {g} step {step} {od}")
