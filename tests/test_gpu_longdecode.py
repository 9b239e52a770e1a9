"""Long decode: 4 layers, context grown to 262,144 slots, 64 append+decode steps.

Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq":
section "Konfiguracja" fixes the context at 262,144 tokens; section "4.
Poprawność w długich sesjach" asks for correct long sessions.  Workload: batch
1, 8 KV / 64 query heads, K/V Student-t (nu = 3) plus a per-(layer, tensor,
head, channel) Gaussian random-walk mean, prefix 262,080 slots, then 64 steps
that each append one token per layer and decode it.  Checked: for one KV head
per layer the whole packed cache row is byte-identical to the oracle's, and
the decode outputs at steps 0, 31 and 63 of every layer are within max-abs
2e-3 (+ half an fp16 ulp) and relative L2 1e-3 of the oracle.
"""

import multiprocessing as mp
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o
from workloads import WORKLOADS, K, V, kv_tensor, q_decode
from _util import check_attn

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CHECK_STEPS = (0, 31, 63)


def test_longdecode_262k_four_layers():
    w = WORKLOADS["longdecode"]
    T = w.n_ctx + w.steps                      # 262,144
    H, G = w.n_kv_heads, w.n_q_heads // w.n_kv_heads
    heads = [(3 * layer + 1) % H for layer in range(w.layers)]   # KV head checked per layer
    caches, new_k, new_v, host_rows = [], [], [], {}
    for layer in range(w.layers):
        cache = tb.KVCache(1, H, T)
        xk = kv_tensor(w, layer, K, 0, T)                  # [1][T][H][128], drift carried
        xv = kv_tensor(w, layer, V, 0, T)
        host_rows[(layer, K)] = xk[0, :, heads[layer]].copy()   # the checked head
        host_rows[(layer, V)] = xv[0, :, heads[layer]].copy()
        new_k.append(torch.from_numpy(xk[:, w.n_ctx:].copy()).cuda())
        new_v.append(torch.from_numpy(xv[:, w.n_ctx:].copy()).cuda())
        for t0 in range(0, w.n_ctx, 32768):
            t1 = min(w.n_ctx, t0 + 32768)
            tb.quantize_append(cache, torch.from_numpy(np.ascontiguousarray(xk[:, t0:t1])).cuda(),
                               torch.from_numpy(np.ascontiguousarray(xv[:, t0:t1])).cuda(), t0)
        del xk, xv
        caches.append(cache)
    torch.cuda.synchronize()

    # the 64 steps: per layer, append one token, then decode over pos + 1 slots
    outs = {}
    ws = torch.empty(tb.decode_workspace_bytes(1, H, w.n_q_heads, T, 0), dtype=torch.uint8,
                     device="cuda")
    for step in range(w.steps):
        pos = w.n_ctx + step
        for layer in range(w.layers):
            tb.quantize_append(caches[layer], new_k[layer][:, step:step + 1].contiguous(),
                               new_v[layer][:, step:step + 1].contiguous(), pos)
            q = torch.from_numpy(q_decode(w, layer, step)).cuda()
            out = tb.attn_decode(caches[layer], q, pos + 1, w.softmax_scale, workspace=ws)
            if step in CHECK_STEPS:
                outs[(layer, step)] = out.float().cpu().numpy()
    torch.cuda.synchronize()

    # oracle: one KV head per layer, quantised in worker processes
    keys = [(layer, tensor) for layer in range(w.layers) for tensor in (K, V)]
    with ProcessPoolExecutor(min(8, len(keys)), mp_context=mp.get_context("spawn")) as ex:
        packed = [r[0] for r in ex.map(o.quantize_blocks, [host_rows[k] for k in keys])]
        deq = list(ex.map(o.dequantize_blocks, packed))
    res = {k: (p, d) for k, p, d in zip(keys, packed, deq)}
    for layer in range(w.layers):
        g = heads[layer]
        kc, kh = res[(layer, K)]
        vc, vh = res[(layer, V)]
        assert np.array_equal(caches[layer].k[0, g].cpu().numpy(), kc), f"layer {layer} K bytes"
        assert np.array_equal(caches[layer].v[0, g].cpu().numpy(), vc), f"layer {layer} V bytes"
        for step in CHECK_STEPS:
            n = w.n_ctx + step + 1
            q = q_decode(w, layer, step)[0, g * G:(g + 1) * G]
            ref = o.attn_decode_rows_ref(q, kh[:n], vh[:n], w.softmax_scale)
            check_attn(outs[(layer, step)][0, g * G:(g + 1) * G], ref, True,
                       f"layer {layer} step {step}")
