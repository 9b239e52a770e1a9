"""Pin of the oracle's row-wise decode attention (``attn_decode_rows_ref``).

The function is the reference behind every check that compares only some
(sequence, KV head) rows of a large workload (decode at 98304 / 131072 slots,
the prefill chunk, the long decode, verify and the mixed formats).  It is
plain softmax attention (page "Kontekst 262K na jednej RTX 4090: co dodałem
do llama.cpp-turboq", section "Od czego zacząłem": flash attention computes
exactly softmax attention), so it is pinned here against two things that do
not share its code: torch's scaled-dot-product attention in fp64 with grouped
query heads, and the oracle's whole-cache ``attn_decode_ref`` on prefix slices
of a packed cache.  Planted mistakes (a dropped softmax scale, a transposed K,
a softmax over the wrong axis, K in place of V, a prefix one key short) each
fail the same checks.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import tbq4_oracle as o


def _pin(fn):
    """Run the checks with ``fn`` standing for attn_decode_rows_ref; returns
    the list of the checks it fails (empty when it passes all of them)."""
    failed = []
    rng = np.random.default_rng(31)
    # 1. against torch SDPA (fp64, enable_gqa) on GQA shapes: every KV head's
    #    G query rows through fn, all heads at once through SDPA
    for (Hkv, G, n, scale) in ((1, 4, 128, 0.3), (3, 8, 77, 1 / np.sqrt(128)), (2, 2, 300, 1.0)):
        K = rng.standard_normal((Hkv, n, 128)) * 1.7
        V = rng.standard_normal((Hkv, n, 128))
        q = rng.standard_normal((Hkv * G, 128))
        want = F.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None], torch.from_numpy(K)[None],
            torch.from_numpy(V)[None], scale=scale, enable_gqa=True)[0, :, 0].numpy()
        for g in range(Hkv):
            try:
                got = fn(q[g * G:(g + 1) * G], K[g], V[g], scale)
            except Exception:                       # a shape error is a failure too
                failed.append(f"sdpa Hkv={Hkv} G={G} n={n}")
                break
            if got.shape != (G, 128) or not np.allclose(got, want[g * G:(g + 1) * G],
                                                        rtol=1e-12, atol=1e-13):
                failed.append(f"sdpa Hkv={Hkv} G={G} n={n}")
                break
    # 2. against attn_decode_ref on prefix slices of a packed cache: rows of
    #    KV head g at length n equal the whole-cache reference's query heads
    B, Hkv, G, T = 2, 2, 4, 96
    x = rng.standard_normal((2, B, Hkv, T, 128)).astype(np.float32)
    x[0, ..., 5] *= 20.0                            # an outlier key channel
    kc = o.quantize_blocks(x[0], seed=7)[0]
    vc = o.quantize_blocks(x[1], seed=7)[0]
    q = rng.standard_normal((B, Hkv * G, 128))
    for n in (1, 2, 33, 95, 96):
        ref = o.attn_decode_ref(q, kc, vc, n, 0.125, seed=7)
        for b in range(B):
            for g in range(Hkv):
                Kd = o.dequantize_blocks(kc[b, g], seed=7)
                Vd = o.dequantize_blocks(vc[b, g], seed=7)
                try:
                    got = fn(q[b, g * G:(g + 1) * G], Kd[:n], Vd[:n], 0.125)
                except Exception:
                    failed.append(f"prefix n={n}")
                    break
                if got.shape != (G, 128) or not np.allclose(got, ref[b, g * G:(g + 1) * G],
                                                            rtol=1e-12, atol=1e-13):
                    failed.append(f"prefix n={n} b={b} g={g}")
                    break
    return failed


def test_rows_ref_matches_sdpa_and_whole_cache_reference():
    assert _pin(o.attn_decode_rows_ref) == []


def _softmax(s, axis=-1):
    e = np.exp(s - s.max(axis=axis, keepdims=True))
    return e / e.sum(axis=axis, keepdims=True)


MUTANTS = {
    "scale dropped": lambda q, K, V, sc: _softmax(np.asarray(q, np.float64) @ K.T) @ V,
    "scale squared": lambda q, K, V, sc: _softmax(sc * sc * (np.asarray(q, np.float64) @ K.T)) @ V,
    "K transposed": lambda q, K, V, sc: _softmax(sc * (np.asarray(q, np.float64) @ K)) @ V,
    "softmax over the query axis": lambda q, K, V, sc: _softmax(sc * (np.asarray(q) @ K.T), 0) @ V,
    "K in place of V": lambda q, K, V, sc: _softmax(sc * (np.asarray(q, np.float64) @ K.T)) @ K,
    "last key dropped": lambda q, K, V, sc: (
        _softmax(sc * (np.asarray(q, np.float64) @ K[:-1].T)) @ V[:-1] if len(K) > 1
        else _softmax(sc * (np.asarray(q, np.float64) @ K.T)) @ V * 0.5),
    "unnormalised": lambda q, K, V, sc: np.exp(sc * (np.asarray(q, np.float64) @ K.T)
                                               - (sc * (np.asarray(q) @ K.T)).max()) @ V,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_the_pin(name):
    assert _pin(MUTANTS[name]) != [], f"the pin does not catch: {name}"


# --------------------------------------------------------------------------
# attn_prefill_rows_ref: causal rows of one head group, batched.  Pinned
# against torch SDPA with a lower-right causal mask (fp64, grouped heads) and
# against the oracle's whole-cache attn_prefill_ref.
# --------------------------------------------------------------------------
def _pin_prefill_rows(fn):
    from torch.nn.attention.bias import causal_lower_right
    failed = []
    rng = np.random.default_rng(32)
    for (G, n_past, n_q, rows, chunk) in ((4, 20, 9, range(9), 64), (8, 0, 70, range(70), 16),
                                          (2, 130, 40, [0, 5, 39, 17, 3], 2)):
        T = n_past + n_q
        K = rng.standard_normal((T + 3, 128)) * 1.5        # keys past T must not count
        V = rng.standard_normal((T + 3, 128))
        q = rng.standard_normal((n_q, G, 128))
        want = F.scaled_dot_product_attention(
            torch.from_numpy(q).transpose(0, 1)[None], torch.from_numpy(K[:T])[None, None],
            torch.from_numpy(V[:T])[None, None], attn_mask=causal_lower_right(n_q, T),
            scale=0.2, enable_gqa=True)[0].transpose(0, 1).numpy()
        rows = list(rows)
        try:
            got = fn(q[rows], K, V, n_past, rows, 0.2, chunk)
        except Exception:
            failed.append(f"sdpa G={G}")
            continue
        if got.shape != (len(rows), G, 128) or not np.allclose(got, want[rows], rtol=1e-12,
                                                               atol=1e-13):
            failed.append(f"sdpa G={G} n_past={n_past}")
    # against attn_prefill_ref on a packed cache
    n_past, n_q, Hkv, G = 33, 20, 2, 4
    x = rng.standard_normal((2, 1, Hkv, n_past + n_q, 128)).astype(np.float32)
    kc, vc = o.quantize_blocks(x[0], seed=5)[0], o.quantize_blocks(x[1], seed=5)[0]
    q = rng.standard_normal((1, n_q, Hkv * G, 128))
    ref = o.attn_prefill_ref(q, kc, vc, n_past, 0.09, seed=5)
    for g in range(Hkv):
        Kd, Vd = o.dequantize_blocks(kc[0, g], 5), o.dequantize_blocks(vc[0, g], 5)
        rows = list(range(n_q))
        got = fn(q[0, :, g * G:(g + 1) * G], Kd, Vd, n_past, rows, 0.09, 8)
        if not np.allclose(got, ref[0, :, g * G:(g + 1) * G], rtol=1e-12, atol=1e-13):
            failed.append(f"whole-cache g={g}")
    return failed


def test_prefill_rows_ref_matches_sdpa_and_whole_cache_reference():
    assert _pin_prefill_rows(o.attn_prefill_rows_ref) == []


def _masked(q_rows, K, V, n_past, rows, sc, chunk, off):
    """attention with keys 0 .. n_past + i + off (off = 0 is the right rule)"""
    out = []
    for j, i in enumerate(rows):
        n = max(1, n_past + int(i) + 1 + off)
        out.append(o.attn_decode_rows_ref(q_rows[j], K[:n], V[:n], sc))
    return np.stack(out)


PREFILL_MUTANTS = {
    "diagonal excluded": lambda q, K, V, n_past, rows, sc, ch: _masked(q, K, V, n_past, rows, sc, ch, -1),
    "one key past the diagonal": lambda q, K, V, n_past, rows, sc, ch: _masked(q, K, V, n_past, rows, sc, ch, 1),
    "no causal mask": lambda q, K, V, n_past, rows, sc, ch: _masked(q, K, V, n_past, rows, sc, ch,
                                                                    10 ** 6),
    "rows ignored": lambda q, K, V, n_past, rows, sc, ch: _masked(q, K, V, n_past,
                                                                  list(range(len(rows))), sc, ch, 0),
}


@pytest.mark.parametrize("name", sorted(PREFILL_MUTANTS))
def test_planted_prefill_mistakes_fail_the_pin(name):
    assert _pin_prefill_rows(PREFILL_MUTANTS[name]) != [], f"the pin does not catch: {name}"
