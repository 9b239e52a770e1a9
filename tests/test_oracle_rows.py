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
