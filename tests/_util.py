"""Shared helpers for the parity tests (no method arithmetic here)."""

import numpy as np

# Attention tolerance: max-abs 2e-3 and relative L2 1e-3 against the fp64
# oracle.  An fp16 output adds its own rounding, at most half an fp16 ulp of
# the reference value (<= 2^-11 |ref|), which is allowed on top of 2e-3.
MAX_ABS = 2e-3
REL_L2 = 1e-3


def attn_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def check_attn(got, ref, out_is_f16, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - ref)
    bound = MAX_ABS + (np.abs(ref) * 2.0 ** -11 if out_is_f16 else 0.0)
    worst = np.unravel_index(np.argmax(d - bound), d.shape)
    assert np.all(d <= bound), (f"{what}: |err| {d[worst]:.3e} > {bound[worst] if np.ndim(bound) else bound:.3e} "
                                f"at {worst} (ref {ref[worst]:.4f})")
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e} > {REL_L2}"
    return float(d.max()), float(rel)


def rising_scores_inputs(rng, B, T, H, G, n_q, vmag):
    """fp32 q [B][n_q][H*G][128], k, v [B][T][H][128] whose scores rise along
    the sequence: every key carries a growing multiple (0 .. 100) of one unit
    direction that the query heads point along (the normalised sum of the
    queries), so new score maxima keep arriving; V rows of every other run of
    512 positions are scaled by vmag (block scales above 256 when vmag is
    large)."""
    q = rng.standard_normal((B, n_q, H * G, 128))
    u = q.reshape(-1, 128).sum(axis=0)
    u /= np.linalg.norm(u)
    ramp = 100.0 * np.arange(T) / T
    k = rng.standard_normal((B, T, H, 128)) + ramp[None, :, None, None] * u
    v = rng.standard_normal((B, T, H, 128))
    v[:, (np.arange(T) // 512) % 2 == 1] *= vmag
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)
