"""Seeded synthetic inputs for TBQ4 attention (shared by tests, bench and smoke).

This module only draws random numbers: it holds none of the quantiser's or of
attention's arithmetic, so both the HIP path and the CPU oracle may take their
inputs from it.  All draws use numpy PCG64 streams keyed by integer tuples, so
any (layer, tensor, sequence, KV head, chunk) slice can be regenerated on its
own without drawing the rest of the tensor.

Workloads (head_dim 128 throughout; G = query heads per KV head):

* ``tiny``        batch 1, 1 KV / 4 Q heads, 1024 cached tokens, K,V,Q ~ N(0,1)
                  from ``default_rng(0)`` in the order K, V, Q, then one key
                  channel scaled x20.  softmax scale 1/sqrt(128).
* ``decode16k``   batch 1, 8 / 64 heads, 16384 tokens; K,V ~ N(0,1) with two
                  outlier channels x15 per (KV head, tensor); Q ~ N(0,1)/sqrt(128)
                  with softmax scale 1.0.
* ``decode96k`` / ``decode128k``  batch 4, 8 / 64 heads, 98304 / 131072 tokens;
                  K,V ~ Student-t(nu=5) times per-(KV head, channel) scales drawn
                  from U[0.5, 4] once per tensor; Q ~ N(0,1), scale 1/sqrt(128).
* ``prefill``     batch 1, 8 / 64 heads, 131072 cached tokens then a chunk of
                  2048 queries; Q,K,V ~ N(0,1) with two outlier channels x15 on K
                  and V; scale 1/sqrt(128).
* ``longdecode``  batch 1, 8 / 64 heads, 4 layers, prefix 262080 tokens then 64
                  steps of (append one token, decode); K,V ~ Student-t(nu=3) plus a
                  per-(layer, tensor, KV head, channel) Gaussian random-walk mean
                  (step std 0.01, starting at 0); Q ~ N(0,1), scale 1/sqrt(128).

The long-context pages measure whole models on needle-in-a-haystack and public
suites; these synthetic tensors stand in for them with the same context lengths
(16K-262K), a GQA d=128 head geometry, and outlier / heavy-tailed KV statistics.
"""

from .gen import (  # noqa: F401
    WORKLOADS, Workload, tiny_inputs, kv_rows, kv_tensor, q_decode, q_prefill,
    K, V, Q,
)
