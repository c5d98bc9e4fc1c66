"""The dense projections around the path -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources: "Model Parallel Strategy Analysis", step 3.1 (MLA's projections:
q_down, q_up, kv_down, kv_up for K and V, o_proj); "[RFC]: Parallel strategy
for Deepseek v3.2 like models", "Problem with tp" (the indexer's wq_b and w_k
projections).  The pages give the structure, not the arithmetic; each
projection is a plain matrix product of activations and a weight stored as
[out, in] (a linear layer), and the latent-form attention folds the K and V
up-projections into per-head products (q_latent = q_nope . W_UK,
o = O_latent . W_UV), written out here from the identity they rest on.

Readings taken (the pages are silent on the sizes): DeepSeek-V3.2's
published dimensions (hidden 7168, q compression 1536, 128 heads of
128 + 64 query dims, latent 512, value head 128; indexer 64 heads x 128).
"""

from __future__ import annotations

import numpy as np


def gemm_nt(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """C[.., m, n] = sum_k a[.., m, k] * b[.., n, k] in float64 (a linear
    layer with the weight stored as [out, in]; batched over leading axes).
    Parity: pinned against an explicit triple loop on small shapes."""
    a64 = np.asarray(a, dtype=np.float64)
    b64 = np.asarray(b, dtype=np.float64)
    return np.matmul(a64, np.swapaxes(b64, -1, -2))


def absorbed_q(q_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """Per head h: q_latent[:, h, :] = q_nope[:, h, :] . W_UK[h] with the
    weight stored as w_uk[h] = W_UK[h]^T ([latent, nope]).  Then
    <q_latent, c> = <q_nope, W_UK c>: the logit against a latent row c
    equals the logit against its up-projected key.  Parity: pinned by that
    identity."""
    return np.stack([gemm_nt(q_nope[:, h, :], w_uk[h]) for h in range(q_nope.shape[1])], axis=1)


def value_up(o_latent: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Per head h: o[:, h, :] = O_latent[:, h, :] . W_UV[h] with the weight
    stored as w_uv[h] = W_UV[h]^T ([v_head, latent]).  Attention output in
    latent form then up-projected equals attention over up-projected values.
    Parity: pinned by that identity."""
    return np.stack([gemm_nt(o_latent[:, h, :], w_uv[h]) for h in range(o_latent.shape[1])], axis=1)
