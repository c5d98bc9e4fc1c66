"""Pins of oracle/projections.py: the matrix product against an explicit
loop, and the absorption identities of the latent-form attention."""

import numpy as np

from oracle import projections as pj
from oracle import sparse_attention as sa


def test_gemm_nt_against_a_triple_loop():
    rng = np.random.default_rng(1)
    for (bt, m, n, k) in ((1, 3, 4, 5), (3, 2, 6, 7)):
        a = rng.standard_normal((bt, m, k))
        b = rng.standard_normal((bt, n, k))
        c = pj.gemm_nt(a, b)
        for t in range(bt):
            for i in range(m):
                for j in range(n):
                    want = 0.0
                    for kk in range(k):
                        want += a[t, i, kk] * b[t, j, kk]
                    assert abs(c[t, i, j] - want) <= 1e-12 * (1 + abs(want))
    a2, b2 = rng.standard_normal((4, 9)), rng.standard_normal((5, 9))
    assert np.allclose(pj.gemm_nt(a2, b2), a2 @ b2.T, rtol=0, atol=1e-12)   # 2-d: a linear layer


def test_absorbed_queries_give_the_up_projected_logits():
    # q_nope . (W_UK c) == (q_nope . W_UK) . c for every head and latent row
    rng = np.random.default_rng(2)
    n, H, dn, dl, rows = 5, 4, 16, 32, 7
    q_nope = rng.standard_normal((n, H, dn))
    W_UK = rng.standard_normal((H, dn, dl))            # key up-projection per head
    c = rng.standard_normal((rows, dl))                # latent rows
    q_lat = pj.absorbed_q(q_nope, np.transpose(W_UK, (0, 2, 1)))
    for h in range(H):
        k_up = c @ W_UK[h].T                           # [rows, dn] up-projected keys
        assert np.allclose(q_lat[:, h, :] @ c.T, q_nope[:, h, :] @ k_up.T, rtol=1e-12, atol=1e-10)


def test_value_up_projection_after_latent_attention():
    # softmax-weighted latent rows then W_UV == softmax-weighted up-projected values
    rng = np.random.default_rng(3)
    n, H, dl, dv, rows = 3, 4, 32, 8, 9
    q = rng.standard_normal((n, H, dl)) / 4
    c = rng.standard_normal((rows, dl))
    W_UV = rng.standard_normal((H, dl, dv))
    o_lat = np.stack([np.stack([sa.sparse_mla_row(q[j], c, 0.3, dl)[0][h] for h in range(H)])
                      for j in range(n)])             # [n, H, dl] latent outputs (oracle MLA)
    o = pj.value_up(o_lat, np.transpose(W_UV, (0, 2, 1)))
    for j in range(n):
        for h in range(H):
            logits = 0.3 * (c @ q[j, h])
            p = np.exp(logits - logits.max())
            p /= p.sum()
            assert np.allclose(o[j, h], p @ (c @ W_UV[h]), rtol=1e-10, atol=1e-12)
