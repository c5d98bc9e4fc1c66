"""The allocation-free decode entry point against sparse_mla_decode.

sparse_mla_decode_noalloc keeps its split partials in the library's own
device array instead of a caller workspace.  Two calls in a row on one
GPU (the second with fewer queries, fewer selected rows and fewer heads, so
it reuses the array over a part of what the first one left there) must
each match sparse_mla_decode on the same inputs within the bf16 gates
(max-abs <= 2e-2, relative max-abs <= 1e-2, lse within 1e-3): the two may
split the rows differently, which changes only the bf16 rounding of the
partials.  A third call, with more queries than the array holds at the
default split count, takes fewer splits and still matches.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import deepseek_v3_context_amd as ds  # noqa: E402
    from tests import gpu_path as gp  # noqa: E402


def _case(n_q, heads, rows, k, valid, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    rng = np.random.default_rng(seed)
    q = (torch.randn(n_q, heads, 576, generator=g) / 24).bfloat16().to(gp.DEV)
    kv = (torch.randn(rows, 576, generator=g) / 24).bfloat16().to(gp.DEV)
    idx = np.full((n_q, k), -1, dtype=np.int32)
    for j in range(n_q):
        cnt = valid if j % 2 == 0 else int(rng.integers(1, valid + 1))   # ragged tails
        idx[j, :cnt] = rng.choice(rows, cnt, replace=False)
    return q, kv, torch.from_numpy(idx).to(gp.DEV)


@pytest.mark.parametrize("call", [
    dict(n_q=32, heads=128, rows=40000, k=2048, valid=2048, seed=61),   # the 32-request decode
    dict(n_q=5, heads=64, rows=3000, k=512, valid=400, seed=62),        # smaller, right after
    dict(n_q=48, heads=128, rows=20000, k=2048, valid=1500, seed=63),   # fewer splits than default
])
def test_noalloc_decode_matches_the_workspace_variant(call):
    scale = 1.0 / 24.0
    q, kv, idx = _case(**call)
    n_q, heads = call["n_q"], call["heads"]
    gp.say(f"[gpu] sparse_mla_decode_noalloc vs sparse_mla_decode: {call}")
    ref_o, ref_l = ds.sparse_mla_decode(q, kv, idx, scale, 512)
    out = torch.full((n_q, heads, 512), float("nan"), dtype=torch.bfloat16, device=gp.DEV)
    lse = torch.full((n_q, heads), float("nan"), dtype=torch.float32, device=gp.DEV)
    got_o, got_l = ds.sparse_mla_decode_noalloc(q, kv, idx, scale, 512, out=out, lse=lse)
    torch.cuda.synchronize()
    a, b = got_o.float().cpu().numpy(), ref_o.float().cpu().numpy()
    assert np.isfinite(a).all() and np.isfinite(got_l.cpu().numpy()).all()
    err = np.abs(a - b).max()
    rel = err / np.abs(b).max()
    lerr = np.abs(got_l.cpu().numpy() - ref_l.cpu().numpy()).max()
    gp.say(f"  max|dO|={err:.3e} rel={rel:.3e} max|dlse|={lerr:.3e}")
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)
    assert lerr <= 1e-3, lerr
