"""GPU parity of the split metadata beyond the round-robin main path.

* the in-sequence split (the contrast mode): metadata and the row gather of
  cp_split_metadata_in_seq, bit-exact against the oracle's enumeration on
  the blog's 8000-token / 8-rank example, its 8000/800/5 batch, the
  six-request batch, and random batches with empty requests; a caller count
  above the rank's real count leaves the tail entries marked empty;
* decode_metadata, bit-exact against the oracle's definition.
"""

import numpy as np
import pytest
import torch

from oracle import pipeline as opl
from oracle import round_robin_cp as orr

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import deepseek_v3_context_amd as ds  # noqa: E402
    from tests import gpu_path as gp  # noqa: E402

KEYS = ("global_idx", "batch_idx", "local_cu", "kv_start", "kv_len")


def _batches():
    rng = np.random.default_rng(71)
    out = [([0, 8000], (8,)), ([0, 8000, 8800, 8805], (8,)),
           ([0, 8000, 8800, 8805, 11805, 13305, 25305], (8,)), ([0, 0, 3, 3, 17, 17], (1, 3, 8))]
    for _ in range(4):
        lens = rng.integers(0, 300, size=int(rng.integers(1, 9)))
        out.append(([0] + np.cumsum(lens).tolist(), (1, 2, 3, 8)))
    # more requests than one workgroup scans in a round (1024)
    lens = rng.integers(0, 9, size=2500)
    out.append(([0] + np.cumsum(lens).tolist(), (4,)))
    return out


@pytest.mark.parametrize("case", range(len(_batches())))
def test_in_seq_split_bit_exact(case):
    cu_host, cps = _batches()[case]
    T = int(cu_host[-1])
    cu = torch.tensor(cu_host, dtype=torch.int32, device=gp.DEV)
    ids = torch.arange(T, dtype=torch.int32, device=gp.DEV) * 7 + 3     # row contents = f(g)
    gp.say(f"[gpu] in-seq split: {len(cu_host) - 1} requests, T={T}, cp {cps}")
    for cp in cps:
        for r in range(cp):
            om = orr.in_seq_split_metadata(cu_host, cp, r)
            n = om["global_idx"].size
            assert ds.cp_in_seq_local_count(cu_host, cp, r) == n
            got = ds.cp_split_metadata_in_seq(cu, T, cp, r, n_local=n, rows_src=ids if T else None)
            torch.cuda.synchronize()
            for k in KEYS:
                assert np.array_equal(got[k].cpu().numpy(), om[k]), (cp, r, k)
            if T and n:
                assert np.array_equal(got["rows"].cpu().numpy(), om["global_idx"] * 7 + 3)


def test_in_seq_split_caller_count_above_the_real_count():
    cu_host = [0, 8000, 8800, 8805]
    cu = torch.tensor(cu_host, dtype=torch.int32, device=gp.DEV)
    om = orr.in_seq_split_metadata(cu_host, 8, 6)
    n = om["global_idx"].size
    rows = torch.full((n + 5,), -7, dtype=torch.int32, device=gp.DEV)
    ids = torch.arange(8805, dtype=torch.int32, device=gp.DEV)
    got = ds.cp_split_metadata_in_seq(cu, 8805, 8, 6, n_local=n + 5, rows_src=ids,
                                      out={"rows": rows})
    torch.cuda.synchronize()
    assert np.array_equal(got["global_idx"][:n].cpu().numpy(), om["global_idx"])
    assert (got["global_idx"][n:].cpu().numpy() == -1).all()
    assert (got["batch_idx"][n:].cpu().numpy() == -1).all()
    assert (got["kv_len"][n:].cpu().numpy() == 0).all()
    assert np.array_equal(rows[:n].cpu().numpy(), om["global_idx"])
    assert (rows[n:].cpu().numpy() == -7).all()            # skipped, left untouched


def test_decode_metadata_bit_exact():
    lengths = np.array([4096, 1, 65536, 0, 777, 33], dtype=np.int32)
    got = ds.decode_metadata(torch.from_numpy(lengths).to(gp.DEV))
    torch.cuda.synchronize()
    want = opl.decode_metadata(lengths)
    for k in ("q_req", "kv_start", "kv_len"):
        assert np.array_equal(got[k].cpu().numpy(), want[k]), k
