"""GPU parity of the sparse-MLA control paths that ordinary inputs never reach.

With N(0,1)/sqrt(D) inputs every logit of a query lies within a few units of
the others, so the kernels' softmax bookkeeping never leaves its fast path.
These cases plant selected rows whose logits exceed every earlier one by a
wide margin, and check the results against the float64 oracle:

* bf16 kernel (prefill, and decode with split partials): a head's softmax
  reference is the maximum of its first tile of 32 rows; a later row more
  than 64 log2 units (about 44 natural units) above it makes the workgroup
  start over with the exact maximum.  128 heads run the lagged schedule,
  32 and 64 heads the plain one; fp8 prefill rows take the same kernel after
  widening.
* fp8 decode kernel: a head's reference moves (and the accumulated output is
  rescaled) whenever a tile of 64 rows raises the maximum by more than 8
  log2 units; rows planted in successive tiles make it move several times.
* rows beyond 4 GiB of latent KV (64-bit gather addresses), selected on both
  sides of the 2^32-byte line, in prefill and decode.
* a NaN row that no query selects: slots of a partial tile must not read it.

Gates as in test_gpu_parity.py: bf16 rows max-abs <= 2e-2 and relative
max-abs <= 1e-2, fp8 rows 6e-2 and 3e-2, lse within 1e-3 (natural log).
"""

import numpy as np
import pytest
import torch

from oracle import pipeline as opl
from synth.draw import to_bf16_bits, to_e4m3fn_blocks

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import deepseek_v3_context_amd as ds  # noqa: E402
    from tests import gpu_path as gp  # noqa: E402

D, DL = 576, 512
SCALE = 1.0 / 24.0


def _gates(fmt):
    return (6e-2, 3e-2) if fmt == "fp8" else (2e-2, 1e-2)


def _inputs(n_q, heads, rows, seed, rope_q):
    """q [n_q, heads, 576], kv [rows, 576] in float32: N(0,1)/24 everywhere,
    except the rope part of q, which is rope_q[h] (a per-head constant), so
    that a kv row whose rope part is c has a logit of about
    SCALE * 64 * c * rope_q[h] for head h."""
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((n_q, heads, D)) / 24).astype(np.float32)
    q[:, :, DL:] = np.asarray(rope_q, dtype=np.float32)[None, :, None]
    kv = (rng.standard_normal((rows, D)) / 24).astype(np.float32)
    return q, kv, rng


def _plant(kv, row, rope, rng):
    """A row with rope part `rope` and a latent part in [-0.5, 0.5]."""
    kv[row, :DL] = rng.uniform(-0.5, 0.5, DL).astype(np.float32)
    kv[row, DL:] = rope


def _run_and_check(q, kv, idx, fmt, decode, label):
    qb = to_bf16_bits(q)
    if fmt == "bf16":
        kvs, scale = to_bf16_bits(kv), None
    else:
        kvs, scale = to_e4m3fn_blocks(kv)
    qd = gp.to_dev(qb, "bf16")
    kvd = gp.to_dev(kvs, fmt)
    sd = None if scale is None else torch.from_numpy(scale).to(gp.DEV)
    fn = ds.sparse_mla_decode if decode else ds.sparse_mla_prefill
    gp.say(f"[gpu] {label}: {fn.__name__} {q.shape[1]} heads {fmt}")
    out, lse = fn(qd, kvd, torch.from_numpy(idx).to(gp.DEV), SCALE, DL, kv_scale=sd)
    torch.cuda.synchronize()
    ref_o, ref_l = opl.sparse_mla_rows(list(range(q.shape[0])), list(idx), qb, "bf16", kvs, fmt,
                                       scale, SCALE, DL)
    got_o = out.float().cpu().numpy()
    err = np.abs(got_o - ref_o).max()
    rel = err / np.abs(ref_o).max()
    lerr = np.abs(lse.cpu().numpy() - ref_l).max()
    gp.say(f"  {label}: max|dO|={err:.3e} rel={rel:.3e} max|dlse|={lerr:.3e} "
           f"lse range [{ref_l.min():.1f}, {ref_l.max():.1f}]")
    abs_gate, rel_gate = _gates(fmt)
    assert np.isfinite(got_o).all(), label
    assert err <= abs_gate and rel <= rel_gate, (label, err, rel)
    assert lerr <= 1e-3, (label, lerr)


@pytest.mark.parametrize("heads", [128, 64, 32])
@pytest.mark.parametrize("decode", [False, True], ids=["prefill", "decode"])
def test_wide_kernel_restart_with_exact_maximum(heads, decode):
    # per-head rope constants: most heads far above the 64-log2 bail
    # margin, a few below it (they restart with their workgroup anyway)
    rope_q = np.linspace(6.0, 30.0, heads).round()
    n_q, rows, k = 6, 3000, 1024
    q, kv, rng = _inputs(n_q, heads, rows, seed=300 + heads + decode, rope_q=rope_q)
    idx = np.full((n_q, k), -1, dtype=np.int32)
    perm = rng.permutation(np.arange(10, rows))
    for j in range(n_q):
        idx[j] = perm[j * 300: j * 300 + k] if j * 300 + k <= perm.size else rng.choice(perm, k, False)
    A, B, C = 1, 2, 3          # planted rows: rope 1, 63/64 and 0.75 (all exact in bf16)
    _plant(kv, A, 1.0, rng)
    _plant(kv, B, 63.0 / 64.0, rng)
    _plant(kv, C, 0.75, rng)
    for r in range(4, 8):      # more rows like A (other latent parts)
        _plant(kv, r, 1.0, rng)
    # query 0: nothing planted (no restart)
    # query 1: two planted rows well past the first tile
    idx[1, 40], idx[1, 77] = A, B
    # query 2: planted rows in the last, partial tile (900 valid slots)
    idx[2, 900:] = -1
    idx[2, 898], idx[2, 899] = A, B
    # query 3: a large row in the first tile, a larger one later within the
    # margin for most heads (weights up to 2^64 without a restart)
    idx[3, 5], idx[3, 700] = C, A
    # query 4: planted rows in every split's range (decode: 256 rows each),
    # past each split's first tile, with empty slots in between
    for i, s0 in enumerate((0, 256, 512, 768)):
        idx[4, s0 + 50] = 4 + i
    idx[4, 256 + 51] = B
    idx[4, 300:400] = -1
    # query 5: the planted rows and few others (ragged: 70 valid slots)
    idx[5, 70:] = -1
    idx[5, 33], idx[5, 69] = B, A
    _run_and_check(q, kv, idx, "bf16", decode, f"restart {heads}h")


def test_wide_kernel_restart_fp8_prefill_rows():
    heads = 128
    rope_q = np.linspace(10.0, 30.0, heads).round()
    n_q, rows, k = 3, 2000, 512
    q, kv, rng = _inputs(n_q, heads, rows, seed=320, rope_q=rope_q)
    idx = np.stack([rng.permutation(np.arange(8, rows))[:k] for _ in range(n_q)]).astype(np.int32)
    _plant(kv, 2, 1.0, rng)
    _plant(kv, 5, 63.0 / 64.0, rng)
    idx[1, 100], idx[1, 101] = 2, 5
    idx[2, 300:] = -1
    idx[2, 299], idx[2, 40] = 2, 5
    _run_and_check(q, kv, idx, "fp8", False, "restart fp8 prefill")


def test_fp8_decode_lazy_rescale_moves_the_reference():
    heads = 128
    rope_q = np.linspace(8.0, 24.0, heads).round()
    n_q, rows, k = 4, 4000, 1024
    q, kv, rng = _inputs(n_q, heads, rows, seed=330, rope_q=rope_q)
    idx = np.stack([rng.permutation(np.arange(16, rows))[:k] for _ in range(n_q)]).astype(np.int32)
    # rows whose logits climb by about 2.7 * rope_q[h] * step natural units
    # per tile: 0.25 -> 0.5 -> 0.75 -> 1.0 of the rope constant
    for i, c in enumerate((0.25, 0.5, 0.75, 1.0)):
        _plant(kv, 1 + i, c, rng)
    # query 1: one planted row per 64-row tile of split 0 (rows 0..255)
    for i in range(4):
        idx[1, 64 * i + 10] = 1 + i
    # query 2: the same within split 2, rising then falling
    for i, r in enumerate((1, 3, 4, 2)):
        idx[2, 512 + 64 * i + 20] = r
    # query 3: climbing across the splits, with empty slots
    for i in range(4):
        idx[3, 256 * i + 100] = 1 + i
    idx[3, 600:700] = -1
    _run_and_check(q, kv, idx, "fp8", True, "fp8 lazy rescale")


@pytest.mark.parametrize("decode", [False, True], ids=["prefill", "decode"])
def test_latent_kv_beyond_4_gib(decode):
    # 3.8 M rows of 1152 bytes (4.38 GB); rows 3 728 271 and up start past
    # byte 2^32.  Only the selected rows hold data; every other row is zero
    # (finite), and the oracle sees the selected rows only.
    rows_total = 3_800_000
    line = -(-(1 << 32) // (2 * D))      # first row that starts at or past 2^32 bytes
    assert line * 2 * D >= (1 << 32) > (line - 1) * 2 * D   # row line-1 straddles it
    heads, n_q, k = 128, 4, 512
    rng = np.random.default_rng(340 + decode)
    below = rng.choice(np.arange(0, line - 1), 600, replace=False)
    above = rng.choice(np.arange(line - 1, rows_total), 600, replace=False)
    pool = np.concatenate([below, above, [line - 1, line, rows_total - 1]]).astype(np.int64)
    pool = np.unique(pool)
    idx = np.stack([rng.choice(pool, k, replace=False) for _ in range(n_q)]).astype(np.int32)
    idx[0, :3] = [line - 1, line, rows_total - 1]   # the rows around the line, and the last
    idx[2, 400:] = -1
    used = np.unique(idx[idx >= 0])
    vals = (rng.standard_normal((used.size, D)) / 4).astype(np.float32)
    qv = (rng.standard_normal((n_q, heads, D)) / 4).astype(np.float32)
    vb, qb = to_bf16_bits(vals), to_bf16_bits(qv)
    kv = torch.zeros((rows_total, D), dtype=torch.bfloat16, device=gp.DEV)
    kv[torch.from_numpy(used).to(gp.DEV)] = gp.to_dev(vb, "bf16")
    fn = ds.sparse_mla_decode if decode else ds.sparse_mla_prefill
    gp.say(f"[gpu] 4 GiB+ latent KV: {fn.__name__}")
    out, lse = fn(gp.to_dev(qb, "bf16"), kv, torch.from_numpy(idx).to(gp.DEV), SCALE, DL)
    torch.cuda.synchronize()
    del kv
    torch.cuda.empty_cache()
    pos = {int(r): i for i, r in enumerate(used)}
    local = np.where(idx >= 0, np.vectorize(lambda r: pos.get(int(r), -1))(idx), -1)
    ref_o, ref_l = opl.sparse_mla_rows(list(range(n_q)), list(local), qb, "bf16", vb, "bf16", None,
                                       SCALE, DL)
    err = np.abs(out.float().cpu().numpy() - ref_o).max()
    rel = err / np.abs(ref_o).max()
    lerr = np.abs(lse.cpu().numpy() - ref_l).max()
    gp.say(f"  4 GiB+ {fn.__name__}: max|dO|={err:.3e} rel={rel:.3e} max|dlse|={lerr:.3e}")
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)
    assert lerr <= 1e-3, lerr


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("decode", [False, True], ids=["prefill", "decode"])
def test_unselected_nan_row_is_never_used(fmt, decode):
    # row 0 holds NaN (and so does every row no query selects); queries
    # with partial tiles and empty slots must not pick it up
    heads, n_q, rows, k = 128, 5, 1500, 512
    rng = np.random.default_rng(350 + decode)
    q = (rng.standard_normal((n_q, heads, D)) / 24).astype(np.float32)
    kv = (rng.standard_normal((rows, D)) / 24).astype(np.float32)
    idx = np.stack([rng.choice(np.arange(1, rows), k, replace=False) for _ in range(n_q)])
    idx = idx.astype(np.int32)
    idx[0, 17:] = -1
    idx[1, 100:200] = -1
    idx[2, 250:] = -1
    idx[3, ::3] = -1
    qb = to_bf16_bits(q)
    if fmt == "bf16":
        kvs, scale = to_bf16_bits(kv), None
        kvs[0] = 0x7FC0                                     # bf16 quiet NaN
    else:
        kvs, scale = to_e4m3fn_blocks(kv)
        kvs[0] = 0x7F                                       # e4m3fn NaN
    fn = ds.sparse_mla_decode if decode else ds.sparse_mla_prefill
    gp.say(f"[gpu] NaN row 0 never selected: {fn.__name__} {fmt}")
    sd = None if scale is None else torch.from_numpy(scale).to(gp.DEV)
    out, lse = fn(gp.to_dev(qb, "bf16"), gp.to_dev(kvs, fmt), torch.from_numpy(idx).to(gp.DEV),
                  SCALE, DL, kv_scale=sd)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all() and np.isfinite(lse.cpu().numpy()).all()
    ref_o, ref_l = opl.sparse_mla_rows(list(range(n_q)), list(idx), qb, "bf16", kvs, fmt, scale,
                                       SCALE, DL)
    err = np.abs(got - ref_o).max()
    abs_gate, rel_gate = _gates(fmt)
    assert err <= abs_gate and err / np.abs(ref_o).max() <= rel_gate, err
    assert np.abs(lse.cpu().numpy() - ref_l).max() <= 1e-3
