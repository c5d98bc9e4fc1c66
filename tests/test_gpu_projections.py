"""GPU parity of the projection GEMM (gemm_bf16_nt) against the oracle.

Every projection around the path at DeepSeek-V3.2's dimensions (hidden
7168, q compression 1536, 128 heads x (128 + 64), latent 512, value head
128; indexer 64 x 128), on ragged token counts that span two row tiles, and
the per-head absorbed products on strided in-place views (the latent part of
the 576-wide MLA query row, the nope part of the q_up output).  Full-size
shapes (the 65536-token prefill's 8192 rank tokens) are checked on sampled
rows.  Gate per element, from bf16 output rounding (relative 2^-8) and fp32
accumulation of K products:
    |gpu - ref| <= 2^-8 |ref| + 1e-4 sum_k |a_k b_k|.
"""

import numpy as np
import pytest
import torch

from oracle import projections as pj

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import deepseek_v3_context_amd as ds  # noqa: E402
    from tests import gpu_path as gp  # noqa: E402

HID, QL, H, DN, DR, DL, DV, HI, DI = 7168, 1536, 128, 128, 64, 512, 128, 64, 128
SHAPES = {                       # name: (N, K)
    "mla_q_down": (QL, HID),
    "mla_q_up": (H * (DN + DR), QL),
    "indexer_wq_b": (HI * DI, QL),
    "indexer_w_k": (DI, HID),
    "o_proj": (HID, H * DV),
}


def _bf16(shape, g, scale):
    return (torch.randn(shape, generator=g) * scale).bfloat16()


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _f64(t):
    return (_u16(t).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _gate(got, a64, b64):
    ref = pj.gemm_nt(a64, b64)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * pj.gemm_nt(np.abs(a64), np.abs(b64))
    err = np.abs(got - ref)
    return float(err.max()), float((err - bound).max()), ref


@pytest.mark.parametrize("name", list(SHAPES))
def test_projection_shapes_ragged_tokens(name):
    N, K = SHAPES[name]
    M = 300
    g = torch.Generator().manual_seed(100 + sorted(SHAPES).index(name))
    a = _bf16((M, K), g, 1.0)
    w = _bf16((N, K), g, K ** -0.5)
    gp.say(f"[gpu] gemm {name}: M={M} N={N} K={K}")
    out = ds.gemm_bf16_nt(a.to(gp.DEV), w.to(gp.DEV))
    torch.cuda.synchronize()
    got = _f64(out.cpu())
    err, over, _ = _gate(got, _f64(a), _f64(w))
    gp.say(f"  max|err|={err:.3e}")
    assert over <= 0, (name, err)


def test_fp32_output_and_split_k_partials():
    # N = 128 and K = 7168 over few row tiles: split over K, summed in order
    g = torch.Generator().manual_seed(7)
    a, w = _bf16((40, 7168), g, 1.0), _bf16((256, 7168), g, 7168 ** -0.5)
    out = ds.gemm_bf16_nt(a.to(gp.DEV), w.to(gp.DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    err, over, _ = _gate(out.cpu().numpy().astype(np.float64), _f64(a), _f64(w))
    assert ds.gemm_bf16_nt_workspace_size(40, 256, 7168, 1) > 0
    assert over <= 0, err


def test_absorbed_products_on_strided_views():
    # q_latent[:, h, :] = q_nope[:, h, :] . W_UK[h] written into the latent
    # part of the 576-wide MLA query; o[:, h, :] = O_latent[:, h, :] . W_UV[h]
    n = 270
    g = torch.Generator().manual_seed(11)
    q_up = _bf16((n, H, DN + DR), g, 1.0).to(gp.DEV)
    w_uk = _bf16((H, DL, DN), g, DN ** -0.5).to(gp.DEV)          # W_UK[h]^T: [latent, nope]
    q_mla = torch.full((n, H, DL + DR), 7.0, dtype=torch.bfloat16, device=gp.DEV)
    ds.gemm_bf16_nt(q_up[:, :, :DN].transpose(0, 1), w_uk, out=q_mla[:, :, :DL].transpose(0, 1))
    o_lat = _bf16((n, H, DL), g, 1.0).to(gp.DEV)
    w_uv = _bf16((H, DV, DL), g, DL ** -0.5).to(gp.DEV)          # W_UV[h]^T: [v_head, latent]
    o = torch.empty((n, H * DV), dtype=torch.bfloat16, device=gp.DEV)
    ds.gemm_bf16_nt(o_lat.transpose(0, 1), w_uv, out=o.view(n, H, DV).transpose(0, 1))
    torch.cuda.synchronize()
    gp.say("[gpu] absorbed q and value up-projection on strided views")
    qn, wk = _f64(q_up.cpu())[:, :, :DN], _f64(w_uk.cpu())
    ref_q = pj.absorbed_q(qn, wk)
    got_q = _f64(q_mla.cpu())
    assert (got_q[:, :, DL:] == 7.0).all()                       # rope part untouched
    bound = 2.0 ** -8 * np.abs(ref_q) + 1e-4 * pj.absorbed_q(np.abs(qn), np.abs(wk))
    assert (np.abs(got_q[:, :, :DL] - ref_q) <= bound).all()
    ol, wv = _f64(o_lat.cpu()), _f64(w_uv.cpu())
    ref_o = pj.value_up(ol, wv)
    bound = 2.0 ** -8 * np.abs(ref_o) + 1e-4 * pj.value_up(np.abs(ol), np.abs(wv))
    assert (np.abs(_f64(o.cpu()).reshape(n, H, DV) - ref_o) <= bound).all()


@pytest.mark.parametrize("name", ["o_proj", "indexer_w_k", "mla_q_up", "mla_q_down"])
def test_full_size_sampled_rows(name):
    # the 65536-token prefill's 8192 rank tokens; 24 sampled rows, all
    # columns.  Tile widths: 256 (o_proj, q_up), 128 with split-K (w_k), 128
    # chosen so that no split is needed (q_down: 192 wide tiles < the CUs)
    N, K = SHAPES[name]
    M = 8192
    g = torch.Generator(device=gp.DEV).manual_seed(5)
    a = (torch.randn((M, K), generator=g, device=gp.DEV)).bfloat16()
    w = (torch.randn((N, K), generator=g, device=gp.DEV) * K ** -0.5).bfloat16()
    gp.say(f"[gpu] gemm {name} full size: M={M} N={N} K={K}")
    out = ds.gemm_bf16_nt(a, w)
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, 255, 256, M - 1]) |
                  set(np.random.default_rng(6).choice(M, 19, replace=False).tolist()))
    got = _f64(out[rows].cpu())
    err, over, _ = _gate(got, _f64(a[rows].cpu()), _f64(w.cpu()))
    gp.say(f"  max|err|={err:.3e}")
    assert over <= 0, (name, err)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N", [128, 256])
def test_output_at_unaligned_address_and_stride(out_dtype, N):
    # the output rows start one element past a 16-byte boundary and have an
    # odd stride, so the row-piece stores of the epilogue cannot be 16-byte
    # stores; M = 130 leaves a partial 64-row block.  Elements around the
    # output window keep their canary value.
    M, K = 130, 192
    g = torch.Generator().manual_seed(21 + N)
    a, w = _bf16((M, K), g, 1.0), _bf16((N, K), g, K ** -0.5)
    ld = N + 3
    buf = torch.full((M + 1, ld), 5.0, dtype=out_dtype, device=gp.DEV)
    out = buf.view(-1)[1: 1 + M * ld].view(M, ld)[:, :N]
    gp.say(f"[gpu] gemm output at an unaligned address: N={N} {out_dtype}")
    ds.gemm_bf16_nt(a.to(gp.DEV), w.to(gp.DEV), out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64) if out_dtype == torch.float32 else _f64(out.cpu())
    err, over, _ = _gate(got, _f64(a), _f64(w))
    assert over <= 0, err
    flat = buf.float().cpu().numpy().reshape(-1)
    mask = np.ones(flat.size, bool)
    for r in range(M):
        mask[1 + r * ld: 1 + r * ld + N] = False
    assert (flat[mask] == 5.0).all()
