"""CPU model of the bf16 sparse-MLA kernel's LDS tile layout.

The kernel gathers a tile of 32 selected latent rows (1152 bytes each) into
LDS with 36 DMA wave-instructions and reads it back two ways: as K
fragments of the QK products and, with the transposing LDS read, as V^T
fragments of the PV products.  The index arithmetic of those three access
patterns is restated here from the kernel's layout rules (sparse_mla.hip:
wide_gather_slot, wide_koff, wide_voff and the DMA's lane placement) and
checked on a tile of distinct byte values: every tile byte is written
exactly once, and every fragment read returns the operand elements that
v_mfma_f32_16x16x32_bf16 expects, with the key order of the V^T fragments
equal to the key order of the P^T fragments the softmax writes.
"""

import numpy as np

ROWS, ROW_BYTES = 32, 1152
BLOCKS = ROW_BYTES // 32          # one DMA wave-instruction per 32-byte column block


def gather_slot(l):               # tile row whose bytes lane l gathers
    return (l & 31) ^ ((l >> 5) << 3)


def koff(l):                      # lane's K-fragment byte offset (kb 0, ks 0)
    hh = (l >> 4) & 1
    return (l >> 5) * 1024 + hh * 512 + ((l & 15) ^ (hh << 3)) * 16


def voff(l, col0):                # lane's transposed-V read offset
    li, g = l & 15, l >> 4
    hh = (li >> 1) & 1
    return (col0 >> 4) * 1024 + hh * 512 + ((4 * g + (li >> 2)) ^ (hh << 3)) * 16 + (li & 1) * 8


def dma_tile(rows):
    """LDS bytes after the 36 DMA instructions: lane l of instruction m
    lands 16 bytes at 1024m + 16l, taken from its row at 32m + 16(l >> 5)."""
    lds = np.full(BLOCKS * 1024, -1, dtype=np.int64)
    for m in range(BLOCKS):
        for l in range(64):
            src = rows[gather_slot(l), 32 * m + 16 * (l >> 5): 32 * m + 16 * (l >> 5) + 16]
            dst = 1024 * m + 16 * l
            assert (lds[dst: dst + 16] == -1).all(), "a byte written twice"
            lds[dst: dst + 16] = src
    return lds


def _tile():
    # byte value = a unique id of (row, byte): the model tracks where each lands
    return np.arange(ROWS * ROW_BYTES, dtype=np.int64).reshape(ROWS, ROW_BYTES)


def test_dma_writes_every_tile_byte_once():
    lds = dma_tile(_tile())
    assert (lds >= 0).all()
    assert np.array_equal(np.sort(lds), np.arange(ROWS * ROW_BYTES))


def test_k_fragments_are_the_mfma_a_operand():
    # A operand of 16x16x32: lane l holds row l % 16 of the 16-key block and
    # k elements 8 (l // 16) .. + 7 of the 32-element k-step: bytes
    # 64 ks + 16 (l // 16) .. + 15 of key 16 kb + l % 16
    rows = _tile()
    lds = dma_tile(rows)
    for kb in range(2):
        for ks in range(18):
            for l in range(64):
                off = koff(l) + kb * 256 + ks * 2048
                got = lds[off: off + 16]
                key = 16 * kb + (l & 15)
                want = rows[key, 64 * ks + 16 * (l >> 4): 64 * ks + 16 * (l >> 4) + 16]
                assert np.array_equal(got, want), (kb, ks, l)


def _read_tr_b16(lds, addrs):
    """ds_read_b64_tr_b16 over one 16-lane group: lane i names 4 bf16 (8
    bytes) at addrs[i]; together the group's lanes name a 4 x 16 block of
    bf16 (row i // 4, columns 4 (i % 4) .. + 3); lane i receives column i of
    the 4 rows.  Returns [16 lanes][4 values] of 2-byte element ids."""
    block = np.empty((4, 16, 2), dtype=np.int64)
    for i in range(16):
        for e in range(4):
            block[i // 4, 4 * (i % 4) + e] = lds[addrs[i] + 2 * e: addrs[i] + 2 * e + 2]
    return [[tuple(block[r, i]) for r in range(4)] for i in range(16)]


def test_v_fragments_are_the_transposed_values_in_p_key_order():
    # A operand of PV (O^T += V^T P^T): lane l holds output column
    # col0 + 16 c + l % 16 and 8 keys; the softmax writes P^T with keys
    # 16 kb + 4 (l // 16) + i (i < 4) for kb = 0, 1 in that order, so the V
    # fragment must hold the same 8 keys in the same order.
    rows = _tile()
    lds = dma_tile(rows)
    for col0 in (0, 128, 256, 384):          # the four waves' column ranges
        for c in range(8):
            for g in range(4):
                lanes = [16 * g + i for i in range(16)]
                lo = _read_tr_b16(lds, [voff(l, col0) + c * 1024 for l in lanes])
                hi = _read_tr_b16(lds, [voff(l, col0) + c * 1024 + 256 for l in lanes])
                for i in range(16):
                    col = col0 + 16 * c + i
                    keys = [4 * g + e for e in range(4)] + [16 + 4 * g + e for e in range(4)]
                    got = lo[i] + hi[i]
                    want = [tuple(rows[k, 2 * col: 2 * col + 2]) for k in keys]
                    assert list(got) == want, (col0, c, g, i)


def test_fragment_reads_stay_inside_the_tile():
    for l in range(64):
        assert 0 <= koff(l) + 256 + 17 * 2048 + 16 <= BLOCKS * 1024
        for col0 in (0, 128, 256, 384):
            assert 0 <= voff(l, col0) + 7 * 1024 + 256 + 8 <= BLOCKS * 1024
