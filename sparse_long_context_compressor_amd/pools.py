"""Byte layouts of the three paged pools the library reads and writes.

Every pool is split into blocks of 64 rows; a per-sequence block table maps
logical block i (rows 64*i .. 64*i+63 of that sequence) to a physical block.
The layouts follow the pages' cache-block pictures (row data first, then the
block's scales after all its rows) with this library's row widths:

  SWA pool   bf16 [n_blocks][64][576]                      73728 B / block
  CMP pool   per block: 64 rows x (512 e4m3 codes | 64 bf16 rope) = 640 B,
             then 64 rows x 8 fp32 scales (one per 64 nope dims)  43008 B
  KEY pool   per block: 64 rows x 128 e4m3 codes, then 64 fp32   8448 B
  KEY4 pool  MXFP4 keys, per block: 64 rows x 64 bytes of e2m1 pairs (even
             element in the low nibble), then 64 rows x 4 E8M0 bytes  4352 B
  fp8 SWA    the CMP layout, rows at positions instead of slots

These helpers only move bytes (torch tensors, any device); they hold none of
the method's arithmetic.
"""
from __future__ import annotations

import torch

BLOCK_ROWS = 64
D_LATENT = 576
D_NOPE = 512
D_ROPE = 64
D_INDEX = 128
N_QBLK = D_NOPE // 64

SWA_BLOCK_BYTES = BLOCK_ROWS * D_LATENT * 2
CMP_ROW_BYTES = D_NOPE + 2 * D_ROPE                 # 640
CMP_SCALE_OFF = BLOCK_ROWS * CMP_ROW_BYTES          # 40960
CMP_BLOCK_BYTES = CMP_SCALE_OFF + BLOCK_ROWS * 4 * N_QBLK   # 43008
KEY_SCALE_OFF = BLOCK_ROWS * D_INDEX                # 8192
KEY_BLOCK_BYTES = KEY_SCALE_OFF + BLOCK_ROWS * 4    # 8448
KEY4_SCALE_OFF = BLOCK_ROWS * D_INDEX // 2          # 4096
KEY4_BLOCK_BYTES = KEY4_SCALE_OFF + BLOCK_ROWS * 4  # 4352


def _u8(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.uint8)


def _phys_rows(table_row: torch.Tensor, rows: torch.Tensor):
    """Physical (block, row-in-block) of logical rows through one table row."""
    blk = table_row.long()[rows // BLOCK_ROWS]
    return blk, rows % BLOCK_ROWS


def _logical_rows(n: int, start: int, device) -> torch.Tensor:
    return torch.arange(start, start + n, device=device, dtype=torch.long)


# --------------------------------------------------------------------- SWA
def swa_pool_empty(n_blocks: int, device="cpu") -> torch.Tensor:
    return torch.zeros(n_blocks, BLOCK_ROWS, D_LATENT, dtype=torch.bfloat16, device=device)


def swa_pool_put(pool: torch.Tensor, table_row: torch.Tensor, pos0: int, rows: torch.Tensor):
    """Write bf16 rows [n,576] for positions pos0 .. pos0+n-1 of one sequence."""
    r = _logical_rows(rows.shape[0], pos0, pool.device)
    b, i = _phys_rows(table_row.to(pool.device), r)
    pool[b, i] = rows.to(pool.device, torch.bfloat16)


def swa_pool_get(pool: torch.Tensor, table_row: torch.Tensor, pos0: int, n: int) -> torch.Tensor:
    r = _logical_rows(n, pos0, pool.device)
    b, i = _phys_rows(table_row.to(pool.device), r)
    return pool[b, i]


# --------------------------------------------------------------------- CMP
def cmp_pool_empty(n_blocks: int, device="cpu") -> torch.Tensor:
    return torch.zeros(n_blocks, CMP_BLOCK_BYTES, dtype=torch.uint8, device=device)


def _cmp_views(pool: torch.Tensor):
    nb = pool.shape[0]
    rows = pool.as_strided((nb, BLOCK_ROWS, CMP_ROW_BYTES), (CMP_BLOCK_BYTES, CMP_ROW_BYTES, 1))
    scl = pool.as_strided((nb, BLOCK_ROWS, 4 * N_QBLK), (CMP_BLOCK_BYTES, 4 * N_QBLK, 1),
                          CMP_SCALE_OFF)
    return rows, scl


def cmp_pool_put(pool, table_row, slot0, codes, scales, rope):
    """codes [n,512] uint8, scales [n,8] float32, rope [n,64] bfloat16 for
    logical slots slot0 .. slot0+n-1 of one sequence."""
    n = codes.shape[0]
    r = _logical_rows(n, slot0, pool.device)
    b, i = _phys_rows(table_row.to(pool.device), r)
    rows, scl = _cmp_views(pool)
    rows[b, i, :D_NOPE] = codes.to(pool.device, torch.uint8)
    rows[b, i, D_NOPE:] = _u8(rope.to(pool.device, torch.bfloat16)).reshape(n, 2 * D_ROPE)
    scl[b, i] = _u8(scales.to(pool.device, torch.float32)).reshape(n, 4 * N_QBLK)


def cmp_pool_get(pool, table_row, slot0, n):
    """Inverse of cmp_pool_put: (codes u8 [n,512], scales f32 [n,8], rope bf16 [n,64])."""
    r = _logical_rows(n, slot0, pool.device)
    b, i = _phys_rows(table_row.to(pool.device), r)
    rows, scl = _cmp_views(pool)
    rr = rows[b, i]
    codes = rr[:, :D_NOPE].contiguous()
    rope = rr[:, D_NOPE:].contiguous().view(torch.bfloat16).reshape(n, D_ROPE)
    scales = scl[b, i].contiguous().view(torch.float32).reshape(n, N_QBLK)
    return codes, scales, rope


# --------------------------------------------------------------------- KEY
def key_pool_empty(n_blocks: int, device="cpu") -> torch.Tensor:
    return torch.zeros(n_blocks, KEY_BLOCK_BYTES, dtype=torch.uint8, device=device)


def _key_views(pool):
    nb = pool.shape[0]
    codes = pool.as_strided((nb, BLOCK_ROWS, D_INDEX), (KEY_BLOCK_BYTES, D_INDEX, 1))
    scl = pool.as_strided((nb, BLOCK_ROWS, 4), (KEY_BLOCK_BYTES, 4, 1), KEY_SCALE_OFF)
    return codes, scl


def key_pool_put(pool, table_row, slot0, codes, scales):
    """codes [n,128] uint8, scales [n] float32 for slots slot0 .. slot0+n-1."""
    n = codes.shape[0]
    r = _logical_rows(n, slot0, pool.device)
    b, i = _phys_rows(table_row.to(pool.device), r)
    c, s = _key_views(pool)
    c[b, i] = codes.to(pool.device, torch.uint8)
    s[b, i] = _u8(scales.to(pool.device, torch.float32)).reshape(n, 4)


def key_pool_get(pool, table_row, slot0, n):
    r = _logical_rows(n, slot0, pool.device)
    b, i = _phys_rows(table_row.to(pool.device), r)
    c, s = _key_views(pool)
    return c[b, i].contiguous(), s[b, i].contiguous().view(torch.float32).reshape(n)


# -------------------------------------------------------------------- KEY4
def key4_pool_empty(n_blocks: int, device="cpu") -> torch.Tensor:
    return torch.zeros(n_blocks, KEY4_BLOCK_BYTES, dtype=torch.uint8, device=device)


def _key4_views(pool):
    nb = pool.shape[0]
    codes = pool.as_strided((nb, BLOCK_ROWS, D_INDEX // 2), (KEY4_BLOCK_BYTES, D_INDEX // 2, 1))
    scl = pool.as_strided((nb, BLOCK_ROWS, 4), (KEY4_BLOCK_BYTES, 4, 1), KEY4_SCALE_OFF)
    return codes, scl


def key4_pool_put(pool, table_row, slot0, codes4, e8m0):
    """codes4 [n,64] uint8 (packed e2m1 pairs), e8m0 [n,4] uint8 for slots
    slot0 .. slot0+n-1."""
    n = codes4.shape[0]
    r = _logical_rows(n, slot0, pool.device)
    b, i = _phys_rows(table_row.to(pool.device), r)
    c, s = _key4_views(pool)
    c[b, i] = codes4.to(pool.device, torch.uint8)
    s[b, i] = e8m0.to(pool.device, torch.uint8)


def key4_pool_get(pool, table_row, slot0, n):
    r = _logical_rows(n, slot0, pool.device)
    b, i = _phys_rows(table_row.to(pool.device), r)
    c, s = _key4_views(pool)
    return c[b, i].contiguous(), s[b, i].contiguous()
