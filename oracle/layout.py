"""Row gather / scatter between padded and packed layouts -- TEST INFRASTRUCTURE ONLY.

Follows the packed-path diagram on the page "Lesson 5: IAW model FA2 vs FA3
measured" (section 1): unpad takes the rows named by ``indices`` out of the
padded (B, total_len, H, D) tensor into a compact (total_valid, H, D) tensor;
pad puts the compact rows back at those positions.  Reading where the page is
silent: rows of the padded result that no index names hold +0.0 (the page's
pad path runs a fill kernel before the index write, section 6).

Both functions work on whole rows of bytes, so they are exact for any dtype.

mask_to_varlen derives the unpad inputs from a padding mask (section 1: the
indices name the rows that are not padding; the varlen attention on the
compact rows needs the sequence offsets).  Reading where the page is silent:
the padded tensor is B slots of L rows, a nonzero mask byte marks a valid row,
each slot's valid rows (in row order) form one sequence, indices list the valid
rows in row-major order, cu_seqlens are the running sums of the per-slot
counts (empty slots give empty sequences), and max_seqlen is the largest count.
"""

from __future__ import annotations

import numpy as np


def _rows(x: np.ndarray, n_rows: int, row_elems: int) -> np.ndarray:
    return np.ascontiguousarray(x).reshape(n_rows, row_elems)


def unpad_gather(src: np.ndarray, indices: np.ndarray, row_shape) -> np.ndarray:
    """dst[r] = src_row[indices[r]] for r in range(len(indices)).

    ``src`` holds ``prod(src.shape) / prod(row_shape)`` rows of shape
    ``row_shape``; the result has shape (len(indices), *row_shape).
    """
    row_elems = int(np.prod(row_shape))
    n_rows = src.size // row_elems
    rows = _rows(src, n_rows, row_elems)
    out = np.empty((len(indices), row_elems), dtype=src.dtype)
    for r, idx in enumerate(np.asarray(indices, dtype=np.int64)):
        out[r] = rows[idx]
    return out.reshape((len(indices),) + tuple(row_shape))


def pad_scatter(src: np.ndarray, indices: np.ndarray, n_rows_total: int) -> np.ndarray:
    """dst = zeros(n_rows_total rows); dst[indices[r]] = src[r] for every r."""
    n_valid = len(indices)
    row_shape = src.shape[1:]
    row_elems = int(np.prod(row_shape))
    rows = _rows(src, n_valid, row_elems)
    out = np.zeros((n_rows_total, row_elems), dtype=src.dtype)
    for r, idx in enumerate(np.asarray(indices, dtype=np.int64)):
        out[idx] = rows[r]
    return out.reshape((n_rows_total,) + tuple(row_shape))


def mask_to_varlen(mask: np.ndarray):
    """mask (B, L), nonzero = valid row.  Returns (indices int32 (n_valid,),
    cu_seqlens int32 (B + 1,), max_seqlen int)."""
    m = np.asarray(mask) != 0
    indices = np.flatnonzero(m.reshape(-1)).astype(np.int32)
    counts = m.sum(axis=1).astype(np.int64)
    cu = np.zeros(m.shape[0] + 1, dtype=np.int64)
    np.cumsum(counts, out=cu[1:])
    return indices, cu.astype(np.int32), int(counts.max()) if counts.size else 0
