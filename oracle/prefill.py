"""Plain CPU oracle of the non-absorbed path's first step (numpy, fp64).

TEST INFRASTRUCTURE: only the tests and the bench's CPU baseline use this module.
It shares nothing with the HIP path.

"DeepSeek-MLA-Principle" eqs. (2) and (4): the content key of head h at position
t is W_UK[h] c_t and its value W_UV[h] c_t ("MLA Matrix Absorption" sec. 2.2, the
decompression that the non-absorbed path of sec. 6 performs).  The attention that
follows is the decode oracle's (oracle.decode, which handles any number of new
tokens per sequence with the causal rule), pinned to the non-absorbed definition
by the oracle's own tests.
"""
from __future__ import annotations

import numpy as np


def decompress_kv(c: np.ndarray, W_UK: np.ndarray, W_UV: np.ndarray):
    """c [n, d_c] latent rows (float64), W [H, d_h, d_c] -> (K [n, H, d_h], V [n, H, d_h])."""
    c = np.asarray(c, dtype=np.float64)
    K = np.einsum("hdm,nm->nhd", np.asarray(W_UK, dtype=np.float64), c)
    V = np.einsum("hdm,nm->nhd", np.asarray(W_UV, dtype=np.float64), c)
    return K, V


def sequence_latents(c_cache: np.ndarray, block_table: np.ndarray, seq_len: int) -> np.ndarray:
    """The latent rows of positions 0 .. seq_len-1 of one sequence, in order."""
    t = np.arange(int(seq_len))
    pages = np.asarray(block_table)[t // 64]
    return np.asarray(c_cache)[pages, t % 64]
