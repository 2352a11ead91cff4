"""Byte and FLOP accounting of one absorbed-MLA decode step.

The per-token figures follow "DeepSeek-MLA-Principle", section 3 ("does
down/up-projection save memory/compute"): the cache holds d_c + d_h^R values
per token, the history-dependent work is 2*L*n_h*d_c + L*n_h*d_h^R
multiplications, and a step reads L*(d_c + d_h^R)*bytes of cache.  Everything
here is plain counting; no attention arithmetic.
"""
from __future__ import annotations

import dataclasses

FORMAT_BYTES = {"f32": 4, "bf16": 2, "fp16": 2}


def cache_values_per_token(d_c: int, d_r: int) -> int:
    """Values cached per token: the latent plus the shared RoPE key."""
    return d_c + d_r


def mha_values_per_token(n_h: int, d_h: int) -> int:
    """Values a standard MHA cache holds per token (K and V of every head)."""
    return 2 * n_h * d_h


def cache_bytes_per_token(d_c: int, d_r: int, fmt: str) -> int:
    """Bytes read per cached token.  'fp8': e4m3 latent + one fp32 scale + bf16 RoPE key."""
    if fmt == "fp8":
        return d_c + 4 + 2 * d_r
    return FORMAT_BYTES[fmt] * (d_c + d_r)


def history_multiplications(L: int, n_h: int, d_c: int, d_r: int) -> int:
    """Multiplications that grow with the history length in one absorbed decode step
    (content logits + latent weighted sum + RoPE logits)."""
    return 2 * L * n_h * d_c + L * n_h * d_r


def mha_history_multiplications(L: int, n_h: int, d_h: int) -> int:
    return 2 * L * n_h * d_h


def visible_positions(seq_lens, Sq: int) -> int:
    """Sum over sequences and query rows of the positions each row attends to."""
    tot = 0
    for n in seq_lens:
        n = int(n)
        for s in range(Sq):
            tot += max(0, n - Sq + 1 + s)
    return tot


@dataclasses.dataclass
class StepCost:
    cache_bytes: int      # latent cache + RoPE keys (+ fp8 scales) of every token read
    weight_bytes: int     # W_UK + W_UV
    query_bytes: int      # q_nope + q_rope
    out_bytes: int        # final per-head output
    flops: int            # 2 * multiply-adds of the four steps
    decode_bytes: int     # algorithmic bytes of the split-KV attention kernel alone
    decode_flops: int

    @property
    def total_bytes(self) -> int:
        return self.cache_bytes + self.weight_bytes + self.query_bytes + self.out_bytes


def step_cost(B: int, Sq: int, H: int, d_h: int, d_c: int, d_r: int, seq_lens,
              fmt: str = "bf16", out_fmt: str = "f32") -> StepCost:
    """Algorithmic bytes/FLOP of absorb + attend + merge + up-projection.

    Intermediates (absorbed query, split partials, merged latent) are excluded:
    a fully fused design never writes them."""
    elem = 4 if fmt == "f32" else 2
    tokens = sum(int(n) for n in seq_lens)
    cache = tokens * cache_bytes_per_token(d_c, d_r, fmt)
    weights = 2 * H * d_h * d_c * elem
    rows = B * Sq * H
    query = rows * (d_h + d_r) * elem
    out = rows * d_h * FORMAT_BYTES[out_fmt]
    vis = visible_positions(seq_lens, Sq)
    attend_flops = 2 * H * (d_c + d_r + d_c) * vis
    proj_flops = 2 * 2 * rows * d_h * d_c
    lat_elem = 4 if fmt == "f32" else 2
    decode_bytes = cache + rows * (d_c + d_r) * lat_elem
    return StepCost(cache, weights, query, out, attend_flops + proj_flops,
                    decode_bytes, attend_flops)


def append_bytes(tokens: int, H: int, d_c: int, d_r: int, in_fmt: str = "bf16", kv_fmt: str = "bf16",
                 pe_fmt: str = "bf16", with_query: bool = False) -> int:
    """Algorithmic bytes of appending `tokens` new tokens: the latent rows and RoPE
    keys read in the activation format and written in the cache formats (fp8:
    e4m3 codes plus one fp32 scale per token), and, with the query rotation, the
    query RoPE parts read and written."""
    a = FORMAT_BYTES[in_fmt]
    c_out = d_c + 4 if kv_fmt == "fp8" else d_c * FORMAT_BYTES[kv_fmt]
    per_tok = (d_c + d_r) * a + c_out + d_r * FORMAT_BYTES[pe_fmt]
    if with_query:
        per_tok += 2 * H * d_r * a
    return tokens * per_tok


def visible_pairs(seq_lens, Sq: int) -> int:
    """visible_positions in closed form: row s of a sequence of n tokens sees
    max(0, n - Sq + 1 + s) positions."""
    tot = 0
    for n in seq_lens:
        lo = max(0, int(n) - Sq + 1)          # positions seen by row 0 (or the first row that sees any)
        hi = int(n)                            # positions seen by the last row
        if hi <= 0:
            continue
        first = max(lo, 1)
        tot += (first + hi) * (hi - first + 1) // 2
    return tot


@dataclasses.dataclass
class PrefillCost:
    decompress_flops: int   # K and V of every cached position, every head
    attention_flops: int    # scores (d_h + d_r) and values (d_h) of every visible pair
    decompress_bytes: int   # latent rows read, K and V written (bf16)
    attention_bytes: int    # Q read, K, V, k_pe read once, output written


def prefill_cost(Sq: int, H: int, d_h: int, d_c: int, d_r: int, seq_lens, out_fmt: str = "bf16") -> PrefillCost:
    """Algorithmic FLOP/bytes of the non-absorbed path ("MLA Matrix Absorption"
    sec. 6): decompression 2 * 2*H*d_h*d_c per cached position, attention
    2*H*(2*d_h + d_r) per visible (query, position) pair (causal pairs only)."""
    tokens = sum(int(n) for n in seq_lens)
    rows = len(seq_lens) * Sq * H
    pairs = visible_pairs(seq_lens, Sq)
    dflops = 2 * 2 * H * d_h * d_c * tokens
    aflops = 2 * H * (2 * d_h + d_r) * pairs
    dbytes = tokens * (2 * d_c + 2 * 2 * H * d_h)
    abytes = rows * (d_h + d_r) * 2 + tokens * (2 * 2 * H * d_h + 2 * d_r) + rows * d_h * FORMAT_BYTES[out_fmt]
    return PrefillCost(dflops, aflops, dbytes, abytes)
