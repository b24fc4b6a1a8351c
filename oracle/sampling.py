"""CPU oracle for the step after the block: token-id hashing, the counter-based
random numbers and the seeded sampler.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the bench's
CPU-baseline leg use anything under ``oracle/``.  It shares no code, table or
helper with the HIP library.

Token hashes.  The "Receipts" page ("Making a receipt": the receipt's
``prompt`` and ``output.tokens`` fields, and the sentence under the field
table) records the prompt and output token ids with their BLAKE3, taken over
the ids as little-endian 32-bit integers.  ``blake3`` below follows the
published BLAKE3 definition (compression function, 1024-byte chunks of 64-byte
blocks, the binary tree whose left subtree holds the largest power of two
chunks that leaves at least one for the right, ROOT flag on the final
compression, 32-byte output); it is pinned by the two hashes the page prints.

Random numbers.  A draw for sequence position p under seed s is the first
64-bit word of Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011) with key (s, 0) and counter
(p, 0, 0, 0), turned into u = (word >> 11) * 2^-53 in [0, 1).  It depends on
nothing but (s, p), so a row's draw does not depend on the batch.

Sampler.  The pages list the receipt's sampler settings (temperature, top-k,
top-p, min-p, repeat / presence / frequency penalties over the last n tokens,
seed) but not the algorithm; this is the plain reading, in this order:
 1. penalties, in float32, for each distinct token of the row's history
    (ids outside the vocabulary are ignored):
    repeat: l > 0 -> l / r, else l * r; then
    presence and frequency: l - (presence + count * frequency);
 2. temperature 0: the largest penalised logit, lowest id on ties (greedy);
 3. otherwise candidates = the top_k largest penalised logits, ordered by
    (logit descending, id ascending); in float64: w_i = exp((l_i - l_0) / T);
    min-p keeps w_i >= min_p (w_0 = 1 is the maximum); top-p keeps the
    shortest prefix whose running sum reaches top_p times the total; the token
    is the first candidate whose running sum of the kept weights exceeds
    u times their total.
Decisions that floating point takes (a top-p cut, the draw) are made in
float64 here and in the kernel; the tests accept the kernel's choice when u
lies within a relative 1e-12 of a boundary, where either neighbour is correct.

Parity status.  BLAKE3 of inputs up to one chunk (1024 bytes, 256 token ids)
is pinned by the page's two printed hashes (one and two 64-byte blocks); the
multi-chunk tree is parity unpinned: no published digest of a longer input is
at hand here.  Philox words are pinned by numpy's own Philox generator.  The
sampler is pinned by closed forms for each step and a chi-square test of its
output distribution (tests/test_oracle_sampling.py).
"""
from __future__ import annotations

import struct

import numpy as np

from .bi_oracle import bf16_decode

# ---------------------------------------------------------------------------
# BLAKE3 (hash mode, 32-byte output)
# ---------------------------------------------------------------------------
_IV = (0x6A09E667, 0xBB67AE85, 0x3C6EF372, 0xA54FF53A, 0x510E527F, 0x9B05688C, 0x1F83D9AB, 0x5BE0CD19)
_PERM = (2, 6, 3, 10, 7, 0, 4, 13, 1, 11, 12, 5, 9, 14, 15, 8)
_CHUNK_START, _CHUNK_END, _PARENT, _ROOT = 1, 2, 4, 8
_CHUNK_LEN, _BLOCK_LEN = 1024, 64
_M32 = 0xFFFFFFFF


def _rotr(x, n):
    return ((x >> n) | (x << (32 - n))) & _M32


def _g(v, a, b, c, d, mx, my):
    v[a] = (v[a] + v[b] + mx) & _M32
    v[d] = _rotr(v[d] ^ v[a], 16)
    v[c] = (v[c] + v[d]) & _M32
    v[b] = _rotr(v[b] ^ v[c], 12)
    v[a] = (v[a] + v[b] + my) & _M32
    v[d] = _rotr(v[d] ^ v[a], 8)
    v[c] = (v[c] + v[d]) & _M32
    v[b] = _rotr(v[b] ^ v[c], 7)


def _compress(cv, block_words, counter, block_len, flags):
    """The BLAKE3 compression function; returns the 16-word output state."""
    v = list(cv) + list(_IV[:4]) + [counter & _M32, (counter >> 32) & _M32, block_len, flags]
    m = list(block_words)
    for rnd in range(7):
        _g(v, 0, 4, 8, 12, m[0], m[1])
        _g(v, 1, 5, 9, 13, m[2], m[3])
        _g(v, 2, 6, 10, 14, m[4], m[5])
        _g(v, 3, 7, 11, 15, m[6], m[7])
        _g(v, 0, 5, 10, 15, m[8], m[9])
        _g(v, 1, 6, 11, 12, m[10], m[11])
        _g(v, 2, 7, 8, 13, m[12], m[13])
        _g(v, 3, 4, 9, 14, m[14], m[15])
        if rnd < 6:
            m = [m[_PERM[i]] for i in range(16)]
    return [v[i] ^ v[i + 8] for i in range(8)] + [v[i + 8] ^ cv[i] for i in range(8)]


def _words(block: bytes):
    block = block + bytes(_BLOCK_LEN - len(block))
    return struct.unpack("<16I", block)


def _chunk(data: bytes, index: int, root: bool):
    """Chaining value (first 8 words) of one chunk; ROOT on its last block when asked."""
    blocks = [data[i:i + _BLOCK_LEN] for i in range(0, len(data), _BLOCK_LEN)] or [b""]
    cv = list(_IV)
    for j, blk in enumerate(blocks):
        flags = (_CHUNK_START if j == 0 else 0) | (_CHUNK_END if j == len(blocks) - 1 else 0)
        if root and j == len(blocks) - 1:
            flags |= _ROOT
        cv = _compress(cv, _words(blk), index, len(blk), flags)[:8]
    return cv


def _subtree(data: bytes, first_chunk: int, root: bool):
    """Chaining value of the subtree over ``data`` starting at chunk ``first_chunk``."""
    n = max(1, -(-len(data) // _CHUNK_LEN))
    if n == 1:
        return _chunk(data, first_chunk, root)
    left = 1 << ((n - 1).bit_length() - 1)     # largest power of two < n
    lcv = _subtree(data[:left * _CHUNK_LEN], first_chunk, False)
    rcv = _subtree(data[left * _CHUNK_LEN:], first_chunk + left, False)
    return _compress(list(_IV), lcv + rcv, 0, _BLOCK_LEN, _PARENT | (_ROOT if root else 0))[:8]


def blake3(data: bytes) -> bytes:
    """BLAKE3 hash (32 bytes) of ``data``."""
    return struct.pack("<8I", *_subtree(bytes(data), 0, True))


def token_hash(ids) -> bytes:
    """BLAKE3 over token ids as little-endian 32-bit integers."""
    return blake3(np.asarray(ids, dtype="<u4").tobytes())


# ---------------------------------------------------------------------------
# Philox4x64-10
# ---------------------------------------------------------------------------
_M64 = (1 << 64) - 1
_PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
_PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def philox4x64_10(counter, key):
    """Philox4x64 with 10 rounds: 4 x uint64 counter, 2 x uint64 key -> 4 x uint64."""
    c = [int(x) & _M64 for x in counter]
    k = [int(x) & _M64 for x in key]
    for rnd in range(10):
        p0 = _PHILOX_M[0] * c[0]
        p1 = _PHILOX_M[1] * c[2]
        c = [((p1 >> 64) ^ c[1] ^ k[0]) & _M64, p1 & _M64, ((p0 >> 64) ^ c[3] ^ k[1]) & _M64, p0 & _M64]
        if rnd < 9:
            k = [(k[0] + _PHILOX_W[0]) & _M64, (k[1] + _PHILOX_W[1]) & _M64]
    return c


def uniform(seed: int, position: int) -> float:
    """The draw in [0, 1) for (seed, position): first Philox word, top 53 bits."""
    w = philox4x64_10((position, 0, 0, 0), (seed, 0))[0]
    return (w >> 11) * 2.0 ** -53


# ---------------------------------------------------------------------------
# sampler
# ---------------------------------------------------------------------------
def penalised_logits(logit_bits, history, repeat=1.0, presence=0.0, frequency=0.0) -> np.ndarray:
    """Float32 logits of one row after the history penalties (step 1 of the header)."""
    l = bf16_decode(logit_bits).astype(np.float32)
    hist = [int(t) for t in history if 0 <= int(t) < l.size]   # other ids are ignored
    r, pr, fr = np.float32(repeat), np.float32(presence), np.float32(frequency)
    for tok in sorted(set(hist)):
        v = l[tok]
        v = v / r if v > 0 else v * r
        cnt = np.float32(hist.count(tok))
        v = v - (pr + cnt * fr)
        l[tok] = np.float32(v)
    return l


def sample_row(logit_bits, seed, position, temperature, top_k, top_p, min_p,
               history=(), repeat=1.0, presence=0.0, frequency=0.0):
    """One row's token id.  Returns (id, detail) where detail holds the kept
    candidates, their running sums and u (None for greedy)."""
    l = penalised_logits(logit_bits, history, repeat, presence, frequency)
    if temperature == 0.0:
        m = l.max()
        return int(np.flatnonzero(l == m)[0]), None
    order = np.lexsort((np.arange(l.size), -l.astype(np.float64)))[:top_k]
    z = l[order].astype(np.float64)
    w = np.exp((z - z[0]) / np.float64(np.float32(temperature)))
    keep = w >= np.float64(np.float32(min_p))
    ids, w = order[keep], w[keep]
    csum = np.cumsum(w)          # sequential in candidate order
    cut = int(np.searchsorted(csum, np.float64(np.float32(top_p)) * csum[-1], side="left")) + 1
    ids, w = ids[:cut], w[:cut]
    csum = np.cumsum(w)
    u = uniform(seed, position)
    target = u * csum[-1]
    pick = int(np.searchsorted(csum, target, side="right"))
    pick = min(pick, len(ids) - 1)
    return int(ids[pick]), dict(ids=ids, csum=csum, u=u, target=target)
