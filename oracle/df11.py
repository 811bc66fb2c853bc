"""DFloat11-style lossless coding of bf16 weights (oracle).  Test infrastructure only.

[DF11] "DFloat11: Nén suy luận GPU không mất dữ liệu, giảm LLM xuống còn 70%
kích thước" (vi.news.hada.io):

* "Dư địa nén còn lại trong exponent của BFloat16": a bf16 word is 1 sign, 8
  exponent and 7 mantissa bits; in LLM weights only the exponent has low
  entropy (about 2.6 of its 8 bits), sign and mantissa are close to full.
* "Định dạng DFloat11": a Huffman code is built from the exponent
  distribution; the exponents are bit-packed into the byte array
  EncodedExponent, sign and mantissa are kept verbatim in the byte array
  PackedSignMantissa; about 11 bits per weight on average.
* "Giải mã dựa trên LUT phân cấp": the code tree is cut into disjoint
  subtrees of height 8, each a 256-entry table; table entries 240..255
  (exponents that do not occur in weights) point to the next table; a
  CodeLengths table gives each exponent's code length.
* "Kernel GPU hai giai đoạn và metadata bổ trợ": each thread owns 8
  consecutive bytes of EncodedExponent and decodes the codes that START in
  them; Gaps holds, per thread, the 5-bit offset of its first code; only the
  output position of each thread block's first element is stored.

Readings taken where the page leaves a step open (each listed in the design
notes):

D1  One code per matrix, from that matrix's exponent histogram.
D2  Huffman: repeatedly merge the two nodes of least (weight, order), where
    leaves are ordered by exponent value and internal nodes come after all
    leaves in creation order; code length = depth.  One used exponent gets a
    1-bit code; no used exponent gives an empty stream.
D3  Code lengths are limited to 32 bits (the page bounds the gap by 31 and
    the code length by 32).  When the Huffman code is deeper, the optimal
    length-limited code is taken instead (package-merge, Larmore and
    Hirschberg 1990), with the merge order fixed below.
D4  Canonical codewords: exponents ordered by (length, exponent) receive
    consecutive code values (the usual canonical Huffman assignment).
D5  The stream is MSB-first: the first code bit is bit 7 of byte 0.
D6  PackedSignMantissa byte = sign << 7 | mantissa.
D7  Segments of 64 bits, n_seg = ceil(total_bits / 64); the gap of segment t
    is (first code start >= 64 t, or total_bits if there is none) - 64 t.
D8  Gaps are packed 5 bits per segment, LSB-first (gap t in stream bits
    5t..5t+4, bit k being bit k % 8 of byte k // 8).
D9  A decoding block is 256 threads (16384 stream bits); block_pos[b] is the
    number of codes that start before bit 16384 b, for b = 0..n_blocks, so
    block_pos[n_blocks] = n.
D10 Sub-tables are numbered 1, 2, ... in the order in which codes, walked in
    canonical order, first need them; table k is referenced by the entry
    value 256 - k, so at most 16 sub-tables.  Exponents >= 240 cannot be
    represented (their values are pointers) and are rejected, as is a code
    needing more than 16 sub-tables.  Unused table entries are 0.
D11 Buffer sizes: EncodedExponent 8 n_seg + 8 bytes (zero padding for the
    last thread's window), Gaps 4 ceil(5 n_seg / 32) + 4 bytes.

Everything here is integer arithmetic; results compare bit for bit.
"""
from __future__ import annotations

import heapq

import numpy as np

MAX_LEN = 32          # D3
SEG_BITS = 64         # 8 bytes per thread
BLOCK_THREADS = 256   # D9
PTR_MIN = 240         # D10
MAX_SUBTABLES = 16


class DF11Error(ValueError):
    """The exponent set cannot be coded in this format (D10)."""


# --------------------------------------------------------------------- fields
def split_fields(bits):
    """bf16 bit patterns (uint16) -> (exponent uint8, sign|mantissa uint8) (D6)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    exp = ((b >> 7) & 0xFF).astype(np.uint8)
    sm = (((b >> 8) & 0x80) | (b & 0x7F)).astype(np.uint8)
    return exp, sm


def join_fields(exp, sm):
    e = np.asarray(exp, dtype=np.uint32)
    s = np.asarray(sm, dtype=np.uint32)
    return (((s & 0x80) << 8) | (e << 7) | (s & 0x7F)).astype(np.uint16)


def exponent_histogram(bits) -> np.ndarray:
    """Counts of the 256 exponent values ("Dư địa nén..." histogram)."""
    exp, _ = split_fields(np.asarray(bits).reshape(-1))
    return np.bincount(exp, minlength=256).astype(np.int64)


# ------------------------------------------------------------ code lengths
def huffman_lengths(hist) -> np.ndarray:
    """Huffman code lengths (D2), unlimited depth."""
    h = np.asarray(hist, dtype=np.int64)
    used = [s for s in range(len(h)) if h[s] > 0]
    lens = np.zeros(len(h), dtype=np.int64)
    if len(used) == 1:
        lens[used[0]] = 1
    if len(used) <= 1:
        return lens
    heap = [(int(h[s]), s, ("leaf", s)) for s in used]
    heapq.heapify(heap)
    order = len(h)
    while len(heap) > 1:
        w0, _, a = heapq.heappop(heap)
        w1, _, b = heapq.heappop(heap)
        heapq.heappush(heap, (w0 + w1, order, ("node", a, b)))
        order += 1
    stack = [(heap[0][2], 0)]
    while stack:
        node, d = stack.pop()
        if node[0] == "leaf":
            lens[node[1]] = d
        else:
            stack.append((node[1], d + 1))
            stack.append((node[2], d + 1))
    return lens


def package_merge_lengths(hist, max_len: int) -> np.ndarray:
    """Optimal code lengths bounded by ``max_len`` (package-merge).

    Leaves sorted by (weight, exponent).  At each of the max_len levels,
    starting from the deepest, the list is the leaves merged with the
    packages (pairs of consecutive items, an odd last item dropped) of the
    previous level's list, by weight, a leaf before a package of equal
    weight and otherwise keeping each list's order.  The first 2(n - 1)
    items of the final list are selected; a symbol's length is the number of
    selected items that contain it (counted with the packages' contents).
    """
    h = np.asarray(hist, dtype=np.int64)
    used = sorted((int(h[s]), s) for s in range(len(h)) if h[s] > 0)
    n = len(used)
    lens = np.zeros(len(h), dtype=np.int64)
    if n <= 1:
        if n == 1:
            lens[used[0][1]] = 1
        return lens
    if (1 << max_len) < n:
        raise DF11Error("max_len too small for the alphabet")
    leaves = [(w, np.eye(1, n, i, dtype=np.int64)[0]) for i, (w, _) in enumerate(used)]
    prev = []
    for _ in range(max_len):
        pk = [(prev[2 * i][0] + prev[2 * i + 1][0], prev[2 * i][1] + prev[2 * i + 1][1])
              for i in range(len(prev) // 2)]
        cur, i, j = [], 0, 0
        while i < len(leaves) or j < len(pk):
            if j >= len(pk) or (i < len(leaves) and leaves[i][0] <= pk[j][0]):
                cur.append(leaves[i]); i += 1
            else:
                cur.append(pk[j]); j += 1
        prev = cur
    cnt = np.sum([c for _, c in prev[:2 * (n - 1)]], axis=0)
    for i, (_, s) in enumerate(used):
        lens[s] = cnt[i]
    return lens


def code_lengths(hist) -> np.ndarray:
    """D2 + D3: Huffman, or package-merge at 32 bits when Huffman is deeper."""
    lens = huffman_lengths(hist)
    if lens.max(initial=0) > MAX_LEN:
        lens = package_merge_lengths(hist, MAX_LEN)
    return lens


def canonical_codes(lens) -> np.ndarray:
    """D4: codewords (right-aligned ints) from lengths."""
    lens = np.asarray(lens, dtype=np.int64)
    codes = np.zeros(len(lens), dtype=np.int64)
    syms = sorted((int(lens[s]), s) for s in range(len(lens)) if lens[s] > 0)
    code, prev = 0, None
    for L, s in syms:
        if prev is not None:
            code = (code + 1) << (L - prev)
        codes[s] = code
        prev = L
    return codes


# ------------------------------------------------------------------ tables
def build_tables(lens, codes):
    """Hierarchical 256-entry tables (D10).  Returns a uint8 array [k, 256]."""
    lens = np.asarray(lens, dtype=np.int64)
    if np.any(lens[PTR_MIN:] > 0):
        raise DF11Error("exponent >= 240 present")
    tables = [np.zeros(256, dtype=np.int64)]
    ptr = [np.zeros(256, dtype=bool)]
    for L, s in sorted((int(lens[s]), s) for s in range(len(lens)) if lens[s] > 0):
        c = int(codes[s])
        t, rem = 0, L
        while rem > 8:
            idx = (c >> (rem - 8)) & 0xFF
            if not ptr[t][idx]:
                k = len(tables)
                if k > MAX_SUBTABLES:
                    raise DF11Error("more than 16 sub-tables")
                tables.append(np.zeros(256, dtype=np.int64))
                ptr.append(np.zeros(256, dtype=bool))
                tables[t][idx] = 256 - k
                ptr[t][idx] = True
            t = 256 - int(tables[t][idx])
            rem -= 8
        low = c & ((1 << rem) - 1)
        lo, hi = low << (8 - rem), (low + 1) << (8 - rem)
        assert not ptr[t][lo:hi].any()
        tables[t][lo:hi] = s
    return np.array(tables, dtype=np.uint8)


def build_code(hist):
    """Everything the host derives from a histogram: (lens uint8[256],
    codes uint32[256], tables uint8[k,256], total_bits)."""
    h = np.asarray(hist, dtype=np.int64)
    lens = code_lengths(h)
    codes = canonical_codes(lens)
    tables = build_tables(lens, codes)
    total = int(np.sum(h * lens))
    return lens.astype(np.uint8), codes.astype(np.uint32), tables, total


# ------------------------------------------------------------------ layout
def sizes(total_bits: int):
    """(n_seg, enc_bytes, gap_bytes, n_blocks) (D7, D9, D11)."""
    n_seg = -(-total_bits // SEG_BITS)
    n_blocks = -(-n_seg // BLOCK_THREADS)
    return n_seg, 8 * n_seg + 8, 4 * (-(-5 * n_seg // 32)) + 4, n_blocks


def encode(bits, lens, codes):
    """bf16 bits -> dict(enc, sm, gaps, block_pos, total_bits) (D5-D9)."""
    exp, sm = split_fields(np.asarray(bits).reshape(-1))
    n = exp.size
    L = np.asarray(lens, dtype=np.int64)[exp]
    C = np.asarray(codes, dtype=np.int64)[exp]
    if n and np.any(L == 0):
        raise DF11Error("exponent without a code")
    starts = np.cumsum(L) - L
    total = int(L.sum())
    n_seg, enc_bytes, gap_bytes, n_blocks = sizes(total)
    stream = np.zeros(8 * enc_bytes, dtype=np.uint8)
    for j in range(MAX_LEN):
        m = L > j
        stream[starts[m] + j] = (C[m] >> (L[m] - 1 - j)) & 1
    enc = np.packbits(stream, bitorder="big")
    seg0 = np.arange(n_seg, dtype=np.int64) * SEG_BITS
    k = np.searchsorted(starts, seg0, side="left")
    first = np.where(k < n, starts[np.minimum(k, max(n - 1, 0))] if n else 0, total)
    gap = first - seg0
    assert np.all((gap >= 0) & (gap <= 31))
    gbits = np.zeros(8 * gap_bytes, dtype=np.uint8)
    for b in range(5):
        gbits[5 * np.arange(n_seg) + b] = (gap >> b) & 1
    gaps = np.packbits(gbits, bitorder="little")
    bounds = np.arange(n_blocks + 1, dtype=np.int64) * SEG_BITS * BLOCK_THREADS
    block_pos = np.searchsorted(starts, bounds, side="left").astype(np.uint32)
    block_pos[-1] = n
    return {"enc": enc, "sm": sm, "gaps": gaps, "block_pos": block_pos, "total_bits": total,
            "n_seg": n_seg, "n_blocks": n_blocks}


# ---------------------------------------------------------------- decoding
def decode_sequential(enc, total_bits: int, lens, codes, sm):
    """Plain prefix-code decoding, bit by bit, of the whole stream (no
    tables, no segments): the definition the table decoder must meet."""
    lookup = {(int(lens[s]), int(codes[s])): s for s in range(len(lens)) if lens[s] > 0}
    bits = np.unpackbits(np.asarray(enc, dtype=np.uint8), bitorder="big")
    out, c, L = [], 0, 0
    for p in range(total_bits):
        c = (c << 1) | int(bits[p])
        L += 1
        s = lookup.get((L, c))
        if s is not None:
            out.append(s)
            c, L = 0, 0
        elif L > MAX_LEN:
            raise DF11Error("invalid code")
    assert L == 0, "stream ends inside a code"
    return join_fields(np.array(out, dtype=np.uint32), sm[:len(out)])


def decode_tables(enc, gaps, block_pos, tables, lens, total_bits: int, sm):
    """The page's parallel decoding, walked serially: per thread segment,
    start at its gap, decode codes that start inside the segment with the
    hierarchical tables; per block, the threads' outputs concatenated
    follow block_pos."""
    enc = np.asarray(enc, dtype=np.uint8)
    gaps = np.asarray(gaps, dtype=np.uint8)
    bits = np.unpackbits(enc, bitorder="big")
    gb = np.unpackbits(gaps, bitorder="little")
    n_seg, _, _, n_blocks = sizes(total_bits)

    def window(p):
        w = 0
        for j in range(32):
            w = (w << 1) | (int(bits[p + j]) if p + j < len(bits) else 0)
        return w

    out = []
    for b in range(n_blocks):
        blk = []
        for t in range(b * BLOCK_THREADS, min(n_seg, (b + 1) * BLOCK_THREADS)):
            g = sum(int(gb[5 * t + k]) << k for k in range(5))
            p, end = t * SEG_BITS + g, min((t + 1) * SEG_BITS, total_bits)
            while p < end:
                w = window(p)
                tab, sh = 0, 24
                v = int(tables[tab][(w >> sh) & 0xFF])
                while v >= PTR_MIN:
                    tab, sh = 256 - v, sh - 8
                    v = int(tables[tab][(w >> sh) & 0xFF])
                blk.append(v)
                p += int(lens[v])
        assert len(blk) == int(block_pos[b + 1]) - int(block_pos[b]), "block_pos mismatch"
        out.extend(blk)
    return join_fields(np.array(out, dtype=np.uint32), np.asarray(sm)[:len(out)])
