"""The LDS tile layout of the attention kernels (DirectTile in rsa_tiles.h).

A tile row of D bf16 is stored as D/8 16-byte chunks, chunk c of row r at
position c ^ swz(r). These host tests take swz from the header itself and
check, on a model of gfx950's LDS (64 banks of 4 bytes; a 16-byte read is
served 16 lanes per cycle, an 8-byte read 32 lanes per cycle), that

* swz permutes the chunks of every row (the copy and the reads agree),
* the fragment read (lane l: row 32x + l % 32, chunk 2k + l / 32) and the
  transposing ds_read_b64_tr_b16 read (16-lane groups over four rows and
  four consecutive 8-byte pieces per row, both row orders) touch 64
  different banks per cycle.

The model reproduces the SQ_LDS_BANK_CONFLICT count measured with the
earlier swizzle 2(r & 3) + ((r >> 2) & 1): 4 extra cycles per fragment read,
none per transposing read.
"""

import os
import re

import pytest

HEADER = os.path.join(os.path.dirname(__file__), "..", "sequence_transformer_attention_rsa_amd", "csrc",
                      "rsa_tiles.h")


def header_swizzles():
    src = open(HEADER).read()
    body = re.search(r"static constexpr int swz\(int r\) \{(.*?)\n    \}", src, re.S).group(1)
    exprs = re.findall(r"return (.*?);", body)
    assert len(exprs) == 2, body
    return {8: exprs[0], 16: exprs[1]}   # chunks per row -> expression


def as_function(expr):
    return lambda r: eval(expr, {}, {"r": r})


def cycles(addrs, width):
    """Cycles of one wave-wide read of `width` bytes per lane at byte addresses `addrs`."""
    per = {16: 16, 8: 32}[width]
    total = 0
    for g in range(0, 64, per):
        banks = {}
        for a in addrs[g:g + per]:
            for w in range(width // 4):
                word = a // 4 + w
                banks.setdefault(word % 64, set()).add(word)
        total += max(len(s) for s in banks.values())
    return total


def extra_cycles(swz, D):
    cpr, rb = D // 8, 2 * D
    frag = tr = 0
    for x in range(2):
        for c in range(0, cpr, 2):
            addrs = []
            for lane in range(64):
                r = 32 * x + (lane & 31)
                addrs.append(r * rb + 16 * ((c + (lane >> 5)) ^ swz(r)))
            frag = max(frag, cycles(addrs, 16) - 4)
    for row0 in range(0, 64, 16):
        for col0 in range(0, D, 32):
            for k in range(2):
                for seq in (False, True):
                    addrs = []
                    for lane in range(64):
                        i, ig, h = lane & 15, (lane >> 4) & 1, lane >> 5
                        e = col0 + 16 * ig + 4 * (i & 3)
                        r = row0 + (8 * h + 4 * k if seq else 8 * k + 4 * h) + (i >> 2)
                        addrs.append(r * rb + 16 * ((e >> 3) ^ swz(r)) + 8 * ((e >> 2) & 1))
                    tr = max(tr, cycles(addrs, 8) - 2)
    return frag, tr


@pytest.mark.parametrize("D", [64, 128])
def test_swizzle_permutes_chunks(D):
    swz = as_function(header_swizzles()[D // 8])
    for r in range(64):
        assert sorted(c ^ swz(r) for c in range(D // 8)) == list(range(D // 8)), r


@pytest.mark.parametrize("D", [64, 128])
def test_swizzle_is_bank_conflict_free(D):
    swz = as_function(header_swizzles()[D // 8])
    assert extra_cycles(swz, D) == (0, 0)


def test_model_reproduces_measured_conflicts_of_the_earlier_swizzle():
    old = lambda r: 2 * (r & 3) + ((r >> 2) & 1)   # noqa: E731
    assert extra_cycles(old, 64) == (4, 0)
