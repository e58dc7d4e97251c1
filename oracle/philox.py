"""Philox4x32-10 counter-based generator, pure Python integers.

Test infrastructure only: this module belongs to the CPU oracle and is never
imported by the product path.

Written from the published description of the Philox family (J. K. Salmon,
M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3", SC'11, section 3 "Philox"): a 4-word counter is passed through ten
rounds; each round multiplies words 0 and 2 by fixed 32-bit multipliers,
keeps the high and low halves of the 64-bit products, XORs the high halves
with the other two counter words and the two key words, and permutes the
words. Between rounds the 2-word key is advanced by two Weyl constants
(golden ratio and sqrt(3)-1, scaled to 32 bits).

The sampling convention built on top of it (which counter and key a verify
row uses, and how a word becomes a uniform) is the library's own choice; the
pages only say that the random target path draws one sample for every verify
row and that per-request seeds are not supported (xLLM docs, "Adaptive
speculative inference", section "Launch example" of the DSpark part).
"""

MASK32 = 0xFFFFFFFF
# Round multipliers and key schedule increments of Philox4x32 (SC'11 paper,
# table of Philox parameters).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10


def _round(ctr, key):
    p0 = PHILOX_M0 * ctr[0]          # exact 64-bit product (Python int)
    p1 = PHILOX_M1 * ctr[2]
    hi0, lo0 = p0 >> 32, p0 & MASK32
    hi1, lo1 = p1 >> 32, p1 & MASK32
    return (
        (hi1 ^ ctr[1] ^ key[0]) & MASK32,
        lo1,
        (hi0 ^ ctr[3] ^ key[1]) & MASK32,
        lo0,
    )


def philox4x32_10(counter, key):
    """Return the 4 output words for a 4-word counter and a 2-word key."""
    ctr = tuple(int(c) & MASK32 for c in counter)
    k = [int(key[0]) & MASK32, int(key[1]) & MASK32]
    for r in range(ROUNDS):
        if r:
            k[0] = (k[0] + PHILOX_W0) & MASK32
            k[1] = (k[1] + PHILOX_W1) & MASK32
        ctr = _round(ctr, k)
    return ctr


def row_uniform(seed, request, row, offset):
    """Uniform in [0, 1) for local verify row `row` of request `request`.

    Counter = (row, request, offset low word, offset high word); key = (seed
    low word, seed high word). The top 24 bits of output word 0 give
    u = (w0 >> 8) * 2**-24, a value exactly representable in float32 and
    float64. Keying on (request, local row) and not on the packed row index
    makes the draw independent of how requests are packed or sharded.
    """
    seed = int(seed)
    offset = int(offset)
    w = philox4x32_10(
        (int(row), int(request), offset & MASK32, (offset >> 32) & MASK32),
        (seed & MASK32, (seed >> 32) & MASK32),
    )
    return (w[0] >> 8) * (1.0 / 16777216.0)
