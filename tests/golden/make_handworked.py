"""Writes q2K, q3K, q4K, q5K and q6K_handworked.txt.

The pages print no worked decode, so these fixtures are worked by hand from the
ggml K-quant layout (the reading the oracle follows).  Everything below is the
hand derivation written down: the raw bytes are chosen, the scale/min fields are
decoded by hand in the comments, and the expected weights are evaluated from that
hand-decoded table.  No decoder (neither the oracle nor the HIP library) is
called.  Run from the repository root:  python tests/golden/make_handworked.py
"""
import os

HERE = os.path.dirname(os.path.abspath(__file__))

# ---------------------------------------------------------------- q4_K
# d = 0.5  (binary16 0x3800, bytes 00 38); dmin = 0.25 (0x3400, bytes 00 34)
# 12 scale bytes and their hand decode:
#   s0 = 0xC1 = 11|000001 : sc0 = 1,  top bits 11 -> sc4 gets 3<<4 = 48
#   s1 = 0x42 = 01|000010 : sc1 = 2,  top bits 01 -> sc5 gets 16
#   s2 = 0x03 = 00|000011 : sc2 = 3,  top bits 00 -> sc6 gets 0
#   s3 = 0xBF = 10|111111 : sc3 = 63, top bits 10 -> sc7 gets 32
#   s4 = 0x05 = 00|000101 : m0 = 5,   top bits 00 -> m4 gets 0
#   s5 = 0x86 = 10|000110 : m1 = 6,   top bits 10 -> m5 gets 32
#   s6 = 0x47 = 01|000111 : m2 = 7,   top bits 01 -> m6 gets 16
#   s7 = 0xC0 = 11|000000 : m3 = 0,   top bits 11 -> m7 gets 48
#   s8 = 0x21 : low nibble 1 -> sc4 = 48+1 = 49 ; high nibble 2 -> m4 = 0+2 = 2
#   s9 = 0x9F : low nibble 15 -> sc5 = 16+15 = 31 ; high nibble 9 -> m5 = 32+9 = 41
#   s10 = 0x00: sc6 = 0 ; m6 = 16
#   s11 = 0xF4: low nibble 4 -> sc7 = 32+4 = 36 ; high nibble 15 -> m7 = 48+15 = 63
Q4_SCALE_BYTES = [0xC1, 0x42, 0x03, 0xBF, 0x05, 0x86, 0x47, 0xC0, 0x21, 0x9F, 0x00, 0xF4]
Q4_SC = [1, 2, 3, 63, 49, 31, 0, 36]
Q4_M = [5, 6, 7, 0, 2, 41, 16, 63]
# quant bytes: in each 32-byte group, byte l holds low nibble l%16 and high nibble
# 15 - l%16.  So sub-block 2g has q = l%16 and sub-block 2g+1 has q = 15 - l%16.
Q4_QS = [(l % 16) | ((15 - l % 16) << 4) for g in range(4) for l in range(32)]


def q4_weights():
    out = []
    for j in range(8):
        for l in range(32):
            q = l % 16 if j % 2 == 0 else 15 - l % 16
            out.append(0.5 * Q4_SC[j] * q - 0.25 * Q4_M[j])
    return out


# ---------------------------------------------------------------- q6_K
# ql byte t = t (so its low nibble is t%16 and its high nibble t//16); every qh
# byte is 0xE4 = 11 10 01 00, so quarter c always gets top bits c.
# Weight i = 128h + 32c + l therefore has q = 16c + (l%16 for c<2, else
# 4h + 2*(c-2) + l//16) and decodes as 0.5 * sc[i//16] * (q - 32).
Q6_SC = [1, -1, 2, -2, 3, -3, 4, -4, 127, -128, 5, -5, 64, -64, 7, 0]


def q6_weights():
    out = []
    for h in range(2):
        for c in range(4):
            for l in range(32):
                low = l % 16 if c < 2 else 4 * h + 2 * (c - 2) + l // 16
                q = 16 * c + low
                out.append(0.5 * Q6_SC[(128 * h + 32 * c + l) // 16] * (q - 32))
    return out


# ---------------------------------------------------------------- q2_K
# d = 0.5 (bytes 00 38), dmin = 0.25 (bytes 00 34), stored after the quants.
# Sub-block byte j holds scale j in its low nibble and min j in its high nibble:
#   0x30 -> sc 0, m 3    0x81 -> sc 1, m 8    0xD2 -> sc 2, m 13   0x23 -> sc 3, m 2
#   0x74 -> sc 4, m 7    0xC5 -> sc 5, m 12   0x16 -> sc 6, m 1    0x67 -> sc 7, m 6
#   0xB8 -> sc 8, m 11   0x09 -> sc 9, m 0    0x5A -> sc 10, m 5   0xAB -> sc 11, m 10
#   0xFC -> sc 12, m 15  0x4D -> sc 13, m 4   0x9E -> sc 14, m 9   0xEF -> sc 15, m 14
Q2_SCALE_BYTES = [0x30, 0x81, 0xD2, 0x23, 0x74, 0xC5, 0x16, 0x67,
                  0xB8, 0x09, 0x5A, 0xAB, 0xFC, 0x4D, 0x9E, 0xEF]
Q2_SC = list(range(16))
Q2_M = [3, 8, 13, 2, 7, 12, 1, 6, 11, 0, 5, 10, 15, 4, 9, 14]
# Quant byte 32h + l repeats E4 39 4E 93 by l % 4.  Bit pairs, low to high:
#   0xE4 = 11 10 01 00 -> quarters 0..3 get 0, 1, 2, 3
#   0x39 = 00 11 10 01 -> 1, 2, 3, 0
#   0x4E = 01 00 11 10 -> 2, 3, 0, 1
#   0x93 = 10 01 00 11 -> 3, 0, 1, 2
# so weight 128h + 32c + l has q = (l % 4 + c) % 4.
Q2_QS = [[0xE4, 0x39, 0x4E, 0x93][l % 4] for h in range(2) for l in range(32)]


def q2_weights():
    out = []
    for h in range(2):
        for c in range(4):
            for l in range(32):
                j = (128 * h + 32 * c + l) // 16
                out.append(0.5 * Q2_SC[j] * ((l % 4 + c) % 4) - 0.25 * Q2_M[j])
    return out


# ---------------------------------------------------------------- q3_K
# Mask byte l is l itself, so weight 128h + 32c + l has its third bit set when
# bit 4h + c of l is set (never for h = 1, c >= 1, since l < 32).
# Low parts: the same bytes as the q2_K quants above, low = (l % 4 + c) % 4;
# q = low where the bit is set, low - 4 where it is clear.
# Scales (stored values u, sc = u - 32), chosen:
#   u = 0 63 32 31 1 62 17 48 5 40 33 20 60 3 44 27
#   low nibbles: 0 F 0 F 1 E 1 0 5 8 1 4 C 3 C B; top two bits: 0 3 2 1 0 3 1 3 0 2 2 1 3 0 2 1
#   bytes 0..3 = low nibbles of u0..u3 | low nibbles of u8..u11 << 4: 50 8F 10 4F
#   bytes 4..7 = low nibbles of u4..u7 | low nibbles of u12..u15 << 4: C1 3E C1 B0
#   byte 8 + k = top(u_k) | top(u_4+k) << 2 | top(u_8+k) << 4 | top(u_12+k) << 6:
#     k = 0: 0 | 0 | 0 | 3<<6 = C0     k = 1: 3 | 3<<2 | 2<<4 | 0 = 2F
#     k = 2: 2 | 1<<2 | 2<<4 | 2<<6 = A6   k = 3: 1 | 3<<2 | 1<<4 | 1<<6 = 5D
# d = 0.5 (bytes 00 38) at the end.
Q3_SCALE_BYTES = [0x50, 0x8F, 0x10, 0x4F, 0xC1, 0x3E, 0xC1, 0xB0, 0xC0, 0x2F, 0xA6, 0x5D]
Q3_SC = [u - 32 for u in [0, 63, 32, 31, 1, 62, 17, 48, 5, 40, 33, 20, 60, 3, 44, 27]]


def q3_weights():
    out = []
    for h in range(2):
        for c in range(4):
            for l in range(32):
                low = (l % 4 + c) % 4
                q = low if (l >> (4 * h + c)) & 1 else low - 4
                out.append(0.5 * Q3_SC[(128 * h + 32 * c + l) // 16] * q)
    return out


# ---------------------------------------------------------------- q5_K
# d = 0.5, dmin = 0.25 and the 12 scale bytes of the q4_K block above (same
# packing, same hand decode Q4_SC / Q4_M).  High-bit byte l is l itself, so
# weight 64g + 32t + l gets +16 when bit 2g + t of l is set.  Low nibbles: the
# q4_K block's quant bytes, low = l % 16 (t = 0) or 15 - l % 16 (t = 1).


def q5_weights():
    out = []
    for g in range(4):
        for t in range(2):
            for l in range(32):
                low = l % 16 if t == 0 else 15 - l % 16
                q = low + (16 if (l >> (2 * g + t)) & 1 else 0)
                out.append(0.5 * Q4_SC[2 * g + t] * q - 0.25 * Q4_M[2 * g + t])
    return out


def write(name, raw, weights, header):
    with open(os.path.join(HERE, name), "w") as f:
        f.write(header)
        f.write("bytes: " + " ".join("%02x" % b for b in raw) + "\n")
        f.write("weights: " + " ".join(repr(float(w)) for w in weights) + "\n")


def main():
    q4 = [0x00, 0x38, 0x00, 0x34] + Q4_SCALE_BYTES + Q4_QS
    assert len(q4) == 144
    write("q4K_handworked.txt", q4, q4_weights(),
          "# One q4_K block decoded by hand (see make_handworked.py for the derivation).\n"
          "# d = 0.5, dmin = 0.25, sc = %s, m = %s\n" % (Q4_SC, Q4_M))
    q6 = list(range(128)) + [0xE4] * 64 + [s & 0xFF for s in Q6_SC] + [0x00, 0x38]
    assert len(q6) == 210
    write("q6K_handworked.txt", q6, q6_weights(),
          "# One q6_K block decoded by hand (see make_handworked.py for the derivation).\n"
          "# d = 0.5, sc = %s\n" % (Q6_SC,))
    q2 = Q2_SCALE_BYTES + Q2_QS + [0x00, 0x38, 0x00, 0x34]
    assert len(q2) == 84
    write("q2K_handworked.txt", q2, q2_weights(),
          "# One q2_K block decoded by hand (see make_handworked.py for the derivation).\n"
          "# d = 0.5, dmin = 0.25, sc = %s, m = %s\n" % (Q2_SC, Q2_M))
    q3 = list(range(32)) + Q2_QS + Q3_SCALE_BYTES + [0x00, 0x38]
    assert len(q3) == 110
    write("q3K_handworked.txt", q3, q3_weights(),
          "# One q3_K block decoded by hand (see make_handworked.py for the derivation).\n"
          "# d = 0.5, sc = %s\n" % (Q3_SC,))
    q5 = [0x00, 0x38, 0x00, 0x34] + Q4_SCALE_BYTES + list(range(32)) + Q4_QS
    assert len(q5) == 176
    write("q5K_handworked.txt", q5, q5_weights(),
          "# One q5_K block decoded by hand (see make_handworked.py for the derivation).\n"
          "# d = 0.5, dmin = 0.25, sc = %s, m = %s\n" % (Q4_SC, Q4_M))


if __name__ == "__main__":
    main()
