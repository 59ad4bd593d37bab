"""Writes q4K_handworked.txt and q6K_handworked.txt.

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


if __name__ == "__main__":
    main()
