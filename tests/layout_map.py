"""Which outputs of a block each payload bit may change, per format.

Written from the DequantizePacked page's "Packed layouts and decoding" table
(field order and sizes) and the element-order definitions of its
"Mathematical decoding rules" (the P(a,w,g) enumeration, the IQ lane
structure i = 4g + l, the TQ1_0 sequences), and from section 3.3 of the
NInfer tensor-formats page for "nvfp4".  It shares nothing with the oracle's
code; the structural test flips every bit of random blocks and checks the
oracle's changed outputs against these predictions.

Each bit maps to (kind, outputs):
  "exact"  - every trial changes a subset of `outputs`; over all trials the
             changes cover `outputs` exactly (code and sign bits);
  "some"   - subset per trial, and some trial changes something
             (codebook index bits: rows are distinct, so a new row differs);
  "within" - subset per trial (scale bits, ternary bytes).
"""


def _plane(w, g):
    """Element index of (byte t, bit b) of a region enumerated by P(a,w,g)."""
    def f(t, b):
        return (t // g) * g * (8 // w) + (b // w) * g + (t % g)
    return f


class Map:
    def __init__(self, B, S):
        self.B, self.S = B, S
        self.m = {}

    def put(self, byte, bit, kind, outs):
        key = byte * 8 + bit
        assert key not in self.m, (byte, bit)
        self.m[key] = (kind, frozenset(outs))

    def scale(self, start, n, outs):
        for t in range(start, start + n):
            for b in range(8):
                self.put(t, b, "within", outs)

    def ignored(self, start, n):
        for t in range(start, start + n):
            for b in range(8):
                self.put(t, b, "exact", ())

    def plane(self, start, n, w, g, base=0):
        f = _plane(w, g)
        for t in range(n):
            for b in range(8):
                self.put(start + t, b, "exact", (base + f(t, b),))

    def done(self):
        assert len(self.m) == 8 * self.S, (len(self.m), self.S)
        return self


def _all(B):
    return range(B)


def build(fmt):
    k = fmt.split(":")[-1]
    if fmt == "nvfp4":
        k = "nvfp4"
    if k in ("q4_0", "iq4_nl"):
        m = Map(32, 18); m.scale(0, 2, _all(32)); m.plane(2, 16, 4, 16)
    elif k == "q4_1":
        m = Map(32, 20); m.scale(0, 4, _all(32)); m.plane(4, 16, 4, 16)
    elif k in ("q5_0", "q5_1"):
        off = 2 if k == "q5_0" else 4
        m = Map(32, off + 20); m.scale(0, off, _all(32))
        for t in range(4):
            for b in range(8):
                m.put(off + t, b, "exact", (8 * t + b,))
        m.plane(off + 4, 16, 4, 16)
    elif k in ("q8_0", "q8_1"):
        S = 34 if k == "q8_0" else 36
        m = Map(32, S); m.scale(0, 2, _all(32))
        if k == "q8_1":
            m.ignored(2, 2)
        q0 = S - 32
        for t in range(32):
            for b in range(8):
                m.put(q0 + t, b, "exact", (t,))
    elif k == "q8_k":
        m = Map(256, 292); m.scale(0, 4, _all(256))
        for t in range(256):
            for b in range(8):
                m.put(4 + t, b, "exact", (t,))
        m.ignored(260, 32)
    elif k == "q1_0":
        m = Map(128, 18); m.scale(0, 2, _all(128))
        for t in range(16):
            for b in range(8):
                m.put(2 + t, b, "exact", (8 * t + b,))
    elif k == "q2_0":
        m = Map(64, 18); m.scale(0, 2, _all(64)); m.plane(2, 16, 2, 1)
    elif k == "q2_k":
        m = Map(256, 84)
        for t in range(16):
            m.scale(t, 1, range(16 * t, 16 * t + 16))
        m.plane(16, 64, 2, 32)
        m.scale(80, 4, _all(256))
    elif k == "q3_k":
        m = Map(256, 110)
        m.plane(0, 32, 1, 32)
        m.plane(32, 64, 2, 32)
        lf, af = _plane(4, 8), _plane(2, 4)
        for t in range(8):
            for b in range(8):
                g = lf(t, b)
                m.put(96 + t, b, "within", range(16 * g, 16 * g + 16))
        for t in range(4):
            for b in range(8):
                g = af(t, b)
                m.put(104 + t, b, "within", range(16 * g, 16 * g + 16))
        m.scale(108, 2, _all(256))
    elif k in ("q4_k", "q5_k"):
        m = Map(256, 144 if k == "q4_k" else 176)
        m.scale(0, 4, _all(256))
        run = lambda kk: range(32 * kk, 32 * kk + 32)
        for i in range(12):
            for b in range(8):
                if i < 4:
                    kk = i if b < 6 else i + 4        # a[i]; top bits feed a[i+4]
                elif i < 8:
                    kk = i - 4 if b < 6 else i        # m[i-4]; top bits feed m[i]
                else:
                    kk = i - 4                        # low nibble a[i-4], high nibble m[i-4]
                m.put(4 + i, b, "within", run(kk))
        if k == "q5_k":
            m.plane(16, 32, 1, 32)
            m.plane(48, 128, 4, 32)
        else:
            m.plane(16, 128, 4, 32)
    elif k == "q6_k":
        m = Map(256, 210)
        m.plane(0, 128, 4, 64)
        m.plane(128, 64, 2, 32)
        for t in range(16):
            m.scale(192 + t, 1, range(16 * t, 16 * t + 16))
        m.scale(208, 2, _all(256))
    elif k == "iq4_xs":
        m = Map(256, 136)
        m.scale(0, 2, _all(256))
        for t in range(2):
            for b in range(8):
                kk = (8 * t + b) // 2
                m.put(2 + t, b, "within", range(32 * kk, 32 * kk + 32))
        for t in range(4):
            for b in range(8):
                kk = 2 * t + (b // 4)
                m.put(4 + t, b, "within", range(32 * kk, 32 * kk + 32))
        m.plane(8, 128, 4, 16)
    elif k == "tq1_0":
        m = Map(256, 54)
        for t in range(32):
            m.scale(t, 1, [32 * p + t for p in range(5)])
        for t in range(16):
            m.scale(32 + t, 1, [160 + 16 * p + t for p in range(5)])
        for t in range(4):
            m.scale(48 + t, 1, [240 + 4 * p + t for p in range(4)])
        m.scale(52, 2, _all(256))
    elif k == "tq2_0":
        m = Map(256, 66); m.plane(0, 64, 2, 32); m.scale(64, 2, _all(256))
    elif k == "mxfp4":
        m = Map(32, 17); m.scale(0, 1, _all(32)); m.plane(1, 16, 4, 16)
    elif k == "nvfp4":
        m = Map(64, 36)
        for g in range(4):
            m.scale(g, 1, range(16 * g, 16 * g + 16))
            m.plane(4 + 8 * g, 8, 4, 8, base=16 * g)
    else:
        m = _build_iq(k)
    return m.done()


def _lane(i):
    return range(8 * i, 8 * i + 8)


def _signs_parity(m, byte0, g):
    """32-bit aux word at byte0: bits 7l..7l+6 are lane l's stored signs, 28..31 the scale."""
    for t in range(4):
        for b in range(8):
            kbit = 8 * t + b
            if kbit < 28:
                l, jj = kbit // 7, kbit % 7
                i = 4 * g + l
                m.put(byte0 + t, b, "exact", (8 * i + jj, 8 * i + 7))
            else:
                m.put(byte0 + t, b, "within", range(32 * g, 32 * g + 32))


def _build_iq(k):
    if k == "iq2_xxs":
        m = Map(256, 66); m.scale(0, 2, _all(256))
        for g in range(8):
            for l in range(4):
                for b in range(8):
                    m.put(2 + 8 * g + l, b, "some", _lane(4 * g + l))
            _signs_parity(m, 6 + 8 * g, g)
    elif k == "iq2_xs":
        m = Map(256, 74); m.scale(0, 2, _all(256))
        for i in range(32):
            for t in range(2):
                for b in range(8):
                    kbit = 8 * t + b
                    if kbit < 9:
                        m.put(2 + 2 * i + t, b, "some", _lane(i))
                    else:
                        jj = kbit - 9
                        m.put(2 + 2 * i + t, b, "exact", (8 * i + jj, 8 * i + 7))
        for g in range(8):
            for b in range(8):
                lanes = (4 * g, 4 * g + 1) if b < 4 else (4 * g + 2, 4 * g + 3)
                m.put(66 + g, b, "within", [o for i in lanes for o in _lane(i)])
    elif k == "iq2_s":
        m = Map(256, 82); m.scale(0, 2, _all(256))
        for i in range(32):
            for b in range(8):
                m.put(2 + i, b, "some", _lane(i))
                m.put(34 + i, b, "exact", (8 * i + b,))
        for g in range(8):
            for b in range(8):
                m.put(66 + g, b, "some", _lane(4 * g + b // 2))
                lanes = (4 * g, 4 * g + 1) if b < 4 else (4 * g + 2, 4 * g + 3)
                m.put(74 + g, b, "within", [o for i in lanes for o in _lane(i)])
    elif k == "iq3_xxs":
        m = Map(256, 98); m.scale(0, 2, _all(256))
        for i in range(32):
            for t in range(2):
                for b in range(8):
                    m.put(2 + 2 * i + t, b, "some", range(8 * i + 4 * t, 8 * i + 4 * t + 4))
        for g in range(8):
            _signs_parity(m, 66 + 4 * g, g)
    elif k == "iq3_s":
        m = Map(256, 110); m.scale(0, 2, _all(256))
        for i in range(32):
            for t in range(2):
                for b in range(8):
                    m.put(2 + 2 * i + t, b, "some", range(8 * i + 4 * t, 8 * i + 4 * t + 4))
            for b in range(8):
                m.put(74 + i, b, "exact", (8 * i + b,))
        for g in range(8):
            for b in range(8):
                l, t = b // 2, b % 2
                i = 4 * g + l
                m.put(66 + g, b, "some", range(8 * i + 4 * t, 8 * i + 4 * t + 4))
        for h in range(4):
            for b in range(8):
                g = 2 * h + b // 4
                m.put(106 + h, b, "within", range(32 * g, 32 * g + 32))
    elif k == "iq1_s":
        m = Map(256, 50); m.scale(0, 2, _all(256))
        for i in range(32):
            for b in range(8):
                m.put(2 + i, b, "some", _lane(i))
        for g in range(8):
            for t in range(2):
                for b in range(8):
                    kbit = 8 * t + b
                    if kbit < 12:
                        m.put(34 + 2 * g + t, b, "some", _lane(4 * g + kbit // 3))
                    else:
                        m.put(34 + 2 * g + t, b, "within", range(32 * g, 32 * g + 32))
    elif k == "iq1_m":
        m = Map(256, 56)
        for i in range(32):
            for b in range(8):
                m.put(i, b, "some", _lane(i))
        for t in range(16):
            for b in range(8):
                i = 2 * t + b // 4
                if b % 4 < 3:
                    m.put(32 + t, b, "some", _lane(i))
                else:
                    m.put(32 + t, b, "exact", _lane(i))
        for kw in range(4):
            for t in range(2):
                for b in range(8):
                    n = 8 * t + b
                    if n < 12:
                        f = n // 3
                        g = 2 * kw + f // 2
                        l0 = 2 * (f % 2)
                        outs = [o for l in (l0, l0 + 1) for o in _lane(4 * g + l)]
                        m.put(48 + 2 * kw + t, b, "within", outs)
                    else:
                        m.put(48 + 2 * kw + t, b, "within", _all(256))
    else:
        raise KeyError(k)
    return m
