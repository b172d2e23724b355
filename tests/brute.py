"""Pure-Python brute force of the MoE layer, for tiny inputs only.

Written independently of the oracle to pin it: formats are decoded from their
bit fields (not from a table), bf16 rounding works on the IEEE-754 bit
pattern, every dot product is a Python loop, the ranking uses sorted() on
(-logit, id), and the layer is evaluated densely: every expert runs on every
token and is weighted by a gate that is zero for experts outside the top-k.
"""
from __future__ import annotations

import math
import struct


def e2m1_value(code: int) -> float:
    """FP4 E2M1 from its bit fields s|ee|m (OCP MX v1.0): exponent bias 1, subnormal at e=0."""
    sign = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return sign * mag


def e8m0_value(byte: int) -> float:
    """E8M0 scale: 2^(byte - 127); 255 encodes NaN (OCP MX v1.0)."""
    return math.nan if byte == 255 else 2.0 ** (byte - 127)


def bf16_bits_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def bf16_round(v: float) -> float:
    """Round a Python float (fp64) to bf16 precision (8 significant bits), ties to even."""
    if v == 0.0 or not math.isfinite(v):
        return v
    bits = struct.unpack("<Q", struct.pack("<d", v))[0]
    keep = 52 - 7                      # fp64 has 52 fraction bits, bf16 keeps 7
    low = bits & ((1 << keep) - 1)
    base = bits >> keep
    half = 1 << (keep - 1)
    if low > half or (low == half and (base & 1)):
        base += 1
    return struct.unpack("<d", struct.pack("<Q", base << keep))[0]


def decode_matrix(codes, scales):
    """codes [R][K/2], scales [R][K/32] (nested sequences of ints) -> list of float rows."""
    out = []
    for crow, srow in zip(codes, scales):
        K = 2 * len(crow)
        row = []
        for kk in range(K):
            byte = int(crow[kk // 2])
            c = byte & 0xF if kk % 2 == 0 else byte >> 4
            row.append(e2m1_value(c) * e8m0_value(int(srow[kk // 32])))
        out.append(row)
    return out


def mxfp4_quantize(row):
    """OCP MX v1.0 conversion of a row to MXFP4 values, block by block of 32: the shared exponent
    is floor(log2 amax) minus E2M1's largest exponent (2); each element goes to the E2M1 value
    nearest to v / 2^E (searched over all sixteen codes), an exact tie to the even code, so past
    6 it stays at 6; an all-zero block stays zero."""
    out = []
    for b0 in range(0, len(row), 32):
        blk = row[b0:b0 + 32]
        amax = max(abs(v) for v in blk)
        if amax == 0.0:
            out.extend([0.0] * len(blk))
            continue
        E = max(-127, min(127, math.floor(math.log2(amax)) - 2))
        for v in blk:
            q = v / 2.0 ** E
            best = min(range(16), key=lambda c: (abs(e2m1_value(c) - q), c & 1, c))
            out.append(e2m1_value(best) * 2.0 ** E)
    return out


def expert_dense(xrow, Wg, Wu, Wd, limit, act4=False):
    """One SwiGLU expert on one token: returns (h list, z list).  act4: the rows entering each
    projection are quantized to MXFP4 first."""
    if act4:
        xrow = mxfp4_quantize(xrow)
    h = []
    for i in range(len(Wg)):
        g = sum(a * b for a, b in zip(xrow, Wg[i]))
        u = sum(a * b for a, b in zip(xrow, Wu[i]))
        g = min(max(g, -limit), limit)
        u = min(max(u, -limit), limit)
        h.append(bf16_round(g / (1.0 + math.exp(-g)) * u))
    if act4:
        h = mxfp4_quantize(h)
    z = [sum(a * b for a, b in zip(h, Wd[n])) for n in range(len(Wd))]
    return h, z


def brute_layer(inp, act4=False):
    """Dense evaluation of the layer; returns dict(logits, idx, w, y) as Python lists."""
    T, D, E, k, I = inp.T, inp.D, inp.E, inp.k, inp.I
    x = [[bf16_bits_value(int(b)) for b in row] for row in inp.x_bf16]
    wr = [[float(v) for v in row] for row in inp.w_router]
    br = [float(v) for v in inp.b_router]
    experts = []
    for e in range(E):
        gu = decode_matrix(inp.gu_codes[e], inp.gu_scales[e])
        dn = decode_matrix(inp.dn_codes[e], inp.dn_scales[e])
        experts.append((gu[:I], gu[I:], dn))
    logits, idx_all, w_all, y_all = [], [], [], []
    for t in range(T):
        lt = [sum(a * b for a, b in zip(x[t], wr[e])) + br[e] for e in range(E)]
        ranked = sorted(range(E), key=lambda e: (-lt[e], e))
        sel = sorted(ranked[:k])
        m = max(lt[e] for e in sel)
        ex = {e: math.exp(lt[e] - m) for e in sel}
        s = sum(ex[e] for e in sel)
        gate = [ex[e] / s if e in ex else 0.0 for e in range(E)]
        y = [0.0] * D
        for e in range(E):                       # every expert, ascending id
            _, z = expert_dense(x[t], *experts[e], inp.swiglu_limit, act4=act4)
            y = [a + gate[e] * b for a, b in zip(y, z)]
        logits.append(lt)
        idx_all.append(sel)
        w_all.append([gate[e] for e in sel])
        y_all.append(y)
    return dict(logits=logits, idx=idx_all, w=w_all, y=y_all)
