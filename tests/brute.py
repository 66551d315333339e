"""Brute-force attention for tiny inputs, written independently of ``oracle``.

Pure Python scalars. Rotation uses complex exponentials: the pair
(x[i], x[i + d/2]) is the complex number x[i] + 1j*x[i + d/2], and R_p
multiplies it by exp(1j * p * theta_i) (RoFormer's complex form). The
visibility rule is stated per segment, from the meaning of the primitives in
"MiniPIC: Flexible Position-Independent Caching in <100LOC", §3.1.1 and
§3.3.1: a token of a PDep segment sees every earlier token; any other token
sees the earlier tokens of its own segment and of GLOBAL (shared-prefix)
segments.
"""
import cmath
import math


def theta(i, d, base):
    return base ** (-(2.0 * i) / d)


def rot(vec, p, base):
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for i in range(h):
        z = complex(vec[i], vec[i + h]) * cmath.exp(1j * p * theta(i, d, base))
        out[i] = z.real
        out[i + h] = z.imag
    return out


def segment_of(c, segments):
    """segments: list of (start, length, kind)."""
    for s in segments:
        if s[0] <= c < s[0] + s[1]:
            return s
    raise ValueError(c)


def visible(c, j, segments):
    if j > c:
        return False
    sc = segment_of(c, segments)
    if sc[2] == "pdep":
        return True
    sj = segment_of(j, segments)
    return sj is sc or sj[2] == "global"


def attention(q, q_ctx, k, v, pos, segments, base, q_rotated):
    """q: [nq][Hq][d] lists; k, v: [L][Hkv][d]; returns [nq][Hq][d]."""
    nq = len(q)
    Hq = len(q[0]) if nq else 0
    L = len(k)
    Hkv = len(k[0])
    d = len(k[0][0])
    G = Hq // Hkv
    out = []
    for n in range(nq):
        c = q_ctx[n]
        row = []
        for h in range(Hq):
            g = h // G
            qv = q[n][h] if q_rotated else rot(q[n][h], pos[c], base)
            scores = []
            for j in range(L):
                if visible(c, j, segments):
                    kv = rot(k[j][g], pos[j], base)
                    s = sum(qv[t] * kv[t] for t in range(d)) / math.sqrt(d)
                    scores.append((j, s))
            mx = max(s for _, s in scores)
            ws = [(j, math.exp(s - mx)) for j, s in scores]
            tot = sum(w for _, w in ws)
            o = [0.0] * d
            for j, w in ws:
                for t in range(d):
                    o[t] += w / tot * v[j][g][t]
            row.append(o)
        out.append(row)
    return out
