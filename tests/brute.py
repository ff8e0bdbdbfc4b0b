"""Scalar brute-force paged attention for tiny inputs (pin for the oracle).

Written independently of ``oracle/``: Python floats, math.exp and math.fsum,
bf16 decoded with struct, each score a dot product over the head dimension,
each key/value row located by its own block-table lookup.
"""
import math
import struct


def bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def scalar(x, dtype):
    return float(x) if dtype == "f32" else bf16_to_float(int(x))


def brute_attention(q, k_pool, v_pool, tables, lens, q_len, scale, block_size, dtype):
    """q: [B][q_len][H_q][d]; k_pool [NB][H_kv][d/32][bs][32]; v_pool [NB][H_kv][d][bs].
    Returns nested lists [B][q_len][H_q][d] of floats."""
    B, _, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    out = []
    for b in range(B):
        L = int(lens[b])
        ob = []
        for i in range(q_len):
            oi = []
            for h in range(Hq):
                g = h // G
                qv = [scalar(q[b, i, h, c], dtype) for c in range(d)]
                scores, vrows = [], []
                for t in range(L - q_len + i + 1):
                    blk = int(tables[b][t // block_size])
                    off = t % block_size
                    kr = [scalar(k_pool[blk, g, c // 32, off, c % 32], dtype) for c in range(d)]
                    vrows.append([scalar(v_pool[blk, g, c, off], dtype) for c in range(d)])
                    scores.append(scale * math.fsum(qv[c] * kr[c] for c in range(d)))
                mx = max(scores)
                e = [math.exp(s - mx) for s in scores]
                z = math.fsum(e)
                oi.append([math.fsum(e[t] * vrows[t][c] for t in range(len(e))) / z for c in range(d)])
            ob.append(oi)
        out.append(ob)
    return out


def brute_attention_logical(q, k, v, q_len, scale, dtype):
    """One sequence from its never-paged K/V: q [q_len][H_q][d]; k, v
    [L][H_kv][d] in token order. No pool, no block table: this pin shares
    nothing with the pool layout or the gather. Drafted token i sees
    positions 0 .. L - q_len + i. Returns nested lists [q_len][H_q][d]."""
    L, Hkv, d = k.shape
    Hq = q.shape[1]
    G = Hq // Hkv
    out = []
    for i in range(q_len):
        oi = []
        for h in range(Hq):
            g = h // G
            qv = [scalar(q[i, h, c], dtype) for c in range(d)]
            scores = []
            for t in range(L - q_len + i + 1):
                scores.append(scale * math.fsum(qv[c] * scalar(k[t, g, c], dtype) for c in range(d)))
            mx = max(scores)
            e = [math.exp(s - mx) for s in scores]
            z = math.fsum(e)
            oi.append([math.fsum(e[t] * scalar(v[t, g, c], dtype) for t in range(len(e))) / z for c in range(d)])
        out.append(oi)
    return out
