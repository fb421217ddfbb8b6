"""Pure-Python brute force for tiny shapes — TEST INFRASTRUCTURE.

Independent of ``oracle.reference``: no NumPy, only ``math`` and nested loops,
so a pin that compares the two catches a mistake in either (a transposed
operand, a wrong head slice of ``B``, a dropped adapter term, a sign in the
rotation).  Inputs are nested Python lists with the layouts documented in
``oracle.reference``.

Definition followed (LRAgent, arXiv 2602.01053v2, App. A.3 and App. D.1):
``K = K_base + rot(L_k B_k)``, ``V = V_base + L_v B_v`` per KV head slice,
``O = softmax(q K^T * scale) V`` with bottom-right causal visibility.
"""
import math


def brute_attention(q, k_base, v_base, l_k, l_v, b_k, b_v, q_pos, scale=None,
                    rope_theta=None):
    n_rows = len(q)
    h_q = len(q[0])
    d = len(q[0][0])
    h_kv = len(k_base)
    kv_len = len(k_base[0])
    r = len(l_k[0])
    g = h_q // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = [[[0.0] * d for _ in range(h_q)] for _ in range(n_rows)]
    for hq in range(h_q):
        h = hq // g
        # materialise the adapted key and value rows of this KV head
        keys, vals = [], []
        for j in range(kv_len):
            dk = [sum(l_k[j][t] * b_k[t][h * d + c] for t in range(r)) for c in range(d)]
            if rope_theta is not None:
                half = d // 2
                rot = [0.0] * d
                for i in range(half):
                    ang = j * rope_theta ** (-2.0 * i / d)
                    c_, s_ = math.cos(ang), math.sin(ang)
                    rot[i] = dk[i] * c_ - dk[i + half] * s_
                    rot[i + half] = dk[i + half] * c_ + dk[i] * s_
                dk = rot
            keys.append([k_base[h][j][c] + dk[c] for c in range(d)])
            vals.append([v_base[h][j][c] + sum(l_v[j][t] * b_v[t][h * d + c] for t in range(r))
                         for c in range(d)])
        for i in range(n_rows):
            vis = [j for j in range(kv_len) if j <= q_pos[i]]
            scores = [scale * sum(q[i][hq][c] * keys[j][c] for c in range(d)) for j in vis]
            mx = max(scores)
            ex = [math.exp(s - mx) for s in scores]
            tot = sum(ex)
            for c in range(d):
                out[i][hq][c] = sum(ex[n] * vals[j][c] for n, j in enumerate(vis)) / tot
    return out


def brute_matmul(x, a):
    """``x @ a`` with explicit loops (for the LR-cache build pin)."""
    n, k = len(x), len(x[0])
    m = len(a[0])
    return [[sum(x[i][t] * a[t][j] for t in range(k)) for j in range(m)] for i in range(n)]
