"""Second, independent FP64 reference: the chunk form of the KDA operator.

Test infrastructure only (it pins the token oracle in ``kda_oracle.c``; it
shares no code with it and none with the GPU path). Tiny sizes only: it forms
pairwise decay factors exp(G_r - G_s) directly, with no blocking or
factorisation, so a reader can check it against the per-chunk operation table
of "KDA at the production shape..." section 2.1 (aqk, akk, w, u, v_new,
intra, inter, state update, triangular inverse) and the state-loop pieces of
section 1.1 (v_new = u - w h, h += k^T v_new, channel decay of h by the last
cumulative gate of the chunk).

One cell of that table is garbled in the extracted text: the u row multiplies
the inverse by an elementwise product of w and v, which is ill-typed (w is
C x K, v is C x V). The reading used here is u = M^-1 (beta * v), the only
one consistent with the rest of the table and with the token recurrence.

Per chunk (rows r = 1..c, entering state h, G = cumulative sum of g within
the chunk):
    Akk[r,s] = beta_r sum_k kh_rk kh_sk exp(G_rk - G_sk)     (s < r)
    Aqk[r,s] = sum_k qh_rk kh_sk exp(G_rk - G_sk)            (s <= r)
    T  = (I + Akk)^-1
    W  = T (beta * kh * e^G),   U = T (beta * v)
    Vn = U - W h
    O  = (qh * e^G) h + Aqk Vn
    h <- Diag(e^{G_c}) h + (kh * e^{G_c - G})^T Vn

``chunk_bwd`` differentiates exactly these chunk operations (reverse over
chunks) and then the prologue.
"""
from __future__ import annotations

import numpy as np


def _prologue(q, k, raw_g, raw_beta, A_log_h, dt_bias_h, scale, lower_bound, eps):
    """Rows of one (sequence, head): q,k,raw_g [L,K], raw_beta [L]."""
    rq = 1.0 / np.sqrt(np.sum(q * q, axis=1) + eps)
    rk = 1.0 / np.sqrt(np.sum(k * k, axis=1) + eps)
    qbar = q * rq[:, None]
    qh = scale * qbar
    kh = k * rk[:, None]
    beta = 1.0 / (1.0 + np.exp(-raw_beta))
    z = np.exp(A_log_h) * (raw_g + dt_bias_h[None, :])
    sz = 1.0 / (1.0 + np.exp(-z))
    g = lower_bound * sz
    return dict(rq=rq, rk=rk, qbar=qbar, qh=qh, kh=kh, beta=beta, z=z, sz=sz, g=g)


def _chunk_mats(qh, kh, beta, G):
    """Pairwise-exponent Akk, Aqk for one chunk (c rows)."""
    c = qh.shape[0]
    E = np.exp(G[:, None, :] - G[None, :, :])  # [r, s, k]
    P = np.einsum("rk,sk,rsk->rs", kh, kh, E)
    Q = np.einsum("rk,sk,rsk->rs", qh, kh, E)
    Akk = beta[:, None] * P * np.tril(np.ones((c, c)), -1)
    Aqk = Q * np.tril(np.ones((c, c)), 0)
    return Akk, Aqk, P, E


def chunk_fwd(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, chunk,
              scale=1.0, lower_bound=-5.0, eps=1e-6, h0=None, return_state=False):
    """Chunk-form forward. Returns O [T,H,V] (float64), or (O, ht) with the
    state after every sequence's last chunk, ht [N,H,K,V], when return_state.
    h0 [N,H,K,V]: the state each sequence enters its first chunk with (zero
    when None)."""
    T, H, K = q.shape
    out = np.zeros((T, H, v.shape[2]))
    ht = np.zeros((len(cu_seqlens) - 1, H, K, v.shape[2]))
    for n in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        for hh in range(H):
            p = _prologue(q[a:b, hh], k[a:b, hh], raw_g[a:b, hh], raw_beta[a:b, hh],
                          A_log[hh], dt_bias[hh], scale, lower_bound, eps)
            h = np.zeros((K, v.shape[2])) if h0 is None else np.array(h0[n, hh], dtype=np.float64)
            for c0 in range(0, b - a, chunk):
                sl = slice(c0, min(c0 + chunk, b - a))
                G = np.cumsum(p["g"][sl], axis=0)
                Akk, Aqk, _, _ = _chunk_mats(p["qh"][sl], p["kh"][sl], p["beta"][sl], G)
                Tm = np.linalg.inv(np.eye(G.shape[0]) + Akk)
                W = Tm @ (p["beta"][sl, None] * p["kh"][sl] * np.exp(G))
                U = Tm @ (p["beta"][sl, None] * v[a:b, hh][sl])
                Vn = U - W @ h
                out[a:b, hh][sl] = (p["qh"][sl] * np.exp(G)) @ h + Aqk @ Vn
                kg = p["kh"][sl] * np.exp(G[-1][None, :] - G)
                h = np.exp(G[-1])[:, None] * h + kg.T @ Vn
            ht[n, hh] = h
    return (out, ht) if return_state else out


def chunk_bwd(q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, dO, chunk,
              scale=1.0, lower_bound=-5.0, eps=1e-6):
    """Chunk-form reverse-mode gradient of sum(O * dO) for all seven inputs."""
    T, H, K = q.shape
    V = v.shape[2]
    res = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               draw_g=np.zeros_like(raw_g), draw_beta=np.zeros_like(raw_beta),
               dA_log=np.zeros(H), ddt_bias=np.zeros((H, K)))
    for n in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        L = b - a
        for hh in range(H):
            p = _prologue(q[a:b, hh], k[a:b, hh], raw_g[a:b, hh], raw_beta[a:b, hh],
                          A_log[hh], dt_bias[hh], scale, lower_bound, eps)
            starts = list(range(0, L, chunk))
            # forward over chunks, keeping the entering states
            hs = []
            h = np.zeros((K, V))
            for c0 in starts:
                sl = slice(c0, min(c0 + chunk, L))
                hs.append(h)
                G = np.cumsum(p["g"][sl], axis=0)
                Akk, Aqk, _, _ = _chunk_mats(p["qh"][sl], p["kh"][sl], p["beta"][sl], G)
                Tm = np.linalg.inv(np.eye(G.shape[0]) + Akk)
                W = Tm @ (p["beta"][sl, None] * p["kh"][sl] * np.exp(G))
                U = Tm @ (p["beta"][sl, None] * v[a:b, hh][sl])
                kg = p["kh"][sl] * np.exp(G[-1][None, :] - G)
                h = np.exp(G[-1])[:, None] * h + kg.T @ (U - W @ h)
            dqh = np.zeros((L, K))
            dkh = np.zeros((L, K))
            dbeta = np.zeros(L)
            dg = np.zeros((L, K))
            dvv = np.zeros((L, V))
            dhp = np.zeros((K, V))  # gradient of the state leaving the chunk
            for ci in range(len(starts) - 1, -1, -1):
                sl = slice(starts[ci], min(starts[ci] + chunk, L))
                h = hs[ci]
                qh, kh, beta = p["qh"][sl], p["kh"][sl], p["beta"][sl]
                vv = v[a:b, hh][sl]
                dOc = dO[a:b, hh][sl]
                c = qh.shape[0]
                G = np.cumsum(p["g"][sl], axis=0)
                Akk, Aqk, P, E = _chunk_mats(qh, kh, beta, G)
                Tm = np.linalg.inv(np.eye(c) + Akk)
                eG = np.exp(G)
                gam = np.exp(G[-1])
                Kb = beta[:, None] * kh * eG
                Bv = beta[:, None] * vv
                W = Tm @ Kb
                U = Tm @ Bv
                Vn = U - W @ h
                qg = qh * eG
                kg = kh * np.exp(G[-1][None, :] - G)
                # state path
                dVn = Aqk.T @ dOc + kg @ dhp
                dh = gam[:, None] * dhp + qg.T @ dOc - W.T @ dVn
                # direct products
                dAqk = np.tril(dOc @ Vn.T)
                dqg = dOc @ h.T
                dkg = Vn @ dhp.T
                dW = -dVn @ h.T
                dGc = np.sum(h * dhp, axis=1) * gam
                # through the inverse
                dBv = Tm.T @ dVn
                dKb = Tm.T @ dW
                dT = dVn @ Bv.T + dW @ Kb.T
                dAkk = np.tril(-Tm.T @ dT @ Tm.T, -1)
                # value and beta
                dvv[sl] += beta[:, None] * dBv
                dbeta[sl] += np.sum(dBv * vv, axis=1) + np.sum(dKb * kh * eG, axis=1) \
                    + np.sum(dAkk * P, axis=1)
                dGl = np.zeros((c, K))
                dqh_l = np.zeros((c, K))
                dkh_l = np.zeros((c, K))
                # gated products X[r,s] = sum_k a_rk c_sk exp(G_rk - G_sk)
                for dX, aa, cc, da, dc in ((beta[:, None] * dAkk, kh, kh, dkh_l, dkh_l),
                                           (dAqk, qh, kh, dqh_l, dkh_l)):
                    t3 = dX[:, :, None] * E  # [r,s,k]
                    da += np.einsum("rsk,sk->rk", t3, cc)
                    dc += np.einsum("rsk,rk->sk", t3, aa)
                    m = np.einsum("rsk,rk,sk->rsk", t3, aa, cc)
                    dGl += m.sum(axis=1)
                    dGl -= m.sum(axis=0)
                dqh_l += dqg * eG
                dGl += dqg * qg
                dkh_l += dkg * np.exp(G[-1][None, :] - G) + beta[:, None] * dKb * eG
                dGl += -dkg * kg + dKb * Kb
                dGl[-1] += np.sum(dkg * kg, axis=0) + dGc
                dqh[sl] += dqh_l
                dkh[sl] += dkh_l
                # G = cumsum(g) within the chunk: dg = reverse cumsum of dG
                dg[sl] += np.cumsum(dGl[::-1], axis=0)[::-1]
                dhp = dh
            # prologue VJP
            qd = np.sum(p["qbar"] * dqh, axis=1)
            kd = np.sum(p["kh"] * dkh, axis=1)
            res["dq"][a:b, hh] = scale * p["rq"][:, None] * (dqh - p["qbar"] * qd[:, None])
            res["dk"][a:b, hh] = p["rk"][:, None] * (dkh - p["kh"] * kd[:, None])
            res["dv"][a:b, hh] = dvv
            res["draw_beta"][a:b, hh] = dbeta * p["beta"] * (1 - p["beta"])
            dz = dg * lower_bound * p["sz"] * (1 - p["sz"])
            dx = dz * np.exp(A_log[hh])
            res["draw_g"][a:b, hh] = dx
            res["ddt_bias"][hh] += dx.sum(axis=0)
            res["dA_log"][hh] += np.sum(dz * p["z"])
    return res
