"""Error bounds for the backward pass, derived from the arithmetic of fa_bwd (test infrastructure).

The GPU backward takes the forward's O (bf16) and LSE (fp32) and, per (query i, key j):
  * recomputes p = exp2(fma(s, scale * log2 e, -LSE * log2 e)) from fp32 scores s (bf16 products,
    fp32 accumulation over d on the matrix core);
  * forms dS = p * (dP - Dr) in fp32, with dP = dO_i . v_j (fp32 accumulation) and
    Dr_i = dO_i . O_i from the forward's bf16 O;
  * rounds p and dS to bf16 (round to nearest even) before dV = P^T dO, dQ = scale dS K and
    dK = scale dS^T Q, which accumulate in fp32 (over the keys for dQ; over the queries of every
    query head sharing the K/V head for dK and dV);
  * rounds dQ, dK, dV to bf16.
The reference (oracle.attention_backward) differentiates the definition in float64 from Q, K, V,
dO alone.  For each step the bound below takes the worst case of its rounding, with
u = 2^-24 (fp32) and u_b = 2^-8 (bf16):
  * p: relative error tau = expm1(|dLSE_i| + eps_s + 2^-22), with dLSE the forward's LSE error
    (known to the test), eps_s = scale 2 d u sum_c |q_ic k_jc| + 3 u |s_ij| + 2 u |LSE_i| the
    error of the exponent (score accumulation, the fp32 scale, the exponent's FMA), 2^-22 the
    hardware exp2;
  * dP: |delta_ij| <= 2 d u sum_c |dO_ic v_jc|;  Dr: |rho_i| <= |dO_i . (O_gpu,i - O_i)| +
    2 d u sum_c |dO_ic O_gpu,ic|;
  * dS (fp32): |F_ij| <= P_ij [(tau + 2u (1 + tau)) A_ij + delta_ij + rho_i], with
    A_ij = |dP_ij - Dr_i| + delta_ij + rho_i; then bf16: E_ij = F_ij + u_b (|dS_ij| + F_ij);
  * dQ_ic: G = scale sum_j E_ij |k_jc| + (2 N_k + 2) u scale sum_j (|dS_ij| + E_ij) |k_jc|, and
    |error| <= G + u_b (|dQ_ic| + G); dK likewise with Q and the N_q * group accumulated queries;
  * dV_jc: with kappa = tau + u_b (1 + tau) the error of bf16(p),
    G = sum_i P_ij kappa_ij |dO_ic| + (2 N_q group + 2) u sum_i P_ij (1 + kappa_ij) |dO_ic|, and
    |error| <= G + u_b (|dV_jc| + G).
The sums treat every rounding as adding up with the same sign, so the bound is loose by about the
square root of the number of terms on random data; it still catches an error confined to a
tile, a row or a column, which a whole-tensor norm can average away.

Beside it, the relative L2 error is held to 1.5 times a prediction from the same roundings
taken as independent: each bf16 rounding contributes an RMS relative error of at most
u_b / sqrt(3), propagated through the products taken over squares (sum_j dS^2 k^2 for dQ, ...),
plus the output rounding, plus the exact effect of the forward's LSE and O errors (known to the
test).  The realised value is about 0.75 of the prediction on random data (the RMS of a
round-to-nearest error over a binade is about 0.74 of u_b / sqrt(3)).
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24
UB = 2.0 ** -8
EXP2_REL = 2.0 ** -22
SIGMA_B = UB / np.sqrt(3.0)
REL_L2_FACTOR = 1.5


def _head(q, k, v, do, o_gpu, lse_gpu, scale, causal, diag):
    """Reference gradients of one query head, the bound terms and the RMS-model terms."""
    q, k, v, do, o_gpu, lse_gpu = (np.asarray(x, np.float64) for x in (q, k, v, do, o_gpu, lse_gpu))
    nq, d = q.shape
    nk = k.shape[0]
    s = scale * (q @ k.T)
    if causal:
        vis = np.arange(nk)[None, :] <= np.arange(nq)[:, None] + diag
        s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    lse = m + np.log(l)
    p = e / l[:, None]
    o = p @ v
    dp = do @ v.T
    dr = (do * o).sum(axis=1)
    ds = p * (dp - dr[:, None])
    s_fin = np.where(np.isfinite(s), s, 0.0)
    dlse = np.abs(lse_gpu - lse)
    eps_s = scale * 2 * d * U * (np.abs(q) @ np.abs(k).T) + 3 * U * np.abs(s_fin) + 2 * U * np.abs(lse)[:, None]
    tau = np.expm1(dlse[:, None] + eps_s + EXP2_REL)
    delta = 2 * d * U * (np.abs(do) @ np.abs(v).T)
    ddr = (do * (o_gpu - o)).sum(axis=1)
    rho = np.abs(ddr) + 2 * d * U * (np.abs(do) * np.abs(o_gpu)).sum(axis=1)
    a = np.abs(dp - dr[:, None]) + delta + rho[:, None]
    f = p * ((tau + 2 * U * (1 + tau)) * a + delta + rho[:, None])
    err_ds = f + UB * (np.abs(ds) + f)
    kappa = tau + UB * (1 + tau)
    ads = np.abs(ds) + err_ds
    return {
        "dq": scale * ds @ k, "dk": scale * ds.T @ q, "dv": p.T @ do,
        # bound parts (before the output rounding)
        "gq_e": scale * err_ds @ np.abs(k), "gq_w": scale * ads @ np.abs(k),
        "gk_e": scale * err_ds.T @ np.abs(q), "gk_w": scale * ads.T @ np.abs(q),
        "gv_e": (p * kappa).T @ np.abs(do), "gv_w": (p * (1 + kappa)).T @ np.abs(do),
        # RMS model: variance of the random roundings, and the systematic part from dLSE and dO
        "vq": (SIGMA_B * scale) ** 2 * ((ds ** 2) @ (k ** 2)),
        "vk": (SIGMA_B * scale) ** 2 * ((ds ** 2).T @ (q ** 2)),
        "vv": SIGMA_B ** 2 * ((p ** 2).T @ (do ** 2)),
        "sq": -(lse_gpu - lse)[:, None] * (scale * ds @ k) - scale * ddr[:, None] * (p @ k),
        "sk": scale * (-(lse_gpu - lse)[:, None] * ds - p * ddr[:, None]).T @ q,
        "sv": (-(lse_gpu - lse)[:, None] * p).T @ do,
        "nq": nq,
    }


def reference_and_bounds(q, k, v, do, o_gpu, lse_gpu, scale, causal=False, diag=0):
    """[B,H,Nq,d] q, do, o_gpu; [B,H_kv,Nk,d] k, v; [B,H,Nq] lse_gpu (float arrays of the values the
    GPU saw and produced).  Returns, for "dq", "dk", "dv": (reference, element-wise bound,
    predicted relative L2 error)."""
    q, do, o_gpu, lse_gpu = (np.asarray(x) for x in (q, do, o_gpu, lse_gpu))
    k, v = np.asarray(k), np.asarray(v)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    grp = H // Hkv
    out = {x: [np.zeros(shape) for _ in range(6)] for x, shape in
           (("dq", (B, H, Nq, d)), ("dk", (B, Hkv, Nk, d)), ("dv", (B, Hkv, Nk, d)))}
    for b in range(B):
        for h in range(H):
            hk = h // grp
            t = _head(q[b, h], k[b, hk], v[b, hk], do[b, h], o_gpu[b, h], lse_gpu[b, h], scale, causal, diag)
            for x, idx, e, wgt, var, sys_ in (("dq", (b, h), "gq_e", "gq_w", "vq", "sq"),
                                              ("dk", (b, hk), "gk_e", "gk_w", "vk", "sk"),
                                              ("dv", (b, hk), "gv_e", "gv_w", "vv", "sv")):
                ref, ge, gw, vv, ss, _ = out[x]
                ref[idx] += t[x]
                ge[idx] += t[e]
                gw[idx] += t[wgt]
                vv[idx] += t[var]
                ss[idx] += t[sys_]
    res = {}
    for x, n_acc in (("dq", Nk), ("dk", Nq * grp), ("dv", Nq * grp)):
        ref, ge, gw, vv, ss, _ = out[x]
        g = ge + (2 * n_acc + 2) * U * gw
        bound = g + UB * (np.abs(ref) + g) + 1e-30
        var = vv + (SIGMA_B * ref) ** 2
        pred = float(np.sqrt((ss ** 2).sum() + var.sum()) / max(np.linalg.norm(ref), 1e-300))
        res[x] = (ref, bound, pred)
    return res


def check(got: dict, res: dict, what: str = ""):
    """got: "dq"/"dk"/"dv" -> GPU gradients (float arrays).  Asserts every element within its bound
    and the relative L2 error within REL_L2_FACTOR x the prediction; returns the figures."""
    figs = {}
    for x in ("dq", "dk", "dv"):
        ref, bound, pred = res[x]
        g = np.asarray(got[x], np.float64)
        ratio = float((np.abs(g - ref) / bound).max())
        rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
        figs[x] = {"worst_err_over_bound": ratio, "rel_l2": rel, "rel_l2_pred": pred,
                   "rel_l2_bar": REL_L2_FACTOR * pred, "finite": bool(np.isfinite(g).all())}
    print(f"    backward {what}: {figs}", flush=True)
    for x, f in figs.items():
        assert f["finite"], (what, x, f)
        assert f["worst_err_over_bound"] <= 1.0, (what, x, f)
        assert f["rel_l2"] <= f["rel_l2_bar"], (what, x, f)
    return figs
