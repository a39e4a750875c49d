"""Per-element error budget of the SSD (Mamba-2) form computed with bf16
matrix-core operands -- test infrastructure.

The kernel rounds three kinds of operand to bf16 (relative error at most
u = 2^-8 each, the unit roundoff of an 8-bit significand), everything else is float32 with a float32 state:
  * the masked score S[t,s] = (C_t . B_s) exp(lam_t - lam_s) dt_s of a pair
    of tokens in the same chunk (intra-chunk product S X);
  * the decay-weighted input X_w[s,:] = x_s dt_s exp(lam_end - lam_s) that a
    token adds to the state (state update X_w^T B);
  * the copy of the state entering a chunk used for its readout C h^T.
Writing w_ts = dt_s exp(sum_{s<r<=t} dt_r A) for the weight of token s in
output t (the definition's decay), the first two roundings perturb each
contribution of token s to out[t,p] by at most u w_ts |C_t . B_s| |x_s,p|
(both carry the dot product C_t . B_s exactly: B and C are bf16 inputs and
the products accumulate in float32), so their total is at most u E1 with
    E1[t,p] = sum_{s<=t} w_ts |C_t . B_s| |x_s,p|.
The third perturbs the readout of the state entering t's chunk by at most
u E2 with
    E2[t,p] = sum_n |C_t,n| |h_start[p,n]| exp(lam_t - lam_start)
(h_start the exact state entering the chunk of 64 tokens holding t, the
chunk size of the kernel's interface).  Before the gate the error is thus
at most u (E1 + E2) up to float32 rounding; the gate multiplies it by
|silu(z)|.  The final state carries only the second rounding: at most u
times sum_s w_Ls |x_s,p| |B_s,n|.

These are bounds built from the definition on the pages ("RWKV-v6 vs.
Mamba-3 Selective State Spaces", section "3.1. State Space Duality (SSD)",
and the recurrence h_t = e^(dt A) h + dt x B^T, y = C h + D x, read as in
the oracle's header), in float64 numpy; nothing here comes from the HIP
path.
"""
import numpy as np

CHUNK = 64


def _softplus(u):
    return np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))


def ssd_budget(x, dt, A, B, C, dt_bias=None, dt_softplus=True, h0=None, chunk=CHUNK):
    """E1 and E2 per output element and the final-state budget.

    x: (batch, L, H, P); dt: (batch, L, H); A: (H,); B, C: (batch, L, G, N);
    h0: (batch, H, P, N) or None.  Returns (E1, E2 (batch, L, H, P),
    S_last (batch, H, P, N)) in float64."""
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    E1 = np.zeros((batch, L, H, P))
    E2 = np.zeros((batch, L, H, P))
    S_last = np.zeros((batch, H, P, N))
    for b in range(batch):
        for h in range(H):
            g = h // hpg
            u = dt[b, :, h] + (0.0 if dt_bias is None else float(dt_bias[h]))
            d = _softplus(u) if dt_softplus else u
            lam = np.cumsum(d * A[h])
            CB = C[b, :, g, :] @ B[b, :, g, :].T                      # (L, L): C_t . B_s
            W = np.tril(np.exp(np.minimum(lam[:, None] - lam[None, :], 0.0)) * d[None, :])
            ax = np.abs(x[b, :, h, :])
            e1 = (np.abs(CB) * W) @ ax                                  # (L, P)
            # exact states entering each chunk, then the readout budget
            st = np.zeros((P, N)) if h0 is None else np.asarray(h0[b, h], np.float64).copy()
            e2 = np.zeros((L, P))
            aC = np.abs(C[b, :, g, :])
            for c0 in range(0, L, chunk):
                c1 = min(L, c0 + chunk)
                lam0 = lam[c0 - 1] if c0 > 0 else 0.0
                dec = np.exp(lam[c0:c1] - lam0)                         # (len,)
                e2[c0:c1] = dec[:, None] * (aC[c0:c1] @ np.abs(st).T)  # (len, P)
                # advance the exact state over the chunk
                wend = np.exp(lam[c1 - 1] - lam[c0:c1]) * d[c0:c1]      # (len,)
                st = np.exp(lam[c1 - 1] - lam0) * st + (x[b, c0:c1, h, :] * wend[:, None]).T @ B[b, c0:c1, g, :]
            E1[b, :, h, :] = e1
            E2[b, :, h, :] = e2
            wL = np.exp(lam[-1] - lam) * d if L else np.zeros(0)
            S_last[b, h] = (ax * wL[:, None]).T @ np.abs(B[b, :, g, :])
    return E1, E2, S_last


def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))
