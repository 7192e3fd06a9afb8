"""Independent numpy fp64 evaluators used to pin the oracle (not the oracle itself).

Both unroll Eq. (1) of the Video-Ma2mba review (pith.science verdict for arXiv
2411.19460, skeptic critique), h_t = exp(dt_t A) h_{t-1} + dt_t B_t x_t^T,
y_t = C_t^T h_t + D x_t, in closed form instead of stepping it:

  quadratic(...)  the matrix ("dual") form of the structured-state-space-duality
                  paper cited on the arXiv index page: y = (L o C B^T) (dt x)
                  + exp(cum) C h0^T + D x, with L[t, s] = exp(sum_{r=s+1..t} l_r)
                  for s <= t, O(L^2).
  chunked(...)    the same sum split into chunks of Q steps: an intra-chunk
                  quadratic term, a carried-state term exp(cs_t) C_t H_{c-1}^T, the
                  chunk state S_c and the inter-chunk recurrence
                  H_c = exp(cs_end) H_{c-1} + S_c.  Q=1 is the recurrence, Q=L the
                  quadratic form.
"""
import numpy as np


def softplus(u):
    return np.logaddexp(0.0, u)


def silu(u):
    return u / (1.0 + np.exp(-u))


def _dt(dt_raw, dt_bias, use_softplus):
    u = dt_raw + (0.0 if dt_bias is None else dt_bias[None, None, :])
    return softplus(u) if use_softplus else u


def quadratic(x, dt_raw, A, Bm, Cm, dt_bias=None, use_softplus=True, D=None, z=None, h0=None):
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dt = _dt(dt_raw, dt_bias, use_softplus)
    y = np.zeros((Bsz, L, H, P))
    hf = np.zeros((Bsz, H, P, N))
    mask = np.tril(np.ones((L, L), dtype=bool))
    for b in range(Bsz):
        for h in range(H):
            g = h // (H // G)
            l = dt[b, :, h] * A[h]
            cum = np.cumsum(l)
            seg = cum[:, None] - cum[None, :]
            Ldec = np.where(mask, np.exp(np.where(mask, seg, 0.0)), 0.0)
            CB = Cm[b, :, g, :] @ Bm[b, :, g, :].T
            X = x[b, :, h, :] * dt[b, :, h][:, None]
            Y = (CB * Ldec) @ X
            if h0 is not None:
                Y += np.exp(cum)[:, None] * (Cm[b, :, g, :] @ h0[b, h].T)
            if D is not None:
                Y += D[h] * x[b, :, h, :]
            y[b, :, h, :] = Y
            w = np.exp(cum[-1] - cum) * dt[b, :, h]
            S = (x[b, :, h, :] * w[:, None]).T @ Bm[b, :, g, :]
            hf[b, h] = S + (np.exp(cum[-1]) * h0[b, h] if h0 is not None else 0.0)
    out = y * silu(z) if z is not None else y
    return out, y, hf


def chunked(x, dt_raw, A, Bm, Cm, Q, dt_bias=None, use_softplus=True, D=None, z=None, h0=None):
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dt = _dt(dt_raw, dt_bias, use_softplus)
    y = np.zeros((Bsz, L, H, P))
    hf = np.zeros((Bsz, H, P, N))
    for b in range(Bsz):
        for h in range(H):
            g = h // (H // G)
            Hs = np.zeros((P, N)) if h0 is None else h0[b, h].copy()
            for c0 in range(0, L, Q):
                c1 = min(L, c0 + Q)
                n = c1 - c0
                l = dt[b, c0:c1, h] * A[h]
                cs = np.cumsum(l)                                   # chunk-local cumsum
                mask = np.tril(np.ones((n, n), dtype=bool))
                Ldec = np.where(mask, np.exp(np.where(mask, cs[:, None] - cs[None, :], 0.0)), 0.0)
                C = Cm[b, c0:c1, g, :]
                Bc = Bm[b, c0:c1, g, :]
                X = x[b, c0:c1, h, :]
                dts = dt[b, c0:c1, h]
                Ydiag = ((C @ Bc.T) * Ldec) @ (X * dts[:, None])
                Yoff = np.exp(cs)[:, None] * (C @ Hs.T)
                Yc = Ydiag + Yoff
                if D is not None:
                    Yc = Yc + D[h] * X
                y[b, c0:c1, h, :] = Yc
                w = np.exp(cs[-1] - cs) * dts
                Sc = (X * w[:, None]).T @ Bc
                Hs = np.exp(cs[-1]) * Hs + Sc
            hf[b, h] = Hs
    out = y * silu(z) if z is not None else y
    return out, y, hf


def conv_np(xraw, w, bias, state_in, use_silu=True):
    """Causal depthwise conv via numpy.convolve per channel (kernel flipped:
    the layer is a cross-correlation whose last tap multiplies the current token)."""
    Bsz, L, Cd = xraw.shape
    K = w.shape[1]
    out = np.zeros((Bsz, L, Cd))
    for b in range(Bsz):
        full = np.concatenate([state_in[b] if state_in is not None else np.zeros((K - 1, Cd)),
                               xraw[b]], axis=0)
        for c in range(Cd):
            out[b, :, c] = np.convolve(full[:, c], w[c, ::-1], mode="valid")
    if bias is not None:
        out += bias[None, None, :]
    return silu(out) if use_silu else out
