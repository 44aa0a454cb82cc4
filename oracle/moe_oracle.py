"""CPU oracle of the Stable LatentMoE layer forward pass and its
quantile-balancing (QB) bias update.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP path and imports nothing from it.

Every step is the plain definition written out in numpy, floating point in
fp64 unless stated.  In bf16 mode the values the GPU stores in bf16 are rounded
to bf16 here at the same points (h, z, shared hidden G, expert hidden H, expert
output Y, combined latent y_lat, out); in f32 mode nothing is rounded and the
result is the fp64 value of the layer.

Sources (page title + place on the page):
  [P1] "Pretraining a Mini Kimi K3" (e-book review), capsule 16 (collapse and
       the noaux_tc bias rule), capsule 20 (3 batched expert matmuls),
       capsule 25 (dispatch buffer that silently fell back).
  [P3] Attention->K3 course, Day 28, design survival table (RMSNorm inside
       LatentMoE; 896-choose-16 Stable LatentMoE; AttnRes replaces x+f(x)).
  [P4] "Kimi K3 MoE lightweight replica demo" article: width separation and
       the shared/routed dual path (architecture paragraph); Tab 1 data flow;
       Tab 2 Fig. 2(a)/(b) (QB balance, histogram vs exact quantile);
       Tab 8-10 (QB reroutes only, weight normalisation, delayed update,
       mean centring, frozen at inference).
  [P5] "K3 tops open source" blog, idle-experts section (hot windows raise
       the threshold, cold ones lower it); fourth-waste section (4-bit
       expert weights, 8-bit run-time data).

Readings where the pages are silent (each is listed with its reason in the
design notes): sigmoid scores; router on the d-wide normalised h; SiLU GLU for
all experts; no residual inside the layer; dropless routing; ties in the
biased top-k go to the lower expert index; histogram of the raw score s on
[0,1]; QB target quantile = the (k/E)-upper quantile (every expert's target
load is T*k/E); bias set outright to mean(q) - q_e.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against closed forms, library routines, brute force or invariants.  The
layer-level equation the demo checks against ("Eq. 11" on [P4], Tab 3) is
not reproduced on the pages: parity with it is unpinned.
"""
from __future__ import annotations

from decimal import Decimal, getcontext
from typing import Dict, Optional

import numpy as np

F32 = np.float32

# --------------------------------------------------------------------------
# bf16 rounding (storage precision of the bf16 mode)
# --------------------------------------------------------------------------


def bf16_round(a) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits, ties to even).

    Written from the definition: with a = m * 2**e, 0.5 <= |m| < 1, keep
    rint(m * 2**8) * 2**(e-8).  Exact in fp64 for finite normal-range values
    (the only ones the layer produces).  Returns fp64.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    """Value after a store in the layer's storage dtype."""
    return bf16_round(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# S1: RMSNorm   ([P3] survival table: RMSNorm without mean subtraction;
#                [P4] Tab 5: RMSNorm stability)
# --------------------------------------------------------------------------


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """h = gamma * x / sqrt(mean(x^2) + eps), per token row (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * x / np.sqrt(ms + eps)


def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a) = a / (1 + exp(-a)) in fp64 (SiLU-gated GLU)."""
    return a / (1.0 + np.exp(-a))


def glu(h: np.ndarray, Wg: np.ndarray, Wu: np.ndarray) -> np.ndarray:
    """silu(h Wg^T) * (h Wu^T), the gated hidden of a GLU expert."""
    return silu(h @ np.asarray(Wg, np.float64).T) * (h @ np.asarray(Wu, np.float64).T)


# --------------------------------------------------------------------------
# S3: scores.  The router score is a sigmoid (reading of the noaux_tc rule,
# [P1] capsule 16).  To make routing decisions bit-reproducible from fp32
# logits, the sigmoid is fixed down to each fp32 operation:
#   y = -clamp(l, -30, 30);  n = rint(y * LOG2E)
#   r = (y - n*LN2_HI) - n*LN2_LO            (Cody & Waite argument reduction)
#   p = degree-7 Taylor polynomial of exp(r), Horner, separate mul and add
#   e = p * 2**n;  s = 1 / (1 + e)           (IEEE fp32 divide)
# --------------------------------------------------------------------------


def _sigmoid_constants():
    """Derive the fp32 constants from ln 2 (50 significant digits)."""
    getcontext().prec = 60
    ln2 = Decimal(2).ln()
    log2e = F32(float(1 / ln2))
    # ln 2 truncated to 16 significant bits: n*LN2_HI is exact for |n| < 2**8
    hi = (ln2 * (1 << 16)).to_integral_value(rounding="ROUND_FLOOR") / (1 << 16)
    ln2_hi = F32(float(hi))
    ln2_lo = F32(float(ln2 - hi))
    taylor = [F32(1.0 / float(np.prod(np.arange(1, i + 1, dtype=np.float64)))) for i in range(8)]
    return log2e, ln2_hi, ln2_lo, taylor


LOG2E, LN2_HI, LN2_LO, _TAYLOR = _sigmoid_constants()
LOGIT_CLAMP = F32(30.0)


def sigmoid_r(logits: np.ndarray) -> np.ndarray:
    """Router score s = 1/(1+exp(-l)) with every step an fp32 op (see above)."""
    l = np.asarray(logits, dtype=F32)
    y = -np.minimum(np.maximum(l, -LOGIT_CLAMP), LOGIT_CLAMP)
    n = np.rint(y * LOG2E).astype(F32)
    r = (y - n * LN2_HI) - n * LN2_LO
    p = _TAYLOR[7]
    for i in range(6, -1, -1):
        p = (p * r).astype(F32) + _TAYLOR[i]
    p = p.astype(F32)
    e = np.ldexp(p, n.astype(np.int32)).astype(F32)
    return (F32(1.0) / (F32(1.0) + e)).astype(F32)


# --------------------------------------------------------------------------
# S5-S6: biased top-k and unbiased gates  ([P4] Tab 8-10: the bias reroutes
# only, gate values are the renormalised scores of the chosen experts)
# --------------------------------------------------------------------------


def topk_select(s: np.ndarray, bias: np.ndarray, k: int) -> np.ndarray:
    """idx[T,k]: the k experts with the largest v = s + b (fp32 add), ordered
    by v descending, equal v by expert index ascending."""
    s = np.asarray(s, dtype=F32)
    assert np.all(np.isfinite(s))
    v = (s + np.asarray(bias, dtype=F32)[None, :]).astype(F32)
    e_idx = np.broadcast_to(np.arange(v.shape[1]), v.shape)
    order = np.lexsort((e_idx, -v), axis=1)      # primary: -v asc; then e asc
    return order[:, :k].astype(np.int32)


def gates_from(s: np.ndarray, idx: np.ndarray, routed_scale: float = 1.0) -> np.ndarray:
    """g_j = s_{idx_j} / S * routed_scale, S the fp32 sum of the selected
    scores in slot order (fp32 throughout)."""
    s_sel = np.take_along_axis(np.asarray(s, dtype=F32), idx.astype(np.int64), axis=1)
    S = s_sel[:, 0].copy()
    for j in range(1, s_sel.shape[1]):
        S = (S + s_sel[:, j]).astype(F32)
    g = (s_sel / S[:, None]).astype(F32)
    return (g * F32(routed_scale)).astype(F32)


# --------------------------------------------------------------------------
# S7-S9: counts, offsets and the stable permutation ([P1] capsule 25 dispatch
# buffer; dropless: every (token, slot) pair gets a row)
# --------------------------------------------------------------------------


def permutation(idx: np.ndarray, E: int):
    """Group the (t, j) pairs by expert, keeping (t, j) order inside a group.

    Returns counts[E], offsets[E+1] (exclusive prefix sum), perm_src[T*k]
    (token of each row) and inv[T,k] (row of each (t, j)).
    """
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")          # rows in expert order
    perm_src = (order // k).astype(np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    inv[order] = np.arange(T * k, dtype=np.int32)
    return counts, offsets, perm_src, inv.reshape(T, k)


# --------------------------------------------------------------------------
# S4 + S18: QB histogram and update ([P4] Tab 2 Fig. 2(b) histogram quantile;
# Tab 8-10 delayed, mean-centred, frozen at inference; [P5] hot experts
# raise their threshold)
# --------------------------------------------------------------------------


def bin_scale(B: int, lo: float = 0.0, hi: float = 1.0) -> np.float32:
    """Bins per unit of score, fp32(B / (hi - lo)) with the quotient taken in
    fp64 on the fp32 range ends (exactly B on [0, 1])."""
    return F32(float(B) / (float(F32(hi)) - float(F32(lo))))


def score_bins(s: np.ndarray, B: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """B equal bins over the score range [lo, hi]:
    bin = clamp(floor(fp32(fp32(s - lo) * scale)), 0, B-1), scale from
    ``bin_scale``; scores outside the range land in the end bins.  On [0, 1]
    this is min(B-1, floor(s*B)) with s*B an fp32 product."""
    t = (np.asarray(s, dtype=F32) - F32(lo)).astype(F32)
    sb = (t * bin_scale(B, lo, hi)).astype(F32)
    return np.clip(np.floor(sb).astype(np.int64), 0, B - 1)


def histogram(s: np.ndarray, B: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """hist[E,B] (int64): per expert, the number of tokens whose score falls
    in each of B equal bins of [lo, hi] (end bins also take what lies beyond)."""
    T, E = s.shape
    bins = score_bins(s, B, lo, hi)
    flat = (np.arange(E)[None, :] * B + bins).reshape(-1)
    return np.bincount(flat, minlength=E * B).reshape(E, B).astype(np.int64)


def qb_quantiles(hist: np.ndarray, N: int, k: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """Histogram estimate q_e of the score each expert must exceed to receive
    its target load m = N*k/E.

    Scanning bins from the top, j is the bin with A_j*E < N*k <= (A_j+c_j)*E
    (A_j = count above bin j, integer comparisons); inside it the estimate is
    linear, as a fraction u of the range: u = (j+1)/B - ((N*k - A_j*E) /
    (E*c_j)) / B, and q = lo + (hi - lo) * u (fp64; q = u on [0, 1]).
    """
    E, B = hist.shape
    target = N * k
    lo64, w64 = float(F32(lo)), float(F32(hi)) - float(F32(lo))
    q = np.zeros(E, dtype=np.float64)
    for e in range(E):
        above = 0
        for j in range(B - 1, -1, -1):
            c = int(hist[e, j])
            if above * E < target <= (above + c) * E:
                frac = float(target - above * E) / float(E * c)
                q[e] = lo64 + w64 * ((j + 1) / B - frac / B)
                break
            above += c
        else:                                   # unreachable for N > 0
            raise AssertionError("no quantile bin")
    return q


def qb_bias(q: np.ndarray) -> np.ndarray:
    """b_e = fp32(mu - q_e), mu the fp64 mean of q summed in expert order."""
    mu = 0.0
    for v in q:
        mu += float(v)
    mu = mu / len(q)
    return np.array([mu - float(v) for v in q], dtype=np.float64).astype(F32)


def qb_update(hist: np.ndarray, N: int, k: int, bias: np.ndarray, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """New bias from the accumulated histogram over [lo, hi]; the old bias is
    kept when no token was seen.  The caller applies it to the next forward
    (one step late)."""
    if N == 0:
        return np.asarray(bias, dtype=F32).copy()
    return qb_bias(qb_quantiles(hist, N, k, lo, hi))


def sign_update(load: np.ndarray, bias: np.ndarray, gamma: float) -> np.ndarray:
    """Sign-rule balancer ([P1] capsule 16, the noaux_tc bias rule with
    gamma = 1e-2 there): every expert's bias moves by gamma towards balance,
    b_e <- b_e + gamma * sign(mean load - load_e), in fp32.

    load_e is the number of (token, slot) pairs routed to e since the last
    update and the mean load is sum(load) / E, so the sign is that of
    sum(load) - E * load_e, decided here in exact integers.  A zero sign leaves
    b_e unchanged.  No mean-centring (the page states none for this rule)."""
    n = [int(v) for v in np.asarray(load).reshape(-1)]
    E = len(n)
    total = sum(n)
    g = F32(gamma)
    out = np.asarray(bias, dtype=F32).copy()
    for e in range(E):
        diff = total - E * n[e]
        if diff > 0:
            out[e] = F32(out[e] + g)
        elif diff < 0:
            out[e] = F32(out[e] - g)
    return out


def exact_quantile(s_col: np.ndarray, N: int, k: int, E: int) -> float:
    """Sort-based counterpart of ``qb_quantiles``: the ceil(N*k/E)-th largest
    score of one expert."""
    m = -(-(N * k) // E)
    return float(np.sort(np.asarray(s_col, dtype=np.float64))[::-1][m - 1])


# --------------------------------------------------------------------------
# The whole layer
# --------------------------------------------------------------------------


# --------------------------------------------------------------------------
# Low-precision experts (the "next" step of FP8 activations and weights):
# OCP microscaling MXFP8 -- blocks of 32 consecutive elements along the
# contraction axis share one power-of-two scale (E8M0 byte), each element is
# an FP8 E4M3 value (bias 7, 3 mantissa bits, largest 448, no infinities).
# --------------------------------------------------------------------------
MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8            # exponent of the largest E4M3 binade (448 = 1.75 * 2^8)


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value (ties to even), saturating at +-448 (fp64 out).

    Normal binade 2^e (e >= -6) has step 2^(e-3); below 2^-6 the
    subnormal step is 2^-9."""
    v = np.asarray(v, dtype=np.float64)
    _, E = np.frexp(v)                       # |v| = m 2^E, 0.5 <= m < 1, so e = E - 1
    step = np.ldexp(1.0, np.maximum(E - 1, -6) - 3)
    q = np.rint(v / step) * step
    return np.clip(q, -E4M3_MAX, E4M3_MAX)


def mx_scale_bytes(a: np.ndarray) -> np.ndarray:
    """E8M0 scale byte of each block of 32 along the last axis:
    2^(floor(log2 amax) - 8) stored as its biased exponent (bias 127),
    clamped to [0, 254]; an all-zero block gets byte 0."""
    a = np.asarray(a, dtype=np.float64)
    blocks = a.reshape(a.shape[:-1] + (a.shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, E = np.frexp(amax)
    b = np.clip(E - 1 - E4M3_EMAX + 127, 0, 254)
    return np.where(amax > 0, b, 0).astype(np.int64)


def mx_quantize(a: np.ndarray):
    """(elements as E4M3 values, scale bytes) of `a` in MXFP8 along the last
    axis (its length a multiple of 32): element = e4m3_round(a / 2^(byte - 127))."""
    a = np.asarray(a, dtype=np.float64)
    sb = mx_scale_bytes(a)
    scale = np.repeat(np.ldexp(1.0, sb - 127), MX_BLOCK, axis=-1)
    return e4m3_round(a / scale), sb


def mx_round(a: np.ndarray) -> np.ndarray:
    """The value an MXFP8 round trip gives: element * scale (fp64)."""
    q, sb = mx_quantize(a)
    return q * np.repeat(np.ldexp(1.0, sb - 127), MX_BLOCK, axis=-1)


# 4-bit expert weights with 8-bit activations ([P5] "K3 tops open source"
# blog, fourth-waste section: expert weights held in 4 bits and the data
# flowing at run time in 8 bits during quantisation-aware training; the
# format is not named -- reading: OCP MXFP4 weights, E2M1 elements (1 sign,
# 2 exponent bits of bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6)
# under the same E8M0 block scale per 32 along K, against MXFP8 activations).
E2M1_MAX = 6.0
E2M1_EMAX = 2            # exponent of the largest E2M1 binade (6 = 1.5 * 2^2)


def e2m1_round(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 value (ties to even), saturating at +-6 (fp64 out).

    Binade 2^e (e >= 0) has step 2^(e-1); below 1 the subnormal step is 1/2."""
    v = np.asarray(v, dtype=np.float64)
    _, E = np.frexp(v)
    step = np.ldexp(1.0, np.maximum(E - 1, 0) - 1)
    q = np.rint(v / step) * step
    return np.clip(q, -E2M1_MAX, E2M1_MAX)


def mx4_scale_bytes(a: np.ndarray) -> np.ndarray:
    """E8M0 scale byte of each block of 32 along the last axis for MXFP4:
    2^(floor(log2 amax) - 2), biased by 127, clamped to [0, 254]; an
    all-zero block gets byte 0."""
    a = np.asarray(a, dtype=np.float64)
    blocks = a.reshape(a.shape[:-1] + (a.shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, E = np.frexp(amax)
    b = np.clip(E - 1 - E2M1_EMAX + 127, 0, 254)
    return np.where(amax > 0, b, 0).astype(np.int64)


def mx4_quantize(a: np.ndarray):
    """(elements as E2M1 values, scale bytes) of `a` in MXFP4 along the last
    axis: element = e2m1_round(a / 2^(byte - 127))."""
    a = np.asarray(a, dtype=np.float64)
    sb = mx4_scale_bytes(a)
    scale = np.repeat(np.ldexp(1.0, sb - 127), MX_BLOCK, axis=-1)
    return e2m1_round(a / scale), sb


def mx4_round(a: np.ndarray) -> np.ndarray:
    """The value an MXFP4 round trip gives: element * scale (fp64)."""
    q, sb = mx4_quantize(a)
    return q * np.repeat(np.ldexp(1.0, sb - 127), MX_BLOCK, axis=-1)


def _expert_rounding(experts: str):
    """(activation rounding, weight rounding) of an expert format; None for
    bf16 experts."""
    if experts == "mxfp8":
        return mx_round, mx_round
    if experts == "mxfp4":
        return mx_round, mx4_round
    if experts != "bf16":
        raise ValueError(f"unknown expert format {experts}")
    return None, None


def router_logits(h: np.ndarray, W_r: np.ndarray, c: Optional[np.ndarray] = None) -> np.ndarray:
    """l = h W_r^T (+ c) in fp64, stored as fp32 ([P4] Tab 1 routing branch)."""
    l = h @ np.asarray(W_r, np.float64).T
    if c is not None:
        l = l + np.asarray(c, np.float64)[None, :]
    return l.astype(F32)


def expert_outputs(X: np.ndarray, offsets: np.ndarray, W: Dict[str, np.ndarray], dtype: str,
                   experts: str = "bf16"):
    """Per expert e on its rows X[off_e:off_e+1]: H = silu(X Wg^T) * (X Wu^T),
    Y = H Wd^T  ([P1] capsule 20: three batched matmuls per expert group).

    experts="mxfp8": both operands of each product are MXFP8 along their
    contraction axis (X and W_g, W_u along l; H, stored first, and W_d along
    f); experts="mxfp4": the weights are MXFP4 instead (activations still
    MXFP8).  The products and sums are exact (fp64) on the rounded values."""
    ra, rw = _expert_rounding(experts)
    mx = ra is not None
    if mx:
        X = ra(X)
    E = len(offsets) - 1
    f = W["W_g"].shape[1]
    lat = W["W_d"].shape[1]
    H = np.zeros((X.shape[0], f), dtype=np.float64)
    Y = np.zeros((X.shape[0], lat), dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        Wg, Wu, Wd = W["W_g"][e], W["W_u"][e], W["W_d"][e]
        if mx:
            Wg, Wu, Wd = rw(Wg), rw(Wu), rw(Wd)
        He = _store(glu(X[a:b], Wg, Wu), dtype)
        H[a:b] = He
        Y[a:b] = _store((ra(He) if mx else He) @ np.asarray(Wd, np.float64).T, dtype)
    return H, Y


def forward(x: np.ndarray, W: Dict[str, np.ndarray], bias: np.ndarray, *, k: int, dtype: str,
            eps: float = 1e-6, B: int = 256, routed_scale: float = 1.0,
            logits: Optional[np.ndarray] = None, with_hist: bool = True,
            experts: str = "bf16", qb_lo: float = 0.0, qb_hi: float = 1.0) -> Dict[str, np.ndarray]:
    """One training (or frozen) forward of the layer on x[T,d].

    ``logits`` (fp32 [T,E]) replaces the router output when given, so that the
    routing decisions can be checked bit for bit against a given set of
    logits; everything else is computed here.

    Returns every intermediate: h, logits, s, idx, gates, counts, offsets,
    perm_src, inv, z, G, H, Y, y_lat, sh, y_r, out, and hist (if with_hist).
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    E = W["W_r"].shape[0]
    r: Dict[str, np.ndarray] = {}
    h = _store(rmsnorm(x, W["gamma"], eps), dtype)                    # S1
    r["h"] = h
    lg = router_logits(h, W["W_r"], W.get("c")) if logits is None else np.asarray(logits, F32)
    r["logits"] = lg                                                   # S2
    s = sigmoid_r(lg)                                                  # S3
    r["s"] = s
    if with_hist:
        r["hist"] = histogram(s, B, qb_lo, qb_hi)                      # S4
    idx = topk_select(s, bias, k)                                      # S5
    g = gates_from(s, idx, routed_scale)                               # S6
    r["idx"], r["gates"] = idx, g
    counts, offsets, perm_src, inv = permutation(idx, E)               # S7-S9
    r.update(counts=counts, offsets=offsets, perm_src=perm_src, inv=inv)
    if W.get("W_sg") is not None and W["W_sg"].shape[0] > 0:           # S10
        G = _store(glu(h, W["W_sg"], W["W_su"]), dtype)
        sh = G @ np.asarray(W["W_sd"], np.float64).T
    else:
        G = np.zeros((T, 0))
        sh = np.zeros((T, x.shape[1]))
    r["G"], r["sh"] = G, sh
    z = _store(h @ np.asarray(W["W_dn"], np.float64).T, dtype)        # S11
    r["z"] = z
    X = z[perm_src]                                                    # S12
    H, Y = expert_outputs(X, offsets, W, dtype, experts)               # S13-S14
    r["H"], r["Y"] = H, Y
    y_lat = np.zeros((T, z.shape[1]), dtype=np.float64)                # S15
    for j in range(k):
        y_lat += g[:, j].astype(np.float64)[:, None] * Y[inv[:, j]]
    y_lat = _store(y_lat, dtype)
    r["y_lat"] = y_lat
    y_r = y_lat @ np.asarray(W["W_up"], np.float64).T                 # S16
    r["y_r"] = y_r
    r["out"] = _store(sh + y_r, dtype)                                 # S17
    return r


def forward_tokens(x_rows: np.ndarray, W: Dict[str, np.ndarray], idx_rows: np.ndarray,
                   gates_rows: np.ndarray, *, dtype: str, eps: float = 1e-6, experts: str = "bf16") -> np.ndarray:
    """Layer output for a few tokens given their routing (idx, gates).

    Every token is independent of the others once its routing is fixed, so
    this evaluates, per token, the same rounding points as ``forward`` without
    any permutation: out = sh(h) + W_up bf(sum_j g_j bf(W_d[e_j] bf(GLU_e_j(z)))).
    Used to check outputs of large batches on sampled tokens.
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    h = _store(rmsnorm(x_rows, W["gamma"], eps), dtype)
    z = _store(h @ np.asarray(W["W_dn"], np.float64).T, dtype)
    out = np.zeros_like(x_rows)
    ra, rw = _expert_rounding(experts)
    mx = ra is not None
    for t in range(x_rows.shape[0]):
        y_lat = np.zeros(z.shape[1])
        zt = ra(z[t:t + 1]) if mx else z[t:t + 1]
        for j in range(idx_rows.shape[1]):
            e = int(idx_rows[t, j])
            Wg, Wu, Wd = W["W_g"][e], W["W_u"][e], W["W_d"][e]
            if mx:
                Wg, Wu, Wd = rw(Wg), rw(Wu), rw(Wd)
            He = _store(glu(zt, Wg, Wu), dtype)
            Ye = _store((ra(He) if mx else He) @ np.asarray(Wd, np.float64).T, dtype)
            y_lat += float(gates_rows[t, j]) * Ye[0]
        y_lat = _store(y_lat, dtype)
        y_r = y_lat @ np.asarray(W["W_up"], np.float64).T
        if W["W_sg"].shape[0] > 0:
            G = _store(glu(h[t:t + 1], W["W_sg"], W["W_su"]), dtype)
            sh = (G @ np.asarray(W["W_sd"], np.float64).T)[0]
        else:
            sh = 0.0
        out[t] = _store(sh + y_r, dtype)
    return out


# --------------------------------------------------------------------------
# Backward pass (the "next" step after the forward: the gradients that train
# the layer).  The routing decisions (idx) are piecewise constant in the
# inputs, so gradients flow through the gates, never into the bias b, which
# only reroutes ([P4] Tab 8-10).
# --------------------------------------------------------------------------


def dsilu(a: np.ndarray) -> np.ndarray:
    """d silu(a) / da = sigma(a) (1 + a (1 - sigma(a))) in fp64."""
    sg = 1.0 / (1.0 + np.exp(-a))
    return sg * (1.0 + a * (1.0 - sg))


def glu_backward(P: np.ndarray, Q: np.ndarray, dG: np.ndarray):
    """G = silu(P) * Q:  dP = dG * Q * silu'(P),  dQ = dG * silu(P)."""
    return dG * Q * dsilu(P), dG * silu(P)


def gates_backward(s: np.ndarray, idx: np.ndarray, dg: np.ndarray, routed_scale: float = 1.0) -> np.ndarray:
    """Router-logit gradient dl[T,E] from the gate gradient dg[T,k].

    g_j = c s_j / S with S = sum_i s_i over the selected experts, so
    ds_m = (c / S) dg_m - (1 / S) sum_j dg_j g_j for a selected m, and
    dl_m = ds_m s_m (1 - s_m) (sigmoid).  Unselected experts get 0."""
    s_sel = np.take_along_axis(np.asarray(s, np.float64), idx.astype(np.int64), axis=1)
    S = s_sel.sum(axis=1, keepdims=True)
    g = routed_scale * s_sel / S
    ds = routed_scale * dg / S - (dg * g).sum(axis=1, keepdims=True) / S
    dl = np.zeros(np.asarray(s).shape, dtype=np.float64)
    np.put_along_axis(dl, idx.astype(np.int64), ds * s_sel * (1.0 - s_sel), axis=1)
    return dl


def rmsnorm_backward(x: np.ndarray, gamma: np.ndarray, eps: float, dh: np.ndarray):
    """h = gamma * x * r, r = (mean(x^2) + eps)^-1/2, per row of width d:
    dx = r (gamma dh) - x r^3 sum(gamma dh x) / d;  dgamma = sum_t dh x r."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    u = np.asarray(gamma, np.float64)[None, :] * dh
    dx = r * u - x * r ** 3 * (u * x).sum(axis=1, keepdims=True) / d
    return dx, (dh * x * r).sum(axis=0)


def backward(x: np.ndarray, W: Dict[str, np.ndarray], dout: np.ndarray, fwd: Dict[str, np.ndarray], *,
             dtype: str, eps: float = 1e-6, routed_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Gradients of sum(out * dout) for the forward ``fwd`` (from ``forward``)
    with respect to x and every weight.

    Chain, in the order the values are formed (bf16 mode rounds to bf16 at the
    points the device stores bf16 operands of its products: the recomputed GLU
    pre-activations P, Q, A, U; dG, dy_lat, dP, dQ, dY, dH, dA, dU, dX, dz
    and the router-logit gradient; dh, the weight gradients and dgamma stay
    unrounded):
      out = G W_sd^T + y_lat W_up^T       -> dG, dy_lat, dW_sd, dW_up
      y_lat = sum_j g_j Y[inv_j]          -> dY rows, dg (combine transpose)
      Y_e = H_e W_d[e]^T                  -> dH, dW_d
      H_e = silu(A) U, A = X W_g^T, U = X W_u^T -> dA, dU, dW_g, dW_u, dX
      X = z[perm_src]                     -> dz[t] = sum_j dX[inv_j]
      g = gates(s), s = sigmoid(l)        -> dl (selected experts only)
      G = silu(P) Q, P = h W_sg^T, Q = h W_su^T -> dP, dQ, dW_sg, dW_su
      z = h W_dn^T, l = h W_r^T (+c)      -> dW_dn, dW_r
      dh = dP W_sg + dQ W_su + dz W_dn + dl W_r;  h = RMSNorm(x) -> dx, dgamma
    """
    f64 = lambda a: np.asarray(a, np.float64)  # noqa: E731
    st = lambda a: _store(a, dtype)            # noqa: E731
    x = f64(x)
    dout = st(dout)
    T = x.shape[0]
    k = fwd["idx"].shape[1]
    E = W["W_r"].shape[0]
    h, z, G, H, Y, y_lat = fwd["h"], fwd["z"], fwd["G"], fwd["H"], fwd["Y"], fwd["y_lat"]
    idx, gates, inv, offsets, perm_src = fwd["idx"], fwd["gates"], fwd["inv"], fwd["offsets"], fwd["perm_src"]
    g: Dict[str, np.ndarray] = {}
    shared = W.get("W_sg") is not None and W["W_sg"].shape[0] > 0
    # output projections
    g["W_up"] = dout.T @ y_lat
    dy = st(dout @ f64(W["W_up"]))
    dh = np.zeros_like(h)
    if shared:
        g["W_sd"] = dout.T @ G
        dG = st(dout @ f64(W["W_sd"]))
        P = st(h @ f64(W["W_sg"]).T)
        Q = st(h @ f64(W["W_su"]).T)
        dP, dQ = glu_backward(P, Q, dG)
        dP, dQ = st(dP), st(dQ)
        g["W_sg"] = dP.T @ h
        g["W_su"] = dQ.T @ h
        dh += dP @ f64(W["W_sg"]) + dQ @ f64(W["W_su"])
    # combine transpose
    dY = np.zeros_like(Y)
    dg = np.zeros((T, k))
    for j in range(k):
        rows = inv[:, j]
        dY[rows] = st(f64(gates[:, j])[:, None] * dy)
        dg[:, j] = (dy * Y[rows]).sum(axis=1)
    # experts
    X = z[perm_src]
    dX = np.zeros_like(X)
    g["W_d"] = np.zeros(np.shape(W["W_d"]))
    g["W_g"] = np.zeros(np.shape(W["W_g"]))
    g["W_u"] = np.zeros(np.shape(W["W_u"]))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        g["W_d"][e] = dY[a:b].T @ H[a:b]
        dH = st(dY[a:b] @ f64(W["W_d"][e]))
        A = st(X[a:b] @ f64(W["W_g"][e]).T)
        U = st(X[a:b] @ f64(W["W_u"][e]).T)
        dA, dU = glu_backward(A, U, dH)
        dA, dU = st(dA), st(dU)
        g["W_g"][e] = dA.T @ X[a:b]
        g["W_u"][e] = dU.T @ X[a:b]
        dX[a:b] = st(dA @ f64(W["W_g"][e]) + dU @ f64(W["W_u"][e]))
    # dispatch transpose
    dz = np.zeros_like(z)
    for j in range(k):
        dz += dX[inv[:, j]]
    dz = st(dz)
    g["W_dn"] = dz.T @ h
    dh += dz @ f64(W["W_dn"])
    # router
    dl = st(gates_backward(fwd["s"], idx, dg, routed_scale))
    g["W_r"] = dl.T @ h
    dh += dl @ f64(W["W_r"])
    dx, dgamma = rmsnorm_backward(x, W["gamma"], eps, dh)
    g["x"] = st(dx)
    g["gamma"] = dgamma
    return g


def load_stats(counts: np.ndarray) -> Dict[str, float]:
    """Balance statistics that do not hide dead experts ([P1] capsule 16: the
    router entropy read 0.9999 while 94.5% of experts were dead)."""
    c = np.asarray(counts, dtype=np.float64)
    live = c[c > 0]
    return {
        "max_over_min": float(c.max() / c.min()) if c.min() > 0 else float("inf"),
        "max_over_mean": float(c.max() / c.mean()),
        "dead": int((c == 0).sum()),
        "cv": float(c.std() / c.mean()),
        "min_live": float(live.min()) if live.size else 0.0,
    }
