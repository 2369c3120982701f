"""fp64 CPU oracle of the sparse MoE feed-forward layer (forward pass).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run this module.  The GPU library
never calls it and shares no code with it; the two meet only in the seeded
input generator (``synth``), which holds none of the layer's arithmetic.

What it computes.  The layer is exact (not an approximation), so the oracle
is the plain definition written out step by step in fp64, reading the exact
stored input values (bf16 expanded by placing its 16 bits on top of an fp32
pattern, fp32 promoted).  Sources, all on the page "MoE: how sparse
activation saves compute" unless another page is named:

  * SwiGLU expert F(u) = W_down (SiLU(W_gate u) * W_up u)        -- §3.1, eq. F(u)
  * router scores z = W_route u and softmax p                     -- §3.2, eqs. z, p
  * top-k set S_t, renormalised weights a = p / sum_{S_t} p,
    combine y_t = sum_{i in S_t} a_{t,i} F_i(u_t)                 -- §3.2, eqs. a, y
  * top-1 (Switch) keeps the selected probability as the weight  -- §3.2, last paragraph
  * capacity C = ceil(c T / N), overflow tokens skip the layer    -- §3.5, eq. C
  * for k > 1 capacity counts dispatches (k T)                   -- §3.5, second paragraph
  * shapes [T,d] -> [T,N] -> [T,k] -> per expert [L_i,d]         -- §3.6
  * f_i, P_i and L_aux = alpha N sum f_i P_i                      -- §3.4, eqs. f, P, L_aux
  * overflow and empty-slot ledgers                               -- §3.8
  * parameter ledger P_all = N 3dh, P_active = k 3dh              -- §3.3
  * dense all-experts reference (every expert evaluated, weight 0
    where unselected)                                             -- appendix, moe_lab.py main()
  * LatentMoE: d->l projection, routed experts at width l, RMSNorm
    after aggregation and before the l->d projection, shared
    experts at width d, SiTU-GLU soft caps on both GLU factors    -- page "Stable LatentMoE
                                                                     interactive demo", the
                                                                     width-separation, RMSNorm
                                                                     and SiTU-GLU passages

Readings where the pages are silent (listed again in the design doc):
  * ties in top-k go to the lower expert index; slots are ordered by
    descending p;
  * capacity ranks are in token order (the first C tokens that reach an
    expert are kept), the order in which the appendix code's
    ``torch.where(top_idx == e)`` lists them;
  * a dropped slot contributes 0 and the remaining weights are not
    renormalised;
  * f_i is the argmax indicator of §3.4's formula, taken before capacity;
  * SiTU-GLU(g, v) = SiLU(beta_g tanh(g / beta_g)) * beta_u tanh(v / beta_u);
  * RMSNorm(r) = r / sqrt(mean(r^2) + eps), no learned gain;
  * LatentMoE routes on the full-width u, adds shared experts with weight 1;
  * Quantile Balancing: score = router logit z, selection on z + b with the
    combine weights from the unbiased p, a_t = k-th largest z_t + b,
    q = round(k T / N), histogram of 256 bins over [min, max] of required;
  * FP8 expert weights: OCP E4M3 codes (the format whose largest value, 448,
    the SiTU-GLU passage quotes) with one fp32 scale per weight row; a
    stored row is its scale times each code's exact value;
  * MXFP4 expert weights (the MCU page stores 4-bit experts): OCP MX FP4,
    E2M1 elements in runs of 32 along a row sharing one E8M0 scale, two
    elements a byte with the even element in the low nibble;
  * router backward: the selected sets, the expert outputs and f are held
    fixed (piecewise-constant or separate steps); the loss is
    <dy, y> + aux_scale * L_aux;
  * LatentMoE backward: the same loss and the same fixed quantities; the
    router's part takes dr (the gradient at the aggregated r) in place of
    dy.

Pins (tests/test_oracle_pins.py): the capacity example [10,3,2,1] -> drops
6/4/0; the balanced/collapsed aux example (1.0000 / 2.8449); the parameter
ledger; the seed-7 routing loads [8,7,8,9]; sparse == dense brute force;
N=1 reduces to a torch.nn.functional SwiGLU; softmax/top-k against torch;
dispatch order against torch.where; RMSNorm against torch's rms_norm;
latent limits (beta -> inf gives SwiGLU; identity projections give
RMSNorm(plain); scale invariance); the 12.4% latent parameter saving.
Quantile Balancing pins: after the exact update every expert admits exactly
q tokens under the fixed cutoffs; a constant shift of b shifts b' by the same
constant; the histogram estimate lies within one bin of the exact value; a
hand-worked 4-token example; b = 0 reproduces the unbiased routing.
FP8 pins: all 256 E4M3 codes decode as torch.float8_e4m3fn does, with the
format's landmarks (448, 2^-9, 2^-6, -0, NaN) and a hand-expanded scaled
matrix.  MXFP4 pins: E8M0 against torch.float8_e8m0fnu; every E2M1 value
against torch's decode of the E4M3 code with the same sign, exponent and
mantissa (E2M1 is a subset of E4M3); a hand-expanded two-block matrix.
Router backward pins: torch autograd of an independently written forward;
central differences of the oracle's own loss; the softmax gradient sums to
zero per token; a balanced f makes the aux gradient vanish; renorm with
k = N equals the prob gate.  Experts backward pins: torch autograd of an
independently written SwiGLU / SiTU-GLU layer (capacity drops included).
LatentMoE backward pins: torch autograd of an independently written latent
layer (routing, capacity, SiTU-GLU, RMSNorm, shared experts, aux term);
unselected experts get exactly zero gradient (the demo's own check); the
RMSNorm backward against torch's rms_norm under autograd and, with eps = 0,
orthogonal to r (the norm is scale-free).
Parity unpinned: the exact SiTU-GLU form, the LatentMoE wiring and the
Quantile Balancing readings (score, cutoff, q, bins) are readings, pinned
only through the limits and invariants above.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# Stored values -> fp64 (exact)
# ---------------------------------------------------------------------------


def e4m3_value(code: int) -> float:
    """Exact value of one OCP FP8 E4M3 code: bit 7 sign, bits 6..3 the
    exponent with bias 7, bits 2..0 the mantissa.  Exponent field 0 holds the
    subnormals m * 2^-9; S.1111.111 is NaN; there are no infinities."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e2m1_value(code: int) -> float:
    """Exact value of one OCP FP4 E2M1 code (4 bits): bit 3 sign, bits 2..1
    the exponent with bias 1, bit 0 the mantissa; exponent field 0 holds the
    subnormal m * 0.5.  No infinities or NaN."""
    sign = -1.0 if code & 0x8 else 1.0
    e, m = (code >> 1) & 0x3, code & 0x1
    if e == 0:
        return sign * m * 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e8m0_value(code: int) -> float:
    """Exact value of one OCP E8M0 scale byte: 2^(code - 127); 0xFF is NaN."""
    return math.nan if code == 0xFF else 2.0 ** (code - 127)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def expand(stored) -> np.ndarray:
    """Exact fp64 value of stored bf16 bit patterns (uint16), fp32 values, or
    an FP8 row-scaled matrix (an object with ``codes`` [..., rows, cols] uint8
    and ``scale`` [..., rows] fp32): element (r, c) = scale[r] * E4M3(code)."""
    if hasattr(stored, "packed") and hasattr(stored, "block_scale"):
        # OCP MXFP4: element 2i of a row in the low nibble of byte i, each run
        # of 32 elements times its E8M0 scale.
        packed = np.asarray(stored.packed)
        assert packed.dtype == np.uint8
        codes = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(
            packed.shape[:-1] + (packed.shape[-1] * 2,))
        vals = E2M1_TABLE[codes]
        sc = E8M0_TABLE[np.asarray(stored.block_scale)]
        assert sc.shape[-1] * 32 == vals.shape[-1]
        return (vals.reshape(vals.shape[:-1] + (-1, 32)) * sc[..., None]).reshape(vals.shape)
    if hasattr(stored, "codes") and hasattr(stored, "scale"):
        codes = np.asarray(stored.codes)
        scale = np.asarray(stored.scale, dtype=np.float32).astype(np.float64)
        assert codes.dtype == np.uint8 and scale.shape == codes.shape[:-1]
        return scale[..., None] * E4M3_TABLE[codes]
    a = np.asarray(stored)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {a.dtype}")


# ---------------------------------------------------------------------------
# Router: scores, softmax, top-k, gate weights  (§3.2)
# ---------------------------------------------------------------------------


def router_logits(u: np.ndarray, w_route: np.ndarray) -> np.ndarray:
    """z[t, i] = (W_route u_t)_i; u [T, d], W_route [N, d]."""
    return u @ w_route.T


def softmax(z: np.ndarray) -> np.ndarray:
    """Row-wise softmax; the row max is subtracted before exponentiating."""
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=1, keepdims=True)


def select_topk(p: np.ndarray, k: int) -> np.ndarray:
    """S_t: the k experts of largest p, by descending p, ties to the lower index."""
    order = np.argsort(-p, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def topk_margin(z: np.ndarray, k: int) -> np.ndarray:
    """z_(k) - z_(k+1) per token (descending order statistics); +inf when k = N."""
    N = z.shape[1]
    if k >= N:
        return np.full(z.shape[0], np.inf)
    zs = -np.sort(-z, axis=1)
    return zs[:, k - 1] - zs[:, k]


def gate_weights(p: np.ndarray, idx: np.ndarray, gate: str) -> np.ndarray:
    """Combine weights of the selected experts.

    renorm: a = p / sum_{j in S_t} p_j (Mixtral-style, §3.2 eq. a);
    prob:   a = p (Switch top-1 keeps the selected probability, §3.2).
    """
    psel = np.take_along_axis(p, idx, axis=1)
    if gate == "renorm":
        return psel / psel.sum(axis=1, keepdims=True)
    if gate == "prob":
        return psel
    raise ValueError(gate)


def route(u: np.ndarray, w_route: np.ndarray, k: int, gate: str,
          bias: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Router.  With a selection bias b (Quantile Balancing, page "Stable
    LatentMoE interactive demo", QB passage) the k experts are the largest
    z_t + b, while the combine weights still come from the unbiased p."""
    z = router_logits(u, w_route)
    p = softmax(z)
    if bias is None:
        idx = select_topk(p, k)
        margin = topk_margin(z, k)
    else:
        sb = z + np.asarray(bias, dtype=np.float64)[None, :]
        idx = select_topk(sb, k)
        margin = topk_margin(sb, k)
    return {"z": z, "p": p, "idx": idx, "a": gate_weights(p, idx, gate), "margin": margin}


# ---------------------------------------------------------------------------
# Router backward  (page "MoE: how sparse activation saves compute", §3.2
# eqs. z, p, a, y and §3.4 eq. L_aux, differentiated)
# ---------------------------------------------------------------------------
#
# For a total loss L = <dy, y> + aux_scale * L_aux, with the selected set S_t
# and the expert outputs F_i(x_t) held fixed (the selection is piecewise
# constant in z and the experts' own gradients are a separate step), and f
# held fixed (an arg-max count), the router's share of the gradient is:
#   da_{t,s} = dy_t . F_{i_s}(x_t) for kept slots, 0 for dropped ones;
#   renorm gate a_s = p_s / sum_S p: dp_j = (da_j - sum_s da_s a_s) / sum_S p
#   for j in S_t (0 elsewhere); prob gate a = p: dp_j = da_j;
#   L_aux = alpha N sum_i f_i P_i with P_i = mean_t p_{t,i} adds
#   aux_scale * alpha * N * f_i / T to every dp_{t,i};
#   softmax: dz_t = p_t * (dp_t - p_t . dp_t);
#   dW_route = dz^T u and du = dz W_route (the router's part of du).


def route_backward(u: np.ndarray, w_route: np.ndarray, idx: np.ndarray, row_of: np.ndarray,
                   y_rows: np.ndarray, dy: np.ndarray, *, gate: str, f: np.ndarray,
                   alpha: float, aux_scale: float,
                   n_tokens: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Router backward, steps as above.  u [T, d], w_route [N, d], idx [T, k],
    row_of [T*k] (-1 for a dropped slot), y_rows [R, d] the experts' outputs
    of the kept rows, dy [T, d], f [N] the forward's arg-max shares.
    n_tokens: the layer's token count in the aux term's 1/T when u holds only
    some of its tokens (default: all of them)."""
    T, d = u.shape
    N = w_route.shape[0]
    k = idx.shape[1]
    z = router_logits(u, w_route)
    p = softmax(z)
    da = np.zeros((T, k))
    for t in range(T):
        for s in range(k):
            r = int(row_of[t * k + s])
            if r >= 0:
                da[t, s] = float(dy[t] @ y_rows[r])
    psel = np.take_along_axis(p, idx, axis=1)
    if gate == "renorm":
        ssum = psel.sum(axis=1, keepdims=True)
        a = psel / ssum
        g = (da - (da * a).sum(axis=1, keepdims=True)) / ssum
    elif gate == "prob":
        g = da
    else:
        raise ValueError(gate)
    dp = np.zeros((T, N))
    np.put_along_axis(dp, idx, g, axis=1)
    dp = dp + aux_scale * alpha * N * np.asarray(f, dtype=np.float64)[None, :] / (
        T if n_tokens is None else n_tokens)
    dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return {"p": p, "da": da, "dp": dp, "dz": dz, "dW_route": dz.T @ u, "du": dz @ w_route}


def act_backward(act: str, g: np.ndarray, v: np.ndarray, dh: np.ndarray,
                 beta_g: float = 4.0, beta_u: float = 25.0):
    """(dg, dv) for h = act(g, v) given dh.  SwiGLU h = silu(g) v with
    silu'(g) = s(g) (1 + g (1 - s(g))), s the logistic function; SiTU-GLU
    caps both factors first (g' = beta_g tanh(g / beta_g), likewise v), which
    adds the factors 1 - tanh^2."""
    if act == "swiglu":
        sg = 1.0 / (1.0 + np.exp(-g))
        return dh * v * sg * (1.0 + g * (1.0 - sg)), dh * g * sg
    if act == "situ":
        tg, tv = np.tanh(g / beta_g), np.tanh(v / beta_u)
        gc, vc = beta_g * tg, beta_u * tv
        sg = 1.0 / (1.0 + np.exp(-gc))
        dgc = dh * vc * sg * (1.0 + gc * (1.0 - sg))
        dvc = dh * gc * sg
        return dgc * (1.0 - tg * tg), dvc * (1.0 - tv * tv)
    raise ValueError(act)


def experts_backward(x: np.ndarray, disp: Dict[str, np.ndarray], a: np.ndarray,
                     experts: ExpertFn, dy: np.ndarray, *, act: str, k: int,
                     beta_g: float = 4.0, beta_u: float = 25.0) -> Dict[str, np.ndarray]:
    """The experts' share of the gradient of <dy, y>, y_t = sum_kept a_{t,s}
    F_{i_s}(x_t) (page "MoE: how sparse activation saves compute", §3.1 eq.
    F and §3.2 eq. y, differentiated): for each kept row of expert i with
    token t and weight a, dY = a dy_t; with G = W_gate x, U = W_up x,
    H = act(G, U): dH = W_down^T dY, (dG, dU) = act'(G, U) dH,
    dx_t += W_gate^T dG + W_up^T dU, dW_down += dY H^T, dW_gate += dG x^T,
    dW_up += dU x^T.  Experts with no kept row get zero gradients."""
    T, w = x.shape
    N = len(disp["counts"])
    dx = np.zeros((T, w))
    dWg, dWu, dWd = [], [], []
    shapes = None
    for e in range(N):
        lo, kept = int(disp["offsets"][e]), int(disp["kept_counts"][e])
        if kept == 0 and shapes is not None:
            # no kept row: zero gradients (the weights are not needed)
            dWd.append(np.zeros(shapes[2]))
            dWg.append(np.zeros(shapes[0]))
            dWu.append(np.zeros(shapes[1]))
            continue
        wg, wu, wd = _expert64(experts, e)
        shapes = (wg.shape, wu.shape, wd.shape)
        ent = disp["perm"][lo:lo + kept]
        toks, slots = ent // k, ent % k
        xr = x[toks]
        g, v = xr @ wg.T, xr @ wu.T
        hh = make_act(act, beta_g, beta_u)(g, v)
        dY = a[toks, slots][:, None] * dy[toks]
        dh = dY @ wd
        dg, dv = act_backward(act, g, v, dh, beta_g, beta_u)
        np.add.at(dx, toks, dg @ wg + dv @ wu)
        dWd.append(dY.T @ hh)
        dWg.append(dg.T @ xr)
        dWu.append(dv.T @ xr)
    return {"dx": dx, "dW_gate": np.stack(dWg), "dW_up": np.stack(dWu),
            "dW_down": np.stack(dWd)}


# ---------------------------------------------------------------------------
# Quantile Balancing  (page "Stable LatentMoE interactive demo", QB passage)
# ---------------------------------------------------------------------------
#
# With token t's cutoff a_t held fixed, expert j takes token t exactly when
# z_tj + b_j >= a_t, i.e. when b_j >= required_tj = a_t - z_tj.  A bias that
# makes expert j take exactly q tokens is therefore the q-th smallest
# required_tj over the tokens: one step, no learning rate.  Readings (the page
# gives only this outline): the score is the router logit z; a_t is the k-th
# largest z_t + b under the current bias; q = round(k T / N); the histogram
# estimate uses 256 equal bins over each expert's [min, max] of required and
# interpolates linearly inside the bin that holds the q-th value.


def qb_target(T: int, N: int, k: int) -> int:
    """Target tokens per expert, q = round(k T / N), at least 1, at most T."""
    return int(min(T, max(1, int(math.floor(k * T / N + 0.5)))))


def qb_cutoff(z: np.ndarray, bias: np.ndarray, k: int) -> np.ndarray:
    """a_t = the k-th largest of z_t + b (descending order statistic)."""
    sb = z + np.asarray(bias, dtype=np.float64)[None, :]
    return -np.sort(-sb, axis=1)[:, k - 1]


def qb_required(z: np.ndarray, bias: np.ndarray, k: int) -> np.ndarray:
    """required[t, j] = a_t - z[t, j]: the smallest b_j that still admits t."""
    return qb_cutoff(z, bias, k)[:, None] - z


def qb_bias_exact(z: np.ndarray, bias: np.ndarray, k: int, q: int) -> np.ndarray:
    """b'_j = the q-th smallest required[:, j] (1-based q)."""
    req = qb_required(z, bias, k)
    return np.sort(req, axis=0)[q - 1, :]


def qb_bias_histogram(z: np.ndarray, bias: np.ndarray, k: int, q: int,
                      bins: int = 256) -> np.ndarray:
    """Histogram estimate of the q-th smallest required value per expert."""
    req = qb_required(z, bias, k)
    T, N = req.shape
    out = np.empty(N)
    for j in range(N):
        col = req[:, j]
        lo, hi = float(col.min()), float(col.max())
        if hi <= lo:
            out[j] = lo
            continue
        width = (hi - lo) / bins
        b = np.minimum(np.floor((col - lo) / width).astype(np.int64), bins - 1)
        counts = np.bincount(b, minlength=bins)
        cum = np.cumsum(counts)
        m = int(np.searchsorted(cum, q))          # first bin with cum >= q
        before = int(cum[m - 1]) if m > 0 else 0
        out[j] = lo + width * (m + (q - before) / counts[m])
    return out


def qb_loads(z: np.ndarray, bias: np.ndarray, k: int) -> np.ndarray:
    """Tokens each expert receives when routing on z + b (no capacity)."""
    sb = z + np.asarray(bias, dtype=np.float64)[None, :]
    idx = select_topk(sb, k)
    return np.bincount(idx.ravel(), minlength=z.shape[1])


# ---------------------------------------------------------------------------
# Capacity and dispatch  (§3.5, §3.6, §3.8)
# ---------------------------------------------------------------------------


def capacity_from_factor(T: int, N: int, k: int, c: float) -> int:
    """Per-expert slots C = ceil(c * k * T / N) (k dispatches per token)."""
    return int(math.ceil((c * k * T) / N))


def dispatch(idx: np.ndarray, N: int, capacity: Optional[int],
             kept: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Group the (token, slot) dispatches by expert, in token order.

    rank(t, s) counts the earlier tokens that chose the same expert; a dispatch
    is kept iff rank < C.  perm lists entries t*k+s sorted by (expert, token);
    row_of gives each kept entry its row in the expert-sorted kept rows.
    ``kept`` [T, k] may give the kept flags instead (a subset of a larger
    dispatch's tokens: its kept entries are still the first of each expert in
    token order); capacity is then ignored.
    """
    T, k = idx.shape
    C = None if capacity is None or capacity < 0 or kept is not None else int(capacity)
    counts = np.zeros(N, dtype=np.int64)
    rank = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for s in range(k):
            e = int(idx[t, s])
            rank[t, s] = counts[e]
            counts[e] += 1
    if kept is not None:
        kept = np.asarray(kept, dtype=bool).reshape(T, k)
        kept_counts = np.bincount(idx[kept].astype(np.int64), minlength=N)
    else:
        kept_counts = counts if C is None else np.minimum(counts, C)
        kept = np.ones((T, k), dtype=bool) if C is None else rank < C
    offsets = np.concatenate([[0], np.cumsum(counts)])
    kept_offsets = np.concatenate([[0], np.cumsum(kept_counts)])
    perm = np.empty(T * k, dtype=np.int64)
    row_of = np.full(T * k, -1, dtype=np.int64)
    for t in range(T):
        for s in range(k):
            e = int(idx[t, s])
            perm[offsets[e] + rank[t, s]] = t * k + s
            if kept[t, s]:
                row_of[t * k + s] = kept_offsets[e] + rank[t, s]
    out = {"counts": counts, "offsets": offsets, "kept_counts": kept_counts,
           "kept_offsets": kept_offsets, "rank": rank.reshape(-1), "perm": perm,
           "row_of": row_of, "drop": (~kept).reshape(-1).astype(np.uint8)}
    if C is not None:
        out["overflow"] = int(np.maximum(counts - C, 0).sum())
        out["empty_slots"] = int(np.maximum(C - counts, 0).sum())
        out["static_slots"] = N * C
    return out


# ---------------------------------------------------------------------------
# Experts  (§3.1; LatentMoE page for SiTU-GLU)
# ---------------------------------------------------------------------------


def silu(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(g: np.ndarray, v: np.ndarray) -> np.ndarray:
    return silu(g) * v


def situ_glu(g: np.ndarray, v: np.ndarray, beta_g: float, beta_u: float) -> np.ndarray:
    """Soft-capped GLU: both factors pass through beta * tanh(x / beta) first."""
    return silu(beta_g * np.tanh(g / beta_g)) * (beta_u * np.tanh(v / beta_u))


def make_act(act: str, beta_g: float = 4.0, beta_u: float = 25.0) -> Callable:
    if act == "swiglu":
        return swiglu
    if act == "situ":
        return lambda g, v: situ_glu(g, v, beta_g, beta_u)
    raise ValueError(act)


def expert_forward(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                   w_down: np.ndarray, act: Callable) -> np.ndarray:
    """F(x) for rows x [M, w]: W_down act(W_gate x, W_up x); gate/up [h, w], down [w, h]."""
    g = x @ w_gate.T
    v = x @ w_up.T
    return act(g, v) @ w_down.T


def rmsnorm(r: np.ndarray, eps: float) -> np.ndarray:
    """r / sqrt(mean(r^2) + eps), per row, no gain."""
    return r / np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + eps)


# ---------------------------------------------------------------------------
# Statistics  (§3.4, §3.3)
# ---------------------------------------------------------------------------


def balance_stats(p: np.ndarray, alpha: float) -> Dict[str, np.ndarray]:
    """f_i = share of tokens whose argmax is i; P_i = mean p; N sum f P; alpha N sum f P."""
    T, N = p.shape
    f = np.bincount(np.argmax(p, axis=1), minlength=N) / T
    P = p.mean(axis=0)
    s = N * float(np.sum(f * P))
    return {"f": f, "P": P, "n_sum_fP": s, "aux": alpha * s}


def param_ledger(N: int, k: int, d: int, h: int) -> Dict[str, int]:
    """Expert parameters: one SwiGLU expert 3dh, all N 3dh, active per token k 3dh."""
    one = d * h + d * h + h * d
    return {"one": one, "all": N * one, "active": k * one}


def latent_param_saving(d: int, l: int, H: int, E: int) -> float:
    """Share of routed-expert-side parameters saved by running experts at width l
    instead of d, counting the added d->l and l->d projections."""
    full = E * 3 * H * d
    latent = E * 3 * H * l + 2 * d * l
    return 1.0 - latent / full


# ---------------------------------------------------------------------------
# Forward passes
# ---------------------------------------------------------------------------

ExpertFn = Callable[[int], Sequence[np.ndarray]]


def _expert64(experts: ExpertFn, e: int):
    return tuple(expand(w) for w in experts(e))


def combine_routed(x: np.ndarray, r: Dict[str, np.ndarray], disp: Dict[str, np.ndarray],
                   experts: ExpertFn, act: Callable, k: int, out_width: int,
                   tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """y_t = sum over kept slots of a_{t,s} F_{idx[t,s]}(x_t), for the given tokens.

    Only selected (and kept) experts run; each expert is evaluated on the rows
    routed to it.  Rows of tokens outside ``tokens`` are skipped.
    """
    want = None if tokens is None else {int(t): i for i, t in enumerate(tokens)}
    n_out = x.shape[0] if tokens is None else len(tokens)
    y = np.zeros((n_out, out_width))
    N = len(disp["counts"])
    for e in range(N):
        lo = int(disp["offsets"][e])
        kept = int(disp["kept_counts"][e])
        ent = disp["perm"][lo:lo + kept]
        toks = ent // k
        slots = ent % k
        if want is not None:
            sel = np.array([int(t) in want for t in toks], dtype=bool)
            toks, slots = toks[sel], slots[sel]
        if toks.size == 0:
            continue
        wg, wu, wd = _expert64(experts, e)
        xe = x[toks] if want is None else x[[want[int(t)] for t in toks]]
        fe = expert_forward(xe, wg, wu, wd, act)
        a = r["a"][toks, slots]
        dst = toks if want is None else np.array([want[int(t)] for t in toks])
        for j in range(toks.size):   # one dispatch per (token, slot): no collisions
            y[dst[j]] += a[j] * fe[j]
    return y


def combine_rows(y_rows: np.ndarray, row_of: np.ndarray, a: np.ndarray,
                 rms_eps: Optional[float] = None) -> np.ndarray:
    """The combine step on its own: y_t = sum over kept slots s of
    a[t, s] * y_rows[row_of[t*k + s]] (rows of dropped slots are -1 and add
    nothing).  With rms_eps, the latent layer's RMSNorm follows."""
    T, k = a.shape
    y = np.zeros((T, y_rows.shape[1]))
    for t in range(T):
        for s in range(k):
            r = int(row_of[t * k + s])
            if r >= 0:
                y[t] += a[t, s] * y_rows[r]
    return y if rms_eps is None else rmsnorm(y, rms_eps)


def expert_rows(x: np.ndarray, disp: Dict[str, np.ndarray], experts: ExpertFn, act: Callable,
                k: int, rows: Optional[np.ndarray] = None) -> Dict[int, np.ndarray]:
    """F_e(x_t) for kept rows of the expert-sorted layout: row kept_offsets[e] + j
    holds the output of the j-th kept entry of expert e.  Returns {row: vector}
    for the requested rows (all kept rows when None)."""
    N = len(disp["counts"])
    want = None if rows is None else set(int(r) for r in rows)
    out = {}
    for e in range(N):
        lo, kept = int(disp["kept_offsets"][e]), int(disp["kept_counts"][e])
        js = [j for j in range(kept) if want is None or lo + j in want]
        if not js:
            continue
        ent = disp["perm"][int(disp["offsets"][e]) + np.array(js)]
        wg, wu, wd = _expert64(experts, e)
        fe = expert_forward(x[ent // k], wg, wu, wd, act)
        for i, j in enumerate(js):
            out[lo + j] = fe[i]
    return out


def forward(u_st: np.ndarray, w_route_st: np.ndarray, experts: ExpertFn, *, k: int,
            gate: str = "renorm", act: str = "swiglu", capacity: Optional[int] = None,
            beta_g: float = 4.0, beta_u: float = 25.0, alpha: float = 0.01,
            tokens: Optional[np.ndarray] = None,
            u_rows_st: Optional[np.ndarray] = None,
            bias: Optional[np.ndarray] = None) -> Dict[str, object]:
    """Plain MoE layer.  Routing and dispatch over all T tokens (capacity depends
    on every token); outputs y for ``tokens`` (all when None); ``bias`` is an
    optional selection bias (see ``route``).

    u_st [T, d], w_route_st [N, d] stored; experts(e) -> stored (gate [h,d],
    up [h,d], down [d,h]).  ``u_rows_st`` may hold the rows of ``tokens`` when
    u_st is only needed for routing (it is the same data)."""
    u = expand(u_st)
    N = w_route_st.shape[0]
    r = route(u, expand(w_route_st), k, gate, bias)
    disp = dispatch(r["idx"], N, capacity)
    x = u if tokens is None else (expand(u_rows_st) if u_rows_st is not None else u[tokens])
    y = combine_routed(x, r, disp, experts, make_act(act, beta_g, beta_u), k, u.shape[1],
                       tokens)
    return {**r, "disp": disp, "y": y, "stats": balance_stats(r["p"], alpha)}


def forward_dense(u_st: np.ndarray, w_route_st: np.ndarray, experts: ExpertFn, *, k: int,
                  gate: str = "renorm", act: str = "swiglu", capacity: Optional[int] = None,
                  beta_g: float = 4.0, beta_u: float = 25.0,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Brute force: evaluate every expert on every token and weight it by the
    token's (kept) combine weight, 0 where unselected."""
    u = expand(u_st)
    T = u.shape[0]
    N = w_route_st.shape[0]
    r = route(u, expand(w_route_st), k, gate, bias)
    disp = dispatch(r["idx"], N, capacity)
    kept = (1 - disp["drop"].reshape(T, k)).astype(np.float64)
    fn = make_act(act, beta_g, beta_u)
    y = np.zeros_like(u)
    for e in range(N):
        wg, wu, wd = _expert64(experts, e)
        w = np.zeros(T)
        for s in range(k):
            w += (r["idx"][:, s] == e) * r["a"][:, s] * kept[:, s]
        y += w[:, None] * expert_forward(u, wg, wu, wd, fn)
    return y


def latent_forward(u_st: np.ndarray, w_route_st: np.ndarray, experts: ExpertFn,
                   w_ldown_st: np.ndarray, w_lup_st: np.ndarray, shared: ExpertFn,
                   n_shared: int, *, k: int, gate: str = "renorm", act: str = "situ",
                   capacity: Optional[int] = None, beta_g: float = 4.0,
                   beta_u: float = 25.0, rms_eps: float = 1e-6, alpha: float = 0.01,
                   tokens: Optional[np.ndarray] = None,
                   u_rows_st: Optional[np.ndarray] = None,
                   bias: Optional[np.ndarray] = None) -> Dict[str, object]:
    """LatentMoE layer: x_l = W_ldown u; route on u; r = sum a E_i(x_l) at width l;
    y = W_lup RMSNorm(r) + sum_j SwiGLU_j(u) over the shared experts."""
    u = expand(u_st)
    N = w_route_st.shape[0]
    rt = route(u, expand(w_route_st), k, gate, bias)
    disp = dispatch(rt["idx"], N, capacity)
    ux = u if tokens is None else (expand(u_rows_st) if u_rows_st is not None else u[tokens])
    w_ldown = expand(w_ldown_st)
    w_lup = expand(w_lup_st)
    xl = ux @ w_ldown.T
    rsum = combine_routed(xl, rt, disp, experts, make_act(act, beta_g, beta_u), k,
                          w_ldown.shape[0], tokens)
    rn = rmsnorm(rsum, rms_eps)
    y = rn @ w_lup.T
    for j in range(n_shared):
        sg, su, sd = (expand(w) for w in shared(j))
        y = y + expert_forward(ux, sg, su, sd, swiglu)
    return {**rt, "disp": disp, "x_l": xl, "r": rsum, "r_norm": rn, "y": y,
            "stats": balance_stats(rt["p"], alpha)}


# ---------------------------------------------------------------------------
# LatentMoE backward  (page "Stable LatentMoE interactive demo": the layer of
# the width-separation and RMSNorm passages, differentiated; the demo's own
# check is that only the selected experts receive gradient)
# ---------------------------------------------------------------------------
#
# With n = RMSNorm(r) = r / rho, rho = sqrt(mean(r^2) + eps) per token:
#   dn_m/dr_j = delta_mj / rho - r_m r_j / (l rho^3), so
#   dr = (dn - n mean(dn * n)) / rho.
# The rest is the chain rule through y = W_lup n + sum_j S_j(u),
# r = sum_kept a E_i(x_l), x_l = W_ldown u; the router's part comes from
# route_backward with dy replaced by dr and the expert outputs at width l.


def rmsnorm_backward(r: np.ndarray, dn: np.ndarray, eps: float) -> np.ndarray:
    """dr for n = r / sqrt(mean(r^2) + eps) (per row), given dn."""
    rho = np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + eps)
    n = r / rho
    return (dn - n * np.mean(dn * n, axis=-1, keepdims=True)) / rho


def latent_backward(u_st: np.ndarray, w_route_st: np.ndarray, experts: ExpertFn,
                    w_ldown_st: np.ndarray, w_lup_st: np.ndarray, shared: ExpertFn,
                    n_shared: int, dy: np.ndarray, *, k: int, gate: str = "renorm",
                    act: str = "situ", capacity: Optional[int] = None, beta_g: float = 4.0,
                    beta_u: float = 25.0, rms_eps: float = 1e-6, alpha: float = 0.01,
                    aux_scale: float = 0.0) -> Dict[str, object]:
    """Gradient of L = <dy, y> + aux_scale L_aux for the LatentMoE layer of
    latent_forward, with the selected sets, the capacity drops and f held
    fixed.  Returns du, dz, dW_route, dW_ldown, dW_lup, the routed experts'
    dW_gate / dW_up / dW_down [N, ...] (zero for an expert with no kept row),
    the shared experts' dWs_gate / dWs_up / dWs_down, and the intermediates
    x_l, r, dn, dr."""
    u = expand(u_st)
    wr, wld, wlu = expand(w_route_st), expand(w_ldown_st), expand(w_lup_st)
    N = wr.shape[0]
    rt = route(u, wr, k, gate)
    disp = dispatch(rt["idx"], N, capacity)
    xl = u @ wld.T
    fn = make_act(act, beta_g, beta_u)
    rows = expert_rows(xl, disp, experts, fn, k)
    y_rows = np.zeros((int(disp["kept_offsets"][-1]), wld.shape[0]))
    for j, v in rows.items():
        y_rows[j] = v
    r = combine_rows(y_rows, disp["row_of"], rt["a"])
    n = rmsnorm(r, rms_eps)
    dn = dy @ wlu
    dr = rmsnorm_backward(r, dn, rms_eps)
    ex = experts_backward(xl, disp, rt["a"], experts, dr, act=act, k=k, beta_g=beta_g,
                          beta_u=beta_u)
    rb = route_backward(u, wr, rt["idx"], disp["row_of"], y_rows, dr, gate=gate,
                        f=balance_stats(rt["p"], alpha)["f"], alpha=alpha, aux_scale=aux_scale)
    du = rb["du"] + ex["dx"] @ wld
    dWs_g, dWs_u, dWs_d = [], [], []
    for j in range(n_shared):
        sg, su, sd = (expand(w) for w in shared(j))
        g, v = u @ sg.T, u @ su.T
        dg, dv = act_backward("swiglu", g, v, dy @ sd)
        du = du + dg @ sg + dv @ su
        dWs_d.append(dy.T @ swiglu(g, v))
        dWs_g.append(dg.T @ u)
        dWs_u.append(dv.T @ u)
    out = {"du": du, "dz": rb["dz"], "dW_route": rb["dW_route"], "dW_ldown": ex["dx"].T @ u,
           "dW_lup": dy.T @ n, "dW_gate": ex["dW_gate"], "dW_up": ex["dW_up"],
           "dW_down": ex["dW_down"], "x_l": xl, "r": r, "dn": dn, "dr": dr, "dx_l": ex["dx"],
           "route": rt, "disp": disp, "y_rows": y_rows}
    if n_shared:
        out.update(dWs_gate=np.stack(dWs_g), dWs_up=np.stack(dWs_u), dWs_down=np.stack(dWs_d))
    return out


def latent_backward_tokens(u_st: np.ndarray, w_route_st: np.ndarray, experts: ExpertFn,
                           w_ldown_st: np.ndarray, w_lup_st: np.ndarray, shared: ExpertFn,
                           n_shared: int, dy_rows: np.ndarray, tokens: np.ndarray, *, k: int,
                           gate: str = "renorm", act: str = "situ",
                           capacity: Optional[int] = None, beta_g: float = 4.0,
                           beta_u: float = 25.0, rms_eps: float = 1e-6, alpha: float = 0.01,
                           aux_scale: float = 0.0) -> Dict[str, object]:
    """latent_backward's du and dz rows of the given tokens only (dy_rows
    [len(tokens), d] their upstream gradient).  Each token's du and dz depend
    only on its own routing, its own rows and, through f and the capacity
    ranks, on the routing of all tokens, which is computed in full; the
    experts run on the sampled tokens' rows only (renumbered 0..n-1)."""
    u = expand(u_st)
    wr, wld, wlu = expand(w_route_st), expand(w_ldown_st), expand(w_lup_st)
    T, N = u.shape[0], wr.shape[0]
    tokens = np.asarray(tokens, dtype=np.int64)
    rt = route(u, wr, k, gate)
    full = dispatch(rt["idx"], N, capacity)
    f = balance_stats(rt["p"], alpha)["f"]
    idx = rt["idx"][tokens]
    a = rt["a"][tokens]
    kept = full["row_of"].reshape(T, k)[tokens] >= 0
    disp = dispatch(idx, N, None, kept=kept)
    ut = u[tokens]
    xl = ut @ wld.T
    rows = expert_rows(xl, disp, experts, make_act(act, beta_g, beta_u), k)
    y_rows = np.zeros((int(disp["kept_offsets"][-1]), wld.shape[0]))
    for j, v in rows.items():
        y_rows[j] = v
    r = combine_rows(y_rows, disp["row_of"], a)
    dr = rmsnorm_backward(r, dy_rows @ wlu, rms_eps)
    ex = experts_backward(xl, disp, a, experts, dr, act=act, k=k, beta_g=beta_g,
                          beta_u=beta_u)
    rb = route_backward(ut, wr, idx, disp["row_of"], y_rows, dr, gate=gate, f=f, alpha=alpha,
                        aux_scale=aux_scale, n_tokens=T)
    du = rb["du"] + ex["dx"] @ wld
    for j in range(n_shared):
        sg, su, sd = (expand(w) for w in shared(j))
        g, v = ut @ sg.T, ut @ su.T
        dg, dv = act_backward("swiglu", g, v, dy_rows @ sd)
        du = du + dg @ sg + dv @ su
    return {"du": du, "dz": rb["dz"], "dr": dr, "idx": idx, "margin": rt["margin"][tokens]}


def relative_error(y: np.ndarray, y_ref: np.ndarray) -> float:
    """max|y - y_ref| / max|y_ref| over every compared element."""
    den = float(np.max(np.abs(y_ref)))
    num = float(np.max(np.abs(np.asarray(y, dtype=np.float64) - y_ref)))
    return num / den if den > 0 else num
