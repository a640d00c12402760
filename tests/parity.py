"""GPU-vs-oracle comparison rules for the verification step (test helper).

The oracle (oracle/verify.py) is the pages' method in fp64.  The kernels
compute in fp32 (fp64 for the accept test and for combining partial sums), so
a discrete decision may differ only where the oracle's result lies within the
kernels' error of a decision boundary.  The bar:

  * argmax mode (T = 0): n_accepted, next_token, alpha, p_draft and q_draft are
    bit-exact.
  * T > 0, n_accepted: exact, except in sequences where an evaluated accept test
    has |u_i - min(1, p_i(x_i) / (l q_i(x_i)))| < 1e-6 (the oracle's u band, the
    exemption the specification fixes).  Counted.
  * T > 0, next_token: exact, except where the oracle's final uniform lies
    within the derived band (below) of a step of the sampled row's CDF.  In
    those rows a differing token must still be a valid draw: positive weight,
    with the uniform inside its CDF interval widened by the band.  Counted.
  * A rejection whose residual mass is within the derived error of zero may
    also have been sampled from p_n (the kernel found no residual mass, the
    pages' zero-mass reading): the token must then have p_n(t) > 0.  Counted.
  * top-p: a sequence with a row whose nucleus decision lies within the derived
    band of top_p is counted and left out (its kept set may legitimately
    differ by the boundary tie group).
  * alpha, p_draft and q_draft agree within 1e-5 absolute.
  * With per-sequence draft counts, the padding positions are NaN on both sides.

Derived bands.  u = 2^-24 is fp32's unit roundoff and k~ = log2(e)/T as the
kernels hold it (log2(e) rounded to fp32, then divided by T in fp32); its
relative error d_k = |k~ / k - 1| is computed exactly for each case.  For a
token x of a row with maximum logit m, A_x = (m - l_x) log2(e) / T >= 0 is its
distance below the maximum in the base-2 exponent the kernels evaluate.  A
kernel weight relative to the row maximum carries at most these relative
errors:

  ln2 d_k A     the tilt of exp2(l k~) against exp2(l k);
  ln2 u A       the exponent argument rounded (one fused multiply-add on the
                fused path; on the multi-pass path a subtraction that is
                exact for logits within a factor of 2^16 of the maximum, then a
                product);
  2 ln2 u A     the scale factors that carry thread and tile sums to the row
                maximum (a difference of two maxima, rounded, twice);
  12 u          three exp2 evaluations (v_exp_f32, 2 ulp each);
  3 u           three products by those factors;
  18 u          the fp32 sums over a thread (32 terms in 4 chains: 9) and over
                a wave or workgroup (a 6-level tree plus 4 waves: 9).

So weight x is within e_x = ln2 (d_k + 3 u) A_x + 33 u of its value, relative,
and the row's total within E = sum_x p(x) e_x.  The kernel compares the final
uniform with its cumulative weights normalised by its total, so at step j
(the CDF C_j = sum_{x <= j} p(x)) its error is at most

  err_j = sum_{x <= j} p(x) e_x + C_j E + 64 u

(64 u: the in-tile fp32 scan, 8-32 terms a thread, a 6-level wave scan and 4
waves, and theta's remainder rounded to fp32).  The token can only differ from
the oracle's t if the uniform lies within err of one of the two steps that
bracket it, C_{t-1} and C_t (err_j is monotone, so no farther step can cross).

Residual rows max(0, p - l q): per token |w~ - w| <= d_x = p (e^p_x + E_p) +
l q (e^q_x + E_q) where the token can carry residual mass at all (p - l q >
-d_x; elsewhere both sides give exactly 0), and the fused path forms its tile
masses as (a + b - |a - b|) / 2, which adds at most 20 u of the p and q mass
before the step.  So the cumulative residual mass at step j is off by at most
D_j = sum_{x <= j} d_x + 20 u (P_j + l Q_j), and the normalised step by
(D_j + C_j D_V) / S_res + 64 u.  A residual mass S_res <= D_V may have been
computed as empty, and then p_n is sampled (the pages' zero-mass reading):
either reading is valid there.

Nucleus: the row and list threshold kernels weigh tokens by exp2((l - m) k~)
in fp32 (the tilt, the argument rounded twice, exp2 at 2 ulp) and sum the
weights in fp64 or 2^-40 fixed point; the streaming nucleus path weighs them by
exp2(fma(l, k~, -c)) (the argument rounded once, exp2 at 2 ulp) and truncates
each to 24 fractional bits of its octave (at most 2 u) before exact integer
sums.  Both stay within e_x = ln2 (d_k + 2 u) A_x + 4 u over the top-k
survivors, and the normalised masses compared with top_p are off by at most
2 E_nuc.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from oracle import verify as ov

PROB_TOL = 1e-5           # alpha, p_draft, q_draft: absolute
U = 2.0 ** -24
LN2 = 0.6931471805599453
LOG2E = 1.4426950408889634
C_0 = 33.0                # per-token constant error, units of u
SCAN = 64.0 * U           # in-tile fp32 scan and theta's remainder
TILE_FORM = 20.0 * U      # fused tile residual masses from the |a - b| form


def kernel_k(T: float) -> float:
    """log2(e)/T as the kernels hold it (two fp32 roundings)."""
    return float(np.float32(np.float32(LOG2E) / np.float32(T)))


@dataclasses.dataclass
class Report:
    rows: int = 0
    u_band: int = 0
    cdf_band: int = 0                 # sampled rows within the derived band of a CDF step
    token_mismatch_valid: int = 0     # of those, rows whose token differs (validly)
    residual_degenerate: int = 0      # rejections whose residual mass is within its error of zero
    residual_zero: int = 0            # rejections whose residual has no mass at all (p_n is sampled)
    thresholds_differ: int = 0        # sequences with a GPU keep threshold unlike the oracle's
    filter_band: int = 0              # sequences left out: a nucleus decision within its band
    max_band: float = 0.0             # the widest CDF band met (normalised)

    def __str__(self):
        return (f"rows={self.rows} u_band={self.u_band} cdf_band={self.cdf_band} "
                f"mismatched-but-valid={self.token_mismatch_valid} "
                f"residual_degenerate={self.residual_degenerate} residual_zero={self.residual_zero} "
                f"filter_band={self.filter_band} thresholds_differ={self.thresholds_differ} "
                f"max_band={self.max_band:.3g}")


# ------------------------------------------------------------ error model

def _row(case, b: int, r: int):
    """Row r of sequence b as fp64 logits: r <= gamma target rows, then drafts."""
    G = case.gamma
    src = case.target[b, r] if r <= G else case.draft[b, r - G - 1]
    return ov.widen(src, case.dtype)


def adjacent_values(x: np.ndarray, tau: float) -> np.ndarray:
    """The keep thresholds a kernel may return for a row whose nucleus boundary
    lies within the band: the oracle's tau or the row's next distinct finite
    logit above or below it (one tie group kept more or less), as float32."""
    vals = np.unique(np.asarray(x, np.float64)[np.isfinite(x)]).astype(np.float32)
    q = int(np.searchsorted(vals, np.float32(tau)))
    return vals[max(q - 1, 0):q + 2]


def row_errors(x: np.ndarray, T: float, tau: float = -np.inf, nucleus: bool = False):
    """(p, e, E) for a row of fp64 logits: p = softmax(x / T) over the kept
    tokens (x >= tau, zero elsewhere), e the per-token relative error bound of
    the kernels' weights and E = sum p e."""
    keep = (x >= tau) & np.isfinite(x)
    m = x[keep].max()
    A = np.where(keep, (m - np.where(keep, x, m)) * (LOG2E / T), 0.0)
    p = np.where(keep, np.exp((np.where(keep, x, m) - m) / T), 0.0)
    p /= p.sum()
    k_exact = LOG2E / T
    dk = abs(kernel_k(T) / k_exact - 1.0)
    if nucleus:
        e = LN2 * (dk + 2.0 * U) * A + 4.0 * U
    else:
        e = LN2 * (dk + 3.0 * U) * A + C_0 * U
    return p, e, float(np.dot(p, e))


def nucleus_bands(rows: np.ndarray, T: float, top_k: int) -> np.ndarray:
    """2 E_nuc per row of fp64 logits [n, V]: how far the threshold kernels'
    normalised nucleus masses may lie from the oracle's."""
    from oracle import adjust
    out = np.empty(rows.shape[0])
    for r in range(rows.shape[0]):
        _, _, E = row_errors(rows[r], T, adjust.topk_threshold(rows[r], top_k), nucleus=True)
        out[r] = 2.0 * E
    return out


def bonus_step_errors(p, e, E):
    """err_j of every CDF step of a row sampled from p itself."""
    return np.cumsum(p * e) + np.cumsum(p) * E + SCAN


def residual_step_errors(p, ep, Ep, q, eq, Eq, lenience):
    """(normalised err_j, S_res, D_V) of the residual max(0, p - l q)."""
    d = p * (ep + Ep) + lenience * q * (eq + Eq)
    live = (p - lenience * q) > -d
    d = np.where(live, d, 0.0)
    r = np.maximum(p - lenience * q, 0.0)
    D = np.cumsum(d) + TILE_FORM * (np.cumsum(p) + lenience * np.cumsum(q))
    S = float(r.sum())
    DV = float(D[-1])
    if S == 0.0:
        return np.full(p.shape, np.inf), S, DV
    C = np.cumsum(r) / S
    return (D + C * DV) / S + SCAN, S, DV


def step_band(errs, cdf, t: int, u_final: float) -> bool:
    """True when u_final lies within the error of a step bracketing token t."""
    lo = cdf[t - 1] if t > 0 else 0.0
    err_lo = errs[t - 1] if t > 0 else SCAN
    return (u_final - lo) <= err_lo or (cdf[t] - u_final) <= errs[t]


# ------------------------------------------------------------- comparison

def _live_rows(G: int, gb: int):
    """Indices (target rows 0..gamma, then drafts) of the rows a sequence uses."""
    return [j for j in range(2 * G + 1) if (j <= gb if j <= G else j - G - 1 < gb)]


def check(case, gpu: dict, seqs=None, where: str = "", lenience: float = 1.0, gamma_seq=None,
          top_k: int = 0, top_p: float = 1.0, workers: int = 1, res=None, gpu_thresholds=None) -> Report:
    """Compare GPU outputs (numpy dict, full batch) with the oracle on `seqs`.

    lenience, gamma_seq (numpy int [B]), top_k and top_p are passed to the
    oracle unchanged.  `res` may hand in the oracle's result for `seqs` (with
    keep_weights) when the caller already has it.

    gpu_thresholds ([B, 2 gamma + 1] float32: target rows, then draft rows, as
    spec_filter_thresholds returns them) narrows the top-p exemption: a
    sequence is then left out only if one of its GPU thresholds differs from
    the oracle's, and every such row must lie within its nucleus band."""
    if seqs is None:
        seqs = np.arange(case.B)
    seqs = np.asarray(seqs)
    if res is None:
        res = ov.verify_case(case, keep_weights=case.temperature > 0, seqs=seqs, lenience=lenience,
                             gamma_seq=gamma_seq, top_k=top_k, top_p=top_p, workers=workers)
    T = float(np.float32(case.temperature))
    lenience = float(np.float32(lenience))
    G = case.gamma
    gb = np.full(len(seqs), G) if gamma_seq is None else np.asarray(gamma_seq)[seqs]
    rep = Report(rows=len(seqs))
    in_filter_band = np.zeros(len(seqs), bool)
    if res.filter_margins is not None:
        for r in range(len(seqs)):
            for j in _live_rows(G, int(gb[r])):
                mg = res.filter_margins[r, j]
                if np.isfinite(mg) and mg <= nucleus_bands(_row(case, int(seqs[r]), j)[None], T, top_k)[0]:
                    in_filter_band[r] = True
                    break
        rep.filter_band = int(in_filter_band.sum())
        if gpu_thresholds is not None:
            thr = np.asarray(gpu_thresholds)[seqs]
            differs = np.zeros(len(seqs), bool)
            for r in range(len(seqs)):
                for j in _live_rows(G, int(gb[r])):
                    if np.float32(res.filter_tau[r, j]) != thr[r, j]:
                        differs[r] = True
                        assert in_filter_band[r], (f"{where}: keep threshold of row {j} of sequence {seqs[r]} "
                                                   f"differs ({thr[r, j]} vs {res.filter_tau[r, j]}) "
                                                   f"outside the nucleus band")
                        near = adjacent_values(_row(case, int(seqs[r]), j), res.filter_tau[r, j])
                        assert thr[r, j] in near, (f"{where}: keep threshold of row {j} of sequence {seqs[r]} "
                                                   f"is {thr[r, j]}, not the oracle's {res.filter_tau[r, j]} "
                                                   f"or an adjacent logit {near}")
            rep.thresholds_differ = int(differs.sum())
            in_filter_band = differs

    g = {k: np.asarray(v)[seqs] for k, v in gpu.items()}
    if case.temperature == 0.0:
        assert np.array_equal(g["n_accepted"], res.n_accepted), where
        assert np.array_equal(g["next_token"], res.next_token), where
        if G:
            for key, ref in (("alpha", res.alpha), ("p_draft", res.p_draft), ("q_draft", res.q_draft)):
                assert np.array_equal(g[key], ref.astype(np.float32), equal_nan=True), f"{where}: {key}"
        return rep

    band = res.u_band
    rep.u_band = int(band.sum())
    bad_n = (g["n_accepted"] != res.n_accepted) & ~band & ~in_filter_band
    assert not bad_n.any(), (f"{where}: n_accepted differs outside the u band in rows {seqs[bad_n][:10]} "
                             f"(gpu {g['n_accepted'][bad_n][:10]}, oracle {res.n_accepted[bad_n][:10]})")

    tau_rows = res.filter_tau
    for r in range(len(seqs)):
        if in_filter_band[r]:
            continue
        b, n = int(seqs[r]), int(res.n_accepted[r])
        t_gpu = int(g["next_token"][r])
        assert 0 <= t_gpu < case.V, f"{where}: token {t_gpu} out of range in row {b}"
        if g["n_accepted"][r] != n:
            continue                      # a u-band row: a different row was sampled
        t_or = int(res.next_token[r])
        u_final = float(np.float32(case.uniforms[b, gb[r]]))
        tau_p = tau_rows[r, n] if tau_rows is not None else -np.inf
        p, ep, Ep = row_errors(_row(case, b, n), T, tau_p)
        degenerate = False
        if res.residual[r] and res.res_mass[r] > 0.0:
            tau_q = tau_rows[r, G + 1 + n] if tau_rows is not None else -np.inf
            q, eq, Eq = row_errors(_row(case, b, G + 1 + n), T, tau_q)
            errs, S, DV = residual_step_errors(p, ep, Ep, q, eq, Eq, lenience)
            degenerate = S <= DV
            rep.residual_degenerate += int(degenerate)
        else:
            # the bonus row, or a residual with no mass at all: both sides sample
            # p_n (the kernel's computed residual can only be within its error of
            # zero there, so a token from it is also accepted below)
            if res.residual[r]:
                rep.residual_zero += 1
                degenerate = True
            errs = bonus_step_errors(p, ep, Ep)
        w = res.weights[r]
        cdf = np.cumsum(w)
        zero = res.residual[r] and res.res_mass[r] == 0.0
        ambiguous = (degenerate and not zero) or step_band(errs, cdf, t_or, u_final)
        rep.cdf_band += int(ambiguous)
        if not degenerate or zero:
            rep.max_band = max(rep.max_band, float(max(errs[t_or], errs[t_or - 1] if t_or else 0.0)))
        if t_gpu == t_or:
            continue
        assert ambiguous or degenerate, (f"{where}: next_token {t_gpu} != oracle {t_or} in row {b} "
                           f"(margin {res.cdf_margin[r]:.3g}, step errors "
                           f"{errs[t_or - 1] if t_or else 0.0:.3g} / {errs[t_or]:.3g})")
        if degenerate:
            # either reading: the kernel's residual (p~ > l q~ needs p > 0) or p_n itself
            assert p[t_gpu] > 0, f"{where}: token {t_gpu} has p = 0 in row {b}"
        else:
            lo = cdf[t_gpu - 1] if t_gpu > 0 else 0.0
            err_lo = errs[t_gpu - 1] if t_gpu > 0 else SCAN
            assert w[t_gpu] > 0 and lo - err_lo <= u_final < cdf[t_gpu] + errs[t_gpu], \
                f"{where}: invalid token {t_gpu} in row {b} (interval [{lo:.9g}, {cdf[t_gpu]:.9g}), u {u_final:.9g})"
        rep.token_mismatch_valid += 1

    if G:
        keep = ~in_filter_band
        for key, ref in (("alpha", res.alpha), ("p_draft", res.p_draft), ("q_draft", res.q_draft)):
            pad = np.isnan(ref)
            assert np.array_equal(np.isnan(g[key]), pad), f"{where}: {key} padding positions differ"
            err = np.abs(g[key].astype(np.float64) - ref)[~pad & keep[:, None]]
            assert err.size == 0 or np.all(err <= PROB_TOL), f"{where}: {key} max error {err.max():.3g}"
    return rep


def oracle_bands(case, seqs=None, lenience: float = 1.0, gamma_seq=None, top_k: int = 0, top_p: float = 1.0,
                 workers: int = 1) -> Report:
    """The band counts of a case from the oracle alone (no GPU): the oracle's
    own outputs stand in for the GPU's, so every token matches and only the
    counts remain."""
    idx = np.arange(case.B) if seqs is None else np.asarray(seqs)
    res = ov.verify_case(case, keep_weights=case.temperature > 0, seqs=idx, lenience=lenience,
                         gamma_seq=gamma_seq, top_k=top_k, top_p=top_p, workers=workers)
    gpu = {}
    for key in ("n_accepted", "next_token", "alpha", "p_draft", "q_draft"):
        val = getattr(res, key)
        full = np.zeros((case.B,) + val.shape[1:], val.dtype)
        full[idx] = val
        gpu[key] = full.astype(np.float32) if key in ("alpha", "p_draft", "q_draft") else full
    return check(case, gpu, seqs=idx, where="oracle", lenience=lenience, gamma_seq=gamma_seq, top_k=top_k,
                 top_p=top_p, res=res)
