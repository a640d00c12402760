"""GPU-vs-oracle comparison rules for the verification step (test helper).

The bar:
  * argmax mode (T = 0): n_accepted, next_token, alpha, p_draft and q_draft are
    bit-exact.
  * T > 0: n_accepted is exact except in rows where an evaluated accept test
    has |u_i - min(1, p_i(x_i)/q_i(x_i))| < U_BAND (1e-6, from the oracle's fp64).
    Such rows are counted and reported.
  * next_token (T > 0) is exact, except in band rows and in rows whose final
    uniform lies within CDF_EPS of a cumulative-weight boundary of the sampled
    row (normalised to total mass 1).  In those ambiguous rows the GPU token
    must still be a valid draw: positive weight, with u inside its CDF interval
    widened by CDF_EPS.
  * A rejection whose residual mass lies in (0, RES_FLOOR_BAND) may land on
    either side of the 2^-20 floor below which both sides sample p_n instead:
    such rows only need an in-range token, and are counted.
  * alpha, p_draft and q_draft agree within 1e-5 absolute.
  * With per-sequence draft counts, the padding positions are NaN on both sides.

CDF_EPS comes from the GPU's fp32 arithmetic.  Each weight carries a few ulps
from exp2 and the 1/S scaling (relative ~1e-6 at exponent arguments near 30).
The residual max(0, p - q) turns the independent errors of p and q into an
absolute error of about 1e-7 (p + q) per token.  A fp32 scan over at most 2^18
tokens adds about 18 ulps of the running sum.  Together that is a few 1e-6 of
the sampled mass when the residual mass is at least a few percent; 1e-5 leaves
headroom.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from oracle import verify as ov

PROB_TOL = 1e-5
CDF_EPS = 1e-5
# v_exp_f32 is within an ulp of the correctly rounded exp2, so the kernel's and
# the oracle's normalised nucleus sums differ by at most 2^-23 of the total.
FILTER_EPS = 2.5e-7
# the GPU's residual mass carries about 1e-6 of absolute error (as alpha does)
RES_FLOOR_BAND = 4 * ov.RESIDUAL_FLOOR


@dataclasses.dataclass
class Report:
    rows: int = 0
    u_band: int = 0
    cdf_ambiguous: int = 0
    token_mismatch_valid: int = 0
    filter_ambiguous: int = 0
    floor_ambiguous: int = 0

    def __str__(self):
        return (f"rows={self.rows} u_band={self.u_band} cdf_ambiguous={self.cdf_ambiguous} "
                f"mismatched-but-valid={self.token_mismatch_valid} filter_ambiguous={self.filter_ambiguous} "
                f"floor_ambiguous={self.floor_ambiguous}")


def _cdf_interval(w: np.ndarray, t: int):
    c = np.cumsum(w)
    lo = c[t - 1] if t > 0 else 0.0
    return lo, c[t]


def check(case, gpu: dict, seqs=None, where: str = "", lenience: float = 1.0, gamma_seq=None,
          top_k: int = 0, top_p: float = 1.0) -> Report:
    """Compare GPU outputs (numpy dict, full batch) with the oracle on `seqs`.

    lenience, gamma_seq (numpy int [B]), top_k and top_p are passed to the
    oracle unchanged.  With top-p, a sequence one of whose rows has its nucleus
    boundary within FILTER_EPS of top_p (fp32 masses may then keep one tie group
    more or fewer) is counted and left out of the comparison."""
    if seqs is None:
        seqs = np.arange(case.B)
    seqs = np.asarray(seqs)
    res = ov.verify_case(case, keep_weights=case.temperature > 0, seqs=seqs, lenience=lenience,
                         gamma_seq=gamma_seq, top_k=top_k, top_p=top_p)
    keep = res.filter_margin >= FILTER_EPS
    if not keep.all():
        sub = np.nonzero(keep)[0]
        rep0 = check(case, gpu, seqs[sub], where, lenience, gamma_seq, top_k, top_p) if sub.size else Report()
        rep0.filter_ambiguous = int((~keep).sum())
        return rep0
    g = {k: np.asarray(v)[seqs] for k, v in gpu.items()}
    rep = Report(rows=len(seqs))
    G = case.gamma
    gb = np.full(len(seqs), G) if gamma_seq is None else np.asarray(gamma_seq)[seqs]

    if case.temperature == 0.0:
        assert np.array_equal(g["n_accepted"], res.n_accepted), where
        assert np.array_equal(g["next_token"], res.next_token), where
        if G:
            for key, ref in (("alpha", res.alpha), ("p_draft", res.p_draft), ("q_draft", res.q_draft)):
                assert np.array_equal(g[key], ref.astype(np.float32), equal_nan=True), f"{where}: {key}"
        return rep

    band = res.u_band
    rep.u_band = int(band.sum())
    bad_n = (g["n_accepted"] != res.n_accepted) & ~band
    assert not bad_n.any(), f"{where}: n_accepted differs outside the u band in rows {seqs[bad_n][:10]}"

    same_n = g["n_accepted"] == res.n_accepted
    ambiguous = res.cdf_margin < CDF_EPS
    rep.cdf_ambiguous = int((ambiguous & same_n).sum())
    with np.errstate(invalid="ignore"):
        near_floor = (res.res_mass > 0) & (res.res_mass < RES_FLOOR_BAND)
    rep.floor_ambiguous = int((near_floor & same_n).sum())
    for r in np.nonzero(same_n)[0]:
        t_gpu = int(g["next_token"][r])
        assert 0 <= t_gpu < case.V, f"{where}: token out of range in row {seqs[r]}"
        if t_gpu == res.next_token[r] or near_floor[r]:
            continue
        assert ambiguous[r], (f"{where}: next_token {t_gpu} != oracle {res.next_token[r]} in row "
                              f"{seqs[r]} (margin {res.cdf_margin[r]:.3g})")
        w = res.weights[r]
        lo, hi = _cdf_interval(w, t_gpu)
        u = float(case.uniforms[seqs[r], gb[r]])
        assert w[t_gpu] > 0 and lo - CDF_EPS <= u < hi + CDF_EPS, f"{where}: invalid token in row {seqs[r]}"
        rep.token_mismatch_valid += 1

    if G:
        for key, ref in (("alpha", res.alpha), ("p_draft", res.p_draft), ("q_draft", res.q_draft)):
            pad = np.isnan(ref)
            assert np.array_equal(np.isnan(g[key]), pad), f"{where}: {key} padding positions differ"
            err = np.abs(g[key].astype(np.float64) - ref)[~pad]
            assert np.all(err <= PROB_TOL), f"{where}: {key} max error {err.max():.3g}"
    return rep
