"""Sort-based reference for filtered categorical sampling (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): nothing in the GPU
library imports, links or runs this module.

Pages cited (titles as they appear; sections by their headings):

* [Blog]  FlashInfer blog, "Sorting-Free GPU Kernels for LLM Sampling"
          (Chinese translation "面向 LLM 采样的免排序 GPU 内核").
* [F4]    gpu-kernel-drills note "F4 讲解：不排序的 top-k / top-p".
* [Expl]  charlestar explainer on FlashInfer Sorting-Free Sampling.

Arithmetic
----------
Every float32 value x >= 0 is an integer multiple of 2**-149, so
``X = x * 2**149`` is an exact Python integer and every mass below is an
exact integer sum.  Parameters p and min_p are float32 numbers, hence exact
rationals; comparisons against ``p * Z`` are done in integers.  There is no
rounding anywhere in the decisions, so the kept sets are the mathematical
ones.  Only reported probabilities and renormalised values are rounded (to
float64 / float32) at the very end.

Readings of the pages (each also listed in the design doc):

* R1 ties: every filter is value-based and keeps all ties, so the kept set is
  always an upper set {i : x_i >= tau}.  [F4 §⑥] states that a threshold keeps
  every tied value; [Expl] "Tie 需要明确定义" asks only that the reference and
  the predicate agree.
* R2 top-p reference mass: the prefix is compared with p * Z_C, Z_C being the
  exact mass of the set entering the top-p stage (the whole row, or the top-k
  set under top-k-then-top-p).  [Expl] "Top-k 与 top-p 的组合顺序会改变分布"
  applies top-p inside the top-k set; for rows that sum to one this equals the
  raw rule of [F4 §②].
* R3 the top-p prefix is the smallest r >= 1 with prefix_r >= p * Z_C
  ([Expl] "Top-p"), so at least the maximum (with its ties) is kept.
* R4 parameter domains: k <= 0 makes the output invalid, k >= V keeps every
  token; p and min_p are clamped to [0, 1]; NaN p or min_p is invalid.
* R5 degenerate rows ([Expl] "退化分布必须可报告"): any value with the sign bit
  set (negative numbers and -0.0), NaN or +-inf, or a zero total, make the row
  invalid; sampling reports token -1 with valid = 0, renorm reports a NaN row.
* R6 min-p threshold is min_p * max as an exact product ([Blog] "Min-P",
  [Expl] "Min-p"); kept set {x >= min_p * max}.
* R18 logits with a temperature: the max is subtracted before the exponent
  (an identity of the formula, needed for range); differences, scaling by
  1/T, exponentials and their sum in float64, each probability rounded once
  to float32; the probabilities then enter the filters like any input row.
* R21 sampling from logits with the softmax fused (the library's default
  for top-k-then-top-p from logits): top-k, top-p (R2) and the draw compare
  values only with each other and with fractions of their sums, so scaling
  every value by one constant changes none of them; the filters and the draw
  then take the softmax's weights w_i = exp((z_i - m) * (1 / T)) in float64,
  rounded once to float32 (w = 1 at the maximum), and the normaliser
  S = sum_j w_j is never formed.  The kept set equals R18's except where the
  one float32 rounding of w_i versus that of w_i / S makes or breaks a tie.
* R19 top-k selection ([Expl] "选择 top-k 值本身": values and indices, not a
  sample): the k largest values of a row in descending order, equal values
  by ascending index, -0.0 equal to +0.0; a NaN makes the row invalid.
* R20 chain speculative verification ([Blog] "社区采用和其他应用" names chain
  speculative sampling as a use of the same rejection sampling and gives no
  algorithm; the standard one, Leviathan, Kalman & Matias 2023 and Chen et
  al. 2023, is taken): for j = 0 .. n-1 in order the draft token d_j is
  accepted iff u_j * q_j(d_j) < p_j(d_j), u_j the row's draw j; at the first
  rejection j* the emitted token is one inverse-transform draw (draw n) from
  the residual max(0, p_j* - q_j*), taken exactly, or from p_j* when that
  residual is zero everywhere; with every draft accepted a bonus token is
  drawn (draw n) from p_n.  Output: d_0 .. d_{j*-1}, the drawn token, then
  -1; accepted = j* (n with the bonus).  Invalid (all -1, accepted 0): a
  draft id outside [0, V), a sign bit / NaN / inf in an examined p_j(d_j) or
  q_j(d_j) or anywhere in the rows the final draw reads, or a zero total in
  the row it draws from.
* R17 the "joint" order ([Blog] footnote on the filter options; [Expl]
  "Top-k 与 top-p 的组合顺序会改变分布") checks the top-k and the top-p
  condition together in every rejection round; the top-p condition then
  refers to the whole row's mass (there is no top-k stage before it), so the
  kept set is where both hold: {x >= max(tau_k, tau_p)} with tau_p taken on
  the whole row.
"""

from bisect import bisect_left, bisect_right
from fractions import Fraction
from itertools import accumulate

import numpy as np

SCALE_EXP = 149          # x * 2**149 is an integer for every float32 x >= 0

OPS = ("none", "top_k", "top_p", "min_p", "top_k_top_p", "top_k_top_p_joint")
K_OPS = ("top_k", "top_k_top_p", "top_k_top_p_joint")
P_OPS = ("top_p", "top_k_top_p", "top_k_top_p_joint")


# ----------------------------------------------------------------------------
# exact arithmetic helpers
# ----------------------------------------------------------------------------

def exact_units(values):
    """Exact integers x * 2**149 for a float32 array of finite x >= 0."""
    scaled = np.ldexp(np.asarray(values, dtype=np.float32).astype(np.float64),
                      SCALE_EXP)
    return [int(t) for t in scaled]


def fraction_of(value):
    """Exact rational value of a float32 (or float64) number."""
    return Fraction(*float(value).as_integer_ratio())


def row_is_valid(row):
    """R5: no sign bit set, no NaN/inf, and a positive total."""
    row = np.asarray(row, dtype=np.float32)
    bits = row.view(np.uint32)
    if np.any(bits >= np.uint32(0x7F800000)):   # sign bit, inf or NaN
        return False
    return bool(np.any(bits != 0))


# ----------------------------------------------------------------------------
# thresholds (the kept set is {x >= tau}, R1)
# ----------------------------------------------------------------------------

def _sorted_desc(row):
    return np.sort(np.asarray(row, dtype=np.float32))[::-1]


def tau_top_k(row, k):
    """k-th largest value [Expl "Top-k"]; k >= V keeps every token."""
    s = _sorted_desc(row)
    kk = min(int(k), s.size)
    return float(s[kk - 1])


def _count_at_least(sorted_desc, tau):
    """Number of entries >= tau in a descending array."""
    asc = sorted_desc[::-1]
    return int(asc.size - np.searchsorted(asc, np.float32(tau), side="left"))


def tau_top_p(sorted_desc, n_c, p):
    """Top-p threshold on the first n_c entries of a descending row.

    m = min{r >= 1 : sum_{j<=r} v_(j) >= p * Z_C} and tau = v_(m)
    ([Expl] "Top-p"; R2, R3).  ``p`` must already be clamped to [0, 1].
    """
    units = exact_units(sorted_desc[:n_c])
    prefix = list(accumulate(units))
    z_c = prefix[-1]
    num, den = fraction_of(p).as_integer_ratio()
    # prefix_r * den >= num * z_c  <=>  prefix_r >= ceil(num * z_c / den)
    need = -((-num * z_c) // den)
    r = bisect_left(prefix, need)
    r = max(0, min(r, n_c - 1))
    return float(sorted_desc[r])


def top_p_boundary_margin(row, p, k=None):
    """Relative distance of the top-p decision from a tie with p * Z_C.

    min(|prefix_m - p Z_C|, |prefix_{m'} - p Z_C|) / Z_C, where m is the
    chosen prefix length and m' the last prefix strictly below it; a float64
    implementation that accumulates masses with relative error e decides
    every boundary exactly when the margin exceeds e.  Reported by the GPU
    tests; not used by any decision here.
    """
    s = _sorted_desc(row)
    n_c = s.size if k is None else _count_at_least(s, tau_top_k(row, k))
    units = exact_units(s[:n_c])
    prefix = list(accumulate(units))
    z_c = prefix[-1]
    pf = fraction_of(clamp01(p)) * z_c
    r = bisect_left(prefix, -((-pf.numerator) // pf.denominator))
    r = max(0, min(r, n_c - 1))
    gaps = [abs(prefix[r] - pf)]
    tau = s[r]
    below = _count_at_least(s[:n_c], np.nextafter(tau, np.float32(np.inf)))
    if below > 0:
        gaps.append(abs(prefix[below - 1] - pf))
    return float(min(gaps) / z_c)


def clamp01(v):
    v = float(np.float32(v))
    return min(max(v, 0.0), 1.0)


def threshold(row, op, k=None, p=None, min_p=None):
    """(valid, tau) for one row and one filter; kept set = {x >= tau}.

    ``tau`` is returned as a float64 holding the exact threshold (for min-p,
    the exact product of two float32 numbers, which float64 represents
    exactly).
    """
    row = np.asarray(row, dtype=np.float32)
    if not row_is_valid(row):
        return False, None
    if op == "none":
        return True, 0.0
    if op in K_OPS and int(k) <= 0:
        return False, None
    if op in P_OPS and np.isnan(np.float32(p)):
        return False, None
    if op == "min_p" and np.isnan(np.float32(min_p)):
        return False, None
    s = _sorted_desc(row)
    if op == "top_k":
        return True, tau_top_k(row, k)
    if op == "top_p":
        return True, tau_top_p(s, s.size, clamp01(p))
    if op == "top_k_top_p":
        tk = tau_top_k(row, k)
        n_c = _count_at_least(s, tk)
        return True, tau_top_p(s, n_c, clamp01(p))
    if op == "top_k_top_p_joint":
        # both conditions at once (R17): the larger of the two thresholds,
        # the top-p one against the whole row
        return True, max(tau_top_k(row, k), tau_top_p(s, s.size, clamp01(p)))
    if op == "min_p":
        # exact: a product of two float32 numbers fits a float64 exactly
        return True, float(np.float64(clamp01(min_p)) * np.float64(s[0]))
    raise ValueError(op)


def kept_mask(row, tau):
    """{x >= tau} (R1)."""
    return np.asarray(row, dtype=np.float32).astype(np.float64) >= float(tau)


def support_mask(row, tau):
    """Support of the filtered distribution: kept and strictly positive."""
    r = np.asarray(row, dtype=np.float32)
    return kept_mask(r, tau) & (r > 0)


def target_distribution(row, tau):
    """p~_i = p_i / sum_{j in S} p_j on S, else 0 ([Expl] "采样流水线究竟在计算什么")."""
    r = np.asarray(row, dtype=np.float32)
    sup = support_mask(r, tau)
    z = sum(exact_units(r[sup]))
    out = np.zeros(r.size, dtype=np.float64)
    # x_i * 2**149 / Z, both exact before the one final rounding of each
    out[sup] = np.ldexp(r[sup].astype(np.float64), SCALE_EXP) / float(z)
    return out


# ----------------------------------------------------------------------------
# renormalisation and logit masking
# ----------------------------------------------------------------------------

def renorm_row(row, tau):
    """out_i = x_i / Z_S on the kept set, 0 elsewhere ([F4 §④] last two passes).

    Z_S is exact; the quotient is formed in float64 from the correctly
    rounded Z_S and rounded once more to float32.
    """
    r = np.asarray(row, dtype=np.float32)
    keep = kept_mask(r, tau)
    z = sum(exact_units(r[keep]))
    zf = np.ldexp(float(z), -SCALE_EXP)
    out = np.zeros(r.size, dtype=np.float32)
    out[keep] = (r[keep].astype(np.float64) / zf).astype(np.float32)
    return out


def top_k_renorm(row, k):
    valid, tau = threshold(row, "top_k", k=k)
    if not valid:
        return False, np.full(np.asarray(row).size, np.nan, dtype=np.float32)
    return True, renorm_row(row, tau)


def top_p_renorm(row, p):
    valid, tau = threshold(row, "top_p", p=p)
    if not valid:
        return False, np.full(np.asarray(row).size, np.nan, dtype=np.float32)
    return True, renorm_row(row, tau)


def mask_logits_row(row, k):
    """Keep the k largest logits (ties kept, R1), set the rest to -inf.

    Logits may be negative, so the order is the numeric order of the values
    ([F4 §⑧]: raw bit patterns of negative floats order backwards).  A NaN
    logit or k <= 0 makes the row invalid (NaN-filled output).
    """
    r = np.asarray(row, dtype=np.float32)
    if np.any(np.isnan(r)) or int(k) <= 0:
        return False, np.full(r.size, np.nan, dtype=np.float32)
    if int(k) >= r.size:
        return True, r.copy()
    tau = np.sort(r)[::-1][int(k) - 1]
    return True, np.where(r >= tau, r, np.float32(-np.inf)).astype(np.float32)


# ----------------------------------------------------------------------------
# inverse-transform draw
# ----------------------------------------------------------------------------

class CdfTable:
    """Exact prefix sums of the masked entries of one row, for repeated draws.

    ``draw(a53)`` is the inverse-transform rule of ``inverse_transform``:
    the first masked index j (index order) whose prefix exceeds u * Z, with
    u = a53 / 2**53 and Z the masked total.
    """

    def __init__(self, row, mask):
        r = np.asarray(row, dtype=np.float32)
        self.idx = np.nonzero(mask)[0]
        self.prefix = list(accumulate(exact_units(r[self.idx])))
        self.total = self.prefix[-1] if self.prefix else 0

    def draw(self, a53):
        if self.total == 0:
            return -1
        thr = (int(a53) * self.total) >> 53       # floor(u * Z)
        return int(self.idx[bisect_right(self.prefix, thr)])


def inverse_transform(row, mask, a53):
    """Index j with F_{j-1} <= u * Z < F_j over the masked entries, in index order.

    [Blog] "逆变换采样" and [Expl] "不带过滤时：inverse transform sampling":
    u ~ U[0, 1), F the prefix sums, return the first j with F_j > u.  Here
    u = a53 / 2**53 and the prefix is scaled by the total Z of the masked
    entries, so unnormalised rows are handled exactly.  Returns -1 if the
    masked mass is zero.
    """
    return CdfTable(row, mask).draw(a53)


def sample_by_cdf(row, op, a53, k=None, p=None, min_p=None):
    """Sort-based filter then one CDF draw: the oracle's own sampler."""
    valid, tau = threshold(row, op, k=k, p=p, min_p=min_p)
    if not valid:
        return -1
    return inverse_transform(row, support_mask(row, tau), a53)


# ----------------------------------------------------------------------------
# probabilities from logits with a temperature (the step before the filters)
# ----------------------------------------------------------------------------

def softmax_row(z, temperature):
    """p_i = exp(z_i / T) / sum_j exp(z_j / T) ([Expl] "采样流水线究竟在计算什么").

    Written out in the order the library fixes (R18): m = max_i z_i,
    t_i = (z_i - m) * (1 / T) in float64 (the difference of two float32 is
    exact there), e_i = exp(t_i) in float64, S = sum_i e_i rounded once
    (math.fsum), and p_i = float32(e_i / S).  Returns (valid, p): a NaN or
    +inf logit, no finite logit, or T not a finite positive number make the
    row invalid.
    """
    import math
    z = np.asarray(z, dtype=np.float32)
    t32 = np.float32(temperature)
    if np.isnan(z).any() or np.isposinf(z).any() or not np.isfinite(z).any():
        return False, None
    if not (np.isfinite(t32) and t32 > 0):
        return False, None
    m = np.float64(z.max())
    inv_t = 1.0 / np.float64(t32)
    with np.errstate(invalid="ignore", over="ignore"):
        t = (z.astype(np.float64) - m) * inv_t
    e = np.exp(t)                                # -inf -> 0
    total = math.fsum(e.tolist())
    return True, (e / total).astype(np.float32)


def softmax_weights(z, temperature):
    """w_i = float32(exp((z_i - m) * (1 / T))), m = max_i z_i (R21): the
    softmax of [Expl] "采样流水线究竟在计算什么" without its normaliser.
    Returns (valid, w); invalid exactly when ``softmax_row`` is."""
    z = np.asarray(z, dtype=np.float32)
    t32 = np.float32(temperature)
    if np.isnan(z).any() or np.isposinf(z).any() or not np.isfinite(z).any():
        return False, None
    if not (np.isfinite(t32) and t32 > 0):
        return False, None
    m = np.float64(z.max())
    inv_t = 1.0 / np.float64(t32)
    with np.errstate(invalid="ignore", over="ignore"):
        t = (z.astype(np.float64) - m) * inv_t
    return True, np.exp(t).astype(np.float32)


# ----------------------------------------------------------------------------
# top-k selection: values and indices (R19)
# ----------------------------------------------------------------------------

def top_k_select(row, k):
    """(valid, values, indices) of the k largest entries of a float32 row,
    values descending, equal values by ascending index (R19); NaN: invalid."""
    row = np.asarray(row, dtype=np.float32)
    if np.isnan(row).any():
        return False, None, None
    key = row.astype(np.float64) + 0.0            # -0.0 -> +0.0
    order = np.lexsort((np.arange(row.size), -key))[:int(k)]
    return True, row[order], order.astype(np.int32)


# ----------------------------------------------------------------------------
# chain speculative verification (R20)
# ----------------------------------------------------------------------------

def _finite_nonneg(values):
    """No sign bit (negative or -0.0), NaN or inf among float32 values."""
    bits = np.atleast_1d(np.asarray(values, dtype=np.float32)).view(np.uint32)
    return not np.any(bits >= np.uint32(0x7F800000))


def draw_from_units(units, a53):
    """Inverse transform on exact weights: the first index whose prefix
    exceeds floor(u * Z), u = a53 / 2**53 (the rule of ``CdfTable``); -1 when
    the total is zero."""
    prefix = list(accumulate(units))
    if not prefix or prefix[-1] == 0:
        return -1
    thr = (int(a53) * prefix[-1]) >> 53
    return bisect_right(prefix, thr)


def chain_speculative(draft_probs, draft_ids, target_probs, a53s):
    """One row of chain speculative verification (R20).

    draft_probs [n, V] (q), draft_ids [n], target_probs [n + 1, V] (p), all
    float32 / integer; a53s: the n + 1 draws (53-bit integers) of the row,
    draw j for the acceptance test at position j, draw n for the final
    token.  Returns (valid, tokens [n + 1] int32, accepted).
    """
    q = np.asarray(draft_probs, dtype=np.float32)
    p = np.asarray(target_probs, dtype=np.float32)
    ids = np.asarray(draft_ids).astype(np.int64)
    n, V = q.shape
    bad = (False, np.full(n + 1, -1, dtype=np.int32), 0)
    out = []
    for j in range(n):
        d = int(ids[j])
        if not 0 <= d < V:
            return bad
        pj, qj = p[j, d], q[j, d]
        if not (_finite_nonneg(pj) and _finite_nonneg(qj)):
            return bad
        # u * q < p with u = a / 2**53, in integers
        (qu,), (pu,) = exact_units([qj]), exact_units([pj])
        if int(a53s[j]) * qu < pu << 53:
            out.append(d)
            continue
        if not (_finite_nonneg(p[j]) and _finite_nonneg(q[j])):
            return bad
        res = [max(0, a - b) for a, b in zip(exact_units(p[j]), exact_units(q[j]))]
        if sum(res) == 0:
            res = exact_units(p[j])
        tok = draw_from_units(res, a53s[n])
        if tok < 0:
            return bad
        out += [tok] + [-1] * (n - j)
        return True, np.array(out, dtype=np.int32), j
    if not _finite_nonneg(p[n]):
        return bad
    tok = draw_from_units(exact_units(p[n]), a53s[n])
    if tok < 0:
        return bad
    return True, np.array(out + [tok], dtype=np.int32), n


# ----------------------------------------------------------------------------
# the rejection predicate f and a plain model of dual-pivot rejection sampling
# ----------------------------------------------------------------------------

class Predicate:
    """f(t) = 1 iff the threshold t already satisfies the filter.

    [Blog] "双枢轴拒绝采样" defines f on probability values; "拒绝采样" says the
    top-p check compares the mass above the pivot with top_p and the top-k
    check counts the tokens above the pivot.  Written with strict
    comparisons (x > t), as the draw range (low, inf) of the same section:

      top_k:        #{x > t} < k
      top_p:        sum_{x > t} x < p * Z_C   or  #{x > t} = 0
      min_p:        t >= min_p * max
      top_k_top_p:  top_k(t)  and  (sum_{x > t} x < p * Z_k  or  #{x > t} = 0)
      top_k_top_p_joint:
                    top_k(t)  and  (sum_{x > t} x < p * Z_C  or  #{x > t} = 0)
      none:         always 1

    Z_C is the whole row's exact mass, Z_k that of {x >= tau_k} (R2, R17).
    The "#{x > t} = 0" clause makes f(max) = 1 also when p = 0.
    """

    def __init__(self, row, op, k=None, p=None, min_p=None):
        self.row = np.asarray(row, dtype=np.float32)
        self.op = op
        self.units = exact_units(self.row)
        self.k = None if k is None else int(k)
        if op in P_OPS:
            self.p_num, self.p_den = fraction_of(clamp01(p)).as_integer_ratio()
        if op in ("top_p", "top_k_top_p_joint"):
            self.z_c = sum(self.units)
        if op == "top_k_top_p":
            tk = tau_top_k(self.row, self.k)
            self.z_c = sum(u for u, x in zip(self.units, self.row) if x >= tk)
        if op == "min_p":
            self.minp_tau = float(np.float64(clamp01(min_p)) *
                                  np.float64(self.row.max()))

    def mass_count_above(self, t):
        above = self.row > np.float32(t)
        return sum(u for u, a in zip(self.units, above) if a), int(above.sum())

    def __call__(self, t):
        if self.op == "none":
            return True
        if self.op == "min_p":
            return float(np.float32(t)) >= self.minp_tau
        mass, count = self.mass_count_above(t)
        ok_k = True if self.op == "top_p" else count < self.k
        if self.op == "top_k":
            return ok_k
        ok_p = (mass * self.p_den < self.p_num * self.z_c) or count == 0
        return ok_k and ok_p


def pivot2_of(pivot1, high):
    """(pivot1 + high) / 2 rounded once to float32 (reading of [Blog] "双枢轴拒绝采样").

    The sum of two float32 numbers and its half are exact in float64, so
    this is the correctly rounded midpoint with no overflow.
    """
    return np.float32((np.float64(pivot1) + np.float64(high)) / 2.0)


def dual_pivot_sample(row, op, stream, k=None, p=None, min_p=None,
                      max_rounds=100000, trace=None):
    """One draw by dual-pivot rejection sampling, following [Blog] "双枢轴拒绝采样".

      low <- 0, high <- max
      repeat: draw j from the tokens with p_j > low by inverse transform;
              pivot1 <- p_j; pivot2 <- (pivot1 + high) / 2
              f(pivot1) = 1                -> return j
              f(pivot1) = 0, f(pivot2) = 1 -> low, high <- pivot1, pivot2
              f(pivot1) = 0, f(pivot2) = 0 -> low <- pivot2

    ``stream.next()`` supplies one 53-bit uniform per draw.  Returns
    (token, rounds); (-1, 0) for an invalid row or parameter.  If ``trace``
    is a list, the (low, high) interval is appended to it at the start and
    after every rejected round.
    """
    row = np.asarray(row, dtype=np.float32)
    valid, _ = threshold(row, op, k=k, p=p, min_p=min_p)
    if not valid:
        return -1, 0
    f = Predicate(row, op, k=k, p=p, min_p=min_p)
    low, high = np.float32(0.0), np.float32(row.max())
    if trace is not None:
        trace.append((low, high))
    for rounds in range(1, max_rounds + 1):
        j = inverse_transform(row, row > low, stream.next())
        pivot1 = row[j]
        if f(pivot1):
            return j, rounds
        pivot2 = pivot2_of(pivot1, high)
        if f(pivot2):
            low, high = pivot1, pivot2
        else:
            low = pivot2
        if trace is not None:
            trace.append((low, high))
    raise RuntimeError("dual-pivot model did not terminate")


def single_pivot_sample(row, op, stream, k=None, p=None, min_p=None, max_rounds=1000000):
    """One draw by single-pivot rejection sampling ([Blog] "拒绝采样"; [Expl]
    "如何在不知道 top-k 边界时拒绝错误样本"):

      low <- 0
      repeat: draw j from the tokens with p_j > low by inverse transform;
              f(p_j) = 1 -> return j;  otherwise low <- p_j

    Same stream, predicate and draw rule as ``dual_pivot_sample``; returns
    (token, rounds), (-1, 0) for an invalid row or parameter.
    """
    row = np.asarray(row, dtype=np.float32)
    valid, _ = threshold(row, op, k=k, p=p, min_p=min_p)
    if not valid:
        return -1, 0
    f = Predicate(row, op, k=k, p=p, min_p=min_p)
    low = np.float32(0.0)
    for rounds in range(1, max_rounds + 1):
        j = inverse_transform(row, row > low, stream.next())
        if f(row[j]):
            return j, rounds
        low = row[j]
    raise RuntimeError("single-pivot model did not terminate")


def single_pivot_law(row, op, k=None, p=None, min_p=None):
    """Exact output law and expected round count of ``single_pivot_sample``
    (enumeration over every reachable low with exact rationals; tiny rows)."""
    row = np.asarray(row, dtype=np.float32)
    f = Predicate(row, op, k=k, p=p, min_p=min_p)
    units = f.units
    memo = {}

    def solve(low):
        key = float(low)
        if key in memo:
            return memo[key]
        cand = [i for i in range(row.size) if row[i] > low]
        s = sum(units[i] for i in cand)
        law, rounds = {}, Fraction(1)
        for i in cand:
            w = Fraction(units[i], s)
            if w == 0:
                continue
            if f(row[i]):
                law[i] = law.get(i, Fraction(0)) + w
                continue
            sub_law, sub_rounds = solve(row[i])
            for j, q in sub_law.items():
                law[j] = law.get(j, Fraction(0)) + w * q
            rounds += w * sub_rounds
        memo[key] = (law, rounds)
        return law, rounds

    return solve(np.float32(0.0))


def dual_pivot_law(row, op, k=None, p=None, min_p=None):
    """Exact output law and expected round count of ``dual_pivot_sample``.

    Enumerates every draw from every reachable (low, high) state with exact
    rationals (draw probability p_i / S(low), S(low) = mass above low, as in
    the recurrence (★) of [Blog] "拒绝采样器正确性的理论证明").  For tiny
    vocabularies only.  Returns ({token: Fraction}, Fraction expected_rounds).
    """
    row = np.asarray(row, dtype=np.float32)
    f = Predicate(row, op, k=k, p=p, min_p=min_p)
    units = f.units
    memo = {}

    def solve(low, high):
        key = (float(low), float(high))
        if key in memo:
            return memo[key]
        cand = [i for i in range(row.size) if row[i] > low]
        s = sum(units[i] for i in cand)
        law, rounds = {}, Fraction(1)
        for i in cand:
            w = Fraction(units[i], s)
            if w == 0:
                continue
            pivot1 = row[i]
            if f(pivot1):
                law[i] = law.get(i, Fraction(0)) + w
                continue
            pivot2 = pivot2_of(pivot1, high)
            sub_law, sub_rounds = (solve(pivot1, pivot2) if f(pivot2)
                                   else solve(pivot2, high))
            for j, q in sub_law.items():
                law[j] = law.get(j, Fraction(0)) + w * q
            rounds += w * sub_rounds
        memo[key] = (law, rounds)
        return law, rounds

    return solve(np.float32(0.0), np.float32(row.max()))


def dual_pivot_rounds_law(row, op, k=None, p=None, min_p=None):
    """Exact law of the number of rounds ``dual_pivot_sample`` takes.

    The same enumeration as ``dual_pivot_law`` ([Blog] "双枢轴拒绝采样":
    draw above low, accept at f(pivot1) = 1, else move (low, high) by the
    three cases), but every accepted path adds its probability to the count
    of rounds it used.  Tiny vocabularies only.  Returns {rounds: Fraction}.
    """
    row = np.asarray(row, dtype=np.float32)
    f = Predicate(row, op, k=k, p=p, min_p=min_p)
    units = f.units
    memo = {}

    def solve(low, high):
        key = (float(low), float(high))
        if key in memo:
            return memo[key]
        cand = [i for i in range(row.size) if row[i] > low]
        s = sum(units[i] for i in cand)
        law = {}
        for i in cand:
            w = Fraction(units[i], s)
            if w == 0:
                continue
            pivot1 = row[i]
            if f(pivot1):
                law[1] = law.get(1, Fraction(0)) + w
                continue
            pivot2 = pivot2_of(pivot1, high)
            sub = solve(pivot1, pivot2) if f(pivot2) else solve(pivot2, high)
            for r, q in sub.items():
                law[r + 1] = law.get(r + 1, Fraction(0)) + w * q
        memo[key] = law
        return law

    return solve(np.float32(0.0), np.float32(row.max()))


# ----------------------------------------------------------------------------
# batch helpers mirroring the library's calling convention
# ----------------------------------------------------------------------------

def per_output(arr, scalar, n):
    """Per-output parameter list: the array if given, else the scalar repeated."""
    if arr is None:
        return [scalar] * n
    return list(np.asarray(arr).reshape(-1)[:n])


def batch_thresholds(probs, op, indices=None, k=None, p=None, min_p=None,
                     num_outputs=None):
    """(valid, tau) per output; ``indices`` maps outputs onto rows.

    ``k``, ``p``, ``min_p`` are scalars or per-output arrays.  An index
    outside [0, rows) makes that output invalid.
    """
    probs = np.asarray(probs, dtype=np.float32)
    rows = probs.shape[0]
    n = rows if num_outputs is None else int(num_outputs)
    rows_of = list(range(n)) if indices is None else [int(v) for v in indices]

    def listify(v):
        return list(np.asarray(v).reshape(-1)) if np.ndim(v) else [v] * n

    ks, ps, ms = listify(k), listify(p), listify(min_p)
    out = []
    for i in range(n):
        r = rows_of[i]
        if r < 0 or r >= rows:
            out.append((False, None))
            continue
        out.append(threshold(probs[r], op, k=ks[i], p=ps[i], min_p=ms[i]))
    return out
