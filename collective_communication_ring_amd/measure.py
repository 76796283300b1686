"""Bandwidth bookkeeping and the alpha-beta fit.

Byte and bandwidth definitions used by the benchmark:
  algBW  = per-rank bytes / time                      (n * s / t)
  busBW  = algBW * 2(R-1)/R for all-reduce, algBW * (R-1)/R for
           reduce-scatter and all-gather
  algorithmic HBM bytes of one ring all-reduce in the one-HBM direct form
  (each of the R-1 reduce steps of a segment reads two operands and writes
  one, each of the R-1 copy steps reads one and writes one):
           5 (R-1) N s
  reduce-scatter: (R-1) reduce steps, partials in the accumulator type A
  (4 bytes) when T is narrower: first step reads 2 T and writes A, middle
  steps read A + T and write A, the last reads A + T and writes T.
  all-gather: one placement (read T, write T) and R-1 copy steps.
The cost model T(n) = alpha + beta * n ("NCCL and NVSHMEM -- two GPU
communication models, side by side", cost-model paragraph: alpha is the
latency floor, beta the reciprocal bandwidth).
"""
import numpy as np


def allreduce_alg_bytes(R, N, s):
    return 5 * (R - 1) * N * s


def reduce_scatter_alg_bytes(R, N, s, acc=4):
    if R == 2:
        return N * (2 * s + s)
    return N * ((2 * s + acc) + (R - 3) * (acc + s + acc) + (acc + s + s))


def all_gather_alg_bytes(R, N, s):
    # N = R * shard: placement of every shard plus R-1 copy steps
    return 2 * N * s + 2 * (R - 1) * N * s


def busbw_factor(op, R):
    return 2.0 * (R - 1) / R if op == "allreduce" else (R - 1) / R


def fit_alpha_beta(n_bytes, t_sec):
    """Least-squares fit of t = alpha + beta * n weighted by 1/t^2 (relative
    error).  Returns dict(alpha_us, inv_beta_GBps, r2, max_rel_residual)."""
    n = np.asarray(n_bytes, dtype=np.float64)
    t = np.asarray(t_sec, dtype=np.float64)
    w = 1.0 / t
    A = np.stack([w, n * w], axis=1)
    coef, *_ = np.linalg.lstsq(A, np.ones_like(t), rcond=None)
    alpha, beta = coef
    pred = alpha + beta * n
    rel = (pred - t) / t
    ss_res = float(np.sum((t - pred) ** 2))
    ss_tot = float(np.sum((t - t.mean()) ** 2))
    return dict(alpha_us=alpha * 1e6,
                inv_beta_GBps=(1.0 / beta / 1e9) if beta > 0 else float("inf"),
                r2=1.0 - ss_res / ss_tot if ss_tot > 0 else 1.0,
                max_rel_residual=float(np.max(np.abs(rel))))
