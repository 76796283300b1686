"""Bandwidth bookkeeping and the alpha-beta fit.

Byte and bandwidth definitions used by the benchmark:
  algBW  = per-rank bytes / time                      (n * s / t)
  busBW  = algBW * 2(R-1)/R for all-reduce, algBW * (R-1)/R for
           reduce-scatter and all-gather

Two byte counts per collective (N elements per rank, s bytes each):
  hop bytes -- every step's loads and stores, as if each hop went through
  memory (the direct one-HBM form, where the receiver reads the sender's
  buffer in place): all-reduce 5 (R-1) N s (each of the R-1 reduce steps of
  a segment reads two operands and writes one, each of the R-1 copy steps
  reads one and writes one); reduce-scatter with partials in the accumulator
  type A (4 bytes) when T is narrower: first step reads 2 T and writes A,
  middle steps read A + T and write A, the last reads A + T and writes T;
  all-gather one placement (read T, write T) and R-1 copy steps.
  HBM bytes -- what must cross the HBM at least: every input element read
  once and every output element written once.  All-reduce 2 R N s;
  reduce-scatter R N s + N s; all-gather N s + R N s.  The fused form moves
  exactly these (its hops are stores and loads of lines still in the XCD's
  L2), so they are its roofline bytes; the counters confirm it.
The cost model T(n) = alpha + beta * n ("NCCL and NVSHMEM -- two GPU
communication models, side by side", cost-model paragraph: alpha is the
latency floor, beta the reciprocal bandwidth).
"""
import numpy as np


def allreduce_alg_bytes(R, N, s, acc=None):
    """Hop bytes of one ring all-reduce: the reduce-scatter's, then R-1 copy
    steps (5 (R-1) N s when the partials are in T itself, acc = s)."""
    return reduce_scatter_alg_bytes(R, N, s, s if acc is None else acc) + 2 * (R - 1) * N * s


def allreduce_hbm_bytes(R, N, s):
    """HBM bytes of one all-reduce: R input rows read, R output rows written."""
    return 2 * R * N * s


def reduce_scatter_hbm_bytes(R, N, s):
    """R input rows of N read, R shards of N / R written."""
    return R * N * s + N * s


def all_gather_hbm_bytes(R, N, s):
    """R shards of N / R read, R output rows of N written."""
    return N * s + R * N * s


def reduce_scatter_alg_bytes(R, N, s, acc=4):
    """Hop bytes of one ring reduce-scatter."""
    if R == 2:
        return N * (2 * s + s)
    return N * ((2 * s + acc) + (R - 3) * (acc + s + acc) + (acc + s + s))


def all_gather_alg_bytes(R, N, s):
    """Hop bytes of one ring all-gather."""
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


def crossover_bytes(fit_small, fit_large):
    """Per-rank size where two alpha-beta lines cross (the first is cheaper
    below it); None when they do not cross at a positive size."""
    # alpha in us, beta in us per byte (1 GB/s moves 1e3 bytes per us)
    a1, b1 = fit_small["alpha_us"], 1e-3 / fit_small["inv_beta_GBps"]
    a2, b2 = fit_large["alpha_us"], 1e-3 / fit_large["inv_beta_GBps"]
    if b1 <= b2:
        return None
    n = (a2 - a1) / (b1 - b2)
    return n if n > 0 else None
