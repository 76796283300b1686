"""Seeded synthetic inputs for the five workloads.

This module only draws random numbers and lays them out rank-major; it holds
none of the collective's arithmetic.  The same arrays feed the GPU library and
the CPU oracle.

Recipe: numpy ``Generator(PCG64)`` with one independent stream per logical
rank from ``SeedSequence(seed).spawn(R)``; bfloat16 inputs are drawn in
float32 and rounded by torch's own float32 -> bfloat16 conversion.  The large
gradient-bucket workload is drawn on the device with a seeded torch generator
(one seed per bucket) so that a gigabyte per rank does not pass through the
host.
"""
import numpy as np

# name -> (R, dtype, elements per rank, distribution, seed)
WORKLOADS = {
    "ring_int32_r4": dict(R=4, dtype="int32", count=4096, dist="int_pm1000", seed=1),
    "ring_f32_r8_64MiB": dict(R=8, dtype="float32", count=16_777_216, dist="normal", seed=2),
    "sweep_f32_r8": dict(R=8, dtype="float32", count=None, dist="normal", seed=3),
    "tree_ll_f32_r8": dict(R=8, dtype="float32", count=None, dist="uniform_pm1", seed=4),
    "buckets_bf16_r16": dict(R=16, dtype="bf16", count=13_107_200, dist="normal_0.02", seed=5,
                             buckets=40),
}


def rank_generators(seed, R):
    """One numpy PCG64 generator per logical rank."""
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(R)]


def draw(dist, R, count, seed):
    """[R, count] host array for a distribution name.

    int_pm1000  : integers uniform on [-1000, 1000], both ends included (int32)
    normal      : standard normal (float32)
    uniform_pm1 : uniform on [-1, 1) (float32)
    normal_0.02 : normal with standard deviation 0.02 (float32, before bf16)
    ones        : all ones (float32)
    """
    gens = rank_generators(seed, R)
    if dist == "int_pm1000":
        return np.stack([g.integers(-1000, 1000, size=count, endpoint=True, dtype=np.int32)
                         for g in gens])
    if dist == "normal":
        return np.stack([g.standard_normal(count, dtype=np.float32) for g in gens])
    if dist == "uniform_pm1":
        return np.stack([(g.random(count, dtype=np.float32) * np.float32(2.0)
                          - np.float32(1.0)) for g in gens])
    if dist == "normal_0.02":
        return np.stack([g.standard_normal(count, dtype=np.float32) * np.float32(0.02)
                         for g in gens])
    if dist == "ones":
        return np.ones((R, count), dtype=np.float32)
    raise ValueError("unknown distribution %r" % (dist,))


def to_bf16_bits(a_f32):
    """float32 numpy array -> bfloat16 bit patterns (uint16) via torch's
    conversion (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def host_inputs(name, count=None, seed=None):
    """Host input array [R, count] for a workload (bf16 as uint16 bits)."""
    w = WORKLOADS[name]
    count = w["count"] if count is None else count
    seed = w["seed"] if seed is None else seed
    a = draw(w["dist"], w["R"], count, seed)
    if w["dtype"] == "bf16":
        return to_bf16_bits(a)
    return a


def device_bucket_bf16(R, count, seed, bucket, device):
    """One gradient bucket [R, count] of bfloat16 N(0, 0.02) drawn on the
    device with a torch generator seeded by (seed, bucket)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + bucket)
    x = torch.randn((R, count), generator=g, device=device, dtype=torch.float32)
    return (x * 0.02).to(torch.bfloat16)


def sweep_counts(min_bytes, max_bytes, elem_size=4):
    """Per-rank element counts for a powers-of-two byte sweep."""
    out = []
    b = min_bytes
    while b <= max_bytes:
        out.append(max(1, b // elem_size))
        b *= 2
    return out
