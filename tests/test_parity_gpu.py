"""GPU parity: libar's HIP kernels against the CPU oracle, on the same seeded
inputs.  The oracle replays the same ring/tree order, so every dtype is
expected bit-exact; float32 is also held to the stated tolerance against the
float64 sum (1e-6 relative + 1e-6*R absolute), bfloat16 to 1e-2 relative.
"""
import re

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

# ring launch forms; "ll" is the ring with the LL protocol
LAUNCHES = ["fused", "step", "pipelined", "ll"]


def ring_opts(launch):
    """Comm keyword arguments for a ring variant name."""
    if launch == "ll":
        return dict(algo="ring", proto="ll")
    return dict(algo="ring", proto="simple", launch=launch)


@pytest.fixture(scope="module")
def env():
    import torch
    from collective_communication_ring_amd import api, inputs
    import oracle
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    api.lib()
    return dict(torch=torch, api=api, inputs=inputs, orc=oracle, dev=torch.device("cuda:0"))


def _np_dtype(dtype):
    return {"int32": np.int32, "float32": np.float32, "bf16": np.uint16}[dtype]


def to_dev(env, x, dtype):
    torch = env["torch"]
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(env["dev"]).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(env["dev"])


def from_dev(env, t, dtype):
    torch = env["torch"]
    torch.cuda.synchronize()
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def poisoned(env, shape, dtype):
    """An output buffer full of 0xFF bytes (NaN / -1), so any element the
    kernel fails to write is caught."""
    torch = env["torch"]
    tdt = {"int32": torch.int32, "float32": torch.float32, "bf16": torch.bfloat16}[dtype]
    t = torch.empty(shape, dtype=tdt, device=env["dev"])
    t.view(torch.uint8).fill_(0xFF)
    return t


def rand_input(env, dtype, R, N, seed):
    inputs = env["inputs"]
    if dtype == "int32":
        return inputs.draw("int_pm1000", R, N, seed)
    if dtype == "float32":
        return inputs.draw("normal", R, N, seed)
    return inputs.to_bf16_bits(inputs.draw("normal_0.02", R, N, seed))


def check_tolerance(env, y, x, dtype):
    orc = env["orc"]
    R = x.shape[0]
    ex = orc.exact_sum(x, dtype)
    if dtype == "float32":
        err = np.abs(y.astype(np.float64) - ex[None, :])
        assert (err <= 1e-6 * np.abs(ex)[None, :] + 1e-6 * R).all()
    elif dtype == "bf16":
        yf = orc.f32_from_bf16(y).astype(np.float64)
        assert (np.abs(yf - ex[None, :]) <= 1e-2 * np.abs(ex)[None, :] + 1e-6 * R).all()


def run_allreduce(env, x, dtype, algo="ring", proto="simple", launch=None, reps=1, **opts):
    api = env["api"]
    R, N = x.shape
    if launch == "ll":
        proto, launch = "ll", None
    comm = api.Comm(R, max(N, 1), dtype, algo, proto, device=env["dev"], launch=launch, **opts)
    send = to_dev(env, x, dtype)
    outs = []
    for _ in range(reps):
        recv = poisoned(env, (R, N), dtype)
        comm.allreduce(send, recv)
        outs.append(from_dev(env, recv, dtype))
    assert comm.check() == api.AR_SUCCESS
    return outs


# ---------------------------------------------------------------- R = 4 int32, 4096 per rank

@pytest.mark.parametrize("launch", LAUNCHES)
def test_ring_int32_r4_4096(env, launch):
    x = env["inputs"].host_inputs("ring_int32_r4")
    R, N = x.shape
    (y,) = run_allreduce(env, x, "int32", launch=launch, chunk_bytes=(N // R) * 4)
    want = x.astype(np.int64).sum(axis=0).astype(np.int32)
    assert np.array_equal(y, env["orc"].ring_allreduce(x))
    assert (y == want[None, :]).all()


# ---------------------------------------------------------------- R = 8 fp32, 64 MiB per rank

@pytest.mark.parametrize("launch", LAUNCHES)
def test_ring_f32_r8_64MiB(env, launch):
    x = env["inputs"].host_inputs("ring_f32_r8_64MiB")
    (y,) = run_allreduce(env, x, "float32", launch=launch, chunk_bytes=512 * 1024)
    ref = env["orc"].ring_allreduce(x)
    assert y.tobytes() == ref.tobytes()
    check_tolerance(env, y, x, "float32")


@pytest.mark.parametrize("form", ["fused", "ll"])
def test_tree_f32_r8_64MiB(env, form):
    """Both tree forms on the same 64 MiB-per-rank inputs (the fused tree in
    16-byte packs, its default grid looping over each half 16 times; the LL
    tree runs 128 pieces): bit-exact against the oracle's tree, and within
    the float32 tolerance of the exact sum."""
    x = env["inputs"].host_inputs("ring_f32_r8_64MiB")
    kw = dict(proto="simple", launch="fused") if form == "fused" else dict(proto="ll")
    (y,) = run_allreduce(env, x, "float32", algo="tree", **kw)
    assert y.tobytes() == env["orc"].tree_allreduce(x).tobytes()
    check_tolerance(env, y, x, "float32")


def test_tree_fused_unaligned_views_take_single_elements(env, capfd):
    """Rows of a view that starts 4 bytes into its allocation are not 16-byte
    aligned: the fused tree takes one element per thread there even where
    the grid (here 4 workgroups) would take 16-byte packs, bit-exact."""
    api, orc = env["api"], env["orc"]
    R, N = 8, 4096
    x = rand_input(env, "float32", R, N, seed=77)
    base = to_dev(env, np.zeros((R * N + 1,), np.float32), "float32")
    send = base[1:].view(R, N)
    send.copy_(to_dev(env, x, "float32"))
    out = poisoned(env, (R * N + 1,), "float32")[1:].view(R, N)
    comm = api.Comm(R, N, "float32", "tree", "simple", device=env["dev"], launch="fused", debug=1,
                    grid=4)
    capfd.readouterr()
    comm.allreduce(send, out)
    assert "vec=1" in capfd.readouterr().err
    aligned = poisoned(env, (R, N), "float32")
    capfd.readouterr()
    comm.allreduce(to_dev(env, x, "float32"), aligned)  # the same call, aligned: packs
    assert "vec=4" in capfd.readouterr().err
    assert from_dev(env, aligned, "float32").tobytes() == orc.tree_allreduce(x).tobytes()
    assert from_dev(env, out, "float32").tobytes() == orc.tree_allreduce(x).tobytes()
    assert comm.check() == api.AR_SUCCESS


def test_tree_fused_bf16_r16_gradient_bucket(env, capfd):
    """The fused tree on one gradient bucket's shape (R = 16 bfloat16,
    13,107,200 elements per rank, N(0,0.02)): 16-byte packs of 8 elements,
    float32 partials in two halves, bit-exact against the oracle's tree."""
    api, orc = env["api"], env["orc"]
    R, N = 16, 13_107_200
    x = rand_input(env, "bf16", R, N, seed=1605)
    (y,) = run_allreduce(env, x, "bf16", algo="tree", launch="fused", debug=1)
    assert "vec=8" in capfd.readouterr().err
    assert y.tobytes() == orc.tree_allreduce(x, "bf16").tobytes()
    check_tolerance(env, y, x, "bf16")


def test_tree_fused_int32_r16_large_ragged(env):
    """The fused tree at R = 16 on 4 Mi + 3 int32 per rank (odd N: one
    element per thread, looping over each half ~16 times, and tree A's half
    one element longer), against the oracle's tree and the exact int64
    sum."""
    R, N = 16, (1 << 22) + 3
    x = rand_input(env, "int32", R, N, seed=1603)
    (y,) = run_allreduce(env, x, "int32", algo="tree", launch="fused")
    assert y.tobytes() == env["orc"].tree_allreduce(x, "int32").tobytes()
    assert (y == x.astype(np.int64).sum(axis=0).astype(np.int32)[None, :]).all()


# ---------------------------------------------------------------- ragged sizes

@pytest.mark.parametrize("launch", LAUNCHES)
@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R", [2, 3, 5, 8, 16])
def test_ring_allreduce_ragged(env, launch, dtype, R):
    orc = env["orc"]
    for N in (1, 2, 7, 13, 64, 1000, 4097, 3 * 4096 + 5, 65536 + 40):
        x = rand_input(env, dtype, R, N, seed=1000 * R + N)
        (y,) = run_allreduce(env, x, dtype, launch=launch)
        assert y.tobytes() == orc.ring_allreduce(x, dtype).tobytes(), (R, N)
        check_tolerance(env, y, x, dtype)


def test_ring_zero_count_is_noop(env):
    torch, api = env["torch"], env["api"]
    comm = api.Comm(4, 16, "float32", device=env["dev"])
    send = torch.ones((4, 0), device=env["dev"])
    recv = torch.ones((4, 0), device=env["dev"])
    comm.allreduce(send, recv)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- summation order

@pytest.mark.parametrize("launch", LAUNCHES)
def test_ring_order_pins_in_random_data(env, launch):
    # In segment c the ring folds x_{c+1}, x_{c+2}, ..., x_c.  With
    # x_c = -T, x_{c+1} = T, every other rank 1 (T = 2^24) the float32 fold is
    # T + 1 -> T (tie to even) repeatedly, then T - T = 0: result 0, exact R-2.
    R, N = 8, 8 * 4096
    T = np.float32(2.0 ** 24)
    x = env["inputs"].draw("normal", R, N, seed=9)
    S = N // R
    for c in range(R):
        for e in (c * S, c * S + 1, c * S + S // 2, c * S + S - 1):
            x[:, e] = 1
            x[c, e] = -T
            x[(c + 1) % R, e] = T
    (y,) = run_allreduce(env, x, "float32", launch=launch)
    for c in range(R):
        for e in (c * S, c * S + 1, c * S + S // 2, c * S + S - 1):
            assert (y[:, e] == 0.0).all()
    assert y.tobytes() == env["orc"].ring_allreduce(x).tobytes()


# ---------------------------------------------------------------- RS / AG

@pytest.mark.parametrize("launch", LAUNCHES)
@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R", [2, 4, 8, 16])
def test_reduce_scatter_all_gather(env, launch, dtype, R):
    api, orc, torch = env["api"], env["orc"], env["torch"]
    for n in (1, 3, 8, 1000, 8192 + 8):
        N = n * R
        x = rand_input(env, dtype, R, N, seed=77 + n + R)
        comm = api.Comm(R, N, dtype, device=env["dev"], **ring_opts(launch))
        send = to_dev(env, x, dtype)
        shard = poisoned(env, (R, n), dtype)
        comm.reduce_scatter(send, shard)
        full = poisoned(env, (R, N), dtype)
        comm.all_gather(shard, full)
        ar = poisoned(env, (R, N), dtype)
        comm.allreduce(send, ar)
        rs, ag, y = from_dev(env, shard, dtype), from_dev(env, full, dtype), from_dev(env, ar, dtype)
        assert rs.tobytes() == orc.ring_reduce_scatter(x, dtype).tobytes(), (R, n)
        assert ag.tobytes() == y.tobytes(), (R, n)                      # RS o AG == AR
        assert ag.tobytes() == orc.ring_all_gather(rs, dtype).tobytes()
        assert y.tobytes() == orc.ring_allreduce(x, dtype).tobytes()
        # all-gather alone on unrelated data
        g = rand_input(env, dtype, R, n, seed=5 + n)
        out = poisoned(env, (R, N), dtype)
        comm.all_gather(to_dev(env, g, dtype), out)
        assert from_dev(env, out, dtype).tobytes() == np.tile(g.reshape(-1), (R, 1)).tobytes()
        assert comm.check() == api.AR_SUCCESS


@pytest.mark.parametrize("launch", ["fused", "step", "pipelined"])
@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R", [2, 8])
def test_scalar_vector_switch_boundary(env, launch, dtype, R):
    """Segments just under, at and over 2 KiB (where the ring forms switch
    from one element per lane to 16-byte slots), whole and with a ragged last
    segment: all-reduce, and reduce-scatter then all-gather, bit-exact."""
    api, orc = env["api"], env["orc"]
    es = 2 if dtype == "bf16" else 4
    for seg_bytes in (2032, 2048, 2064):
        S = seg_bytes // es
        for N in (R * S, R * S - 1):
            x = rand_input(env, dtype, R, N, seed=31 * seg_bytes + N)
            (y,) = run_allreduce(env, x, dtype, launch=launch)
            assert y.tobytes() == orc.ring_allreduce(x, dtype).tobytes(), (seg_bytes, N)
        comm = api.Comm(R, R * S, dtype, device=env["dev"], **ring_opts(launch))
        x = rand_input(env, dtype, R, R * S, seed=7 * seg_bytes)
        shard = poisoned(env, (R, S), dtype)
        comm.reduce_scatter(to_dev(env, x, dtype), shard)
        rs = from_dev(env, shard, dtype)
        assert rs.tobytes() == orc.ring_reduce_scatter(x, dtype).tobytes(), seg_bytes
        full = poisoned(env, (R, R * S), dtype)
        comm.all_gather(shard, full)
        assert from_dev(env, full, dtype).tobytes() == orc.ring_all_gather(rs, dtype).tobytes()
        assert comm.check() == api.AR_SUCCESS


@pytest.mark.parametrize("chunk_bytes", [16384, 49152, 524288])
@pytest.mark.parametrize("R", [3, 8, 16])
def test_pipelined_bf16_chunk_layouts(env, chunk_bytes, R):
    """The pipelined ring keeps a bf16 chunk's float32 partials as one run
    per 16-byte half, laid out by the chunk's number of whole slots: chunks
    of three sizes (two workgroups per rank, so no chunk is cut finer), each
    segment two whole chunks and a ragged third (125 whole 8-element slots
    and 3 elements).  All-reduce and reduce-scatter, bit-exact."""
    api, orc = env["api"], env["orc"]
    U = chunk_bytes // 2
    S = 2 * U + 1003
    N = R * S
    x = rand_input(env, "bf16", R, N, seed=R * 7 + chunk_bytes)
    (y,) = run_allreduce(env, x, "bf16", launch="pipelined", chunk_bytes=chunk_bytes, grid=2 * R)
    assert y.tobytes() == orc.ring_allreduce(x, "bf16").tobytes()
    comm = api.Comm(R, N, "bf16", device=env["dev"], launch="pipelined", chunk_bytes=chunk_bytes,
                    grid=2 * R)
    shard = poisoned(env, (R, S), "bf16")
    comm.reduce_scatter(to_dev(env, x, "bf16"), shard)
    assert from_dev(env, shard, "bf16").tobytes() == orc.ring_reduce_scatter(x, "bf16").tobytes()
    assert comm.check() == api.AR_SUCCESS
    comm.close()


def test_pipelined_bf16_largest_chunk(env):
    """The largest pipelined chunk: R = 3 bf16, segments of 2^29 + 512
    elements, whole-segment chunks (chunk size 0) and two workgroups per rank,
    so chunks stay as large as the library allows.  A chunk's float32
    partials take 4 bytes per element and must stay addressable by one buffer
    resource (below 2 GiB).  Sampled outputs -- each segment's ends and the
    elements around 2^28 and 2^29 into it -- against the oracle, and no
    output element left unwritten."""
    torch, api, orc = env["torch"], env["api"], env["orc"]
    R = 3
    S = (1 << 29) + 512
    N = R * S
    g = torch.Generator(device=env["dev"])
    g.manual_seed(29)
    send = torch.randn((R, N), generator=g, device=env["dev"], dtype=torch.bfloat16)
    recv = torch.full_like(send, float("nan"))
    comm = api.Comm(R, N, "bf16", device=env["dev"], launch="pipelined", chunk_bytes=0,
                    grid=2 * R, timeout_us=30_000_000)
    comm.allreduce(send, recv)
    torch.cuda.synchronize()
    assert comm.check() == api.AR_SUCCESS
    offs = sorted({0, 1, 2, 3, S - 4, S - 3, S - 2, S - 1}
                  | {b + d for b in (1 << 28, 1 << 29) for d in range(-8, 8)})
    idx = np.array([c * S + o for c in range(R) for o in offs], dtype=np.int64)
    ti = torch.from_numpy(idx).to(env["dev"])
    xs = send[:, ti].view(torch.int16).cpu().numpy().view(np.uint16)
    ys = recv[:, ti].view(torch.int16).cpu().numpy().view(np.uint16)
    # segment c's samples sit in columns [c*m, (c+1)*m) of [R, R*m]: the same fold
    assert ys.tobytes() == orc.ring_allreduce(np.ascontiguousarray(xs), "bf16").tobytes()
    assert not torch.isnan(recv).any().item()
    comm.close()
    del send, recv, comm
    torch.cuda.empty_cache()


def test_ll_epochs_restart_before_they_wrap(env):
    """LL flags are 32-bit epochs advanced once per launch; every 2^30 tree or
    ring + LL launches the library clears the lines and epochs on the stream
    before the next such launch.  Forced from the host: the ring + LL epoch
    word (control word 4 of the workspace) set to 2^31 - 1, where the next
    launch's reduce flag 2 * epoch would wrap to 0 -- the value of every line
    not written since the clear -- and the launch count set to the reset
    point.  The next call, over more lines than any before, must match the
    oracle, and the count restarts; the tree likewise."""
    torch, api, orc = env["torch"], env["api"], env["orc"]
    R = 4
    comm = api.Comm(R, 1 << 16, "float32", "ring", "ll", device=env["dev"])
    for N, reset in ((1000, False), (1 << 16, True)):
        x = rand_input(env, "float32", R, N, seed=N)
        if reset:
            comm.workspace[:256].view(torch.int32)[4] = 2 ** 31 - 1
            comm.set_option(api.AR_OPT_DEBUG_LL_LAUNCHES, 1 << 30)
        recv = poisoned(env, (R, N), "float32")
        comm.allreduce(to_dev(env, x, "float32"), recv)
        assert from_dev(env, recv, "float32").tobytes() == orc.ring_allreduce(x).tobytes(), N
        assert comm.check() == api.AR_SUCCESS
    launches = comm.get_option(api.AR_OPT_DEBUG_LL_LAUNCHES)
    assert 1 <= launches < 100  # counted again from the reset
    assert int(comm.workspace[:256].view(torch.int32)[4].item()) == launches
    comm.close()
    tree = api.Comm(R, 1 << 16, "float32", "tree", "ll", device=env["dev"])
    for N in (1000, 1 << 16):
        x = rand_input(env, "float32", R, N, seed=N + 1)
        tree.set_option(api.AR_OPT_DEBUG_LL_LAUNCHES, 1 << 30)
        recv = poisoned(env, (R, N), "float32")
        tree.allreduce(to_dev(env, x, "float32"), recv)
        assert from_dev(env, recv, "float32").tobytes() == orc.tree_allreduce(x).tobytes(), N
        assert 1 <= tree.get_option(api.AR_OPT_DEBUG_LL_LAUNCHES) < 100
    assert tree.check() == api.AR_SUCCESS
    tree.close()


def _ncu(env):
    import torch
    return torch.cuda.get_device_properties(env["dev"]).multi_processor_count


@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R", [3, 8, 16])
@pytest.mark.parametrize("channels", [1, 2])
def test_fused_scalar_tiles_up_to_one_per_cu(env, dtype, R, channels):
    """The fused form keeps its scalar path (tiles of 256 elements, one per
    thread) while those tiles number at most one per CU, and takes the vector
    path beyond: 16-byte aligned segments just under, at and just over the
    switch (so both sides run), whole and ragged (a ragged count is not
    aligned and stays scalar), out of place and in place, and reduce-scatter
    then all-gather, bit-exact against the oracle."""
    api, orc = env["api"], env["orc"]
    ncu = _ncu(env)
    per_seg = max(1, ncu // R) * 256 * channels  # elements per segment at the switch
    for S in (per_seg - 8, per_seg, per_seg + 8):
        for N in (R * S, R * S - 3):
            x = rand_input(env, dtype, R, N, seed=17 * S + N + R)
            comm = api.Comm(R, N, dtype, device=env["dev"], launch="fused", channels=channels)
            strides = [api.ar_ring_channel_stride(comm.handle, k) for k in range(channels)]
            ref = orc.ring_allreduce(x, dtype, strides=strides)
            send = to_dev(env, x, dtype)
            recv = poisoned(env, (R, N), dtype)
            comm.allreduce(send, recv)
            assert from_dev(env, recv, dtype).tobytes() == ref.tobytes(), (S, N)
            comm.allreduce(send, send)  # in place: the hand-off goes through the workspace
            assert from_dev(env, send, dtype).tobytes() == ref.tobytes(), (S, N, "in place")
            assert comm.check() == api.AR_SUCCESS
        comm = api.Comm(R, R * S, dtype, device=env["dev"], launch="fused", channels=channels)
        strides = [api.ar_ring_channel_stride(comm.handle, k) for k in range(channels)]
        x = rand_input(env, dtype, R, R * S, seed=5 * S + R)
        shard = poisoned(env, (R, S), dtype)
        comm.reduce_scatter(to_dev(env, x, dtype), shard)
        rs = from_dev(env, shard, dtype)
        assert rs.tobytes() == orc.ring_reduce_scatter(x, dtype, strides=strides).tobytes(), S
        full = poisoned(env, (R, R * S), dtype)
        comm.all_gather(shard, full)
        assert from_dev(env, full, dtype).tobytes() == \
            orc.ring_all_gather(rs, dtype, strides=strides).tobytes(), S
        assert comm.check() == api.AR_SUCCESS


@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R", [3, 8])
def test_ll_one_line_per_thread_switch(env, dtype, R):
    """The LL kernels take one line per thread while every workgroup has at
    most one 256-line sub-block, four above: ring + LL and the tree at counts
    on both sides of that switch, bit-exact against the oracle."""
    orc = env["orc"]
    ncu = _ncu(env)
    # ring + LL: sub-blocks per segment up to the workgroups per rank (ncu / R)
    s_ring = max(1, ncu // R) * 256
    # tree: lines per tree half up to the workgroups per (tree, rank) (ncu / 2R)
    h_tree = max(1, ncu // (2 * R)) * 256
    for N in (R * s_ring, R * s_ring + R, R * (s_ring + 256) + 1):
        x = rand_input(env, dtype, R, N, seed=N + R)
        (y,) = run_allreduce(env, x, dtype, launch="ll")
        assert y.tobytes() == orc.ring_allreduce(x, dtype).tobytes(), ("ring-LL", N)
    for N in (2 * h_tree, 2 * h_tree + 2, 2 * (h_tree + 256) + 1):
        x = rand_input(env, dtype, R, N, seed=3 * N + R)
        (y,) = run_allreduce(env, x, dtype, "tree", "ll")
        assert y.tobytes() == orc.tree_allreduce(x, dtype).tobytes(), ("tree", N)


# ---------------------------------------------------------------- tree + LL, R = 8, 8 B .. 256 KiB per rank

def test_tree_ll_r8_8B_to_256KiB(env):
    orc, inputs = env["orc"], env["inputs"]
    for nbytes in [2 ** k for k in range(3, 19)]:
        N = nbytes // 4
        x = inputs.draw("uniform_pm1", 8, N, seed=4)
        outs = run_allreduce(env, x, "float32", "tree", "ll", reps=3)
        ref = orc.tree_allreduce(x)
        for y in outs:  # repeated calls: the LL epoch advances each time
            assert y.tobytes() == ref.tobytes(), nbytes
        check_tolerance(env, outs[0], x, "float32")


@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R", [2, 3, 5, 8, 13, 16, 64])
def test_tree_ll_ragged(env, dtype, R):
    orc = env["orc"]
    for N in (1, 2, 3, 17, 1000, 2 * 65536 + 7):
        x = rand_input(env, dtype, R, N, seed=31 * R + N)
        outs = run_allreduce(env, x, dtype, "tree", "ll", reps=2)
        ref = orc.tree_allreduce(x, dtype)
        for y in outs:
            assert y.tobytes() == ref.tobytes(), (R, N)


@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R", list(range(2, 18)) + [32, 33, 64])
def test_tree_fused_matches_the_tree_order(env, capfd, dtype, R):
    """The fused tree (a tree call with the fused launch and a protocol other
    than LL, R <= 16 or R = 32 or 64, the trees compiled in for each R;
    bfloat16 partials in two 16-bit halves): the LL tree's fold order, so
    bit-exact against the oracle's tree -- every
    operator, ragged sizes and sizes taking 16-byte packs, in place, and a
    grid of 3 workgroups that loops over the elements -- and the library's
    debug line shows the fused kernel ran, and in which width.  At other R
    the same call takes the LL tree."""
    api, orc = env["api"], env["orc"]
    fused = R <= 16 or R in (32, 64)
    ops = ["sum", "max", "min"] + ([] if dtype == "int32" else ["avg"])
    Nmax = 4 * 4096 + 37
    # (a grid of 3 for the fused form only: the LL tree needs 2R resident
    # workgroups and refuses a smaller grid)
    for op, grid in [(op, None) for op in ops] + ([("sum", 3)] if fused else []):
        opts = {} if grid is None else {"grid": grid}
        comm = api.Comm(R, Nmax, dtype, "tree", "simple", device=env["dev"], launch="fused",
                        redop=op, debug=1, **opts)
        want = ((api.AR_TREE, api.AR_SIMPLE, api.AR_LAUNCH_FUSED) if fused
                else (api.AR_TREE, api.AR_LL, api.AR_LAUNCH_AUTO))
        assert comm.plan(Nmax)[:3] == want
        # N a multiple of two packs above the grid's threads takes 16-byte
        # packs (4 or 8 elements per thread): here with the grid of 3 (768
        # threads)
        for N in (1, 2, 7, 8, 1000, 4097, 4 * 4096, Nmax):
            x = rand_input(env, dtype, R, N, seed=R * 131 + N + len(op))
            ref = orc.tree_allreduce(x, dtype, op=op)
            capfd.readouterr()
            send = to_dev(env, x, dtype)
            recv = poisoned(env, (R, N), dtype)
            comm.allreduce(send, recv)
            assert from_dev(env, recv, dtype).tobytes() == ref.tobytes(), (op, grid, N)
            err = capfd.readouterr().err
            assert ("ar: tree-fused" in err) == fused and ("ar: tree-LL" in err) != fused, err
            if fused:
                pack = 8 if dtype == "bf16" else 4
                vec = grid is not None and N % (2 * pack) == 0 and N > grid * 256 and R <= 16
                assert ("vec=%d" % (pack if vec else 1)) in err, err
            if fused and grid is not None:
                assert int(re.search(r"tree-fused .* grid=(\d+)", err).group(1)) <= grid, err
            comm.allreduce(send, send)  # in place
            assert from_dev(env, send, dtype).tobytes() == ref.tobytes(), (op, grid, N, "in place")
        assert comm.check() == api.AR_SUCCESS
        comm.close()


def test_tree_epochs_across_sizes(env):
    """The tree keeps one epoch per group of 64 lines.  Calls of different
    sizes on one communicator use different grids and different sets of
    groups (a group one call leaves alone is used again by a later one, over
    lines that still hold older flags), and the largest takes two launches;
    every call must match the oracle."""
    api, orc = env["api"], env["orc"]
    R, Nmax = 8, 2 * 65536 + 7
    comm = api.Comm(R, Nmax, "float32", "tree", "ll", device=env["dev"])
    for N in (Nmax, 1, 300, 40_000, 3, Nmax, 5000, 129, 40_000, 1, 70_001):
        x = rand_input(env, "float32", R, N, seed=N + 1)
        out = poisoned(env, (R, N), "float32")
        comm.allreduce(to_dev(env, x, "float32"), out)
        assert from_dev(env, out, "float32").tobytes() == orc.tree_allreduce(x).tobytes(), N
    assert comm.check() == api.AR_SUCCESS


def test_tree_order_pin(env):
    # Tree A at R = 8: P(2) = x2 + x1 + x3 = (T + 1) -> T, T - T = 0 with
    # x2 = T, x1 = 1, x3 = -T; exact sum 1.
    T = np.float32(2.0 ** 24)
    x = np.zeros((8, 64), np.float32)
    x[2, 0], x[1, 0], x[3, 0] = T, 1, -T
    (y,) = run_allreduce(env, x, "float32", "tree", "ll")
    assert (y[:, 0] == 0.0).all()


def test_auto_selects_tree_then_ring(env):
    api = env["api"]
    x = env["inputs"].draw("normal", 8, 1 << 16, seed=12)
    comm = api.Comm(8, 1 << 16, "float32", "auto", device=env["dev"], tree_max_bytes=4096,
                    launch="pipelined")
    assert comm.plan(1024)[0] == api.AR_TREE and comm.plan(1 << 16)[0] == api.AR_RING
    for N, ref in ((1024, env["orc"].tree_allreduce(x[:, :1024].copy())),
                   (1 << 16, env["orc"].ring_allreduce(x))):
        send = to_dev(env, x[:, :N].copy(), "float32")
        recv = poisoned(env, (8, N), "float32")
        comm.allreduce(send, recv)
        assert from_dev(env, recv, "float32").tobytes() == ref.tobytes()


@pytest.mark.parametrize("launch", ["pipelined", "step"])
def test_protocol_auto_runs_the_planned_protocol(env, capfd, launch):
    """With AR_PROTO_AUTO each call runs the algorithm and protocol ar_plan
    reports (the library's debug line names the kernels it launched):
    tree + LL, ring + LL or the simple-protocol ring by size; all-reduce,
    and reduce-scatter + all-gather weighed by the full row, bit-exact."""
    api, orc = env["api"], env["orc"]
    R, Nmax = 8, 1 << 20
    x = env["inputs"].draw("normal", R, Nmax, seed=13)
    comm = api.Comm(R, Nmax, "float32", "auto", "auto", device=env["dev"], launch=launch, debug=1)
    tree_max = api.ar_auto_tree_max_bytes(comm.handle)
    assert 0 < tree_max < 600_000 // 4 * 4
    seen = set()
    # 4 KiB (tree), 600 KB (ring + LL), 4 MiB (the simple form) per rank
    for N in (1024, 150_000, Nmax):
        algo, proto, _ = comm.plan(N)
        kind = "tree" if algo == api.AR_TREE else "ring-ll" if proto == api.AR_LL else "simple"
        seen.add(kind)
        xs = np.ascontiguousarray(x[:, :N])
        send = to_dev(env, xs, "float32")
        recv = poisoned(env, (R, N), "float32")
        capfd.readouterr()
        comm.allreduce(send, recv)
        got = from_dev(env, recv, "float32")
        err = capfd.readouterr().err
        ref = orc.tree_allreduce(xs) if kind == "tree" else orc.ring_allreduce(xs)
        assert got.tobytes() == ref.tobytes(), (N, kind)
        assert ("ar: tree-LL" in err) == (kind == "tree"), (N, kind, err)
        assert ("ar: ring-LL" in err) == (kind == "ring-ll"), (N, kind, err)
        assert ("launch=" + launch in err) == (kind == "simple"), (N, kind, err)
    assert seen == {"tree", "ring-ll", "simple"}
    # reduce-scatter and all-gather are ring only; their size is the full row
    for N in (150_000 // R * R, Nmax):
        proto = comm.plan(N)[1] if comm.plan(N)[0] == api.AR_RING else api.AR_LL
        xs = np.ascontiguousarray(x[:, :N])
        shard = poisoned(env, (R, N // R), "float32")
        full = poisoned(env, (R, N), "float32")
        capfd.readouterr()
        comm.reduce_scatter(to_dev(env, xs, "float32"), shard)
        comm.all_gather(shard, full)
        rs = from_dev(env, shard, "float32")
        err = capfd.readouterr().err
        assert rs.tobytes() == orc.ring_reduce_scatter(xs).tobytes()
        assert from_dev(env, full, "float32").tobytes() == orc.ring_all_gather(rs).tobytes()
        assert ("ar: ring-LL" in err) == (proto == api.AR_LL), (N, err)
    assert comm.check() == api.AR_SUCCESS
    comm.close()


# ---------------------------------------------------------------- wave tiles

# 16-byte slots per lane of the fused form's wave tile (kWaveSlots): a tile is
# 64 * 2 slots, i.e. 512 elements of 32-bit T or 1024 of bf16, per rank row
TILE_SLOTS = 128


@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R", [2, 3, 8, 16])
@pytest.mark.parametrize("channels", [1, 2])
def test_fused_wave_tile_seams(env, dtype, R, channels):
    """The fused vector path around tile boundaries: every segment a whole
    number of tiles (the lean kernel), one element more or less (the kernel
    with the checked path for a segment's last tile), and only the last
    segment short.  All-reduce (out of place and in place), reduce-scatter and
    all-gather against the oracle, with one and two ring channels."""
    api, orc, torch = env["api"], env["orc"], env["torch"]
    V = 8 if dtype == "bf16" else 4
    te = TILE_SLOTS * V  # elements per rank row in one tile
    K = min(channels, len([m for m in range(1, R) if np.gcd(m, R) == 1]))
    strides = [1, R - 1][:K]
    for segs in (te, 3 * te, te + V, 3 * te - V, 2 * te + 8):
        for N in (R * segs, R * segs - V if R * segs - V > (R - 1) * segs else R * segs - 1):
            x = rand_input(env, dtype, R, N, seed=N * 7 + R)
            comm = api.Comm(R, N, dtype, device=env["dev"], launch="fused", channels=K)
            send = to_dev(env, x, dtype)
            recv = poisoned(env, (R, N), dtype)
            comm.allreduce(send, recv)
            want = orc.ring_allreduce(x, dtype, strides=strides)
            assert from_dev(env, recv, dtype).tobytes() == want.tobytes(), (N, "ar")
            inplace = to_dev(env, x, dtype)
            comm.allreduce(inplace, inplace)
            assert from_dev(env, inplace, dtype).tobytes() == want.tobytes(), (N, "in place")
            if N % R == 0:
                shard = poisoned(env, (R, N // R), dtype)
                comm.reduce_scatter(send, shard)
                rs = orc.ring_reduce_scatter(x, dtype, strides=strides)
                assert from_dev(env, shard, dtype).tobytes() == rs.tobytes(), (N, "rs")
                full = poisoned(env, (R, N), dtype)
                comm.all_gather(to_dev(env, rs, dtype), full)
                ag = orc.ring_all_gather(rs, dtype, strides=strides)
                assert from_dev(env, full, dtype).tobytes() == ag.tobytes(), (N, "ag")
            assert comm.check() == api.AR_SUCCESS
            comm.close()


@pytest.mark.parametrize("grid", [1, 3, 64, 4096])
def test_fused_staging_with_any_grid(env, grid):
    """bf16 hands its float32 running value on through one staging slot per
    wave; the launch is capped at the waves the staging holds, whatever grid
    is asked for, and a grid smaller than the tiles loops over them."""
    api, orc = env["api"], env["orc"]
    R, N = 16, 16 * 1024 * 40 + 16 * 8
    x = rand_input(env, "bf16", R, N, seed=grid)
    (y,) = run_allreduce(env, x, "bf16", launch="fused", grid=grid)
    assert y.tobytes() == orc.ring_allreduce(x, "bf16").tobytes()


# ---------------------------------------------------------------- gradient buckets, R = 16 bf16, 40 x 25 MiB

def test_gradient_buckets_bf16_r16_40x25MiB(env):
    """40 buckets x 13,107,200 bf16 per rank, R = 16: reduce-scatter then
    all-gather equals all-reduce bit for bit on every bucket.  Every bucket is
    also compared with the oracle: 64 sampled elements of each segment (the
    fold of an element depends only on its segment, so the samples laid out
    as [R, R*64] fold in the same order), the all-reduce output and the
    reduce-scatter shards at those elements; buckets 0 and 39 in full."""
    api, orc, inputs, torch = env["api"], env["orc"], env["inputs"], env["torch"]
    w = inputs.WORKLOADS["buckets_bf16_r16"]
    R, N, B = w["R"], w["count"], w["buckets"]
    n = N // R
    comm = api.Comm(R, N, "bf16", "ring", device=env["dev"])
    shard = torch.empty((R, n), dtype=torch.bfloat16, device=env["dev"])
    full = torch.empty((R, N), dtype=torch.bfloat16, device=env["dev"])
    ar = torch.empty((R, N), dtype=torch.bfloat16, device=env["dev"])
    rng, m = np.random.default_rng(5), 64
    for b in range(B):
        x = inputs.device_bucket_bf16(R, N, w["seed"], b, env["dev"])
        full.fill_(float("nan"))
        comm.reduce_scatter(x, shard)
        comm.all_gather(shard, full)
        comm.allreduce(x, ar)
        assert torch.equal(full.view(torch.int16), ar.view(torch.int16)), b
        assert torch.equal(ar.view(torch.int16), ar[0:1].expand(R, N).view(torch.int16)), b
        idx = _segment_samples(rng, N, R, m)
        ti = torch.from_numpy(idx).to(env["dev"])
        ref = orc.ring_allreduce(from_dev(env, x[:, ti].contiguous(), "bf16"), "bf16")
        assert from_dev(env, ar[:, ti].contiguous(), "bf16").tobytes() == ref.tobytes(), b
        sh = from_dev(env, shard, "bf16")
        for c in range(R):
            cols = idx[c * m:(c + 1) * m]
            assert np.array_equal(sh[c, cols - c * n], ref[c, c * m:(c + 1) * m]), (b, c)
        if b in (0, B - 1):
            xh = from_dev(env, x, "bf16")
            y = from_dev(env, ar, "bf16")
            assert y.tobytes() == orc.ring_allreduce(xh, "bf16").tobytes(), b
            assert from_dev(env, shard, "bf16").tobytes() == orc.ring_reduce_scatter(xh, "bf16").tobytes()
            check_tolerance(env, y[:1], xh, "bf16")
    assert comm.check() == api.AR_SUCCESS


# ---------------------------------------------------------------- edges

def test_unaligned_views_use_the_scalar_path(env):
    torch, api, orc = env["torch"], env["api"], env["orc"]
    R, N = 8, 4099
    x = env["inputs"].draw("normal", R, N, seed=3)
    base = torch.zeros(R * N + 1, dtype=torch.float32, device=env["dev"])
    send = base[1:].view(R, N)                           # 4-byte misaligned
    send.copy_(torch.from_numpy(x).to(env["dev"]))
    rbase = torch.full((R * N + 3,), float("nan"), device=env["dev"])
    recv = rbase[3:].view(R, N)
    for launch in LAUNCHES:
        comm = api.Comm(R, N, "float32", device=env["dev"], **ring_opts(launch))
        comm.allreduce(send, recv)
        assert from_dev(env, recv, "float32").tobytes() == orc.ring_allreduce(x).tobytes()


def _offset_view(env, shape, dtype, off):
    """A contiguous [rows, cols] view starting `off` elements into an
    allocation of 0xFF bytes, so that its rows are not 16-byte aligned."""
    torch = env["torch"]
    tdt = {"int32": torch.int32, "float32": torch.float32, "bf16": torch.bfloat16}[dtype]
    base = torch.empty(shape[0] * shape[1] + off, dtype=tdt, device=env["dev"])
    base.view(torch.uint8).fill_(0xFF)
    return base[off:].view(*shape)


@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
def test_unaligned_views_with_more_tiles_than_the_grid(env, dtype):
    """Rows that are not 16-byte aligned take the fused form's scalar path at
    any size.  Its default grid is 8 workgroups per CU; here the segments hold
    more 256-element tiles than that, so each workgroup loops over several,
    with a ragged last segment; then a small call with a grid of 3.
    All-reduce, reduce-scatter and all-gather, bit-exact."""
    api, orc = env["api"], env["orc"]
    R = 8
    S = 256 * _ncu(env) + 300  # ceil(S / 256) * R tiles > 8 per CU
    for N, grid in ((R * S - 3, None), (R * 700 - 5, 3)):
        opts = {} if grid is None else {"grid": grid}
        comm = api.Comm(R, N, dtype, device=env["dev"], launch="fused", **opts)
        x = rand_input(env, dtype, R, N, seed=N)
        send = _offset_view(env, (R, N), dtype, 1)
        send.copy_(to_dev(env, x, dtype))
        recv = _offset_view(env, (R, N), dtype, 3)
        comm.allreduce(send, recv)
        assert from_dev(env, recv, dtype).tobytes() == orc.ring_allreduce(x, dtype).tobytes(), \
            (N, grid, "ar")
        n = N // R
        xs = np.ascontiguousarray(x[:, :R * n])
        rsend = _offset_view(env, (R, R * n), dtype, 1)
        rsend.copy_(to_dev(env, xs, dtype))
        shard = _offset_view(env, (R, n), dtype, 3)
        comm.reduce_scatter(rsend, shard)
        rs = orc.ring_reduce_scatter(xs, dtype)
        assert from_dev(env, shard, dtype).tobytes() == rs.tobytes(), (N, grid, "rs")
        full = _offset_view(env, (R, R * n), dtype, 1)
        comm.all_gather(shard, full)
        assert from_dev(env, full, dtype).tobytes() == orc.ring_all_gather(rs, dtype).tobytes(), \
            (N, grid, "ag")
        assert comm.check() == api.AR_SUCCESS
        comm.close()


def test_argument_errors(env):
    torch, api = env["torch"], env["api"]
    comm = api.Comm(4, 64, "float32", device=env["dev"])
    a = torch.zeros((4, 64), device=env["dev"])
    big = torch.zeros((4, 65), device=env["dev"])
    with pytest.raises(api.ArError) as e:
        comm.allreduce(big, torch.zeros_like(big))
    assert e.value.status == api.AR_ERR_INVALID_ARG
    tcomm = api.Comm(4, 64, "float32", "tree", "ll", device=env["dev"])
    with pytest.raises(api.ArError) as e:
        tcomm.reduce_scatter(a, torch.zeros((4, 16), device=env["dev"]))
    assert e.value.status == api.AR_ERR_UNSUPPORTED
    # shard counts whose product with R wraps around size_t are refused
    # before anything is launched (raw C calls: the pointers are never used)
    L = api.lib()
    huge = (1 << 64) // 4 + 1  # 4 * huge wraps to 4
    p = a.data_ptr()
    assert L.ar_reduce_scatter(comm.handle, p, p + 4096, huge, None) == api.AR_ERR_INVALID_ARG
    assert L.ar_all_gather(comm.handle, p, p + 4096, huge, None) == api.AR_ERR_INVALID_ARG
    assert L.ar_reduce_scatter(comm.handle, p, p + 4096, 17, None) == api.AR_ERR_INVALID_ARG
    assert comm.check() == api.AR_SUCCESS


@pytest.mark.parametrize("launch", LAUNCHES)
def test_repeat_runs_bit_identical(env, launch):
    x = env["inputs"].draw("normal", 8, 1 << 20, seed=21)
    outs = run_allreduce(env, x, "float32", launch=launch, reps=5)
    for y in outs[1:]:
        assert y.tobytes() == outs[0].tobytes()


# ---------------------------------------------------------------- graphs

@pytest.mark.parametrize("variant", ["fused", "step", "pipelined", "ll", "tree", "tree-fused"])
def test_graph_replay_matches_eager(env, variant):
    """Capture one call in a HIP graph and replay it several times with eager
    calls and synchronizations in between; every replay must equal the eager
    result (the tree's LL epoch and the pipelined flags' base live on the
    device, so replays stay correct)."""
    torch, api = env["torch"], env["api"]
    R, N = 8, 40_000
    x = env["inputs"].draw("normal", R, N, seed=17)
    if variant.startswith("tree"):
        kw = dict(proto="ll") if variant == "tree" else dict(proto="simple", launch="fused")
        comm = api.Comm(R, N, "float32", "tree", device=env["dev"], **kw)
        ref = env["orc"].tree_allreduce(x)
    else:
        comm = api.Comm(R, N, "float32", device=env["dev"], **ring_opts(variant))
        ref = env["orc"].ring_allreduce(x)
    send = to_dev(env, x, "float32")
    eager = poisoned(env, (R, N), "float32")
    comm.allreduce(send, eager)
    assert from_dev(env, eager, "float32").tobytes() == ref.tobytes()
    out = poisoned(env, (R, N), "float32")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        comm.allreduce(send, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        comm.allreduce(send, out)
    for i in range(4):
        out.view(torch.uint8).fill_(0xFF)
        comm.allreduce(send, eager)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert from_dev(env, out, "float32").tobytes() == ref.tobytes(), i
        assert from_dev(env, eager, "float32").tobytes() == ref.tobytes(), i
    assert comm.check() == api.AR_SUCCESS


# ---------------------------------------------------------------- the sweep's largest size, 1 GiB per rank

def _segment_samples(rng, N, R, m):
    """m element indices from each ring segment of an N-element row, in
    segment order, always including each segment's first and last element."""
    S = -(-N // R)
    idx = []
    for c in range(R):
        lo, hi = min(c * S, N), min((c + 1) * S, N)
        pick = set([lo, hi - 1]) | set(rng.integers(lo, hi, size=m - 2).tolist())
        pick = sorted(pick)
        while len(pick) < m:  # keep exactly m per segment
            pick.append(pick[-1])
        idx.extend(pick[:m])
    return np.array(idx, dtype=np.int64)


@pytest.mark.parametrize("variant", LAUNCHES + ["tree", "tree-fused", "tree-fused-packed"])
def test_counts_beyond_2_32_elements_sampled(env, variant):
    """R = 2 bf16 with 2^32 + 1000 elements (8 GiB) per rank, so element
    indices pass both 2^31 and 2^32: every form, sampled outputs -- each
    segment's ends and the elements around 2^31 and 2^32 -- against the
    oracle (with two ranks the fold is one float32 addition, the same in
    every order and layout), and no output element left unwritten.  The
    fused tree runs one element per thread there, and 16-byte packs at
    2^32 + 1008 (a multiple of two packs)."""
    torch, api, orc = env["torch"], env["api"], env["orc"]
    R, N = 2, (1 << 32) + (1008 if variant == "tree-fused-packed" else 1000)
    g = torch.Generator(device=env["dev"])
    g.manual_seed(32)
    send = torch.randn((R, N), generator=g, device=env["dev"], dtype=torch.bfloat16)
    recv = torch.full_like(send, float("nan"))
    if variant == "tree":
        comm = api.Comm(R, N, "bf16", "tree", "ll", device=env["dev"])
    elif variant.startswith("tree-fused"):
        comm = api.Comm(R, N, "bf16", "tree", device=env["dev"], launch="fused")
    else:
        comm = api.Comm(R, N, "bf16", device=env["dev"], **ring_opts(variant))
    comm.allreduce(send, recv)
    torch.cuda.synchronize()
    assert comm.check() == api.AR_SUCCESS
    S = -(-N // R)
    picks = {0, 1, S - 1, S, S + 1, N - 2, N - 1}
    picks |= {b + d for b in (1 << 31, 1 << 32) for d in range(-4, 4)}
    idx = np.array(sorted(picks), dtype=np.int64)
    ti = torch.from_numpy(idx).to(env["dev"])
    xs = send[:, ti].view(torch.int16).cpu().numpy().view(np.uint16)
    ys = recv[:, ti].view(torch.int16).cpu().numpy().view(np.uint16)
    assert ys.tobytes() == orc.ring_allreduce(np.ascontiguousarray(xs), "bf16").tobytes()
    assert not torch.isnan(recv).any().item()
    comm.close()
    del send, recv, comm
    torch.cuda.empty_cache()


@pytest.mark.parametrize("launch", ["auto", "step", "pipelined", "ll"])
def test_ring_f32_r8_1GiB_sampled(env, launch):
    """R = 8, fp32, 1 GiB per rank (the sweep's largest size) in the launch form
    the benchmark times: sampled outputs against the oracle.  The ring's fold
    for an element depends only on its segment, so m samples from each
    segment, laid out as an [R, R*m] array, have the same fold order there."""
    torch, api, orc = env["torch"], env["api"], env["orc"]
    R, N, m = 8, 1 << 28, 64
    g = torch.Generator(device=env["dev"])
    g.manual_seed(3)
    send = torch.randn((R, N), generator=g, device=env["dev"], dtype=torch.float32)
    recv = torch.full_like(send, float("nan"))
    comm = api.Comm(R, N, "float32", device=env["dev"],
                    **(dict(algo="ring") if launch == "auto" else ring_opts(launch)))
    comm.allreduce(send, recv)
    torch.cuda.synchronize()
    assert comm.check() == api.AR_SUCCESS
    idx = _segment_samples(np.random.default_rng(0), N, R, m)
    ti = torch.from_numpy(idx).to(env["dev"])
    xs = send[:, ti].cpu().numpy()
    ys = recv[:, ti].cpu().numpy()
    ref = orc.ring_allreduce(np.ascontiguousarray(xs))
    assert ys.tobytes() == ref.tobytes()
    check_tolerance(env, ys, xs, "float32")
    # every element written: no NaN left anywhere (checked on the device)
    assert not torch.isnan(recv).any().item()
    del send, recv, comm
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- watchdog

@pytest.mark.parametrize("variant,mute", [("tree", 3), ("tree", 0), ("pipelined", 3), ("ll", 3)])
def test_watchdog_reports_timeout_and_recovers(env, variant, mute):
    """Forced from the host: one logical rank skips publishing, so its
    consumers' bounded waits (5 ms here) expire.  The kernel still finishes,
    ar_check reports AR_ERR_TIMEOUT once (clearing the LL lines and epochs
    too), and the next call is correct.  Rank
    0 is tree A's root: muted, it sends nothing down, but must still advance
    its line groups' epochs so that the next call uses fresh flags."""
    import time
    torch, api, orc = env["torch"], env["api"], env["orc"]
    R, N = 8, 4096
    x = env["inputs"].draw("normal", R, N, seed=23)
    if variant == "tree":
        comm = api.Comm(R, N, "float32", "tree", "ll", device=env["dev"], timeout_us=5000)
        ref = orc.tree_allreduce(x)
    else:
        comm = api.Comm(R, N, "float32", device=env["dev"], timeout_us=5000, **ring_opts(variant))
        ref = orc.ring_allreduce(x)
    send = to_dev(env, x, "float32")
    recv = poisoned(env, (R, N), "float32")
    comm.allreduce(send, recv)            # warm (first call initialises the device facts)
    torch.cuda.synchronize()
    assert comm.check() == api.AR_SUCCESS
    comm.set_option(api.AR_OPT_DEBUG_MUTE_RANK, mute)
    t0 = time.perf_counter()
    comm.allreduce(send, recv)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert comm.check() == api.AR_ERR_TIMEOUT
    if variant in ("tree", "ll"):
        # the LL lines and epochs were cleared with the error word
        assert comm.get_option(api.AR_OPT_DEBUG_LL_LAUNCHES) == 0
    assert comm.check() == api.AR_SUCCESS  # the error word was cleared
    assert dt < 1.0, dt
    comm.set_option(api.AR_OPT_DEBUG_MUTE_RANK, -1)
    for _ in range(2):
        recv = poisoned(env, (R, N), "float32")
        comm.allreduce(send, recv)
        assert from_dev(env, recv, "float32").tobytes() == ref.tobytes()
    assert comm.check() == api.AR_SUCCESS


def test_measurement_utilities(env):
    """The streaming references and the LL ping-pong probe run and finish."""
    torch, api = env["torch"], env["api"]
    st = torch.cuda.current_stream().cuda_stream
    a = torch.randn(4099, device=env["dev"])
    b = torch.randn(4099, device=env["dev"])
    c = torch.empty_like(a)
    api.ar_stream_add(a.data_ptr(), b.data_ptr(), c.data_ptr(), a.numel(), st)
    torch.cuda.synchronize()
    assert torch.equal(c, a + b)
    d = torch.empty_like(a)
    api.ar_stream_copy(a.data_ptr(), d.data_ptr(), 4096 * 4, st)
    torch.cuda.synchronize()
    assert torch.equal(d[:4096], a[:4096])
    for rows in (1, 3, 8, 11):  # whole groups of 8 rows and a remainder
        src = torch.randn((rows, 12 * 512), device=env["dev"])  # 12 tiles of 2 KiB per row
        dst = torch.zeros_like(src)
        api.ar_stream_rows(src.data_ptr(), dst.data_ptr(), rows, src.shape[1] * 4, st)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), rows
    lines = torch.zeros(64, dtype=torch.int64, device=env["dev"])
    res = torch.ones(1, dtype=torch.int32, device=env["dev"])
    for apart in (1, 0):
        api.ar_ll_pingpong(lines.data_ptr(), res.data_ptr(), 1000, apart, 2_000_000, st)
        torch.cuda.synchronize()
        assert int(res.item()) == 0
        assert (int(lines[0].item()) >> 32) == 1000 and (int(lines[16].item()) >> 32) == 1000


# ---------------------------------------------------------------- operators, in place

@pytest.mark.parametrize("variant", LAUNCHES + ["tree"])
@pytest.mark.parametrize("dtype,op", [(d, o) for d in ("int32", "float32", "bf16")
                                      for o in ("max", "min", "avg")
                                      if not (d == "int32" and o == "avg")])  # refused: see below
def test_reduction_operators(env, variant, dtype, op):
    api, orc = env["api"], env["orc"]
    for R, N in ((3, 1001), (8, 8 * 4096 + 24), (16, 16 * 5)):
        x = rand_input(env, dtype, R, N, seed=R * 7 + N)
        if variant == "tree":
            (y,) = run_allreduce(env, x, dtype, "tree", "ll", redop=op)
            ref = orc.tree_allreduce(x, dtype, op=op)
        else:
            (y,) = run_allreduce(env, x, dtype, launch=variant, redop=op)
            ref = orc.ring_allreduce(x, dtype, op=op)
        assert y.tobytes() == ref.tobytes(), (R, N)
        if variant != "tree" and N % R == 0:
            comm = api.Comm(R, N, dtype, device=env["dev"], redop=op, **ring_opts(variant))
            shard = poisoned(env, (R, N // R), dtype)
            comm.reduce_scatter(to_dev(env, x, dtype), shard)
            assert from_dev(env, shard, dtype).tobytes() == orc.ring_reduce_scatter(x, dtype, op=op).tobytes()


def test_int32_average_is_refused(env):
    api = env["api"]
    comm = api.Comm(4, 64, "int32", device=env["dev"])
    with pytest.raises(api.ArError) as e:
        comm.set_option(api.AR_OPT_REDOP, api.AR_AVG)
    assert e.value.status == api.AR_ERR_INVALID_ARG


@pytest.mark.parametrize("variant", LAUNCHES + ["tree"])
@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
def test_in_place_allreduce(env, variant, dtype):
    api, orc, torch = env["api"], env["orc"], env["torch"]
    for R, N in ((2, 7), (5, 1003), (8, 1 << 16), (16, 16 * 4096 + 3)):
        x = rand_input(env, dtype, R, N, seed=31 + R + N)
        if variant == "tree":
            comm = api.Comm(R, N, dtype, "tree", "ll", device=env["dev"])
            ref = orc.tree_allreduce(x, dtype)
        else:
            comm = api.Comm(R, N, dtype, device=env["dev"], **ring_opts(variant))
            ref = orc.ring_allreduce(x, dtype)
        buf = to_dev(env, x, dtype)
        comm.allreduce(buf, buf)
        assert from_dev(env, buf, dtype).tobytes() == ref.tobytes(), (R, N)
        assert comm.check() == api.AR_SUCCESS
    # partial overlap is refused
    comm = api.Comm(4, 64, "float32", device=env["dev"])
    base = torch.zeros(4 * 64 + 64, device=env["dev"])
    with pytest.raises(api.ArError) as e:
        comm.allreduce(base[:256].view(4, 64), base[64:320].view(4, 64))
    assert e.value.status == api.AR_ERR_INVALID_USAGE


@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R", [2, 8, 64])
def test_ring_ll_multiple_pieces(env, dtype, R):
    """Counts whose segments exceed one launch's line capacity run as several
    ring-LL launches (each with a fresh epoch)."""
    orc = env["orc"]
    cap = min(10 ** 9, max(64, (1 << 21) // (R * R)))
    N = R * (2 * cap + 37) + 5
    x = rand_input(env, dtype, R, N, seed=R + 91)
    outs = run_allreduce(env, x, dtype, launch="ll", reps=2)
    ref = orc.ring_allreduce(x, dtype)
    for y in outs:
        assert y.tobytes() == ref.tobytes()


# ---------------------------------------------------------------- R = 64, concurrency

@pytest.mark.parametrize("launch", LAUNCHES)
@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
def test_ring_largest_rank_count(env, launch, dtype):
    """R = 64, the largest communicator, in every ring form: ragged and whole
    segments, all-reduce and reduce-scatter."""
    api, orc = env["api"], env["orc"]
    R = 64
    for N in (R * 1000 + 7, R * 4096):
        x = rand_input(env, dtype, R, N, seed=640 + N)
        (y,) = run_allreduce(env, x, dtype, launch=launch)
        assert y.tobytes() == orc.ring_allreduce(x, dtype).tobytes(), N
        check_tolerance(env, y, x, dtype)
    n = 1024
    x = rand_input(env, dtype, R, R * n, seed=641)
    comm = api.Comm(R, R * n, dtype, device=env["dev"], **ring_opts(launch))
    shard = poisoned(env, (R, n), dtype)
    comm.reduce_scatter(to_dev(env, x, dtype), shard)
    assert from_dev(env, shard, dtype).tobytes() == orc.ring_reduce_scatter(x, dtype).tobytes()
    assert comm.check() == api.AR_SUCCESS


@pytest.mark.parametrize("pair", [("fused", "fused"), ("fused", "step"), ("step", "step")])
def test_two_comms_on_two_streams(env, pair):
    """Two communicators, each with its own workspace, run at the same time on
    two streams and both stay exact (the forms without cross-workgroup waits;
    LL and pipelined launches need the whole device resident and must not
    overlap each other)."""
    torch, api, orc = env["torch"], env["api"], env["orc"]
    xs = [env["inputs"].draw("normal", 8, 1 << 20, seed=51),
          env["inputs"].draw("normal", 4, (1 << 20) + 13, seed=52)]
    refs = [orc.ring_allreduce(x) for x in xs]
    comms = [api.Comm(x.shape[0], x.shape[1], "float32", device=env["dev"], launch=l)
             for x, l in zip(xs, pair)]
    sends = [to_dev(env, x, "float32") for x in xs]
    recvs = [poisoned(env, x.shape, "float32") for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for c, s_, r, st in zip(comms, sends, recvs, streams):
            with torch.cuda.stream(st):
                for _ in range(2):
                    c.allreduce(s_, r)
        torch.cuda.synchronize()
        for r, ref in zip(recvs, refs):
            assert from_dev(env, r, "float32").tobytes() == ref.tobytes()
    for c in comms:
        assert c.check() == api.AR_SUCCESS


@pytest.mark.parametrize("variant", LAUNCHES + ["tree"])
def test_comm_on_a_cu_masked_stream_then_teardown(env, variant):
    """A comm used on a caller-owned stream held to 32 CUs, with AR_OPT_GRID
    at one workgroup per CU (the forms whose workgroups must all be resident
    fit those CUs): exact in every form, and closing the comm before
    destroying the stream releases the workspace cleanly (the workspace is
    recorded on every stream the comm ran on)."""
    torch, api, orc = env["torch"], env["api"], env["orc"]
    ncu = torch.cuda.get_device_properties(env["dev"]).multi_processor_count
    raw = api.ar_stream_create_cu_masked(range(32), ncu)
    try:
        st = torch.cuda.ExternalStream(raw, device=env["dev"])
        x = env["inputs"].draw("normal", 8, 1 << 16, seed=61)
        if variant == "tree":
            comm = api.Comm(8, 1 << 16, "float32", "tree", "ll", device=env["dev"], grid=32)
            ref = orc.tree_allreduce(x)
        else:
            comm = api.Comm(8, 1 << 16, "float32", device=env["dev"], grid=32, **ring_opts(variant))
            ref = orc.ring_allreduce(x)
        send = to_dev(env, x, "float32")
        recv = poisoned(env, x.shape, "float32")
        st.wait_stream(torch.cuda.current_stream())
        comm.allreduce(send, recv, stream=st)
        torch.cuda.synchronize()
        assert from_dev(env, recv, "float32").tobytes() == ref.tobytes()
        assert comm.check() == api.AR_SUCCESS
        comm.close()
        del comm
        torch.cuda.synchronize()
    finally:
        api.ar_stream_destroy(raw)
    torch.cuda.empty_cache()  # the allocator handles the recorded stream's events
    torch.cuda.synchronize()


# ---------------------------------------------------------------- special values

def _special_f32(R, N, seed):
    """float32 inputs mixing normal values with denormals, signed zeros,
    infinities of both signs and NaNs, placed column by column."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, N)).astype(np.float32)
    cols = rng.permutation(N)
    q = N // 8
    den, zer, negz, inf1, infpm, nan1, big = (cols[i * q:(i + 1) * q] for i in range(7))
    x[:, den] *= np.float32(1e-39)               # float32 denormals (below 1.18e-38)
    x[:, zer] = 0.0
    x[rng.integers(0, R, len(zer)), zer] = -0.0  # one -0 among +0
    x[:, negz] = -0.0                            # all -0: the sum stays -0
    x[rng.integers(0, R, len(inf1)), inf1] = np.inf
    r = rng.integers(0, R, len(infpm))
    x[r, infpm] = np.inf
    x[(r + 1 + rng.integers(0, R - 1, len(infpm))) % R, infpm] = -np.inf  # inf - inf = NaN
    x[rng.integers(0, R, len(nan1)), nan1] = np.nan
    x[:, big] = np.float32(3.0e38) * np.sign(x[:, big])  # overflow to +-inf mid-fold
    return x


def _assert_same_special(y, ref, dtype, what):
    """Bit-exact except that a NaN result must be a NaN (IEEE fixes no NaN
    payload or sign, and x86 and gfx950 differ there)."""
    if dtype == "bf16":
        yf, rf = y.astype(np.uint32) << 16, ref.astype(np.uint32) << 16
        yf, rf = yf.view(np.float32), rf.view(np.float32)
    else:
        yf, rf = y, ref
    nan = np.isnan(rf)
    assert (np.isnan(yf) == nan).all(), what
    assert y[~nan].tobytes() == ref[~nan].tobytes(), what


@pytest.mark.parametrize("variant", LAUNCHES + ["tree", "tree-fused"])
@pytest.mark.parametrize("dtype", ["float32", "bf16"])
@pytest.mark.parametrize("op", ["sum", "max", "min", "avg"])
def test_special_values(env, variant, dtype, op):
    """Denormals, signed zeros, infinities and NaNs go through every form and
    operator exactly as the oracle folds them (no flush to zero, no fused or
    reassociated adds, max/min by the same strict comparison); the fused
    tree also with a grid of 16, so that 32,816 elements take 16-byte
    packs."""
    orc = env["orc"]
    for R, N in ((8, 8 * 4096 + 48), (5, 1003)):
        x = _special_f32(R, N, seed=R * 131 + N)
        if dtype == "bf16":
            x = orc.bf16_from_f32(x)
        if variant == "tree":
            runs = [dict(algo="tree", proto="ll")]
        elif variant == "tree-fused":
            runs = [dict(algo="tree", launch="fused"), dict(algo="tree", launch="fused", grid=16)]
        else:
            runs = [dict(launch=variant)]
        for kw in runs:
            (y,) = run_allreduce(env, x, dtype, redop=op, **kw)
            ref = (orc.tree_allreduce(x, dtype, op=op) if variant.startswith("tree")
                   else orc.ring_allreduce(x, dtype, op=op))
            _assert_same_special(y, ref, dtype, (variant, dtype, op, R, N, kw))


@pytest.mark.parametrize("variant", LAUNCHES + ["tree", "tree-fused"])
def test_int32_sum_wraps(env, variant):
    """int32 sums wrap modulo 2^32 in every form, as in the oracle and as
    numpy's int64 sum reduced modulo 2^32."""
    orc = env["orc"]
    R, N = 8, 4 * 4096 + 3
    rng = np.random.default_rng(77)
    x = rng.integers(-2 ** 31, 2 ** 31, size=(R, N), dtype=np.int64).astype(np.int32)
    want = (x.astype(np.int64).sum(axis=0) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
    if variant.startswith("tree"):
        kw = dict(proto="ll") if variant == "tree" else dict(launch="fused")
        (y,) = run_allreduce(env, x, "int32", "tree", **kw)
        assert y.tobytes() == orc.tree_allreduce(x).tobytes()
    else:
        (y,) = run_allreduce(env, x, "int32", launch=variant)
        assert y.tobytes() == orc.ring_allreduce(x).tobytes()
    assert (y == want[None, :]).all()


# ---------------------------------------------------------------- channels

def _strides(api, R, K):
    c = api.ar_init(R, 64, api.AR_FLOAT32, api.AR_RING, api.AR_SIMPLE)
    try:
        return [api.ar_ring_channel_stride(c, k) for k in range(K)]
    finally:
        api.ar_destroy(c)


@pytest.mark.parametrize("launch", LAUNCHES)
@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R,K", [(2, 1), (5, 2), (5, 4), (8, 2), (8, 4), (16, 3), (16, 8)])
def test_multi_channel_rings(env, launch, dtype, R, K):
    """K channels: channel k reduces sub-range k of every segment around its
    own ring q -> q + m_k; the fold order is the one the oracle replays with
    the same strides."""
    api, orc = env["api"], env["orc"]
    strides = _strides(api, R, K)
    for N in (1, 13, 1000, 4097, 16 * 4096 + 40):
        x = rand_input(env, dtype, R, N, seed=3 * R + K + N)
        (y,) = run_allreduce(env, x, dtype, launch=launch, channels=K)
        assert y.tobytes() == orc.ring_allreduce(x, dtype, strides=strides).tobytes(), (R, K, N)
        check_tolerance(env, y, x, dtype)


@pytest.mark.parametrize("launch", LAUNCHES)
@pytest.mark.parametrize("dtype", ["float32", "bf16"])
def test_multi_channel_reduce_scatter_all_gather_operators(env, launch, dtype):
    api, orc = env["api"], env["orc"]
    R, K = 8, 4
    strides = _strides(api, R, K)
    for n in (3, 1000, 8192 + 8):
        N = n * R
        x = rand_input(env, dtype, R, N, seed=n + 401)
        for op in ("sum", "max", "avg"):
            comm = api.Comm(R, N, dtype, device=env["dev"], channels=K, redop=op,
                            **ring_opts(launch))
            assert comm.channel_strides() == strides
            send = to_dev(env, x, dtype)
            shard = poisoned(env, (R, n), dtype)
            comm.reduce_scatter(send, shard)
            rs = from_dev(env, shard, dtype)
            assert rs.tobytes() == orc.ring_reduce_scatter(x, dtype, op=op,
                                                           strides=strides).tobytes(), (n, op)
            full = poisoned(env, (R, N), dtype)
            comm.all_gather(shard, full)
            assert from_dev(env, full, dtype).tobytes() == \
                orc.ring_all_gather(rs, dtype, strides=strides).tobytes(), (n, op)
            ar = poisoned(env, (R, N), dtype)
            comm.allreduce(send, ar)
            assert from_dev(env, ar, dtype).tobytes() == \
                orc.ring_allreduce(x, dtype, op=op, strides=strides).tobytes(), (n, op)
            assert comm.check() == api.AR_SUCCESS


def test_multi_channel_full_size_order_differs_from_one_channel(env):
    """At 64 MiB per rank, 8 ranks, float32: four channels match the oracle
    with four strides bit for bit, and (the fold order being different) not
    the single-ring result everywhere."""
    api, orc = env["api"], env["orc"]
    x = env["inputs"].host_inputs("ring_f32_r8_64MiB")
    strides = _strides(api, 8, 4)
    (y4,) = run_allreduce(env, x, "float32", launch="fused", channels=4)
    assert y4.tobytes() == orc.ring_allreduce(x, strides=strides).tobytes()
    (y1,) = run_allreduce(env, x, "float32", launch="fused")
    assert y1.tobytes() != y4.tobytes()
    check_tolerance(env, y4, x, "float32")


@pytest.mark.parametrize("launch", ["fused", "step", "tree-fused"])
def test_concurrent_with_compute_on_another_stream(env, launch):
    """A ring (or fused tree) all-reduce on a second stream while GEMMs run
    on the first (the overlap pattern) stays exact."""
    torch, api, orc = env["torch"], env["api"], env["orc"]
    R, N = 8, 1 << 20
    x = env["inputs"].draw("normal", R, N, seed=44)
    if launch == "tree-fused":
        ref = orc.tree_allreduce(x)
        comm = api.Comm(R, N, "float32", "tree", device=env["dev"], launch="fused")
    else:
        ref = orc.ring_allreduce(x)
        comm = api.Comm(R, N, "float32", device=env["dev"], launch=launch)
    send = to_dev(env, x, "float32")
    recv = poisoned(env, (R, N), "float32")
    a = torch.randn((2048, 2048), device=env["dev"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(side):
            comm.allreduce(send, recv)
        c = a
        for _ in range(4):
            c = c @ a / 2048.0
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert from_dev(env, recv, "float32").tobytes() == ref.tobytes()
    assert comm.check() == api.AR_SUCCESS


# ---------------------------------------------------------------- random combinations

def test_random_automatic_choices_match_oracle(env):
    """60 seeded draws with the algorithm and the protocol both chosen by the
    library (AR_AUTO, AR_PROTO_AUTO) over a random ring launch form, ranks,
    dtype, operator, channels and sizes up to 2 MB per rank, so the fused
    tree, tree + LL, ring + LL and the simple-protocol ring all run: each
    result bit-exact against the oracle's replay of the schedule ar_plan
    reports."""
    api, orc = env["api"], env["orc"]
    rng = np.random.default_rng(20261204)
    kinds = set()
    for case in range(60):
        R = int(rng.integers(2, 17))
        dtype = ["int32", "float32", "bf16"][int(rng.integers(3))]
        launch = ["pipelined", "step", "fused"][int(rng.integers(3))]
        ops = ["sum", "max", "min"] + ([] if dtype == "int32" else ["avg"])
        op = ops[int(rng.integers(len(ops)))]
        K = 1 if R == 2 else int(rng.integers(1, 3))
        es = 2 if dtype == "bf16" else 4
        # bytes per rank: half log-uniform over 8 B .. 2 MB, half uniform over
        # 300 KB .. 2 MB, where ring + LL lies between the tree and the simple form
        nbytes = np.exp(rng.uniform(np.log(8), np.log(2e6))) if case % 2 else rng.uniform(3e5, 2e6)
        N = max(1, int(nbytes) // es)
        what = (case, R, dtype, launch, op, K, N)
        x = rand_input(env, dtype, R, N, seed=1000 + case)
        comm = api.Comm(R, N, dtype, "auto", "auto", device=env["dev"], launch=launch, redop=op,
                        channels=K)
        algo, proto, plaunch = comm.plan(N)
        kinds.add(("tree-fused" if plaunch == api.AR_LAUNCH_FUSED else "tree") if algo == api.AR_TREE
                  else "ring-ll" if proto == api.AR_LL else "simple")
        if algo == api.AR_TREE:
            ref = orc.tree_allreduce(x, dtype, op=op)
        else:
            ref = orc.ring_allreduce(x, dtype, op=op, strides=comm.channel_strides())
        recv = poisoned(env, (R, N), dtype)
        comm.allreduce(to_dev(env, x, dtype), recv)
        assert from_dev(env, recv, dtype).tobytes() == ref.tobytes(), what
        assert comm.check() == api.AR_SUCCESS, what
        comm.close()
    assert kinds == {"tree", "tree-fused", "ring-ll", "simple"}, kinds


def test_random_configurations_match_oracle(env):
    """200 seeded draws over the option space at once: ranks, ragged sizes,
    dtype, launch form (and the LL or fused tree), ring channels, reduction
    operator, in place, and all-reduce or reduce-scatter then all-gather; each
    result bit-exact against the oracle's replay of the same schedule."""
    api, orc = env["api"], env["orc"]
    rng = np.random.default_rng(20261203)
    for case in range(200):
        R = int(rng.integers(2, 17))
        dtype = ["int32", "float32", "bf16"][int(rng.integers(3))]
        variant = (LAUNCHES + ["tree", "tree-fused"])[int(rng.integers(len(LAUNCHES) + 2))]
        ops = ["sum", "max", "min"] + ([] if dtype == "int32" else ["avg"])
        op = ops[int(rng.integers(len(ops)))]
        tree = variant.startswith("tree")
        coll = "ar" if tree else ["ar", "rs_ag"][int(rng.integers(2))]
        K = 1 if tree or R == 2 else int(rng.integers(1, 3))  # R = 2 has one stride
        what = (case, R, dtype, variant, op, coll, K)
        if coll == "ar":
            N = int(np.exp(rng.uniform(0, np.log(300000))))
            x = rand_input(env, dtype, R, N, seed=case)
            if tree:
                # the fused tree for R <= 16, else the LL tree
                tree_opts = (dict(proto="simple", launch="fused") if variant == "tree-fused"
                             else dict(proto="ll"))
                comm = api.Comm(R, N, dtype, "tree", device=env["dev"], redop=op, **tree_opts)
                ref = orc.tree_allreduce(x, dtype, op=op)
            else:
                comm = api.Comm(R, N, dtype, device=env["dev"], redop=op, channels=K,
                                **ring_opts(variant))
                ref = orc.ring_allreduce(x, dtype, op=op, strides=comm.channel_strides())
            send = to_dev(env, x, dtype)
            if rng.integers(2):
                comm.allreduce(send, send)  # in place
                got = from_dev(env, send, dtype)
            else:
                recv = poisoned(env, (R, N), dtype)
                comm.allreduce(send, recv)
                got = from_dev(env, recv, dtype)
            assert got.tobytes() == ref.tobytes(), what + (N,)
        else:
            n = int(np.exp(rng.uniform(0, np.log(20000))))
            N = n * R
            x = rand_input(env, dtype, R, N, seed=case)
            comm = api.Comm(R, N, dtype, device=env["dev"], redop=op, channels=K,
                            **ring_opts(variant))
            strides = comm.channel_strides()
            shard = poisoned(env, (R, n), dtype)
            comm.reduce_scatter(to_dev(env, x, dtype), shard)
            rs = from_dev(env, shard, dtype)
            assert rs.tobytes() == orc.ring_reduce_scatter(x, dtype, op=op,
                                                           strides=strides).tobytes(), what + (n,)
            full = poisoned(env, (R, N), dtype)
            comm.all_gather(shard, full)
            assert from_dev(env, full, dtype).tobytes() == \
                orc.ring_all_gather(rs, dtype, strides=strides).tobytes(), what + (n,)
        assert comm.check() == api.AR_SUCCESS, what
