"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and its host-side logic (argument checks, schedule views)
behaves -- without any compute call (there is no GPU here)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "ar.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(ar_[a-z_]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def api():
    from collective_communication_ring_amd import api
    if not os.path.exists(api.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    api.lib()
    return api


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("ar_init", "ar_allreduce", "ar_reduce_scatter", "ar_all_gather",
              "ar_workspace_bytes", "ar_set_workspace", "ar_check", "ar_destroy",
              "ar_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(api):
    L = api.lib()
    missing = [n for n in _declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_python_constants_match_the_header(api):
    """Every enumerator ar.h defines has the same value in the Python binding."""
    src = open(os.path.join(ROOT, "include", "ar.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    vals = {}
    for body in re.findall(r"typedef enum\s*\{(.*?)\}", src, flags=re.S):
        for name, v in re.findall(r"(AR_[A-Z0-9_]+)\s*=\s*(-?\d+)", body):
            vals[name] = int(v)
    assert len(vals) > 30
    missing = [n for n in vals if n != "AR_COST_FORMS" and not hasattr(api, n)]
    assert not missing, missing
    wrong = {n: (v, getattr(api, n)) for n, v in vals.items() if hasattr(api, n) and getattr(api, n) != v}
    assert not wrong, wrong


def test_init_argument_checks(api):
    import ctypes
    L = api.lib()
    h = ctypes.c_void_p()
    assert L.ar_init(ctypes.byref(h), 1, 16, api.AR_FLOAT32, api.AR_RING, api.AR_SIMPLE) == api.AR_ERR_INVALID_ARG
    assert h.value is None
    assert L.ar_init(ctypes.byref(h), 65, 16, api.AR_FLOAT32, api.AR_RING, api.AR_SIMPLE) == api.AR_ERR_INVALID_ARG
    assert L.ar_init(ctypes.byref(h), 4, 16, 7, api.AR_RING, api.AR_SIMPLE) == api.AR_ERR_INVALID_ARG
    assert L.ar_init(ctypes.byref(h), 4, 16, api.AR_FLOAT32, 9, api.AR_SIMPLE) == api.AR_ERR_INVALID_ARG
    assert L.ar_init(None, 4, 16, api.AR_FLOAT32, api.AR_RING, api.AR_SIMPLE) == api.AR_ERR_INVALID_ARG
    c = api.ar_init(8, 1024, api.AR_FLOAT32)
    try:
        assert api.ar_workspace_bytes(c) >= 256 + 1024 * 4  # one accumulator row
        # no workspace yet: a collective is refused before touching the device
        assert L.ar_allreduce(c, 16, 4096, 8, None) == api.AR_ERR_INVALID_USAGE
        assert L.ar_set_workspace(c, None, 1 << 20, None) == api.AR_ERR_INVALID_ARG
        assert L.ar_set_workspace(c, 257, 1 << 30, None) == api.AR_ERR_INVALID_ARG  # misaligned
        assert L.ar_set_workspace(c, 4096, 16, None) == api.AR_ERR_INVALID_ARG      # too small
    finally:
        api.ar_destroy(c)
    assert api.ar_destroy(None) == 0


def test_options_round_trip(api):
    c = api.ar_init(4, 100, api.AR_INT32)
    try:
        for opt, val in ((api.AR_OPT_CHUNK_BYTES, 4096), (api.AR_OPT_LAUNCH, api.AR_LAUNCH_STEP),
                         (api.AR_OPT_GRID, 512), (api.AR_OPT_TIMEOUT_US, 1000),
                         (api.AR_OPT_ALGO, api.AR_TREE), (api.AR_OPT_PROTO, api.AR_LL),
                         (api.AR_OPT_TREE_MAX_BYTES, 1 << 20), (api.AR_OPT_DEBUG_MUTE_RANK, 2),
                         (api.AR_OPT_DEBUG_MUTE_RANK, -1), (api.AR_OPT_DEBUG_LL_LAUNCHES, 1 << 30),
                         (api.AR_OPT_DEBUG_LL_LAUNCHES, 0)):
            api.ar_set_option(c, opt, val)
            assert api.ar_get_option(c, opt) == val
        with pytest.raises(api.ArError):
            api.ar_set_option(c, api.AR_OPT_LAUNCH, 99)
        with pytest.raises(api.ArError):
            api.ar_set_option(c, 1234, 1)
        with pytest.raises(api.ArError):
            api.ar_set_option(c, api.AR_OPT_DEBUG_MUTE_RANK, 4)  # R = 4
        with pytest.raises(api.ArError):
            api.ar_set_option(c, api.AR_OPT_DEBUG_LL_LAUNCHES, (1 << 30) + 1)
    finally:
        api.ar_destroy(c)


def test_plan_picks_tree_for_small_and_ring_for_large(api):
    c = api.ar_init(8, 1 << 22, api.AR_FLOAT32, api.AR_AUTO)
    try:
        assert api.ar_get_option(c, api.AR_OPT_TREE_MAX_BYTES) == -1  # by the cost model
        # the default launch: the fused tree's line against the fused ring's,
        # crossing between 2 and 4 MiB per rank
        ua, ub = api.ar_get_cost(c, api.AR_COST_TREE_FUSED)
        fa, fb = api.ar_get_cost(c, api.AR_COST_RING_FUSED)
        n = api.ar_auto_tree_max_bytes(c)
        cross = (fa - ua) / (1e-3 / ub - 1e-3 / fb)
        assert 2 << 20 < n <= cross < n + 2 and cross < 4 << 20
        assert api.ar_plan(c, 1)[:3] == (api.AR_TREE, api.AR_SIMPLE, api.AR_LAUNCH_FUSED)
        assert api.ar_plan(c, n // 4)[0] == api.AR_TREE
        assert api.ar_plan(c, n // 4 + 1)[:3] == (api.AR_RING, api.AR_SIMPLE, api.AR_LAUNCH_FUSED)
        # the LL tree's line is above the fused ring's at every size, so where
        # the tree cannot be fused (R of 17 .. 63 other than 32) AUTO keeps the
        # ring
        ta, tb = api.ar_get_cost(c, api.AR_COST_TREE_LL)
        assert fa < ta and fb > tb
        for R, dt in ((16, api.AR_BF16), (32, api.AR_FLOAT32), (64, api.AR_INT32)):
            b = api.ar_init(R, 1 << 22, dt, api.AR_AUTO)
            try:  # R = 2..16, 32 and 64 have the fused tree, every dtype
                assert api.ar_plan(b, 1)[:3] == (api.AR_TREE, api.AR_SIMPLE, api.AR_LAUNCH_FUSED)
            finally:
                api.ar_destroy(b)
        for R, dt in ((17, api.AR_BF16), (17, api.AR_FLOAT32), (48, api.AR_FLOAT32)):
            d = api.ar_init(R, 1 << 22, dt, api.AR_AUTO)
            try:
                assert api.ar_auto_tree_max_bytes(d) == 0
                assert api.ar_plan(d, 1)[0] == api.AR_RING
            finally:
                api.ar_destroy(d)
        # with the pipelined ring the lines cross: tree below, ring above
        api.ar_set_option(c, api.AR_OPT_LAUNCH, api.AR_LAUNCH_PIPELINED)
        n = api.ar_auto_tree_max_bytes(c)
        pa, pb = api.ar_get_cost(c, api.AR_COST_RING_PIPELINED)
        cross = (pa - ta) / (1e-3 / tb - 1e-3 / pb)  # bytes where the lines meet
        assert 0 < n <= cross < n + 2
        assert api.ar_plan(c, 1)[0] == api.AR_TREE
        assert api.ar_plan(c, n // 4)[0] == api.AR_TREE
        assert api.ar_plan(c, n // 4 + 1)[0] == api.AR_RING
        # a caller's own fits move the crossing
        api.ar_set_cost(c, api.AR_COST_RING_PIPELINED, pa, pb * 4)
        assert api.ar_auto_tree_max_bytes(c) < n
        # ring + LL uses its own line
        api.ar_set_option(c, api.AR_OPT_PROTO, api.AR_LL)
        la, lb = api.ar_get_cost(c, api.AR_COST_RING_LL)
        assert abs(api.ar_auto_tree_max_bytes(c) - (la - ta) / (1e-3 / tb - 1e-3 / lb)) < 2
        api.ar_set_option(c, api.AR_OPT_PROTO, api.AR_SIMPLE)
        # a fixed threshold overrides the model
        api.ar_set_option(c, api.AR_OPT_TREE_MAX_BYTES, 64 * 1024)
        assert api.ar_auto_tree_max_bytes(c) == 64 * 1024
        assert api.ar_plan(c, 16)[0] == api.AR_TREE
        assert api.ar_plan(c, 16 * 1024)[0] == api.AR_TREE
        assert api.ar_plan(c, 16 * 1024 + 1)[0] == api.AR_RING
        assert api.ar_plan(c, 1 << 20)[0] == api.AR_RING
        api.ar_set_option(c, api.AR_OPT_TREE_MAX_BYTES, -1)
        assert api.ar_auto_tree_max_bytes(c) < n
        # bad models are refused
        for form, a, b in ((6, 1.0, 1.0), (-1, 1.0, 1.0), (0, -1.0, 1.0), (0, 1.0, 0.0),
                           (0, float("nan"), 1.0), (0, 1.0, float("nan"))):
            with pytest.raises(api.ArError):
                api.ar_set_cost(c, form, a, b)
        with pytest.raises(api.ArError):
            api.ar_set_option(c, api.AR_OPT_TREE_MAX_BYTES, -2)
    finally:
        api.ar_destroy(c)


def _line_cross(a, b):
    """Bytes per rank where two cost lines (alpha_us, GB/s) meet."""
    return (b[0] - a[0]) / (1e-3 / a[1] - 1e-3 / b[1])


def _cost(line, n):
    return line[0] + n / (line[1] * 1e3)


def test_plan_protocol_auto(api):
    """AR_PROTO_AUTO takes ring + LL where its line is strictly below the
    simple form's, and AR_AUTO weighs the tree against that cheaper ring."""
    c = api.ar_init(8, 1 << 24, api.AR_FLOAT32, api.AR_AUTO, api.AR_PROTO_AUTO)
    try:
        assert api.ar_get_option(c, api.AR_OPT_PROTO) == api.AR_PROTO_AUTO
        tree = api.ar_get_cost(c, api.AR_COST_TREE_LL)
        ll = api.ar_get_cost(c, api.AR_COST_RING_LL)
        # the default fused launch: ring + LL never beats the fused ring, so
        # the fused tree below its crossing with the fused ring, the fused ring
        # above
        fused = (api.ar_get_cost(c, api.AR_COST_TREE_FUSED), api.ar_get_cost(c, api.AR_COST_RING_FUSED))
        t_max = api.ar_auto_tree_max_bytes(c)
        assert abs(t_max - _line_cross(*fused)) < 2
        for n in (1, 1000, t_max // 4):
            assert api.ar_plan(c, n) == (api.AR_TREE, api.AR_SIMPLE, api.AR_LAUNCH_FUSED)
        for n in (t_max // 4 + 1, 1 << 20, 1 << 24):
            assert api.ar_plan(c, n) == (api.AR_RING, api.AR_SIMPLE, api.AR_LAUNCH_FUSED)
        for launch, form in ((api.AR_LAUNCH_PIPELINED, api.AR_COST_RING_PIPELINED),
                             (api.AR_LAUNCH_STEP, api.AR_COST_RING_STEP)):
            api.ar_set_option(c, api.AR_OPT_LAUNCH, launch)
            simple = api.ar_get_cost(c, form)
            t_max = api.ar_auto_tree_max_bytes(c)
            # the tree goes up to the lower of its two crossings (with ring + LL here)
            assert abs(t_max - min(_line_cross(tree, ll), _line_cross(tree, simple))) < 2
            ll_max = _line_cross(ll, simple)  # ring + LL below the simple form up to here
            assert t_max < ll_max
            assert api.ar_plan(c, 1) == (api.AR_TREE, api.AR_LL, api.AR_LAUNCH_AUTO)
            assert api.ar_plan(c, t_max // 4) == (api.AR_TREE, api.AR_LL, api.AR_LAUNCH_AUTO)
            assert api.ar_plan(c, t_max // 4 + 1) == (api.AR_RING, api.AR_LL, api.AR_LAUNCH_AUTO)
            # the switch to the simple form sits where the two ring lines cross
            k = int(ll_max) // 4
            for n in range(k - 2, k + 3):
                want = api.AR_LL if _cost(ll, 4 * n) < _cost(simple, 4 * n) else api.AR_SIMPLE
                got = api.ar_plan(c, n)
                assert got[:2] == (api.AR_RING, want), (launch, n, got)
            assert api.ar_plan(c, 1 << 22) == (api.AR_RING, api.AR_SIMPLE, launch)
            # a ring-only comm keeps the same protocol choice
            api.ar_set_option(c, api.AR_OPT_ALGO, api.AR_RING)
            assert api.ar_plan(c, 1) == (api.AR_RING, api.AR_LL, api.AR_LAUNCH_AUTO)
            assert api.ar_plan(c, 1 << 22) == (api.AR_RING, api.AR_SIMPLE, launch)
            api.ar_set_option(c, api.AR_OPT_ALGO, api.AR_AUTO)
        # a fixed protocol still wins over the model (step form, 1.2 MB per
        # rank: above the tree's crossing, below ring + LL's)
        assert api.ar_plan(c, 1_200_000 // 4)[:2] == (api.AR_RING, api.AR_LL)
        api.ar_set_option(c, api.AR_OPT_PROTO, api.AR_SIMPLE)
        assert api.ar_plan(c, 1_200_000 // 4) == (api.AR_RING, api.AR_SIMPLE, api.AR_LAUNCH_STEP)
        with pytest.raises(api.ArError):
            api.ar_set_option(c, api.AR_OPT_PROTO, 3)
    finally:
        api.ar_destroy(c)
    with pytest.raises(api.ArError):
        api.ar_init(8, 1024, api.AR_FLOAT32, api.AR_AUTO, 3)


def test_auto_tree_max_bytes_for_any_lines(api):
    """ar_auto_tree_max_bytes for lines a caller may set: a prefix of sizes
    by tree, none, all, or (lines crossing the other way) -2; answers at once
    even where the lines meet far out."""
    c = api.ar_init(8, 1024, api.AR_FLOAT32, api.AR_AUTO, api.AR_SIMPLE)
    try:
        api.ar_set_option(c, api.AR_OPT_LAUNCH, api.AR_LAUNCH_PIPELINED)
        P, T = api.AR_COST_RING_PIPELINED, api.AR_COST_TREE_LL
        # the tree cheaper only for large messages
        api.ar_set_cost(c, T, 100.0, 1000.0)
        api.ar_set_cost(c, P, 10.0, 100.0)
        assert api.ar_auto_tree_max_bytes(c) == -2
        assert api.ar_plan(c, 1)[0] == api.AR_RING
        assert api.ar_plan(c, 1 << 30)[0] == api.AR_TREE
        # never, always, and equal lines (strictly below: never)
        api.ar_set_cost(c, T, 20.0, 100.0)
        assert api.ar_auto_tree_max_bytes(c) == 0
        api.ar_set_cost(c, T, 1.0, 1000.0)
        assert api.ar_auto_tree_max_bytes(c) == 2 ** 63 - 1
        api.ar_set_cost(c, T, 10.0, 100.0)
        assert api.ar_auto_tree_max_bytes(c) == 0
        # meeting points far out: ~5e8 bytes (a prefix), ~1e9 bytes (a suffix)
        api.ar_set_cost(c, T, 0.0, 1e-3)
        api.ar_set_cost(c, P, 5e8, 1e8)
        b = api.ar_auto_tree_max_bytes(c)
        assert abs(b - _line_cross((0.0, 1e-3), (5e8, 1e8))) < 2
        assert api.ar_plan(c, b // 4)[0] == api.AR_TREE
        assert api.ar_plan(c, b // 4 + 1)[0] == api.AR_RING
        api.ar_set_cost(c, T, 1e8, 1e8)
        api.ar_set_cost(c, P, 0.0, 1e-2)
        assert api.ar_auto_tree_max_bytes(c) == -2
        # lines that meet beyond any size: the side that wins at n = 0 everywhere
        api.ar_set_cost(c, T, 0.0, 1e8)
        api.ar_set_cost(c, P, 1e8, 1e8 * 0.999999)
        assert api.ar_auto_tree_max_bytes(c) == 2 ** 63 - 1
    finally:
        api.ar_destroy(c)


@pytest.mark.parametrize("R", [2, 3, 4, 5, 7, 8, 16, 64])
def test_library_schedule_matches_oracle(api, orc, R):
    """The library's host scheduler and the oracle are separate code; their
    segment bounds and tree shapes must agree."""
    c = api.ar_init(R, 10 ** 6, api.AR_FLOAT32)
    try:
        for t in (0, 1):
            assert [api.ar_tree_parent(c, t, r) for r in range(R)] == orc.tree_parents(R, t)
        assert api.ar_tree_parent(c, 2, 0) == -2
        for count in (0, 1, R - 1, R, 10 * R + 3, 999_983):
            S = -(-count // R)
            prev = 0
            for s in range(R):
                lo, hi = api.ar_ring_segment(c, count, s)
                assert (lo, hi) == (min(s * S, count), min((s + 1) * S, count))
                assert lo == prev
                prev = hi
            assert prev == count
    finally:
        api.ar_destroy(c)


def test_status_strings(api):
    for s in range(7):
        assert api.ar_status_string(s)
    assert "timeout" in api.ar_status_string(api.AR_ERR_TIMEOUT)


def test_utilities_reject_bad_arguments(api):
    L = api.lib()
    assert L.ar_stream_add(None, None, None, 16, None) == api.AR_ERR_INVALID_ARG
    assert L.ar_stream_add(None, None, None, 0, None) == api.AR_SUCCESS
    assert L.ar_stream_copy(16, 32, 15, None) == api.AR_ERR_INVALID_ARG  # not a multiple of 16
    assert L.ar_stream_rows(16, 32, 8, 1024, None) == api.AR_ERR_INVALID_ARG  # not whole tiles
    assert L.ar_stream_rows(None, None, 8, 2048, None) == api.AR_ERR_INVALID_ARG
    assert L.ar_stream_rows(8, 32, 8, 2048, None) == api.AR_ERR_INVALID_ARG  # misaligned
    assert L.ar_stream_rows(16, 32, -1, 2048, None) == api.AR_ERR_INVALID_ARG
    assert L.ar_stream_rows(None, None, 0, 2048, None) == api.AR_SUCCESS    # nothing to do
    assert L.ar_ll_pingpong(None, None, 10, 1, 1000, None) == api.AR_ERR_INVALID_ARG
    assert L.ar_ll_pingpong(256, 512, 0, 1, 1000, None) == api.AR_ERR_INVALID_ARG


@pytest.mark.parametrize("R", [2, 3, 4, 5, 6, 7, 8, 9, 12, 16, 30, 64])
def test_channel_strides(api, R):
    """Channel strides: every integer in [1, R) coprime with R, each once,
    ordered 1, R-1, 3, R-3, ... with duplicates dropped; each stride walks a
    Hamiltonian ring (q -> q + m visits every rank), and a stride and its
    complement traverse the same undirected ring in opposite directions."""
    import math
    c = api.ar_init(R, 1024, api.AR_FLOAT32, api.AR_RING, api.AR_SIMPLE)
    try:
        got = []
        k = 0
        while True:
            m = api.ar_ring_channel_stride(c, k)
            if m < 0:
                break
            got.append(m)
            k += 1
        assert sorted(got) == [m for m in range(1, R) if math.gcd(m, R) == 1]
        assert got[0] == 1
        if R > 2:
            assert got[1] == R - 1
        for m in got:
            seen, q = set(), 0
            for _ in range(R):
                seen.add(q)
                q = (q + m) % R
            assert seen == set(range(R)) and q == 0
        # the option accepts 1 .. len(strides) and nothing else
        for K in range(1, len(got) + 1):
            api.ar_set_option(c, api.AR_OPT_CHANNELS, K)
            assert api.ar_get_option(c, api.AR_OPT_CHANNELS) == K
        for bad in (0, len(got) + 1, -3):
            with pytest.raises(api.ArError):
                api.ar_set_option(c, api.AR_OPT_CHANNELS, bad)
        assert api.ar_ring_channel_stride(c, -1) == -1
    finally:
        api.ar_destroy(c)


def test_counts_are_checked_before_the_device(api):
    """Sizes are validated before anything touches the device, and a shard
    count whose product with R would wrap around size_t is refused."""
    L = api.lib()
    c = api.ar_init(4, 64, api.AR_FLOAT32)
    try:
        huge = (1 << 64) // 4 + 1  # 4 * huge wraps to 4, below the capacity
        for fn in (L.ar_reduce_scatter, L.ar_all_gather):
            assert fn(c, 4096, 8192, huge, None) == api.AR_ERR_INVALID_ARG
            assert fn(c, 4096, 8192, 17, None) == api.AR_ERR_INVALID_ARG   # 4 * 17 > 64
            assert fn(c, 4096, 8192, 16, None) == api.AR_ERR_INVALID_USAGE  # fits: no workspace yet
        assert L.ar_allreduce(c, 4096, 8192, 65, None) == api.AR_ERR_INVALID_ARG
        assert L.ar_allreduce(c, 4096, 8192, 64, None) == api.AR_ERR_INVALID_USAGE
    finally:
        api.ar_destroy(c)
