"""The allocation-free all-reduce (ar_allreduce_noalloc) against ar_allreduce.

It is called through the C ABI with device pointers.  Its output must equal
ar_allreduce's on the same inputs, bit for bit.  Each case runs two calls in
a row, the second with a smaller input: the device array keeps the last
call's contents and must not leak them into the next call.  The cases cover:
- bfloat16 and in-place float32, whose wave tiles cut short by a segment's
  end stage the float32 running value in the library's device array (whole
  tiles hand it on through LDS);
- out-of-place float32 and int32;
- the scalar path, which hands off through LDS, at any count.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    from collective_communication_ring_amd import api, inputs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    api.lib()
    return dict(torch=torch, api=api, inputs=inputs, dev=torch.device("cuda:0"))


def _input(env, dtype, R, N, seed):
    torch, inputs = env["torch"], env["inputs"]
    if dtype == "bf16":
        x = inputs.to_bf16_bits(inputs.draw("normal_0.02", R, N, seed))
        return torch.from_numpy(x.view(np.int16)).to(env["dev"]).view(torch.bfloat16)
    if dtype == "int32":
        return torch.from_numpy(inputs.draw("int_pm1000", R, N, seed)).to(env["dev"])
    return torch.from_numpy(inputs.draw("normal", R, N, seed)).to(env["dev"])


def _bits(env, t):
    torch = env["torch"]
    torch.cuda.synchronize()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else t.dtype).cpu().numpy().tobytes()


@pytest.mark.parametrize("dtype,R,sizes,in_place", [
    ("bf16", 16, (13_107_200, 1_048_576 + 16 * 8), False),  # a 25 MiB gradient bucket, then a smaller one
    ("float32", 8, (16_777_216, 65_536 * 8 + 8), True),     # the headline, in place
    ("float32", 8, (16_777_216, 4096 * 8), False),
    ("int32", 4, (1 << 20, 4096), False),
    ("bf16", 8, (8 * 100 + 3, 8 * 7 + 1), False),            # odd sizes: the scalar path
    ("float32", 5, (4099, 13), True),
])
def test_noalloc_matches_allreduce(env, dtype, R, sizes, in_place):
    torch, api = env["torch"], env["api"]
    comm = api.Comm(R, sizes[0], dtype, "ring", device=env["dev"], launch="fused")
    st = torch.cuda.current_stream().cuda_stream
    for k, N in enumerate(sizes):
        x = _input(env, dtype, R, N, seed=1000 + 17 * k + N % 97)
        want = torch.empty_like(x)
        comm.allreduce(x, want)
        got = x.clone() if in_place else torch.full_like(x, float("nan")) \
            if dtype != "int32" else torch.full_like(x, -1)
        src = got if in_place else x
        api.ar_allreduce_noalloc(comm.handle, src.data_ptr(), got.data_ptr(), N, st)
        assert _bits(env, got) == _bits(env, want), (dtype, R, N, in_place)
    assert comm.check() == api.AR_SUCCESS
    comm.close()


def test_noalloc_runs_a_scalar_path_call_of_any_size(env):
    """Odd bf16 rows (not 16-byte aligned) take the scalar path, which hands
    its running value on through LDS and uses none of the 8 MiB array: a
    count above what the array could hold as one float32 per element
    (2,097,152) runs, on two calls in a row, and equals ar_allreduce."""
    torch, api = env["torch"], env["api"]
    R, N = 2, (8 << 20) // 4 + 1001
    comm = api.Comm(R, N, "bf16", "ring", device=env["dev"])
    g = torch.Generator(device=env["dev"])
    g.manual_seed(71)
    x = torch.randn((R, N), generator=g, device=env["dev"]).to(torch.bfloat16)
    L = api.lib()
    st = torch.cuda.current_stream().cuda_stream
    for n in (N, N - 2000):
        xs = x[:, :n].contiguous()
        y = torch.full_like(xs, float("nan"))
        assert L.ar_allreduce_noalloc(comm.handle, xs.data_ptr(), y.data_ptr(), n, st) == \
            api.AR_SUCCESS
        ref = torch.full_like(xs, float("nan"))
        comm.allreduce(xs, ref)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), n
    comm.close()
