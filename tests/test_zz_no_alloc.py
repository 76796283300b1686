"""The allocation-free all-reduce (ar_allreduce_noalloc) against ar_allreduce.

It is called through the C ABI with device pointers.  Its output must equal
ar_allreduce's on the same inputs, bit for bit.  Each case runs two calls in
a row, the second with a smaller input: the device array keeps the last
call's contents and must not leak them into the next call.  The cases cover:
- bfloat16 and in-place float32, which stage the float32 running value in
  the library's device array;
- out-of-place float32 and int32, whose running value lives in the owner's
  row;
- the scalar path.
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


def test_noalloc_refuses_a_scalar_path_call_too_large_for_its_array(env):
    """Odd bf16 rows (not 16-byte aligned) take the scalar path, which keeps
    one float32 per element in the 8 MiB array: above 2,097,152 elements the
    call is refused on the host, before anything is launched."""
    torch, api = env["torch"], env["api"]
    R, N = 2, (8 << 20) // 4 + 1
    comm = api.Comm(R, N, "bf16", "ring", device=env["dev"])
    x = torch.zeros((R, N), dtype=torch.bfloat16, device=env["dev"])
    y = torch.empty_like(x)
    L = api.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert L.ar_allreduce_noalloc(comm.handle, x.data_ptr(), y.data_ptr(), N, st) == \
        api.AR_ERR_INVALID_ARG
    # an odd count just under the limit (still the scalar path) runs
    assert L.ar_allreduce_noalloc(comm.handle, x.data_ptr(), y.data_ptr(), N - 2, st) == \
        api.AR_SUCCESS
    torch.cuda.synchronize()
    comm.close()
