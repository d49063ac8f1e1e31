"""ssm_scan_fwd_noalloc (through the C ABI) against ssm_scan_fwd on the same inputs.

The no-allocation entry point runs the same plan and kernels with its scratch in the library's fixed
device array, so its results must equal the allocating entry point's. Two calls in a row, the second on
a smaller input, catch state kept from one call to the next; a plan too large for the fixed array must
be refused before any launch.
"""
import numpy as np
import pytest
import torch

from gpu_util import TAU, assert_close, from_torch, upload
from selective_state_space_82_amd import api
from selective_state_space_82_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    api.lib()


def both(inp, **kw):
    """(allocating y, h), (no-allocation y, h) on one upload of `inp`; the outputs of the no-allocation
    call are preallocated and filled with a sentinel first."""
    t = upload(inp)
    y_ref, h_ref = api.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], **kw)
    y = torch.full_like(y_ref, 7.0)
    h = torch.full_like(h_ref, 7.0)
    api.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], y=y, final_state=h, noalloc=True,
                     **kw)
    torch.cuda.synchronize()
    return (from_torch(y_ref), from_torch(h_ref)), (from_torch(y), from_torch(h))


def check(inp, what, **kw):
    (y_ref, h_ref), (y, h) = both(inp, **kw)
    tau = TAU[inp["dtype"]]
    assert_close(y, y_ref, tau, f"{what} y")
    assert_close(h, h_ref, tau, f"{what} final state")
    # the same plan and kernels: identical bits
    assert np.array_equal(y, y_ref) and np.array_equal(h, h_ref), f"{what}: results differ from ssm_scan_fwd"


def test_small_problem_needs_no_scratch():
    """A short sequence on few channel blocks (the small-problem kernel) through the no-allocation entry point:
    no scratch at all, and the same bits as ssm_scan_fwd."""
    plan = api.ssm_scan_fwd_plan(2, 40, 200, 16)
    assert plan["scratch_bytes"] == 0 and plan["groups_aggregate_pass"] == 0
    check(I.random_prefill(2, 40, 200, 16, dtype="bf16", seed=8), "small-problem kernel")


def test_two_calls_in_a_row_second_smaller():
    """32 segments (a carry kernel chains the aggregates: carries in scratch too), then 11 segments on a
    smaller input (each output wavefront chains them)."""
    b, d, L, N = 2, 96, 4096, 16
    plan = api.ssm_scan_fwd_plan(b, d, L, N, torch.bfloat16, seg_len=128)
    assert plan["n_segments"] == 32 and 0 < plan["scratch_bytes"] <= api.NOALLOC_SCRATCH_BYTES
    check(I.random_prefill(b, d, L, N, dtype="bf16", seed=51), "noalloc first call (32 segments)", seg_len=128)
    plan2 = api.ssm_scan_fwd_plan(1, 40, 700, N, torch.float32, seg_len=64)
    assert plan2["n_segments"] == 11 and plan2["scratch_bytes"] < plan["scratch_bytes"]
    check(I.random_prefill(1, 40, 700, N, dtype="f32", seed=52), "noalloc second call (11 segments)", seg_len=64)


def test_default_plan_and_initial_state():
    b, d, L, N = 1, 512, 8192, 16
    plan = api.ssm_scan_fwd_plan(b, d, L, N, torch.bfloat16)
    assert plan["n_segments"] > 1 and plan["scratch_bytes"] <= api.NOALLOC_SCRATCH_BYTES
    inp = I.random_prefill(b, d, L, N, dtype="bf16", seed=53)
    h0 = torch.from_numpy((np.random.default_rng(5).standard_normal((b, d, N)) * 0.5).astype(np.float32)).cuda()
    check(inp, "noalloc default plan + initial state", initial_state=h0)


def test_no_split_needs_no_scratch():
    inp = I.random_prefill(4, 1024, 256, 16, dtype="f32", seed=54)
    assert api.ssm_scan_fwd_plan(4, 1024, 256, 16, torch.float32)["scratch_bytes"] == 0
    check(inp, "noalloc single segment")


def test_plan_beyond_the_fixed_scratch_is_refused():
    """A plan needing 793 MB of scratch: SSM_ERR_SCRATCH, and the outputs stay untouched."""
    b, d, L, N = 1, 16384, 2048, 64
    plan = api.ssm_scan_fwd_plan(b, d, L, N, torch.float32, seg_len=32)
    assert plan["scratch_bytes"] > api.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((b, d, L), device="cuda")
    dl = torch.full((b, d, L), 0.1, device="cuda")
    A = -torch.ones((d, N), device="cuda")
    B = torch.zeros((b, L, N), device="cuda")
    y = torch.full((b, d, L), 7.0, device="cuda")
    h = torch.full((b, d, N), 7.0, device="cuda")
    with pytest.raises(api.SsmError) as e:
        api.ssm_scan_fwd(x, dl, A, B, B, y=y, final_state=h, seg_len=32, noalloc=True)
    assert e.value.status == api.SSM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0)) and bool(torch.all(h == 7.0))


def test_empty_sequence_zeroes_final_state():
    t = upload(I.random_prefill(2, 3, 0, 4, dtype="f32"))
    y = torch.empty((2, 3, 0), device="cuda")
    h = torch.full((2, 3, 4), 7.0, device="cuda")
    api.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], y=y, final_state=h, noalloc=True)
    torch.cuda.synchronize()
    assert bool(torch.all(h == 0))
