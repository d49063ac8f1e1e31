"""Every entry point runs on the caller's current stream (scratch included, taken stream-ordered from it):
the same call issued on a side stream gives bit-identical results to the default stream."""
import numpy as np
import pytest
import torch

from gpu_util import to_torch, upload
from selective_state_space_82_amd import api
from selective_state_space_82_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    api.lib()


def _on(stream, fn):
    with torch.cuda.stream(stream):
        out = fn()
    stream.synchronize()
    return out


def test_all_entry_points_on_a_side_stream():
    side = torch.cuda.Stream()
    inp = I.random_prefill(2, 96, 700, 16, dtype="bf16", seed=41)
    t = upload(inp)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(4)
    dy = to_torch(I.store(rng.standard_normal((2, 96, 700)), "bf16"), "bf16", dev)
    lti = I.random_lti(2, 8, 700, 16, dtype="f32", seed=42)
    ssd = I.random_ssd(1, 2, 300, 64, dtype="f32", seed=43)
    dl = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    conv_w = torch.randn(96, 4, device=dev)

    def run():
        y, h = api.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], seg_len=256)
        st = h.clone()
        ys = api.ssm_scan_step(st, t["x"][:, :, 0].contiguous(), t["delta"][:, :, 0].contiguous(), t["A"],
                               t["B"][:, 0].contiguous(), t["C"][:, 0].contiguous(), t["D"], t["z"][:, :, 0].contiguous())
        g = api.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], dy=dy)
        xc, sc = api.ssm_conv1d_fwd(t["x"], conv_w)
        yl = api.ssm_lti_fwd(dl(lti["x"]), dl(lti["delta"]), dl(lti["A"]), dl(lti["B"]), dl(lti["C"]), dl(lti["D"]),
                             dl(lti["z"]))
        yd, hd = api.ssm_ssd_fwd(dl(ssd["x"]), dl(ssd["delta"]), dl(ssd["A"]), dl(ssd["B"]), dl(ssd["C"]),
                                 dl(ssd["D"]), dl(ssd["z"]))
        return [y, h, ys, st, g["dx"], g["ddelta"], g["dz"], xc, sc, yl, yd, hd]

    ref = run()
    torch.cuda.synchronize()
    got = _on(side, run)
    # the summed gradients (float atomics) may differ in their last bits; everything else is deterministic
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(a, b), f"output {i} differs between the default and a side stream"
