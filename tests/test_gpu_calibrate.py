"""Bonus-guided calibration on the device against the oracle: calibrated logits within
the tolerance, top-16 exactly the stable order of the device's own calibrated logits and
equal to the oracle's up to near ties."""
import sys

import numpy as np
import pytest

import oracle
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
import block_diffusion_drafter_feature_amd as D  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


# (workload, batch, cal_dim); c2 is the full Qwen3-8B-shaped vocabulary and width
CASES = [("t_small", 3, 64), ("t_f32", 2, 128), ("t_batch", 12, 64), ("c2", 1, 256)]


@pytest.mark.parametrize("name,B,C", CASES)
def test_calibrate_parity(name, B, C):
    say(f"calibrate {name} batch {B} width {C}")
    wl = synth.workload(name)
    dims = wl.dims
    W = synth.make_weights(dims, wl.seed, names=["embed"])
    W.update(synth.make_cal_weights(dims, wl.seed, C, std=0.05))
    dr = D.Drafter(dims, W)
    assert dr.cfg.cal_dim == C
    r = np.random.default_rng(wl.seed)
    xh = r.standard_normal((B, 16, dims.d)).astype(np.float32)
    lg = r.standard_normal((B, 16, dims.vocab)).astype(np.float32)
    bonus = r.integers(0, dims.vocab - 1, size=B).astype(np.int32)
    lg_d = torch.from_numpy(lg).cuda()
    ci = torch.zeros((B, 16, 16), dtype=torch.int32, device="cuda")
    cl = torch.zeros((B, 16, 16), dtype=torch.float32, device="cuda")
    nb = D.dflash_calibrate_workspace_bytes(dr.cfg, B)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    D.dflash_calibrate(dr.cfg, dr.w, torch.from_numpy(xh).cuda(), i32(bonus), B, lg_d, ci, cl, ws, nb)
    torch.cuda.synchronize()
    got, ci, cl = lg_d.cpu().numpy(), ci.cpu().numpy(), cl.cpu().numpy()
    m = oracle.Model(dims, W)
    t = H.tol(dims)
    near = 0
    for b in range(B):
        want = oracle.calibrate(m, xh[b], int(bonus[b]), lg[b])
        # the bias against the oracle's bias (the logits themselves are shared inputs)
        H.assert_close_rows(f"bias b{b}", got[b] - lg[b], want - lg[b], t)
        np.testing.assert_array_equal(ci[b], H.exact_topk_of(got[b]))
        np.testing.assert_array_equal(cl[b], np.take_along_axis(got[b], ci[b].astype(np.int64), axis=1))
        near += H.topk_with_margin(ci[b], want, got[b])
        moved = np.mean([len(set(ci[b, i]) ^ set(oracle.topk(lg[b, i:i + 1], 16)[0][0])) > 0 for i in range(16)])
        say(f"  b{b}: bias max {np.abs(want - lg[b]).max():.3f}, rows whose top-16 set moved {moved:.2f}")
    say(f"  near-tie top-16 swaps: {near}")
