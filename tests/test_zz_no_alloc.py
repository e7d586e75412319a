"""dflash_verify_noalloc (the verification entry point that allocates nothing) against
dflash_verify on the same inputs: equal accept lengths and bonus tokens, bit for bit, on two
calls in a row, the second with a smaller input (the fixed scratch keeps the first call's
contents, which the second must not read)."""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
import block_diffusion_drafter_feature_amd as D  # noqa: E402


def _case(name, batch, n_draft, seed):
    dims = synth.workload(name).dims
    draft = np.random.default_rng(seed).integers(0, dims.vocab - 1, size=(batch, n_draft)).astype(np.int32)
    T = synth.make_target_logits(dims, batch, n_draft, seed + 1, planted="prefix", draft=draft)
    tdt = D.DFLASH_BF16 if dims.dtype == "bf16" else D.DFLASH_F32
    return dims, torch.from_numpy(draft).cuda(), D.to_device(T, dims), tdt


def test_verify_noalloc_matches_verify_twice():
    for name, batch, n_draft, seed in (("c5", 64, 15, 11), ("t_small", 3, 5, 12)):
        print(f"noalloc verify: {name} batch {batch} drafts {n_draft}", file=sys.stderr, flush=True)
        dims, draft, T, tdt = _case(name, batch, n_draft, seed)
        V = dims.vocab
        acc0 = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
        bon0 = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
        nb = D.dflash_verify_workspace_bytes(batch, n_draft, V)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        D.dflash_verify(draft, T, tdt, batch, n_draft, V, acc0, bon0, ws, nb)
        acc1 = torch.full((batch,), -9, dtype=torch.int32, device="cuda")
        bon1 = torch.full((batch,), -9, dtype=torch.int32, device="cuda")
        D.dflash_verify_noalloc(draft, T, tdt, batch, n_draft, V, acc1, bon1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc1.cpu().numpy(), acc0.cpu().numpy())
        np.testing.assert_array_equal(bon1.cpu().numpy(), bon0.cpu().numpy())
        assert (acc0.cpu().numpy() >= 0).all() and (acc0.cpu().numpy() <= n_draft).all()
        assert len(set(acc0.cpu().numpy().tolist())) > 1 or batch < 8


def test_verify_noalloc_refuses_oversize_without_launch():
    dims, draft, T, tdt = _case("c5", 2, 15, 13)
    acc = torch.zeros(432, dtype=torch.int32, device="cuda")
    with pytest.raises(D.DflashError) as e:
        D.dflash_verify_noalloc(draft, T, tdt, 432, 15, dims.vocab, acc, acc)
    assert e.value.status == D.DFLASH_E_WORKSPACE
