"""The allocation-free decode layer (ssm_mamba1_decode_layer_noalloc, its
workspace in the library's per-GPU device array) against the layer that takes
a caller workspace: the same inputs through both, two calls in a row, the
second with a smaller batch and other dimensions, so that it runs over the
first call's leftovers in the array.  Both run the same kernels in the same
order, so hidden and both caches must agree bit for bit (within the parity
bar of tests/_parity.py by construction)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import state_space_model_causal_amd as ssm

    ssm.load_library()
    return torch.device("cuda:0")


CALLS = [
    # Mamba-1 2.8B layer at the 245-request decode batch, then a small bf16
    # layer with padded requests
    (dict(batch=245, nslots=300, io="f16", state="f32"), 0),
    (dict(d_model=128, d_inner=256, d_state=16, dt_rank=16, batch=6, nslots=8, io="bf16",
          state="bf16"), 3),
]


def test_noalloc_layer_matches_workspace_layer(dev):
    import state_space_model_causal_amd as ssm

    for call, (kw, pad) in enumerate(CALLS):
        print(f"no-alloc layer call {call}: {kw}", flush=True)
        t = W.mamba1_layer(seed=60 + call, device=dev, **kw)
        idx = t["slot_idx"].clone()
        if pad:
            idx[::pad] = -1
        desc = ssm.mamba1_layer(t["w"], eps=1e-5)
        a = [t["hidden"].clone(), t["conv_state"].clone(), t["ssm_state"].clone()]
        b = [t["hidden"].clone(), t["conv_state"].clone(), t["ssm_state"].clone()]
        ssm.mamba1_decode_layer(desc, *a, slot_idx=idx)
        ssm.mamba1_decode_layer_noalloc(desc, *b, slot_idx=idx)
        torch.cuda.synchronize()
        for name, x, y in zip(("hidden", "conv_state", "ssm_state"), a, b):
            assert torch.equal(x, y), f"call {call}: {name} differs"
        # the call did something: hidden rows of named requests moved
        live = (idx >= 0).nonzero().flatten()
        assert not torch.equal(b[0][live], t["hidden"][live])
        padded = (idx < 0).nonzero().flatten()
        np.testing.assert_array_equal(b[0][padded].cpu().float().numpy(),
                                      t["hidden"][padded].cpu().float().numpy())
