"""MOE_GG_VALIDATE=1: the weight gradient, data gradient and grouped GEMM entry points reject
malformed offsets with EINVAL before launching; without it they launch (results unspecified)."""
import numpy as np
import pytest

from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu

GOOD = [0, 100, 200, 256]
BAD = {"decreasing": [0, 200, 100, 256], "first_not_zero": [8, 100, 200, 256], "last_not_M": [0, 100, 200, 255]}


def _calls(torch, mg):
    d = torch.device("cuda:0")
    M, N, K, E = 256, 256, 256, 3
    u8 = dict(dtype=torch.uint8, device=d)
    wg = lambda off: mg.wgrad_mxfp8(torch.zeros((N, M), **u8), torch.zeros((K, M), **u8),
                                    torch.full((N, M // 32), 127, **u8), torch.full((K, M // 32), 127, **u8), off)
    dg = lambda off: mg.dgrad_f32(torch.zeros((M, N), dtype=torch.float32, device=d),
                                  torch.zeros((E, N, K), dtype=torch.float32, device=d), off)
    gg = lambda off: mg.grouped_mxfp8(torch.zeros((M, K), **u8), torch.zeros((E, N, K), **u8),
                                      torch.full((M, K // 32), 127, **u8), torch.full((E, N, K // 32), 127, **u8), off)
    return {"wgrad": wg, "dgrad": dg, "grouped": gg}


@pytest.mark.parametrize("entry", ["wgrad", "dgrad", "grouped"])
def test_validate_env_rejects_malformed_offsets(entry, monkeypatch):
    torch, mg = require_gpu()
    call = _calls(torch, mg)[entry]
    off = lambda v: torch.tensor(v, dtype=torch.int32, device="cuda:0")
    monkeypatch.setenv("MOE_GG_VALIDATE", "1")
    say("validate", entry)
    out = call(off(GOOD))
    torch.cuda.synchronize()
    assert float(out.float().abs().max()) == 0.0              # zero operands, well-formed offsets
    for name, bad in BAD.items():
        with pytest.raises(mg.MoeGGError) as err:
            call(off(bad))
        assert err.value.status == mg.EINVAL, name
    monkeypatch.delenv("MOE_GG_VALIDATE")
    call(off(BAD["decreasing"]))                              # not checked: launches, no access outside
    torch.cuda.synchronize()
