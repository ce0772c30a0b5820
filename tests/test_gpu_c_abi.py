"""The library called from plain C (tests/c_abi/rehydrate_demo.c: hipMalloc'd buffers,
kamera_batch_workspace_bytes, kamera_rehydrate_batched on the null stream, or
kamera_rehydrate_batched_noalloc without a workspace), checked
against the fp64 oracle: one GQA chunk of 2 heads x 128, 2 layers, rank-8 factors on K
and V (Kamera preprint Eq. 1), bf16 tolerance as in the other parity tests."""
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle.kamera_oracle as O
from oracle import tolerance as tol
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

DEMO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "rehydrate_demo")
L, H, HD, F, M = 2, 2, 128, 256, 8


def bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


@pytest.mark.parametrize("T,delta,noalloc", [(1, 3, False), (77, -40000, False), (300, 123456, False),
                                             (300, 123456, True), (33, -7, True)])
def test_plain_c_caller_matches_oracle(T, delta, noalloc):
    assert os.path.exists(DEMO), f"{DEMO} is missing: build it with __graft_entry__.build()"
    say(f"[c-abi] T={T} delta={delta} noalloc={noalloc}")
    rng = np.random.default_rng(T)
    k, v = bf16(rng.standard_normal((L, T, F))), bf16(rng.standard_normal((L, T, F)))
    uk, vk = bf16(0.2 * rng.standard_normal((L, T, M))), bf16(0.2 * rng.standard_normal((L, F, M)))
    uv, vv = bf16(0.2 * rng.standard_normal((L, T, M))), bf16(0.2 * rng.standard_normal((L, F, M)))
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        np.concatenate([a.ravel() for a in (k, v, uk, vk, uv, vv)]).astype("<u2").tofile(fin)
        r = subprocess.run([DEMO, fin, fout, str(T), str(delta)] + (["noalloc"] if noalloc else []),
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        say("  " + r.stdout.strip())
        out = np.fromfile(fout, dtype="<u2").reshape(2, L, T, F)
    for layer in range(L):
        facs = [O.Factor(0, 0, O.upcast(uk[layer], O.BF16), O.upcast(vk[layer], O.BF16).T),
                O.Factor(1, 0, O.upcast(uv[layer], O.BF16), O.upcast(vv[layer], O.BF16).T)]
        xk, xv = O.upcast(k[layer], O.BF16), O.upcast(v[layer], O.BF16)
        yk, yv = O.rehydrate_gqa(xk, xv, delta, num_kv_heads=H, head_dim=HD, base=1e6, factors=facs)
        for t, (x, y) in enumerate(((xk, yk), (xv, yv))):
            S = O.abs_terms(x, tensor=t, delta=delta, rotate_this=t == 0, bands=O.band_offsets(O.GQA, H, HD),
                            d_rot=HD, base=1e6, pairing=O.NEOX, factors=facs)
            res = tol.check_bf16(out[t, layer], y, O.round_to(y, O.BF16), S, M + 4)
            assert res["fail"] == 0, (layer, t, res["n"])
