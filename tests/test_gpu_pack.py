"""GPU: moe_q4_pack (row-major Q4 -> the library's 16-row groups) through the C ABI, byte for byte against
the permutation written here in numpy from the layout the header states, and DeviceWeights.upload (which
uses it) against the same permutation."""
import numpy as np
import pytest
import torch

import synth
from sparse_moe_expert_sigmoid_amd import abi
from sparse_moe_expert_sigmoid_amd.layer import DeviceWeights, to_device
from gpu_util import say


def ref_pack_codes(qs: np.ndarray) -> np.ndarray:
    """[..., rows, K/2] -> [..., rows/16, K/32, 16, 16]: the 16-byte block b of row r moves to byte
    ((r/16)*(K/32) + b)*256 + (r%16)*16 of its matrix."""
    *lead, rows, half_k = qs.shape
    nkb = half_k // 16
    return np.ascontiguousarray(qs.reshape(*lead, rows // 16, 16, nkb, 16).swapaxes(-3, -2))


def ref_pack_scales(sc: np.ndarray) -> np.ndarray:
    """[..., rows, K/32] -> [..., rows/16, K/32, 16]: the scale of row r, block b moves to element
    ((r/16)*(K/32) + b)*16 + r%16 of its matrix."""
    *lead, rows, nkb = sc.shape
    return np.ascontiguousarray(sc.reshape(*lead, rows // 16, 16, nkb).swapaxes(-1, -2))


def test_reference_permutation_by_explicit_indexing():
    """The numpy reference above, checked element by element against the header's index formulas."""
    rng = np.random.default_rng(1)
    rows, K = 48, 96
    nkb = K // 32
    qs = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    sc = rng.integers(0, 65536, (rows, nkb), dtype=np.uint16)
    pq, ps = ref_pack_codes(qs).ravel(), ref_pack_scales(sc).ravel()
    for r in range(rows):
        for b in range(nkb):
            o = ((r // 16) * nkb + b) * 256 + (r % 16) * 16
            assert bytes(pq[o:o + 16]) == bytes(qs[r, 16 * b:16 * b + 16])
            assert ps[((r // 16) * nkb + b) * 16 + r % 16] == sc[r, b]


@pytest.mark.gpu
@pytest.mark.parametrize("n_mats,rows,K", [(1, 16, 32), (3, 48, 96), (5, 64, 4096), (2, 4096, 1024),
                                           (1, 2048, 8192)])
def test_q4_pack_matches_the_permutation(n_mats, rows, K):
    say(f"[case] q4_pack n_mats={n_mats} rows={rows} K={K}")
    rng = np.random.default_rng(n_mats * 1000 + rows + K)
    qs = rng.integers(0, 256, (n_mats, rows, K // 2), dtype=np.uint8)
    sc = rng.integers(0, 65536, (n_mats, rows, K // 32), dtype=np.uint16)
    qi, si = to_device(qs, "cuda"), to_device(sc, "cuda")
    qo = torch.full_like(qi, 0x5A)
    so = torch.full_like(si, 0x5A5A)
    abi.moe_q4_pack(n_mats, rows, K, qi, si, qo, so)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qo.cpu().numpy().reshape(-1), ref_pack_codes(qs).reshape(-1))
    np.testing.assert_array_equal(so.cpu().numpy().view(np.uint16).reshape(-1), ref_pack_scales(sc).reshape(-1))
    # 2-byte aligned input scales (a row-major slice that starts mid-way) are accepted
    if n_mats == 3:
        big = torch.zeros(si.numel() + 1, dtype=si.dtype, device="cuda")
        big[1:] = si.reshape(-1)
        so2 = torch.empty_like(so)
        abi.moe_q4_pack(n_mats, rows, K, qi, big[1:], qo, so2)
        torch.cuda.synchronize()
        assert torch.equal(so2, so)


@pytest.mark.gpu
def test_device_weights_upload_uses_the_layout():
    dims = synth.Dims(T=4, d=256, E=3, k=2, I=64, I_shared=96)
    inp = synth.make_inputs(dims, seed=5)
    w = DeviceWeights.upload(inp)
    torch.cuda.synchronize()
    for name in ("w13", "w2", "s13", "s2"):
        np.testing.assert_array_equal(w[name + "_qs"].cpu().numpy().reshape(-1),
                                      ref_pack_codes(inp[name + "_qs"]).reshape(-1), err_msg=name)
        np.testing.assert_array_equal(w[name + "_sc"].cpu().numpy().view(np.uint16).reshape(-1),
                                      ref_pack_scales(inp[name + "_sc"]).reshape(-1), err_msg=name)
