"""The weight packer (moe_pack_mxfp4) through the C ABI: a byte permutation, so
its output must equal, byte for byte, the packed layout of include/moe.h written
out with numpy index arithmetic here (no GPU code involved in the expectation),
including the zero padding of the last K step when K % 128 == 64."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def pack_reference(codes: np.ndarray, scales: np.ndarray):
    """Packed layout of include/moe.h from codes [E][N][K/2], scales [E][N][K/32]."""
    E, N, Kh = codes.shape
    K = 2 * Kh
    S, G, nblk = (K + 127) // 128, N // 32, K // 32
    blocks = np.zeros((E, N, 4 * S, 16), np.uint8)           # per-block 16-byte code runs
    blocks[:, :, :nblk] = codes.reshape(E, N, nblk, 16)
    sc = np.zeros((E, N, 4 * S), np.uint8)
    sc[:, :, :nblk] = scales
    l = np.arange(64)
    row = l % 32
    pc = np.zeros((E, G, S, 2, 64, 16), np.uint8)
    ps = np.zeros((E, G, S, 64, 2), np.uint8)
    for g in range(G):
        for j in range(S):
            for s in range(2):
                pc[:, g, j, s] = blocks[:, 32 * g + row, 4 * j + 2 * (l // 32) + s]
            b0 = 4 * j + 2 * (l // 32)
            ps[:, g, j, :, 0] = sc[:, 32 * g + row, b0]
            ps[:, g, j, :, 1] = sc[:, 32 * g + row, b0 + 1]
    return pc.reshape(-1), ps.reshape(-1)


@pytest.mark.parametrize("E,N,K", [(3, 64, 128), (2, 128, 192), (1, 2880, 2880), (5, 320, 4160)])
def test_pack_matches_layout(E, N, K):
    import torch

    import sparse_moe_transformer_gemm_amd as moe
    rng = np.random.default_rng(E * 1000 + N + K)
    codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(100, 140, (E, N, K // 32), dtype=np.uint8)
    print(f"[pack] E={E} N={N} K={K}", flush=True)
    pc, ps = moe.pack_mxfp4(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda())
    torch.cuda.synchronize()
    rc, rs = pack_reference(codes, scales)
    assert np.array_equal(pc.cpu().numpy(), rc)
    assert np.array_equal(ps.cpu().numpy(), rs)
