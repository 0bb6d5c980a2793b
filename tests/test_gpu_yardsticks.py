"""GPU checks of the measurement kernels behind the benchmark's measured ceilings: the read
stream's XOR and the copy, bit for bit on ragged sizes, and the bf16 MFMA loop against a host
model of the 16x16x32 MFMA operand and result lane layout (exact: short bf16 inputs)."""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_canvas_amd import driver

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (3 << 20) + 48, (64 << 20) + 16 * 1001])
def test_read_stream_xor_and_copy(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    src = torch.from_numpy(host).to(DEV)
    word = torch.full((1,), 12345, dtype=torch.int32, device=DEV)   # overwritten by the call
    driver.read_stream(src, nbytes, word)
    dst = torch.zeros_like(src)
    driver.copy_bytes(dst, src, nbytes)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert np.uint32(word.cpu().numpy().view(np.uint32)[0]) == want
    assert torch.equal(dst, src)


def _bf16(bits):
    return np.array([b << 16 for b in bits], dtype=np.uint32).view(np.float32).astype(np.float64)


def _operand(lane, words):
    # 8 bf16 elements of a lane's 16-byte operand: element e is half e % 2 of word e // 2
    return _bf16([(words[e // 2] >> (16 * (e % 2))) & 0xFFFF for e in range(8)])


@pytest.mark.parametrize("iters", [1, 3])
def test_mfma_loop_matches_lane_layout_model(iters):
    blocks = driver.mfma_loop_blocks()
    out = torch.zeros(blocks * 256, dtype=torch.float32, device=DEV)
    driver.mfma_loop(iters, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(blocks, 4, 64)
    # operands of lane l (the kernel's constants)
    a = [_operand(l, [0x3F803F80 ^ l, 0x3F003F00, 0x3E803E80, 0x3F803F80]) for l in range(64)]
    b = [_operand(l, [0x3F803F80, 0x3F803F80 ^ (l << 1), 0x3F003F00, 0x3E803E80]) for l in range(64)]
    # A[i][k] is element k % 8 of lane i + 16 (k // 8); B[k][j] likewise for lane j + 16 (k // 8)
    A = np.array([[a[i + 16 * (k // 8)][k % 8] for k in range(32)] for i in range(16)])
    B = np.array([[b[j + 16 * (k // 8)][k % 8] for j in range(16)] for k in range(32)])
    Cm = A @ B
    # lane (column j, group g) holds C[4 g + r][j], r < 4; 8 chains of `iters` MFMAs each
    want = np.array([iters * 8 * sum(Cm[4 * (l // 16) + r][l % 16] for r in range(4))
                     for l in range(64)], dtype=np.float64)
    assert np.array_equal(got, np.broadcast_to(want.astype(np.float32), got.shape))
