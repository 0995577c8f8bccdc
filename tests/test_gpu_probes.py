"""Measurement probes (include/nvq_probe.h) on the GPU: each reads exactly the bytes
it documents (the XOR of its per-wavefront words equals the XOR of those bytes when
every byte is read once) and the MFMA loop returns the closed-form accumulator sum."""
import numpy as np
import pytest
import torch

import gemm_q8_act_amd as nvq
from gemm_q8_act_amd import synth

pytestmark = pytest.mark.gpu


def _xor32(a):
    """XOR of a uint32 array (numpy)."""
    return int(np.bitwise_xor.reduce(a.astype(np.uint32))) if a.size else 0


def test_probe_read_covers_every_byte():
    rng = np.random.default_rng(17)
    nbytes = 16 * 12345  # not a multiple of the grid's stride: ragged last pass
    host = rng.integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    for blocks in (1, 7, 64):
        sink = torch.zeros(4 * blocks, dtype=torch.int32, device="cuda")
        nvq.nvq_probe_read(src, blocks, sink)
        torch.cuda.synchronize()
        got = _xor32(sink.cpu().numpy().view(np.uint32))
        assert got == _xor32(host.view(np.uint32)), f"blocks={blocks}"


@pytest.mark.parametrize("splits,waves,batch", [(1, 8, 5), (2, 4, 5)])
def test_probe_gemv_loads_reads_the_packed_matrix_once(splits, waves, batch):
    # K = 5120: 40 chunks per tile; with these shapes every wavefront's batch stays
    # inside its share, so each code word and scale pair is loaded exactly once
    N, K = 100, 5120
    codes, scales, _ = synth.nvfp4_weights(N, K, 5, "uniform")
    packed = nvq.nvq_pack_nvfp4(codes, scales)
    w = torch.from_numpy(packed).cuda()
    ntiles, nch = (N + 15) // 16, K // 128
    sink = torch.zeros(waves * ntiles * splits, dtype=torch.int32, device="cuda")
    nvq.nvq_probe_gemv_loads(w, N, K, splits, waves, batch, sink)
    torch.cuda.synchronize()
    cbytes = ntiles * nch * 1024
    want = _xor32(packed[:cbytes].view(np.uint32)) ^ _xor32(packed[cbytes:cbytes + ntiles * nch * 128].view(np.uint16))
    assert _xor32(sink.cpu().numpy().view(np.uint32)) == want


def test_probe_mfma_closed_form():
    blocks, iters = 8, 50
    out = torch.empty(256 * blocks, dtype=torch.float32, device="cuda")
    nvq.nvq_probe_mfma(blocks, iters, False, out)
    torch.cuda.synchronize()
    a = np.array([np.float16(0.001 * (i + 1)) for i in range(8)], np.float64)
    b = np.array([np.float16(0.002 * (i + 3)) for i in range(8)], np.float64)
    # every accumulator element gains sum over k < 16 of a[k % 8] * b[k % 8] per MFMA,
    # 3 MFMAs per accumulator and iteration; each thread sums 16 elements x 4 accumulators
    want = 64 * 3 * iters * 2 * float(np.dot(a, b))
    got = out.cpu().numpy().astype(np.float64)
    assert np.allclose(got, want, rtol=1e-4), (got[:4], want)
    nvq.nvq_probe_mfma(blocks, iters, True, out)
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
