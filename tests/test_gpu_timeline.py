"""The calibration stream's timeline (ar_stream_timeline): it performs the
in-place N-read / N-write XOR stream bit for bit, whatever the LDS
reservation, and every block leaves a start and an end on the device clock."""

import numpy as np
import pytest
import torch

import ring_allreduce_rs_amd as ar

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LDS_PER_CU = 160 << 10


def reservation(w):
    return 0 if w == 0 else (2 * LDS_PER_CU // (2 * w + 1)) & ~255


@pytest.mark.parametrize("n,nbytes,waves", [(8, (1 << 20) + 48, 5), (8, 4096, 0),
                                             (3, (1 << 20) + 16, 0), (12, 65536 + 1008, 6)])
def test_timeline_stream_xors_in_place_and_stamps_every_block(n, nbytes, waves):
    g = torch.Generator(device="cuda")
    g.manual_seed(n * 1000 + nbytes)
    bufs = [torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda",
                          generator=g) for _ in range(n)]
    want = bufs[0].clone()
    for t in bufs[1:]:
        want ^= t
    blocks = -(-nbytes // 1024)
    ts = torch.zeros(2 * blocks + 6, dtype=torch.int64, device="cuda")
    nblk, khz = ar.stream_timeline(bufs, reservation(waves), ts)
    torch.cuda.synchronize()
    assert nblk == blocks and khz > 0
    for t in bufs:
        assert torch.equal(t, want)
    stamps = ts[:2 * blocks].view(-1, 2).cpu().numpy()
    assert (stamps[:, 0] > 0).all() and (stamps[:, 1] >= stamps[:, 0]).all()
    span_us = (stamps[:, 1].max() - stamps[:, 0].min()) / (khz / 1e3)
    assert 0 < span_us < 1e6
    assert (ts[2 * blocks:] == 0).all()      # nothing written past the last block's entries


def test_timeline_rejects_bad_arguments():
    bufs = [torch.zeros(1024, dtype=torch.int32, device="cuda") for _ in range(2)]
    ts = torch.zeros(8, dtype=torch.int64, device="cuda")
    with pytest.raises(ar.ArError):
        ar.stream_timeline(bufs, 0, ts[:7])                   # 4 blocks need 8 entries
    with pytest.raises(ar.ArError):
        ar.stream_timeline(bufs, (64 << 10) + 1, ts)          # reservation above 64 KiB
    with pytest.raises(ar.ArError):
        ar.stream_timeline([bufs[0], bufs[0]], 0, ts)         # overlapping buffers
