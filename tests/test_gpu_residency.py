"""The mechanism behind the one-pass kernels' residency caps, measured on the
device: under the dynamic LDS reservation of a cap W, every compute unit
holds exactly W one-wave blocks at once (ar_residency_probe); without a
reservation it holds more than any cap."""

import pytest
import torch

import ring_allreduce_rs_amd as ar

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LDS_PER_CU = 160 << 10
CAPS = [3, 4, 5, 6, 7, 8, 10, 14]     # every cap the library chooses


def reservation(w):
    # 160 KiB / (w + 1/2), rounded down to 256 bytes
    return (2 * LDS_PER_CU // (2 * w + 1)) & ~255


@pytest.mark.parametrize("w", CAPS)
def test_reservation_holds_every_cu_at_its_cap(w):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    r = ar.context(0).residency_probe(reservation(w))
    assert r == {"max_per_cu": w, "min_per_cu": w, "cus": cus}, r


def test_no_reservation_holds_more_than_any_cap():
    r = ar.context(0).residency_probe(0)
    assert r["min_per_cu"] > max(CAPS), r


def test_probe_rejects_bad_arguments():
    with pytest.raises(ar.ArError):
        ar.context(0).residency_probe((64 << 10) + 1)
    with pytest.raises(ar.ArError):
        ar.context(0).residency_probe(0, blocks=0)
