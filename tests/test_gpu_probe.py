"""The read-only gather probe (a measurement aid) runs over any row list,
skipping entries that name no row, and writes nothing in practice."""

import pytest
import torch

import nvfp4_compressed_sparse_mla_amd as mla

pytestmark = pytest.mark.gpu


def test_gather_probe_runs_and_skips_rows_outside_the_cache():
    dev = torch.device("cuda:0")
    cache = torch.zeros((1000, 352), dtype=torch.uint8, device=dev)
    rows = torch.tensor([0, 999, -1, 1000, 5, 5, 1 << 30], dtype=torch.int32, device=dev)
    sink = mla.gather_probe(cache, rows)
    torch.cuda.synchronize()
    assert sink.item() == 0                    # all-zero rows fold to 0
    empty = torch.empty(0, dtype=torch.int32, device=dev)
    mla.gather_probe(cache, empty, sink)
    big = torch.randint(0, 1000, (100_000,), dtype=torch.int32, device=dev)
    mla.gather_probe(cache, big, sink)
    torch.cuda.synchronize()
    assert sink.item() == 0
