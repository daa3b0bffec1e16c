"""The Python binding rejects tensors the C ABI cannot take safely (host
memory, another device, a wrongly shaped or strided output) before any
launch.  The C ABI takes plain pointers and writes outputs densely, so these
checks are what keeps a host pointer or a short buffer away from a kernel.

CPU part: host tensors are refused.  GPU part: mixed devices are impossible
with one GPU, so it checks shapes, dtypes and contiguity; every case raises
in Python and nothing is launched.
"""

import pytest
import torch

import nvfp4_compressed_sparse_mla_amd as mla


def _cpu_args(T=2, H=32, K=16, rows=64):
    q = torch.zeros((T, H, 576), dtype=torch.float16)
    cache = torch.zeros((rows, 352), dtype=torch.uint8)
    idx = torch.zeros((T, K), dtype=torch.int32)
    return q, cache, idx


def test_host_tensors_are_refused_by_decode():
    q, cache, idx = _cpu_args()
    with pytest.raises(ValueError, match="GPU memory"):
        mla.sparse_decode(q, cache, idx, 0.1)


def test_host_tensors_are_refused_by_append_and_staging():
    lat = torch.zeros((3, 512), dtype=torch.float16)
    rope = torch.zeros((3, 64), dtype=torch.float16)
    slots = torch.arange(3)
    cache = torch.zeros((8, 352), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU memory"):
        mla.quantize_append(lat, rope, slots, cache)
    with pytest.raises(ValueError, match="GPU memory"):
        mla.fp8_quantize_append(lat, rope, slots, torch.zeros((8, 576), dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU memory"):
        mla.gather_dequant_fp8(cache, torch.zeros((2, 4), dtype=torch.int32))


@pytest.mark.gpu
def test_bad_outputs_and_operands_raise_before_launch():
    dev = "cuda:0"
    T, H, K = 2, 32, 16
    q = torch.zeros((T, H, 576), dtype=torch.float16, device=dev)
    cache = torch.zeros((64, 352), dtype=torch.uint8, device=dev)
    idx = torch.zeros((T, K), dtype=torch.int32, device=dev)
    bad = [
        dict(out=torch.empty((T, H, 256), dtype=torch.float16, device=dev)),
        dict(out=torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)),
        dict(out=torch.empty((T, 512, H), dtype=torch.float16, device=dev).transpose(1, 2)),
        dict(lse=torch.empty((T, H), dtype=torch.float16, device=dev)),
        dict(lse=torch.empty((T, H + 1), dtype=torch.float32, device=dev)),
        dict(out=torch.empty((T, H, 512), dtype=torch.float16)),            # host memory
        dict(workspace=torch.zeros(4096, dtype=torch.int32, device=dev)),
        dict(fmt="fp4"),
        dict(block_table=torch.zeros((1, 4), dtype=torch.int32, device=dev)),   # no token_seq
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            mla.sparse_decode(q, cache, idx, 0.1, **kw)
    with pytest.raises(ValueError):
        mla.sparse_decode(q, cache, idx.to(torch.int64), 0.1)
    with pytest.raises(ValueError):
        mla.sparse_decode(q, torch.zeros((64, 576), dtype=torch.uint8, device=dev), idx, 0.1)
    with pytest.raises(ValueError):
        mla.gather_dequant_fp8(cache, idx, rows=torch.empty((T * K - 1, 576), dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        mla.gather_dequant_fp8(cache, idx, staged_indices=torch.empty((T, K), dtype=torch.int64, device=dev))
    lat = torch.zeros((3, 512), dtype=torch.float16, device=dev)
    rope = torch.zeros((3, 64), dtype=torch.float16, device=dev)
    with pytest.raises(ValueError):
        mla.quantize_append(lat, rope, torch.arange(3), cache)                 # slots in host memory
    torch.cuda.synchronize()
