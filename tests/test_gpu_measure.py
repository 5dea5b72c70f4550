"""The measurement aids on the device: moe_stream_read and moe_tile_copy_read
run, size their buffers as documented, and fold what they read into the
sink deterministically (the same call twice gives the same words)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_layer_lds_amd as m
    return m


def test_stream_read_folds_deterministically(lib):
    buf = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    s1 = torch.zeros(64, dtype=torch.int32, device="cuda")
    s2 = torch.zeros(64, dtype=torch.int32, device="cuda")
    lib.moe_stream_read(buf, s1)
    lib.moe_stream_read(buf, s2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)


@pytest.mark.parametrize("pattern", [0, 1, 2])
def test_tile_copy_read_patterns(lib, pattern):
    cus = lib.moe_device_cu_count()
    if cus < 128:
        pytest.skip("the tile-copy measurement needs at least 128 compute units")
    row_bytes = 2048
    nbytes = (cus // 128) * 8 * 160 * row_bytes
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    s1 = torch.zeros(cus, dtype=torch.int32, device="cuda")
    s2 = torch.zeros(cus, dtype=torch.int32, device="cuda")
    lib.moe_tile_copy_read(pattern, buf, row_bytes, 2, s1)
    lib.moe_tile_copy_read(pattern, buf, row_bytes, 2, s2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    # one byte short of the documented size, or one sink word short: refused
    with pytest.raises(lib.MoeError):
        lib.moe_tile_copy_read(pattern, buf[:-1], row_bytes, 1, s1)
    with pytest.raises(lib.MoeError):
        lib.moe_tile_copy_read(pattern, buf, row_bytes, 1, s1[:-1])
