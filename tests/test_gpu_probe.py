"""The measurement aid gdn_stream_copy copies exactly (whole blocks and a
partial last block)."""
import pytest

pytestmark = pytest.mark.gpu


def test_stream_copy_exact():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_chunk_amd as gdn

    g = torch.Generator(device="cuda").manual_seed(7)
    for nbytes in (16, 32768, (1 << 20) + 48, 3 * 32768 + 4096):
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
        dst = torch.zeros_like(src)
        gdn.stream_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), nbytes
