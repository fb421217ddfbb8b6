"""The device-ceiling kernels: the read stream touches every 16-byte word exactly once
(checked through its guard store), and the MFMA stream launches and completes."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

MAGIC = 0x6a09e667


def _planted(n_bytes, word):
    """A zero buffer whose 16-byte word `word` XOR-folds to the guard value."""
    import torch
    buf = np.zeros(n_bytes // 4, dtype=np.uint32)
    buf[4 * word: 4 * word + 4] = [0x12345678, 0x0f0f0f0f, 0xa5a5a5a5, MAGIC ^ 0x12345678 ^ 0x0f0f0f0f ^ 0xa5a5a5a5]
    return torch.from_numpy(buf.view(np.uint8)).cuda()


@pytest.mark.parametrize("n_bytes,n_wg", [(16, 0), (4096, 0), (1 << 20, 0), (1 << 20, 7), (3 * 16 * 1000 + 16, 3),
                                          (16 * 4097, 0), (16 * 4097, 65535), (64 << 20, 0), (64 << 20, 4096),
                                          (64 << 20, 8192)])
@pytest.mark.parametrize("nt,chunked", [(True, False), (False, False), (True, True), (False, True)])
def test_read_stream_reaches_every_word(n_bytes, n_wg, nt, chunked):
    import torch
    import attention_shared_base_amd as lra
    n16 = n_bytes // 16
    for word in sorted({0, n16 // 2, n16 - 1, (n16 * 7) // 11}):
        buf = _planted(n_bytes, word)
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        lra.ceiling_hbm_read(buf, sink, n_workgroups=n_wg, nontemporal=nt, chunked=chunked)
        torch.cuda.synchronize()
        assert int(sink[0].item()) & 0xffffffff == MAGIC, (n_bytes, n_wg, word)
        # the guard store writes the first word only
        assert int(sink[1:].abs().sum().item()) == 0


def test_read_stream_quiet_on_zero_buffer():
    import torch
    import attention_shared_base_amd as lra
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    lra.ceiling_hbm_read(buf, sink)
    lra.ceiling_hbm_read(buf, sink, chunked=True)
    torch.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0


@pytest.mark.parametrize("lds", [0, 1, 2])
def test_mfma_stream_runs(lds):
    import torch
    import attention_shared_base_amd as lra
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    flops = lra.ceiling_mfma_bf16(sink, n_workgroups=512, iters=64, lds_operands=lds)
    torch.cuda.synchronize()
    assert flops == 512 * 64 * 524288
    assert int(sink.abs().sum().item()) == 0
