"""The read-rate reference kernel (mfa_stream_read) reads every byte of its
buffer exactly once: the XOR of its sink equals the XOR of the buffer's
32-bit words, on sizes that do and do not split evenly over the workgroups,
and a sink shorter than one word per thread is refused."""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 16 * 7, 64 << 20, (64 << 20) + 16 * 12345])
def test_stream_read_touches_every_word_once(nbytes):
    rng = np.random.default_rng(nbytes % 1000)
    words = rng.integers(-2**31, 2**31, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(words).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.full((cus * 512,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    mfa.mfa_stream_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words.view(np.uint32))
    assert got == want


def test_stream_read_refuses_a_short_sink():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    sink = torch.zeros(cus * 512 - 1, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="MFA_ERR_SHAPE"):
        mfa.mfa_stream_read(src, sink)
