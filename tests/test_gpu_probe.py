"""The read-bandwidth probe reads what it is given: a buffer of zeros leaves
the sink clear, one 16-byte word whose xor is the probe's constant sets it,
wherever that word lies (every decomposition the bench uses, ragged chunks)."""
import ctypes

import pytest
import torch

import commit_step_amd as dc
from gpu_util import log

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("nbytes,wgs,nt", [(1 << 20, 256, 512), (1 << 20, 2048, 256),
                                           (16 * 12345, 7, 256), (16 * 5, 64, 512)])
def test_read_probe_reads_every_word(nbytes, wgs, nt):
    lib = dc.load_library()
    dev = torch.device("cuda:0")
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    log(f"read probe {nbytes} bytes, {wgs} x {nt}")
    assert lib.dllm_read_probe(buf.data_ptr(), nbytes, wgs, nt, sink.data_ptr(), s) == 0
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    for word in (0, nbytes // 16 // 2, nbytes // 16 - 1):
        buf.zero_()
        buf[4 * word] = ctypes.c_int32(MAGIC).value          # xor of the word = MAGIC
        sink.zero_()
        assert lib.dllm_read_probe(buf.data_ptr(), nbytes, wgs, nt, sink.data_ptr(), s) == 0
        torch.cuda.synchronize()
        assert int(sink.item()) == 1, f"word {word} not read"
