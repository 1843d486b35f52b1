"""The measurement kernels behind the benchmark's ceilings
(libmoedc_ceiling.so, include/moedc_ceiling.h) do the work they are
credited with: the write and copy streams write every byte, the scatter
writes exactly the slot bytes dispatch writes, the gather reads every row
it is charged for (its output is their XOR), and the MFMA floor runs."""
import numpy as np
import pytest
import torch

import bench
from gpu_common import log

pytestmark = pytest.mark.gpu


def _lib():
    return bench._ceiling_lib()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def test_write_and_copy_streams_cover_every_byte():
    L = _lib()
    n = (3 << 20) + 48                              # not a multiple of a workgroup's 4 or 16 KiB
    a = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    b = torch.zeros(n, dtype=torch.uint8, device="cuda")
    assert L.moedc_ceiling_copy(b.data_ptr(), a.data_ptr(), n, _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    c = torch.zeros(n, dtype=torch.uint8, device="cuda")
    assert L.moedc_ceiling_write(c.data_ptr(), n, _stream()) == 0
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert L.moedc_ceiling_read(a.data_ptr(), n, sink.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    words = c.view(torch.int32).view(-1, 4).cpu().numpy()
    assert (words[:, 2] == 0x5A5A5A5A).all() and (words[:, 3] == 0).all()   # every 16 B written
    assert int(sink.item()) == 0


def test_scatter_writes_the_slot_bytes_and_nothing_else():
    L = _lib()
    T, K, stride, row = 300, 4, 7680, 7424
    rng = np.random.default_rng(3)
    S = 2000
    slots = np.full((T, K), -1, np.int32)
    for t in range(T):
        slots[t] = rng.choice(S, K, replace=False)
    slots[rng.random((T, K)) < 0.1] = -1
    buf = torch.full((S, stride), 0xA5, dtype=torch.uint8, device="cuda")
    sd = torch.from_numpy(slots).cuda()
    assert L.moedc_ceiling_scatter(sd.data_ptr(), T, K, buf.data_ptr(), stride, row, _stream()) == 0
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    used = np.unique(slots[slots >= 0])
    unused = np.setdiff1d(np.arange(S), used)
    assert (h[unused] == 0xA5).all()
    assert (h[used][:, row:] == 0xA5).all()        # the stride's tail untouched
    # each written slot holds its (last) token's pattern: the token id in word 0 of every 8 B
    w = h[used][:, :row].view(np.uint32).reshape(len(used), -1, 2)
    owner = {}
    for t in range(T):
        for s in slots[t]:
            if s >= 0:
                owner.setdefault(int(s), set()).add(t)
    for i, s in enumerate(used):
        assert set(np.unique(w[i, :, 0]).tolist()) <= owner[int(s)]
    log(f"  scatter: {len(used)} slots written, {len(unused)} untouched")


def test_gather_reads_every_row_it_is_charged_for():
    L = _lib()
    T, K, S, rb = 257, 8, 3000, 2 * 1152
    rng = np.random.default_rng(4)
    rows = torch.from_numpy(rng.integers(0, 2 ** 16, (S, rb // 2), dtype=np.uint16).view(np.int16)).cuda()
    slots = rng.integers(0, S, (T, K)).astype(np.int32)
    slots[rng.random((T, K)) < 0.2] = -1
    out = torch.zeros((T, rb // 2), dtype=torch.int16, device="cuda")
    sd = torch.from_numpy(slots).cuda()
    assert L.moedc_ceiling_gather(rows.data_ptr(), sd.data_ptr(), T, K, rb, rb, out.data_ptr(),
                                  _stream()) == 0
    torch.cuda.synchronize()
    hr = rows.cpu().numpy().view(np.uint32)
    want = np.zeros((T, rb // 4), np.uint32)
    for t in range(T):
        for s in slots[t]:
            if s >= 0:
                want[t] ^= hr[s]
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("fold", [0, 1])
def test_mfma_floor_runs(fold):
    L = _lib()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert L.moedc_ceiling_mfma(256 * 8 * 32 * 10, fold, sink.data_ptr(), _stream()) == 0
    assert L.moedc_ceiling_mfma(0, fold, sink.data_ptr(), _stream()) != 0   # rejected, no launch
    torch.cuda.synchronize()
