"""Exhaustive check of the device quantizer: for every positive finite BF16
amax and every BF16 x with |x| <= amax (about 1.07e9 pairs), the INT8 code
and the fp32 scale written by moedc_dispatch equal the oracle's bit for bit.
Each 128-value group holds amax followed by 127 test values; tokens of 7168
values are dispatched to one slot each."""
import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M

from gpu_common import dev, dev_i16, log

pytestmark = pytest.mark.gpu

H = 7168
G = H // 128


def groups_for(amax_lo, amax_hi):
    """All groups for amax bit patterns in [amax_lo, amax_hi)."""
    out = []
    for a in range(amax_lo, amax_hi):
        mags = np.arange(a + 1, dtype=np.uint16)
        vals = np.concatenate([mags, mags | np.uint16(0x8000)])
        pad = (-vals.size) % 127
        if pad:
            vals = np.concatenate([vals, np.zeros(pad, np.uint16)])
        g = vals.reshape(-1, 127)
        out.append(np.concatenate([np.full((g.shape[0], 1), a, np.uint16), g], axis=1))
    return np.concatenate(out)


@pytest.mark.parametrize("chunk", range(8))
def test_quantizer_every_bf16_pair(chunk):
    edges = np.linspace(1, 0x7F80, 9).astype(int)
    lo, hi = int(edges[chunk]), int(edges[chunk + 1])
    g = groups_for(lo, hi)
    ntok = -(-g.shape[0] // G)
    pad = ntok * G - g.shape[0]
    if pad:
        g = np.concatenate([g, np.zeros((pad, 128), np.uint16)])
    x = g.reshape(ntok, H)
    log(f"[case] amax bits [{lo:#06x}, {hi:#06x}): {x.size:,} values in {ntok} tokens")
    plan = M.Plan(max_tokens=ntok, hidden=H, num_logical=1, num_phys=1, top_k=1,
                  capacity=[ntok])
    sd = plan.sizes.slot_stride
    dbuf = torch.empty((ntok, sd), dtype=torch.uint8, device="cuda")
    slots = np.arange(ntok, dtype=np.int32).reshape(ntok, 1)
    plan.dispatch(dev_i16(x), dev(slots), dbuf)
    torch.cuda.synchronize()
    got = dbuf[:, : H + 4 * G].cpu().numpy()
    del dbuf
    q, s = oracle.quantize_tokens(x)
    assert np.array_equal(got[:, :H], q.view(np.uint8)), "INT8 codes differ"
    assert np.array_equal(got[:, H:], s.view(np.uint8)), "scales differ"
