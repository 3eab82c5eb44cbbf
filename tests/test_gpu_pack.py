"""GPU: the packed weight layout written by pkv_pack_weight, checked
bit-exactly against a numpy re-layout written here from the layout's
definition (blocks of 16 rows x 32 columns, lane chunk l = 16 i + m holds
row(G, m), columns 32 s + 8 i .. + 8)."""
import numpy as np
import pytest
import torch

import paged_kv_transformer_amd as pkv
import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu


def row_of(layout, rows, G, m):
    if layout in (pkv.PACK_QKV, pkv.PACK_QKV128):
        D = 64 if layout == pkv.PACK_QKV else 128
        j = 8 * (G % (D // 16)) + (m % 8)
        r = D * (G // (D // 16)) + (j if m < 8 else D // 2 + j)
        return r if r < rows else -1
    if layout == pkv.PACK_GATE_UP:
        I = rows // 2
        i = 8 * G + (m % 8)
        return (i if m < 8 else I + i) if i < I else -1
    r = 16 * G + m
    return r if r < rows else -1


def reference_pack(W, layout):
    rows, cols = W.shape
    S = cols // 32
    groups = (rows // 2 + 7) // 8 if layout == pkv.PACK_GATE_UP else (rows + 15) // 16
    out = np.zeros((groups, S, 4, 16, 8), dtype=np.uint16)
    for G in range(groups):
        for m in range(16):
            r = row_of(layout, rows, G, m)
            if r < 0:
                continue
            out[G, :, :, m, :] = W[r].reshape(S, 4, 8)
    return out.reshape(-1)


@pytest.mark.parametrize("rows,cols,layout", [
    (37, 64, pkv.PACK_ROWS), (1000, 128, pkv.PACK_ROWS), (3 * 64 * 3, 96, pkv.PACK_QKV),
    (3 * 128 * 2, 96, pkv.PACK_QKV128),
    (2 * 48, 160, pkv.PACK_GATE_UP), (2 * 64, 64, pkv.PACK_GATE_UP),
])
def test_pack_weight_matches_reference_layout(rows, cols, layout):
    W = synth.bf16_normal(9, "w_o", (rows, cols), 1.0, 0.0, (rows, layout))
    got = pkv.pack_weight(dev(W), layout)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint16), reference_pack(W, layout))
