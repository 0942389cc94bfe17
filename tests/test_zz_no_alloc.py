"""archead_logits_noalloc (the library's own per-GPU workspace, no allocation)
against archead_logits (the caller's workspace), through the C ABI.

Two calls in a row on one head: first 300 tokens (the tile path), then a
smaller call of 5 tokens (the decode path), which reuses the array the first
call left behind.  Each is compared with archead_logits on the same inputs:
max|dY| <= 2e-3 max|Y| and the same per-row argmax (with less room for the
split-tile partial sums, the tile path may split a tile's hidden dimension
differently, which changes the fp32 summation order), and with the oracle.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL, ah_mod, check_parity, device_H, log, to_f64, torch_mod


def _call(fn, head, H_bits):
    torch = torch_mod()
    H = device_H(H_bits)
    Y = torch.full((H.shape[0], head.V), float("nan"), dtype=torch.float32, device="cuda")
    fn(H, head, Y)
    torch.cuda.synchronize()
    return to_f64(Y)


@pytest.mark.gpu
def test_noalloc_matches_logits_on_two_calls():
    ah = ah_mod()
    inp = synth.make("tiny", seed=17, V=3000, D=1024, N=300, r_c=32, r_r=32, g=128, n_outlier=4)
    head = ah.PackedHead.from_components(inp.head)
    for n in (300, 5):  # the second call is smaller and takes the other path
        Hb = np.ascontiguousarray(inp.H_bits[:n])
        log(f"noalloc V=3000 D=1024 r_c=r_r=32 g=128 N={n}")
        Ya = _call(ah.archead_logits_noalloc, head, Hb)
        Yb = _call(ah.archead_logits, head, Hb)
        assert not np.isnan(Ya).any()
        scale = np.abs(Yb).max()
        assert np.abs(Ya - Yb).max() <= TOL * scale, (n, np.abs(Ya - Yb).max() / scale)
        assert np.array_equal(np.argmax(Ya, 1), np.argmax(Yb, 1))
        check_parity(Ya, oracle.logits(Hb, inp.head), f"noalloc N={n}")


def test_noalloc_rejects_calls_beyond_its_array():
    """A call whose workspace exceeds the library's array is refused before
    anything touches the GPU (the pointers are never dereferenced)."""
    ah = ah_mod()
    V, D, r_c, r_r, g = 151936, 4096, 64, 64, 128
    dims = ah.ArcheadDims(V, D, r_c, r_r, g)

    def call(n):
        H = ah.ArcheadTensor(16, n, D, D, ah.ARCHEAD_BF16)
        Y = ah.ArcheadTensor(16, n, V, V, ah.ARCHEAD_F32)
        P = ah.ArcheadPackedHead(dims, 256, 1 << 40, None, 0)
        return ah.lib.archead_logits_noalloc(ctypes.byref(H), ctypes.byref(P), ctypes.byref(Y), None)

    assert call(4096) == 7        # ARCHEAD_E_WORKSPACE: 4096 tokens need 32 MiB of converted H alone
    assert call(0) == 0           # no tokens: nothing to do
    assert ah.lib.archead_logits_noalloc(None, None, None, None) == 1  # ARCHEAD_E_NULL
    assert ah.ARCHEAD_NOALLOC_SCRATCH_BYTES == 16 << 20
