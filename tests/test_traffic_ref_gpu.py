"""The measurement references that bench.py times beside the kernels
(libtrafficref.so): each must move every byte its op moves, so their outputs
are checked bit for bit against their definitions -- residual_out = x ^
residual and y = residual_out ^ gate ^ scale ^ shift with the frame-major
(B, F, 1, C) modulation rows; y = x ^ scale ^ shift with broadcast rows for
the norm-only one -- and the rows past the problem stay untouched."""
import ctypes
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

pytestmark = pytest.mark.gpu


def _lib():
    lib = ctypes.CDLL(bench.REF_LIB)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.rn_traffic_ref.argtypes = [P] * 7 + [I64] * 4 + [P]
    lib.rn_traffic_ref.restype = ctypes.c_int
    lib.rn_traffic_ref_nss.argtypes = [P] * 4 + [I64] * 3 + [P]
    lib.rn_traffic_ref_nss.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("B,L,F", [(2, 6, 3), (1, 13, 1), (3, 35, 7)])
def test_reference_moves_every_byte(B, L, F):
    import torch
    print("traffic reference B=%d L=%d F=%d" % (B, L, F), flush=True)
    D, dev = 5120, torch.device("cuda:0")
    g = torch.Generator().manual_seed(B * 1000 + L * 10 + F)
    rows, guard = B * L, 3

    def rnd(n):
        return torch.randint(-2 ** 15, 2 ** 15, (n, D), generator=g, dtype=torch.int16).to(dev)
    x, r = rnd(rows), rnd(rows)
    gate, sc, sh = rnd(B * F), rnd(B * F), rnd(B * F)
    y = torch.full((rows + guard, D), 0x1234, dtype=torch.int16, device=dev)
    ro = torch.full((rows + guard, D), 0x4321, dtype=torch.int16, device=dev)
    st = _lib().rn_traffic_ref(y.data_ptr(), ro.data_ptr(), x.data_ptr(), r.data_ptr(), gate.data_ptr(),
                               sc.data_ptr(), sh.data_ptr(), B, L, D, F,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    frame = torch.tensor([b * F + l // (L // F) for b in range(B) for l in range(L)], device=dev)
    want_ro = x ^ r
    want_y = want_ro ^ gate[frame] ^ sc[frame] ^ sh[frame]
    assert torch.equal(ro[:rows], want_ro)
    assert torch.equal(y[:rows], want_y)
    assert bool((ro[rows:] == 0x4321).all()) and bool((y[rows:] == 0x1234).all())


@pytest.mark.parametrize("B,L", [(1, 13), (2, 8), (3, 1)])
def test_norm_only_reference_moves_every_byte(B, L):
    import torch
    print("norm-only traffic reference B=%d L=%d" % (B, L), flush=True)
    D, dev = 5120, torch.device("cuda:0")
    g = torch.Generator().manual_seed(B * 100 + L)
    rows, guard = B * L, 3

    def rnd(n):
        return torch.randint(-2 ** 15, 2 ** 15, (n, D), generator=g, dtype=torch.int16).to(dev)
    x, sc, sh = rnd(rows), rnd(1), rnd(1)
    y = torch.full((rows + guard, D), 0x1234, dtype=torch.int16, device=dev)
    st = _lib().rn_traffic_ref_nss(y.data_ptr(), x.data_ptr(), sc.data_ptr(), sh.data_ptr(), B, L, D,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(y[:rows], x ^ sc ^ sh)
    assert bool((y[rows:] == 0x1234).all())
