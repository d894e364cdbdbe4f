"""CPU tests of the chunked feed-forward block: the oracle against what
PyTorch and the mathematics fix, and the host-side checks of the C ABI."""
import ctypes

import numpy as np
import pytest

import oracle
from memory_efficient_tiled_amd import binding


def test_gelu_matches_torch():
    import torch
    import torch.nn.functional as F
    a = np.linspace(-8.0, 8.0, 2001)
    ref = F.gelu(torch.from_numpy(a), approximate="tanh").numpy()
    assert np.max(np.abs(oracle.gelu_tanh(a) - ref)) <= 1e-15


def test_gelu_closed_forms():
    g = oracle.gelu_tanh(np.array([0.0, 40.0, -40.0]))
    assert g[0] == 0.0 and g[1] == 40.0 and abs(g[2]) < 1e-300


def test_ffn_matches_torch_mlp():
    """Against a PyTorch Linear -> GELU(tanh) -> Linear chain in float64."""
    import torch
    rng = np.random.default_rng(1)
    N, Dm, F = 37, 24, 80
    x = rng.standard_normal((N, Dm))
    w1, b1 = rng.standard_normal((F, Dm)) / 5, rng.standard_normal(F)
    w2, b2 = rng.standard_normal((Dm, F)) / 9, rng.standard_normal(Dm)
    lin1 = torch.nn.Linear(Dm, F).double()
    lin2 = torch.nn.Linear(F, Dm).double()
    with torch.no_grad():
        lin1.weight.copy_(torch.from_numpy(w1)); lin1.bias.copy_(torch.from_numpy(b1))
        lin2.weight.copy_(torch.from_numpy(w2)); lin2.bias.copy_(torch.from_numpy(b2))
        ref = lin2(torch.nn.functional.gelu(lin1(torch.from_numpy(x)), approximate="tanh"))
    assert np.max(np.abs(oracle.ffn(x, w1, b1, w2, b2) - ref.numpy())) <= 1e-12
    # without biases
    with torch.no_grad():
        ref0 = torch.from_numpy(x) @ torch.from_numpy(w1).T
        ref0 = torch.nn.functional.gelu(ref0, approximate="tanh") @ torch.from_numpy(w2).T
    assert np.max(np.abs(oracle.ffn(x, w1, None, w2, None) - ref0.numpy())) <= 1e-12


@pytest.mark.parametrize("chunk", [1, 5, 16, 37, 100])
def test_chunking_changes_nothing(chunk):
    """Rows are independent: any chunking gives the same rows (to float64
    rounding: the BLAS products block differently for other row counts)."""
    rng = np.random.default_rng(2)
    x, w1, b1 = rng.standard_normal((37, 8)), rng.standard_normal((20, 8)), rng.standard_normal(20)
    w2, b2 = rng.standard_normal((8, 20)), rng.standard_normal(8)
    rows = np.concatenate([oracle.ffn(x[i:i + 1], w1, b1, w2, b2) for i in range(37)])
    assert np.max(np.abs(oracle.ffn_chunked(x, w1, b1, w2, b2, chunk) - rows)) <= 1e-12


def test_ffn_validation():
    lib = binding.load_library()
    X, W1, B1, W2, B2, Y = (0x10000000 + i * 0x1000000 for i in range(6))

    def chk(N=100, Dm=128, F=512, chunk=64, dtype=binding.ATTN_BF16, **kw):
        a = dict(x=X, w1=W1, b1=B1, w2=W2, b2=B2, y=Y)
        a.update(kw)
        return lib.ffn_chunked_check(a["x"], a["w1"], a["b1"], a["w2"], a["b2"], a["y"], N, Dm,
                                     F, 0, chunk, dtype)
    assert chk() == 0 and chk(b1=None, b2=None) == 0 and chk(chunk=0) == 0
    assert chk(Dm=100) == binding.ATTN_EINVAL          # rows must be multiples of 8 elements
    assert chk(N=0) == binding.ATTN_EINVAL and chk(chunk=-1) == binding.ATTN_EINVAL
    assert chk(dtype=5) == binding.ATTN_EINVAL
    assert chk(y=X + 64) == binding.ATTN_EINVAL        # output overlaps x
    assert lib.ffn_workspace_bytes(64, 512, 128, binding.ATTN_BF16) >= 64 * 512 * 2


def test_library_exports_ffn_header():
    import os
    import re
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "include", "ffn.h")
    names = set(re.findall(r"^\s*(?:size_t|int)\s+(ffn_\w+)\s*\(", open(hdr).read(), re.M))
    assert names == {"ffn_chunked", "ffn_chunked_check", "ffn_workspace_bytes", "ffn_verify"}
    so = ctypes.CDLL(binding.lib_path())
    for n in names:
        assert hasattr(so, n), n
