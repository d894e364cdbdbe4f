"""GPU parity of the chunked feed-forward block against the oracle.

Tolerance (derived): the first product is rounded to the 16-bit type
(relative u = 2^-8 bf16, 2^-11 fp16) before bias and GELU, which moves
h_f = gelu(a_f + b1_f) by about |gelu'(z_f)| |a_f| u; h is rounded again
(|h_f| u); the second product sums these with weights w2 in fp32, so y_d is
off by a sum of independent errors of standard deviation
sqrt(sum_f ((|gelu'(z_f)| |a_f| + |h_f|) u w2_df)^2 / 3), bounded by 6 of
them; its rounding, the bias add and the final rounding add
(|W2 h|_d + |y_d|) u.  Mean error within 1.5 times the mean standard
deviation plus the rounding terms' mean.
"""
import numpy as np
import pytest

import oracle
from memory_efficient_tiled_amd import inputs
from tests.parity import log, to_device

pytestmark = pytest.mark.gpu

U = {inputs.BF16: 2.0 ** -8, inputs.F16: 2.0 ** -11}


def _bound(x, w1, b1, w2, b2, dtype):
    a = x @ w1.T
    z = a + (0.0 if b1 is None else b1)
    h = oracle.gelu_tanh(z)
    eps = 1e-6
    dg = (oracle.gelu_tanh(z + eps) - oracle.gelu_tanh(z - eps)) / (2 * eps)
    u = U[dtype]
    e = (np.abs(dg) * np.abs(a) + np.abs(h)) * u               # [R, F]
    sigma = np.sqrt((e ** 2) @ (w2 ** 2).T / 3.0)               # [R, Dm]
    yg = h @ w2.T
    y = yg + (0.0 if b2 is None else b2)
    rnd = (np.abs(yg) + np.abs(y)) * u
    return 6.0 * sigma + rnd, 1.5 * sigma + rnd, y


def _run(device, N, Dm, F, dtype, chunk, seed, bias=True, rows=None, verify=False):
    import torch
    from memory_efficient_tiled_amd import ffn_chunked
    log(f"ffn N={N} Dm={Dm} F={F} {dtype} chunk={chunk} bias={bias} seed={seed}")
    xi = inputs.make_ffn_inputs(N, Dm, F, dtype, seed=seed)
    dev = [to_device(a, dtype, device) for a in (xi.x, xi.w1, xi.b1, xi.w2, xi.b2)]
    x, w1, b1, w2, b2 = dev
    if not bias:
        b1 = b2 = None
    y = ffn_chunked(x, w1, b1, w2, b2, chunk_rows=chunk, verify=verify)
    torch.cuda.synchronize(device)
    got = y.float().cpu().numpy().astype(np.float64)
    dec = [oracle.decode(a, dtype) for a in (xi.x, xi.w1, xi.b1, xi.w2, xi.b2)]
    if not bias:
        dec[2] = dec[4] = None
    ri = np.arange(N) if rows is None else rows
    bound, mbound, ref = _bound(dec[0][ri], dec[1], dec[2], dec[3], dec[4], dtype)
    assert np.max(np.abs(ref - oracle.ffn(dec[0][ri], *dec[1:]))) <= 1e-9
    err = np.abs(got[ri] - ref)
    log(f"  max|err| {err.max():.3e} mean|err| {err.mean():.3e} worst err/bound "
        f"{np.max(err / bound):.3f} rms(y) {np.sqrt(np.mean(ref ** 2)):.3e}")
    assert np.all(np.isfinite(got[ri]))
    assert np.all(err <= bound), "error above the bound"
    assert err.mean() <= mbound.mean(), "mean error above the bound"


@pytest.mark.parametrize("dtype", [inputs.F16, inputs.BF16])
@pytest.mark.parametrize("chunk", [0, 1, 37, 64, 1000])
def test_ffn_chunks(gpu_device, chunk, dtype):
    _run(gpu_device, 300, 64, 256, dtype, chunk, seed=chunk + 1)


def test_ffn_no_bias(gpu_device):
    _run(gpu_device, 130, 128, 512, inputs.BF16, 50, seed=7, bias=False)


def test_ffn_verify(gpu_device):
    """The runtime chunking check passes for a correct chunking."""
    _run(gpu_device, 700, 256, 1024, inputs.BF16, 200, seed=8, verify=True)


def test_ffn_video_width_sampled(gpu_device):
    """Model width 1536, hidden 8960 (a 1.3B video DiT), 4100 rows in chunks
    of 1000; 64 sampled rows against the oracle (first, last, chunk edges)."""
    rows = np.unique(np.concatenate([[0, 999, 1000, 1999, 2000, 3999, 4000, 4099],
                                     np.random.default_rng(9).choice(4100, 56, replace=False)]))
    _run(gpu_device, 4100, 1536, 8960, inputs.BF16, 1000, seed=9, rows=rows, verify=True)


@pytest.mark.parametrize("chunk", [4864, 0])
def test_ffn_verify_14b_width(gpu_device, chunk):
    """Model width 5120, hidden 13824 (the 14B video DiT's block), 10000 rows.
    With 4864-row chunks the check evaluates the first 2 * 4864 + 1 = 9729
    rows as one chunk, the product shape whose GEMM workspace selection is
    fixed (a candidate is taken only if its stated workspace fits the
    buffer); 0 takes the library's chunk (3072 rows at this width).  Output
    finite, 48 sampled rows (chunk edges included) against the oracle."""
    N, Dm, F = 10000, 5120, 13824
    rows = np.unique(np.concatenate([[0, 3071, 3072, 4863, 4864, 9727, 9728, 9729, 9999],
                                     np.random.default_rng(10).choice(N, 39, replace=False)]))
    _run(gpu_device, N, Dm, F, inputs.BF16, chunk, seed=10, rows=rows, verify=True)


def test_ffn_verify_rejects_nan(gpu_device):
    """A NaN in the input gives NaN rows in both evaluations; the check must
    fail on it rather than drop it."""
    import torch
    from memory_efficient_tiled_amd import ffn_chunked
    dtype = inputs.BF16
    xi = inputs.make_ffn_inputs(300, 64, 256, dtype, seed=11)
    x, w1, b1, w2, b2 = (to_device(a, dtype, gpu_device)
                         for a in (xi.x, xi.w1, xi.b1, xi.w2, xi.b2))
    x[5, 3] = float("nan")
    with pytest.raises(RuntimeError, match="chunking check failed"):
        ffn_chunked(x, w1, b1, w2, b2, chunk_rows=100, verify=True)
    torch.cuda.synchronize(gpu_device)
