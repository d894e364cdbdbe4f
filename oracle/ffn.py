"""CPU oracle (float64) for the chunked feed-forward block -- test infrastructure only.

Only tests, the smoke check and the bench's CPU-baseline leg may use it; it
shares no code with the HIP library.

The English noflash-attention post (ai-navigate-news.com, section "The DIY
approach", its list of what worked) names FFN chunking, with a runtime
safety check, as its second memory saver.  Reading (the post gives no
formula): the transformer's position-wise feed-forward block

    y_i = W2 act(W1 x_i + b1) + b2        for every token row i

evaluated over chunks of rows, so the N x F hidden activation never exists
at once; act is GELU with the tanh approximation (the video DiT the post
runs uses it),

    gelu(a) = a/2 (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))).

Chunking changes the order of evaluation only, so the oracle is the
definition, row by row in float64; ``ffn_chunked`` evaluates it chunk by
chunk to pin that invariance.
"""
from __future__ import annotations

import math

import numpy as np


def gelu_tanh(a: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation, float64."""
    a = np.asarray(a, dtype=np.float64)
    return 0.5 * a * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (a + 0.044715 * a ** 3)))


def ffn(x, w1, b1, w2, b2) -> np.ndarray:
    """y = W2 gelu(W1 x + b1) + b2 for every row of x, float64.

    x [N, Dm], w1 [F, Dm], b1 [F] or None, w2 [Dm, F], b2 [Dm] or None.
    """
    x = np.asarray(x, dtype=np.float64)
    h = x @ np.asarray(w1, dtype=np.float64).T
    if b1 is not None:
        h = h + np.asarray(b1, dtype=np.float64)
    y = gelu_tanh(h) @ np.asarray(w2, dtype=np.float64).T
    if b2 is not None:
        y = y + np.asarray(b2, dtype=np.float64)
    return y


def ffn_chunked(x, w1, b1, w2, b2, chunk_rows: int) -> np.ndarray:
    """The same block evaluated over chunks of ``chunk_rows`` rows."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty((x.shape[0], np.asarray(w2).shape[0]))
    for r0 in range(0, x.shape[0], chunk_rows):
        out[r0:r0 + chunk_rows] = ffn(x[r0:r0 + chunk_rows], w1, b1, w2, b2)
    return out
