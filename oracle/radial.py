"""The radial network's last layer joined to the convolution (oracle; test infrastructure).

The convolution's per-edge weights come from a radial network of the edge
length ([COURSE] 06a: m_ij = (R(|r_ij|) Y(rhat_ij)) (x)_w h_j; [V2106]: radial
features feed Convolution). Its last layer is a linear map of the hidden
activations h[e] (reading: no bias, Linear(hidden -> W) as in the benchmark's
radial MLP). [E3J] E.4 and F.1 fuse message formation and avoid materialising
edge-wise intermediates in HBM; [XNN] "What to expect from fast
implementations" notes that above a million edges the radial networks are
recomputed rather than stored. Forming w inside the convolution changes where
it is computed, not what is computed:

  w[e, k] = sum_j h[e, j] W2[j, k]               h [E][H], W2 [H][W] row-major
  out     = conv.forward(x, Y, w, scale)

Backward (chain rule through the linear layer), with (dx, dY, dw) the
convolution's cotangents for the output cotangent g:

  dh  = dw W2^T                 [E][H]
  dW2 = sum over edges of h^T dw  [H][W]
"""

import numpy as np

from . import conv


def edge_weights(h, W2):
    """w = h W2, one matrix product."""
    return np.asarray(h, np.float64) @ np.asarray(W2, np.float64)


def forward(L, row_ptr, src, x, Y, h, W2, scale, pad_node=None):
    return conv.forward(L, row_ptr, src, x, Y, edge_weights(h, W2), scale, pad_node)


def backward(L, row_ptr, src, x, Y, h, W2, scale, g, pad_node=None):
    """Cotangents (dx, dY, dh, dW2) for the output cotangent g."""
    h = np.asarray(h, np.float64)
    W2 = np.asarray(W2, np.float64)
    dx, dY, dw = conv.backward(L, row_ptr, src, x, Y, edge_weights(h, W2), scale, g, pad_node)
    return dx, dY, dw @ W2.T, h.T @ dw
