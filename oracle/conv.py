"""Plain float64 oracle of the two-tap dynamic depthwise convolution.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Shares no code with
the HIP library and imports nothing from it.

Source: P1 "DFlash 2: Block diffusion, wearing a drafter's coat", section "The
architecture", sub-section "Suffix-decay convolution" (a short convolution
whose taps depend on the input, added so that the last positions of a block
are drafted as well as the first ones); P2 "A 2B Drafter Made a 27B Model
3.4x Faster. Same Exact Output.", section "The two fixes" (each block
position is combined with the one just before it).

Reading of what the pages leave open (the tap generator is not given):
  * depthwise, two taps: channel c of position t mixes only channel c of
    positions t and t-1;
  * dynamic: the two taps of every channel are generated from the position's
    own representation by one linear map, [w0_t | w1_t] = Wt @ x_t with
    Wt of shape [2 * hidden, hidden] (row c generates w0[c], row hidden + c
    generates w1[c]; 2 * hidden^2 parameters, about 16.6 M at hidden 2880,
    the size P1 states);
  * y_t = w0_t * x_t + w1_t * x_{t-1}, where the predecessor of the block's
    first position is x0, the representation of the last verified position
    (an input).
"""

import numpy as np


def conv2tap(x, x0, Wt):
    """y [L, hidden] of one stream, all float64.

    ``x`` [L, hidden] are the block's representations, ``x0`` [hidden] the
    predecessor of the first position, ``Wt`` [2 * hidden, hidden] the tap
    generator.  Plain definition: the taps of position t are the matrix-vector
    product Wt @ x_t, split into the current tap (first hidden rows) and the
    previous tap (last hidden rows); each channel is then mixed with the same
    channel of the previous position.

    Pinned by ``tests/test_oracle_conv.py``: identity and shift generators
    (closed forms x * x and x * x_prev), a cyclic permutation generator (the
    orientation of Wt), quadratic homogeneity, linearity in Wt, and causality.
    """
    x = np.asarray(x, dtype=np.float64)
    x0 = np.asarray(x0, dtype=np.float64)
    Wt = np.asarray(Wt, dtype=np.float64)
    L, H = x.shape
    assert x0.shape == (H,) and Wt.shape == (2 * H, H)
    y = np.empty((L, H))
    prev = x0
    for t in range(L):
        taps = Wt @ x[t]                 # [2H]
        y[t] = taps[:H] * x[t] + taps[H:] * prev
        prev = x[t]
    return y


def conv2tap_batch(x, x0, Wt):
    """y [B, L, hidden] for B independent streams (a loop over ``conv2tap``)."""
    x = np.asarray(x, dtype=np.float64)
    return np.stack([conv2tap(x[b], x0[b], Wt) for b in range(x.shape[0])])
