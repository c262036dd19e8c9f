"""Weight layouts: gate/up interleave at granularity 8 and the K-major form.

README ("NVFP4 MegaMoE Kernel"):
  * "Fused SwiGLU — How It Works", "The Solution": the L1 weight's gate and up
    columns are interleaved at granularity 8 along N, so the GEMM output holds
    eight gate columns, then the eight matching up columns, and so on;
  * same section, "The //2 Bug": the granularity is 8 (a leftover //2 once
    gave 4), because the interleave runs along N, not along the packed K axis;
  * "What We Have" (bridge layer): weights are quantised along K and the B
    operand is converted to K-major.

Readings: the logical L1 weight of an expert is (K, 2I) = [gate | up] (gate
columns first); the interleaved, K-major weight is (2I, K) whose row n is
logical column src(n) below.
"""

import numpy as np

GRANULARITY = 8


def interleave_src(two_i, g=GRANULARITY):
    """src[n] = logical column read by interleaved row n.

    Interleaved position n lies in group n // (2g); the first g positions of a
    group are gate columns, the next g are the matching up columns.
    """
    if two_i % (2 * g):
        raise ValueError("2I must be a multiple of 2*granularity")
    half = two_i // 2
    n = np.arange(two_i)
    grp, pos = n // (2 * g), n % (2 * g)
    col = grp * g + (pos % g)
    return np.where(pos < g, col, half + col)


def interleave_l1(w1, g=GRANULARITY):
    """Logical (E, K, 2I) [gate | up] -> interleaved K-major (E, 2I, K)."""
    w1 = np.asarray(w1)
    src = interleave_src(w1.shape[-1], g)
    return np.ascontiguousarray(np.swapaxes(w1, -1, -2)[..., src, :])


def deinterleave_cols(y, g=GRANULARITY):
    """Interleaved output columns (.., 2I) -> (gate (.., I), up (.., I))."""
    y = np.asarray(y)
    two_i = y.shape[-1]
    src = interleave_src(two_i, g)
    logical = np.empty_like(y)
    logical[..., src] = y
    return logical[..., :two_i // 2], logical[..., two_i // 2:]


def k_major(w):
    """(E, K, N) -> (E, N, K): the B operand with K contiguous."""
    return np.ascontiguousarray(np.swapaxes(np.asarray(w), -1, -2))
