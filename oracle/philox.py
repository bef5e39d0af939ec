"""Oracle: the counter-based noise behind Gumbel-max sampling (test infrastructure).

The pages ask for Gumbel-max sampling "with an explicit key" and "a fresh key per
step" (mlx-arsenal "dLLM block decoding", function table in "What mlx-arsenal
ships" and the "Sampling" swap under "Reference loop"); mojo-dllm ("The loop
LLaDA uses") adds Gumbel noise to the logits before the argmax.  They name no
generator.  This build uses Philox4x32-10, the counter-based generator of
J. K. Salmon, M. A. Moraes, R. O. Dror and D. E. Shaw, "Parallel Random Numbers:
As Easy as 1, 2, 3" (SC'11), written here from that paper's definition:

  * state: a 4 x 32-bit counter (c0, c1, c2, c3) and a 2 x 32-bit key (k0, k1);
  * one round: two 32x32->64-bit products, (hi0, lo0) = M0 * c0 and
    (hi1, lo1) = M1 * c2, then the new counter is
    (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0);
  * after every round the key is bumped by the Weyl constants (k0 += W0, k1 += W1);
  * ten rounds.

Noise layout (a choice of this build; the pages leave it open): for the logit of
token v at position (b, l) and decoding step ``step`` with 64-bit ``seed``,
key = (low 32 bits of seed, high 32 bits of seed) and
counter = (v // 4, l, b, step); word v % 4 of the output is the draw.  The noise is
therefore a pure function of (seed, step, b, l, v), independent of how a GPU
launch is laid out, and any step can be recomputed on its own.

Word -> uniform: u = (w >> 9 + 0.5) * 2**-23, an odd multiple of 2**-24 in (0, 1),
exactly representable in float32.  Gumbel(0, 1): g = -log(-log u) (float64 here).
"""
import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32-10 on numpy arrays.

    counter: 4 arrays (or ints) of 32-bit values, broadcastable together.
    key:     2 ints (k0, k1).
    Returns the 4 output words as uint64 arrays holding 32-bit values.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _MASK32 for c in counter)
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = int(key[0]) & 0xFFFFFFFF
    k1 = int(key[1]) & 0xFFFFFFFF
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for _ in range(10):
        p0 = m0 * c0                      # < 2**64: no wrap in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
        k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
    return c0, c1, c2, c3


def philox_words(seed, step, b, l, V):
    """The V noise words of position (b, l) at ``step`` (uint64 array of 32-bit words)."""
    seed = int(seed)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    nblk = (int(V) + 3) // 4
    j = np.arange(nblk, dtype=np.uint64)
    w = philox4x32_10((j, l, b, step), key)
    words = np.stack(w, axis=1).reshape(-1)      # word (v % 4) of block v // 4
    return words[:V]


def uniform_from_word(w):
    """u = ((w >> 9) + 0.5) * 2**-23 in (0, 1); float64 (exact)."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel_noise(seed, step, b, l, V):
    """g_v = -log(-log u_v) for v in [0, V), float64."""
    u = uniform_from_word(philox_words(seed, step, b, l, V))
    return -np.log(-np.log(u))
