"""Small seeded inputs for the oracle's CPU pins (no method arithmetic)."""
import numpy as np

from bit_trainable_attention_block_amd import workloads as wl


def gaussian_head(N, D, seed, dtype=wl.BF16, sigma=1.0, k_offset=0.0, q_offset=0.0):
    """One head of Q, K, V, dO rounded to the I/O dtype; returns float64 arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for t in range(4):
        x = rng.standard_normal((N, D)).astype(np.float32)
        if t < 2:
            x = x * np.float32(sigma)
        if t == 1 and k_offset:
            x = x + (rng.standard_normal(D).astype(np.float32) * np.float32(k_offset))[None, :]
        if t == 0 and q_offset:
            x = x + (rng.standard_normal(D).astype(np.float32) * np.float32(q_offset))[None, :]
        bits = wl.to_io_bits(x.astype(np.float32), dtype)
        out.append(wl.bits_to_float32(bits, dtype).astype(np.float64))
    return out
