"""Counter-keyed random streams and fp32/bf16 encodings.

Streams are NumPy PCG64 generators keyed by a SeedSequence spawn key, so each
(workload, tensor, index...) tuple names one independent stream.  Large
tensors are filled in fixed-size blocks, each block from its own stream, on a
thread pool: the bits depend only on the seed and the block layout, never on
the number of threads.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# One stable integer per tensor name, used inside spawn keys.
_TENSOR_IDS = {
    "h": 1, "w1": 2, "b1": 3, "wlm": 4, "tree": 5, "topk_ids": 6, "root": 7,
    "q": 8, "k": 9, "v": 10, "logits": 11, "plant": 12, "cache_k": 13,
    "cache_v": 14, "prefix": 15, "misc": 16, "h_tree": 17, "w_base": 18,
    "uniforms": 19,
}

_BLOCK = 1 << 20  # elements per independently seeded block


def _tid(tensor):
    return _TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)


def stream(seed, workload_id, tensor, *keys):
    """A NumPy Generator for one (workload, tensor, keys...) stream."""
    key = (int(workload_id), _tid(tensor)) + tuple(int(k) for k in keys)
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(int(seed), spawn_key=key)))


def _threads():
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed, workload_id, tensor, keys, n, std=1.0, mean=0.0):
    """``n`` float32 normal variates N(mean, std^2), filled block by block.

    Block ``i`` comes from ``stream(seed, workload_id, tensor, *keys, i)``.
    """
    out = np.empty(int(n), dtype=np.float32)
    nblk = (int(n) + _BLOCK - 1) // _BLOCK

    def fill(i):
        g = stream(seed, workload_id, tensor, *keys, i)
        lo = i * _BLOCK
        hi = min(int(n), lo + _BLOCK)
        blk = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        if mean != 0.0:
            blk += np.float32(mean)
        out[lo:hi] = blk

    if nblk <= 1:
        for i in range(nblk):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def bf16_bits(x):
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    n = flat_u.size

    def conv(lo, hi):
        s = flat_u[lo:hi].astype(np.uint64)
        r = (s + 0x7FFF + ((s >> 16) & 1)) >> 16
        nan = (s & 0x7FFFFFFF) > 0x7F800000
        r = np.where(nan, (s >> 16) | 0x40, r)
        flat_o[lo:hi] = r.astype(np.uint16)

    step = 1 << 22
    spans = [(lo, min(n, lo + step)) for lo in range(0, n, step)]
    if len(spans) <= 1:
        for lo, hi in spans:
            conv(lo, hi)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda s: conv(*s), spans))
    return out


def bf16_to_f32(bits):
    """Decode uint16 bf16 bits to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_round(x):
    """Round to float32 (the exact value a float32 buffer would hold)."""
    return np.asarray(x, dtype=np.float32)
