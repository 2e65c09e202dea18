"""Counter-based random numbers and the sampled next token -- TEST
INFRASTRUCTURE ONLY.

Definitions followed:
  * API reference page, ``medusa_generate`` and ``generate_candidates``
    (arguments ``temperature``, ``posterior_threshold``, ``posterior_alpha``,
    ``top_p``, ``sampling='typical'``): with a positive temperature the
    tree's root -- the base model's token after the last accepted one -- is
    drawn from the base distribution under the sampling mode rather than
    taken as its argmax.  The pages name the arguments and nothing more.
    Reading taken: in typical mode the token is drawn from
    p = softmax(logits / temperature) restricted to the tokens the typical
    rule would accept, p(x) > min(eps, delta * exp(-H(p))) (the same test
    and float32 comparison as the acceptance), renormalised; in nucleus mode
    it is the nucleus draw of ``nucleus.py``.  A draw walks the allowed
    tokens in token-id order and returns the first whose running mass
    exceeds u times the allowed mass (the highest allowed id if none).  The
    argmax always qualifies when delta < 1 (p_max >= exp(-H) > delta *
    exp(-H)), so the allowed set is never empty.
  * Philox4x64-10, J. K. Salmon, M. A. Moraes, R. O. Dror and D. E. Shaw,
    "Parallel random numbers: as easy as 1, 2, 3", SC 2011: a 4 x 64-bit
    counter and a 2 x 64-bit key; ten rounds, each multiplying two counter
    words by the constants 0xD2E7470EE14C6C93 and 0xCA5A826395121157 (full
    128-bit products), exchanging halves and xoring in the key, the key
    bumped by the Weyl constants 0x9E3779B97F4A7C15 and 0xBB67AE8584CAA73B
    between rounds.

Keying (a choice of this library, stated in its header): the random number
of (seed, step, sequence b, tree node n, purpose) is the top 24 bits of the
first output word of Philox4x64-10 with counter (n, b, step, purpose) and
key (seed, 0), as u = bits * 2^-24 in [0, 1) (exact in float32).  Purpose 0
draws a node's nucleus sample, purpose 1 the typical-mode next token.
"""

import numpy as np

from .common import as_f64

_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B
_MASK = (1 << 64) - 1

PURPOSE_NUCLEUS = 0
PURPOSE_NEXT_TOKEN = 1


def philox4x64(counter, key, rounds=10):
    """Philox4x64 block: four 64-bit output words for a 4-word counter and a
    2-word key (Python integers)."""
    c0, c1, c2, c3 = (int(x) & _MASK for x in counter)
    k0, k1 = (int(x) & _MASK for x in key)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = (p1 >> 64) ^ c1 ^ k0, p1 & _MASK, (p0 >> 64) ^ c3 ^ k1, p0 & _MASK
    return [c0, c1, c2, c3]


def uniform(seed, step, b, node, purpose):
    """The float32 uniform in [0, 1) of one (seed, step, sequence, node,
    purpose): the top 24 bits of the first Philox word, times 2^-24."""
    w = philox4x64([node, b, step, purpose], [seed, 0])[0]
    return np.float32((w >> 40) * 2.0 ** -24)


def uniforms(seed, step, B, T, purpose):
    """float32 [B][T] of uniform() over sequences and nodes."""
    out = np.empty((B, T), dtype=np.float32)
    for b in range(B):
        for n in range(T):
            out[b, n] = uniform(seed, step, b, n, purpose)
    return out


def _f32(x):
    return float(np.float32(x))


def typical_allowed(logits_row, temperature, eps, delta):
    """The tokens the typical rule accepts at one node, ascending, and
    their probabilities p = softmax(logits / temperature)."""
    t = _f32(temperature)
    if not t > 0.0:
        raise ValueError("temperature must be positive")
    z = as_f64(logits_row) / t
    m = z.max()
    e = np.exp(z - m)
    S = e.sum()
    H = np.log(S) - ((z - m) * e).sum() / S
    thr = min(_f32(eps), _f32(delta) * np.exp(-H))
    p = e / S
    keep = p.astype(np.float32) > np.float32(thr)
    ids = np.flatnonzero(keep)
    return ids, p[ids]


def typical_sample(logits_row, temperature, eps, delta, u):
    """The token drawn from the typical set of one node with uniform u."""
    ids, p = typical_allowed(logits_row, temperature, eps, delta)
    target = min(max(_f32(u), 0.0), 1.0) * p.sum()
    run = 0.0
    for v, pv in zip(ids, p):
        run += pv
        if run > target:
            return int(v)
    return int(ids[-1])


def sample_next_typical(logits, retrieve, best_path, accept_len, temperature, eps, delta, seed, step):
    """The typical-mode next token of each sequence: drawn at the last
    accepted node (retrieve[best_path[b]][accept_len[b]]) with the purpose-1
    uniform of (seed, step, b, node 0).  logits [B][T][V] float32."""
    logits = np.asarray(logits)
    B = logits.shape[0]
    out = np.zeros(B, dtype=np.int64)
    for b in range(B):
        node = int(np.asarray(retrieve)[int(best_path[b]), int(accept_len[b])])
        u = uniform(seed, step, b, 0, PURPOSE_NEXT_TOKEN)
        out[b] = typical_sample(logits[b, node], temperature, eps, delta, u)
    return out
