"""Seeded random inputs (no method arithmetic).

Host arrays come from numpy's PCG64 seeded by ``SeedSequence([root, *key])``;
device arrays (large workloads that do not fit a host round trip) come from a
torch generator on the device seeded from the same key.  Weights are
N(0, sigma) with sigma the standard deviation; activations are N(0, 1)
rounded to bf16 by torch's own conversion; router logits are N(0, 1) fp32.

Keys: (workload, layer, matrix id, role) with role W=0, x=1, logits=2.
"""

import numpy as np

ROLE_W, ROLE_X, ROLE_LOGITS = 0, 1, 2
ROOT_SEED = 0


def seed_for(*key):
    """A 63-bit integer seed derived from the key (for torch generators)."""
    ss = np.random.SeedSequence([ROOT_SEED, *[int(k) for k in key]])
    return int(ss.generate_state(1, np.uint64)[0] >> np.uint64(1))


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, *[int(k) for k in key]])))


def host_normal(shape, sigma, *key):
    """fp32 N(0, sigma) array of the given shape."""
    r = _rng(*key).standard_normal(shape, dtype=np.float32)
    return (r * np.float32(sigma)).astype(np.float32)


def to_bf16_bits(a32):
    """fp32 -> bf16 bit patterns via torch's CPU conversion (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host_bf16_normal(shape, *key):
    """bf16 activations N(0, 1) as uint16 bit patterns."""
    return to_bf16_bits(_rng(*key).standard_normal(shape, dtype=np.float32))


def host_logits(n, *key):
    """fp32 N(0, 1) router logits."""
    return _rng(*key).standard_normal(n, dtype=np.float32)


def device_normal(shape, sigma, device, *key):
    """torch fp32 N(0, sigma) tensor generated on ``device``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*key))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, 1.0, generator=g)
    t.mul_(sigma)
    return t


def device_bf16_normal(shape, device, *key):
    """torch bf16 N(0, 1) activations generated on ``device``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*key))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, 1.0, generator=g)
    return t.to(torch.bfloat16)
