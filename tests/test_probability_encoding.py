"""The probabilities of the attention kernel's value product, modelled on the CPU.

The kernel writes each 32-token block's probabilities as a two-term E4M3 pair relative to
the block's integer maximum m_b (log2 units): with p256 = 2^(x - m_b + 8) in (0, 256],
hi = E4M3(p256) and lo = E4M3(16 (p256 - hi)), and the value product applies the E8M0
scales 2^(m_b - m_ref - 8) and 2^(m_b - m_ref - 12) (m_ref: the accumulator's reference).
These tests model that arithmetic (fp32, round-to-nearest-even E4M3 as the conversion
instructions do) and check the error bound stated for it: |p~ - p| <= 2^-8 p + 2^-14 2^(m_b-8),
and its effect on an attention output against the tolerance of the GPU parity tests,
including a dominant token and latents with a large common mean.
"""
import numpy as np
import pytest
import torch

O_ATOL, O_RTOL = 2e-2, 1e-2  # the GPU parity tolerance of the attention output


def e4m3(x):
    t = torch.from_numpy(np.asarray(x, np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def encode_blocks(x_log2):
    """x_log2: [n] logits in log2 units (n a multiple of 32).  Returns the represented
    probabilities relative to 2^m_ref (m_ref = the largest block maximum), like the kernel's
    scaled value product sees them, and the block maxima."""
    x = np.asarray(x_log2, np.float32).reshape(-1, 32)
    m_b = np.ceil(x.max(axis=1)).astype(np.int64)  # integer block maximum
    m_ref = m_b.max()
    p256 = np.exp2((x - m_b[:, None] + 8).astype(np.float32)).astype(np.float32)
    hi = e4m3(p256)
    lo = e4m3(np.float32(16.0) * (p256 - hi.astype(np.float32)))
    rep = (hi + lo / 16.0) * np.exp2((m_b - m_ref - 8).astype(np.float64))[:, None]
    return rep.reshape(-1), m_b, m_ref


def exact_rel(x_log2, m_ref):
    return np.exp2(np.asarray(x_log2, np.float64) - m_ref)


@pytest.mark.parametrize("seed", range(6))
def test_two_term_e4m3_error_bound(seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 3 + 4 * seed, 2048)  # spreads from a few to ~70 log2 units
    rep, m_b, m_ref = encode_blocks(x)
    p = exact_rel(x.astype(np.float32), m_ref)
    bound = 2.0 ** -8 * p + 2.0 ** -14 * np.repeat(np.exp2((m_b - m_ref - 8).astype(np.float64)), 32)
    assert (np.abs(rep - p) <= bound * (1 + 1e-6)).all()


def test_block_maximum_is_exact_and_small_blocks_keep_their_precision():
    # a block far below the dominant one is represented relative to its own maximum
    x = np.full(64, -40.0)
    x[:32] = 0.0
    x[40] = -39.5
    rep, _, m_ref = encode_blocks(x)
    p = exact_rel(x, m_ref)
    assert rep[0] == p[0] == 1.0
    assert abs(rep[40] - p[40]) <= 2.0 ** -8 * p[40]


def _attention_error(logits_nat, v, seed=0):
    """max |O~ - O| for one head: O = sum_t softmax(logits)_t v_t, with the kernel's
    probability encoding in O~ (the softmax sum uses the unquantised probabilities)."""
    x = np.asarray(logits_nat, np.float64) / np.log(2.0)
    rep, _, m_ref = encode_blocks(x)
    p = exact_rel(x.astype(np.float32), m_ref)
    z = p.sum()
    o_exact = (p[:, None] * v).sum(0) / z
    o_enc = (rep[:, None] * v).sum(0) / z
    return np.abs(o_enc - o_exact), np.abs(o_exact)


@pytest.mark.parametrize("case", ["random", "dominant", "two_dominant", "large_mean"])
def test_encoded_attention_within_the_parity_tolerance(case):
    rng = np.random.default_rng(11)
    n = 2048
    v = e4m3(rng.normal(0, 1, (n, 64)))           # E4M3 latent values
    logits = rng.normal(0, 2, n)
    if case == "dominant":
        logits[777] += 30.0                        # one token carries almost all the weight
    elif case == "two_dominant":
        logits[5] += 25.0
        logits[2040] += 24.3
    elif case == "large_mean":
        v = e4m3(rng.normal(3.0, 1.0, (n, 64)))    # every value shares a large mean
        logits = rng.normal(0, 4, n)
    err, mag = _attention_error(logits, v)
    assert (err <= 0.25 * (O_ATOL + O_RTOL * mag)).all(), err.max()
    # the encoding alone moves O by far less than the tolerance: about 2^-8 of |v|
    assert err.max() <= 2.0 ** -7 * np.abs(v).max()
