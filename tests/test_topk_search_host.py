"""The top-k kernel's search for the k-th key, emulated on the host and checked against brute force.

The selection rule ("feat(laguna): Laguna-S-2.1 decode on the CUDA engine": the k experts with the
largest biased scores s + b, ties to the lower id) fixes one chosen set.  The kernel finds it from
order-preserving 32-bit keys held 64 per register (lanes past E hold key 0): it takes the largest key
M, counts the keys at or above v0, the start of the binade below M's, and, when at least k are there,
starts the bit-by-bit search below the leading bits those keys all share (their AND and OR); exactly k
there are the chosen set outright, and fewer send the search to the top bit.  The search keeps a
candidate bit when at least k keys reach it and stops at a candidate exactly k keys reach; the chosen
set is the keys above the threshold plus the lowest ids among the keys equal to it.  These tests
run that procedure on integers (as the kernel does) and compare its chosen set with a full sort, on
random, tied, subnormal, NaN and mixed-sign keys; each case also names the start it took, and every
start must occur.
"""
import collections
import struct

import numpy as np


def ordered_bits(f: np.float32) -> int:
    """The kernel's key: NaN just above empty slots, -0 == +0, order-preserving otherwise."""
    if f != f:
        return 1
    if f == 0:
        f = np.float32(0.0)
    u = struct.unpack("<I", struct.pack("<f", float(f)))[0]
    return (~u) & 0xFFFFFFFF if u & 0x80000000 else u | 0x80000000


def kernel_search(slots, k):
    """Chosen slot indices and the start taken, following the kernel's integer steps."""
    tau, top, start = 0, 31, "top_bit"
    M = max(slots)
    v0 = ((M & 0xFF800000) - 0x00800000) if M >= 0x01000000 else 0
    contenders = [x for x in slots if x >= v0]
    if len(contenders) == k and v0 != 0:
        tau, top, start = v0 - 1, -1, "exactly_k"
    elif len(contenders) >= k:
        A = O = contenders[0]
        for x in contenders[1:]:
            A &= x
            O |= x
        if A == O:
            tau, top, start = A, -1, "all_equal"
        else:
            top = (A ^ O).bit_length() - 1
            tau = 0 if top == 31 else A & ~((2 << top) - 1) & 0xFFFFFFFF
            start = "shared_bits"
    for bit in range(top, -1, -1):
        cand = tau | (1 << bit)
        cnt = sum(1 for x in slots if x >= cand)
        if cnt == k:
            tau = cand - 1
            break
        if cnt > k:
            tau = cand
    chosen = {i for i, x in enumerate(slots) if x > tau}
    for i, x in enumerate(slots):
        if len(chosen) < k and x == tau:
            chosen.add(i)
    return chosen, start


def brute_force(keys, k):
    return set(sorted(range(len(keys)), key=lambda i: (-keys[i], i))[:k])


def case_values(kind, E, rng):
    if kind == "sigmoid_bias":
        s = 1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.3, E)))
        return (s + rng.uniform(-0.1, 0.1, E)).astype(np.float32)
    if kind == "all_equal":
        return np.full(E, np.float32(rng.uniform(-1, 1)), dtype=np.float32)
    if kind == "few_values":
        return rng.choice(np.float32([0.25, 0.5, 0.5000001, 1.0, -0.0, 0.0]), E).astype(np.float32)
    if kind == "normal":
        return rng.normal(0.0, 1.0, E).astype(np.float32)
    if kind == "subnormal":
        return rng.uniform(-1e-39, 1e-39, E).astype(np.float32)
    if kind == "nan_and_huge":
        return rng.choice(np.float32([np.nan, 1.0, 0.5, -3.0, 1e30, -1e30]), E).astype(np.float32)
    if kind == "one_high":  # one key far above the rest: too few contenders
        v = (0.5 + rng.uniform(-0.4, 0.4, E)).astype(np.float32)
        v[rng.integers(E)] = np.float32(4.0)
        return v
    if kind == "k_high":  # k keys in [1, 2), the rest below 1/2: exactly k contenders
        return None
    raise ValueError(kind)


KINDS = ["sigmoid_bias", "all_equal", "few_values", "normal", "subnormal", "nan_and_huge", "one_high", "k_high"]


def test_search_matches_brute_force():
    rng = np.random.default_rng(2024)
    starts = collections.Counter()
    for trial in range(1600):
        E = int(rng.choice([4, 20, 63, 64, 100, 256, 500, 1024]))
        k = int(min(E, rng.choice([1, 2, 4, 10, 16, 32, E])))
        kind = KINDS[trial % len(KINDS)]
        if kind == "k_high":
            v = (0.25 + rng.uniform(0.0, 0.2, E)).astype(np.float32)
            v[rng.choice(E, size=k, replace=False)] = (1.25 + rng.uniform(0.0, 0.5, k)).astype(np.float32)
        else:
            v = case_values(kind, E, rng)
        keys = [ordered_bits(x) for x in v]
        slots = keys + [0] * (64 * ((E + 63) // 64) - E)  # lanes past E hold key 0
        chosen, start = kernel_search(slots, k)
        starts[start] += 1
        assert chosen == brute_force(keys, k), (trial, kind, E, k, start)
    assert set(starts) == {"top_bit", "exactly_k", "all_equal", "shared_bits"}, starts


def test_ordered_bits_preserve_order():
    # the key order is the float order (NaN lowest of the real keys, -0 == +0), above empty slots (0)
    vals = np.float32([-np.inf, -1e30, -1.0, -1e-45, -0.0, 0.0, 1e-45, 1e-38, 0.5, 1.0, 3e38, np.inf])
    keys = [ordered_bits(x) for x in vals]
    assert keys[4] == keys[5]
    assert all(a < b for a, b in zip(keys[:4] + keys[5:-1], keys[1:4] + keys[6:]))
    assert 0 < ordered_bits(np.float32(np.nan)) < keys[0]
