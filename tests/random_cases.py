"""Seeded random plan and launch shapes shared by the GPU parity tests and
the CPU emulation tests (so that every random case the GPU runs has first
run through the emulator's bounds checks)."""
import numpy as np


def case(seed):
    """Plan shape (N, B, S, Hq, Hkv, d), mode name, layout and tuning fields
    of random case `seed`: a valid plan of at most 2M elements per tensor and
    every tuning field drawn from its valid range."""
    rng = np.random.default_rng(1000 + seed)
    while True:
        N = int(rng.choice([1, 2, 3, 4, 6, 8]))
        mode = int(rng.integers(0, 2))
        if mode == 1:
            B = int(rng.choice([x for x in (1, 2, 3, 4, 6, 8) if N % x == 0] + [N * int(rng.integers(2, 4))]))
            P = N // B if B <= N else 1
        else:
            B = int(rng.integers(1, 5))
            P = N
        S = P * int(rng.integers(1, 40))
        Hkv = P * int(rng.integers(1, 4))
        Hq = Hkv * int(rng.integers(1, 4))
        d = int(rng.choice([1, 2, 3, 5, 8, 16, 24, 40, 64]))
        if B * S * Hq * d <= 2_000_000:
            break
    tuning = dict(block_size=int(rng.choice([0, 64, 128, 256])), vectors_per_thread=int(rng.choice([0, 1, 2, 4, 8])),
                  tile_heads=int(rng.integers(0, 5)), tile_tokens=int(rng.choice([0, 0, 1, 3, 17])),
                  tile_order=int(rng.integers(0, 4)), lane_order=int(rng.integers(0, 3)),
                  xcd_remap=int(rng.integers(0, 3)), stage=int(rng.integers(0, 3)),
                  batch_order=int(rng.integers(0, 3)), cache_policy=int(rng.integers(0, 6)),
                  max_grid=int(rng.choice([0, 0, 1, 7, 33])))
    return (N, B, S, Hq, Hkv, d), ("basp" if mode else "ulysses"), int(rng.integers(0, 2)), tuning


COUNT = 200


def group_case(seed):
    """Plan shape, number of groups G (dividing N and B, 1 < G < B and G < N
    when possible), layout and tuning of random general-G case `seed`."""
    rng = np.random.default_rng(5000 + seed)
    while True:
        N = int(rng.choice([2, 4, 6, 8, 12]))
        B = int(rng.choice([2, 3, 4, 6, 8, 12, 16]))
        Gs = [g for g in range(1, N + 1) if N % g == 0 and B % g == 0]
        inner = [g for g in Gs if 1 < g < min(B, N)]
        G = int(rng.choice(inner or Gs))
        P = N // G
        S = P * int(rng.integers(1, 30))
        Hkv = P * int(rng.integers(1, 4))
        Hq = Hkv * int(rng.integers(1, 4))
        d = int(rng.choice([1, 3, 8, 24, 40, 64]))
        if B * S * Hq * d <= 1_500_000:
            break
    tuning = dict(block_size=int(rng.choice([0, 64, 128, 256])), vectors_per_thread=int(rng.choice([0, 1, 2, 4, 8])),
                  tile_heads=int(rng.integers(0, 5)), tile_tokens=int(rng.choice([0, 0, 1, 3, 17])),
                  tile_order=int(rng.integers(0, 4)), lane_order=int(rng.integers(0, 3)),
                  xcd_remap=int(rng.integers(0, 3)), stage=int(rng.integers(0, 3)),
                  batch_order=int(rng.integers(0, 3)), cache_policy=int(rng.integers(0, 6)),
                  max_grid=int(rng.choice([0, 0, 1, 7, 33])))
    return (N, B, S, Hq, Hkv, d), G, int(rng.integers(0, 2)), tuning


GROUP_COUNT = 100
