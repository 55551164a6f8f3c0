"""The launch plan (attn_launch_plan) without a GPU: the schedules and dispatch chunks that
the entry points choose, pinned on the headline shapes, on hand-computed chunk sizes and
on the rule's invariants over random shapes."""

import ctypes
import random

import pytest

import exact_attention_27_amd as ea

MIB = 1 << 20
FOUR, EIGHT = ea.ATTN_VARIANT_FOURWAVE, ea.ATTN_VARIANT_PINGPONG


def plan(B, Hq, Hkv, S, d, causal=True, **kw):
    return ea.attn_launch_plan(B, Hq, Hkv, S, d, causal, **kw)


@pytest.mark.parametrize("shape, causal, expect", [
    # 2k prefill: one chunk of its 64 groups, four-wave everywhere.
    ((4, 16, 16, 2048, 128), True, dict(fwd_schedule=FOUR, fwd_chunk=64, dq_chunk=64, dkdv_chunk=64, dkdv_schedule=FOUR)),
    # 32k forward and its backward: S > 4096 keeps one chunk; the dK/dV walk is 512 blocks.
    ((1, 16, 16, 32768, 128), True, dict(fwd_schedule=FOUR, fwd_chunk=16, dq_chunk=16, dkdv_chunk=16, dkdv_schedule=EIGHT)),
    # 4k backward: 64 groups x 2 MiB = 128 MiB, under the 160 MiB threshold; walk 64.
    ((4, 16, 16, 4096, 128), True, dict(fwd_schedule=FOUR, fwd_chunk=64, dq_chunk=64, dkdv_chunk=64, dkdv_schedule=FOUR)),
    # GQA step: walk 4 x 128 = 512 -> eight waves.
    ((2, 32, 8, 8192, 128), True, dict(fwd_schedule=FOUR, fwd_chunk=16, dq_chunk=16, dkdv_chunk=16, dkdv_schedule=EIGHT)),
    # Dense non-causal 32k: the ping-pong forward (B Hq ceil(S/256) = 2048 >= 256 workgroups).
    ((1, 16, 16, 32768, 128), False, dict(fwd_schedule=EIGHT, fwd_chunk=16, dq_chunk=16, dkdv_chunk=16, dkdv_schedule=EIGHT)),
    # 256 groups x 1 MiB = 256 MiB: 3 chunks -> ceil(256 / 3) = 86 -> 88 groups.
    ((16, 16, 16, 2048, 128), True, dict(fwd_chunk=88, dq_chunk=88, dkdv_chunk=88, dkdv_schedule=FOUR)),
    # 355 groups x 512,000 B (173 MiB): 2 chunks -> 178 -> 184.
    ((71, 5, 5, 1000, 128), True, dict(fwd_chunk=184, dq_chunk=184, dkdv_chunk=184)),
    # 96 groups: K/V 49 MB in all (one chunk); fp16 Q/dO of 4 heads, 2,048,000 B per group
    # (188 MiB): 2 chunks of 48.
    ((24, 16, 4, 1000, 128), True, dict(fwd_chunk=96, dq_chunk=96, dkdv_chunk=48)),
    # d = 64: 660 groups x 256,000 B (161 MiB): 2 chunks -> 330 -> 336.
    ((132, 5, 5, 1000, 64), True, dict(fwd_chunk=336, dq_chunk=336, dkdv_chunk=336, dkdv_schedule=FOUR)),
    # 26 groups of 8 query heads: dK/dV 8 MiB per group (208 MiB): 3 chunks -> 9 -> 16.
    ((13, 16, 2, 2048, 128), True, dict(fwd_chunk=26, dq_chunk=26, dkdv_chunk=16)),
])
def test_plan_of_known_shapes(shape, causal, expect):
    p = plan(*shape, causal=causal)
    for k, v in expect.items():
        assert p[k] == v, (shape, k, p)


def test_plan_options():
    # Forced schedules.
    assert plan(4, 16, 16, 2048, 128, variant=EIGHT)["fwd_schedule"] == EIGHT
    assert plan(4, 16, 16, 2048, 128, variant=EIGHT)["dkdv_schedule"] == EIGHT
    assert plan(2, 32, 8, 8192, 128, variant=FOUR)["dkdv_schedule"] == FOUR
    assert plan(1, 16, 16, 32768, 128, causal=False, variant=FOUR)["fwd_schedule"] == FOUR
    # d = 64 always runs four-wave dK/dV workgroups; the cubic exponential at d = 128 eight.
    assert plan(4, 16, 16, 2048, 64, variant=EIGHT)["dkdv_schedule"] == FOUR
    assert plan(4, 16, 16, 2048, 128, exp_mode=ea.ATTN_EXP_POLY3, variant=FOUR)["dkdv_schedule"] == EIGHT
    # Options do not move the chunks.
    assert plan(16, 16, 16, 2048, 128, variant=EIGHT, tau=0.0)["fwd_chunk"] == 88


def test_plan_errors():
    L = ea.lib()
    out = ea.attn_plan()
    assert L.attn_launch_plan(1, 2, 2, 128, 64, 1, None, None) == 1  # ATTN_ERR_NULL
    assert L.attn_launch_plan(1, 3, 2, 128, 64, 1, None, ctypes.byref(out)) == 2  # Hq % Hkv
    assert L.attn_launch_plan(-1, 2, 2, 128, 64, 1, None, ctypes.byref(out)) == 2
    assert L.attn_launch_plan(1, 2, 2, 128, 96, 1, None, ctypes.byref(out)) == 3  # d
    bad = ea.attn_default_options()
    bad.tau = float("nan")
    assert L.attn_launch_plan(1, 2, 2, 128, 64, 1, ctypes.byref(bad), ctypes.byref(out)) == 7
    with pytest.raises(Exception):
        plan(1, 2, 2, 128, 80)


def test_plan_of_empty_launches():
    p = plan(0, 4, 2, 1024, 128)
    assert p["fwd_chunk"] == 0 and p["dq_chunk"] == 0 and p["dkdv_chunk"] == 0
    p = plan(3, 4, 2, 0, 128)
    assert p["fwd_chunk"] == 6 and p["dkdv_chunk"] == 6


def test_chunk_rule_invariants():
    """Over random shapes: one chunk when S > 4096 or the re-read operands of all groups
    fit in 160 MiB; otherwise chunks are a multiple of 8 groups, the fewest of at most
    96 MiB (up to the rounding to 8 groups), and equal but for the last."""
    rng = random.Random(7)
    for _ in range(400):
        d = rng.choice([64, 128])
        Hkv = rng.choice([1, 2, 4, 5, 8, 16])
        G = rng.choice([1, 2, 4, 8])
        B = rng.randint(1, 400)
        S = rng.choice([rng.randint(1, 4096), rng.randint(4097, 20000)])
        p = plan(B, Hkv * G, Hkv, S, d)
        ngrp = B * Hkv
        for key, per_group in (("fwd_chunk", 4 * S * d), ("dq_chunk", 4 * S * d), ("dkdv_chunk", 4 * G * S * d)):
            c = p[key]
            total = ngrp * per_group
            if S > 4096 or total <= 160 * MIB:
                assert c == ngrp, (B, Hkv, G, S, d, key, c)
                continue
            nch = -(-total // (96 * MIB))
            assert c == ngrp or c % 8 == 0, (key, c)
            assert 1 <= c <= ngrp
            chunks = -(-ngrp // c)
            assert chunks <= nch, (key, c, chunks, nch)
            assert c - 8 < -(-ngrp // nch) <= c, (key, c, nch)
