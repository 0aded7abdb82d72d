"""Exact closed forms the pages build their accounting on -- TEST INFRASTRUCTURE.

Each function states the relation it follows.  Units are plain SI (bytes,
bytes per second, seconds, sums per second) unless the name says otherwise.

Sources (cited by short tag; see oracle.c):
  [roofline-holds]  research.arkey.ai, "The roofline holds on a second GPU"
  [one-serial-kernel] vocodex.ai, "From 22.8 to 42.8 tokens a second ..."
"""
from __future__ import annotations

from fractions import Fraction

# bits per weight of each format, as exact fractions ([roofline-holds]
# "The Math": 4.5 and 6.5625 bits per weight once the scales are counted;
# "The search space": 256 weights in 144 and in 210 bytes).  The 2-bit
# format spends one fp16 scale per 32 codes: 2 + 16/32 = 2.5.
BITS_PER_WEIGHT = {
    0: Fraction(16),                       # bf16
    1: Fraction(4) + Fraction(16, 32),     # 4-bit codes + fp16 per 32
    2: Fraction(6) + Fraction(8, 16) + Fraction(16, 256),  # 6-bit + int8/16 + fp16/256
    3: Fraction(2) + Fraction(16, 32),     # 2-bit codes + fp16 per 32
}


def weight_bytes(fmt: int, n_weights: int) -> Fraction:
    """Bytes of a table of n_weights weights in format fmt."""
    return BITS_PER_WEIGHT[fmt] * n_weights / 8


def sums_per_byte(bits_per_weight: float) -> float:
    """Arithmetic intensity of one decode token: a weight of w bits costs w/8
    bytes of traffic and contributes a multiply and an add, so 2 / (w/8)
    operations per byte ([roofline-holds] "The Math")."""
    return 2.0 / (bits_per_weight / 8.0)


def m_star(bits_per_weight: float, sums_per_s: float, bytes_per_s: float) -> float:
    """Token count at which sums and bytes take equal time:
    2 M P / R = P w / (8 BW)  =>  M* = (w/16) (R/BW)  ([roofline-holds] "The Math")."""
    return (bits_per_weight / 16.0) * (sums_per_s / bytes_per_s)


def tokens_per_s_limit(bytes_per_s: float, bytes_per_token: float) -> float:
    """Roofline speed limit for decode: tokens/s <= BW / B
    ([roofline-holds] "The question", "The Math")."""
    return bytes_per_s / bytes_per_token


def floor_seconds(bytes_read: float, bytes_per_s: float) -> float:
    """Shortest time to read a table once: B / BW."""
    return bytes_read / bytes_per_s


def token_time(bytes_per_token: float, bytes_per_s: float, flops: float,
               flops_per_s: float, t_gaps: float) -> float:
    """Lower bound T >= max(B/BW, F/R) + T_gaps
    ([roofline-holds] "How the breakouts tie out: Little and Volkov")."""
    return max(bytes_per_token / bytes_per_s, flops / flops_per_s) + t_gaps


def bytes_in_flight(bytes_per_s: float, wait_s: float) -> float:
    """Little's law for a memory: L = lambda W  =>  bytes in flight = BW x W
    ([roofline-holds] "How the breakouts tie out: Little and Volkov")."""
    return bytes_per_s * wait_s


# ---------------------------------------------------------------------------
# The per-token table census of the 36-layer model the pages measure
# ([roofline-holds] "The Math": gate and up 12288 x 4096, attention 4096 x 4096
# plus key and value 1024 x 4096, down 4096 x 12288, vocabulary 151936 x 4096;
# 4-bit for gate, up and attention; 6-bit for the vocabulary and for the down
# table of every other layer).
# ---------------------------------------------------------------------------

LAYERS = 36
D_MODEL = 4096
D_KV = 1024
D_FF = 12288
VOCAB = 151936


def layer_tables(layer: int):
    """(name, fmt, N, K) of every table one layer reads; the 6-bit down table
    sits in the even layers (the pages say only "half")."""
    down_fmt = 2 if layer % 2 == 0 else 1
    return [
        ("q", 1, D_MODEL, D_MODEL),
        ("k", 1, D_KV, D_MODEL),
        ("v", 1, D_KV, D_MODEL),
        ("o", 1, D_MODEL, D_MODEL),
        ("gate", 1, D_FF, D_MODEL),
        ("up", 1, D_FF, D_MODEL),
        ("down", down_fmt, D_MODEL, D_FF),
    ]


def token_weight_bytes() -> int:
    """Exact weight bytes one token of the 36-layer stack reads."""
    total = Fraction(0)
    for layer in range(LAYERS):
        for _, fmt, n, k in layer_tables(layer):
            total += weight_bytes(fmt, n * k)
    total += weight_bytes(2, VOCAB * D_MODEL)
    assert total.denominator == 1
    return int(total)
