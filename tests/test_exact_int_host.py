"""The integer arithmetic behind the GPU hash's exact probe order
(csrc/exact_int.h), built for the host with g++ and checked against exact
rationals: the sign of (x.a)^2 |b|^2 - (x.b)^2 |a|^2 on bf16 and float32
vectors with ties, near ties ~2^-40 .. 2^-60 apart, zero vectors and wide
exponent ranges.  A scratch array too small for the integers must give "no
room", never a write past its end (the build runs under AddressSanitizer
where the toolchain has it)."""

import os
import shutil
import struct
import subprocess
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(HERE, "..", "kv_compressed_attention_amd", "csrc", "exact_int.h")
NO_ROOM = 2


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    d = tmp_path_factory.mktemp("exact_int")
    src = open(HEADER).read().replace('#include "common.h"', "")
    (d / "exact_int_host.h").write_text(src)
    exe = str(d / "harness")
    base = [gxx, "-O1", "-std=c++17", "-w", "-I", str(d), os.path.join(HERE, "exact_int_harness.cpp"), "-o", exe]
    r = subprocess.run(base[:1] + ["-fsanitize=address,undefined"] + base[1:], capture_output=True, text=True)
    if r.returncode != 0:
        r = subprocess.run(base, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return exe, d


def _bf16_bits(a):
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _ratio_sign(x, a, b):
    fx, fa, fb = ([Fraction(float(t)) for t in v] for v in (x, a, b))
    dot = lambda u, v: sum((p * q for p, q in zip(u, v)), Fraction(0))  # noqa: E731
    na, nb = dot(fa, fa), dot(fb, fb)
    if na == 0 or nb == 0:
        return NO_ROOM
    t = dot(fx, fa) ** 2 * nb - dot(fx, fb) ** 2 * na
    return (t > 0) - (t < 0)


def _cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dt, D = int(rng.integers(2)), (64, 128)[int(rng.integers(2))]
        s = 2.0 ** rng.integers(-30, 30, size=3)
        x, a = rng.standard_normal(D) * s[0], rng.standard_normal(D) * s[1]
        mode = int(rng.integers(6))
        if mode == 0:                      # the same hyperplane twice
            b = a.copy()
        elif mode == 1:                    # a scaled copy: equal distances
            b = a * 2.0 ** int(rng.integers(-5, 5))
        elif mode == 2:                    # a near tie
            b = a.copy()
            b[rng.integers(D)] += np.abs(a).max() * 2.0 ** -int(rng.integers(20, 60))
        elif mode == 3:                    # a zero vector
            b = np.zeros(D)
        elif mode == 4:                    # sparse, exponents over +-2^60
            a = np.where(rng.random(D) < .2, a * 2.0 ** rng.integers(-60, 60, size=D), 0)
            b = np.where(rng.random(D) < .2, rng.standard_normal(D) * 2.0 ** rng.integers(-60, 60, size=D), 0)
        else:
            b = rng.standard_normal(D) * s[2]
        cap = int(rng.choice([256, 40, 12]))
        out.append((dt, D, cap, x, a, b))
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_exact_ratio_sign_matches_rationals(harness, seed):
    exe, d = harness
    cases = _cases(seed, 300)
    blob, want = [], []
    for dt, D, cap, x, a, b in cases:
        if dt == 0:
            bx, ba, bb = _bf16_bits(x), _bf16_bits(a), _bf16_bits(b)
            vals = [_bf16_value(v) for v in (bx, ba, bb)]
            raw = bx.tobytes() + ba.tobytes() + bb.tobytes()
        else:
            vs = [np.asarray(v, np.float32) for v in (x, a, b)]
            vals = [v.astype(np.float64) for v in vs]
            raw = b"".join(v.tobytes() for v in vs)
        blob.append(struct.pack("3i", dt, D, cap) + raw)
        want.append(_ratio_sign(*vals))
    path = d / f"cases{seed}.bin"
    path.write_bytes(b"".join(blob))
    r = subprocess.run([exe, str(path)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    got = [int(t) for t in r.stdout.split()]
    assert len(got) == len(want)
    decided = 0
    for (dt, D, cap, *_), g, w in zip(cases, got, want):
        if g == NO_ROOM:
            assert w == NO_ROOM or cap < 256, (dt, D, cap, w)
        else:
            assert g == w, (dt, D, cap, g, w)
            decided += 1
    # every case with the full scratch is decided; ties and near ties among them
    assert decided >= sum(1 for c, w in zip(cases, want) if c[2] == 256 and w != NO_ROOM)
    assert sum(1 for w in want if w == 0) > 10
