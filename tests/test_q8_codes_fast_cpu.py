"""The argument behind the one-division-per-block Q8 encoder of the fused
quantize + Q4_K x Q8 launch, checked on the CPU (no GPU).

The device encoder forms each quotient as v * (1/d) and falls back to the
exact division when that product's fractional part lies within 2^-13 of 0.5,
or when d is zero, subnormal or not finite.  Its claim: the codes equal
round-half-away(RN(v / d)) clamped to [-127, 127] (the Q8 rule, with the
correctly rounded f32 quotient) for every input.  This program restates the
encoder's steps in C with IEEE f32 arithmetic (no contraction) and compares
them with the exact rule on random blocks over 220 binades, on block maxima,
on quotients placed within 4 ulps of every k + 0.5, and on the special
values zero, infinity and the extremes of the f32 range.  The GPU parity
test on half-way activations checks the device code itself.
"""
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
static int code_exact(float v, float d) {
    int q = 0;
    if (d != 0.0f) { volatile float t = v / d; float r = roundf(t); r = fminf(fmaxf(r, -127.0f), 127.0f); q = (int)r; }
    return q;
}
static int code_fast(float v, float d, int *slow_out) {
    const float y = 1.0f / d;
    int slow = !(d >= 0x1p-126f && d <= 0x1p+126f);
    const float q = v * y;
    const float t = truncf(q);
    const float f = fabsf(q - t);
    slow = slow || !(fabsf(f - 0.5f) >= 0x1p-13f);
    const float r = f >= 0.5f ? t + copysignf(1.0f, q) : t;
    int c = (int)fminf(fmaxf(r, -127.0f), 127.0f);
    if (slow) c = code_exact(v, d);
    *slow_out = slow;
    return c;
}
static uint64_t s = 88172645463325252ull;
static uint64_t rnd(void) { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return s; }
static float unif(void) { return (float)((rnd() >> 11) * 0x1p-53); }
int main(int argc, char **argv) {
    const long cases = atol(argv[1]);
    long bad = 0, n = 0, fast = 0;
    int slow;
    for (long it = 0; it < cases; ++it) {
        const float amax = ldexpf(1.0f + unif(), (int)(rnd() % 220) - 110);
        const volatile float d = amax / 127.0f;
        float v;
        const int mode = (int)(rnd() % 4);
        if (mode == 0) {
            v = (2.0f * unif() - 1.0f) * amax;
        } else if (mode == 1) {
            v = (rnd() & 1) ? amax : -amax;
        } else {
            const int k = (int)(rnd() % 127);
            float w = ((float)k + 0.5f) * d;
            const int steps = (int)(rnd() % 9) - 4;
            for (int j = 0; j < abs(steps); ++j) w = nextafterf(w, steps > 0 ? INFINITY : -INFINITY);
            if (fabsf(w) > amax) w = amax;
            v = mode == 3 ? -w : w;
        }
        const int a = code_exact(v, d), b = code_fast(v, d, &slow);
        fast += !slow; ++n;
        if (a != b) { if (bad < 5) printf("mismatch v=%a d=%a exact=%d fast=%d\n", v, d, a, b); ++bad; }
    }
    const float sp[] = {0.0f, -0.0f, INFINITY, -INFINITY, 0x1p-149f, 0x1p-126f, 1.0f, 0x1.fffffep127f};
    for (int i = 0; i < 8; ++i)
        for (int j = 0; j < 8; ++j) {
            const float v = sp[i];
            const volatile float d = fabsf(sp[j]) / 127.0f;
            const int a = code_exact(v, d), b = code_fast(v, d, &slow);
            ++n;
            if (a != b) { printf("mismatch special v=%a d=%a exact=%d fast=%d\n", v, d, a, b); ++bad; }
        }
    printf("cases %ld mismatches %ld fast-path %ld\n", n, bad, fast);
    return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_q8_codes_fast_equal_exact_division(tmp_path):
    src = tmp_path / "q8fast.c"
    exe = tmp_path / "q8fast"
    src.write_text(SRC)
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", str(src), "-o", str(exe), "-lm"],
                   check=True, capture_output=True)
    p = subprocess.run([str(exe), "20000000"], capture_output=True, text=True)
    assert p.returncode == 0, p.stdout + p.stderr
    words = p.stdout.split()
    assert words[words.index("mismatches") + 1] == "0"
    # the fast path is the common one (every random-block and block-maximum case)
    assert int(words[words.index("fast-path") + 1]) > 5_000_000
