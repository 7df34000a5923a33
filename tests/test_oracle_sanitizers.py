"""The oracle (plain C) built with AddressSanitizer and UndefinedBehaviorSanitizer
and driven over a sweep of shapes, strides, dtypes, operator flags and special
values, with every buffer allocated at exactly the size the call may touch, so
that any read or write outside a view, any signed overflow or shift out of
range, and any misaligned access stops the run.  CPU only."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "ggrms_oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {  /* xorshift64*: a test input stream, nothing more */
    state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
    return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float pick(int special) {
    const float sp[] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN, 1e-40f, -1e-40f, 65504.0f,
                        -90.0f, 100.0f, 3e38f, -3e38f};
    if (special && next32() % 5 == 0) return sp[next32() % (sizeof sp / sizeof sp[0])];
    return ((float)(next32() % 20001) - 10000.0f) / 2500.0f;
}
/* exact-size heap copies: the sanitizer reports any access past either end */
static void* dup_bytes(const void* src, size_t n) {
    void* p = malloc(n ? n : 1);
    memcpy(p, src, n);
    return p;
}

int main(void) {
    const int64_t Gs[] = {1, 2, 3, 7, 8, 63, 64, 65, 100, 128, 960};
    long calls = 0, rejected = 0;
    for (size_t gi = 0; gi < sizeof Gs / sizeof Gs[0]; ++gi)
    for (int groups = 1; groups <= 3; ++groups)
    for (int64_t rows = 0; rows <= 3; ++rows)
    for (int dt = 0; dt < 3; ++dt)
    for (int pad = 0; pad < 2; ++pad)
    for (int flags = 0; flags < 8; ++flags) {
        const int64_t G = Gs[gi], width = G * groups;
        const int64_t sy = width + 3 * pad, sg = width + 5 * pad, so = width + pad;
        const size_t es = dt == 0 ? 4 : 2;
        const int64_t ny = rows ? (rows - 1) * sy + width : 0;
        const int64_t ng = rows ? (rows - 1) * sg + width : 0;
        const int64_t no = rows ? (rows - 1) * so + width : 0;
        const int64_t nw = (flags & 4) ? G : width;
        float* tmp = malloc(sizeof(float) * (size_t)(ny + ng + nw + 1));
        for (int64_t i = 0; i < ny + ng + nw; ++i) tmp[i] = pick(1);
        uint16_t* h = malloc(2 * (size_t)(ny + ng + 1));
        void *y, *gate;
        if (dt == 0) {
            y = dup_bytes(tmp, 4 * (size_t)ny);
            gate = dup_bytes(tmp + ny, 4 * (size_t)ng);
        } else {
            ggrms_oracle_round_array(tmp, h, ny + ng, dt);
            y = dup_bytes(h, 2 * (size_t)ny);
            gate = dup_bytes(h + ny, 2 * (size_t)ng);
        }
        float* w = dup_bytes(tmp + ny + ng, 4 * (size_t)nw);
        void* out = malloc(es * (size_t)no + (no ? 0 : 1));
        float* scratch = malloc(sizeof(float) * (size_t)G);
        const float eps = (flags & 1) ? 1e-5f : 0.0f;
        const int rc = ggrms_oracle_forward_ex(y, gate, w, out, rows, width, G, sy, sg, so, eps,
                                               dt, flags, scratch);
        ++calls;
        rejected += rc != 0;
        if (rc == 0 && (flags & 4) == 0 && (flags & 2) == 0) {
            ggrms_oracle_forward(y, gate, w, out, rows, width, G, sy, sg, so, eps, dt,
                                 flags & 1, scratch);
            ++calls;
        }
        free(y); free(gate); free(w); free(out); free(scratch); free(tmp); free(h);
    }
    /* the element-wise helpers over every f32 exponent */
    for (int dt = 1; dt < 3; ++dt) {
        uint16_t* o = malloc(2 * 4096);
        for (uint32_t hi = 0; hi < 512; ++hi)
            ggrms_oracle_round_bits_range(hi << 23 | (next32() & 0x7FF000u), 4096, o, dt);
        float* f = malloc(4 * 4096);
        for (int i = 0; i < 4096; ++i) o[i] = (uint16_t)(i * 16 + (i & 15));
        ggrms_oracle_widen_array(o, f, 4096, dt);
        ggrms_oracle_silu_array(f, f, 4096);
        free(o); free(f);
    }
    printf("%ld %ld\n", calls, rejected);
    return calls > 0 ? 0 : 1;
}
"""


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    drv = tmp_path / "oracle_sweep.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "oracle_sweep"
    odir = os.path.join(ROOT, "oracle")
    # the oracle's own arithmetic flags (strict IEEE f32) plus the sanitizers
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-I", odir, str(drv),
                    os.path.join(odir, "ggrms_oracle.c"), "-lm", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    calls, rejected = map(int, r.stdout.split())
    # the norm-first operator refuses the intermediate cast: flags 3 and 7 are rejected
    assert calls > 2000 and 0 < rejected < calls // 3, r.stdout
