"""GPU: the library is safe to call from several host threads at once.

Eight threads, each with its own stream (default priority) and its own jobs
-- different dtypes, group sizes, operators and kernel families -- call
ggrms_forward_ex concurrently through ctypes (which releases the interpreter
lock around the call).  The kernels are deterministic, so every output must
equal, bit for bit, the output of the same call made alone beforehand, which
is itself checked against the oracle.
"""
import threading

import numpy as np
import pytest
import torch

from gpu_util import (BF16, F16, F32, FLAG_NBG, FLAG_PER_GROUP, FLAG_RI, assert_parity, dev_buf,
                      host_bits, random_case, say)

pytestmark = pytest.mark.gpu

# (dtype, G, groups, rows, flags)
JOBS = [
    (BF16, 960, 8, 64, FLAG_RI),           # BLOCK, 4 rows per workgroup
    (F16, 128, 64, 48, FLAG_RI),           # WAVE, 16 lanes
    (F32, 64, 4, 100, 0),                  # WAVE, f32
    (BF16, 5120, 1, 24, FLAG_RI),          # BLOCK 256 x 3
    (F16, 128, 16, 40, FLAG_NBG | FLAG_PER_GROUP),  # norm first, shared weight
    (F16, 100, 48, 32, FLAG_RI),           # packed groups
    (BF16, 40960, 1, 3, FLAG_RI),          # two-pass
    (BF16, 8, 100, 30, 0),                 # one lane per group
]


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_group_rmsnorm_amd as g  # raises if libggrms.so is missing

    return g


@pytest.fixture(scope="module")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


def test_concurrent_calls_from_threads(g, orc):
    prepared = []
    for k, (dtype, G, groups, rows, flags) in enumerate(JOBS):
        width = G * groups
        y, gt, w = random_case(rows, width, dtype, seed=900 + k)
        if flags & FLAG_PER_GROUP:
            w = np.ascontiguousarray(w[:G])
        yd, gd, wd = dev_buf(y, dtype), dev_buf(gt, dtype), torch.from_numpy(w).cuda()
        args = (rows, width, G, width, width, width, 1e-5, dtype, flags)
        od = torch.empty_like(yd)
        st = g.ggrms_forward_ex(yd.data_ptr(), gd.data_ptr(), wd.data_ptr(), od.data_ptr(), *args,
                                torch.cuda.current_stream().cuda_stream)
        assert st == g.SUCCESS, g.ggrms_status_string(st)
        torch.cuda.synchronize()
        alone = host_bits(od, dtype)
        ref = orc.forward(y, gt, w, rows=rows, width=width, group_size=G, y_row_stride=width,
                          gate_row_stride=width, out_row_stride=width, eps=1e-5, dtype=dtype,
                          round_intermediate=flags & FLAG_RI,
                          norm_before_gate=bool(flags & FLAG_NBG),
                          weight_per_group=bool(flags & FLAG_PER_GROUP))
        assert_parity(alone, ref, dtype, f"job {k} alone")
        prepared.append((yd, gd, wd, args, dtype, alone))

    n_threads, calls = 8, 25
    failures = []
    barrier = threading.Barrier(n_threads)

    def worker(t):
        try:
            stream = torch.cuda.Stream()  # default priority
            outs = [torch.empty_like(p[0]) for p in prepared]
            used = set()
            barrier.wait()
            for c in range(calls):
                k = (t + c) % len(prepared)
                used.add(k)
                yd, gd, wd, args, dtype, alone = prepared[k]
                st = g.ggrms_forward_ex(yd.data_ptr(), gd.data_ptr(), wd.data_ptr(),
                                        outs[k].data_ptr(), *args, stream.cuda_stream)
                if st != g.SUCCESS:
                    failures.append(f"thread {t} call {c}: status {st}")
                    return
                if c % 5 == 4:
                    stream.synchronize()
                    got = host_bits(outs[k], dtype)
                    if not np.array_equal(got.view(np.uint8), alone.view(np.uint8)):
                        failures.append(f"thread {t} call {c}: job {k} differs from the lone call")
            stream.synchronize()
            for k in sorted(used):  # the last call of every job this thread ran
                got = host_bits(outs[k], prepared[k][4])
                if not np.array_equal(got.view(np.uint8), prepared[k][5].view(np.uint8)):
                    failures.append(f"thread {t}: job {k} differs from the lone call at the end")
        except Exception as e:  # reported below; a thread must not die silently
            failures.append(f"thread {t}: {e!r}")

    say(f"case threads {n_threads} x {calls} calls over {len(prepared)} jobs")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
        assert not th.is_alive(), "a calling thread did not finish"
    torch.cuda.synchronize()
    assert not failures, failures[:5]
