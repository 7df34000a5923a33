"""The unfused PyTorch op chains that bench.py times beside the fused kernel,
run on the GPU on the workloads' own inputs, against the CPU oracle: the
decode layers (1 x 7680 bf16, groups of 960, intermediate cast on and off),
rows of the 8192 x 7680 bf16 prefill, and the norm-first chain on rows of the
16384 x 8192 fp16 Gated-DeltaNet-shaped job with its 128-value head scale.

Bar: the 2-ulp parity bar and at least 99% of outputs equal to the oracle's
bit for bit (a chain with the intermediate cast misplaced or missing equals
it on only about 74%; the reasoning is in test_bench_cpu.py)."""
import numpy as np
import pytest
import torch

import synthetic as S
from gpu_util import BF16, F16, TDT, assert_parity, host_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bench_mod():
    import importlib.util
    import os

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(root, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.fixture(scope="module")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


def _dev(a, dtype, rows, width):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(TDT[dtype])
    return t.reshape(rows, width).cuda()


def _check(got, ref, dtype, what):
    st = assert_parity(host_bits(got, dtype), ref, dtype, what)
    assert st["exact"] >= 0.99, (what, st)
    return st


@pytest.mark.parametrize("ri", [1, 0])
def test_unfused_chain_decode_layers(bench_mod, orc, ri):
    w = S.WORKLOADS["mamba2_decode_1x7680_bf16_g960"]
    for layer in range(S.DECODE_LAYERS):
        y, gt, wt, _ = S.make_inputs(w, layer)
        say(f"case unfused chain decode layer {layer} ri={ri}")
        got = bench_mod.unfused_chain(torch, _dev(y, BF16, 1, w.width), _dev(gt, BF16, 1, w.width),
                                      torch.from_numpy(wt).cuda(), w.group_size, w.eps, ri)
        torch.cuda.synchronize()
        ref = orc.forward(y, gt, wt, rows=1, width=w.width, group_size=w.group_size,
                          y_row_stride=w.width, gate_row_stride=w.width, out_row_stride=w.width,
                          eps=w.eps, dtype=BF16, round_intermediate=ri)
        _check(got, ref, BF16, f"decode layer {layer} ri={ri}")


@pytest.mark.parametrize("ri", [1, 0])
def test_unfused_chain_prefill_rows(bench_mod, orc, ri):
    w = S.WORKLOADS["mamba2_prefill_8192x7680_bf16_g960"]
    idx = np.array([0, 1, 2, 3, 1000, 4095, 4096, 8191] + list(range(7000, 7056)))
    y, gt = S.make_rows(w, idx)
    wt = S.make_weight(w)
    rows = len(idx)
    say(f"case unfused chain prefill rows={rows} ri={ri}")
    got = bench_mod.unfused_chain(torch, _dev(y, BF16, rows, w.width),
                                  _dev(gt, BF16, rows, w.width), torch.from_numpy(wt).cuda(),
                                  w.group_size, w.eps, ri)
    torch.cuda.synchronize()
    ref = orc.forward(y.reshape(-1), gt.reshape(-1), wt, rows=rows, width=w.width,
                      group_size=w.group_size, y_row_stride=w.width, gate_row_stride=w.width,
                      out_row_stride=w.width, eps=w.eps, dtype=BF16, round_intermediate=ri)
    _check(got, ref, BF16, f"prefill rows ri={ri}")


def test_unfused_chain_norm_first_gdn_rows(bench_mod, orc):
    w = S.WORKLOADS["gdn_head_16384x8192_f16_g128"]
    idx = np.array([0, 1, 8191, 16383] + list(range(12000, 12060)))
    y, gt = S.make_rows(w, idx)
    wg = np.ascontiguousarray(S.make_weight(w)[:w.group_size])
    rows = len(idx)
    say(f"case unfused norm-first chain gdn rows={rows}")
    got = bench_mod.unfused_chain_norm_first(torch, _dev(y, F16, rows, w.width),
                                             _dev(gt, F16, rows, w.width),
                                             torch.from_numpy(wg).cuda(), w.group_size, w.eps)
    torch.cuda.synchronize()
    ref = orc.forward(y.reshape(-1), gt.reshape(-1), wg, rows=rows, width=w.width,
                      group_size=w.group_size, y_row_stride=w.width, gate_row_stride=w.width,
                      out_row_stride=w.width, eps=w.eps, dtype=F16, norm_before_gate=True,
                      weight_per_group=True)
    _check(got, ref, F16, "gdn rows norm first")
