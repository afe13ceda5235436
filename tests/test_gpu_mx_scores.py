"""GPU parity of the prefill's MX score variants (dequant mode 4: MXFP4 keys,
mode 5: MXFP8 keys; MXFP8 queries, S^T = K Q^T on gfx950's scaled f8f6f4
matrix instruction).

Two checks per case, on the same seeded inputs:
* against the fp64 emulation of the recipe (tests/mx_emulation.py: the
  attention over the requantized operands) within the exact path's
  1e-2 + 1e-2 |ref|: the kernel computes what the recipe says (operand layout,
  pairing of NVFP4 blocks into MX blocks, exponents, rounding);
* against the fp64 oracle within the mode's contract (MX_CONTRACT[mode]: per
  element and over the batch), derived on the CPU in
  test_mx_variant_accuracy.py.
"""
import numpy as np
import pytest
import torch

import mx_emulation as M
import workloads as W
from gpu_helpers import assert_close, banner, oracle_outputs, run_gpu

pytestmark = pytest.mark.gpu

Q_LENS = [1, 37, 200, 64, 3, 129]
KV_LENS = [1, 37, 333, 700, 3, 130]


@pytest.fixture(scope="module")
def K():
    import nvfp4_paged_kv_amd as K
    K.lib()
    return K


def _mx_plan(K, w, mode, split_len=-1):
    return K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads, w.num_kv_heads,
                  w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr), split_len=split_len,
                  tile_waves=4, dequant_mode=mode)


def _check(K, O, w, plan, mode):
    out, _, _ = run_gpu(K, w, plan=plan)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    emu, rows = M.mx_outputs(O, w, mode=mode)
    got = out.index_select(0, torch.from_numpy(rows).cuda())
    e_emu = assert_close(got, emu, w.name + " vs MX emulation")
    ref, _ = oracle_outputs(O, w)
    g = got.float().cpu().double().numpy()
    err = np.abs(g - ref)
    elem = float((err / (1 + np.abs(ref))).max())
    rms = float(np.sqrt((err ** 2).mean() / (ref ** 2).mean()))
    elem_max, rms_max = M.MX_CONTRACT[mode]
    print(f"mode {mode}: max err vs emulation {e_emu:.3g}; vs oracle: elem {elem:.3f} (<= {elem_max}), "
          f"rms {rms:.4f} (<= {rms_max})", flush=True)
    assert elem <= elem_max and rms <= rms_max, (elem, rms)
    return out


MODES = [4, 5]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("split_len", [-1, 2])
@pytest.mark.parametrize("scales", ["amax", "lognormal"])
def test_mx_scores_ragged(K, oracle, split_len, scales, mode):
    banner(f"MX scores mode {mode}, ragged batch, {scales} scales, split_len {split_len}")
    kw = dict(scales="amax") if scales == "amax" else dict(scales="lognormal", lognormal=(-3.0, 0.5))
    w = W.make_attention(f"mx_ragged_{scales}", Q_LENS, KV_LENS, 32, 8, 128, 16, 120, seed=31, device="cuda", **kw)
    plan = _mx_plan(K, w, mode, split_len)
    if split_len > 0:
        assert plan.num_split_tiles > 0
    _check(K, oracle, w, plan, mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("page_size", [32, 64])
def test_mx_scores_page_sizes(K, oracle, page_size, mode):
    banner(f"MX scores mode {mode}, page size {page_size}")
    pool = sum((k + page_size - 1) // page_size for k in KV_LENS) + 4
    w = W.make_attention(f"mx_ps{page_size}", Q_LENS, KV_LENS, 32, 8, 128, page_size, pool, seed=32,
                         device="cuda", scales="amax")
    _check(K, oracle, w, _mx_plan(K, w, mode), mode)


@pytest.mark.parametrize("mode", MODES)
def test_mx_scores_2k(K, oracle, mode):
    """The 2048x2048 batch the ablation times, every output row."""
    banner(f"MX scores mode {mode}, 2048x2048")
    w = W.prefill_2k("cuda")
    _check(K, oracle, w, _mx_plan(K, w, mode), mode)


@pytest.mark.parametrize("mode", MODES)
def test_mx_scores_repeatable_and_exact_path_unchanged(K, mode):
    """An MX mode gives the same bits on every run, and the exact path's
    output on the same cache is the one it gives without it having run."""
    banner(f"MX scores mode {mode}, repeatability")
    w = W.make_attention("mx_repeat", Q_LENS, KV_LENS, 32, 8, 128, 16, 120, seed=33, device="cuda", scales="amax")
    exact_plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), 32, 8, 128, 16,
                        kv_indptr=torch.from_numpy(w.kv_indptr), tile_waves=4)
    base, cache, _ = run_gpu(K, w, plan=exact_plan)
    plan = _mx_plan(K, w, mode)
    first, _, _ = run_gpu(K, w, cache=cache, plan=plan)
    again, _, _ = run_gpu(K, w, cache=cache, plan=plan)
    after, _, _ = run_gpu(K, w, cache=cache, plan=exact_plan)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), again.view(torch.int16))
    assert torch.equal(after.view(torch.int16), base.view(torch.int16))
    assert not torch.equal(first.view(torch.int16), base.view(torch.int16))
