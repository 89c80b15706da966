"""Why the bf16 scans use the absorbed form or the T form (CPU): with highly correlated keys
(which the NPU page, section "How it works", says real keys are) and weak decay, rounding
D = T X to bf16 as an operand (the direct form of that page, and the WY form of the Candle
page) loses the cancelling sums of T's alternating columns and misses the 1e-2 bar on the
final state; the absorbed form (W = K^T lambda T and M = A T formed before any rounding) and
the T form (T, lambda Y, A and Y carried as hi/lo bf16 pairs) do not.  The reference is the
fp64 oracle; the rounding points are emulated (tests/rounding_forms.py)."""
import torch

import oracle
from gated_deltanet_scan_amd import synthetic as S
from rounding_forms import max_rel, run


def _errors(key_law, g_law):
    inp = S.make_inputs([1024], 1, 2, 128, 128, torch.bfloat16, seed=1011, g_law=g_law, s0_std=None,
                        key_law=key_law)
    o_ref, s_ref = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"], None)
    errs = {}
    for form in ("direct", "wy", "absorbed", "tform"):
        eo = es = 0.0
        for h in range(2):
            o, st = run(inp["q"][:, 0], inp["k"][:, 0], inp["v"][:, h], inp["g"][:, h], inp["beta"][:, h], form)
            eo, es = max(eo, max_rel(o, o_ref[:, h])), max(es, max_rel(st, s_ref[0, h]))
        errs[form] = (eo, es)
    return errs


def test_correlated_keys_weak_decay_need_the_absorbed_or_t_form():
    e = _errors("correlated", "weak")
    assert e["direct"][1] > 1e-2 and e["wy"][1] > 1e-2, e          # both miss the state bar
    assert e["absorbed"][1] < 5e-3 and e["absorbed"][0] < 1e-2, e   # well inside both bars
    assert e["tform"][1] < 5e-3 and e["tform"][0] < 1e-2, e         # so is the T form


def test_all_forms_agree_on_gaussian_keys():
    e = _errors("gaussian", "uniform")
    for form, (eo, es) in e.items():
        assert eo < 1e-2 and es < 1e-2, (form, e)
