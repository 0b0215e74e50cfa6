"""Pins for the oracle's FP4 paged MQA-logits scorer.

The scorer's formula is a reading (the pages name the scorer and its inputs:
ROCm/aiter PR 5484 intro, "API" and "Verification"); what is pinned here is
that the oracle evaluates that formula: against an independent numpy
evaluation over the (already pinned) dequantized tensors, one-hot weights,
ReLU and linearity, the causal mask, untouched entries past the context, and
invalid block-table entries."""
import numpy as np
import pytest

import oracle
from pack_token_amd import workloads


def numpy_logits(sc, weights_scale=1.0, relu=True):
    qd = oracle.dequant_q(sc.q_out, sc.q_scale_out).astype(np.float64)        # [T,H,128]
    kd = oracle.dequant_kcache(sc.kv_cache, sc.kv_cache_scale).astype(np.float64)  # [NB*64,128]
    T = sc.B * sc.next_n
    stride = sc.max_blocks * 64
    out = np.full((T, stride), np.nan)
    for b in range(sc.B):
        ctx = int(sc.context_lens[b])
        s = np.arange(ctx)
        blk = sc.block_table[b, s // 64]
        ok = (blk >= 0) & (blk < sc.NB)
        slots = np.where(ok, blk, 0) * 64 + s % 64
        k = kd[slots]                                     # [ctx,128]
        for j in range(sc.next_n):
            t = b * sc.next_n + j
            sc_h = qd[t] @ k.T                            # [H,ctx]
            if relu:
                sc_h = np.maximum(sc_h, 0.0)
            v = weights_scale * (sc.weights[t].astype(np.float64) @ sc_h)
            pos = ctx - sc.next_n + j
            v[(s > pos) | ~ok] = -np.inf
            out[t, :ctx] = v
    return out


@pytest.mark.parametrize("next_n,H", [(1, 16), (4, 32), (2, 64)])
@pytest.mark.parametrize("relu", [True, False])
def test_scorer_matches_numpy(next_n, H, relu):
    sc = workloads.scorer_case(5 + next_n + H, 3, next_n, H, 1, 200, signed_weights=True)
    got, bound = oracle.paged_mqa_logits(sc.q_out, sc.q_scale_out, sc.weights, sc.kv_cache,
                                         sc.kv_cache_scale, sc.block_table, sc.context_lens,
                                         next_n, weights_scale=0.75, apply_relu=relu,
                                         with_bound=True)
    want = numpy_logits(sc, 0.75, relu)
    fin = np.isfinite(want)
    assert np.array_equal(np.isnan(got), np.isnan(want))          # untouched past the context
    assert np.array_equal(np.isneginf(got), np.isneginf(want))    # masked keys
    err = np.abs(got[fin].astype(np.float64) - want[fin])
    # the oracle rounds once to fp32 at the end
    assert np.all(err <= 2.0 ** -24 * np.abs(want[fin]) + 1e-300)
    assert np.all(bound[fin] >= np.abs(want[fin]) * (1 - 1e-12))


def test_scorer_one_hot_weight_is_relu_of_one_head():
    sc = workloads.scorer_case(9, 2, 1, 32, 64, 130)
    qd = oracle.dequant_q(sc.q_out, sc.q_scale_out).astype(np.float64)
    kd = oracle.dequant_kcache(sc.kv_cache, sc.kv_cache_scale).astype(np.float64)
    for h in (0, 17, 31):
        w = np.zeros_like(sc.weights)
        w[:, h] = 1.0
        got = oracle.paged_mqa_logits(sc.q_out, sc.q_scale_out, w, sc.kv_cache, sc.kv_cache_scale,
                                      sc.block_table, sc.context_lens, 1)
        for b in range(sc.B):
            ctx = int(sc.context_lens[b])
            s = np.arange(ctx)
            slots = sc.block_table[b, s // 64] * 64 + s % 64
            ref = np.maximum(kd[slots] @ qd[b, h], 0.0)
            assert np.array_equal(got[b, :ctx], ref.astype(np.float32))


def test_scorer_masks_and_invalid_blocks():
    sc = workloads.scorer_case(10, 2, 4, 16, 70, 140)
    sc.block_table[1, 0] = sc.NB + 5        # invalid entry: its 64 keys are -inf
    got = oracle.paged_mqa_logits(sc.q_out, sc.q_scale_out, sc.weights, sc.kv_cache,
                                  sc.kv_cache_scale, sc.block_table, sc.context_lens, 4)
    for b in range(2):
        ctx = int(sc.context_lens[b])
        for j in range(4):
            t = b * 4 + j
            pos = ctx - 4 + j
            assert np.isneginf(got[t, pos + 1:ctx]).all()
            assert np.isfinite(got[t, 64 if b == 1 else 0:pos + 1]).all()
            assert np.isnan(got[t, ctx:]).all()
    assert np.isneginf(got[4:8, :64]).all()
    # ReLU makes every visible logit >= 0 with non-negative weights
    fin = np.isfinite(got)
    assert (got[fin] >= 0).all()


# ---- worked cases with hand-derived logits -----------------------------------

import json
import os

WORKED = os.path.join(os.path.dirname(__file__), "golden", "scorer_worked_cases.json")


def worked_case_inputs(doc, case):
    """The fixture's structured description turned into the scorer's byte
    inputs: every 32-group holds one nibble value and one exponent."""
    H, next_n = case["H"], case["next_n"]
    B = len(case["context_lens"])
    T = B * next_n
    J = oracle.q_scale_cols(H)
    q_out = np.zeros((T, H, 64), np.uint8)
    q_scale = np.zeros((T, 1, 4, 16, J), np.uint8)
    for t in range(T):
        for h, groups in enumerate(doc["q_heads"][:H]):
            for g, (n, e) in enumerate(groups):
                q_out[t, h, 16 * g:16 * g + 16] = n | (n << 4)
                q_scale[t, 0, g, h % 16, h // 16] = e
    NB = case["NB"]
    kv = np.zeros((NB, 1, 4, 64, 16), np.uint8)
    ks = np.full((NB, 1, 4, 64), 140, np.uint8)
    for blk, pos, name in case["keys_at"]:
        for g, (n, e) in enumerate(doc["keys"][name]):
            kv[blk, 0, g, pos, :] = n | (n << 4)
            ks[blk, 0, g, (pos % 16) * 4 + pos // 16] = e
    table = np.array(case["block_table"], np.int32)
    ctx = np.array(case["context_lens"], np.int32)
    w = np.array(case["weights"], np.float32)
    return q_out, q_scale, w, kv, ks, table, ctx


def worked_case_expected(case):
    """[T, stride] float32: the listed logits, NaN (untouched) after them."""
    rows = []
    for row in case["expected"]:
        vals = []
        for item in row:
            if isinstance(item, list):
                v = {"-inf": -np.inf, "zeros": 0.0}[item[0]]
                vals += [v] * item[1]
            else:
                vals.append(-np.inf if item == "-inf" else float(item))
        rows.append(vals)
    out = np.full((len(rows), case["stride"]), np.nan, np.float32)
    for t, vals in enumerate(rows):
        out[t, :len(vals)] = vals
    return out


def worked_cases():
    with open(WORKED) as f:
        doc = json.load(f)
    return doc, doc["cases"]


@pytest.mark.parametrize("idx", range(5))
def test_scorer_worked_cases(idx):
    """Hand-derived logits (tests/golden/scorer_worked_cases.json): the ReLU
    before the weighting, the weights and weights_scale, per-head and
    per-group scale bytes, the interleaved key scale row, the causal mask,
    invalid block entries and untouched entries, each with exact values."""
    doc, cases = worked_cases()
    case = cases[idx]
    q_out, q_scale, w, kv, ks, table, ctx = worked_case_inputs(doc, case)
    got = oracle.paged_mqa_logits(q_out, q_scale, w, kv, ks, table, ctx, case["next_n"],
                                  weights_scale=case["weights_scale"], apply_relu=case["relu"],
                                  stride=case["stride"])
    want = worked_case_expected(case)
    assert np.array_equal(np.isnan(got), np.isnan(want)), case["name"]
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32)), case["name"]
