"""GPU parity of the FP4 paged MQA-logits scorer (scaled-FP4 MFMA) against
the oracle.  The scorer accumulates in fp32 on the matrix cores, so parity is
a tolerance: every finite logit within (K + H + 8) * 2^-24 of the oracle's
error scale |weights_scale| * sum_h |w| * sum_d |q_d k_d| (a forward error
bound of fp32 summation over the 128 products and the H heads), cosine >=
0.9999 over all finite logits, and -inf / untouched entries identical."""
import numpy as np
import pytest

import oracle
from pack_token_amd import workloads
from harness import say

pytestmark = pytest.mark.gpu

SENT = np.float32(-12345.0)


def run_gpu_scorer(sc, weights_scale=1.0, relu=True, stride=None):
    import torch

    from pack_token_amd import fp4idx

    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    stride = stride or sc.max_blocks * 64
    logits = torch.full((sc.B * sc.next_n, stride), float(SENT), dtype=torch.float32, device=dev)
    fp4idx.paged_mqa_logits(t(sc.q_out), t(sc.q_scale_out), t(sc.weights), t(sc.kv_cache),
                            t(sc.kv_cache_scale), t(sc.block_table), t(sc.context_lens),
                            sc.next_n, weights_scale=weights_scale, apply_relu=relu, logits=logits)
    torch.cuda.synchronize()
    return logits.cpu().numpy()


def check_scorer(got, ref, bound, H):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    assert np.array_equal(got == SENT, np.isnan(ref))            # untouched past the context
    g, r = got[fin].astype(np.float64), ref[fin].astype(np.float64)
    tol = (128 + H + 8) * 2.0 ** -24 * bound[fin] + 1e-37
    bad = np.abs(g - r) > tol
    assert not bad.any(), (int(bad.sum()), float(np.max(np.abs(g - r) / np.maximum(tol, 1e-300))))
    if g.size:
        cos = float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r) + 1e-300))
        assert cos >= 0.9999, cos
    return fin


@pytest.mark.parametrize("next_n", [1, 2, 3, 4])
@pytest.mark.parametrize("H", [16, 32, 48, 64])
@pytest.mark.parametrize("relu", [True, False])
def test_scorer_random_bytes(next_n, H, relu):
    sc = workloads.scorer_case(100 * next_n + H, 5, next_n, H, 1, 700, signed_weights=not relu)
    say(f"case scorer next_n={next_n} H={H} relu={relu} ctx={list(sc.context_lens)}")
    got = run_gpu_scorer(sc, 0.5, relu)
    ref, bound = oracle.paged_mqa_logits(sc.q_out, sc.q_scale_out, sc.weights, sc.kv_cache,
                                         sc.kv_cache_scale, sc.block_table, sc.context_lens,
                                         next_n, weights_scale=0.5, apply_relu=relu,
                                         with_bound=True)
    check_scorer(got, ref, bound, H)


def test_scorer_edge_cases():
    """Contexts shorter than next_n, exactly one block, ragged tails, longer than
    the table (clamped), invalid block entries, and a stride wider than the table."""
    sc = workloads.scorer_case(7, 6, 4, 32, 1, 200, spare_blocks=3)
    sc.context_lens[:] = [0, 2, 64, 65, 191, 10_000]   # last one is clamped to max_blocks*64
    sc.block_table[4, 1] = -7
    sc.block_table[3, 1] = sc.NB
    stride = sc.max_blocks * 64 + 37
    got = run_gpu_scorer(sc, 1.0, True, stride)
    ref, bound = oracle.paged_mqa_logits(sc.q_out, sc.q_scale_out, sc.weights, sc.kv_cache,
                                         sc.kv_cache_scale, sc.block_table, sc.context_lens, 4,
                                         stride=stride, with_bound=True)
    check_scorer(got, ref, bound, 32)


@pytest.mark.parametrize("next_n", [1, 4])
def test_producer_to_scorer_end_to_end(next_n):
    """The producer's own bytes fed to the scorer at H=32, D=128, kv_block=64 with
    next_n 1 and 4 (the shapes of ROCm/aiter PR 5484 "Verification", which reports
    cosine 1.000000 and top-64 overlap 1.00 against its reference): GPU producer +
    GPU scorer against oracle producer + oracle scorer."""
    import torch

    from pack_token_amd import fp4idx
    from harness import gpu_run, oracle_run, assert_all_same

    B, H = 16, 32
    ctx = np.random.default_rng(3).integers(300, 1500, B).astype(np.int32)
    n_keys = int(ctx.sum())
    rng = np.random.Generator(np.random.PCG64(77 + next_n))
    # one producer call writes the keys of all sequences (contiguous slots) and the
    # queries of the last next_n positions of every sequence
    T = B * next_n
    wl = workloads.sweep_case(55 + next_n, T, H, True, 64)
    keys = workloads.sweep_case(66 + next_n, n_keys, 16, True, 64)
    starts = np.concatenate([[0], np.cumsum(ctx)[:-1]])
    NB = -(-n_keys // 64) + B
    # each sequence starts on a fresh block
    blk_starts = np.concatenate([[0], np.cumsum(-(-ctx // 64))[:-1]])
    slots = np.concatenate([blk_starts[b] * 64 + np.arange(ctx[b]) for b in range(B)])
    keys.slot_mapping = slots.astype(np.int64)
    keys.positions = np.concatenate([np.arange(c) for c in ctx]).astype(np.int64)
    keys.cos_sin = workloads.cos_sin_table(int(ctx.max()))
    keys.NB = NB
    wl.positions = np.concatenate([np.arange(c - next_n, c) for c in ctx]).astype(np.int64)
    wl.cos_sin = keys.cos_sin
    wl.NB = NB
    max_blocks = int(-(-ctx.max() // 64))
    table = np.full((B, max_blocks), -1, np.int32)
    for b in range(B):
        nb = -(-int(ctx[b]) // 64)
        table[b, :nb] = blk_starts[b] + np.arange(nb)
    say(f"case e2e next_n={next_n}: {B} sequences, {n_keys} keys")
    gq = gpu_run(wl)                         # queries (the cache part is ignored)
    gk = gpu_run(keys)                       # keys into the cache
    rq = oracle_run(wl)
    rk = oracle_run(keys)
    assert_all_same(gq[:3] + (None, None), rq[:3] + (None, None))
    assert_all_same((None, None, None) + gk[3:], (None, None, None) + rk[3:])
    sc = workloads.ScorerCase("e2e", B, next_n, H, gq[0], gq[1], wl.weights, gk[3], gk[4], table, ctx)
    got = run_gpu_scorer(sc)
    ref, bound = oracle.paged_mqa_logits(rq[0], rq[1], wl.weights, rk[3], rk[4], table, ctx,
                                         next_n, with_bound=True)
    fin = check_scorer(got, ref, bound, H)
    # top-64 overlap per query row
    overlaps = []
    for t in range(T):
        f = np.isfinite(ref[t])
        if f.sum() < 64:
            continue
        a = set(np.argsort(-np.where(f, got[t], -np.inf))[:64])
        b = set(np.argsort(-np.where(f, ref[t], -np.inf))[:64])
        overlaps.append(len(a & b) / 64)
    say(f"top-64 overlap mean {np.mean(overlaps):.4f} min {np.min(overlaps):.4f}")
    assert np.mean(overlaps) >= 0.99
    # Against bf16 ground truth: the same scores evaluated in float64 on the
    # rotated bf16 queries and keys before any quantization.  The pages report
    # cosine 0.980 for this pipeline against independent bf16 ground truth
    # (ROCm/aiter PR 5484, "Verification"); the bar is 0.97.
    from pack_token_amd.workloads import bf16_bits_to_f32
    qr = oracle.rope_rows(bf16_bits_to_f32(wl.q).reshape(-1, 128),
                          np.repeat(wl.cos_sin[wl.positions], H, 0)).reshape(T, H, 128)
    kr = oracle.rope_rows(bf16_bits_to_f32(keys.k), keys.cos_sin[keys.positions])
    qr, kr = qr.astype(np.float64), kr.astype(np.float64)
    gt = np.full_like(ref, np.nan, dtype=np.float64)
    for b in range(B):
        kb = kr[starts[b]:starts[b] + ctx[b]]                       # [ctx, 128]
        for j in range(next_n):
            t = b * next_n + j
            pos = int(ctx[b]) - next_n + j
            dots = np.maximum(qr[t] @ kb[:pos + 1].T, 0.0)          # [H, pos + 1]
            gt[t, :pos + 1] = wl.weights[t].astype(np.float64) @ dots
    vis = np.isfinite(gt)
    assert np.array_equal(vis, np.isfinite(ref))
    g, r, x = got[vis].astype(np.float64), ref[vis].astype(np.float64), gt[vis]
    cos_gpu = float(g @ x / (np.linalg.norm(g) * np.linalg.norm(x)))
    cos_ref = float(r @ x / (np.linalg.norm(r) * np.linalg.norm(x)))
    say(f"cosine vs bf16 ground truth: GPU {cos_gpu:.5f}, oracle {cos_ref:.5f} (pages: 0.980)")
    assert cos_gpu >= 0.97


@pytest.mark.parametrize("next_n,H,relu", [(5, 32, True), (8, 64, False), (67, 32, True),
                                           (130, 16, True), (21, 48, False)])
def test_scorer_prefill_tiles(next_n, H, relu):
    """next_n above 4 (chunked prefill): query tiles of 4 with a ragged last
    tile, contexts shorter than, equal to and longer than next_n (queries at
    negative positions see only -inf), whole key blocks after a tile's last
    query (written -inf without being read) and invalid block entries."""
    sc = workloads.scorer_case(900 + next_n + H, 4, next_n, H, 1, 700, signed_weights=not relu)
    sc.context_lens[0] = max(1, next_n - 3)
    sc.context_lens[1] = next_n
    nb1 = -(-int(sc.context_lens[2]) // 64)
    if nb1 > 1:
        sc.block_table[2, nb1 // 2] = -1
    say(f"case scorer prefill next_n={next_n} H={H} relu={relu} ctx={list(sc.context_lens)}")
    got = run_gpu_scorer(sc, 0.75, relu)
    ref, bound = oracle.paged_mqa_logits(sc.q_out, sc.q_scale_out, sc.weights, sc.kv_cache,
                                         sc.kv_cache_scale, sc.block_table, sc.context_lens,
                                         next_n, weights_scale=0.75, apply_relu=relu,
                                         with_bound=True)
    check_scorer(got, ref, bound, H)


@pytest.mark.parametrize("next_n,H", [(1, 32), (4, 32), (3, 48), (67, 32), (130, 64), (9, 16)])
def test_scorer_sparse_invalid_blocks(next_n, H):
    """Block tables where about a third of the entries are invalid (negative or
    past the cache), so that an invalid block falls at every place of a
    wavefront's window of 4 (decode) or 8 (query tiles) blocks: first, last,
    several in a row, and whole windows.  The scorer fetches each block one
    ahead while it scores the previous one; an invalid block is never fetched
    and its keys are -inf.  Contexts run from one block to 40 blocks with
    ragged tails."""
    sc = workloads.scorer_case(4100 + 7 * next_n + H, 6, next_n, H, 1, 40 * 64 - 5)
    rng = np.random.default_rng(next_n * 131 + H)
    bad = rng.random(sc.block_table.shape) < 0.35
    bad[0, :8] = True                       # a whole window of the first sequence
    bad[1, ::4] = True                      # first block of every decode window
    bad[2, 7::8] = True                     # last block of every tiled window
    vals = np.where(rng.random(sc.block_table.shape) < 0.5, -1, sc.NB + 3).astype(np.int32)
    sc.block_table[bad] = vals[bad]
    say(f"case scorer sparse next_n={next_n} H={H} ctx={list(sc.context_lens)} "
        f"invalid={int(bad.sum())}")
    got = run_gpu_scorer(sc, 1.25, True)
    ref, bound = oracle.paged_mqa_logits(sc.q_out, sc.q_scale_out, sc.weights, sc.kv_cache,
                                         sc.kv_cache_scale, sc.block_table, sc.context_lens,
                                         next_n, weights_scale=1.25, apply_relu=True,
                                         with_bound=True)
    check_scorer(got, ref, bound, H)
    assert np.isneginf(ref).any() and np.isfinite(ref).any()


def _check_row_pattern(row, pos, ctx):
    """A logit row of a query at position pos of a context of ctx keys: finite up
    to pos, -inf after it inside the context, untouched past it."""
    assert np.isfinite(row[:max(pos + 1, 0)]).all()
    assert np.isneginf(row[max(pos + 1, 0):ctx]).all()
    assert (row[ctx:] == SENT).all()


def test_scorer_decode_full_size_sampled():
    """The decode-scoring batch at full size, in the launch the benchmark times
    (64 sequences x next_n 4, H = 32, contexts U[4096, 131072], 4.6 M keys):
    two whole sequences against the oracle, the -inf / untouched pattern of
    every row."""
    B, next_n, H = 64, 4, 32
    sc = workloads.scorer_case(7, B, next_n, H, 4096, 131072)
    say(f"case scorer decode full size: {int(sc.context_lens.sum())} keys")
    got = run_gpu_scorer(sc)
    for b in range(B):
        for j in range(next_n):
            ctx = int(sc.context_lens[b])
            _check_row_pattern(got[b * next_n + j], ctx - next_n + j, ctx)
    for b in (int(np.argmax(sc.context_lens)), 5):
        rows = slice(b * next_n, (b + 1) * next_n)
        ref, bound = oracle.paged_mqa_logits(sc.q_out[rows], sc.q_scale_out[rows],
                                             sc.weights[rows], sc.kv_cache, sc.kv_cache_scale,
                                             sc.block_table[b:b + 1], sc.context_lens[b:b + 1],
                                             next_n, with_bound=True)
        check_scorer(got[rows], ref, bound, H)


@pytest.mark.parametrize("B,next_n,H", [(1024, 1, 16), (1025, 2, 32), (700, 4, 64), (1024, 7, 32),
                                         (1030, 6, 16), (300, 9, 48)])
def test_scorer_many_sequences(B, next_n, H):
    """Batches at the flat scorer's sequence limit (1,024: the per-sequence item
    counts are scanned in 16 chunks of 64) and past it (1,025 and 1,030: the
    grid kernels), decode and query tiles (next_n 6, 7, 9 with a short last
    tile), with contexts of 0 to 300 keys, so that many wavefronts cross one or
    more sequence and tile boundaries."""
    sc = workloads.scorer_case(5000 + B + next_n, B, next_n, H, 0, 300)
    rng = np.random.default_rng(B)
    bad = rng.random(sc.block_table.shape) < 0.1
    sc.block_table[bad] = -1
    say(f"case scorer many sequences B={B} next_n={next_n} H={H}")
    got = run_gpu_scorer(sc, 0.5, True)
    ref, bound = oracle.paged_mqa_logits(sc.q_out, sc.q_scale_out, sc.weights, sc.kv_cache,
                                         sc.kv_cache_scale, sc.block_table, sc.context_lens,
                                         next_n, weights_scale=0.5, with_bound=True)
    check_scorer(got, ref, bound, H)


def test_scorer_decode_long_ranges():
    """100 sequences of 131,072 keys (204,800 blocks, 891 MB of cache) with
    next_n = 1, H = 16: more blocks than 64 per wavefront of the resident grid,
    so every wavefront walks several windows of block-table entries; the row
    pattern of every query and three whole sequences against the oracle."""
    B, next_n, H = 100, 1, 16
    sc = workloads.scorer_case(8, B, next_n, H, 131072, 131072)
    say(f"case scorer long ranges: {int(sc.context_lens.sum())} keys")
    got = run_gpu_scorer(sc)
    for b in range(B):
        ctx = int(sc.context_lens[b])
        _check_row_pattern(got[b], ctx - 1, ctx)
    for b in (0, 37, B - 1):
        rows = slice(b, b + 1)
        ref, bound = oracle.paged_mqa_logits(sc.q_out[rows], sc.q_scale_out[rows],
                                             sc.weights[rows], sc.kv_cache, sc.kv_cache_scale,
                                             sc.block_table[b:b + 1], sc.context_lens[b:b + 1],
                                             next_n, with_bound=True)
        check_scorer(got[rows], ref, bound, H)


def test_scorer_prefill_full_size_sampled():
    """The chunked-prefill scoring case at full size, in the launch the benchmark
    times (one sequence of 65,536 keys, its last 4,096 tokens as queries, H = 64,
    query tiles of 2, 8 blocks per wavefront): the row pattern of every query,
    and three groups of 4 queries (the first, a middle and the last) against
    the oracle, each as a 4-query case whose context ends 4 keys after its
    queries' positions, i.e. at exactly the positions of the full run."""
    B, next_n, H, ctx_len = 1, 4096, 64, 65536
    sc = workloads.scorer_case(11, B, next_n, H, ctx_len, ctx_len)
    say("case scorer prefill full size: 4096 x 65536, H = 64")
    got = run_gpu_scorer(sc)
    for j in range(next_n):
        _check_row_pattern(got[j], ctx_len - next_n + j, ctx_len)
    for r0 in (0, 2050, next_n - 4):
        ctx_sub = ctx_len - next_n + r0 + 4
        rows = slice(r0, r0 + 4)
        ref, bound = oracle.paged_mqa_logits(sc.q_out[rows], sc.q_scale_out[rows],
                                             sc.weights[rows], sc.kv_cache, sc.kv_cache_scale,
                                             sc.block_table, np.array([ctx_sub], np.int32), 4,
                                             with_bound=True)
        check_scorer(got[rows, :ctx_sub], ref[:, :ctx_sub], bound[:, :ctx_sub], H)


@pytest.mark.parametrize("idx", range(5))
def test_scorer_worked_cases(idx):
    """The hand-derived worked cases of tests/golden/scorer_worked_cases.json on
    the GPU scorer: every value is a small integer that the matrix cores and
    the fp32 epilogue produce exactly, so the logits must equal the fixture's
    bit for bit (ReLU before the weighting, weights and weights_scale, head and
    group scale bytes, the interleaved key scales, causal mask, invalid
    blocks, untouched entries)."""
    from test_oracle_scorer import worked_case_expected, worked_case_inputs, worked_cases
    from pack_token_amd.workloads import ScorerCase

    doc, cases = worked_cases()
    case = cases[idx]
    q_out, q_scale, w, kv, ks, table, ctx = worked_case_inputs(doc, case)
    sc = ScorerCase(case["name"], len(ctx), case["next_n"], case["H"], q_out, q_scale, w, kv, ks,
                    table, ctx)
    say(f"case scorer worked {case['name']}")
    got = run_gpu_scorer(sc, case["weights_scale"], case["relu"], case["stride"])
    want = worked_case_expected(case)
    untouched = np.isnan(want)
    assert (got[untouched] == SENT).all(), case["name"]
    assert np.array_equal(got[~untouched].view(np.uint32), want[~untouched].view(np.uint32)), \
        case["name"]


def test_scorer_logits_past_32_bit_offsets():
    """Chunked prefill whose logits tensor holds more than 2^32 bytes (20,000
    queries x 131,072 keys, 10.5 GB): rows near the end are addressed past
    every 32-bit offset.  On the device, the -inf count is exactly the causal
    triangle and no entry is left untouched; four groups of queries (the first,
    two in the middle, the last) against the oracle, each as a case whose
    context ends right after its queries, as in the full run."""
    import torch

    from pack_token_amd import fp4idx

    B, next_n, H, ctx_len = 1, 20000, 16, 131072
    sc = workloads.scorer_case(13, B, next_n, H, ctx_len, ctx_len)
    say("case scorer logits past 32-bit offsets: 20000 x 131072, H = 16")
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    logits = torch.full((next_n, ctx_len), float(SENT), dtype=torch.float32, device=dev)
    assert logits.numel() * 4 > 2 ** 32
    fp4idx.paged_mqa_logits(t(sc.q_out), t(sc.q_scale_out), t(sc.weights), t(sc.kv_cache),
                            t(sc.kv_cache_scale), t(sc.block_table), t(sc.context_lens),
                            next_n, logits=logits)
    torch.cuda.synchronize()
    n_inf = int(torch.isneginf(logits).sum().item())
    n_sent = int((logits == float(SENT)).sum().item())
    n_fin = int(torch.isfinite(logits).sum().item())
    assert n_inf == next_n * (next_n - 1) // 2
    assert n_sent == 0
    assert n_fin + n_inf == logits.numel()
    for r0 in (0, 9998, 12001, next_n - 4):
        got = logits[r0:r0 + 4].cpu().numpy()
        for j in range(4):
            _check_row_pattern(got[j], ctx_len - next_n + r0 + j, ctx_len)
        ctx_sub = ctx_len - next_n + r0 + 4
        rows = slice(r0, r0 + 4)
        ref, bound = oracle.paged_mqa_logits(sc.q_out[rows], sc.q_scale_out[rows],
                                             sc.weights[rows], sc.kv_cache, sc.kv_cache_scale,
                                             sc.block_table, np.array([ctx_sub], np.int32), 4,
                                             with_bound=True)
        check_scorer(got[:, :ctx_sub], ref[:, :ctx_sub], bound[:, :ctx_sub], H)
    del logits
    torch.cuda.empty_cache()
