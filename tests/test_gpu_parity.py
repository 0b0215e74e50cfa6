"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, byte
for byte on all five outputs, on the five workloads and a sweep of shapes and
modes (tokens x heads x is_neox x rotated slice, mirroring the 16-config
matrix of ROCm/aiter PR 5484 "Verification")."""
import numpy as np
import pytest

import oracle
from pack_token_amd import workloads
from pack_token_amd.workloads import SENTINEL
from harness import (assert_all_same, assert_same, gpu_run, large_prefill, oracle_run,
                     random_case, say)

pytestmark = pytest.mark.gpu


def check(wl, **kw):
    say(f"case {wl.name}: T={wl.T} H={wl.H} neox={wl.is_neox} ro={wl.rope_offset} "
        f"had={wl.apply_hadamard} norm={wl.k_norm_gamma is not None} fused={kw.get('fused')}")
    got = gpu_run(wl, **kw)
    ref = oracle_run(wl, with_weights=kw.get("with_weights", True))
    assert_all_same(got, ref)
    return got


FUSED = pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])


@FUSED
def test_tiny(fused):
    check(workloads.tiny(), fused=fused)


@FUSED
@pytest.mark.parametrize("pos32", [False, True])
@pytest.mark.parametrize("T", [300, 700])
def test_edge_mix(T, pos32, fused):
    check(workloads.edge_mix(T=T, positions_int32=pos32), fused=fused)


@FUSED
@pytest.mark.parametrize("T", [8, 32])
@pytest.mark.parametrize("H", [32, 64])
@pytest.mark.parametrize("is_neox", [True, False])
@pytest.mark.parametrize("rope_offset", [0, 64])
def test_sweep(T, H, is_neox, rope_offset, fused):
    check(workloads.sweep_case(100 + T + H, T, H, is_neox, rope_offset), fused=fused)


@FUSED
@pytest.mark.parametrize("is_neox", [True, False])
@pytest.mark.parametrize("rope_offset", [0, 64])
@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("had", [False, True])
def test_modes_ragged(is_neox, rope_offset, norm, had, fused):
    """Every kernel variant on a ragged token count (not a multiple of the 4
    or 16 tokens a block covers) and 16, 48 and 80 heads; below 512 tokens the
    query side runs the small-batch kernel, at 613 the per-token kernels."""
    for T, H in [(1, 16), (37, 48), (301, 80), (613, 48)]:
        wl = workloads.sweep_case(7 * T + H, T, H, is_neox, rope_offset)
        wl.apply_hadamard = had
        if norm:
            rng = np.random.default_rng(T)
            wl.k_norm_gamma = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal(128)).astype(np.float32))
        check(wl, fused=fused)


@FUSED
@pytest.mark.parametrize("is_neox", [True, False])
@pytest.mark.parametrize("rope_offset", [0, 64])
@pytest.mark.parametrize("had", [False, True])
def test_overflow_rows(is_neox, rope_offset, had, fused):
    """Finite inputs whose rotation leaves the fp32 range: half of the query
    and key rows carry one RoPE pair of largest-magnitude bf16 values, so one
    output of the pair is +-inf.  Its group amax is infinite, amax / 6 too, and
    the exponent field 255 clamps to e = 254 (the block-exponent rule of
    sgl-project/sglang PR 39656, review); the infinite value takes code 7.
    With the Hadamard the infinity reaches every value of its row (no NaN: a
    row holds one infinity).  T = 40 runs the small-batch kernel, T = 613 the
    per-token ones."""
    for T in (40, 613):
        wl = workloads.overflow_case(31 + T, T, 16 if T < 100 else 48, is_neox, rope_offset, had)
        say(f"case {wl.name}: T={wl.T} H={wl.H} fused={fused}")
        got = gpu_run(wl, fused=fused)
        ref = oracle_run(wl)
        assert (ref[1] == 254).any() and (ref[4] == 254).any()  # the case reaches e = 254
        assert_all_same(got, ref)


@FUSED
@pytest.mark.parametrize("had", [False, True])
def test_maximum_heads(had, fused):
    """H = 2048, the largest head count the ABI accepts (J = 128 q-scale
    columns; 32 KB of LDS per block), on 6 tokens including a skipped slot."""
    wl = workloads.sweep_case(777, 6, 2048, True, 64)
    wl.apply_hadamard = had
    wl.slot_mapping[2] = -1
    check(wl, fused=fused)


@FUSED
@pytest.mark.parametrize("had", [False, True])
def test_maximum_heads_per_token_kernels(had, fused):
    """H = 2048 above the small-batch threshold (521 tokens): the per-token
    kernels loop 128 times over 16 heads, and the Hadamard query path stages
    its code bytes in LDS beside the 32 KB scale rows; interleaved RoPE on
    dims 0..63 with key RMSNorm."""
    wl = workloads.sweep_case(778, 521, 2048, False, 0)
    wl.apply_hadamard = had
    rng = np.random.default_rng(778)
    wl.k_norm_gamma = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal(128)).astype(np.float32))
    wl.slot_mapping[5] = -1
    check(wl, fused=fused)


@FUSED
def test_no_weights_and_scale_floor(fused):
    wl = workloads.edge_mix(seed=21, T=64)
    wl.scale_floor = float(np.float32(1e-10))   # all-zero groups get e = 94
    check(wl, with_weights=False, fused=fused)


@FUSED
def test_out_of_range_positions_and_slots(fused):
    wl = workloads.sweep_case(5, 40, 32, True, 64)
    wl.positions[:4] = [-3, wl.max_pos, wl.max_pos + 99, 2 ** 40]
    wl.slot_mapping[4:8] = [-1, -5, wl.NB * 64, wl.NB * 64 + 12345]
    check(wl, fused=fused)


@FUSED
def test_decode_with_background_cache(fused):
    wl = workloads.decode()
    got = check(wl, fused=fused)
    # every slot was written by the background keys: no sentinel row is left
    assert not (got[4] == SENTINEL).all(axis=-1).any()


@FUSED
def test_prefill_norm_rotate(fused):
    check(workloads.prefill_norm_rotate(), fused=fused)


def _cancelling_rows(rng, n):
    """bf16 rows whose Hadamard transform meets exact zeros, where only the
    IEEE rules for signed zeros and exact cancellation (x - x = +0) decide the
    sign bit of a code: all +0, all -0, mixed +-0, one nonzero among zeros,
    period 8 (every stride-8 difference cancels), x[j + 8] = -x[j] (every
    stride-8 sum cancels), equal pairs (every stride-1 difference cancels), and
    subnormal-only rows."""
    rows = np.zeros((n, 128), np.uint16)
    for i in range(n):
        kind = i % 8
        base = workloads.to_bf16_bits(rng.standard_normal(128).astype(np.float32))
        signs = (rng.integers(0, 2, 128) * 0x8000).astype(np.uint16)
        if kind == 0:
            r = np.zeros(128, np.uint16)
        elif kind == 1:
            r = np.full(128, 0x8000, np.uint16)
        elif kind == 2:
            r = signs
        elif kind == 3:
            r = signs.copy()
            r[rng.integers(0, 128)] = base[0]
        elif kind == 4:
            r = np.tile(base[:8], 16)
        elif kind == 5:
            r = np.tile(base[:8], 16) ^ np.repeat(np.tile(np.array([0, 0x8000], np.uint16), 8), 8)
        elif kind == 6:
            r = np.repeat(base[:64], 2)
        else:
            r = rng.integers(1, 0x80, 128).astype(np.uint16) | signs
        rows[i] = r
    return rows


@FUSED
@pytest.mark.parametrize("is_neox", [True, False])
@pytest.mark.parametrize("T", [37, 613])
def test_hadamard_signed_zeros_and_cancellation(T, is_neox, fused):
    """The Hadamard path on rows built so that exact zeros reach the
    quantizer: the sign of each zero code must follow the IEEE operations of
    the natural-order transform exactly (the cross-lane butterflies included).
    Half the tokens sit at position 0 (cos 1, sin 0), so the patterns also
    cross the rotated slice; 37 tokens take the small-batch kernel, 613 the
    per-token one."""
    H = 48
    rng = np.random.default_rng(1000 + T)
    wl = workloads.sweep_case(31 * T, T, H, is_neox, 64)
    wl.apply_hadamard = True
    wl.positions[::2] = 0
    q = wl.q.reshape(T * H, 128)
    pick = rng.random(T * H) < 0.5
    q[pick] = _cancelling_rows(rng, int(pick.sum()))
    kp = rng.random(T) < 0.5
    wl.k[kp] = _cancelling_rows(rng, int(kp.sum()))
    wl.k_norm_gamma = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal(128)).astype(np.float32))
    got = check(wl, fused=fused)
    # the case must actually reach zero codes of both signs
    codes = np.concatenate([got[0].reshape(-1) & 0x0F, got[0].reshape(-1) >> 4])
    assert (codes == 0x0).any() and (codes == 0x8).any()


def test_non_default_stream():
    import torch

    s = torch.cuda.Stream()
    wl = workloads.sweep_case(9, 96, 64, True, 64)
    with torch.cuda.stream(s):
        got = gpu_run(wl, stream=s)
    assert_all_same(got, oracle_run(wl))


def test_empty_batch():
    import torch

    from pack_token_amd import fp4idx

    dev = "cuda:0"
    q = torch.empty((0, 32, 128), dtype=torch.bfloat16, device=dev)
    pos = torch.empty(0, dtype=torch.int64, device=dev)
    cs = torch.zeros((1, 64), dtype=torch.float32, device=dev)
    q_out, qs, _ = fp4idx.q_rope_pack(q, pos, cs)
    kv = torch.full((1, 1, 4, 64, 16), SENTINEL, dtype=torch.uint8, device=dev)
    ks = torch.full((1, 1, 4, 64), SENTINEL, dtype=torch.uint8, device=dev)
    fp4idx.k_rope_pack_store(torch.empty((0, 128), dtype=torch.bfloat16, device=dev), pos, cs,
                             torch.empty(0, dtype=torch.int64, device=dev), kv, ks)
    torch.cuda.synchronize()
    assert q_out.shape == (0, 32, 64) and (kv == SENTINEL).all() and (ks == SENTINEL).all()


def test_converter_exhaustive():
    """Every finite bf16 value under every block exponent e in [1, 253] it can
    meet (|v| <= 6 * 2^(e-127)), through the unrotated groups of the query
    path: one anchor element per group forces e, the other 31 carry the test
    values.  Compares codes and exponents with the oracle."""
    import torch

    from pack_token_amd import fp4idx

    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[((allb.astype(np.uint32) >> 7) & 0xFF) != 0xFF]
    mag = finite & 0x7FFF
    groups = []
    for e in range(1, 254):
        anchor = 0x7F7F if e == 253 else int(workloads.to_bf16_bits(
            np.array([6.0 * 2.0 ** (e - 127)], np.float32))[0])
        vals = finite[mag <= anchor]
        n = -(-vals.size // 31) * 31
        vals = np.concatenate([vals, np.zeros(n - vals.size, np.uint16)]).reshape(-1, 31)
        g = np.empty((vals.shape[0], 32), np.uint16)
        g[:, 0] = anchor
        g[:, 1:] = vals
        groups.append(g)
    groups = np.concatenate(groups)
    H = 64
    rows = -(-groups.shape[0] // 2)
    T = -(-rows // H)
    q = np.zeros((T * H, 128), np.uint16)
    flat = np.zeros((T * H * 2, 32), np.uint16)
    flat[: groups.shape[0]] = groups
    q[:, :64] = flat.reshape(T * H, 64)           # groups 0 and 1: not rotated (rope_offset 64)
    q = q.reshape(T, H, 128)
    pos = np.zeros(T, np.int64)
    cs = workloads.cos_sin_table(1)
    say(f"case converter_exhaustive: {groups.shape[0]} groups, T={T} H={H}")
    dev = "cuda:0"
    q_out, qs, _ = fp4idx.q_rope_pack(torch.from_numpy(q.view(np.int16)).to(dev),
                                      torch.from_numpy(pos).to(dev), torch.from_numpy(cs).to(dev))
    torch.cuda.synchronize()
    ref_q, ref_qs, _ = oracle.q_rope_pack(q, pos, cs, None, threads=8)
    assert_same("q_out", q_out.cpu().numpy(), ref_q)
    assert_same("q_scale_out", qs.cpu().numpy(), ref_qs)


def test_dequant_debug_matches_oracle():
    import torch

    from pack_token_amd import fp4idx

    wl = workloads.edge_mix(seed=33, T=120)
    got = gpu_run(wl)
    q_out, qs, _, kv, ks = got
    dev = "cuda:0"
    qd = fp4idx.dequant_q(torch.from_numpy(q_out).to(dev), torch.from_numpy(qs).to(dev))
    slots = np.concatenate([wl.slot_mapping, np.array([-1, wl.NB * 64, 3], np.int64)])
    kd = fp4idx.dequant_kcache(torch.from_numpy(kv).to(dev), torch.from_numpy(ks).to(dev),
                               torch.from_numpy(slots).to(dev))
    kall = fp4idx.dequant_kcache(torch.from_numpy(kv).to(dev), torch.from_numpy(ks).to(dev))
    torch.cuda.synchronize()
    assert_same("dequant_q", qd.cpu().numpy(), oracle.dequant_q(q_out, qs))
    assert_same("dequant_k", kd.cpu().numpy(), oracle.dequant_kcache(kv, ks, slots))
    assert_same("dequant_k_all", kall.cpu().numpy(), oracle.dequant_kcache(kv, ks))


_LARGE = {}


def _large_prefill_with_oracle():
    """The large-prefill workload and the oracle's five outputs on all of its
    tokens (computed once per test session: about 1 s on 16 threads)."""
    if not _LARGE:
        wl = large_prefill()
        say(f"case {wl.name}: T={wl.T} H={wl.H} (inputs generated)")
        _LARGE["wl"] = wl
        _LARGE["ref"] = oracle_run(wl)
        say("case large_prefill: oracle outputs computed for every token")
    return _LARGE["wl"], _LARGE["ref"]


@FUSED
def test_large_prefill_full_size(fused):
    """T = 131072, H = 64 in the launch configurations the benchmark times:
    all 131,072 tokens against the oracle, byte for byte, on all five outputs
    (the whole q_out, q_scale_out and weights_out, and the whole key cache and
    its scale rows after every token's key was stored)."""
    wl, ref = _large_prefill_with_oracle()
    got = gpu_run(wl, fused=fused)
    say(f"case large_prefill fused={fused}: GPU outputs copied back")
    assert_all_same(got, ref)
    # no sentinel byte is left anywhere in the cache: every slot was written
    assert (got[3].reshape(wl.NB, 4, 64, 16) != SENTINEL).any(axis=-1).all()
    assert got[4].min() >= 1 and got[4].max() <= 253
    assert got[1].min() >= 1 and got[1].max() <= 253    # H = 64: no pad columns


def _cosine_accumulate(acc, a, b):
    acc[0] += float((a.double() * b.double()).sum())
    acc[1] += float((a.double() ** 2).sum())
    acc[2] += float((b.double() ** 2).sum())


def test_decode_score_cosine():
    """Dequantized per-head q.k scores of the 256 decode queries (x 32 heads)
    against all 262,144 cached keys: cosine >= 0.9999 between the GPU's and the
    oracle's dequantized values, and >= 0.97 against the unquantized rotated
    bf16 vectors (the pages report 0.980 for an FP4 indexer pipeline against bf16
    ground truth, ROCm/aiter PR 5484 "Verification")."""
    import torch

    from pack_token_amd import fp4idx
    from pack_token_amd.workloads import bf16_bits_to_f32

    wl = workloads.decode()
    say(f"case decode scores: {wl.T}x{wl.H} queries vs {wl.NB * 64} keys")
    got = gpu_run(wl, fused=True)
    ref = oracle_run(wl)
    assert_all_same(got, ref)
    q_out, qs, _, kv, ks = got
    dev = "cuda:0"
    # GPU-side dequantization of the GPU's bytes; oracle-side of the oracle's bytes
    qd_gpu = fp4idx.dequant_q(torch.from_numpy(q_out).to(dev), torch.from_numpy(qs).to(dev))
    kd_gpu = fp4idx.dequant_kcache(torch.from_numpy(kv).to(dev), torch.from_numpy(ks).to(dev))
    qd_ref = torch.from_numpy(oracle.dequant_q(ref[0], ref[1])).to(dev)
    kd_ref = torch.from_numpy(oracle.dequant_kcache(ref[3], ref[4])).to(dev)
    # unquantized reference: the same RoPE on the bf16 inputs, keys as the cache holds them
    cs = wl.cos_sin[wl.positions]
    qr = oracle.rope_rows(bf16_bits_to_f32(wl.q).reshape(-1, 128), np.repeat(cs, wl.H, 0))
    k_all = bf16_bits_to_f32(wl.background["k"]).copy()
    pos_all = wl.background["positions"].copy()
    k_all[wl.slot_mapping] = bf16_bits_to_f32(wl.k)
    pos_all[wl.slot_mapping] = wl.positions
    kr = oracle.rope_rows(k_all, wl.cos_sin[pos_all])
    qr = torch.from_numpy(qr).to(dev)
    kr = torch.from_numpy(kr).to(dev)
    Q = [qd_gpu.reshape(-1, 128), qd_ref.reshape(-1, 128), qr]
    acc_ref, acc_bf16 = [0.0, 0.0, 0.0], [0.0, 0.0, 0.0]
    for a in range(0, kd_gpu.shape[0], 32768):
        kt = [x[a:a + 32768].t().contiguous() for x in (kd_gpu, kd_ref, kr)]
        s_gpu = Q[0] @ kt[0]
        s_ref = Q[1] @ kt[1]
        s_bf = Q[2] @ kt[2]
        _cosine_accumulate(acc_ref, s_gpu, s_ref)
        _cosine_accumulate(acc_bf16, s_gpu, s_bf)
    cos_ref = acc_ref[0] / np.sqrt(acc_ref[1] * acc_ref[2])
    cos_bf = acc_bf16[0] / np.sqrt(acc_bf16[1] * acc_bf16[2])
    say(f"score cosine: vs oracle {cos_ref:.7f}, vs bf16 {cos_bf:.5f}")
    assert cos_ref >= 0.9999
    assert cos_bf >= 0.97


def test_graph_replay_matches_oracle():
    """The fused call captured in a HIP graph, replayed three times with new
    inputs copied in (eager work) between replays; every replay equals the
    oracle on that replay's inputs."""
    import torch

    from pack_token_amd import fp4idx

    dev = "cuda:0"
    base = workloads.sweep_case(31, 48, 32, True, 64)
    from harness import dev_tensors
    d = dev_tensors(base, dev)
    T, H = base.T, base.H
    q_out = torch.empty((T, H, 64), dtype=torch.uint8, device=dev)
    qs = torch.empty((T, 1, 4, 16, base.J), dtype=torch.uint8, device=dev)
    w_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    kv = torch.empty((base.NB, 1, 4, 64, 16), dtype=torch.uint8, device=dev)
    ks = torch.empty((base.NB, 1, 4, 64), dtype=torch.uint8, device=dev)

    def step():
        fp4idx.qk_rope_pack_store(d["q"], d["k"], d["positions"], d["cos_sin"], d["slot_mapping"],
                                  kv, ks, d["weights"], q_out=q_out, q_scale_out=qs,
                                  weights_out=w_out)

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        wl = workloads.sweep_case(40 + rep, T, H, True, 64)
        wl.slot_mapping = base.slot_mapping
        wl.positions = base.positions
        for name, arr in (("q", wl.q.view(np.int16)), ("k", wl.k.view(np.int16)),
                          ("weights", wl.weights)):
            d[name].copy_(torch.from_numpy(arr).to(dev))
        kv.fill_(SENTINEL)
        ks.fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (q_out.cpu().numpy(), qs.cpu().numpy(), w_out.cpu().numpy(), kv.cpu().numpy(),
               ks.cpu().numpy())
        assert_all_same(got, oracle_run(wl))


@FUSED
@pytest.mark.parametrize("T", [1, 5, 64, 300])
@pytest.mark.parametrize("pos32", [False, True])
def test_sglang_row_matrix(T, pos32, fused):
    """Rows {1, 5, 64, 300} x scales {1, 40, 1e-3} plus zero, subnormal and
    half-way groups x int32/int64 positions, the matrix of sgl-project/sglang
    PR 39656 "Verification" (compress ratios are a different producer)."""
    check(workloads.edge_mix(seed=200 + T, T=T, positions_int32=pos32), fused=fused)


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes_and_modes(seed):
    """Seeded random cases over shapes and modes, both the two-call path and the
    fused launch, byte for byte against the oracle."""
    wl, with_weights = random_case(seed)
    ref = oracle_run(wl, with_weights=with_weights)
    for fused in (False, True):
        say(f"case {wl.name}: neox={wl.is_neox} ro={wl.rope_offset} had={wl.apply_hadamard} "
            f"norm={wl.k_norm_gamma is not None} floor={wl.scale_floor:g} "
            f"pos={wl.positions.dtype} weights={with_weights} fused={fused}")
        assert_all_same(gpu_run(wl, with_weights=with_weights, fused=fused), ref)
