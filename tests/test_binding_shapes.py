"""The Python binding's shape checks (CPU only).

The C ABI takes plain pointers, so the binding is the last place where a
tensor of the wrong size can be caught before a kernel reads or writes past
it.  Every entry function checks the sizes of all its tensors before it looks
at devices: here each call gets CPU tensors with one argument of the wrong
size and must raise a ValueError naming that argument, and with every size
right it must get past the shape checks to the device check ("must be on the
GPU")."""
import pytest
import torch

from pack_token_amd import fp4idx as F

T, H, D, NB = 5, 32, 128, 3
J = F.q_scale_cols(H)
U8, BF, I64, I32, F32 = torch.uint8, torch.bfloat16, torch.int64, torch.int32, torch.float32


def z(*shape, dtype=U8):
    return torch.zeros(shape, dtype=dtype)


def fp4_args():
    return dict(q=z(T, H, D, dtype=BF), k=z(T, D, dtype=BF), positions=z(T, dtype=I64),
                cos_sin=z(16, 64, dtype=F32), weights=z(T, H, dtype=F32),
                slot_mapping=z(T, dtype=I64), kv_cache=z(NB, 1, 4, 64, 16),
                kv_cache_scale=z(NB, 1, 4, 64))


def call_q(a, **kw):
    return F.q_rope_pack(a["q"], a["positions"], a["cos_sin"], a["weights"], **kw)


def call_k(a, **kw):
    return F.k_rope_pack_store(a["k"], a["positions"], a["cos_sin"], a["slot_mapping"],
                               a["kv_cache"], a["kv_cache_scale"], **kw)


def call_qk(a, **kw):
    return F.qk_rope_pack_store(a["q"], a["k"], a["positions"], a["cos_sin"], a["slot_mapping"],
                                a["kv_cache"], a["kv_cache_scale"], a["weights"], **kw)


def call_q8(a, **kw):
    return F.q_rope_pack_fp8(a["q"], a["positions"], a["cos_sin"], a["weights"], **kw)


def call_k8(a, **kw):
    return F.k_rope_pack_store_fp8(a["k"], a["positions"], a["cos_sin"], a["slot_mapping"],
                                   a.get("kv8", z(NB, 64, 128)), a.get("ks8", z(NB, 64, dtype=F32)),
                                   **kw)


def call_qs(a, **kw):
    return F.q_rope_pack_sglang(a["q"], a["positions"], a["cos_sin"], **kw)


def call_ks(a, **kw):
    return F.k_rope_pack_store_sglang(a["k"], a["positions"], a["cos_sin"], a["slot_mapping"],
                                      a.get("idx", z(64, 68)), **kw)


def call_fq(a, **kw):
    return F.rope_fake_quant(a["q"], a["positions"], a["cos_sin"], rows_per_position=H, **kw)


def scorer_args():
    B, next_n, max_blocks = 2, 2, 4
    return dict(q_out=z(B * next_n, H, 64), q_scale_out=z(B * next_n, 1, 4, 16, J),
                weights=z(B * next_n, H, dtype=F32), kv_cache=z(NB, 1, 4, 64, 16),
                kv_cache_scale=z(NB, 1, 4, 64), block_table=z(B, max_blocks, dtype=I32),
                context_lens=z(B, dtype=I32), next_n=next_n)


def call_sc(a, **kw):
    a = dict(a)
    next_n = a.pop("next_n")
    return F.paged_mqa_logits(a["q_out"], a["q_scale_out"], a["weights"], a["kv_cache"],
                              a["kv_cache_scale"], a["block_table"], a["context_lens"], next_n,
                              **kw)


CALLS = [call_q, call_k, call_qk, call_q8, call_k8, call_qs, call_ks, call_fq]


@pytest.mark.parametrize("call", CALLS + [call_sc], ids=lambda c: c.__name__)
def test_right_sizes_reach_the_device_check(call):
    a = scorer_args() if call is call_sc else fp4_args()
    with pytest.raises(ValueError, match="must be on the GPU"):
        call(a)


BAD_ARGS = [
    (call_q, "positions", z(T + 1, dtype=I64)),
    (call_q, "cos_sin", z(16, 32, dtype=F32)),
    (call_q, "weights", z(T, H + 16, dtype=F32)),
    (call_k, "positions", z(T - 1, dtype=I64)),
    (call_k, "slot_mapping", z(T + 3, dtype=I64)),
    (call_k, "kv_cache_scale", z(NB - 1, 1, 4, 64)),
    (call_k, "kv_cache", z(NB, 1, 4, 32, 16)),
    (call_qk, "k", z(T + 1, D, dtype=BF)),
    (call_qk, "weights", z(T, 16, dtype=F32)),
    (call_qk, "kv_cache_scale", z(NB, 1, 4, 32)),
    (call_q8, "weights", z(T - 1, H, dtype=F32)),
    (call_k8, "slot_mapping", z(1, dtype=I64)),
    (call_k8, "kv_cache_scale", z(NB, 32, dtype=F32)),
    (call_qs, "positions", z(2 * T, dtype=I64)),
    (call_ks, "slot_mapping", z(T + 1, dtype=I64)),
]


@pytest.mark.parametrize("call,name,bad", BAD_ARGS,
                         ids=[f"{c.__name__}-{n}" for c, n, _ in BAD_ARGS])
def test_wrong_input_size_is_refused(call, name, bad):
    a = fp4_args()
    a[{"kv_cache_scale": "ks8"}.get(name, name) if call is call_k8 else name] = bad
    with pytest.raises(ValueError, match=name):
        call(a)


BAD_OUTPUTS = [
    (call_q, "q_out", dict(q_out=z(T, H, 63))),
    (call_q, "q_scale_out", dict(q_scale_out=z(T, 1, 4, 16, J - 1))),
    (call_q, "weights_out", dict(weights_out=z(T, H - 1, dtype=F32))),
    (call_k, "k_norm_gamma", dict(k_norm_gamma=z(64, dtype=BF))),
    (call_qk, "q_scale_out", dict(q_scale_out=z(T - 1, 1, 4, 16, J))),
    (call_qk, "k_norm_gamma", dict(k_norm_gamma=z(129, dtype=BF))),
    (call_q8, "q_out", dict(q_out=z(T, H, 64))),
    (call_q8, "weights_out", dict(weights_out=z(T, 1, dtype=BF))),
    (call_k8, "k_norm_gamma", dict(k_norm_gamma=z(127, dtype=BF))),
    (call_ks, "k_norm_gamma", dict(k_norm_gamma=z(1, dtype=BF))),
    (call_fq, "y", dict(y=z(T, H, 127, dtype=BF))),
]


@pytest.mark.parametrize("call,name,kw", BAD_OUTPUTS,
                         ids=[f"{c.__name__}-{n}" for c, n, _ in BAD_OUTPUTS])
def test_wrong_output_or_option_size_is_refused(call, name, kw):
    with pytest.raises(ValueError, match=name):
        call(fp4_args(), **kw)


@pytest.mark.parametrize("name,bad", [
    ("q_scale_out", z(4, 1, 4, 16, J + 4)),
    ("weights", z(4, H - 16, dtype=F32)),
    ("kv_cache_scale", z(NB + 1, 1, 4, 64)),
    ("context_lens", z(3, dtype=I32)),
])
def test_scorer_wrong_size_is_refused(name, bad):
    a = scorer_args()
    a[name] = bad
    with pytest.raises(ValueError, match=name):
        call_sc(a)


def test_scorer_logits_and_stride():
    a = scorer_args()
    with pytest.raises(ValueError, match="logits"):
        call_sc(a, logits=z(3, 256, dtype=F32))
    with pytest.raises(ValueError, match="stride"):
        call_sc(a, logits=z(4, 256, dtype=F32), stride=128)


def test_dequant_sizes():
    with pytest.raises(ValueError, match="q_scale_out"):
        F.dequant_q(z(T, H, 64), z(T, 1, 4, 16, J + 1))
    with pytest.raises(ValueError, match="out"):
        F.dequant_q(z(T, H, 64), z(T, 1, 4, 16, J), out=z(T, H, 64, dtype=F32))
    with pytest.raises(ValueError, match="kv_cache_scale"):
        F.dequant_kcache(z(NB, 1, 4, 64, 16), z(NB, 1, 4, 63))
    with pytest.raises(ValueError, match="out"):
        F.dequant_kcache(z(NB, 1, 4, 64, 16), z(NB, 1, 4, 64), z(7, dtype=I64),
                         out=z(6, 128, dtype=F32))
