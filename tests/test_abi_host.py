"""CPU-only checks of the C ABI: the library loads, exports every entry point
declared in include/fp4idx.h, and rejects bad arguments on the host with a
specific message before any GPU work (ROCm/aiter PR 5484 "API": shapes
outside head_dim 128, rope_dim 64, group 32, kv block 64, n_heads % 16 are
refused on the host).  These calls never reach a kernel launch."""
import ctypes
import os
import re

import pytest

from pack_token_amd import fp4idx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4idx.h")

ALIGNED = 1 << 20       # a fake, well-aligned non-null address; never dereferenced
MISALIGNED = ALIGNED + 2


def declared_functions(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(fp4idx_\w+)\(", text, re.M)))


def test_exports_every_measurement_symbol():
    names = declared_functions(os.path.join(ROOT, "include", "fp4idx_ceiling.h"))
    assert names == ["fp4idx_ceiling_paged_gather", "fp4idx_ceiling_stream", "fp4idx_ceiling_valu"]
    lib = ctypes.CDLL(fp4idx.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_measurement_entry_points_reject_bad_arguments():
    L = fp4idx.lib()
    assert L.fp4idx_ceiling_stream(ALIGNED, 1024, None, 0, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_stream(ALIGNED, 1040, ALIGNED, 1024, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_stream(MISALIGNED, 1024, ALIGNED, 1024, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_stream(ALIGNED, (1 << 40) + 1024, ALIGNED, 0, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_paged_gather(ALIGNED, ALIGNED, 4, ALIGNED, 8, ALIGNED, 1025, 1,
                                         ALIGNED, 64, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_paged_gather(ALIGNED, ALIGNED, 4, ALIGNED, 8, ALIGNED, 4, 65,
                                         ALIGNED, 64, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_valu(5, 8, 16, ALIGNED, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_valu(-1, 8, 16, ALIGNED, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_valu(0, 0, 16, ALIGNED, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_valu(0, (1 << 20) + 1, 16, ALIGNED, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_valu(0, 8, -1, ALIGNED, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_valu(0, 8, (1 << 32) + 1, ALIGNED, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_valu(0, 8, 16, None, None) == fp4idx.EINVAL
    assert L.fp4idx_ceiling_valu(0, 8, 16, ALIGNED + 2, None) == fp4idx.EINVAL


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert names == ["fp4idx_dequant_debug", "fp4idx_k_rope_pack_store",
                     "fp4idx_k_rope_pack_store_fp8", "fp4idx_k_rope_pack_store_sglang",
                     "fp4idx_last_error", "fp4idx_paged_mqa_logits", "fp4idx_q_rope_pack",
                     "fp4idx_q_rope_pack_fp8", "fp4idx_q_rope_pack_sglang",
                     "fp4idx_qk_rope_pack_store", "fp4idx_rope_fake_quant"]
    lib = ctypes.CDLL(fp4idx.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def q_call(**over):
    a = dict(q=ALIGNED, positions=ALIGNED, positions_int64=1, cos_sin=ALIGNED, max_pos=16,
             weights=None, T=4, H=32, D=128, R=64, rope_offset=64, group_size=32, is_neox=1,
             apply_hadamard=0, scale_floor=2.0 ** -126, q_out=ALIGNED, q_scale_out=ALIGNED,
             weights_out=None, stream=None)
    a.update(over)
    return fp4idx.lib().fp4idx_q_rope_pack(*a.values())


def k_call(**over):
    a = dict(k=ALIGNED, positions=ALIGNED, positions_int64=1, cos_sin=ALIGNED, max_pos=16,
             slot_mapping=ALIGNED, k_norm_gamma=None, k_norm_eps=1e-6, T=4, D=128, R=64,
             rope_offset=64, group_size=32, is_neox=1, apply_hadamard=0,
             scale_floor=2.0 ** -126, kv_cache=ALIGNED, kv_cache_scale=ALIGNED, NB=2, BS=64,
             stream=None)
    a.update(over)
    return fp4idx.lib().fp4idx_k_rope_pack_store(*a.values())


def qk_call(**over):
    a = dict(q=ALIGNED, k=ALIGNED, positions=ALIGNED, positions_int64=1, cos_sin=ALIGNED,
             max_pos=16, weights=None, slot_mapping=ALIGNED, k_norm_gamma=None, k_norm_eps=1e-6,
             T=4, H=32, D=128, R=64, rope_offset=64, group_size=32, is_neox=1, apply_hadamard=0,
             scale_floor=2.0 ** -126, q_out=ALIGNED, q_scale_out=ALIGNED, weights_out=None,
             kv_cache=ALIGNED, kv_cache_scale=ALIGNED, NB=2, BS=64, stream=None)
    a.update(over)
    return fp4idx.lib().fp4idx_qk_rope_pack_store(*a.values())


def d_call(**over):
    a = dict(which=0, packed=ALIGNED, scales=ALIGNED, rows=4, H=32, slots=None, NB=2, BS=64,
             out=ALIGNED, stream=None)
    a.update(over)
    return fp4idx.lib().fp4idx_dequant_debug(*a.values())


Q_REJECT = [
    (dict(D=64), fp4idx.EUNSUPPORTED, "head_dim"),
    (dict(R=32), fp4idx.EUNSUPPORTED, "rope_dim"),
    (dict(group_size=16), fp4idx.EUNSUPPORTED, "group_size"),
    (dict(H=24), fp4idx.EUNSUPPORTED, "n_heads"),
    (dict(H=0), fp4idx.EUNSUPPORTED, "n_heads"),
    (dict(H=4096), fp4idx.EUNSUPPORTED, "n_heads"),
    (dict(rope_offset=32), fp4idx.EUNSUPPORTED, "rope_offset"),
    (dict(is_neox=2), fp4idx.EINVAL, "is_neox"),
    (dict(apply_hadamard=-1), fp4idx.EINVAL, "apply_hadamard"),
    (dict(positions_int64=3), fp4idx.EINVAL, "positions_int64"),
    (dict(T=-1), fp4idx.EINVAL, "T must be"),
    (dict(max_pos=0), fp4idx.EINVAL, "max_pos"),
    (dict(scale_floor=-1.0), fp4idx.EINVAL, "scale_floor"),
    (dict(scale_floor=float("nan")), fp4idx.EINVAL, "scale_floor"),
    (dict(scale_floor=float("inf")), fp4idx.EINVAL, "scale_floor"),
    (dict(weights=ALIGNED), fp4idx.EINVAL, "weights and weights_out"),
    (dict(weights_out=ALIGNED), fp4idx.EINVAL, "weights and weights_out"),
    (dict(q=None), fp4idx.EINVAL, "q must not be NULL"),
    (dict(q=MISALIGNED), fp4idx.EINVAL, "q must be 16-byte aligned"),
    (dict(positions=ALIGNED + 4), fp4idx.EINVAL, "positions must be 8-byte"),
    (dict(cos_sin=ALIGNED + 4), fp4idx.EINVAL, "cos_sin must be 16-byte"),
    (dict(q_out=ALIGNED + 8), fp4idx.EINVAL, "q_out must be 16-byte"),
    (dict(q_scale_out=ALIGNED + 1), fp4idx.EINVAL, "q_scale_out must be 4-byte"),
    (dict(q_scale_out=None), fp4idx.EINVAL, "q_scale_out must not be NULL"),
    (dict(weights=ALIGNED + 1, weights_out=ALIGNED), fp4idx.EINVAL, "weights must be 4-byte"),
    (dict(T=1 << 58), fp4idx.EINVAL, "T too large"),
]


@pytest.mark.parametrize("over,code,msg", Q_REJECT)
def test_q_rejections(over, code, msg):
    assert q_call(**over) == code
    assert msg in fp4idx.last_error(), fp4idx.last_error()
    assert fp4idx.last_error().startswith("fp4idx_q_rope_pack:")


K_REJECT = [
    (dict(D=256), fp4idx.EUNSUPPORTED, "head_dim"),
    (dict(BS=128), fp4idx.EUNSUPPORTED, "kv_block_size"),
    (dict(rope_offset=1), fp4idx.EUNSUPPORTED, "rope_offset"),
    (dict(NB=-1), fp4idx.EINVAL, "NB must be"),
    (dict(k_norm_gamma=ALIGNED, k_norm_eps=-1.0), fp4idx.EINVAL, "k_norm_eps"),
    (dict(k_norm_gamma=ALIGNED, k_norm_eps=float("nan")), fp4idx.EINVAL, "k_norm_eps"),
    (dict(k_norm_gamma=ALIGNED + 2), fp4idx.EINVAL, "k_norm_gamma must be 16-byte"),
    (dict(slot_mapping=None), fp4idx.EINVAL, "slot_mapping must not be NULL"),
    (dict(slot_mapping=ALIGNED + 4), fp4idx.EINVAL, "slot_mapping must be 8-byte"),
    (dict(kv_cache=ALIGNED + 4), fp4idx.EINVAL, "kv_cache must be 16-byte"),
    (dict(kv_cache_scale=ALIGNED + 2), fp4idx.EINVAL, "kv_cache_scale must be 4-byte"),
    (dict(k=None), fp4idx.EINVAL, "k must not be NULL"),
    (dict(positions_int64=0, positions=ALIGNED + 2), fp4idx.EINVAL, "positions must be 4-byte"),
]


@pytest.mark.parametrize("over,code,msg", K_REJECT)
def test_k_rejections(over, code, msg):
    assert k_call(**over) == code
    assert msg in fp4idx.last_error(), fp4idx.last_error()


D_REJECT = [
    (dict(which=2), fp4idx.EINVAL, "which"),
    (dict(rows=-1), fp4idx.EINVAL, "rows"),
    (dict(H=8), fp4idx.EUNSUPPORTED, "n_heads"),
    (dict(which=1, BS=32), fp4idx.EUNSUPPORTED, "kv_block_size"),
    (dict(out=ALIGNED + 4), fp4idx.EINVAL, "out must be 16-byte"),
    (dict(which=1, slots=ALIGNED + 4), fp4idx.EINVAL, "slots must be 8-byte"),
    (dict(packed=None), fp4idx.EINVAL, "packed must not be NULL"),
]


@pytest.mark.parametrize("over,code,msg", D_REJECT)
def test_dequant_rejections(over, code, msg):
    assert d_call(**over) == code
    assert msg in fp4idx.last_error(), fp4idx.last_error()


QK_REJECT = [
    (dict(D=64), fp4idx.EUNSUPPORTED, "head_dim"),
    (dict(H=40), fp4idx.EUNSUPPORTED, "n_heads"),
    (dict(BS=16), fp4idx.EUNSUPPORTED, "kv_block_size"),
    (dict(q=None), fp4idx.EINVAL, "q must not be NULL"),
    (dict(k=None), fp4idx.EINVAL, "k must not be NULL"),
    (dict(k=MISALIGNED), fp4idx.EINVAL, "k must be 16-byte aligned"),
    (dict(slot_mapping=None), fp4idx.EINVAL, "slot_mapping must not be NULL"),
    (dict(weights=ALIGNED), fp4idx.EINVAL, "weights and weights_out"),
    (dict(kv_cache=ALIGNED + 8), fp4idx.EINVAL, "kv_cache must be 16-byte"),
    (dict(q_scale_out=ALIGNED + 2), fp4idx.EINVAL, "q_scale_out must be 4-byte"),
    (dict(k_norm_gamma=ALIGNED, k_norm_eps=-2.0), fp4idx.EINVAL, "k_norm_eps"),
    (dict(NB=-3), fp4idx.EINVAL, "NB must be"),
]


@pytest.mark.parametrize("over,code,msg", QK_REJECT)
def test_qk_rejections(over, code, msg):
    assert qk_call(**over) == code
    assert msg in fp4idx.last_error(), fp4idx.last_error()
    assert fp4idx.last_error().startswith("fp4idx_qk_rope_pack_store:")


def s_call(**over):
    a = dict(q_out=ALIGNED, q_scale_out=ALIGNED, weights=ALIGNED, weights_scale=1.0,
             kv_cache=ALIGNED, kv_cache_scale=ALIGNED, NB=4, block_table=ALIGNED, max_blocks=8,
             context_lens=ALIGNED, B=2, next_n=4, H=32, apply_relu=1, logits=ALIGNED,
             stride=512, stream=None)
    a.update(over)
    return fp4idx.lib().fp4idx_paged_mqa_logits(*a.values())


S_REJECT = [
    (dict(H=128), fp4idx.EUNSUPPORTED, "n_heads"),
    (dict(H=24), fp4idx.EUNSUPPORTED, "n_heads"),
    (dict(next_n=2 * 65535 + 1), fp4idx.EUNSUPPORTED, "next_n"),
    (dict(next_n=0), fp4idx.EUNSUPPORTED, "next_n"),
    (dict(apply_relu=2), fp4idx.EINVAL, "apply_relu"),
    (dict(weights_scale=float("inf")), fp4idx.EINVAL, "weights_scale"),
    (dict(B=70000), fp4idx.EINVAL, "B must be"),
    (dict(NB=-1), fp4idx.EINVAL, "NB"),
    (dict(stride=0), fp4idx.EINVAL, "stride"),
    (dict(weights=ALIGNED + 4), fp4idx.EINVAL, "weights must be 16-byte"),
    (dict(q_out=None), fp4idx.EINVAL, "q_out must not be NULL"),
    (dict(block_table=ALIGNED + 2), fp4idx.EINVAL, "block_table must be 4-byte"),
    (dict(kv_cache=ALIGNED + 4), fp4idx.EINVAL, "kv_cache must be 16-byte"),
    (dict(logits=None), fp4idx.EINVAL, "logits must not be NULL"),
]


@pytest.mark.parametrize("over,code,msg", S_REJECT)
def test_scorer_rejections(over, code, msg):
    assert s_call(**over) == code
    assert msg in fp4idx.last_error(), fp4idx.last_error()


def sq_call(**over):
    a = dict(q=ALIGNED, positions=ALIGNED, positions_int64=1, cos_sin=ALIGNED, max_pos=16, T=4,
             H=32, D=128, R=64, rope_offset=64, group_size=32, is_neox=1,
             fake_quant_floor=2.0 ** -126, pack_floor=1e-10, q_packed=ALIGNED, stream=None)
    a.update(over)
    return fp4idx.lib().fp4idx_q_rope_pack_sglang(*a.values())


def sk_call(**over):
    a = dict(k=ALIGNED, positions=ALIGNED, positions_int64=1, cos_sin=ALIGNED, max_pos=16,
             slot_mapping=ALIGNED, k_norm_gamma=None, k_norm_eps=1e-6, T=4, D=128, R=64,
             rope_offset=64, group_size=32, is_neox=1, compress_ratio=1,
             fake_quant_floor=2.0 ** -126, pack_floor=1e-10, index_k_cache=ALIGNED, num_slots=128,
             stream=None)
    a.update(over)
    return fp4idx.lib().fp4idx_k_rope_pack_store_sglang(*a.values())


SQ_REJECT = [
    (dict(D=64), fp4idx.EUNSUPPORTED, "head_dim"),
    (dict(H=8), fp4idx.EUNSUPPORTED, "n_heads"),
    (dict(rope_offset=16), fp4idx.EUNSUPPORTED, "rope_offset"),
    (dict(fake_quant_floor=-1.0), fp4idx.EINVAL, "fake_quant_floor"),
    (dict(pack_floor=float("nan")), fp4idx.EINVAL, "pack_floor"),
    (dict(pack_floor=float("inf")), fp4idx.EINVAL, "pack_floor"),
    (dict(is_neox=5), fp4idx.EINVAL, "is_neox"),
    (dict(q_packed=None), fp4idx.EINVAL, "q_packed must not be NULL"),
    (dict(q_packed=ALIGNED + 2), fp4idx.EINVAL, "q_packed must be 16-byte"),
    (dict(q_packed=ALIGNED + 4), fp4idx.EINVAL, "q_packed must be 16-byte"),
    (dict(q=ALIGNED + 4), fp4idx.EINVAL, "q must be 16-byte"),
    (dict(T=1 << 58), fp4idx.EINVAL, "T too large"),
]


@pytest.mark.parametrize("over,code,msg", SQ_REJECT)
def test_sglang_q_rejections(over, code, msg):
    assert sq_call(**over) == code
    assert msg in fp4idx.last_error(), fp4idx.last_error()
    assert fp4idx.last_error().startswith("fp4idx_q_rope_pack_sglang:")


SK_REJECT = [
    (dict(group_size=64), fp4idx.EUNSUPPORTED, "group_size"),
    (dict(compress_ratio=3), fp4idx.EUNSUPPORTED, "compress_ratio"),
    (dict(compress_ratio=0), fp4idx.EUNSUPPORTED, "compress_ratio"),
    (dict(num_slots=-1), fp4idx.EINVAL, "num_slots"),
    (dict(num_slots=1 << 62), fp4idx.EINVAL, "num_slots"),
    (dict(fake_quant_floor=float("-inf")), fp4idx.EINVAL, "fake_quant_floor"),
    (dict(pack_floor=-0.5), fp4idx.EINVAL, "pack_floor"),
    (dict(k_norm_gamma=ALIGNED, k_norm_eps=-1.0), fp4idx.EINVAL, "k_norm_eps"),
    (dict(k_norm_gamma=ALIGNED + 8), fp4idx.EINVAL, "k_norm_gamma must be 16-byte"),
    (dict(index_k_cache=ALIGNED + 1), fp4idx.EINVAL, "index_k_cache must be 4-byte"),
    (dict(index_k_cache=None), fp4idx.EINVAL, "index_k_cache must not be NULL"),
    (dict(slot_mapping=ALIGNED + 4), fp4idx.EINVAL, "slot_mapping must be 8-byte"),
    (dict(positions_int64=0, positions=ALIGNED + 2), fp4idx.EINVAL, "positions must be 4-byte"),
]


@pytest.mark.parametrize("over,code,msg", SK_REJECT)
def test_sglang_k_rejections(over, code, msg):
    assert sk_call(**over) == code
    assert msg in fp4idx.last_error(), fp4idx.last_error()
    assert fp4idx.last_error().startswith("fp4idx_k_rope_pack_store_sglang:")


def fq_call(**over):
    a = dict(q=ALIGNED, positions=ALIGNED, positions_int64=1, cos_sin=ALIGNED, max_pos=16,
             weights=ALIGNED, weights_scale=1.0, T=4, H=32, D=128, R=64, rope_offset=64,
             is_neox=1, apply_hadamard=0, scale_fmt=0, scale_floor=2.0 ** -126, q_out=ALIGNED,
             weights_out=ALIGNED, stream=None)
    a.update(over)
    return fp4idx.lib().fp4idx_q_rope_pack_fp8(*a.values())


def fk_call(**over):
    a = dict(k=ALIGNED, positions=ALIGNED, positions_int64=1, cos_sin=ALIGNED, max_pos=16,
             slot_mapping=ALIGNED, k_norm_gamma=None, k_norm_eps=1e-6, T=4, D=128, R=64,
             rope_offset=64, is_neox=1, apply_hadamard=0, scale_fmt=1, scale_floor=2.0 ** -126,
             kv_cache=ALIGNED, kv_cache_scale=ALIGNED, NB=2, BS=64, stream=None)
    a.update(over)
    return fp4idx.lib().fp4idx_k_rope_pack_store_fp8(*a.values())


FQ_REJECT = [
    (dict(D=64), fp4idx.EUNSUPPORTED, "head_dim"),
    (dict(H=40), fp4idx.EUNSUPPORTED, "n_heads"),
    (dict(scale_fmt=2), fp4idx.EINVAL, "scale_fmt"),
    (dict(scale_fmt=1, scale_floor=0.0), fp4idx.EINVAL, "scale_floor must be >= 2^-126"),
    (dict(scale_fmt=1, scale_floor=1e-40), fp4idx.EINVAL, "scale_floor must be >= 2^-126"),
    (dict(scale_floor=-1.0), fp4idx.EINVAL, "scale_floor"),
    (dict(weights_scale=float("nan")), fp4idx.EINVAL, "weights_scale"),
    (dict(weights=None), fp4idx.EINVAL, "weights must not be NULL"),
    (dict(weights_out=None), fp4idx.EINVAL, "weights_out must not be NULL"),
    (dict(weights_out=ALIGNED + 1), fp4idx.EINVAL, "weights_out must be 2-byte"),
    (dict(q_out=ALIGNED + 8), fp4idx.EINVAL, "q_out must be 16-byte"),
    (dict(apply_hadamard=3), fp4idx.EINVAL, "apply_hadamard"),
]


@pytest.mark.parametrize("over,code,msg", FQ_REJECT)
def test_fp8_q_rejections(over, code, msg):
    assert fq_call(**over) == code
    assert msg in fp4idx.last_error(), fp4idx.last_error()
    assert fp4idx.last_error().startswith("fp4idx_q_rope_pack_fp8:")


FK_REJECT = [
    (dict(BS=32), fp4idx.EUNSUPPORTED, "kv_block_size"),
    (dict(NB=-1), fp4idx.EINVAL, "NB out of range"),
    (dict(scale_fmt=-1), fp4idx.EINVAL, "scale_fmt"),
    (dict(scale_floor=0.0), fp4idx.EINVAL, "scale_floor must be >= 2^-126"),
    (dict(kv_cache=ALIGNED + 8), fp4idx.EINVAL, "kv_cache must be 16-byte"),
    (dict(kv_cache_scale=ALIGNED + 2), fp4idx.EINVAL, "kv_cache_scale must be 4-byte"),
    (dict(k_norm_gamma=ALIGNED, k_norm_eps=float("inf")), fp4idx.EINVAL, "k_norm_eps"),
    (dict(slot_mapping=None), fp4idx.EINVAL, "slot_mapping must not be NULL"),
]


@pytest.mark.parametrize("over,code,msg", FK_REJECT)
def test_fp8_k_rejections(over, code, msg):
    assert fk_call(**over) == code
    assert msg in fp4idx.last_error(), fp4idx.last_error()
    assert fp4idx.last_error().startswith("fp4idx_k_rope_pack_store_fp8:")


def fq8_call(**over):
    a = dict(x=ALIGNED, rows=64, rows_per_position=16, positions=ALIGNED, positions_int64=1,
             cos_sin=ALIGNED, max_pos=16, D=128, R=64, rope_offset=64, is_neox=1,
             compress_ratio=1, mode=1, scale_floor=2.0 ** -126, y=ALIGNED, stream=None)
    a.update(over)
    return fp4idx.lib().fp4idx_rope_fake_quant(*a.values())


FQUANT_REJECT = [
    (dict(mode=2), fp4idx.EINVAL, "mode"),
    (dict(compress_ratio=8), fp4idx.EUNSUPPORTED, "compress_ratio"),
    (dict(rows_per_position=0), fp4idx.EINVAL, "rows_per_position"),
    (dict(rows=-1), fp4idx.EINVAL, "T must be"),
    (dict(D=256), fp4idx.EUNSUPPORTED, "head_dim"),
    (dict(rope_offset=8), fp4idx.EUNSUPPORTED, "rope_offset"),
    (dict(scale_floor=float("nan")), fp4idx.EINVAL, "scale_floor"),
    (dict(x=ALIGNED + 4), fp4idx.EINVAL, "x must be 16-byte"),
    (dict(y=None), fp4idx.EINVAL, "y must not be NULL"),
    (dict(positions=None), fp4idx.EINVAL, "positions must not be NULL"),
]


@pytest.mark.parametrize("over,code,msg", FQUANT_REJECT)
def test_fake_quant_rejections(over, code, msg):
    assert fq8_call(**over) == code
    assert msg in fp4idx.last_error(), fp4idx.last_error()
    assert fp4idx.last_error().startswith("fp4idx_rope_fake_quant:")


def test_zero_tokens_is_a_noop_even_with_null_buffers():
    assert q_call(T=0, q=None, positions=None, cos_sin=None, q_out=None, q_scale_out=None) == 0
    assert k_call(T=0, k=None, positions=None, cos_sin=None, slot_mapping=None, kv_cache=None,
                  kv_cache_scale=None) == 0
    assert d_call(rows=0, packed=None, scales=None, out=None) == 0
    assert qk_call(T=0, q=None, k=None, positions=None, cos_sin=None, slot_mapping=None,
                   q_out=None, q_scale_out=None, kv_cache=None, kv_cache_scale=None) == 0
    assert s_call(B=0, q_out=None, logits=None, block_table=None) == 0
    assert sq_call(T=0, q=None, positions=None, cos_sin=None, q_packed=None) == 0
    assert fq_call(T=0, q=None, positions=None, cos_sin=None, weights=None, q_out=None,
                   weights_out=None) == 0
    assert fk_call(T=0, k=None, positions=None, cos_sin=None, slot_mapping=None, kv_cache=None,
                   kv_cache_scale=None) == 0
    assert fq8_call(rows=0, x=None, positions=None, cos_sin=None, y=None) == 0
    assert sk_call(T=0, k=None, positions=None, cos_sin=None, slot_mapping=None,
                   index_k_cache=None) == 0
    # but shapes are still checked first
    assert q_call(T=0, D=64) == fp4idx.EUNSUPPORTED


def test_error_message_is_thread_local():
    import threading

    assert q_call(D=64) == fp4idx.EUNSUPPORTED
    seen = {}

    def other():
        seen["msg"] = fp4idx.last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "head_dim" in fp4idx.last_error()


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fp4idx, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fp4idx, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU or PyTorch fallback"):
        fp4idx.lib()
