"""The C-ABI library loads, exports every symbol include/kvarn.h declares, and
rejects bad arguments on the host before anything is queued (no GPU needed)."""
import ctypes
import os
import re

import pytest

from kv_cache_quantization_seal_amd import kvarn as K
from oracle import kvarn_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # never dereferenced: every call below fails validation first


def _declared():
    text = open(os.path.join(ROOT, "include", "kvarn.h")).read()
    return sorted(set(re.findall(r"\b(kvarn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = K.lib()
    names = _declared()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(K.EXPORTS)


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 4), (256, 2), (256, 4)])
def test_record_bytes_match_oracle(d, bits):
    assert K.record_bytes(d, bits) == O.record_bytes(d, bits)


def test_record_bytes_unsupported():
    assert K.record_bytes(96, 2) == 0 and K.record_bytes(128, 7) == 0 and K.record_bytes(128, 1) == 0
    for bits in (3, 5, 6, 8):
        assert K.record_bytes(128, bits) == O.record_bytes(128, bits)


def test_group_and_workspace_bytes():
    cfg = K.make_config(128, 32, 8, 2, 4)
    assert K.group_bytes(cfg) == 4608 + 8704
    ws = K.decode_workspace_bytes(cfg, 1, 255)
    assert ws > 0 and ws % 256 == 0
    assert K.decode_workspace_bytes(cfg, 0, 255) == 0


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, K.EUNSUPPORTED), ("k_bits", 7, K.EUNSUPPORTED), ("v_bits", 1, K.EUNSUPPORTED),
    ("group", 64, K.EUNSUPPORTED), ("sink", 0, K.EUNSUPPORTED), ("num_q_heads", 12, K.EINVAL),
    ("num_q_heads", 64, K.EUNSUPPORTED), ("num_kv_heads", 0, K.EINVAL), ("sinkhorn_iters", -1, K.EINVAL),
])
def test_check_config_rejects(field, value, status):
    cfg = K.make_config(128, 32, 8, 2, 2)
    assert K.check_config(cfg) == K.OK
    setattr(cfg, field, value)
    assert K.check_config(cfg) == status
    assert K.lib().kvarn_last_error().decode() != ""


def _view(batch=2, max_groups=4, **over):
    v = K.CacheView(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, batch, max_groups)
    for k, val in over.items():
        setattr(v, k, val)
    return v


def test_entry_points_validate_before_launch():
    L = K.lib()
    cfg = K.make_config(128, 32, 8, 2, 2)
    r = ctypes.byref
    assert L.kvarn_append(None, r(_view()), FAKE, FAKE, None) == K.EINVAL
    assert L.kvarn_append(r(cfg), None, FAKE, FAKE, None) == K.EINVAL
    assert L.kvarn_append(r(cfg), r(_view()), None, FAKE, None) == K.EINVAL
    assert L.kvarn_append(r(cfg), r(_view(sink_k=None)), FAKE, FAKE, None) == K.EINVAL
    assert L.kvarn_append(r(cfg), r(_view(batch=0)), FAKE, FAKE, None) == K.EINVAL
    assert L.kvarn_append(r(cfg), r(_view(sink_v=FAKE + 2)), FAKE, FAKE, None) == K.EINVAL
    assert L.kvarn_seal_group(r(cfg), r(_view(max_groups=-1)), None, None, 2, None) == K.EINVAL
    bad = K.make_config(96, 32, 8, 2, 2)
    assert L.kvarn_seal_group(r(bad), r(_view()), None, None, 2, None) == K.EUNSUPPORTED
    # Predicate form: n must be the batch; list form: both lists or neither.
    assert L.kvarn_seal_group(r(cfg), r(_view()), None, None, 1, None) == K.EINVAL
    assert L.kvarn_seal_group(r(cfg), r(_view()), FAKE, None, 1, None) == K.EINVAL
    assert L.kvarn_seal_group(r(cfg), r(_view()), None, FAKE, 1, None) == K.EINVAL
    assert L.kvarn_seal_group(r(cfg), r(_view()), FAKE, FAKE, -1, None) == K.EINVAL
    assert L.kvarn_seal_group(r(cfg), r(_view()), FAKE + 2, FAKE, 1, None) == K.EINVAL
    assert L.kvarn_seal_group(r(cfg), r(_view()), FAKE, FAKE, 0, None) == K.OK   # empty list: no launch
    assert L.kvarn_seal_group(r(cfg), r(_view()), None, None, 0, None) == K.OK
    ws = K.decode_workspace_bytes(cfg, 2, 4)
    assert L.kvarn_decode_attn(r(cfg), r(_view()), FAKE, FAKE, 0.1, FAKE, ws - 1, None) == K.EWORKSPACE
    assert L.kvarn_decode_attn(r(cfg), r(_view()), FAKE, FAKE, 0.1, None, ws, None) == K.EWORKSPACE
    assert L.kvarn_decode_attn(r(cfg), r(_view()), None, FAKE, 0.1, FAKE, ws, None) == K.EINVAL
    assert L.kvarn_decode_attn(r(cfg), r(_view()), FAKE, FAKE, 0.1, FAKE + 16, ws, None) == K.EINVAL
    assert L.kvarn_decode_attn(r(cfg), r(_view()), FAKE, FAKE, float("nan"), FAKE, ws, None) == K.EINVAL


def test_decode_noalloc_validates_before_launch():
    """The no-alloc decode rejects bad arguments, and a cache whose workspace
    exceeds the library's fixed scratch, before anything is queued."""
    L = K.lib()
    r = ctypes.byref
    cfg = K.make_config(128, 32, 8, 2, 2)
    assert L.kvarn_decode_attn_noalloc(r(cfg), r(_view()), None, FAKE, 0.1, None) == K.EINVAL
    assert L.kvarn_decode_attn_noalloc(r(cfg), r(_view()), FAKE, FAKE + 4, 0.1, None) == K.EINVAL
    assert L.kvarn_decode_attn_noalloc(r(cfg), r(_view()), FAKE, FAKE, float("nan"), None) == K.EINVAL
    big = K.make_config(256, 64, 16, 2, 2)
    assert L.kvarn_decode_attn_noalloc(r(big), r(_view(batch=128, max_groups=1)), FAKE, FAKE, 0.1,
                                       None) == K.EWORKSPACE
    assert "scratch" in L.kvarn_last_error().decode()


def test_prefill_range_checks():
    L = K.lib()
    cfg = K.make_config(128, 8, 2, 2, 2)
    r = ctypes.byref
    cap = 128 + 128 * 4 + 127
    lens = (ctypes.c_int32 * 2)(10, cap + 1)
    assert L.kvarn_prefill(r(cfg), r(_view()), FAKE, FAKE, 4096, lens, None) == K.ERANGE
    assert "capacity" in L.kvarn_last_error().decode()
    lens = (ctypes.c_int32 * 2)(10, 300)
    assert L.kvarn_prefill(r(cfg), r(_view()), FAKE, FAKE, 200, lens, None) == K.ERANGE
    lens = (ctypes.c_int32 * 2)(10, -1)
    assert L.kvarn_prefill(r(cfg), r(_view()), FAKE, FAKE, 200, lens, None) == K.EINVAL
    assert L.kvarn_prefill(r(cfg), r(_view()), FAKE, FAKE, 200, None, None) == K.EINVAL


def test_prefill_layers_validates():
    L = K.lib()
    cfg = K.make_config(128, 8, 2, 2, 2)
    r = ctypes.byref
    views = (K.CacheView * 2)(_view(), _view())
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    lens = (ctypes.c_int32 * 2)(10, 300)
    assert L.kvarn_prefill_layers(r(cfg), views, 0, ptrs, ptrs, 400, lens, None) == K.OK   # no layer: no launch
    assert L.kvarn_prefill_layers(r(cfg), views, -1, ptrs, ptrs, 400, lens, None) == K.EINVAL
    assert L.kvarn_prefill_layers(r(cfg), None, 2, ptrs, ptrs, 400, lens, None) == K.EINVAL
    assert L.kvarn_prefill_layers(r(cfg), views, 2, None, ptrs, 400, lens, None) == K.EINVAL
    bad = (K.CacheView * 2)(_view(), _view(batch=3))
    assert L.kvarn_prefill_layers(r(cfg), bad, 2, ptrs, ptrs, 400, lens, None) == K.EINVAL
    assert "batch and max_groups" in L.kvarn_last_error().decode()
    bad = (K.CacheView * 2)(_view(), _view(max_groups=5))
    assert L.kvarn_prefill_layers(r(cfg), bad, 2, ptrs, ptrs, 400, lens, None) == K.EINVAL
    nullk = (ctypes.c_void_p * 2)(FAKE, None)
    assert L.kvarn_prefill_layers(r(cfg), views, 2, nullk, ptrs, 400, lens, None) == K.EINVAL
    big = (ctypes.c_int32 * 2)(10, 128 + 128 * 4 + 128)
    assert L.kvarn_prefill_layers(r(cfg), views, 2, ptrs, ptrs, 4096, big, None) == K.ERANGE


def test_prefill_attn_validates():
    L = K.lib()
    cfg = K.make_config(128, 8, 2, 2, 2)
    r = ctypes.byref
    assert L.kvarn_prefill_attn(r(cfg), r(_view()), FAKE, 0, FAKE, 0.1, None) == K.OK   # empty chunk: no launch
    assert L.kvarn_prefill_attn(r(cfg), r(_view()), FAKE, -1, FAKE, 0.1, None) == K.EINVAL
    assert L.kvarn_prefill_attn(r(cfg), r(_view()), None, 4, FAKE, 0.1, None) == K.EINVAL
    assert L.kvarn_prefill_attn(r(cfg), r(_view()), FAKE, 4, FAKE + 8, 0.1, None) == K.EINVAL
    assert L.kvarn_prefill_attn(r(cfg), r(_view()), FAKE, 4, FAKE, float("nan"), None) == K.EINVAL
    assert L.kvarn_prefill_attn(r(cfg), r(_view(max_groups=1)), FAKE, 384, FAKE, 0.1, None) == K.ERANGE


def test_tile_entry_points_validate():
    L = K.lib()
    assert L.kvarn_seal_tiles(64, 2, 0, 16, FAKE, FAKE, 4608, None, 1, None) == K.EUNSUPPORTED
    assert L.kvarn_seal_tiles(128, 7, 0, 16, FAKE, FAKE, 4608, None, 1, None) == K.EUNSUPPORTED
    assert L.kvarn_seal_tiles(128, 2, 2, 16, FAKE, FAKE, 4608, None, 1, None) == K.EINVAL
    assert L.kvarn_seal_tiles(128, 2, 0, 16, FAKE, FAKE, 4600, None, 1, None) == K.EINVAL
    assert L.kvarn_seal_tiles(128, 2, 0, 99, FAKE, FAKE, 4608, None, 1, None) == K.EINVAL
    assert L.kvarn_seal_tiles(128, 2, 0, 16, None, FAKE, 4608, None, 1, None) == K.EINVAL
    assert L.kvarn_seal_tiles(128, 2, 0, 16, FAKE, FAKE, 4608, None, 0, None) == K.OK
    assert L.kvarn_dequant_records(128, 2, 1, FAKE, 100, FAKE, 1, None) == K.EINVAL
    assert L.kvarn_dequant_records(256, 4, 0, FAKE, 17152, FAKE, -1, None) == K.EINVAL


def test_status_strings():
    L = K.lib()
    assert L.kvarn_status_string(K.EWORKSPACE) == b"KVARN_EWORKSPACE"


def test_append_seal_validates_before_launch():
    L = K.lib()
    cfg = K.make_config(128, 32, 8, 2, 2)
    r = ctypes.byref
    assert L.kvarn_append_seal(None, r(_view()), FAKE, FAKE, None) == K.EINVAL
    assert L.kvarn_append_seal(r(cfg), None, FAKE, FAKE, None) == K.EINVAL
    assert L.kvarn_append_seal(r(cfg), r(_view()), FAKE, None, None) == K.EINVAL
    assert L.kvarn_append_seal(r(cfg), r(_view()), FAKE + 8, FAKE, None) == K.EINVAL
    assert L.kvarn_append_seal(r(cfg), r(_view(tail_v=None)), FAKE, FAKE, None) == K.EINVAL
    # The per-request arrival count shares seq_len with lengths below 2^23.
    assert L.kvarn_append_seal(r(cfg), r(_view(max_groups=(1 << 23) // 128)), FAKE, FAKE, None) == K.ERANGE
    assert "2^23" in L.kvarn_last_error().decode()


@pytest.mark.parametrize("kb", [2, 3, 4, 5, 6, 8])
def test_every_width_pair_is_supported(kb):
    for vb in (2, 3, 4, 5, 6, 8):
        assert K.check_config(K.make_config(128, 8, 2, kb, vb)) == K.OK
        assert K.check_config(K.make_config(256, 8, 2, kb, vb)) == K.OK
    for vb in (1, 7, 9):
        assert K.check_config(K.make_config(128, 8, 2, kb, vb)) == K.EUNSUPPORTED


def test_paged_view_validates_before_launch():
    """A block table needs a positive block count and 4-byte alignment."""
    L = K.lib()
    cfg = K.make_config(128, 32, 8, 2, 2)
    r = ctypes.byref
    field_names = [f[0] for f in K.CacheView._fields_]
    assert field_names[-2:] == ["block_table", "num_blocks"]
    assert L.kvarn_seal_group(r(cfg), r(_view(block_table=FAKE, num_blocks=0)), None, None, 2, None) == K.EINVAL
    assert L.kvarn_append_seal(r(cfg), r(_view(block_table=FAKE + 2, num_blocks=8)), FAKE, FAKE, None) == K.EINVAL
    ws = K.decode_workspace_bytes(cfg, 2, 4)
    assert L.kvarn_decode_attn(r(cfg), r(_view(block_table=FAKE, num_blocks=-1)), FAKE, FAKE, 0.1, FAKE, ws,
                               None) == K.EINVAL


def test_read_probe_validates():
    """The read probe (its own library, not the KVarN ABI) rejects bad
    arguments before anything is queued."""
    from kv_cache_quantization_seal_amd import probe
    L = probe.lib()
    assert L.kvarn_probe_read(FAKE, 0, FAKE, None) == 0   # nothing to read: no launch
    assert L.kvarn_probe_read(None, 16, FAKE, None) == -1
    assert L.kvarn_probe_read(FAKE, 16, None, None) == -1
    assert L.kvarn_probe_read(FAKE, 24, FAKE, None) == -1
    assert L.kvarn_probe_read(FAKE + 8, 16, FAKE, None) == -1
    assert L.kvarn_probe_read(FAKE, 16, FAKE + 2, None) == -1
    assert "kvarn_probe_read" not in K.EXPORTS
