"""Host-side checks of the libdash C ABI: the library loads, exports every function the header
declares, and rejects bad arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dash.h")


@pytest.fixture(scope="module")
def L():
    import sparse_hierarchical_attention_amd as d
    if not os.path.exists(d.library_path):
        from sparse_hierarchical_attention_amd import build
        build.build()
    return d.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dash_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_stages():
    names = declared_functions()
    for fn in ("dash_pool_keys", "dash_block_entmax", "dash_sparse_attn_prefill",
               "dash_sparse_attn_decode"):
        assert fn in names


def test_every_declared_symbol_is_exported(L):
    missing = [fn for fn in declared_functions() if not hasattr(L, fn)]
    assert not missing, missing


def test_status_strings(L):
    for code, name in enumerate(["DASH_OK", "DASH_ERR_INVALID", "DASH_ERR_UNSUPPORTED",
                                 "DASH_ERR_WORKSPACE", "DASH_ERR_HIP"]):
        assert L.dash_status_string(code).decode() == name


def err(L):
    return L.dash_last_error().decode()


def test_pool_rejects_bad_shapes(L):
    assert L.dash_pool_keys(None, 1, None, 1, 64, 2, 96, 64, None) == 2
    assert "head_dim" in err(L)
    assert L.dash_pool_keys(None, 1, None, 1, 64, 2, 128, 48, None) == 2
    assert "block" in err(L)
    assert L.dash_pool_keys(None, 1, None, 0, 64, 2, 128, 64, None) == 1
    assert L.dash_pool_keys(None, 7, None, 1, 64, 2, 128, 64, None) == 1
    assert L.dash_pool_keys(None, 1, None, 1, 64, 2, 128, 64, None) == 1  # null pointers
    assert "null" in err(L)


def test_block_entmax_rejects_bad_arguments(L):
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails before any launch
    args = dict(q=p, dt=1, kbar=p, batch=1, n_q=64, q_pos0=0, n_kv=64, h_q=4, h_kv=2, d=128,
                block=64, alpha=1.5, gamma=1.0, sigma=1.0, mask=p, bias=p, tau=None, ws=p,
                wsb=1 << 40, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return L.dash_block_entmax(*a.values())

    assert call(alpha=1.0) == 1 and "alpha" in err(L)
    assert call(alpha=2.5) == 1
    assert call(gamma=0.0) == 1 and "gamma" in err(L)
    assert call(sigma=0.0) == 1 and "sigma" in err(L)
    assert call(sigma=-1.0) == 1
    assert call(h_q=5) == 1 and "multiple" in err(L)
    assert call(h_q=64, h_kv=2) == 2 and "group" in err(L)
    assert call(q_pos0=1) == 1 and "q_pos0" in err(L)
    assert call(mask=None) == 1 and "null" in err(L)
    need = L.dash_block_entmax_workspace_bytes(1, 1, 64, 0, 64, 4, 2, 128, 64)
    assert need == 1 * 2 * 32 * 3 * 128 * 2  # bf16 prefill: a tile of 32 summaries, three bf16 terms
    assert L.dash_block_entmax_workspace_bytes(1, 1, 40, 0, 40, 4, 2, 128, 64) == 0  # no summary
    need = L.dash_block_entmax_workspace_bytes(0, 1, 64, 0, 64, 4, 2, 128, 64)
    assert need == 64 * 4 * 1 * 4  # fp32 scores through the workspace
    assert call(dt=0, wsb=need - 1) == 3 and "workspace" in err(L)
    need = L.dash_block_entmax_workspace_bytes(1, 2, 1, 4095, 4096, 8, 2, 128, 64)
    assert need == 2 * 8 * 64 * 4  # decode scores through the workspace
    # a 256K prefill off the fused path (fp32) scores in slabs of query rows: 512 MiB, not 64 GiB
    assert L.dash_block_entmax_workspace_bytes(0, 1, 262144, 0, 262144, 32, 8, 128, 128) == 512 << 20
    # in bf16 its 2048-chunk rows stay on chip; the workspace holds the split summaries
    assert L.dash_block_entmax_workspace_bytes(1, 1, 262144, 0, 262144, 32, 8, 128, 128) == \
        1 * 8 * 64 * 32 * 3 * 128 * 2
    # past 2048 chunks bf16 leaves the fused path too
    assert L.dash_block_entmax_workspace_bytes(1, 1, 262144, 0, 262144, 32, 8, 128, 64) == 512 << 20


def test_attention_rejects_bad_arguments(L):
    p = ctypes.c_void_p(16)
    assert L.dash_sparse_attn_prefill(p, p, p, 1, p, p, p, None, 1, 64, 4, 2, 128, 64, 0.0, None) == 1
    assert "scale" in err(L)
    assert L.dash_sparse_attn_prefill(p, p, p, 1, p, p, None, None, 1, 64, 4, 2, 128, 64, 0.1, None) == 1
    need = L.dash_decode_workspace_bytes(2, 4096, 8, 2, 128, 64)
    # ticket counters (256 B), then the partial records of up to 128 slots (32 workgroups of
    # four slots at g = 4) for each (sequence, group)
    assert need == 256 + 2 * 2 * 32 * 4 * (128 + 4) * 4
    assert L.dash_sparse_attn_decode(p, p, p, 1, p, p, p, 2, 4096, 8, 2, 128, 64, 0.1, p,
                                     need - 1, None) == 3
    assert L.dash_sparse_attn_decode(p, p, p, 1, p, p, p, 2, 4096, 8, 2, 128, 64, 0.1, None,
                                     0, None) == 3
    assert L.dash_sparse_attn_decode(p, p, p, 1, p, p, p, 2, 4096, 8, 2, 128, 64, 0.0, None,
                                     0, None) == 1 and "scale" in err(L)


def test_empty_calls_are_invalid(L):
    # a zero batch, sequence length or row count is rejected before any launch (no silent no-op)
    p = ctypes.c_void_p(16)
    assert L.dash_sparse_attn_prefill(p, p, p, 1, p, p, p, None, 0, 64, 4, 2, 128, 64, 0.1, None) == 1
    assert "positive" in err(L)
    assert L.dash_sparse_attn_prefill(p, p, p, 1, p, p, p, None, 1, 0, 4, 2, 128, 64, 0.1, None) == 1
    assert L.dash_sparse_attn_prefill_ex(p, p, p, 1, p, p, p, None, 1, 0, 0, 64, 4, 2, 128, 64,
                                         0.1, None) == 1
    assert L.dash_sparse_attn_decode(p, p, p, 1, p, p, p, 0, 4096, 8, 2, 128, 64, 0.1, p,
                                     1 << 30, None) == 1
    assert L.dash_block_entmax(p, 1, p, 1, 0, 0, 64, 4, 2, 128, 64, 1.5, 1.0, 1.0, p, p, None, p,
                               1 << 40, None) == 1
    assert L.dash_pool_keys(p, 1, p, 1, 0, 2, 128, 64, None) == 1


def test_streaming_and_window_entry_points_reject_bad_arguments(L):
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation
    # per-sequence lengths need one query per sequence
    assert L.dash_block_entmax_ex(p, 1, p, p, 2, 2, 0, 4096, 8, 2, 128, 64, 1.5, 1.0, 1.0, 1,
                                  p, p, None, p, 1 << 30, None) == 1 and "n_q = 1" in err(L)
    assert L.dash_block_entmax_ex(p, 1, p, None, 1, 64, 0, 64, 4, 2, 128, 64, 1.5, 1.0, 1.0, 0,
                                  p, p, None, p, 1 << 30, None) == 1 and "window" in err(L)
    assert L.dash_block_entmax_ex(p, 1, p, None, 1, 64, 0, 64, 4, 2, 128, 64, 3.0, 1.0, 1.0, 2,
                                  p, p, None, p, 1 << 30, None) == 1 and "alpha" in err(L)
    assert L.dash_sparse_attn_decode_varlen(p, p, p, 1, None, p, p, p, 2, 4096, 8, 2, 128, 64,
                                            0.1, p, 1 << 20, None) == 1 and "null" in err(L)
    assert L.dash_sparse_attn_decode_varlen(p, p, p, 1, p, p, p, p, 2, 4096, 8, 2, 128, 64,
                                            0.1, None, 0, None) == 3
    assert L.dash_pool_keys_append(p, 1, None, None, p, 2, 4096, 2, 128, 64, None) == 1
    assert L.dash_pool_keys_append(p, 1, None, p, p, 2, 4096, 2, 96, 64, None) == 2


def test_backward_rejects_bad_arguments(L):
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation
    need = L.dash_sparse_attn_backward_workspace_bytes(2, 300, 8)
    assert need == 2 * 300 * 8 * 4
    assert L.dash_sparse_attn_backward_workspace_bytes(0, 300, 8) == 0
    args = [p] * 5 + [1] + [p] * 6
    assert L.dash_sparse_attn_prefill_backward(*args, 2, 300, 8, 2, 128, 32, 0.1, p, need - 1,
                                               None) == 3
    assert L.dash_sparse_attn_prefill_backward(*args, 2, 300, 8, 2, 128, 32, 0.0, p, need,
                                               None) == 1 and "scale" in err(L)
    assert L.dash_sparse_attn_prefill_backward(*args, 2, 300, 8, 3, 128, 32, 0.1, p, need,
                                               None) == 1
    assert L.dash_sparse_attn_prefill_backward(*args, 2, 300, 8, 2, 96, 32, 0.1, p, need,
                                               None) == 2
    nulls = [p] * 4 + [None] + [1] + [p] * 6
    assert L.dash_sparse_attn_prefill_backward(*nulls, 2, 300, 8, 2, 128, 32, 0.1, p, need,
                                               None) == 1 and "null" in err(L)
    # dbias may be NULL: validation passes up to the (absent) workspace
    no_dbias = [p] * 5 + [1] + [p] * 5 + [None]
    assert L.dash_sparse_attn_prefill_backward(*no_dbias, 2, 300, 8, 2, 128, 32, 0.1, None, 0,
                                               None) == 3


def test_learned_query_backward_rejects_bad_arguments(L):
    """dash_block_entmax_backward_query: strides must be non-negative multiples of 4, queries of
    distinct (sequence, chunk) pairs may coincide but not partly overlap, qbar and dqbar are
    16-byte aligned, and the workspace (which includes each chunk's dqbar) is 256-byte aligned."""
    i64 = ctypes.c_int64
    a = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below fails validation
    B, n, hq, hkv, d, blk = 2, 640, 8, 2, 128, 64
    tc = n // blk
    need = L.dash_block_entmax_backward_query_workspace_bytes(B, n, hq, hkv, d, blk)
    assert need == ((B * n * (hq + hkv) * 4 + 255) // 256) * 256 + B * tc * hkv * d * 4

    def call(sb, sc, qbar=a, dqbar=a, ws=a, ws_bytes=need, dt=1):
        return L.dash_block_entmax_backward_query(
            a, a, dt, a, qbar, i64(sb), i64(sc), a, a, a, a, a, dqbar, B, n, hq, hkv, d, blk,
            ctypes.c_float(1.5), ctypes.c_float(1.0), ctypes.c_float(1.0), 1, ws,
            ctypes.c_size_t(ws_bytes), None)

    assert call(-4, 0) == 1 and "strides" in err(L)
    assert call(0, 6) == 1 and "strides" in err(L)
    assert call(hkv * d, 4) == 1 and "overlap" in err(L)      # chunks 4 floats apart
    assert call(4, tc * hkv * d) == 1 and "overlap" in err(L)  # sequences 4 floats apart
    assert call(0, 0, qbar=ctypes.c_void_p((1 << 20) + 4)) == 1 and "aligned" in err(L)
    assert call(0, 0, dqbar=ctypes.c_void_p((1 << 20) + 8)) == 1 and "aligned" in err(L)
    assert call(0, 0, ws_bytes=need - 1) == 3
    assert call(0, 0, ws=ctypes.c_void_p((1 << 20) + 16)) == 1 and "256-byte" in err(L)
    assert call(0, 0, qbar=None) == 1 and "null" in err(L)
    assert call(0, 0, dt=7) == 1


def test_binding_rejects_non_fp32_side_inputs():
    """The binding checks the fp32 operands' dtype before anything reaches the library (a float64
    buffer passed as float * would be read as garbage)."""
    import torch
    import sparse_hierarchical_attention_amd as d
    k = torch.zeros(1, 64, 1, 64)
    with pytest.raises(TypeError, match="qbar"):
        d.dash_pool_keys_query(k, torch.zeros(1, 64, dtype=torch.float64), 64)
    with pytest.raises(TypeError, match="kbar"):
        d.dash_pool_keys(k, 64, kbar=torch.zeros(1, 1, 1, 64, dtype=torch.float64))
