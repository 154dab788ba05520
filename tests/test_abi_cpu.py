"""The C ABI library without a GPU: it loads, exports every declared entry
point, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from long_context_decode_landmark_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lowram.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(native.SYMBOLS)


def test_library_loads_and_exports_every_symbol():
    L = native.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert native.abi_version() == 3
    assert native.strerror(-4) == "workspace too small"


def test_peaks_library_loads_and_checks_its_arguments():
    """The benchmark's peak probes live in their own library; argument errors
    return before any HIP call."""
    from long_context_decode_landmark_amd import build as lbuild
    P = ctypes.CDLL(lbuild.PEAKS_LIB)
    P.peaks_read_gbs.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_double)]
    P.peaks_mfma_tfs.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
    v = ctypes.c_double(1.0)
    assert P.peaks_read_gbs(None, 1000, 4, None, ctypes.byref(v)) == -2  # not a multiple of n_wg * 32 KiB
    assert P.peaks_read_gbs(None, 1 << 20, 0, None, ctypes.byref(v)) == -2
    assert P.peaks_mfma_tfs(0, 10, None, ctypes.byref(v)) == -2
    assert P.peaks_mfma_tfs(4, 0, None, ctypes.byref(v)) == -2


def shape(**kw):
    import synth
    return native.make_shape(synth.C0, **kw)


def ws_bytes(**kw):
    return native.workspace_bytes(shape(**kw))


@pytest.mark.parametrize("kw,code", [
    (dict(n_heads_q=7), -2),            # Hq % Hkv
    (dict(prefix_len=4031), -2),        # P % S
    (dict(topk=0), -2),
    (dict(prefix_len=0, window=0), -2),
    (dict(n_resid=5000), -2),           # more residuals than prefix tokens
    (dict(coeff_fmt=3), -2),
    (dict(n_cand=600), -2),             # more candidates than chunks
    (dict(rope_theta=-1.0), -2),
    (dict(head_dim=64), -3),
    (dict(chunk=16, prefix_len=4032, n_cand=252), -3),
    (dict(mlp_hidden=128), -3),
    (dict(rank=96), -3),
    (dict(n_heads_q=64, n_heads_kv=2), -3),   # GQA group above 16
    (dict(coeff_fmt=1), -3),            # int4 needs rank % 128 == 0 (rank 64 here)
    (dict(batch=65536), -3),            # sequences index a grid dimension of at most 65535
    (dict(n_heads_q=65536, n_heads_kv=65536), -3),
    # (sequence, KV head, tile) workgroups of 256 work-items: at most (2^32 - 1) / 256, padded to 8
    (dict(batch=1024, n_heads_q=32, n_heads_kv=16, prefix_len=0, n_cand=0, n_resid=0, window=1025 * 128), -3),
    # the merge: (sequence, query head) workgroups of 512 work-items, at most (2^32 - 1) / 512, padded to 8
    (dict(batch=32769, n_heads_q=256, n_heads_kv=16), -3),
    (dict(n_cand=0, window=0), -2),     # a prefix but no candidate and no window: nothing to attend
])
def test_workspace_bytes_rejects_shapes(kw, code):
    with pytest.raises(native.LowramError) as e:
        ws_bytes(**kw)
    assert e.value.status == code


def test_workspace_bytes_formula():
    import synth
    cfg = synth.C3
    s = native.make_shape(cfg, batch=28)
    heads = 28 * 8
    keff = min(cfg.topk, cfg.n_cand)
    # selection tiles of 16 chunks (4 waves x 32 tokens), window tiles of 128
    # tokens; partial slots reserved per head: 2 per selection tile + 6 (the
    # producer/consumer kernel's 4 per group of >= 2 tiles) and 1 per window tile
    # and, for those producer/consumer slots, one PH row of 256 hidden units
    # per query head
    n_sel = -(-keff // 16)
    n_ph = 2 * n_sel + 6
    n_part = n_ph + -(-cfg.window // 128)
    al = lambda x: (x + 255) // 256 * 256
    want = (al(heads * cfg.n_cand * 4) + al(heads * keff * 4) + al(heads * n_part * 4 * 130 * 4)
            + al(heads * n_ph * 4 * 256 * 4))
    assert native.workspace_bytes(s) == want


class FakeTensor:
    """A stand-in with a device address that is never dereferenced: every
    call below fails argument checks before the library touches HIP."""

    def __init__(self, addr, n=1 << 30):
        self.addr, self.n = addr, n

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def fake_cache(base=0x10000000):
    return {n: FakeTensor(base + 0x1000000 * i) for i, n in enumerate(native.CACHE_FIELDS)
            if n not in ("cand_ids", "coeff_scale", "res_scale")}


def call_step(s, cache, q=FakeTensor(0x7000000000), out=FakeTensor(0x7100000000), ws=None):
    ws = ws or FakeTensor(0x7200000000, n=native.workspace_bytes(s) if s.topk > 0 else 1)
    with pytest.raises(native.LowramError) as e:
        native.decode_step(s, cache, q, out, ws, stream=0)
    return e.value.status


def test_step_rejects_null_pointers():
    s = shape()
    for n in ("coeff", "basis", "landmark", "w1", "res_chunk_desc", "win_k", "win_v"):
        c = fake_cache()
        c[n] = None
        assert call_step(s, c) == -1, n
    assert call_step(s, fake_cache(), q=None) == -1


def test_step_rejects_short_workspace():
    s = shape()
    need = native.workspace_bytes(s)
    assert call_step(s, fake_cache(), ws=FakeTensor(0x7200000000, n=need - 1)) == -4


def test_step_rejects_misalignment():
    s = shape()
    c = fake_cache()
    c["landmark"] = FakeTensor(0x10000008)
    assert call_step(s, c) == -5
    c = fake_cache()
    c["res_idx"] = FakeTensor(0x10000002)
    assert call_step(s, c) == -5


def test_step_rejects_more_partial_states_than_the_merge_combines():
    # a window of 4096 tiles of 128 tokens gives the merge its most partial
    # states per (sequence, KV head), 4096; one token more is refused before
    # any HIP call
    s = shape(prefix_len=0, n_cand=0, n_resid=0, window=4096 * 128 + 1)
    assert call_step(s, fake_cache()) == -3
    assert native.decode_plan(shape(prefix_len=0, n_cand=0, n_resid=0, window=4096 * 128), 256)[
        "partial_slots"] == 4096


def test_shapes_at_the_grid_limits_are_accepted():
    # one below each limit that a rejection test above crosses
    assert ws_bytes(batch=65535) > 0
    assert ws_bytes(batch=1023, n_heads_q=32, n_heads_kv=16, prefix_len=0, n_cand=0, n_resid=0,
                    window=1025 * 128) > 0
    assert ws_bytes(n_cand=0, window=1) > 0
    assert ws_bytes(batch=32767, n_heads_q=256, n_heads_kv=16) > 0
    assert native.dense_workspace_bytes(native.dense_shape(65535, 100, 8, 2)) > 0
    assert native.dense_workspace_bytes(native.dense_shape(1023, 1025 * 2048, 32, 16)) > 0
    assert native.dense_workspace_bytes(native.dense_shape(32767, 100, 256, 16)) > 0


def call_noalloc(s, cache, q=FakeTensor(0x7000000000), out=FakeTensor(0x7100000000)):
    with pytest.raises(native.LowramError) as e:
        native.decode_step_noalloc(s, cache, q, out, stream=0)
    return e.value.status


def test_noalloc_scratch_size_matches_the_header():
    m = re.search(r"#define\s+LOWRAM_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == native.NOALLOC_SCRATCH_BYTES


def test_noalloc_refuses_shapes_past_its_scratch_before_any_hip_call():
    import synth
    big = native.make_shape(synth.C3, batch=9)             # ~70 MB of workspace
    assert native.workspace_bytes(big) > native.NOALLOC_SCRATCH_BYTES
    assert call_noalloc(big, fake_cache()) == -7
    assert "no-allocation scratch" in native.strerror(-7)
    fits = native.make_shape(synth.C3, batch=8)
    assert native.workspace_bytes(fits) <= native.NOALLOC_SCRATCH_BYTES
    # argument errors come first, as for lowram_decode_step
    c = fake_cache()
    c["coeff"] = None
    assert call_noalloc(big, c) == -1
    assert call_noalloc(shape(n_heads_q=7), fake_cache()) == -2
    assert call_noalloc(shape(), fake_cache(), q=FakeTensor(0x7000000008)) == -5


def test_step_requires_int4_scales_and_candidates():
    s = shape(rank=128, coeff_fmt=1)
    assert call_step(s, fake_cache()) == -1          # coeff_scale missing
    s = shape(n_cand=200)
    assert call_step(s, fake_cache()) == -2          # fewer candidates but no cand_ids


def test_dense_rejects():
    with pytest.raises(native.LowramError) as e:
        native.dense_workspace_bytes(native.dense_shape(1, 100, 7, 2))
    assert e.value.status == -2
    for bad in (native.dense_shape(65536, 100, 8, 2),          # grid dimension limit
                native.dense_shape(1024, 1025 * 2048, 32, 16),   # over (2^32 - 1) / 256 workgroups
                native.dense_shape(32769, 100, 256, 16)):        # merge: over (2^32 - 1) / 512 workgroups
        with pytest.raises(native.LowramError) as e:
            native.dense_workspace_bytes(bad)
        assert e.value.status == -3
    s = native.dense_shape(1, 100, 8, 2)
    need = native.dense_workspace_bytes(s)
    with pytest.raises(native.LowramError) as e:
        native.dense_decode_step(s, FakeTensor(0x1000), FakeTensor(0x2000), FakeTensor(0x3000),
                                 FakeTensor(0x4000), FakeTensor(0x5000, n=need - 1), stream=0)
    assert e.value.status == -4


def test_build_shapes_at_the_grid_limits_are_accepted():
    assert native.build_layer_workspace_bytes(bshape(batch=32767)) > 0     # 65534 lists
    assert native.build_layer_workspace_bytes(bshape(n_heads_kv=8, ctx_len=(1 << 28) - 1024, window=0,
                                                     n_resid=0)) > 0


def test_chunk_desc_rejects():
    with pytest.raises(native.LowramError) as e:
        native.resid_chunk_desc(FakeTensor(0x1002), 4, 16, 10, 8, FakeTensor(0x2000), stream=0)
    assert e.value.status == -5
    with pytest.raises(native.LowramError) as e:
        native.resid_chunk_desc(FakeTensor(0x1000), 4, 16, 10, 16, FakeTensor(0x2000), stream=0)
    assert e.value.status == -3
    with pytest.raises(native.LowramError) as e:      # lists index a grid dimension of at most 65535
        native.resid_chunk_desc(FakeTensor(0x1000), 65536, 16, 10, 8, FakeTensor(0x2000), stream=0)
    assert e.value.status == -3


# ---------------------------------------------------------- cache builder --
def bshape(**kw):
    import synth
    return native.make_build_shape(synth.C0, **kw)


@pytest.mark.parametrize("kw,code", [
    (dict(window=5000), -2),            # W > T
    (dict(window=63), -2),              # P % S
    (dict(n_resid=5000), -2),           # more residuals than prefix tokens
    (dict(resid_fmt=2), -2),
    (dict(rope_theta=0.0), -2),
    (dict(group_layers=0), -2),
    (dict(head_dim=64), -3),
    (dict(chunk=16), -3),
    (dict(rank=96), -3),
    (dict(mlp_hidden=512), -3),
    (dict(coeff_fmt=1), -3),            # int4 coefficients need rank % 128 == 0
    (dict(batch=65536), -3),            # sequences index a grid dimension of at most 65535
    (dict(batch=32768), -3),            # (sequence, KV head) lists index one of at most 65535
    # 128-token prediction tiles of (sequence, KV head): at most (2^32 - 1) / 256 workgroups
    (dict(n_heads_kv=8, ctx_len=1 << 28, window=0, n_resid=0), -3),
])
def test_build_workspace_rejects_shapes(kw, code):
    with pytest.raises(native.LowramError) as e:
        native.build_layer_workspace_bytes(bshape(**kw))
    assert e.value.status == code


def test_build_workspace_formula():
    import synth
    cfg = synth.C3
    s = native.make_build_shape(cfg, batch=2)
    heads, P = 2 * cfg.n_heads_kv, cfg.prefix
    r_bytes = -(-heads * P * 128 * 4 // 256) * 256
    sel_bytes = -(-(heads * 4096 + heads * 4 + heads * -(-P // 8192) * 2) * 4 // 256) * 256
    assert native.build_layer_workspace_bytes(s) == r_bytes + -(-heads * P * 4 // 256) * 256 + sel_bytes
    assert native.build_layer_workspace_bytes(bshape(window=4096, n_resid=0)) == 0   # no prefix


def build_io(**over):
    io = {n: FakeTensor(0x7000000000 + 0x1000000 * i) for i, n in enumerate(native.BUILD_FIELDS)}
    io.update(over)
    return io


def call_build(s, io, layer=0, ws=None):
    ws = ws or FakeTensor(0x7f00000000, n=native.build_layer_workspace_bytes(s))
    with pytest.raises(native.LowramError) as e:
        native.build_layer(s, layer, io, ws, stream=0)
    return e.value.status


def test_build_layer_rejects():
    s = bshape()
    for n in ("keys", "group_basis", "basis", "coeff", "w1", "values", "landmark", "res_idx", "res_val",
              "res_chunk_desc", "win_k"):
        assert call_build(s, build_io(**{n: None})) == -1, n
    assert call_build(s, build_io(), layer=2) == -2              # C0 has 2 layers per group
    assert call_build(s, build_io(landmark=FakeTensor(0x10000008))) == -5
    need = native.build_layer_workspace_bytes(s)
    assert call_build(s, build_io(), ws=FakeTensor(0x7f00000000, n=need - 1)) == -4
    s4 = bshape(rank=128, coeff_fmt=1, resid_fmt=1)
    assert call_build(s4, build_io(coeff_scale=None)) == -1
    assert call_build(s4, build_io(res_scale=None)) == -1


def test_build_coeff_rejects():
    with pytest.raises(native.LowramError) as e:
        native.build_coeff(bshape(), FakeTensor(0x1000), None, FakeTensor(0x3000), stream=0)
    assert e.value.status == -1
    with pytest.raises(native.LowramError) as e:
        native.build_coeff(bshape(), FakeTensor(0x1008), FakeTensor(0x2000), FakeTensor(0x3000), stream=0)
    assert e.value.status == -5
    with pytest.raises(native.LowramError) as e:
        native.build_coeff(bshape(rank=128, coeff_fmt=1), FakeTensor(0x1000), FakeTensor(0x2000),
                           FakeTensor(0x3000), stream=0)
    assert e.value.status == -1                                   # int4 scales missing


# ------------------------------------------------------ capacities / rollover --
@pytest.mark.parametrize("kw,code", [
    (dict(prefix_cap=4000), -2),        # below prefix_len
    (dict(prefix_cap=4036), -2),        # not a multiple of S
    (dict(window_cap=10), -2),          # below window
    (dict(prefix_cap=-8), -2),
])
def test_caps_rejected(kw, code):
    with pytest.raises(native.LowramError) as e:
        ws_bytes(**kw)
    assert e.value.status == code


def test_caps_with_eviction_rejected():
    s = shape(n_cand=200, prefix_cap=4040)
    c = fake_cache()
    c["cand_ids"] = FakeTensor(0x7300000000)
    assert call_step(s, c) == -2


def test_append_rejects():
    s = shape(prefix_cap=4040, n_resid=600)
    io = {n: FakeTensor(0x7400000000 + 0x100000 * i) for i, n in enumerate(native.APPEND_FIELDS)}
    def status(fn):
        with pytest.raises(native.LowramError) as e:
            fn()
        return e.value.status
    assert status(lambda: native.append_layer(s, 2, 0, fake_cache(), dict(io, res_thresh=None), stream=0)) == -1
    assert status(lambda: native.append_layer(s, 2, 2, fake_cache(), io, stream=0)) == -2       # layer >= G
    assert status(lambda: native.append_layer(shape(prefix_cap=4032, n_resid=600), 2, 0, fake_cache(), io,
                                              stream=0)) == -2                                   # no room
    assert status(lambda: native.append_layer(shape(prefix_cap=0), 2, 0, fake_cache(), io, stream=0)) == -2
    assert status(lambda: native.append_layer(shape(prefix_cap=4040, window=4, prefix_len=4032), 2, 0,
                                              fake_cache(), io, stream=0)) == -2                 # window < S
    assert status(lambda: native.append_coeff(s, 2, FakeTensor(0x1008), FakeTensor(0x2000), FakeTensor(0x3000),
                                              stream=0)) == -5
    assert status(lambda: native.append_coeff(s, 0, FakeTensor(0x1000), FakeTensor(0x2000), FakeTensor(0x3000),
                                              stream=0)) == -2


@pytest.mark.parametrize("kw,code", [
    (dict(prefix_cap=4000), -2), (dict(window_cap=10), -2), (dict(resid_cap=100), -2),
])
def test_build_caps_rejected(kw, code):
    with pytest.raises(native.LowramError) as e:
        native.build_layer_workspace_bytes(bshape(**kw))
    assert e.value.status == code


def test_fit_basis_rejects():
    def st(s):
        with pytest.raises(native.LowramError) as e:
            native.fit_basis_workspace_bytes(s)
        return e.value.status
    assert st(native.fit_shape(1, 4096, 4000, 512, 64)) == -3      # P not a multiple of 64
    assert st(native.fit_shape(65536, 4096, 4096, 512, 64)) == -3  # a grid dimension of at most 65535
    assert st(native.fit_shape(1, 64, 64, 1 << 20, 64)) == -3      # 64-column key blocks in such a dimension
    assert native.fit_basis_workspace_bytes(native.fit_shape(1, 64, 64, (1 << 20) - 128, 64)) > 0
    assert st(native.fit_shape(1, 4096, 4032, 500, 64)) == -3      # D not a multiple of 128
    assert st(native.fit_shape(1, 4096, 4032, 512, 96)) == -3      # rank
    assert st(native.fit_shape(1, 4096, 8192, 512, 64)) == -2      # P > T
    assert st(native.fit_shape(1, 4096, 4032, 512, 64, power=-1)) == -2
    s = native.fit_shape(1, 4096, 4032, 512, 64)
    need = native.fit_basis_workspace_bytes(s)
    with pytest.raises(native.LowramError) as e:
        native.fit_basis(s, FakeTensor(0x1000), FakeTensor(0x2000), FakeTensor(0x3000), FakeTensor(0x4000),
                         FakeTensor(0x5000, n=need - 1), stream=0)
    assert e.value.status == -4
