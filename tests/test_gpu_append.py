"""GPU parity of the window rollover (lowram_append_coeff + lowram_append_layer).

A cache is built with capacities (lowram_build_layer), then the oldest
chunk of the window is rolled into the prefix three times.  Against the
oracle (``compress.append_chunk`` after the oracle's build of the same bf16
inputs): each appended chunk's coefficients and landmark within one bf16
step, its residual decisions equal except tokens within SEL_BAND of the
threshold, the residual rows within one step, the counts and descriptors
exact, the window shifted exactly; the build threshold against the oracle's.
The grown cache then decodes like the oracle's grown cache (decode parity
rule), and decoding the capacity layout equals decoding a dense copy bit for
bit.  As in the builder tests, the layer stages read the oracle's stored
coefficients so both sides predict from identical data.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import DEV, check_output, check_selection, down_bf16, up  # noqa: E402
from long_context_decode_landmark_amd import native  # noqa: E402
from oracle import codecs, compress, decode, fixture  # noqa: E402
from test_gpu_builder import close_bf16, close_int4  # noqa: E402

SEL_BAND = 1e-4
N_APP = 3


def host(t):
    t = t.contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.int16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dense_view(t, n):
    """First n rows along axis 2 of a capacity-layout [NB][Hkv][cap][...] array."""
    return t[:, :, :n].contiguous()


@pytest.mark.parametrize("name,cfg,layer", [
    ("c0_b2", synth.C0.with_(name="app_c0", batch=2), 1),
    ("int4_r128", synth.C0.with_(name="app_int4", rank=128, int4=True, resid_frac=0.25), 0),
])
def test_rollover(name, cfg, layer):
    nb, S, P, W, r, hkv, d = cfg.batch, cfg.chunk, cfg.prefix, cfg.window, cfg.rank, cfg.n_heads_kv, cfg.head_dim
    nR, G, lig = cfg.n_resid, cfg.group_layers, layer % cfg.group_layers
    pcap, wcap, rcap = P + N_APP * S, W, nR + N_APP * S
    inp, exp = fixture.builder_io(cfg, layer)
    bshape = native.make_build_shape(cfg, batch=nb, prefix_cap=pcap, window_cap=wcap, resid_cap=rcap)
    t = {k: up(v) for k, v in inp.items()}
    bf = torch.bfloat16
    c = dict(t)
    if cfg.int4:
        c["coeff"] = torch.zeros((nb, pcap, r // 2), dtype=torch.uint8, device=DEV)
        c["coeff_scale"] = torch.zeros((nb, pcap, r // 32), dtype=torch.int16, device=DEV)
        c["res_val"] = torch.zeros((nb, hkv, rcap, d // 2), dtype=torch.uint8, device=DEV)
        c["res_scale"] = torch.zeros((nb, hkv, rcap, d // 32), dtype=torch.int16, device=DEV)
    else:
        c["coeff"] = torch.zeros((nb, pcap, r), dtype=bf, device=DEV)
        c["res_val"] = torch.zeros((nb, hkv, rcap, d), dtype=bf, device=DEV)
    c["basis"] = torch.zeros((nb, hkv, d, r), dtype=bf, device=DEV)
    c["landmark"] = torch.zeros((nb, hkv, pcap // S, d), dtype=bf, device=DEV)
    c["res_idx"] = torch.full((nb, hkv, rcap), -1, dtype=torch.int32, device=DEV)
    c["res_chunk_desc"] = torch.zeros((nb, hkv, pcap // S), dtype=torch.int32, device=DEV)
    c["win_k"] = torch.zeros((nb, hkv, wcap, d), dtype=bf, device=DEV)
    c["win_v"] = torch.zeros((nb, hkv, wcap, d), dtype=bf, device=DEV)
    c["res_thresh"] = torch.zeros((nb, hkv), dtype=torch.float32, device=DEV)
    c["res_count"] = torch.zeros((nb, hkv), dtype=torch.int32, device=DEV)
    dropped = torch.zeros((nb, hkv), dtype=torch.int32, device=DEV)

    # oracle coefficients of every token the test will compress
    x_all = codecs.bf16_decode(inp["keys"])
    c_or = [compress.store_coeff(compress.project(x_all[b, :pcap], codecs.bf16_decode(inp["group_basis"][b])),
                                 cfg.int4) for b in range(nb)]

    def put_coeff(r0, r1):
        if cfg.int4:
            c["coeff"][:, r0:r1] = up(np.stack([co[0][r0:r1] for co in c_or]))
            c["coeff_scale"][:, r0:r1] = up(np.stack([co[1][r0:r1] for co in c_or]))
        else:
            c["coeff"][:, r0:r1] = up(np.stack([co[r0:r1] for co in c_or])).view(bf)

    def check_coeff(r0, r1, what):
        got = host(c["coeff"][:, r0:r1])
        if cfg.int4:
            close_int4(got, host(c["coeff_scale"][:, r0:r1]), np.stack([co[0][r0:r1] for co in c_or]),
                       np.stack([co[1][r0:r1] for co in c_or]), what, min_exact=0.95)
        else:
            close_bf16(got, np.stack([co[r0:r1] for co in c_or]), what, min_exact=0.95)

    native.build_coeff(bshape, c["keys"], c["group_basis"], c["coeff"], c.get("coeff_scale"))
    torch.cuda.synchronize()
    check_coeff(0, P, "build coefficients")
    put_coeff(0, P)
    ws = torch.empty(native.build_layer_workspace_bytes(bshape), dtype=torch.uint8, device=DEV)
    native.build_layer(bshape, lig, c, ws)
    torch.cuda.synchronize()
    thr_g = host(c["res_thresh"])
    assert np.all(np.abs(thr_g - exp["res_thresh"]) <= 1e-5 * exp["res_thresh"]), (thr_g, exp["res_thresh"])
    assert np.all(host(c["res_count"]) == nR)

    # the capacity layout decodes exactly like a dense copy
    dshape = native.make_shape(cfg, batch=nb, n_resid=rcap, prefix_cap=pcap, window_cap=wcap)
    q = up(np.stack([codecs.bf16_encode(synth.queries(cfg, b, layer)) for b in range(nb)]))
    cache_keys = ("coeff", "coeff_scale", "basis", "landmark", "w1", "b1", "w2", "b2", "res_idx", "res_val",
                  "res_scale", "res_chunk_desc", "win_k", "win_v")
    capc = {k: c[k] for k in cache_keys if k in c}
    dense = dict(capc)
    dense["coeff"] = c["coeff"][:, :P].contiguous()
    if cfg.int4:
        dense["coeff_scale"] = c["coeff_scale"][:, :P].contiguous()
    dense["landmark"] = dense_view(c["landmark"], P // S)
    dense["res_chunk_desc"] = dense_view(c["res_chunk_desc"], P // S)
    ws_d = torch.empty(native.workspace_bytes(dshape), dtype=torch.uint8, device=DEV)
    out_cap, out_dense = torch.empty_like(q), torch.empty_like(q)
    native.decode_step(dshape, capc, q, out_cap, ws_d)
    native.decode_step(native.make_shape(cfg, batch=nb, n_resid=rcap), dense, q, out_dense, ws_d)
    torch.cuda.synchronize()
    assert torch.equal(out_cap.view(torch.int16), out_dense.view(torch.int16))

    # oracle state per (b, h): residual ids and rows (stored), descriptors
    o_idx = {(b, h): list(exp["res_idx"][b, h]) for b in range(nb) for h in range(hkv)}
    o_rows = {(b, h): [exp["res_val"][b, h][i] for i in range(nR)] for b in range(nb) for h in range(hkv)}
    o_scale = {(b, h): [exp["res_scale"][b, h][i] for i in range(nR)] for b in range(nb) for h in range(hkv)} \
        if cfg.int4 else None
    o_lm = {(b, h): list(exp["landmark"][b, h]) for b in range(nb) for h in range(hkv)}
    win0_k, win0_v = host(c["win_k"]).copy(), host(c["win_v"]).copy()
    flips = 0
    for k in range(N_APP):
        P0, W0 = P + k * S, W - k * S
        sh = native.make_shape(cfg, batch=nb, prefix_len=P0, window=W0, n_cand=P0 // S, n_resid=rcap,
                               prefix_cap=pcap, window_cap=wcap)
        keys_new = c["keys"][:, P0:P0 + S].contiguous()
        native.append_coeff(sh, G, keys_new, c["group_basis"], c["coeff"], c.get("coeff_scale"))
        torch.cuda.synchronize()
        check_coeff(P0, P0 + S, f"appended coefficients {k}")
        put_coeff(P0, P0 + S)
        io = dict(keys_new=keys_new, res_thresh=c["res_thresh"], res_count=c["res_count"], res_dropped=dropped,
                  landmark=c["landmark"], res_idx=c["res_idx"], res_val=c["res_val"], res_scale=c.get("res_scale"),
                  res_chunk_desc=c["res_chunk_desc"], win_k=c["win_k"], win_v=c["win_v"])
        native.append_layer(sh, G, lig, capc, io)
        torch.cuda.synchronize()
        g_idx, g_cnt = host(c["res_idx"]), host(c["res_count"])
        g_desc = host(c["res_chunk_desc"]).view(np.uint32)
        for b in range(nb):
            xb = x_all[b]
            cdec = compress.decode_coeff(tuple(a[P0:P0 + S] for a in c_or[b]) if cfg.int4 else c_or[b][P0:P0 + S],
                                         cfg.int4)
            for h in range(hkv):
                cols = synth.layer_cols(cfg, layer, h)
                w = [codecs.bf16_decode(inp[n][b, h]) for n in ("w1", "b1", "w2", "b2")]
                v_new = codecs.bf16_decode(inp["values"][b, h, P0:P0 + S])
                app = compress.append_chunk(xb[P0:P0 + S, cols], v_new, cdec, codecs.bf16_decode(exp["basis"][b, h]),
                                            *w, exp["res_thresh"][b, h], P0, cfg.rope_theta)
                o_lm[(b, h)].append(codecs.bf16_encode(app["landmark"]))
                before = len(o_idx[(b, h)])
                got_new = [int(t_) for t_ in g_idx[b, h, before:g_cnt[b, h]]]
                want_new = [P0 + int(i) for i in app["keep"]]
                tau = exp["res_thresh"][b, h]
                for t_ in set(got_new) ^ set(want_new):
                    assert abs(app["errors"][t_ - P0] - tau) <= SEL_BAND * tau, (b, h, t_)
                flips += len(set(got_new) ^ set(want_new))
                # descriptor of the new chunk from the GPU's own decisions
                mask = sum(1 << (t_ - P0) for t_ in got_new)
                assert int(g_desc[b, h, P0 // S]) == (before << 8) | mask
                # oracle rows of the kept tokens (stored), for the decode comparison below
                rows = app["rows"]
                if cfg.int4:
                    codes, sc = codecs.int4_encode(rows)
                    o_rows[(b, h)] += list(codes)
                    o_scale[(b, h)] += list(sc)
                else:
                    o_rows[(b, h)] += list(codecs.bf16_encode(rows))
                o_idx[(b, h)] += want_new
                assert got_new == want_new or flips > 0
        assert np.all(host(dropped) == 0)
    # landmarks and residual rows of the appended chunks
    nC = P // S
    g_lm = host(c["landmark"])
    for b in range(nb):
        for h in range(hkv):
            close_bf16(g_lm[b, h, nC:nC + N_APP], np.stack(o_lm[(b, h)][nC:nC + N_APP]), f"landmarks {b} {h}",
                       min_exact=0.9)
            n = g_cnt[b, h]
            if n > nR:
                if cfg.int4:
                    close_int4(host(c["res_val"])[b, h, nR:n], host(c["res_scale"])[b, h, nR:n],
                               np.stack(o_rows[(b, h)][nR:n]), np.stack(o_scale[(b, h)][nR:n]), "appended rows",
                               min_exact=0.9)
                else:
                    close_bf16(host(c["res_val"])[b, h, nR:n], np.stack(o_rows[(b, h)][nR:n]), "appended rows",
                               min_exact=0.9)
    # the window moved down by N_APP chunks
    keep_w = W - N_APP * S
    assert np.array_equal(host(c["win_k"])[:, :, :keep_w], win0_k[:, :, N_APP * S:W])
    assert np.array_equal(host(c["win_v"])[:, :, :keep_w], win0_v[:, :, N_APP * S:W])

    # the grown cache decodes like the oracle's grown cache
    P1, W1 = P + N_APP * S, W - N_APP * S
    cfg1 = cfg.with_(ctx=P1 + W1, window=W1)
    sh1 = native.make_shape(cfg, batch=nb, prefix_len=P1, window=W1, n_cand=P1 // S, n_resid=rcap,
                            prefix_cap=pcap, window_cap=wcap)
    out = torch.empty_like(q)
    sel = torch.full((nb, hkv, cfg.topk), -7, dtype=torch.int32, device=DEV)
    native.decode_step(sh1, capc, q, out, ws_d, sel_out=sel)
    torch.cuda.synchronize()
    counts = [len(o_idx[(b, h)]) for b in range(nb) for h in range(hkv)]
    oc = {
        "coeff": (np.stack([co[0][:P1] for co in c_or]) if cfg.int4 else np.stack([co[:P1] for co in c_or])),
        "basis": exp["basis"], "w1": inp["w1"], "b1": inp["b1"], "w2": inp["w2"], "b2": inp["b2"],
        "landmark": np.stack([np.stack([np.stack(o_lm[(b, h)]) for h in range(hkv)]) for b in range(nb)]),
        "win_k": exp["win_k"][:, :, N_APP * S:W], "win_v": exp["win_v"][:, :, N_APP * S:W],
    }
    if cfg.int4:
        oc["coeff_scale"] = np.stack([co[1][:P1] for co in c_or])
    # residual lists may differ in length per head: the oracle decode reads one head at a time
    sel_h = sel.cpu().numpy()
    got = down_bf16(out)
    g = cfg.gqa
    for b in range(nb):
        for h in range(hkv):
            sl = {k: (v[b:b + 1] if k in ("coeff", "coeff_scale") else v[b:b + 1, h:h + 1]) for k, v in oc.items()}
            sl["res_idx"] = np.asarray(o_idx[(b, h)], np.int32)[None, None]
            sl["res_val"] = np.stack(o_rows[(b, h)])[None, None]
            if cfg.int4:
                sl["res_scale"] = np.stack(o_scale[(b, h)])[None, None]
            cfg_h = cfg1
            qs = decode.widen(host(q)[b, h * g:(h + 1) * g])
            _, st = decode.decode_head(cfg_h, sl, qs, 0, 0)
            check_selection(cfg_h, {(0, 0): st}, sel_h[b:b + 1, h:h + 1], 0, 0)
            ref, _ = decode.decode_head(cfg_h, sl, qs, 0, 0, sel_override=sel_h[b, h])
            check_output(got[b, h * g:(h + 1) * g], ref, f"{name} grown b{b} h{h}")
    print(f"\nrollover {name}: {N_APP} chunks, residual counts {sorted(set(counts))}, flips {flips}", flush=True)
