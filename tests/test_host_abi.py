"""The C-ABI library on the host: every symbol include/pie.h declares is
exported, and a host-only context (no weights, no GPU) keeps working sets, the
page pool and the batch packer exactly as the working-set rules state
("How Pie thinks", section 4 Working sets; section 3 ForwardPass): fork
shares frozen pages without copying, a shared page is never written again,
uncommitted tokens are not inherited, and a call that fails changes nothing.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import synth
from paged_kv_forward_amd import _native as N
from paged_kv_forward_amd.runtime import Pass, PieRuntime, model_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 16


def header_functions():
    text = open(os.path.join(ROOT, "include", "pie.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pie_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 16
    L = N.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(N.EXPORTS) == names


def test_sizes():
    d = model_desc(synth.TINY)
    t = synth.TINY
    assert N.lib().pie_kv_page_bytes(ctypes.byref(d)) == t.n_layers * 2 * t.n_kv_heads * P * t.head_dim * 2
    lim = N.pie_limits(256, 8, 8, 1024)
    assert N.lib().pie_workspace_bytes(ctypes.byref(d), ctypes.byref(lim)) > 0
    bad = model_desc(synth.TINY)
    bad.head_dim = 96
    assert N.lib().pie_kv_page_bytes(ctypes.byref(bad)) == 0
    bad = model_desc(synth.TINY)
    bad.n_q_heads = 3
    assert N.lib().pie_workspace_bytes(ctypes.byref(bad), ctypes.byref(lim)) == 0
    assert N.lib().pie_workspace_bytes(ctypes.byref(d), ctypes.byref(N.pie_limits(0, 8, 8, 1024))) == 0


def host_rt(pages=64, max_rows=256, max_seqs=8, max_readout=8, max_ctx=1024):
    page_bytes = N.lib().pie_kv_page_bytes(ctypes.byref(model_desc(synth.TINY)))
    return PieRuntime(synth.TINY, None, pages * page_bytes, max_rows=max_rows, max_seqs=max_seqs,
                      max_readout=max_readout, max_ctx=max_ctx)


def toks(n, base=1):
    return [(base + i) % synth.TINY.vocab for i in range(n)]


def fwd(rt, passes):
    return rt.forward(passes, flags=N.PIE_FLAG_NO_LAUNCH)


def snapshot(rt, handles):
    return ([(rt.ws_info(h)["len"], rt.ws_info(h)["frozen_len"], tuple(rt.ws_info(h)["pages"]))
             for h in handles], rt.pool_stats())


def test_fp8_weight_sizes_and_argument_checks():
    """Sizes of the block-scaled FP8 copies (tiled codes padded to 64 x 64
    blocks, one scale per 128 x 128 block) and the calls' argument checks,
    none of which needs a GPU."""
    L = N.lib()
    assert L.pie_packed_weight_fp8_bytes(100, 70) == 128 * 128
    assert L.pie_packed_weight_fp8_bytes(4096, 4096) == 4096 * 4096
    assert L.pie_packed_weight_fp8_bytes(0, 64) == 0
    assert L.pie_fp8_scale_count(300, 200) == 3 * 2
    assert L.pie_fp8_scale_count(128, 128) == 1
    assert L.pie_fp8_scale_count(-1, 128) == 0
    assert L.pie_pack_weight_fp8(None, ctypes.c_void_p(16), ctypes.c_void_p(16), 64, 64, None) == N.PIE_EINVAL
    assert L.pie_pack_weight_fp8(ctypes.c_void_p(16), ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21),
                                 0, 64, None) == N.PIE_EINVAL
    # codes overlapping the source
    assert L.pie_pack_weight_fp8(ctypes.c_void_p(1 << 20), ctypes.c_void_p((1 << 20) + 64),
                                 ctypes.c_void_p(1 << 24), 64, 64, None) == N.PIE_EINVAL
    rt = PieRuntime(synth.TINY, None, 64 * 1024 * 1024, 128, 4, 8, 256)
    assert L.pie_attach_fp8_weights(rt.ctx, None) == N.PIE_EINVAL
    empty = N.pie_fp8_weights()  # null arrays
    assert L.pie_attach_fp8_weights(rt.ctx, ctypes.byref(empty)) == N.PIE_EINVAL
    assert L.pie_attach_fp8_weights(None, ctypes.byref(empty)) == N.PIE_EINVAL
    rt.close()


def test_profile_repeat_argument_checks():
    """pie_profile_repeat takes 1..64 back-to-back runs; anything else is
    PIE_EINVAL and leaves the setting as it was."""
    L = N.lib()
    rt = PieRuntime(synth.TINY, None, 64 * 1024 * 1024, 128, 4, 8, 256)
    assert L.pie_profile_repeat(rt.ctx, 0) == N.PIE_EINVAL
    assert L.pie_profile_repeat(rt.ctx, 65) == N.PIE_EINVAL
    assert L.pie_profile_repeat(rt.ctx, -3) == N.PIE_EINVAL
    assert L.pie_profile_repeat(None, 4) == N.PIE_EINVAL
    assert L.pie_profile_repeat(rt.ctx, 1) == N.PIE_OK
    assert L.pie_profile_repeat(rt.ctx, 64) == N.PIE_OK
    rt.close()


def test_fork_shares_frozen_pages_and_never_writes_them():
    rt = host_rt(pages=32)
    a = rt.alloc()
    fwd(rt, [Pass(a, toks(40))])
    ia = rt.ws_info(a)
    assert ia["len"] == 40 and ia["frozen_len"] == 40 and len(ia["pages"]) == 3
    free0 = rt.pool_stats()["pages_free"]
    b = rt.fork(a)
    ib = rt.ws_info(b)
    assert ib["len"] == 40 and ib["frozen_len"] == 40
    assert list(ib["pages"]) == list(ia["pages"])
    assert rt.pool_stats()["pages_free"] == free0  # fork takes no page
    # the last shared page holds 8 tokens: both sides append into fresh pages
    fwd(rt, [Pass(b, toks(5)), Pass(a, toks(3))])
    pl = rt.plan()
    shared = set(ia["pages"])
    assert not (set(pl["slot"] // P) & shared)
    ib, ia2 = rt.ws_info(b), rt.ws_info(a)
    assert len(ib["pages"]) == 4 and len(ia2["pages"]) == 4
    assert ib["pages"][3] != ia2["pages"][3]
    assert rt.pool_stats()["pages_free"] == free0 - 2
    rt.free(a)
    assert rt.pool_stats()["pages_free"] == free0 - 1  # only a's private page returns
    rt.free(b)
    st = rt.pool_stats()
    assert st["pages_free"] == st["pages_total"] and st["kv_bytes_copied"] == 0
    assert st["pages_ever_allocated"] == 5
    rt.close()


def test_uncommitted_tokens_not_inherited_and_truncate():
    rt = host_rt(pages=32)
    a = rt.alloc()
    fwd(rt, [Pass(a, toks(20))])
    fwd(rt, [Pass(a, toks(13), commit=False)])
    ia = rt.ws_info(a)
    assert ia["len"] == 33 and ia["frozen_len"] == 20 and len(ia["pages"]) == 3
    c = rt.fork(a)
    ic = rt.ws_info(c)
    assert ic["len"] == 20 and ic["frozen_len"] == 20 and list(ic["pages"]) == list(ia["pages"][:2])
    with pytest.raises(N.PieError) as e:
        rt.truncate(a, 19)
    assert e.value.code == N.PIE_EINVAL
    with pytest.raises(N.PieError):
        rt.truncate(a, 34)
    free = rt.pool_stats()["pages_free"]
    rt.truncate(a, 20)
    ia = rt.ws_info(a)
    assert ia["len"] == 20 and len(ia["pages"]) == 2
    assert rt.pool_stats()["pages_free"] == free + 1
    # a's last page is now shared with c (refcount 2): a's next token opens a fresh page
    fwd(rt, [Pass(a, toks(1))])
    assert len(rt.ws_info(a)["pages"]) == 3
    rt.close()


def test_stale_handles_rejected():
    rt = host_rt()
    a = rt.alloc()
    rt.free(a)
    b = rt.alloc()  # reuses the slot with a new generation
    assert b != a
    for call in (lambda: rt.free(a), lambda: rt.fork(a), lambda: rt.truncate(a, 0),
                 lambda: rt.ws_info(a), lambda: fwd(rt, [Pass(a, toks(1))])):
        with pytest.raises(N.PieError) as e:
            call()
        assert e.value.code == N.PIE_EINVAL
    h = ctypes.c_uint64()
    assert N.lib().pie_fork(rt.ctx, 0, ctypes.byref(h)) == N.PIE_EINVAL
    rt.close()


def test_enomem_is_all_or_nothing():
    rt = host_rt(pages=10)
    a, b = rt.alloc(), rt.alloc()
    fwd(rt, [Pass(a, toks(9))])
    before = snapshot(rt, [a, b])
    with pytest.raises(N.PieError) as e:
        fwd(rt, [Pass(a, toks(20)), Pass(b, toks(9 * P))])  # 2 + 9 pages > 9 free
    assert e.value.code == N.PIE_ENOMEM
    assert snapshot(rt, [a, b]) == before
    fwd(rt, [Pass(a, toks(7)), Pass(b, toks(8 * P))])  # exactly fits: 0 + 8 pages, 1 left
    assert rt.pool_stats()["pages_free"] == 1
    rt.close()


@pytest.mark.parametrize("case", [
    "no_passes", "dup", "no_tokens", "tok_high", "tok_neg", "pos_neg", "ro_high", "ro_neg",
    "temp0", "temp_nan", "temp_inf", "kind", "max_ctx", "max_rows", "max_seqs", "max_readout"])
def test_invalid_batches_change_nothing(case):
    rt = host_rt(max_rows=80, max_seqs=3, max_readout=4, max_ctx=100)
    a, b, c, d = rt.alloc(), rt.alloc(), rt.alloc(), rt.alloc()
    fwd(rt, [Pass(a, toks(30))])
    before = snapshot(rt, [a, b, c, d])
    V = synth.TINY.vocab
    ok = Pass(b, toks(4), [3], [(0, 1.0, 0)])
    bad = {
        "no_passes": ([], N.PIE_EINVAL),
        "dup": ([ok, Pass(a, toks(1)), Pass(a, toks(1))], N.PIE_EINVAL),
        "no_tokens": ([ok, Pass(a, [])], N.PIE_EINVAL),
        "tok_high": ([ok, Pass(a, [1, V])], N.PIE_EINVAL),
        "tok_neg": ([ok, Pass(a, [-1])], N.PIE_EINVAL),
        "pos_neg": ([ok, Pass(a, [1, 2], positions=[5, -1])], N.PIE_EINVAL),
        "ro_high": ([ok, Pass(a, toks(2), [2], [(0, 1.0, 0)])], N.PIE_EINVAL),
        "ro_neg": ([ok, Pass(a, toks(2), [-1], [(0, 1.0, 0)])], N.PIE_EINVAL),
        "temp0": ([ok, Pass(a, toks(2), [1], [(1, 0.0, 5)])], N.PIE_EINVAL),
        "temp_nan": ([ok, Pass(a, toks(2), [1], [(1, math.nan, 5)])], N.PIE_EINVAL),
        "temp_inf": ([ok, Pass(a, toks(2), [1], [(1, math.inf, 5)])], N.PIE_EINVAL),
        "kind": ([ok, Pass(a, toks(2), [1], [(7, 1.0, 5)])], N.PIE_EINVAL),
        "max_ctx": ([ok, Pass(a, toks(71))], N.PIE_EINVAL),
        "max_rows": ([ok, Pass(c, toks(77))], N.PIE_ENOMEM),
        "max_seqs": ([ok, Pass(a, toks(1)), Pass(c, toks(1)), Pass(d, toks(1))], N.PIE_ENOMEM),
        "max_readout": ([ok, Pass(a, toks(4), [0, 1, 2, 3], [(0, 1.0, 0)] * 4)], N.PIE_ENOMEM),
    }[case]
    with pytest.raises(N.PieError) as e:
        fwd(rt, bad[0])
    assert e.value.code == bad[1], str(e.value)
    assert snapshot(rt, [a, b, c, d]) == before
    fwd(rt, [ok, Pass(a, toks(70))])  # the limits themselves are reachable
    rt.close()


def test_host_only_context_refuses_launch():
    rt = host_rt()
    a = rt.alloc()
    with pytest.raises(N.PieError) as e:
        rt.forward([Pass(a, toks(3))])
    assert e.value.code == N.PIE_ESTATE
    assert rt.ws_info(a)["len"] == 0
    rt.close()


def test_async_decode_refused_without_a_gpu_context():
    """pie_decode_async needs a context with device state; pie_sync of a
    host-only context has nothing to wait for; a null context is refused."""
    import ctypes
    rt = host_rt()
    a = rt.alloc()
    ws = (ctypes.c_uint64 * 1)(a)
    epi = (N.pie_epilogue * 1)()
    rc = N.lib().pie_decode_async(rt.ctx, ws, 1, ctypes.c_void_p(16), ctypes.c_void_p(16), epi, None)
    assert rc == N.PIE_ESTATE
    assert rt.ws_info(a)["len"] == 0
    assert N.lib().pie_sync(rt.ctx) == N.PIE_OK
    assert N.lib().pie_decode_async(None, ws, 1, ctypes.c_void_p(16), ctypes.c_void_p(16), epi, None) == N.PIE_EINVAL
    assert N.lib().pie_sync(None) == N.PIE_EINVAL
    rt.close()


def test_plan_layout_of_a_mixed_batch():
    """Packed rows, slots and page tables of a batch that mixes a prefill chunk,
    a decode row, a forked branch and explicit positions."""
    rt = host_rt(pages=64)
    a, b = rt.alloc(), rt.alloc()
    fwd(rt, [Pass(a, toks(40)), Pass(b, toks(17))])
    c = rt.fork(a)
    new = rt.alloc()
    passes = [Pass(new, toks(37, 5), [36, 0], [(0, 1.0, 0), (1, 0.5, 99)]),
              Pass(b, toks(1, 9), [0], [(0, 1.0, 0)]),
              Pass(c, toks(5, 3), [4], [(1, 0.7, 7)], positions=[100, 101, 102, 103, 104]),
              Pass(a, toks(2, 4), [], [], commit=False)]
    ctx_before = [0, 17, 40, 40]
    n_new = [37, 1, 5, 2]
    out, _ = fwd(rt, passes)
    assert list(out) == [-1] * 4
    pl = rt.plan()
    assert list(pl["seq_row0"]) == [0, 37, 38, 43, 45]
    assert list(pl["seq_ctx"]) == ctx_before
    assert list(pl["seq_len"]) == [c0 + n for c0, n in zip(ctx_before, n_new)]
    assert list(pl["row_seq"]) == sum(([s] * n for s, n in enumerate(n_new)), [])
    assert list(pl["tok"]) == sum((list(p.tokens) for p in passes), [])
    exp_pos = list(range(37)) + [17] + [100, 101, 102, 103, 104] + [40, 41]
    assert list(pl["pos"]) == exp_pos
    assert list(pl["ro_row"]) == [36, 0, 37, 42]
    assert list(pl["ro_lane"]) == [0, 1, 0, 0]
    assert len(set(pl["slot"])) == len(pl["slot"])  # no two rows write one slot
    tables = {}
    for s, h in enumerate([new, b, c, a]):
        lo, hi = pl["seq_pg0"][s], pl["seq_pg0"][s + 1]
        ids, valid, start = pl["pg_id"][lo:hi], pl["pg_valid"][lo:hi], pl["pg_start"][lo:hi]
        assert list(ids) == list(rt.ws_info(h)["pages"])
        assert list(start) == list(np.concatenate([[0], np.cumsum(valid)[:-1]]))
        assert int(np.sum(valid)) == pl["seq_len"][s]
        assert np.all((valid >= 1) & (valid <= P))
        tables[s] = (ids, valid, start)
        # row i of the pass sits at logical index seq_ctx + i of its working set
        for i in range(n_new[s]):
            j = pl["seq_ctx"][s] + i
            e = int(np.searchsorted(start, j, side="right") - 1)
            assert pl["slot"][pl["seq_row0"][s] + i] == ids[e] * P + (j - start[e])
    # pages a and its fork c share are written by neither
    shared = set(tables[2][0]) & set(tables[3][0])
    assert len(shared) == 3
    assert not (set(pl["slot"] // P) & shared)
    ia = rt.ws_info(a)
    assert ia["len"] == 42 and ia["frozen_len"] == 40
    rt.close()


def test_working_set_churn_keeps_pool_consistent():
    """Random alloc / fork / append / commit / truncate / free sequences: every
    page is either free or referenced by live working sets, with matching counts."""
    rng = np.random.default_rng(5)
    rt = host_rt(pages=48, max_rows=64, max_ctx=400)
    live = []
    for it in range(400):
        op = rng.integers(0, 6)
        if op == 0 or not live:
            live.append(rt.alloc())
        elif op == 1:
            live.append(rt.fork(live[rng.integers(len(live))]))
        elif op == 2:
            h = live.pop(rng.integers(len(live)))
            rt.free(h)
        elif op == 3:
            h = live[rng.integers(len(live))]
            info = rt.ws_info(h)
            rt.truncate(h, int(rng.integers(info["frozen_len"], info["len"] + 1)))
        else:
            k = int(rng.integers(1, 4))
            hs = [live[i] for i in rng.choice(len(live), size=min(k, len(live)), replace=False)]
            ps = [Pass(h, toks(int(rng.integers(1, 20))), commit=bool(rng.integers(2))) for h in hs]
            try:
                fwd(rt, ps)
            except N.PieError as e:
                assert e.code in (N.PIE_ENOMEM, N.PIE_EINVAL)
        refs = {}
        for h in live:
            for p in rt.ws_info(h)["pages"]:
                refs[p] = refs.get(p, 0) + 1
        st = rt.pool_stats()
        assert st["pages_free"] + len(refs) == st["pages_total"]
    for h in live:
        rt.free(h)
    st = rt.pool_stats()
    assert st["pages_free"] == st["pages_total"] and st["kv_bytes_copied"] == 0
    rt.close()


def test_noise_bounds_rule(tmp_path):
    """Full-size parity bounds: twice the largest measured float32-twin
    difference for logits, the difference itself for the token margin, never
    below the 2e-2 of the tiny configuration."""
    import json
    from tests.parity import noise_bounds
    a, b = tmp_path / "a.json", tmp_path / "b.json"
    a.write_text(json.dumps({"max_abs_dlogit": 0.031}))
    b.write_text(json.dumps({"max_abs_dlogit": 0.004}))
    tol, tau = noise_bounds([str(a), str(b)])
    assert abs(tol - 0.062) < 1e-12 and abs(tau - 0.031) < 1e-12
    assert noise_bounds([str(b)]) == (2e-2, 2e-2)


def test_noise_mean_bound_rule(tmp_path):
    """The mean |dlogit| bound is twice the largest twin mean of the files."""
    import json
    from tests.parity import Report, noise_mean_bound
    a, b = tmp_path / "a.json", tmp_path / "b.json"
    a.write_text(json.dumps({"max_abs_dlogit": 1.3, "mean_abs_dlogit": 0.21}))
    b.write_text(json.dumps({"max_abs_dlogit": 0.1, "mean_abs_dlogit": 0.02}))
    assert abs(noise_mean_bound([str(a), str(b)]) - 0.42) < 1e-12
    rep = Report()
    rep.add(1, 1, 0.5, 2.0)  # excluded: margin below tau
    rep.sum_err = 0.5
    rep.max_err = 0.5
    rep.check(tol=1.0, max_excluded_frac=1.0, mean_tol=0.6, min_compared=0)
    with pytest.raises(AssertionError):
        rep.check(tol=1.0, max_excluded_frac=1.0, mean_tol=0.4, min_compared=0)
    with pytest.raises(AssertionError):
        rep.check(tol=1.0, max_excluded_frac=0.6, mean_tol=0.6, min_compared=0)
    # by default some token must be compared
    with pytest.raises(AssertionError):
        rep.check(tol=1.0, max_excluded_frac=1.0, mean_tol=0.6)


def test_report_accumulates_the_mean_error_of_rows_given_logits():
    """Report.add with logits adds the row's mean |dlogit| to the sum the mean
    bound uses (a row given no logits adds nothing)."""
    import numpy as np
    from tests.parity import Report
    rep = Report()
    rep.add(3, 3, 1.0, 0.02, np.array([0.0, 1.0, 2.0]), np.array([0.1, 1.0, 1.7]))
    rep.add(4, 4, 1.0, 0.02)
    assert abs(rep.sum_err - (0.1 + 0.0 + 0.3) / 3) < 1e-12 and abs(rep.max_err - 0.3) < 1e-12
    rep.check(tol=0.3 + 1e-9, mean_tol=0.1)
    with pytest.raises(AssertionError):
        rep.check(tol=1.0, mean_tol=0.05)


def test_noise_bounds_take_2e2_where_the_twin_is_below_it(tmp_path):
    import json
    from tests.parity import noise_bounds
    a, b = tmp_path / "a.json", tmp_path / "b.json"
    a.write_text(json.dumps({"max_abs_dlogit": 0.019, "mean_abs_dlogit": 0.003}))
    b.write_text(json.dumps({"max_abs_dlogit": 0.031, "mean_abs_dlogit": 0.005}))
    assert noise_bounds([str(a)]) == (2e-2, 2e-2)
    assert noise_bounds([str(a), str(b)]) == (2 * 0.031, 0.031)


def test_stored_conditioning_files_are_complete():
    import glob
    import json
    for path in glob.glob(os.path.join(ROOT, "tests", "golden", "conditioning_*.json")):
        d = json.load(open(path))
        for k in ("model", "n_layers", "context", "max_abs_dlogit", "mean_abs_dlogit", "twin", "logit_std"):
            assert k in d, (path, k)
        # the float32 noise floor grows with depth (80 layers of the 70B shape
        # reach about 1.3) but stays below the spread of the logits themselves
        assert 0 < d["mean_abs_dlogit"] <= d["max_abs_dlogit"] < d["logit_std"]


def test_prefix_lookup_shares_whole_committed_pages():
    """pie_prefix_lookup: a request whose tokens start with a committed
    prefix gets that prefix's whole pages (no new page, no copy), at most
    n - 1 tokens; a different token anywhere in a page stops the match there."""
    rt = host_rt(pages=32)
    a = rt.alloc()
    pre = toks(40, 7)
    fwd(rt, [Pass(a, pre)])                      # committed: pages 0, 1 full, page 2 holds 8
    pages_a = list(rt.ws_info(a)["pages"])
    st0 = rt.pool_stats()
    b, k = rt.prefix_lookup(pre[:32] + toks(5, 900))
    assert k == 32
    ib = rt.ws_info(b)
    assert ib["len"] == ib["frozen_len"] == 32 and list(ib["pages"]) == pages_a[:2]
    assert rt.pool_stats()["pages_ever_allocated"] == st0["pages_ever_allocated"]
    assert rt.pool_stats()["kv_bytes_copied"] == 0
    # continue the shared prefix: new tokens go to a fresh page of b's own
    fwd(rt, [Pass(b, toks(5, 900), [4], [(0, 1.0, 0)])])
    assert list(rt.ws_info(b)["pages"][:2]) == pages_a[:2] and rt.ws_info(b)["pages"][2] not in pages_a
    # the whole input matches: at most n - 1 tokens are shared
    c, k = rt.prefix_lookup(pre[:32])
    assert k == 16
    # a changed token in page 1 stops the match after page 0
    alt = list(pre[:40])
    alt[20] = (alt[20] + 1) % synth.TINY.vocab
    d, k = rt.prefix_lookup(alt)
    assert k == 16 and list(rt.ws_info(d)["pages"]) == pages_a[:1]
    # nothing in common
    e, k = rt.prefix_lookup(toks(40, 3000))
    assert k == 0 and rt.ws_info(e)["len"] == 0
    rt.close()


def test_prefix_registry_rules():
    """Only host-known tokens at default positions are remembered; the
    writable buffer is not; a page is forgotten when its last holder frees it."""
    rt = host_rt(pages=32)
    a = rt.alloc()
    fwd(rt, [Pass(a, toks(20, 11), commit=0)])   # not committed: nothing to share
    _, k = rt.prefix_lookup(toks(30, 11))
    assert k == 0
    fwd(rt, [Pass(a, toks(20, 31), commit=1)])   # commits all 40
    _, k = rt.prefix_lookup(toks(20, 11) + toks(20, 31))
    assert k == 32
    # explicit positions that differ from the index: never remembered
    p = rt.alloc()
    fwd(rt, [Pass(p, toks(33, 500), positions=list(range(100, 133)))])
    _, k = rt.prefix_lookup(toks(33, 500))
    assert k == 0
    # pages freed by every holder are forgotten
    q = rt.alloc()
    fwd(rt, [Pass(q, toks(17, 700))])
    h, k = rt.prefix_lookup(toks(17, 700))
    assert k == 16
    rt.free(q)
    h2, k = rt.prefix_lookup(toks(17, 700))
    assert k == 16                               # h still holds the page
    rt.free(h)
    rt.free(h2)                                  # (every lookup result holds it too)
    _, k = rt.prefix_lookup(toks(17, 700))
    assert k == 0
    # a fork of a page-aligned prefix inherits it and extends it
    g = rt.alloc()
    fwd(rt, [Pass(g, toks(48, 200))])
    f = rt.fork(g)
    fwd(rt, [Pass(f, toks(20, 60))])
    _, k = rt.prefix_lookup(toks(48, 200) + toks(20, 60))
    assert k == 64
    # behind a partly filled page shared by a fork, token blocks no longer
    # line up with pages: the match stops there
    f2 = rt.fork(a)                              # a's third page holds 8 tokens
    fwd(rt, [Pass(f2, toks(30, 60))])
    _, k = rt.prefix_lookup(toks(20, 11) + toks(20, 31) + toks(30, 60))
    assert k == 32
    with pytest.raises(N.PieError) as e:
        rt.prefix_lookup([synth.TINY.vocab])
    assert e.value.code == N.PIE_EINVAL
    rt.close()
