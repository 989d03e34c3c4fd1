"""The C ABI on the CPU: the library loads, exports every declared entry point,
rejects bad arguments before touching the GPU, and builds sound job tables."""
import ctypes
import os
import re

import numpy as np
import pytest

import causal_flashattention_prefill_amd as zy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "zyfa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zyfa_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "zyfa_fwd" in names and "zyfa_fp8_quantize" in names and "zyfa_prepare" in names
    L = zy.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert zy.zyfa_status_string(0) == "ok"
    for code in zy.STATUS.values():
        assert zy.zyfa_status_string(code) != "unknown status"


def _fwd(**kw):
    a = dict(q=16, k=16, v=16, out=16, lse=None, B=1, S=128, H=4, Hk=2, dqk=128, dv=128, layout=0, dtype=0,
             qd=None, kd=None, vd=None, stream=None)
    a.update(kw)
    return zy.lib().zyfa_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["S"], a["H"], a["Hk"], a["dqk"],
                             a["dv"], a["layout"], a["dtype"], a["qd"], a["kd"], a["vd"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), "ZYFA_ERR_SHAPE"), (dict(S=0), "ZYFA_ERR_SHAPE"), (dict(H=-1), "ZYFA_ERR_SHAPE"),
    (dict(dqk=64, dv=64), "ZYFA_ERR_HEADDIM"), (dict(dqk=128, dv=192), "ZYFA_ERR_HEADDIM"),
    (dict(dqk=192, dv=192), "ZYFA_ERR_HEADDIM"), (dict(H=6, Hk=4), "ZYFA_ERR_GQA"),
    (dict(dtype=7), "ZYFA_ERR_DTYPE"), (dict(layout=3), "ZYFA_ERR_LAYOUT"), (dict(q=None), "ZYFA_ERR_NULL"),
    (dict(out=None), "ZYFA_ERR_NULL"), (dict(dtype=1), "ZYFA_ERR_DESCALE"), (dict(dtype=1, qd=16, kd=16), "ZYFA_ERR_DESCALE"),
    (dict(k=24), "ZYFA_ERR_ALIGN"),
])
def test_fwd_argument_errors(kw, status):
    assert _fwd(**kw) == zy.STATUS[status]


@pytest.mark.parametrize("p_mode", [-1, 4, 100])
def test_fwd_ex_rejects_unknown_p_mode(p_mode):
    L = zy.lib()
    rc = L.zyfa_fwd_ex(16, 16, 16, 16, None, 1, 128, 4, 2, 128, 128, 0, 1, 16, 16, 16, 0.0, p_mode, None)
    assert rc == zy.STATUS["ZYFA_ERR_PMODE"]


def test_quantize_argument_errors():
    L = zy.lib()
    assert L.zyfa_fp8_quantize(16, 5, 10, 16, 16, None) == zy.STATUS["ZYFA_ERR_DTYPE"]
    assert L.zyfa_fp8_quantize(16, 0, -1, 16, 16, None) == zy.STATUS["ZYFA_ERR_SHAPE"]
    assert L.zyfa_fp8_quantize(16, 0, 10, 16, None, None) == zy.STATUS["ZYFA_ERR_NULL"]
    assert L.zyfa_fp8_quantize(None, 0, 10, 16, 16, None) == zy.STATUS["ZYFA_ERR_NULL"]
    assert L.zyfa_fp8_quantize(8, 0, 10, 16, 16, None) == zy.STATUS["ZYFA_ERR_ALIGN"]


def test_prepare_argument_errors():
    L = zy.lib()
    assert L.zyfa_prepare(1, 128, 4, 3, 128, 128, 0, 0, 0, None) == zy.STATUS["ZYFA_ERR_GQA"]
    assert L.zyfa_prepare(1, 128, 4, 4, 96, 128, 0, 0, 0, None) == zy.STATUS["ZYFA_ERR_HEADDIM"]


def _random_shapes(n):
    rng = np.random.default_rng(77)
    out = []
    for _ in range(n):
        hk = int(rng.integers(1, 9))
        out.append((int(rng.integers(1, 5)), int(rng.integers(1, 40000)), hk * int(rng.integers(1, 9)), hk))
    return out


@pytest.mark.parametrize("B,S,H,Hk", [(1, 256, 4, 4), (1, 8192, 32, 8), (1, 16384, 32, 8), (1, 16384, 16, 16),
                                      (2, 32000, 32, 8), (3, 1000, 6, 2), (1, 1, 1, 1), (1, 300, 2, 1),
                                      (1, 16384, 4, 1)] + _random_shapes(24))
def test_job_table_covers_every_tile_once(B, S, H, Hk):
    tq, nw, jp, table = zy.zyfa_plan_jobs(B, S, H, Hk)
    n = -(-S // tq)
    assert 1 <= nw <= 256
    seen = {}
    work = np.zeros(nw)
    for w in range(nw):
        ended = False
        for r in range(jp):
            bh, i = table[r, w]
            if bh < 0:
                ended = True
                continue
            assert not ended, "a job after the end marker"
            assert 0 <= bh < B * H and 0 <= i <= n - 1 - i
            for t in {i, n - 1 - i}:
                key = (bh, t)
                assert key not in seen
                seen[key] = w
                work[w] += t + 1          # key tiles ~ tile index + 1
    assert len(seen) == B * H * n
    # every workgroup's job count differs by at most one
    counts = (table[:, :, 0] >= 0).sum(axis=0)
    assert counts.max() - counts.min() <= 1


@pytest.mark.parametrize("B,S,H,Hk,tq", [(1, 16384, 32, 8, 256), (2, 32000, 32, 8, 256), (1, 8192, 32, 8, 256),
                                         (1, 16384, 16, 16, 256), (1, 16384, 4, 1, 128), (1, 8192, 8, 8, 128),
                                         (1, 4096, 4, 1, 128)])
def test_tile_height_choice(B, S, H, Hk, tq):
    # 128-row tiles only where 256-row pairs leave compute units idle: one
    # GPU's share of the 16K GQA case over 8 GPUs (4 / 1 heads) has 128
    # pairs of 256-row tiles for 256 compute units
    assert zy.zyfa_plan_jobs(B, S, H, Hk)[0] == tq


def test_set_tile_q_argument_errors():
    L = zy.lib()
    for bad in (-1, 64, 129, 512):
        assert L.zyfa_set_tile_q(1, 1024, 4, 4, 128, 0, bad) == zy.STATUS["ZYFA_ERR_SHAPE"]
    assert L.zyfa_set_tile_q(1, 1024, 6, 4, 128, 0, 128) == zy.STATUS["ZYFA_ERR_GQA"]
    assert L.zyfa_set_tile_q(1, 1024, 4, 4, 96, 0, 128) == zy.STATUS["ZYFA_ERR_HEADDIM"]
    assert L.zyfa_set_tile_q(0, 1024, 4, 4, 128, 0, 128) == zy.STATUS["ZYFA_ERR_SHAPE"]


def test_job_pairs_have_equal_work():
    tq, nw, jp, table = zy.zyfa_plan_jobs(1, 16384, 32, 8)
    n = -(-16384 // tq)
    for bh, i in table.reshape(-1, 2):
        if bh >= 0:
            assert (i + 1) + (n - 1 - i + 1) == n + 1


def test_job_table_xcd_locality():
    # in each table row, the workgroups of one XCD (blockIdx % 8) hold
    # consecutive jobs: one KV head, and every query head of its group at
    # each pair index they hold (they read the same K and V tiles)
    tq, nw, jp, table = zy.zyfa_plan_jobs(1, 16384, 32, 8, dtype=zy.DTYPE_FP8)
    assert tq == 256 and nw == 256 and jp == 4
    for r in range(jp):
        for x in range(8):
            jobs = [tuple(int(v) for v in table[r, w]) for w in range(x, nw, 8)]
            assert len({h // 4 for h, _ in jobs}) == 1
            for i in {i for _, i in jobs}:
                assert sorted(h % 4 for h, t in jobs if t == i) == [0, 1, 2, 3]


def _range(**kw):
    a = dict(q=16, k=16, v=16, out=16, lse=None, B=1, Sq=128, Sk=300, qp=172, kp=0, H=4, Hk=2, dqk=128, dv=128,
             layout=0, dtype=0, qd=None, kd=None, vd=None, scale=0.0, p_mode=0, stream=None)
    a.update(kw)
    return zy.lib().zyfa_fwd_range(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Sq"], a["Sk"], a["qp"],
                                   a["kp"], a["H"], a["Hk"], a["dqk"], a["dv"], a["layout"], a["dtype"], a["qd"],
                                   a["kd"], a["vd"], a["scale"], a["p_mode"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Sk=0), "ZYFA_ERR_SHAPE"), (dict(Sq=0), "ZYFA_ERR_SHAPE"), (dict(dqk=64, dv=64), "ZYFA_ERR_HEADDIM"),
    (dict(H=6, Hk=4), "ZYFA_ERR_GQA"), (dict(layout=2), "ZYFA_ERR_LAYOUT"), (dict(v=None), "ZYFA_ERR_NULL"),
    (dict(dtype=1), "ZYFA_ERR_DESCALE"), (dict(out=8), "ZYFA_ERR_ALIGN"), (dict(p_mode=5), "ZYFA_ERR_PMODE"),
])
def test_fwd_range_argument_errors(kw, status):
    assert _range(**kw) == zy.STATUS[status]


def _merge(**kw):
    a = dict(oa=16, la=16, ob=16, lb=16, out=16, lse=16, B=1, S=100, H=4, dv=128, layout=0, stream=None)
    a.update(kw)
    return zy.lib().zyfa_lse_merge(a["oa"], a["la"], a["ob"], a["lb"], a["out"], a["lse"], a["B"], a["S"], a["H"],
                                   a["dv"], a["layout"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), "ZYFA_ERR_SHAPE"), (dict(S=-3), "ZYFA_ERR_SHAPE"), (dict(dv=192), "ZYFA_ERR_HEADDIM"),
    (dict(layout=4), "ZYFA_ERR_LAYOUT"), (dict(lb=None), "ZYFA_ERR_NULL"), (dict(lse=None), "ZYFA_ERR_NULL"),
    (dict(ob=24), "ZYFA_ERR_ALIGN"), (dict(la=18), "ZYFA_ERR_ALIGN"),
])
def test_lse_merge_argument_errors(kw, status):
    assert _merge(**kw) == zy.STATUS[status]


def _rot(**kw):
    import numpy as np
    a = dict(x=16, xd=0, rows=10, d=128, signs=None, x8=16, ds=16, stream=None)
    a.update(kw)
    sg = a["signs"]
    ptr = None if sg is None else sg.ctypes.data
    return zy.lib().zyfa_fp8_quantize_rotated(a["x"], a["xd"], a["rows"], a["d"], ptr, a["x8"], a["ds"], a["stream"])


def test_quantize_rotated_argument_errors():
    import numpy as np
    S = zy.STATUS
    assert _rot(xd=1) == S["ZYFA_ERR_DTYPE"]
    assert _rot(rows=-1) == S["ZYFA_ERR_SHAPE"]
    assert _rot(d=64) == S["ZYFA_ERR_HEADDIM"]
    assert _rot(d=192) == S["ZYFA_ERR_HEADDIM"]     # the Hadamard rotation is for d = 128
    bad = np.ones(128, dtype=np.int8)
    bad[7] = 0
    assert _rot(signs=bad) == S["ZYFA_ERR_SIGNS"]
    bad[7] = 2
    assert _rot(signs=bad) == S["ZYFA_ERR_SIGNS"]
    assert _rot(x=None) == S["ZYFA_ERR_NULL"]
    assert _rot(ds=None) == S["ZYFA_ERR_NULL"]
    assert _rot(x8=24) == S["ZYFA_ERR_ALIGN"]
    assert _rot(ds=18) == S["ZYFA_ERR_ALIGN"]


def test_key_mean_and_shifted_argument_errors():
    S = zy.STATUS
    L = zy.lib()
    # zyfa_key_mean(k, k_dtype, batch, seqlen, nheads_k, d, layout, mean, stream)
    assert L.zyfa_key_mean(16, 1, 1, 10, 2, 128, 0, 16, None) == S["ZYFA_ERR_DTYPE"]
    assert L.zyfa_key_mean(16, 0, 0, 10, 2, 128, 0, 16, None) == S["ZYFA_ERR_SHAPE"]
    assert L.zyfa_key_mean(16, 0, 1, 10, 2, 64, 0, 16, None) == S["ZYFA_ERR_HEADDIM"]
    assert L.zyfa_key_mean(16, 0, 1, 10, 2, 128, 5, 16, None) == S["ZYFA_ERR_LAYOUT"]
    assert L.zyfa_key_mean(None, 0, 1, 10, 2, 128, 0, 16, None) == S["ZYFA_ERR_NULL"]
    assert L.zyfa_key_mean(24, 0, 1, 10, 2, 128, 0, 16, None) == S["ZYFA_ERR_ALIGN"]
    # zyfa_fp8_quantize_rotated_shifted(x, xd, batch, seqlen, nheads, d, layout, signs, shift, x8, ds, stream)
    f = L.zyfa_fp8_quantize_rotated_shifted
    assert f(16, 0, 1, 10, 2, 128, 0, None, None, 16, 16, None) == S["ZYFA_ERR_NULL"]
    assert f(16, 0, 1, 10, 2, 128, 7, None, 16, 16, 16, None) == S["ZYFA_ERR_LAYOUT"]
    assert f(16, 0, 0, 10, 2, 128, 0, None, 16, 16, 16, None) == S["ZYFA_ERR_SHAPE"]
    assert f(16, 0, 1 << 20, 1 << 12, 1, 128, 0, None, 16, 16, 16, None) == S["ZYFA_ERR_RANGE"]
    assert f(16, 0, 1, 10, 2, 128, 0, None, 24, 16, 16, None) == S["ZYFA_ERR_ALIGN"]
    assert f(16, 0, 1, 10, 2, 96, 0, None, 16, 16, 16, None) == S["ZYFA_ERR_HEADDIM"]
    assert f(16, 0, 1, 10, 2, 192, 0, None, 16, 16, 16, None) == S["ZYFA_ERR_HEADDIM"]
