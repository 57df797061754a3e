"""Host-side tests of liblcsa through its C ABI: the library loads and exports
every symbol include/lcsa.h declares, the plan reproduces the oracle's
geometry, budget, windows and CSR row pointer, and each error status is
reachable from the host.  No kernel is launched."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import lcsa_inputs as li
import oracle

lcsa = pytest.importorskip("block_sparse_attention_lcsa_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcsa.h")


def _declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lcsa_[a-z_]+)\s*\(", txt)))


def test_header_declares_what_binding_lists():
    assert _declared_functions() == sorted(lcsa.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(lcsa.lib_path())
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lcsa.lib_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in _declared_functions():
        assert name in exported, name


def test_abi_version_and_status_strings():
    assert lcsa.abi_version() == 7
    lib = ctypes.CDLL(lcsa.lib_path())
    lib.lcsa_status_string.restype = ctypes.c_char_p
    texts = {lib.lcsa_status_string(i).decode() for i in range(9)}
    assert len(texts) == 9
    assert lib.lcsa_status_string(99) == b"unknown status"


@pytest.mark.parametrize("name", list(li.CONFIGS))
def test_plan_matches_oracle_geometry(name):
    desc = li.CONFIGS[name]
    g = oracle.geometry(desc)
    p = lcsa.Plan.from_desc(desc)
    inf = p.info
    assert inf["kv_frames"] == g.kv_frames
    assert (inf["nbh"], inf["nbw"], inf["blocks_per_frame"]) == (g.nbh, g.nbw, g.nbf)
    assert (inf["nqb"], inf["nkb"]) == (g.nqb, g.nkb)
    assert (inf["block_h"], inf["block_w"], inf["block_tokens"]) == (g.block_h, g.block_w, g.block_tokens)
    assert inf["k"] == min(g.k, g.nkb)
    assert inf["half_window"] == g.half
    assert inf["q_tokens"] == g.q_tokens and inf["kv_tokens"] == g.kv_tokens
    assert abs(inf["scale"] - g.scale) < 1e-15
    sizes = [len(oracle.window(g, qb)) for qb in range(g.nqb)]
    assert (inf["min_window"], inf["max_window"]) == (min(sizes), max(sizes))
    counts = [min(g.k, n) for n in sizes]
    assert inf["max_row_nnz"] == max(counts)
    rp = np.concatenate([[0], np.cumsum(counts * (g.batch * g.heads))])
    assert inf["rows"] == len(rp) - 1 and inf["nnz"] == rp[-1]
    assert np.array_equal(p.row_ptr(), rp)
    assert inf["useful_flops"] == oracle.useful_flops(g, rp)
    bt = g.block_tokens
    # one device-wide round of split pieces (256 CUs x 8 waves), then the
    # row lengths and row order of lcsa_attend_varlen
    assert inf["attend_workspace_bytes"] == (256 * (8 // (bt // 32)) * bt * (128 + 2) * 4
                                             + -(-8 * inf["rows"] // 256) * 256)
    # pooled K per frame slot, positions in groups of 8 (the last padded)
    assert inf["kcache_slot_bytes"] == g.batch * g.heads * 128 * (-(-g.nbf // 8) * 8) * 8
    assert inf["select_workspace_bytes"] == (g.batch * g.heads * 128 * g.nqb * 8
                                             + g.kv_frames * inf["kcache_slot_bytes"])
    for qb in range(0, g.nqb, max(1, g.nqb // 37)):
        assert np.array_equal(p.window(qb), oracle.window(g, qb))


def _desc(**over):
    d = dict(li.CONFIGS["first_768x1280"])
    d.update(over)
    return d


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=64), "LCSA_ERR_INVALID"),
    (dict(heads=0), "LCSA_ERR_INVALID"),
    (dict(q_frames=0), "LCSA_ERR_INVALID"),
    (dict(cached_frames=-1), "LCSA_ERR_INVALID"),
    (dict(local_range=10), "LCSA_ERR_INVALID"),
    (dict(local_range=0), "LCSA_ERR_INVALID"),
    (dict(kv_ratio=0.5), "LCSA_ERR_INVALID"),
    (dict(topk_ratio=0.0, topk=0), "LCSA_ERR_INVALID"),
    (dict(topk=-2), "LCSA_ERR_INVALID"),
    (dict(scale=-1.0), "LCSA_ERR_INVALID"),
    (dict(block_t=2), "LCSA_ERR_INVALID"),
    (dict(block_h=8, block_w=0), "LCSA_ERR_INVALID"),
    (dict(grid_h=44, grid_w=44), "LCSA_ERR_SHAPE"),
    (dict(block_t=1, block_h=4, block_w=4), "LCSA_ERR_SHAPE"),
    (dict(block_t=1, block_h=8, block_w=32), "LCSA_ERR_SHAPE"),
    (dict(grid_h=48, grid_w=72, block_t=1, block_h=8, block_w=16), "LCSA_ERR_SHAPE"),
])
def test_plan_rejects(over, status):
    with pytest.raises(lcsa.LcsaError) as ei:
        lcsa.Plan.from_desc(_desc(**over))
    assert ei.value.name == status
    assert str(ei.value).count(":") >= 2   # carries the detail message


def test_plan_auto_block_16x8_and_null_args():
    p = lcsa.Plan.from_desc(_desc(grid_w=88))
    assert (p.info["block_h"], p.info["block_w"]) == (16, 8)
    lib = ctypes.CDLL(lcsa.lib_path())
    lib.lcsa_plan_create.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert lib.lcsa_plan_create(None, None) == 1
    lib.lcsa_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.lcsa_plan_destroy(None)   # no-op


def test_row_ptr_capacity_and_window_range():
    p = lcsa.Plan.from_desc(li.CONFIGS["tiny"])
    lib = ctypes.CDLL(lcsa.lib_path())
    lib.lcsa_plan_row_ptr.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    buf = np.zeros(4, dtype=np.int32)
    assert lib.lcsa_plan_row_ptr(p.handle, buf.ctypes.data, 4) == 5   # WORKSPACE
    with pytest.raises(lcsa.LcsaError) as ei:
        p.window(p.info["nqb"])
    assert ei.value.name == "LCSA_ERR_INVALID"


def _fake_view(addr=0x10000, sb=0, ss=256, sh=128, plan=None, tokens="q", heads=None, dim=128):
    """A view of a fake device address with the extents a plan expects:
    tokens "q" (q_tokens), "kv" (kv_tokens) or a number."""
    p = plan if plan is not None else _TINY
    t = {"q": p.info["q_tokens"], "kv": p.info["kv_tokens"]}.get(tokens, tokens)
    return lcsa.LcsaTensor(data=addr, dtype=1, reserved=0, stride_b=sb, stride_s=ss, stride_h=sh,
                           batch=p.desc["batch"], tokens=t,
                           heads=p.desc["heads"] if heads is None else heads, head_dim=dim)


_TINY = lcsa.Plan.from_desc(li.CONFIGS["tiny"])


def _select(p, q, k, rp=0x20000, ci=0x30000, ws=0x40000, ws_bytes=None):
    lib = lcsa._lib
    wsb = p.info["select_workspace_bytes"] if ws_bytes is None else ws_bytes
    return lib.lcsa_select(p.handle, ctypes.byref(q), ctypes.byref(k), rp, ci, None, ws, wsb, None)


def _attend(p, q, k, v, o, nnz=8, ws=None, ws_bytes=0):
    lib = lcsa._lib
    return lib.lcsa_attend(p.handle, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                           0x20000, 0x30000, nnz, ctypes.byref(o), None, ws, ws_bytes, None)


def test_entry_point_validation_statuses():
    """Argument checks run on the host before any HIP call; the fake device
    addresses are never dereferenced because every call here fails first."""
    p = _TINY
    good = _fake_view()
    assert _select(p, _fake_view(addr=0x10008), good) == 4            # ALIGN data
    assert _select(p, _fake_view(ss=250), good) == 4                  # ALIGN stride
    assert _select(p, _fake_view(addr=0), good) == 1                  # NULL data
    assert _select(p, good, good, rp=0) == 1                          # NULL CSR
    assert _select(p, good, good, ws_bytes=16) == 5                   # WORKSPACE
    assert _select(p, good, good, ws=0x40010) == 4                    # ALIGN workspace
    bad_dtype = _fake_view(); bad_dtype.dtype = 7
    assert _select(p, bad_dtype, good) == 2                           # INVALID dtype
    assert _attend(p, good, good, good, good, nnz=-1) == 2            # INVALID nnz
    assert _attend(p, good, good, _fake_view(addr=0x10004), good) == 4
    assert _attend(p, good, good, good, good, ws=0x40040, ws_bytes=1 << 20) == 4  # ALIGN workspace
    assert lcsa._lib.lcsa_select(None, None, None, None, None, None, None, 0, None) == 1
    big = lcsa.Plan.from_desc(dict(li.CONFIGS["first_2048x3840"], local_range=15))
    assert big.info["max_window"] > 1024
    bq, bk = _fake_view(plan=big), _fake_view(plan=big, tokens="kv")
    assert _select(big, bq, bk) == 3                                  # SHAPE: window limit


def test_entry_point_extent_statuses():
    """Tensor extents that disagree with the plan are LCSA_ERR_SHAPE, checked
    on the host before any HIP call (after pointer, dtype and alignment)."""
    p = lcsa.Plan.from_desc(li.CONFIGS["small_edges"])    # q 4096 tokens, kv 6144
    q, kv = _fake_view(plan=p), _fake_view(plan=p, tokens="kv")
    assert p.info["q_tokens"] != p.info["kv_tokens"]
    assert _select(p, kv, kv) == 3                                    # q with kv's tokens
    assert _select(p, q, q) == 3                                      # k with q's tokens
    assert _select(p, q, _fake_view(plan=p, tokens="kv", heads=2)) == 3
    assert _select(p, q, _fake_view(plan=p, tokens="kv", dim=64)) == 3
    wrong_batch = _fake_view(plan=p); wrong_batch.batch = 2
    assert _select(p, wrong_batch, kv) == 3
    assert _attend(p, q, kv, kv, kv) == 3                             # o with kv's tokens
    assert _attend(p, q, kv, q, q) == 3                               # v with q's tokens
    assert _attend(p, q, _fake_view(plan=p, tokens=0), kv, q) == 3
    assert _select(p, _fake_view(plan=p, addr=0x10008, tokens=1), kv) == 4   # ALIGN first
    if not torch.cuda.is_available():
        assert _select(p, q, kv) == 6 and _attend(p, q, kv, kv, q) == 6      # DEVICE


def test_ring_entry_point_validation_statuses():
    """Frame-ring arguments are checked on the host before any HIP call."""
    p = lcsa.Plan.from_desc(li.CONFIGS["small_edges"])      # kv_frames 3
    kvf = p.info["kv_frames"]
    q = _fake_view(plan=p)
    ft = p.desc["grid_h"] * p.desc["grid_w"]
    ring4 = _fake_view(plan=p, tokens=4 * ft)                # a ring of 4 frame slots
    lib = lcsa._lib
    ws, wsb = 0x40000, p.info["select_workspace_bytes"]

    def sel(ring, new=1, kc=0x80000, kview=ring4):
        r = ctypes.byref(ring) if ring is not None else None
        return lib.lcsa_select_ring(p.handle, ctypes.byref(q), ctypes.byref(kview), r, new, kc,
                                    0x20000, 0x30000, None, ws, wsb, None)

    def att(ring, kview=ring4):
        r = ctypes.byref(ring) if ring is not None else None
        return lib.lcsa_attend_ring(p.handle, ctypes.byref(q), ctypes.byref(kview),
                                    ctypes.byref(kview), r, 0x20000, 0x30000, 8, ctypes.byref(q),
                                    None, None, 0, None)
    ok = lcsa.kv_ring(4, [3, 0, 1])
    assert sel(None) == 1                                            # NULL ring
    assert sel(lcsa.kv_ring(0, [0, 0, 0])) == 2                      # no slots
    assert sel(lcsa.kv_ring(4, [3, 4, 1])) == 2                      # slot out of range
    assert sel(lcsa.kv_ring(4, [3, 0, -1])) == 2
    assert sel(ok, new=kvf + 1) == 2 and sel(ok, new=-1) == 2        # new_frames
    assert sel(ok, kc=0) == 1                                        # NULL cache
    assert sel(ok, kc=0x80008) == 4                                  # ALIGN cache
    assert att(None) == 1 and att(lcsa.kv_ring(2, [0, 1, 2])) == 2
    kv3 = _fake_view(plan=p, tokens="kv")                     # 3 frames: not the ring's 4
    assert sel(ok, kview=kv3) == 3 and att(ok, kview=kv3) == 3      # SHAPE: ring extents
    if not torch.cuda.is_available():
        assert sel(ok) == 6 and att(ok) == 6                         # DEVICE on CPU hosts
    too_many = dict(li.CONFIGS["tiny"], q_frames=65, kv_ratio=0.0)
    with pytest.raises(lcsa.LcsaError) as ei:
        lcsa.Plan.from_desc(too_many)
    assert ei.value.name == "LCSA_ERR_SHAPE"


def test_rope_entry_point_validation_statuses():
    """Rotary-embedding arguments are checked on the host before any HIP call."""
    p = lcsa.Plan.from_desc(li.CONFIGS["small_edges"])
    q, kv = _fake_view(plan=p), _fake_view(plan=p, tokens="kv")
    ring4 = _fake_view(plan=p, tokens=4 * p.desc["grid_h"] * p.desc["grid_w"])
    lib = lcsa._lib
    ws, wsb = 0x40000, p.info["select_workspace_bytes"]

    def rope(pt=22, ph=21, pw=21, tt=0x50000, th=0x60000, tw=0x70000, reserved=0):
        return lcsa.LcsaRope(pairs_t=pt, pairs_h=ph, pairs_w=pw, reserved=reserved,
                             table_t=tt, table_h=th, table_w=tw)

    def sel(r, q_rot=q, k_rot=kv):
        rr = ctypes.byref(r) if r is not None else None
        qr = ctypes.byref(q_rot) if q_rot is not None else None
        kr = ctypes.byref(k_rot) if k_rot is not None else None
        return lib.lcsa_select_rope(p.handle, ctypes.byref(q), ctypes.byref(kv), rr, qr, kr,
                                    0x20000, 0x30000, None, ws, wsb, None)

    def sel_ring(r, ring, new=1, k_rot=ring4):
        rr = ctypes.byref(r) if r is not None else None
        return lib.lcsa_select_ring_rope(p.handle, ctypes.byref(q), ctypes.byref(ring4),
                                         ctypes.byref(ring), new, 0x80000, rr, ctypes.byref(q),
                                         ctypes.byref(k_rot), 0x20000, 0x30000, None, ws, wsb, None)
    assert sel(None) == 1                                             # NULL rope
    assert sel(rope(pt=23)) == 2 and sel(rope(pt=-1, ph=44)) == 2     # pairs must sum to 64
    assert sel(rope(reserved=1)) == 2
    assert sel(rope(th=0)) == 1                                       # table with pairs NULL
    assert sel(rope(pt=0, ph=43, tt=0)) != 1                          # no pairs: table may be NULL
    assert sel(rope(tw=0x70004)) == 4                                 # ALIGN table
    assert sel(rope(), q_rot=None) == 1                               # NULL output
    assert sel(rope(), k_rot=_fake_view(plan=p, addr=0x10008, tokens="kv")) == 4  # ALIGN output
    assert sel(rope(), q_rot=kv) == 3 and sel(rope(), k_rot=q) == 3   # SHAPE: output extents
    assert sel_ring(rope(), lcsa.kv_ring(4, [3, 0, 1]), k_rot=kv) == 3
    assert sel_ring(None, lcsa.kv_ring(4, [3, 0, 1])) == 1
    assert sel_ring(rope(), lcsa.kv_ring(4, [3, 4, 1])) == 2          # slot out of range
    assert sel_ring(rope(), lcsa.kv_ring(4, [3, 0, 1]), new=9) == 2
    if not torch.cuda.is_available():
        assert sel(rope()) == 6                                       # DEVICE on CPU hosts
        assert sel_ring(rope(), lcsa.kv_ring(4, [3, 0, 1])) == 6


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device status on CPU hosts")
def test_no_device_status_on_cpu_host():
    p = _TINY
    good = _fake_view()
    assert _select(p, good, good) == 6                                # DEVICE
    assert _attend(p, good, good, good, good) == 6


def test_plan_collected_at_interpreter_exit_is_quiet():
    # A plan held in __main__ of a script that imported torch first is
    # collected after the binding's globals are torn down; its destructor must
    # not raise then.
    code = ("import sys; sys.path.insert(0, %r); import torch; import lcsa_inputs as li; "
            "import block_sparse_attention_lcsa_amd as lcsa; "
            "plan = lcsa.Plan.from_desc(li.CONFIGS['tiny'])" % ROOT)
    r = subprocess.run([os.sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "Exception ignored" not in r.stderr, r.stderr


def test_threshold_entry_point_validation_statuses():
    """Arguments of the steady-threshold calls are checked on the host before
    any HIP call; the ring and the rotary tables are each optional."""
    p = lcsa.Plan.from_desc(li.CONFIGS["small_edges"])
    q, kv = _fake_view(plan=p), _fake_view(plan=p, tokens="kv")
    ring4 = _fake_view(plan=p, tokens=4 * p.desc["grid_h"] * p.desc["grid_w"])
    lib = lcsa._lib
    ws, wsb = 0x40000, p.info["select_workspace_bytes"]
    ok_ring = lcsa.kv_ring(4, [3, 0, 1])

    def steady(kth=0x90000, ring=None, new=1, kc=0x80000, rope=None):
        rg = ctypes.byref(ring) if ring is not None else None
        rp = ctypes.byref(rope) if rope is not None else None
        k = ring4 if ring is not None else kv
        return lib.lcsa_select_steady(p.handle, ctypes.byref(q), ctypes.byref(k), rg, new,
                                      kc, rp, ctypes.byref(q), ctypes.byref(k), 0x20000,
                                      0x30000, kth, None, ws, wsb, None)

    def reuse(tau=0x90000, ring=None, new=1, kc=0x80000):
        rg = ctypes.byref(ring) if ring is not None else None
        k = ring4 if ring is not None else kv
        return lib.lcsa_select_reuse(p.handle, ctypes.byref(q), ctypes.byref(k), rg, new, kc,
                                     None, None, None, tau, 0x20000, 0x30000, None, ws, wsb, None)
    assert steady(kth=0) == 1 and reuse(tau=0) == 1                  # NULL thresholds
    assert steady(kth=0x90004) == 4 and reuse(tau=0x90004) == 4      # ALIGN thresholds
    assert steady(ring=lcsa.kv_ring(4, [3, 4, 1])) == 2              # ring checked when given
    assert reuse(ring=ok_ring, new=9) == 2
    assert reuse(ring=ok_ring, kc=0) == 1 and reuse(ring=ok_ring, kc=0x80008) == 4
    bad_rope = lcsa.LcsaRope(pairs_t=23, pairs_h=21, pairs_w=21, reserved=0, table_t=0x50000,
                             table_h=0x60000, table_w=0x70000)
    assert steady(rope=bad_rope) == 2                                # rope checked when given
    if not torch.cuda.is_available():
        assert steady() == 6 and reuse() == 6 and reuse(ring=ok_ring) == 6   # DEVICE


def test_noalloc_select_statuses():
    """lcsa_select_noalloc refuses a NULL plan and a plan whose workspace
    exceeds the library's scratch array before any HIP call."""
    lib = lcsa._lib
    assert lib.lcsa_select_noalloc(None, None, None, None, None, None, None) == 1
    big = lcsa.Plan.from_desc(dict(li.CONFIGS["first_2048x3840"], batch=2))
    assert big.info["select_workspace_bytes"] > lcsa.SELECT_NOALLOC_MAX_BYTES
    bq, bk = _fake_view(plan=big), _fake_view(plan=big, tokens="kv")
    assert lib.lcsa_select_noalloc(big.handle, ctypes.byref(bq), ctypes.byref(bk), 0x20000,
                                   0x30000, None, None) == 5                 # WORKSPACE
    assert "scratch" in lib.lcsa_last_error().decode()
    p4k = lcsa.Plan.from_desc(li.CONFIGS["first_2048x3840"])
    assert p4k.info["select_workspace_bytes"] <= lcsa.SELECT_NOALLOC_MAX_BYTES
    if not torch.cuda.is_available():
        good = _fake_view()
        assert lib.lcsa_select_noalloc(_TINY.handle, ctypes.byref(good), ctypes.byref(good),
                                       0x20000, 0x30000, None, None) == 6    # DEVICE


def test_attend_varlen_validation_statuses():
    """lcsa_attend_varlen needs its workspace (the split pieces, then the row
    lengths and order): NULL or short is LCSA_ERR_WORKSPACE, checked on the
    host with the other arguments before any HIP call; a ring out of range is
    INVALID as for lcsa_attend_ring."""
    p = lcsa.Plan.from_desc(li.CONFIGS["small_edges"])      # kv_frames 3
    q, kv = _fake_view(plan=p), _fake_view(plan=p, tokens="kv")
    need = p.info["attend_workspace_bytes"]
    lib = lcsa._lib

    def varlen(k=kv, v=kv, ring=None, ws=0x40000, ws_bytes=need, nnz=8):
        return lib.lcsa_attend_varlen(p.handle, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                      ctypes.byref(ring) if ring is not None else None,
                                      0x20000, 0x30000, nnz, ctypes.byref(q), None, ws, ws_bytes,
                                      None)
    assert varlen(ws=None, ws_bytes=0) == 5                           # WORKSPACE: NULL
    assert varlen(ws_bytes=need - 1) == 5                             # WORKSPACE: short
    assert varlen(ws=0x40040) == 4                                    # ALIGN workspace
    assert varlen(nnz=-1) == 2                                        # INVALID nnz
    assert varlen(v=q) == 3                                           # SHAPE: v extents
    ft = p.desc["grid_h"] * p.desc["grid_w"]
    ring4 = _fake_view(plan=p, tokens=4 * ft)
    assert varlen(k=ring4, v=ring4, ring=lcsa.kv_ring(4, [3, 0, 4])) == 2   # INVALID slot
    assert lib.lcsa_attend_varlen(None, None, None, None, None, None, None, 0, None, None, None,
                                  0, None) == 1                        # NULL plan
    if not torch.cuda.is_available():
        assert varlen() == 6                                          # DEVICE on CPU hosts
        assert varlen(k=ring4, v=ring4, ring=lcsa.kv_ring(4, [3, 0, 1])) == 6
