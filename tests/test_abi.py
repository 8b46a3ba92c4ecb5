"""CPU checks of the C-ABI library: it loads, exports every symbol its header
declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m3scan.h")
LIB = os.path.join(ROOT, "selective_state_space_mimo_amd", "libm3scan.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(m3_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("m3_scan_fwd", "m3_decode_step", "m3_scan_workspace_size", "m3_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "build the library first (__graft_entry__.build())"
    lib = ctypes.CDLL(LIB)
    for n in _declared():
        assert hasattr(lib, n), n


def test_header_compiles_as_c():
    import shutil
    import subprocess
    import tempfile
    if not shutil.which("gcc"):
        pytest.skip("no gcc")
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "t.c")
        open(c, "w").write('#include "m3scan.h"\nint main(void){ m3_desc d; (void)d; return 0; }\n')
        subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                               "-c", c, "-o", os.path.join(td, "t.o")])


@pytest.fixture(scope="module")
def m3():
    import selective_state_space_mimo_amd as m
    return m


def _desc(m3, **kw):
    d = dict(batch=2, seqlen=8, nheads=4, ngroups=2, headdim=16, dstate=16, rank=2, npairs=2,
             chunk=4, io_dtype=m3.M3_F32, state_dtype=m3.M3_F32, nsegments=0, rate_law=m3.M3_RATE_STATIC)
    d.update(kw)
    return m3.Desc(**d)


FAKE = 0x7f0000000000   # never dereferenced: every call below fails argument checks first


def _scan(m3, desc, **ptrs):
    p = dict(x=FAKE, B=FAKE + 0x100000, C=FAKE + 0x200000, dt=FAKE + 0x300000, lam=FAKE + 0x400000,
             theta=FAKE + 0x500000, A_log=FAKE + 0x600000, Bb=None, Cb=None, y=FAKE + 0x700000)
    p.update(ptrs)
    return m3.lib.m3_scan_fwd(ctypes.byref(desc), p["x"], p["B"], p["C"], p["dt"], p["lam"], p["theta"],
                              p["A_log"], p["Bb"], p["Cb"], None, p["y"], None, None, 0, None)


def test_status_strings(m3):
    for s in range(6):
        assert m3.lib.m3_status_string(s)
    assert m3.lib.m3_version() > 0


def test_invalid_descriptors(m3):
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_scan_workspace_size(None, ctypes.byref(n)) == 1
    bad = [dict(nheads=3, ngroups=2), dict(npairs=9), dict(dstate=15), dict(batch=0), dict(chunk=0),
           dict(rank=0), dict(io_dtype=7), dict(seqlen=-1), dict(rate_law=2)]
    for kw in bad:
        assert m3.lib.m3_scan_workspace_size(ctypes.byref(_desc(m3, **kw)), ctypes.byref(n)) == 1, kw
        assert _scan(m3, _desc(m3, **kw)) == 1, kw
    assert m3.lib.m3_scan_workspace_size(ctypes.byref(_desc(m3, dstate=512)), ctypes.byref(n)) == 2
    assert m3.lib.m3_scan_workspace_size(ctypes.byref(_desc(m3)), ctypes.byref(n)) == 0


def test_null_misaligned_and_aliased_pointers(m3):
    d = _desc(m3)
    assert _scan(m3, d, x=None) == 1
    assert _scan(m3, d, theta=None) == 1                 # npairs > 0 needs theta
    assert _scan(m3, d, y=None) == 1
    assert _scan(m3, d, dt=FAKE + 0x300004) == 3         # not 16-byte aligned
    assert _scan(m3, d, y=FAKE + 0x10) == 1              # y overlaps x
    desc = _desc(m3, seqlen=1)
    c = m3.Carry(FAKE + 0x800000, FAKE + 0x900000, FAKE + 0xa00000, FAKE + 0xb00000)
    assert m3.lib.m3_decode_step(ctypes.byref(desc), FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000,
                                 FAKE + 0x400000, None, FAKE + 0x600000, None, None, ctypes.byref(c),
                                 FAKE + 0x700000, None) == 1     # theta missing
    # per-token rates: the rate input spans [b, L, H], here reaching into y
    assert _scan(m3, _desc(m3, rate_law=m3.M3_RATE_HEAVY_TAIL), A_log=FAKE + 0x700000 - 64) == 1
    c2 = m3.Carry(FAKE + 0x800000, FAKE + 0x900000, FAKE + 0x800010, FAKE + 0xb00000)   # B_prev inside h
    assert m3.lib.m3_decode_step(ctypes.byref(desc), FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000,
                                 FAKE + 0x400000, FAKE + 0x500000, FAKE + 0x600000, None, None, ctypes.byref(c2),
                                 FAKE + 0x700000, None) == 1


def _block(m3, d, p=None, ws_bytes=None, **kw):
    a = dict(z=FAKE, x=FAKE + 0x100000, B=FAKE + 0x200000, C=FAKE + 0x300000, dt=FAKE + 0x400000,
             A=FAKE + 0x500000, lam=FAKE + 0x600000, th=FAKE + 0x680000, out=FAKE + 0x700000, ws=FAKE + 0x1000000)
    a.update(kw)
    if p is None:
        p = m3.BlockParams(None, None, None, None, None, FAKE + 0x900000, FAKE + 0x940000, None, 1e-6)
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_block_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == 0
    return m3.lib.m3_block_fwd(ctypes.byref(d), ctypes.byref(p), a["z"], a["x"], a["B"], a["C"], a["dt"], a["A"],
                               a["lam"], a["th"], None, a["out"], None, a["ws"],
                               n.value if ws_bytes is None else ws_bytes, None)


def test_block_entry_points_reject_bad_arguments(m3):
    """The layer entry points check parameters, pointers, alignment, the
    workspace size and overlaps before launching anything."""
    d = _desc(m3, rate_law=m3.M3_RATE_HEAVY_TAIL)
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_block_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == 0 and n.value > 0
    n1 = ctypes.c_size_t(0)
    assert m3.lib.m3_block_workspace_size(ctypes.byref(d), 1, ctypes.byref(n1)) == 0 and 0 < n1.value < n.value
    assert m3.lib.m3_block_workspace_size(None, 0, ctypes.byref(n)) == 1
    no_lift = m3.BlockParams(None, None, None, None, None, None, FAKE + 0x940000, None, 1e-6)
    assert _block(m3, d, p=no_lift) == 1
    zero_eps = m3.BlockParams(None, None, None, None, None, FAKE + 0x900000, FAKE + 0x940000, None, 0.0)
    assert _block(m3, d, p=zero_eps) == 1
    assert _block(m3, d, z=None) == 1
    assert _block(m3, d, th=None) == 1                    # npairs > 0 needs the raw angles
    assert _block(m3, d, z=FAKE + 8) == 3                 # not 16-byte aligned
    assert _block(m3, d, ws_bytes=64) == 1                # workspace too small
    assert _block(m3, d, out=FAKE + 0x100010) == 1        # out overlaps x
    assert _block(m3, d, ws=FAKE + 0x400000) == 1         # workspace overlaps dt_raw


def _bwd(m3, d, ws_bytes=None, grads=None, **kw):
    a = dict(x=FAKE, B=FAKE + 0x100000, C=FAKE + 0x200000, dt=FAKE + 0x300000, lam=FAKE + 0x400000,
             theta=FAKE + 0x500000, A=FAKE + 0x600000, dy=FAKE + 0x700000, ws=FAKE + 0x4000000)
    a.update(kw)
    if grads is None:
        grads = m3.Grads(FAKE + 0x1000000, FAKE + 0x1100000, FAKE + 0x1200000, FAKE + 0x1300000, FAKE + 0x1400000,
                         FAKE + 0x1500000, FAKE + 0x1600000, None, None, m3.CarryGrad(None, None, None, None))
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_scan_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    return m3.lib.m3_scan_bwd(ctypes.byref(d), a["x"], a["B"], a["C"], a["dt"], a["lam"], a["theta"], a["A"],
                              None, None, None, a["dy"], None, ctypes.byref(grads), a["ws"],
                              n.value if ws_bytes is None else ws_bytes, None)


def test_backward_entry_point_rejects_bad_arguments(m3):
    """m3_scan_bwd checks shapes, pointers, alignment, the workspace size and
    overlaps (outputs with inputs and with each other) before launching."""
    d = _desc(m3)
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_scan_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0 and n.value > 0
    assert m3.lib.m3_scan_bwd_workspace_size(None, ctypes.byref(n)) == 1
    assert m3.lib.m3_scan_bwd_workspace_size(ctypes.byref(_desc(m3, headdim=80)), ctypes.byref(n)) == 2
    assert m3.lib.m3_scan_bwd_workspace_size(ctypes.byref(_desc(m3, rank=5)), ctypes.byref(n)) == 2
    assert _bwd(m3, d, dy=None) == 1
    assert _bwd(m3, d, theta=None) == 1                    # npairs > 0 needs theta
    assert _bwd(m3, d, dt=FAKE + 0x300004) == 3            # not 16-byte aligned
    assert _bwd(m3, d, ws_bytes=64) == 1                   # workspace too small
    assert _bwd(m3, d, ws=FAKE + 0x700000) == 1            # workspace overlaps dy
    g = m3.Grads(FAKE + 0x1000000, FAKE + 0x1100000, FAKE + 0x1200000, FAKE + 0x1300000, FAKE + 0x1400000,
                 None, FAKE + 0x1600000, None, None, m3.CarryGrad(None, None, None, None))
    assert _bwd(m3, d, grads=g) == 1                       # dtheta required when npairs > 0
    g = m3.Grads(FAKE + 0x10, FAKE + 0x1100000, FAKE + 0x1200000, FAKE + 0x1300000, FAKE + 0x1400000,
                 FAKE + 0x1500000, FAKE + 0x1600000, None, None, m3.CarryGrad(None, None, None, None))
    assert _bwd(m3, d, grads=g) == 1                       # dx overlaps x
    g = m3.Grads(FAKE + 0x1000000, FAKE + 0x1000010, FAKE + 0x1200000, FAKE + 0x1300000, FAKE + 0x1400000,
                 FAKE + 0x1500000, FAKE + 0x1600000, None, None, m3.CarryGrad(None, None, None, None))
    assert _bwd(m3, d, grads=g) == 1                       # dB overlaps dx


def test_final_carry_must_not_overlap_inputs(m3):
    """The final carry is written while other workgroups still read the inputs:
    m3_scan_fwd and m3_block_fwd reject a final carry that overlaps any input,
    the output or the workspace."""
    d = _desc(m3)
    p = dict(x=FAKE, B=FAKE + 0x100000, C=FAKE + 0x200000, dt=FAKE + 0x300000, lam=FAKE + 0x400000,
             theta=FAKE + 0x500000, A_log=FAKE + 0x600000, y=FAKE + 0x700000)

    def scan_with_final(fin):
        return m3.lib.m3_scan_fwd(ctypes.byref(d), p["x"], p["B"], p["C"], p["dt"], p["lam"], p["theta"],
                                  p["A_log"], None, None, None, p["y"], ctypes.byref(fin), None, 0, None)
    ok = m3.Carry(FAKE + 0x800000, FAKE + 0x900000, FAKE + 0xa00000, FAKE + 0xb00000)
    for k, bad in (("h", FAKE + 0x100000), ("phi", FAKE + 0x300000), ("B_prev", FAKE + 0x10),
                   ("x_prev", FAKE + 0x600000)):
        f = m3.Carry(ok.h, ok.phi, ok.B_prev, ok.x_prev)
        setattr(f, k, bad)
        assert scan_with_final(f) == 1, k
    db = _desc(m3, rate_law=m3.M3_RATE_HEAVY_TAIL)
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_block_workspace_size(ctypes.byref(db), 0, ctypes.byref(n)) == 0
    prm = m3.BlockParams(None, None, None, None, None, FAKE + 0x900000, FAKE + 0x940000, None, 1e-6)
    for bad in (FAKE + 0x200000, FAKE + 0x700000, FAKE + 0x1000000):      # B_raw, out, workspace
        f = m3.Carry(bad, FAKE + 0x2900000, FAKE + 0x2a00000, FAKE + 0x2b00000)
        assert m3.lib.m3_block_fwd(ctypes.byref(db), ctypes.byref(prm), FAKE, FAKE + 0x100000, FAKE + 0x200000,
                                   FAKE + 0x300000, FAKE + 0x400000, FAKE + 0x500000, FAKE + 0x600000,
                                   FAKE + 0x680000, None, FAKE + 0x700000, ctypes.byref(f), FAKE + 0x1000000,
                                   n.value, None) == 1, hex(bad)


def test_noalloc_rejects_a_schedule_beyond_its_scratch(m3):
    """m3_scan_fwd_noalloc refuses, before any HIP call, a schedule whose workspace
    exceeds its per-GPU scratch (here the long-context shape split into 64
    segments per stream), and names the limit."""
    G4 = 1 << 32
    d = _desc(m3, batch=1, seqlen=65536, nheads=64, ngroups=1, headdim=64, dstate=128, rank=4, npairs=32,
              chunk=16, io_dtype=m3.M3_BF16, nsegments=64)
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_scan_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value > m3.lib.m3_scan_noalloc_max_workspace() == 64 << 20
    st = m3.lib.m3_scan_fwd_noalloc(ctypes.byref(d), FAKE, FAKE + G4, FAKE + 2 * G4, FAKE + 3 * G4, FAKE + 4 * G4,
                                    FAKE + 5 * G4, FAKE + 6 * G4, None, None, None, FAKE + 7 * G4, None, None)
    assert st == m3.M3_ERR_TOO_LARGE == 5
    assert b"64 MiB" in m3.lib.m3_status_string(st)


def _pcs_desc(m3, **kw):
    d = dict(batch=2, seqlen=300, channels=128, ngroups=1, dstate=16, io_dtype=m3.M3_BF16, nsegments=0)
    d.update(kw)
    return m3.PcsDesc(**d)


def _pcs(m3, d, ws_bytes=None, **kw):
    a = dict(x=FAKE, dt=FAKE + 0x100000, A=FAKE + 0x200000, B=FAKE + 0x300000, C=FAKE + 0x400000, h0=None,
             y=FAKE + 0x500000, h1=None, ws=FAKE + 0x1000000)
    a.update(kw)
    n = ctypes.c_size_t(0)
    st = m3.lib.m3_pcs_workspace_size(ctypes.byref(d), ctypes.byref(n))
    if st != 0:
        return st
    return m3.lib.m3_pcs_fwd(ctypes.byref(d), a["x"], a["dt"], a["A"], a["B"], a["C"], a["h0"], a["y"], a["h1"],
                             a["ws"], n.value if ws_bytes is None else ws_bytes, None)


def test_pcs_entry_points_reject_bad_arguments(m3):
    """m3_pcs_workspace_size / m3_pcs_fwd: invalid descriptors, sizes outside
    the kernels' range, NULL / misaligned / overlapping pointers and a short
    workspace are refused before any HIP call."""
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_pcs_workspace_size(None, ctypes.byref(n)) == 1
    assert m3.lib.m3_pcs_workspace_size(ctypes.byref(_pcs_desc(m3)), None) == 1
    for bad in (dict(batch=0), dict(seqlen=-1), dict(channels=0), dict(ngroups=3), dict(dstate=0),
                dict(io_dtype=7), dict(nsegments=-1)):
        assert _pcs(m3, _pcs_desc(m3, **bad)) == 1, bad
    for uns in (dict(dstate=12), dict(dstate=4), dict(dstate=128), dict(channels=132),      # 132 % 8 != 0 (bf16)
                dict(channels=192, ngroups=2), dict(nsegments=65)):
        assert _pcs(m3, _pcs_desc(m3, **uns)) == 2, uns
    assert _pcs(m3, _pcs_desc(m3, channels=132, io_dtype=m3.M3_F32), y=None) == 1    # f32 rows: 132 % 4 == 0
    d = _pcs_desc(m3)
    assert _pcs(m3, d, C=None) == 1
    assert _pcs(m3, d, dt=FAKE + 0x100008) == 3                                    # not 16-byte aligned
    assert _pcs(m3, d, h1=FAKE + 0x600004) == 3
    assert _pcs(m3, d, y=FAKE + 0x10) == 1                                         # y overlaps x
    assert _pcs(m3, d, h1=FAKE + 0x300000) == 1                                    # h1 overlaps B
    assert _pcs(m3, d, h0=FAKE + 0x600000, h1=FAKE + 0x600000) == 1                # state updated in place
    # a forced segmented schedule needs a workspace that overlaps nothing
    ds = _pcs_desc(m3, nsegments=3)
    assert m3.lib.m3_pcs_workspace_size(ctypes.byref(ds), ctypes.byref(n)) == 0 and n.value > 0
    assert _pcs(m3, ds, ws_bytes=16) == 1
    assert _pcs(m3, ds, ws=None) == 1
    assert _pcs(m3, ds, ws=FAKE + 0x200000) == 1                                   # workspace overlaps A_log


def test_pcs_schedule_sizes(m3):
    """The library's segment choice: none when the (batch, channel tile)
    workgroups fill the chip, several for few long sequences; a forced count is
    clamped to the number of 32-token blocks.  Workspace: two [b, D, nseg, N]
    fp32 state sets and one [b, D, nseg] step sum."""
    def ws(**kw):
        n = ctypes.c_size_t(0)
        assert m3.lib.m3_pcs_workspace_size(ctypes.byref(_pcs_desc(m3, **kw)), ctypes.byref(n)) == 0
        return n.value
    assert ws(batch=16, seqlen=2048, channels=4096) == 0
    b, D, N = 2, 2048, 16
    nseg = 64          # 64 tiles of 64 channels, one wave each when segmented: 64 segments, four waves per SIMD
    assert ws(batch=b, seqlen=32768, channels=D) == (2 * b * D * nseg * N + b * D * nseg) * 4
    assert ws(batch=1, seqlen=100, channels=64, nsegments=64) == (2 * 64 * 4 * 16 + 64 * 4) * 4   # 4 blocks of 32
    assert ws(batch=1, seqlen=0, channels=64, nsegments=5) == 0
    # a segment's rows must stay under 2 GiB: 2^20 tokens of 4096 channels need at least 9
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_pcs_workspace_size(ctypes.byref(_pcs_desc(m3, batch=1, seqlen=1 << 20, channels=4096,
                                                                nsegments=1)), ctypes.byref(n)) == 0
    assert n.value == (2 * 4096 * 9 * 16 + 4096 * 9) * 4
    assert m3.lib.m3_pcs_workspace_size(ctypes.byref(_pcs_desc(m3, batch=1, seqlen=1 << 23, channels=4096)),
                                        ctypes.byref(n)) == 2     # would need more than 64 segments


def test_layer_workspace_follows_the_path(m3):
    """m3_block_workspace_size sizes what the path taken uses: on the fused bf16
    matrix-core path (P 64, N 128, R 4, chunk 64) only the normalised B, C and the
    scan's own workspace (the scan writes the layer's output itself); the unfused
    path also holds the lifted x, the activated dt / lambda / theta and R readouts."""
    n = ctypes.c_size_t(0)
    kw = dict(batch=2, seqlen=256, nheads=4, ngroups=1, headdim=64, dstate=128, rank=4, npairs=32, chunk=64,
              nsegments=1)
    assert m3.lib.m3_block_workspace_size(ctypes.byref(_desc(m3, io_dtype=m3.M3_BF16, **kw)), 0, ctypes.byref(n)) == 0
    fused = n.value
    b, L, H, P, N, R = 2, 256, 4, 64, 128, 4
    assert fused == 2 * (b * L * R * N * 2)                              # Bn, Cn (256-byte multiples)
    assert m3.lib.m3_block_workspace_size(ctypes.byref(_desc(m3, io_dtype=m3.M3_F32, **kw)), 0, ctypes.byref(n)) == 0
    unfused = n.value
    assert unfused >= b * L * H * R * P * 4 * 2 + 2 * b * L * R * N * 4 + b * L * H * (2 + 32) * 4
