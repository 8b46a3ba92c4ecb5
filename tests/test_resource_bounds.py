"""CPU replay of every buffer resource the kernels build: base, record count and
the offsets each load or store forms, checked against the tensor's extent.

A buffer access whose offset is at or past the resource's record count reads zero
or is dropped, so a resource may reach past its tensor (the output rows of one head
span whole tokens of all heads); what must hold is that every offset *inside* the
record count addresses bytes of the tensor.  The replay below restates the kernels'
base, record-count and offset arithmetic (the matrix-core chunked scan in
csrc/scan_mfma.hip, the single-rank scan and its score pass in csrc/scan_siso.hip,
both per-coordinate kernels in csrc/pcs.hip, the raw loads, row prefetch, start-phase
loads and theta-gradient stores of the backward's chunked form in csrc/bwd_chunk.hip) and checks it for
the edge workgroups (first and last batch, head, channel tile and segment, every
chunk of the segment) of every shape the GPU tests and the benchmark run.  The
segment schedule is the library's, restated here and cross-checked against the
workspace size the library reports.
"""
import ctypes

import numpy as np
import pytest

from m3inputs import config_by_name
from m3inputs.pcs import PCS_CONFIGS

KP, KN = 64, 128                      # the matrix-core path's head and state widths


@pytest.fixture(scope="module")
def m3():
    import selective_state_space_mimo_amd as m
    return m


def _check(what, base, records, offsets, size, extent):
    """offsets (bytes from base) of accesses of `size` bytes: those inside the record
    count must lie within [0, extent) of the tensor."""
    o = np.asarray(offsets, np.int64).ravel()
    inside = o[o < records]
    if inside.size == 0:
        return
    lo = base + inside.min()
    hi = base + inside.max() + size
    assert lo >= 0 and hi <= extent, "%s: bytes [%d, %d) of a %d-byte tensor (base %d, records %d)" % (
        what, lo, hi, extent, base, records)


# ---------------------------------------------------------------------------
# chunked scan (matrix-core path)
# ---------------------------------------------------------------------------
def executed_chunk(R, Q):
    built = Q in (16, 32, 64, 128) and 64 <= Q * R <= 256
    return Q if built else 64 // R


def scan_segments(b, H, L, R, Q, nsegments):
    nchunks = -(-L // Q)
    k = nsegments
    if k == 0:
        streams = b * H
        slots = 256 * (2 if (R == 4 and Q == 16) else 1)
        k = 1 if streams >= slots else -(-slots // streams)
    k = max(1, min(k, max(1, nchunks)))
    seglen = -(-nchunks // k) * Q
    return max(1, -(-L // seglen)), seglen


def _ctile(nc, c, k):
    """Query tile k of consumer c (tiles dealt in groups of 2 nc: c and 2 nc - 1 - c)."""
    return 2 * nc * (k >> 1) + ((2 * nc - 1 - c) if (k & 1) else c)


def layer_pieces(R, Q, n_cons):
    """(token of the chunk, 16-byte piece) pairs of the layer's output rows as the
    consumers' lanes take them: piece p of consumer c (token u = p / 8 of its tiles,
    rows R u .. R u + R - 1 in tile order) goes to lane p % 64, slot p / 64; pieces past
    the consumer's tokens are not issued."""
    tpc = Q * R // 16 // n_cons
    xu = tpc * 16 // R
    slots = (8 * xu + 63) // 64
    out = []
    for c in range(n_cons):
        for sl in range(slots):
            for ln in range(64):
                p = 64 * sl + ln
                if p >= 8 * xu:
                    continue
                rr = R * (p >> 3)
                row = 16 * _ctile(n_cons, c, rr >> 4) + (rr & 15)
                out.append((row // R, p & 7))
    return out


def replay_scan(b, L, H, G, R, Q, np_, nseg, seglen, layer=False):
    n_cons = 8 if (R == 4 and Q == 64) else 4
    n_threads = 64 * (n_cons + 4)
    lanes = np.arange(64)
    tids = np.arange(n_threads)
    B_bytes = b * L * G * R * KN * 2
    xrows = 1 if layer else R
    X_bytes = b * L * H * xrows * KP * 2
    Y_bytes = b * L * H * (1 if layer else R) * KP * 2
    TH_bytes = b * L * H * np_ * 4
    bstride = G * R * KN
    xstride = H * xrows * KP
    bsb, xsb, ysb = bstride * 2, xstride * 2, H * R * KP * 2
    for bi in sorted({0, b - 1}):
        for h in sorted({0, H - 1}):
            g = h * G // H
            for seg in sorted({0, nseg - 1}):
                T0 = seg * seglen
                T1 = min(L, T0 + seglen)
                tokbase = bi * L
                chunks = list(range(T0, T1, Q))
                # angles: one buffer load per value, THU values per thread and token round
                if np_:
                    THU = 8 if Q >= 64 else Q // 8
                    THG = 64 // THU
                    THP = (Q + 63) // 64
                    tt = tids & 1023
                    th_t, th_i = tt // THG, (tt % THG) * THU
                    for cst in chunks:
                        nt = min(max(T1 - cst, 0), Q)
                        rec = ((nt - 1) * H * np_ + np_) * 4 if nt > 0 else 0
                        base = ((tokbase + cst) * H + h) * np_ * 4
                        offs = []
                        for pp in range(THP):
                            vo = np.where(th_i < np_, ((th_t + 64 * pp) * H * np_ + th_i) * 4, 0x7FFFFF00)
                            for u in range(THU):
                                offs.append(vo + 4 * u)
                        _check("theta", base, rec, np.concatenate(offs), 4, TH_bytes)
                # C rows of a chunk, straight into the operand layout
                Cg = (tokbase * G + g) * R * KN * 2
                qi = np.arange(Q * R)[:, None, None]
                ks = np.arange(4)[None, :, None]
                j4 = np.arange(4)[None, None, :]
                for cst in chunks:
                    nv = max(0, min(Q, T1 - cst))
                    base = Cg + (cst if nv > 0 else 0) * bstride * 2
                    t, r = qi // R, qi % R
                    _check("C rows", base, nv * bsb, t * bsb + r * (KN * 2) + 64 * ks + 16 * j4, 16, B_bytes)
                # outputs: whole staged rows (the layer: one P-wide row per token, in 16-byte
                # pieces dealt to the consumers' lanes; the x and gate pieces are read at the
                # same offsets of their [b, L, H, P] tensors)
                for cst in chunks:
                    nv = max(0, min(Q, T1 - cst))
                    k8 = np.arange(8)[None, None, :]
                    tq = np.arange(Q)[:, None, None]
                    if layer:
                        base = ((tokbase + cst) * H + h) * KP * 2
                        offs = np.array([t * (H * KP * 2) + 16 * k for t, k in layer_pieces(R, Q, n_cons)])
                        for what in ("layer out", "layer x", "layer gate"):
                            _check(what, base, nv * H * KP * 2, offs, 16, Y_bytes)
                    else:
                        rr = np.arange(R)[None, :, None]
                        base = ((tokbase + cst) * H + h) * R * KP * 2
                        _check("y", base, nv * ysb, tq * ysb + rr * (KP * 2) + 16 * k8, 16, Y_bytes)
                # key rows of B and x, fetched per producer in blocks of 32 / R tokens
                TPB = 32 // R
                NTK = 16 // R + 3 // R + 1
                h2, l2 = lanes >> 5, lanes & 31
                Bg = (tokbase * G + g) * R * KN
                Xg = (tokbase * H + h) * xrows * KP
                rstride = 0 if layer else 128
                for pw in range(4):
                    s0 = T0 + 4 * pw // R
                    f_rem = T1 - s0
                    fb, fx = Bg + s0 * bstride, Xg + s0 * xstride
                    while f_rem > -TPB:
                        nt = min(max(f_rem, 0), NTK)
                        ob = [((h2 * (16 // R) + i // R) * bsb + 256 * (i % R) + 8 * l2) for i in range(4)]
                        _check("B rows", fb * 2, nt * bsb, np.stack(ob), 8, B_bytes)
                        ox = [((rr_ >> 2) * (16 // R) + (rr_ & 3) // R) * xsb + rstride * ((rr_ & 3) % R) + 4 * l2
                              for rr_ in range(8)]
                        _check("x rows", fx * 2, nt * xsb, np.stack(ox), 4, X_bytes)
                        f_rem -= TPB
                        fb += TPB * bstride
                        fx += TPB * xstride


SISO_PREP_CHUNK = 10 * 1024 + 8 * 2 * 64 * 16      # score tiles and B^T operands of one chunk


def siso_path(R, Q, np_, bias):
    """Whether the library runs the single-rank scan (bf16, fp32 state, no rotation or bias)."""
    return R == 1 and Q == 64 and np_ == 0 and not bias


def replay_siso(b, L, H, G):
    """The score pass (per batch, group and chunk) and the scan (per batch, head and half
    of P; every chunk, and the inputs it fetches one chunk past the last)."""
    PS = 32
    xb = 8                                            # bytes of the x tile per thread (512 threads)
    nch = -(-L // 64)
    lanes = np.arange(64)
    l16, g4 = lanes & 15, lanes >> 4
    tids = np.arange(512)
    rowb = G * KN * 2
    xrow = H * KP * 2
    BC_bytes = b * L * G * KN * 2
    X_bytes = b * L * H * KP * 2
    T_bytes = b * L * H * 4
    for bi in sorted({0, b - 1}):
        for g in sorted({0, G - 1}):
            for c in sorted({0, nch - 1}):
                c0 = c * 64
                nv = min(64, L - c0)
                base = ((bi * L + c0) * G + g) * KN * 2
                for q in range(4):
                    offs = [(16 * q + l16) * rowb + (32 * ks + 8 * g4) * 2 for ks in range(4)]
                    offs += [(16 * kt + l16) * rowb + (32 * ks + 8 * g4) * 2 for kt in range(q + 1) for ks in range(4)]
                    for what in ("prep C rows", "prep B rows"):
                        _check(what, base, nv * rowb, np.stack(offs), 16, BC_bytes)
                    gath = [(32 * us + key) * rowb + (16 * (2 * q + j) + l16) * 2
                            for j in range(2) for us in range(2) for key in range(32)]
                    _check("prep B gathers", base, nv * rowb, np.asarray(gath), 2, BC_bytes)
        for h in sorted({0, H - 1}):
            g = h * G // H
            tok0 = bi * L
            for ph in range(KP // PS):
                p0 = PS * ph
                xbase = ((tok0 * H + h) * KP + p0) * 2
                xrec = (L - 1) * xrow + PS * 2
                cbase = (tok0 * G + g) * KN * 2
                crec = (L - 1) * rowb + KN * 2
                tbase = (tok0 * H + h) * 4
                trec = ((L - 1) * H + 1) * 4
                for c in sorted({0, max(0, nch - 1), nch}):
                    c0 = c * 64
                    _check("siso x", xbase, xrec, (c0 + (tids >> 3)) * xrow + xb * (tids & 7), xb, X_bytes)
                    for q in range(4):
                        yo = [(c0 + 16 * q + l16) * xrow + (16 * pt + 4 * g4) * 2 for pt in range(PS // 16)]
                        _check("siso y", xbase, xrec, np.stack(yo), 8, X_bytes)
                        co = [(c0 + 16 * q + l16) * rowb + (32 * ks + 8 * g4) * 2 for ks in range(4)]
                        _check("siso C", cbase, crec, np.stack(co), 16, BC_bytes)
                    _check("siso dt, lam", tbase, trec, np.concatenate([(c0 + lanes) * H * 4, [(c0 + 64) * H * 4]]), 4,
                           T_bytes)


def _scan_ws(m3, b, L, H, G, R, Q, np_, nseg):
    d = m3.Desc(b, L, H, G, KP, KN, R, np_, Q, m3.M3_BF16, m3.M3_F32, nseg, m3.M3_RATE_STATIC)
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_scan_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    return n.value


# the GPU parity sweeps (batch 2, 4 heads) and the many-segment cases, then the workloads
SCAN_SHAPES = [
    # b, L, H, G, R, Q, np, nsegments
    (2, 77, 4, 2, 4, 16, 64, 1), (2, 96, 4, 1, 4, 16, 32, 6), (2, 99, 4, 1, 4, 32, 32, 2),
    (2, 150, 4, 1, 4, 64, 32, 1), (2, 250, 4, 1, 4, 64, 32, 3), (2, 64, 4, 1, 4, 64, 0, 1),
    (2, 300, 4, 1, 4, 128, 32, 1), (2, 520, 4, 1, 4, 128, 32, 4), (2, 200, 4, 1, 4, 128, 64, 2),
    (2, 150, 4, 2, 1, 128, 64, 1), (1, 512, 2, 1, 4, 64, 32, 8), (1, 2000, 2, 1, 4, 16, 32, 16),
    (1, 2000, 2, 1, 4, 16, 32, 33), (1, 2000, 2, 1, 4, 16, 32, 100), (1, 1000, 4, 1, 4, 64, 64, 0),
    (1, 300, 2, 1, 2, 32, 32, 0),
]


@pytest.mark.parametrize("shape", SCAN_SHAPES, ids=lambda s: "b%d_L%d_H%d_G%d_R%d_Q%d_np%d_s%d" % s)
def test_scan_resources_stay_in_their_tensors(m3, shape):
    b, L, H, G, R, Q, np_, nsegments = shape
    Qe = executed_chunk(R, Q)
    nseg, seglen = scan_segments(b, H, L, R, Qe, nsegments)
    ws = _scan_ws(m3, b, L, H, G, R, Q, np_, nsegments)
    S = b * H * nseg
    assert ws == (0 if nseg == 1 else S * (2 * KP * KN + 1 + 2 * np_) * 4), "segment schedule differs from the library's"
    replay_scan(b, L, H, G, R, Qe, np_, nseg, seglen)
    replay_scan(b, L, H, G, R, Qe, np_, nseg, seglen, layer=True)


@pytest.mark.parametrize("shape", [(2, 130, 4, 1), (2, 200, 4, 1), (2, 64, 4, 2), (2, 1, 2, 1), (2, 37, 3, 1),
                                   (2, 300, 4, 2), (2, 2048, 2, 1)], ids=lambda s: "b%d_L%d_H%d_G%d" % s)
def test_siso_resources_stay_in_their_tensors(m3, shape):
    """The single-rank path at the shapes its GPU parity cases run."""
    b, L, H, G = shape
    ws = _scan_ws(m3, b, L, H, G, 1, 64, 0, 0)
    assert ws >= b * G * (-(-L // 64)) * SISO_PREP_CHUNK
    replay_siso(b, L, H, G)


@pytest.mark.parametrize("rq", [(1, 64), (2, 32), (2, 64), (4, 16), (4, 32), (4, 64)])
def test_layer_pieces_cover_each_output_once(rq):
    """The layer variant's lanes store every (token, 16-byte piece) of a chunk's
    outputs exactly once, and each key block's share is whole tokens of one slot."""
    R, Q = rq
    n_cons = 8 if (R == 4 and Q == 64) else 4
    pieces = layer_pieces(R, Q, n_cons)
    assert sorted(pieces) == [(t, k) for t in range(Q) for k in range(8)]
    rpb = 32 // n_cons
    npc = 8 * rpb // R
    assert 64 % npc == 0 and rpb % R == 0


@pytest.mark.parametrize("name", ["siso_bf16_mamba2", "mimo_bf16_prefill", "mimo_bf16_long"])
def test_scan_resources_at_the_workloads(m3, name):
    cfg = config_by_name(name)
    b, L, H, G, R, np_ = cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups, cfg.rank, cfg.npairs
    for Q in sorted({cfg.chunk, 16 if R == 4 else cfg.chunk}):
        Qe = executed_chunk(R, Q)
        ws = _scan_ws(m3, b, L, H, G, R, Q, np_, 0)
        nseg, seglen = scan_segments(b, H, L, R, Qe, 0)
        seg_ws = 0 if nseg == 1 else b * H * nseg * (2 * KP * KN + 1 + 2 * np_) * 4
        if siso_path(R, Qe, np_, False):
            # room for either path (the descriptor does not say whether biases come)
            assert ws == max(seg_ws, b * G * (-(-L // 64)) * SISO_PREP_CHUNK), "workspace differs from the library's"
            replay_siso(b, L, H, G)
            if not siso_path(R, Qe, np_, cfg.bias):
                replay_scan(b, L, H, G, R, Qe, np_, nseg, seglen)
            continue
        assert ws == seg_ws
        replay_scan(b, L, H, G, R, Qe, np_, nseg, seglen)
    replay_scan(b, L, H, G, R, executed_chunk(R, cfg.chunk), np_, *scan_segments(b, H, L, R, executed_chunk(R, cfg.chunk), 0),
                layer=True)


# ---------------------------------------------------------------------------
# per-coordinate scan
# ---------------------------------------------------------------------------
def pcs_segments(b, L, D, G, N, nsegments):
    TB = 32
    nblocks = -(-L // TB)
    k = nsegments
    if k == 0:
        tiles = b * (-(-D // 64))
        waves = tiles * (2 if N == 16 else N // 4 * 64 // 64)
        seg_waves = tiles * (1 if N == 16 else N // 4 * 64 // 64)
        k = 1 if waves >= 1024 else min(64, -(-4096 // seg_waves))
    max_rows = (1 << 31) // (max(D, G * N) * 4) - 64
    k = max(k, -(-L // max_rows))
    k = max(1, min(k, max(1, nblocks)))
    seglen = max(1, -(-nblocks // k)) * TB
    return max(1, -(-L // seglen)), seglen


def replay_pcs(b, L, D, G, N, bf16, nseg, seglen):
    ES = 2 if bf16 else 4
    X_bytes, DT_bytes = b * L * D * ES, b * L * D * 4
    BC_bytes = b * L * G * N * ES
    lanes = np.arange(64)
    ntile = -(-D // 64)
    for bi in sorted({0, b - 1}):
        for tile in sorted({0, ntile - 1}):
            d0 = tile * 64
            g = d0 * G // D
            for seg in sorted({0, nseg - 1}):
                T0, T1 = seg * seglen, min(L, seg * seglen + seglen)
                nrow = T1 - T0
                row0 = bi * L + T0
                bx, bd, bbc = row0 * D * ES, row0 * D * 4, row0 * G * N * ES
                if N == 16:
                    # streaming kernel: per-lane x, dt and y of a token row, PF = 16 ahead
                    d = d0 + lanes
                    live = d < D
                    lo = np.where(live, d * ES, 0x7FFFFFF0)
                    lod = np.where(live, d * 4, 0x7FFFFFF0)
                    for r in range(0, nrow + 16):
                        _check("pcs x", bx, nrow * D * ES, lo + r * D * ES, ES, X_bytes)
                        _check("pcs dt", bd, nrow * D * 4, lod + r * D * 4, 4, DT_bytes)
                        _check("pcs y", bx, nrow * D * ES, lo + r * D * ES, ES, X_bytes)
                    # B, C tiles: each wave's half of the coordinates (two waves) or all (one)
                    for NW in (1, 2):
                        K = N // NW
                        PPR = K * ES // 16
                        TP = 16 * PPR
                        e = lanes % TP
                        row, part = e // PPR, e % PPR
                        for w in range(NW):
                            for rt in range(0, nrow + 32, 16):
                                o = ((rt + row) * G + g) * N * ES + w * K * ES + part * 16
                                _check("pcs B/C tile", bbc, nrow * G * N * ES, o, 16, BC_bytes)
                else:
                    # tiled kernel: whole 16-byte pieces of token rows, 32 tokens per block
                    K = 4
                    NT = 64 * (N // K)
                    e = np.arange(NT * 8)
                    for t0 in range(0, nrow + 32, 32):
                        XPR = 64 * ES // 16
                        r, k = e // XPR, e % XPR
                        dd = d0 + k * (16 // ES)
                        ok = (e < 32 * 64 * ES // 16) & (dd < D)
                        _check("pcs tiled x", bx, nrow * D * ES, np.where(ok, ((t0 + r) * D + dd) * ES, 0x7FFFFFF0), 16,
                               X_bytes)
                        _check("pcs tiled y", bx, nrow * D * ES, np.where(ok, ((t0 + r) * D + dd) * ES, 0x7FFFFFF0), 16,
                               X_bytes)
                        DPR = 64 * 4 // 16
                        r, k = e // DPR, e % DPR
                        dd = d0 + k * 4
                        ok = (e < 32 * 64 * 4 // 16) & (dd < D)
                        _check("pcs tiled dt", bd, nrow * D * 4, np.where(ok, ((t0 + r) * D + dd) * 4, 0x7FFFFFF0), 16,
                               DT_bytes)
                        BPR = N * ES // 4
                        r, k = e // BPR, e % BPR
                        ok = e < 32 * N * ES // 4
                        _check("pcs tiled B/C", bbc, nrow * G * N * ES,
                               np.where(ok, ((t0 + r) * G + g) * N * ES + 4 * k, 0x7FFFFFF0), 4, BC_bytes)


PCS_SHAPES = [
    # b, L, D, G, N, bf16, nsegments (the GPU sweep)
    (2, 200, 200, 1, 16, True, 0), (1, 64, 64, 1, 8, True, 0), (2, 130, 256, 2, 32, True, 0),
    (1, 77, 128, 1, 64, True, 0), (2, 150, 100, 1, 16, False, 0), (1, 65, 256, 4, 8, False, 0),
    (1, 1, 64, 1, 16, True, 0), (2, 1000, 128, 1, 16, True, 5), (1, 640, 64, 1, 32, False, 64),
    (1, 3000, 64, 1, 64, True, 64), (1, 96, 128, 2, 8, True, 3), (2, 6000, 128, 1, 16, True, 7),
    (2, 6000, 128, 1, 16, True, 64), (1, 2048, 64, 1, 16, False, 16),
]


def _pcs_ws(m3, b, L, D, G, N, bf16, nsegments):
    d = m3.PcsDesc(b, L, D, G, N, m3.M3_BF16 if bf16 else m3.M3_F32, nsegments)
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_pcs_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    return n.value


@pytest.mark.parametrize("shape", PCS_SHAPES, ids=lambda s: "b%d_L%d_D%d_G%d_N%d_bf%d_s%d" % s)
def test_pcs_resources_stay_in_their_tensors(m3, shape):
    b, L, D, G, N, bf16, nsegments = shape
    nseg, seglen = pcs_segments(b, L, D, G, N, nsegments)
    S = b * D * nseg
    want = 0 if nseg == 1 else ((2 * S * N + S + 63) // 64 * 64) * 4
    assert _pcs_ws(m3, b, L, D, G, N, bf16, nsegments) == want, "segment schedule differs from the library's"
    replay_pcs(b, L, D, G, N, bf16, nseg, seglen)


@pytest.mark.parametrize("name", sorted(PCS_CONFIGS))
def test_pcs_resources_at_the_workloads(m3, name):
    c = PCS_CONFIGS[name]
    b, L, D, G, N = c["batch"], c["seqlen"], c["channels"], c["ngroups"], c["dstate"]
    nseg, seglen = pcs_segments(b, L, D, G, N, 0)
    S = b * D * nseg
    assert _pcs_ws(m3, b, L, D, G, N, True, 0) == (0 if nseg == 1 else ((2 * S * N + S + 63) // 64 * 64) * 4)
    replay_pcs(b, L, D, G, N, True, nseg, seglen)


def test_the_replay_catches_a_head_offset_record_count():
    """The angle resource's record count measured from the head's offset but spanning
    whole tokens of all heads (the form of an earlier out-of-bounds read) fails the
    replay: lanes of pairs past npairs then address floats beyond the tensor."""
    b, L, H, np_ = 1, 64, 4, 32
    h, cst, nt = H - 1, 0, 64
    base = ((b - 1) * L * H + cst * H + h) * np_ * 4
    rec = nt * H * np_ * 4                          # whole tokens from the head's offset
    offs = (np.arange(64)[:, None] * H * np_ + np.arange(64)[None, :]) * 4     # pairs 0 .. 63
    with pytest.raises(AssertionError):
        _check("theta (planted)", base, rec, offs, 4, b * L * H * np_ * 4)


# ---------------------------------------------------------------------------
# backward, chunked form (csrc/bwd_chunk.hip: bf16, P 64, N 128, R 4, 16-token chunks)
# ---------------------------------------------------------------------------
BQ, BR = 16, 4


def bwd_prefetch_pieces():
    """The row prefetch's pieces as prefetch_rows deals them: waves 2..7 issue eight
    16-byte loads per lane, instruction k of wave v covering pieces q0 .. q0 + 63 with
    q0 = 384 k + 64 v; piece q is kind q // 512 (x, dy, the two halves of B, of C),
    thread j = q % 512 of that kind (row j / 8, 16-byte group j % 8)."""
    kinds, js = [], []
    lane = np.arange(64)
    for k in range(8):
        for v in range(6):
            q0 = 384 * k + 64 * v
            kind = q0 >> 9
            assert (q0 + 63) >> 9 == kind       # one kind per instruction
            kinds.append(np.full(64, kind))
            js.append((q0 & 511) + lane)
    kinds, js = np.concatenate(kinds), np.concatenate(js)
    q = kinds * 512 + js
    assert np.array_equal(np.sort(q), np.arange(3072))   # every piece of the LDS buffer once
    return kinds, js


def bwd_state_prefetch_pieces():
    """The state pass's row prefetch (prefetch_xb): all eight waves issue three 16-byte
    loads per lane, instruction k of wave v covering pieces 512 k + 64 v .. + 63 of kind k
    (x, the first and the second half of B), thread j = 64 v + lane of that kind."""
    kinds, js = [], []
    lane = np.arange(64)
    for k in range(3):
        for v in range(8):
            kinds.append(np.full(64, k))
            js.append(64 * v + lane)
    kinds, js = np.concatenate(kinds), np.concatenate(js)
    assert np.array_equal(np.sort(kinds * 512 + js), np.arange(1536))   # every piece once
    return kinds, js


def replay_bwd_chunked(b, L, H, G, np_):
    """The raw per-token loads (theta, dt, lambda, the rate input), the row prefetch
    (x, dy, B, C), the chunk's start phases (from the state pass's workspace) and the
    theta-gradient stores of every edge stream and chunk, and the state pass's x and B row
    prefetch, as load_raw, prefetch_rows, prefetch_xb and the angle phase form them: per-chunk resources whose record counts end at the
    chunk's last valid token."""
    nch = -(-L // BQ)
    tids = np.arange(512)
    kinds, js = bwd_prefetch_pieces()
    m, q8 = js >> 3, js & 7
    t, r = m >> 2, m & 3
    X_bytes = b * L * H * BR * KP * 2
    BC_bytes = b * L * G * BR * KN * 2
    T_bytes = b * L * H * 4
    TH_bytes = b * L * H * np_ * 4
    PH_bytes = b * H * nch * np_ * 4
    lane = np.arange(64)
    kOOB = 0x7ffffff0
    for bi in sorted({0, b - 1}):
        for h in sorted({0, H - 1}):
            gg = h * G // H
            bh = bi * H + h
            for c in sorted({0, nch - 1}):
                c0 = c * BQ
                nv, ns = min(BQ, L - c0), min(BQ + 1, L - c0)
                t0 = (bi * L + c0) * H + h
                if np_ > 0:
                    e = np.concatenate([tids, tids + 512])
                    e = e[e < BQ * np_]
                    te, je = e // np_, e % np_
                    _check("bwd theta", t0 * np_ * 4, ((nv - 1) * H * np_ + np_) * 4, (te * H * np_ + je) * 4, 4,
                           TH_bytes)
                    # d theta: voffset 4 lane (kOOB past np) plus the token's soffset
                    vo = np.where(lane < np_, lane * 4, kOOB)
                    offs = np.concatenate([vo + tt * H * np_ * 4 for tt in range(BQ)])
                    _check("bwd d theta", t0 * np_ * 4, ((nv - 1) * H * np_ + np_) * 4, offs, 4, TH_bytes)
                    _check("bwd start phases", (bh * nch + c) * np_ * 4, np_ * 4, lane * 4, 4, PH_bytes)
                ts = np.arange(BQ + 1)
                _check("bwd dt, lambda, rate", t0 * 4, ((ns - 1) * H + 1) * 4, ts * H * 4, 4, T_bytes)
                xbase = ((bi * L + c0) * H + h) * BR * KP * 2
                xo = (t * H * BR * KP + r * KP + 8 * q8) * 2
                _check("bwd x, dy rows", xbase, ((nv - 1) * H + 1) * BR * KP * 2, xo[kinds < 2], 16, X_bytes)
                bbase = ((bi * L + c0) * G + gg) * BR * KN * 2
                bo = (t * G * BR * KN + r * KN + 16 * q8) * 2 + np.where(kinds & 1, 16, 0)
                _check("bwd B, C rows", bbase, ((nv - 1) * G + 1) * BR * KN * 2, bo[kinds >= 2], 16, BC_bytes)
                # the state pass: x and B rows
                sk, sj = bwd_state_prefetch_pieces()
                sm, sq8 = sj >> 3, sj & 7
                st_, sr = sm >> 2, sm & 3
                sxo = (st_ * H * BR * KP + sr * KP + 8 * sq8) * 2
                _check("bwd state x rows", xbase, ((nv - 1) * H + 1) * BR * KP * 2, sxo[sk == 0], 16, X_bytes)
                sbo = (st_ * G * BR * KN + sr * KN + 16 * sq8) * 2 + np.where(sk == 2, 16, 0)
                _check("bwd state B rows", bbase, ((nv - 1) * G + 1) * BR * KN * 2, sbo[sk >= 1], 16, BC_bytes)


def _bwd_ws(m3, b, L, H, G, np_):
    d = m3.Desc(b, L, H, G, KP, KN, BR, np_, 64, m3.M3_BF16, m3.M3_F32, 0, m3.M3_RATE_STATIC)
    n = ctypes.c_size_t(0)
    assert m3.lib.m3_scan_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    return n.value


# (batch, L, heads, groups, pairs): the chunked form's GPU parity cases, the full-size,
# all-heads and long-sequence tests
BWD_SHAPES = [(1, 1, 2, 1, 32), (2, 16, 2, 2, 64), (1, 17, 3, 1, 7), (2, 45, 2, 1, 0), (1, 80, 2, 1, 32),
              (1, 300, 2, 1, 16), (2, 70, 4, 1, 32), (8, 2048, 64, 1, 32), (1, 256, 64, 1, 32), (1, 16384, 64, 1, 32)]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "b%d_L%d_H%d_G%d_np%d" % s)
def test_bwd_chunked_resources_stay_in_their_tensors(m3, shape):
    b, L, H, G, np_ = shape
    replay_bwd_chunked(b, L, H, G, np_)
    # the workspace holds the B, C sums and every chunk's state and phases
    nch = -(-L // BQ)
    need = 2 * b * L * G * BR * KN * 4 + b * H * nch * (KN * KP * 2 + np_ * 4) + b * H * np_ * 4
    assert _bwd_ws(m3, b, L, H, G, np_) >= need
