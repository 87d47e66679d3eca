"""CPU model of every global load and store the lookup-combine kernels issue,
checked against the allocations they touch (no GPU).

For each launch shape the library's dispatch picks (token ids in [0, V) are
the caller's contract), the model enumerates every lane of every workgroup
and evaluates the address expressions of combine_dense.hip,
combine_common.hpp (the matrix-core and vector-unit routers, the staged
gates), combine_nf3.hip (NF3 / NF4 / int8 code and scale loads) and
combine_grouped.hip, including the clamps that make unconditional loads
safe, and asserts that each access [offset, offset + width) lies inside its
buffer.  The sweep covers N = 1..64, D not a multiple of the 16-byte chunk
or of the router's 32-wide K step, and batches on both sides of every
dispatch threshold.

The model is written from the kernels' index arithmetic; it is a check of
that arithmetic (and of the dispatch limits), not of the compiled code.
One case replays the matrix-core router without its expert clamp: with
N < 16 the padded expert rows of the 16-wide tile read past W_r, the
address fault a router of that form takes.
"""
import numpy as np
import pytest

BF16, F32 = 2, 4
WAVE = 64
MAX_TPB = 16


def next_pow2(x):
    p = 1
    while p < x:
        p <<= 1
    return p


def pick_group(C, lo, hi):
    G = lo
    while G < C and G < hi:
        G <<= 1
    return G


def pick_tokens_per_block(T, G):
    tpb = min(256 // G, 16)
    min_tpb = 1 if G >= 64 else 64 // G
    while tpb > min_tpb and (T + tpb - 1) // tpb < 512:
        tpb >>= 1
    return tpb


class Buffers:
    """Byte sizes of the buffers a combine touches; records every access."""

    def __init__(self, **sizes):
        self.size = sizes
        self.bad = []

    def access(self, name, off, width):
        off = np.asarray(off, dtype=np.int64)
        if off.size == 0:
            return
        lo, hi = int(off.min()), int(off.max()) + width
        if lo < 0 or hi > self.size[name]:
            self.bad.append((name, lo, hi, self.size[name]))


def lanes(blocks, threads):
    b = np.repeat(np.arange(blocks, dtype=np.int64), threads)
    tid = np.tile(np.arange(threads, dtype=np.int64), blocks)
    return b, tid


# ----------------------------------------------------------------------------
# routers (combine_common.hpp)
# ----------------------------------------------------------------------------

def mfma_router_loads(buf, b, tid, t0, T, tpb, D, N, NP, nwaves, clamp_expert=True, ub=0, one_batch=False):
    """MfmaRouter: lane l of wave w supplies token row l%16 and expert column
    l%16 with 8 consecutive d of k-group l/16; the waves take every nw-th
    32-wide K step, UB steps per batch (ub overrides, as the wide blocks'
    router does; one_batch: only the first batch, which must then cover the
    row)."""
    NT = (NP + 15) // 16
    UB = ub if ub else (8 if NT == 1 else (4 if NT == 2 else 2))
    if one_batch:
        assert (D + 31) // 32 <= UB * nwaves, "one batch of K steps must cover the row"
    lane = tid & 63
    wave = tid >> 6
    row, kg = lane & 15, lane >> 4
    tok = t0 + row
    tok_ok = (row < tpb) & (tok < T)
    hrow = np.where(tok_ok, tok, 0) * D
    ksteps = (D + 31) // 32
    base = wave.copy()
    while True:
        active = base < ksteps
        if not active.any():
            break
        for u in range(UB):
            ks = base + u * nwaves
            k_ok = (ks < ksteps) & (ks * 32 + kg * 8 < D)
            kc = np.where(k_ok, ks * 32 + kg * 8, 0)
            buf.access("h", ((hrow + kc) * BF16)[active], 16)
            for nt in range(NT):
                e = nt * 16 + row
                ec = np.where(e < N, e, N - 1) if clamp_expert else e
                buf.access("w_r", ((ec * D + kc) * BF16)[active], 16)
        if one_batch:
            break
        base = base + UB * nwaves


def lane_router_loads(buf, tt, lig, G, D, N, NP, esz, valid):
    """LaneRouter: load_first from clamped chunk and expert indices, then the
    further chunks (r = lig + G, ...) of lanes inside the row."""
    V = 16 // esz
    C = D // V
    c = np.minimum(lig, C - 1)
    buf.access("h", (tt * D + c * V) * esz, 16)
    for e in range(NP):
        buf.access("w_r", (min(e, N - 1) * D + c * V) * esz, 16)
    ok = valid & (lig < C)
    r = lig + G
    while True:
        m = ok & (r < C)
        if not m.any():
            break
        buf.access("h", ((tt * D + r * V) * esz)[m], 16)
        for e in range(min(NP, N)):
            buf.access("w_r", ((e * D + r * V) * esz)[m], 16)
        r = r + G


def elementwise_router_loads(buf, tt, lig, G, D, N, NP, esz, valid, vector=False):
    """router_partials: 16-byte chunks r = lig, lig + G, ... < D / V of aligned
    rows, else single elements d = lig, lig + G, ... < D."""
    V = 16 // esz if vector else 1
    d = lig.copy()
    while True:
        m = valid & (d < D // V)
        if not m.any():
            break
        buf.access("h", ((tt * D + d * V) * esz)[m], V * esz)
        for e in range(min(NP, N)):
            buf.access("w_r", ((e * D + d * V) * esz)[m], V * esz)
        d = d + G


# ----------------------------------------------------------------------------
# dense table (combine_dense.hip)
# ----------------------------------------------------------------------------

def dense_plan(T, D, N, esz):
    NP = next_pow2(N)
    vec = 16 // esz
    vector = D % vec == 0
    C = D // vec if vector else D
    G = pick_group(C, 16, 256)
    bf = esz == BF16
    one_token = vector and bf and NP <= 16 and G >= 64 and T <= 1024
    tpb = 1 if one_token else pick_tokens_per_block(T, G)
    if vector and bf and NP <= 16 and G >= 128 and T >= 1024 and C <= G:
        # four tokens per workgroup of 4 G threads, matrix-core router
        return dict(NP=NP, vector=vector, C=C, G=G, tpb=4, mode="wide", CH=vec)
    if vector and bf and T >= 2048 and tpb >= 2 and NP <= D:
        mode = "staged"
    elif vector and bf and NP <= 16 and G >= 64 and tpb == 1:
        mode = "lane"
    elif vector and bf:
        mode = "mfma"
    elif vector and NP <= 16:
        mode = "lane"
    else:
        mode = "elementwise"
    return dict(NP=NP, vector=vector, C=C, G=G, tpb=tpb, mode=mode, CH=vec if vector else 1)


def model_dense(T, V, D, N, esz, ids, clamp_expert=True):
    p = dense_plan(T, D, N, esz)
    NP, G, tpb, C, CH = p["NP"], p["G"], p["tpb"], p["C"], p["CH"]
    buf = Buffers(ids=8 * T, h=T * D * esz, w_r=N * D * esz, lut=V * N * D * esz, y=T * D * 4)
    blocks = (T + tpb - 1) // tpb
    b, tid = lanes(blocks, G * tpb)
    grp, lig = tid // G, tid % G
    t0 = b * tpb
    t = t0 + grp
    valid = t < T
    tt = np.where(valid, t, 0)
    buf.access("ids", tt * 8, 8)
    if p["mode"] == "mfma":
        mfma_router_loads(buf, b, tid, t0, T, tpb, D, N, NP, (G * tpb) // WAVE, clamp_expert)
    elif p["mode"] == "wide":
        mfma_router_loads(buf, b, tid, t0, T, tpb, D, N, NP, (G * tpb) // WAVE, clamp_expert, ub=4, one_batch=True)
    elif p["mode"] == "lane":
        lane_router_loads(buf, tt, lig, G, D, N, NP, esz, valid)
    elif p["mode"] == "staged":
        for q in range((NP + 3) // 4):
            buf.access("y", (tt * D + 4 * q) * 4, 16)
    else:
        elementwise_router_loads(buf, tt, lig, G, D, N, NP, esz, valid, p["vector"])
    idv = ids[tt]
    slab = idv * N * D
    EC = min(NP, 16)
    c0 = np.minimum(lig, C - 1)
    for e in range(EC):
        ec = min(e, N - 1)
        buf.access("lut", (slab + ec * D + c0 * CH) * esz, 16 if p["vector"] else esz)
    k = 0
    while True:
        c = k * G + lig
        m = valid & (c < C)
        if not m.any():
            break
        for e in range(min(NP, N)):
            buf.access("lut", ((slab + e * D + c * CH) * esz)[m], 16 if p["vector"] else esz)
        buf.access("y", ((tt * D + c * CH) * 4)[m], 4 * CH)
        k += 1
    return p, buf


# ----------------------------------------------------------------------------
# quantised tables (combine_nf3.hip)
# ----------------------------------------------------------------------------

QFMT = {  # chunk bytes (32 elements), row bytes, scale bytes per row, batch
    "nf3": (12, lambda D: 3 * D // 8, lambda D: 2 * (D // 64), 8),
    "nf4": (16, lambda D: D // 2, lambda D: 2 * (D // 64), 4),
    "int8": (32, lambda D: D, lambda D: 4, 4),
}


def q_plan(fmt, T, D, N, esz):
    NP = next_pow2(N)
    CP = pick_group(D // 32, 8, 64)
    S = min(64 // CP, NP)
    G = CP * S
    bf = esz == BF16
    full_wave = G == WAVE and bf and NP <= 16
    one_token = full_wave and T < 1024
    # four or eight tokens per workgroup of full wavefronts (eight where that
    # takes no more rounds of token slots over the 256 compute units)
    r8, r4 = ((T + 7) // 8 + 255) // 256, ((T + 3) // 4 + 255) // 256
    tpb = 1 if one_token else ((8 if 8 * r8 <= 4 * r4 else 4) if full_wave else pick_tokens_per_block(T, G))
    W = 1
    if bf and NP <= 16 and tpb == 1 and G == WAVE:
        while W < 4 and 2 * W * S <= NP and T * 2 * W <= 2 * 1024:
            W *= 2
    if bf and NP <= 16 and tpb == 1:
        mode = "lane"
    elif bf:
        mode = "mfma"
    elif NP <= 16:
        mode = "lane"
    else:
        mode = "elementwise"
    return dict(NP=NP, CP=CP, S=S, G=G, tpb=tpb, W=W, mode=mode)


def model_q(fmt, T, V, D, N, esz, ids):
    chunk, row_bytes_f, srow_f, batch = QFMT[fmt]
    p = q_plan(fmt, T, D, N, esz)
    NP, CP, S, G, tpb, W = p["NP"], p["CP"], p["S"], p["G"], p["tpb"], p["W"]
    rb, sb = row_bytes_f(D), srow_f(D)
    buf = Buffers(ids=8 * T, h=T * D * esz, w_r=N * D * esz, codes=V * N * rb, scales=V * N * sb, y=T * D * 4)
    threads = G * W if W > 1 else G * tpb
    blocks = (T + tpb - 1) // tpb
    b, tid = lanes(blocks, threads)
    grp, lig = tid // G, tid % G
    sp, ch = lig // CP, lig % CP
    wsp = grp if W > 1 else 0
    t0 = b * tpb
    t = t0 if W > 1 else t0 + grp
    valid = t < T
    tt = np.where(valid, t, 0)
    buf.access("ids", (tt * 8)[valid], 8)
    idv = np.where(valid, ids[tt], 0)
    C = D // 32
    EPL = (NP + S * W - 1) // (S * W)
    EC = min(EPL, batch)

    def load_batch(c, j0, m):
        for j in range(EC):
            e = ((j0 + j) * W + wsp) * S + sp
            mm = m & (e < N)
            buf.access("codes", (idv * N * rb + e * rb + c * chunk)[mm], chunk)
            if fmt == "int8":
                buf.access("scales", ((idv * N + e) * 4)[mm], 4)
            else:
                buf.access("scales", ((idv * N * (D // 64) + e * (D // 64) + (c >> 1)) * 2)[mm], 2)

    if p["mode"] == "mfma" and G == WAVE and W == 1:
        # one token per wavefront: router operands first, then the first
        # batch branch-free (expert and chunk clamped, every lane loads);
        # eight-wavefront blocks take 4 K steps per wavefront and batch
        ub = 2048 // (G * tpb) if (NP <= 16 and G * tpb > 256) else 0
        mfma_router_loads(buf, b, tid, t0, T, tpb, D, N, NP, (G * tpb) // WAVE, ub=ub)
        cc = np.minimum(ch, C - 1)
        for j in range(EC):
            e = (j * W + wsp) * S + sp
            ec = np.minimum(e, N - 1)
            buf.access("codes", idv * N * rb + ec * rb + cc * chunk, chunk)
            if fmt == "int8":
                buf.access("scales", (idv * N + ec) * 4, 4)
            else:
                buf.access("scales", (idv * N * (D // 64) + ec * (D // 64) + (cc >> 1)) * 2, 2)
    else:
        load_batch(ch, 0, valid & (ch < C))
    if p["mode"] == "mfma" and not (G == WAVE and W == 1):
        mfma_router_loads(buf, b, tid, t0, T, tpb, D, N, NP, (G * tpb) // WAVE)
    elif p["mode"] == "lane":
        lane_router_loads(buf, tt, tid if W > 1 else lig, G * W if W > 1 else G, D, N, NP, esz, valid)
    else:
        elementwise_router_loads(buf, tt, lig, G, D, N, NP, esz, valid)
    rounds = (C + CP - 1) // CP
    OUT = 32 // S
    OW = OUT // W
    for k in range(rounds):
        c = k * CP + ch
        act = valid & (c < C)
        for j0 in range(0, EPL, EC):
            if k != 0 or j0 != 0:
                load_batch(c, j0, act)
        # output: the lane's share of the chunk after the split reduce
        off = np.zeros_like(sp)
        bit, span = 0, 16
        while (1 << bit) < S:
            off = off + np.where((sp >> bit) & 1, span, 0)
            bit += 1
            span //= 2
        buf.access("y", ((tt * D + c * 32 + off + wsp * OW) * 4)[act], 4 * OW)
    return p, buf


# ----------------------------------------------------------------------------
# grouped combine (combine_grouped.hip)
# ----------------------------------------------------------------------------

def group_route_accesses(buf, T, D, N, NP):
    """The grouping and routing launch (group_route_kernel)."""
    # grouping workgroups: one per 4096-token chunk, 1024 threads, 4 tokens each
    nchunks = (T + 4095) // 4096
    b, tid = lanes(nchunks, 1024)
    for i in range(4):
        q = tid + i * 1024
        base = b * 4096
        ln = np.minimum(T - base, 4096)
        buf.access("ids", (base + np.where(q < ln, q, 0)) * 8, 8)
        buf.access("pos", ((base + q) * 4)[q < ln], 4)  # written at a position of the chunk
    # routing workgroups: 16 tokens each, 16 wavefronts splitting D
    rt = (T + 15) // 16
    b, tid = lanes(rt, 1024)
    mfma_router_loads(buf, b, tid, b * 16, T, 16, D, N, NP, 16)
    gi = b * 16 * NP + tid
    buf.access("gates", (gi * 4)[(tid < 16 * NP) & (b * 16 + tid // NP < T)], 4)


def model_grouped(T, V, D, N, ids):
    NP = next_pow2(N)
    buf = Buffers(ids=8 * T, h=T * D * 2, w_r=N * D * 2, lut=V * N * D * 2, y=T * D * 4,
                  pos=4 * T, gates=T * 16 * 4)
    group_route_accesses(buf, T, D, N, NP)
    # combine: one workgroup per position; positions hold a permutation of the tokens
    order = np.argsort(ids, kind="stable")
    rows = ids[order]
    C = D // 8
    lanes_n = 64 if C <= 64 else (128 if C <= 128 else 256)
    b, tid = lanes(T, lanes_n)
    buf.access("pos", b * 4, 4)
    buf.access("pos", ((b - 1) * 4)[b > 0], 4)
    start = (b == 0) | (b % 16 == 0) | (rows[np.maximum(b - 1, 0)] != rows[b])
    slab = rows[b] * N * D
    cc = np.minimum(tid, C - 1)
    for e in range(NP):
        buf.access("lut", ((slab + min(e, N - 1) * D + cc * 8) * 2)[start], 16)
    lim = np.minimum((b // 16 + 1) * 16, T)
    ln = np.ones_like(b)
    for _ in range(16):
        nxt = b + ln
        ok = start & (nxt < lim)
        buf.access("pos", (np.minimum(nxt, T - 1) * 4)[ok], 4)
        same = ok & (rows[np.minimum(nxt, T - 1)] == rows[b])
        ln = ln + same
    for q in range(16):
        m = start & (q < ln)
        tok = order[np.minimum(b + q, T - 1)]
        for e in range(NP):
            buf.access("gates", ((tok * NP + e) * 4)[m & (tid == 0)], 4)
        c = tid.copy()
        while True:
            mc = m & (c < C)
            if not mc.any():
                break
            buf.access("y", ((tok * D + c * 8) * 4)[mc], 32)
            c = c + lanes_n
    return buf


def model_nf3_grouped(T, V, D, N, ids):
    """The NF3 combine over the grouped positions (lookup_combine_nf3_grouped_kernel):
    one position per wavefront, four per workgroup; lane (s, c) decodes chunk
    c (+ CP per round) of experts s, s + S, ...; loads guarded by c < C and
    e < N, gates at gates[token][NP], staged 16-byte stores of the row."""
    NP = next_pow2(N)
    rb, sb = 3 * D // 8, D // 64
    buf = Buffers(ids=8 * T, h=T * D * 2, w_r=N * D * 2, codes=V * N * rb, scales=V * N * sb * 2, y=T * D * 4,
                  pos=4 * T, gates=T * 16 * 4)
    group_route_accesses(buf, T, D, N, NP)
    C = D // 32
    CP = pick_group(C, 8, 64)
    while CP * NP < 64:
        CP *= 2
    S = 64 // CP
    EPL = (NP + S - 1) // S
    order = np.argsort(ids, kind="stable")
    b, tid = lanes((T + 3) // 4, 256)
    p = b * 4 + tid // 64
    lane = tid % 64
    live = p < T
    pc = np.minimum(p, T - 1)
    buf.access("pos", (pc * 4)[live], 4)
    tok, row = order[pc], ids[order[pc]]
    sp, ch = lane // CP, lane % CP
    for j in range(EPL):
        e = j * S + sp
        buf.access("gates", ((tok * NP + e) * 4)[live & (e < N)], 4)
    rounds = (C + CP - 1) // CP
    for k in range(rounds):
        c = k * CP + ch
        act = live & (c < C)
        for j in range(EPL):
            e = j * S + sp
            m = act & (e < N)
            buf.access("codes", (row * N * rb + e * rb + c * 12)[m], 12)
            buf.access("scales", ((row * N * sb + e * sb + (c >> 1)) * 2)[m], 2)
        for q in range(max(CP * 32 // 256, 1)):
            el = k * CP * 32 + 4 * lane + 256 * q
            buf.access("y", ((tok * D + el) * 4)[live & (el < D)], 16)
    return buf


# ----------------------------------------------------------------------------
# sweeps
# ----------------------------------------------------------------------------

def ids_for(T, V, seed):
    r = np.random.default_rng(seed)
    ids = r.integers(0, V, T).astype(np.int64)
    ids[: min(T, 3)] = [0, V - 1, V // 2][: min(T, 3)]  # table edges
    return ids


NS = [1, 3, 4, 5, 8, 12, 16, 17, 33, 64]
DS_BF16 = [8, 24, 136, 1000, 1032, 2048, 4096, 60, 30]
TS = [1, 17, 1023, 1024, 1025, 2051]


@pytest.mark.parametrize("esz", [BF16, F32])
def test_dense_combine_loads_stay_in_bounds(esz):
    V = 97
    for N in NS:
        for D in DS_BF16:
            for T in TS:
                if esz == F32 and T > 1025:
                    continue
                p, buf = model_dense(T, V, D, N, esz, ids_for(T, V, N + D + T))
                assert not buf.bad, (N, D, T, p, buf.bad[:3])


@pytest.mark.parametrize("fmt", ["nf3", "nf4", "int8"])
def test_quantised_combine_loads_stay_in_bounds(fmt):
    V = 41
    for N in NS:
        for D in (64, 192, 1024, 2048, 4096):
            for T in (1, 17, 1023, 1024, 1025, 2047, 2049, 4097):
                for esz in (BF16, F32):
                    if esz == F32 and T > 17:
                        continue
                    if T in (2047, 4097) and (D > 1024 or N not in (4, 12, 16)):
                        continue  # the eight-token launch: a few shapes keep the CPU model quick
                    p, buf = model_q(fmt, T, V, D, N, esz, ids_for(T, V, N + D + T))
                    assert not buf.bad, (fmt, N, D, T, esz, p, buf.bad[:3])


def test_grouped_combine_loads_stay_in_bounds():
    V = 50
    for N in (1, 3, 4, 8, 16):
        for D in (8, 64, 136, 1024, 2048, 4096):
            for T in (1, 16, 17, 300, 4097):
                buf = model_grouped(T, V, D, N, ids_for(T, V, N + D + T))
                assert not buf.bad, (N, D, T, buf.bad[:3])


def test_nf3_grouped_combine_loads_stay_in_bounds():
    V = 50
    for N in (1, 2, 3, 4, 8, 16):
        for D in (64, 192, 1024, 2048, 4096):
            for T in (1, 5, 17, 300, 4097):
                buf = model_nf3_grouped(T, V, D, N, ids_for(T, V, N + D + T))
                assert not buf.bad, (N, D, T, buf.bad[:3])


def test_router_without_expert_clamp_reads_past_w_r():
    """The matrix-core router tile is 16 experts wide; N = 4 pads it with 12
    expert rows.  Without the clamp to N - 1 those rows are read past the end
    of W_r (N x D), the out-of-bounds read behind an aperture fault of a
    combine of that form: 256 one-token workgroups of 128 lanes (N = 4,
    D = 768, T = 256), and the several-token launches the dispatch still
    sends to this router.  With the clamp every load stays inside."""
    T, V, D, N = 256, 64, 768, 4
    for clamp in (True, False):
        buf = Buffers(h=T * D * BF16, w_r=N * D * BF16)
        b, tid = lanes(T, 128)
        mfma_router_loads(buf, b, tid, b, T, 1, D, N, next_pow2(N), 2, clamp_expert=clamp)
        if clamp:
            assert not buf.bad
        else:
            assert buf.bad and all(name == "w_r" and hi > size for name, lo, hi, size in buf.bad)
    T = 1025  # past the one-token limit: several tokens per block, matrix-core router
    ids = ids_for(T, V, 1)
    p, buf = model_dense(T, V, D, N, BF16, ids)
    assert p["mode"] in ("mfma", "wide") and p["tpb"] >= 2 and not buf.bad
    _, bad = model_dense(T, V, D, N, BF16, ids, clamp_expert=False)
    assert bad.bad and all(name == "w_r" for name, *_ in bad.bad)
