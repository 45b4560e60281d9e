"""CPU model of every memory access of the bf16 chunked-prefill kernels' block
ring (k_linear_prefill_bf16 and k_linear_prefill_m32 in
linear_attention_attn_amd/csrc/k_linear.hip, which issue the same loads),
checked against the buffers they may touch.

The kernel streams each (request, head)'s tokens in 32-token blocks through a
3-slot LDS ring: per block, each of the 4 waves issues IPB global-to-LDS loads
of 16 bytes per lane (K, V and Q pieces of RPI rows each, round-robin over the
waves) and, in the gated instantiation, one 4-byte load per lane of the
block's log forget factors; the wave then clears the V rows of its pieces that
lie past the request's end, and reads its operands from the landed slot. This
module recomputes, for every (request, head, block, wave, lane, load), the
global element each load reads and the LDS bytes it and every later LDS access
of the block touch, with the same integer arithmetic as the kernel, and checks
each against the extent of q/k/v/log_gamma and of the dynamic LDS allocation.
It covers the ragged gated case whose earlier load-addressing variant faulted
on the GPU (request lengths 1, 77, 0, 300, 16; H = 8; D = 128), the plain
instantiation of the same case, and shapes of the hybrid and prefill workloads.
"""
import numpy as np
import pytest

BLOCK = 32  # tokens per block of the ring
RING = 3    # slots


def swz(tensor, row, D):
    """Chunk XOR of row `row` of a staged K (0), V (1) or Q (2) tile."""
    if D == 128:
        return [((row >> 3) & 3) | ((row & 3) << 2), ((row & 3) << 1) | (row & 8), row & 15][tensor]
    return [((row >> 3) & 3) | (((row >> 1) & 1) << 2), (row & 2) | (((row >> 3) & 1) << 2),
            (row >> 1) & 7][tensor]


def geometry(D, gated):
    tile = BLOCK * D
    gate = 4 * 64 * 2 if gated else 0
    slot = 3 * tile + gate
    cpr = D // 8
    rpi = 64 // cpr
    ipt = BLOCK // rpi
    ipb = 3 * ipt // 4
    return dict(tile=tile, slot=slot, cpr=cpr, rpi=rpi, ipt=ipt, ipb=ipb,
                lds_bytes=RING * slot * 2)


def model_request(tok0, T, H, D, N, gated, g):
    """Check every access of the (request, head) units of one request of T tokens
    starting at token tok0 of an N-token batch. Returns the number of accesses."""
    if T <= 0:
        return 0  # the kernel returns before any access
    ldx = H * D
    assert ldx < (1 << 23), "the launcher refuses H * D >= 2^23 (24-bit row offsets)"
    tile, slot, cpr, rpi, ipt, ipb = (g[x] for x in ("tile", "slot", "cpr", "rpi", "ipt", "ipb"))
    lds = g["lds_bytes"]
    n_elem = N * H * D  # elements of q, k, v (and o)
    nb = (T + BLOCK - 1) // BLOCK
    lanes = np.arange(64)
    count = 0
    for h in range(H):
        head0 = tok0 * ldx + h * D  # element of the request's first token row, head h
        for b in range(nb):
            sl = b % RING
            last = T - 1 - BLOCK * b
            n = min(BLOCK, T - BLOCK * b)
            for w in range(4):
                for i in range(ipb):
                    tensor = 4 * i // ipt
                    prow = (4 * i) % ipt + w
                    row = prow * rpi + lanes // cpr
                    rr = np.minimum(row, last)
                    assert (rr >= 0).all() and (rr < (1 << 23)).all()
                    x = np.array([swz(tensor, int(r), D) for r in row])
                    off = rr * ldx + 8 * ((lanes % cpr) ^ x)  # 24-bit multiply, 32-bit sum
                    assert (off < (1 << 31)).all()
                    src = head0 + BLOCK * b * ldx + off
                    assert (src >= 0).all() and (src + 8 <= n_elem).all(), (h, b, w, i)
                    # the row read belongs to this request and head
                    tok = src // ldx
                    assert ((tok >= tok0) & (tok < tok0 + T)).all()
                    assert ((src % ldx) // D == h).all()
                    dst = 2 * (sl * slot + tensor * tile + prow * rpi * D) + 16 * lanes
                    assert (dst >= 0).all() and (dst + 16 <= lds).all()
                    assert (dst // (2 * slot) == sl).all(), "a load crosses into another slot"
                    count += 64
                    # clear_tail: V rows past the request's end become zeros
                    if tensor == 1:
                        clr = 2 * (sl * slot + tile + prow * rpi * D + 8 * lanes)
                        assert ((clr >= 2 * sl * slot) & (clr + 16 <= 2 * (sl * slot + 2 * tile))).all()
                if gated:
                    t = np.minimum(BLOCK * b + (lanes & 31), T - 1)
                    gsrc = (tok0 + t) * H + h
                    assert (gsrc >= 0).all() and (gsrc < N * H).all()
                    gdst = 2 * (sl * slot + 3 * tile + w * 128) + 4 * lanes
                    assert (gdst >= 0).all() and (gdst + 4 <= 2 * (sl + 1) * slot).all()
                    count += 64
            # LDS reads of the block: Q and K fragments (rows 0..31 of their tiles) and
            # the transposing reads of V and K^T (rows 8 (l / 16) + (l % 16) / 4, + 4)
            lr, lg = lanes & 15, lanes >> 4
            for s in range(D // 32):
                for t2 in range(2):
                    qrow = 16 * t2 + lr
                    e = qrow * D + 8 * (((32 * s + 8 * lg) >> 3) ^ np.array([swz(2, int(r), D) for r in qrow]))
                    assert ((e >= 0) & (e + 8 <= tile)).all()
                for u in range(2):
                    krow = 8 * (lr >> 2) + 4 * u + (lr & 3)
                    e = krow * D + 8 * (((32 * s + 8 * lg) >> 3) ^ np.array([swz(0, int(r), D) for r in krow]))
                    assert ((e >= 0) & (e + 8 <= tile)).all()
            trow = 8 * lg + (lr >> 2)
            assert (trow + 4 < BLOCK).all()
            count += 1
    return count


CASES = {
    "ragged gated (the faulted case)": dict(lens=(1, 77, 0, 300, 16), H=8, D=128, gated=True),
    "ragged plain": dict(lens=(1, 77, 0, 300, 16), H=8, D=128, gated=False),
    "ragged gated D=64": dict(lens=(1, 77, 0, 300, 16), H=8, D=64, gated=True),
    "block edges": dict(lens=(31, 32, 33, 63, 64, 65, 96), H=2, D=128, gated=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_block_ring_accesses_stay_in_bounds(name):
    c = CASES[name]
    g = geometry(c["D"], c["gated"])
    lens = np.array(c["lens"])
    cu = np.concatenate([[0], np.cumsum(lens)])
    N = int(cu[-1])
    total = sum(model_request(int(cu[r]), int(lens[r]), c["H"], c["D"], N, c["gated"], g)
                for r in range(len(lens)))
    assert total > 0
    # the launcher asks for this much dynamic LDS (two workgroups fit in 160 KiB)
    assert g["lds_bytes"] == RING * (3 * BLOCK * c["D"] + (512 if c["gated"] else 0)) * 2
    assert 2 * g["lds_bytes"] <= 160 * 1024


def test_block_ring_accesses_at_workload_shapes():
    """The first and last blocks of a request at the far end of large batches: the
    hybrid step's 16 x 4096-token prefill and the 8 x 8192-token prefill workload
    (H = 32, D = 128), plain and gated, with a ragged last request."""
    for gated in (False, True):
        g = geometry(128, gated)
        for lens in ((4096,) * 15 + (4095,), (8192,) * 7 + (8161,)):
            lens = np.array(lens)
            cu = np.concatenate([[0], np.cumsum(lens)])
            N = int(cu[-1])
            # model the last request only, on two heads (first and last), every block
            r = len(lens) - 1
            tok0, T = int(cu[r]), int(lens[r])
            for h in (0, 31):
                _model_one_head(tok0, T, 32, 128, N, gated, g, h)


def _model_one_head(tok0, T, H, D, N, gated, g, h):
    """model_request restricted to one head (the far corners of a large batch)."""
    ldx = H * D
    tile, slot, cpr, rpi, ipt, ipb = (g[x] for x in ("tile", "slot", "cpr", "rpi", "ipt", "ipb"))
    lanes = np.arange(64)
    nb = (T + BLOCK - 1) // BLOCK
    for b in (0, nb - 1):
        last = T - 1 - BLOCK * b
        for w in range(4):
            for i in range(ipb):
                tensor = 4 * i // ipt
                prow = (4 * i) % ipt + w
                row = prow * rpi + lanes // cpr
                rr = np.minimum(row, last)
                x = np.array([swz(tensor, int(r), D) for r in row])
                src = tok0 * ldx + h * D + BLOCK * b * ldx + rr * ldx + 8 * ((lanes % cpr) ^ x)
                assert (src >= 0).all() and (src + 8 <= N * H * D).all()
            if gated:
                t = np.minimum(BLOCK * b + (lanes & 31), T - 1)
                assert ((tok0 + t) * H + h < N * H).all()


def perm32(m):
    g = m >> 3
    return 16 * (g >> 1) + 8 * ((m >> 2) & 1) + 4 * (g & 1) + (m & 3)


def test_perm32_is_a_permutation_with_the_stated_lane_layout():
    """Row m of a 32-row operand stands for index perm32(m); the 32x32x16 product's
    accumulator element i of a lane in half h holds row 8 (i / 4) + 4 h + i % 4, so
    that lane must see index 16 (i / 8) + 8 h + i % 8."""
    assert sorted(perm32(m) for m in range(32)) == list(range(32))
    for h in range(2):
        for i in range(16):
            assert perm32(8 * (i // 4) + 4 * h + i % 4) == 16 * (i // 8) + 8 * h + i % 8


def test_m32_fragment_and_state_accesses_stay_in_bounds():
    """Every LDS read of the 32x32-tile kernel (Q and K fragments, transposing
    reads of V and of K, the gated factors) stays inside its tile of the slot,
    and every state and output element it touches lies in the head's D x D state
    and in the block's rows (D = 128)."""
    D, tile = 128, BLOCK * 128
    lanes = np.arange(64)
    lc, hl = lanes & 31, lanes >> 5
    gi, gq = lanes & 15, (lanes >> 4) & 1
    krow = np.array([perm32(int(m)) for m in lc])
    for s in range(8):
        col = 16 * s + 8 * hl
        for rows, t in ((lc, 2), (krow, 0)):
            x = np.array([swz(t, int(r), D) for r in rows])
            e = rows * D + 8 * ((col >> 3) ^ x)
            assert ((e >= 0) & (e + 8 <= tile)).all()
    for w in range(4):
        v0 = 32 * w
        for tensor, bases in ((1, [v0]), (0, [32 * t for t in range(4)])):
            for base in bases:
                for c in range(2):
                    row = 16 * c + 8 * hl + (gi >> 2)
                    col = base + 16 * gq + 8 * (gi & 1) + 4 * ((gi >> 1) & 1)
                    assert (col + 4 <= D).all() and (row + 4 < BLOCK).all()
                    x = np.array([swz(tensor, int(r), D) for r in row])
                    p = row * D + 8 * ((col >> 3) ^ x) + (col & 7)
                    assert ((p >= 0) & (p + 4 + 4 * D <= tile)).all()
                    # within each 16-lane group the transposing read hands lane i
                    # element i % 4 of the chunk that source lane i / 4 (mod 4)
                    # points at: column base + perm32(16 gq + i)
                    for g in range(4):
                        for i in range(16):
                            got = int(col[16 * g + i // 4]) + i % 4
                            assert got == base + perm32(16 * (g & 1) + i), (g, i, base)
        # gated: each wave's 64 floats of forget factors after the three tiles
        gsl = 2 * 3 * tile + 4 * (w * 64 + (lanes & 31))
        assert ((gsl >= 2 * 3 * tile) & (gsl + 4 <= 2 * (3 * tile + 4 * 64 * 2))).all()
        # state: rows 32 t + 16 (i >> 3) + 8 hl + (i & 7), column v0 + perm32(lc)
        vcol = v0 + np.array([perm32(int(m)) for m in lc])
        for t in range(4):
            for i in range(16):
                row = 32 * t + 16 * (i >> 3) + 8 * hl + (i & 7)
                assert ((row >= 0) & (row < D) & (vcol >= 0) & (vcol < D)).all()
        # output: row lc of the block (stored only when lc < n), 16-byte pieces at
        # columns v0 + 8 hl + 16 a
        for a in range(2):
            c0 = v0 + 8 * hl + 16 * a
            assert ((c0 >= 0) & (c0 + 8 <= D)).all()
    # the state elements the four waves hold are each of the D x D elements once
    seen = np.zeros((D, D), int)
    for w in range(4):
        vcol = 32 * w + np.array([perm32(int(m)) for m in lc])
        for t in range(4):
            for i in range(16):
                seen[32 * t + 16 * (i >> 3) + 8 * hl + (i & 7), vcol] += 1
    assert (seen == 1).all()
