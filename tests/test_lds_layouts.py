"""Host replay of the LDS and DMA address arithmetic of the attention kernels
(forward and backward), for every head dim and block size built.  No GPU:
the index formulas of the kernels are evaluated here for every lane, wave and
load, and checked to stay inside the tiles they address.

Checked: the XOR swizzles are bijections on a row's 16-byte chunks; a K or V
tile's DMA pieces (forward: issue_tile / tile_lane_offset; backward:
load_tile) write every byte of the tile exactly once and nothing outside it;
the backward's row-statistics DMA covers its 2 * block floats exactly once;
every MFMA operand read (forward K rows, V^T transposed reads; backward
row-major and transposed reads of 32-row sub-blocks) lands inside its tile.
The formulas mirror
dynamic_block_sparse_dsa_amd/csrc/attn_common.hpp, attn_fwd.hip and
attn_bwd.hip.
"""

import itertools

import pytest

DIMS = (64, 128)
BLOCKS = (64, 128)


def kswz(D, r):
    return (r & 15) if D == 128 else ((r >> 1) & 7)


def vswz(D, r):
    return 4 * (r & 3) if D == 128 else 4 * ((r >> 1) & 1)


def qswz(D, r):
    return 4 * (r & 3) + ((r >> 2) & 3) if D == 128 else 4 * ((r >> 1) & 1) + ((r >> 2) & 3)


@pytest.mark.parametrize("D", DIMS)
def test_swizzles_are_chunk_bijections(D):
    CH = D // 8
    for sw in (kswz, vswz, qswz):
        for r in range(256):
            assert sorted(c ^ sw(D, r) for c in range(CH)) == list(range(CH)), (sw.__name__, r)


def fwd_cfg(D, BLK, HG):
    slabs = BLK // 32
    waves = HG * slabs
    loads = BLK * D * 2 // 1024
    assert loads % waves == 0
    return dict(waves=waves, rpi=1024 // (2 * D), ch=D // 8, loads=loads, lpw=loads // waves)


@pytest.mark.parametrize("D,BLK,HG", [(d, b, hg) for d in DIMS for b in BLOCKS for hg in ((1, 2, 4) if b == 64 else (1, 2))])
def test_forward_tile_dma_writes_each_byte_once(D, BLK, HG):
    c = fwd_cfg(D, BLK, HG)
    tile_bytes = BLK * D * 2
    for v_swizzle in (False, True):
        written = [0] * (tile_bytes // 16)
        for wave, n, lane in itertools.product(range(c["waves"]), range(c["lpw"]), range(64)):
            inst = wave + n * c["waves"]
            r = inst * c["rpi"] + lane // c["ch"]
            ch = (lane % c["ch"]) ^ (vswz(D, r) if v_swizzle else kswz(D, r))
            src = (r * D + ch * 8) * 2           # byte offset of the source chunk in the tile's rows
            dst = inst * 1024 + 16 * lane        # LDS byte offset the lane's 16 bytes land at
            assert 0 <= src < tile_bytes and src % 16 == 0
            assert 0 <= dst < tile_bytes
            written[dst // 16] += 1
            # the destination slot holds row r, chunk (lane % CH) swizzled: the reads below undo it
            assert dst == r * D * 2 + (lane % c["ch"]) * 16
        assert written == [1] * len(written)


@pytest.mark.parametrize("D,BLK", [(d, b) for d in DIMS for b in BLOCKS])
def test_forward_operand_reads_stay_in_the_tile(D, BLK):
    tile_elems = BLK * D
    for lane in range(64):
        half = lane >> 5
        # K rows (A operand of S^T): row kr, k-step ks
        for st, ks in itertools.product(range(BLK // 32), range(D // 16)):
            kr = st * 32 + (lane & 31)
            ch = (2 * ks + half) ^ kswz(D, kr)
            e = kr * D + ch * 8
            assert 0 <= e and e + 8 <= tile_elems
        # V^T transposed reads: d-tile dt, key-step kk, two 8-byte reads
        grp, si = (lane >> 4) & 1, lane & 15
        for dt, kk, sg in itertools.product(range(D // 32), range(BLK // 16), range(2)):
            d = dt * 32 + 16 * grp + 4 * (si & 3)
            key = 16 * kk + 8 * sg + 4 * half + (si >> 2)
            ch = (d >> 3) ^ vswz(D, key)
            byte = (key * D + ch * 8) * 2 + (d & 7) * 2
            assert 0 <= byte and byte + 8 <= tile_elems * 2 and key < BLK


def vtsw(D, r):
    return 2 * ((r & 3) + 4 * ((r >> 2) & 1)) if D == 128 else 2 * (((r >> 1) & 1) + 2 * ((r >> 2) & 1))


@pytest.mark.parametrize("D", DIMS)
def test_token_attention_v_tile(D):
    """Token attention (indexer.hip, token_attn_kernel): the V DMA of a
    32-key chunk writes each byte of the wave's tile once; every transposed
    read returns V[key][d] for the d and key order the MFMA expects (A operand
    of O^T += V^T P^T: lane 16 g + i holds dim 16 db + i, slot 4 sg + j key
    4 g + 16 sg + j -- the order P leaves the S accumulators in); and the 32
    lanes of two groups read 64 distinct four-byte banks."""
    CK, CH = 32, D // 8
    rpi, nl = 64 // CH, 32 // (64 // CH)
    tile = [None] * (CK * D)  # logical (row, d) held by each bf16 slot
    for i, lane in itertools.product(range(nl), range(64)):
        rr = i * rpi + lane // CH
        ch = (lane % CH) ^ vtsw(D, rr)
        dst = i * 1024 + 16 * lane
        assert dst == rr * D * 2 + (lane % CH) * 16
        for e in range(8):
            assert tile[dst // 2 + e] is None
            tile[dst // 2 + e] = (rr, ch * 8 + e)
    assert all(x is not None for x in tile)
    for db, sg in itertools.product(range(D // 16), range(2)):
        banks = {0: [], 1: []}
        got = {}
        for lane in range(64):
            g, s = lane >> 4, lane & 15
            r = 4 * g + 16 * sg + (s >> 2)
            d0 = db * 16 + 4 * (s & 3)
            byte = r * D * 2 + ((d0 >> 3) ^ vtsw(D, r)) * 16 + (d0 & 7) * 2
            assert byte % 8 == 0 and 0 <= byte and byte + 8 <= CK * D * 2
            banks[lane >> 5] += [(byte // 4) % 64, (byte // 4 + 1) % 64]
            for e in range(4):  # destination lane 16 g + 4 (s & 3) + e, slot s >> 2
                got[(16 * g + 4 * (s & 3) + e, s >> 2)] = tile[byte // 2 + e]
        for half in (0, 1):
            assert sorted(banks[half]) == list(range(64)), (db, sg, half)
        for lane in range(64):
            g, i = lane >> 4, lane & 15
            for j in range(4):
                assert got[(lane, j)] == (4 * g + 16 * sg + j, 16 * db + i)


@pytest.mark.parametrize("D", DIMS)
def test_decode_v_tile(D):
    """Decode (decode_common.hpp, WaveAttn::step): the wave's V rows go from
    registers into its LDS tile -- lane (pk, pc) = (lane / (D/8), lane % (D/8))
    writes dims 8 pc .. 8 pc + 7 of rows pk + (64 / (D/8)) v at chunk
    pc ^ dec_vsw(row) -- covering each bf16 slot of the tile once; the
    transposed reads (the same addressing as the token attention's) then return
    V[key][d] in the MFMA A-operand order that matches the P layout (lane
    16 g + i: dim 16 db + i, slot 4 sg + j: key 4 g + 16 sg + j)."""
    CK, CHK = 32, D // 8
    KGR = 64 // CHK
    VPL = CK // KGR
    tile = [None] * (CK * D)
    for lane, v in itertools.product(range(64), range(VPL)):
        pk, pc = lane // CHK, lane % CHK
        rr = pk + KGR * v
        ch = pc ^ vtsw(D, rr)
        assert 0 <= ch < CHK
        for e in range(8):
            slot = rr * D + ch * 8 + e
            assert tile[slot] is None
            tile[slot] = (rr, pc * 8 + e)
    assert all(x is not None for x in tile)
    for db, sg in itertools.product(range(D // 16), range(2)):
        for lane in range(64):
            g, s_ = lane >> 4, lane & 15
            r = 4 * g + 16 * sg + (s_ >> 2)
            d0 = db * 16 + 4 * (s_ & 3)
            byte = r * D * 2 + ((d0 >> 3) ^ vtsw(D, r)) * 16 + (d0 & 7) * 2
            assert byte % 8 == 0 and 0 <= byte and byte + 8 <= CK * D * 2
            for e in range(4):  # destination lane 16 g + 4 (s & 3) + e, slot 4 sg + (s >> 2)
                dst_lane, slot = 16 * g + 4 * (s_ & 3) + e, s_ >> 2
                key, d = tile[byte // 2 + e]
                assert (key, d) == (4 * g + 16 * sg + slot, 16 * db + (dst_lane & 15))


def bwd_kv_cfg(D, BLK):
    kg = BLK // 32
    qs = 2 if BLK == 64 else 1
    waves = kg * qs
    tile = BLK * D
    stage = 2 * tile * 2 + 2 * BLK * 4
    nbuf = 4 if 4 * stage <= 136 * 1024 else 3 if 3 * stage <= 136 * 1024 else 2
    return dict(waves=waves, tile=tile, nbuf=nbuf, stat_bpw=2 * BLK * 4 // waves, qb_per_wave=(BLK // 32) // qs, qs=qs)


@pytest.mark.parametrize("D,BLK", [(d, b) for d in DIMS for b in BLOCKS])
def test_backward_stage_dma_and_reads_stay_in_their_buffers(D, BLK):
    c = bwd_kv_cfg(D, BLK)
    assert c["nbuf"] * (2 * c["tile"] * 2 + 2 * BLK * 4) <= 160 * 1024
    # load_tile: every byte of a stage tile once
    rpi, ch_n = 1024 // (2 * D), D // 8
    loads = BLK * D * 2 // 1024
    assert loads % c["waves"] == 0
    written = [0] * (c["tile"] * 2 // 16)
    for wave, n, lane in itertools.product(range(c["waves"]), range(loads // c["waves"]), range(64)):
        inst = wave + n * c["waves"]
        r = inst * rpi + lane // ch_n
        ch = (lane % ch_n) ^ qswz(D, r)
        assert 0 <= (r * D + ch * 8) * 2 < c["tile"] * 2
        written[(inst * 1024 + 16 * lane) // 16] += 1
    assert written == [1] * len(written)
    # row statistics: one DMA per wave, 16 bytes per active lane
    assert c["stat_bpw"] % 16 == 0 and c["stat_bpw"] <= 1024
    stat = [0] * (2 * BLK * 4 // 16)
    for wave, lane in itertools.product(range(c["waves"]), range(64)):
        if lane < c["stat_bpw"] // 16:
            stat[(wave * c["stat_bpw"] + 16 * lane) // 16] += 1
    assert stat == [1] * len(stat)
    # reads of 32-query sub-blocks: row-major (read_row) and transposed (read_tr)
    for wave_qs, qq, lane in itertools.product(range(c["qs"]), range(c["qb_per_wave"]), range(64)):
        qb = wave_qs * c["qb_per_wave"] + qq
        half = lane >> 5
        for ks in range(D // 16):
            r = qb * 32 + (lane & 31)
            ch = (2 * ks + half) ^ qswz(D, r)
            assert r < BLK and 0 <= r * D + ch * 8 and r * D + ch * 8 + 8 <= c["tile"]
        si = lane & 15
        for d0, t in itertools.product(range(0, D, 32), range(2)):
            d = d0 + 16 * ((lane >> 4) & 1) + 4 * (si & 3)
            for sg in range(2):
                row = qb * 32 + 16 * t + 4 * half + (si >> 2) + 8 * sg
                ch = (d >> 3) ^ qswz(D, row)
                byte = (row * D + ch * 8) * 2 + (d & 7) * 2
                assert row < BLK and byte + 8 <= c["tile"] * 2


@pytest.mark.parametrize("D,BLK", [(d, b) for d in DIMS for b in BLOCKS])
def test_backward_dq_transposed_key_reads_stay_in_the_tile(D, BLK):
    """dQ^T += K^T dS^T reads K^T by transposed reads of the K tile: rows
    16 kk + 4 half + s / 4 + 8 sg for every key step kk < BLK / 16."""
    for lane, kk, dt, sg in itertools.product(range(64), range(BLK // 16), range(D // 32), range(2)):
        half, si = lane >> 5, lane & 15
        d = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (si & 3)
        row = 16 * kk + 4 * half + (si >> 2) + 8 * sg
        ch = (d >> 3) ^ qswz(D, row)
        byte = (row * D + ch * 8) * 2 + (d & 7) * 2
        assert row < BLK and byte + 8 <= BLK * D * 2
