"""Index identities the kernels' register paths rely on (host-side, CPU).

The M/N-contiguous loader (256-row panel, 256 threads, 8 vectors of 8
elements per thread) maps thread t to k-group kb = (t >> 2) & 7 and
mn-chunk mc = (t & 3) | ((t >> 5) << 2), and stores unit i (row mc*8 + i)
of its transposed block at LDS element row*64 + ((kb ^ swz(row)) << 3) with
swz(row) = (row >> 1) & 7.  The gradient-on-load loop relies on three
consequences, checked here for every thread and unit:

- one offset register per thread covers the eight units:
  byte offset of unit i == (off0 ^ ((i >> 1) << 4)) + 128 i;
- every vector of wave w lies in the tile's 64-row chunk w, so a wave
  applies one column of the scale table;
- the K-contiguous loader's thread t holds token rows t/8 + 32 i, and lane
  l of wave w stages row 8w + l/8 + 32 (l % 8): each thread's 8 rows are 8
  consecutive staged words of its own wave, starting at word 8 ((t >> 3) & 7).
"""


def swz(row):
    return (row >> 1) & 7


def kb_of(t):
    return (t >> 2) & 7


def mc_of(t):
    return (t & 3) | ((t >> 5) << 2)


def test_unit_offsets_from_one_register():
    for t in range(256):
        kb, mc = kb_of(t), mc_of(t)
        off0 = (mc * 8 * 64 + ((kb ^ swz(mc * 8)) << 3)) * 2
        for i in range(8):
            row = mc * 8 + i
            ref = (row * 64 + ((kb ^ swz(row)) << 3)) * 2
            assert ref == (off0 ^ ((i >> 1) << 4)) + i * 128


def test_threads_cover_the_panel_once():
    seen = {(kb_of(t), mc_of(t)) for t in range(256)}
    assert seen == {(kb, mc) for kb in range(8) for mc in range(32)}


def test_a_wave_stays_in_one_scale_chunk():
    for t in range(256):
        rows = {mc_of(t) * 8 + e for e in range(8)}
        assert {r // 64 for r in rows} == {t >> 6}


def test_k_major_rows_are_consecutive_staged_words():
    for t in range(256):
        w, l = t >> 6, t & 63
        staged = [8 * w + (x >> 3) + 32 * (x & 7) for x in range(64)]  # word x of wave w
        idx0 = ((t >> 3) & 7) * 8
        rows = [t // 8 + 32 * i for i in range(8)]
        assert staged[idx0:idx0 + 8] == rows
    # and the 4 waves stage all 256 rows exactly once
    allrows = sorted(8 * w + (x >> 3) + 32 * (x & 7) for w in range(4) for x in range(64))
    assert allrows == list(range(256))
