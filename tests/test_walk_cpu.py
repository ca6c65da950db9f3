"""The workgroup deals of the forward kernels, restated from their
documentation as a model on the CPU (no GPU): every group of a column block,
and every flat-walk group including the partial one, goes to exactly one
workgroup, with the XCD-weighted deal as with the round-robin one.

Tiled walk (make_walk): G workgroups, nb column blocks, ng groups per block.
Round-robin: workgroup w serves block w mod nb and takes groups
w div nb, + G/nb, ... With share q (G a multiple of 2 nb): pair p = w div 2
serves block p mod nb; the workgroup of the pair whose parity equals flip
(the launch-wide XCD parity hint) takes groups i, i + G/(2 nb), ... below
e = round(ng q / 1024), the other one groups e + i, e + i + G/(2 nb), ...
below ng (i = p div nb).

Flat walk: ngroups whole groups and possibly a partial one (index ngroups).
Round-robin: w takes w, w + G, ...; the partial group goes to ngroups mod G.
Weighted (G even): w of parity flip takes w div 2, + G/2, ... below e; the
others take e + w div 2, ... below ngroups; the partial group goes to the
workgroup of the other parity with w div 2 = (ngroups - e) mod G/2. Its column offset advances by
(G' B V) mod N per group, G' = G/2 weighted, G otherwise.
"""
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402


def even_groups(ng, q):
    return (ng * q + 512) >> 10


def tiled_deal(G, nb, ng, q, flip=0, rq=0):
    """{(block, group): workgroup} of the main loop. With rq (G a multiple
    of 4 nb) the first G/2 workgroups take groups [0, round(ng rq / 1024))
    and the second half the rest, each half split by the XCD classes as
    above with index i among the half's pairs."""
    weighted = q != 0 and G % (2 * nb) == 0
    rounds = weighted and rq != 0 and G % (4 * nb) == 0
    H = G // 2 if rounds else G
    out = {}
    for w in range(G):
        half = 1 if rounds and w >= H else 0
        wl = w - half * H
        pair, odd = wl >> 1, wl & 1
        cls = odd ^ flip
        b = pair % nb if weighted else w % nb
        gcount = G // nb
        if weighted:
            n0 = even_groups(ng, rq) if rounds else ng
            lo, nr = (n0, ng - n0) if half else (0, n0)
            ne = even_groups(nr, q)
            first = lo + (ne if cls else 0) + pair // nb
            stride = H // nb // 2
            end = lo + (nr if cls else ne)
        else:
            first, stride, end = w // nb, gcount, ng
        for gi in range(first, end, stride):
            assert (b, gi) not in out, (G, nb, ng, q, w, gi)
            out[(b, gi)] = w
    return out


def flat_deal(G, ngroups, partial, q, flip=0):
    weighted = q != 0 and G % 2 == 0
    ne = even_groups(ngroups, q) if weighted else ngroups
    stride = G // 2 if weighted else G
    out = {}
    for w in range(G):
        cls = (w & 1) ^ flip
        first = ((ne if cls else 0) + (w >> 1)) if weighted else w
        end = ngroups if (weighted and cls) or not weighted else ne
        last_next = None
        for gi in range(first, end, stride):
            assert gi not in out
            out[gi] = w
            last_next = gi + stride
        owns = (cls and (w >> 1) == (ngroups - ne) % stride) if weighted else w == ngroups % G
        if partial and owns:
            assert ngroups not in out
            out[ngroups] = w
            # the owner's sequence reaches the partial group exactly
            nxt = first if last_next is None else last_next
            assert nxt == ngroups, (G, ngroups, q, w, first, nxt)
    return out


@settings(max_examples=400, deadline=None)
@given(st.sampled_from([2, 4, 8, 64, 128, 256, 512, 1024, 6, 254, 510]),
       st.sampled_from([1, 2, 3, 4]), st.integers(0, 5000), st.sampled_from([0, 512, 543, 560, 600]),
       st.sampled_from([0, 1]), st.sampled_from([0, 532, 548, 600]))
def test_tiled_deal_covers_every_group_once(G, nb, ng, q, flip, rq):
    if G % nb:
        return
    d = tiled_deal(G, nb, ng, q, flip, rq)
    assert set(d) == {(b, gi) for b in range(nb) for gi in range(ng)}
    if q and not rq and G % (2 * nb) == 0 and ng >= 4 * G:
        favoured = sum(1 for w in d.values() if w % 2 == flip)
        assert abs(favoured - nb * even_groups(ng, q)) == 0
    if q and rq and G % (4 * nb) == 0 and ng >= 4 * G:
        first = sum(1 for w in d.values() if w < G // 2)
        assert first == nb * even_groups(ng, rq)


@settings(max_examples=400, deadline=None)
@given(st.sampled_from([2, 4, 8, 128, 129, 256]), st.integers(0, 20000), st.booleans(),
       st.sampled_from([0, 512, 527, 543, 600]), st.sampled_from([0, 1]))
def test_flat_deal_covers_every_group_once(G, ngroups, partial, q, flip):
    d = flat_deal(G, ngroups, partial, q, flip)
    assert set(d) == set(range(ngroups + (1 if partial else 0)))
