"""CPU checks of the log-linear decode kernel's addressing (no GPU).

The kernel (csrc/kla_loglinear.hip, loglinear_decode_kernel) gives each of its NT threads
4 adjacent columns (c4) of NP rows (rg + p * RPP) of a bucket, with TPR = dv / 4 threads per
row and RPP = NT / TPR rows per pass, and walks the levels of position t as: levels 0..j
(j = trailing zeros of t) summed into level j + 1, then each higher set bit of t in place,
then level 0 written. These tests replay that index arithmetic and check it against the
definitions: every element of a bucket is owned by exactly one thread, and the levels read
and written at each position are exactly the occupied levels of the Log-Linear page's
Fenwick buckets before and after the token (oracle/loglinear.py's occupied_levels, itself
pinned by hand-derived cases in tests/test_oracle_loglinear.py).
"""
import pytest

from oracle import loglinear


def ll_threads(dk, dv):
    return 512 if dk * dv >= 128 * 128 else 256  # the kernel's thread count per (sequence, head)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128), (256, 64), (256, 128)])
def test_thread_tiles_cover_each_bucket_element_once(dk, dv):
    nt = ll_threads(dk, dv)
    tpr = dv // 4
    rpp = nt // tpr
    np_ = dk // rpp
    assert dk % rpp == 0 and dk <= nt
    owner = {}
    for tid in range(nt):
        rg, c4 = divmod(tid, tpr)
        for p in range(np_):
            for j in range(4):
                e = (rg + p * rpp, 4 * c4 + j)
                assert e not in owner, f"{e} owned by threads {owner[e]} and {tid}"
                owner[e] = tid
    assert len(owner) == dk * dv
    # 16-byte accesses: a thread's four columns are contiguous and 16-byte aligned in a row
    for tid in range(nt):
        assert (4 * (tid % tpr) * 4) % 16 == 0
    # the reduction over rows sums spa[g][c4] for g < RPP: every row of a column lands in
    # exactly one (rg, p) pair, so the column sums see each row once
    for c4 in range(tpr):
        rows = sorted(rg + p * rpp for rg in range(rpp) for p in range(np_))
        assert rows == list(range(dk))


def kernel_levels(t):
    """Levels the kernel reads and writes at position t >= 1, in its order."""
    j = (t & -t).bit_length() - 1          # trailing zeros of t
    read = list(range(j + 1))              # load_add of levels 0..j
    written = [j + 1]                      # their sum, transformed, into level j + 1
    dest = j + 1
    while True:
        rest = t >> dest
        nxt = dest + ((rest & -rest).bit_length() - 1) + 1 if rest else -1
        if nxt < 0:
            break
        read.append(nxt)                   # a higher occupied level, transformed in place
        written.append(nxt)
        dest = nxt
    written.append(0)                      # the token opens level 0
    return read, written


@pytest.mark.parametrize("L", [4, 8, 16])
def test_levels_read_and_written_are_the_occupied_buckets(L):
    for t in range(1, 1 << (L - 1)):
        read, written = kernel_levels(t)
        assert sorted(read) == sorted(loglinear.occupied_levels(t - 1)), t
        assert sorted(written) == sorted(loglinear.occupied_levels(t)), t
        assert len(set(written)) == len(written) and max(written) < L, t
        # a level written in place is read first; the merge destination j + 1 is not read
        j = (t & -t).bit_length() - 1
        assert j + 1 not in read
