"""Host tests of the prefix cache of KDA states (include/kda_prefix_cache.h).

No GPU: the cache only bookkeeps slots.  Besides the individual rules
(longest match, chained keys, prompt-end entries, deferred visibility,
pinning, LRU eviction, second-hit retention) a randomized run is checked
against a brute-force model that keys entries by the full token tuple.
"""
import numpy as np
import pytest

import linear_attention_recurrence_decode_amd as kda

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(kda.LIB_PATH), reason="libkda.so not built")


def toks(rng, n, vocab=1000):
    return rng.integers(0, vocab, n).astype(np.int32)


def put(c, t, pos, step=0):
    slot = int(c.reserve(1)[0])
    kept = c.insert(t, pos, slot, step)
    return slot if kept else None


def test_longest_aligned_prefix_and_max_len():
    rng = np.random.default_rng(1)
    c = kda.PrefixCache(16, unit=128)
    a = toks(rng, 1000)
    s256, s512 = put(c, a, 256), put(c, a, 512)
    c.commit(0)
    b = np.concatenate([a[:700], toks(rng, 300)])
    assert c.lookup(b) == (512, s512)
    c.release(s512)
    assert c.lookup(b, max_len=511) == (256, s256)
    c.release(s256)
    assert c.lookup(b, max_len=255) == (0, -1)


def test_chained_keys_name_the_whole_prefix():
    rng = np.random.default_rng(2)
    c = kda.PrefixCache(8, unit=64)
    a = toks(rng, 256)
    put(c, a, 256)
    c.commit(0)
    b = a.copy()
    b[10] += 1                      # same last unit, different earlier token
    assert c.lookup(b) == (0, -1)
    assert c.lookup(a)[0] == 256


def test_prompt_end_entries_between_units():
    rng = np.random.default_rng(3)
    c = kda.PrefixCache(8, unit=128)
    a = toks(rng, 900)
    s_end = put(c, a, 700)          # prompt end, not on a unit boundary
    s_small = put(c, a, 50)         # shorter than one unit
    s_aligned = put(c, a, 640)
    c.commit(0)
    assert c.lookup(np.concatenate([a[:700], toks(rng, 5)])) == (700, s_end)
    c.release(s_end)
    assert c.lookup(a[:699]) == (640, s_aligned)
    c.release(s_aligned)
    assert c.lookup(np.concatenate([a[:60], toks(rng, 10)])) == (50, s_small)
    c.release(s_small)
    assert c.lookup(a[:49]) == (0, -1)


def test_entries_are_invisible_until_their_step_commits():
    rng = np.random.default_rng(4)
    c = kda.PrefixCache(8, unit=64)
    a = toks(rng, 300)
    s = put(c, a, 128, step=5)
    assert c.lookup(a) == (0, -1)
    c.commit(4)
    assert c.lookup(a) == (0, -1)
    c.commit(5)
    assert c.lookup(a) == (128, s)


def test_pinned_and_uncommitted_entries_are_not_evicted_lru_order_otherwise():
    rng = np.random.default_rng(5)
    c = kda.PrefixCache(3, unit=64)
    a, b, d = toks(rng, 64), toks(rng, 64), toks(rng, 64)
    sa, sb, sd = put(c, a, 64), put(c, b, 64), put(c, d, 64)
    c.commit(0)
    assert c.lookup(a) == (64, sa)          # a is now most recent and pinned
    got = c.reserve(1)                       # evicts the least recent unpinned: b
    assert int(got[0]) == sb and c.lookup(b) == (0, -1)
    c.unreserve(int(got[0]))
    got = c.reserve(2)                       # free slot + evict d; a stays (pinned)
    assert sorted(int(x) for x in got) == sorted([sb, sd])
    with pytest.raises(kda.KdaError):
        c.reserve(1)                         # only the pinned entry is left
    c.release(sa)
    assert int(c.reserve(1)[0]) == sa
    st = c.stats()
    assert st["evictions"] == 3 and st["entries"] == 0


def test_second_hit_policy_keeps_only_repeated_prefixes():
    rng = np.random.default_rng(6)
    c = kda.PrefixCache(8, unit=64, policy=kda.KDA_PCACHE_SECOND_HIT)
    a, b = toks(rng, 200), toks(rng, 200)
    assert put(c, a, 128) is None            # first sighting: declined, slot free again
    assert put(c, b, 128) is None
    s = put(c, a, 128)                       # second: kept
    assert s is not None
    c.commit(0)
    assert c.lookup(a)[0] == 128 and c.lookup(b) == (0, -1)
    st = c.stats()
    assert st["declined"] == 2 and st["entries"] == 1 and st["free_slots"] == 7


def test_duplicates_declined_and_errors_reported():
    rng = np.random.default_rng(7)
    c = kda.PrefixCache(4, unit=64)
    a = toks(rng, 100)
    assert put(c, a, 64) is not None
    assert put(c, a, 64) is None             # same prefix again
    with pytest.raises(kda.KdaError):
        c.release(0)                         # not pinned
    with pytest.raises(kda.KdaError):
        c.insert(a, 64, 3, 0)                # slot 3 was never reserved
    with pytest.raises(kda.KdaError):
        kda.PrefixCache(0, unit=64)


def test_randomized_against_brute_force_model():
    """Random inserts, lookups, releases and commits over prompts that share
    prefixes; the cache must return the same (p, slot) as a model keyed by
    the full token tuple, while capacity never forces an eviction."""
    rng = np.random.default_rng(8)
    unit, nslots = 16, 400
    c = kda.PrefixCache(nslots, unit=unit)
    roots = [toks(rng, 200, vocab=5) for _ in range(6)]     # small vocab: many shared prefixes
    model = {}                                              # tuple(prefix) -> (slot, step)
    step, pinned = 0, []
    for it in range(600):
        base = roots[int(rng.integers(len(roots)))]
        cut = int(rng.integers(1, 200))
        t = np.concatenate([base[:cut], toks(rng, int(rng.integers(0, 40)), vocab=5)])
        op = rng.random()
        if op < 0.45:
            pos = int(rng.integers(1, len(t) + 1))
            if rng.random() < 0.5:
                pos = max(unit, pos // unit * unit) if len(t) >= unit else pos
            key = tuple(t[:pos])
            slot = int(c.reserve(1)[0])
            kept = c.insert(t, pos, slot, step)
            assert kept == (key not in model)
            if kept:
                model[key] = (slot, step)
        elif op < 0.9:
            max_len = int(rng.integers(0, len(t) + 1))
            # model: longest committed prefix with p <= max_len that is a unit multiple or a prompt-end entry
            best = (0, -1)
            for p in range(1, max_len + 1):
                e = model.get(tuple(t[:p]))
                if e is not None and e[1] <= step - 1:
                    best = (p, e[0])
            got = c.lookup(t, max_len=max_len)
            assert got == best, (it, got, best)
            if got[0]:
                pinned.append(got[1])
        elif op < 0.95 and pinned:
            c.release(pinned.pop(int(rng.integers(len(pinned)))))
        else:
            c.commit(step)
            step += 1
    assert c.stats()["evictions"] == 0


def test_insert_many_equals_single_inserts():
    rng = np.random.default_rng(9)
    a = toks(rng, 2000)
    pos = [128, 256, 300, 384, 1000, 1024, 1999]
    c1, c2 = kda.PrefixCache(16, unit=128), kda.PrefixCache(16, unit=128)
    s1 = [put(c1, a, p) for p in pos]
    s2 = c2.reserve(len(pos))
    assert c2.insert_many(a, pos, s2, 0).all()
    c1.commit(0)
    c2.commit(0)
    for n in (129, 300, 301, 999, 1000, 1500, 2000):
        p1, q1 = c1.lookup(a, max_len=n)
        p2, q2 = c2.lookup(a, max_len=n)
        assert p1 == p2 and (p1 == 0 or pos.index(p1) == list(s1).index(q1) == list(s2).index(q2))
    with pytest.raises(kda.KdaError):
        c2.insert_many(a, [5, 4], c2.reserve(2), 1)            # positions must increase


def test_shared_prompt_end_offset_survives_eviction():
    """Two prompts that share the prefix up to a unit boundary and end at the
    same offset after it are listed under that boundary together; evicting one
    must leave the other reachable."""
    rng = np.random.default_rng(10)
    c = kda.PrefixCache(2, unit=16)
    base = toks(rng, 32)
    a = np.concatenate([base, np.array([1, 2], np.int32)])
    b = np.concatenate([base, np.array([3, 4], np.int32)])
    sa, sb = put(c, a, 34), put(c, b, 34)
    c.commit(0)
    assert c.lookup(b) == (34, sb)
    c.release(sb)
    # b was used last, so the next reservation evicts a
    s = int(c.reserve(1)[0])
    assert s == sa and c.stats()["evictions"] == 1
    c.unreserve(s)
    assert c.lookup(b) == (34, sb)
    c.release(sb)
    assert c.lookup(a) == (0, -1)


def test_refused_reservation_evicts_nothing():
    rng = np.random.default_rng(11)
    c = kda.PrefixCache(2, unit=16)
    a, b = toks(rng, 32), toks(rng, 32)
    put(c, a, 32)
    put(c, b, 32)
    c.commit(0)
    p, s = c.lookup(a)              # a pinned: only b can be evicted
    assert p == 32
    with pytest.raises(kda.KdaError):
        c.reserve(2)
    st = c.stats()
    assert st["entries"] == 2 and st["evictions"] == 0 and st["free_slots"] == 0
    assert c.lookup(b)[0] == 32
