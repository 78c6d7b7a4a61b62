"""Pins of the expert-cache model (oracle/expert_cache.py): hand-worked LRU
sequences, and a brute force that recomputes recency from the whole request
history on random request streams.  Co-inference page, section 2.2."""

import random

import pytest

from oracle.expert_cache import ExpertCacheModel


def test_lru_sequence_worked_by_hand():
    c = ExpertCacheModel(num_sets=1, ways=2, num_experts=8)
    assert c.request(0, [1]) == ([0], [(1, 0)])        # empty ways fill from way 0
    assert c.request(0, [2]) == ([1], [(2, 1)])
    assert c.request(0, [1]) == ([0], [])              # hit: 1 is now the most recent
    assert c.request(0, [3]) == ([1], [(3, 1)])        # 2 is least recent: evicted
    assert c.request(0, [2]) == ([0], [(2, 0)])        # now 1 is least recent
    assert c.slot_table(0) == [-1, -1, 0, 1, -1, -1, -1, -1]
    assert (c.hits, c.misses) == (1, 4)


def test_experts_of_one_request_never_evict_each_other():
    c = ExpertCacheModel(num_sets=1, ways=2, num_experts=8)
    c.request(0, [1, 2])
    slots, loads = c.request(0, [3, 1])                # 1 hits; 3 may only take 2's way
    assert slots == [1, 0] and loads == [(3, 1)]
    assert c.slot_table(0)[2] == -1


def test_layers_map_to_sets_modulo_the_set_count():
    c = ExpertCacheModel(num_sets=2, ways=2, num_experts=4)
    assert c.request(0, [0, 1])[0] == [0, 1]           # layer 0 -> set 0 (slots 0, 1)
    assert c.request(1, [0, 1])[0] == [2, 3]           # layer 1 -> set 1 (slots 2, 3)
    slots, loads = c.request(2, [3])                    # layer 2 shares set 0 with layer 0
    assert slots == [0] and loads == [(3, 0)]          # layer 0's expert 0 was least recent
    assert c.slot_table(0) == [-1, 1, -1, -1]
    assert c.slot_table(1) == [2, 3, -1, -1]


def test_duplicates_and_capacity():
    c = ExpertCacheModel(num_sets=1, ways=2, num_experts=4)
    slots, loads = c.request(0, [2, 2])
    assert slots == [0, 0] and loads == [(2, 0)]
    with pytest.raises(ValueError):
        c.request(0, [0, 1, 3])
    with pytest.raises(ValueError):
        c.request(0, [4])


def _history_lru(num_sets, ways, seq):
    """Brute force: recency comes from scanning the whole request history (the
    index of the last request that used a way's current key), not from
    stamps kept up to date."""
    occupant = {}          # slot -> (layer, expert)
    history = []           # per request: set of (layer, expert) used
    out = []
    for layer, experts in seq:
        wanted = list(dict.fromkeys(experts))
        base = (layer % num_sets) * ways
        where = {e: s for e in wanted for s, k in occupant.items() if k == (layer, e)}
        loads = []
        for e in wanted:
            if e in where:
                continue
            cands = [base + w for w in range(ways) if base + w not in where.values()]
            empty = [s for s in cands if s not in occupant]
            if empty:
                slot = min(empty)
            else:
                def last_use(s):
                    return max(i for i, used in enumerate(history) if occupant[s] in used)
                slot = min(cands, key=lambda s: (last_use(s), s))
            occupant[slot] = (layer, e)
            where[e] = slot
            loads.append((e, slot))
        history.append({(layer, e) for e in wanted})
        out.append(([where[e] for e in experts], loads))
    return out


def test_tied_recency_evicts_the_lowest_way():
    c = ExpertCacheModel(num_sets=1, ways=2, num_experts=8)
    c.request(0, [1, 2])                               # both used by the same request
    assert c.request(0, [3]) == ([0], [(3, 0)])


@pytest.mark.parametrize("seed", range(6))
def test_model_matches_history_brute_force(seed):
    rng = random.Random(seed)
    num_sets, ways, E, L = rng.choice([1, 2, 3]), rng.choice([2, 3, 4]), 8, 5
    seq = []
    for _ in range(200):
        layer = rng.randrange(L)
        seq.append((layer, [rng.randrange(E) for _ in range(rng.randint(1, ways))]))
    c = ExpertCacheModel(num_sets, ways, E)
    got = [c.request(layer, ex) for layer, ex in seq]
    assert got == _history_lru(num_sets, ways, seq)


def _golden(name):
    import os
    vals = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (x.strip() for x in line.split("=", 1))
                vals[k] = v
    return vals


def test_cache_geometry_reproduces_the_pages_worked_example():
    """19 GB free, 340 MB experts: about 56 slots, and the (N, M) pairs (14, 4),
    (11, 5), (7, 8) of the page's configuration table (binary units)."""
    from oracle.expert_cache import cache_geometry
    g = _golden("coinference_cache_sizing.txt")
    free, expert = int(g["free_gb"]) << 30, int(g["expert_mb_mixtral"]) << 20
    pairs = [tuple(int(x) for x in p.split("x")) for p in g["sets_ways"].split()]
    for n, m in pairs:
        slots, sets = cache_geometry(free, expert, m)
        assert sets == n
        assert abs(slots - int(g["slots_approx"])) <= 1
        assert sets * m <= slots


def test_page_expert_sizes_match_the_synthetic_shapes():
    """One fp16 expert (gate, up, down) of the Mixtral-8x7B- and Phi-3.5-MoE-shaped
    layers against the sizes the page prints (within its rounding, binary MB)."""
    import synth
    g = _golden("coinference_cache_sizing.txt")
    for case, key in (("mixtral_decode", "expert_mb_mixtral"), ("phi35_skew", "expert_mb_phi35")):
        shp = synth.case_shape(case)
        fp16_bytes = 3 * shp.d_model * shp.d_ff * 2
        assert abs(fp16_bytes / (1 << 20) / int(g[key]) - 1) < 0.02, (case, fp16_bytes)
