"""Plain model of the GPU expert cache: which pool slot holds which expert.

TEST INFRASTRUCTURE.  Only the tests may import this module; the library's
own cache policy is written separately and never calls it.

Co-inference page, section 2.2 (the expert cache mechanism):
  * the GPU holds S expert slots, S = floor(free GPU memory / size of one
    expert);
  * the slots form an N-way set-associative cache: M ways per set and
    N = floor(S / M) sets (the page writes a configuration as (N, M), e.g.
    (14, 4): 14 indices of 4 ways);
  * replacement is LRU, motivated by expert reuse across consecutive layers
    and consecutive tokens.
Co-inference page, section 3.1, and Strata page, section 2.2: the weights of
the experts a layer will need are copied host -> device on a second stream
while the GPU computes, so the cache is asked for a layer's experts before
that layer runs.

cache_geometry gives (S, N) for a memory budget, an expert size and M.

Readings where the page is silent (each is listed in the design notes):
  * the set of an expert of layer L is L mod N (the page's N indices cover
    the layers; with more layers than sets, layers share sets);
  * slot number = set * M + way;
  * one request = the experts one layer needs for one step.  Its experts that
    are resident are hits; each missing one takes a way of the set that holds
    no expert of the same request: an empty way if there is one (lowest way
    first), else the least recently used way (lowest way first among equals),
    whose expert is evicted.  Every expert of the request is then stamped as
    used at this request, so "improved LRU" is read as plain LRU at request
    granularity;
  * a request needing more distinct experts than M at once is an error.
"""


def cache_geometry(free_bytes: int, expert_bytes: int, ways: int):
    """Co-inference page, section 2.2: S = floor(free memory / size of one
    expert) slots, grouped into N = floor(S / M) sets of M ways.  Returns
    (S, N); the slots past N * M stay unused."""
    if free_bytes < 0 or expert_bytes <= 0 or ways <= 0:
        raise ValueError("need free_bytes >= 0, expert_bytes > 0, ways > 0")
    slots = free_bytes // expert_bytes
    return slots, slots // ways


class ExpertCacheModel:
    def __init__(self, num_sets: int, ways: int, num_experts: int):
        if num_sets < 1 or ways < 1 or num_experts < 1:
            raise ValueError("num_sets, ways and num_experts must be positive")
        self.num_sets, self.ways, self.num_experts = num_sets, ways, num_experts
        # per slot: (layer, expert) or None, and the request counter of its last use
        self.key = [None] * (num_sets * ways)
        self.stamp = [0] * (num_sets * ways)
        self.clock = 0
        self.hits = 0
        self.misses = 0

    def slot_of(self, layer: int, expert: int):
        s = layer % self.num_sets
        for w in range(self.ways):
            if self.key[s * self.ways + w] == (layer, expert):
                return s * self.ways + w
        return None

    def request(self, layer: int, experts):
        """Returns (slots of `experts` in order, loads as [(expert, slot)])."""
        wanted = []
        for e in experts:
            if not 0 <= e < self.num_experts:
                raise ValueError(f"expert {e} out of range")
            if e not in wanted:
                wanted.append(e)
        if len(wanted) > self.ways:
            raise ValueError(f"{len(wanted)} experts do not fit {self.ways} ways")
        self.clock += 1
        s = layer % self.num_sets
        base = s * self.ways
        where = {}
        for e in wanted:  # hits
            slot = self.slot_of(layer, e)
            if slot is not None:
                where[e] = slot
                self.hits += 1
        loads = []
        for e in wanted:  # misses, in request order
            if e in where:
                continue
            self.misses += 1
            taken = set(where.values())
            free = [base + w for w in range(self.ways) if self.key[base + w] is None and base + w not in taken]
            if free:
                slot = free[0]
            else:
                cands = [base + w for w in range(self.ways) if base + w not in taken]
                slot = min(cands, key=lambda x: (self.stamp[x], x))
            self.key[slot] = (layer, e)
            where[e] = slot
            loads.append((e, slot))
        for e in wanted:
            self.stamp[where[e]] = self.clock
        return [where[e] for e in experts], loads

    def slot_table(self, layer: int):
        """Slot of every expert of `layer`, -1 where it is not resident."""
        return [(-1 if self.slot_of(layer, e) is None else self.slot_of(layer, e)) for e in range(self.num_experts)]
