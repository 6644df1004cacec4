"""Model check of the partial-logit exchange between the two halves of a CU
pair (the d = 2048 vocabulary head): a plain-Python model of the schedule the
kernel follows, run under random relative delays of the two halves.

Half h, iteration t (t = 0 .. nt + 2):
  * stores its partial of tile t-1 (if 0 <= t-1 < nt) into its slot (t-1) % 4,
    tagged with the generation bit of tile t-1;
  * reads the other half's slot (t-2) % 4 and waits until the bit matches the
    generation of tile t-2 (if 0 <= t-2 < nt).
Slots start cleared (bit 0).  The model asserts that a reader only ever
accepts the record of the tile it wants: not the cleared slot, not an older
tile.  The generation bit is ((tile // 4) + 1) % 2; with (tile // 4) % 2 the
cleared slot matches the first four tiles, which the second check shows.
"""
import random


def gen(tile, offset=1):
    return ((tile >> 2) + offset) & 1


def simulate(nt, seed, offset, cap=200000):
    """Accepted (wanted tile, tile found) pairs, or None if the halves stop
    making progress (a reader waiting for a record that was overwritten)."""
    rng = random.Random(seed)
    CLEARED = (None, 0)
    slots = [[CLEARED] * 4 for _ in range(2)]  # slots[h][s] = (tile, bit)
    t = [0, 0]
    phase = [0, 0]  # 0: store, 1: read
    accepted = []
    steps = 0
    while min(t) <= nt + 2:
        steps += 1
        if steps > cap:
            return None
        h = rng.randrange(2)
        if t[h] > nt + 2:
            h ^= 1
        if phase[h] == 0:
            tile = t[h] - 1
            if 0 <= tile < nt:
                slots[h][tile % 4] = (tile, gen(tile, offset))
            phase[h] = 1
        else:
            tile = t[h] - 2
            if 0 <= tile < nt:
                got, bit = slots[h ^ 1][tile % 4]
                if bit != gen(tile, offset):
                    continue  # still waiting; the other half must make progress
                accepted.append((tile, got))
            phase[h] = 0
            t[h] += 1
    return accepted


def test_reader_accepts_only_the_wanted_tile():
    for nt in (1, 2, 3, 4, 5, 8, 13):
        for seed in range(300):
            acc = simulate(nt, seed, offset=1)
            assert acc is not None, (nt, seed)
            assert len(acc) == 2 * nt
            for tile, got in acc:
                assert got == tile, (nt, seed, tile, got)


def test_unshifted_generation_breaks():
    # with bit (tile // 4) % 2 a cleared slot passes for tiles 0..3: wrong
    # records are accepted, or a half runs ahead and the other one then waits
    # for a record that was already overwritten
    broken = 0
    for seed in range(100):
        acc = simulate(8, seed, offset=0, cap=20000)
        broken += acc is None or any(got != tile for tile, got in acc)
    assert broken > 0


# ---- the start handshake of a CU group ------------------------------------------------------

SOLO = 1 << 8


def handshake(Q, arrive, spin, seed):
    """Plain-Python model of the group handshake: member m becomes runnable at
    step arrive[m] (None: never, within the run) and then runs
      v = fetch_or(word, bit m); loop: decided if SOLO set or all Q bits set;
      after `spin` polls try CAS(word, v, v | SOLO), on failure re-read;
    one atomic operation of one member per step, members picked at random.
    A bound of 0 sets the member's bit and the solo mark at once.
    Returns each member's decision (True = solo; None if never arrived)."""
    rng = random.Random(seed)
    full = (1 << Q) - 1
    word = 0
    state = [None] * Q        # None: not started; else dict
    decision = [None] * Q
    for step in range(100000):
        ready = [m for m in range(Q) if arrive[m] is not None and arrive[m] <= step and decision[m] is None]
        if not ready:
            if all(decision[m] is not None or arrive[m] is None for m in range(Q)):
                break
            continue
        m = rng.choice(ready)
        st = state[m]
        if st is None:
            old = word
            word |= (1 << m) | (SOLO if spin == 0 else 0)
            state[m] = st = {"v": word if spin == 0 else old | (1 << m), "n": 0}
        v = st["v"]
        if (v & SOLO) or (v & full) == full:
            decision[m] = bool(v & SOLO)
            continue
        if st["n"] >= spin:
            if word == v:                      # compare-and-swap
                word = v | SOLO
                st["v"] = word
            else:
                st["v"] = word
            continue
        st["v"] = word                         # a poll
        st["n"] += 1
    return decision, word


def test_group_handshake_members_agree():
    for Q in (2, 4):
        for seed in range(400):
            rng = random.Random(seed)
            arrive = [rng.choice([0, rng.randrange(0, 60), rng.randrange(0, 400)]) for _ in range(Q)]
            spin = rng.choice([0, 1, 3, 20, 200])
            dec, word = handshake(Q, arrive, spin, seed)
            assert None not in dec, (Q, seed)
            assert len(set(dec)) == 1, (Q, seed, dec, arrive, spin)   # one decision per group
            if not dec[0]:
                assert word == (1 << Q) - 1                            # paired: everyone arrived, no mark


def test_group_handshake_pairs_when_members_arrive_together():
    for Q in (2, 4):
        for seed in range(50):
            dec, _ = handshake(Q, [0] * Q, 10 ** 6, seed)
            assert dec == [False] * Q


def test_group_handshake_goes_solo_without_a_partner():
    # the last member arrives only after the others have given up waiting
    for Q in (2, 4):
        for seed in range(50):
            dec, word = handshake(Q, [0] * (Q - 1) + [10 ** 4], 5, seed)
            assert dec == [True] * Q and word & SOLO
