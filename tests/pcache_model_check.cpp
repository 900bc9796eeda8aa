// Model-based check of the host prefix cache (include/kda_prefix_cache.h),
// built with g++ and run under AddressSanitizer / UndefinedBehaviorSanitizer
// by tests/test_prefix_cache_sanitized.py.  Random operations (reserve,
// insert, insert_many, lookup, release, commit, unreserve) on a few token
// sequences that branch off one another are applied both to the cache and to
// a plain reference model (an ordered map from prefix to entry); every return
// value and every counter is compared after each operation.
//
//   pcache_model_check <seed> <ops> <unit> <slots> [<policy> <ghost_capacity>]
//
// policy 0 keeps every inserted state, 1 only a prefix's second insertion
// (first sightings are remembered in a FIFO of ghost_capacity keys).
//
// Prints "ok <ops>" and exits 0, or prints the first mismatch and exits 1.

#include "kda_prefix_cache.h"

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <deque>
#include <map>
#include <set>
#include <random>
#include <vector>

namespace {

using Seq = std::vector<int32_t>;

struct ModelEntry {
    int32_t slot;
    int64_t step;
    int32_t pins;
    int64_t last_use;   // for the least-recently-used eviction order
};

int g_op = 0;

#define CHECK(c)                                                                               \
    do {                                                                                       \
        if (!(c)) {                                                                            \
            std::printf("mismatch at op %d (line %d): %s [%s]\n", g_op, __LINE__, #c,          \
                        kda_pcache_last_error());                                              \
            std::exit(1);                                                                      \
        }                                                                                      \
    } while (0)

}  // namespace

int main(int argc, char** argv) {
    if (argc != 5 && argc != 7) {
        std::printf("usage: %s seed ops unit slots [policy ghost_capacity]\n", argv[0]);
        return 2;
    }
    const int32_t policy = argc == 7 ? std::atoi(argv[5]) : KDA_PCACHE_KEEP_ALL;
    const int32_t ghost_arg = argc == 7 ? std::atoi(argv[6]) : 0;
    const uint64_t seed = std::strtoull(argv[1], nullptr, 10);
    const int ops = std::atoi(argv[2]);
    const int32_t unit = std::atoi(argv[3]);
    const int32_t num_slots = std::atoi(argv[4]);
    std::mt19937_64 rng(seed);
    auto rnd = [&](int64_t n) { return static_cast<int64_t>(rng() % static_cast<uint64_t>(n)); };

    // token sequences that share prefixes: each branches off an earlier one
    std::vector<Seq> seqs;
    {
        Seq s(1 + rnd(200));
        for (auto& t : s) t = static_cast<int32_t>(rnd(4));
        seqs.push_back(s);
        for (int i = 1; i < 8; i++) {
            const Seq& parent = seqs[rnd(i)];
            Seq b(parent.begin(), parent.begin() + rnd(static_cast<int64_t>(parent.size()) + 1));
            const int64_t extra = 1 + rnd(150);
            for (int64_t j = 0; j < extra; j++) b.push_back(static_cast<int32_t>(rnd(4)));
            seqs.push_back(b);
        }
    }

    kda_pcache* c = kda_pcache_create(num_slots, unit, policy, ghost_arg);
    CHECK(c != nullptr);
    std::map<Seq, ModelEntry> model;
    std::vector<int> state(num_slots, 0);    // 0 free, 1 reserved, 2 owned by an entry
    std::vector<Seq> owner(num_slots);
    std::vector<int32_t> reserved, pinned;
    int64_t committed = INT64_MIN, step = 0, clock = 0;
    int64_t hits = 0, misses = 0, evictions = 0, declined = 0;
    const size_t ghost_cap = ghost_arg > 0 ? static_cast<size_t>(ghost_arg) : static_cast<size_t>(num_slots) * 4;
    std::set<Seq> ghosts;          // first sightings remembered by the second-hit policy
    std::deque<Seq> ghost_order;
    // expected result of inserting key: 1 kept, 0 declined (updates the ghosts)
    auto expect_insert = [&](const Seq& key) {
        if (model.count(key)) return 0;
        if (policy == KDA_PCACHE_SECOND_HIT && !ghosts.count(key)) {
            ghosts.insert(key);
            ghost_order.push_back(key);
            while (ghost_order.size() > ghost_cap) {
                ghosts.erase(ghost_order.front());
                ghost_order.pop_front();
            }
            return 0;
        }
        return 1;
    };

    auto visible_best = [&](const Seq& s, int64_t max_len) {
        int64_t best = 0;
        for (int64_t p = 1; p <= max_len; p++) {
            auto it = model.find(Seq(s.begin(), s.begin() + p));
            if (it != model.end() && it->second.step <= committed) best = p;
        }
        return best;
    };
    auto take_reserved = [&]() {
        const int64_t i = rnd(static_cast<int64_t>(reserved.size()));
        const int32_t s = reserved[i];
        reserved.erase(reserved.begin() + i);
        return s;
    };

    for (g_op = 0; g_op < ops; g_op++) {
        const int64_t r = rnd(100);
        if (r < 20) {
            // reserve: free slots first, then least recently used evictable entries
            const int32_t n = static_cast<int32_t>(1 + rnd(3));
            int64_t nfree = 0;
            std::vector<std::pair<int64_t, int32_t>> evictable;   // (last use, slot)
            for (int32_t s = 0; s < num_slots; s++) {
                if (state[s] == 0) nfree++;
                if (state[s] == 2) {
                    const ModelEntry& e = model.at(owner[s]);
                    if (e.pins == 0 && e.step <= committed) evictable.push_back({e.last_use, s});
                }
            }
            std::sort(evictable.begin(), evictable.end());
            int32_t out[3] = {-1, -1, -1};
            const int32_t got = kda_pcache_reserve(c, n, out);
            if (nfree + static_cast<int64_t>(evictable.size()) < n) {
                CHECK(got == -1);
                continue;
            }
            CHECK(got == n);
            const int64_t need = std::max<int64_t>(0, n - nfree);
            std::vector<int32_t> expect_evicted;
            for (int64_t i = 0; i < need; i++) expect_evicted.push_back(evictable[i].second);
            int64_t evicted = 0;
            for (int32_t i = 0; i < n; i++) {
                const int32_t s = out[i];
                CHECK(s >= 0 && s < num_slots);
                for (int32_t j = 0; j < i; j++) CHECK(out[j] != s);
                CHECK(state[s] != 1);
                if (state[s] == 2) {
                    CHECK(std::find(expect_evicted.begin(), expect_evicted.end(), s) != expect_evicted.end());
                    model.erase(owner[s]);
                    evicted++;
                }
                state[s] = 1;
                reserved.push_back(s);
            }
            CHECK(evicted == need);
            evictions += need;
        } else if (r < 45 && !reserved.empty()) {
            // insert one state
            const Seq& s = seqs[rnd(static_cast<int64_t>(seqs.size()))];
            const int64_t p = 1 + rnd(static_cast<int64_t>(s.size()));
            const int32_t slot = take_reserved();
            const Seq key(s.begin(), s.begin() + p);
            const int32_t expect = expect_insert(key);
            CHECK(kda_pcache_insert(c, s.data(), p, slot, step) == expect);
            if (expect) {
                model[key] = ModelEntry{slot, step, 0, ++clock};
                state[slot] = 2;
                owner[slot] = key;
            } else {
                state[slot] = 0;
                declined++;
            }
        } else if (r < 55 && reserved.size() >= 2) {
            // insert several states of one sequence at increasing positions
            const Seq& s = seqs[rnd(static_cast<int64_t>(seqs.size()))];
            const int32_t n = static_cast<int32_t>(std::min<int64_t>(2 + rnd(3), static_cast<int64_t>(reserved.size())));
            if (static_cast<int64_t>(s.size()) < n) continue;
            std::vector<int64_t> pos;
            while (static_cast<int32_t>(pos.size()) < n) {
                const int64_t p = 1 + rnd(static_cast<int64_t>(s.size()));
                if (std::find(pos.begin(), pos.end(), p) == pos.end()) pos.push_back(p);
            }
            std::sort(pos.begin(), pos.end());
            std::vector<int32_t> slots, kept(n, -1);
            for (int32_t i = 0; i < n; i++) slots.push_back(take_reserved());
            int32_t expect_count = 0;
            std::vector<int32_t> expect(n);
            for (int32_t i = 0; i < n; i++) {
                expect[i] = expect_insert(Seq(s.begin(), s.begin() + pos[i]));
                expect_count += expect[i];
            }
            CHECK(kda_pcache_insert_many(c, s.data(), n, pos.data(), slots.data(), step, kept.data()) == expect_count);
            for (int32_t i = 0; i < n; i++) {
                CHECK(kept[i] == expect[i]);
                if (expect[i]) {
                    const Seq key(s.begin(), s.begin() + pos[i]);
                    model[key] = ModelEntry{slots[i], step, 0, ++clock};
                    state[slots[i]] = 2;
                    owner[slots[i]] = key;
                } else {
                    state[slots[i]] = 0;
                    declined++;
                }
            }
        } else if (r < 75) {
            // lookup: the longest visible prefix, pinned on a hit
            const Seq& s = seqs[rnd(static_cast<int64_t>(seqs.size()))];
            const int64_t max_len = rnd(static_cast<int64_t>(s.size()) + 1);
            const int64_t best = visible_best(s, max_len);
            int32_t slot = -2;
            CHECK(kda_pcache_lookup(c, s.data(), max_len, &slot) == best);
            if (best > 0) {
                ModelEntry& e = model.at(Seq(s.begin(), s.begin() + best));
                CHECK(slot == e.slot);
                e.pins++;
                e.last_use = ++clock;
                pinned.push_back(slot);
                hits++;
            } else {
                CHECK(slot == -1);
                misses++;
            }
        } else if (r < 85 && !pinned.empty()) {
            const int64_t i = rnd(static_cast<int64_t>(pinned.size()));
            const int32_t slot = pinned[i];
            pinned.erase(pinned.begin() + i);
            CHECK(kda_pcache_release(c, slot) == 0);
            model.at(owner[slot]).pins--;
        } else if (r < 88) {
            // refused calls change nothing: releasing a slot without a pin, inserting
            // into a slot that is not reserved, repeated slots, non-increasing positions
            const int32_t slot = static_cast<int32_t>(rnd(num_slots));
            const Seq& s = seqs[rnd(static_cast<int64_t>(seqs.size()))];
            if (std::find(pinned.begin(), pinned.end(), slot) == pinned.end()) CHECK(kda_pcache_release(c, slot) == -1);
            if (state[slot] != 1) CHECK(kda_pcache_insert(c, s.data(), 1, slot, step) == -1);
            if (!reserved.empty() && s.size() >= 2) {
                const int32_t two[2] = {reserved[0], reserved[0]};
                const int64_t pos2[2] = {1, 2};
                CHECK(kda_pcache_insert_many(c, s.data(), 2, pos2, two, step, nullptr) == -1);
            }
            if (reserved.size() >= 2 && s.size() >= 2) {
                const int32_t two[2] = {reserved[0], reserved[1]};
                const int64_t pos2[2] = {2, 2};
                CHECK(kda_pcache_insert_many(c, s.data(), 2, pos2, two, step, nullptr) == -1);
            }
        } else if (r < 95) {
            kda_pcache_commit(c, step);
            committed = std::max(committed, step);
            step++;
        } else if (!reserved.empty()) {
            const int32_t slot = take_reserved();
            CHECK(kda_pcache_unreserve(c, slot) == 0);
            state[slot] = 0;
        }

        int64_t st[8];
        kda_pcache_stats(c, st, 8);
        int64_t nfree = 0, npinned = 0;
        for (int32_t s = 0; s < num_slots; s++) nfree += state[s] == 0;
        for (int32_t s = 0; s < num_slots; s++)
            if (state[s] == 2 && model.at(owner[s]).pins > 0) npinned++;
        CHECK(st[0] == static_cast<int64_t>(model.size()));
        CHECK(st[1] == nfree);
        CHECK(st[2] == npinned);
        CHECK(st[3] == hits);
        CHECK(st[4] == misses);
        CHECK(st[5] == evictions);
        CHECK(st[6] == declined);
        CHECK(st[7] == static_cast<int64_t>(ghosts.size()));
    }
    kda_pcache_destroy(c);
    std::printf("ok %d\n", ops);
    return 0;
}
