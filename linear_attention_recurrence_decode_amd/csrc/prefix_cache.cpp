// prefix_cache.cpp -- host-side prefix cache of KDA states (see
// include/kda_prefix_cache.h for the contract and the passages it follows).
//
// Keys: a 128-bit chained hash folded over the prefix tokens (two 64-bit
// lanes with independent mixing), finalised with the prefix length, so a key
// names the whole prefix.  Entries live in one hash map keyed that way; the
// prompt-end entries that do not sit on a multiple of the match unit are also
// listed, by their offset, under the key of the unit boundary before them, so
// a lookup only probes unit boundaries plus those listed offsets.
// Eviction: least recently used among committed, unpinned entries.

#include "kda_prefix_cache.h"

#include <cstdio>
#include <cstring>
#include <deque>
#include <list>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

namespace {

thread_local std::string g_err;

int fail(const char* msg) {
    g_err = msg;
    return -1;
}

// 64-bit finaliser of MurmurHash3 (a published bijective mixer).
inline uint64_t fmix64(uint64_t k) {
    k ^= k >> 33;
    k *= 0xff51afd7ed558ccdULL;
    k ^= k >> 33;
    k *= 0xc4ceb9fe1a85ec53ULL;
    k ^= k >> 33;
    return k;
}

struct Key {
    uint64_t a, b;
    bool operator==(const Key& o) const { return a == o.a && b == o.b; }
};

struct KeyHash {
    size_t operator()(const Key& k) const { return static_cast<size_t>(k.a ^ (k.b * 0x9e3779b97f4a7c15ULL)); }
};

// Running chain state over a token sequence.
struct Chain {
    uint64_t a = 0x6a09e667f3bcc908ULL, b = 0xbb67ae8584caa73bULL;
    void push(int32_t tok) {
        const uint64_t t = static_cast<uint32_t>(tok);
        a = fmix64(a ^ (t + 0x9e3779b97f4a7c15ULL));
        b = fmix64(b + t * 0xd6e8feb86659fd93ULL + 0x632be59bd9b4e019ULL);
    }
    Key key(int64_t len) const {
        const uint64_t l = static_cast<uint64_t>(len);
        return Key{fmix64(a ^ (l * 0xff51afd7ed558ccdULL)), fmix64(b + l + 0xc4ceb9fe1a85ec53ULL)};
    }
};

struct Entry {
    int32_t slot;
    int64_t pos;
    int64_t step;          // visible once committed_step >= step
    int32_t pins = 0;
    bool tail = false;     // listed under the unit boundary before pos
    Key boundary{0, 0};
    std::list<Key>::iterator lru;   // position in the LRU list (front = most recent)
};

}  // namespace

struct kda_pcache {
    int32_t num_slots, unit, policy;
    size_t ghost_cap;
    int64_t committed = INT64_MIN;
    std::unordered_map<Key, Entry, KeyHash> entries;
    // unit boundary -> (offset, number of entries at that offset) of the entries
    // after it: prompts that share the boundary prefix can end at one offset
    std::unordered_map<Key, std::vector<std::pair<int32_t, int32_t>>, KeyHash> tails;
    std::list<Key> lru;
    std::vector<int32_t> free_slots;
    std::vector<uint8_t> state;            // per slot: 0 free, 1 reserved, 2 owned by an entry
    std::vector<Key> owner;                // key of the entry owning a slot
    std::vector<int32_t> pins;             // per slot pin count
    std::unordered_set<Key, KeyHash> ghosts;
    std::deque<Key> ghost_order;
    int64_t hits = 0, misses = 0, evictions = 0, declined = 0;

    void touch(Entry& e, const Key& k) {
        lru.erase(e.lru);
        lru.push_front(k);
        e.lru = lru.begin();
    }

    void drop_entry(const Key& k) {
        auto it = entries.find(k);
        Entry& e = it->second;
        if (e.tail) {
            auto t = tails.find(e.boundary);
            if (t != tails.end()) {
                const int32_t off = static_cast<int32_t>(e.pos % unit);
                auto& v = t->second;
                for (size_t i = 0; i < v.size(); i++)
                    if (v[i].first == off) {
                        if (--v[i].second == 0) {
                            v[i] = v.back();
                            v.pop_back();
                        }
                        break;
                    }
                if (v.empty()) tails.erase(t);
            }
        }
        lru.erase(e.lru);
        state[e.slot] = 0;
        free_slots.push_back(e.slot);
        entries.erase(it);
    }

    int64_t evictable() const {
        int64_t n = 0;
        for (const auto& kv : entries) n += kv.second.pins == 0 && kv.second.step <= committed;
        return n;
    }

    bool evict_one() {
        for (auto it = lru.end(); it != lru.begin();) {
            --it;
            auto e = entries.find(*it);
            if (e->second.pins == 0 && e->second.step <= committed) {
                drop_entry(*it);
                evictions++;
                return true;
            }
        }
        return false;
    }

    void remember(const Key& k) {
        if (ghost_cap == 0) return;
        if (ghosts.insert(k).second) {
            ghost_order.push_back(k);
            while (ghost_order.size() > ghost_cap) {
                ghosts.erase(ghost_order.front());
                ghost_order.pop_front();
            }
        }
    }
};

extern "C" {

kda_pcache* kda_pcache_create(int32_t num_slots, int32_t unit, int32_t policy, int32_t ghost_capacity) {
    if (num_slots < 1 || unit < 1 || (policy != KDA_PCACHE_KEEP_ALL && policy != KDA_PCACHE_SECOND_HIT) ||
        ghost_capacity < 0) {
        fail("kda_pcache_create: num_slots >= 1, unit >= 1, a known policy and ghost_capacity >= 0 are required");
        return nullptr;
    }
    auto* c = new kda_pcache();
    c->num_slots = num_slots;
    c->unit = unit;
    c->policy = policy;
    c->ghost_cap = ghost_capacity > 0 ? static_cast<size_t>(ghost_capacity) : static_cast<size_t>(num_slots) * 4;
    c->state.assign(num_slots, 0);
    c->owner.assign(num_slots, Key{0, 0});
    c->pins.assign(num_slots, 0);
    c->free_slots.reserve(num_slots);
    for (int32_t s = num_slots - 1; s >= 0; s--) c->free_slots.push_back(s);
    g_err.clear();
    return c;
}

void kda_pcache_destroy(kda_pcache* c) { delete c; }

int64_t kda_pcache_lookup(kda_pcache* c, const int32_t* tokens, int64_t max_len, int32_t* slot) {
    if (!c || (max_len > 0 && !tokens) || !slot) return fail("kda_pcache_lookup: bad arguments");
    *slot = -1;
    Chain ch;
    int64_t best = 0;
    Key best_key{0, 0};
    std::vector<int64_t> wanted;   // prompt-end positions listed under the last unit boundary
    {
        auto t = c->tails.find(ch.key(0));
        if (t != c->tails.end())
            for (const auto& oc : t->second) wanted.push_back(oc.first);
    }
    auto probe = [&](int64_t p) {
        const Key k = ch.key(p);
        auto it = c->entries.find(k);
        if (it != c->entries.end() && it->second.step <= c->committed && it->second.pos == p && p > best) {
            best = p;
            best_key = k;
        }
        return k;
    };
    for (int64_t p = 1; p <= max_len; p++) {
        ch.push(tokens[p - 1]);
        bool listed = false;
        for (size_t i = 0; i < wanted.size(); i++) {
            if (wanted[i] == p) {
                listed = true;
                break;
            }
        }
        if (p % c->unit == 0) {
            const Key k = probe(p);
            wanted.clear();
            auto t = c->tails.find(k);
            if (t != c->tails.end())
                for (const auto& oc : t->second) wanted.push_back(p + oc.first);
        } else if (listed) {
            probe(p);
        }
    }
    if (best == 0) {
        c->misses++;
        return 0;
    }
    Entry& e = c->entries.find(best_key)->second;
    c->touch(e, best_key);
    e.pins++;
    c->pins[e.slot]++;
    c->hits++;
    *slot = e.slot;
    return best;
}

int32_t kda_pcache_release(kda_pcache* c, int32_t slot) {
    if (!c || slot < 0 || slot >= c->num_slots || c->pins[slot] == 0 || c->state[slot] != 2)
        return fail("kda_pcache_release: slot is not pinned");
    c->pins[slot]--;
    c->entries.find(c->owner[slot])->second.pins--;
    return 0;
}

int32_t kda_pcache_reserve(kda_pcache* c, int32_t n, int32_t* slots) {
    if (!c || n < 0 || (n > 0 && !slots)) return fail("kda_pcache_reserve: bad arguments");
    const int64_t short_by = static_cast<int64_t>(n) - static_cast<int64_t>(c->free_slots.size());
    // a refused call evicts nothing
    if (short_by > 0 && c->evictable() < short_by) return fail("kda_pcache_reserve: not enough free or evictable slots");
    while (static_cast<int32_t>(c->free_slots.size()) < n) c->evict_one();
    for (int32_t i = 0; i < n; i++) {
        const int32_t s = c->free_slots.back();
        c->free_slots.pop_back();
        c->state[s] = 1;
        slots[i] = s;
    }
    return n;
}

int32_t kda_pcache_unreserve(kda_pcache* c, int32_t slot) {
    if (!c || slot < 0 || slot >= c->num_slots || c->state[slot] != 1)
        return fail("kda_pcache_unreserve: slot is not reserved");
    c->state[slot] = 0;
    c->free_slots.push_back(slot);
    return 0;
}

}  // extern "C"

namespace {

int32_t insert_key(kda_pcache* c, const Key& k, const Key& boundary, int64_t pos, int32_t slot, int64_t step) {
    auto decline = [&]() {
        c->state[slot] = 0;
        c->free_slots.push_back(slot);
        c->declined++;
        return 0;
    };
    if (c->entries.count(k)) return decline();
    if (c->policy == KDA_PCACHE_SECOND_HIT && !c->ghosts.count(k)) {
        c->remember(k);
        return decline();
    }
    c->lru.push_front(k);
    Entry e;
    e.slot = slot;
    e.pos = pos;
    e.step = step;
    e.lru = c->lru.begin();
    e.tail = pos % c->unit != 0;
    e.boundary = boundary;
    c->entries.emplace(k, e);
    c->state[slot] = 2;
    c->owner[slot] = k;
    if (e.tail) {
        auto& offs = c->tails[boundary];
        const int32_t off = static_cast<int32_t>(pos % c->unit);
        bool have = false;
        for (auto& oc : offs)
            if (oc.first == off) {
                oc.second++;
                have = true;
            }
        if (!have) offs.push_back({off, 1});
    }
    return 1;
}

}  // namespace

extern "C" {

int32_t kda_pcache_insert_many(kda_pcache* c, const int32_t* tokens, int32_t n, const int64_t* pos,
                               const int32_t* slots, int64_t step, int32_t* kept) {
    if (!c || n < 0 || (n > 0 && (!tokens || !pos || !slots))) return fail("kda_pcache_insert: bad arguments");
    for (int32_t i = 0; i < n; i++) {
        if (pos[i] < 1 || (i > 0 && pos[i] <= pos[i - 1]) || slots[i] < 0 || slots[i] >= c->num_slots ||
            c->state[slots[i]] != 1)
            return fail("kda_pcache_insert: positions must be >= 1 and increasing, slots reserved");
        for (int32_t j = 0; j < i; j++)
            if (slots[j] == slots[i]) return fail("kda_pcache_insert: a slot appears twice");
    }
    Chain ch;
    Key boundary = ch.key(0);
    int32_t i = 0, count = 0;
    for (int64_t p = 1; i < n; p++) {
        ch.push(tokens[p - 1]);
        if (p % c->unit == 0) boundary = ch.key(p);
        while (i < n && pos[i] == p) {
            const int32_t r = insert_key(c, ch.key(p), boundary, p, slots[i], step);
            if (kept) kept[i] = r;
            count += r;
            i++;
        }
    }
    return count;
}

int32_t kda_pcache_insert(kda_pcache* c, const int32_t* tokens, int64_t pos, int32_t slot, int64_t step) {
    int32_t kept = 0;
    const int32_t r = kda_pcache_insert_many(c, tokens, 1, &pos, &slot, step, &kept);
    return r < 0 ? r : kept;
}

void kda_pcache_commit(kda_pcache* c, int64_t step) {
    if (c && step > c->committed) c->committed = step;
}

void kda_pcache_stats(const kda_pcache* c, int64_t* out, int32_t n) {
    if (!c || !out) return;
    int64_t pinned = 0;
    for (int32_t p : c->pins) pinned += p > 0;
    const int64_t v[8] = {static_cast<int64_t>(c->entries.size()), static_cast<int64_t>(c->free_slots.size()), pinned,
                          c->hits, c->misses, c->evictions, c->declined, static_cast<int64_t>(c->ghosts.size())};
    for (int32_t i = 0; i < n && i < 8; i++) out[i] = v[i];
}

const char* kda_pcache_last_error(void) { return g_err.c_str(); }

}  // extern "C"
