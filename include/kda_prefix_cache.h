/*
 * kda_prefix_cache.h -- host-side prefix cache of KDA states.
 *
 * A recurrent layer can only resume a shared prefix from the state stored at
 * that exact prefix boundary.  This cache maps token prefixes to slots of a
 * state pool (the checkpoint layout of kda.h) that hold the state and conv
 * state after that prefix.  It runs on the host and touches no device memory:
 * the caller moves states with kda_resume / kda_state_checkpoint.
 * [vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM", section
 *  "The Hardest Part: Prefix Caching for KDA": a prefix-match unit finer than
 *  the physical state block, chained fine-grained hashes so that a boundary
 *  identifies the whole prefix, copy-on-write of a hit into a private
 *  destination, and same-step reuse deferred until the state is safe;
 *  agentlenshq "vLLM Kimi K3 Support", section "Agentic Cache Retention
 *  Policies": interval-based retention (fixed intervals and prompt
 *  boundaries) and selective retention that keeps a prefix's state only on
 *  its second hit.]
 *
 * Keys: the prefix tokens[0:p] is identified by a 128-bit chained hash of
 * all p tokens and of p.  Lookups visit every multiple of the match unit and,
 * under each such boundary, the few prompt-end entries registered between it
 * and the next one; the longest visible entry wins.
 *
 * Lifecycle of a slot: kda_pcache_reserve hands out free slots (evicting the
 * least recently used unpinned entries when needed); the caller copies a
 * state into each and registers it with kda_pcache_insert, which either
 * keeps it (entry owns the slot) or declines it (slot back to the free list:
 * duplicate key, or a first sighting under the second-hit policy).  An entry
 * inserted during step s is invisible to lookups until kda_pcache_commit(s)
 * (call it once the copies of step s have completed on the device).  A hit
 * pins its slot until kda_pcache_release; pinned and uncommitted entries are
 * never evicted.
 *
 * Not thread-safe: one engine thread owns a cache.  Errors are reported by
 * return values (negative) and kda_pcache_last_error().
 */
#ifndef KDA_PREFIX_CACHE_H
#define KDA_PREFIX_CACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kda_pcache kda_pcache;

typedef enum {
    KDA_PCACHE_KEEP_ALL = 0,     /* keep every inserted state (interval-based retention) */
    KDA_PCACHE_SECOND_HIT = 1    /* keep a prefix's state only when it is inserted a second time */
} kda_pcache_policy;

/* A cache over slots [0, num_slots) of a state pool.  unit: prefix-match
 * unit in tokens (>= 1).  ghost_capacity: how many first sightings the
 * second-hit policy remembers (0 = num_slots * 4).  NULL on bad arguments. */
kda_pcache* kda_pcache_create(int32_t num_slots, int32_t unit, int32_t policy, int32_t ghost_capacity);
void kda_pcache_destroy(kda_pcache* c);

/* Longest visible cached prefix of tokens[0:p] with p <= max_len.  Returns p
 * (0: no hit) and, on a hit, the slot in *slot (pinned until released). */
int64_t kda_pcache_lookup(kda_pcache* c, const int32_t* tokens, int64_t max_len, int32_t* slot);

/* Unpin a slot returned by kda_pcache_lookup.  Returns 0, or -1 if it was not pinned. */
int32_t kda_pcache_release(kda_pcache* c, int32_t slot);

/* Hand out n free slots into slots[0..n): free ones first, then by evicting
 * least recently used unpinned, committed entries.  Returns n, or -1 (nothing
 * handed out, nothing evicted) if not enough slots can be freed. */
int32_t kda_pcache_reserve(kda_pcache* c, int32_t n, int32_t* slots);

/* Register the state after tokens[0:pos] (pos >= 1) held in a reserved slot,
 * as part of step `step`.  Returns 1 if kept, 0 if declined (the slot is free
 * again), -1 on bad arguments (slot not reserved). */
int32_t kda_pcache_insert(kda_pcache* c, const int32_t* tokens, int64_t pos, int32_t slot, int64_t step);

/* The same for n states of one token sequence at increasing positions
 * pos[0..n) in the reserved slots[0..n), hashing the prefix once; kept[i]
 * (may be NULL) receives 1 or 0 per state.  Returns how many were kept, or -1
 * (nothing registered) on bad arguments. */
int32_t kda_pcache_insert_many(kda_pcache* c, const int32_t* tokens, int32_t n, const int64_t* pos,
                               const int32_t* slots, int64_t step, int32_t* kept);

/* Return a reserved slot that will not be inserted to the free list. */
int32_t kda_pcache_unreserve(kda_pcache* c, int32_t slot);

/* Make the entries inserted in steps <= step visible to lookups. */
void kda_pcache_commit(kda_pcache* c, int64_t step);

/* Counters: [0] entries, [1] free slots, [2] pinned slots, [3] hits,
 * [4] misses, [5] evictions, [6] declined inserts, [7] remembered first
 * sightings.  n = number of counters wanted (<= 8). */
void kda_pcache_stats(const kda_pcache* c, int64_t* out, int32_t n);

/* Message of the last error of this thread ("" if none). */
const char* kda_pcache_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_PREFIX_CACHE_H */
