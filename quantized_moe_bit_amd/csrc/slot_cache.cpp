// Host-side expert slot planner.
//
// The Mference system design keeps a fixed number of expert slots per layer and decides which
// expert occupies which slot with least-frequently-used eviction, recency breaking ties; a hit
// reuses its slot and a miss takes an evictable slot ("Load and ownership"). This planner is
// that bookkeeping for one layer: per slot, the resident expert, the uses of that expert since
// the slot was filled, and the request of its last use. A request lists the experts one call
// needs; its own experts are never evicted by it, so every expert it lists is resident after
// it (the slots its misses need are at most the slots its hits leave free).
//
// Deterministic order: hits first (all of them, in one step), then the missing experts in
// ascending expert order, each taking the lowest free slot, else the evictable slot with the
// lowest use count, then the oldest last use, then the lowest slot index. A request may also name
// protected experts: resident ones keep their slots (not evictable by this request) without
// counting a use, which lets a caller plan the next tile of a chunk while the current tile's
// experts still serve queued work (Mference system design, "Prefill": the next tile is fetched
// while the current one is queued; "Correctness and safety invariants": a slot is not reused
// while queued work owns it).
#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

struct moe_slot_cache {
    int32_t n_experts = 0, n_slots = 0;
    std::vector<int32_t> slot_of;    // [n_experts]: slot or -1
    std::vector<int32_t> expert_in;  // [n_slots]: expert or -1 (free)
    std::vector<int64_t> uses;       // [n_slots]: uses of the resident expert since the fill
    std::vector<int64_t> last;       // [n_slots]: request of the last use
    int64_t request = 0;
};

using qmoe::fail;

moe_status moe_slot_cache_create(int32_t n_experts, int32_t n_slots, moe_slot_cache **out) {
    qmoe::clear_error();
    if (!out) return fail(MOE_E_INVALID, "moe_slot_cache_create: out is NULL");
    *out = nullptr;
    if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS)
        return fail(MOE_E_SHAPE, "moe_slot_cache_create: n_experts %d out of range [1, %d]", n_experts,
                    MOE_MAX_EXPERTS);
    if (n_slots < 1 || n_slots > n_experts)
        return fail(MOE_E_SHAPE, "moe_slot_cache_create: n_slots %d out of range [1, n_experts = %d]", n_slots,
                    n_experts);
    moe_slot_cache *c = new (std::nothrow) moe_slot_cache;
    if (!c) return fail(MOE_E_NOMEM, "moe_slot_cache_create: out of host memory");
    c->n_experts = n_experts;
    c->n_slots = n_slots;
    c->slot_of.assign(n_experts, -1);
    c->expert_in.assign(n_slots, -1);
    c->uses.assign(n_slots, 0);
    c->last.assign(n_slots, -1);
    *out = c;
    return MOE_OK;
}

void moe_slot_cache_destroy(moe_slot_cache *cache) { delete cache; }

moe_status moe_slot_cache_plan(moe_slot_cache *c, const int32_t *experts, int32_t n, int32_t *slot_of,
                               int32_t *fill_expert, int32_t *fill_slot, int32_t *n_fill) {
    return moe_slot_cache_plan_protected(c, experts, n, nullptr, 0, slot_of, fill_expert, fill_slot, n_fill);
}

moe_status moe_slot_cache_plan_protected(moe_slot_cache *c, const int32_t *experts, int32_t n,
                                         const int32_t *protect, int32_t n_protect, int32_t *slot_of,
                                         int32_t *fill_expert, int32_t *fill_slot, int32_t *n_fill) {
    qmoe::clear_error();
    if (!c || !n_fill || (n > 0 && (!experts || !slot_of || !fill_expert || !fill_slot)) ||
        (n_protect > 0 && !protect))
        return fail(MOE_E_INVALID, "moe_slot_cache_plan: NULL argument");
    if (n < 0 || n_protect < 0) return fail(MOE_E_SHAPE, "moe_slot_cache_plan: n = %d or n_protect = %d is negative", n, n_protect);
    *n_fill = 0;
    // the request's distinct experts, ascending
    std::vector<int32_t> want(experts, experts + n);
    for (int32_t e : want)
        if (e < 0 || e >= c->n_experts)
            return fail(MOE_E_INVALID, "moe_slot_cache_plan: expert %d out of range [0, %d)", e, c->n_experts);
    for (int32_t i = 0; i < n_protect; ++i)
        if (protect[i] < 0 || protect[i] >= c->n_experts)
            return fail(MOE_E_INVALID, "moe_slot_cache_plan: protected expert %d out of range [0, %d)", protect[i],
                        c->n_experts);
    std::sort(want.begin(), want.end());
    want.erase(std::unique(want.begin(), want.end()), want.end());
    // slots the request may not evict: those of its own experts (marked below) and of the
    // resident protected experts it does not list
    std::vector<char> in_request(c->n_slots, 0);
    int32_t n_kept = 0;
    for (int32_t i = 0; i < n_protect; ++i) {
        const int32_t s = c->slot_of[protect[i]];
        if (s >= 0 && !in_request[s] && !std::binary_search(want.begin(), want.end(), protect[i])) {
            in_request[s] = 1;
            ++n_kept;
        }
    }
    if ((int32_t)want.size() + n_kept > c->n_slots)
        return fail(MOE_E_CAPACITY, "moe_slot_cache_plan: %zu distinct experts (and %d protected) need more than the %d slots",
                    want.size(), n_kept, c->n_slots);
    const int64_t req = c->request++;
    std::vector<int32_t> misses;
    for (int32_t e : want) {
        const int32_t s = c->slot_of[e];
        if (s >= 0) {
            c->uses[s] += 1;
            c->last[s] = req;
            in_request[s] = 1;
        } else {
            misses.push_back(e);
        }
    }
    int32_t nf = 0;
    for (int32_t e : misses) {
        int32_t pick = -1;
        for (int32_t s = 0; s < c->n_slots && pick < 0; ++s)
            if (c->expert_in[s] < 0) pick = s;
        if (pick < 0) {
            for (int32_t s = 0; s < c->n_slots; ++s) {
                if (in_request[s]) continue;
                if (pick < 0 || c->uses[s] < c->uses[pick] ||
                    (c->uses[s] == c->uses[pick] && c->last[s] < c->last[pick]))
                    pick = s;   // ties beyond count and last use keep the lower slot
            }
        }
        // pick >= 0: the request's distinct experts fit the slots, and none of its own is evictable
        if (c->expert_in[pick] >= 0) c->slot_of[c->expert_in[pick]] = -1;
        c->expert_in[pick] = e;
        c->slot_of[e] = pick;
        c->uses[pick] = 1;
        c->last[pick] = req;
        in_request[pick] = 1;
        fill_expert[nf] = e;
        fill_slot[nf] = pick;
        ++nf;
    }
    for (int32_t i = 0; i < n; ++i) slot_of[i] = c->slot_of[experts[i]];
    *n_fill = nf;
    return MOE_OK;
}

moe_status moe_slot_cache_table(const moe_slot_cache *c, int32_t *expert_slot) {
    qmoe::clear_error();
    if (!c || !expert_slot) return fail(MOE_E_INVALID, "moe_slot_cache_table: NULL argument");
    std::copy(c->slot_of.begin(), c->slot_of.end(), expert_slot);
    return MOE_OK;
}
