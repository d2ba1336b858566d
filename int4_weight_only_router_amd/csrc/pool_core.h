// pool_core.h -- expert slot pool for partial residency: policy, slot
// bookkeeping and the generation protocol, independent of how bytes move.
//
// Horizon RunMap "03 / Arquitetura" (resident-qpacked-cache-v1) and "07 / De
// volta à oficina": the complete compact source stays immutable in host RAM;
// a missing expert is copied through pinned memory into a temporary GPU slot
// while readers keep the previous generation; once the routed group's copies
// complete, a new complete generation is published; a discarded copy is
// dropped without write-back and its slot is reused only after its
// consumers retire; capacity is fixed before requests and a profile with too
// few spares is rejected; a failure before publication keeps the previous
// generation.  Strata article ("Como 125 bilhões..."): eviction by an access
// counter whose old hits decay.  Constants are a reading: decay
// c <- c - (c >> shift) per routed event of the layer, +65536 per routed
// expert, hits then misses touched in ascending id on a use clock, victim =
// resident non-routed expert with lowest (counter, last use, id).
// Local-inference explainer (lucashiago.com.br), step 4: the other policy
// measures usage first and fixes the most used experts.  A pinned layer
// (pin()) keeps a fixed set of C experts; any other routed expert is copied
// into a spare slot for that generation only and dropped at the next one, so
// a non-pinned expert is paid at every use and nothing is ever evicted.
//
// The Backend provides: init(), slot_ptr(l, s), wait_retired(l),
// copy(l, dst, src, n), upload_table(l, buf, entries) -> device table ptr,
// publish(l, compute), retire(l, compute), sync(), destroy().
#pragma once

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "moe_w4a16.h"

namespace moe {

int set_error(int code, const char *fmt, ...);

template <class Backend>
class SlotPool {
  public:
    moe_pool_config cfg{};
    std::vector<const void *> src;   // [L*E] pinned host blobs
    Backend be;

    struct Layer {
        std::vector<int64_t> cnt, last;  // per expert
        std::vector<int> slot_of;        // expert -> slot or -1
        std::vector<int> expert_in;      // slot -> expert or -1
        int cur_buf = 0;
        bool prepared = false;
        bool publish_pending = false;   // prepared with the compute-stream wait deferred
        const void *const *table = nullptr;
        bool pinned = false;             // fixed resident set (pin())
        std::vector<int> transient;      // pinned layer: this generation's copied misses
    };
    std::vector<Layer> layers;
    int64_t clock = 0;
    moe_pool_stats_t tot{};
    // per (layer, expert), index l*E + e: routed uses that hit a resident
    // slot and uses that missed, since creation or the last reset
    std::vector<int64_t> use_hits, use_misses;

    int nslots() const { return cfg.capacity + cfg.spares; }

    // a committed generation: every routed expert is a use, a hit unless it
    // is among the misses
    void count_uses(int l, const std::vector<char> &inR, const std::vector<int> &misses)
    {
        const size_t b = (size_t)l * cfg.experts;
        for (int e = 0; e < cfg.experts; ++e)
            use_hits[b + e] += inR[e] ? 1 : 0;
        for (int m : misses) {
            use_hits[b + m] -= 1;
            use_misses[b + m] += 1;
        }
    }

    void access_counts(int64_t *hits, int64_t *misses) const
    {
        std::copy(use_hits.begin(), use_hits.end(), hits);
        std::copy(use_misses.begin(), use_misses.end(), misses);
    }

    int create(const moe_pool_config &c, const void *const *pinned_src)
    {
        cfg = c;
        if (c.layers <= 0 || c.experts <= 0 || c.topk <= 0 || c.expert_bytes <= 0 || !pinned_src)
            return set_error(MOE_EINVAL, "moe_pool_create: bad configuration");
        if (c.capacity < c.topk || c.capacity > c.experts || c.spares < c.topk)
            return set_error(MOE_ECAPACITY,
                             "moe_pool_create: profile rejected (C=%d, S=%d, k=%d, E=%d): need "
                             "k <= C <= E and S >= k",
                             c.capacity, c.spares, c.topk, c.experts);
        if (c.expert_bytes % 256)
            return set_error(MOE_EINVAL, "moe_pool_create: expert_bytes must be a multiple of 256");
        src.assign(pinned_src, pinned_src + (size_t)c.layers * c.experts);
        for (const void *p : src)
            if (!p)
                return set_error(MOE_EINVAL, "moe_pool_create: null source blob");
        int rc = be.init(cfg);
        if (rc)
            return rc;
        return place_initial();
    }

    int place_initial()
    {
        layers.assign(cfg.layers, Layer{});
        clock = 0;
        tot = moe_pool_stats_t{};
        use_hits.assign((size_t)cfg.layers * cfg.experts, 0);
        use_misses.assign((size_t)cfg.layers * cfg.experts, 0);
        for (int l = 0; l < cfg.layers; ++l) {
            Layer &L = layers[l];
            L.cnt.assign(cfg.experts, 0);
            L.last.assign(cfg.experts, 0);
            L.slot_of.assign(cfg.experts, -1);
            L.expert_in.assign(nslots(), -1);
            for (int e = 0; e < cfg.capacity; ++e) {
                L.slot_of[e] = e;
                L.expert_in[e] = e;
                L.last[e] = (int64_t)e - cfg.capacity;
                int rc = be.copy(l, be.slot_ptr(l, e), src[(size_t)l * cfg.experts + e],
                                 (size_t)cfg.expert_bytes);
                if (rc)
                    return rc;
            }
            std::vector<const void *> tab(cfg.experts, nullptr);
            for (int e = 0; e < cfg.experts; ++e)
                if (L.slot_of[e] >= 0)
                    tab[e] = be.slot_ptr(l, L.slot_of[e]);
            L.cur_buf = 0;
            int rc = be.upload_table(l, 0, tab.data(), &L.table);
            if (rc)
                return rc;
        }
        return be.sync();
    }

    // defer_publish: the compute stream is not yet made to wait for the
    // copies; the caller enqueues work that reads only the previous
    // generation's experts first, then calls publish().
    int prepare(int l, const int32_t *ids, int n, hipStream_t compute,
                const void *const **table_out, moe_pool_stats_t *step,
                bool defer_publish = false)
    {
        if (l < 0 || l >= cfg.layers || n < 0 || (n > 0 && !ids) || !table_out)
            return set_error(MOE_EINVAL, "moe_pool_prepare: bad arguments");
        Layer &L0 = layers[l];
        if (L0.prepared)
            return set_error(MOE_ESTATE,
                             "moe_pool_prepare: layer %d generation not retired", l);
        const int E = cfg.experts;
        std::vector<char> inR(E, 0);
        int nR = 0;
        for (int i = 0; i < n; ++i) {
            if (ids[i] < 0 || ids[i] >= E)
                return set_error(MOE_EINVAL, "moe_pool_prepare: expert id %d out of range",
                                 ids[i]);
            if (!inR[ids[i]]) {
                inR[ids[i]] = 1;
                ++nR;
            }
        }
        if (nR > cfg.capacity)
            return set_error(MOE_ECAPACITY,
                             "moe_pool_prepare: %d distinct experts exceed capacity %d", nR,
                             cfg.capacity);
        if (L0.pinned)
            return prepare_pinned(l, inR, compute, table_out, step, defer_publish);
        // policy on a copy of the layer state
        Layer L = L0;
        int64_t clk = clock;
        if (cfg.decay_shift >= 0)
            for (int e = 0; e < E; ++e)
                L.cnt[e] -= L.cnt[e] >> cfg.decay_shift;
        for (int e = 0; e < E; ++e)
            if (inR[e])
                L.cnt[e] += 65536;
        int hits = 0;
        std::vector<int> misses, victims;
        for (int e = 0; e < E; ++e)
            if (inR[e] && L.slot_of[e] >= 0) {
                L.last[e] = ++clk;
                ++hits;
            }
        for (int e = 0; e < E; ++e)
            if (inR[e] && L.slot_of[e] < 0)
                misses.push_back(e);
        std::vector<int> spares;
        for (int s = 0; s < nslots(); ++s)
            if (L.expert_in[s] < 0)
                spares.push_back(s);
        if ((int)misses.size() > (int)spares.size())
            return set_error(MOE_ECAPACITY, "moe_pool_prepare: %d misses exceed %d spare slots",
                             (int)misses.size(), (int)spares.size());
        std::vector<int> fill_slot, victim_slot;
        for (size_t i = 0; i < misses.size(); ++i) {
            const int m = misses[i];
            int v = -1;
            for (int c = 0; c < E; ++c) {
                if (L.slot_of[c] < 0 || inR[c])
                    continue;
                if (v < 0 || L.cnt[c] < L.cnt[v] || (L.cnt[c] == L.cnt[v] && L.last[c] < L.last[v]) ||
                    (L.cnt[c] == L.cnt[v] && L.last[c] == L.last[v] && c < v))
                    v = c;
            }
            const int sp = spares[i];
            victims.push_back(v);
            victim_slot.push_back(L.slot_of[v]);
            fill_slot.push_back(sp);
            // the victim leaves the table now; its slot stays occupied (not a
            // spare) until this generation is published and retired
            L.slot_of[v] = -1;
            L.expert_in[sp] = m;
            L.slot_of[m] = sp;
            L.last[m] = ++clk;
        }
        const void *const *dtab = L0.table;
        if (!misses.empty()) {
            // copies of the misses into spare slots (side stream, after earlier
            // readers of those slots retired); table of the new generation
            int rc = be.wait_retired(l);
            if (rc)
                return rc;
            for (size_t i = 0; i < misses.size(); ++i) {
                rc = be.copy(l, be.slot_ptr(l, fill_slot[i]), src[(size_t)l * E + misses[i]],
                             (size_t)cfg.expert_bytes);
                if (rc)
                    return rc;   // nothing published: previous generation and counters intact
            }
            std::vector<const void *> tab(E, nullptr);
            for (int e = 0; e < E; ++e)
                if (L.slot_of[e] >= 0)
                    tab[e] = be.slot_ptr(l, L.slot_of[e]);
            const int nbuf = L.cur_buf ^ 1;
            rc = be.upload_table(l, nbuf, tab.data(), &dtab);
            if (rc)
                return rc;
            if (!defer_publish) {
                rc = be.publish(l, compute);
                if (rc)
                    return rc;
            }
            L.publish_pending = defer_publish;
            L.cur_buf = nbuf;
        }
        // (all hits: the new generation holds the same experts in the same
        // slots, so the published table is the current one, unchanged)
        // commit: the victims' slots become spares (reusable after retirement)
        for (int vs : victim_slot)
            L.expert_in[vs] = -1;
        L.table = dtab;
        L.prepared = true;
        L0 = std::move(L);
        clock = clk;
        moe_pool_stats_t st{};
        st.hits = hits;
        st.misses = (int64_t)misses.size();
        st.evictions = (int64_t)victims.size();
        st.h2d_bytes = st.misses * cfg.expert_bytes;
        count_uses(l, inR, misses);
        tot.hits += st.hits;
        tot.misses += st.misses;
        tot.evictions += st.evictions;
        tot.h2d_bytes += st.h2d_bytes;
        tot.generation += 1;
        st.generation = tot.generation;
        if (step)
            *step = st;
        *table_out = dtab;
        return MOE_OK;
    }

    // Fixes layer l's resident set to experts[0..n) (n = C, distinct): they
    // are copied into the C resident slots (ascending id), the spares are
    // emptied, and from now on the layer follows the pinned policy (until
    // reset()).  Synchronous; the layer's last generation must be retired.
    int pin(int l, const int32_t *experts, int n)
    {
        if (l < 0 || l >= cfg.layers || n != cfg.capacity || !experts)
            return set_error(MOE_EINVAL, "moe_pool_pin: need layer in range and n = C = %d",
                             cfg.capacity);
        Layer &L = layers[l];
        if (L.prepared)
            return set_error(MOE_ESTATE, "moe_pool_pin: layer %d generation not retired", l);
        const int E = cfg.experts;
        std::vector<char> in(E, 0);
        for (int i = 0; i < n; ++i) {
            if (experts[i] < 0 || experts[i] >= E || in[experts[i]])
                return set_error(MOE_EINVAL, "moe_pool_pin: bad or repeated expert id %d",
                                 experts[i]);
            in[experts[i]] = 1;
        }
        int rc = be.wait_retired(l);
        if (rc)
            return rc;
        std::vector<int> slot_of(E, -1), expert_in(nslots(), -1);
        int s = 0;
        for (int e = 0; e < E; ++e)
            if (in[e]) {
                slot_of[e] = s;
                expert_in[s] = e;
                rc = be.copy(l, be.slot_ptr(l, s), src[(size_t)l * E + e], (size_t)cfg.expert_bytes);
                if (rc)
                    return rc;
                ++s;
            }
        std::vector<const void *> tab(E, nullptr);
        for (int e = 0; e < E; ++e)
            if (slot_of[e] >= 0)
                tab[e] = be.slot_ptr(l, slot_of[e]);
        const void *const *dtab = nullptr;
        const int nbuf = L.cur_buf ^ 1;
        rc = be.upload_table(l, nbuf, tab.data(), &dtab);
        if (rc)
            return rc;
        rc = be.sync();
        if (rc)
            return rc;
        L.slot_of = std::move(slot_of);
        L.expert_in = std::move(expert_in);
        L.cnt.assign(E, 0);
        L.last.assign(E, 0);
        L.cur_buf = nbuf;
        L.table = dtab;
        L.pinned = true;
        L.transient.clear();
        return MOE_OK;
    }

    // Pinned layer: hits are the routed experts of the fixed set; every other
    // routed expert (ascending id) is copied into a spare slot for this
    // generation; the previous generation's copies are dropped first.
    int prepare_pinned(int l, const std::vector<char> &inR, hipStream_t compute,
                       const void *const **table_out, moe_pool_stats_t *step, bool defer_publish)
    {
        Layer &L0 = layers[l];
        const int E = cfg.experts;
        Layer L = L0;
        const bool had_transient = !L.transient.empty();
        for (int e : L.transient) {
            L.expert_in[L.slot_of[e]] = -1;
            L.slot_of[e] = -1;
        }
        L.transient.clear();
        int hits = 0;
        std::vector<int> misses;
        for (int e = 0; e < E; ++e) {
            if (!inR[e])
                continue;
            if (L.slot_of[e] >= 0)
                ++hits;
            else
                misses.push_back(e);
        }
        std::vector<int> spares;
        for (int s = 0; s < nslots(); ++s)
            if (L.expert_in[s] < 0)
                spares.push_back(s);
        if (misses.size() > spares.size())
            return set_error(MOE_ECAPACITY, "moe_pool_prepare: %d misses exceed %d spare slots",
                             (int)misses.size(), (int)spares.size());
        for (size_t i = 0; i < misses.size(); ++i) {
            L.expert_in[spares[i]] = misses[i];
            L.slot_of[misses[i]] = spares[i];
            L.transient.push_back(misses[i]);
        }
        const void *const *dtab = L0.table;
        if (!misses.empty() || had_transient) {
            // the spare slots and the older table buffer are rewritten only
            // after the kernels of earlier generations retired
            int rc = be.wait_retired(l);
            if (rc)
                return rc;
            if (!misses.empty()) {
                for (size_t i = 0; i < misses.size(); ++i) {
                    rc = be.copy(l, be.slot_ptr(l, spares[i]), src[(size_t)l * E + misses[i]],
                                 (size_t)cfg.expert_bytes);
                    if (rc)
                        return rc;   // nothing published: previous generation intact
                }
            }
            std::vector<const void *> tab(E, nullptr);
            for (int e = 0; e < E; ++e)
                if (L.slot_of[e] >= 0)
                    tab[e] = be.slot_ptr(l, L.slot_of[e]);
            const int nbuf = L.cur_buf ^ 1;
            rc = be.upload_table(l, nbuf, tab.data(), &dtab);
            if (rc)
                return rc;
            if (!defer_publish) {
                rc = be.publish(l, compute);
                if (rc)
                    return rc;
            }
            L.publish_pending = defer_publish;
            L.cur_buf = nbuf;
        }
        L.table = dtab;
        L.prepared = true;
        L0 = std::move(L);
        moe_pool_stats_t st{};
        st.hits = hits;
        st.misses = (int64_t)misses.size();
        st.evictions = 0;
        st.h2d_bytes = st.misses * cfg.expert_bytes;
        count_uses(l, inR, misses);
        tot.hits += st.hits;
        tot.misses += st.misses;
        tot.h2d_bytes += st.h2d_bytes;
        tot.generation += 1;
        st.generation = tot.generation;
        if (step)
            *step = st;
        *table_out = dtab;
        return MOE_OK;
    }

    // Makes `compute` wait for the copies of a deferred prepare (no-op otherwise).
    int publish(int l, hipStream_t compute)
    {
        Layer &L = layers[l];
        if (!L.publish_pending)
            return MOE_OK;
        int rc = be.publish(l, compute);
        if (rc)
            return rc;
        L.publish_pending = false;
        return MOE_OK;
    }

    int retire(int l, hipStream_t compute)
    {
        if (l < 0 || l >= cfg.layers)
            return set_error(MOE_EINVAL, "moe_pool_retire: bad layer %d", l);
        if (!layers[l].prepared)
            return set_error(MOE_ESTATE, "moe_pool_retire: layer %d has nothing to retire", l);
        int rc = publish(l, compute);   // a deferred publish never outlives its generation
        if (rc)
            return rc;
        rc = be.retire(l, compute);
        if (rc)
            return rc;
        layers[l].prepared = false;
        return MOE_OK;
    }

    int reset()
    {
        int rc = be.sync();
        if (rc)
            return rc;
        return place_initial();
    }
};

}  // namespace moe
