// pool_fake.cpp -- host-only build of the slot pool for CPU tests: "device"
// slots and tables are host memory, copies are memcpy, streams and events do
// nothing, and copy failures can be injected.  Copies can also be held back
// (queued, applied only when the test says so) to check that the previous
// generation stays intact while a generation's copies are in flight.  Built
// into libmoe_pool_host.so; exports the same moe_pool_* entry points plus the
// moe_pool_fake_* test hooks.  Not part of the GPU library.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <new>
#include <string>
#include <vector>

#include "pool_core.h"

namespace moe {

static thread_local std::string g_err;

int set_error(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

struct FakeBackend {
    moe_pool_config cfg{};
    int nslots = 0;
    uint8_t *slots = nullptr;
    const void **tables = nullptr;
    long fail_after = -1;   // copies allowed before one fails; -1 = never
    long copies = 0;
    bool delay = false;     // queue copies until complete_copies()
    struct Pending {
        void *dst;
        const void *src;
        size_t n;
    };
    std::vector<Pending> pending;

    int init(const moe_pool_config &c)
    {
        cfg = c;
        nslots = c.capacity + c.spares;
        slots = (uint8_t *)calloc((size_t)c.layers * nslots, (size_t)c.expert_bytes);
        tables = (const void **)calloc((size_t)c.layers * 2 * c.experts, sizeof(void *));
        if (!slots || !tables)
            return set_error(MOE_ENOMEM, "fake pool: out of memory");
        return MOE_OK;
    }
    void *slot_ptr(int l, int s) { return slots + ((size_t)l * nslots + s) * cfg.expert_bytes; }
    int wait_retired(int) { return MOE_OK; }
    int copy(int, void *dst, const void *src, size_t n)
    {
        if (fail_after >= 0 && copies >= fail_after)
            return set_error(MOE_EHIP, "fake pool: injected copy failure after %ld copies", copies);
        if (delay)
            pending.push_back({dst, src, n});
        else
            memcpy(dst, src, n);
        ++copies;
        return MOE_OK;
    }
    int upload_table(int l, int buf, const void *const *entries, const void *const **dtab)
    {
        const void **dt = tables + ((size_t)l * 2 + buf) * cfg.experts;
        for (int e = 0; e < cfg.experts; ++e)
            dt[e] = entries[e];
        *dtab = dt;
        return MOE_OK;
    }
    int publish(int, hipStream_t) { return MOE_OK; }
    int retire(int, hipStream_t) { return MOE_OK; }
    int sync()
    {
        complete_copies();   // a synchronisation point lands every copy
        return MOE_OK;
    }
    long complete_copies()
    {
        for (const Pending &p : pending)
            memcpy(p.dst, p.src, p.n);
        const long n = (long)pending.size();
        pending.clear();
        return n;
    }
    void destroy()
    {
        free(slots);
        free(tables);
        slots = nullptr;
        tables = nullptr;
    }
};

}  // namespace moe

struct moe_pool {
    moe::SlotPool<moe::FakeBackend> p;
};

extern "C" {

const char *moe_last_error(void) { return moe::g_err.c_str(); }

int moe_pool_create(const moe_pool_config *cfg, const void *const *src, moe_pool_t *out)
{
    moe::g_err.clear();
    if (!cfg || !out)
        return moe::set_error(MOE_EINVAL, "moe_pool_create: null argument");
    moe_pool *pool = new (std::nothrow) moe_pool();
    if (!pool)
        return moe::set_error(MOE_ENOMEM, "moe_pool_create: out of memory");
    int rc = pool->p.create(*cfg, src);
    if (rc) {
        pool->p.be.destroy();
        delete pool;
        return rc;
    }
    *out = pool;
    return MOE_OK;
}

int moe_pool_prepare(moe_pool_t pool, int layer, const int32_t *ids, int n, hipStream_t compute,
                     const void *const **tab, moe_pool_stats_t *step)
{
    moe::g_err.clear();
    return pool ? pool->p.prepare(layer, ids, n, compute, tab, step)
                : moe::set_error(MOE_EINVAL, "null pool");
}

int moe_pool_pin(moe_pool_t pool, int layer, const int32_t *experts, int n)
{
    moe::g_err.clear();
    return pool ? pool->p.pin(layer, experts, n) : moe::set_error(MOE_EINVAL, "null pool");
}

int moe_pool_retire(moe_pool_t pool, int layer, hipStream_t compute)
{
    moe::g_err.clear();
    return pool ? pool->p.retire(layer, compute) : moe::set_error(MOE_EINVAL, "null pool");
}

int moe_pool_stats(moe_pool_t pool, moe_pool_stats_t *out)
{
    if (!pool || !out)
        return moe::set_error(MOE_EINVAL, "null argument");
    *out = pool->p.tot;
    return MOE_OK;
}

int moe_pool_access_counts(moe_pool_t pool, int64_t *hits, int64_t *misses)
{
    if (!pool || !hits || !misses)
        return moe::set_error(MOE_EINVAL, "null argument");
    pool->p.access_counts(hits, misses);
    return MOE_OK;
}

int moe_pool_reset(moe_pool_t pool)
{
    return pool ? pool->p.reset() : moe::set_error(MOE_EINVAL, "null pool");
}

int moe_pool_destroy(moe_pool_t pool)
{
    if (pool) {
        pool->p.be.destroy();
        delete pool;
    }
    return MOE_OK;
}

// Injection: the next `n` copies succeed, the one after fails (n < 0: never).
int moe_pool_fake_fail_after(moe_pool_t pool, long n)
{
    if (!pool)
        return MOE_EINVAL;
    pool->p.be.fail_after = n < 0 ? -1 : pool->p.be.copies + n;
    return MOE_OK;
}

// Held-back copies: on != 0 queues every later copy until
// moe_pool_fake_complete_copies() (or a synchronising call) applies them in
// order.  pending() is the queue length, pending_dst(i) the destination of
// queued copy i (NULL out of range).
int moe_pool_fake_set_delay(moe_pool_t pool, int on)
{
    if (!pool)
        return MOE_EINVAL;
    pool->p.be.delay = on != 0;
    return MOE_OK;
}

long moe_pool_fake_complete_copies(moe_pool_t pool)
{
    return pool ? pool->p.be.complete_copies() : -1;
}

long moe_pool_fake_pending(moe_pool_t pool)
{
    return pool ? (long)pool->p.be.pending.size() : -1;
}

void *moe_pool_fake_pending_dst(moe_pool_t pool, long i)
{
    if (!pool || i < 0 || i >= (long)pool->p.be.pending.size())
        return nullptr;
    return pool->p.be.pending[(size_t)i].dst;
}

}  // extern "C"
