// pool_hip.cpp -- HIP backend of the expert slot pool and its C ABI.
// Slots live in HBM; misses are hipMemcpyAsync H2D from the pinned source on
// a side stream; the compute stream waits on an event recorded after the
// copies and the table upload; a per-layer retirement event recorded on the
// compute stream guards reuse of evicted slots and of the older table buffer.
// A pooled layer of one token gets its routed ids from the routing kernel
// itself, written into coherent pinned host memory with a sequence flag.
#include <chrono>
#include <cstring>

#include <hip/hip_runtime.h>

#include "moe_common.h"
#include "trace.h"
#include "pool_core.h"

namespace moe {

struct HipPoolBackend {
    moe_pool_config cfg{};
    int nslots = 0;
    uint8_t *slots = nullptr;            // [L][C+S][bytes]
    const void **tables = nullptr;       // device [L][2][E]
    const void **staging = nullptr;      // pinned host [L][2][E]
    hipStream_t side = nullptr;
    std::vector<hipEvent_t> retire_ev, copies_ev, upload_ev;
    hipEvent_t ids_ev = nullptr;         // routed ids on the host (moe_pool_layer_forward)
    // one token's routed ids written into host memory by the routing kernel
    // (coherent pinned memory: 64 ids, then the flag at byte 256)
    void *mirror = nullptr;
    int32_t *mirror_ids_dev = nullptr;
    unsigned *mirror_flag_dev = nullptr;
    unsigned mirror_seq = 0;
    std::vector<char> retired, uploaded;

    int init(const moe_pool_config &c)
    {
        cfg = c;
        nslots = c.capacity + c.spares;
        const size_t slot_bytes = (size_t)c.layers * nslots * (size_t)c.expert_bytes;
        const size_t tab_bytes = (size_t)c.layers * 2 * c.experts * sizeof(void *);
        size_t freeb = 0, totalb = 0;
        MOE_HIP_TRY(hipMemGetInfo(&freeb, &totalb));
        if (slot_bytes + tab_bytes + (64u << 20) > freeb)
            return set_error(MOE_ECAPACITY,
                             "moe_pool_create: %zu slot bytes do not fit in %zu free bytes",
                             slot_bytes, freeb);
        MOE_HIP_TRY(hipMalloc(&slots, slot_bytes));
        MOE_HIP_TRY(hipMalloc(&tables, tab_bytes));
        MOE_HIP_TRY(hipHostMalloc((void **)&staging, tab_bytes, hipHostMallocDefault));
        MOE_HIP_TRY(hipStreamCreateWithFlags(&side, hipStreamNonBlocking));
        retire_ev.assign(c.layers, nullptr);
        copies_ev.assign(c.layers, nullptr);
        upload_ev.assign((size_t)c.layers * 2, nullptr);
        retired.assign(c.layers, 0);
        uploaded.assign((size_t)c.layers * 2, 0);
        for (auto *v : {&retire_ev, &copies_ev, &upload_ev})
            for (auto &ev : *v)
                MOE_HIP_TRY(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
        MOE_HIP_TRY(hipEventCreateWithFlags(&ids_ev, hipEventDisableTiming));
        MOE_HIP_TRY(hipHostMalloc(&mirror, 512, hipHostMallocCoherent));
        std::memset(mirror, 0, 512);
        void *dev = nullptr;
        MOE_HIP_TRY(hipHostGetDevicePointer(&dev, mirror, 0));
        mirror_ids_dev = static_cast<int32_t *>(dev);
        mirror_flag_dev = reinterpret_cast<unsigned *>(static_cast<char *>(dev) + 256);
        return MOE_OK;
    }
    const int32_t *mirror_ids() const { return static_cast<const int32_t *>(mirror); }
    const unsigned *mirror_flag() const
    {
        return reinterpret_cast<const unsigned *>(static_cast<const char *>(mirror) + 256);
    }
    void *slot_ptr(int l, int s) { return slots + ((size_t)l * nslots + s) * cfg.expert_bytes; }
    int wait_retired(int l)
    {
        if (retired[l])
            MOE_HIP_TRY(hipStreamWaitEvent(side, retire_ev[l], 0));
        return MOE_OK;
    }
    int copy(int, void *dst, const void *src, size_t n)
    {
        MOE_HIP_TRY(hipMemcpyAsync(dst, src, n, hipMemcpyHostToDevice, side));
        return MOE_OK;
    }
    int upload_table(int l, int buf, const void *const *entries, const void *const **dtab)
    {
        const size_t i = (size_t)l * 2 + buf;
        const void **st = staging + i * cfg.experts;
        if (uploaded[i])
            MOE_HIP_TRY(hipEventSynchronize(upload_ev[i]));
        for (int e = 0; e < cfg.experts; ++e)
            st[e] = entries[e];
        const void **dt = tables + i * cfg.experts;
        MOE_HIP_TRY(hipMemcpyAsync((void *)dt, (const void *)st, cfg.experts * sizeof(void *),
                                   hipMemcpyHostToDevice, side));
        MOE_HIP_TRY(hipEventRecord(upload_ev[i], side));
        uploaded[i] = 1;
        *dtab = dt;
        return MOE_OK;
    }
    int publish(int l, hipStream_t compute)
    {
        MOE_HIP_TRY(hipEventRecord(copies_ev[l], side));
        MOE_HIP_TRY(hipStreamWaitEvent(compute, copies_ev[l], 0));
        return MOE_OK;
    }
    int retire(int l, hipStream_t compute)
    {
        MOE_HIP_TRY(hipEventRecord(retire_ev[l], compute));
        retired[l] = 1;
        return MOE_OK;
    }
    int sync()
    {
        MOE_HIP_TRY(hipDeviceSynchronize());
        std::fill(retired.begin(), retired.end(), 0);
        return MOE_OK;
    }
    void destroy()
    {
        if (side)
            (void)hipStreamSynchronize(side);
        (void)hipDeviceSynchronize();
        for (auto *v : {&retire_ev, &copies_ev, &upload_ev})
            for (auto &ev : *v)
                if (ev)
                    (void)hipEventDestroy(ev);
        if (ids_ev)
            (void)hipEventDestroy(ids_ev);
        ids_ev = nullptr;
        if (side)
            (void)hipStreamDestroy(side);
        if (staging)
            (void)hipHostFree(staging);
        if (mirror)
            (void)hipHostFree(mirror);
        mirror = nullptr;
        if (tables)
            (void)hipFree(tables);
        if (slots)
            (void)hipFree(slots);
        side = nullptr;
        staging = nullptr;
        tables = nullptr;
        slots = nullptr;
    }
};

}  // namespace moe

namespace moe {
int launch_ffn_decode(const void *, const int32_t *, const int32_t *, const void *const *,
                      const void *const *, int, int, int, int, int, int, int, int, float *,
                      hipStream_t, const DecodeRoute *);
int route_permute_mirror(const void *, const void *, const float *, int, int, int, int, unsigned,
                         int32_t *, float *, int32_t *, int32_t *, int32_t *, int32_t *, void *,
                         size_t, HostMirror, bool *, hipStream_t);
constexpr double MIRROR_WAIT_S = 10.0;   // far beyond any routing launch
}

struct moe_pool {
    moe::SlotPool<moe::HipPoolBackend> p;
};

extern "C" {

int moe_pool_create(const moe_pool_config *cfg, const void *const *pinned_src, moe_pool_t *out)
{
    MOE_API_RANGE();
    moe::clear_error();
    if (!cfg || !out)
        return moe::set_error(MOE_EINVAL, "moe_pool_create: null argument");
    moe_pool *pool = new (std::nothrow) moe_pool();
    if (!pool)
        return moe::set_error(MOE_ENOMEM, "moe_pool_create: out of host memory");
    int rc = pool->p.create(*cfg, pinned_src);
    if (rc) {
        pool->p.be.destroy();
        delete pool;
        return rc;
    }
    *out = pool;
    return MOE_OK;
}

int moe_pool_prepare(moe_pool_t pool, int layer, const int32_t *host_ids, int n,
                     hipStream_t compute, const void *const **d_table_out, moe_pool_stats_t *step)
{
    MOE_API_RANGE();
    moe::clear_error();
    if (!pool)
        return moe::set_error(MOE_EINVAL, "moe_pool_prepare: null pool");
    return pool->p.prepare(layer, host_ids, n, compute, d_table_out, step);
}

int moe_pool_layer_forward(moe_pool_t pool, int layer, const moe_pool_layer_args *a,
                           hipStream_t stream, moe_pool_stats_t *step)
{
    MOE_API_RANGE();
    moe::clear_error();
    if (!pool || !a || !a->host_ids)
        return moe::set_error(MOE_EINVAL, "moe_pool_layer_forward: null argument");
    auto &P = pool->p;
    if (layer < 0 || layer >= P.cfg.layers)
        return moe::set_error(MOE_EINVAL, "moe_pool_layer_forward: bad layer %d", layer);
    const int E = P.cfg.experts;
    const int n = a->T * a->k;
    // one token: the routing kernel writes the routed ids and then a fresh
    // sequence number into host memory, and this thread spins on it (no
    // device-to-host copy, no event); other shapes copy the ids and wait on
    // an event
    unsigned seq = ++P.be.mirror_seq;
    if (seq == 0)
        seq = ++P.be.mirror_seq;
    bool mirrored = false;
    int rc = moe::route_permute_mirror(
        a->x_f16, a->w_router_f16, a->logit_bias, a->T, a->H, E, a->k, a->flags, a->topk_idx,
        a->topk_w, a->counts, a->offsets, a->perm, a->inv_perm, a->route_ws, a->route_ws_bytes,
        moe::HostMirror{P.be.mirror_ids_dev, P.be.mirror_flag_dev, seq}, &mirrored, stream);
    if (rc)
        return rc;
    if (mirrored) {
        const auto t0 = std::chrono::steady_clock::now();
        for (unsigned it = 0; __atomic_load_n(P.be.mirror_flag(), __ATOMIC_ACQUIRE) != seq; ++it) {
            if ((it & 4095) == 4095 &&
                std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() >
                    moe::MIRROR_WAIT_S) {
                const hipError_t e = hipStreamQuery(stream);
                return moe::set_error(MOE_EHIP,
                                      "moe_pool_layer_forward: routed ids not in host memory "
                                      "after %.0f s (stream: %s)",
                                      moe::MIRROR_WAIT_S, hipGetErrorString(e));
            }
        }
        std::memcpy(a->host_ids, P.be.mirror_ids(), (size_t)n * sizeof(int32_t));
    } else if (n > 0) {
        hipError_t err = hipMemcpyAsync(a->host_ids, a->topk_idx, (size_t)n * sizeof(int32_t),
                                        hipMemcpyDeviceToHost, stream);
        if (err == hipSuccess)
            err = hipEventRecord(P.be.ids_ev, stream);
        if (err == hipSuccess)
            err = hipEventSynchronize(P.be.ids_ev);
        if (err != hipSuccess)
            return moe::set_error(MOE_EHIP, "moe_pool_layer_forward: routed ids: %s",
                                  hipGetErrorString(err));
    }
    // Hits first: every routed expert that was already resident is in the
    // previous generation's table (same slot), a missed one is not, so the
    // decode FFN of the hits runs on that table while the misses are being
    // copied; after the copies, a second launch on the new table computes
    // only the experts the previous one lacked.
    const void *const *old_table = P.layers[layer].table;
    const void *const *table = nullptr;
    moe_pool_stats_t st{};
    rc = P.prepare(layer, a->host_ids, n, stream, &table, &st, /*defer_publish=*/true);
    if (rc)
        return rc;
    if (step)
        *step = st;
    const bool tok = (a->regime & MOE_Y_TOKEN_ORDER) != 0;   // decode: y in token order
    int resolved = 0;
    rc = moe_expert_ffn_plan(a->T, a->H, a->I, E, a->k, a->group, a->regime, &resolved, nullptr,
                             nullptr, nullptr);
    // (a pinned layer's previous table can hold last generation's copies,
    // whose slots this generation's copies may reuse: no split there)
    const bool split = !rc && st.misses > 0 && st.hits > 0 && resolved == MOE_REGIME_DECODE &&
                       !P.layers[layer].pinned;
    if (split) {
        rc = moe_expert_ffn_w4a16(a->x_f16, a->perm, a->offsets, old_table, a->T, a->H, a->I, E,
                                  a->k, a->group, a->regime, a->y, a->y_dtype, a->y_slices,
                                  a->ffn_ws, a->ffn_ws_bytes, stream);
        if (!rc)
            rc = P.publish(layer, stream);
        if (!rc)
            rc = moe::launch_ffn_decode(a->x_f16, a->perm, a->offsets, table, old_table, a->T,
                                        a->H, a->I, E, a->k, a->group,
                                        (a->regime & MOE_W4_ZERO_POINT) ? moe::FMT_ZP
                                                                        : moe::FMT_SYM,
                                        moe::decode_yflags(a->regime),
                                        static_cast<float *>(a->y), stream, nullptr);
    } else if (!rc) {
        rc = P.publish(layer, stream);
        if (!rc)
            rc = moe_expert_ffn_w4a16(a->x_f16, a->perm, a->offsets, table, a->T, a->H, a->I, E,
                                      a->k, a->group, a->regime, a->y, a->y_dtype, a->y_slices,
                                      a->ffn_ws, a->ffn_ws_bytes, stream);
    }
    const int rr = P.retire(layer, stream);   // the generation is released even on failure
    if (rc)
        return rc;
    if (rr)
        return rr;
    return moe_combine(a->y, a->y_dtype, a->y_slices, tok ? nullptr : a->inv_perm, a->topk_w,
                       a->shared_f32,
                       a->residual_f16, a->T, a->H, a->k, a->out_f16, stream);
}

int moe_pool_pin(moe_pool_t pool, int layer, const int32_t *experts, int n)
{
    MOE_API_RANGE();
    moe::clear_error();
    if (!pool)
        return moe::set_error(MOE_EINVAL, "moe_pool_pin: null pool");
    return pool->p.pin(layer, experts, n);
}

int moe_pool_retire(moe_pool_t pool, int layer, hipStream_t compute)
{
    MOE_API_RANGE();
    moe::clear_error();
    if (!pool)
        return moe::set_error(MOE_EINVAL, "moe_pool_retire: null pool");
    return pool->p.retire(layer, compute);
}

int moe_pool_stats(moe_pool_t pool, moe_pool_stats_t *out)
{
    moe::clear_error();
    if (!pool || !out)
        return moe::set_error(MOE_EINVAL, "moe_pool_stats: null argument");
    *out = pool->p.tot;
    return MOE_OK;
}

int moe_pool_access_counts(moe_pool_t pool, int64_t *hits, int64_t *misses)
{
    moe::clear_error();
    if (!pool || !hits || !misses)
        return moe::set_error(MOE_EINVAL, "moe_pool_access_counts: null argument");
    pool->p.access_counts(hits, misses);
    return MOE_OK;
}

int moe_pool_reset(moe_pool_t pool)
{
    MOE_API_RANGE();
    moe::clear_error();
    if (!pool)
        return moe::set_error(MOE_EINVAL, "moe_pool_reset: null pool");
    return pool->p.reset();
}

int moe_pool_destroy(moe_pool_t pool)
{
    MOE_API_RANGE();
    moe::clear_error();
    if (!pool)
        return MOE_OK;
    pool->p.be.destroy();
    delete pool;
    return MOE_OK;
}

}  // extern "C"
