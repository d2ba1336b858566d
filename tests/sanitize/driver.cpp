// Exercises the CPU oracle and the host-only slot pool under AddressSanitizer
// and UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py with g++ /
// gcc only; no GPU code).  Every call's return code is checked; a sanitizer
// report aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "moe_w4a16.h"

extern "C" {
void oracle_set_threads(int n);
int oracle_blob_layout(int H, int I, int g, int64_t off[6], int64_t *total);
int oracle_blob_layout_zp(int H, int I, int g, int64_t off[9], int64_t *total);
int oracle_pack_expert(const float *, const float *, const float *, int, int, int, uint8_t *);
int oracle_pack_expert_zp(const float *, const float *, const float *, int, int, int, uint8_t *);
int oracle_quantize_rows(const float *, int, int, int, uint8_t *, uint16_t *);
int oracle_dequant_rows(const uint8_t *, const uint16_t *, int, int, int, double *);
int oracle_quantize_rows_zp(const float *, int, int, int, uint8_t *, uint16_t *, uint8_t *);
int oracle_dequant_rows_zp(const uint8_t *, const uint16_t *, const uint8_t *, int, int, int,
                           double *);
int oracle_route(const uint16_t *, const uint16_t *, const float *, int, int, int, int, int,
                 int32_t *, float *, float *);
int oracle_permute(const int32_t *, int, int, int, int32_t *, int32_t *, int32_t *, int32_t *);
int oracle_expert_ffn_fmt(const uint16_t *, const int32_t *, const int32_t *,
                          const uint8_t *const *, int, int, int, int, int, int, int,
                          const int32_t *, int, double *);
int oracle_shared_ffn(const uint16_t *, const uint16_t *, const uint16_t *, const uint16_t *, int,
                      int, int, const int32_t *, int, double *);
int oracle_shared_gate(const uint16_t *, const uint16_t *, int, int, const int32_t *, int,
                       double *);
int oracle_combine(const double *, const int32_t *, const float *, const double *,
                   const double *, const uint16_t *, int, int, int, uint16_t *, double *);
int oracle_pool_sim(int, int, int, int, int, const int32_t *, const int32_t *, int, int32_t *,
                    int32_t *, int32_t *, int32_t *);
int oracle_profile_pin(const int64_t *, int, int, int, int32_t *);
int oracle_pool_sim_pinned(int, int, int, const int32_t *, int, const int32_t *, const int32_t *,
                           int, int32_t *, int32_t *, int32_t *);
uint16_t oracle_f64_to_f16(double);
int moe_pool_fake_fail_after(moe_pool_t, long);
int moe_pool_fake_set_delay(moe_pool_t, int);
long moe_pool_fake_complete_copies(moe_pool_t);
}

#define CHECK(x)                                                            \
    do {                                                                    \
        int _rc = (x);                                                      \
        if (_rc != 0) {                                                     \
            std::fprintf(stderr, "%s:%d: %s returned %d\n", __FILE__, __LINE__, #x, _rc); \
            std::exit(2);                                                   \
        }                                                                   \
    } while (0)

static void oracle_layer(std::mt19937 &rng, int fmt, int threads)
{
    oracle_set_threads(threads);
    const int H = 64, I = 64, E = 5, k = 2, g = 32, T = 7, Is = 64;
    std::normal_distribution<float> nd(0.0f, 1.0f);
    int64_t off[9], total;
    CHECK(fmt ? oracle_blob_layout_zp(H, I, g, off, &total) : oracle_blob_layout(H, I, g, off, &total));
    std::vector<std::vector<uint8_t>> blobs(E, std::vector<uint8_t>((size_t)total));
    std::vector<const uint8_t *> bp(E);
    for (int e = 0; e < E; ++e) {
        std::vector<float> wg(I * H), wu(I * H), wd(H * I);
        for (auto *v : {&wg, &wu, &wd})
            for (float &f : *v)
                f = 0.02f * nd(rng);
        CHECK(fmt ? oracle_pack_expert_zp(wg.data(), wu.data(), wd.data(), H, I, g, blobs[e].data())
                  : oracle_pack_expert(wg.data(), wu.data(), wd.data(), H, I, g, blobs[e].data()));
        bp[e] = blobs[e].data();
    }
    std::vector<uint16_t> x(T * H), wr(E * H), sg(Is * H), su(Is * H), sd(H * Is), gw(H),
        res(T * H);
    for (auto &v : x) v = oracle_f64_to_f16(nd(rng));
    for (auto &v : res) v = oracle_f64_to_f16(nd(rng));
    for (auto &v : wr) v = oracle_f64_to_f16(0.02 * nd(rng));
    for (auto *a : {&sg, &su, &sd, &gw})
        for (auto &v : *a) v = oracle_f64_to_f16(0.02 * nd(rng));
    std::vector<float> bias(E), w(T * k), lg(T * E);
    for (auto &b : bias) b = nd(rng);
    std::vector<int32_t> idx(T * k), cnt(E), offs(E + 1), perm(T * k), inv(T * k);
    CHECK(oracle_route(x.data(), wr.data(), bias.data(), T, H, E, k, 1, idx.data(), w.data(),
                       lg.data()));
    CHECK(oracle_permute(idx.data(), T, k, E, cnt.data(), offs.data(), perm.data(), inv.data()));
    std::vector<double> y((size_t)T * k * H), s((size_t)T * H), gt(T), o64((size_t)T * H);
    std::vector<int32_t> rows = {0, 3, T * k - 1};
    CHECK(oracle_expert_ffn_fmt(x.data(), perm.data(), offs.data(), bp.data(), T, H, I, E, k, g,
                                fmt, rows.data(), (int)rows.size(), y.data()));
    CHECK(oracle_expert_ffn_fmt(x.data(), perm.data(), offs.data(), bp.data(), T, H, I, E, k, g,
                                fmt, nullptr, 0, y.data()));
    CHECK(oracle_shared_ffn(x.data(), sg.data(), su.data(), sd.data(), T, H, Is, nullptr, 0,
                            s.data()));
    CHECK(oracle_shared_gate(x.data(), gw.data(), T, H, nullptr, 0, gt.data()));
    std::vector<uint16_t> out((size_t)T * H);
    CHECK(oracle_combine(y.data(), inv.data(), w.data(), s.data(), gt.data(), res.data(), T, H, k,
                         out.data(), o64.data()));
    // quantiser round trips on their own
    std::vector<float> m(8 * 128);
    for (float &f : m) f = nd(rng);
    std::vector<uint8_t> q(8 * 64), z(8 * 4);
    std::vector<uint16_t> sc(8 * 4);
    std::vector<double> dq(8 * 128);
    CHECK(oracle_quantize_rows(m.data(), 8, 128, 32, q.data(), sc.data()));
    CHECK(oracle_dequant_rows(q.data(), sc.data(), 8, 128, 32, dq.data()));
    CHECK(oracle_quantize_rows_zp(m.data(), 8, 128, 32, q.data(), sc.data(), z.data()));
    CHECK(oracle_dequant_rows_zp(q.data(), sc.data(), z.data(), 8, 128, 32, dq.data()));
}

static void oracle_policies(std::mt19937 &rng)
{
    const int L = 3, E = 10, C = 4, k = 3, n = 200;
    std::vector<int32_t> lay(n), ids(n * k), hits(n), miss(n), ml(n * k), el(n * k);
    for (int i = 0; i < n; ++i) {
        lay[i] = (int)(rng() % L);
        std::vector<int> all(E);
        for (int e = 0; e < E; ++e) all[e] = e;
        for (int j = 0; j < k; ++j) {
            std::swap(all[j], all[j + rng() % (E - j)]);
            ids[i * k + j] = all[j];
        }
    }
    for (int shift : {3, 0, -1})
        CHECK(oracle_pool_sim(L, E, C, shift, k, lay.data(), ids.data(), n, hits.data(),
                              miss.data(), ml.data(), el.data()));
    std::vector<int64_t> counts(L * E);
    for (auto &c : counts) c = rng() % 50;
    std::vector<int32_t> pinned(L * C);
    CHECK(oracle_profile_pin(counts.data(), L, E, C, pinned.data()));
    CHECK(oracle_pool_sim_pinned(L, E, C, pinned.data(), k, lay.data(), ids.data(), n, hits.data(),
                                 miss.data(), ml.data()));
}

static void fake_pool(std::mt19937 &rng)
{
    const int L = 2, E = 9, k = 3, C = 4, S = 3;
    const int64_t nb = 256;
    std::vector<uint8_t> src((size_t)L * E * nb);
    for (auto &b : src) b = (uint8_t)rng();
    std::vector<const void *> ptrs(L * E);
    for (int i = 0; i < L * E; ++i) ptrs[i] = src.data() + (size_t)i * nb;
    moe_pool_config cfg{L, E, k, C, S, 3, nb};
    moe_pool_t pool = nullptr;
    CHECK(moe_pool_create(&cfg, ptrs.data(), &pool));
    for (int round = 0; round < 2; ++round) {
        CHECK(moe_pool_fake_set_delay(pool, round));
        for (int i = 0; i < 150; ++i) {
            const int l = (int)(rng() % L);
            std::vector<int> all(E);
            for (int e = 0; e < E; ++e) all[e] = e;
            int32_t ids[3];
            for (int j = 0; j < k; ++j) {
                std::swap(all[j], all[j + rng() % (E - j)]);
                ids[j] = all[j];
            }
            const void *const *tab = nullptr;
            moe_pool_stats_t st{};
            if (i == 77) {   // an injected copy failure keeps the previous generation
                moe_pool_fake_fail_after(pool, 0);
                const int rc = moe_pool_prepare(pool, l, ids, k, nullptr, &tab, &st);
                moe_pool_fake_fail_after(pool, -1);
                if (rc == 0)
                    CHECK(moe_pool_retire(pool, l, nullptr));
                continue;
            }
            CHECK(moe_pool_prepare(pool, l, ids, k, nullptr, &tab, &st));
            moe_pool_fake_complete_copies(pool);
            CHECK(moe_pool_retire(pool, l, nullptr));
        }
        int32_t pin[4] = {0, 2, 4, 6};
        CHECK(moe_pool_pin(pool, 1, pin, C));
        moe_pool_stats_t tot{};
        CHECK(moe_pool_stats(pool, &tot));
        CHECK(moe_pool_reset(pool));
    }
    CHECK(moe_pool_destroy(pool));
}

int main()
{
    std::mt19937 rng(12345);
    for (int fmt : {0, 1})
        for (int threads : {1, 3})
            oracle_layer(rng, fmt, threads);
    oracle_policies(rng);
    fake_pool(rng);
    std::printf("sanitized run clean\n");
    return 0;
}
