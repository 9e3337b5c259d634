// Host-only driver for the sanitizer builds (test infrastructure): layout queries on random
// tensor lists and the threaded host AdamW at ragged sizes, offsets and thread counts, from
// several threads at once.  No GPU is used.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <thread>
#include <vector>
#include "zr.h"
int main() {
    std::mt19937_64 rng(1);
    long frags_total = 0;
    for (int it = 0; it < 300; ++it) {
        int nt = 1 + rng() % 40;
        std::vector<int64_t> numels(nt);
        for (auto &x : numels) x = rng() % 4 == 0 ? rng() % 200 : rng() % 300000;
        int nd = 1 + rng() % 70;
        zr_layout *L = nullptr;
        if (zr_layout_create(numels.data(), nt, nd, rng() % 3 ? 100000 : 0, &L)) { printf("create: %s\n", zr_last_error()); return 1; }
        zr_layout_info info; zr_layout_query(L, &info);
        for (int r = 0; r < nd; ++r) {
            int64_t b, e; zr_layout_rank_range(L, r, &b, &e);
            int32_t count = 0;
            zr_layout_fragments(L, b, e, nullptr, 0, &count);
            std::vector<zr_fragment> f(count + 1);
            int32_t got = 0;
            if (zr_layout_fragments(L, b, e, f.data(), count, &got)) { printf("frags: %s\n", zr_last_error()); return 1; }
            frags_total += got;
        }
        for (int s = 0; s < 4; ++s) { int64_t bytes; zr_layout_ledger_bytes(L, s, &bytes); }
        zr_layout_destroy(L);
    }
    zr_adamw_hparams hp = {5e-5, 0.9, 0.999, 1e-8, 0.01, 1.0, 10};
    auto work = [&](int seed) {
        std::mt19937_64 r(seed);
        for (int it = 0; it < 20; ++it) {
            int64_t n = r() % 300000, off = r() % 7;
            std::vector<uint16_t> g(n + off + 1), p(n + off + 1);
            std::vector<float> t(n + off + 1), m(n + off + 1), v(n + off + 1);
            for (int64_t i = 0; i < n + off + 1; ++i) { g[i] = 0x3a00 + (r() & 0xff); t[i] = 0.01f; m[i] = 1e-4f; v[i] = 1e-6f; }
            if (zr_host_adamw_step(g.data() + off, t.data() + off, m.data() + off, v.data() + off, p.data() + off, n, &hp, r() % 5))
                printf("host adamw: %s\n", zr_last_error());
        }
    };
    std::vector<std::thread> th;
    for (int k = 0; k < 4; ++k) th.emplace_back(work, k);
    for (auto &x : th) x.join();
    printf("ok: %ld fragments, simd %s\n", frags_total, zr_host_simd());
    return 0;
}
