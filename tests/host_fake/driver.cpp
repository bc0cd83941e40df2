// driver.cpp -- runs the library's host code against the fake HIP runtime
// (fake_hip.cpp) under AddressSanitizer / UndefinedBehaviorSanitizer.  Test
// infrastructure only: prints "ALL OK" and exits 0 when every check passes.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "ar.h"
#include "fake_hip.h"

namespace {

int g_fail = 0;
#define CHECK(c, ...)                                                      \
    do {                                                                   \
        if (!(c)) {                                                        \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);      \
            std::fprintf(stderr, __VA_ARGS__);                             \
            std::fprintf(stderr, "\n");                                    \
            ++g_fail;                                                      \
        }                                                                  \
    } while (0)

// Rank r's fake buffer lives at kBase + r * kStride; nothing is dereferenced.
constexpr uintptr_t kBase = uintptr_t(1) << 44;
constexpr uintptr_t kStride = uintptr_t(1) << 43;   // 8 TiB per rank
constexpr int kMaxN = AR_MAX_RANKS;
// device-0 memory after the rank buffers, for the checker's reference and result
constexpr uintptr_t kAux = kBase + (uintptr_t)kMaxN * kStride;

void* rank_addr(int r, size_t byte_shift) {
    return reinterpret_cast<void*>(kBase + (uintptr_t)r * kStride + byte_shift);
}

size_t eb_of(ar_dtype d) { return d == AR_BFLOAT16 ? 2 : 4; }
bool pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }
int log2i(int n) {
    int l = 0;
    while ((1 << l) < n) ++l;
    return l;
}

// ----------------------------------------------------------- chunk layout
void check_chunk_range() {
    const size_t counts[] = {0, 1, 2, 3, 37, 1000003, (size_t(1) << 40) + 3, SIZE_MAX / 8};
    for (int n = 1; n <= kMaxN; ++n) {
        for (size_t count : counts) {
            const size_t per = count / (size_t)n + (count % (size_t)n ? 1 : 0);
            size_t next = 0, total = 0;
            for (int c = 0; c < n; ++c) {
                size_t off = 0, len = 0;
                CHECK(ar_chunk_range(count, n, c, &off, &len) == AR_OK, "chunk_range n=%d c=%d", n, c);
                const size_t lo = (size_t)c * per < count ? (size_t)c * per : count;
                CHECK(off == lo, "chunk offset n=%d count=%zu c=%d: %zu vs %zu", n, count, c, off, lo);
                CHECK(off == next, "chunks not contiguous n=%d count=%zu c=%d", n, count, c);
                CHECK(len <= per, "chunk longer than L");
                next = off + len;
                total += len;
            }
            CHECK(total == count, "chunks do not cover count=%zu n=%d", count, n);
        }
        size_t o, l;
        CHECK(ar_chunk_range(10, n, -1, &o, &l) == AR_ERR_INVALID_ARG, "chunk -1");
        CHECK(ar_chunk_range(10, n, n, &o, &l) == AR_ERR_INVALID_ARG, "chunk n");
        CHECK(ar_chunk_range(10, n, 0, nullptr, &l) == AR_ERR_INVALID_ARG, "null offset");
    }
    size_t o, l;
    CHECK(ar_chunk_range(10, 0, 0, &o, &l) == AR_ERR_INVALID_ARG, "nranks 0");
    CHECK(ar_chunk_range(10, kMaxN + 1, 0, &o, &l) == AR_ERR_INVALID_ARG, "nranks 65");
}

// ------------------------------------------------------------- cost model
void check_cost_model() {
    const ar_algo algos[] = {AR_ALGO_RING_STEP, AR_ALGO_RING_FUSED, AR_ALGO_TREE,
                             AR_ALGO_HALVING_DOUBLING, AR_ALGO_DOUBLE_TREE, AR_ALGO_TREE_FUSED,
                             AR_ALGO_HALVING_DOUBLING_FUSED, AR_ALGO_DOUBLE_TREE_FUSED};
    const ar_dtype dts[] = {AR_INT32, AR_FLOAT32, AR_BFLOAT16};
    for (int n = 1; n <= kMaxN; ++n)
        for (ar_dtype dt : dts)
            for (int lg = 0; lg <= 40; lg += 5) {
                const size_t count = size_t(1) << lg;
                double best = 1e300;
                ar_algo best_algo = AR_ALGO_RING_FUSED;
                for (ar_algo a : algos) {
                    double us = -1;
                    const ar_status st = ar_predict_us(a, n, count, dt, &us);
                    const bool needs_pow2 = a == AR_ALGO_TREE || a == AR_ALGO_HALVING_DOUBLING ||
                                            a == AR_ALGO_DOUBLE_TREE || a == AR_ALGO_TREE_FUSED ||
                                            a == AR_ALGO_HALVING_DOUBLING_FUSED ||
                                            a == AR_ALGO_DOUBLE_TREE_FUSED;
                    if (needs_pow2 && !pow2(n)) {
                        CHECK(st == AR_ERR_UNSUPPORTED, "predict needs pow2");
                        continue;
                    }
                    CHECK(st == AR_OK && std::isfinite(us) && us > 0, "predict n=%d lg=%d", n, lg);
                    if (us < best) {
                        best = us;
                        best_algo = a;
                    }
                }
                ar_algo got;
                CHECK(ar_auto_algo(n, count, dt, &got) == AR_OK, "auto_algo");
                double got_us = 0;
                (void)ar_predict_us(got, n, count, dt, &got_us);
                CHECK(got_us <= best * (1 + 1e-12), "AUTO is not the argmin n=%d lg=%d (%d vs %d)",
                      n, lg, (int)got, (int)best_algo);
            }
    double us;
    CHECK(ar_predict_us(AR_ALGO_AUTO, 8, 8, AR_FLOAT32, &us) == AR_ERR_INVALID_ARG, "AUTO predict");
    CHECK(ar_predict_us(AR_ALGO_RING_STEP, 8, 8, AR_FLOAT32, nullptr) == AR_ERR_INVALID_ARG, "null");
    CHECK(ar_predict_us((ar_algo)99, 8, 8, AR_FLOAT32, &us) == AR_ERR_INVALID_ARG, "bad algo");
}

// ------------------------------------------------------------ validation
void check_validation(ar_ctx* ctx) {
    fake_clear_executed();
    const long before = fake_counters().kernel_launches;
    void* bufs[kMaxN];
    for (int r = 0; r < kMaxN; ++r) bufs[r] = rank_addr(r, 0);
    auto rejected = [&](ar_status st, ar_status want, const char* what) {
        CHECK(st == want, "%s: got %d want %d (%s)", what, (int)st, (int)want, ar_last_error(ctx));
        CHECK(std::strlen(ar_last_error(ctx)) > 0, "%s: empty last_error", what);
    };
    rejected(ar_allreduce(ctx, nullptr, 4, 16, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "NULL bufs");
    rejected(ar_allreduce(ctx, bufs, 0, 16, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "nranks 0");
    rejected(ar_allreduce(ctx, bufs, kMaxN + 1, 16, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "nranks 65");
    rejected(ar_allreduce(ctx, bufs, 4, 16, (ar_dtype)7, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "bad dtype");
    rejected(ar_allreduce(ctx, bufs, 4, 16, AR_FLOAT32, (ar_op)5, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "bad op");
    rejected(ar_allreduce(ctx, bufs, 4, 16, AR_FLOAT32, AR_SUM, (ar_algo)9), AR_ERR_INVALID_ARG,
             "bad algo");
    rejected(ar_allreduce(ctx, bufs, 4, 16, AR_INT32, AR_AVG, AR_ALGO_RING_FUSED),
             AR_ERR_UNSUPPORTED, "int32 AVG");
    rejected(ar_allreduce(ctx, bufs, 6, 16, AR_FLOAT32, AR_SUM, AR_ALGO_TREE), AR_ERR_UNSUPPORTED,
             "tree on 6 ranks");
    rejected(ar_reduce_scatter(ctx, bufs, 8, 16, AR_FLOAT32, AR_SUM, AR_ALGO_DOUBLE_TREE),
             AR_ERR_UNSUPPORTED, "double tree RS");
    rejected(ar_allgather(ctx, bufs, 8, 16, AR_FLOAT32, AR_ALGO_TREE), AR_ERR_UNSUPPORTED,
             "tree AG");
    rejected(ar_allreduce(ctx, bufs, 4, SIZE_MAX / 2, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "size overflow");

    void* bad[4] = {bufs[0], bufs[1], nullptr, bufs[3]};
    rejected(ar_allreduce(ctx, bad, 4, 16, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "NULL rank");
    void* mis[4] = {bufs[0], rank_addr(1, 2), bufs[2], bufs[3]};
    rejected(ar_allreduce(ctx, mis, 4, 16, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "misaligned fp32");
    void* dup[4] = {bufs[0], bufs[1], bufs[1], bufs[3]};
    rejected(ar_allreduce(ctx, dup, 4, 16, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "overlap");
    void* near[2] = {bufs[0], rank_addr(0, 60)};
    rejected(ar_allreduce(ctx, near, 2, 16, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "partial overlap");
    void* host[2] = {bufs[0], reinterpret_cast<void*>(uintptr_t(0x1000))};
    rejected(ar_allreduce(ctx, host, 2, 16, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "unregistered pointer");
    void* past[2] = {bufs[0], rank_addr(1, kStride - 32)};
    rejected(ar_allreduce(ctx, past, 2, 16, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "runs past its allocation");
    void* other[2] = {bufs[0], reinterpret_cast<void*>(kBase - kStride)};   // device 1 range
    rejected(ar_allreduce(ctx, other, 2, 16, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED),
             AR_ERR_INVALID_ARG, "other device");
    rejected(ar_ring_rs_step(ctx, bufs, 4, 16, AR_FLOAT32, AR_SUM, 3), AR_ERR_INVALID_ARG,
             "RS step 3 of 4 ranks");
    rejected(ar_ring_ag_step(ctx, bufs, 4, 16, AR_FLOAT32, -1), AR_ERR_INVALID_ARG, "AG step -1");
    rejected(ar_tree_step(ctx, bufs, 8, 16, AR_FLOAT32, AR_SUM, 3), AR_ERR_INVALID_ARG,
             "tree step 3 of 8 ranks");
    rejected(ar_dtree_step(ctx, bufs, 8, 16, AR_FLOAT32, AR_SUM, 6), AR_ERR_INVALID_ARG,
             "dtree step 6 of 8 ranks");
    rejected(ar_hd_rs_step(ctx, bufs, 6, 16, AR_FLOAT32, AR_SUM, 0), AR_ERR_UNSUPPORTED,
             "hd step on 6 ranks");
    rejected(ar_copy(ctx, bufs[0], rank_addr(1, 4), 64), AR_ERR_INVALID_ARG, "copy misaligned");
    CHECK(fake_counters().kernel_launches == before, "a rejected call launched a kernel");

    CHECK(ar_allreduce(ctx, bufs, 5, 0, AR_FLOAT32, AR_SUM, AR_ALGO_RING_STEP) == AR_OK, "count 0");
    CHECK(ar_allreduce(ctx, bufs, 1, 99, AR_FLOAT32, AR_AVG, AR_ALGO_TREE) == AR_OK, "one rank");
    CHECK(fake_counters().kernel_launches == before, "a no-op launched a kernel");
}

// ------------------------------------------------------- launch sequences
struct Expect {
    arlib::Kind kind;
    int step;
};

int order_of(int coll, ar_algo algo) {
    if (algo == AR_ALGO_TREE_FUSED) return arlib::ORDER_PAIR;
    if (algo == AR_ALGO_DOUBLE_TREE_FUSED) return arlib::ORDER_DTREE;
    if (algo == AR_ALGO_HALVING_DOUBLING_FUSED && coll != 2) return arlib::ORDER_PAIR_BITREV;
    return arlib::ORDER_RING;
}

std::vector<Expect> expected(int coll, ar_algo algo, int n) {
    std::vector<Expect> e;
    const bool rs = coll != 2, ag = coll != 1;
    const int L = log2i(n);
    switch (algo) {
        case AR_ALGO_RING_FUSED:
        case AR_ALGO_TREE_FUSED:
        case AR_ALGO_HALVING_DOUBLING_FUSED:
        case AR_ALGO_DOUBLE_TREE_FUSED:
            e.push_back({coll == 0 ? arlib::KIND_FUSED_AR
                                   : coll == 1 ? arlib::KIND_FUSED_RS : arlib::KIND_FUSED_AG, 0});
            break;
        case AR_ALGO_TREE:
            for (int s = 0; s < L; ++s) e.push_back({arlib::KIND_TREE_STEP, s});
            break;
        case AR_ALGO_DOUBLE_TREE:
            for (int s = 0; s < 2 * L; ++s) e.push_back({arlib::KIND_DT_STEP, s});
            break;
        case AR_ALGO_HALVING_DOUBLING:
            if (rs) for (int s = 0; s < L; ++s) e.push_back({arlib::KIND_HD_RS_STEP, s});
            if (ag) for (int s = 0; s < L; ++s) e.push_back({arlib::KIND_HD_AG_STEP, s});
            break;
        default:
            if (rs) for (int k = 0; k < n - 1; ++k) e.push_back({arlib::KIND_RS_STEP, k});
            if (ag) for (int k = 0; k < n - 1; ++k) e.push_back({arlib::KIND_AG_STEP, k});
            break;
    }
    return e;
}

ar_status call(ar_ctx* ctx, int coll, void** bufs, int n, size_t count, ar_dtype dt, ar_op op,
               ar_algo algo) {
    if (coll == 0) return ar_allreduce(ctx, bufs, n, count, dt, op, algo);
    if (coll == 1) return ar_reduce_scatter(ctx, bufs, n, count, dt, op, algo);
    return ar_allgather(ctx, bufs, n, count, dt, algo);
}

void check_sequence(const std::vector<FakeLaunch>& got, int coll, ar_algo algo, int n,
                    size_t count, ar_dtype dt, ar_op op, void** bufs, const char* what) {
    const std::vector<Expect> want = expected(coll, algo, n);
    CHECK(got.size() == want.size(), "%s: %zu launches, want %zu", what, got.size(), want.size());
    for (size_t i = 0; i < got.size() && i < want.size(); ++i) {
        const FakeLaunch& l = got[i];
        CHECK(l.plan.kind == want[i].kind && l.plan.step == want[i].step,
              "%s: launch %zu is kind %d step %d", what, i, (int)l.plan.kind, l.plan.step);
        CHECK(l.plan.nranks == n && l.plan.count == count && l.plan.dtype == dt, "%s: plan", what);
        const bool is_ag = l.plan.kind == arlib::KIND_AG_STEP ||
                           l.plan.kind == arlib::KIND_HD_AG_STEP ||
                           l.plan.kind == arlib::KIND_FUSED_AG;
        if (!is_ag) {   // copy kernels ignore the operator
            CHECK(l.plan.op == op, "%s: op", what);
            CHECK(l.args.avg == (op == AR_AVG ? 1 : 0), "%s: avg flag", what);
        }
        for (int r = 0; r < n; ++r) CHECK(l.args.t.p[r] == bufs[r], "%s: rank %d pointer", what, r);
        for (int r = n; r < kMaxN; ++r) CHECK(l.args.t.p[r] == nullptr, "%s: stale pointer", what);
    }
}

void check_launches(ar_ctx* ctx) {
    std::mt19937_64 rng(12345);
    const ar_algo algos[] = {AR_ALGO_RING_STEP, AR_ALGO_RING_FUSED, AR_ALGO_TREE,
                             AR_ALGO_HALVING_DOUBLING, AR_ALGO_DOUBLE_TREE, AR_ALGO_AUTO,
                             AR_ALGO_TREE_FUSED, AR_ALGO_HALVING_DOUBLING_FUSED,
                             AR_ALGO_DOUBLE_TREE_FUSED};
    const ar_dtype dts[] = {AR_INT32, AR_FLOAT32, AR_BFLOAT16};
    const ar_op ops[] = {AR_SUM, AR_MAX, AR_AVG};
    // (the 2^22 .. 2^25 counts put most rank counts over the 128 MiB and 256 MiB
    // thresholds of the residency-capped shapes)
    const size_t special[] = {1, 2, 3, 7, 15, 16, 17, 63, 64, 65, 4095, 4096, 4097, 65536,
                              1000003, (size_t(1) << 22) + 3, (size_t(1) << 23) + 8,
                              (size_t(1) << 24) + 1, (size_t(1) << 25) + 16, size_t(1) << 31,
                              (size_t(1) << 40) + 5};
    int calls = 0;
    for (int iter = 0; iter < 4000; ++iter) {
        const int n = 1 + (int)(rng() % kMaxN);
        const ar_algo algo = algos[rng() % (sizeof algos / sizeof algos[0])];
        const int coll = (int)(rng() % 3);
        const ar_dtype dt = dts[rng() % 3];
        ar_op op = ops[rng() % 3];
        if (dt == AR_INT32 && op == AR_AVG) op = AR_SUM;
        size_t count = rng() % 3 == 0 ? special[rng() % (sizeof special / sizeof special[0])]
                                      : (size_t)(rng() % 200000);
        if (rng() % 4 == 0) count = (size_t)n * (count % 5000 + 1);   // N divides count
        const size_t eb = eb_of(dt);
        // common alignment shift (vector path) or mixed shifts (element path)
        const bool mixed = rng() % 5 == 0;
        const size_t shift = (rng() % (16 / eb)) * eb;
        void* bufs[kMaxN];
        for (int r = 0; r < n; ++r)
            bufs[r] = rank_addr(r, mixed ? ((size_t)r % (16 / eb)) * eb : shift);
        fake_clear_executed();
        const ar_status st = call(ctx, coll, bufs, n, count, dt, op, algo);
        const bool tree_only = algo == AR_ALGO_TREE || algo == AR_ALGO_DOUBLE_TREE ||
                               algo == AR_ALGO_TREE_FUSED || algo == AR_ALGO_DOUBLE_TREE_FUSED;
        const bool needs_pow2 = tree_only || algo == AR_ALGO_HALVING_DOUBLING ||
                                algo == AR_ALGO_HALVING_DOUBLING_FUSED;
        char what[160];
        std::snprintf(what, sizeof what, "coll %d algo %d n %d count %zu dtype %d op %d shift %zu%s",
                      coll, (int)algo, n, count, (int)dt, (int)op, shift, mixed ? " mixed" : "");
        if (tree_only && coll != 0) {
            CHECK(st == AR_ERR_UNSUPPORTED, "%s: %d", what, (int)st);
            continue;
        }
        if (needs_pow2 && !pow2(n)) {
            CHECK(st == AR_ERR_UNSUPPORTED, "%s: %d", what, (int)st);
            continue;
        }
        ar_algo resolved = algo;
        if (algo == AR_ALGO_AUTO) {
            (void)ar_auto_algo(n, count, dt, &resolved);
            if ((resolved == AR_ALGO_TREE || resolved == AR_ALGO_DOUBLE_TREE ||
                 resolved == AR_ALGO_TREE_FUSED || resolved == AR_ALGO_DOUBLE_TREE_FUSED) &&
                coll != 0)
                resolved = AR_ALGO_RING_FUSED;
        }
        // a call whose kernels do not all fit one grid is refused before any launch
        bool fits = true;
        if (n > 1)
            for (const Expect& e : expected(coll, resolved, n)) {
                arlib::Plan p{};
                p.kind = e.kind;
                p.dtype = dt;
                p.op = op;
                p.nranks = n;
                p.count = count;
                p.step = e.step;
                p.vec = !mixed;
                p.mis = mixed ? 0u : (unsigned)shift;
                p.order = order_of(coll, resolved);
                const size_t parts = resolved == AR_ALGO_DOUBLE_TREE_FUSED ? 2 : (size_t)n;
                const size_t cb = (count + parts - 1) / parts * eb;
                const bool fused_kind = e.kind == arlib::KIND_FUSED_AR ||
                                        e.kind == arlib::KIND_FUSED_RS || e.kind == arlib::KIND_FUSED_AG;
                p.lead = fused_kind && p.vec &&
                         !((reinterpret_cast<uintptr_t>(bufs[0]) & 127u) == 0 && cb % 128 == 0);
                arlib::Shape sh;
                fits = fits && arlib::plan_shape(p, &sh);
            }
        if (!fits) {
            CHECK(st == AR_ERR_INVALID_ARG && fake_executed().empty(),
                  "%s: oversized call gave %d and %zu launches", what, (int)st,
                  fake_executed().size());
            continue;
        }
        CHECK(st == AR_OK, "%s: status %d (%s)", what, (int)st, ar_last_error(ctx));
        if (st != AR_OK) continue;
        ++calls;
        if (n == 1) {
            CHECK(fake_executed().empty(), "%s: one rank launched", what);
            continue;
        }
        check_sequence(fake_executed(), coll, resolved, n, count, dt, op, bufs, what);
        const size_t parts = resolved == AR_ALGO_DOUBLE_TREE_FUSED ? 2 : (size_t)n;
        const bool lines = (reinterpret_cast<uintptr_t>(bufs[0]) & 127u) == 0 &&
                           (count + parts - 1) / parts * eb % 128 == 0;
        for (const FakeLaunch& l : fake_executed()) {
            CHECK(l.plan.order == order_of(coll, resolved), "%s: fold order %d", what, l.plan.order);
            const bool vec = !mixed;
            CHECK(l.plan.vec == vec, "%s: vec flag", what);
            CHECK(l.plan.mis == (vec ? (unsigned)shift : 0u), "%s: mis %u", what, l.plan.mis);
            const bool fused_kind = l.plan.kind == arlib::KIND_FUSED_AR ||
                                    l.plan.kind == arlib::KIND_FUSED_RS ||
                                    l.plan.kind == arlib::KIND_FUSED_AG;
            CHECK(l.plan.lead == (fused_kind && vec && !lines), "%s: lead flag %d", what,
                  (int)l.plan.lead);
        }
    }
    CHECK(calls > 1000, "too few accepted calls (%d)", calls);

    // single-step entry points launch exactly one kernel of their kind
    void* bufs[kMaxN];
    for (int r = 0; r < kMaxN; ++r) bufs[r] = rank_addr(r, 0);
    for (int n : {2, 3, 8, 64}) {
        for (int k = 0; k < n - 1; ++k) {
            fake_clear_executed();
            CHECK(ar_ring_rs_step(ctx, bufs, n, 1000, AR_FLOAT32, AR_AVG, k) == AR_OK, "rs step");
            CHECK(ar_ring_ag_step(ctx, bufs, n, 1000, AR_FLOAT32, k) == AR_OK, "ag step");
            CHECK(fake_executed().size() == 2 && fake_executed()[0].plan.kind == arlib::KIND_RS_STEP &&
                      fake_executed()[1].plan.kind == arlib::KIND_AG_STEP &&
                      fake_executed()[0].plan.step == k,
                  "single ring steps n=%d k=%d", n, k);
        }
    }
}

// ----------------------------------------------------------- graph replay
bool same_launch(const FakeLaunch& x, const FakeLaunch& y) {
    const arlib::Args &a = x.args, &b = y.args;
    for (int r = 0; r < kMaxN; ++r)
        if (a.t.p[r] != b.t.p[r]) return false;
    return x.grid == y.grid && x.plan.kind == y.plan.kind && x.plan.step == y.plan.step &&
           a.count == b.count && a.per == b.per && a.n == b.n && a.step == b.step &&
           a.tiles == b.tiles && a.mis == b.mis && a.avg == b.avg && a.nf == b.nf &&
           a.inv == b.inv;
}

void check_graphs(ar_ctx* ctx) {
    FakeCounters& fc = fake_counters();
    void* bufs[kMaxN];
    for (int r = 0; r < kMaxN; ++r) bufs[r] = rank_addr(r, 0);
    const ar_algo multi[] = {AR_ALGO_RING_STEP, AR_ALGO_TREE, AR_ALGO_HALVING_DOUBLING,
                             AR_ALGO_DOUBLE_TREE};
    for (ar_algo algo : multi) {
        CHECK(ar_set_graphs(ctx, 0) == AR_OK, "graphs off");
        fake_clear_executed();
        CHECK(ar_allreduce(ctx, bufs, 8, 5000, AR_FLOAT32, AR_AVG, algo) == AR_OK, "direct");
        const std::vector<FakeLaunch> direct = fake_executed();
        CHECK(ar_set_graphs(ctx, SIZE_MAX) == AR_OK, "graphs on");
        for (int rep = 0; rep < 3; ++rep) {
            const long cap = fc.captures, gl = fc.graph_launches;
            fake_clear_executed();
            CHECK(ar_allreduce(ctx, bufs, 8, 5000, AR_FLOAT32, AR_AVG, algo) == AR_OK, "replay");
            CHECK(fc.graph_launches == gl + 1, "algo %d rep %d: no graph launch", (int)algo, rep);
            CHECK(fc.captures == cap + (rep == 0 ? 1 : 0), "algo %d rep %d: captures", (int)algo, rep);
            const std::vector<FakeLaunch>& got = fake_executed();
            CHECK(got.size() == direct.size(), "algo %d: replay launches %zu vs %zu", (int)algo,
                  got.size(), direct.size());
            for (size_t i = 0; i < got.size() && i < direct.size(); ++i)
                CHECK(same_launch(got[i], direct[i]), "algo %d: replayed launch %zu differs",
                      (int)algo, i);
        }
    }
    // the fused pass is one launch: never replayed
    {
        const long gl = fc.graph_launches;
        CHECK(ar_allreduce(ctx, bufs, 8, 5000, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED) == AR_OK, "fused");
        CHECK(fc.graph_launches == gl, "fused call went through a graph");
    }
    // threshold: 1024 bytes per rank
    CHECK(ar_set_graphs(ctx, 1024) == AR_OK, "threshold");
    {
        const long gl = fc.graph_launches;
        CHECK(ar_allreduce(ctx, bufs, 4, 256, AR_FLOAT32, AR_SUM, AR_ALGO_RING_STEP) == AR_OK, "small");
        CHECK(fc.graph_launches == gl + 1, "1024-byte call not replayed");
        CHECK(ar_allreduce(ctx, bufs, 4, 257, AR_FLOAT32, AR_SUM, AR_ALGO_RING_STEP) == AR_OK, "big");
        CHECK(fc.graph_launches == gl + 1, "1028-byte call replayed");
    }
    // eviction: more distinct shapes than the cache holds
    CHECK(ar_set_graphs(ctx, SIZE_MAX) == AR_OK, "graphs on");
    {
        const long destroyed = fc.execs_destroyed, syncs = fc.event_syncs;
        for (int i = 0; i < 80; ++i)
            CHECK(ar_allreduce(ctx, bufs, 4, 100 + (size_t)i, AR_INT32, AR_SUM,
                               AR_ALGO_RING_STEP) == AR_OK, "eviction call %d", i);
        CHECK(fc.execs_destroyed > destroyed, "no graph was evicted");
        CHECK(fc.event_syncs - syncs >= fc.execs_destroyed - destroyed,
              "an evicted graph was destroyed without waiting for its last replay");
    }
    // a caller capturing the context's stream gets direct launches in its capture
    {
        std::vector<FakeLaunch> sink;
        fake_set_null_stream_capturing(true, &sink);
        const long gl = fc.graph_launches, cap = fc.captures;
        CHECK(ar_allreduce(ctx, bufs, 8, 777, AR_FLOAT32, AR_SUM, AR_ALGO_DOUBLE_TREE) == AR_OK,
              "under caller capture");
        fake_set_null_stream_capturing(false, nullptr);
        CHECK(fc.graph_launches == gl && fc.captures == cap, "library graph used under capture");
        CHECK(sink.size() == 6, "caller capture got %zu launches, want 6", sink.size());
    }
    CHECK(ar_set_graphs(ctx, 0) == AR_OK, "graphs off");
    CHECK(fc.execs_created == fc.execs_destroyed, "graphs left after turning replay off");
    CHECK(fc.events_created == fc.events_destroyed, "events left after turning replay off");
    CHECK(fc.graphs_created == fc.graphs_destroyed, "captured graphs not destroyed");
    CHECK(ar_set_graphs(nullptr, 1) == AR_ERR_INVALID_ARG, "NULL ctx");
}

}  // namespace

// ------------------------------------------------------------- checker
void check_checker(ar_ctx* ctx) {
    FakeCounters& fc = fake_counters();
    void* bufs[kMaxN];
    for (int r = 0; r < kMaxN; ++r) bufs[r] = rank_addr(r, 0);
    auto* res = reinterpret_cast<ar_check_result*>(kAux);
    const auto* ref = reinterpret_cast<const double*>(kAux + 4096);
    const auto* bound = reinterpret_cast<const double*>(kAux + (kStride >> 1));
    // an address the fake runtime does not know (not device memory)
    const auto* host_ref = reinterpret_cast<const double*>(uintptr_t(1) << 40);
    const long l0 = fc.kernel_launches, a0 = fc.device_allocs;
    auto bad = [&](ar_status st, const char* what) {
        CHECK(st == AR_ERR_INVALID_ARG, "%s: status %d", what, (int)st);
    };
    bad(ar_check(ctx, bufs, 8, 100, AR_FLOAT32, nullptr, nullptr, nullptr), "NULL result");
    bad(ar_check(ctx, bufs, 8, 100, AR_FLOAT32, nullptr, nullptr,
                 reinterpret_cast<ar_check_result*>(kAux + 4)), "misaligned result");
    bad(ar_check(ctx, bufs, 8, 100, AR_FLOAT32, nullptr, bound, res), "bound without ref");
    bad(ar_check(ctx, bufs, 8, 4, AR_FLOAT32, host_ref, nullptr, res), "host ref");
    bad(ar_check(ctx, bufs, 8, 100, AR_FLOAT32,
                 reinterpret_cast<const double*>(kAux + kStride - 64), nullptr, res), "short ref");
    bad(ar_check(ctx, bufs, 8, 100, AR_FLOAT32, ref,
                 reinterpret_cast<const double*>(kAux + kStride - 64), res), "short bound");
    bad(ar_check(ctx, bufs, 8, 100, AR_FLOAT32, ref, nullptr,
                 reinterpret_cast<ar_check_result*>(kBase - kStride)), "result on device 1");
    bad(ar_check(ctx, bufs, 0, 100, AR_FLOAT32, nullptr, nullptr, res), "no ranks");
    bad(ar_check(ctx, bufs, 8, 100, (ar_dtype)9, nullptr, nullptr, res), "bad dtype");
    CHECK(fc.kernel_launches == l0 && fc.device_allocs == a0, "a rejected check launched");
    CHECK(ar_check(ctx, bufs, 8, 100000, AR_BFLOAT16, ref, bound, res) == AR_OK, "check");
    CHECK(fc.kernel_launches == l0 + 2 && fc.device_allocs == a0 + 1, "check: 2 launches, 1 alloc");
    CHECK(ar_check(ctx, bufs, 3, 7, AR_INT32, nullptr, nullptr, res) == AR_OK, "check again");
    CHECK(fc.kernel_launches == l0 + 4 && fc.device_allocs == a0 + 1, "scratch kept");
    CHECK(ar_check(ctx, bufs, 3, 0, AR_INT32, nullptr, nullptr, res) == AR_OK, "check count 0");
    CHECK(fc.kernel_launches == l0 + 5, "count 0: the final pass only");
    // the allocation-free variant: same validation, no allocation
    bad(ar_check_noalloc(ctx, bufs, 8, 100, AR_FLOAT32, nullptr, bound, res), "noalloc bound");
    bad(ar_check_noalloc(ctx, bufs, 8, 100, AR_FLOAT32, nullptr, nullptr, nullptr), "noalloc NULL");
    CHECK(fc.kernel_launches == l0 + 5, "a rejected noalloc check launched");
    CHECK(ar_check_noalloc(ctx, bufs, 8, (size_t)1 << 33, AR_FLOAT32, nullptr, nullptr, res) ==
              AR_OK, "noalloc check");
    CHECK(ar_check_noalloc(ctx, bufs, 2, 5, AR_BFLOAT16, ref, bound, res) == AR_OK, "noalloc 2");
    CHECK(fc.kernel_launches == l0 + 9 && fc.device_allocs == a0 + 1, "noalloc allocated");
    CHECK(ar_check_noalloc(nullptr, bufs, 2, 5, AR_INT32, nullptr, nullptr, res) ==
              AR_ERR_INVALID_ARG, "noalloc NULL ctx");
}

void register_all() {
    // rank buffers of device 0, one range on device 1, the checker's arrays
    for (int r = 0; r < kMaxN; ++r) fake_register(rank_addr(r, 0), kStride, 0);
    fake_register(reinterpret_cast<void*>(kBase - kStride), kStride, 1);
    fake_register(reinterpret_cast<void*>(kAux), kStride, 0);
}

// ------------------------------------------------------- pointer cache
// A buffer freed and re-allocated smaller at the same address: rejected on
// the next call unless the caller turned the pointer-set cache on.
void check_pointer_cache() {
    const uintptr_t a = kBase - 3 * kStride, b = a + 8192;
    void* bufs[2] = {reinterpret_cast<void*>(a), reinterpret_cast<void*>(b)};
    auto shrink_to = [&](size_t size) {
        fake_reset_ranges();
        register_all();
        fake_register(bufs[0], size, 0);
        fake_register(bufs[1], size, 0);
    };
    for (int cache = 0; cache <= 1; ++cache) {
        ar_ctx* c = nullptr;
        CHECK(ar_create(&c, 0, nullptr) == AR_OK, "create");
        CHECK(ar_set_pointer_cache(c, cache) == AR_OK, "set pointer cache");
        shrink_to(4096);
        CHECK(ar_allreduce(c, bufs, 2, 1024, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED) == AR_OK,
              "4 KiB buffers, 4 KiB call");
        shrink_to(2048);
        const ar_status st = ar_allreduce(c, bufs, 2, 1024, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED);
        if (cache) CHECK(st == AR_OK, "cache on: the documented stale-size case is not re-checked");
        else CHECK(st == AR_ERR_INVALID_ARG, "cache off: re-allocated smaller buffers rejected");
        CHECK(ar_set_pointer_cache(c, 0) == AR_OK, "cache off again");
        CHECK(ar_allreduce(c, bufs, 2, 1024, AR_FLOAT32, AR_SUM, AR_ALGO_RING_FUSED) ==
                  AR_ERR_INVALID_ARG, "turning the cache off clears it");
        CHECK(ar_destroy(c) == AR_OK, "destroy");
    }
    CHECK(ar_set_pointer_cache(nullptr, 1) == AR_ERR_INVALID_ARG, "NULL ctx");
    fake_reset_ranges();
    register_all();
}

// Residency caps of the fused launches: the LDS a capped block reserves lets
// exactly the cap's number of blocks share a CU's LDS (and never exceeds what
// one block may take); the PACED shape appears only from 8 ranks, on the
// 16-byte path, above its size threshold; AllGather and uncapped shapes
// reserve nothing.
// Calls just below and just above the size thresholds of the capped shapes,
// through the public entry points: every launch they plan passes record()'s
// grid-coverage check, and the PACED and capped DEEP plans among them carry
// the LDS reservation of their cap.
void check_capped_launches(ar_ctx* ctx) {
    using namespace arlib;
    CHECK(ar_set_residency_caps(nullptr, 1) == AR_ERR_INVALID_ARG, "caps on a NULL context");
    for (int on = 1; on >= 0; --on) {
        CHECK(ar_set_residency_caps(ctx, on) == AR_OK, "set residency caps");
        int paced = 0, capped = 0;
        const ar_algo algos[] = {AR_ALGO_RING_FUSED, AR_ALGO_TREE_FUSED,
                                 AR_ALGO_HALVING_DOUBLING_FUSED, AR_ALGO_DOUBLE_TREE_FUSED};
        for (int n : {8, 9, 12, 16, 17, 32, 64})
            for (ar_dtype dt : {AR_INT32, AR_FLOAT32, AR_BFLOAT16})
                for (ar_op op : {AR_SUM, AR_MAX, AR_AVG})
                    for (int coll = 0; coll < 2; ++coll)
                        for (ar_algo algo : algos)
                            for (size_t mib : {128, 256})
                                for (long delta : {-17L, 3L, 4096L})
                                    for (size_t shift : {size_t(0), size_t(4)}) {
                                        if (dt == AR_INT32 && op == AR_AVG) continue;
                                        if (algo != AR_ALGO_RING_FUSED && !pow2(n)) continue;
                                        if ((algo == AR_ALGO_TREE_FUSED ||
                                             algo == AR_ALGO_DOUBLE_TREE_FUSED) && coll != 0)
                                            continue;
                                        const size_t eb = eb_of(dt);
                                        const size_t count = (size_t)((long)((mib << 20) / eb / n) + delta);
                                        void* bufs[kMaxN];
                                        for (int r = 0; r < n; ++r) bufs[r] = rank_addr(r, shift);
                                        fake_clear_executed();
                                        const ar_status st = call(ctx, coll, bufs, n, count, dt, op, algo);
                                        CHECK(st == AR_OK, "capped sweep n=%d dt=%d op=%d coll=%d algo=%d: %d",
                                              n, (int)dt, (int)op, coll, (int)algo, (int)st);
                                        for (const FakeLaunch& l : fake_executed()) {
                                            const unsigned w = fused_waves_per_cu(l.plan);
                                            paced += fused_variant(l.plan) == CFG_PACED;
                                            capped += w > 0;
                                            CHECK(fused_lds_reserve(l.plan) == lds_for_waves(w),
                                                  "reservation and cap disagree");
                                        }
                                    }
        // the AllGather around its two thresholds (8 ranks: 128 MiB over all
        // ranks; more ranks: 512 MiB), ring and halving-doubling algos
        int ag_paced = 0;
        for (int n : {8, 12, 16, 24, 32, 64})
            for (ar_dtype dt : {AR_INT32, AR_BFLOAT16})
                for (ar_algo algo : {AR_ALGO_RING_FUSED, AR_ALGO_HALVING_DOUBLING_FUSED})
                    for (size_t mib : {128, 512})
                        for (long delta : {-17L, 3L, 4096L})
                            for (size_t shift : {size_t(0), size_t(4)}) {
                                if (algo != AR_ALGO_RING_FUSED && !pow2(n)) continue;
                                const size_t count = (size_t)((long)((mib << 20) / eb_of(dt) / n) + delta);
                                void* bufs[kMaxN];
                                for (int r = 0; r < n; ++r) bufs[r] = rank_addr(r, shift);
                                fake_clear_executed();
                                CHECK(call(ctx, 2, bufs, n, count, dt, AR_SUM, algo) == AR_OK,
                                      "AllGather sweep n=%d dt=%d algo=%d", n, (int)dt, (int)algo);
                                for (const FakeLaunch& l : fake_executed()) {
                                    const unsigned w = fused_waves_per_cu(l.plan);
                                    ag_paced += fused_variant(l.plan) == CFG_PACED;
                                    CHECK(fused_lds_reserve(l.plan) == lds_for_waves(w),
                                          "AllGather reservation and cap disagree");
                                    CHECK((w > 0) == (fused_variant(l.plan) == CFG_PACED),
                                          "AllGather cap without PACED");
                                }
                            }
        CHECK(on ? ag_paced > 20 : ag_paced == 0, "AllGather PACED plans: %d (caps %d)", ag_paced, on);
        if (on)
            CHECK(paced > 100 && capped > paced, "capped shapes barely planned (%d PACED, %d capped)",
                  paced, capped);
        else
            CHECK(paced == 0 && capped == 0, "caps off, yet %d PACED and %d capped plans", paced,
                  capped);
    }
    CHECK(ar_set_residency_caps(ctx, 1) == AR_OK, "caps back on");

    // a device with another LDS size per CU: the caps start off and cannot be
    // turned on, and the same large call plans no capped launch
    fake_set_lds_per_cu(64 << 10);
    ar_ctx* other = nullptr;
    CHECK(ar_create(&other, 0, nullptr) == AR_OK && other, "create on a 64 KiB-LDS device");
    if (other) {
        CHECK(ar_set_residency_caps(other, 1) == AR_ERR_UNSUPPORTED, "caps on a 64 KiB-LDS device");
        CHECK(ar_set_residency_caps(other, 0) == AR_OK, "caps off on a 64 KiB-LDS device");
        void* bufs[8];
        for (int r = 0; r < 8; ++r) bufs[r] = rank_addr(r, 0);
        fake_clear_executed();
        CHECK(ar_allreduce(other, bufs, 8, (size_t)64 << 20, AR_FLOAT32, AR_AVG,
                           AR_ALGO_RING_FUSED) == AR_OK, "large call without caps");
        for (const FakeLaunch& l : fake_executed())
            CHECK(fused_variant(l.plan) != CFG_PACED && fused_lds_reserve(l.plan) == 0,
                  "capped launch on a 64 KiB-LDS device");
        CHECK(!fake_executed().empty(), "no launch recorded");
        CHECK(ar_destroy(other) == AR_OK, "destroy");
    }
    fake_set_lds_per_cu(160 << 10);
}

void check_residency_caps() {
    using namespace arlib;
    int paced = 0, capped = 0;
    for (int n : {2, 4, 7, 8, 9, 16, 17, 24, 25, 32, 33, 64})
        for (int dt : {AR_INT32, AR_FLOAT32, AR_BFLOAT16})
            for (int op : {AR_SUM, AR_MAX, AR_AVG})
                for (int kind : {KIND_FUSED_AR, KIND_FUSED_RS, KIND_FUSED_AG})
                    for (int order : {ORDER_RING, ORDER_PAIR, ORDER_PAIR_BITREV, ORDER_DTREE})
                        for (size_t mib : {1, 16, 64, 127, 129, 300, 511, 513, 4096})
                            for (bool vec : {false, true}) {
                                if (order != ORDER_RING && !pow2(n)) continue;
                                Plan p{};
                                p.kind = (Kind)kind;
                                p.dtype = (ar_dtype)dt;
                                p.op = (ar_op)op;
                                p.nranks = n;
                                p.order = order;
                                p.vec = vec;
                                const size_t eb = dt == AR_BFLOAT16 ? 2 : 4;
                                // mib: MiB over all ranks
                                p.count = (mib << 20) / eb / (size_t)n;
                                const size_t total = p.count * eb * (size_t)n;
                                const int cfg = fused_variant(p);
                                const unsigned w = fused_waves_per_cu(p);
                                const unsigned lds = fused_lds_reserve(p);
                                // bf16: only the 8-rank ring SUM / AVG AllReduce
                                const bool bf16_ok = dt != AR_BFLOAT16 ||
                                                     (n == kBatch && kind == KIND_FUSED_AR &&
                                                      order == ORDER_RING && op != AR_MAX);
                                // the AllGather (a copy: any dtype, and the order
                                // plays no part), a higher threshold beyond 8 ranks
                                const size_t ag_min = n == kBatch ? kPacedMinBytes : kAgPacedMinBytes;
                                const bool ag_paced = kind == KIND_FUSED_AG && n >= kBatch && vec &&
                                                      total > ag_min;
                                if (kind == KIND_FUSED_AG)
                                    CHECK((cfg == CFG_PACED) == ag_paced && (cfg == CFG_PACED || cfg == CFG_WIDE),
                                          "AllGather shape n=%d total=%zu cfg=%d", n, total, cfg);
                                if (cfg == CFG_PACED && kind == KIND_FUSED_AG)
                                    CHECK(w == (n <= 8 ? 14u : n <= 16 ? 8u : n <= 24 ? 5u : n <= 32 ? 4u : 3u),
                                          "AllGather cap %u at n=%d", w, n);
                                if (cfg == CFG_PACED && kind != KIND_FUSED_AG)
                                    CHECK(n >= kBatch && vec && bf16_ok && total > kPacedMinBytes,
                                          "PACED n=%d dt=%d kind=%d total=%zu", n, dt, kind, total);
                                if (cfg != CFG_PACED && dt == AR_BFLOAT16 && n == kBatch && vec &&
                                    kind == KIND_FUSED_AR && order == ORDER_RING && op != AR_MAX &&
                                    total > kPacedMinBytes)
                                    CHECK(false, "8-rank bf16 AllReduce not PACED above the threshold");
                                if (kind == KIND_FUSED_AR && n >= kBatch && vec && dt != AR_BFLOAT16 &&
                                    total > kPacedMinBytes && (cfg == CFG_WIDE))
                                    CHECK(false, "WIDE kept above the threshold n=%d", n);
                                // the ReduceScatter's DEEP caps: beyond 16 ranks and
                                // 256 MiB, bf16 MAX excepted
                                if (cfg == CFG_DEEP && kind == KIND_FUSED_RS) {
                                    const unsigned want =
                                        total <= kDeepCapMinBytes || n <= 16 ? 0u
                                        : dt == AR_BFLOAT16 ? (op == AR_MAX ? 0u : 8u)
                                                            : 5u;
                                    CHECK(w == want, "ReduceScatter DEEP cap %u (want %u) n=%d dt=%d op=%d",
                                          w, want, n, dt, op);
                                }
                                if (cfg == CFG_WIDE || cfg == CFG_TINY)
                                    CHECK(w == 0 && lds == 0, "uncapped shape reserves LDS");
                                if (cfg == CFG_PACED) {
                                    CHECK(w >= 3, "PACED without a cap");
                                    ++paced;
                                }
                                if (w == 0) {
                                    CHECK(lds == 0, "LDS without a cap");
                                    continue;
                                }
                                CHECK(lds > 0 && lds <= (64u << 10) && lds % 256 == 0,
                                      "reservation %u", lds);
                                CHECK(kLdsBytesPerCU / lds == w, "cap %u but %u blocks fit (lds %u)",
                                      w, kLdsBytesPerCU / lds, lds);
                                // slack for a coarser allocation granule: rounding
                                // the reservation up by 256 bytes still fits w blocks
                                CHECK(kLdsBytesPerCU / (lds + 256) == w, "cap %u too tight", w);
                                ++capped;
                            }
    CHECK(paced > 50 && capped > paced, "caps barely exercised (%d PACED, %d capped)", paced, capped);
}

int main() {
    register_all();
    check_residency_caps();

    check_chunk_range();
    check_cost_model();

    ar_ctx* bad = nullptr;
    CHECK(ar_create(nullptr, 0, nullptr) == AR_ERR_INVALID_ARG, "create NULL out");
    CHECK(ar_create(&bad, 1, nullptr) == AR_ERR_INVALID_ARG && bad == nullptr, "create device 1");
    CHECK(std::strlen(ar_last_error(nullptr)) > 0, "create error text");
    CHECK(ar_destroy(nullptr) == AR_OK, "destroy NULL");
    for (int s = 0; s <= 5; ++s) CHECK(ar_status_string((ar_status)s) != nullptr, "status string");

    ar_ctx* ctx = nullptr;
    CHECK(ar_create(&ctx, 0, nullptr) == AR_OK && ctx, "create");
    if (ctx) {
        check_validation(ctx);
        check_launches(ctx);
        check_capped_launches(ctx);
        check_graphs(ctx);
        check_checker(ctx);
        check_pointer_cache();
        // the residency probe: argument checks, and its tables freed again
        // (no kernel runs here, so no CU reports)
        unsigned hi = 9, lo = 9, ncu = 9;
        CHECK(ar_residency_probe(nullptr, 0, 1, &hi, &lo, &ncu) == AR_ERR_INVALID_ARG, "probe NULL ctx");
        CHECK(ar_residency_probe(ctx, 0, 1, nullptr, &lo, &ncu) == AR_ERR_INVALID_ARG, "probe NULL out");
        CHECK(ar_residency_probe(ctx, 0, 0, &hi, &lo, &ncu) == AR_ERR_INVALID_ARG, "probe 0 blocks");
        CHECK(ar_residency_probe(ctx, (64u << 10) + 1, 1, &hi, &lo, &ncu) == AR_ERR_INVALID_ARG,
              "probe LDS above 64 KiB");
        const long allocs = fake_counters().device_allocs, frees = fake_counters().device_frees;
        CHECK(ar_residency_probe(ctx, 29696, 1024, &hi, &lo, &ncu) == AR_OK && hi == 0 && lo == 0 &&
                  ncu == 0, "probe on the fake device");
        CHECK(fake_counters().device_allocs - allocs == 1 && fake_counters().device_frees - frees == 1,
              "probe tables not freed");
        // the stream timeline: argument checks, one launch when they pass
        {
            void* tb[8];
            for (int r = 0; r < 8; ++r) tb[r] = rank_addr(r, 0);
            auto* ts = reinterpret_cast<unsigned long long*>(kAux);
            const size_t bytes = (size_t)25 << 20, nblk = bytes / 1024;
            size_t blocks = 0;
            unsigned khz = 0;
            const long launches = fake_counters().kernel_launches;
            CHECK(ar_stream_timeline(nullptr, tb, 8, bytes, 0, ts, 2 * nblk, &blocks, &khz) ==
                      AR_ERR_INVALID_ARG, "timeline NULL ctx");
            CHECK(ar_stream_timeline(ctx, nullptr, 8, bytes, 0, ts, 2 * nblk, &blocks, &khz) ==
                      AR_ERR_INVALID_ARG, "timeline NULL bufs");
            CHECK(ar_stream_timeline(ctx, tb, 0, bytes, 0, ts, 2 * nblk, &blocks, &khz) ==
                      AR_ERR_INVALID_ARG, "timeline 0 buffers");
            CHECK(ar_stream_timeline(ctx, tb, 8, bytes + 8, 0, ts, 2 * nblk + 2, &blocks, &khz) ==
                      AR_ERR_INVALID_ARG, "timeline bytes not a multiple of 16");
            CHECK(ar_stream_timeline(ctx, tb, 8, 0, 0, ts, 2 * nblk, &blocks, &khz) ==
                      AR_ERR_INVALID_ARG, "timeline 0 bytes");
            CHECK(ar_stream_timeline(ctx, tb, 8, bytes, (64u << 10) + 1, ts, 2 * nblk, &blocks,
                                     &khz) == AR_ERR_INVALID_ARG, "timeline LDS above 64 KiB");
            CHECK(ar_stream_timeline(ctx, tb, 8, bytes, 0, ts, 2 * nblk - 1, &blocks, &khz) ==
                      AR_ERR_INVALID_ARG, "timeline ts too short");
            CHECK(ar_stream_timeline(ctx, tb, 8, bytes, 0, ts, 2 * nblk, &blocks, &khz) ==
                      AR_OK, "timeline");
            CHECK(ar_stream_timeline(ctx, tb, 8, bytes, 0,
                                     reinterpret_cast<unsigned long long*>(kAux + 4), 2 * nblk,
                                     &blocks, &khz) == AR_ERR_INVALID_ARG, "timeline ts misaligned");
            CHECK(ar_stream_timeline(ctx, tb, 8, bytes, 0,
                                     reinterpret_cast<unsigned long long*>(rank_addr(3, 4096)),
                                     2 * nblk, &blocks, &khz) == AR_ERR_INVALID_ARG,
                  "timeline ts overlapping a buffer");
            CHECK(ar_stream_timeline(ctx, tb, 8, bytes, 0,
                                     reinterpret_cast<unsigned long long*>(kBase - kStride), 2 * nblk,
                                     &blocks, &khz) == AR_ERR_INVALID_ARG, "timeline ts on device 1");
            void* mis[2] = {tb[0], rank_addr(1, 8)};
            CHECK(ar_stream_timeline(ctx, mis, 2, bytes, 0, ts, 2 * nblk, &blocks, &khz) ==
                      AR_ERR_INVALID_ARG, "timeline buffer not 16-byte aligned");
            blocks = 0;
            khz = 0;
            CHECK(ar_stream_timeline(ctx, tb, 8, bytes - 16, 29696, ts, 2 * nblk, &blocks, &khz) ==
                      AR_OK && blocks == nblk && khz == 100000, "timeline blocks %zu, clock %u kHz",
                  blocks, khz);
            CHECK(ar_stream_timeline(ctx, tb, 8, bytes, 0, ts, 2 * nblk, nullptr, nullptr) == AR_OK,
                  "timeline without outputs");
            CHECK(fake_counters().kernel_launches - launches == 3, "timeline launches: %ld",
                  fake_counters().kernel_launches - launches);
        }
        // leave a few graphs recorded: ar_destroy must release them
        CHECK(ar_set_graphs(ctx, SIZE_MAX) == AR_OK, "graphs on");
        void* bufs[kMaxN];
        for (int r = 0; r < kMaxN; ++r) bufs[r] = rank_addr(r, 0);
        for (int i = 0; i < 3; ++i)
            (void)ar_allreduce(ctx, bufs, 4, 10 + (size_t)i, AR_FLOAT32, AR_SUM, AR_ALGO_TREE);
        CHECK(ar_destroy(ctx) == AR_OK, "destroy");
    }
    const FakeCounters& fc = fake_counters();
    CHECK(fc.execs_created == fc.execs_destroyed && fc.events_created == fc.events_destroyed &&
              fc.streams_created == fc.streams_destroyed && fc.device_allocs == fc.device_frees,
          "ar_destroy left graphs, events, streams or scratch behind");
    // one allocation for the checker's scratch, one for the residency probe's tables
    CHECK(fc.device_allocs == 2 && fc.stream_syncs >= 1, "checker scratch: %ld allocs, %ld syncs",
          fc.device_allocs, fc.stream_syncs);
    const char* msg = nullptr;
    CHECK(fake_coverage_ok(&msg), "launch coverage: %s", msg);
    std::printf("launches %ld, graph launches %ld, captures %ld, evictions %ld\n",
                fc.kernel_launches, fc.graph_launches, fc.captures, fc.execs_destroyed);
    if (g_fail) {
        std::printf("%d FAILED\n", g_fail);
        return 1;
    }
    std::printf("ALL OK\n");
    return 0;
}
