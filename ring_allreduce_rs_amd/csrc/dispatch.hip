// dispatch.hip -- launch shapes and the Plan -> kernel-argument translation
// shared by every kernel family (host code).
#include "common.h"

namespace arlib {

int fused_variant(const Plan& p) {
    if (p.kind == KIND_FUSED_AG) {
        // The AllGather (one read, N - 1 writes per element) takes PACED on
        // large calls, with the cap below.  Measured on MI355X against WIDE
        // without a cap: 8 x 25 MiB fp32 37.2 -> 35.6 us, 8 x 200 MiB 305 ->
        // 269 us, 8 x 2 GiB bf16 3100 -> 2649 us, 16 x 1 GiB int32 3412 ->
        // 2975 us, 32 x 32 MiB 219 -> 175 us, 64 x 64 MiB 941 -> 719 us.  The
        // run-time-N form loses on calls of 512 MiB or less (64 x 8 MiB 93.5
        // -> 97.2 us, 24 x 16 MiB 73.0 -> 75.8, 16 x 9 MiB 26.2 -> 28.7) and
        // the 8-rank form at 8 x 12.5 MiB (17.9 -> 18.4 us).
        const size_t total = p.count * (size_t)elem_bytes(p.dtype) * (size_t)p.nranks;
        const size_t min = p.nranks == kBatch ? kPacedMinBytes : kAgPacedMinBytes;
        return p.caps && p.vec && p.nranks >= kBatch && total > min ? CFG_PACED : CFG_WIDE;
    }
    if (p.kind != KIND_FUSED_AR && p.kind != KIND_FUSED_RS) return CFG_WIDE;
    // Among the uncapped shapes (measured on MI355X, fused AllReduce, inputs
    // cold in HBM): WIDE is best for fp32 / int32 at 8 and 16 ranks
    // (8 x 25 MiB: 74 us vs 83 us DEEP; 16 x 1 GiB: 6.9 ms vs 7.7 ms); DEEP for
    // 64 ranks (64 x 64 MiB: 1.60 ms vs 1.88 ms) and for bf16, whose per-hop
    // rounding makes the fold ALU-heavier and favours the higher occupancy
    // (8 x 2 GiB: 5.97 ms vs 6.39 ms); small chunks are latency-bound and also
    // favour DEEP.  Large calls then trade WIDE for PACED (below).  Beyond
    // DEEP's 32 ranks of loads per batch, chunks of at most 4 KiB take TINY
    // (every rank's element load in flight at once: 64 x 4 KiB 8.3 -> 5.0 us,
    // 64 x 64 KiB 8.1 -> 5.5 us); at 16 KiB chunks its 4-byte loads lose
    // (64 x 1 MiB: 23 -> 32 us).
    const size_t per = ceil_div(p.count, (size_t)fused_parts(p.order, p.nranks)) *
                       (size_t)elem_bytes(p.dtype);
    // (not the double tree: its 64-position in-order scan does not unroll in
    // the TINY shape, and the compiler would keep the pending values in
    // scratch memory; DEEP serves it)
    if (p.nranks > FusedDeep::B && per <= kTinyMaxChunkBytes && p.order != ORDER_DTREE)
        return CFG_TINY;
    const size_t total = p.count * (size_t)elem_bytes(p.dtype) * (size_t)p.nranks;
    const bool big = p.vec && total > kPacedMinBytes;
    // bf16 SUM / AVG AllReduce over 8 ranks: PACED with the 8-rank loop
    // (8 x 2 GiB 5.40 -> 5.34 ms, 8 x 12.5 Mi elements AVG 75.9 -> 68.9 us
    // against capped / uncapped DEEP); bf16 MAX, whose fold is the most ALU
    // per byte here, keeps DEEP without a cap (8 x 128 Mi: 704 us, PACED at
    // best 696 with 10 waves).
    if (p.caps && p.dtype == AR_BFLOAT16 && big && p.nranks == kBatch && p.kind == KIND_FUSED_AR &&
        p.order == ORDER_RING && p.op != AR_MAX)
        return CFG_PACED;
    if (p.dtype == AR_BFLOAT16 || p.nranks > 16) return CFG_DEEP;
    // From 8 ranks up, calls over kPacedMinBytes in all take PACED (WIDE's
    // batches at one unit per lane, residency capped).  Measured on MI355X,
    // fp32 SUM, cold inputs, WIDE -> PACED: 8 x 25 MiB 75.3 -> 69.7 us,
    // 8 x 200 MiB 631 -> 540 us, 16 x 64 MiB 422 -> 342 us, 16 x 1 GiB int32
    // 6.38 -> 5.58 ms, 10 x 64 MiB AVG 246 -> 226 us; at 8 x 16 MiB (128 MiB
    // in all) WIDE still wins, 47.6 vs 49.1 us, and by 17-30 % at 8 x 4-8 MiB.
    // Below 8 ranks a wave's batch is only N KiB; there PACED lost at every
    // cap (2 x 100 MiB: 67.8 us uncapped, 85 us at best capped; 4 x 25 MiB
    // WIDE 36.1 us vs 37.5 us).
    const int wide = p.caps && big && p.nranks >= kBatch ? CFG_PACED : CFG_WIDE;
    // the tree orders have a WIDE kernel for 8 ranks only (a wider one would
    // need a deeper stack of subtree results in registers)
    if (p.order != ORDER_RING) return p.nranks == 8 && p.vec ? wide : CFG_DEEP;
    if (p.nranks <= kBatch) return wide;
    return per <= kDeepMaxChunkBytes ? CFG_DEEP : wide;
}

int fused_units_per_lane(int cfg) {
    return cfg == CFG_DEEP    ? FusedDeep::U
           : cfg == CFG_TINY  ? FusedTiny::U
           : cfg == CFG_PACED ? FusedPaced::U
                              : FusedWide::U;
}

unsigned fused_waves_per_cu(const Plan& p) {
    if (!p.caps) return 0;
    const int cfg = fused_variant(p);
    if (p.kind == KIND_FUSED_AG) {
        if (cfg != CFG_PACED) return 0;
        // A wave writes its 1 KiB tile to N - 1 ranks, so the best cap falls
        // as N grows: about 100-190 KiB of stores in flight per CU.  Sweeps
        // of 2-28 waves per CU on MI355X: 8 ranks best at 14 (8 x 25 MiB
        // 35.6 us, 36.4 at 16, 36.7 at 12; 8 x 2 GiB bf16 2649 us, 2743 at
        // 16, 2694 at 12), 16 at 8 (16 x 1 GiB int32 2975 us, 3008 at 6,
        // 3037 at 12), 24 at 5 (24 x 32 MiB 138.5 us, 149.5 at 4, 152.1 at
        // 6), 32 at 4 (32 x 32 MiB 174.8 us, 191.1 at 5, 197.8 at 3), 48 and
        // 64 at 3 (64 x 64 MiB 719 us, 826 at 2, 754 at 4).
        return p.nranks <= 8 ? 14 : p.nranks <= 16 ? 8 : p.nranks <= 24 ? 5 : p.nranks <= 32 ? 4 : 3;
    }
    if (p.kind != KIND_FUSED_AR && p.kind != KIND_FUSED_RS) return 0;
    // How many waves a CU needs depends on the bytes a wave keeps in flight
    // and on the fold's ALU work per byte: bf16 (widening, rounding, and for
    // MAX the NaN rules hop by hop) wants more waves than an add, an integer
    // max or fp32 MAX (one hardware maximum per hop).  Each cap is the best
    // of a sweep over 3-16 waves per CU (or none), measured on MI355X with
    // cold inputs (fp32 unless named):
    if (cfg == CFG_PACED) {
        // ReduceScatter (N reads, one write): 8 x 25 MiB 39.8 -> 38.6 us,
        // 16 x 256 MiB int32 787 -> 720 us
        if (p.kind == KIND_FUSED_RS) return 10;
        // the pairwise orders: 8 x 25 MiB 77.8 -> 71.9 us (PAIR), 77.3 ->
        // 71.2 us (PAIR_BITREV)
        if (p.order == ORDER_PAIR || p.order == ORDER_PAIR_BITREV) return 7;
        // bf16 SUM / AVG: 8 x 2 GiB 5.34 ms at 6 (5.26 at 5, 5.37 at 7),
        // 8 x 128 Mi elements 693 us at 6-7, 8 x 12.5 Mi AVG 68.9 us at 6
        // (71.0 at 5)
        if (p.dtype == AR_BFLOAT16) return 6;
        // ring and double-tree SUM / AVG / MAX: 8 x 25 MiB 69.7 us at 5
        // (70.7 at 4 and 6), 12 x 64 MiB 261 us at 5, 16 x 64 MiB 342 us at
        // 4-5, 16 x 1 GiB int32 MAX 5.68 ms at 5 (6.20 uncapped), fp32 MAX
        // 8 x 25 MiB 70.1 us at 5 (71.4 at 6), 16 x 268,435,459 5.72 ms at
        // 5 (5.77 at 6).  (How the
        // rank buffers sit in HBM moves the best cap by one: with
        // back-to-back buffers 8 x 25 MiB ran 67.8 us at 4 and 68.9 at 5.)
        return kPacedRingWaves;
    }
    if (cfg == CFG_DEEP && p.kind == KIND_FUSED_AR) {
        // DEEP keeps up to 32 ranks of loads in flight (32 KiB per wave).
        // Small calls lose under any cap (64 x 4 MiB: 107.9 us uncapped,
        // 111.6 at best).  Measured, uncapped -> capped:
        const size_t total = p.count * (size_t)elem_bytes(p.dtype) * (size_t)p.nranks;
        if (total <= kDeepCapMinBytes) return 0;
        if (p.dtype == AR_BFLOAT16) {
            // bf16 MAX: 64 x 16 MiB 476 us uncapped, 473 at 8, 626 at 4;
            // 8 x 256 MiB 704 uncapped, 791 at 8
            if (p.op == AR_MAX) return 0;
            // SUM / AVG: 32 x 32 MiB 410 -> 366 us (4; 3 gave 408), 64 x
            // 16 MiB 458 -> 411 us (4), 16 x 128 MiB 742 -> 703 us (7)
            return p.nranks > 16 ? 4 : 7;
        }
        if (p.nranks <= 16) return 0;
        // fp32 / int32: 64 x 8 MiB 230.5 -> 202.5 us, 64 x 64 MiB 1572 ->
        // 1490 us, 32 x 32 MiB 403 -> 350 us, 64 x 16 MiB int32 MAX 464 ->
        // 383 us, fp32 MAX 476 -> 394 us, 32 x 32 MiB fp32 MAX 407 -> 354
        // us (all at 3)
        return 3;
    }
    if (cfg == CFG_DEEP && p.kind == KIND_FUSED_RS) {
        // The ReduceScatter issues the AllReduce's loads but stores once per
        // element, so its caps sit higher.  Beyond 16 ranks, measured
        // uncapped -> capped (calls of 256 MiB or less lose: 64 x 4 MiB int32
        // 50.3 -> 52.6 us at 5):
        const size_t total = p.count * (size_t)elem_bytes(p.dtype) * (size_t)p.nranks;
        if (total <= kDeepCapMinBytes || p.nranks <= 16) return 0;
        if (p.dtype == AR_BFLOAT16) {
            // bf16 MAX: 64 x 16 MiB 220.8 us uncapped, 242.1 at 10; SUM /
            // AVG: 64 x 16 MiB 193.8 -> 185.7 us, 32 x 32 MiB 181.8 -> 175.4
            // (8; 198 at 6, 179 at 10)
            return p.op == AR_MAX ? 0 : 8;
        }
        // fp32 / int32 at 5: 64 x 16 MiB 191.7 -> 172.3 us, 64 x 8 MiB 98.2
        // -> 91.5, 32 x 32 MiB 179.5 -> 167.9, 32 x 32 MiB int32 MAX 181.5 ->
        // 168.9, 64 x 64 MiB 684.5 -> 656.4, fp32 MAX 64 x 16 MiB 190.5 ->
        // 172.8, 32 x 32 MiB 180.0 -> 167.8 (4 and 6 within 1-3 % of 5, 3,
        // 8 and 10 worse)
        return 5;
    }
    return 0;
}

unsigned fused_lds_reserve(const Plan& p) { return lds_for_waves(fused_waves_per_cu(p)); }

bool plan_shape(const Plan& p, Shape* out) {
    const size_t eb = (size_t)elem_bytes(p.dtype);
    const bool fused = p.kind == KIND_FUSED_AR || p.kind == KIND_FUSED_RS || p.kind == KIND_FUSED_AG;
    // the TINY fused shape moves elements, not 16-byte units
    const size_t epu = p.vec && !(fused && fused_variant(p) == CFG_TINY) ? 16 / eb : 1;
    const size_t threads = fused ? kFusedThreads : kThreads;
    const size_t per_tile =
        threads * (fused ? (size_t)fused_units_per_lane(fused_variant(p)) : (size_t)kUnroll);
    size_t tiles, groups;
    if (p.kind == KIND_TREE_STEP) {
        tiles = ceil_div(ceil_div(p.count, epu), per_tile);
        groups = (size_t)p.nranks / 2;
    } else if (p.kind == KIND_DT_STEP) {
        int L = 0;
        while ((1 << L) < p.nranks) ++L;
        const int s = p.step;
        size_t nodes = 1;
        if (s < L - 1) nodes = (size_t)p.nranks >> (s + 2);
        else if (s > L) nodes = (size_t)p.nranks >> (2 * L - s + 1);
        tiles = ceil_div(ceil_div((p.count + 1) / 2, epu), per_tile);
        groups = 2 * nodes;
    } else if (p.kind == KIND_HD_RS_STEP || p.kind == KIND_HD_AG_STEP) {
        // a step moves d consecutive chunks per rank
        const size_t per = ceil_div(p.count, (size_t)p.nranks);
        const size_t d = p.kind == KIND_HD_RS_STEP ? ((size_t)p.nranks >> (p.step + 1))
                                                   : ((size_t)1 << p.step);
        tiles = ceil_div(ceil_div(per * d, epu), per_tile);
        groups = (size_t)p.nranks;
    } else {
        // ring steps and fused kinds: one group per chunk (fused double tree:
        // per half)
        const size_t parts = fused ? (size_t)fused_parts(p.order, p.nranks) : (size_t)p.nranks;
        const size_t per = ceil_div(p.count, parts);
        const size_t slack = fused && p.lead && epu > 1 ? kLeadUnits : 0;
        tiles = ceil_div(ceil_div(per, epu) + slack, per_tile);
        groups = parts;
    }
    if (tiles == 0) tiles = 1;
    const size_t blocks = tiles * groups;
    if (blocks == 0 || blocks > 0x7fffffffu || tiles > 0xffffffffu) return false;
    out->blocks = (unsigned)blocks;
    out->threads = (unsigned)threads;
    out->tiles = (unsigned)tiles;
    return true;
}

hipError_t launch(const Plan& p, const RankTable& t, hipStream_t stream) {
    Shape sh;
    if (!plan_shape(p, &sh)) return hipErrorInvalidConfiguration;
    const bool fused = p.kind == KIND_FUSED_AR || p.kind == KIND_FUSED_RS || p.kind == KIND_FUSED_AG;
    Args a;
    a.t = t;
    a.count = p.count;
    a.per = ceil_div(p.count, (size_t)(fused ? fused_parts(p.order, p.nranks) : p.nranks));
    a.n = p.nranks;
    a.step = p.step;
    a.tiles = sh.tiles;
    a.mis = p.mis;
    a.avg = p.op == AR_AVG ? 1 : 0;
    a.nf = (float)p.nranks;
    a.inv = (p.nranks & (p.nranks - 1)) == 0 ? 1.0f / (float)p.nranks : 0.0f;
    const dim3 grid(sh.blocks);
    return fused ? launch_fused_kind(p, a, grid, stream) : launch_step_kind(p, a, grid, stream);
}

}  // namespace arlib
