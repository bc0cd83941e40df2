/*
 * ar.h -- C ABI of the single-GPU AllReduce library (libar.so).
 *
 * N logical ranks are N equal-length buffers in one GPU's HBM.  The library
 * reduces them elementwise (SUM, MAX, or AVG = SUM then divide by N) so that
 * every buffer ends with the same result, the way an AllReduce leaves every
 * participant with the reduction of all participants' data ("AllReduce",
 * compassingai.com, section 3 技术原理; "AllReduce 集合通信", zzmblog.top,
 * section 语义).  Operations are in place, like torch.distributed.all_reduce
 * ("Allreduce：大模型分布式训练的核心通信算法与优化实践", pwwt.cn, section 3.2).
 *
 * Conventions shared by every call below:
 *  - bufs: a HOST array of nranks DEVICE pointers, read only during the call.
 *    The caller owns the buffers; each holds `count` elements of `dtype`,
 *    contiguous, naturally aligned, on the context's device, and no two
 *    buffers overlap.  1 <= nranks <= AR_MAX_RANKS.
 *  - Chunks: element range of chunk c is given by ar_chunk_range: chunk length
 *    L = ceil(count / nranks); chunk c = [min(c*L, count), min((c+1)*L, count)).
 *    Trailing chunks may be short or empty when nranks does not divide count.
 *  - Every compute call validates its arguments first and returns an error
 *    before launching anything if they are invalid.  Otherwise it enqueues the
 *    kernels on the context's stream and returns AR_OK without waiting; a
 *    device fault surfaces at the caller's next synchronisation of that stream.
 *  - count == 0 and nranks == 1 are successful no-ops (AVG over one rank is
 *    the identity).
 *  - No call allocates device memory for data: the pointer table travels by
 *    value in the kernel arguments.  (With ar_set_graphs on, the HIP runtime
 *    allocates what an instantiated graph needs, once per recorded graph; the
 *    first ar_check on a context allocates the checker's 80 KiB scratch.)
 *  - No C++ exception crosses this interface.  A context is not thread-safe;
 *    use one per host thread / stream.
 *  - ar_last_error(ctx) describes the most recent failure on that context.
 *  - Alignment and speed: any element-aligned address is accepted.  Buffers
 *    that share their address modulo 16 take the 16-byte path (element-wise
 *    heads and tails per chunk); otherwise the whole call runs element by
 *    element.  On the 16-byte path, chunks whose bodies start off a 128-byte
 *    line of bufs[0] have their tiles shifted onto lines, so they move no
 *    more bytes than aligned ones.
 *  - Every call checks that each buffer is device memory of the context's
 *    device and that `count` elements lie inside its allocation (the runtime
 *    reports an allocation's extent; a sub-allocation of a caching allocator
 *    is checked against the whole segment).  ar_set_pointer_cache can trade
 *    that per-call check for a cache of recently checked pointer sets.
 *  - Large one-pass AllReduce / ReduceScatter / AllGather calls launch with
 *    dynamic LDS that no kernel uses for data: it caps the waves resident
 *    per compute unit (ar_set_residency_caps turns this off).
 */
#ifndef RING_ALLREDUCE_AR_H
#define RING_ALLREDUCE_AR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AR_MAX_RANKS 64

/* Under C++ the enums below have int as their fixed underlying type, so any
 * int a C caller passes (including out-of-range values, which the library
 * rejects) is a valid value of the enum type; the ABI is the same as C's. */
#ifdef __cplusplus
#define AR_ENUM_INT : int
#else
#define AR_ENUM_INT
#endif

typedef struct ar_ctx ar_ctx;

typedef enum ar_status AR_ENUM_INT {
    AR_OK = 0,
    AR_ERR_INVALID_ARG = 1,   /* bad pointer, size, enum, overlap, step index */
    AR_ERR_UNSUPPORTED = 2,   /* valid but not defined: int32 AVG, the tree algorithms
                                 (TREE, HALVING_DOUBLING, DOUBLE_TREE and their fused forms)
                                 on non-power-of-two N, TREE / TREE_FUSED / DOUBLE_TREE /
                                 DOUBLE_TREE_FUSED on ReduceScatter / AllGather */
    AR_ERR_RUNTIME = 3,       /* the HIP runtime reported an error */
    AR_ERR_NO_MEMORY = 4      /* host allocation of the context failed */
} ar_status;

typedef enum ar_dtype AR_ENUM_INT { AR_INT32 = 0, AR_FLOAT32 = 1, AR_BFLOAT16 = 2 } ar_dtype;

/* Reduction operator.  Per-hop arithmetic: int32 SUM wraps (two's complement);
 * fp32 SUM is one binary32 round-to-nearest-even add per hop; bf16 SUM adds in
 * fp32 and rounds the sum to bf16 (nearest-even) at every hop; MAX is
 * IEEE-754-2019 maximum (NaN wins, +0 > -0; a NaN result is the canonical
 * quiet NaN).  AVG is SUM followed by one division of the finished sum by N
 * (DDP's divide by world size: pwwt.cn page, sections 3.1-3.2): fp32 correctly
 * rounded, bf16 rounded from the fp32 quotient.  AVG on int32 is
 * AR_ERR_UNSUPPORTED. */
typedef enum ar_op AR_ENUM_INT { AR_SUM = 0, AR_MAX = 1, AR_AVG = 2 } ar_op;

/* Algorithm.
 *  RING_STEP  -- the ring as the pages lay it out: N-1 ReduceScatter steps then
 *                N-1 AllGather steps, one kernel launch per step ("AllReduce",
 *                compassingai.com, section 3; pwwt.cn page, section 2.2).
 *                Chunk c is folded over ranks c+1, c+2, ..., c in that order.
 *  RING_FUSED -- one kernel that reads each element from all N ranks, folds in
 *                the same ring order with the same per-hop rounding, and writes
 *                all N outputs: bitwise equal to RING_STEP, with the minimum
 *                HBM traffic (N*K read + N*K written, K = bytes per rank).
 *  TREE       -- recursive doubling ("集合通信基础AllReduce、Ring算法与NCCL全解析",
 *                xdnf.cn, section 4.1): log2 N steps, partner r XOR 2^s, whole
 *                vectors.  Pairwise fold order ((x0+x1)+(x2+x3))...  Power-of-two
 *                N only; AllReduce only.
 *  HALVING_DOUBLING -- the same page's "Recursive Doubling / Halving" read as the
 *                bandwidth-optimal variant: recursive-halving ReduceScatter
 *                (partners at distance N/2, N/4, ..., 1; rank r ends with chunk
 *                r) then recursive-doubling AllGather; 2 log2 N steps, (N-1)/N*K
 *                sent per rank per phase like the ring.  Fold order
 *                ((x0+x4)+(x2+x6))+((x1+x5)+(x3+x7)) for N = 8.  Power-of-two N
 *                only; AllReduce, ReduceScatter and AllGather.
 *  DOUBLE_TREE -- two complementary binary trees, each reducing half of the
 *                vector from the leaves to its root and broadcasting it back
 *                ("AllReduce", compassingai.com, section 3).  In-order shape:
 *                position 0 is the root with the single child N/2; position v
 *                with lowest set bit b > 1 has children v - b/2 and v + b/2.
 *                Tree 0 places rank v at position v and carries elements
 *                [0, ceil(count/2)); tree 1 places rank (v-1) mod N at position
 *                v and carries the rest.  A node folds (left + own) + right;
 *                the root folds own + child.  2 log2 N steps; power-of-two N;
 *                AllReduce only.
 *  TREE_FUSED -- the TREE result (same bits) in one pass: every element is read
 *                once from each rank, folded as the pairwise tree of recursive
 *                doubling in registers, and written to all N ranks (the
 *                minimum N*K read + N*K written, like RING_FUSED).
 *                Power-of-two N; AllReduce only.
 *  HALVING_DOUBLING_FUSED -- the HALVING_DOUBLING result (same bits) in one
 *                pass: the pairwise tree over ranks in bit-reversed order
 *                (partners at distance N/2 first).  Power-of-two N;
 *                AllReduce, ReduceScatter (owner chunk written) and AllGather
 *                (a copy, as for every algorithm).
 *  DOUBLE_TREE_FUSED -- the DOUBLE_TREE result (same bits) in one pass: the
 *                two trees run side by side, every element of each half read
 *                once from each rank, folded in its tree's in-order order in
 *                registers, and written to all N ranks (N*K read + N*K
 *                written).  Power-of-two N; AllReduce only.
 *  AUTO       -- pick the algorithm with the smallest predicted time under the
 *                latency/bandwidth model of ar_predict_us (the pages' size-based
 *                choice between ring and tree: "AllReduce", compassingai.com,
 *                sections 4-5; xdnf.cn page, section 4.3).  On one GPU a
 *                one-pass form needs one launch and the fewest bytes; the model
 *                gives every one-pass form the same time, ties go to
 *                RING_FUSED, so AUTO picks RING_FUSED at every size measured. */
typedef enum ar_algo AR_ENUM_INT {
    AR_ALGO_RING_STEP = 0,
    AR_ALGO_RING_FUSED = 1,
    AR_ALGO_TREE = 2,
    AR_ALGO_HALVING_DOUBLING = 3,
    AR_ALGO_AUTO = 4,
    AR_ALGO_DOUBLE_TREE = 5,
    AR_ALGO_TREE_FUSED = 6,
    AR_ALGO_HALVING_DOUBLING_FUSED = 7,
    AR_ALGO_DOUBLE_TREE_FUSED = 8
} ar_algo;

/* Create a context bound to HIP device `device` and stream `stream`
 * (a hipStream_t; NULL = the device's null stream).  *out receives the
 * context, owned by the library until ar_destroy.  Errors: out == NULL or a
 * bad device -> AR_ERR_INVALID_ARG; allocation failure -> AR_ERR_NO_MEMORY. */
ar_status ar_create(ar_ctx** out, int device, void* stream);

/* Rebind the context to another stream (hipStream_t, NULL = null stream) of
 * the same device.  Subsequent calls enqueue there. */
ar_status ar_set_stream(ar_ctx* ctx, void* stream);

/* Graph replay of the multi-launch algorithms (RING_STEP, TREE,
 * HALVING_DOUBLING, DOUBLE_TREE), for ar_allreduce, ar_reduce_scatter and
 * ar_allgather.  Each of their steps is a dependent kernel launch, the
 * one-GPU counterpart of the per-message latency alpha in the pages' cost
 * model ("AllReduce", compassingai.com, section 4); replaying the recorded
 * sequence as one graph cuts that per-step cost where it dominates, i.e. for
 * small messages.
 * max_bytes_per_rank > 0: a collective of at most that many bytes per rank
 * (count * element size) is replayed: its first call on a given pointer set
 * and shape (collective, algo, dtype, op, nranks, count) records the kernel
 * sequence into a HIP graph on a private stream the library creates, and that
 * call and every later identical one launch the instantiated graph on the
 * context's stream.  Larger collectives launch directly.  The same kernels
 * run in the same order, so results are bitwise those of direct launches.
 * Up to 64 graphs are kept per context; the least recently used is released
 * (after its last replay has finished) to make room.  While the context's
 * stream is itself being captured by the caller, kernels are launched
 * directly so they land in the caller's graph.
 * max_bytes_per_rank == 0 (the default) launches everything directly and
 * releases every recorded graph, waiting for its last replay.  On MI355X,
 * replay halves a 64-rank per-step ring at 4 KiB per rank and is a few
 * percent slower than direct launches from about 16 MiB per rank, hence
 * AR_GRAPHS_MAX_BYTES_DEFAULT.  RING_FUSED and the single-step calls are one
 * launch and are not affected.  Errors: ctx == NULL -> AR_ERR_INVALID_ARG; a
 * failed capture or instantiation makes the collective call return
 * AR_ERR_RUNTIME. */
#define AR_GRAPHS_MAX_BYTES_DEFAULT ((size_t)8 << 20)
ar_status ar_set_graphs(ar_ctx* ctx, size_t max_bytes_per_rank);

/* Pointer-set cache (off by default).  enable != 0: the device-memory check
 * of bufs is remembered for the 32 most recent pointer sets and skipped when
 * the same set comes back with at most the byte size it was checked for --
 * for callers that reduce the same buckets every step and can guarantee that
 * a buffer is never freed and re-allocated smaller at the same address while
 * it is in use (that case would not be re-checked).  enable == 0 clears the
 * cache and checks every call.  Errors: ctx == NULL -> AR_ERR_INVALID_ARG. */
ar_status ar_set_pointer_cache(ar_ctx* ctx, int enable);

/* Residency caps of the one-pass kernels (on by default).  Large one-pass
 * AllReduce / ReduceScatter calls (more than 128 MiB over all ranks, from 8
 * ranks up; DEEP shapes above 256 MiB) and AllGather calls (from 8 ranks up,
 * more than 128 MiB at 8 ranks and 512 MiB beyond) launch with dynamic LDS
 * that no kernel touches, so that only 3-14 of their one-wave blocks fit on
 * a compute unit at once: fewer, smaller memory requests per CU stream HBM
 * faster (on MI355X, 8 x 25 MiB fp32 AllReduce: 70 us capped, 75 us
 * uncapped).  While such a call
 * runs it holds most of each CU's LDS; a caller that overlaps it with kernels
 * needing LDS (GEMMs on another stream) can turn the caps off (enable == 0):
 * the same calls then run the uncapped shapes and reserve no LDS.  Results
 * are bitwise the same either way.  ar_stream follows the setting.  The
 * reservations are sized for the 160 KiB of LDS per compute unit of gfx950;
 * on a device that reports another size the caps start off.  Errors: ctx ==
 * NULL -> AR_ERR_INVALID_ARG; enable != 0 on such a device ->
 * AR_ERR_UNSUPPORTED (the caps stay off). */
ar_status ar_set_residency_caps(ar_ctx* ctx, int enable);

/* Residency probe, a diagnostic of the mechanism behind the caps: launches
 * `blocks` one-wave blocks, each reserving `lds_bytes` of dynamic LDS and
 * staying resident for a bounded time (about 0.7 ms), and reports the most
 * blocks found resident at once on a compute unit -- the largest (*max_per_cu)
 * and the smallest (*min_per_cu) of those per-CU maxima -- and how many
 * compute units ran a block (*cus).  With lds_bytes the reservation of a cap
 * W, every CU should hold exactly W.  Synchronous on the context's stream;
 * allocates and frees 32 KiB of device memory.  Errors: NULL ctx or output,
 * blocks == 0 or above 1 << 20, lds_bytes above 64 KiB ->
 * AR_ERR_INVALID_ARG; AR_ERR_NO_MEMORY / AR_ERR_RUNTIME from the runtime. */
ar_status ar_residency_probe(ar_ctx* ctx, unsigned lds_bytes, unsigned blocks,
                             unsigned* max_per_cu, unsigned* min_per_cu, unsigned* cus);

/* AllReduce in place: every bufs[r][0:count) ends with the reduction of all
 * ranks' inputs.  RING_STEP and RING_FUSED give identical bits; TREE and
 * HALVING_DOUBLING give their tree-order results. */
ar_status ar_allreduce(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                       ar_dtype dtype, ar_op op, ar_algo algo);

/* ReduceScatter in place ("AllReduce 集合通信", zzmblog.top, section 语义: each
 * process ends with one shard of the reduction).  On return bufs[r] holds the
 * finished chunk r at its natural offset (ar_chunk_range(count, nranks, r));
 * the other chunks of bufs[r] are unspecified.  RING_STEP, RING_FUSED or
 * HALVING_DOUBLING. */
ar_status ar_reduce_scatter(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                            ar_dtype dtype, ar_op op, ar_algo algo);

/* AllGather in place ("AllReduce 集合通信", zzmblog.top, section 语义: every
 * process ends with every process's shard, assembled in rank order; the ring
 * runs it as N-1 forwarding steps without accumulation, section 两阶段流程):
 * chunk r of bufs[r] is copied, bit for bit, into chunk r of every other
 * buffer.  ar_reduce_scatter then ar_allgather with the same
 * algo equals ar_allreduce bitwise.  RING_STEP, RING_FUSED or
 * HALVING_DOUBLING. */
ar_status ar_allgather(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                       ar_dtype dtype, ar_algo algo);

/* One ReduceScatter step k (0 <= k <= nranks-2) of the ring: for every rank r,
 * chunk c = (r-k-1) mod N of bufs[r] is folded into chunk c of bufs[(r+1)%N].
 * With AR_AVG the last step (k = N-2) also divides the finished chunk by N.
 * Calling k = 0..N-2 in order equals ar_reduce_scatter(RING_STEP). */
ar_status ar_ring_rs_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                          ar_dtype dtype, ar_op op, int step);

/* One AllGather step k (0 <= k <= nranks-2): for every rank r, chunk
 * c = (r-k) mod N of bufs[r] is copied into chunk c of bufs[(r+1)%N]. */
ar_status ar_ring_ag_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                          ar_dtype dtype, int step);

/* One recursive-doubling step s (0 <= s < log2 N): every pair (r, r XOR 2^s)
 * replaces both vectors by their elementwise combination; with AR_AVG the
 * last step divides by N.  Power-of-two nranks only. */
ar_status ar_tree_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                       ar_dtype dtype, ar_op op, int step);

/* One recursive-halving ReduceScatter step s (0 <= s < log2 N): with
 * d = N >> (s+1), every rank r folds partner (r XOR d)'s copy of the d chunks
 * starting at (r & ~(d-1)) into its own; with AR_AVG the last step divides
 * the finished chunk r by N.  Power-of-two nranks only.  Calling s = 0..log2N-1
 * in order equals ar_reduce_scatter(HALVING_DOUBLING). */
ar_status ar_hd_rs_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                        ar_dtype dtype, ar_op op, int step);

/* One recursive-doubling AllGather step t (0 <= t < log2 N): with d = 2^t,
 * every rank r copies the d finished chunks of partner (r XOR d), i.e. chunks
 * ((r XOR d) & ~(d-1)) ... + d-1.  Power-of-two nranks only. */
ar_status ar_hd_ag_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                        ar_dtype dtype, int step);

/* One double-binary-tree step s (0 <= s < 2 log2 N), both trees at once:
 * s < L-1 reduces tree level s+1, s = L-1 folds the roots (AVG divides
 * there), s = L copies each root to position N/2, s > L broadcasts level
 * 2L-s to its children (L = log2 N).  Power-of-two nranks only.  Calling
 * s = 0..2L-1 in order equals ar_allreduce(DOUBLE_TREE). */
ar_status ar_dtree_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                        ar_dtype dtype, ar_op op, int step);

/* Chunk c's element range (host-only; touches no GPU).  The ring splits each
 * rank's data into N chunks ("AllReduce", compassingai.com, section 3 技术原理;
 * pwwt.cn page, section 2.2) and says nothing of counts that N does not
 * divide; the reading here is a ceiling split: L = ceil(count / N), chunk c =
 * [min(c*L, count), min((c+1)*L, count)), so trailing chunks are short or
 * empty.  Exact for every count up to SIZE_MAX.  Errors: nranks out of range,
 * chunk outside [0, nranks), NULL outputs -> AR_ERR_INVALID_ARG. */
ar_status ar_chunk_range(size_t count, int nranks, int chunk, size_t* offset, size_t* len);

/* Predicted time in microseconds of one ar_allreduce with `algo` (not AUTO),
 * from the alpha-beta model T = t_call + launches * alpha + bytes / BW(algo):
 * the pages' T_ring ~ 2(N-1) alpha + ... D beta and T_tree ~ 2 log2 N alpha +
 * ... ("AllReduce", compassingai.com, section 4) with one-GPU launches and HBM
 * bytes in place of link messages.  Constants were fitted on MI355X over the
 * 64-rank message-size sweep (host-only; touches no GPU).  Errors: bad
 * algo / nranks / dtype, NULL us, TREE or HALVING_DOUBLING with a
 * non-power-of-two nranks -> AR_ERR_INVALID_ARG / AR_ERR_UNSUPPORTED. */
ar_status ar_predict_us(ar_algo algo, int nranks, size_t count, ar_dtype dtype, double* us);

/* The algorithm AR_ALGO_AUTO resolves to for an AllReduce of this shape
 * (host-only). */
ar_status ar_auto_algo(int nranks, size_t count, ar_dtype dtype, ar_algo* out);

/* Plain device-to-device copy of `bytes` bytes (16-byte aligned pointers and
 * size), used to calibrate bandwidth and hardware byte counters against a
 * kernel of known traffic.  Enqueued on the context's stream. */
ar_status ar_copy(ar_ctx* ctx, void* dst, const void* src, size_t bytes);

/* Calibration stream with the fused AllReduce kernel's memory pattern and no
 * reduction: reads `bytes` bytes from each of the nsrc buffers src[0..nsrc)
 * and writes their bitwise XOR (zeros when nsrc == 0) to each of the ndst
 * buffers dst[0..ndst), with the fused kernel's tiling (one 64-lane wave per
 * block, 8 sources of loads in flight, streaming loads and stores; 4 KiB of
 * every buffer per block, or -- from 8 sources holding more than 128 MiB in
 * all, like the fused AllReduce -- 1 KiB per block with the same cap on the
 * blocks resident per compute unit).  nsrc = ndst = N is the ceiling of an N-rank
 * fused AllReduce's N*K-read / N*K-written pattern on this hardware; other
 * mixes separate the cost of read streams from that of write streams.
 * src and dst are HOST arrays of DEVICE pointers (read during the call),
 * every buffer 16-byte aligned, device memory of the context's device, no two
 * overlapping, except that dst[i] may equal src[i] (in place, as an
 * AllReduce works); bytes a multiple of 16; nsrc and ndst at most
 * AR_MAX_RANKS each, not both 0, and at most AR_MAX_RANKS distinct buffers.
 * Enqueued on the context's stream.  Errors: AR_ERR_INVALID_ARG for any of
 * the above, AR_ERR_RUNTIME if the launch fails. */
ar_status ar_stream(ar_ctx* ctx, const void* const* src, int nsrc, void* const* dst, int ndst,
                    size_t bytes);

/* Timeline of the calibration stream, a diagnostic of where a one-pass
 * kernel's time goes: the in-place N-read / N-write XOR stream of ar_stream
 * over bufs[0..nbufs) (each buffer read, then overwritten with the XOR of all
 * of them) in the paced shape: one 64-lane block per 1 KiB tile of every
 * buffer, one 16-byte unit per lane, launched with lds_bytes of dynamic LDS
 * per block (0: none) to cap the blocks resident per compute unit.  Block b
 * writes the device's constant-rate wall clock at its start to ts[2b] and,
 * once all of its loads and stores have completed, to ts[2b + 1]; from them a
 * caller reads the ramp, the steady rate and the drain of the launch.
 * bufs is a HOST array of DEVICE pointers, 16-byte aligned, device memory of
 * the context's device, not overlapping; bytes > 0, a multiple of 16; ts is
 * DEVICE memory of that device, 8-byte aligned, holding ts_len >= 2 *
 * ceil(bytes / 1024) entries, overlapping no buffer.  *blocks (if not NULL)
 * receives ceil(bytes / 1024), *clock_khz (if not NULL) the clock's rate in
 * kHz.  Enqueued on the context's stream.  Errors: AR_ERR_INVALID_ARG for any
 * of the above or lds_bytes above 64 KiB; AR_ERR_RUNTIME if the launch
 * fails. */
ar_status ar_stream_timeline(ar_ctx* ctx, void* const* bufs, int nbufs, size_t bytes,
                             unsigned lds_bytes, unsigned long long* ts, size_t ts_len,
                             size_t* blocks, unsigned* clock_khz);

/* On-device check of an AllReduce result, a test utility: the whole array is
 * checked where it lies, without copying it to the host.  An AllReduce leaves
 * every participant with the same data ("AllReduce", compassingai.com,
 * section 3 技术原理), and a floating-point SUM is judged against the exact
 * sum through an error bound.
 *  mismatched      positions i in [0, count) where some bufs[r][i] differs bit
 *                  for bit from bufs[0][i]
 *  first_mismatch  the smallest such i (count if there is none)
 *  over_bound      with ref: positions where |bufs[0][i] - ref[i]| (binary64,
 *                  the element widened exactly) exceeds bound[i] (bound given)
 *                  or is NaN
 *  max_abs_err     with ref: the largest |bufs[0][i] - ref[i]|; NaN if any
 *                  difference is NaN; 0 without ref
 * ref and bound: NULL, or DEVICE arrays of `count` binary64 values (bound
 * needs ref).  result: a DEVICE pointer to one ar_check_result (8-byte
 * aligned), written asynchronously on the context's stream: synchronise
 * before reading it.  bufs: as for ar_allreduce (they are only read).  The
 * per-block partial records live in a scratch array of 2048 records that the
 * context allocates on its first ar_check and frees in ar_destroy.  Errors:
 * AR_ERR_INVALID_ARG for bad buffers, a NULL or misplaced result, bound
 * without ref, or ref/bound not holding count doubles of device memory;
 * AR_ERR_NO_MEMORY if the scratch array cannot be allocated; AR_ERR_RUNTIME
 * if a launch fails. */
typedef struct ar_check_result {
    unsigned long long mismatched;
    unsigned long long first_mismatch;
    unsigned long long over_bound;
    double max_abs_err;
} ar_check_result;

ar_status ar_check(ar_ctx* ctx, void* const* bufs, int nranks, size_t count, ar_dtype dtype,
                   const double* ref, const double* bound, ar_check_result* result);

/* ar_check for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, validation and results as ar_check, and the same kernels; the
 * partial records live in a device-resident array of AR_CHECK_MAX_RECORDS
 * records (80 KiB) that each GPU the library runs on holds until the process
 * ends, located once per device by ar_create.  The call allocates nothing
 * (no hipMalloc, no hipFree) and launches two kernels.  Every count fits: the
 * first pass never uses more than AR_CHECK_MAX_RECORDS blocks, each writing
 * the one record the second pass reads, so no state carries over between
 * calls.  All calls on one GPU share that array: calls that overlap on one
 * GPU (several streams or contexts at once) race and give wrong results, so
 * run them one after another.  Errors: as ar_check, and AR_ERR_RUNTIME if
 * the array could not be located on this device when the context was made. */
#define AR_CHECK_MAX_RECORDS 2048
ar_status ar_check_noalloc(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                           ar_dtype dtype, const double* ref, const double* bound,
                           ar_check_result* result);

/* Static description of a status code (never NULL). */
const char* ar_status_string(ar_status s);

/* Detail of the last failure on ctx (empty string if none; never NULL).
 * ar_last_error(NULL) describes the last ar_create failure of this thread. */
const char* ar_last_error(const ar_ctx* ctx);

/* Destroy a context.  ar_destroy(NULL) is a no-op returning AR_OK.  Work
 * already enqueued is not waited for, except that a context which ran
 * ar_check first waits for its stream, then frees the checker's scratch. */
ar_status ar_destroy(ar_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* RING_ALLREDUCE_AR_H */
