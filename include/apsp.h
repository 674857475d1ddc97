/*
 * apsp.h -- C ABI of the gfx950 (MI355X) blocked Floyd-Warshall library.
 *
 * The library computes all-pairs shortest-path distances of a weighted
 * digraph held as a dense row-major distance matrix in device memory, by the
 * blocked Floyd-Warshall method of the page "Katz and Kider" (thesis section
 * 4.6 and its Algorithms 16-18): the matrix is cut into square pivot blocks;
 * round K closes the diagonal block (K,K) (Phase 1), then updates the blocks
 * in pivot row K and pivot column K (Phase 2), then every remaining block
 * (Phase 3), and the pivot moves one block down the diagonal.  Next to it:
 * many small graphs at once (apsp_fw_batched_*) and Johnson's algorithm for
 * sparse graphs with negative weights (apsp_johnson_*), whose own contracts
 * are stated at their declarations.
 *
 * Only plain C types cross this boundary.  `stream` is a hipStream_t passed
 * as an opaque pointer (NULL = the null stream).
 *
 * Matrix contract (all entry points):
 *   d      device pointer to element (0,0); element (i,j) is d[i*ld + j].
 *          Must be 4-byte aligned.  When d is 16-byte aligned and ld is a
 *          multiple of 4, 128-bit loads and stores are used.
 *   n      number of vertices, n >= 0 (n = 0 is a no-op).
 *   ld     leading dimension in elements, ld >= max(n, 1).
 *   inf    the "no edge / no path" sentinel.
 * Input preconditions (not checked; results are undefined otherwise):
 *   d[i][i] = 0; 0 <= d[i][j] <= inf; no NaN; every true shortest distance
 *   between connected vertices is < inf.
 * Output: on completion of the enqueued work, d[i][j] (i, j < n) holds the
 * shortest-path distance from i to j, and exactly `inf` when j is not
 * reachable from i.  Elements outside the leading n x n block are never read
 * or written.  int32 results are exact; float32 results are within a few
 * units in the last place per path edge of the exact real-number distances,
 * and bit-identical from run to run.
 *
 * Ownership and concurrency: the caller owns d.  An int32 call takes 256
 * bytes of stream-ordered scratch (hipMallocAsync / hipFreeAsync on
 * `stream`); float32 calls allocate nothing.  Beyond that the library keeps
 * only a per-device "is gfx950" cache, so calls on different streams with
 * different matrices may run concurrently.  Work is enqueued asynchronously
 * on `stream`; the caller synchronises.
 *
 * Arithmetic of int32 calls: when every finite entry is an integer in
 * [0, 2^24] and either no off-diagonal entry equals inf or (n - 1) times the
 * largest finite entry is at most 2^24, every value the recurrence stores is
 * an integer of at most 2^24, so the kernels compute in binary32, which is
 * exact there and twice as fast on gfx950; the first round's loads convert
 * the entries to binary32 and the last round's stores (and a short pass over
 * its pivot row and column) convert them back, in place within the call.  Otherwise they compute in int32.  A scan kernel
 * makes this choice on the device (no host synchronisation), and the
 * results are identical either way (see apsp_set_int32_arith).
 *
 * Errors: argument errors return APSP_ERR_INVALID_VALUE before any HIP call
 * (nothing is enqueued, d is untouched).  A current device that is not
 * gfx950 returns APSP_ERR_NO_DEVICE.  A failed launch returns APSP_ERR_LAUNCH
 * (d is then undefined) and apsp_last_hip_error() gives the hipError_t value
 * for the calling thread.  Nothing is printed; nothing aborts.
 */
#ifndef APSP_H
#define APSP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  APSP_OK = 0,
  APSP_ERR_INVALID_VALUE = 1,
  APSP_ERR_NO_DEVICE = 2,
  APSP_ERR_LAUNCH = 3,
  APSP_ERR_NEGATIVE_CYCLE = 4,  /* the graph has a cycle of negative weight */
  APSP_ERR_RANGE = 5            /* a value the call must represent is out of range */
};

/*
 * All-pairs shortest paths on an int32 matrix, in place (all rounds).
 * Arithmetic: plain int32 add and signed min.  inf must satisfy
 * 1 <= inf <= 0x3FFFFFFF so that inf + inf cannot overflow.
 * Defines: "Katz and Kider" page, section 4.6 (three phases per round).
 */
int apsp_fw_i32(int32_t *d, int64_t n, int64_t ld, int32_t inf, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, results and arguments as apsp_fw_i32, with no allocation of
 * any kind.  The int32 call's scan result (8 bytes) lives in a static
 * 256-byte device array of the library instead of stream-ordered scratch;
 * the need is 8 bytes whatever n, so no input is too large for it.  Each
 * GPU holds one copy of that array from the first call on it until the
 * process ends, and every call on that GPU shares it: each call clears it
 * (with a kernel) before use, and calls that overlap in time on one GPU
 * (different streams, or other host threads) race on it and must be
 * serialised by the caller.  The first call on a device looks up the
 * array's device address (hipGetSymbolAddress); a failure there returns
 * APSP_ERR_LAUNCH.  Other errors as for apsp_fw_i32.
 */
int apsp_fw_i32_noalloc(int32_t *d, int64_t n, int64_t ld, int32_t inf, void *stream);

/*
 * All-pairs shortest paths on a float32 matrix, in place (all rounds).
 * Arithmetic: IEEE binary32 add (round to nearest even) and min.
 * inf must be > 0 and not NaN; +infinity is allowed.
 * Defines: "Katz and Kider" page, section 4.6 (three phases per round).
 */
int apsp_fw_f32(float *d, int64_t n, int64_t ld, float inf, void *stream);

/*
 * All-pairs shortest paths of a dense matrix whose weights may be negative
 * (the setting of the page "Johnson's APSP in Glushkov algorithmic
 * algebras", where a path through "no edge" must never count): in place, the
 * same blocked rounds ("Katz and Kider" page, section 4.6), no sum ever
 * passes through the sentinel.
 * Input: d[i][i] = 0; off-diagonal entries are weights in (-inf, inf) or
 * exactly inf ("no edge").  int32: 1 <= inf <= 0x3FFFFFFF.  float32: inf > 0
 * or +infinity; weights finite.
 * int32 arithmetic (W = the largest |weight|): binary32 with "no edge" as
 * +infinity when (n - 1) * W <= 2^24 (exact, as for apsp_fw_i32; subject to
 * the arithmetic policy below); else int32 with the sentinel as a large
 * number, exact when (2n - 3) * W < inf (or (n - 1) * W < 2^30 when no entry
 * is inf), followed by a pass that restores inf on unreachable pairs.
 * Otherwise APSP_ERR_RANGE before anything is written.  float32: the
 * sentinel becomes +infinity for the rounds and comes back as inf; results
 * as for apsp_fw_f32.
 * Returns APSP_ERR_INVALID_VALUE (nothing written) for a non-zero diagonal
 * entry or an int32 entry outside (-inf, inf] (checked on the device), and
 * APSP_ERR_NEGATIVE_CYCLE when some d[i][i] < 0 after the rounds (a negative
 * cycle through i); d then holds the unspecified partial results.
 * Synchronous: returns after the work on `stream` has completed.  Takes 16
 * bytes of stream-ordered scratch.  Other errors as for apsp_fw_i32.
 */
int apsp_fw_signed_i32(int32_t *d, int64_t n, int64_t ld, int32_t inf, void *stream);
int apsp_fw_signed_f32(float *d, int64_t n, int64_t ld, float inf, void *stream);

/*
 * Rounds [round_begin, round_end) only, in place, with pivot blocks of
 * apsp_pivot_block(n) vertices; round r uses pivots [r*B, min((r+1)*B, n)).
 * After rounds [0, r) the matrix holds the shortest distances over paths
 * whose intermediate vertices all lie in [0, r*B) -- the state of the
 * Floyd-Warshall recurrence after its first r*B pivots -- so a run can stop
 * and later resume from that state.  Calling [0, R) and then [R, rounds)
 * equals one full call.  Requires 0 <= round_begin <= round_end <=
 * ceil(n / B).  Defines: "Katz and Kider" page, section 4.6 (the primary
 * block moves one block down the diagonal per round).
 */
int apsp_fw_rounds_i32(int32_t *d, int64_t n, int64_t ld, int32_t inf,
                       int64_t round_begin, int64_t round_end, void *stream);
int apsp_fw_rounds_f32(float *d, int64_t n, int64_t ld, float inf,
                       int64_t round_begin, int64_t round_end, void *stream);

/*
 * Measurement variant of apsp_fw_i32 / apsp_fw_f32: the same kernels on
 * the same stream, with HIP events recorded around each launch (or group
 * of launches).  It synchronises the stream before returning and writes:
 *   phase_ms[p]     summed event time of the launches of kind p, in ms;
 *   phase_launch[p] number of timed launches (or groups) of kind p;
 *   *arith          1 if the call computed in binary32, 0 if in int32;
 * kinds (arrays of 4): 0 = standalone Phase 1 (first round only),
 * 1 = Phase 2, 2 = Phase 3 (which also carries the next round's Phase 1),
 * 3 = the int32 scan before the rounds and, when the call computed in
 * binary32 over more than one block, the conversion of the last round's
 * pivot row and column back to int32 after them (the other conversions ride
 * in the first round's loads and the last round's Phase-3 stores).  Any
 * pointer may be NULL.  Errors as for apsp_fw_i32.
 */
int apsp_fw_timed_i32(int32_t *d, int64_t n, int64_t ld, int32_t inf, void *stream,
                      double *phase_ms, int64_t *phase_launch, int *arith);
int apsp_fw_timed_f32(float *d, int64_t n, int64_t ld, float inf, void *stream,
                      double *phase_ms, int64_t *phase_launch, int *arith);

/*
 * Min-plus matrix product C <- min(C, A (x) B), (A (x) B)[i][j] = min over t
 * of A[i][t] + B[t][j]: the update inside Phases 2 and 3 of the "Katz and
 * Kider" page (thesis section 4.6, Algorithms 17 and 18), for operands in
 * separate device buffers and of any depth k.
 *   C  m x n, element (i, j) at C[i*ldc + j], ldc >= n;
 *   A  m x k, at A[i*lda + t], lda >= k;   B  k x n, at B[t*ldb + j], ldb >= n.
 * Device pointers, 4-byte aligned (128-bit access when all three are 16-byte
 * aligned and every leading dimension is a multiple of 4).  C must not
 * overlap A or B.  m, n or k = 0 is a no-op.
 * int32 entries lie in [0, inf] with 1 <= inf <= 0x3FFFFFFF (sums cannot
 * overflow, and inf + x never improves an entry).  float32 entries are <=
 * inf (inf > 0 or +infinity); with +infinity as "no path", finite entries
 * may be negative (+infinity plus anything finite stays +infinity).  int32 results are exact; float32 results are
 * each the minimum of single rounded sums (deterministic).  Asynchronous on
 * `stream`; allocates nothing.  Errors: APSP_ERR_INVALID_VALUE for bad
 * arguments before any HIP call, else as for apsp_fw_i32.
 */
int apsp_minplus_gemm_i32(int32_t *C, int64_t ldc, const int32_t *A, int64_t lda,
                          const int32_t *B, int64_t ldb, int64_t m, int64_t n, int64_t k,
                          int32_t inf, void *stream);
int apsp_minplus_gemm_f32(float *C, int64_t ldc, const float *A, int64_t lda, const float *B,
                          int64_t ldb, int64_t m, int64_t n, int64_t k, float inf, void *stream);

/*
 * All-pairs shortest paths of a matrix in HOST memory, for graphs larger
 * than device memory ("Katz and Kider" page, section 4.6.1: the in-core
 * method needs the whole graph in global memory).  The blocked rounds run on
 * outer blocks of S pivots (S a multiple of 128): the S x S diagonal block is
 * closed on the device by the in-core rounds, the S-wide pivot-row and
 * pivot-column panels are updated and held in device memory, and every other
 * S x S super-tile streams to the device, takes its min-plus product of
 * depth S, and streams back.  The panels go back to the host while the
 * super-tiles are computed.
 *   h, n, ld, inf   the matrix, in place in host memory, with the contract
 *                   of apsp_fw_i32 / apsp_fw_f32 (element (i,j) at h[i*ld+j]).
 *                   Allocate it pinned (hipHostMalloc) for copies that
 *                   overlap the products; pageable memory works, slower.
 *   device_bytes    device memory the call may use (0: half of the free
 *                   memory).  How it is used is apsp_fw_host_plan's answer:
 *                   a matrix that fits is copied in whole and computed
 *                   in-core; else S and one or two panel sets are chosen to
 *                   fit (about 4 (2 S n + 4 S^2) bytes with one set,
 *                   4 (4 S n + 4 S^2) with two).  A budget too small for
 *                   S = 128 returns APSP_ERR_RANGE with the matrix untouched.
 *   outer_block     optional output (may be NULL): the S used (n rounded up
 *                   to 128 when in-core).
 * int32 matrices compute in binary32 when that is exact, as for apsp_fw_i32
 * (the arithmetic policy applies), decided by a device scan streamed over
 * the matrix first.  Results equal apsp_fw_i32 / apsp_fw_f32 on the same
 * matrix (int32 exactly).  Synchronous: returns after all work, on `stream`
 * and on three internal streams of default priority, has completed.
 * Errors as for apsp_fw_i32.
 */
int apsp_fw_host_i32(int32_t *h, int64_t n, int64_t ld, int32_t inf, int64_t device_bytes,
                     void *stream, int64_t *outer_block);
int apsp_fw_host_f32(float *h, int64_t n, int64_t ld, float inf, int64_t device_bytes,
                     void *stream, int64_t *outer_block);

/*
 * How apsp_fw_host_* would run an n x n matrix of elem_bytes-byte elements
 * (4: int32 or float) in device_bytes of device memory, without running it:
 *   *panel_sets = 0   the matrix fits: in-core (outer_block = n rounded up
 *                     to 128);
 *               = 1   outer block S, one panel set, reloaded every round;
 *               = 2   outer block S, two panel sets: the next round's panels
 *                     are computed in place, never reloaded.
 * S is the largest multiple of 128 that fits, then lowered to the smallest
 * multiple of 128 with the same number of rounds.  Two sets are taken when
 * they fit at S >= min(S with one set, 4096).  Host logic only: with
 * device_bytes > 0 it makes no HIP call; 0 asks the device for half of its
 * free memory.  Returns APSP_ERR_RANGE when S = 128 does not fit,
 * APSP_ERR_INVALID_VALUE for bad arguments; outputs may be NULL.
 */
int apsp_fw_host_plan(int64_t n, int64_t elem_bytes, int64_t device_bytes, int64_t *outer_block,
                      int32_t *panel_sets);

/*
 * Path reconstruction: the successor (first-hop) matrix.  For i != j,
 * nxt[i][j] = the smallest u != i minimising w[i][u] + d[u][j] (a first hop
 * of a shortest path i -> j, by Bellman's equation d(i,j) = min over u != i
 * of w(i,u) + d(u,j)); nxt[i][i] = i; -1 where no candidate is below inf (j
 * unreachable).  It is the page "Johnson's APSP in Glushkov algorithmic
 * algebras" relaxation RelaxEdge(i, u, j) taken once more over the final
 * distances, keeping the argument of the minimum, so it does not depend on
 * the order in which the distances were found.
 *   w, ldw   device, the n x n weights (as given to apsp_fw_*: w[i][i] = 0,
 *            inf for "no edge"; int32 entries in [0, inf]);
 *   d, ldd   device, the n x n shortest distances of w (e.g. apsp_fw_*'s
 *            output);
 *   nxt, ldn device int32 output, n x n, ldn >= n.
 * Pointers 4-byte aligned (128-bit loads when w and d are 16-byte aligned and
 * ldw, ldd are multiples of 4).
 * Precondition for walkable successors: no cycle of total weight 0 (with
 * weights >= 0, a cycle of 0-weight edges).  Then following nxt from i
 * reaches j within n - 1 hops along a path whose weights sum to d[i][j]:
 * each hop keeps d(., j) + the weight walked constant and d(., j) never
 * increases, so a vertex seen twice would close a 0-weight cycle.  With
 * such a cycle the matrix is still the one defined above (ties go to the
 * smallest u), but two vertices of the cycle can name each other as first
 * hop towards the same j, and apsp_path then returns -3 for the pairs whose
 * walk enters that loop.
 * Work: n^3 candidates when w has more than n^2/16 finite off-diagonal
 * entries; else only the neighbours of each i are tried (n candidates per
 * edge).  For n^3 candidates in int32, when every finite weight and distance
 * is >= 0 and the largest finite weight plus the largest finite distance is
 * below inf and 2^(31 - ceil(log2 n)), each candidate is one 32-bit key
 * (w + d) << ceil(log2 n) | u and the argmin is a minimum of keys.  The same
 * matrix in every case.  Asynchronous on `stream` (the choices are made on
 * the device); uses 24 * (1 + min(n, 1024)) bytes of stream-ordered
 * scratch.  Errors as for apsp_fw_i32.
 */
int apsp_successors_i32(const int32_t *w, int64_t ldw, const int32_t *d, int64_t ldd,
                        int32_t *nxt, int64_t ldn, int64_t n, int32_t inf, void *stream);
int apsp_successors_f32(const float *w, int64_t ldw, const float *d, int64_t ldd, int32_t *nxt,
                        int64_t ldn, int64_t n, float inf, void *stream);

/*
 * Distances and successors in one call: d in place (the apsp_fw_* result)
 * and nxt (the apsp_successors_* matrix of the weights d held on entry).
 * Same preconditions as those two (w[i][i] = 0, int32 entries in [0, inf]).
 *
 * int32, one-pass form: when the weights are dense (more than n^2/16 finite
 * off-diagonal entries), none is negative, the diagonal is zero, and every
 * value the rounds can store stays below 2^(30-s) - 1 with s the bit width
 * of n (2^(s-1) <= n < 2^s) -- the largest weight when no off-diagonal
 * entry is inf, else n - 1 times it -- the rounds run once, in int32
 * arithmetic, on keys v << s | h: the weight or distance v and the first
 * hop h (the diagonal carries h = 2^s - 1, "no edge" is 2^30 - 2^s).  A
 * pivot-row operand enters each sum with its low s bits cleared, so
 * (a << s | h) + (b << s) is the walk i -> k -> j with the first hop of its
 * i -> k part, and the minimum of keys picks the shortest distance and,
 * among shortest paths, the smallest first hop: the same nxt as
 * apsp_successors_*, with no n^3 successor pass.  Defines: "Katz and
 * Kider" page, section 4.6 (the rounds); "Study of Betweenness Centrality
 * Algorithms in GPU" (predecessor arrays).  Deciding reads 24 bytes of
 * statistics back, so int32 calls synchronise `stream` once (on a stream
 * under graph capture the call does not, and takes the form below).
 *
 * Otherwise (and always for float32): apsp_fw_* in place on d, then
 * apsp_successors_* from a copy of the weights kept in n*n elements of
 * stream-ordered scratch, asynchronously on `stream`.
 */
int apsp_fw_paths_i32(int32_t *d, int64_t ld, int32_t *nxt, int64_t ldn, int64_t n, int32_t inf,
                      void *stream);
int apsp_fw_paths_f32(float *d, int64_t ld, int32_t *nxt, int64_t ldn, int64_t n, float inf,
                      void *stream);

/*
 * Diagnostic: the form the calling thread's last apsp_fw_paths_i32 call
 * took -- 1 the one-pass key form, 0 the rounds followed by the successor
 * pass, -1 no call yet or the call returned an error before choosing.
 */
int apsp_fw_paths_last_form(void);

/*
 * The path i -> j from a successor matrix in HOST memory (copy nxt back
 * first): writes the vertices i, ..., j into path[0 .. min(len, cap)) and
 * returns len, the number of vertices (1 when i = j).  Returns -1 when j is
 * unreachable from i, -2 for bad arguments, -3 when the successors do not
 * reach j within n hops (possible only when the graph has a cycle of total
 * weight 0; see apsp_successors_*).  Host code only.
 */
int64_t apsp_path(const int32_t *nxt, int64_t ldn, int64_t n, int64_t i, int64_t j,
                  int32_t *path, int64_t cap);

/*
 * Measurement across calls: after apsp_trace_begin(max_launches), every
 * apsp_fw_i32 / apsp_fw_f32 / apsp_fw_rounds_* call made by this thread
 * records HIP events around each launch (or launch group, as for
 * apsp_fw_timed_i32), on the call's stream, without synchronising.
 * apsp_trace_end synchronises on the last recorded event, ends the trace and
 * writes the summed event time and the number of launches per kind (the
 * kinds of apsp_fw_timed_i32) and the number of launches beyond max_launches
 * that were not recorded (any pointer may be NULL).  Events come from a
 * per-thread pool that lives until the process ends.  apsp_trace_begin
 * returns APSP_ERR_INVALID_VALUE for max_launches outside [1, 2^24] or when
 * a trace is already on; apsp_trace_end returns it when none is on.
 */
int apsp_trace_begin(int64_t max_launches);
int apsp_trace_end(double *phase_ms, int64_t *phase_launch, int64_t *dropped);

/*
 * Many small graphs at once: all-pairs shortest paths of `batch` independent
 * graphs of n <= 128 vertices each, in place, one workgroup per graph.
 * Defines: the page "Loops into zones", section "Many small graphs" (each
 * graph is one GPU block, graphs never interact), with the per-graph work
 * being the diagonal-block closure of the "Katz and Kider" page (thesis
 * section 4.6, Phase 1 / Algorithm 16) on the whole graph.
 *   d       device pointer; graph g's element (i, j) is d[g*stride + i*ld + j].
 *           4-byte aligned; 128-bit access when d is 16-byte aligned and ld
 *           and stride are multiples of 4.
 *   batch   number of graphs, >= 0 (0 is a no-op).
 *   n       vertices per graph, 0 <= n <= 128 (0 is a no-op).
 *   ld      leading dimension of each graph, ld >= n.
 *   stride  elements between consecutive graphs, stride >= (n-1)*ld + n (the
 *           graphs must not overlap).
 *   inf     sentinel, as for apsp_fw_i32 / apsp_fw_f32.
 * Input preconditions and output as for apsp_fw_i32 / apsp_fw_f32, per graph.
 * Arithmetic: int32 add and min (i32), IEEE binary32 add and min (f32); every
 * graph is closed pivot by pivot in order, so float32 results equal the plain
 * sequential Floyd-Warshall on that graph bit for bit.  Elements outside each
 * graph's n x n block are never read or written.  Allocates nothing; work is
 * enqueued on `stream`.  Errors: APSP_ERR_INVALID_VALUE for bad arguments
 * (including n > 128) before any HIP call; otherwise as for apsp_fw_i32.
 */
int apsp_fw_batched_i32(int32_t *d, int64_t batch, int64_t n, int64_t ld, int64_t stride,
                        int32_t inf, void *stream);
int apsp_fw_batched_f32(float *d, int64_t batch, int64_t n, int64_t ld, int64_t stride,
                        float inf, void *stream);

/*
 * Johnson's all-pairs shortest paths of a sparse digraph whose edge weights
 * may be negative, written as a dense distance matrix.
 * Defines: the page "Johnson's APSP in Glushkov algorithmic algebras" (CEUR
 * Vol-1631): extendGraph (an added vertex q with 0-weight edges to every
 * vertex), BellmanFord from q with the negative-cycle condition cnc, giving
 * the potentials h; UpdateWeights w'(u,v) = w(u,v) + h(u) - h(v) >= 0; a
 * single-source search D(i) from every vertex on w'; and to(D, i), d(i,j) =
 * D'(j) - h(i) + h(j).  The single-source searches follow the delta-stepping
 * scheme of the page "Delta-stepping SSSP on CPU and GPU" (CEUR Vol-1662,
 * Algorithm 1) with the threshold rule of the Johnson page's parallel
 * ExtractMin.
 *   row_ptr  device, n + 1 int64 offsets: the out-edges of vertex u are
 *            e in [row_ptr[u], row_ptr[u+1]); row_ptr[0] = 0, non-decreasing,
 *            row_ptr[n] = nnz.  8-byte aligned.
 *   col, w   device, nnz int32 each: edge e goes to col[e] (0 <= col[e] < n)
 *            with weight w[e], -inf < w[e] < inf.  Self loops and parallel
 *            edges are allowed (the lightest parallel edge counts; a
 *            negative self loop is a negative cycle).  May be NULL when
 *            nnz = 0.
 *   n, nnz   vertices (0 <= n < 2^31 - 1; n = 0 is a no-op) and edges
 *            (0 <= nnz < 2^31).
 *   d, ld    device output, element (i, j) at d[i*ld + j], ld >= n, 4-byte
 *            aligned; only the leading n x n block is written.  Must not
 *            overlap the graph arrays or h.
 *   inf      the "no path" sentinel written for unreachable pairs,
 *            1 <= inf <= 0x3FFFFFFF.
 *   h        optional device output (NULL or n int32): the potentials h(v),
 *            the shortest distance from the added vertex q (always <= 0;
 *            all zero when no weight is negative).
 *   delta    bucket width of the searches (>= 0), or < 0 for automatic (the
 *            mean reweighted edge weight).  0 takes one distance value per
 *            step, like Dijkstra.  The result does not depend on delta.
 * Output: d[i][j] = the shortest-path distance from i to j (exact), d[i][i]
 * = 0, and exactly inf where j is unreachable from i.
 * Preconditions checked on the device before anything is written: the CSR
 * structure and the weight range above (else APSP_ERR_INVALID_VALUE).
 * Results must be representable: every finite distance lies strictly between
 * -inf and inf (else APSP_ERR_RANGE; d is then partly written).
 * Negative cycle: returns APSP_ERR_NEGATIVE_CYCLE and leaves d untouched (h,
 * when given, is left untouched too).
 * Synchronous: the call reads device results between its steps and returns
 * after all of its work on `stream` has completed.  It takes stream-ordered
 * scratch (hipMallocAsync on `stream`) of about 14n + 8nnz bytes and frees
 * it before returning.  The tentative distances of each source live in one
 * workgroup's LDS (4n bytes plus a small queue) up to n of about 38 000 on
 * gfx950; beyond that they live in the source's own row of d in global
 * memory (slower), with a bitmap of n/8 bytes and the queue still in LDS,
 * which bounds n to about 1.2 million (else APSP_ERR_RANGE before any work).
 * Other errors as for apsp_fw_i32.
 */
int apsp_johnson_i32(const int64_t *row_ptr, const int32_t *col, const int32_t *w,
                     int64_t n, int64_t nnz, int32_t *d, int64_t ld, int32_t inf,
                     int32_t *h, int32_t delta, void *stream);

/*
 * Measurement variant of apsp_johnson_i32: the same work, with HIP events on
 * `stream` around each step.  phase_ms (4 doubles, may be NULL) receives the
 * event time of: 0 = validation, 1 = Bellman-Ford (including its host
 * checks; no rounds run when no weight is negative) and the int32
 * potentials, 2 = reweighting, 3 = the
 * single-source searches with the write-out.  counts (4 int64, may be
 * NULL) receives: 0 = Bellman-Ford rounds launched, 1 = search steps, 2 =
 * vertices removed from the marks, 3 = edge relaxations (1-3 summed over
 * all sources; every source relaxes each edge it reaches at least once).
 */
int apsp_johnson_timed_i32(const int64_t *row_ptr, const int32_t *col, const int32_t *w,
                           int64_t n, int64_t nnz, int32_t *d, int64_t ld, int32_t inf,
                           int32_t *h, int32_t delta, void *stream, double *phase_ms,
                           int64_t *counts);

/*
 * Destroys the HIP timing events that the measurement entry points
 * (apsp_fw_timed_*, apsp_trace_begin) keep pooled for the calling thread,
 * on every device, and frees their host arrays.  Later measurement calls
 * create them again.  Call it before the HIP runtime shuts down (for
 * example from an exit handler that runs before static destructors); the
 * library itself makes no HIP call from a static destructor.  Returns
 * APSP_ERR_INVALID_VALUE while a launch trace is open, APSP_ERR_LAUNCH if a
 * HIP call failed (the events are then released as far as possible).
 */
int apsp_release_events(void);

/*
 * Arithmetic policy of int32 calls (process-wide; affects calls made after
 * it is set).  APSP_ARITH_AUTO (default): binary32 when it is exact (see
 * above) and n > 384 (at least nine Phase-3 tiles; below that the scan that
 * checks exactness costs more than binary32 saves); otherwise int32.  The
 * negative-weight entry points keep int32 below two Phase-3 tiles per
 * compute unit.  APSP_ARITH_F32_WHEN_EXACT: binary32 whenever it is exact.
 * APSP_ARITH_INT32: always int32.  Results are identical under every
 * policy.  Returns APSP_ERR_INVALID_VALUE for an unknown mode.
 */
enum { APSP_ARITH_AUTO = 0, APSP_ARITH_F32_WHEN_EXACT = 1, APSP_ARITH_INT32 = 2 };
int apsp_set_int32_arith(int mode);
int apsp_get_int32_arith(void);

/*
 * Diagnostic: the empirical VALU ceiling of the min-plus core on the current
 * device, in relaxations per second.  Runs a register-only replica of the
 * Phase-3 inner step (8 x 8 accumulators per thread, two candidates per
 * three-input min, no memory traffic) at 2 and at 4 waves per SIMD on the
 * null stream, synchronises, and reports the faster rate.  arith: 0 = int32
 * arithmetic, 1 = binary32, 2 = the packed (sum, index) keys of
 * apsp_successors_i32 (unsigned saturating adds, unsigned three-input min;
 * candidates per second).  Allocates
 * and frees a small device buffer.  Returns APSP_ERR_INVALID_VALUE for a bad
 * argument, APSP_ERR_LAUNCH on a HIP failure.
 */
int apsp_minplus_ceiling(int arith, double *relax_per_s);

/*
 * Diagnostic: the same replica at exactly waves_per_simd waves per SIMD
 * (1 to 4; one 256-thread workgroup per CU per wave).  gfx950's double
 * issue pairs two waves of a SIMD, so an odd count leaves one wave at the
 * single rate; at 3 waves per SIMD (the Phase-3 kernels' occupancy, set by
 * their registers) this is the rate those kernels can reach.  Same
 * arith codes, stream, synchronisation and errors as apsp_minplus_ceiling.
 */
int apsp_minplus_ceiling_waves(int arith, int waves_per_simd, double *relax_per_s);

/* Pivot block edge B used for an n-vertex matrix (rounds = ceil(n / B)). */
int64_t apsp_pivot_block(int64_t n);

/* Static text for a status code (never NULL). */
const char *apsp_status_string(int status);

/* hipError_t of the calling thread's last APSP_ERR_LAUNCH (0 if none). */
int apsp_last_hip_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int apsp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* APSP_H */
