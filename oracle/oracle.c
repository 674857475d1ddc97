/*
 * CPU oracle for all-pairs shortest paths -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the bench's CPU-baseline leg load
 * this library.  It is a plain, slow, obviously correct statement of what the
 * GPU path must compute, and it shares no code, header or constant with it.
 *
 * What is computed.  For a weighted digraph given as a dense row-major matrix
 * W (W[i][i] = 0, W[i][j] = edge weight, or the caller's "infinity" sentinel
 * when there is no edge), the all-pairs shortest-path distance
 *     delta(i, j) = min over directed paths i -> j of the sum of the weights,
 * with delta(i, i) = 0 and delta(i, j) = inf when j is unreachable from i.
 * Weights are non-negative, so a shortest simple path exists whenever j is
 * reachable and the minimum is well defined.
 *
 * Two independent routes to delta are given:
 *
 *  1. oracle_fw_*: the textbook Floyd-Warshall recurrence
 *        d(i,j) <- min(d(i,j), d(i,k) + d(k,j))   for k = 0, 1, ..., n-1
 *     with k outermost.  This is the recurrence that the blocked algorithm on
 *     the page "Katz and Kider" (thesis section 4.6; its Phase 1 runs
 *     "standard Floyd-Warshall" on a block) reorganises into tiles; the
 *     blocked form performs the same relaxations in another order and reaches
 *     the same distances (section 4.6, "the parallel versions giving the same
 *     values as the serial one" is the corresponding claim on the
 *     "Loops into zones" page, section "What it does not change").
 *     An optional k_end < n stops after the first k_end pivots, which exposes
 *     the intermediate matrices of the recurrence to the tests.
 *
 *  2. oracle_sssp_*: Dijkstra's algorithm from one source, written the way the
 *     Johnson's-algorithm page formalises it (Ukrainian/Russian CEUR paper on
 *     Johnson's APSP with Glushkov algebras, operators init, ExtractMin and
 *     RelaxEdge): all distances start at infinity except the source's 0; the
 *     unsettled vertex with the smallest tentative distance is settled; each
 *     of its out-edges (u,v) relaxes d(v) when d(v) > d(u) + w(u,v).
 *     One call yields one row of delta, so sampled rows of very large
 *     matrices can be checked without the cubic recurrence.
 *
 * Arithmetic.  int32 inputs: every candidate sum is formed in int64, so no
 * overflow can occur whatever the sentinel.  Floating-point inputs are
 * computed in binary64 (the caller widens float32 weights exactly); sums are
 * single IEEE additions, min is exact, no fused or reassociated operations.
 *
 * Parallelism.  Within one pivot k, the rows i are independent: row k and
 * column k do not change during step k because d(k,k) = 0 (or >= 0), so
 * d(i,k) + d(k,k) >= d(i,k) and d(k,k) + d(k,j) >= d(k,j).  Each element
 * therefore sees exactly the same sequence of operations whether the i loop
 * runs serially or under OpenMP, and the results are bit-identical.
 */
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 0; /* 0 = OpenMP default */

void oracle_set_threads(int t) { g_threads = t < 0 ? 0 : t; }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

int oracle_version(void) { return 2; }

/* Floyd-Warshall on int32 distances, in place; pivots k = k_begin .. k_end-1
 * taken in order.  Given the recurrence's state after pivots 0 .. k_begin-1,
 * it leaves the state after pivots 0 .. k_end-1, so a long run can be split
 * into consecutive ranges. */
void oracle_fw_range_i32(int32_t *d, int64_t n, int64_t ld, int64_t k_begin, int64_t k_end) {
  if (k_begin < 0) k_begin = 0;
  if (k_end > n) k_end = n;
  int nt = oracle_max_threads();
  for (int64_t k = k_begin; k < k_end; ++k) {
    const int32_t *row_k = d + k * ld;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t i = 0; i < n; ++i) {
      int32_t *row_i = d + i * ld;
      int64_t d_ik = row_i[k];
      for (int64_t j = 0; j < n; ++j) {
        int64_t cand = d_ik + (int64_t)row_k[j];
        if (cand < row_i[j]) row_i[j] = (int32_t)cand;
      }
    }
  }
}

/* Pivots 0 .. k_end-1 (the whole recurrence when k_end >= n). */
void oracle_fw_i32(int32_t *d, int64_t n, int64_t ld, int64_t k_end) {
  oracle_fw_range_i32(d, n, ld, 0, k_end);
}

/* Floyd-Warshall on binary64 distances, in place; pivots k = k_begin ..
 * k_end-1 in order, as for int32 above. */
void oracle_fw_range_f64(double *d, int64_t n, int64_t ld, int64_t k_begin, int64_t k_end) {
  if (k_begin < 0) k_begin = 0;
  if (k_end > n) k_end = n;
  int nt = oracle_max_threads();
  for (int64_t k = k_begin; k < k_end; ++k) {
    const double *row_k = d + k * ld;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t i = 0; i < n; ++i) {
      double *row_i = d + i * ld;
      double d_ik = row_i[k];
      for (int64_t j = 0; j < n; ++j) {
        double cand = d_ik + row_k[j];
        if (cand < row_i[j]) row_i[j] = cand;
      }
    }
  }
}

void oracle_fw_f64(double *d, int64_t n, int64_t ld, int64_t k_end) {
  oracle_fw_range_f64(d, n, ld, 0, k_end);
}

/*
 * Many independent graphs (the "many small graphs" case of the page "Loops
 * into zones"): graph g is the n x n matrix at d + g * stride with leading
 * dimension ld, closed by the same recurrence as above.  Graphs run in
 * parallel (an inner parallel region, when nested, runs on its one thread,
 * and the recurrence's results do not depend on its thread count).
 */
void oracle_fw_batched_i32(int32_t *d, int64_t batch, int64_t n, int64_t ld, int64_t stride) {
  int nt = oracle_max_threads();
#pragma omp parallel for schedule(dynamic, 8) num_threads(nt)
  for (int64_t g = 0; g < batch; ++g) oracle_fw_i32(d + g * stride, n, ld, n);
}

void oracle_fw_batched_f64(double *d, int64_t batch, int64_t n, int64_t ld, int64_t stride) {
  int nt = oracle_max_threads();
#pragma omp parallel for schedule(dynamic, 8) num_threads(nt)
  for (int64_t g = 0; g < batch; ++g) oracle_fw_f64(d + g * stride, n, ld, n);
}

/*
 * Floyd-Warshall that also admits negative weights (the setting of Johnson's
 * algorithm on the page "Johnson's APSP in Glushkov algorithmic algebras"):
 * a candidate through k is formed only when both of its parts are finite,
 * so the sentinel is never treated as a number.  int64 distances, in place
 * on an int64 matrix.  Without a negative cycle the result is delta (a
 * shortest walk is then a shortest simple path).  With one, some vertex on
 * it ends with d(i, i) < 0; the function returns 1 in that case, else 0.
 */
int oracle_fw_guarded_i64(int64_t *d, int64_t n, int64_t ld, int64_t inf) {
  int nt = oracle_max_threads();
  for (int64_t k = 0; k < n; ++k) {
    const int64_t *row_k = d + k * ld;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t i = 0; i < n; ++i) {
      int64_t *row_i = d + i * ld;
      int64_t d_ik = row_i[k];
      if (d_ik == inf) continue;
      for (int64_t j = 0; j < n; ++j) {
        if (row_k[j] == inf) continue;
        int64_t cand = d_ik + row_k[j];
        if (cand < row_i[j]) row_i[j] = cand;
      }
    }
  }
  for (int64_t i = 0; i < n; ++i)
    if (d[i * ld + i] < 0) return 1;
  return 0;
}

/*
 * Dijkstra from `src` on the dense int32 weight matrix w (edge u->v exists
 * when u != v and w[u][v] != inf).  Writes delta(src, .) to out[0..n-1]:
 * unreachable vertices get exactly `inf`.  Returns 0, or -1 on bad arguments
 * or allocation failure.
 */
int oracle_sssp_i32(const int32_t *w, int64_t n, int64_t ld, int32_t inf,
                    int64_t src, int32_t *out) {
  if (n <= 0 || src < 0 || src >= n) return -1;
  int64_t *dist = (int64_t *)malloc((size_t)n * sizeof(int64_t));
  unsigned char *settled = (unsigned char *)calloc((size_t)n, 1);
  if (!dist || !settled) { free(dist); free(settled); return -1; }
  for (int64_t v = 0; v < n; ++v) dist[v] = INT64_MAX; /* "infinity" */
  dist[src] = 0;
  for (;;) {
    /* ExtractMin over the unsettled vertices with a finite distance. */
    int64_t u = -1;
    for (int64_t v = 0; v < n; ++v)
      if (!settled[v] && dist[v] != INT64_MAX && (u < 0 || dist[v] < dist[u])) u = v;
    if (u < 0) break;
    settled[u] = 1;
    const int32_t *wu = w + u * ld;
    for (int64_t v = 0; v < n; ++v) { /* RelaxEdge(u, v) */
      if (v == u || wu[v] == inf) continue;
      int64_t cand = dist[u] + (int64_t)wu[v];
      if (dist[v] > cand) dist[v] = cand;
    }
  }
  for (int64_t v = 0; v < n; ++v)
    out[v] = dist[v] == INT64_MAX ? inf : (int32_t)dist[v];
  free(dist);
  free(settled);
  return 0;
}

/* Dijkstra from `src` on a dense binary64 weight matrix; see above. */
int oracle_sssp_f64(const double *w, int64_t n, int64_t ld, double inf,
                    int64_t src, double *out) {
  if (n <= 0 || src < 0 || src >= n) return -1;
  double *dist = (double *)malloc((size_t)n * sizeof(double));
  unsigned char *reached = (unsigned char *)calloc((size_t)n, 1);
  unsigned char *settled = (unsigned char *)calloc((size_t)n, 1);
  if (!dist || !reached || !settled) {
    free(dist); free(reached); free(settled); return -1;
  }
  dist[src] = 0.0;
  reached[src] = 1;
  for (;;) {
    int64_t u = -1;
    for (int64_t v = 0; v < n; ++v)
      if (!settled[v] && reached[v] && (u < 0 || dist[v] < dist[u])) u = v;
    if (u < 0) break;
    settled[u] = 1;
    const double *wu = w + u * ld;
    for (int64_t v = 0; v < n; ++v) {
      if (v == u || wu[v] == inf) continue;
      double cand = dist[u] + wu[v];
      if (!reached[v] || dist[v] > cand) { dist[v] = cand; reached[v] = 1; }
    }
  }
  for (int64_t v = 0; v < n; ++v) out[v] = reached[v] ? dist[v] : inf;
  free(dist);
  free(reached);
  free(settled);
  return 0;
}

/* Many sources at once (each source independent; OpenMP over sources). */
int oracle_sssp_rows_i32(const int32_t *w, int64_t n, int64_t ld, int32_t inf,
                         const int64_t *srcs, int64_t nsrc, int32_t *out,
                         int64_t ldo) {
  int bad = 0;
  int nt = oracle_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : bad)
  for (int64_t s = 0; s < nsrc; ++s)
    bad |= oracle_sssp_i32(w, n, ld, inf, srcs[s], out + s * ldo) != 0;
  return bad ? -1 : 0;
}

int oracle_sssp_rows_f64(const double *w, int64_t n, int64_t ld, double inf,
                         const int64_t *srcs, int64_t nsrc, double *out,
                         int64_t ldo) {
  int bad = 0;
  int nt = oracle_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : bad)
  for (int64_t s = 0; s < nsrc; ++s)
    bad |= oracle_sssp_f64(w, n, ld, inf, srcs[s], out + s * ldo) != 0;
  return bad ? -1 : 0;
}

/*
 * Bellman-Ford from `src` over a graph in compressed sparse rows (edge e of
 * vertex u goes to col[e] with weight w[e], for e in [row_ptr[u],
 * row_ptr[u+1])), following the Bellman-Ford operator of the page "Johnson's
 * APSP in Glushkov algorithmic algebras": init (source 0, every other vertex
 * unreached), rounds of RelaxEdges over every edge, then the negative-cycle
 * condition cnc (some edge can still be relaxed).  A round that changes
 * nothing leaves every later round unchanged too, so the rounds stop early
 * there; after n rounds without that happening, an edge is still relaxable,
 * which is the cnc condition.  Weights may be negative; sums are int64.
 * Writes the shortest walk length from src to every vertex into dist
 * (INT64_MAX when unreached).  Returns 1 when a negative cycle is reachable
 * from src, 0 otherwise, -1 on bad arguments.
 */
int oracle_sssp_bf_csr_i64(const int64_t *row_ptr, const int32_t *col, const int64_t *w,
                           int64_t n, int64_t src, int64_t *dist) {
  if (n <= 0 || src < 0 || src >= n) return -1;
  for (int64_t v = 0; v < n; ++v) dist[v] = INT64_MAX;
  dist[src] = 0;
  for (int64_t round = 0; round < n; ++round) {
    int changed = 0;
    for (int64_t u = 0; u < n; ++u) {
      if (dist[u] == INT64_MAX) continue;
      for (int64_t e = row_ptr[u]; e < row_ptr[u + 1]; ++e) {
        const int64_t v = col[e];
        const int64_t cand = dist[u] + w[e];
        if (cand < dist[v]) { dist[v] = cand; changed = 1; }
      }
    }
    if (!changed) return 0;
  }
  return 1;
}

/* Bellman-Ford from many sources (independent; OpenMP over sources).  Row s
 * of out (leading dimension ldo) receives the distances from srcs[s];
 * neg[s] the negative-cycle result.  Returns -1 if any call rejected its
 * arguments, else 0. */
int oracle_sssp_bf_rows_i64(const int64_t *row_ptr, const int32_t *col, const int64_t *w,
                            int64_t n, const int64_t *srcs, int64_t nsrc, int64_t *out,
                            int64_t ldo, int32_t *neg) {
  int bad = 0;
  int nt = oracle_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt) reduction(| : bad)
  for (int64_t s = 0; s < nsrc; ++s) {
    const int r = oracle_sssp_bf_csr_i64(row_ptr, col, w, n, srcs[s], out + s * ldo);
    if (r < 0) bad = 1;
    else neg[s] = r;
  }
  return bad ? -1 : 0;
}

/*
 * Min-plus product C <- min(C, A (x) B), (A (x) B)[i][j] = min over t of
 * A[i][t] + B[t][j]: the update of a block from its pivot-row and
 * pivot-column blocks on the "Katz and Kider" page (thesis section 4.6,
 * Algorithms 17-18), written as the definition.  Entries equal to inf are
 * "no path": a candidate through one is not formed.  int64 (exact) and
 * binary64 (single IEEE additions, exact min) versions; OpenMP over rows.
 */
void oracle_minplus_i64(int64_t *c, int64_t ldc, const int64_t *a, int64_t lda,
                        const int64_t *b, int64_t ldb, int64_t m, int64_t n, int64_t k,
                        int64_t inf) {
  int nt = oracle_max_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t i = 0; i < m; ++i)
    for (int64_t t = 0; t < k; ++t) {
      const int64_t ait = a[i * lda + t];
      if (ait == inf) continue;
      for (int64_t j = 0; j < n; ++j) {
        const int64_t btj = b[t * ldb + j];
        if (btj == inf) continue;
        const int64_t cand = ait + btj;
        if (cand < c[i * ldc + j]) c[i * ldc + j] = cand;
      }
    }
}

void oracle_minplus_f64(double *c, int64_t ldc, const double *a, int64_t lda, const double *b,
                        int64_t ldb, int64_t m, int64_t n, int64_t k) {
  int nt = oracle_max_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t i = 0; i < m; ++i)
    for (int64_t t = 0; t < k; ++t) {
      const double ait = a[i * lda + t];
      for (int64_t j = 0; j < n; ++j) {
        const double cand = ait + b[t * ldb + j];
        if (cand < c[i * ldc + j]) c[i * ldc + j] = cand;
      }
    }
}

/*
 * Successor (first-hop) matrix, by its definition: for i != j, nxt[i][j] is
 * the smallest u != i minimising w[i][u] + d[u][j] over the u whose two
 * terms are both below inf (RelaxEdge of the Johnson's-APSP page over the
 * final distances, keeping the argument), -1 when there is none; nxt[i][i] =
 * i.  w and d are n x n int64 (leading dimension ld), nxt int32 (ld).
 */
void oracle_successors_i64(const int64_t *w, const int64_t *d, int32_t *nxt, int64_t n, int64_t ld,
                           int64_t inf) {
  int nt = oracle_max_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < n; ++j) {
      if (i == j) { nxt[i * ld + j] = (int32_t)i; continue; }
      int64_t best = 0, arg = -1;
      for (int64_t u = 0; u < n; ++u) {
        if (u == i || w[i * ld + u] == inf || d[u * ld + j] == inf) continue;
        const int64_t cand = w[i * ld + u] + d[u * ld + j];
        if (cand >= inf) continue;  /* not below the sentinel: no path, as for the distances */
        if (arg < 0 || cand < best) { best = cand; arg = u; }
      }
      nxt[i * ld + j] = (int32_t)arg;
    }
}

/*
 * The same definition for listed rows only, for spot checks of large
 * matrices: row k of nxt_rows is row rows[k] of the successor matrix, from
 * row k of w_rows (the out-weights of vertex rows[k]) and all of d.  w_rows
 * and nxt_rows are r x n, d is n x n (leading dimension n).
 */
void oracle_successors_rows_i64(const int64_t *w_rows, const int64_t *d, const int64_t *rows,
                                int64_t r, int32_t *nxt_rows, int64_t n, int64_t inf) {
  int nt = oracle_max_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t k = 0; k < r; ++k) {
    const int64_t i = rows[k];
    const int64_t *wi = w_rows + k * n;
    for (int64_t j = 0; j < n; ++j) {
      if (i == j) { nxt_rows[k * n + j] = (int32_t)i; continue; }
      int64_t best = 0, arg = -1;
      for (int64_t u = 0; u < n; ++u) {
        if (u == i || wi[u] == inf || d[u * n + j] == inf) continue;
        const int64_t cand = wi[u] + d[u * n + j];
        if (cand >= inf) continue;
        if (arg < 0 || cand < best) { best = cand; arg = u; }
      }
      nxt_rows[k * n + j] = (int32_t)arg;
    }
  }
}
