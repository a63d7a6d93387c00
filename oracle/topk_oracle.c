/*
 * CPU oracle for exact row-wise Top-K.  TEST INFRASTRUCTURE ONLY: the tests,
 * the smoke check and the benchmark's CPU-baseline leg may call it; the
 * selector library never does.  It shares no code with the GPU path.
 *
 * What it computes is the plain definition of the operator contract in
 * "Sample-Guided Exact Top-K Selection for Long-Context Sparse Attention",
 * Sec. 2.1 ("Operator contract") and the exactness criterion of Sec. 6.1
 * (Eq. 30):
 *   - row r has valid length L = ke[r] clamped to [0, N];
 *   - if L <= K the answer is every valid index, then -1 sentinels;
 *   - otherwise the answer is K distinct indices such that no unselected
 *     valid value exceeds a selected one; ties at rank K are free.
 *
 * The row's valid values are sorted once, completely, in descending value
 * order (the C library qsort is the only primitive), and the first K
 * positions are taken.  Values are float32 and NaN-free; +-inf and
 * subnormals compare numerically (compile without flush-to-zero).  The pages
 * do not order -0.0 against +0.0; this oracle places +0.0 above -0.0 (a
 * refinement of the numeric order, so Eq. 30 still holds) and breaks the
 * remaining ties by ascending index only to make the sort deterministic.
 *
 * Per row it reports:
 *   sel_bits[r][0..K)  bit patterns of the K selected values, in sorted order
 *   sel_idx[r][0..K)   the indices in that order
 *   n_strict[r]        how many of them lie strictly above the K-th value;
 *                      those indices (the first n_strict) belong to every
 *                      exact answer, the rest are one valid choice among ties.
 * For L <= K: sel_idx = 0..L-1 then -1, sel_bits = those values then 0,
 * n_strict = L.
 *
 * Rows at or beyond min(m_live, M) are left untouched.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    float v;
    int32_t i;
} entry;

static uint32_t bits_of(float v) {
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    return u;
}

/* Descending value order; +0.0 before -0.0; then ascending index. */
static int cmp_desc(const void* pa, const void* pb) {
    const entry* a = (const entry*)pa;
    const entry* b = (const entry*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    /* numerically equal: only +0.0 against -0.0 can still differ */
    int sa = (int)(bits_of(a->v) >> 31);
    int sb = (int)(bits_of(b->v) >> 31);
    if (sa != sb) return sa - sb; /* sign clear (+0.0) first */
    if (a->i < b->i) return -1;
    if (a->i > b->i) return 1;
    return 0;
}

static void one_row(const float* row, int64_t L, int32_t K, entry* scratch,
                    uint32_t* sel_bits, int32_t* sel_idx, int32_t* n_strict) {
    if (L <= K) {
        for (int64_t j = 0; j < K; ++j) {
            sel_idx[j] = j < L ? (int32_t)j : -1;
            sel_bits[j] = j < L ? bits_of(row[j]) : 0u;
        }
        *n_strict = (int32_t)L;
        return;
    }
    for (int64_t j = 0; j < L; ++j) {
        scratch[j].v = row[j];
        scratch[j].i = (int32_t)j;
    }
    qsort(scratch, (size_t)L, sizeof(entry), cmp_desc);
    for (int32_t j = 0; j < K; ++j) {
        sel_bits[j] = bits_of(scratch[j].v);
        sel_idx[j] = scratch[j].i;
    }
    /* entries before the first copy of the K-th value are strictly above it */
    uint32_t kth = sel_bits[K - 1];
    int32_t s = 0;
    while (s < K && sel_bits[s] != kth) ++s;
    *n_strict = s;
}

typedef struct {
    const float* x;
    int64_t n, stride, rows;
    const int32_t* ke;
    int32_t k;
    uint32_t* sel_bits;
    int32_t* sel_idx;
    int32_t* n_strict;
    int64_t next; /* shared row counter, taken under the mutex */
    pthread_mutex_t mu;
    int failed;
} job;

static void* worker(void* p) {
    job* jb = (job*)p;
    entry* scratch = (entry*)malloc(sizeof(entry) * (size_t)(jb->n > 0 ? jb->n : 1));
    if (!scratch) {
        pthread_mutex_lock(&jb->mu);
        jb->failed = 1;
        pthread_mutex_unlock(&jb->mu);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&jb->mu);
        int64_t r = jb->next++;
        pthread_mutex_unlock(&jb->mu);
        if (r >= jb->rows) break;
        int64_t L = jb->ke[r];
        if (L < 0) L = 0;
        if (L > jb->n) L = jb->n;
        one_row(jb->x + r * jb->stride, L, jb->k, scratch, jb->sel_bits + r * jb->k,
                jb->sel_idx + r * jb->k, jb->n_strict + r);
    }
    free(scratch);
    return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int oracle_topk(const float* x, int64_t m, int64_t n, int64_t stride, const int32_t* ke,
                int64_t m_live, int32_t k, int32_t nthreads, uint32_t* sel_bits,
                int32_t* sel_idx, int32_t* n_strict) {
    if (m < 0 || n < 0 || stride < n || k < 1 || nthreads < 1) return -1;
    int64_t rows = m_live < m ? m_live : m;
    if (rows < 0) rows = 0;
    job jb;
    jb.x = x;
    jb.n = n;
    jb.stride = stride;
    jb.rows = rows;
    jb.ke = ke;
    jb.k = k;
    jb.sel_bits = sel_bits;
    jb.sel_idx = sel_idx;
    jb.n_strict = n_strict;
    jb.next = 0;
    jb.failed = 0;
    pthread_mutex_init(&jb.mu, NULL);
    int nt = nthreads;
    if (nt > 256) nt = 256;
    pthread_t th[256];
    int started = 0;
    for (int t = 0; t < nt; ++t) {
        if (pthread_create(&th[t], NULL, worker, &jb) != 0) break;
        ++started;
    }
    if (started == 0) worker(&jb);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    pthread_mutex_destroy(&jb.mu);
    return jb.failed ? -2 : 0;
}

/*
 * Coarse key c(x) of Sec. 4.2, Eq. 11, checked against a device's values for
 * every float32 bit pattern in [start, start + n):
 *   h  = the binary16 pattern of x under IEEE round-to-nearest-even (the
 *        host CPU's F16C conversion, _mm256_cvtps_ph with rounding mode 0);
 *   k  = h ^ 0x7FFF when the sign bit is clear, h when it is set (a larger
 *        value gets a smaller key);
 *   c  = k >> 5 (its top 11 bits).
 * got[i] is the device's c for pattern start + i.  NaN patterns are skipped
 * (the operator contract excludes NaN).  Returns the number of mismatches and
 * sets *first to the first mismatching pattern (unchanged when none); -1 when
 * the host CPU lacks F16C, -2 on bad arguments.
 */
#include <immintrin.h>

typedef struct {
    uint32_t start;
    int64_t lo, hi;
    const uint16_t* got;
    int64_t bad;
    int64_t first;  /* offset of the first mismatch, or -1 */
} coarse_job;

__attribute__((target("avx,f16c")))
static void* coarse_worker(void* arg) {
    coarse_job* j = (coarse_job*)arg;
    j->bad = 0;
    j->first = -1;
    for (int64_t i = j->lo; i < j->hi; i += 8) {
        uint32_t pat[8];
        int cnt = (int)(j->hi - i < 8 ? j->hi - i : 8);
        for (int u = 0; u < 8; ++u) pat[u] = j->start + (uint32_t)(i + (u < cnt ? u : 0));
        __m256 v;
        memcpy(&v, pat, sizeof pat);
        const __m128i hv = _mm256_cvtps_ph(v, 0);  /* 0: round to nearest even */
        uint16_t h[8];
        memcpy(h, &hv, sizeof h);
        for (int u = 0; u < cnt; ++u) {
            if ((pat[u] & 0x7FFFFFFFu) > 0x7F800000u) continue;  /* NaN */
            const uint32_t k16 = (h[u] & 0x8000u) ? h[u] : (uint32_t)(h[u] ^ 0x7FFFu);
            if ((k16 >> 5) != j->got[i + u]) {
                if (j->first < 0) j->first = i + u;
                ++j->bad;
            }
        }
    }
    return NULL;
}

int64_t oracle_coarse_check(uint32_t start, int64_t n, const uint16_t* got, int32_t nthreads,
                            uint32_t* first) {
    if (n < 0 || n > ((int64_t)1 << 32) - (int64_t)start || (n > 0 && !got) || !first ||
        nthreads < 1)
        return -2;
    __builtin_cpu_init();
    if (!__builtin_cpu_supports("f16c") || !__builtin_cpu_supports("avx")) return -1;
    int nt = nthreads > 256 ? 256 : nthreads;
    coarse_job jobs[256];
    pthread_t th[256];
    int started[256];
    const int64_t per = (n + nt - 1) / nt;
    for (int t = 0; t < nt; ++t) {
        jobs[t].start = start;
        jobs[t].lo = per * t < n ? per * t : n;
        jobs[t].hi = per * (t + 1) < n ? per * (t + 1) : n;
        jobs[t].got = got;
        started[t] = pthread_create(&th[t], NULL, coarse_worker, &jobs[t]) == 0;
        if (!started[t]) coarse_worker(&jobs[t]);
    }
    int64_t bad = 0;
    int64_t firsti = -1;
    for (int t = 0; t < nt; ++t) {
        if (started[t]) pthread_join(th[t], NULL);
        bad += jobs[t].bad;
        if (jobs[t].first >= 0 && (firsti < 0 || jobs[t].first < firsti)) firsti = jobs[t].first;
    }
    if (firsti >= 0) *first = start + (uint32_t)firsti;
    return bad;
}
