/*
 * CPU model of the single-batch-overlap protocol between the signalled down
 * GEMM and the polling combine (DeepGEMM single-batch-overlap pull request,
 * section 2: a counter per block of rows, incremented once part of the work
 * is done, polled by the consumer until it reaches a threshold; section 3:
 * the increment is release-ordered).  Run under ThreadSanitizer by the CPU
 * test suite; it checks the synchronisation pattern, not the arithmetic.
 *
 * Producer: "workgroups" = (row tile, column panel) pairs in tile-major order,
 * each executed by a team of threads: every thread stores its share of the
 * tile's panel (plain stores), the team meets at a barrier, then one thread
 * publishes: a release add of the panel's column count to the tile's counter
 * (the adds of all panels form one release sequence; the GPU code instead
 * stores the rows at device scope, waits for them to complete and adds with
 * no fence -- see below).  Consumer:
 * threads walk the layout rows in chunks and combine each token at its last
 * row: poll every counter the token reads (relaxed loads) until it reaches H,
 * then an acquire load of it, then plain reads of the rows; tokens with no
 * row are combined in a second pass.
 *
 * What this model does not cover: C11 has no memory scopes, and
 * ThreadSanitizer does not follow standalone fences, so the acquire load
 * stands for "relaxed poll, then acquire", and the release add for "stores,
 * then release".  The GPU producer stores its rows at device scope and waits
 * for them to complete before a relaxed add; the GPU consumer issues a
 * workgroup-scope fence after its polls and reads the rows with device-scope
 * loads.  Neither side writes back or invalidates an XCD's L2 (the down
 * GEMM's weight panels live there).  That is not a C11 pattern; it relies on
 * the GPU's cache rules, which test_sbo_hw_model.py states and checks
 * exhaustively on an operational model of per-XCD write-back L2 caches.
 *
 * Build with -DBROKEN to drop the consumer's wait: ThreadSanitizer must then
 * report a race (the test checks that the model can fail).
 */
#include <pthread.h>
#include <stdatomic.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

enum { R = 8, H = 24, C = 6, P = H / C, TEAM = 3, TEAMS = 2, CONSUMERS = 3, RC = 4, K = 3 };

static int n_tokens, n_rows, n_tiles;
static int* pos;      /* [T*K] layout row or -1 */
static int* row_src;  /* [n_rows] t*K+k or -1 */
static float* wgt;    /* [T*K] */
static float* y;      /* [n_rows][H] */
static float* out;    /* [T][H] */
static atomic_int* sig;

static float yval(int r, int c) { return (float)((r * 131 + c * 7) % 97) * 0.25f; }

typedef struct {
    int team, member;
    pthread_barrier_t* bar;
} prod_arg;

static void* producer(void* p) {
    prod_arg* a = (prod_arg*)p;
    for (int wg = a->team; wg < n_tiles * P; wg += TEAMS) {
        const int tile = wg / P, panel = wg % P;  /* tile-major */
        for (int i = a->member; i < R * C; i += TEAM) {
            const int r = tile * R + i / C, c = panel * C + i % C;
            y[r * H + c] = yval(r, c);
        }
        pthread_barrier_wait(a->bar);
        if (a->member == 0) atomic_fetch_add_explicit(&sig[tile], C, memory_order_release);
        pthread_barrier_wait(a->bar); /* the team moves on together */
    }
    return NULL;
}

static void combine_token(int t) {
    float acc[H];
    memset(acc, 0, sizeof acc);
#ifndef BROKEN
    for (int k = 0; k < K; ++k) {
        const int p = pos[t * K + k];
        if (p < 0) continue;
        while (atomic_load_explicit(&sig[p / R], memory_order_relaxed) < H) sched_yield();
        (void)atomic_load_explicit(&sig[p / R], memory_order_acquire);
    }
#endif
    for (int k = 0; k < K; ++k) {
        const int p = pos[t * K + k];
        if (p < 0) continue;
        for (int c = 0; c < H; ++c) acc[c] += wgt[t * K + k] * y[p * H + c];
    }
    memcpy(out + (size_t)t * H, acc, sizeof acc);
}

static int last_row(int t) {
    int last = -1;
    for (int k = 0; k < K; ++k) last = pos[t * K + k] > last ? pos[t * K + k] : last;
    return last;
}

static void* consumer(void* p) {
    const int id = (int)(size_t)p;
    const int row_units = (n_rows + RC - 1) / RC, units = row_units + (n_tokens + RC - 1) / RC;
    for (int u = id; u < units; u += CONSUMERS) {
        for (int i = 0; i < RC; ++i) {
            if (u < row_units) {
                const int r = u * RC + i;
                if (r >= n_rows || row_src[r] < 0) continue;
                const int t = row_src[r] / K;
                if (last_row(t) == r) combine_token(t);
            } else {
                const int t = (u - row_units) * RC + i;
                if (t < n_tokens && last_row(t) < 0) combine_token(t);
            }
        }
    }
    return NULL;
}

int main(int argc, char** argv) {
    const unsigned seed = argc > 1 ? (unsigned)atoi(argv[1]) : 1u;
    srand(seed);
    n_tokens = 40;
    const int n_exp = 4;
    /* a contiguous layout: experts' segments padded to R rows; slot k of a
       token goes to about expert (2k + t) % (n_exp + 4), experts >= n_exp are not
       local (-1), so some tokens have no local row */
    int count[8] = {0}, off[9] = {0};
    int* eid = malloc(sizeof(int) * n_tokens * K);
    for (int t = 0; t < n_tokens; ++t)
        for (int k = 0; k < K; ++k) {
            int e = (k * 2 + t + rand() % 3) % (n_exp + 4);
            for (int j = 0; j < k; ++j)
                if (eid[t * K + j] == e) e = -1; /* a token hits an expert once */
            eid[t * K + k] = e < n_exp ? e : -1;
            if (eid[t * K + k] >= 0) count[eid[t * K + k]]++;
        }
    for (int e = 0; e < n_exp; ++e) off[e + 1] = off[e] + (count[e] + R - 1) / R * R;
    n_rows = off[n_exp];
    n_tiles = n_rows / R;
    pos = malloc(sizeof(int) * n_tokens * K);
    row_src = malloc(sizeof(int) * (n_rows > 0 ? n_rows : 1));
    wgt = malloc(sizeof(float) * n_tokens * K);
    for (int r = 0; r < n_rows; ++r) row_src[r] = -1;
    int fill[8] = {0};
    for (int t = 0; t < n_tokens; ++t)
        for (int k = 0; k < K; ++k) {
            const int e = eid[t * K + k];
            wgt[t * K + k] = 0.5f + 0.25f * k;
            if (e < 0) { pos[t * K + k] = -1; continue; }
            pos[t * K + k] = off[e] + fill[e]++;
            row_src[pos[t * K + k]] = t * K + k;
        }
    y = calloc((size_t)n_rows * H, sizeof(float));
    out = malloc(sizeof(float) * n_tokens * H);
    for (int i = 0; i < n_tokens * H; ++i) out[i] = -1.0f;
    sig = calloc((size_t)n_tiles, sizeof(atomic_int));

    pthread_t th[TEAMS * TEAM + CONSUMERS];
    pthread_barrier_t bars[TEAMS];
    prod_arg args[TEAMS * TEAM];
    int n = 0;
    for (int c = 0; c < CONSUMERS; ++c) pthread_create(&th[n++], NULL, consumer, (void*)(size_t)c);
    for (int tm = 0; tm < TEAMS; ++tm) {
        pthread_barrier_init(&bars[tm], NULL, TEAM);
        for (int m = 0; m < TEAM; ++m) {
            args[tm * TEAM + m] = (prod_arg){tm, m, &bars[tm]};
            pthread_create(&th[n++], NULL, producer, &args[tm * TEAM + m]);
        }
    }
    for (int i = 0; i < n; ++i) pthread_join(th[i], NULL);

    int bad = 0;
    for (int t = 0; t < n_tokens; ++t)
        for (int c = 0; c < H; ++c) {
            float want = 0.0f;
            for (int k = 0; k < K; ++k)
                if (pos[t * K + k] >= 0) want += wgt[t * K + k] * yval(pos[t * K + k], c);
            if (out[t * H + c] != want) bad++;
        }
    for (int i = 0; i < n_tiles; ++i)
        if (atomic_load(&sig[i]) != H) bad++;
    int orphans = 0;
    for (int t = 0; t < n_tokens; ++t) orphans += last_row(t) < 0;
    printf("tiles %d rows %d tokens %d orphans %d mismatches %d\n", n_tiles, n_rows, n_tokens, orphans, bad);
    return bad ? 1 : 0;
}
