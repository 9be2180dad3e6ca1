/*
 * sched_fuzz.c - random operation sequences against the host scheduler of
 * include/pakv_sched.h, for a build with AddressSanitizer and UBSan
 * (tests/test_sched_sanitized.py). Every entry point is called, including
 * its error paths (unknown ids, wrong states, oversize requests, NULL
 * arguments), and the block tables and page accounting are checked after
 * every operation:
 *   - page ids in the rows are inside the pool, and the distinct pages the
 *     rows reference plus the free pages never exceed the pool (pages held
 *     for queued requests that share a prefix make up the rest);
 *   - every running request's row holds exactly its budget of pages per
 *     layer, then -1; empty slots hold -1 and context length 0; one request
 *     per slot, the running count as reported;
 *   - once every request has finished, the whole pool is free again.
 * Usage: sched_fuzz <seed> <operations>. Exit status 0 when every check
 * holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pakv_sched.h"

#define P 96
#define L 2
#define MB 5
#define STRIDE 12
#define MAXREQ 4096

static uint64_t g_state;
static uint32_t rnd(uint32_t n) {   /* splitmix64 */
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return n ? (uint32_t)(z % n) : 0u;
}

static void fail(const char* what, long op) {
  fprintf(stderr, "sched_fuzz: %s (operation %ld)\n", what, op);
  exit(1);
}

/* what the driver knows about each request it submitted */
static int64_t g_id[MAXREQ];
static int g_total[MAXREQ];   /* prompt + max_new */
static int g_live[MAXREQ];    /* 1 while not finished */
static int g_n;
static int g_nlive;

static void check_tables(const pa_sched* s, long op) {
  const int32_t* bt = pa_sched_block_tables(s);
  const int32_t* ctx = pa_sched_context_lens(s);
  static int refs[P];
  memset(refs, 0, sizeof refs);
  int running_seen = 0;
  int owner_of[MB];
  for (int b = 0; b < MB; ++b) owner_of[b] = -1;
  for (int i = 0; i < g_n; ++i) {
    int32_t slot = -2;
    if (!g_live[i]) continue;
    if (pa_sched_slot(s, g_id[i], &slot) != PA_OK) fail("slot of a live request", op);
    if (slot < -1 || slot >= MB) fail("slot out of range", op);
    if (slot >= 0) {
      if (owner_of[slot] >= 0) fail("two requests in one slot", op);
      owner_of[slot] = i;
    }
  }
  for (int b = 0; b < MB; ++b) {
    const int owner = owner_of[b];
    for (int l = 0; l < L; ++l) {
      const int32_t* row = bt + ((size_t)l * MB + b) * STRIDE;
      int used = 0;
      while (used < STRIDE && row[used] >= 0) {
        if (row[used] >= P) fail("page id outside the pool", op);
        ++refs[row[used]];
        ++used;
      }
      for (int j = used; j < STRIDE; ++j)
        if (row[j] != -1) fail("entry after the budget is not -1", op);
      if (owner < 0 && used != 0) fail("empty slot holds pages", op);
      if (owner >= 0 && used != (g_total[owner] + 15) / 16) fail("row is not the budget", op);
    }
    if (owner < 0 && ctx[b] != 0) fail("empty slot has a context", op);
    if (owner >= 0) {
      ++running_seen;
      if (ctx[b] < 0 || ctx[b] > g_total[owner]) fail("context out of range", op);
    }
  }
  int referenced = 0;
  for (int p = 0; p < P; ++p) referenced += refs[p] > 0;
  int32_t free_pages = -1, queued = -1, running = -1;
  if (pa_sched_stats(s, &free_pages, &queued, &running) != PA_OK) fail("stats", op);
  if (running != running_seen) fail("running count", op);
  if (free_pages + referenced > P) fail("pages counted twice", op);
  if (queued < 0 || free_pages < 0) fail("negative counts", op);
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: sched_fuzz <seed> <operations>\n");
    return 2;
  }
  g_state = strtoull(argv[1], NULL, 10);
  const long ops = strtol(argv[2], NULL, 10);
  pa_sched* s = NULL;

  /* argument errors */
  if (pa_sched_create(NULL, P, L, MB, STRIDE, PA_BATCH_CONTINUOUS) != PA_ERR_NULL) fail("create NULL", -1);
  if (pa_sched_create(&s, 0, L, MB, STRIDE, PA_BATCH_CONTINUOUS) != PA_ERR_INVALID) fail("create 0 pages", -1);
  if (pa_sched_create(&s, P, L, MB, STRIDE, 7) != PA_ERR_INVALID) fail("create bad mode", -1);
  const int mode = (int)(g_state & 1u) ? PA_BATCH_STATIC : PA_BATCH_CONTINUOUS;
  if (pa_sched_create(&s, P, L, MB, STRIDE, mode) != PA_OK) fail("create", -1);
  int64_t id = 0;
  if (pa_sched_submit(s, 0, 0, &id) != PA_ERR_INVALID) fail("empty request", -1);
  if (pa_sched_submit(s, STRIDE * 16 + 1, 0, &id) != PA_ERR_CAPACITY) fail("row overflow", -1);
  if (pa_sched_submit(s, 1, 1, NULL) != PA_ERR_NULL) fail("submit NULL", -1);
  if (pa_sched_finish(s, 12345) != PA_ERR_INVALID) fail("finish unknown", -1);
  if (pa_sched_advance(s, 12345, 1) != PA_ERR_INVALID) fail("advance unknown", -1);
  int32_t slot = 0;
  if (pa_sched_slot(s, 12345, &slot) != PA_ERR_INVALID) fail("slot unknown", -1);
  if (pa_sched_submit_shared(s, 12345, 16, 20, 1, &id) == PA_OK) fail("shared from unknown", -1);

  int64_t admitted[MB];
  for (long op = 0; op < ops; ++op) {
    const uint32_t kind = rnd(100);
    if (kind < 30 && g_n < MAXREQ && g_nlive < 40) {        /* submit */
      const int prompt = (int)rnd(STRIDE * 16 / 2);
      const int max_new = 1 + (int)rnd(40);
      const pa_status st = pa_sched_submit(s, prompt, max_new, &id);
      if (st == PA_OK) {
        g_id[g_n] = id; g_total[g_n] = prompt + max_new; g_live[g_n] = 1; ++g_n; ++g_nlive;
      } else if (st != PA_ERR_CAPACITY) {
        fail("submit status", op);
      }
    } else if (kind < 40 && g_n > 0 && g_n < MAXREQ && g_nlive < 40) {   /* submit sharing a prefix */
      const int parent = (int)rnd((uint32_t)g_n);
      const int shared = (int)rnd(64);
      const int prompt = shared + (int)rnd(40);
      const int max_new = 1 + (int)rnd(20);
      const pa_status st = pa_sched_submit_shared(s, g_id[parent], shared, prompt, max_new, &id);
      if (st == PA_OK) {
        g_id[g_n] = id; g_total[g_n] = prompt + max_new; g_live[g_n] = 1; ++g_n; ++g_nlive;
      } else if (st != PA_ERR_STATE && st != PA_ERR_CAPACITY && st != PA_ERR_INVALID) {
        fail("submit_shared status", op);
      }
    } else if (kind < 60) {                                  /* admit */
      int32_t n = -1;
      if (pa_sched_admit(s, admitted, MB, &n) != PA_OK || n < 0 || n > MB) fail("admit", op);
    } else if (kind < 85 && g_n > 0) {                       /* advance */
      const int i = (int)rnd((uint32_t)g_n);
      const pa_status st = pa_sched_advance(s, g_id[i], (int)rnd(20));
      if (g_live[i] && st != PA_OK && st != PA_ERR_STATE && st != PA_ERR_INVALID) fail("advance status", op);
      if (!g_live[i] && st != PA_ERR_INVALID) fail("advance of a finished request", op);
    } else if (g_n > 0) {                                    /* finish */
      const int i = (int)rnd((uint32_t)g_n);
      const pa_status st = pa_sched_finish(s, g_id[i]);
      if (g_live[i] && st != PA_OK) fail("finish", op);
      if (!g_live[i] && st != PA_ERR_INVALID) fail("finish twice", op);
      if (g_live[i]) --g_nlive;
      g_live[i] = 0;
    }
    check_tables(s, op);
  }
  for (int i = 0; i < g_n; ++i)
    if (g_live[i] && pa_sched_finish(s, g_id[i]) != PA_OK) fail("final finish", ops);
  int32_t free_pages = -1, queued = -1, running = -1;
  if (pa_sched_stats(s, &free_pages, &queued, &running) != PA_OK) fail("stats", ops);
  if (free_pages != P || queued != 0 || running != 0) fail("pool not whole at the end", ops);
  pa_sched_destroy(s);
  printf("sched_fuzz: %ld operations, %d requests, mode %d: ok\n", ops, g_n, mode);
  return 0;
}
