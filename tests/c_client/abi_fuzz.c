/*
 * abi_fuzz.c - the host-side code of libpakv (pakv.hip compiled for the
 * host only) under AddressSanitizer and UBSan (tests/test_abi_sanitized.py):
 *   - pa_decode_plan on random context lengths, block-table widths, head
 *     dims and group sizes: whole items of 8 words, each with 1 .. ucap
 *     units (4, or 2 when more than 8 query heads share a KV head); every
 *     existing (sequence, split) exactly once (an empty context once, as
 *     split 0); a sequence with 2 .. ucap splits whole, in split order, in one
 *     item; each unit's rotation the pairs before it in its item mod the
 *     workgroup's waves; the bins' chains (item b < bins first, each item
 *     naming the next) reach every item once, moving forward past the first
 *     items; bin costs (pairs + 2 per unit) within one group's cost of each
 *     other; and the same call into a buffer one word short of the plan
 *     refused, nothing written past it;
 *   - pa_prefill_plan on random cache and chunk lengths (negative and past
 *     the bounds included): every row block that holds rows appears once
 *     and no other, costs never increase along the plan outside the
 *     reversed tiers of a one-round grid, and a capacity one short is
 *     refused;
 *   - the sizing calls and pa_status_str over every code and beyond;
 *   - the argument checks of every entry point that queues work, always with
 *     an argument they must refuse, so nothing reaches the HIP runtime.
 * Usage: abi_fuzz <seed> <rounds>. Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pakv.h"

static uint64_t g_state;
static uint32_t rnd(uint32_t n) {   /* splitmix64 */
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return n ? (uint32_t)(z % n) : 0u;
}

static void fail(const char* what, long round) {
  fprintf(stderr, "abi_fuzz: %s (round %ld)\n", what, round);
  exit(1);
}

/* fake device pointers: never dereferenced by the host code */
#define DEV ((void*)(uintptr_t)0x100000)
#define DEV_MIS ((void*)(uintptr_t)0x100002)

static int64_t clamp_ctx64(int32_t c, int32_t stride) {
  int64_t n = c < 0 ? 0 : c;
  return n > (int64_t)stride * 16 ? (int64_t)stride * 16 : n;
}

static void plan_round(long round) {
  const int d = rnd(2) ? 64 : 128;
  const int hkv = 1 + (int)rnd(8);
  const int group = 1 + (int)rnd(16);
  const int hq = hkv * group;
  const int ucap = group <= 8 ? 4 : 2;
  const int waves = d == 64 ? 16 : 8;
  pa_pool* pool = NULL;
  if (pa_pool_create(&pool, DEV, DEV, 1 + (int)rnd(100000), 16, hkv, d) != PA_OK) fail("pool", round);
  const int32_t num_seqs = (int32_t)rnd(300);
  const int32_t stride = 1 + (int32_t)rnd(rnd(4) ? 300 : 3000);
  const int64_t cap = pa_decode_plan_capacity(pool, num_seqs, stride);
  if (cap < 0) fail("capacity", round);
  int32_t* ctx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(num_seqs ? num_seqs : 1));
  if (!ctx) fail("oom", round);
  for (int b = 0; b < num_seqs; ++b) {
    const uint32_t k = rnd(10);
    ctx[b] = k == 0 ? 0 : k == 1 ? -(int32_t)rnd(100) : k == 2 ? stride * 16 + (int32_t)rnd(5000)
                                                              : (int32_t)rnd((uint32_t)stride * 16 + 1);
  }
  const int split_tok = pa_split_tokens(d);
  if (split_tok != (d == 64 ? 2048 : 1024)) fail("split tokens", round);
  const int sp = split_tok / 16;
  int64_t units = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t pages = (clamp_ctx64(ctx[b], stride) + 15) / 16;
    units += pages == 0 ? 1 : (pages + sp - 1) / sp;
  }
  if (units * 8 > cap) fail("units above capacity", round);
  int32_t* plan = (int32_t*)malloc(sizeof(int32_t) * (size_t)(cap ? cap : 1));
  if (!plan) fail("oom", round);
  int32_t words = -1;
  if (pa_decode_plan(pool, ctx, num_seqs, hq, stride, plan, cap, &words) != PA_OK) fail("plan", round);
  if (num_seqs == 0) {
    if (words != 0) fail("empty plan", round);
  } else {
    if (words <= 0 || words % 8 != 0 || words > units * 8) fail("word count", round);
    /* one word short: refused, nothing written past the buffer (ASan watches) */
    int32_t* short_buf = (int32_t*)malloc(sizeof(int32_t) * (size_t)(words - 1 ? words - 1 : 1));
    if (!short_buf) fail("oom", round);
    int32_t w2 = -1;
    if (pa_decode_plan(pool, ctx, num_seqs, hq, stride, short_buf, words - 1, &w2) == PA_OK) fail("short capacity", round);
    free(short_buf);
  }
  char* seen = (char*)calloc((size_t)(num_seqs ? num_seqs : 1) * 2048, 1);
  if (!seen) fail("oom", round);
  const int32_t nitems = words / 8;
  int64_t* item_cost = (int64_t*)calloc((size_t)(nitems ? nitems : 1), sizeof(int64_t));
  if (!item_cost) fail("oom", round);
  int64_t max_group = 0;
  int64_t placed = 0;
  for (int32_t i = 0; i < words; i += 8) {
    const int32_t* it = plan + i;
    if (it[6] != 0 || it[7] != 0) fail("unused words", round);
    int nu = 0;
    int64_t before = 0, pairs_item = 0;
    for (int u = 0; u < 4; ++u) {
      if (it[u] < 0) {
        for (int v = u; v < 4; ++v)
          if (it[v] != -1) fail("unit after a gap", round);
        break;
      }
      ++nu;
      const int b = (int)((uint32_t)it[u] & 0xFFFFFu);
      const int s = (int)((uint32_t)it[u] >> 20);
      if (b >= num_seqs || s >= 2048) fail("unit out of range", round);
      if (seen[(size_t)b * 2048 + s]++) fail("unit twice", round);
      ++placed;
      const int64_t pages = (clamp_ctx64(ctx[b], stride) + 15) / 16;
      const int64_t ns = pages == 0 ? 1 : (pages + sp - 1) / sp;
      if (s >= ns) fail("split past the context", round);
      if (((uint32_t)it[4] >> (4 * u) & 15u) != (uint32_t)(before % waves)) fail("rotation", round);
      const int64_t pg = pages == 0 ? 0 : (pages - (int64_t)s * sp < sp ? pages - (int64_t)s * sp : sp);
      before += (pg + 1) / 2;
      pairs_item += (pg + 1) / 2;
      if (s == 0 && ns >= 2 && ns <= ucap) {   /* a short sequence: whole, in order, from here */
        int64_t gp = 0;
        for (int64_t v = 0; v < ns; ++v) {
          const int64_t pv = pages - v * sp < sp ? pages - v * sp : sp;
          gp += (pv + 1) / 2;
        }
        if (gp + 2 * ns > max_group) max_group = gp + 2 * ns;
        if (u + ns > 4) fail("short sequence cut", round);
        for (int v = 1; v < ns; ++v)
          if (it[u + v] != (int32_t)((uint32_t)b | ((uint32_t)v << 20))) fail("short sequence cut", round);
      }
      if (s > 0 && ns <= ucap && (u == 0 || it[u - 1] != (int32_t)((uint32_t)b | ((uint32_t)(s - 1) << 20))))
        fail("split of a short sequence out of place", round);
    }
    if (nu == 0 || nu > ucap) fail("units per item", round);
    if ((uint32_t)it[4] >> (4 * nu) != 0u) fail("rotation bits past the units", round);
    item_cost[i / 8] = pairs_item + 2 * nu;
    /* a group of one unit (a single split, or one split of a long sequence) */
    for (int u = 0; u < nu; ++u) {
      const int b = (int)((uint32_t)it[u] & 0xFFFFFu);
      const int s = (int)((uint32_t)it[u] >> 20);
      const int64_t pages = (clamp_ctx64(ctx[b], stride) + 15) / 16;
      const int64_t ns = pages == 0 ? 1 : (pages + sp - 1) / sp;
      if (ns == 1 || ns > ucap) {
        const int64_t pg = pages == 0 ? 0 : (pages - (int64_t)s * sp < sp ? pages - (int64_t)s * sp : sp);
        if ((pg + 1) / 2 + 2 > max_group) max_group = (pg + 1) / 2 + 2;
      }
    }
  }
  if (placed != (num_seqs ? units : 0)) fail("units missing", round);
  /* the bins' chains: every item once, forward, past the first items */
  const int32_t slots = 256 / hkv > 0 ? 256 / hkv : 1;
  const int32_t nb = nitems < slots ? nitems : slots;
  char* reached = (char*)calloc((size_t)(nitems ? nitems : 1), 1);
  if (!reached) fail("oom", round);
  int64_t cmin = INT64_MAX, cmax = 0;
  for (int32_t b = 0; b < nb; ++b) {
    int64_t cost = 0;
    for (int32_t k = b;;) {
      if (reached[k]++) fail("item reached twice", round);
      cost += item_cost[k];
      const int32_t nxt = plan[(size_t)k * 8 + 5];
      if (nxt == 0) break;
      if (nxt <= k || nxt < nb || nxt >= nitems) fail("chain step", round);
      k = nxt;
    }
    if (cost < cmin) cmin = cost;
    if (cost > cmax) cmax = cost;
  }
  for (int32_t k = 0; k < nitems; ++k)
    if (!reached[k]) fail("item not reached", round);
  if (nb > 0 && cmax - cmin > max_group) fail("bin balance", round);
  free(reached);
  free(item_cost);
  free(seen);
  free(plan);
  free(ctx);
  pa_pool_destroy(pool);
}

static void prefill_plan_round(long round) {
  const int d = rnd(2) ? 64 : 128;
  static const int kv_choices[4] = {1, 2, 4, 8};
  const int hkv = kv_choices[rnd(4)];
  const int group = 1 + (int)rnd(16);
  const int hq = hkv * group;
  pa_pool* pool = NULL;
  if (pa_pool_create(&pool, DEV, DEV, 1 + (int)rnd(100000), 16, hkv, d) != PA_OK) fail("pool", round);
  const int32_t num_seqs = (int32_t)rnd(40);
  const int32_t stride = 1 + (int32_t)rnd(400);
  const int32_t max_chunk = (int32_t)rnd(rnd(4) ? 700 : 5000);
  const int64_t cap = pa_prefill_plan_capacity(pool, num_seqs, hq, max_chunk);
  const int64_t row_blocks = ((int64_t)max_chunk * group + 127) / 128;
  if (cap != (int64_t)num_seqs * row_blocks) fail("prefill capacity", round);
  int32_t* ctx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(num_seqs ? num_seqs : 1));
  int32_t* chunk = (int32_t*)malloc(sizeof(int32_t) * (size_t)(num_seqs ? num_seqs : 1));
  if (!ctx || !chunk) fail("oom", round);
  int64_t need = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const uint32_t k = rnd(8);
    ctx[b] = k == 0 ? -(int32_t)rnd(50) : k == 1 ? stride * 16 + (int32_t)rnd(100) : (int32_t)rnd((uint32_t)stride * 16 + 1);
    chunk[b] = k == 2 ? -(int32_t)rnd(50) : k == 3 ? max_chunk + (int32_t)rnd(100) : (int32_t)rnd((uint32_t)max_chunk + 1);
    const int64_t c = ctx[b] < 0 ? 0 : (ctx[b] > stride * 16 ? stride * 16 : ctx[b]);
    int64_t n = chunk[b] < 0 ? 0 : (chunk[b] > max_chunk ? max_chunk : chunk[b]);
    if (n > stride * 16 - c) n = stride * 16 - c;
    need += (n * group + 127) / 128;
  }
  int32_t* plan = (int32_t*)malloc(sizeof(int32_t) * (size_t)(need ? need : 1));
  if (!plan) fail("oom", round);
  int32_t items = -1;
  if (need > 0 &&
      pa_prefill_plan(pool, ctx, chunk, num_seqs, hq, stride, max_chunk, plan, need - 1, &items) == PA_OK)
    fail("prefill short capacity", round);
  if (pa_prefill_plan(pool, ctx, chunk, num_seqs, hq, stride, max_chunk, plan, need, &items) != PA_OK)
    fail("prefill plan", round);
  if (items != need) fail("prefill item count", round);
  char* seen = (char*)calloc((size_t)(num_seqs ? num_seqs : 1) * (size_t)(row_blocks ? row_blocks : 1), 1);
  if (!seen) fail("oom", round);
  int64_t prev = INT64_MAX;
  int breaks = 0;
  for (int32_t i = 0; i < items; ++i) {
    const uint32_t it = (uint32_t)plan[i];
    const int b = (int)(it & 0xFFFFFu);
    const int64_t rb = (int64_t)(it >> 20);
    if (b >= num_seqs || rb >= row_blocks) fail("prefill item out of range", round);
    if (seen[(size_t)b * row_blocks + rb]++) fail("prefill item twice", round);
    const int64_t c = ctx[b] < 0 ? 0 : (ctx[b] > stride * 16 ? stride * 16 : ctx[b]);
    int64_t n = chunk[b] < 0 ? 0 : (chunk[b] > max_chunk ? max_chunk : chunk[b]);
    if (n > stride * 16 - c) n = stride * 16 - c;
    const int64_t rows = n * group;
    if (rb * 128 >= rows) fail("prefill item past the chunk", round);
    const int64_t last = c + ((rb * 128 + 127 < rows - 1 ? rb * 128 + 127 : rows - 1) / group);
    const int64_t pairs = ((last + 16) / 16 + 1) / 2;
    if (pairs > prev) ++breaks;
    prev = pairs;
  }
  /* 256 CUs x prefill workgroups per CU (4 at head_dim 64, 2 at 128) */
  if (breaks > 0 && (int64_t)items * hkv > 256 * (d == 64 ? 4 : 2)) fail("prefill plan order", round);
  free(seen);
  free(plan);
  free(chunk);
  free(ctx);
  pa_pool_destroy(pool);
}

static void validation_round(long round) {
  pa_pool* pool = NULL;
  const int d = rnd(2) ? 64 : 128;
  if (pa_pool_create(&pool, DEV, DEV, 64, 16, 8, d) != PA_OK) fail("pool", round);
  float* out = (float*)DEV;
  /* each call carries one argument the host checks refuse */
  switch (rnd(12)) {
    case 0:
      if (pa_decode(pool, DEV, 4, 30, DEV, 4, DEV, 0.1f, out, NULL, 0, NULL) != PA_ERR_INVALID) fail("decode heads", round);
      break;
    case 1:
      if (pa_decode(pool, DEV_MIS, 4, 32, DEV, 4, DEV, 0.1f, out, NULL, 0, NULL) != PA_ERR_ALIGN) fail("decode align", round);
      break;
    case 2:
      /* 600 pages: more splits than a workgroup finishes, at either head_dim */
      if (pa_decode(pool, DEV, 4, 32, DEV, 600, DEV, 0.1f, out, NULL, 0, NULL) != PA_ERR_WORKSPACE) fail("decode workspace", round);
      break;
    case 3:
      if (pa_decode(pool, DEV, 4, 32, DEV, 4, DEV, INFINITY, out, NULL, 0, NULL) != PA_ERR_INVALID) fail("decode scale", round);
      break;
    case 4:
      if (pa_decode_planned(pool, DEV, 4, 32, DEV, 4, DEV, 0.1f, out, NULL, 0, NULL, 1, NULL) != PA_ERR_NULL) fail("planned", round);
      break;
    case 5:
      if (pa_decode_planned(pool, DEV, 4, 32, DEV, 4, DEV, 0.1f, out, NULL, 0, DEV, -8, NULL) != PA_ERR_INVALID) fail("planned items", round);
      if (pa_decode_planned(pool, DEV, 4, 32, DEV, 4, DEV, 0.1f, out, NULL, 0, DEV, 12, NULL) != PA_ERR_INVALID) fail("planned whole items", round);
      break;
    case 6:
      if (pa_decode_append(pool, DEV, NULL, DEV, DEV, 4, 32, DEV, 4, DEV, 0.1f, out, NULL, 0, NULL) != PA_ERR_NULL) fail("append", round);
      break;
    case 7:
      if (pa_kv_append(pool, DEV_MIS, DEV, 4, DEV, 4, DEV, NULL) != PA_ERR_ALIGN) fail("kv_append", round);
      break;
    case 8:
      if (pa_kv_write(pool, DEV, DEV, 4, 10, 8, DEV, DEV, 0, DEV, NULL) != PA_ERR_INVALID) fail("kv_write", round);
      break;
    case 9:
      if (pa_prefill(pool, DEV, DEV, DEV, 2, 8 * 17, 10, 8, DEV, DEV, 4, DEV, 0.1f, out, NULL) != PA_ERR_UNSUPPORTED) fail("prefill group", round);
      break;
    case 10:
      if (pa_prefill(pool, NULL, DEV, DEV, 2, 32, 10, 8, DEV, DEV, 4, DEV, 0.1f, out, NULL) != PA_ERR_NULL) fail("prefill null", round);
      break;
    default: {
      pa_pool* other = NULL;
      if (pa_pool_create(&other, DEV, DEV, 64, 16, 8, 96) != PA_ERR_UNSUPPORTED) fail("head dim", round);
      if (other) pa_pool_destroy(other);
      break;
    }
  }
  if (pa_decode_workspace_bytes(pool, (int32_t)rnd(1000), 32, 1 + (int32_t)rnd(5000)) > ((size_t)1 << 40)) fail("workspace size", round);
  pa_pool_destroy(pool);
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: abi_fuzz <seed> <rounds>\n");
    return 2;
  }
  g_state = strtoull(argv[1], NULL, 10);
  const long rounds = strtol(argv[2], NULL, 10);
  for (int st = -3; st < 20; ++st) {
    const char* t = pa_status_str((pa_status)st);
    if (!t || !t[0]) fail("status text", -1);
  }
  if (pa_decode_plan_capacity(NULL, 1, 1) >= 0) fail("capacity NULL", -1);
  int32_t items = 0;
  if (pa_decode_plan(NULL, NULL, 0, 32, 1, NULL, 0, &items) != PA_ERR_NULL) fail("plan NULL", -1);
  for (long r = 0; r < rounds; ++r) {
    plan_round(r);
    prefill_plan_round(r);
    validation_round(r);
  }
  printf("abi_fuzz: %ld rounds: ok\n", rounds);
  return 0;
}
