/*
 * pakv_client.c - a plain C client of libpakv (no Python, no torch): the C
 * ABI of include/pakv.h and include/pakv_sched.h plus the HIP runtime's C
 * API for device memory. Test infrastructure: tests/test_gpu_c_client.py
 * writes seeded inputs into a directory, runs this program on it, and checks
 * every output against the FP64 oracle.
 *
 * Flow (one small serving run):
 *   - the page pool is uploaded from k_pool.bin / v_pool.bin;
 *   - a scheduler (continuous batching) over the pool admits the requests of
 *     config.txt;
 *   - their prompts are prefilled layer by layer, layer 0 through a launch
 *     plan (pa_prefill_plan + pa_prefill_planned), the other layers through
 *     pa_prefill (prefill_{q,k,v}_<layer>.bin in, prefill_out_<layer>.bin
 *     out);
 *   - then `steps` decode steps: per layer pa_kv_append of the new token
 *     (step<s>_{k,v}_<layer>.bin), then attention, layer 0 through a launch
 *     plan (pa_decode_plan + pa_decode_planned), the other layers through
 *     pa_decode (step<s>_q_<layer>.bin in, step<s>_out_<layer>.bin out);
 *   - the block tables and context lengths used are written out
 *     (bt_prefill.bin, ctx_prefill.bin, bt_step<s>.bin, pos_step<s>.bin,
 *     ctx_step<s>.bin), and the final pool (k_final.bin, v_final.bin).
 *
 * config.txt: num_pages kv_heads q_heads head_dim layers max_batch
 *             max_pages_per_seq steps num_requests, then one
 *             "prompt_tokens max_new_tokens" line per request.
 * Exit status 0 on success; any library status other than PA_OK is printed
 * with pa_status_str and ends the run with status 1.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pakv.h"
#include "pakv_sched.h"

static const char* g_dir;

static void die(const char* what) {
  fprintf(stderr, "pakv_client: %s\n", what);
  exit(1);
}

static void check(pa_status st, const char* what) {
  if (st != PA_OK) {
    fprintf(stderr, "pakv_client: %s: %s (%d)\n", what, pa_status_str(st), (int)st);
    exit(1);
  }
}

static void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "pakv_client: %s: %s\n", what, hipGetErrorString(e));
    exit(1);
  }
}

static void path_of(char* out, size_t cap, const char* name) {
  if ((size_t)snprintf(out, cap, "%s/%s", g_dir, name) >= cap) die("path too long");
}

static void read_file(const char* name, void* dst, size_t bytes) {
  char p[4096];
  path_of(p, sizeof p, name);
  FILE* f = fopen(p, "rb");
  if (!f) die(p);
  if (fread(dst, 1, bytes, f) != bytes) die(p);
  fclose(f);
}

static void write_file(const char* name, const void* src, size_t bytes) {
  char p[4096];
  path_of(p, sizeof p, name);
  FILE* f = fopen(p, "wb");
  if (!f) die(p);
  if (fwrite(src, 1, bytes, f) != bytes) die(p);
  fclose(f);
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  hip_check(hipMalloc(&p, bytes ? bytes : 16), "hipMalloc");
  return p;
}

static void upload(void* dst, const void* src, size_t bytes) {
  hip_check(hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice), "copy to device");
}

static void download(void* dst, const void* src, size_t bytes) {
  hip_check(hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost), "copy to host");
}

/* A device array filled from a file of the given size. */
static void* dev_from_file(const char* name, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  if (!host) die("out of memory");
  read_file(name, host, bytes);
  void* d = dev_alloc(bytes);
  upload(d, host, bytes);
  free(host);
  return d;
}

int main(int argc, char** argv) {
  if (argc != 2) die("usage: pakv_client <directory>");
  g_dir = argv[1];

  char cfg[4096];
  path_of(cfg, sizeof cfg, "config.txt");
  FILE* f = fopen(cfg, "r");
  if (!f) die(cfg);
  int P, Hkv, Hq, D, L, MB, stride, steps, nreq;
  if (fscanf(f, "%d %d %d %d %d %d %d %d %d", &P, &Hkv, &Hq, &D, &L, &MB, &stride, &steps, &nreq) != 9)
    die("bad config header");
  if (MB < 1 || MB > 64) die("max_batch must be in 1..64 (fixed-size host arrays)");
  if (nreq < 1 || nreq > MB) die("bad request count");
  int prompt[64], max_new[64];
  for (int i = 0; i < nreq; ++i)
    if (fscanf(f, "%d %d", &prompt[i], &max_new[i]) != 2) die("bad request line");
  fclose(f);
  const float scale = 1.0f / sqrtf((float)D);

  /* the pool */
  const size_t page_elems = (size_t)Hkv * 16 * D;
  const size_t pool_bytes = (size_t)P * page_elems * 2;
  void* k_pool = dev_from_file("k_pool.bin", pool_bytes);
  void* v_pool = dev_from_file("v_pool.bin", pool_bytes);
  pa_pool* pool = NULL;
  check(pa_pool_create(&pool, k_pool, v_pool, P, 16, Hkv, D), "pa_pool_create");

  /* admission */
  pa_sched* sched = NULL;
  check(pa_sched_create(&sched, P, L, MB, stride, PA_BATCH_CONTINUOUS), "pa_sched_create");
  int64_t ids[64];
  for (int i = 0; i < nreq; ++i) check(pa_sched_submit(sched, prompt[i], max_new[i], &ids[i]), "pa_sched_submit");
  int64_t admitted[64];
  int32_t n_admitted = 0;
  check(pa_sched_admit(sched, admitted, 64, &n_admitted), "pa_sched_admit");
  if (n_admitted != nreq) die("not every request was admitted");
  int32_t slot_of[64];
  for (int i = 0; i < nreq; ++i) check(pa_sched_slot(sched, ids[i], &slot_of[i]), "pa_sched_slot");
  const int32_t* bt_host = pa_sched_block_tables(sched);
  const int32_t* ctx_host = pa_sched_context_lens(sched);
  const size_t bt_layer = (size_t)MB * stride;

  /* device copies of one layer's block tables and of the per-slot arrays */
  int32_t* bt_dev = (int32_t*)dev_alloc(bt_layer * 4);
  int32_t* ctx_dev = (int32_t*)dev_alloc((size_t)MB * 4);
  int32_t* pos_dev = (int32_t*)dev_alloc((size_t)MB * 4);
  int32_t* qs_dev = (int32_t*)dev_alloc((size_t)(MB + 1) * 4);
  int32_t* bt_clean = (int32_t*)malloc(bt_layer * 4);   /* -1 entries (empty) mapped to page 0 */
  if (!bt_clean) die("out of memory");

  /* ---- prefill: every slot's prompt is its chunk; empty slots have none */
  int32_t qs[65];
  qs[0] = 0;
  for (int b = 0; b < MB; ++b) {
    int chunk = 0;
    for (int i = 0; i < nreq; ++i)
      if (slot_of[i] == b) chunk = prompt[i];
    qs[b + 1] = qs[b] + chunk;
  }
  const int N = qs[MB];
  int max_chunk = 0;
  for (int i = 0; i < nreq; ++i)
    if (prompt[i] > max_chunk) max_chunk = prompt[i];
  upload(qs_dev, qs, (size_t)(MB + 1) * 4);
  upload(ctx_dev, ctx_host, (size_t)MB * 4);
  write_file("bt_prefill.bin", bt_host, (size_t)L * bt_layer * 4);
  write_file("ctx_prefill.bin", ctx_host, (size_t)MB * 4);
  float* out_dev = (float*)dev_alloc((size_t)(N > MB ? N : MB) * Hq * D * 4);
  float* out_host = (float*)malloc((size_t)(N > MB ? N : MB) * Hq * D * 4);
  if (!out_host) die("out of memory");
  /* the prefill launch plan from the host's cache and chunk lengths */
  int32_t chunk_host[64];
  for (int b = 0; b < MB; ++b) chunk_host[b] = qs[b + 1] - qs[b];
  const int64_t pplan_cap = pa_prefill_plan_capacity(pool, MB, Hq, max_chunk);
  if (pplan_cap < 0) die("pa_prefill_plan_capacity");
  int32_t* pplan = (int32_t*)malloc((size_t)(pplan_cap > 0 ? pplan_cap : 1) * 4);
  if (!pplan) die("out of memory");
  int32_t pplan_items = 0;
  check(pa_prefill_plan(pool, ctx_host, chunk_host, MB, Hq, stride, max_chunk, pplan, pplan_cap, &pplan_items),
        "pa_prefill_plan");
  int32_t* pplan_dev = (int32_t*)dev_alloc((size_t)(pplan_items > 0 ? pplan_items : 1) * 4);
  upload(pplan_dev, pplan, (size_t)pplan_items * 4);
  for (int l = 0; l < L; ++l) {
    char name[256];
    for (size_t e = 0; e < bt_layer; ++e) bt_clean[e] = bt_host[l * bt_layer + e] < 0 ? 0 : bt_host[l * bt_layer + e];
    upload(bt_dev, bt_clean, bt_layer * 4);
    snprintf(name, sizeof name, "prefill_q_%d.bin", l);
    void* q = dev_from_file(name, (size_t)N * Hq * D * 2);
    snprintf(name, sizeof name, "prefill_k_%d.bin", l);
    void* kr = dev_from_file(name, (size_t)N * Hkv * D * 2);
    snprintf(name, sizeof name, "prefill_v_%d.bin", l);
    void* vr = dev_from_file(name, (size_t)N * Hkv * D * 2);
    if (l == 0)
      check(pa_prefill_planned(pool, q, kr, vr, MB, Hq, N, max_chunk, qs_dev, bt_dev, stride, ctx_dev,
                               scale, out_dev, pplan_dev, pplan_items, NULL),
            "pa_prefill_planned");
    else
      check(pa_prefill(pool, q, kr, vr, MB, Hq, N, max_chunk, qs_dev, bt_dev, stride, ctx_dev, scale,
                       out_dev, NULL),
            "pa_prefill");
    hip_check(hipDeviceSynchronize(), "prefill");
    download(out_host, out_dev, (size_t)N * Hq * D * 4);
    snprintf(name, sizeof name, "prefill_out_%d.bin", l);
    write_file(name, out_host, (size_t)N * Hq * D * 4);
    hip_check(hipFree(q), "hipFree");
    hip_check(hipFree(kr), "hipFree");
    hip_check(hipFree(vr), "hipFree");
  }
  for (int i = 0; i < nreq; ++i) check(pa_sched_advance(sched, ids[i], prompt[i]), "pa_sched_advance");

  /* ---- decode steps */
  const size_t ws_bytes = pa_decode_workspace_bytes(pool, MB, Hq, stride);
  void* ws = dev_alloc(ws_bytes);
  const int64_t plan_cap = pa_decode_plan_capacity(pool, MB, stride);
  if (plan_cap < 0) die("pa_decode_plan_capacity");
  int32_t* plan = (int32_t*)malloc((size_t)(plan_cap > 0 ? plan_cap : 1) * 4);
  int32_t* plan_dev = (int32_t*)dev_alloc((size_t)(plan_cap > 0 ? plan_cap : 1) * 4);
  if (!plan) die("out of memory");
  for (int s = 0; s < steps; ++s) {
    char name[256];
    int32_t pos[64];
    for (int b = 0; b < MB; ++b) pos[b] = -1;
    for (int i = 0; i < nreq; ++i) pos[slot_of[i]] = ctx_host[slot_of[i]];
    upload(pos_dev, pos, (size_t)MB * 4);
    snprintf(name, sizeof name, "bt_step%d.bin", s);
    write_file(name, bt_host, (size_t)L * bt_layer * 4);
    snprintf(name, sizeof name, "pos_step%d.bin", s);
    write_file(name, pos, (size_t)MB * 4);
    for (int l = 0; l < L; ++l) {
      for (size_t e = 0; e < bt_layer; ++e) bt_clean[e] = bt_host[l * bt_layer + e] < 0 ? 0 : bt_host[l * bt_layer + e];
      upload(bt_dev, bt_clean, bt_layer * 4);
      snprintf(name, sizeof name, "step%d_k_%d.bin", s, l);
      void* kn = dev_from_file(name, (size_t)MB * Hkv * D * 2);
      snprintf(name, sizeof name, "step%d_v_%d.bin", s, l);
      void* vn = dev_from_file(name, (size_t)MB * Hkv * D * 2);
      check(pa_kv_append(pool, kn, vn, MB, bt_dev, stride, pos_dev, NULL), "pa_kv_append");
      hip_check(hipDeviceSynchronize(), "append");
      hip_check(hipFree(kn), "hipFree");
      hip_check(hipFree(vn), "hipFree");
    }
    for (int i = 0; i < nreq; ++i) check(pa_sched_advance(sched, ids[i], 1), "pa_sched_advance");
    upload(ctx_dev, ctx_host, (size_t)MB * 4);
    snprintf(name, sizeof name, "ctx_step%d.bin", s);
    write_file(name, ctx_host, (size_t)MB * 4);
    int32_t items = 0;
    check(pa_decode_plan(pool, ctx_host, MB, Hq, stride, plan, plan_cap, &items), "pa_decode_plan");
    upload(plan_dev, plan, (size_t)(items > 0 ? items : 1) * 4);
    for (int l = 0; l < L; ++l) {
      for (size_t e = 0; e < bt_layer; ++e) bt_clean[e] = bt_host[l * bt_layer + e] < 0 ? 0 : bt_host[l * bt_layer + e];
      upload(bt_dev, bt_clean, bt_layer * 4);
      snprintf(name, sizeof name, "step%d_q_%d.bin", s, l);
      void* q = dev_from_file(name, (size_t)MB * Hq * D * 2);
      if (l == 0)
        check(pa_decode_planned(pool, q, MB, Hq, bt_dev, stride, ctx_dev, scale, out_dev, ws, ws_bytes,
                                plan_dev, items, NULL),
              "pa_decode_planned");
      else
        check(pa_decode(pool, q, MB, Hq, bt_dev, stride, ctx_dev, scale, out_dev, ws, ws_bytes, NULL),
              "pa_decode");
      hip_check(hipDeviceSynchronize(), "decode");
      download(out_host, out_dev, (size_t)MB * Hq * D * 4);
      snprintf(name, sizeof name, "step%d_out_%d.bin", s, l);
      write_file(name, out_host, (size_t)MB * Hq * D * 4);
      hip_check(hipFree(q), "hipFree");
    }
  }

  /* ---- the final pool, then everything freed */
  void* pool_host = malloc(pool_bytes);
  if (!pool_host) die("out of memory");
  download(pool_host, k_pool, pool_bytes);
  write_file("k_final.bin", pool_host, pool_bytes);
  download(pool_host, v_pool, pool_bytes);
  write_file("v_final.bin", pool_host, pool_bytes);
  for (int i = 0; i < nreq; ++i) check(pa_sched_finish(sched, ids[i]), "pa_sched_finish");
  int32_t free_pages = -1;
  check(pa_sched_stats(sched, &free_pages, NULL, NULL), "pa_sched_stats");
  if (free_pages != P) die("pages not returned to the pool");
  pa_sched_destroy(sched);
  pa_pool_destroy(pool);
  free(pool_host);
  free(plan);
  free(pplan);
  free(out_host);
  free(bt_clean);
  hip_check(hipFree(plan_dev), "hipFree");
  hip_check(hipFree(pplan_dev), "hipFree");
  hip_check(hipFree(ws), "hipFree");
  hip_check(hipFree(out_dev), "hipFree");
  hip_check(hipFree(qs_dev), "hipFree");
  hip_check(hipFree(pos_dev), "hipFree");
  hip_check(hipFree(ctx_dev), "hipFree");
  hip_check(hipFree(bt_dev), "hipFree");
  hip_check(hipFree(v_pool), "hipFree");
  hip_check(hipFree(k_pool), "hipFree");
  printf("pakv_client: %d requests, %d prefill rows, %d decode steps, %d layers: ok\n", nreq, N, steps, L);
  return 0;
}
