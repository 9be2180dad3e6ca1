/*
 * pakv_graph.c - a decode step captured into a HIP graph through the HIP
 * runtime's C API, by a plain C client of libpakv (test infrastructure,
 * built as libpakv_graph.so by build_client.py and driven from
 * tests/test_gpu_graph_hip.py with device buffers the test allocates).
 *
 * A step is, per layer l: pa_kv_append of the new tokens (when the step
 * appends), then pa_decode_planned with the launch plan in a device buffer.
 * pg_capture records one step on a stream (hipStreamBeginCapture /
 * hipStreamEndCapture), checks that the graph holds kernel nodes only and
 * instantiates it. Every step, replayed or eager, first copies its plan
 * from pinned host memory into the device plan buffer with hipMemcpyAsync
 * on the stream (outside the graph; two staging buffers, each rewritten
 * only after its previous copy has run); pg_replay then launches the graph,
 * pg_eager queues the step's calls one by one. Both time `count` steps
 * between two HIP events on the stream (device time) and with the host's
 * monotonic clock around the loop that queues them (host time).
 */
#define _POSIX_C_SOURCE 199309L
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "pakv.h"

#define PG_MAX_LAYERS 64

/* One decode step's arguments: per-layer device pointers in arrays. */
typedef struct {
  const pa_pool* pool;
  int32_t layers, num_seqs, num_q_heads, max_pages_per_seq;
  float scale;
  const void* q[PG_MAX_LAYERS];            /* BF16 [B][Hq][D] per layer */
  const void* k_new[PG_MAX_LAYERS];        /* BF16 [B][Hkv][D] per layer (NULL: no append) */
  const void* v_new[PG_MAX_LAYERS];
  const int32_t* block_tables[PG_MAX_LAYERS];
  float* out[PG_MAX_LAYERS];
  const int32_t* context_lens;             /* [B] */
  const int32_t* positions;                /* [B] */
  void* workspace;
  size_t workspace_bytes;
  int32_t* plan_dev;                       /* device buffer the decodes read */
  int32_t plan_words;
} pg_step;

typedef struct {
  hipGraphExec_t exec;
} pg_graph;

/* Two pinned staging buffers for the per-step plan copy. */
typedef struct {
  int32_t* pinned[2];
  hipEvent_t copied[2];
  int used[2];
  int32_t words;
} pg_staging;

static void staging_free(pg_staging* st) {
  for (int k = 0; k < 2; ++k) {
    if (st->pinned[k]) hipHostFree(st->pinned[k]);
    if (st->copied[k]) hipEventDestroy(st->copied[k]);
  }
}

static int staging_init(pg_staging* st, int32_t words) {
  memset(st, 0, sizeof *st);
  st->words = words;
  for (int k = 0; k < 2; ++k) {
    if (hipHostMalloc((void**)&st->pinned[k], (size_t)(words > 0 ? words : 1) * 4, 0) != hipSuccess) return 2;
    if (hipEventCreateWithFlags(&st->copied[k], hipEventDisableTiming) != hipSuccess) return 2;
  }
  return 0;
}

/* Step i's plan into plan_dev, through staging buffer i % 2. */
static int upload_plan(pg_staging* st, int i, const int32_t* plan_host, int32_t* plan_dev, hipStream_t stream) {
  const int k = i & 1;
  const size_t bytes = (size_t)st->words * 4;
  if (st->used[k] && hipEventSynchronize(st->copied[k]) != hipSuccess) return 2;
  memcpy(st->pinned[k], plan_host, bytes);
  if (bytes && hipMemcpyAsync(plan_dev, st->pinned[k], bytes, hipMemcpyHostToDevice, stream) != hipSuccess) return 2;
  if (hipEventRecord(st->copied[k], stream) != hipSuccess) return 2;
  st->used[k] = 1;
  return 0;
}

static double now_us(void) {
  struct timespec t;
  clock_gettime(CLOCK_MONOTONIC, &t);
  return (double)t.tv_sec * 1e6 + (double)t.tv_nsec * 1e-3;
}

/* Status: 0 ok; 1 a library call failed; 2 a HIP call failed; 3 the graph
 * holds a node that is not a kernel; 4 bad arguments. */
static int queue_step(const pg_step* s, hipStream_t stream) {
  if (s->layers < 1 || s->layers > PG_MAX_LAYERS) return 4;
  for (int l = 0; l < s->layers; ++l) {
    if (s->k_new[l]) {
      if (pa_kv_append(s->pool, s->k_new[l], s->v_new[l], s->num_seqs, s->block_tables[l], s->max_pages_per_seq,
                       s->positions, stream) != PA_OK)
        return 1;
    }
    if (pa_decode_planned(s->pool, s->q[l], s->num_seqs, s->num_q_heads, s->block_tables[l], s->max_pages_per_seq,
                          s->context_lens, s->scale, s->out[l], s->workspace, s->workspace_bytes, s->plan_dev,
                          s->plan_words, stream) != PA_OK)
      return 1;
  }
  return 0;
}

static int time_region(hipStream_t stream, hipEvent_t e0, hipEvent_t e1, float* ms) {
  if (hipEventRecord(e1, stream) != hipSuccess) return 2;
  if (hipEventSynchronize(e1) != hipSuccess) return 2;
  if (hipEventElapsedTime(ms, e0, e1) != hipSuccess) return 2;
  return 0;
}

/* `count` eager steps on `stream`, each with its plan copy (plan_host into
 * s->plan_dev); *ms: their device time (HIP events), *host_us: the host's
 * time to queue them. */
int pg_eager(const pg_step* s, const int32_t* plan_host, void* stream_, int count, float* ms, double* host_us) {
  hipStream_t stream = (hipStream_t)stream_;
  pg_staging stg;
  hipEvent_t e0 = NULL, e1 = NULL;
  int st = staging_init(&stg, s->plan_words);
  if (st == 0 && hipEventCreate(&e0) != hipSuccess) st = 2;
  if (st == 0 && hipEventCreate(&e1) != hipSuccess) st = 2;
  if (st == 0 && hipStreamSynchronize(stream) != hipSuccess) st = 2;
  if (st == 0 && hipEventRecord(e0, stream) != hipSuccess) st = 2;
  const double t0 = now_us();
  for (int i = 0; i < count && st == 0; ++i) {
    st = upload_plan(&stg, i, plan_host, s->plan_dev, stream);
    if (st == 0) st = queue_step(s, stream);
  }
  *host_us = now_us() - t0;
  if (st == 0) st = time_region(stream, e0, e1, ms);
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  staging_free(&stg);
  return st;
}

/* One step captured on `stream` and instantiated; *nodes: the graph's node
 * count. The plan the captured decodes read is s->plan_dev. */
int pg_capture(const pg_step* s, void* stream_, pg_graph** out, int* nodes) {
  hipStream_t stream = (hipStream_t)stream_;
  *out = NULL;
  if (hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal) != hipSuccess) return 2;
  int st = queue_step(s, stream);
  hipGraph_t g = NULL;
  if (hipStreamEndCapture(stream, &g) != hipSuccess || !g) return 2;
  if (st != 0) {
    hipGraphDestroy(g);
    return st;
  }
  size_t n = 0;
  if (hipGraphGetNodes(g, NULL, &n) != hipSuccess) st = 2;
  hipGraphNode_t* list = st == 0 ? (hipGraphNode_t*)calloc(n ? n : 1, sizeof(hipGraphNode_t)) : NULL;
  if (st == 0 && !list) st = 4;
  if (st == 0 && hipGraphGetNodes(g, list, &n) != hipSuccess) st = 2;
  for (size_t i = 0; st == 0 && i < n; ++i) {
    hipGraphNodeType t;
    if (hipGraphNodeGetType(list[i], &t) != hipSuccess) st = 2;
    else if (t != hipGraphNodeTypeKernel) st = 3;
  }
  free(list);
  *nodes = (int)n;
  pg_graph* pg = NULL;
  if (st == 0) {
    pg = (pg_graph*)calloc(1, sizeof(pg_graph));
    if (!pg) st = 4;
  }
  if (st == 0 && hipGraphInstantiate(&pg->exec, g, NULL, NULL, 0) != hipSuccess) st = 2;
  hipGraphDestroy(g);
  if (st != 0) {
    if (pg) {
      if (pg->exec) hipGraphExecDestroy(pg->exec);
      free(pg);
    }
    return st;
  }
  *out = pg;
  return 0;
}

/* `count` replayed steps, each with its plan copy (plan_host, plan_words
 * words: the length the graph was captured with, into plan_dev) before the
 * graph launch; *ms: their device time (HIP events), *host_us: the host's
 * time to queue them. */
int pg_replay(pg_graph* pg, const int32_t* plan_host, int32_t* plan_dev, int32_t plan_words, void* stream_,
              int count, float* ms, double* host_us) {
  hipStream_t stream = (hipStream_t)stream_;
  pg_staging stg;
  hipEvent_t e0 = NULL, e1 = NULL;
  int st = staging_init(&stg, plan_words);
  if (st == 0 && hipEventCreate(&e0) != hipSuccess) st = 2;
  if (st == 0 && hipEventCreate(&e1) != hipSuccess) st = 2;
  if (st == 0 && hipStreamSynchronize(stream) != hipSuccess) st = 2;
  if (st == 0 && hipEventRecord(e0, stream) != hipSuccess) st = 2;
  const double t0 = now_us();
  for (int i = 0; i < count && st == 0; ++i) {
    st = upload_plan(&stg, i, plan_host, plan_dev, stream);
    if (st == 0 && hipGraphLaunch(pg->exec, stream) != hipSuccess) st = 2;
  }
  *host_us = now_us() - t0;
  if (st == 0) st = time_region(stream, e0, e1, ms);
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  staging_free(&stg);
  return st;
}

void pg_destroy(pg_graph* pg) {
  if (!pg) return;
  if (pg->exec) hipGraphExecDestroy(pg->exec);
  free(pg);
}
