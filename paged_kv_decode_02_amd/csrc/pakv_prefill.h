// pakv_prefill.h - gfx950 device code of libpakv's paged prefill (included by
// pakv.hip after pakv_kernels.h).
//
// Prefill takes a chunk of new tokens per sequence: it writes their K/V into
// the sequence's pages (prefill fills a request's pages: comrad404.com review
// of the samir-vllm README, section "Что README говорит о KV-кэше и пакетном
// декодировании") and computes causal grouped-query attention for all of
// them at once ("Construye tu propio motor de inferencia LLM ..." (aibit.im),
// sections "Prefill vs. Decode" and "Atención de Consulta Agrupada (GQA)").
// The token at position p attends over positions 0 .. p of its sequence,
// read in place from the pages; positions before the chunk were cached
// earlier.
//
// Attention work decomposition. For one (sequence, KV head) the chunk's
// query rows are the (token, head) pairs of the G query heads of that KV
// head, row index rho = token * G + head. A workgroup of 4 wavefronts takes
// 64 consecutive rows, 16 per wave; each wave streams the key pages its rows
// can see (up to the position of its last token), two pages per step:
//
//   S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16): A = the 16
//     keys of a page x 32 head dims, B = 32 head dims x the wave's 16 rows;
//     lane (r = lane % 16, grp = lane / 16) gets keys 4 grp + 0..3 of row r;
//   causal mask by select, FP32 online softmax per row (the 4 lanes holding a
//     row reduce their maxima with two xor shuffles);
//   O^T += V^T P^T on the matrix cores: A = V^T (16 head dims x 32 keys: for
//     lane group grp, keys 4 grp + 0..3 of each of the two pages, which are
//     8 contiguous bytes of a slot-minor V row), B = P^T in the same key
//     order, P split into BF16 hi + lo as in decode.
// The waves share nothing; there is no LDS and no barrier.
#pragma once

namespace pakv {

struct PrefillArgs {
  const uint16_t* kpool;
  const uint16_t* vpool;
  const uint16_t* q;            // [N][Hq][D]
  const int32_t* query_start;   // [B + 1]
  const int32_t* block_tables;  // [B][stride]
  const int32_t* ctx_before;    // [B]
  float* out;                   // [N][Hq][D]
  int32_t num_pages;
  int32_t num_seqs;
  int32_t num_rows;             // N
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t stride;
  int32_t max_chunk;            // host bound on every chunk's length
  int32_t row_blocks;           // 64-row blocks per (sequence, KV head) in the grid
  float scale_log2;
};

struct WriteArgs {
  uint16_t* kpool;
  uint16_t* vpool;
  const uint16_t* k_rows;       // [N][Hkv][D]
  const uint16_t* v_rows;
  const int32_t* query_start;
  const int32_t* block_tables;
  const int32_t* ctx_before;
  int32_t num_pages;
  int32_t num_seqs;
  int32_t num_rows;
  int32_t num_kv_heads;
  int32_t stride;
  int32_t max_chunk;
  int32_t pages_per_seq;        // page blocks per sequence in the grid
};

// A sequence's chunk as the kernels see it: rows [r0, r0 + n) of the row
// arrays, positions [c, c + n); clamped so that nothing leaves the row arrays
// or the block-table row.
struct Chunk {
  int r0, n, c;
};

__device__ __forceinline__ Chunk load_chunk(const int32_t* query_start, const int32_t* ctx_before,
                                            int b, int num_rows, int max_chunk, int stride) {
  Chunk ch;
  int r0 = query_start[b];
  int r1 = query_start[b + 1];
  int c = ctx_before[b];
  r0 = r0 < 0 ? 0 : (r0 > num_rows ? num_rows : r0);
  r1 = r1 < r0 ? r0 : (r1 > num_rows ? num_rows : r1);
  c = c < 0 ? 0 : (c > stride * kPage ? stride * kPage : c);
  int n = r1 - r0;
  n = n > max_chunk ? max_chunk : n;
  n = n > stride * kPage - c ? stride * kPage - c : n;
  ch.r0 = r0;
  ch.n = n;
  ch.c = c;
  return ch;
}

// ------------------------------------------------------------ chunk write
// One 256-thread block per (sequence, page the chunk touches): K rows are
// 16-byte copies; every V slot row (32 bytes, one head dim of one KV head) of
// the page is built from the chunk's tokens, reading the old row first only
// when the chunk covers part of the page.
template <int D>
__global__ __launch_bounds__(256) void kv_write_kernel(WriteArgs a) {
  const int b = blockIdx.x % a.num_seqs;
  const int j = blockIdx.x / a.num_seqs;
  const Chunk ch = load_chunk(a.query_start, a.ctx_before, b, a.num_rows, a.max_chunk, a.stride);
  if (ch.n <= 0) return;
  const int first_page = ch.c / kPage;
  const int last_page = (ch.c + ch.n - 1) / kPage;
  const int pg = first_page + j;
  if (pg > last_page) return;
  const int pid = a.block_tables[(size_t)b * a.stride + pg];
  if (pid < 0 || pid >= a.num_pages) return;
  const int s0 = max(ch.c, pg * kPage) - pg * kPage;             // slots [s0, s1) are written
  const int s1 = min(ch.c + ch.n, (pg + 1) * kPage) - pg * kPage;
  const int row_of_slot0 = ch.r0 + pg * kPage - ch.c;             // chunk row of slot 0
  const int H = a.num_kv_heads;
  const size_t tile0 = (size_t)pid * H;
  // K: (slot, kv head, 16-byte chunk)
  const int kchunks = (s1 - s0) * H * (D / 8);
  for (int e = threadIdx.x; e < kchunks; e += 256) {
    const int part = e % (D / 8);
    const int g = (e / (D / 8)) % H;
    const int slot = s0 + e / ((D / 8) * H);
    const size_t row = (size_t)(row_of_slot0 + slot);
    *(u32x4*)(a.kpool + ((tile0 + g) * kPage + slot) * D + 8 * part) =
        *(const u32x4*)(a.k_rows + (row * H + g) * D + 8 * part);
  }
  // V: one slot row per (kv head, head dim)
  const bool whole = s0 == 0 && s1 == kPage;
  for (int e = threadIdx.x; e < H * D; e += 256) {
    const int g = e / D;
    const int dd = e - g * D;
    u32x4* vrow = (u32x4*)(a.vpool + ((tile0 + g) * D + dd) * kPage);
    u32x4 h0, h1;
    if (whole) {
      h0 = u32x4{0u, 0u, 0u, 0u};
      h1 = h0;
    } else {
      h0 = vrow[0];
      h1 = vrow[1];
    }
    for (int slot = s0; slot < s1; ++slot) {
      const uint32_t nv = a.v_rows[((size_t)(row_of_slot0 + slot) * H + g) * D + dd];
      const int w = (slot & 7) >> 1;
      const uint32_t sh = (slot & 1) * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i != w) continue;
        if (slot < 8) h0[i] = (h0[i] & ~(0xFFFFu << sh)) | (nv << sh);
        else h1[i] = (h1[i] & ~(0xFFFFu << sh)) | (nv << sh);
      }
    }
    vrow[0] = h0;
    vrow[1] = h1;
  }
}

// -------------------------------------------------------------- attention
template <int D>
struct PrefillPair {
  u32x4 k[2][D / 32];     // S^T A operands: page j of the pair, k-step kk
  u32x4 v[D / 16];        // O^T A operands: dwords 0-1 page 0, 2-3 page 1
};

template <int D>
struct PrefillWave {
  const uint16_t* ktile;  // K pool + KV head tile of page 0
  const uint16_t* vtile;
  const int32_t* bt_row;  // the sequence's block-table row
  size_t page_elems;
  int num_pages;          // pool size (page ids are clamped into it)
  int key_pages;          // pages holding positions 0 .. last_pos
  int last_pos;           // position of the wave's last token (keys past it are zeroed)
  int pos;                // this lane's query position (rows past the chunk: last_pos)
  uint32_t koff;          // lane's element offset inside a K tile: key r, dims 8 grp
  uint32_t voff;          // lane's element offset inside a V tile: dim r, slots 4 grp
  float sl2;
  bf16x8 qf[D / 32];      // the lane's query row, B operand
};

template <int D>
__device__ __forceinline__ int clamp_pid(const PrefillWave<D>& w, int logical) {
  const int p = w.bt_row[logical];
  return p < 0 ? 0 : (p >= w.num_pages ? w.num_pages - 1 : p);
}

template <int D>
__device__ __forceinline__ void prefill_issue(const PrefillWave<D>& w, PrefillPair<D>& buf, int pr) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  const int pa = clamp_pid(w, 2 * pr);
  const int pb = clamp_pid(w, min(2 * pr + 1, w.key_pages - 1));   // a missing page re-reads the first
  const uint16_t* ka = w.ktile + (size_t)pa * w.page_elems + w.koff;
  const uint16_t* kb = w.ktile + (size_t)pb * w.page_elems + w.koff;
  const uint16_t* va = w.vtile + (size_t)pa * w.page_elems + w.voff;
  const uint16_t* vb = w.vtile + (size_t)pb * w.page_elems + w.voff;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    buf.k[0][kk] = *(const u32x4*)(ka + 32 * kk);
    buf.k[1][kk] = *(const u32x4*)(kb + 32 * kk);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const u32x2 lo = *(const u32x2*)(va + mt * 16 * kPage);
    const u32x2 hi = *(const u32x2*)(vb + mt * 16 * kPage);
    buf.v[mt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int D>
__device__ __forceinline__ void prefill_compute(const PrefillWave<D>& w, PrefillPair<D>& buf, int pr,
                                                SoftmaxState<D>& st, int grp) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  f32x4 sc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    sc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf.k[j][kk]), w.qf[kk], sc[j], 0, 0, 0);
  }
  // element e = 4 j + i is key position 32 pr + 16 j + 4 grp + i
  const int key0 = 32 * pr + 4 * grp;
  float sv[8];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = sc[j][i] * w.sl2;
      x = (key0 + 16 * j + i <= w.pos) ? x : -INFINITY;
      sv[4 * j + i] = x;
      mx = fmaxf(mx, x);
    }
  mx = xor_max(mx, 16);
  mx = xor_max(mx, 32);
  const float m_new = fmaxf(st.m, mx);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  float psum = 0.f;
  bf16x8 ph, pl;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = __builtin_amdgcn_exp2f(sv[e] - m_new);
    psum += p;
    const __bf16 hi = (__bf16)p;
    ph[e] = hi;
    pl[e] = (__bf16)(p - (float)hi);
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) st.acc[mt] *= alpha;
  }
  // keys past the wave's last position may be unwritten (NaN): zero their V
  // (dword w holds keys 2w, 2w+1 of the lane's 8: page w / 2, slots 4 grp + 2 (w % 2))
  if (32 * pr + 32 > w.last_pos + 1) {
    uint32_t keep[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k0 = key0 + 16 * (q >> 1) + 2 * (q & 1);
      keep[q] = (k0 <= w.last_pos ? 0x0000FFFFu : 0u) | (k0 + 1 <= w.last_pos ? 0xFFFF0000u : 0u);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) buf.v[mt][q] &= keep[q];
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    st.acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf.v[mt]), ph, st.acc[mt], 0, 0, 0);
    st.acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf.v[mt]), pl, st.acc[mt], 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// All pairs 0 .. npairs-1 of one wave, the next pair's loads in flight while
// the current one computes (two register buffers, exact peeled loop).
template <int D>
__device__ __forceinline__ void prefill_stream(const PrefillWave<D>& w, int npairs, SoftmaxState<D>& st,
                                               int grp) {
  const int n = __builtin_amdgcn_readfirstlane(npairs);
  if (n <= 0) return;
  PrefillPair<D> b0, b1;
  prefill_issue(w, b0, 0);
  int it = 0;
  for (; it + 2 < n; it += 2) {
    prefill_issue(w, b1, it + 1);
    prefill_compute(w, b0, it, st, grp);
    prefill_issue(w, b0, it + 2);
    prefill_compute(w, b1, it + 1, st, grp);
  }
  if (it + 1 < n) {
    prefill_issue(w, b1, it + 1);
    prefill_compute(w, b0, it, st, grp);
    prefill_compute(w, b1, it + 1, st, grp);
  } else {
    prefill_compute(w, b0, it, st, grp);
  }
}

// Grid: (KV head fastest, then sequence, then row block from the last one
// down, so the blocks that see the most keys start first).
template <int D>
__global__ __launch_bounds__(256, occupancy(D)) void prefill_kernel(PrefillArgs a) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int grp = lane >> 4;
  const int kvh = blockIdx.x % a.num_kv_heads;
  const int rest = blockIdx.x / a.num_kv_heads;
  const int b = rest % a.num_seqs;
  const int rb = a.row_blocks - 1 - rest / a.num_seqs;
  const int G = a.group;
  const Chunk ch = load_chunk(a.query_start, a.ctx_before, b, a.num_rows, a.max_chunk, a.stride);
  const int rows = ch.n * G;
  const int rho0 = rb * 64 + wave * 16;        // the wave's first row
  if (rho0 >= rows) return;
  const int rho_last = min(rho0 + 15, rows - 1);
  const int rho = rho0 + r;
  const bool valid = rho < rows;
  const int t = (valid ? rho : rho_last) / G;  // chunk token of this lane's row
  const int h = (valid ? rho : rho_last) - t * G;

  PrefillWave<D> w;
  w.last_pos = ch.c + rho_last / G;
  w.pos = ch.c + t;
  w.key_pages = (w.last_pos + kPage) / kPage;
  w.num_pages = a.num_pages;
  w.bt_row = a.block_tables + (size_t)b * a.stride;
  w.page_elems = (size_t)a.num_kv_heads * kPage * D;
  w.ktile = a.kpool + (size_t)kvh * kPage * D;
  w.vtile = a.vpool + (size_t)kvh * kPage * D;
  w.koff = (uint32_t)(r * D + 8 * grp);
  w.voff = (uint32_t)(r * kPage + 4 * grp);
  w.sl2 = a.scale_log2;
  const size_t qrow = ((size_t)(ch.r0 + t) * a.num_q_heads + (size_t)kvh * G + h) * D;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    w.qf[kk] = as_bf16x8(valid ? *(const u32x4*)(a.q + qrow + 32 * kk + 8 * grp) : u32x4{0u, 0u, 0u, 0u});

  SoftmaxState<D> st;
  init_state(st);
  prefill_stream(w, (w.key_pages + 1) >> 1, st, grp);
  st.l += __shfl_xor(st.l, 16, 64);
  st.l += __shfl_xor(st.l, 32, 64);
  if (valid) {
    const float inv = 1.f / st.l;
    float* o = a.out + qrow + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *(f32x4*)(o + 16 * mt) = st.acc[mt] * inv;
  }
}

}  // namespace pakv
