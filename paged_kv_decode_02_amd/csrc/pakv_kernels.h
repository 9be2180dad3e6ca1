// pakv_kernels.h - gfx950 device code of libpakv (included by pakv.hip only).
//
// Decode attention over paged BF16 K/V (one shared pool, 16-token pages, one
// block table per sequence and layer, pages read where they lie, FP32 online
// softmax: "Curso gratuito recorre la inferencia de LLM ..." (news-factory.app),
// section "¿Cómo administra el motor la memoria de la caché KV?"), with
// contiguous grouped-query heads ("Construye tu propio motor de inferencia LLM
// ..." (aibit.im), section "Atención de Consulta Agrupada (GQA)").
//
// Work decomposition. A context is cut into splits of SPLIT_PAGES pages (a
// fixed count per head_dim). One workgroup of W wavefronts handles one
// (split, sequence, KV head); wave w takes page pairs w, w + W, ... of the
// split. Per page pair (32 tokens) a wave does:
//
//   QK^T on the matrix cores, v_mfma_f32_16x16x32_bf16 with
//     A = 16 key rows (tokens) x 32 head dims, B = 32 head dims x 16 columns
//     (the G query heads of the group, zero-padded to 16), so
//     S^T[token][head] lands with head = lane % 16 in every lane;
//   the FP32 online-softmax update for that head, lane-locally plus two
//     cross-lane max steps (lanes 16 and 32 apart hold the same head);
//   PV on the matrix cores with A = V^T (16 head dims x 32 tokens, straight
//     from the slot-minor V page layout) and B = P^T (32 tokens x 16 heads).
//     P (FP32) is split as hi = bf16(p), lo = bf16(p - hi) and both halves go
//     through the MFMA, so the weights keep ~16 significant bits.
//
// Every K/V byte is loaded once, 16 bytes per lane per load, straight into the
// registers of its MFMA operand, with the nontemporal (streaming) hint where
// it measured faster; the next pair's loads are issued before the current
// pair is computed. Waves merge (m, l, acc) through LDS; a split that
// is not alone writes its partial to the workspace and merge_splits combines
// the splits of a sequence by log-sum-exp in split order.
//
// Lane roles (lane = 0..63, r = lane % 16, grp = lane / 16):
//   QK A operand   row r = token: page (r / 8) of the pair,
//                  slot 8 * ((r / 4) % 2) + 4 * j + r % 4 for MFMA j = 0, 1;
//                  k = head dims 8 * grp + 32 * kk + 0..7 (K slab kk: one
//                  load instruction fills 8 whole 128-byte lines)
//   QK result      lane holds S for head r, tokens 8 * grp + 4 * j + i
//   PV B operand   same lane, same 8 tokens (k = 8 * grp + e)
//   PV A operand   row = head dim 16 * mt + r, tokens 8 * grp + 0..7 ->
//                  page grp / 2, slots 8 * (grp % 2) + 0..7 (16 contiguous bytes)
//   PV result      lane holds acc for head r, dims 16 * mt + 4 * grp + i
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pakv {

constexpr int kPage = 16;

// Offset of element (slot t, dim e) inside one (page, KV head) K tile: the
// dims come in slabs of 32, each holding 64 bytes of all 16 slots, so the
// pieces one matrix-core K-step reads from 16 tokens are whole cache lines.
__host__ __device__ constexpr int k_offset(int t, int e) {
  return (e >> 5) * (kPage * 32) + t * 32 + (e & 31);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DecodeArgs {
  const uint16_t* kpool;
  const uint16_t* vpool;
  const uint16_t* q;
  const int32_t* block_tables;
  const int32_t* ctx;
  float* out;
  float* ws_acc;      // [B][Hq][S_max][D] unnormalised partial outputs
  float* ws_ml;       // [B][Hq][S_max][2] (running max in log2 units, sum)
  int32_t num_pages;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t stride;     // max_pages_per_seq
  int32_t s_max;      // splits per sequence the grid covers
  float scale_log2;   // scale * log2(e)
  // fused append (all NULL for a plain decode): the new token's K/V rows
  // [B][Hkv][D] and their positions [B]
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* positions;
  // optional launch plan: workgroup (item, KV head) takes the split
  // plan[item] = b | s << 20; NULL = every (sequence, split) in split-major order
  const int32_t* plan;
};

struct AppendArgs {
  uint16_t* kpool;
  uint16_t* vpool;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* block_tables;
  const int32_t* positions;
  int32_t num_pages;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t stride;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

__device__ __forceinline__ int clamp_ctx(int n, int stride) {
  return n < 0 ? 0 : (n > stride * kPage ? stride * kPage : n);
}

// K/V pages are read once per launch: they are loaded with the nontemporal
// hint (streaming cache policy), measured faster for d = 64 (K and V) and for
// the V tiles of d = 128; the d = 128 K tiles measured no faster with it
// (slightly slower), so they keep the default policy.
template <int D>
__host__ __device__ constexpr bool nt_k() { return D == 64; }
template <int D>
__host__ __device__ constexpr bool nt_v() { return true; }

// Head dims held by lane group grp for QK k-step kk (8 consecutive dims):
// k-step kk covers K slab kk. The keys (A operand), the query (B operand),
// the fused append and the prefill use it.
template <int D>
__host__ __device__ constexpr int kdim(int grp, int kk) { return 8 * grp + 32 * kk; }

template <bool NT>
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int D>
struct PairBuf {
  u32x4 k[2][D / 32];   // QK A operands: MFMA j, k-step kk
  u32x4 v[D / 16];      // PV A operands: dim tile mt
};

// ---------------------------------------------------------------- decode
// Per-lane constants for streaming one split of one (sequence, KV head).
template <int D>
struct SplitCtx {
  const uint16_t* kbase;   // K pool + KV head tile + this lane's offset
  const uint16_t* vbase;   // V pool + KV head tile + this lane's offset
  size_t page_elems;       // elements per physical page in each pool
  int my_pid;              // lane i: physical page of the split's logical page i
  int npages;              // pages in this split
  int pair_tok0;           // first token of the split
  int tok1;                // one past the split's last token
  bool k_second;           // this lane's K row lies in the pair's second page
  bool v_second;           // this lane's V tokens lie in the pair's second page
  float sl2;               // softmax scale * log2(e)
  bf16x8 qf[D / 32];       // query group, MFMA B operand
};

// Running softmax state of one wave: head = lane % 16.
template <int D>
struct SoftmaxState {
  float m;                 // running max (log2 units), same in the 4 lanes of a head
  float l;                 // this lane's share of the running sum
  f32x4 acc[D / 16];       // unnormalised output, dims 16 * mt + 4 * grp + i
};

template <int D>
__device__ __forceinline__ void issue_pair(const SplitCtx<D>& c, PairBuf<D>& buf, int pr) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  const int pa = __builtin_amdgcn_readlane(c.my_pid, 2 * pr);
  const int pb = __builtin_amdgcn_readlane(c.my_pid, min(2 * pr + 1, c.npages - 1));  // a missing second page re-reads the first (all masked)
  const uint16_t* kp = c.kbase + (size_t)(c.k_second ? pb : pa) * c.page_elems;
  const uint16_t* vp = c.vbase + (size_t)(c.v_second ? pb : pa) * c.page_elems;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) buf.k[j][kk] = ld_stream<nt_k<D>()>((const u32x4*)(kp + k_offset(4 * j, kdim<D>(0, kk))));
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) buf.v[mt] = ld_stream<nt_v<D>()>((const u32x4*)(vp + mt * 16 * kPage));
  // keep later pairs' loads and this pair's math in program order, so the
  // registers in use are the buffers as written
  __builtin_amdgcn_sched_barrier(0);
}

template <int D>
__device__ __forceinline__ void compute_pair(const SplitCtx<D>& c, PairBuf<D>& buf, int pr,
                                             SoftmaxState<D>& st, int grp) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  const int pair_tok = c.pair_tok0 + 2 * kPage * pr;
  f32x4 sc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    sc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf.k[j][kk]), c.qf[kk], sc[j], 0, 0, 0);
  }
  // scores in log2 units; tokens past the split end are masked by select
  const int t_lane = pair_tok + 8 * grp;
  float sv[8];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = sc[j][i] * c.sl2;
      x = (t_lane + 4 * j + i < c.tok1) ? x : -INFINITY;
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
  if (__ballot(alpha != 1.f)) {   // skip the rescale when no head's max moved
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) st.acc[mt] *= alpha;
  }
  // tail pair: zero V of masked tokens (0 * NaN would poison the product)
  if (pair_tok + 2 * kPage > c.tok1) {
    int cnt = c.tok1 - t_lane;
    cnt = cnt < 0 ? 0 : (cnt > 8 ? 8 : cnt);
    uint32_t keep[4];
#pragma unroll
    for (int w = 0; w < 4; ++w)
      keep[w] = (2 * w < cnt ? 0x0000FFFFu : 0u) | (2 * w + 1 < cnt ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int w = 0; w < 4; ++w) buf.v[mt][w] &= keep[w];
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    st.acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf.v[mt]), ph, st.acc[mt], 0, 0, 0);
    st.acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf.v[mt]), pl, st.acc[mt], 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Stream pairs first, first + step, ... (< npairs) of a split into st. The
// next pair's loads are in flight while the current one is computed (two
// register buffers). The steady-state loop issues unconditionally and the last
// one or two pairs are peeled, so every wait for loaded data counts exactly
// the loads issued after it and never waits for the prefetch.
template <int D>
__device__ __forceinline__ void stream_pairs(const SplitCtx<D>& c, int first, int step, int npairs,
                                             SoftmaxState<D>& st, int grp) {
  const int my_n = first < npairs ? (npairs - first + step - 1) / step : 0;
  if (my_n <= 0) return;
  PairBuf<D> b0, b1;
  issue_pair(c, b0, first);
  int it = 0;
  for (; it + 2 < my_n; it += 2) {
    issue_pair(c, b1, first + (it + 1) * step);
    compute_pair(c, b0, first + it * step, st, grp);
    issue_pair(c, b0, first + (it + 2) * step);
    compute_pair(c, b1, first + (it + 1) * step, st, grp);
  }
  if (it + 1 < my_n) {
    issue_pair(c, b1, first + (it + 1) * step);
    compute_pair(c, b0, first + it * step, st, grp);
    compute_pair(c, b1, first + (it + 1) * step, st, grp);
  } else {
    compute_pair(c, b0, first + it * step, st, grp);
  }
}

// Lane i's raw block-table entry for logical page s * SPLIT_PAGES + i (0 past
// the row). Needs no context length, so it is loaded alongside it.
template <int SPLIT_PAGES>
__device__ __forceinline__ int load_split_pages(const DecodeArgs& a, int b, int s, int lane) {
  const int p = s * SPLIT_PAGES + lane;
  return (lane < SPLIT_PAGES && p < a.stride) ? a.block_tables[(size_t)b * a.stride + p] : 0;
}

template <int D, int SPLIT_PAGES>
__device__ __forceinline__ void make_split_ctx(const DecodeArgs& a, int b, int kvh, int s, int n,
                                               int lane, int raw_pid, SplitCtx<D>& c) {
  constexpr int KK = D / 32;
  constexpr int TILE = kPage * D;
  constexpr int SPLIT_TOK = SPLIT_PAGES * kPage;
  const int r = lane & 15;
  const int grp = lane >> 4;
  const int G = a.group;
  const int tok0 = s * SPLIT_TOK;
  c.tok1 = min(tok0 + SPLIT_TOK, n);
  c.pair_tok0 = tok0;
  const int p0 = tok0 / kPage;
  c.npages = (c.tok1 - tok0 + kPage - 1) / kPage;
  // this split's physical page ids, one per lane, clamped into the pool
  (void)p0;
  c.my_pid = lane < c.npages ? (raw_pid < 0 ? 0 : (raw_pid >= a.num_pages ? a.num_pages - 1 : raw_pid)) : 0;
  // query group as the MFMA B operand (columns = heads, zero past G)
  if (r < G) {
    const uint16_t* qp = a.q + ((size_t)b * a.num_q_heads + (size_t)kvh * G + r) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) c.qf[kk] = as_bf16x8(*(const u32x4*)(qp + kdim<D>(grp, kk)));
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) c.qf[kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  c.page_elems = (size_t)a.num_kv_heads * TILE;
  const int koff = k_offset(8 * ((r >> 2) & 1) + (r & 3), kdim<D>(grp, 0));
  const int voff = r * kPage + 8 * (grp & 1);
  c.k_second = (r >> 3) != 0;
  c.v_second = (grp >> 1) != 0;
  c.kbase = a.kpool + (size_t)kvh * TILE + koff;
  c.vbase = a.vpool + (size_t)kvh * TILE + voff;
  c.sl2 = a.scale_log2;
}

template <int D>
__device__ __forceinline__ void init_state(SoftmaxState<D>& st) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) st.acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Write one V column (the D values of one token) into a slot-minor V tile by
// rewriting whole 32-byte slot rows: lane i handles rows i, i + 64, ...
template <int D>
__device__ __forceinline__ void write_v_column(uint16_t* vtile, const uint16_t* vn, int slot, int lane) {
  const int w = (slot & 7) >> 1;
  const int half = slot >> 3;
  const uint32_t sh = (slot & 1) * 16;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const int dd = lane + 64 * i;
    u32x4* row = (u32x4*)(vtile + (size_t)dd * kPage);
    u32x4 h0 = row[0];
    u32x4 h1 = row[1];
    const uint32_t nv = vn[dd];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t upd0 = (h0[e] & ~(0xFFFFu << sh)) | (nv << sh);
      const uint32_t upd1 = (h1[e] & ~(0xFFFFu << sh)) | (nv << sh);
      h0[e] = (half == 0 && e == w) ? upd0 : h0[e];
      h1[e] = (half == 1 && e == w) ? upd1 : h1[e];
    }
    row[0] = h0;
    row[1] = h1;
  }
}

// Fused append of a position the decode does not attend over (at or past the
// context length): plain stores by wave 0 of the workgroup of the split the
// position falls in; nothing in this launch reads that slot.
template <int D>
__device__ __forceinline__ void append_unattended(const DecodeArgs& a, int b, int kvh, int pos,
                                                  int lane) {
  const int pid = a.block_tables[(size_t)b * a.stride + pos / kPage];
  if (pid < 0 || pid >= a.num_pages) return;
  const int slot = pos % kPage;
  const size_t tile = (size_t)pid * a.num_kv_heads + kvh;
  const uint16_t* kn = a.k_new + ((size_t)b * a.num_kv_heads + kvh) * D;
  const uint16_t* vn = a.v_new + ((size_t)b * a.num_kv_heads + kvh) * D;
  uint16_t* ktile = const_cast<uint16_t*>(a.kpool) + tile * kPage * D;
  uint16_t* vdst = const_cast<uint16_t*>(a.vpool) + tile * D * kPage + slot;
  if (lane < D / 8) *(u32x4*)(ktile + k_offset(slot, 8 * lane)) = *(const u32x4*)(kn + 8 * lane);
  write_v_column<D>(vdst - slot, vn, slot, lane);
}

// Fused append of an attended position, by the wave that will read its page
// pair: every lane stores exactly the bytes of the new token that it loads
// itself later (its chunks of the K row, its elements of the V column), so
// program order within the lane makes its own later loads return them. No
// other lane, wave or workgroup reads that slot in this launch, so no fence
// or barrier is needed. pid is the token's page, p_in_pair 0/1 its page
// within the pair, slot its slot.
template <int D>
__device__ __forceinline__ void append_by_reader(const DecodeArgs& a, int b, int kvh, int pid,
                                                 int p_in_pair, int slot, int lane) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  const int r = lane & 15;
  const int grp = lane >> 4;
  const size_t tile = (size_t)pid * a.num_kv_heads + kvh;
  const uint16_t* kn = a.k_new + ((size_t)b * a.num_kv_heads + kvh) * D;
  const uint16_t* vn = a.v_new + ((size_t)b * a.num_kv_heads + kvh) * D;
  // K: the QK row of this token is r = 8 * page-in-pair + 4 * (slot / 8) + slot % 4
  if (r == 8 * p_in_pair + 4 * (slot >> 3) + (slot & 3)) {
    uint16_t* ktile = const_cast<uint16_t*>(a.kpool) + tile * kPage * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      *(u32x4*)(ktile + k_offset(slot, kdim<D>(grp, kk))) = *(const u32x4*)(kn + kdim<D>(grp, kk));
  }
  // V: the two lane groups 2 * page-in-pair and 2 * page-in-pair + 1 load the
  // two 16-byte halves of every 32-byte slot row of this page. They read their
  // halves, put v_new into the token's element and write the halves back, so
  // each row is written whole (a lone 2-byte write would make the memory side
  // read-modify-write the sector).
  if ((grp >> 1) == p_in_pair) {
    const bool mine = (grp & 1) == (slot >> 3);
    const int w = (slot & 7) >> 1;
    const uint32_t sh = (slot & 1) * 16;
    uint16_t* vrow = const_cast<uint16_t*>(a.vpool) + tile * D * kPage + r * kPage + 8 * (grp & 1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      u32x4 h = *(const u32x4*)(vrow + mt * 16 * kPage);
      const uint32_t nv = vn[16 * mt + r];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (mine && e == w) h[e] = (h[e] & ~(0xFFFFu << sh)) | (nv << sh);
      *(u32x4*)(vrow + mt * 16 * kPage) = h;
    }
  }
}

// Waves per SIMD the register budget must allow (512 registers per lane).
__host__ __device__ constexpr int occupancy(int d) { return d == 64 ? 4 : 2; }

// Decode: one workgroup of W waves per (split, sequence, KV head); wave w
// takes pairs w, w + W, ...; the waves merge through LDS. With FUSED the
// launch also appends each sequence's new token (pa_decode_append).

template <int D, int W, int SPLIT_PAGES, bool FUSED>
__global__ __launch_bounds__(64 * W, occupancy(D)) void decode_split_kernel(DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(SPLIT_PAGES % 2 == 0 && SPLIT_PAGES <= 64, "split pages: even, at most one per lane");
  constexpr int MT = D / 16;
  constexpr int SPLIT_TOK = SPLIT_PAGES * kPage;
  constexpr int LDS_ROW = D + 4;
  extern __shared__ float smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int grp = lane >> 4;
  const int wg = blockIdx.x;
  const int kvh = wg % a.num_kv_heads;
  const int rest = wg / a.num_kv_heads;
  int b, s;
  if (a.plan) {
    const uint32_t item = (uint32_t)a.plan[rest];
    b = (int)(item & 0xFFFFFu);
    s = (int)(item >> 20);
    if (b >= a.num_seqs || s >= a.s_max) return;
  } else {
    b = rest % a.num_seqs;
    s = rest / a.num_seqs;
  }
  const int G = a.group;

  // the independent loads of the prologue are issued together
  int pos = FUSED ? a.positions[b] : -1;
  const int raw_pid = load_split_pages<SPLIT_PAGES>(a, b, s, lane);
  const int ctx_b = a.ctx[b];
  const int n = clamp_ctx(ctx_b, a.stride);
  if (FUSED && pos >= 0 && pos < a.stride * kPage && pos / SPLIT_TOK == s) {
    if (pos >= n) {
      if (wave == 0) append_unattended<D>(a, b, kvh, pos, lane);
    } else {
      const int lp = pos / kPage - s * SPLIT_PAGES;          // page within this split
      if (wave == (lp >> 1) % W) {                           // the wave reading its pair
        const int v = __builtin_amdgcn_readlane(raw_pid, lp);
        if (v >= 0 && v < a.num_pages) append_by_reader<D>(a, b, kvh, v, lp & 1, pos % kPage, lane);
      }
    }
  }
  if (n == 0) {
    if (s == 0) {
      float* o = a.out + ((size_t)b * a.num_q_heads + (size_t)kvh * G) * D;
      for (int e = threadIdx.x; e < G * D; e += 64 * W) o[e] = 0.f;
    }
    return;
  }
  const int nsplit = (n + SPLIT_TOK - 1) / SPLIT_TOK;
  if (s >= nsplit) return;

  SplitCtx<D> c;
  make_split_ctx<D, SPLIT_PAGES>(a, b, kvh, s, n, lane, raw_pid, c);
  SoftmaxState<D> st;
  init_state(st);
  stream_pairs(c, wave, W, (c.npages + 1) >> 1, st, grp);
  st.l += __shfl_xor(st.l, 16, 64);
  st.l += __shfl_xor(st.l, 32, 64);

  float* sm_m = smem;
  float* sm_l = smem + W * 16;
  float* sm_acc = smem + 2 * W * 16;
  if (grp == 0) {
    sm_m[wave * 16 + r] = st.m;
    sm_l[wave * 16 + r] = st.l;
  }
  if (r < G) {
    float* dst = sm_acc + (size_t)(wave * G + r) * LDS_ROW + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *(f32x4*)(dst + 16 * mt) = st.acc[mt];
  }
  // LDS-only fences: the barrier must not wait for global stores in flight
  // (a fused append's pool writes)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  const bool alone = nsplit == 1;
  const size_t head0 = (size_t)b * a.num_q_heads + (size_t)kvh * G;
  for (int e = threadIdx.x; e < G * D; e += 64 * W) {
    const int hh = e / D;
    const int dd = e - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w * 16 + hh]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float cw = __builtin_amdgcn_exp2f(sm_m[w * 16 + hh] - M);
      L += cw * sm_l[w * 16 + hh];
      A += cw * sm_acc[(size_t)(w * G + hh) * LDS_ROW + dd];
    }
    if (alone) {
      a.out[(head0 + hh) * D + dd] = A / L;
    } else {
      const size_t slot = (head0 + hh) * a.s_max + s;
      a.ws_acc[slot * D + dd] = A;
      if (dd == 0) {
        a.ws_ml[slot * 2] = M;
        a.ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// One wave per (sequence, query head): combine the splits of sequences that
// have more than one, in split order. Lane i holds split i's (m, l); they are
// loaded together with the context length, so the partial outputs (read four
// splits at a time) are two dependent loads away from the start.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void merge_splits_kernel(DecodeArgs a, int split_tokens) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.num_seqs * a.num_q_heads) return;
  const int b = item / a.num_q_heads;
  const float* ml = a.ws_ml + (size_t)item * a.s_max * 2;
  const float* acc = a.ws_acc + (size_t)item * a.s_max * D;
  // the context length and the first 64 splits' (m, l) are loaded together;
  // lanes past the sequence's split count drop theirs
  const int ctx_b = a.ctx[b];
  float m0 = -INFINITY, l0 = 0.f;
  if (lane < a.s_max) {
    m0 = ml[2 * lane];
    l0 = ml[2 * lane + 1];
  }
  const int n = clamp_ctx(ctx_b, a.stride);
  const int nsplit = (n + split_tokens - 1) / split_tokens;
  if (nsplit <= 1) return;
  float M = lane < nsplit ? m0 : -INFINITY;
  for (int s0 = 64; s0 < nsplit; s0 += 64)
    if (s0 + lane < nsplit) M = fmaxf(M, ml[2 * (s0 + lane)]);
  M = wave_max(M);
  float L = 0.f;
  float A[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) A[i] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int cnt = min(64, nsplit - s0);
    float c = 0.f;
    if (lane < cnt) {
      const float mm = s0 == 0 ? m0 : ml[2 * (s0 + lane)];
      const float ll = s0 == 0 ? l0 : ml[2 * (s0 + lane) + 1];
      c = __builtin_amdgcn_exp2f(mm - M);
      L += c * ll;
    }
    int j = 0;
    for (; j + 4 <= cnt; j += 4) {
      float v[4][PER];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < PER; ++i) v[u][i] = acc[(size_t)(s0 + j + u) * D + lane + 64 * i];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float cu = __shfl(c, j + u, 64);
#pragma unroll
        for (int i = 0; i < PER; ++i) A[i] += cu * v[u][i];
      }
    }
    for (; j < cnt; ++j) {
      const float cu = __shfl(c, j, 64);
#pragma unroll
      for (int i = 0; i < PER; ++i) A[i] += cu * acc[(size_t)(s0 + j) * D + lane + 64 * i];
    }
  }
  L = wave_sum(L);
  const float inv = 1.f / L;
  float* o = a.out + (size_t)item * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[lane + 64 * i] = A[i] * inv;
}

// ---------------------------------------------------------------- append
// One 256-thread block per sequence: a bit copy of the new token's K row
// (16-byte chunks, each to its slab of the K tile) and of its V values into
// the slot-minor V layout, each V slot row (32 bytes) read, patched and
// written whole.
template <int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int t = threadIdx.x;
  const int b = blockIdx.x;
  const int pos = a.positions[b];
  if (pos < 0 || pos >= a.stride * kPage) return;
  const int pid = a.block_tables[(size_t)b * a.stride + pos / kPage];
  if (pid < 0 || pid >= a.num_pages) return;
  const int slot = pos % kPage;
  const int H = a.num_kv_heads;
  const size_t tile0 = (size_t)pid * H;
  const uint16_t* kn = a.k_new + (size_t)b * H * D;
  const uint16_t* vn = a.v_new + (size_t)b * H * D;
  for (int c = t; c < H * (D / 8); c += 256) {
    const int g = c / (D / 8);
    const int part = c - g * (D / 8);
    *(u32x4*)(a.kpool + (tile0 + g) * kPage * D + k_offset(slot, 8 * part)) =
        *(const u32x4*)(kn + (size_t)g * D + 8 * part);
  }
  const int w = (slot & 7) >> 1;
  const int half = slot >> 3;
  const uint32_t sh = (slot & 1) * 16;
  for (int e = t; e < H * D; e += 256) {     // row e = (kv head, dim)
    u32x4* row = (u32x4*)(a.vpool + (tile0 * D + e) * kPage);
    u32x4 h0 = row[0];
    u32x4 h1 = row[1];
    const uint32_t nv = vn[e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t upd0 = (h0[i] & ~(0xFFFFu << sh)) | (nv << sh);
      const uint32_t upd1 = (h1[i] & ~(0xFFFFu << sh)) | (nv << sh);
      h0[i] = (half == 0 && i == w) ? upd0 : h0[i];
      h1[i] = (half == 1 && i == w) ? upd1 : h1[i];
    }
    row[0] = h0;
    row[1] = h1;
  }
}

// ------------------------------------------------------- read ceiling
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* sink) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t x = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace pakv
