// pakv_kernels.h - gfx950 device code of libpakv (included by pakv.hip only).
//
// Decode attention over paged BF16 K/V (one shared pool, 16-token pages, one
// block table per sequence and layer, pages read where they lie, FP32 online
// softmax: "Curso gratuito recorre la inferencia de LLM ..." (news-factory.app),
// section "¿Cómo administra el motor la memoria de la caché KV?"), with
// contiguous grouped-query heads ("Construye tu propio motor de inferencia LLM
// ..." (aibit.im), section "Atención de Consulta Agrupada (GQA)").
//
// Reduction structure (fixed per head_dim, so a sequence's result never
// depends on the rest of the batch). A context is cut into splits of
// SPLIT_PAGES pages. Inside a split, logical wave lw (0 <= lw < W) streams
// page pairs lw, lw + W, lw + 2 W, ... with its own online-softmax state; the
// W partial states of a split are merged in logical-wave order, and the
// splits of a sequence by log-sum-exp in split order.
//
// Work decomposition. One workgroup of W wavefronts takes one work item: up
// to four units of one KV head, a unit being one split of one sequence.
// Physical wave p runs logical wave (p - rot_u) mod W of every unit u in
// turn, so that the pairs of all the item's units are dealt round-robin over
// the W waves (rot_u, from the launch plan, is the running count of pairs
// before unit u, mod W) and every wave gets the same count to within one.
// A wave's pairs form one stream: the next pair is always in flight while
// the current one is computed, across unit boundaries too. At a unit's end
// the wave parks its partial state in LDS. When every wave is done, the
// workgroup merges each unit's W partials; a sequence whose splits all lie
// in the item (at most four; two when G > 8) is finished in LDS, by the
// same log-sum-exp code the merge kernel runs for longer sequences, whose
// split partials go to the workspace.
//
// Per page pair (32 tokens), per wave:
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
// it measured faster.
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

// Decode geometry per head_dim: pages per split and waves per workgroup
// (= logical waves per split). Both give at most 4 page pairs per logical
// wave of a full split.
template <int D> struct DecodeGeom;
template <> struct DecodeGeom<64> {
  static constexpr int W = 16;
  static constexpr int SPLIT_PAGES = 128;
};
template <> struct DecodeGeom<128> {
  static constexpr int W = 8;
  static constexpr int SPLIT_PAGES = 64;
};

constexpr int kItemUnits = 4;   // units a work item can name
constexpr int kItemInts = 8;    // int32 words per plan item: 4 units, the rotations, the next item, 2 unused
constexpr int kMaxPairsPerUnit = 4;
// Units a workgroup can finish together: the LDS holds the partials of
// (units x G) <= 32 query-head rows per wave.
__host__ __device__ constexpr int units_cap(int group) { return group <= 8 ? 4 : 2; }

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
  int32_t ucap;       // units_cap(group)
  int32_t num_items;  // work items the plan lists (or the grid covers, without one)
  int32_t num_bins;   // workgroups per KV head: the grid's (y, z) extent
  float scale_log2;   // scale * log2(e)
  // optional launch plan: workgroup (bin, KV head) runs item bin, then the
  // chain of items each item names as its next. Item i runs the units of
  // plan[i * kItemInts + 0..3] (b | s << 20, or -1 for none) with the
  // rotations packed 4 bits per unit in plan[i * kItemInts + 4]; its
  // successor is plan[i * kItemInts + 5] (the chain ends at an index that is
  // not above i, or not in [num_bins, num_items)). NULL = one item per
  // workgroup: per sequence, its splits in consecutive groups of ucap.
  const int32_t* plan;
};

// A launch plan carried by value in the kernel's arguments (the runtime
// copies the arguments at launch, so the host array is free again when the
// call returns); NW words: NW / kItemInts items.
template <int NW>
struct InlinePlan {
  int32_t w[NW];
};
constexpr int kInlineSmall = 256;     // 32 items, 1 KiB of arguments
constexpr int kInlineLarge = 2048;    // 256 items, 8 KiB

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

// Cross-lane steps with gfx950's permlane swaps (VALU, no LDS round trip):
// a swap of a value with itself leaves, in every lane, the pair {own value,
// value of lane ^ 16} (permlane16) or {own, lane ^ 32} (permlane32), in one
// order or the other; max and sum of the pair are exact and order-free.
__device__ __forceinline__ float pair_max16(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_max32(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum16(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float pair_sum32(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
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
// k-step kk covers K slab kk. The keys (A operand), the query (B operand)
// and the prefill use it.
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
// Per-lane constants of one wave's stream. Every unit of a work item belongs
// to the same KV head, so the tile offsets are shared; the pair list is held
// one pair per lane and read with readlane.
template <int D>
struct StreamCtx {
  const uint16_t* kbase;   // K pool + KV head tile + this lane's offset
  const uint16_t* vbase;   // V pool + KV head tile + this lane's offset
  size_t page_elems;       // elements per physical page in each pool
  bool k_second;           // this lane's K row lies in the pair's second page
  bool v_second;           // this lane's V tokens lie in the pair's second page
  float sl2;               // softmax scale * log2(e)
  int pa;                  // lane i: physical page of the first page of the wave's pair i
  int pb;                  // lane i: of its second page (the first again when there is none)
  int ptu;                 // lane i: (first token of pair i) / 32, shifted left 2, | its unit
};

// Running softmax state of one wave: head = lane % 16.
template <int D>
struct SoftmaxState {
  float m;                 // running max (log2 units), same in the 4 lanes of a head
  float l;                 // this lane's share of the running sum
  f32x4 acc[D / 16];       // unnormalised output, dims 16 * mt + 4 * grp + i
};

template <int D>
__device__ __forceinline__ void init_state(SoftmaxState<D>& st) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) st.acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ int sel4(int i, int x0, int x1, int x2, int x3) {
  return i == 0 ? x0 : (i == 1 ? x1 : (i == 2 ? x2 : x3));
}

template <int D>
__device__ __forceinline__ void issue_pair(const StreamCtx<D>& c, PairBuf<D>& buf, int i) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  const int pa = __builtin_amdgcn_readlane(c.pa, i);
  const int pb = __builtin_amdgcn_readlane(c.pb, i);
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

// One page pair (tokens pair_tok .. pair_tok + 31; those at or past tok1 are
// masked) into the running state.
template <int D>
__device__ __forceinline__ void compute_pair(const bf16x8 (&qf)[D / 32], float sl2, int pair_tok, int tok1,
                                             PairBuf<D>& buf, SoftmaxState<D>& st, int grp) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  f32x4 sc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    sc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf.k[j][kk]), qf[kk], sc[j], 0, 0, 0);
  }
  // scores in log2 units; tokens past the split end are masked by select
  const int t_lane = pair_tok + 8 * grp;
  float sv[8];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = sc[j][i] * sl2;
      x = (t_lane + 4 * j + i < tok1) ? x : -INFINITY;
      sv[4 * j + i] = x;
      mx = fmaxf(mx, x);
    }
  mx = pair_max16(mx);   // the 4 lanes of a head: r, r + 16, r + 32, r + 48
  mx = pair_max32(mx);
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
  if (pair_tok + 2 * kPage > tok1) {
    int cnt = tok1 - t_lane;
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

// LDS of the decode workgroup, in floats: the item's query rows (BF16), then
// per (unit, logical wave) the partial max and sum of 16 heads, the partial
// accumulators of (unit, logical wave, head) rows, and the units' merged
// max and sum.
template <int D>
struct DecodeLds {
  static constexpr int W = DecodeGeom<D>::W;
  static constexpr int ROW = D + 4;                               // padded accumulator row
  static constexpr int Q = 0;                                     // BF16 query rows [unit][16][D]
  static constexpr int WM = Q + kItemUnits * 16 * D / 2;          // [unit][lw][16]
  static constexpr int WL = WM + kItemUnits * W * 16;
  static constexpr int ACC = WL + kItemUnits * W * 16;            // [(unit * W + lw) * G + head][ROW]
  static constexpr int UM = ACC + 32 * W * ROW;                   // [unit][16]
  static constexpr int UL = UM + kItemUnits * 16;
  static constexpr int TOTAL = UL + kItemUnits * 16;
};

// A wave's partial state of one unit (logical wave lw) into LDS slot
// (unit * W + lw).
template <int D>
__device__ __forceinline__ void park_partial(float* smem, int slot, int G, const SoftmaxState<D>& st, int r,
                                             int grp) {
  using L = DecodeLds<D>;
  float l = pair_sum16(st.l);
  l = pair_sum32(l);
  if (grp == 0) {
    smem[L::WM + slot * 16 + r] = st.m;
    smem[L::WL + slot * 16 + r] = l;
  }
  if (r < G) {
    float* dst = smem + L::ACC + (size_t)(slot * G + r) * L::ROW + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) *(f32x4*)(dst + 16 * mt) = st.acc[mt];
  }
}

template <int D>
__device__ __forceinline__ void load_query(const float* smem, int u, int G, int r, int grp, bf16x8 (&qf)[D / 32]) {
  const u32x4* sq = (const u32x4*)(smem + DecodeLds<D>::Q);
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    qf[kk] = r < G ? as_bf16x8(sq[(u * 16 + r) * (D / 8) + grp + 4 * kk]) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
}

// The wave's pairs 0 .. T-1 (of all units in turn; pair 0 already issued
// into b0). The next pair's loads are in flight while the current one is
// computed (two register buffers), also across a unit boundary; at a
// boundary the finished unit's state is parked in LDS. The steady-state loop issues unconditionally and the last one or
// two pairs are peeled, so a wait for loaded data never covers the prefetch.
template <int D>
__device__ __forceinline__ void stream_item(const StreamCtx<D>& c, int T, PairBuf<D>& b0, float* smem, int G,
                                            int r, int grp, int lw0, int lw1, int lw2, int lw3, int te0, int te1,
                                            int te2, int te3) {
  constexpr int W = DecodeGeom<D>::W;
  if (T <= 0) return;
  SoftmaxState<D> st;
  init_state(st);
  bf16x8 qf[D / 32];
  int cur = -1;
  int tok1 = 0;
  auto step = [&](PairBuf<D>& buf, int i) {
    const int tu = __builtin_amdgcn_readlane(c.ptu, i);
    const int u = tu & 3;
    if (u != cur) {
      if (cur >= 0) {
        park_partial<D>(smem, cur * W + sel4(cur, lw0, lw1, lw2, lw3), G, st, r, grp);
        init_state(st);
      }
      cur = u;
      load_query<D>(smem, u, G, r, grp, qf);
      tok1 = sel4(u, te0, te1, te2, te3);
    }
    compute_pair<D>(qf, c.sl2, (tu >> 2) << 5, tok1, buf, st, grp);
  };
  PairBuf<D> b1;   // pair 0 is already in flight in b0
  int it = 0;
  for (; it + 2 < T; it += 2) {
    issue_pair(c, b1, it + 1);
    step(b0, it);
    issue_pair(c, b0, it + 2);
    step(b1, it + 1);
  }
  if (it + 1 < T) {
    issue_pair(c, b1, it + 1);
    step(b0, it);
    step(b1, it + 1);
  } else {
    step(b0, it);
  }
  park_partial<D>(smem, cur * W + sel4(cur, lw0, lw1, lw2, lw3), G, st, r, grp);
}

// Max over lanes 0 .. N-1 of each row of 16 lanes (N = 8 or 16), in every
// one of those lanes: DPP quad swaps, then the half-row and row mirrors.
template <int N>
__device__ __forceinline__ float row_max(float v) {
  static_assert(N == 8 || N == 16, "row_max: 8 or 16 lanes");
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  if (N == 16) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

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

// Log-sum-exp merge of nsplit split partials of one (sequence, query head),
// in split order, by one wave: ml(s) gives split s's (max in log2 units, sum),
// acc(s, e) its unnormalised output element e. The decode workgroup (from
// LDS) and the merge kernel (from the workspace) run this same code.
template <int D, class ML, class ACC>
__device__ __forceinline__ void lse_merge(int nsplit, int lane, ML ml, ACC acc, float* o) {
  constexpr int PER = D / 64;
  float M = -INFINITY;
  for (int s0 = 0; s0 < nsplit; s0 += 64)
    if (s0 + lane < nsplit) M = fmaxf(M, ml(s0 + lane).x);
  M = wave_max(M);
  float L = 0.f;
  float A[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) A[i] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int cnt = min(64, nsplit - s0);
    float c = 0.f;
    if (lane < cnt) {
      const float2 v = ml(s0 + lane);
      c = __builtin_amdgcn_exp2f(v.x - M);
      L = __builtin_fmaf(c, v.y, L);
    }
#pragma unroll 4
    for (int j = 0; j < cnt; ++j) {
      const float cu = __shfl(c, j, 64);
#pragma unroll
      for (int i = 0; i < PER; ++i) A[i] = __builtin_fmaf(cu, acc(s0 + j, lane + 64 * i), A[i]);
    }
  }
  L = wave_sum(L);
  const float inv = 1.f / L;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[lane + 64 * i] = A[i] * inv;
}

// Waves per SIMD the register budget must allow (512 registers per lane).
__host__ __device__ constexpr int occupancy(int d) { return d == 64 ? 4 : 2; }

// One work item of KV head kvh: its units streamed by the workgroup's waves,
// their partials merged. Returns the index of the item the plan chains after
// it (-1 without a plan). Every wave of the workgroup takes the same path.
template <int D, int NW>
__device__ __forceinline__ int decode_item(const DecodeArgs& a, const InlinePlan<NW>& ip, int kvh, int tid,
                                           int item, float* smem) {
  constexpr int W = DecodeGeom<D>::W;
  constexpr int SP = DecodeGeom<D>::SPLIT_PAGES;
  constexpr int SPLIT_TOK = SP * kPage;
  constexpr int TILE = kPage * D;
  using L = DecodeLds<D>;
  constexpr bool kInline = NW > kItemInts;

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;
  const int grp = lane >> 4;
  const int Hkv = a.num_kv_heads;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int ucap = a.ucap;

  // the item's units (sequence -1: none) and their rotations. The variants
  // with an inline plan (NW > one item) read it from the kernel's arguments,
  // together with the other arguments, in the first round of loads.
  const int32_t* ctxp = a.ctx;
  const int32_t* btp = a.block_tables;
  const uint16_t* qp = a.q;
  const int num_seqs = a.num_seqs;
  const int s_max = a.s_max;
  const int stride = a.stride;
  int ub[kItemUnits], us[kItemUnits];
  int rot = 0;
  int next = -1;
  int prefetched = 0;
  if (kInline || a.plan) {
    int it[kItemUnits + 2];
    if (kInline) {
#pragma unroll
      for (int k = 0; k < kItemUnits + 2; ++k) it[k] = ip.w[item * kItemInts + k];
    } else {
      // the plan does not change during a launch: scalar loads through the
      // constant address space
      typedef __attribute__((address_space(4))) const int32_t cint;
      const cint* cplan = (const cint*)a.plan;
#pragma unroll
      for (int k = 0; k < kItemUnits + 2; ++k) it[k] = cplan[(size_t)item * kItemInts + k];
    }
    // every argument the next round of loads needs, in registers together
    asm volatile("" ::"s"(it[0]), "s"(it[1]), "s"(it[2]), "s"(it[3]), "s"(it[4]), "s"(it[5]), "s"(ctxp),
                 "s"(btp), "s"(qp), "s"(num_seqs), "s"(s_max), "s"(stride));
    next = it[kItemUnits + 1];
    if constexpr (!kInline) {
      // the chain's next record, touched now so that its load meets a warm
      // scalar cache when this item is done (consumed below, at the end)
      typedef __attribute__((address_space(4))) const int32_t cint;
      const cint* cplan = (const cint*)a.plan;
      prefetched = cplan[(size_t)min(max(next, 0), a.num_items - 1) * kItemInts];
    }
#pragma unroll
    for (int u = 0; u < kItemUnits; ++u) {
      const int e = it[u];
      const int b = e & 0xFFFFF;
      const int s = (int)((uint32_t)e >> 20);
      const bool ok = u < ucap && e >= 0 && b < num_seqs && s < s_max;
      ub[u] = ok ? b : -1;
      us[u] = ok ? s : 0;
    }
    rot = it[kItemUnits];
  } else {
    const int b = item % num_seqs;
    const int j = item / num_seqs;
#pragma unroll
    for (int u = 0; u < kItemUnits; ++u) {
      const int s = j * ucap + u;
      ub[u] = (u < ucap && s < s_max) ? b : -1;
      us[u] = s;
    }
  }
  if (ub[0] < 0 && ub[1] < 0 && ub[2] < 0 && ub[3] < 0) {
    asm volatile("" ::"s"(prefetched));
    return next;
  }

  // the second round, issued together and unconditionally (absent units read
  // sequence 0, whose row always exists, and are masked after): the context
  // lengths, this lane's block-table entry, this thread's query chunks
  int raw_n[kItemUnits];
  {
    // the context lengths do not change during a launch: scalar loads
    // through the constant address space
    typedef __attribute__((address_space(4))) const int32_t cint;
    const cint* cctx = (const cint*)ctxp;
#pragma unroll
    for (int u = 0; u < kItemUnits; ++u) raw_n[u] = cctx[max(ub[u], 0)];
  }
  // lane t < 32: page j = t % 2 of pair k = (t / 2) % 4 of unit t / 8
  const int tu = (lane >> 3) & 3;
  const int tk = (lane >> 1) & 3;
  const int tj = lane & 1;
  const int t_b = sel4(tu, ub[0], ub[1], ub[2], ub[3]);
  const int t_lw = (wave - ((rot >> (4 * tu)) & 15)) & (W - 1);
  const int t_pi = 2 * (t_lw + W * tk) + tj;                                 // page within the split
  const int t_lp = sel4(tu, us[0], us[1], us[2], us[3]) * SP + t_pi;        // logical page
  const bool t_ok = lane < 32 && t_b >= 0 && t_lp < stride;
  int raw = btp[t_ok ? (size_t)t_b * stride + t_lp : 0];
  // query rows: 16-byte chunk t = (unit * 16 + head) * (D / 8) + c of the
  // LDS copy, thread tid + i * 64 * W for i < QCH
  constexpr int QCHUNKS = kItemUnits * 16 * (D / 8);
  constexpr int QCH = (QCHUNKS + 64 * W - 1) / (64 * W);
  u32x4 qv[QCH];
  bool qok[QCH];
#pragma unroll
  for (int i = 0; i < QCH; ++i) {
    const int t = tid + i * 64 * W;
    const int u = (t / (16 * (D / 8))) & 3;
    const int h = (t / (D / 8)) & 15;
    const int ch = t % (D / 8);
    const int b = sel4(u, ub[0], ub[1], ub[2], ub[3]);
    qok[i] = t < QCHUNKS && b >= 0 && h < G;
    qv[i] = *(const u32x4*)(qp + ((size_t)(qok[i] ? b : 0) * Hq + (size_t)kvh * G + (qok[i] ? h : 0)) * D + 8 * ch);
  }
  raw &= -(int)t_ok;
  int n[kItemUnits];
#pragma unroll
  for (int u = 0; u < kItemUnits; ++u) n[u] = clamp_ctx(raw_n[u], stride) & -(int)(ub[u] >= 0);

  // per unit: tokens, pages, pairs; this wave's logical wave and its pairs
  int nsplit[kItemUnits], te[kItemUnits], np[kItemUnits], lw[kItemUnits], cnt[kItemUnits];
#pragma unroll
  for (int u = 0; u < kItemUnits; ++u) {
    nsplit[u] = (n[u] + SPLIT_TOK - 1) / SPLIT_TOK;
    const bool live = ub[u] >= 0 && us[u] < nsplit[u];
    const int tok0 = us[u] * SPLIT_TOK;
    te[u] = live ? min(tok0 + SPLIT_TOK, n[u]) : 0;
    np[u] = live ? (te[u] - tok0 + kPage - 1) / kPage : 0;
    const int npairs = (np[u] + 1) >> 1;
    lw[u] = (wave - ((rot >> (4 * u)) & 15)) & (W - 1);
    cnt[u] = npairs > lw[u] ? (npairs - lw[u] + W - 1) / W : 0;
  }
  // page ids: clamped into the pool; a pair's missing second page re-reads
  // its first (all its tokens are masked)
  int pid = raw < 0 ? 0 : (raw >= a.num_pages ? a.num_pages - 1 : raw);
  const int first = __shfl(pid, lane & ~1, 64);
  pid = t_pi < sel4(tu, np[0], np[1], np[2], np[3]) ? pid : first;
  // the wave's pairs in stream order: lane f holds pair f
  const int F1 = cnt[0], F2 = F1 + cnt[1], F3 = F2 + cnt[2], T = F3 + cnt[3];
  const int fu = (lane >= F1) + (lane >= F2) + (lane >= F3);
  const int fk = lane - sel4(fu, 0, F1, F2, F3);
  const int src = (lane < T) ? 8 * fu + 2 * fk : 0;
  StreamCtx<D> c;
  c.pa = __shfl(pid, src, 64);
  c.pb = __shfl(pid, src + 1, 64);
  {
    const int ptok = sel4(fu, us[0], us[1], us[2], us[3]) * SPLIT_TOK +
                     2 * kPage * (sel4(fu, lw[0], lw[1], lw[2], lw[3]) + W * fk);
    c.ptu = ((ptok >> 5) << 2) | fu;
  }
  c.page_elems = (size_t)Hkv * TILE;
  c.k_second = (r >> 3) != 0;
  c.v_second = (grp >> 1) != 0;
  c.kbase = a.kpool + (size_t)kvh * TILE + k_offset(8 * ((r >> 2) & 1) + (r & 3), kdim<D>(grp, 0));
  c.vbase = a.vpool + (size_t)kvh * TILE + r * kPage + 8 * (grp & 1);
  c.sl2 = a.scale_log2;

  // pair 0's loads go out before the barrier that publishes the query rows
  // in LDS (LDS-only fences: the barrier does not wait for them)
  // (unconditional, so that the wait for the query rows below counts these
  // loads; a wave without pairs reads its lane 0 page, a valid one, for nothing)
  PairBuf<D> b0;
  issue_pair(c, b0, 0);
  {
    u32x4* sq = (u32x4*)(smem + L::Q);
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int t = tid + i * 64 * W;
      const uint32_t m = -(uint32_t)qok[i];
      if (t < QCHUNKS) sq[t] = u32x4{qv[i][0] & m, qv[i][1] & m, qv[i][2] & m, qv[i][3] & m};
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  // units this wave has no pair of still get their (empty) partial
#pragma unroll
  for (int u = 0; u < kItemUnits; ++u) {
    if (np[u] > 0 && cnt[u] == 0) {
      SoftmaxState<D> e;
      init_state(e);
      park_partial<D>(smem, u * W + lw[u], G, e, r, grp);
    }
  }
  stream_item<D>(c, T, b0, smem, G, r, grp, lw[0], lw[1], lw[2], lw[3], te[0], te[1], te[2], te[3]);

  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  // sequences whose splits (2 .. ucap of them) all lie in this item, in
  // split order from unit u0: finished here
  bool whole[kItemUnits];
  bool any_whole = false;
#pragma unroll
  for (int u0 = 0; u0 < kItemUnits; ++u0) {
    const int ns = nsplit[u0];
    bool ok = ub[u0] >= 0 && us[u0] == 0 && ns >= 2 && ns <= ucap && u0 + ns <= kItemUnits;
#pragma unroll
    for (int v = 1; v < kItemUnits; ++v) {
      const int uv = u0 + v < kItemUnits ? u0 + v : kItemUnits - 1;
      if (v < ns) ok = ok && u0 + v < kItemUnits && ub[uv] == ub[u0] && us[uv] == v;
    }
    whole[u0] = ok;
    any_whole = any_whole || ok;
  }

  // merge each unit's W partials in logical-wave order: one wave per
  // (unit, head) row, lane w reading logical wave w's max and sum, each lane
  // its elements of the W partial accumulator rows
  constexpr int PER = D / 64;
  const size_t head_kv = (size_t)kvh * G;
  for (int row = wave; row < kItemUnits * G; row += W) {
    const int u = row / G;
    const int hh = row - u * G;
    const int b = sel4(u, ub[0], ub[1], ub[2], ub[3]);
    if (b < 0) continue;
    const int s = sel4(u, us[0], us[1], us[2], us[3]);
    const int nn = sel4(u, n[0], n[1], n[2], n[3]);
    const int ns = sel4(u, nsplit[0], nsplit[1], nsplit[2], nsplit[3]);
    const size_t head = (size_t)b * Hq + head_kv + hh;
    if (nn == 0) {
      if (s == 0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) a.out[head * D + lane + 64 * i] = 0.f;
      }
      continue;
    }
    if (s >= ns) continue;
    const float* pacc = smem + L::ACC + (size_t)(u * W * G + hh) * L::ROW + lane;
    float x[W][PER];
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int i = 0; i < PER; ++i) x[w][i] = pacc[(size_t)w * G * L::ROW + 64 * i];
    const float mv = lane < W ? smem[L::WM + (u * W + lane) * 16 + hh] : -INFINITY;
    const float lv = lane < W ? smem[L::WL + (u * W + lane) * 16 + hh] : 0.f;
    const float M = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row_max<W>(mv))));
    const float cw = __builtin_amdgcn_exp2f(mv - M);   // 0 in lanes >= W
    float Ls = 0.f, A[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) A[i] = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cw), w));
      Ls += c * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), w));
#pragma unroll
      for (int i = 0; i < PER; ++i) A[i] += c * x[w][i];
    }
    if (ns == 1) {
#pragma unroll
      for (int i = 0; i < PER; ++i) a.out[head * D + lane + 64 * i] = A[i] / Ls;
    } else if (ns <= ucap) {
      // logical wave 0's row of this head (this wave's own) takes the unit's merged accumulator
#pragma unroll
      for (int i = 0; i < PER; ++i) smem[L::ACC + (size_t)((u * W) * G + hh) * L::ROW + lane + 64 * i] = A[i];
      if (lane == 0) {
        smem[L::UM + u * 16 + hh] = M;
        smem[L::UL + u * 16 + hh] = Ls;
      }
    } else {
      const size_t slot = head * a.s_max + s;
#pragma unroll
      for (int i = 0; i < PER; ++i) a.ws_acc[slot * D + lane + 64 * i] = A[i];
      if (lane == 0) {
        a.ws_ml[slot * 2] = M;
        a.ws_ml[slot * 2 + 1] = Ls;
      }
    }
  }
  if (!any_whole) {
    asm volatile("" ::"s"(prefetched));
    return next;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
  for (int u0 = 0; u0 < kItemUnits; ++u0) {
    if (!whole[u0]) continue;
    for (int hh = wave; hh < G; hh += W) {
      auto ml = [&](int s) {
        return make_float2(smem[L::UM + (u0 + s) * 16 + hh], smem[L::UL + (u0 + s) * 16 + hh]);
      };
      auto acc = [&](int s, int e) { return smem[L::ACC + (size_t)(((u0 + s) * W) * G + hh) * L::ROW + e]; };
      lse_merge<D>(nsplit[u0], lane, ml, acc, a.out + ((size_t)ub[u0] * Hq + head_kv + hh) * D);
    }
  }
  asm volatile("" ::"s"(prefetched));
  return next;
}

// One workgroup per (KV head, bin): the bin's items in turn. Consecutive
// items need no barrier between them: an item writes the query rows (read
// only while streaming, which ended at the previous item's merge barrier)
// before its first barrier, and the partials only after it, when every wave
// has finished the previous item's merge. CHAIN = false is the form for
// launches in which no item can be chained (no more items than bins): each
// workgroup runs its one item, without the loop, which measured ~0.5 us
// faster on such one-round launches (64 sequences of up to 2048 tokens).
template <int D, int NW, bool CHAIN>
__global__ __launch_bounds__(64 * DecodeGeom<D>::W, occupancy(D)) void decode_kernel(DecodeArgs a,
                                                                                   InlinePlan<NW> ip) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int W = DecodeGeom<D>::W;
  constexpr int SP = DecodeGeom<D>::SPLIT_PAGES;
  static_assert(SP / 2 <= kMaxPairsPerUnit * W, "at most 4 pairs per logical wave");
  static_assert((W & (W - 1)) == 0 && W <= 16, "W: a power of two, rotations in 4 bits");
  __shared__ __align__(16) float smem[DecodeLds<D>::TOTAL];
  // grid: x = KV head, (y, z) = bin; linear workgroup order is KV head
  // fastest, so with 8 KV heads each XCD takes one head of every bin
  const int kvh = blockIdx.x;
  const int bin = blockIdx.z * 65535 + blockIdx.y;
  constexpr bool kInline = NW > kItemInts;
  // only a grid past 65535 bins has a ragged end; an inline plan holds at
  // most 256 items, so its grid is exact
  if constexpr (!kInline) {
    if (bin >= a.num_bins) return;
  }
  if constexpr (!CHAIN) {
    decode_item<D, NW>(a, ip, kvh, threadIdx.x, bin, smem);
  } else {
    int item = bin;
    for (;;) {
      // each item derives its per-lane values afresh (opaque copies of the
      // thread and KV head indices): none is held in registers across items
      int h = kvh;
      int tid = threadIdx.x;
      asm volatile("" : "+s"(h), "+v"(tid));
      const int next = decode_item<D, NW>(a, ip, h, tid, item, smem);
      // a chain only moves forward, past the bins' first items and inside
      // the plan: it ends after at most num_items items whatever the plan holds
      if (next <= item || next < a.num_bins || next >= a.num_items) break;
      item = next;
    }
  }
}

// One wave per (sequence, query head) of the sequences with more splits than
// a work item holds: their split partials, merged in split order.
template <int D>
__global__ __launch_bounds__(256) void merge_splits_kernel(DecodeArgs a) {
  constexpr int SPLIT_TOK = DecodeGeom<D>::SPLIT_PAGES * kPage;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.num_seqs * a.num_q_heads) return;
  const int b = item / a.num_q_heads;
  const int n = clamp_ctx(a.ctx[b], a.stride);
  const int nsplit = (n + SPLIT_TOK - 1) / SPLIT_TOK;
  if (nsplit <= a.ucap) return;
  const float* ml = a.ws_ml + (size_t)item * a.s_max * 2;
  const float* acc = a.ws_acc + (size_t)item * a.s_max * D;
  lse_merge<D>(
      nsplit, lane, [&](int s) { return make_float2(ml[2 * s], ml[2 * s + 1]); },
      [&](int s, int e) { return acc[(size_t)s * D + e]; }, a.out + (size_t)item * D);
}

// ---------------------------------------------------------------- append
// One 256-thread block per sequence: a bit copy of the new token's K row
// (16-byte chunks, each to its slab of the K tile) and of its V values into
// the slot-minor V layout, each V slot row (32 bytes) read, patched and
// written whole. The new token's values do not depend on where it goes, so
// they are loaded first, in flight while the position and the block-table
// entry are read; the V rows it patches are then all loaded together. The
// block's first kAppendK chunks and kAppendV values are held this way (all
// of them for up to 8 KV heads of 64 dims); larger shapes loop over the
// rest. Streaming (nontemporal) stores: the rows are read again only by a
// later step, and lines left dirty in L2 would be written back at the end
// of this launch, ahead of the decode that follows.
constexpr int kAppendK = 1;   // 16-byte K chunks per thread held in registers
constexpr int kAppendV = 2;   // V values (and their slot rows) per thread held in registers

template <int D>
__device__ __forceinline__ u32x4 patch_slot(u32x4 h, int half, int q, int w, uint32_t sh, uint32_t nv) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t upd = (h[i] & ~(0xFFFFu << sh)) | (nv << sh);
    h[i] = (half == q && i == w) ? upd : h[i];
  }
  return h;
}

template <int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int t = threadIdx.x;
  const int b = blockIdx.x;
  const int H = a.num_kv_heads;
  const uint16_t* kn = a.k_new + (size_t)b * H * D;
  const uint16_t* vn = a.v_new + (size_t)b * H * D;
  const int kchunks = H * (D / 8);
  const int vvals = H * D;
  u32x4 kv[kAppendK];
  uint32_t vv[kAppendV];
#pragma unroll
  for (int i = 0; i < kAppendK; ++i) {
    const int c = t + 256 * i;
    kv[i] = c < kchunks ? *(const u32x4*)(kn + 8 * (size_t)c) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < kAppendV; ++i) {
    const int e = t + 256 * i;
    vv[i] = e < vvals ? (uint32_t)vn[e] : 0u;
  }
  const int pos = a.positions[b];
  if (pos < 0 || pos >= a.stride * kPage) return;
  const int pid = a.block_tables[(size_t)b * a.stride + pos / kPage];
  if (pid < 0 || pid >= a.num_pages) return;
  const int slot = pos % kPage;
  const size_t tile0 = (size_t)pid * H;
  const int w = (slot & 7) >> 1;
  const int half = slot >> 3;
  const uint32_t sh = (slot & 1) * 16;
  // the V slot rows of the held values, loaded together
  u32x4 h0[kAppendV], h1[kAppendV];
#pragma unroll
  for (int i = 0; i < kAppendV; ++i) {
    const int e = t + 256 * i;   // row e = (kv head, dim)
    if (e < vvals) {
      const u32x4* row = (const u32x4*)(a.vpool + (tile0 * D + e) * kPage);
      h0[i] = row[0];
      h1[i] = row[1];
    }
  }
#pragma unroll
  for (int i = 0; i < kAppendK; ++i) {
    const int c = t + 256 * i;
    if (c < kchunks) {
      const int g = c / (D / 8);
      const int part = c - g * (D / 8);
      __builtin_nontemporal_store(kv[i], (u32x4*)(a.kpool + (tile0 + g) * kPage * D + k_offset(slot, 8 * part)));
    }
  }
#pragma unroll
  for (int i = 0; i < kAppendV; ++i) {
    const int e = t + 256 * i;
    if (e < vvals) {
      u32x4* row = (u32x4*)(a.vpool + (tile0 * D + e) * kPage);
      __builtin_nontemporal_store(patch_slot<D>(h0[i], half, 0, w, sh, vv[i]), row);
      __builtin_nontemporal_store(patch_slot<D>(h1[i], half, 1, w, sh, vv[i]), row + 1);
    }
  }
  // shapes beyond what the registers hold
  for (int c = t + 256 * kAppendK; c < kchunks; c += 256) {
    const int g = c / (D / 8);
    const int part = c - g * (D / 8);
    __builtin_nontemporal_store(*(const u32x4*)(kn + 8 * (size_t)c),
                                (u32x4*)(a.kpool + (tile0 + g) * kPage * D + k_offset(slot, 8 * part)));
  }
  for (int e = t + 256 * kAppendV; e < vvals; e += 256) {
    u32x4* row = (u32x4*)(a.vpool + (tile0 * D + e) * kPage);
    const uint32_t nv = vn[e];
    const u32x4 r0 = row[0];
    const u32x4 r1 = row[1];
    __builtin_nontemporal_store(patch_slot<D>(r0, half, 0, w, sh, nv), row);
    __builtin_nontemporal_store(patch_slot<D>(r1, half, 1, w, sh, nv), row + 1);
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
