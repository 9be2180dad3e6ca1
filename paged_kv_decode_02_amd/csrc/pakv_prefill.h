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
// 128 consecutive rows, 32 per wave in two groups of 16, and streams the key
// pages its rows can see (up to the position of its last token), two pages
// per step. The workgroup loads each page pair's K and V once into LDS,
// stored in matrix-core operand order; every wave reads its operands from
// there and feeds both of its row groups with them:
//
//   S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16): A = 16 keys
//     x 32 head dims, B = 32 head dims x one group's 16 rows. The 16 A rows
//     of MFMA j mix the two pages (row r is page r / 8, slot
//     8 ((r / 4) % 2) + 4 j + r % 4), so that lane (r = lane % 16,
//     grp = lane / 16) ends up with slots 8 (grp % 2) + 0..7 of page grp / 2
//     for row r: 8 consecutive keys, positions 32 pair + 8 grp + 0..7
//     (both row groups' scores are issued before either group's softmax);
//   causal mask by select (only on pairs that cross the diagonal), FP32
//     online softmax per row: weights against the running max as it stands;
//     the row maxima (over the 4 lanes holding a row, by lane swaps) are
//     found only when some lane's weight sum passes 2^8, and the running max
//     moves only when it trails the row's max by more than 8 (log2 units);
//   O^T += V^T P^T on the matrix cores: A = V^T (16 head dims x those 8 keys
//     per lane group: 16 contiguous bytes of a slot-minor V row), B = P^T,
//     P split into BF16 hi + lo as in decode.
// The row blocks that see the most keys are launched first.
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
  int32_t row_blocks;           // 128-row blocks per (sequence, KV head) in the grid
  float scale_log2;
  // optional launch plan: workgroup (item, KV head) takes row block
  // plan[item] = b | rb << 20; NULL = every (sequence, row block) in the
  // rotated order below
  const int32_t* plan;
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
// 16-byte copies into their slabs; every V slot row (32 bytes, one head dim of one KV head) of
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
  // K: (slot, kv head, 16-byte chunk); four loads in flight per thread
  const int kchunks = (s1 - s0) * H * (D / 8);
  for (int e0 = threadIdx.x; e0 < kchunks; e0 += 4 * 256) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * 256;
      if (e < kchunks) {
        const int part = e % (D / 8);
        const int g = (e / (D / 8)) % H;
        const size_t row = (size_t)(row_of_slot0 + s0 + e / ((D / 8) * H));
        v[u] = *(const u32x4*)(a.k_rows + (row * H + g) * D + 8 * part);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * 256;
      if (e < kchunks) {
        const int part = e % (D / 8);
        const int g = (e / (D / 8)) % H;
        const int slot = s0 + e / ((D / 8) * H);
        *(u32x4*)(a.kpool + (tile0 + g) * kPage * D + k_offset(slot, 8 * part)) = v[u];
      }
    }
  }
  // V: one slot row per (kv head, head dim). The chunk's values of that dim
  // for the page's slots are loaded together (independent 2-byte loads; a
  // wave covers 64 consecutive dims, so each load is 128 contiguous bytes),
  // then packed into the row; slots outside the chunk keep their bits.
  const bool whole = s0 == 0 && s1 == kPage;
  for (int e = threadIdx.x; e < H * D; e += 256) {
    const int g = e / D;
    const int dd = e - g * D;
    u32x4* vrow = (u32x4*)(a.vpool + ((tile0 + g) * D + dd) * kPage);
    uint32_t nv[kPage];
#pragma unroll
    for (int slot = 0; slot < kPage; ++slot)
      nv[slot] = (slot >= s0 && slot < s1)
                     ? (uint32_t)a.v_rows[((size_t)(row_of_slot0 + slot) * H + g) * D + dd] : 0u;
    u32x4 h[2];
    if (whole) {
      h[0] = u32x4{0u, 0u, 0u, 0u};
      h[1] = h[0];
    } else {
      h[0] = vrow[0];
      h[1] = vrow[1];
    }
    // dword i of half q holds slots 8 q + 2 i (low 16 bits) and 8 q + 2 i + 1
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sa = 8 * q + 2 * i;
        const uint32_t lo = (sa >= s0 && sa < s1) ? nv[sa] : (h[q][i] & 0xFFFFu);
        const uint32_t hi = (sa + 1 >= s0 && sa + 1 < s1) ? nv[sa + 1] : (h[q][i] >> 16);
        h[q][i] = lo | (hi << 16);
      }
    vrow[0] = h[0];
    vrow[1] = h[1];
  }
}

// -------------------------------------------------------------- attention
template <int D, int RG>
struct PrefillWave {
  const uint16_t* ktile;  // K pool + KV head tile of page 0
  const uint16_t* vtile;
  const int32_t* bt_row;  // the sequence's block-table row
  size_t page_elems;
  int num_pages;          // pool size (page ids are clamped into it)
  int key_pages;          // pages the workgroup reads (positions 0 .. its last token)
  int last_pos;           // position of the wave's last token (keys past it are zeroed)
  int first_pos;          // position of the wave's first token (keys up to it are seen by every row)
  int pos[RG];            // this lane's query position per row group (rows past the chunk: last_pos)
  float sl2;
  uint32_t neg_lo, neg_hi;  // BF16 pairs (-1, 0) and (0, -1), held opaque (see split_low)
  bf16x8 qf[RG][D / 32];  // the lane's query row per row group, B operand
};

// The page ids of a pair are the same for every lane, and the block tables
// do not change during the launch: read through the constant address space
// they are scalar loads (both issued before either is used), and the clamp
// into the pool and the pages' addresses are scalar arithmetic, not per-lane
// 64-bit multiplies.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

template <int D, int RG>
__device__ __forceinline__ void pair_pages(const PrefillWave<D, RG>& w, int first, int second, int& pa,
                                           int& pb) {
  const const_i32_ptr row = (const_i32_ptr)(uintptr_t)w.bt_row;
  const int ra = row[first];
  const int rb = row[second];
  pa = ra < 0 ? 0 : (ra >= w.num_pages ? w.num_pages - 1 : ra);
  pb = rb < 0 ? 0 : (rb >= w.num_pages ? w.num_pages - 1 : rb);
}

// Maximum over the 4 lanes that hold one row (l, l ^ 16, l ^ 32, l ^ 48),
// with gfx950's lane-swap instructions instead of LDS permutes: swapping a
// value with a copy of itself leaves the values of lanes l and l ^ 16 (or
// l ^ 32) in the two results. The copy is made opaque, so the compiler keeps
// the two results apart (handed one value twice, it merged them).
__device__ __forceinline__ float row_max4(float v) {
  uint32_t a = __float_as_uint(v), b = a;
  asm volatile("" : "+v"(b));
  const auto s16 = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  v = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  a = __float_as_uint(v);
  b = a;
  asm volatile("" : "+v"(b));
  const auto s32 = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}

// How far (log2 units) a row's running max may trail its true max before the
// accumulators are rescaled: weights then stay at most 2^8, and a rescale
// happens only when a row's maximum grows by more than that. A lane whose
// weight sum is within kLazyBound has every weight within it.
constexpr float kLazyMax = 8.f;
constexpr float kLazyBound = 256.f;   // 2^kLazyMax

// The pair's scores and weights: S^T = K Q^T for every row group, then the
// online softmax; ph / pl receive the weights' BF16 high and low parts.
template <int D, int RG>
__device__ __forceinline__ void prefill_softmax(const PrefillWave<D, RG>& w, const u32x4 (&kop)[2][D / 32], int pr,
                                                SoftmaxState<D> (&st)[RG], int grp, bf16x8 (&ph)[RG],
                                                bf16x8 (&pl)[RG]) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  // element e = 4 j + i is key position key0 + e
  const int key0 = 32 * pr + 8 * grp;
  // only a pair that some row of the wave cannot see whole needs the mask
  const bool diag = 32 * pr + 31 > w.first_pos;
  // every row group's scores first, so that the matrix cores work on the
  // next group's while the VALU does this group's weights
  f32x4 scg[RG][2];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      scg[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        scg[g][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[j][kk]), w.qf[g][kk], scg[g][j], 0, 0, 0);
    }
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = scg[g][e >> 2][e & 3];
    if (diag) {
      const int lim = w.pos[g] - key0;     // key0 + e is visible iff e <= lim
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = (e <= lim) ? sv[e] : -INFINITY;
    }
    // Weights against the running max as it stands. Each is at most the
    // lane's sum, so while every lane's sum stays within 2^kLazyMax the row
    // maxima need not be found; otherwise (and on a row's first keys, while
    // its max is -inf and the sums are not finite) the wave finds them,
    // moves a max that trails by more than kLazyMax, and recomputes.
    const float m_old = st[g].m;
    f32x2 pv[4];
    float psum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pv[q] = f32x2{__builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * q], w.sl2, -m_old)),
                    __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * q + 1], w.sl2, -m_old))};
      psum = q == 0 ? pv[q][0] + pv[q][1] : psum + (pv[q][0] + pv[q][1]);
    }
    float alpha = 1.f;
    if (__ballot(!(psum <= kLazyBound))) {
      float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                       fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mx = row_max4(mx);
      // raw scores times a positive sl2 (the sign of the scale is folded into q)
      const float mx2 = mx * w.sl2;
      const float m_new = mx2 > m_old + kLazyMax ? mx2 : m_old;
      alpha = __builtin_amdgcn_exp2f(m_old - m_new);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pv[q] = f32x2{__builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * q], w.sl2, -m_new)),
                      __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * q + 1], w.sl2, -m_new))};
        psum = q == 0 ? pv[q][0] + pv[q][1] : psum + (pv[q][0] + pv[q][1]);
      }
      if (__ballot(m_new != m_old)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) st[g].acc[mt] *= alpha;
      }
      st[g].m = m_new;
    }
    st[g].l = st[g].l * alpha + psum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x2 hi = __builtin_convertvector(pv[q], bf16x2);
      // low halves p - float(hi), exactly: hi . (-1, 0) + p0 and hi . (0, -1) + p1
      // (BF16 products are exact in FP32 and the sums are representable)
      const f32x2 low = {__builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2, w.neg_lo), pv[q][0], false),
                         __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2, w.neg_hi), pv[q][1], false)};
      const bf16x2 lo = __builtin_convertvector(low, bf16x2);
      ph[g][2 * q] = hi[0];
      ph[g][2 * q + 1] = hi[1];
      pl[g][2 * q] = lo[0];
      pl[g][2 * q + 1] = lo[1];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// O^T += V^T P^T for every row group, P as its BF16 high and low parts.
template <int D, int RG>
__device__ __forceinline__ void prefill_pv(const PrefillWave<D, RG>& w, u32x4 (&vop)[D / 16], int pr,
                                           SoftmaxState<D> (&st)[RG], int grp, const bf16x8 (&ph)[RG],
                                           const bf16x8 (&pl)[RG]) {
  constexpr int MT = D / 16;
  const int key0 = 32 * pr + 8 * grp;
  // keys past the wave's last position may be unwritten (NaN): zero their V
  // (dword q holds the lane's keys 2q, 2q+1: positions key0 + 2q, key0 + 2q + 1)
  if (32 * pr + 32 > w.last_pos + 1) {
    uint32_t keep[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k0 = key0 + 2 * q;
      keep[q] = (k0 <= w.last_pos ? 0x0000FFFFu : 0u) | (k0 + 1 <= w.last_pos ? 0xFFFF0000u : 0u);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) vop[mt][q] &= keep[q];
  }
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      st[g].acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vop[mt]), ph[g], st[g].acc[mt], 0, 0, 0);
      st[g].acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vop[mt]), pl[g], st[g].acc[mt], 0, 0, 0);
    }
  __builtin_amdgcn_sched_barrier(0);
}

// Two groups of 16 rows per wave: every K/V operand loaded feeds both.
template <int D>
__host__ __device__ constexpr int prefill_row_groups() { return 2; }
// Waves per SIMD: 4 at d = 64 (at most 128 registers per lane, the kernel
// needs 126; more waves overlap one wave's softmax with another's
// matrix-core work and measured faster than 2 or 3), 2 at d = 128 (at most
// 256 registers per lane, the kernel needs about 200; a bound of 1 gave 2
// waves as well).
// The launch plan counts on these as the workgroups a CU holds.
template <int D>
__host__ __device__ constexpr int prefill_occupancy() { return D == 64 ? 4 : 2; }
// rows per workgroup: 4 waves x 16 rows x row groups
template <int D>
__host__ __device__ constexpr int prefill_block_rows() { return 64 * prefill_row_groups<D>(); }

// Grid: KV head fastest, then sequence, then row block from the last one
// down, so the blocks that see the most keys start first. Within each row
// block the sequences are rotated by rbp + rbp / 4 (rbp: the block's rank
// from the last): the workgroups reach the 8 XCDs round-robin and then a CU
// of their XCD in order, so in a grid the device holds at once a CU takes
// positions t, t + 32, t + 64, ... of its XCD's sequence; without the
// rotation, whenever the sequence count divides 32 those are row blocks of
// one sequence, and the CU that draws the longest cache does its four
// longest blocks while others idle. With it, a CU's four blocks belong to
// four sequences (8 sequences: offsets 0, 5, 2, 7). A launch plan made on
// the host from the chunk and cache lengths (pa_prefill_plan) replaces this
// order with one by work. Wave w of a block takes rows w * 32 .. w * 32 + 31
// in two groups of 16.
//
// The 4 waves share every K/V tile through LDS. Per page pair the
// workgroup copies K and V from the pages into LDS with direct-to-LDS
// buffer loads (buffer_load_dwordx4 ... lds: 16 bytes per lane, written at
// the wave's LDS base + 16 x lane, no registers on the way), in the order
// the matrix cores read them. An operand area (K, or V) is 2 x 128
// NPT 16-byte slots, the first half from the pair's first page, the second
// from its second: slot t of a half holds, for K, piece (MFMA j, k-step kk
// = block t / 32, lane group t % 32 / 8, key row t % 8 of the half's page)
// and for V piece (dim tile t / 32, lane t % 32 of the half's page). A
// wave's 64 slots therefore come from one page, so its load addresses are
// that page's base (scalar) plus a fixed per-lane offset; a lane reading
// its operand takes slot half x 128 NPT + block x 32 + (K) grp x 8 + r % 8
// / (V) lane % 32: every run of 8 lanes reads 128 contiguous bytes, free of
// bank conflicts. Four LDS buffers form a ring: pair p + 4's copies are
// issued while pair p is computed, so three pairs' copies are in flight;
// each wave waits for its own copies with vmcnt and one barrier per pair
// makes all of them visible (and frees the buffer of the pair before).
template <int D>
struct PrefillLds {
  static constexpr int kKBytes = 2 * kPage * D * 2;     // K of a pair (two pages)
  static constexpr int kPairBytes = 2 * kKBytes;        // K and V
  static constexpr int kPerThread = (4 * D) / 256;      // 16-byte K (and V) pieces per thread
  static constexpr int kHalfSlots = 128 * kPerThread;   // slots of one page in an operand area
};
// Fourth word of a raw buffer descriptor on gfx9: 32-bit data format, no
// swizzle, no thread-id offsets (a zero data format would make loads return 0).
constexpr int kBufferWord3 = 0x00020000;
// Pairs whose copies are in the LDS ring at once (at d = 64 four
// workgroups hold 4 x 32 KiB of a CU's 160 KiB; at d = 128, two hold 2 x 64 KiB).
constexpr int kPrefillRing = 4;

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt bits 3:0, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Waits until at most N of this wave's copies are in flight (the copies
// issued after those of the pair about to be read), then a bare barrier:
// every wave's copies of that pair have landed and every wave is done with
// the buffer the next copy reuses (each wave's own LDS reads have returned:
// lgkmcnt(0)). The empty asm statements keep the compiler from moving
// memory accesses across it.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  wait_vm<N>();
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(256, prefill_occupancy<D>()) void prefill_kernel(PrefillArgs a) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  constexpr int RG = prefill_row_groups<D>();
  constexpr int WROWS = 16 * RG;
  constexpr int BROWS = 4 * WROWS;
  constexpr int NPT = PrefillLds<D>::kPerThread;
  constexpr int KB = PrefillLds<D>::kKBytes;
  constexpr int PB = PrefillLds<D>::kPairBytes;
  constexpr int HS = PrefillLds<D>::kHalfSlots;
  static_assert(kPrefillRing == 4, "the loop below is unrolled for a ring of 4");
  // separate arrays, indexed statically, so that the compiler can tell the
  // ring's buffers apart and waits only for the copies a read needs
  __shared__ __attribute__((aligned(16))) char ring0[PB], ring1[PB], ring2[PB], ring3[PB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;
  const int grp = lane >> 4;
  const int kvh = blockIdx.x % a.num_kv_heads;
  const int rest = blockIdx.x / a.num_kv_heads;
  int b, rb;
  if (a.plan) {
    const uint32_t item = (uint32_t)a.plan[rest];
    b = (int)(item & 0xFFFFFu);
    rb = (int)(item >> 20);
    if (b >= a.num_seqs || rb >= a.row_blocks) return;
  } else {
    const int rbp = rest / a.num_seqs;
    b = (rest % a.num_seqs + rbp + rbp / 4) % a.num_seqs;
    rb = a.row_blocks - 1 - rbp;
  }
  const int G = a.group;
  const Chunk ch = load_chunk(a.query_start, a.ctx_before, b, a.num_rows, a.max_chunk, a.stride);
  const int rows = ch.n * G;
  if (rb * BROWS >= rows) return;                      // the whole block is past the chunk
  const int blk_last_pos = ch.c + min(rb * BROWS + BROWS - 1, rows - 1) / G;
  const int blk_pages = (blk_last_pos + kPage) / kPage;
  const int npairs = (blk_pages + 1) >> 1;
  const int rho0 = rb * BROWS + wave * WROWS;          // the wave's first row
  const bool active = rho0 < rows;                     // a wave past the chunk only loads
  const int rho_last = active ? min(rho0 + WROWS - 1, rows - 1) : rows - 1;

  PrefillWave<D, RG> w;
  w.last_pos = ch.c + rho_last / G;
  w.first_pos = ch.c + min(rho0, rows - 1) / G;
  w.key_pages = blk_pages;
  w.num_pages = a.num_pages;
  w.bt_row = a.block_tables + (size_t)b * a.stride;
  w.page_elems = (size_t)a.num_kv_heads * kPage * D;
  w.ktile = a.kpool + (size_t)kvh * kPage * D;
  w.vtile = a.vpool + (size_t)kvh * kPage * D;
  const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  const bool qzero = a.scale_log2 == 0.f;
  w.sl2 = qzero ? 1.f : fabsf(a.scale_log2);
  // Held in registers the compiler cannot see into: folded to an inline
  // constant, the pair (-1, 0) was encoded as FP32 -1.0, which
  // v_dot2_f32_bf16 reads as the pair (0, -1).
  w.neg_lo = 0x0000BF80u;
  w.neg_hi = 0xBF800000u;
  asm volatile("" : "+s"(w.neg_lo));
  asm volatile("" : "+s"(w.neg_hi));
  size_t qrow[RG];
  bool valid[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int rho = rho0 + 16 * g + r;
    valid[g] = active && rho < rows;
    const int t = (valid[g] ? rho : rho_last) / G;
    const int h = (valid[g] ? rho : rho_last) - t * G;
    w.pos[g] = ch.c + t;
    qrow[g] = ((size_t)(ch.r0 + t) * a.num_q_heads + (size_t)kvh * G + h) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      w.qf[g][kk] = as_bf16x8((valid[g] && !qzero) ? *(const u32x4*)(a.q + qrow[g] + kdim<D>(grp, kk)) ^ qflip
                                                    : u32x4{0u, 0u, 0u, 0u});
  }

  // this thread's copies of a pair: piece i fills slot tid + 256 i of the K
  // (and of the V) area; the slot's half, hence the page, is the same for
  // the whole wave
  uint32_t kgo[NPT], vgo[NPT];   // byte offsets within the page's KV-head tile
  bool second[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int slot = tid + 256 * i;
    const int t = slot % HS;
    second[i] = slot >= HS;
    {  // K: block (j, kk) = t / 32, lane group t % 32 / 8, key row t % 8 of the page
      const int jk = t >> 5;
      const int j = jk / KK;
      const int kk = jk - j * KK;
      const int lg = (t >> 3) & 3;
      const int lr = t & 7;                              // QK row lr (+ 8 on the second page)
      const int key = 8 * ((lr >> 2) & 1) + 4 * j + (lr & 3);
      kgo[i] = (uint32_t)(2 * k_offset(key, kdim<D>(lg, kk)));
    }
    {  // V: dim tile mt = t / 32, operand lane t % 32 (+ 32 on the second page)
      const int mt = t >> 5;
      const int ln = t & 31;
      vgo[i] = (uint32_t)(2 * ((16 * mt + (ln & 15)) * kPage + 8 * (ln >> 4)));
    }
  }
  // LDS byte offsets of this lane's operands in a buffer
  const uint32_t kread = (uint32_t)(16 * ((r >> 3) * HS + grp * 8 + (r & 7)));
  const uint32_t vread = (uint32_t)(KB + 16 * ((grp >> 1) * HS + (lane & 31)));
  typedef __attribute__((address_space(3))) void* lds_ptr;
  constexpr int kTileBytes = kPage * D * 2;        // one page's K (or V) of one KV head
  // The pair's copies into buffer `dst`, from pages pa and pb. They are
  // buffer loads with the LDS destination (buffer_load_dwordx4 ... lds):
  // with them the compiler still waits for LDS reads one by one (lgkmcnt
  // n), which it does not after the flat-encoded global-to-LDS form. Every step
  // issues one pair's copies, also past the last pair (then the last pair's
  // pages again, which no one reads), so that the wait before each pair is
  // the same count. The page half of piece i is the same for the whole wave.
  auto copy_pair = [&](int pa, int pb, char* dst) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int pid = (64 * wave + 256 * i) >= HS ? pb : pa;
      // buffer descriptors of the page's K and V tiles of this KV head
      // (offsets checked against the tile's bytes)
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(w.ktile + (size_t)pid * w.page_elems), (short)0, kTileBytes, kBufferWord3);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(w.vtile + (size_t)pid * w.page_elems), (short)0, kTileBytes, kBufferWord3);
      char* wbase = dst + 16 * (64 * wave + 256 * i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_ptr)wbase, 16, (int)kgo[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_ptr)(wbase + KB), 16, (int)vgo[i], 0, 0, 0);
    }
  };
  // page ids of pair pr (clamped to the block's last pair)
  auto pages_of = [&](int pr, int& pa, int& pb) {
    pr = min(pr, npairs - 1);
    pair_pages(w, 2 * pr, min(2 * pr + 1, blk_pages - 1), pa, pb);
  };
  SoftmaxState<D> st[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) init_state(st[g]);
  // this lane's operands of the pair being computed: K for the scores, V
  // for the weighted sum; each is read from LDS one phase before its use
  u32x4 kop[2][KK], vop[MT];
  auto read_k = [&](const char* buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kop[j][kk] = *(const u32x4*)(buf + kread + 512 * (j * KK + kk));
  };
  auto read_v = [&](const char* buf) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) vop[mt] = *(const u32x4*)(buf + vread + 512 * mt);
  };
  // page ids of the pair a copy is for, read right before the barrier that
  // precedes the copy, whose wait (lgkmcnt(0)) covers their scalar loads
  int pa, pb;
  // the first four pairs' copies fill the ring; pair p lives in buffer p % 4
  constexpr int NL = 2 * NPT;   // copies per pair and thread
  pages_of(0, pa, pb);
  copy_pair(pa, pb, ring0);
  pages_of(1, pa, pb);
  copy_pair(pa, pb, ring1);
  pages_of(2, pa, pb);
  copy_pair(pa, pb, ring2);
  pages_of(3, pa, pb);
  copy_pair(pa, pb, ring3);
  ring_barrier<3 * NL>();   // pair 0 (pairs 1-3 may be in flight)
  read_k(ring0);
  read_v(ring0);
  // One step computes pair pr (its K and V already in registers): the
  // scores and weights; the barrier for pair pr + 1 (its copies have
  // landed, and every wave is done with pair pr's buffer); the copy of
  // pair pr + 4 into that buffer; the read of pair pr + 1's K, then the
  // weighted sum of pair pr, then the read of pair pr + 1's V. Every LDS
  // read thus has a phase of matrix-core work to land in.
  auto step = [&](int pr, char* cur, const char* nxt, bool issue) {
    const bool doit = active && 32 * pr <= w.last_pos;
    bf16x8 ph[RG], pl[RG];
    if (doit) prefill_softmax(w, kop, pr, st, grp, ph, pl);
    if (issue) {
      pages_of(pr + 4, pa, pb);
      ring_barrier<2 * NL>();   // pair pr + 1 (pairs pr + 2, pr + 3 may be in flight)
      copy_pair(pa, pb, cur);
    } else {
      // the last pairs: every copy was issued already; wait for all of them
      asm volatile("" ::: "memory");
      wait_vm<0>();
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    read_k(nxt);
    if (doit) prefill_pv(w, vop, pr, st, grp, ph, pl);
    read_v(nxt);
  };
  // whole rounds of four pairs (a loop without early exits, so that the
  // compiler's own wait analysis sees the ring's buffers apart), then the
  // last 0-3 pairs, which issue no copies
  int pr = 0;
  for (; pr + 4 <= npairs; pr += 4) {
    step(pr, ring0, ring1, true);
    step(pr + 1, ring1, ring2, true);
    step(pr + 2, ring2, ring3, true);
    step(pr + 3, ring3, ring0, true);
  }
  if (pr < npairs) step(pr, ring0, ring1, false);
  if (pr + 1 < npairs) step(pr + 1, ring1, ring2, false);
  if (pr + 2 < npairs) step(pr + 2, ring2, ring3, false);
  // no copy may still be writing this workgroup's LDS when it ends
  wait_vm<0>();
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    float l = st[g].l;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (valid[g]) {
      const float inv = 1.f / l;
      float* o = a.out + qrow[g] + 4 * grp;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) *(f32x4*)(o + 16 * mt) = st[g].acc[mt] * inv;
    }
  }
}

}  // namespace pakv
