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
// registers of its MFMA operand; the next pair's loads are issued before the
// current pair is computed. Waves merge (m, l, acc) through LDS; a split that
// is not alone writes its partial to the workspace and merge_splits combines
// the splits of a sequence by log-sum-exp in split order.
//
// Lane roles (lane = 0..63, r = lane % 16, grp = lane / 16):
//   QK A operand   row r = token: page (r / 8) of the pair,
//                  slot 8 * ((r / 4) % 2) + 4 * j + r % 4 for MFMA j = 0, 1;
//                  k = head dims (D / 4) * grp + 8 * kk + 0..7
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

template <int D>
struct PairBuf {
  u32x4 k[2][D / 32];   // QK A operands: MFMA j, k-step kk
  u32x4 v[D / 16];      // PV A operands: dim tile mt
};

// ---------------------------------------------------------------- decode
template <int D, int W, int SPLIT_PAGES>
__global__ __launch_bounds__(64 * W) void decode_split_kernel(DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(SPLIT_PAGES % 2 == 0 && SPLIT_PAGES <= 64, "split pages: even, at most one per lane");
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  constexpr int TILE = kPage * D;           // elements of one (page, kv head) tile
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
  const int b = rest % a.num_seqs;
  const int s = rest / a.num_seqs;
  const int G = a.group;

  const int n = clamp_ctx(a.ctx[b], a.stride);
  if (n == 0) {
    if (s == 0) {
      float* o = a.out + ((size_t)b * a.num_q_heads + (size_t)kvh * G) * D;
      for (int e = threadIdx.x; e < G * D; e += 64 * W) o[e] = 0.f;
    }
    return;
  }
  const int nsplit = (n + SPLIT_TOK - 1) / SPLIT_TOK;
  if (s >= nsplit) return;

  const int tok0 = s * SPLIT_TOK;
  const int tok1 = min(tok0 + SPLIT_TOK, n);
  const int p0 = tok0 / kPage;
  const int npages = (tok1 - tok0 + kPage - 1) / kPage;
  const int npairs = (npages + 1) >> 1;

  // This split's physical page ids, one per lane, clamped into the pool.
  int my_pid = 0;
  if (lane < npages) {
    int v = a.block_tables[(size_t)b * a.stride + p0 + lane];
    my_pid = v < 0 ? 0 : (v >= a.num_pages ? a.num_pages - 1 : v);
  }

  // Query group as the MFMA B operand (columns = heads, zero past G).
  bf16x8 qf[KK];
  if (r < G) {
    const uint16_t* qp = a.q + ((size_t)b * a.num_q_heads + (size_t)kvh * G + r) * D + (D / 4) * grp;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = as_bf16x8(*(const u32x4*)(qp + 8 * kk));
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }

  const size_t page_elems = (size_t)a.num_kv_heads * TILE;
  const int koff = (8 * ((r >> 2) & 1) + (r & 3)) * D + (D / 4) * grp;
  const int voff = r * kPage + 8 * (grp & 1);
  const bool k_second = (r >> 3) != 0;    // this lane's K row comes from the pair's second page
  const bool v_second = (grp >> 1) != 0;  // this lane's V tokens come from the second page
  const uint16_t* kbase = a.kpool + (size_t)kvh * TILE + koff;
  const uint16_t* vbase = a.vpool + (size_t)kvh * TILE + voff;
  const float sl2 = a.scale_log2;

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](PairBuf<D>& buf, int pr) {
    const int la = 2 * pr;
    const int lb = min(2 * pr + 1, npages - 1);     // a missing second page re-reads the first (all masked)
    const int pa = __builtin_amdgcn_readlane(my_pid, la);
    const int pb = __builtin_amdgcn_readlane(my_pid, lb);
    const uint16_t* kp = kbase + (size_t)(k_second ? pb : pa) * page_elems;
    const uint16_t* vp = vbase + (size_t)(v_second ? pb : pa) * page_elems;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) buf.k[j][kk] = *(const u32x4*)(kp + 4 * j * D + 8 * kk);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) buf.v[mt] = *(const u32x4*)(vp + mt * 16 * kPage);
  };

  auto compute = [&](PairBuf<D>& buf, int pr) {
    const int pair_tok = (p0 + 2 * pr) * kPage;
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
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
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
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {   // skip the rescale when no head's max moved
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
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
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf.v[mt]), ph, acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(buf.v[mt]), pl, acc[mt], 0, 0, 0);
    }
  };

  // This wave's pairs are wave, wave + W, ...; the next pair's loads are in
  // flight while the current one is computed (two register buffers). The
  // steady-state loop issues unconditionally and the last one or two pairs
  // are peeled, so every wait for loaded data counts exactly the loads issued
  // after it and never waits for the prefetch.
  const int my_n = wave < npairs ? (npairs - wave + W - 1) / W : 0;
  if (my_n > 0) {
    PairBuf<D> b0, b1;
    issue(b0, wave);
    int it = 0;
    for (; it + 2 < my_n; it += 2) {
      issue(b1, wave + (it + 1) * W);
      compute(b0, wave + it * W);
      issue(b0, wave + (it + 2) * W);
      compute(b1, wave + (it + 1) * W);
    }
    if (it + 1 < my_n) {
      issue(b1, wave + (it + 1) * W);
      compute(b0, wave + it * W);
      compute(b1, wave + (it + 1) * W);
    } else {
      compute(b0, wave + it * W);
    }
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // Merge the W waves through LDS: m, l per head, acc per (head, dim).
  float* sm_m = smem;
  float* sm_l = smem + W * 16;
  float* sm_acc = smem + 2 * W * 16;
  if (grp == 0) {
    sm_m[wave * 16 + r] = m_run;
    sm_l[wave * 16 + r] = l_run;
  }
  if (r < G) {
    float* dst = sm_acc + (size_t)(wave * G + r) * LDS_ROW + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *(f32x4*)(dst + 16 * mt) = acc[mt];
  }
  __syncthreads();

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
      const float c = __builtin_amdgcn_exp2f(sm_m[w * 16 + hh] - M);
      L += c * sm_l[w * 16 + hh];
      A += c * sm_acc[(size_t)(w * G + hh) * LDS_ROW + dd];
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
// have more than one, in split order.
template <int D>
__global__ __launch_bounds__(256) void merge_splits_kernel(DecodeArgs a, int split_tokens) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.num_seqs * a.num_q_heads) return;
  const int b = item / a.num_q_heads;
  const int n = clamp_ctx(a.ctx[b], a.stride);
  const int nsplit = (n + split_tokens - 1) / split_tokens;
  if (nsplit <= 1) return;
  const float* ml = a.ws_ml + (size_t)item * a.s_max * 2;
  const float* acc = a.ws_acc + (size_t)item * a.s_max * D;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f;
  float A[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) A[i] = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float c = __builtin_amdgcn_exp2f(ml[2 * s] - M);
    L += c * ml[2 * s + 1];
#pragma unroll
    for (int i = 0; i < PER; ++i) A[i] += c * acc[(size_t)s * D + lane + 64 * i];
  }
  float* o = a.out + (size_t)item * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[lane + 64 * i] = A[i] / L;
}

// ---------------------------------------------------------------- append
// Four sequences per 256-thread block; a bit copy of the new token's K row
// (16-byte stores) and V values (into the slot-minor V layout).
template <int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= a.num_seqs) return;
  const int pos = a.positions[b];
  if (pos < 0 || pos >= a.stride * kPage) return;
  const int pid = a.block_tables[(size_t)b * a.stride + pos / kPage];
  if (pid < 0 || pid >= a.num_pages) return;
  const int slot = pos % kPage;
  const int H = a.num_kv_heads;
  const size_t tile0 = (size_t)pid * H;
  const uint16_t* kn = a.k_new + (size_t)b * H * D;
  const uint16_t* vn = a.v_new + (size_t)b * H * D;
  for (int c = lane; c < H * (D / 8); c += 64) {
    const int g = c / (D / 8);
    const int part = c - g * (D / 8);
    *(u32x4*)(a.kpool + ((tile0 + g) * kPage + slot) * D + 8 * part) =
        *(const u32x4*)(kn + (size_t)g * D + 8 * part);
  }
  for (int e = lane; e < H * D; e += 64) {
    const int g = e / D;
    const int dd = e - g * D;
    a.vpool[((tile0 + g) * D + dd) * kPage + slot] = vn[e];
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
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * stride];
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
