// Synthetic dynamic page selector: sel_pages from Q and the FP8 K pages.
//
// "PageWeaver: KV-Guided Query Unions for Sparse Attention", Abstract: each
// query of dynamic sparse attention comes with its own set of selected KV
// pages; the method takes that relation as given.  This is a stand-in
// selector of our own in the block-sparse style, so that the path can run
// on selections derived from Q and K:
//   fixed pages  the sink (page 0) and the L local pages p, p-1, ..., p-L+1
//                of the query's own page p;
//   candidates   pages 1..p not fixed;
//   score(u)     ks[u][h] * <qs_t, C_u>, qs_t = sum of the query's G head rows
//                of KV head h, C_u[d] = sum of e4m3(K[u][h][j][d]) over keys j;
//   choice       the min(S - |fixed|, |candidates|) largest scores, ties to the
//                lower page; the row is ascending, padded with -1.
//
// Per KV head, three kernels on the caller's stream:
//   1. prep: qs (fp32 sum of the bf16 rows) and C (exact fp32 sum of the
//      e4m3 codes) as bf16 hi + lo pairs;
//   2. scores: <qs, C> for every (query, page <= own page) on the bf16 MFMA,
//      hi*hi + hi*lo + lo*hi (relative error ~2^-16 of sum |qs||C|);
//   3. top-k: one wave per query, a 4-pass 8-bit radix select on the ordered
//      fp32 score bits over LDS histograms, then the ascending row.
#include "pw_internal.h"

namespace pw {
namespace {

constexpr int kMaxPages = 1024;     // candidates per query held by one wave (16 per lane)

struct SelLayout {
  size_t off_qh, off_ql, off_ch, off_cl, off_sc, total;
};

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

SelLayout layout(const pw_shape& s) {
  SelLayout l;
  const size_t tq = (size_t)s.T * s.D * 2, nc = (size_t)s.N_pages * s.D * 2;
  l.off_qh = 0;
  l.off_ql = al256(tq);
  l.off_ch = l.off_ql + al256(tq);
  l.off_cl = l.off_ch + al256(nc);
  l.off_sc = l.off_cl + al256(nc);
  l.total = l.off_sc + al256((size_t)s.T * s.N_pages * 4);
  return l;
}

__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// qs and C of KV head h as bf16 hi/lo pairs: threads [0, T*D) do qs, the rest C.
__global__ __launch_bounds__(256) void sel_prep_kernel(const uint16_t* __restrict__ Q,
                                                       const uint8_t* __restrict__ K, int T,
                                                       int Hq, int Hkv, int D, int P, int N,
                                                       int h, __bf16* qh, __bf16* ql,
                                                       __bf16* ch, __bf16* cl) {
  const int G = Hq / Hkv;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nq = (size_t)T * D;
  if (i < nq) {
    const int t = (int)(i / D), d = (int)(i % D);
    const uint16_t* q = Q + ((size_t)t * Hq + h * G) * D + d;
    float acc = 0.f;
    for (int j = 0; j < G; ++j) acc += __uint_as_float((uint32_t)q[(size_t)j * D] << 16);
    split_bf16(acc, qh[i], ql[i]);
  } else if (i < nq + (size_t)N * D) {
    const size_t c = i - nq;
    const int u = (int)(c / D), d = (int)(c % D);
    const uint8_t* k = K + ((size_t)u * Hkv + h) * P * D + d;
    float acc = 0.f;                  // every partial sum of e4m3 values here is exact in fp32
    for (int j = 0; j < P; j += 2) {
      const int pair = (int)k[(size_t)j * D] | ((int)k[(size_t)(j + 1) * D] << 8);
      const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(pair, false);
      acc += f[0];
      acc += f[1];
    }
    split_bf16(acc, ch[c], cl[c]);
  }
}

// scores[t][u] = <qs_t, C_u> for one 32 x 32 (query, page) tile per wave; tiles
// whose pages all lie after the tile's last query are skipped.
__global__ __launch_bounds__(256) void sel_score_kernel(const __bf16* __restrict__ qh,
                                                        const __bf16* __restrict__ ql,
                                                        const __bf16* __restrict__ ch,
                                                        const __bf16* __restrict__ cl, int T,
                                                        int D, int P, int N, int n_ut,
                                                        float* __restrict__ sc) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int tt = wid / n_ut, ut = wid % n_ut;
  const int t0 = 32 * tt, u0 = 32 * ut;
  if (t0 >= T || u0 > (min(T, t0 + 32) - 1) / P) return;
  const int row = lane & 31, half = lane >> 5;
  const int t = min(t0 + row, T - 1), u = min(u0 + row, N - 1);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int k0 = 0; k0 < D; k0 += 16) {
    const size_t qo = (size_t)t * D + k0 + 8 * half, co = (size_t)u * D + k0 + 8 * half;
    const bf16x8 a_h = *reinterpret_cast<const bf16x8*>(qh + qo);
    const bf16x8 a_l = *reinterpret_cast<const bf16x8*>(ql + qo);
    const bf16x8 b_h = *reinterpret_cast<const bf16x8*>(ch + co);
    const bf16x8 b_l = *reinterpret_cast<const bf16x8*>(cl + co);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_l, b_h, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_h, b_l, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_h, b_h, acc, 0, 0, 0);
  }
  // lane holds column u0 + row, rows 8*(r/4) + 4*half + r%4 of the tile
  const int uc = u0 + row;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tr = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (tr < T && uc < N) sc[(size_t)tr * N + uc] = acc[r];
  }
}

// Larger float -> larger key (fp32 bits made unsigned-ordered).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One wave per query: fixed pages, then the k largest candidate scores.
__global__ __launch_bounds__(256) void sel_topk_kernel(const float* __restrict__ sc,
                                                       const float* __restrict__ kscale, int T,
                                                       int Hkv, int P, int N, int S, int L, int h,
                                                       int32_t* __restrict__ sel) {
  __shared__ uint32_t hist_all[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  uint32_t* hist = hist_all[wave];
  const int p = t / P;
  const int lo_local = max(0, p - L + 1);          // local pages lo_local..p
  const int n_fixed = (p - lo_local + 1) + (lo_local > 0 ? 1 : 0);
  const int n_cand = max(0, lo_local - 1);         // pages 1 .. lo_local-1
  const int k = min(S - n_fixed, n_cand);
  constexpr int R = kMaxPages / 64;
  uint32_t key[R];
  uint32_t valid = 0, chosen = 0;                  // bit i: page lane + 64 i
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int u = lane + 64 * i;
    key[i] = 0;
    if (u >= 1 && u < lo_local) {
      key[i] = order_key(sc[(size_t)t * N + u] * kscale[(size_t)u * Hkv]);
      valid |= 1u << i;
    }
  }
  if (k > 0) {
    uint32_t prefix = 0, mask = 0;
    int need = k;                                   // still to take at or below the prefix
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int b = lane; b < 256; b += 64) hist[b] = 0;
      wave_sync();
#pragma unroll
      for (int i = 0; i < R; ++i)
        if (((valid >> i) & 1u) && (key[i] & mask) == prefix)
          atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
      wave_sync();
      // lane holds bins 4*lane .. 4*lane+3; suffix counts from the top bin down
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = hist[4 * lane + j];
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      uint32_t above = mine;                      // inclusive suffix over lanes >= lane
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_down(above, d);
        if (lane + d < 64) above += y;
      }
      above -= mine;                              // bins of higher lanes only
      // the bin b where the count of digits >= b first reaches need
      int found = -1;
      uint32_t gt = 0;
      uint32_t run = above;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (found < 0 && run + c[j] >= (uint32_t)need) {
          found = 4 * lane + j;
          gt = run;
        }
        run += c[j];
      }
      const uint64_t bal = __ballot(found >= 0);
      const int src = 63 - __builtin_clzll(bal);  // highest lane that found it: the largest bin
      const int b = __shfl(found, src);
      need -= (int)__shfl(gt, src);
      prefix |= (uint32_t)b << shift;
      mask |= 0xFFu << shift;
      wave_sync();
    }
    // keys above the k-th value, then the lowest pages among those equal to it
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (((valid >> i) & 1u) && key[i] > prefix) chosen |= 1u << i;
      const bool eq = ((valid >> i) & 1u) && key[i] == prefix;
      const uint64_t be = __ballot(eq);
      const int rank = __builtin_popcountll(be & ((1ull << lane) - 1ull));
      if (eq && rank < need) chosen |= 1u << i;
      need -= min(need, __popcll(be));
    }
  }
  // the row: fixed and chosen pages in ascending order, then -1
  int32_t* out = sel + ((size_t)h * T + t) * S;
  int pos = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int u = lane + 64 * i;
    const bool take = u <= p && (u == 0 || u >= lo_local || ((chosen >> i) & 1u));
    const uint64_t bt = __ballot(take);
    if (take) out[pos + __builtin_popcountll(bt & ((1ull << lane) - 1ull))] = u;
    pos += __popcll(bt);
  }
  for (int j = pos + lane; j < S; j += 64) out[j] = -1;
}

}  // namespace

size_t select_workspace(const pw_shape& s) { return layout(s).total; }

hipError_t launch_select(const pw_shape& s, const uint16_t* Q, const uint8_t* K,
                         const float* scales, int L, int32_t* sel, void* ws,
                         hipStream_t stream) {
  const SelLayout l = layout(s);
  char* base = static_cast<char*>(ws);
  __bf16* qh = reinterpret_cast<__bf16*>(base + l.off_qh);
  __bf16* ql = reinterpret_cast<__bf16*>(base + l.off_ql);
  __bf16* ch = reinterpret_cast<__bf16*>(base + l.off_ch);
  __bf16* cl = reinterpret_cast<__bf16*>(base + l.off_cl);
  float* sc = reinterpret_cast<float*>(base + l.off_sc);
  const int n_tt = (s.T + 31) / 32, n_ut = (s.N_pages + 31) / 32;
  const size_t n_prep = (size_t)(s.T + s.N_pages) * s.D;
  for (int h = 0; h < s.H_kv; ++h) {
    hipLaunchKernelGGL(sel_prep_kernel, dim3((unsigned)((n_prep + 255) / 256)), dim3(256), 0,
                       stream, Q, K, s.T, s.H_q, s.H_kv, s.D, s.P, s.N_pages, h, qh, ql, ch, cl);
    hipLaunchKernelGGL(sel_score_kernel, dim3((n_tt * n_ut + 3) / 4), dim3(256), 0, stream, qh,
                       ql, ch, cl, s.T, s.D, s.P, s.N_pages, n_ut, sc);
    hipLaunchKernelGGL(sel_topk_kernel, dim3((s.T + 3) / 4), dim3(256), 0, stream, sc,
                       scales + h, s.T, s.H_kv, s.P, s.N_pages, s.S, L, h, sel);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pw
