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
//      hi*hi + hi*lo + lo*hi (relative error ~2^-16 of sum |qs||C|), 128 x 128
//      tiles per workgroup with D staged through LDS;
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

// qs and C of KV head h as bf16 hi/lo pairs, 8 d per thread (16-byte loads and
// stores): threads [0, T*D/8) do qs, the rest C.
__global__ __launch_bounds__(256) void sel_prep_kernel(const uint16_t* __restrict__ Q,
                                                       const uint8_t* __restrict__ K, int T,
                                                       int Hq, int Hkv, int D, int P, int N,
                                                       int h, __bf16* qh, __bf16* ql,
                                                       __bf16* ch, __bf16* cl) {
  const int G = Hq / Hkv, D8 = D / 8;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nq = (size_t)T * D8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  __bf16 *hi, *lo;
  if (i < nq) {
    const int t = (int)(i / D8), d8 = (int)(i % D8);
    const uint16_t* q = Q + ((size_t)t * Hq + h * G) * D + 8 * d8;
    for (int j = 0; j < G; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(q + (size_t)j * D);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += __uint_as_float(w[k] << 16);
        acc[2 * k + 1] += __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
    hi = qh + (size_t)t * D + 8 * d8;
    lo = ql + (size_t)t * D + 8 * d8;
  } else if (i < nq + (size_t)N * D8) {
    const size_t c = i - nq;
    const int u = (int)(c / D8), d8 = (int)(c % D8);
    const uint8_t* k = K + ((size_t)u * Hkv + h) * P * D + 8 * d8;
#pragma unroll 8
    for (int j = 0; j < P; ++j) {        // every partial sum of e4m3 values here is exact in fp32
      const uint2 w = *reinterpret_cast<const uint2*>(k + (size_t)j * D);
      const uint32_t ww[2] = {w.x, w.y};
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(ww[k2], false);
        const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(ww[k2], true);
        acc[4 * k2] += f01[0];
        acc[4 * k2 + 1] += f01[1];
        acc[4 * k2 + 2] += f23[0];
        acc[4 * k2 + 3] += f23[1];
      }
    }
    hi = ch + (size_t)u * D + 8 * d8;
    lo = cl + (size_t)u * D + 8 * d8;
  } else {
    return;
  }
  bf16x8 vh, vl;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 a, b;
    split_bf16(acc[e], a, b);
    vh[e] = a;
    vl[e] = b;
  }
  *reinterpret_cast<bf16x8*>(hi) = vh;
  *reinterpret_cast<bf16x8*>(lo) = vl;
}

// scores[t][u] = <qs_t, C_u> for one 128 x 128 (query, page) tile per workgroup;
// tiles whose pages all lie after the tile's last query exit.  D is staged in
// LDS 32 at a time (the next slice's loads in flight during the current one's
// MFMAs); each wave owns a 64 x 64 quarter as 2 x 2 MFMA tiles, three MFMAs
// per 16-d step (lo*hi + hi*lo + hi*hi).
constexpr int kSelTile = 128;
constexpr int kSelKD = 32;                    // d per staged slice
constexpr int kSelStride = kSelKD + 8;        // LDS row stride in bf16 (conflict-spreading pad)

__global__ __launch_bounds__(256) void sel_score_kernel(const __bf16* __restrict__ qh,
                                                        const __bf16* __restrict__ ql,
                                                        const __bf16* __restrict__ ch,
                                                        const __bf16* __restrict__ cl, int T,
                                                        int D, int P, int N, int n_ut,
                                                        float* __restrict__ sc) {
  __shared__ __align__(16) __bf16 lds[4][kSelTile * kSelStride];   // qh, ql, ch, cl slices
  const int tt = blockIdx.x / n_ut, ut = blockIdx.x % n_ut;
  const int t0 = kSelTile * tt, u0 = kSelTile * ut;
  if (u0 > (min(T, t0 + kSelTile) - 1) / P) return;               // uniform: all after the tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wy = wave >> 1, wx = wave & 1;
  const int row = lane & 31, half = lane >> 5;
  const __bf16* src[4] = {qh, ql, ch, cl};
  // loader: 4 arrays x 128 rows x 4 segments of 8 bf16; thread covers segments tid, tid + 256
  uint4 pre[4][2];
  auto load = [&](int d0) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int sidx = tid + 256 * j, r = sidx >> 2, part = sidx & 3;
        const int g = (a < 2 ? t0 : u0) + r;
        const int lim = a < 2 ? T : N;
        pre[a][j] = g < lim ? *reinterpret_cast<const uint4*>(src[a] + (size_t)g * D + d0 + 8 * part)
                            : make_uint4(0, 0, 0, 0);
      }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  load(0);
  for (int d0 = 0; d0 < D; d0 += kSelKD) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int sidx = tid + 256 * j, r = sidx >> 2, part = sidx & 3;
        *reinterpret_cast<uint4*>(&lds[a][r * kSelStride + 8 * part]) = pre[a][j];
      }
    __syncthreads();
    if (d0 + kSelKD < D) load(d0 + kSelKD);
#pragma unroll
    for (int k0 = 0; k0 < kSelKD; k0 += 16) {
      bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = 64 * wy + 32 * i + row, rb = 64 * wx + 32 * i + row;
        const int o = k0 + 8 * half;
        ah[i] = *reinterpret_cast<const bf16x8*>(&lds[0][ra * kSelStride + o]);
        al[i] = *reinterpret_cast<const bf16x8*>(&lds[1][ra * kSelStride + o]);
        bh[i] = *reinterpret_cast<const bf16x8*>(&lds[2][rb * kSelStride + o]);
        bl[i] = *reinterpret_cast<const bf16x8*>(&lds[3][rb * kSelStride + o]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
        }
    }
    __syncthreads();                      // the slice is overwritten next
  }
  // lane holds column (page) row of each 32 x 32 tile, rows 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int uc = u0 + 64 * wx + 32 * j + row;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = t0 + 64 * wy + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (tr < T && uc < N) sc[(size_t)tr * N + uc] = acc[i][j][r];
      }
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
  // all loads first (clamped to the row, so none needs a branch), then the keys
  float sv[R], kv[R];
  const int n_load = min(lo_local, N);             // candidates lie below lo_local
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int u = min(lane + 64 * i, N - 1);
    if (64 * i < n_load) {                         // uniform: skip chunks past the candidates
      sv[i] = sc[(size_t)t * N + u];
      kv[i] = kscale[(size_t)u * Hkv];
    } else {
      sv[i] = 0.f;
      kv[i] = 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int u = lane + 64 * i;
    const bool ok = u >= 1 && u < lo_local;
    key[i] = ok ? order_key(sv[i] * kv[i]) : 0u;
    valid |= ok ? 1u << i : 0u;
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
  const int n_tt = (s.T + kSelTile - 1) / kSelTile, n_ut = (s.N_pages + kSelTile - 1) / kSelTile;
  const size_t n_prep = (size_t)(s.T + s.N_pages) * (s.D / 8);
  for (int h = 0; h < s.H_kv; ++h) {
    hipLaunchKernelGGL(sel_prep_kernel, dim3((unsigned)((n_prep + 255) / 256)), dim3(256), 0,
                       stream, Q, K, s.T, s.H_q, s.H_kv, s.D, s.P, s.N_pages, h, qh, ql, ch, cl);
    hipLaunchKernelGGL(sel_score_kernel, dim3(n_tt * n_ut), dim3(256), 0, stream, qh,
                       ql, ch, cl, s.T, s.D, s.P, s.N_pages, n_ut, sc);
    hipLaunchKernelGGL(sel_topk_kernel, dim3((s.T + 3) / 4), dim3(256), 0, stream, sc,
                       scales + h, s.T, s.H_kv, s.P, s.N_pages, s.S, L, h, sel);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pw
