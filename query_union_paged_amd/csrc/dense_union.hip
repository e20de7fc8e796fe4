// Direct KV-page union: the pages' design-study alternative to query unions.
//
// "PageWeaver: KV-Guided Query Unions for Sparse Attention", Abstract: a
// direct KV-page union implementation studies non-local reuse against the
// cost of reducing partial outputs.  AI Radio episode on the paper, "Paper
// summary": it works on disjoint page pairs and uses the full membership of
// each page to form common or exclusive query lists.
//
// Pairs are either adjacent page IDs (2k, 2k + 1) or a caller-given table that
// partitions the pages (e.g. the affinity matching of pair_match.hip); a page
// map sends page u to slot 2k + (0 | 1) of its pair.  The FP8 pages are first
// re-tiled in MFMA operand order (as for the query union).  Then per chunk of
// Tc queries (all KV heads), on the caller's stream:
//   1. zero the per-pair list lengths;
//   2. pair_entries_kernel: one thread per (KV head, query) sets its pair-slot
//      bitset in LDS, walks its pairs in ascending order and appends
//      (query, partial slot, which pages) to pair k's list -- the pair's full
//      membership; an entry with both pages is on the common list, one page
//      on an exclusive list; list ranges are reserved once per (wave, pair);
//   3. tile_scan_kernel: per KV head, the lists cut into tiles of 8 entries are
//      numbered consecutively (an exclusive scan over the pairs), so the
//      attention grid covers at most entries / 8 + pairs tiles per head;
//   4. pair attention (union_attn.hip, pair mode): tiles of 8 entries of a
//      list compute (m, l, acc) over their own visible keys of the pair;
//   5. merge_kernel: one wave per (KV head, query) combines its partials by
//      log-sum-exp into O (maximum first, then independent weighted loads).
// The list order within a pair depends on atomics, but every partial has a
// fixed slot and a row's arithmetic does not depend on the other rows of its
// tile, so the result is deterministic.
#include "pw_internal.h"

namespace pw {
namespace {

constexpr size_t kBudget = size_t(4) << 30;   // workspace bound (bytes)

struct DUPlan {
  int Np, maxp, Tc, NW;   // Np: pair capacity per head (N: any partition fits)
  size_t off_tiles, off_count, off_tstart, off_pmap, off_npairs, off_list, off_part, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

DUPlan plan(const pw_shape& s) {
  DUPlan d;
  const int G = s.H_q / s.H_kv;
  d.Np = s.N_pages;
  d.maxp = s.S < d.Np ? s.S : d.Np;
  d.NW = (2 * d.Np + 31) / 32;      // words of a query's pair-slot bitset
  const size_t per_token = (size_t)s.H_kv * ((size_t)d.maxp * G * (s.D + 4) * 4 + (size_t)d.Np * 8 + 4);
  size_t tc = kBudget / per_token;
  tc = tc / 64 * 64;
  if (tc < 64) tc = 64;
  const size_t tmax = ((size_t)s.T + 63) / 64 * 64;
  if (tc > tmax) tc = tmax;
  d.Tc = (int)tc;
  d.off_tiles = 0;
  d.off_count = align256(tiled_kv_bytes(s));
  d.off_tstart = d.off_count + align256((size_t)s.H_kv * d.Np * 4);
  d.off_pmap = d.off_tstart + align256((size_t)s.H_kv * (d.Np + 1) * 4);
  d.off_npairs = d.off_pmap + align256((size_t)s.H_kv * s.N_pages * 4);
  d.off_list = d.off_npairs + align256((size_t)s.H_kv * d.Tc * 4);
  d.off_part = d.off_list + align256((size_t)s.H_kv * d.Np * d.Tc * 8);
  d.total = d.off_part + align256((size_t)s.H_kv * d.Tc * d.maxp * G * (s.D + 4) * 4);
  return d;
}

__global__ void fill_kernel(int* p, int n, int v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

// pmap[h][u] = 2k + position of page u in pair k of the table (pmap starts at -1:
// pages in no pair stay -1).  One thread per table row; rows (-1, -1) end it.
__global__ void pair_map_kernel(const int2* __restrict__ pairs, int N, int Hkv, int* pmap) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Hkv * N) return;
  const int h = i / N, k = i - h * N;
  const int2 pr = pairs[i];
  if (pr.x >= 0 && pr.x < N) pmap[h * N + pr.x] = 2 * k;
  if (pr.y >= 0 && pr.y < N) pmap[h * N + pr.y] = 2 * k + 1;
}

// Per KV head: tstart[k] = tiles (8 entries each) of pairs 0..k-1 and
// tstart[Np] = all of the head's tiles.  One 1024-thread block per head; wave
// scans by shuffles, wave totals through LDS.
__global__ __launch_bounds__(1024) void tile_scan_kernel(const int* __restrict__ pcount, int Np,
                                                         int* __restrict__ tstart) {
  __shared__ int wsum[16];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int* pc = pcount + (size_t)h * Np;
  int* ts = tstart + (size_t)h * (Np + 1);
  int running = 0;
  for (int base = 0; base < Np; base += 1024) {
    const int k = base + tid;
    const int n = k < Np ? (pc[k] + 7) >> 3 : 0;
    int x = n;                                     // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int woff = 0, all = 0;
    for (int v = 0; v < 16; ++v) {
      const int c = wsum[v];
      woff += v < wv ? c : 0;
      all += c;
    }
    if (k < Np) ts[k] = running + woff + x - n;
    running += all;
    __syncthreads();                               // wsum is rewritten next round
  }
  if (tid == 0) ts[Np] = running;
}

// One wave per 64 queries of one KV head.  Each lane sets its query's pair-slot
// bitset in LDS (bit 2k + position for each selected page) and walks its pairs
// in ascending order.  The wave first
// counts its entries per pair in LDS, reserves one range per pair in the global
// list (one atomic per (wave, pair) instead of one per entry: the sink and
// local pairs are in every query's support), then writes its entries there.
__global__ __launch_bounds__(64) void pair_entries_kernel(const int32_t* __restrict__ sel,
                                                         const int* __restrict__ pmap, int T,
                                                         int S, int N, int NW, int Np, int Tc,
                                                         int maxp, int t0, int* pcount,
                                                         int* npairs, int2* plist) {
  extern __shared__ uint32_t sh[];                 // [64][NW + 1] bitsets, cnt[Np], pos[Np]
  const int h = blockIdx.y, lane = threadIdx.x;
  const int tl = blockIdx.x * 64 + lane;           // query within the chunk
  const int t = t0 + tl;
  uint32_t* w = sh + lane * (NW + 1);
  int* cnt = reinterpret_cast<int*>(sh + 64 * (NW + 1));
  int* pos = cnt + Np;
  for (int i = 0; i < NW; ++i) w[i] = 0;
  for (int k = lane; k < Np; k += 64) cnt[k] = 0;
  const bool ok = tl < Tc && t < T;
  if (ok) {
    const int32_t* row = sel + ((size_t)h * T + t) * S;
    const int* pm = pmap != nullptr ? pmap + (size_t)h * N : nullptr;
    for (int s2 = 0; s2 < S; ++s2) {
      const int u = row[s2];
      if (u >= 0 && u < N) {
        const int v = pm != nullptr ? pm[u] : u;   // adjacent pairs: slot = page
        if (v >= 0) w[v >> 5] |= 1u << (v & 31);
      }
    }
  }
  wave_sync();
  // f(k, kind) for every pair of this lane's query, ascending
  auto for_pairs = [&](auto&& f) {
    for (int i = 0; i < NW; ++i) {
      const uint32_t x = w[i];
      uint32_t pm = (x | (x >> 1)) & 0x55555555u;  // pairs with at least one page
      while (pm) {
        const int bit = __builtin_ctz(pm);
        pm &= pm - 1;
        f(i * 16 + (bit >> 1), (int)((x >> bit) & 3));   // kind 1: first page, 2: second, 3: both
      }
    }
  };
  if (ok) for_pairs([&](int k, int) { atomicAdd(&cnt[k], 1); });
  wave_sync();
  for (int k = lane; k < Np; k += 64) {
    const int c = cnt[k];
    pos[k] = c ? atomicAdd(&pcount[h * Np + k], c) : 0;
  }
  wave_sync();
  if (ok) {
    int j = 0;
    for_pairs([&](int k, int kind) {
      const int slot = (h * Tc + tl) * maxp + j++;
      const int at = atomicAdd(&pos[k], 1);
      plist[((size_t)h * Np + k) * Tc + at] = make_int2(tl, slot | (kind << 30));
    });
    npairs[h * Tc + tl] = j;
  }
}

// One wave per (KV head, query).  For each of the G heads: the partials'
// (m, l) are read one per lane, their maximum M fixes the weights
// w_i = 2^(m_i - M), and every lane accumulates its d values over the
// partials with independent loads (no serial running-max chain).
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(const float* __restrict__ partials,
                                                   const int* __restrict__ npairs,
                                                   uint16_t* __restrict__ O, int T, int Hq,
                                                   int G, int Tc, int maxp, int t0) {
  constexpr int PER = D / 64;                      // d values per lane
  const int h = blockIdx.y;
  const int tl = blockIdx.x;
  const int t = t0 + tl;
  if (t >= T) return;
  const int lane = threadIdx.x;
  const int n = npairs[h * Tc + tl];
  const size_t slot0 = ((size_t)h * Tc + tl) * maxp;
  for (int j = 0; j < G; ++j) {
    auto part = [&](int i) { return partials + ((slot0 + i) * G + j) * (D + 4); };
    float M = -INFINITY;
    for (int i = lane; i < n; i += 64) {
      const float* pp = part(i);
      if (pp[1] > 0.f) M = fmaxf(M, pp[0]);        // l > 0: the pair had a visible key
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.f, A[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) A[q] = 0.f;
    if (M > -INFINITY) {
      for (int i0 = 0; i0 < n; i0 += 64) {
        float wgt = 0.f;
        if (i0 + lane < n) {
          const float* pp = part(i0 + lane);
          wgt = (pp[1] > 0.f) ? exp2f(pp[0] - M) : 0.f;
          L += wgt * pp[1];
        }
        const int cnt = min(64, n - i0);
        for (int r = 0; r < cnt; ++r) {
          const float wr = __shfl(wgt, r);
          const float* pp = part(i0 + r);
#pragma unroll
          for (int q = 0; q < PER; ++q) A[q] += wr * pp[4 + lane + 64 * q];
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    uint16_t* op = O + ((size_t)t * Hq + h * G + j) * D;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const __bf16 v = (__bf16)(A[q] * inv);
      op[lane + 64 * q] = __builtin_bit_cast(uint16_t, v);
    }
  }
}

}  // namespace

size_t dense_union_workspace(const pw_shape& s) { return plan(s).total; }

hipError_t launch_dense_union(const pw_shape& s, const uint16_t* Q, const uint8_t* K,
                              const uint8_t* V, const float* scales, const int32_t* sel,
                              const int32_t* pairs, uint16_t* O, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  const DUPlan d = plan(s);
  if (ws_bytes < d.total) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  int* pcount = reinterpret_cast<int*>(base + d.off_count);
  int* tstart = reinterpret_cast<int*>(base + d.off_tstart);
  int* pmap = nullptr;
  const int2* ptab = reinterpret_cast<const int2*>(pairs);
  // pairs in use per head: adjacent IDs need ceil(N / 2); a table may use up to N
  const int Np = pairs != nullptr ? d.Np : (s.N_pages + 1) / 2;
  const int NW = (2 * Np + 31) / 32;
  const int maxp = s.S < Np ? s.S : Np;
  int* npairs = reinterpret_cast<int*>(base + d.off_npairs);
  int2* plist = reinterpret_cast<int2*>(base + d.off_list);
  float* partials = reinterpret_cast<float*>(base + d.off_part);
  const int G = s.H_q / s.H_kv;
  uint8_t* tiles = reinterpret_cast<uint8_t*>(base + d.off_tiles);
  hipError_t e0 = tile_kv(s, K, V, scales, tiles, stream);
  if (e0 != hipSuccess) return e0;
  const int n_map = s.H_kv * s.N_pages;
  if (pairs != nullptr) {
    pmap = reinterpret_cast<int*>(base + d.off_pmap);
    hipLaunchKernelGGL(fill_kernel, dim3((n_map + 255) / 256), dim3(256), 0, stream, pmap, n_map,
                       -1);
    hipLaunchKernelGGL(pair_map_kernel, dim3((n_map + 255) / 256), dim3(256), 0, stream, ptab,
                       s.N_pages, s.H_kv, pmap);
  }
  // tile slots per head: at most entries / 8 + one partial tile per pair
  const int tiles_head = (int)(((size_t)d.Tc * maxp + 7) / 8) + Np;
  for (int t0 = 0; t0 < s.T; t0 += d.Tc) {
    const int n_count = s.H_kv * Np;
    hipLaunchKernelGGL(fill_kernel, dim3((n_count + 255) / 256), dim3(256), 0, stream, pcount,
                       n_count, 0);
    const int tcur = (s.T - t0 < d.Tc) ? s.T - t0 : d.Tc;
    hipLaunchKernelGGL(pair_entries_kernel, dim3((tcur + 63) / 64, s.H_kv), dim3(64),
                       ((size_t)64 * (NW + 1) + 2 * (size_t)Np) * 4, stream, sel, pmap, s.T, s.S,
                       s.N_pages, NW, Np, d.Tc, maxp, t0, pcount, npairs, plist);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tile_scan_kernel, dim3(s.H_kv), dim3(1024), 0, stream, pcount, Np, tstart);
    e = launch_pair_attention(s, Q, tiles, scales, plist, pcount, tstart, ptab, tiles_head,
                              partials, Np, d.Tc, t0, stream);
    if (e != hipSuccess) return e;
    if (s.D == 128)
      hipLaunchKernelGGL(merge_kernel<128>, dim3(tcur, s.H_kv), dim3(64), 0, stream, partials,
                         npairs, O, s.T, s.H_q, G, d.Tc, maxp, t0);
    else
      hipLaunchKernelGGL(merge_kernel<64>, dim3(tcur, s.H_kv), dim3(64), 0, stream, partials,
                         npairs, O, s.T, s.H_q, G, d.Tc, maxp, t0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pw
