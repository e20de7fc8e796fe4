// Affinity page pairs for the direct KV-page union.
//
// "PageWeaver: KV-Guided Query Unions for Sparse Attention", Abstract: the
// direct KV-page union weighs non-local reuse against the cost of reducing
// partials.  AI Radio episode on the paper, "Paper summary": it works on
// disjoint page pairs with common and exclusive query lists.  Pairing pages
// that many queries select together puts more entries on common lists and
// fewer (query, pair) partials in the reduction.
//
// Per KV head:
//   co[u][v] = number of queries whose support holds both u and v (diagonal 0);
//   the pairing is the greedy matching on the edges co > 0 in the order
//   (larger count, lower first page, lower second page); unmatched pages stay
//   single; pairs are numbered by their lower page.
//
// Kernels:
//   colbits_kernel  one wave per 64 queries: page columns as bitsets over the
//                   queries (LDS atomics, then coalesced stores, word-major);
//   gram_kernel     64 x 64 page tiles of co: per 4-word step each thread ANDs
//                   and popcounts a 4 x 4 block of page columns (v_bcnt), the
//                   column chunks staged in LDS; chunks where either side is
//                   all zero are skipped (a page is only selected after it
//                   exists, so early query blocks of late pages are empty).
//                   Each page's best partner over all pages (the first-round
//                   pointer of the matching) is folded in with atomicMax on
//                   the key (count << 12 | 4095 - partner);
//   match_kernel    one 1024-thread block per head: rounds in which every free
//                   page points at its best free partner and mutual pointers
//                   match.  A pair that points at each other is the first
//                   remaining edge at both ends, which is exactly the edge the
//                   sequential greedy takes there, so the result is the greedy
//                   matching (bit-exact).  A pointer is recomputed only when
//                   its target got matched: the free set only shrinks, so a
//                   free target stays the best.
#include "pw_internal.h"

namespace pw {
namespace {

constexpr int kMaxPairN = 2048;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct PMPlan {
  int TW;                      // 32-query words per page column (even)
  size_t off_cols, off_best, off_first, off_co, total;
};

PMPlan pm_plan(const pw_shape& s) {
  PMPlan d;
  d.TW = ((s.T + 63) / 64) * 2;
  d.off_cols = 0;
  d.off_best = align256((size_t)s.H_kv * s.N_pages * d.TW * 4);
  d.off_first = d.off_best + align256((size_t)s.H_kv * s.N_pages * 4);
  d.off_co = d.off_first + align256((size_t)s.H_kv * s.N_pages * 4);
  d.total = d.off_co + align256((size_t)s.H_kv * s.N_pages * s.N_pages * 4);
  return d;
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

__device__ __forceinline__ uint32_t pair_key(uint32_t c, int v) {
  return (c << 12) | (uint32_t)(4095 - v);      // larger count first, then the lower page
}

// cols[h][w][u]: bit j of word w = query 32 w + j selects page u.  first[h][u]:
// lowest word with a bit of page u (starts at TW: never selected).
__global__ __launch_bounds__(64) void colbits_kernel(const int32_t* __restrict__ sel, int T,
                                                     int S, int N, int TW,
                                                     uint32_t* __restrict__ cols,
                                                     int* __restrict__ first) {
  extern __shared__ uint32_t cw[];                 // [N][2]: the block's two words per page
  const int h = blockIdx.y, lane = threadIdx.x;
  const int t0 = blockIdx.x * 64;
  const int nq = min(64, T - t0);
  for (int i = lane; i < 2 * N; i += 64) cw[i] = 0;
  wave_sync();
  // the block's selection rows are contiguous: read them coalesced, 8 loads in flight
  const int32_t* rows = sel + ((size_t)h * T + t0) * S;
  const int n = nq * S;
  for (int i0 = 0; i0 < n; i0 += 64 * 8) {
    int e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j + lane;
      e[j] = i < n ? rows[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = (i0 + 64 * j + lane) / S;     // query within the block
      if (e[j] >= 0 && e[j] < N) atomicOr(&cw[2 * e[j] + (q >> 5)], 1u << (q & 31));
    }
  }
  wave_sync();
  uint32_t* base = cols + ((size_t)h * TW + 2 * blockIdx.x) * N;
  for (int u = lane; u < N; u += 64) {
    const uint32_t a = cw[2 * u], b = cw[2 * u + 1];
    base[u] = a;
    base[N + u] = b;
    if (a | b) atomicMin(&first[(size_t)h * N + u], 2 * blockIdx.x + (a ? 0 : 1));
  }
}

__global__ void fill_i32_kernel(int* p, int n, int v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

// One 64 x 64 tile (pages u0.., v0..) of co per block, u0 <= v0; writes both
// (u, v) and (v, u).  256 threads: thread (ty, tx) owns pages u0 + 4 ty + i and
// v0 + 4 tx + j.
constexpr int kGW = 32;                 // words per staged chunk
constexpr int kGS = kGW + 4;            // LDS row stride (16-byte aligned rows)

__global__ __launch_bounds__(256) void gram_kernel(const uint32_t* __restrict__ cols,
                                                   const int* __restrict__ first, int N,
                                                   int TW, int n_tiles, int* __restrict__ co,
                                                   uint32_t* __restrict__ best) {
  __shared__ __align__(16) uint32_t As[64 * kGS];
  __shared__ __align__(16) uint32_t Bs[64 * kGS];
  __shared__ int wmin[2][4];
  const int h = blockIdx.y;
  // blockIdx.x -> (ti, tj) with ti <= tj, row-major over the upper triangle
  int ti = 0, rem = blockIdx.x;
  while (rem >= n_tiles - ti) {
    rem -= n_tiles - ti;
    ++ti;
  }
  const int tj = ti + rem;
  const int u0 = 64 * ti, v0 = 64 * tj;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const uint32_t* ch = cols + (size_t)h * TW * N;
  // loader: thread t stages page t % 64 (row of the LDS chunk), words 8 (t / 64) .. + 8
  const int lr = tid & 63, lw = 8 * (tid >> 6);
  uint32_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0;
  // words before the first one where both tiles have a selected page are zero on
  // one side: start there (tile minimum of each side's first words, then the max)
  {
    const int* fh = first + (size_t)h * N;
    int fa = (u0 + (tid & 63) < N) ? fh[u0 + (tid & 63)] : TW;
    int fb = (v0 + (tid & 63) < N) ? fh[v0 + (tid & 63)] : TW;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      fa = min(fa, __shfl_xor(fa, off));
      fb = min(fb, __shfl_xor(fb, off));
    }
    if ((tid & 63) == 0) {
      wmin[0][tid >> 6] = fa;
      wmin[1][tid >> 6] = fb;
    }
  }
  __syncthreads();
  const int wstart = max(wmin[0][0], wmin[1][0]) / kGW * kGW;

  for (int w0 = wstart; w0 < TW; w0 += kGW) {
    uint32_t a[8], b[8];
    uint32_t any_a = 0, any_b = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int w = w0 + lw + q;
      const int ua = u0 + lr, vb = v0 + lr;
      a[q] = (w < TW && ua < N) ? ch[(size_t)w * N + ua] : 0u;
      b[q] = (w < TW && vb < N) ? ch[(size_t)w * N + vb] : 0u;
      any_a |= a[q];
      any_b |= b[q];
    }
    const int live_a = __syncthreads_or(any_a != 0);
    const int live_b = __syncthreads_or(any_b != 0);
    if (!live_a || !live_b) continue;               // uniform over the block
#pragma unroll
    for (int q = 0; q < 8; q += 4) {
      *reinterpret_cast<uint4*>(&As[lr * kGS + lw + q]) = make_uint4(a[q], a[q + 1], a[q + 2], a[q + 3]);
      *reinterpret_cast<uint4*>(&Bs[lr * kGS + lw + q]) = make_uint4(b[q], b[q + 1], b[q + 2], b[q + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kGW; w += 4) {
      uint4 ra[4], rb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const uint4*>(&As[(4 * ty + i) * kGS + w]);
        rb[i] = *reinterpret_cast<const uint4*>(&Bs[(4 * tx + i) * kGS + w]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t c = acc[i][j];
          c += __builtin_popcount(ra[i].x & rb[j].x);
          c += __builtin_popcount(ra[i].y & rb[j].y);
          c += __builtin_popcount(ra[i].z & rb[j].z);
          c += __builtin_popcount(ra[i].w & rb[j].w);
          acc[i][j] = c;
        }
    }
    __syncthreads();                                // As / Bs are rewritten next chunk
  }
  int* coh = co + (size_t)h * N * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = u0 + 4 * ty + i, v = v0 + 4 * tx + j;
      if (u == v || u >= N || v >= N) acc[i][j] = 0;   // no self pairs, no padding pages
    }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = u0 + 4 * ty + i;
    if (u < N)
      for (int j = 0; j < 4; ++j)
        if (v0 + 4 * tx + j < N) coh[(size_t)u * N + v0 + 4 * tx + j] = (int)acc[i][j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = v0 + 4 * tx + j;
    if (v < N)
      for (int i = 0; i < 4; ++i)
        if (u0 + 4 * ty + i < N) coh[(size_t)v * N + u0 + 4 * ty + i] = (int)acc[i][j];
  }
  // best partner keys: rows u over this tile's v (lanes of equal ty: tx = lane & 15),
  // and rows v over this tile's u (lanes of equal tx: the four ty of the wave)
  uint32_t* bh = best + (size_t)h * N;
  const int lane = tid & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t k = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (acc[i][j]) k = max(k, pair_key(acc[i][j], v0 + 4 * tx + j));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) k = max(k, (uint32_t)__shfl_xor((int)k, off));
    const int u = u0 + 4 * ty + i;
    if ((lane & 15) == 0 && k && u < N) atomicMax(&bh[u], k);
  }
  if (u0 != v0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t k = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (acc[i][j]) k = max(k, pair_key(acc[i][j], u0 + 4 * ty + i));
      k = max(k, (uint32_t)__shfl_xor((int)k, 16));
      k = max(k, (uint32_t)__shfl_xor((int)k, 32));
      const int v = v0 + 4 * tx + j;
      if (lane < 16 && k && v < N) atomicMax(&bh[v], k);
    }
  }
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}

// One block per KV head.  pairs[h][k] = (lower page, partner or -1), numbered
// by the lower page; rows past the head's pairs are (-1, -1).
__global__ __launch_bounds__(1024) void match_kernel(const int* __restrict__ co,
                                                     const uint32_t* __restrict__ best0, int N,
                                                     int2* __restrict__ pairs) {
  __shared__ int mate[kMaxPairN], ptr[kMaxPairN], todo[kMaxPairN];
  __shared__ int wsum[16];
  __shared__ int n_new, n_todo;
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int* C = co + (size_t)h * N * N;
  // first-round pointers: the best partner over all pages (every page is free)
  for (int u = tid; u < N; u += 1024) {
    const uint32_t k = best0[(size_t)h * N + u];
    mate[u] = -1;
    ptr[u] = k ? 4095 - (int)(k & 4095u) : -1;
  }
  __syncthreads();
  // Each round either matches at least one edge (the first remaining edge in
  // the order is mutual) or finds no edge between free pages and ends.
  for (int round = 0; round <= N; ++round) {
    // pages needing a new pointer (free, and the target got matched) are listed,
    // then the waves rescan the listed rows round-robin
    if (tid == 0) n_todo = 0;
    __syncthreads();
    for (int u = tid; u < N; u += 1024) {
      if (mate[u] != -1) continue;
      const int p = ptr[u];
      if (p >= 0 && mate[p] != -1) todo[atomicAdd(&n_todo, 1)] = u;
    }
    __syncthreads();
    const int nt = n_todo;
    for (int i = wv; i < nt; i += 16) {
      const int u = __builtin_amdgcn_readfirstlane(todo[i]);
      uint32_t kb = 0;
      const int* row = C + (size_t)u * N;
      for (int v0 = 0; v0 < N; v0 += 64 * 16) {     // 16 loads in flight per lane
        int c[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int v = v0 + 64 * j + lane;
          c[j] = v < N ? row[v] : 0;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int v = v0 + 64 * j + lane;
          if (c[j] > 0 && mate[v] == -1) kb = max(kb, pair_key((uint32_t)c[j], v));
        }
      }
      kb = wave_max_u32(kb);
      if (lane == 0) ptr[u] = kb ? 4095 - (int)(kb & 4095u) : -1;
    }
    if (tid == 0) n_new = 0;
    __syncthreads();
    int mine = 0;
    for (int u = tid; u < N; u += 1024) {
      if (mate[u] != -1) continue;
      const int p = ptr[u];
      if (p >= 0 && ptr[p] == u) {
        mate[u] = p;                              // each page writes only its own entry
        mine = 1;
      }
    }
    if (mine) atomicAdd(&n_new, 1);
    __syncthreads();
    const int done = n_new == 0;
    __syncthreads();                              // n_new is reset next round
    if (done) break;
  }
  // pair rows: leaders are single pages and the lower page of each pair
  int2* out = pairs + (size_t)h * N;
  int running = 0;
  for (int base = 0; base < N; base += 1024) {
    const int u = base + tid;
    const int m = u < N ? mate[u] : 0;
    const int lead = (u < N && (m < 0 || m > u)) ? 1 : 0;
    int x = lead;
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
    if (lead) out[running + woff + x - 1] = make_int2(u, m > u ? m : -1);
    running += all;
    __syncthreads();
  }
  for (int k = running + tid; k < N; k += 1024) out[k] = make_int2(-1, -1);
}

}  // namespace

size_t page_pairs_workspace(const pw_shape& s) { return pm_plan(s).total; }

hipError_t launch_page_pairs(const pw_shape& s, const int32_t* sel, int32_t* pairs, void* ws,
                             hipStream_t stream) {
  const PMPlan d = pm_plan(s);
  char* base = static_cast<char*>(ws);
  uint32_t* cols = reinterpret_cast<uint32_t*>(base + d.off_cols);
  uint32_t* best = reinterpret_cast<uint32_t*>(base + d.off_best);
  int* first = reinterpret_cast<int*>(base + d.off_first);
  int* co = reinterpret_cast<int*>(base + d.off_co);
  const int N = s.N_pages;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((s.H_kv * N + 255) / 256), dim3(256), 0, stream, best,
                     s.H_kv * N);
  hipLaunchKernelGGL(fill_i32_kernel, dim3((s.H_kv * N + 255) / 256), dim3(256), 0, stream, first,
                     s.H_kv * N, d.TW);
  hipLaunchKernelGGL(colbits_kernel, dim3((s.T + 63) / 64, s.H_kv), dim3(64), (size_t)2 * N * 4,
                     stream, sel, s.T, s.S, N, d.TW, cols, first);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nt = (N + 63) / 64;
  hipLaunchKernelGGL(gram_kernel, dim3(nt * (nt + 1) / 2, s.H_kv), dim3(256), 0, stream, cols,
                     first, N, d.TW, nt, co, best);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(match_kernel, dim3(s.H_kv), dim3(1024), 0, stream, co, best, N,
                     reinterpret_cast<int2*>(pairs));
  return hipGetLastError();
}

}  // namespace pw
