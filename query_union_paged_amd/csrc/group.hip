// Bounded-window greedy grouping of queries by selected-page affinity.
//
// "PageWeaver: KV-Guided Query Unions for Sparse Attention", Abstract: a
// bounded GPU search produces query IDs (nothing else).  AI Radio episode on
// the paper, "Paper summary": within a bounded window the members of a
// query-owned group are collected greedily, taking queries whose selected
// sets add few new pages; g is fixed independently of the window W.
//
// One wave per (KV head, aligned window).  Lane l owns candidates l, l+64,
// l+128, ... (C = ceil(W/64) of them) and keeps their page bitsets in VGPRs
// over the window's pages only (page -> its rank among the distinct pages the
// window selects, so the width is set by how many pages the window uses, not
// by their spread); the bitsets are built 64 candidates at a time in LDS from
// 16-byte loads of the selection rows.  A
// step is a wave minimum of key = (cost << 10 | local index) over the
// available candidates (DPP within rows of 16, then four readlanes), so the
// lowest index wins ties and the result is bit-exact.  The winner's words
// come to scalar registers by readlane; only the words where it brings new
// pages (delta = B_best & ~U) touch the candidates, whose cost is kept as
// |B_c| - |B_c & U| with |B_c & U| accumulated popcount by popcount.
// On request the search also records each group's union size as it closes the
// group; group_order_kernel (below) turns those sizes into an execution order
// of the groups for the attention.
#include "pw_internal.h"

namespace pw {
namespace {

constexpr uint32_t kNone = 0xFFFFFFFFu;
constexpr int kStride = 33;   // LDS words per candidate bitset (32 + 1 pad: conflict-free rows)

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_min(uint32_t v) {
  // every lane has a source lane for these permutes, so the move folds into v_min_u32_dpp
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
  return min(v, o);
}

// Minimum over the 64 lanes, returned as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t v) {
  v = dpp_min<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_min<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_min<0x141>(v);   // row_half_mirror
  v = dpp_min<0x140>(v);   // row_mirror: every lane holds its row's minimum
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// The greedy loop of one window.  The window's bitsets are staged 64
// candidates at a time (LDS `stage`) and kept in registers over page ranks
// (`rank`: a page's index among the window's distinct pages), NWB words wide;
// words past the last rank are zero for every candidate and cost nothing.
// With NWV > 1 waves per window, wave wv owns candidates
// 64 C wv + 64 c + lane; each step then takes the minimum over the waves' minima
// through LDS (`xch`), and the owner of the chosen candidate publishes its
// words there (two workgroup barriers per step).
template <int C, int NWB, int NWV>
__device__ __forceinline__ void window_body(const int32_t* __restrict__ wbase, int S, int N,
                                            int Wr, int g, const uint16_t* rank,
                                            uint32_t* stage, int* order, uint32_t* xch,
                                            int32_t* __restrict__ usz) {
  const int lane = threadIdx.x & 63;
  const int wv = NWV > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  static_assert(NWV == 1 || (C & (C - 1)) == 0, "several waves need C in {1, 2, 4}");
  // candidate index -> owning wave (log2(64 C); one wave: always 0)
  constexpr int kShift = NWV == 1 ? 16 : C == 4 ? 8 : C == 2 ? 7 : 6;
  const int cbase = 64 * C * wv;             // first candidate of this wave
  uint32_t b[C][NWB];
  // one 64-candidate chunk: bits set in LDS, then each lane takes its row
  auto build_chunk = [&](uint32_t(&bc)[NWB], const int c) __attribute__((always_inline)) {
    for (int i = lane; i < 64 * kStride; i += 64) stage[i] = 0;
    wave_sync();
    const int r0 = cbase + 64 * c;
    const int nrows = max(0, min(64, Wr - r0));
    const int32_t* base = wbase + (size_t)r0 * S;
    auto put = [&](int r, int u) __attribute__((always_inline)) {
      if (u >= 0 && u < N) {
        const int k = rank != nullptr ? rank[u] : u;   // the page's index among the window's pages
        atomicOr(&stage[r * kStride + (k >> 5)], 1u << (k & 31));
      }
    };
    if ((S & 3) == 0) {          // 16-byte loads, 8 per lane in flight
      const int n4 = (nrows * S) >> 2;
      const int4* b4 = reinterpret_cast<const int4*>(base);
      for (int i0 = 0; i0 < n4; i0 += 64 * 8) {
        int4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = i0 + 64 * j + lane;
          v[j] = (i < n4) ? b4[i] : make_int4(-1, -1, -1, -1);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // the four entries belong to one row (S is a multiple of 4) and selection rows are
          // usually sorted: entries that fall into the same bitset word share one LDS atomic
          const int r = ((i0 + 64 * j + lane) << 2) / S;
          const int e4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
          int wcur = -1;
          uint32_t bits = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int u = e4[q];
            const int k = (u >= 0 && u < N) ? (rank != nullptr ? (int)rank[u] : u) : -1;
            const int wq = k >= 0 ? (k >> 5) : -1;
            if (wq != wcur) {
              if (bits) atomicOr(&stage[r * kStride + wcur], bits);
              wcur = wq;
              bits = 0;
            }
            if (k >= 0) bits |= 1u << (k & 31);
          }
          if (bits) atomicOr(&stage[r * kStride + wcur], bits);
        }
      }
    } else {
      for (int i = lane; i < nrows * S; i += 64) put(i / S, base[i]);
    }
    wave_sync();
#pragma unroll
    for (int jj = 0; jj < NWB; ++jj) bc[jj] = stage[lane * kStride + jj];
    wave_sync();
  };
  build_chunk(b[0], 0);
  if constexpr (C > 1) build_chunk(b[1], 1);
  if constexpr (C > 2) build_chunk(b[2], 2);
  if constexpr (C > 3) build_chunk(b[3], 3);

  // cost(c) = |B_c \ U| = tot_c - gain_c with gain_c = |B_c & U|, kept
  // incrementally: a word where U grows by delta adds popcount(B_c & delta)
  uint32_t tot[C], gain[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    tot[c] = 0;
#pragma unroll
    for (int jj = 0; jj < NWB; ++jj) tot[c] += __builtin_popcount(b[c][jj]);
  }
  uint32_t avail = 0;                      // bit c: candidate 64c + lane unassigned
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (cbase + 64 * c + lane < Wr) avail |= 1u << c;
  uint32_t U[NWB];                         // the group's union (wave-uniform)
  uint32_t w[NWB];                         // the chosen candidate's words

  // the chosen candidate's words, read from its lane (wave-uniform result);
  // across waves the owner publishes them in LDS
  auto fetch = [&](int wb, int cb, int lb) __attribute__((always_inline)) {
    if (wb == wv) {
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (c == cb) {
#pragma unroll
          for (int jj = 0; jj < NWB; ++jj) w[jj] = __builtin_amdgcn_readlane(b[c][jj], lb);
        }
    }
    if constexpr (NWV > 1) {
      uint32_t* row = xch + 4;   // [32]
      if (wb == wv && lane == 0) {
#pragma unroll
        for (int jj = 0; jj < NWB; ++jj) row[jj] = w[jj];
      }
      __syncthreads();
#pragma unroll
      for (int jj = 0; jj < NWB; ++jj) w[jj] = __builtin_amdgcn_readfirstlane(row[jj]);
    }
  };
  // the window-wide minimum of a key (the wave's own minimum when NWV == 1)
  auto window_min = [&](uint32_t key) __attribute__((always_inline)) -> uint32_t {
    uint32_t m = __builtin_amdgcn_readfirstlane(wave_min_dpp(key));
    if constexpr (NWV > 1) {
      if (lane == 0) xch[wv] = m;
      __syncthreads();
#pragma unroll
      for (int v = 0; v < NWV; ++v) m = min(m, xch[v]);
      m = __builtin_amdgcn_readfirstlane(m);
    }
    return m;
  };
  // every candidate gains the pages of delta in word jj
  auto add_gain = [&](int jj, uint32_t delta) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < C; ++c) gain[c] += __builtin_popcount(b[c][jj] & delta);
  };

  int pos = 0, grp = 0;
  while (pos < Wr) {
    // ---- seed: the lowest unassigned ID owns the next group
    uint32_t key = kNone;
#pragma unroll
    for (int c = 0; c < C; ++c)
      if ((avail >> c) & 1u) key = min(key, (uint32_t)(cbase + 64 * c + lane));
    uint32_t best = window_min(key);
    int wb = best >> kShift, cb = (best >> 6) - C * wb, lb = best & 63;
    if (wb == wv && lane == lb) avail &= ~(1u << cb);
    if (wv == 0 && lane == 0) order[pos] = (int)best;
    ++pos;
    fetch(wb, cb, lb);
#pragma unroll
    for (int c = 0; c < C; ++c) gain[c] = 0;
#pragma unroll
    for (int jj = 0; jj < NWB; ++jj) {
      U[jj] = w[jj];
      if (w[jj]) add_gain(jj, w[jj]);
    }
    // ---- joins: the unassigned query adding the fewest new pages
    for (int members = 1; members < g && pos < Wr; ++members) {
      key = kNone;
#pragma unroll
      for (int c = 0; c < C; ++c)
        if ((avail >> c) & 1u)
          key = min(key, ((tot[c] - gain[c]) << 10) | (uint32_t)(cbase + 64 * c + lane));
      best = window_min(key) & 1023u;
      wb = best >> kShift;
      cb = (best >> 6) - C * wb;
      lb = best & 63;
      if (wb == wv && lane == lb) avail &= ~(1u << cb);
      if (wv == 0 && lane == 0) order[pos] = (int)best;
      ++pos;
      fetch(wb, cb, lb);
#pragma unroll
      for (int jj = 0; jj < NWB; ++jj) {
        const uint32_t d = w[jj] & ~U[jj];
        if (d) {
          U[jj] |= d;
          add_gain(jj, d);
        }
      }
    }
    // ---- the closed group's union size (pages), when the caller asks for it
    if (usz != nullptr) {
      int n = 0;
#pragma unroll
      for (int jj = 0; jj < NWB; ++jj) n += __builtin_popcount(U[jj]);
      if (wv == 0 && lane == 0) usz[grp] = n;
    }
    ++grp;
  }
}

// blockDim = 64 NWV: one wave per window (NWV = 1, W <= 256) or NWV waves
// of 256 candidates each (W <= 1024).
template <int C, int NWV>
__global__ __launch_bounds__(64 * NWV) void group_kernel(const int32_t* __restrict__ sel,
                                                         int32_t* __restrict__ ids, int T, int S,
                                                         int N, int W, int g, int n_windows,
                                                         int32_t* __restrict__ usize) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wv = NWV > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  uint32_t* stage = lds + wv * 64 * kStride;                      // [64][kStride] per wave
  int* order = reinterpret_cast<int*>(lds + NWV * 64 * kStride);  // [NWV C 64] emission order
  uint32_t* xch = lds + NWV * 64 * kStride + NWV * C * 64;        // [4 keys | 32 words]
  uint32_t* apg = xch + 36;                                       // [32] the window's pages
  int* wpre = reinterpret_cast<int*>(apg + 32);                   // [32] ranks before each word
  uint16_t* rank = reinterpret_cast<uint16_t*>(wpre + 32);        // [N] page -> rank
  const int h = blockIdx.x / n_windows;
  const int w0 = (blockIdx.x % n_windows) * W;
  const int Wr = min(W, T - w0);
  const int32_t* wbase = sel + ((size_t)h * T + w0) * S;
  // union sizes of this window's groups (W is a multiple of g: they start at group w0 / g)
  int32_t* usz = usize != nullptr ? usize + (size_t)h * ((T + g - 1) / g) + w0 / g : nullptr;
  // this wave's candidate rows
  const int r_lo = min(Wr, 64 * C * wv), r_hi = min(Wr, 64 * C * (wv + 1));

  // the window's pages (bitset apg over N <= 1024 pages), then every page's rank
  // among them: bitsets are kept over ranks, so their width follows the number
  // of distinct pages in the window, not how widely those pages are spread
  auto sync = [&]() __attribute__((always_inline)) {
    if constexpr (NWV > 1) __syncthreads(); else wave_sync();
  };
  if (N <= 256) {            // every page fits in 8 words: pages are their own ranks
    window_body<C, 8, NWV>(wbase, S, N, Wr, g, nullptr, stage, order, xch, usz);
    sync();
    for (int i = threadIdx.x; i < Wr; i += 64 * NWV) ids[(size_t)h * T + w0 + i] = w0 + order[i];
    return;
  }
  if (threadIdx.x < 32) apg[threadIdx.x] = 0;
  sync();
  if ((S & 3) == 0) {
    const int lo4 = (r_lo * S) >> 2, n4 = (r_hi * S) >> 2;
    const int4* w4 = reinterpret_cast<const int4*>(wbase);
    for (int i0 = lo4; i0 < n4; i0 += 64 * 8) {
      int4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + 64 * j + lane;
        v[j] = (i < n4) ? w4[i] : make_int4(-1, -1, -1, -1);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // one LDS atomic per run of entries in the same word of the page set
        const int e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        int wcur = -1;
        uint32_t bits = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bool ok = e[k] >= 0 && e[k] < N;
          const int wq = ok ? (e[k] >> 5) : -1;
          if (wq != wcur) {
            if (bits) atomicOr(&apg[wcur], bits);
            wcur = wq;
            bits = 0;
          }
          if (ok) bits |= 1u << (e[k] & 31);
        }
        if (bits) atomicOr(&apg[wcur], bits);
      }
    }
  } else {
    for (int i = r_lo * S + lane; i < r_hi * S; i += 64) {
      const int u = wbase[i];
      if (u >= 0 && u < N) atomicOr(&apg[u >> 5], 1u << (u & 31));
    }
  }
  sync();
  // exclusive prefix of the words' page counts (lanes 0..31 of every wave)
  const uint32_t aw = lane < 32 ? apg[lane] : 0u;
  int x = __builtin_popcount(aw);
#pragma unroll
  for (int d = 1; d < 32; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  const int n_act = __builtin_amdgcn_readlane(x, 31);
  if (wv == 0 && lane < 32) wpre[lane] = x - __builtin_popcount(aw);
  sync();
  for (int u = threadIdx.x; u < N; u += 64 * NWV)
    rank[u] = (uint16_t)(wpre[u >> 5] + __builtin_popcount(apg[u >> 5] & ((1u << (u & 31)) - 1u)));
  sync();
  if (n_act <= 256)
    window_body<C, 8, NWV>(wbase, S, N, Wr, g, rank, stage, order, xch, usz);
  else if (n_act <= 512)
    window_body<C, 16, NWV>(wbase, S, N, Wr, g, rank, stage, order, xch, usz);
  else
    window_body<C, 32, NWV>(wbase, S, N, Wr, g, rank, stage, order, xch, usz);
  sync();
  for (int i = threadIdx.x; i < Wr; i += 64 * NWV) ids[(size_t)h * T + w0 + i] = w0 + order[i];
}

template <int C, int NWV>
hipError_t launch_c(const pw_shape& s, const int32_t* sel, int W, int g, int32_t* ids,
                    int32_t* usize, hipStream_t stream) {
  const int n_windows = (s.T + W - 1) / W;
  const size_t lds =
      ((size_t)NWV * 64 * kStride + (size_t)NWV * C * 64 + 36 + 32 + 32) * 4 + (size_t)s.N_pages * 2;
  hipLaunchKernelGGL((group_kernel<C, NWV>), dim3(s.H_kv * n_windows), dim3(64 * NWV), lds,
                     stream, sel, ids, s.T, s.S, s.N_pages, W, g, n_windows, usize);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_group(const pw_shape& s, const int32_t* sel, int W, int g, int32_t* ids,
                        hipStream_t stream, int32_t* usize) {
  const int C = (W + 63) / 64;
  if (C <= 1) return launch_c<1, 1>(s, sel, W, g, ids, usize, stream);
  if (C == 2) return launch_c<2, 1>(s, sel, W, g, ids, usize, stream);
  if (C == 3) return launch_c<3, 1>(s, sel, W, g, ids, usize, stream);
  if (C == 4) return launch_c<4, 1>(s, sel, W, g, ids, usize, stream);
  if (W <= 512) return launch_c<4, 2>(s, sel, W, g, ids, usize, stream);
  if (W <= 768) return launch_c<4, 3>(s, sel, W, g, ids, usize, stream);
  return launch_c<4, 4>(s, sel, W, g, ids, usize, stream);
}

// ---- execution order of the groups: per KV head and block of consecutive
// groups, the block's groups by ascending union size, equal sizes in index
// order (a stable counting sort).  One workgroup of 16 waves per (KV head,
// block); wave w owns a contiguous segment of the block's groups.  The waves count their segments' sizes into per-wave LDS
// histograms; an exclusive scan over (size, wave) turns those into the first
// output position of every (wave, size); each wave then walks its segment 64
// groups at a time in index order, the lanes holding equal sizes finding each
// other with eleven ballots (one per bit of the size), so positions follow
// the index order without atomics.
namespace {

constexpr int kMaxUnion = 1024;          // union sizes are at most N_pages <= 1024
constexpr int kKeys = kMaxUnion + 1;
constexpr int kOrderWaves = 16;
// The attention keeps 256 waves resident per XCD (32 CUs x 8 waves); the groups
// those waves run at once are the ones whose page sweeps should stay in step, so
// the order sorts blocks of that many groups (256 / waves per group) and keeps
// the blocks themselves in index order.
constexpr int kResidentWavesPerXcd = 256;

__global__ __launch_bounds__(64 * kOrderWaves) void group_order_kernel(
    const int32_t* __restrict__ usize, int ngroups_head, int block, int32_t* __restrict__ order) {
  __shared__ int cnt[kOrderWaves][kKeys];
  __shared__ int wsum[kOrderWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this workgroup's block: `block` consecutive groups of one KV head
  const int nblk = (ngroups_head + block - 1) / block;
  const int hh = blockIdx.x / nblk, b0 = (blockIdx.x - hh * nblk) * block;
  const int ngroups = min(block, ngroups_head - b0);
  const int32_t* sz = usize + (size_t)hh * ngroups_head + b0;
  int32_t* out = order + (size_t)hh * ngroups_head + b0;
  const int seg = (ngroups + kOrderWaves - 1) / kOrderWaves;
  const int s0 = min(ngroups, wave * seg), s1 = min(ngroups, s0 + seg);
  auto key_of = [&](int i) __attribute__((always_inline)) {
    return min(max((int)sz[i], 0), kMaxUnion);
  };
  for (int i = tid; i < kOrderWaves * kKeys; i += 64 * kOrderWaves) (&cnt[0][0])[i] = 0;
  __syncthreads();
  // per-wave histograms of the segments (8 loads in flight per lane)
  for (int i0 = s0; i0 < s1; i0 += 64 * 8) {
    int k[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j + lane;
      k[j] = i < s1 ? key_of(i) : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k[j] >= 0) atomicAdd(&cnt[wave][k[j]], 1);
  }
  __syncthreads();
  // exclusive scan over keys of the totals (thread t: key t; the positions of the last
  // key, 1024, follow those of key 1023 and are set by thread 1023)
  constexpr int kT = 64 * kOrderWaves;
  static_assert(kT == kKeys - 1, "one key per thread plus the last");
  int tot = 0;
#pragma unroll
  for (int w = 0; w < kOrderWaves; ++w) tot += cnt[w][tid];
  int incl = tot;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int off = before + incl - tot;                       // first position of key tid
  // first position of every (wave, key): keys ascending, waves in index order
#pragma unroll
  for (int w = 0; w < kOrderWaves; ++w) {
    const int c = cnt[w][tid];
    cnt[w][tid] = off;
    off += c;
  }
  if (tid == kT - 1) {                                  // key kMaxUnion follows key 1023
#pragma unroll
    for (int w = 0; w < kOrderWaves; ++w) {
      const int c = cnt[w][kMaxUnion];
      cnt[w][kMaxUnion] = off;
      off += c;
    }
  }
  __syncthreads();
  // stable placement within each wave's segment
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i0 = s0; i0 < s1; i0 += 64) {
    const int i = i0 + lane;
    const bool live = i < s1;
    const int key = live ? key_of(i) : 0;
    uint64_t eq = __ballot(live);
#pragma unroll
    for (int b = 0; b < 11; ++b) {
      const uint64_t m = __ballot((key >> b) & 1);
      eq &= ((key >> b) & 1) ? m : ~m;
    }
    const int pos = live ? cnt[wave][key] + __popcll(eq & below) : 0;
    wave_sync();
    if (live) {
      out[pos] = b0 + i;
      if ((eq >> lane) == 1ull) cnt[wave][key] += __popcll(eq);   // the highest lane of its size
    }
    wave_sync();
  }
}

}  // namespace

hipError_t launch_group_order(const pw_shape& s, int g, const int32_t* usize, int32_t* order,
                              hipStream_t stream) {
  const int ngroups = (s.T + g - 1) / g;
  const int waves_per_group = (g * (s.H_q / s.H_kv) + 31) / 32;
  const int block = max(1, kResidentWavesPerXcd / waves_per_group);
  const int nblk = (ngroups + block - 1) / block;
  hipLaunchKernelGGL(group_order_kernel, dim3(s.H_kv * nblk), dim3(64 * kOrderWaves), 0, stream,
                     usize, ngroups, block, order);
  return hipGetLastError();
}

}  // namespace pw

// ---- query-ID check: per KV head, the number of entries that are out of
// range or repeat an earlier ID (0 for every head <=> each row is a permutation).
namespace pw {
namespace {

__global__ void ids_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

__global__ void ids_check_kernel(const int32_t* __restrict__ ids, int T, int Hkv,
                                 uint32_t* __restrict__ seen, int32_t* __restrict__ bad) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)T * Hkv) return;
  const int h = (int)(i / T);
  const int t = ids[i];
  bool wrong = t < 0 || t >= T;
  if (!wrong) {
    const size_t bit = (size_t)h * T + t;
    wrong = (atomicOr(&seen[bit >> 5], 1u << (bit & 31)) >> (bit & 31)) & 1u;
  }
  if (wrong) atomicAdd(&bad[h], 1);
}

}  // namespace

size_t check_ids_workspace(const pw_shape& s) {
  return ((size_t)s.H_kv * s.T + 31) / 32 * 4;
}

hipError_t launch_check_ids(const pw_shape& s, const int32_t* ids, int32_t* bad, void* ws,
                            hipStream_t stream) {
  uint32_t* seen = static_cast<uint32_t*>(ws);
  const size_t nw = check_ids_workspace(s) / 4;
  hipLaunchKernelGGL(ids_zero_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream,
                     seen, nw);
  hipLaunchKernelGGL(ids_zero_kernel, dim3(1), dim3(64), 0, stream,
                     reinterpret_cast<uint32_t*>(bad), (size_t)s.H_kv);
  const size_t n = (size_t)s.H_kv * s.T;
  hipLaunchKernelGGL(ids_check_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     ids, s.T, s.H_kv, seen, bad);
  return hipGetLastError();
}

}  // namespace pw
