// Bounded-window greedy grouping of queries by selected-page affinity.
//
// "PageWeaver: KV-Guided Query Unions for Sparse Attention", Abstract: a
// bounded GPU search produces query IDs (nothing else).  AI Radio episode on
// the paper, "Paper summary": within a bounded window the members of a
// query-owned group are collected greedily, taking queries whose selected
// sets add few new pages; g is fixed independently of the window W.
//
// One wave per (KV head, aligned window).  Lane l owns candidates l, l+64,
// l+128, ... (C = ceil(W/64) of them) and keeps their page bitsets in VGPRs;
// the group union U is wave-uniform and lives in scalar registers.  A step is
// a wave minimum of key = (cost << 10 | local index) over the available
// candidates (DPP within rows of 16, then four readlanes), so the lowest
// index wins ties and the result is bit-exact.  The winner's words are read
// with readlane from the owning lane; only the words where the winner brings
// new pages (delta = B_best & ~U) touch the candidates' costs.
#include "pw_internal.h"

namespace pw {
namespace {

constexpr uint32_t kNone = 0xFFFFFFFFu;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_min(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
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

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false);
  return __builtin_amdgcn_readlane(v, 0) | __builtin_amdgcn_readlane(v, 16) |
         __builtin_amdgcn_readlane(v, 32) | __builtin_amdgcn_readlane(v, 48);
}

// The greedy loop of one window, with the window's active words compacted into
// NWB register words per candidate (NWB >= number of active words; the words
// past it are zero for every candidate and cost nothing).
template <int C, int NWB>
__device__ __forceinline__ void window_body(const int32_t* __restrict__ wbase, int S, int N,
                                            int Wr, int g, uint32_t act, uint32_t* stage,
                                            int* order) {
  constexpr int STR = NWB + 1;             // padded row: conflict-free column reads
  const int lane = threadIdx.x;
  uint32_t b[C][NWB];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    for (int i = lane; i < 64 * STR; i += 64) stage[i] = 0;
    wave_sync();
    const int r0 = 64 * c;
    const int nrows = max(0, min(64, Wr - r0));
    const int32_t* base = wbase + (size_t)r0 * S;
    for (int i = lane; i < nrows * S; i += 64) {
      const int u = base[i];
      if (u >= 0 && u < N) {
        const int jj = __builtin_popcount(act & ((1u << (u >> 5)) - 1u));   // compacted word
        atomicOr(&stage[(i / S) * STR + jj], 1u << (u & 31));
      }
    }
    wave_sync();
#pragma unroll
    for (int jj = 0; jj < NWB; ++jj) b[c][jj] = stage[lane * STR + jj];
    wave_sync();
  }

  uint32_t U[NWB];
  uint32_t cost[C];
  uint32_t avail = 0;                      // bit c: candidate 64c + lane unassigned
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (64 * c + lane < Wr) avail |= 1u << c;

  int pos = 0;
  while (pos < Wr) {
    // ---- seed: the lowest unassigned ID owns the next group
    uint32_t key = kNone;
#pragma unroll
    for (int c = 0; c < C; ++c)
      if ((avail >> c) & 1u) key = min(key, (uint32_t)(64 * c + lane));
    uint32_t best = __builtin_amdgcn_readfirstlane(wave_min_dpp(key));
    int cb = best >> 6, lb = best & 63;
    if (lane == lb) avail &= ~(1u << cb);
    if (lane == 0) order[pos] = (int)best;
    ++pos;
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (c == cb) {
#pragma unroll
        for (int jj = 0; jj < NWB; ++jj) U[jj] = __builtin_amdgcn_readlane(b[c][jj], lb);
      }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      uint32_t x = 0;
#pragma unroll
      for (int jj = 0; jj < NWB; ++jj) x += __builtin_popcount(b[c][jj] & ~U[jj]);
      cost[c] = x;
    }
    // ---- joins: the unassigned query adding the fewest new pages
    for (int members = 1; members < g && pos < Wr; ++members) {
      key = kNone;
#pragma unroll
      for (int c = 0; c < C; ++c)
        if ((avail >> c) & 1u) key = min(key, (cost[c] << 10) | (uint32_t)(64 * c + lane));
      best = __builtin_amdgcn_readfirstlane(wave_min_dpp(key) & 1023u);
      cb = best >> 6;
      lb = best & 63;
      if (lane == lb) avail &= ~(1u << cb);
      if (lane == 0) order[pos] = (int)best;
      ++pos;
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (c == cb) {
#pragma unroll
          for (int jj = 0; jj < NWB; ++jj) {
            const uint32_t d = __builtin_amdgcn_readlane(b[c][jj], lb) & ~U[jj];
            if (d) {
              U[jj] |= d;
#pragma unroll
              for (int c2 = 0; c2 < C; ++c2) cost[c2] -= __builtin_popcount(b[c2][jj] & d);
            }
          }
        }
    }
  }
}

template <int C>
__global__ __launch_bounds__(64) void group_kernel(const int32_t* __restrict__ sel,
                                                   int32_t* __restrict__ ids, int T, int S,
                                                   int N, int W, int g, int n_windows) {
  extern __shared__ uint32_t lds[];
  uint32_t* stage = lds;                                  // [64][33] one candidate chunk
  int* order = reinterpret_cast<int*>(lds + 64 * 33);     // [C * 64] emission order
  const int lane = threadIdx.x;
  const int h = blockIdx.x / n_windows;
  const int w0 = (blockIdx.x % n_windows) * W;
  const int Wr = min(W, T - w0);
  const int32_t* wbase = sel + ((size_t)h * T + w0) * S;

  // words (32 pages each) that some candidate of the window uses
  uint32_t act = 0;
  for (int i = lane; i < Wr * S; i += 64) {
    const int u = wbase[i];
    if (u >= 0 && u < N) act |= 1u << (u >> 5);
  }
  act = wave_or(act);
  const int nact = __builtin_popcount(act);
  if (nact <= 8)
    window_body<C, 8>(wbase, S, N, Wr, g, act, stage, order);
  else if (nact <= 16)
    window_body<C, 16>(wbase, S, N, Wr, g, act, stage, order);
  else
    window_body<C, 32>(wbase, S, N, Wr, g, act, stage, order);
  wave_sync();
  for (int i = lane; i < Wr; i += 64) ids[(size_t)h * T + w0 + i] = w0 + order[i];
}

template <int C>
hipError_t launch_c(const pw_shape& s, const int32_t* sel, int W, int g, int32_t* ids,
                    hipStream_t stream) {
  const int n_windows = (s.T + W - 1) / W;
  const size_t lds = (size_t)64 * 33 * 4 + (size_t)C * 64 * 4;
  hipLaunchKernelGGL(group_kernel<C>, dim3(s.H_kv * n_windows), dim3(64), lds, stream, sel, ids,
                     s.T, s.S, s.N_pages, W, g, n_windows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_group(const pw_shape& s, const int32_t* sel, int W, int g, int32_t* ids,
                        hipStream_t stream) {
  const int C = (W + 63) / 64;
  if (C <= 1) return launch_c<1>(s, sel, W, g, ids, stream);
  if (C == 2) return launch_c<2>(s, sel, W, g, ids, stream);
  if (C == 3) return launch_c<3>(s, sel, W, g, ids, stream);
  return launch_c<4>(s, sel, W, g, ids, stream);
}

}  // namespace pw
