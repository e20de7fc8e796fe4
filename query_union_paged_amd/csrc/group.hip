// Bounded-window greedy grouping of queries by selected-page affinity.
//
// "PageWeaver: KV-Guided Query Unions for Sparse Attention", Abstract: a
// bounded GPU search produces query IDs (nothing else).  AI Radio episode on
// the paper, "Paper summary": within a bounded window the members of a
// query-owned group are collected greedily, taking queries whose selected
// sets add few new pages; g is fixed independently of the window W.
//
// One workgroup per (KV head, aligned window).  Thread c owns candidate c of
// the window and keeps its page bitset in registers; the window's bitsets
// also sit in LDS (word-major, so thread c's words are conflict-free and the
// winner's words are read as broadcasts).  Every step is one workgroup-wide
// minimum over the key (cost << 10 | local index): the lowest index wins
// ties, so the result is deterministic and bit-exact.  After a join only the
// newly added pages (delta = B_best & ~U) are subtracted from each
// candidate's cost.
#include "pw_internal.h"

namespace pw {
namespace {

constexpr uint32_t kNone = 0xFFFFFFFFu;

// Workgroup minimum.  `red` holds two slot sets used on alternate steps, so
// one barrier per step suffices: a wave can only overwrite a slot set after
// every wave has passed the barrier of the step in between.
__device__ __forceinline__ uint32_t block_min(uint32_t v, uint32_t* red, int parity,
                                              int nwaves) {
  v = wave_min_u32(v);
  if (nwaves == 1) return v;
  if ((threadIdx.x & 63) == 0) red[parity * 4 + (threadIdx.x >> 6)] = v;
  __syncthreads();
  uint32_t r = red[parity * 4];
  for (int i = 1; i < nwaves; ++i) r = min(r, red[parity * 4 + i]);
  return r;
}

template <int NWMAX>
__global__ __launch_bounds__(256) void group_kernel(const int32_t* __restrict__ sel,
                                                    int32_t* __restrict__ ids, int T, int S,
                                                    int N, int W, int g, int n_windows) {
  extern __shared__ uint32_t lds[];
  const int nw = (N + 31) >> 5;
  const int nthreads = blockDim.x;            // multiple of 64, >= W
  const int nwaves = nthreads >> 6;
  const int h = blockIdx.x / n_windows;
  const int w0 = (blockIdx.x % n_windows) * W;
  const int Wr = min(W, T - w0);
  const int tid = threadIdx.x;

  uint32_t* bits = lds;                                   // [nw][nthreads]
  int* order = reinterpret_cast<int*>(lds + nw * nthreads);   // [nthreads]
  uint32_t* red = reinterpret_cast<uint32_t*>(order + nthreads);  // [2][4]

  for (int i = tid; i < nw * nthreads; i += nthreads) bits[i] = 0;
  __syncthreads();
  // The window's selection rows are one contiguous block: read it coalesced.
  const int32_t* base = sel + ((size_t)h * T + w0) * S;
  for (int i = tid; i < Wr * S; i += nthreads) {
    const int u = base[i];
    if (u >= 0 && u < N) atomicOr(&bits[(u >> 5) * nthreads + i / S], 1u << (u & 31));
  }
  __syncthreads();

  uint32_t b[NWMAX];
#pragma unroll
  for (int j = 0; j < NWMAX; ++j) b[j] = (j < nw) ? bits[j * nthreads + tid] : 0u;
  uint32_t U[NWMAX];
  bool avail = tid < Wr;
  uint32_t cost = 0;
  int pos = 0, step = 0;

  while (pos < Wr) {
    // Seed: the lowest unassigned ID owns the next group.
    const uint32_t seed = block_min(avail ? (uint32_t)tid : kNone, red, step++ & 1, nwaves);
    if (tid == (int)seed) avail = false;
    if (tid == 0) order[pos] = (int)seed;
    ++pos;
    cost = 0;
#pragma unroll
    for (int j = 0; j < NWMAX; ++j) {
      U[j] = (j < nw) ? bits[j * nthreads + seed] : 0u;
      cost += __builtin_popcount(b[j] & ~U[j]);
    }
    for (int members = 1; members < g && pos < Wr; ++members) {
      const uint32_t key = avail ? ((cost << 10) | (uint32_t)tid) : kNone;
      const uint32_t best = block_min(key, red, step++ & 1, nwaves) & 1023u;
      if (tid == (int)best) avail = false;
      if (tid == 0) order[pos] = (int)best;
      ++pos;
#pragma unroll
      for (int j = 0; j < NWMAX; ++j) {
        if (j < nw) {
          const uint32_t d = bits[j * nthreads + best] & ~U[j];
          U[j] |= d;
          cost -= __builtin_popcount(b[j] & d);
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < Wr; i += nthreads) ids[(size_t)h * T + w0 + i] = w0 + order[i];
}

template <int NWMAX>
hipError_t launch_nw(const pw_shape& s, const int32_t* sel, int W, int g, int32_t* ids,
                     hipStream_t stream) {
  const int n_windows = (s.T + W - 1) / W;
  const int threads = ((W + 63) / 64) * 64;
  const int nw = (s.N_pages + 31) / 32;
  const size_t lds = (size_t)nw * threads * 4 + (size_t)threads * 4 + 8 * 4;
  hipLaunchKernelGGL(group_kernel<NWMAX>, dim3(s.H_kv * n_windows), dim3(threads), lds, stream,
                     sel, ids, s.T, s.S, s.N_pages, W, g, n_windows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_group(const pw_shape& s, const int32_t* sel, int W, int g, int32_t* ids,
                        hipStream_t stream) {
  const int nw = (s.N_pages + 31) / 32;
  if (nw <= 2) return launch_nw<2>(s, sel, W, g, ids, stream);
  if (nw <= 4) return launch_nw<4>(s, sel, W, g, ids, stream);
  if (nw <= 8) return launch_nw<8>(s, sel, W, g, ids, stream);
  if (nw <= 16) return launch_nw<16>(s, sel, W, g, ids, stream);
  return launch_nw<32>(s, sel, W, g, ids, stream);
}

}  // namespace pw
