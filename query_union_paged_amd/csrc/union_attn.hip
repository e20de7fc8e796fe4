// ID-aware query-union attention over a paged FP8 KV cache (gfx950).
//
// "PageWeaver: KV-Guided Query Unions for Sparse Attention", Abstract: query
// unions share page loads and fill matrix-core tiles; every query keeps its
// original support and sole ownership of its output; the kernel consumes
// query IDs without materialising a reordered Q tensor or cross-page partial
// outputs.
//
// Mapping on CDNA4.  A pre-pass (tile_kv_kernel) rewrites the FP8 K and V
// pages of the call into MFMA operand order, 64 key slots per page.  One wave
// then owns one 32-row tile of one group (g query IDs of one KV head, M = g*G
// query rows <= 64, so one or two waves per group) and walks the group's union
// of pages in ascending page order; four waves share a workgroup only for
// scheduling.  Per page (64 keys):
//   S^T = K_page * Q^T     v_mfma_scale_f32_32x32x64_f8f6f4 on the e4m3 codes
//                          and a two-part e4m3 split of each bf16 Q row
//                          (hi + lo: exact for elements >= 2^-2 after the
//                          row's power-of-two scaling, within 2^-10 below);
//                          keys are the MFMA rows and query rows the columns,
//                          so each lane holds one query row (lane & 31) and 32
//                          of its 64 keys;
//   online softmax         fp32 in registers, log2 domain, lazy rescale; row
//                          max/sum finished with one cross-half lane swap; the
//                          max pass is skipped when |q| * max |k| shows that no
//                          score of the page can move any row's reference;
//   O^T += V_page^T * P^T  v_mfma_f32_32x32x16_bf16 with the V codes converted
//                          to bf16 exactly; d is the MFMA row.
// Page loads are contiguous 1 KB wave reads of the tiled copy straight into
// operand registers.  A group of at most 32 rows (G = 4, g = 8) is one wave,
// which loads each union page once; a 64-row group (G = 8) is two waves, each
// walking the union of its own four members' pages (pages selected in both
// halves cross the vector memory path twice per group).  The per-page scales are folded into the
// scores (k) and into the exponent (v).  The key order inside the 32-row K
// tiles is permuted so that the PV operands of every lane are 32 consecutive
// keys of one d in the tiled V copy.
//
// Ownership.  A row whose query did not select a page gets p = 0 and its
// running max untouched on that page (alpha = 1 exactly), so its result is
// the same whichever group it sits in; each (query, Q head) row is written
// once, by its wave.  There are no atomics and no partial outputs.
#include "attn_common.h"

#ifndef PW_UA_WG_WAVES
#define PW_UA_WG_WAVES 4  // waves (independent groups) per workgroup
#endif

namespace pw {
namespace {

struct UAParams {
  const uint16_t* Q;
  const uint8_t* Kt;   // tiled copies of the FP8 K and V pages (see tile_kv_kernel)
  const uint8_t* Vt;
  const float* scales;
  const float4* pf;    // [N][Hkv] page factors (tile_kv_kernel): k_scale * qk_scale,
                       // score bound factor, log2(v_scale), 1 / v_scale
  const int32_t* sel;
  const int32_t* ids;
  uint16_t* O;
  int T, Hq, Hkv, G, P, N, S, g;
  int groups_per_head, total_groups;
  const int32_t* order;  // optional [H_kv][groups_per_head]: execution order of each head's groups
  int h_begin;       // first KV head of the call (groups cover heads h_begin ...)
  int n_rt;          // 32-row tiles per group (ceil(g * G / 32)): one wave each
  int total_items;   // total_groups * n_rt
  int n_umax;        // list capacity per wave (>= any union size)
  int lds_wave;      // bytes of LDS per wave
  float qk_scale;    // log2(e) / sqrt(D)
  // page-pair mode (direct KV-page union): per (KV head, pair) entry lists
  const int2* plist;   // [H_kv][Np][Tc] (token - t0, partial slot | pages << 30)
  const int* pcount;   // [H_kv][Np] entries per list
  const int* tstart;   // [H_kv][Np + 1] first tile of each pair's list; [Np] = tiles of the head
  const int2* pairs;   // [H_kv][Np] the pair's pages (lower first, second -1 if single);
                       // null: pair k is pages (2k, 2k + 1)
  float* partials;     // [slot][G][D + 4]: m, l, -, -, acc[D]
  int Np, Tc, t0, tiles_head;
};

enum : int { kUnionMode = 0, kPairMode = 1, kFp8Mode = 2 };

// Re-tiles the FP8 pages of one layer into MFMA operand order (one workgroup
// per (page, KV head) block of 64 key slots x D bytes, for K and for V; both
// cache pages are token-major [P][D]):
//   K chunk (kt, c, l) = K[tile_key(l % 32, kt)][(D/2)(l/32) + 16c .. +16)
//   V chunk (dt, j, l) = V[32 (l/32) + 16 j .. +16][32 dt + l % 32]   (16 keys of one d)
// at byte 16 * ((kt * D/32 + c) * 64 + l), resp. 16 * ((2 dt + j) * 64 + l);
// key slots >= P are zero.  The attention loop then reads each page with
// contiguous 1 KB wave loads instead of one 128-byte row per lane.  A V chunk
// gathers one column of the page: the page is staged in LDS and each thread
// transposes 4 x 4 byte blocks (4 keys x 4 consecutive d) into 4 chunks of
// consecutive lanes.
// The same pass stores the page's uniform softmax factors pf[u][h] = {c, kn * |c|,
// log2(v_scale), 1 / v_scale} with c = k_scale * log2(e) / sqrt(D) and kn =
// (1 + 2^-9) * the largest Euclidean norm of the page's decoded e4m3 key codes:
// kn * |c| times the norm of a query row bounds every score of that row on the
// page (log2 units).  The attention loop then reads them with one scalar load.
template <int D>
__global__ __launch_bounds__(256) void tile_kv_kernel(const uint8_t* __restrict__ K,
                                                      const uint8_t* __restrict__ V,
                                                      const float* __restrict__ scales,
                                                      float qk_scale,
                                                      uint8_t* __restrict__ Kt,
                                                      uint8_t* __restrict__ Vt,
                                                      float4* __restrict__ pf, int N, int P,
                                                      int Hkv, int h_begin, int h_count) {
  constexpr int KCH = D / 32, DT = D / 32;
  __shared__ uint4 vpage[64 * D / 16];        // the V page, 64 key rows (rows >= P zero)
  // one block per (page, head) of heads h_begin .. h_begin + h_count - 1
  const size_t blk = (size_t)(blockIdx.x / h_count) * Hkv + h_begin + blockIdx.x % h_count;
  const uint8_t* kp = K + blk * P * D;
  const uint8_t* vp = V + blk * P * D;
  uint8_t* kt_out = Kt + blk * 64 * D;
  uint8_t* vt_out = Vt + blk * 64 * D;
  for (int i = threadIdx.x; i < 64 * D / 16; i += blockDim.x) {
    const int key = i / (D / 16);
    vpage[i] = (key < P) ? load16(vp + 16 * (size_t)i) : make_uint4(0, 0, 0, 0);
  }
  for (int q = threadIdx.x; q < 2 * KCH * 64; q += blockDim.x) {
    const int l = q & 63, kc = q >> 6, kt = kc / KCH, c = kc - kt * KCH;
    const int key = tile_key(l & 31, kt);
    const uint4 v = (key < P) ? load16(kp + (size_t)key * D + (D / 2) * (l >> 5) + 16 * c)
                              : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(kt_out + 16 * q) = v;
  }
  __syncthreads();
  // V: work item (dt, j, l4) writes the chunks of lanes 4 l4 .. 4 l4 + 3 of
  // chunk row 2 dt + j: d = d0 .. d0 + 3, keys k0 .. k0 + 15.
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(vpage);
  for (int w = threadIdx.x; w < 2 * DT * 16; w += blockDim.x) {
    const int l = 4 * (w & 15), dj = w >> 4, dt = dj >> 1, j = dj & 1;
    const int d0 = 32 * dt + (l & 31), k0 = 32 * (l >> 5) + 16 * j;
    uint32_t out[4][4];                       // out[i][kq]: d0 + i, keys k0 + 4 kq .. + 3
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      uint32_t r[4];                          // r[m]: bytes d0 .. d0 + 3 of key k0 + 4 kq + m
#pragma unroll
      for (int m = 0; m < 4; ++m) r[m] = vw[((k0 + 4 * kq + m) * D + d0) >> 2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[i][kq] = ((r[0] >> (8 * i)) & 0xFFu) | (((r[1] >> (8 * i)) & 0xFFu) << 8) |
                     (((r[2] >> (8 * i)) & 0xFFu) << 16) | (((r[3] >> (8 * i)) & 0xFFu) << 24);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(vt_out + 16 * ((2 * dt + j) * 64 + l + i)) =
          make_uint4(out[i][0], out[i][1], out[i][2], out[i][3]);
  }
  // key norms: four threads per key slot, D / 4 codes each
  __shared__ float wmax[4];
  const int key = threadIdx.x >> 2, part = threadIdx.x & 3;
  float ss = 0.f;
  if (key < P) {
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      const uint4 v = load16(kp + (size_t)key * D + (D / 4) * part + 16 * c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
        const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
        ss = fmaf(a[0], a[0], ss);
        ss = fmaf(a[1], a[1], ss);
        ss = fmaf(b[0], b[0], ss);
        ss = fmaf(b[1], b[1], ss);
      }
    }
  }
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) ss = fmaxf(ss, __shfl_xor(ss, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float kn = sqrtf(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))) * kNormSlack;
    const float c = scales[blk] * qk_scale;
    const float vs = scales[(size_t)N * Hkv + blk];
    pf[blk] = make_float4(c, kn * fabsf(c), __builtin_amdgcn_logf(vs), __builtin_amdgcn_rcpf(vs));
  }
}

// MODE kUnionMode: groups of query IDs, union of their selected pages, O out.
// MODE kPairMode: up to 8 entries of one page pair's membership list, the pair's
// pages they selected, unnormalised partials out (direct KV-page union).
// MODE kFp8Mode: as kUnionMode with Q and P rounded to e4m3fn per row, QK^T on
// K Qhi^T alone and PV on the FP8 MFMA (a lower-precision variant).
template <int D, int P, int MODE>
__global__ __launch_bounds__(64 * PW_UA_WG_WAVES, 2) void union_attn_kernel(UAParams p) {
  // P in {16, 32, 64} keys per page; the tiled pages always hold 64 key slots
  // (slots >= P are zero and masked here).
  constexpr int KCH = D / 32;    // uint4 chunks of K per lane per key tile
  constexpr int DT = D / 32;     // output tiles over d (PV)
  extern __shared__ __align__(16) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5;      // lane half
  const int col = lane & 31;     // query row within a tile

  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
  // each XCD sweeps a contiguous range of groups (one KV head's pages stay in
  // that XCD's L2).
  // Each XCD takes its range from the top down: late queries have the largest
  // supports, so the cheap early groups are the ones left for the tail.  With a
  // group order, sweep position k of a head runs group order[h][k] instead (the
  // search's order by ascending union size: largest unions first, and unions of
  // similar size side by side, whose ascending page sweeps stay in step).
  const int nb = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, per = nb >> 3, extra = nb & 7;
  const int cnt = per + (xcd < extra ? 1 : 0);       // workgroups of this XCD
  const int lb = xcd * per + min(xcd, extra) + (cnt - 1 - (b >> 3));
  const int wid = lb * PW_UA_WG_WAVES + wave;
  if (wid >= p.total_items) return;
  const int rt = wid % p.n_rt;              // which 32-row tile of the group
  const int gid = wid / p.n_rt;

  unsigned char* wbase = smem + (size_t)wave * p.lds_wave;
  uint32_t* list = reinterpret_cast<uint32_t*>(wbase);        // page | members << 16
  int h, gm, n_u = 0;
  int my_t = -1, my_slot = -1;              // lane i < gm: member i's token (and slot)
  // The slots (members) whose rows this wave holds: rows 32 rt .. 32 rt + 31 are slot * G +
  // head.  A page that none of them selected leaves every row of the wave as it is (p = 0,
  // alpha = 1), so with two row tiles per group each wave walks only its own slots' pages.
  const int s_lo = (32 * rt) / p.G, s_hi = (32 * rt + 31) / p.G;       // inclusive

  if constexpr (MODE != kPairMode) {
  const int hl = gid / p.groups_per_head;
  h = p.h_begin + hl;
  int k = gid - hl * p.groups_per_head;
  if (p.order != nullptr) {
    k = p.order[(size_t)h * p.groups_per_head + k];
    if (k < 0 || k >= p.groups_per_head) return;       // not a group index: nothing to run
  }
  const int g0 = k * p.g;
  gm = min(p.g, p.T - g0);
  const int nw = (p.N + 31) >> 5;              // words of the page bitset
  uint32_t* bits = reinterpret_cast<uint32_t*>(wbase + (size_t)p.n_umax * 4);
  int* prefix = reinterpret_cast<int*>(bits + nw);  // union pages before each word
  if (lane < gm) {
    const int t = p.ids[(size_t)h * p.T + g0 + lane];
    my_t = (t >= 0 && t < p.T) ? t : -1;
  }

  // ---- union + membership.  A page bitset marks the union; a scan of its words
  // gives the ascending page list and, per word, the list position of its first
  // page; then each (page, member) entry ORs its member bit into the upper half
  // of that page's list entry.  LDS use is N/4 bytes + 4 per list entry, so N
  // up to the supported maximum fits.
  for (int i = lane; i < nw; i += 64) bits[i] = 0;
  wave_sync();
  constexpr int MAXIT = 16;          // g * S <= 1024 entries
  int pg[MAXIT];
  {
    const int n_ent = gm * p.S;
    if ((p.S & 3) == 0) {
      // lane l takes slots 4 (l + 64 j) .. + 3, four consecutive slots of one member (one
      // 16-byte load); selection rows are usually sorted, so entries in the same bitset word
      // share one LDS atomic
#pragma unroll
      for (int j = 0; j < MAXIT / 4; ++j) {
        const int e0 = 4 * (lane + 64 * j);
        const int i = e0 / p.S;
        const int t = __shfl(my_t, i & 63);
        int4 v = make_int4(-1, -1, -1, -1);
        if (e0 < n_ent && t >= 0)
          v = *reinterpret_cast<const int4*>(p.sel + ((size_t)h * p.T + t) * p.S + (e0 - i * p.S));
        const int e4[4] = {v.x, v.y, v.z, v.w};
        int wcur = -1;
        uint32_t word_bits = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = e4[q];
          const bool ok = u >= 0 && u < p.N && i >= s_lo && i <= s_hi;
          pg[4 * j + q] = ok ? (u | (i << 16)) : -1;
          const int wq = ok ? (u >> 5) : -1;
          if (wq != wcur) {
            if (word_bits) atomicOr(&bits[wcur], word_bits);
            wcur = wq;
            word_bits = 0;
          }
          if (ok) word_bits |= 1u << (u & 31);
        }
        if (word_bits) atomicOr(&bits[wcur], word_bits);
      }
    } else {
#pragma unroll
      for (int it = 0; it < MAXIT; ++it) {
        const int e = lane + 64 * it;
        const int i = e / p.S;
        const int t = __shfl(my_t, i & 63);
        pg[it] = -1;
        if (e < n_ent && t >= 0) pg[it] = p.sel[((size_t)h * p.T + t) * p.S + (e - i * p.S)];
        pg[it] = (pg[it] >= 0 && pg[it] < p.N && i >= s_lo && i <= s_hi) ? (pg[it] | (i << 16)) : -1;
      }
#pragma unroll
      for (int it = 0; it < MAXIT; ++it)
        if (pg[it] >= 0) atomicOr(&bits[(pg[it] & 0xFFFF) >> 5], 1u << (pg[it] & 31));
    }
  }
  wave_sync();
  for (int c0 = 0; c0 < nw; c0 += 64) {
    const int w = c0 + lane;
    uint32_t x = (w < nw) ? bits[w] : 0u;
    const int cnt = __builtin_popcount(x);
    int incl = cnt;                    // inclusive scan of the word counts over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    int pos = n_u + incl - cnt;
    if (w < nw) prefix[w] = pos;
    while (x) {
      list[pos++] = (uint32_t)(32 * w + __builtin_ctz(x));
      x &= x - 1u;
    }
    n_u += __shfl(incl, 63);
  }
  wave_sync();
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    if (pg[it] >= 0) {
      const int u = pg[it] & 0xFFFF, i = pg[it] >> 16;
      const int r = prefix[u >> 5] + __builtin_popcount(bits[u >> 5] & ((1u << (u & 31)) - 1u));
      atomicOr(&list[r], (1u << i) << 16);
    }
  }
  wave_sync();
  } else {
  // Tile slot j of KV head h: the pairs' lists are cut into tiles of 8 entries,
  // numbered consecutively over the pairs (tstart); slots past the head's
  // last tile exit.  Pair k is the one with tstart[k] <= j < tstart[k + 1].
  const int j = gid % p.tiles_head;
  h = gid / p.tiles_head;
  const int* ts = p.tstart + (size_t)h * (p.Np + 1);
  if (j >= __builtin_amdgcn_readfirstlane(ts[p.Np])) return;
  int lo = 0, hi = p.Np;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(ts[mid]) <= j) lo = mid; else hi = mid;
  }
  const int k = lo;
  const int tile = j - __builtin_amdgcn_readfirstlane(ts[k]);
  const int hk = h * p.Np + k;
  const int cnt = p.pcount[hk];
  gm = min(8, cnt - 8 * tile);
  if (gm <= 0) return;
  int pa = 2 * k, pb = 2 * k + 1;
  if (p.pairs != nullptr) {
    const int2 pr = p.pairs[hk];
    pa = __builtin_amdgcn_readfirstlane(pr.x);
    pb = __builtin_amdgcn_readfirstlane(pr.y);
  }
  int kind = 0;
  if (lane < gm) {
    const int2 e = p.plist[(size_t)hk * p.Tc + 8 * tile + lane];
    my_t = p.t0 + e.x;
    my_slot = e.y & 0x3FFFFFFF;
    kind = (e.y >> 30) & 3;                 // bit 0: the pair's first page selected, bit 1: second
  }
  const uint32_t own = ((2u << s_hi) - (1u << s_lo)) & 0xFFu;    // this wave's slots
  const uint32_t m0 = (uint32_t)__ballot(kind & 1) & own;
  const uint32_t m1 = (uint32_t)__ballot(kind & 2) & own;
  if (m0) list[n_u++] = (uint32_t)pa | (m0 << 16);
  if (m1) list[n_u++] = (uint32_t)pb | (m1 << 16);
  wave_sync();
  }
  const int tmin = __builtin_amdgcn_readfirstlane(
      (int)wave_min_u32(my_t >= 0 ? (uint32_t)my_t : 0xFFFFFFFFu));

  // ---- the lane's query row (32 rows per wave: row n = slot * G + head)
  const int n = 32 * rt + col;
  const int s_ = n / p.G;
  const int t_ = __shfl(my_t, s_ & 63);
  const bool ok = (s_ < gm) && (t_ >= 0);
  const int slot = ok ? s_ : -1, trow = ok ? t_ : -1;
  const int pslot = __shfl(my_slot, s_ & 63);
  const int qhead = h * p.G + (n - s_ * p.G);
  QRow<D> qr;
  load_q_row<D, MODE != kFp8Mode>(p.Q + ((size_t)(ok ? t_ : 0) * p.Hq + qhead) * D + (D / 2) * hf,
                                  ok, qr);

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  // K and V come from the tiled copies (tile_kv_kernel): the block of (page u,
  // KV head h) holds 64 key slots x D in MFMA operand order, so every load
  // below is one contiguous 1 KB read of the wave (lane l at 16 * l).
  uint4 kbuf[2][KCH], vbuf[DT][2];
  f32x16 sacc[2];
  float4 pfr = make_float4(0.f, 0.f, 0.f, 0.f);
  const int block_bytes = 64 * D;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Kt, (short)0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Vt, (short)0, 0x7FFFFFFF, 0x00020000);
  const int loff = 16 * lane;       // the only per-lane part of a page load's address
  auto block_of = [&](int u) {     // wave-uniform: a scalar offset, no per-lane address
    return __builtin_amdgcn_readfirstlane((u * p.Hkv + h) * block_bytes);
  };
  auto load_k = [&](uint4 (&kr)[2][KCH], int u) {
    const int so = block_of(u);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < KCH; ++c)
        kr[kt][c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  krs, loff, so + 1024 * (kt * KCH + c), 0));
  };
  auto load_v = [&](uint4 (&vr)[DT][2], int u) {
    const int so = block_of(u);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        vr[dt][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  vrs, loff, so + 1024 * (2 * dt + j), 0));
  };
  const float4* pfac = p.pf + h;                            // [N][Hkv]

  // One page of K/V ahead, two waves per SIMD overlapping each other's matrix
  // and vector work.  (Software-pipelined schedules that keep the next page's
  // scores in flight during the softmax need more than the 256 registers a
  // wave has at this occupancy; they spilled and ran slower.)
  // The list entry of the next page (page in the low half, member mask in the
  // high half) is read once, one page ahead, and carried into the next step:
  // one LDS read per page, and none after the page factors' scalar load, whose
  // wait therefore falls a whole page later.
  uint32_t ent_nx = 0;
  if (n_u > 0) {
    ent_nx = (uint32_t)__builtin_amdgcn_readfirstlane((int)list[0]);
    const int u0 = (int)(ent_nx & 0xFFFF);
    load_k(kbuf, u0);
    load_v(vbuf, u0);
    pfr = pfac[(size_t)u0 * p.Hkv];
  }
  bf16x8 pB[4];
  i32x8 pF;
  int vsb = 127;
  for (int up = 0; up < n_u; ++up) {
    const uint32_t ent = ent_nx;
    const float4 pf_c = pfr;
    ent_nx = (uint32_t)__builtin_amdgcn_readfirstlane((int)list[min(up + 1, n_u - 1)]);
    const int u1 = (int)(ent_nx & 0xFFFF);
    qk_page<D, MODE == kFp8Mode ? 1 : 2>(kbuf, qr, sacc);
    load_k(kbuf, u1);                     // K registers are free once the MFMAs have read them
    pfr = pfac[(size_t)u1 * p.Hkv];
    mask_page<P>(sacc, ent & 0xFFFF, tmin, trow, hf);
    const bool member = slot >= 0 && (((ent >> 16) >> slot) & 1u);
    if constexpr (MODE == kFp8Mode) {
      const float alpha =
          softmax_page_fp8(sacc, member, pf_c, qr.rscale, qr.qn, m_run, l_run, pF, vsb);
      rescale_acc<D>(acc, alpha);
      pv_page_fp8<D>(vbuf, pF, vsb, acc);
    } else {
      const float alpha = softmax_page(sacc, member, pf_c, qr.rscale, qr.qn, m_run, l_run, pB);
      rescale_acc<D>(acc, alpha);
      pv_page<D>(vbuf, pB, acc);
    }
    load_v(vbuf, u1);
  }

  if constexpr (MODE == kPairMode) {
    // ---- partials of the page pair: (m, l, acc) per owned row, merged later
    const float l_tot = half_sum(l_run);
    if (trow < 0) return;
    float* pp = p.partials + ((size_t)pslot * p.G + (qhead - h * p.G)) * (D + 4);
    if (hf == 0) *reinterpret_cast<float2*>(pp) = make_float2(m_run, l_tot);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<float4*>(pp + 4 + 32 * dt + 8 * rq + 4 * hf) =
            make_float4(acc[dt][4 * rq], acc[dt][4 * rq + 1], acc[dt][4 * rq + 2],
                        acc[dt][4 * rq + 3]);
    return;
  }
  // ---- epilogue: normalise and write each owned row once
  store_row<D>(acc, l_run, trow >= 0 ? p.O + ((size_t)trow * p.Hq + qhead) * D : nullptr, hf);
}


template <int D, int MODE>
hipError_t launch_d(const UAParams& prm, int blocks, size_t lds, hipStream_t stream) {
  const dim3 grid(blocks), block(64 * PW_UA_WG_WAVES);
  if (prm.P == 64)
    hipLaunchKernelGGL((union_attn_kernel<D, 64, MODE>), grid, block, lds, stream, prm);
  else if (prm.P == 32)
    hipLaunchKernelGGL((union_attn_kernel<D, 32, MODE>), grid, block, lds, stream, prm);
  else
    hipLaunchKernelGGL((union_attn_kernel<D, 16, MODE>), grid, block, lds, stream, prm);
  return hipGetLastError();
}

void common_params(UAParams& prm, const pw_shape& s, const uint16_t* Q, const float* scales) {
  prm = UAParams{};
  prm.Q = Q; prm.scales = scales;
  prm.T = s.T; prm.Hq = s.H_q; prm.Hkv = s.H_kv; prm.G = s.H_q / s.H_kv; prm.P = s.P;
  prm.N = s.N_pages; prm.S = s.S;
  prm.qk_scale = kLog2e / sqrtf((float)s.D);
}

}  // namespace

// Workspace of the re-tiled pages: K tiles, V tiles, then the page factors.
size_t tiled_pf_offset(const pw_shape& s) { return (size_t)2 * s.N_pages * s.H_kv * 64 * s.D; }
size_t tiled_kv_bytes(const pw_shape& s) {
  return tiled_pf_offset(s) + ((size_t)16 * s.N_pages * s.H_kv + 255) / 256 * 256;
}

hipError_t tile_kv(const pw_shape& s, const uint8_t* K, const uint8_t* V, const float* scales,
                   uint8_t* tiles, hipStream_t stream, int h_begin, int h_count) {
  if (h_count < 0) h_count = s.H_kv;
  uint8_t* Kt = tiles;
  uint8_t* Vt = tiles + tiled_pf_offset(s) / 2;
  float4* pf = reinterpret_cast<float4*>(tiles + tiled_pf_offset(s));
  const float qk_scale = kLog2e / sqrtf((float)s.D);
  const dim3 grid(s.N_pages * h_count);
  if (s.D == 128)
    hipLaunchKernelGGL(tile_kv_kernel<128>, grid, dim3(256), 0, stream, K, V, scales, qk_scale,
                       Kt, Vt, pf, s.N_pages, s.P, s.H_kv, h_begin, h_count);
  else
    hipLaunchKernelGGL(tile_kv_kernel<64>, grid, dim3(256), 0, stream, K, V, scales, qk_scale,
                       Kt, Vt, pf, s.N_pages, s.P, s.H_kv, h_begin, h_count);
  return hipGetLastError();
}

hipError_t launch_union_attention_tiled(const pw_shape& s, const uint16_t* Q, const int32_t* sel,
                                        const int32_t* ids, int g, int h_begin, int h_count,
                                        uint16_t* O, const void* ws, hipStream_t stream,
                                        const int32_t* order, bool fp8_qp) {
  const uint8_t* tiles = static_cast<const uint8_t*>(ws);
  UAParams prm;
  common_params(prm, s, Q, nullptr);
  prm.Kt = tiles;
  prm.Vt = tiles + tiled_pf_offset(s) / 2;
  prm.pf = reinterpret_cast<const float4*>(tiles + tiled_pf_offset(s));
  prm.sel = sel; prm.ids = ids; prm.O = O; prm.g = g;
  prm.groups_per_head = (s.T + g - 1) / g;
  prm.order = order;
  prm.total_groups = prm.groups_per_head * h_count;
  prm.h_begin = h_begin;
  prm.n_umax = (g * s.S < s.N_pages) ? g * s.S : s.N_pages;
  const int nw = (s.N_pages + 31) / 32;           // page bitset words, then their list offsets
  prm.lds_wave = ((prm.n_umax * 4 + 2 * nw * 4) + 15) / 16 * 16;
  prm.n_rt = (g * prm.G + 31) / 32;
  prm.total_items = prm.total_groups * prm.n_rt;
  const int blocks = (prm.total_items + PW_UA_WG_WAVES - 1) / PW_UA_WG_WAVES;
  const size_t lds = (size_t)prm.lds_wave * PW_UA_WG_WAVES;
  if (fp8_qp)
    return s.D == 128 ? launch_d<128, kFp8Mode>(prm, blocks, lds, stream)
                      : launch_d<64, kFp8Mode>(prm, blocks, lds, stream);
  return s.D == 128 ? launch_d<128, kUnionMode>(prm, blocks, lds, stream)
                    : launch_d<64, kUnionMode>(prm, blocks, lds, stream);
}

hipError_t launch_union_attention(const pw_shape& s, const uint16_t* Q, const uint8_t* K,
                                  const uint8_t* V, const float* scales, const int32_t* sel,
                                  const int32_t* ids, int g, int h_begin, int h_count,
                                  uint16_t* O, void* ws, hipStream_t stream) {
  hipError_t e = tile_kv(s, K, V, scales, static_cast<uint8_t*>(ws), stream, h_begin, h_count);
  if (e != hipSuccess) return e;
  return launch_union_attention_tiled(s, Q, sel, ids, g, h_begin, h_count, O, ws, stream);
}

hipError_t launch_pair_attention(const pw_shape& s, const uint16_t* Q, const uint8_t* tiles,
                                 const float* scales, const int2* plist, const int* pcount,
                                 const int* tstart, const int2* pairs, int tiles_head,
                                 float* partials, int Np, int Tc, int t0, hipStream_t stream) {
  UAParams prm;
  common_params(prm, s, Q, scales);
  prm.Kt = tiles;
  prm.Vt = tiles + tiled_pf_offset(s) / 2;
  prm.pf = reinterpret_cast<const float4*>(tiles + tiled_pf_offset(s));
  prm.plist = plist; prm.pcount = pcount; prm.partials = partials;
  prm.tstart = tstart; prm.pairs = pairs; prm.tiles_head = tiles_head;
  prm.Np = Np; prm.Tc = Tc; prm.t0 = t0;
  prm.g = 8;
  prm.n_rt = (8 * prm.G + 31) / 32;
  prm.total_items = s.H_kv * tiles_head * prm.n_rt;
  prm.n_umax = 2;
  prm.lds_wave = 16;
  const int blocks = (prm.total_items + PW_UA_WG_WAVES - 1) / PW_UA_WG_WAVES;
  const size_t lds = (size_t)prm.lds_wave * PW_UA_WG_WAVES;
  return s.D == 128 ? launch_d<128, kPairMode>(prm, blocks, lds, stream)
                    : launch_d<64, kPairMode>(prm, blocks, lds, stream);
}

}  // namespace pw
