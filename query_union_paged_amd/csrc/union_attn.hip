// ID-aware query-union attention over a paged FP8 KV cache (gfx950).
//
// "PageWeaver: KV-Guided Query Unions for Sparse Attention", Abstract: query
// unions share page loads and fill matrix-core tiles; every query keeps its
// original support and sole ownership of its output; the kernel consumes
// query IDs without materialising a reordered Q tensor or cross-page partial
// outputs.
//
// Mapping on CDNA4.  One wave owns one group (g query IDs of one KV head,
// M = g*G query rows <= 64 = NT tiles of 32) and walks the group's union of
// pages in ascending page order; four waves (four groups) share a workgroup
// only for scheduling.  Per page (64 keys):
//   S^T = K_page * Q^T     v_mfma_f32_32x32x16_bf16, keys are the MFMA rows
//                          and query rows the columns, so each lane holds one
//                          query row (lane & 31) and 32 of its 64 keys;
//   online softmax         fp32 in registers, row max/sum finished with one
//                          cross-half exchange (lane ^ 32);
//   O^T += V_page^T * P^T  v_mfma_f32_32x32x16_bf16, d is the MFMA row.
// The e4m3fn codes go straight from global memory into MFMA operand registers
// (each byte is used by exactly one wave once, so LDS staging would only add
// traffic) and are converted to bf16 exactly; the per-page scales are folded
// into the scores (k) and into the exponent (v).  The key order inside the
// 32-row K tiles is permuted so that the PV operands of every lane are 32
// contiguous tokens of a dim-major V page.
//
// Ownership.  A row whose query did not select a page gets p = 0 and its
// running max untouched on that page (alpha = 1 exactly), so its result is
// the same whichever group it sits in; each (query, Q head) row is written
// once, by its wave.  There are no atomics and no partial outputs.
#include "pw_internal.h"

namespace pw {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 8.0f;   // lazy-rescale threshold (log2 units): p <= 2^8

struct UAParams {
  const uint16_t* Q;
  const uint8_t* K;
  const uint8_t* V;
  const float* scales;
  const int32_t* sel;
  const int32_t* ids;
  uint16_t* O;
  int T, Hq, Hkv, G, P, N, S, g;
  int groups_per_head, total_groups;
  int n_umax;        // list capacity per wave (>= any union size)
  int lds_wave;      // bytes of LDS per wave
  float qk_scale;    // log2(e) / sqrt(D)
};

// Physical key held by MFMA row i of key tile kt.  Output register r of a lane
// in half `hf` holds MFMA row 8*(r/4) + 4*hf + r%4; with this map it holds
// key 32*hf + 16*kt + r, i.e. each lane sees 32 consecutive keys.
__device__ __forceinline__ int tile_key(int i, int kt) {
  return 32 * ((i >> 2) & 1) + 16 * kt + 4 * (i >> 3) + (i & 3);
}

__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <int D, int NT>
__global__ __launch_bounds__(256) void union_attn_kernel(UAParams p) {
  constexpr int KS = D / 16;     // MFMA k-steps over d (QK^T)
  constexpr int KCH = D / 32;    // uint4 chunks of K per lane per key tile
  constexpr int DT = D / 32;     // output tiles over d (PV)
  extern __shared__ __align__(16) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hf = lane >> 5;      // lane half
  const int col = lane & 31;     // query row within a tile

  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
  // each XCD sweeps a contiguous range of groups (one KV head's pages stay in
  // that XCD's L2).
  const int nb = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, per = nb >> 3, extra = nb & 7;
  const int lb = xcd * per + min(xcd, extra) + (b >> 3);
  const int gid = lb * 4 + wave;
  if (gid >= p.total_groups) return;
  const int h = gid / p.groups_per_head;
  const int g0 = (gid - h * p.groups_per_head) * p.g;
  const int gm = min(p.g, p.T - g0);

  unsigned char* wbase = smem + (size_t)wave * p.lds_wave;
  uint32_t* list = reinterpret_cast<uint32_t*>(wbase);        // page | members << 16
  uint32_t* mask32 = reinterpret_cast<uint32_t*>(wbase + (size_t)p.n_umax * 4);
  const int n_mwords = (p.N + 3) >> 2;

  // Members of the group (lane i < gm holds member i's token).
  int my_t = -1;
  if (lane < gm) {
    const int t = p.ids[(size_t)h * p.T + g0 + lane];
    my_t = (t >= 0 && t < p.T) ? t : -1;
  }
  int tmin = wave_min_u32(my_t >= 0 ? (uint32_t)my_t : 0xFFFFFFFFu);

  // ---- union + membership: mask byte per page, bit i = member i selected it
  for (int i = lane; i < n_mwords; i += 64) mask32[i] = 0;
  wave_sync();
  {
    constexpr int MAXIT = 16;        // g * S <= 1024 entries
    const int n_ent = gm * p.S;
    int pg[MAXIT];
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      const int e = lane + 64 * it;
      const int i = e / p.S;
      const int t = __shfl(my_t, i & 63);
      pg[it] = -1;
      if (e < n_ent && t >= 0) pg[it] = p.sel[((size_t)h * p.T + t) * p.S + (e - i * p.S)];
      pg[it] = (pg[it] >= 0 && pg[it] < p.N) ? (pg[it] | (i << 16)) : -1;
    }
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      if (pg[it] >= 0) {
        const int u = pg[it] & 0xFFFF, i = pg[it] >> 16;
        atomicOr(&mask32[u >> 2], (1u << i) << ((u & 3) * 8));
      }
    }
  }
  wave_sync();
  int n_u = 0;
  for (int c0 = 0; c0 < p.N; c0 += 64) {
    const int u = c0 + lane;
    const uint32_t m = (u < p.N) ? ((mask32[u >> 2] >> ((u & 3) * 8)) & 0xFFu) : 0u;
    const uint64_t bal = __ballot(m != 0);
    if (m) list[n_u + lane_prefix(bal)] = (uint32_t)u | (m << 16);
    n_u += __popcll(bal);
  }
  wave_sync();

  // ---- per-lane query rows and Q operands (B of S^T = K Q^T)
  int slot[NT], trow[NT], qhead[NT];
  bf16x8 qB[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = 32 * nt + col;
    const int s = n / p.G;
    const int t = __shfl(my_t, s & 63);
    const bool ok = (s < gm) && (t >= 0);
    slot[nt] = ok ? s : -1;
    trow[nt] = ok ? t : -1;
    qhead[nt] = h * p.G + (n - s * p.G);
    const uint16_t* qp = p.Q + ((size_t)(ok ? t : 0) * p.Hq + qhead[nt]) * D + (D / 2) * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = ok ? *reinterpret_cast<const uint4*>(qp + 8 * ks) : make_uint4(0, 0, 0, 0);
      qB[nt][ks] = as_bf16x8(v);
    }
  }

  float m_run[NT], l_run[NT];
  f32x16 acc[NT][DT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nt][dt][r] = 0.f;
  }

  const size_t page_stride = (size_t)p.Hkv * p.P * D;   // bytes between pages
  const uint8_t* kbase = p.K + (size_t)h * p.P * D;
  const uint8_t* vbase = p.V + (size_t)h * D * p.P;
  int krow[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) krow[kt] = tile_key(col, kt);
  const int vbytes = min(max(p.P - 32 * hf, 0), 32);   // valid V bytes of this lane's row

  uint4 kraw[2][KCH], vraw[DT][2];
  auto load_k = [&](int u) {
    const uint8_t* kp = kbase + (size_t)u * page_stride + (D / 2) * hf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < KCH; ++c)
        kraw[kt][c] = (krow[kt] < p.P) ? load16(kp + (size_t)krow[kt] * D + 16 * c)
                                       : make_uint4(0, 0, 0, 0);
  };
  auto load_v = [&](int u) {
    const uint8_t* vp = vbase + (size_t)u * page_stride + 32 * hf;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint8_t* row = vp + (size_t)(32 * dt + col) * p.P;
      vraw[dt][0] = (vbytes >= 16) ? load16(row) : make_uint4(0, 0, 0, 0);
      vraw[dt][1] = (vbytes >= 32) ? load16(row + 16) : make_uint4(0, 0, 0, 0);
    }
  };

  const float* kscale = p.scales + h;                       // [N][Hkv]
  const float* vscale = p.scales + (size_t)p.N * p.Hkv + h;
  float ks_raw = 1.f, vs_raw = 1.f;
  if (n_u > 0) {
    const int u0 = list[0] & 0xFFFF;
    load_k(u0);
    load_v(u0);
    ks_raw = kscale[(size_t)u0 * p.Hkv];
    vs_raw = vscale[(size_t)u0 * p.Hkv];
  }

  for (int up = 0; up < n_u; ++up) {
    const uint32_t ent = list[up];
    const int u = ent & 0xFFFF;
    const uint32_t mbits = ent >> 16;
    const float ksc = ks_raw * p.qk_scale;
    const float lvs = __builtin_amdgcn_logf(vs_raw);    // log2
    const float ivs = __builtin_amdgcn_rcpf(vs_raw);
    const int u_next = (up + 1 < n_u) ? (int)(list[up + 1] & 0xFFFF) : -1;
    if (u_next >= 0) {
      ks_raw = kscale[(size_t)u_next * p.Hkv];
      vs_raw = vscale[(size_t)u_next * p.Hkv];
    }

    // S^T = K Q^T
    f32x16 sacc[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[nt][kt][r] = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 w = kraw[kt][ks >> 1];
        const bf16x8 a = (ks & 1) ? fp8x8_to_bf16(w.z, w.w) : fp8x8_to_bf16(w.x, w.y);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          sacc[nt][kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qB[nt][ks], sacc[nt][kt], 0, 0, 0);
      }
    }
    if (u_next >= 0) load_k(u_next);

    // causal / page-size mask, only where some key can lie after a member
    const bool need_mask = (p.P < 64) || (u * p.P + p.P - 1 > tmin);
    if (need_mask) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * hf + 16 * kt + r;
            if (key >= p.P || u * p.P + key > trow[nt]) sacc[nt][kt][r] = -INFINITY;
          }
    }

    // online softmax (log2 domain, v_scale folded into the exponent)
    bf16x8 pB[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nt][kt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool member = slot[nt] >= 0 && ((mbits >> slot[nt]) & 1u);
      const float mx2 = mx * ksc;
      const float m_new = (member && mx2 > m_run[nt] + kTau) ? mx2 : m_run[nt];
      const float alpha = (m_new == m_run[nt]) ? 1.f : __builtin_amdgcn_exp2f(m_run[nt] - m_new);
      m_run[nt] = m_new;
      const float bias = (member && m_new > -INFINITY) ? (lvs - m_new) : -INFINITY;
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[nt][kt][r], ksc, bias));
          sacc[nt][kt][r] = e;
          ps += e;
        }
      l_run[nt] = l_run[nt] * alpha + ps * ivs;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[nt][dt][r] *= alpha;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)sacc[nt][q >> 1][8 * (q & 1) + e];
        pB[nt][q] = v;
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 w = vraw[dt][q >> 1];
        const bf16x8 a = (q & 1) ? fp8x8_to_bf16(w.z, w.w) : fp8x8_to_bf16(w.x, w.y);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pB[nt][q], acc[nt][dt], 0, 0, 0);
      }
    }
    if (u_next >= 0) load_v(u_next);
  }

  // ---- epilogue: normalise and write each owned row once
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l_tot = l_run[nt] + __shfl_xor(l_run[nt], 32);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (trow[nt] < 0) continue;
    uint16_t* op = p.O + ((size_t)trow[nt] * p.Hq + qhead[nt]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x2 lo, hi;
        lo[0] = (__bf16)(acc[nt][dt][4 * rq + 0] * inv);
        lo[1] = (__bf16)(acc[nt][dt][4 * rq + 1] * inv);
        hi[0] = (__bf16)(acc[nt][dt][4 * rq + 2] * inv);
        hi[1] = (__bf16)(acc[nt][dt][4 * rq + 3] * inv);
        uint2 v = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        *reinterpret_cast<uint2*>(op + 32 * dt + 8 * rq + 4 * hf) = v;
      }
  }
}

template <int D, int NT>
hipError_t launch_dn(const UAParams& prm, int blocks, size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL((union_attn_kernel<D, NT>), dim3(blocks), dim3(256), lds, stream, prm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_union_attention(const pw_shape& s, const uint16_t* Q, const uint8_t* K,
                                  const uint8_t* V, const float* scales, const int32_t* sel,
                                  const int32_t* ids, int g, uint16_t* O, hipStream_t stream) {
  UAParams prm;
  prm.Q = Q; prm.K = K; prm.V = V; prm.scales = scales; prm.sel = sel; prm.ids = ids; prm.O = O;
  prm.T = s.T; prm.Hq = s.H_q; prm.Hkv = s.H_kv; prm.G = s.H_q / s.H_kv; prm.P = s.P;
  prm.N = s.N_pages; prm.S = s.S; prm.g = g;
  prm.groups_per_head = (s.T + g - 1) / g;
  prm.total_groups = prm.groups_per_head * s.H_kv;
  prm.n_umax = (g * s.S < s.N_pages) ? g * s.S : s.N_pages;
  const int mask_bytes = ((s.N_pages + 3) / 4) * 4;
  prm.lds_wave = ((prm.n_umax * 4 + mask_bytes) + 15) / 16 * 16;
  prm.qk_scale = kLog2e / sqrtf((float)s.D);
  const int blocks = (prm.total_groups + 3) / 4;
  const size_t lds = (size_t)prm.lds_wave * 4;
  const int nt = (g * prm.G + 31) / 32;
  if (s.D == 128) return nt == 1 ? launch_dn<128, 1>(prm, blocks, lds, stream)
                                 : launch_dn<128, 2>(prm, blocks, lds, stream);
  return nt == 1 ? launch_dn<64, 1>(prm, blocks, lds, stream)
                 : launch_dn<64, 2>(prm, blocks, lds, stream);
}

}  // namespace pw
