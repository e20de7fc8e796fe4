// Device helpers shared by the union-attention kernels (gfx950): softmax
// constants, the key permutation of the re-tiled K pages, raw maxima, lane-half
// reductions and the two-part e4m3 split of a Q row.
#pragma once

#include "pw_internal.h"

namespace pw {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Lazy-rescale threshold (log2 units): a row's reference maximum moves only
// when a score exceeds it by more than kTau, so p <= 2^kTau.  At 24, the
// Cauchy-Schwarz bound below usually proves on N(0,1)-like data that no score
// of a page can move the reference, and the wave skips its max pass.
constexpr float kTau = 24.0f;
// Relative slack of the norm bounds: covers the fp32 rounding of the sums of
// squares, of the square roots and of the score accumulation, and the residual
// of the two-part e4m3 split of Q (below 1e-4 of a row's norm).
constexpr float kNormSlack = 1.0f + 1.0f / 512;
// The FP8 Q and P variant rounds p to e4m3fn (largest value 448): its threshold
// keeps p <= 2^kTauFp8 * phi < 2^7 with the V scale's mantissa phi in [1, 2).
constexpr float kTauFp8 = 6.0f;


// Physical key held by MFMA row i of key tile kt.  Output register r of a lane
// in half `hf` holds MFMA row 8*(r/4) + 4*hf + r%4; with this map it holds
// key 32*hf + 16*kt + r, i.e. each lane sees 32 consecutive keys.
__device__ __forceinline__ int tile_key(int i, int kt) {
  return 32 * ((i >> 2) & 1) + 16 * kt + 4 * (i >> 3) + (i & 3);
}

// Maxima of scores that come straight from the matrix cores (never a
// signalling NaN): plain v_max3 / v_max, without the quieting v_max x, x that
// fmaxf adds per operand in IEEE mode.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Lanes l and l ^ 32 hold the two key halves of the same query row: combine
// them with one VALU lane swap (no LDS round trip).
__device__ __forceinline__ float half_max(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_raw(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ---- one lane's query row: the B operand of S^T = K Q^T ------------------
// Lane (hf, col) holds d in [(D/2) hf, (D/2) hf + D/2) of its row.  The bf16
// row is scaled by a power of two 2^e (its largest magnitude into [128, 256))
// and split into two e4m3fn parts, hi = e4m3(q) and lo = e4m3(q - hi): hi + lo
// is the scaled bf16 value for elements >= 2^-2 and within 2^-10 below, so
// K^T runs on the FP8 MFMA straight from the cache bytes; rscale = 2^-e is
// folded back into the score scale.  qn bounds the norm of the scaled row.
// Without SPLIT (the FP8 Q and P variant) the row is hi alone, and qn bounds
// the norm of hi.
template <int D>
struct QRow {
  i32x8 hi[D / 64], lo[D / 64];
  float rscale, qn;
};

template <int D, bool SPLIT = true>
__device__ __forceinline__ void load_q_row(const uint16_t* qp, bool ok, QRow<D>& r) {
  constexpr int KQ = D / 64;
  float q[D / 2];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const uint4 v = ok ? *reinterpret_cast<const uint4*>(qp + 8 * c) : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      q[8 * c + 2 * k] = __uint_as_float(w[k] << 16);
      q[8 * c + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < D / 2; ++i) amax = fmaxf(amax, fabsf(q[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  int e = 0;
  if (amax > 0.f) {
    int ex;
    frexpf(amax, &ex);
    e = 8 - ex;                  // amax * 2^e in [128, 256)
  }
  r.rscale = ldexpf(1.f, -e);
  float ssq = 0.f;
#pragma unroll
  for (int ks = 0; ks < KQ; ++ks) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const float* x = q + 32 * ks + 4 * w;
      const float x0 = ldexpf(x[0], e), x1 = ldexpf(x[1], e);
      const float x2 = ldexpf(x[2], e), x3 = ldexpf(x[3], e);
      if constexpr (SPLIT) ssq = fmaf(x0, x0, fmaf(x1, x1, fmaf(x2, x2, fmaf(x3, x3, ssq))));
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hi, true);
      const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
      const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
      if constexpr (SPLIT) {
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - h01[0], x1 - h01[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - h23[0], x3 - h23[1], lo, true);
        r.hi[ks][w] = hi;
        r.lo[ks][w] = lo;
      } else {
        ssq = fmaf(h01[0], h01[0], fmaf(h01[1], h01[1], fmaf(h23[0], h23[0], fmaf(h23[1], h23[1], ssq))));
        r.hi[ks][w] = hi;
      }
    }
  }
  r.qn = sqrtf(ssq + __shfl_xor(ssq, 32)) * kNormSlack;
}

// ---- S^T = K (Qhi + Qlo)^T on the FP8 MFMA, one page of 64 key slots ------
// kr[kt][c]: the lane's 16-byte K chunks of key tile kt (tiled page order).
// Key tiles innermost, so consecutive MFMAs accumulate into different tiles.
// PARTS = 1: K Qhi^T only (the FP8 Q and P variant).
template <int D, int PARTS = 2>
__device__ __forceinline__ void qk_page(const uint4 (&kr)[2][D / 32], const QRow<D>& q,
                                        f32x16 (&sc)[2]) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[kt][r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 64; ++ks) {
#pragma unroll
    for (int part = 0; part < PARTS; ++part) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint4 w0 = kr[kt][2 * ks], w1 = kr[kt][2 * ks + 1];
        const i32x8 a = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w,
                         (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
        sc[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a, part ? q.lo[ks] : q.hi[ks], sc[kt], 0, 0, 0, 127, 0, 127);
      }
    }
  }
}

// ---- causal / page-size mask: key slot 32 hf + 16 kt + r of page u is kept
// iff it is a real key (< P) and not after the row's token.  Only pages that
// reach past the group's lowest token (tmin) need it.
template <int P>
__device__ __forceinline__ void mask_page(f32x16 (&sc)[2], int u, int tmin, int trow, int hf) {
  const bool need_mask = P < 64 || (u * P + P - 1 > tmin);
  if (need_mask) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * hf + 16 * kt + r;
        if (key >= P || u * P + key > trow) sc[kt][r] = -INFINITY;
      }
  }
}

// ---- online softmax of one page in the log2 domain ------------------------
// f = the page's factors {k_scale * log2(e) / sqrt(D), score bound factor,
// log2(v_scale), 1 / v_scale}.  The reference maximum m of a row moves only when
// a score passes it by more than kTau (lazy rescale, p <= 2^kTau); v_scale is
// folded into the exponent, so P V on the codes gives v_scale * p * v.  The
// probabilities come out as bf16 MFMA operands pB; returns the rescale factor
// of the accumulator (exactly 1 unless the reference moved).  A row whose query
// did not select the page (member false) gets p = 0 and keeps m and l.
__device__ __forceinline__ float softmax_page(f32x16 (&sc)[2], bool member, const float4 f,
                                              float rscale, float qn, float& m_run,
                                              float& l_run, bf16x8 (&pB)[4]) {
  const float ksc = f.x * rscale;
  const float lim = m_run + kTau;
  // Cauchy-Schwarz: no score of the row on this page exceeds |q| * max |k| *
  // |scale|; when that cannot pass the reference by kTau for any member row of
  // the wave, the row maxima are not needed (the computed maximum would leave
  // every reference where it is: same result).
  const bool may_move = member && !(qn * f.y * rscale <= lim);
  float m_new = m_run, alpha = 1.f;
  if (__ballot(may_move)) {
    float mx = max_raw(sc[0][0], sc[0][1]);
#pragma unroll
    for (int i = 2; i < 32; i += 2) mx = max3_raw(mx, sc[i >> 4][i & 15], sc[i >> 4][(i & 15) + 1]);
    mx = half_max(mx);
    const float mx2 = mx * ksc;
    m_new = (member && mx2 > lim) ? mx2 : m_run;
    // exp2(0) = 1 exactly when the reference max is unchanged
    alpha = __builtin_amdgcn_exp2f((m_new == m_run) ? 0.f : m_run - m_new);
  }
  m_run = m_new;
  const float bias = (member && m_new > -INFINITY) ? (f.z - m_new) : -INFINITY;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float ps = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[q >> 1][8 * (q & 1) + e], ksc, bias));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[q >> 1][8 * (q & 1) + e + 1], ksc, bias));
      bf16x2 pr;
      pr[0] = (__bf16)e0;
      pr[1] = (__bf16)e1;
      ps = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps, false);
      v[e] = pr[0];
      v[e + 1] = pr[1];
    }
    pB[q] = v;
  }
  l_run = fmaf(ps, f.w, l_run * alpha);
  return alpha;
}

// ---- the same page for the FP8 Q and P variant ----------------------------
// The threshold is kTauFp8, and the V scale is split as v_scale = phi 2^vk with
// vk = floor(log2 v_scale): phi folds into the exponent (p = 2^(s - m) phi <=
// 2^7), 2^vk becomes the E8M0 scale *vsb of the P operand of the PV MFMA.  The
// probabilities are rounded to e4m3fn (round to nearest even) into pF, byte i
// of a lane being key 32 hf + i, and the row sums add those rounded values
// (converted back exactly) times 1 / phi, so the weights of a row sum to one.
__device__ __forceinline__ float softmax_page_fp8(f32x16 (&sc)[2], bool member, const float4 f,
                                                  float rscale, float qn, float& m_run,
                                                  float& l_run, i32x8& pF, int& vsb) {
  const float ksc = f.x * rscale;
  const float lim = m_run + kTauFp8;
  const bool may_move = member && !(qn * f.y * rscale <= lim);
  float m_new = m_run, alpha = 1.f;
  if (__ballot(may_move)) {
    float mx = max_raw(sc[0][0], sc[0][1]);
#pragma unroll
    for (int i = 2; i < 32; i += 2) mx = max3_raw(mx, sc[i >> 4][i & 15], sc[i >> 4][(i & 15) + 1]);
    mx = half_max(mx);
    const float mx2 = mx * ksc;
    m_new = (member && mx2 > lim) ? mx2 : m_run;
    alpha = __builtin_amdgcn_exp2f((m_new == m_run) ? 0.f : m_run - m_new);
  }
  m_run = m_new;
  const float vk = floorf(f.z);
  vsb = min(max(127 + (int)vk, 0), 254);
  const float bias = (member && m_new > -INFINITY) ? ((f.z - vk) - m_new) : -INFINITY;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float ps = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const f32x16& t = sc[w >> 2];
    const int r = 4 * (w & 3);
    const float e0 = __builtin_amdgcn_exp2f(fmaf(t[r], ksc, bias));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(t[r + 1], ksc, bias));
    const float e2 = __builtin_amdgcn_exp2f(fmaf(t[r + 2], ksc, bias));
    const float e3 = __builtin_amdgcn_exp2f(fmaf(t[r + 3], ksc, bias));
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
    x = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, x, true);
    pF[w] = x;
    ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false),
                                         ones, ps, false);
    ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true),
                                         ones, ps, false);
  }
  l_run = fmaf(ps, ldexpf(f.w, (int)vk), l_run * alpha);
  return alpha;
}

template <int D>
__device__ __forceinline__ void rescale_acc(f32x16 (&acc)[D / 32], float alpha) {
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
  }
}

// ---- O^T += V^T P^T on the bf16 MFMA (d tiles innermost: consecutive MFMAs
// are independent); vr[dt][j]: the lane's 16-byte V chunks, codes converted to
// bf16 exactly.
template <int D>
__device__ __forceinline__ void pv_page(const uint4 (&vr)[D / 32][2], const bf16x8 (&pB)[4],
                                        f32x16 (&acc)[D / 32]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const uint4 w = vr[dt][q >> 1];
      const bf16x8 a = (q & 1) ? fp8x8_to_bf16(w.z, w.w) : fp8x8_to_bf16(w.x, w.y);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pB[q], acc[dt], 0, 0, 0);
    }
  }
}

// ---- O^T += V^T P^T on the FP8 MFMA (the FP8 Q and P variant): one MFMA per
// d tile over all 64 keys; A = the lane's 32 V codes of one d (keys 32 hf ..
// 32 hf + 31), B = the lane's 32 e4m3 probabilities of the same keys, scaled
// by 2^(vsb - 127).
template <int D>
__device__ __forceinline__ void pv_page_fp8(const uint4 (&vr)[D / 32][2], const i32x8& pF, int vsb,
                                            f32x16 (&acc)[D / 32]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const uint4 w0 = vr[dt][0], w1 = vr[dt][1];
    const i32x8 a = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w,
                     (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
    acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pF, acc[dt], 0, 0, 0, 127, 0, vsb);
  }
}

// ---- epilogue: normalise and write the lane's half of its row (bf16 RNE) ---
template <int D>
__device__ __forceinline__ void store_row(const f32x16 (&acc)[D / 32], float l_run, uint16_t* op,
                                          int hf) {
  const float l_tot = half_sum(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (op == nullptr) return;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      bf16x2 lo, hi;
      lo[0] = (__bf16)(acc[dt][4 * rq + 0] * inv);
      lo[1] = (__bf16)(acc[dt][4 * rq + 1] * inv);
      hi[0] = (__bf16)(acc[dt][4 * rq + 2] * inv);
      hi[1] = (__bf16)(acc[dt][4 * rq + 3] * inv);
      uint2 v = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      *reinterpret_cast<uint2*>(op + 32 * dt + 8 * rq + 4 * hf) = v;
    }
}

}  // namespace
}  // namespace pw
