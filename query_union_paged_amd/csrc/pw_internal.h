// Internal declarations shared by the HIP sources of libpageweaver (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pageweaver.h"

namespace pw {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

// Make this wave's earlier LDS writes visible to its later LDS reads (the
// lanes of one wave exchange data through LDS without a workgroup barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}

// Eight e4m3fn bytes (two dwords) -> eight bf16, exactly (every e4m3fn value,
// subnormals included, is a bf16 value).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// Host-side launchers (implemented next to their kernels).
// usize (optional): the union size of every group, int32 [H_kv][ceil(T / g)]
hipError_t launch_group(const pw_shape& s, const int32_t* sel, int W, int g, int32_t* ids,
                        hipStream_t stream, int32_t* usize = nullptr);
// Per KV head and block of consecutive groups (the groups the attention runs at
// once on one XCD), the block's groups by ascending union size (equal sizes in
// index order); blocks stay in index order.
hipError_t launch_group_order(const pw_shape& s, int g, const int32_t* usize, int32_t* order,
                              hipStream_t stream);
// FP8 K/V pages re-tiled in MFMA operand order (K tiles, then V tiles), then
// 16 bytes of softmax factors per (page, KV head).
size_t tiled_kv_bytes(const pw_shape& s);
// KV heads h_begin .. h_begin + h_count - 1 (h_count < 0: all heads)
hipError_t tile_kv(const pw_shape& s, const uint8_t* K, const uint8_t* V, const float* scales,
                   uint8_t* tiles, hipStream_t stream, int h_begin = 0, int h_count = -1);
hipError_t launch_union_attention(const pw_shape& s, const uint16_t* Q, const uint8_t* K,
                                  const uint8_t* V, const float* scales, const int32_t* sel,
                                  const int32_t* ids, int g, int h_begin, int h_count,
                                  uint16_t* O, void* ws, hipStream_t stream);
// The attention alone, on a workspace that tile_kv has filled for heads
// h_begin .. h_begin + h_count - 1.
// order (optional): per KV head, the execution order of its groups (a
// permutation of 0 .. ceil(T / g) - 1, the last entries run first).
// fp8_qp: the lower-precision variant with Q and P rounded to e4m3fn.
hipError_t launch_union_attention_tiled(const pw_shape& s, const uint16_t* Q, const int32_t* sel,
                                        const int32_t* ids, int g, int h_begin, int h_count,
                                        uint16_t* O, const void* ws, hipStream_t stream,
                                        const int32_t* order = nullptr, bool fp8_qp = false);
hipError_t launch_pair_attention(const pw_shape& s, const uint16_t* Q, const uint8_t* tiles,
                                 const float* scales, const int2* plist, const int* pcount,
                                 const int* tstart, const int2* pairs, int tiles_head,
                                 float* partials, int Np, int Tc, int t0, hipStream_t stream);
// Device address and size of the calling device's no-alloc scratch array
// (looked up once per device).
hipError_t noalloc_scratch(void** ptr, size_t* bytes);
size_t check_ids_workspace(const pw_shape& s);
hipError_t launch_check_ids(const pw_shape& s, const int32_t* ids, int32_t* bad, void* ws,
                            hipStream_t stream);
size_t select_workspace(const pw_shape& s);
hipError_t launch_select(const pw_shape& s, const uint16_t* Q, const uint8_t* K,
                         const float* scales, int L, int32_t* sel, void* ws, hipStream_t stream);
size_t dense_union_workspace(const pw_shape& s);
// pairs: null = adjacent pages (2k, 2k + 1); else int32 [H_kv][N][2] pair table
hipError_t launch_dense_union(const pw_shape& s, const uint16_t* Q, const uint8_t* K,
                              const uint8_t* V, const float* scales, const int32_t* sel,
                              const int32_t* pairs, uint16_t* O, void* ws, size_t ws_bytes,
                              hipStream_t stream);
size_t page_pairs_workspace(const pw_shape& s);
hipError_t launch_page_pairs(const pw_shape& s, const int32_t* sel, int32_t* pairs, void* ws,
                             hipStream_t stream);

}  // namespace pw
