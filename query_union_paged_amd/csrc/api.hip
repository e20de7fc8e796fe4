// extern "C" entry points of libpageweaver: host-side validation, then the
// launches on the caller's stream.  Declarations and contracts live in
// include/pageweaver.h.
#include <stdarg.h>
#include <stdio.h>

#include <initializer_list>

#include "pw_internal.h"

namespace {

thread_local char g_last_error[512] = "";

pw_status fail(pw_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

pw_status ok() {
  g_last_error[0] = '\0';
  return PW_OK;
}

pw_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PW_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checks shared by every call: consistent, positive dimensions.
pw_status check_shape(const pw_shape* s) {
  if (!s) return fail(PW_ERR_NULL, "shape is NULL");
  if (s->T <= 0 || s->H_q <= 0 || s->H_kv <= 0 || s->D <= 0 || s->P <= 0 || s->N_pages <= 0 ||
      s->S <= 0)
    return fail(PW_ERR_DIMS, "all dimensions must be positive (T=%d H_q=%d H_kv=%d D=%d P=%d N=%d S=%d)",
                s->T, s->H_q, s->H_kv, s->D, s->P, s->N_pages, s->S);
  if ((int64_t)s->N_pages * s->P != s->T)
    return fail(PW_ERR_DIMS, "T (%d) must equal N_pages * P (%d * %d)", s->T, s->N_pages, s->P);
  if (s->H_q % s->H_kv != 0)
    return fail(PW_ERR_DIMS, "H_q (%d) must be a multiple of H_kv (%d)", s->H_q, s->H_kv);
  return PW_OK;
}

pw_status check_attention_support(const pw_shape* s, int g) {
  const int G = s->H_q / s->H_kv;
  if (g < 1 || g > 16) return fail(PW_ERR_UNSUPPORTED, "g = %d outside [1, 16]", g);
  if (g * G > 64) return fail(PW_ERR_UNSUPPORTED, "g * G = %d exceeds 64 query rows", g * G);
  if (s->D != 64 && s->D != 128) return fail(PW_ERR_UNSUPPORTED, "D = %d not in {64, 128}", s->D);
  if (s->P != 16 && s->P != 32 && s->P != 64)
    return fail(PW_ERR_UNSUPPORTED, "P = %d not in {16, 32, 64}", s->P);
  if (s->N_pages > 32768) return fail(PW_ERR_UNSUPPORTED, "N_pages = %d exceeds 32768", s->N_pages);
  if (g * s->S > 1024) return fail(PW_ERR_UNSUPPORTED, "g * S = %d exceeds 1024", g * s->S);
  return PW_OK;
}

// The kernels move whole vectors: rows of Q, K, V and O 16 bytes at a time, selection rows 16
// bytes at a time when S is a multiple of 4, page pairs as 8-byte pairs, and the other int32 /
// fp32 arrays element by element.  NULL entries are checked elsewhere.
struct Aligned {
  const char* name;
  const void* p;
  unsigned bytes;
};
pw_status check_aligned(std::initializer_list<Aligned> xs) {
  for (const Aligned& x : xs)
    if (x.p != nullptr && ((uintptr_t)x.p & (x.bytes - 1)) != 0)
      return fail(PW_ERR_DIMS, "%s must be %u-byte aligned", x.name, x.bytes);
  return PW_OK;
}
unsigned sel_align(const pw_shape* s) { return s->S % 4 == 0 ? 16u : 4u; }

// The re-tiled K/V copy of pw_tile_kv: size, alignment, and the 2 GiB reach of
// the 32-bit offsets its readers form.
pw_status check_tiled_workspace(const pw_shape* s, const void* ws, size_t ws_bytes) {
  const size_t need = pw::tiled_kv_bytes(*s);
  if (!ws) return fail(PW_ERR_NULL, "workspace of %zu bytes required", need);
  if (ws_bytes < need) return fail(PW_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (((uintptr_t)ws & 255) != 0) return fail(PW_ERR_DIMS, "workspace must be 256-byte aligned");
  if (pw::tiled_kv_bytes(*s) / 2 > 0x7FFFFFFFu)
    return fail(PW_ERR_UNSUPPORTED, "tiled K/V of %zu bytes exceeds 2 GiB",
                pw::tiled_kv_bytes(*s) / 2);
  return PW_OK;
}

}  // namespace

extern "C" {

const char* pw_status_string(pw_status st) {
  switch (st) {
    case PW_OK: return "ok";
    case PW_ERR_NULL: return "null pointer";
    case PW_ERR_DIMS: return "invalid dimensions";
    case PW_ERR_UNSUPPORTED: return "unsupported configuration";
    case PW_ERR_WORKSPACE: return "workspace too small";
    case PW_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* pw_last_error(void) { return g_last_error; }

int32_t pw_abi_version(void) { return PW_ABI_VERSION; }

size_t pw_group_workspace_bytes(const pw_shape*, int32_t, int32_t) { return 0; }

static pw_status check_group_args(const pw_shape* shape, const int32_t* sel_pages, int32_t W,
                                  int32_t g, const int32_t* query_ids) {
  pw_status st = check_shape(shape);
  if (st != PW_OK) return st;
  if (!sel_pages || !query_ids) return fail(PW_ERR_NULL, "sel_pages and query_ids are required");
  if (W < 1 || W > 1024) return fail(PW_ERR_UNSUPPORTED, "W = %d outside [1, 1024]", W);
  if (g < 1 || g > 16) return fail(PW_ERR_UNSUPPORTED, "g = %d outside [1, 16]", g);
  if (W % g != 0)
    return fail(PW_ERR_UNSUPPORTED,
                "W = %d is not a multiple of g = %d (attention groups would straddle windows)", W, g);
  if (shape->N_pages > 1024)
    return fail(PW_ERR_UNSUPPORTED, "N_pages = %d exceeds 1024 for the search", shape->N_pages);
  return check_aligned({{"sel_pages", sel_pages, sel_align(shape)}, {"query_ids", query_ids, 4}});
}

pw_status pw_group(const pw_shape* shape, const int32_t* sel_pages, int32_t W, int32_t g,
                   int32_t* query_ids, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  pw_status st = check_group_args(shape, sel_pages, W, g, query_ids);
  if (st != PW_OK) return st;
  return hip_status(pw::launch_group(*shape, sel_pages, W, g, query_ids, (hipStream_t)stream),
                    "pw_group launch");
}

size_t pw_group_ordered_workspace_bytes(const pw_shape* shape, int32_t W, int32_t g) {
  (void)W;
  if (check_shape(shape) != PW_OK || g < 1) return 0;
  return (size_t)shape->H_kv * ((shape->T + g - 1) / g) * sizeof(int32_t);
}

pw_status pw_group_ordered(const pw_shape* shape, const int32_t* sel_pages, int32_t W, int32_t g,
                           int32_t* query_ids, int32_t* group_order, void* ws, size_t ws_bytes,
                           void* stream) {
  pw_status st = check_group_args(shape, sel_pages, W, g, query_ids);
  if (st != PW_OK) return st;
  if (!group_order) return fail(PW_ERR_NULL, "group_order is required");
  const size_t need = pw_group_ordered_workspace_bytes(shape, W, g);
  if (!ws) return fail(PW_ERR_NULL, "workspace of %zu bytes required", need);
  if (ws_bytes < need) return fail(PW_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (((uintptr_t)ws & 3) != 0 || ((uintptr_t)group_order & 3) != 0)
    return fail(PW_ERR_DIMS, "workspace and group_order must be 4-byte aligned");
  int32_t* usize = static_cast<int32_t*>(ws);
  hipError_t e = pw::launch_group(*shape, sel_pages, W, g, query_ids, (hipStream_t)stream, usize);
  if (e != hipSuccess) return hip_status(e, "pw_group_ordered search launch");
  return hip_status(pw::launch_group_order(*shape, g, usize, group_order, (hipStream_t)stream),
                    "pw_group_ordered order launch");
}

size_t pw_check_ids_workspace_bytes(const pw_shape* shape) {
  if (check_shape(shape) != PW_OK) return 0;
  return pw::check_ids_workspace(*shape);
}

pw_status pw_check_ids(const pw_shape* shape, const int32_t* query_ids, int32_t* bad_counts,
                       void* ws, size_t ws_bytes, void* stream) {
  pw_status st = check_shape(shape);
  if (st != PW_OK) return st;
  if (!query_ids || !bad_counts) return fail(PW_ERR_NULL, "query_ids and bad_counts are required");
  st = check_aligned({{"query_ids", query_ids, 4}, {"bad_counts", bad_counts, 4}});
  if (st != PW_OK) return st;
  const size_t need = pw::check_ids_workspace(*shape);
  if (!ws) return fail(PW_ERR_NULL, "workspace of %zu bytes required", need);
  if (ws_bytes < need) return fail(PW_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(pw::launch_check_ids(*shape, query_ids, bad_counts, ws, (hipStream_t)stream),
                    "pw_check_ids launch");
}

size_t pw_union_attention_workspace_bytes(const pw_shape* shape, int32_t) {
  if (check_shape(shape) != PW_OK) return 0;
  return pw::tiled_kv_bytes(*shape);
}

static pw_status union_attention_range(const pw_shape* shape, const uint16_t* Q,
                                       const uint8_t* K_fp8, const uint8_t* V_fp8,
                                       const float* scales, const int32_t* sel_pages,
                                       const int32_t* query_ids, int32_t g, int32_t h_begin,
                                       int32_t h_count, uint16_t* O, void* ws, size_t ws_bytes,
                                       void* stream, const char* what) {
  pw_status st = check_shape(shape);
  if (st != PW_OK) return st;
  if (!Q || !K_fp8 || !V_fp8 || !scales || !sel_pages || !query_ids || !O)
    return fail(PW_ERR_NULL, "Q, K_fp8, V_fp8, scales, sel_pages, query_ids and O are required");
  st = check_aligned({{"Q", Q, 16}, {"K_fp8", K_fp8, 16}, {"V_fp8", V_fp8, 16}, {"scales", scales, 4},
                      {"sel_pages", sel_pages, sel_align(shape)}, {"query_ids", query_ids, 4},
                      {"O", O, 16}});
  if (st != PW_OK) return st;
  st = check_attention_support(shape, g);
  if (st != PW_OK) return st;
  if (h_begin < 0 || h_count < 1 || h_begin + h_count > shape->H_kv)
    return fail(PW_ERR_DIMS, "KV heads [%d, %d) outside [0, %d)", h_begin, h_begin + h_count,
                shape->H_kv);
  st = check_tiled_workspace(shape, ws, ws_bytes);
  if (st != PW_OK) return st;
  return hip_status(pw::launch_union_attention(*shape, Q, K_fp8, V_fp8, scales, sel_pages,
                                               query_ids, g, h_begin, h_count, O, ws,
                                               (hipStream_t)stream),
                    what);
}

pw_status pw_union_attention(const pw_shape* shape, const uint16_t* Q, const uint8_t* K_fp8,
                             const uint8_t* V_fp8, const float* scales, const int32_t* sel_pages,
                             const int32_t* query_ids, int32_t g, uint16_t* O, void* ws,
                             size_t ws_bytes, void* stream) {
  return union_attention_range(shape, Q, K_fp8, V_fp8, scales, sel_pages, query_ids, g, 0,
                               shape ? shape->H_kv : 0, O, ws, ws_bytes, stream,
                               "pw_union_attention launch");
}

pw_status pw_union_attention_heads(const pw_shape* shape, const uint16_t* Q,
                                   const uint8_t* K_fp8, const uint8_t* V_fp8,
                                   const float* scales, const int32_t* sel_pages,
                                   const int32_t* query_ids, int32_t g, int32_t h_begin,
                                   int32_t h_count, uint16_t* O, void* ws, size_t ws_bytes,
                                   void* stream) {
  return union_attention_range(shape, Q, K_fp8, V_fp8, scales, sel_pages, query_ids, g, h_begin,
                               h_count, O, ws, ws_bytes, stream, "pw_union_attention_heads launch");
}

pw_status pw_union_attention_noalloc(const pw_shape* shape, const uint16_t* Q,
                                     const uint8_t* K_fp8, const uint8_t* V_fp8,
                                     const float* scales, const int32_t* sel_pages,
                                     const int32_t* query_ids, int32_t g, uint16_t* O,
                                     void* stream) {
  pw_status st = check_shape(shape);
  if (st != PW_OK) return st;
  if (!Q || !K_fp8 || !V_fp8 || !scales || !sel_pages || !query_ids || !O)
    return fail(PW_ERR_NULL, "Q, K_fp8, V_fp8, scales, sel_pages, query_ids and O are required");
  st = check_aligned({{"Q", Q, 16}, {"K_fp8", K_fp8, 16}, {"V_fp8", V_fp8, 16}, {"scales", scales, 4},
                      {"sel_pages", sel_pages, sel_align(shape)}, {"query_ids", query_ids, 4},
                      {"O", O, 16}});
  if (st != PW_OK) return st;
  st = check_attention_support(shape, g);
  if (st != PW_OK) return st;
  const size_t need = pw::tiled_kv_bytes(*shape);
  if (need > PW_NOALLOC_SCRATCH_BYTES)
    return fail(PW_ERR_UNSUPPORTED,
                "re-tiled K/V of %zu bytes exceeds the %zu-byte no-alloc scratch "
                "(use pw_union_attention with a workspace)",
                need, (size_t)PW_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipError_t e = pw::noalloc_scratch(&ws, &ws_bytes);
  if (e != hipSuccess) return hip_status(e, "pw_union_attention_noalloc scratch lookup");
  if (ws_bytes < need) return fail(PW_ERR_WORKSPACE, "no-alloc scratch %zu < %zu bytes", ws_bytes, need);
  return hip_status(pw::launch_union_attention(*shape, Q, K_fp8, V_fp8, scales, sel_pages,
                                               query_ids, g, 0, shape->H_kv, O, ws,
                                               (hipStream_t)stream),
                    "pw_union_attention_noalloc launch");
}

pw_status pw_tile_kv(const pw_shape* shape, const uint8_t* K_fp8, const uint8_t* V_fp8,
                     const float* scales, void* ws, size_t ws_bytes, void* stream) {
  pw_status st = check_shape(shape);
  if (st != PW_OK) return st;
  if (!K_fp8 || !V_fp8 || !scales) return fail(PW_ERR_NULL, "K_fp8, V_fp8 and scales are required");
  st = check_aligned({{"K_fp8", K_fp8, 16}, {"V_fp8", V_fp8, 16}, {"scales", scales, 4}});
  if (st != PW_OK) return st;
  st = check_attention_support(shape, 1);
  if (st != PW_OK) return st;
  st = check_tiled_workspace(shape, ws, ws_bytes);
  if (st != PW_OK) return st;
  return hip_status(pw::tile_kv(*shape, K_fp8, V_fp8, scales, static_cast<uint8_t*>(ws),
                                (hipStream_t)stream),
                    "pw_tile_kv launch");
}

static pw_status tiled_attention(const pw_shape* shape, const uint16_t* Q,
                                 const int32_t* sel_pages, const int32_t* query_ids,
                                 const int32_t* group_order, int32_t g, uint16_t* O,
                                 const void* ws, size_t ws_bytes, void* stream, const char* what,
                                 bool fp8_qp = false) {
  pw_status st = check_shape(shape);
  if (st != PW_OK) return st;
  if (!Q || !sel_pages || !query_ids || !O)
    return fail(PW_ERR_NULL, "Q, sel_pages, query_ids and O are required");
  st = check_aligned({{"Q", Q, 16}, {"sel_pages", sel_pages, sel_align(shape)},
                      {"query_ids", query_ids, 4}, {"group_order", group_order, 4}, {"O", O, 16}});
  if (st != PW_OK) return st;
  st = check_attention_support(shape, g);
  if (st != PW_OK) return st;
  st = check_tiled_workspace(shape, ws, ws_bytes);
  if (st != PW_OK) return st;
  return hip_status(pw::launch_union_attention_tiled(*shape, Q, sel_pages, query_ids, g, 0,
                                                     shape->H_kv, O, ws, (hipStream_t)stream,
                                                     group_order, fp8_qp),
                    what);
}

pw_status pw_union_attention_tiled(const pw_shape* shape, const uint16_t* Q,
                                   const int32_t* sel_pages, const int32_t* query_ids, int32_t g,
                                   uint16_t* O, const void* ws, size_t ws_bytes, void* stream) {
  return tiled_attention(shape, Q, sel_pages, query_ids, nullptr, g, O, ws, ws_bytes, stream,
                         "pw_union_attention_tiled launch");
}

pw_status pw_union_attention_tiled_ordered(const pw_shape* shape, const uint16_t* Q,
                                           const int32_t* sel_pages, const int32_t* query_ids,
                                           const int32_t* group_order, int32_t g, uint16_t* O,
                                           const void* ws, size_t ws_bytes, void* stream) {
  if (!group_order) return fail(PW_ERR_NULL, "group_order is required");
  return tiled_attention(shape, Q, sel_pages, query_ids, group_order, g, O, ws, ws_bytes, stream,
                         "pw_union_attention_tiled_ordered launch");
}

pw_status pw_union_attention_tiled_fp8qp(const pw_shape* shape, const uint16_t* Q,
                                         const int32_t* sel_pages, const int32_t* query_ids,
                                         const int32_t* group_order, int32_t g, uint16_t* O,
                                         const void* ws, size_t ws_bytes, void* stream) {
  return tiled_attention(shape, Q, sel_pages, query_ids, group_order, g, O, ws, ws_bytes, stream,
                         "pw_union_attention_tiled_fp8qp launch", true);
}

size_t pw_dense_union_ref_workspace_bytes(const pw_shape* shape) {
  if (check_shape(shape) != PW_OK) return 0;
  return pw::dense_union_workspace(*shape);
}

pw_status pw_dense_union_ref(const pw_shape* shape, const uint16_t* Q, const uint8_t* K_fp8,
                             const uint8_t* V_fp8, const float* scales, const int32_t* sel_pages,
                             uint16_t* O, void* ws, size_t ws_bytes, void* stream) {
  pw_status st = check_shape(shape);
  if (st != PW_OK) return st;
  if (!Q || !K_fp8 || !V_fp8 || !scales || !sel_pages || !O)
    return fail(PW_ERR_NULL, "Q, K_fp8, V_fp8, scales, sel_pages and O are required");
  st = check_aligned({{"Q", Q, 16}, {"K_fp8", K_fp8, 16}, {"V_fp8", V_fp8, 16}, {"scales", scales, 4},
                      {"sel_pages", sel_pages, sel_align(shape)}, {"O", O, 16}});
  if (st != PW_OK) return st;
  st = check_attention_support(shape, 1);
  if (st != PW_OK) return st;
  if (shape->H_q / shape->H_kv > 8)
    return fail(PW_ERR_UNSUPPORTED, "G = %d exceeds 8 for the page-pair tiles", shape->H_q / shape->H_kv);
  if (shape->N_pages > 4096)
    return fail(PW_ERR_UNSUPPORTED, "N_pages = %d exceeds 4096 for the page-pair lists", shape->N_pages);
  if (pw::tiled_kv_bytes(*shape) / 2 > 0x7FFFFFFFu)
    return fail(PW_ERR_UNSUPPORTED, "tiled K/V of %zu bytes exceeds 2 GiB",
                pw::tiled_kv_bytes(*shape) / 2);
  const size_t need = pw::dense_union_workspace(*shape);
  if (need > 0 && !ws) return fail(PW_ERR_NULL, "workspace of %zu bytes required", need);
  if (ws_bytes < need) return fail(PW_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (((uintptr_t)ws & 255) != 0) return fail(PW_ERR_DIMS, "workspace must be 256-byte aligned");
  return hip_status(pw::launch_dense_union(*shape, Q, K_fp8, V_fp8, scales, sel_pages, nullptr, O,
                                           ws, ws_bytes, (hipStream_t)stream),
                    "pw_dense_union_ref launch");
}

pw_status pw_dense_union_paired(const pw_shape* shape, const uint16_t* Q, const uint8_t* K_fp8,
                                const uint8_t* V_fp8, const float* scales,
                                const int32_t* sel_pages, const int32_t* pairs, uint16_t* O,
                                void* ws, size_t ws_bytes, void* stream) {
  pw_status st = check_shape(shape);
  if (st != PW_OK) return st;
  if (!Q || !K_fp8 || !V_fp8 || !scales || !sel_pages || !pairs || !O)
    return fail(PW_ERR_NULL, "Q, K_fp8, V_fp8, scales, sel_pages, pairs and O are required");
  st = check_aligned({{"Q", Q, 16}, {"K_fp8", K_fp8, 16}, {"V_fp8", V_fp8, 16}, {"scales", scales, 4},
                      {"sel_pages", sel_pages, sel_align(shape)}, {"pairs", pairs, 8}, {"O", O, 16}});
  if (st != PW_OK) return st;
  st = check_attention_support(shape, 1);
  if (st != PW_OK) return st;
  if (shape->H_q / shape->H_kv > 8)
    return fail(PW_ERR_UNSUPPORTED, "G = %d exceeds 8 for the page-pair tiles", shape->H_q / shape->H_kv);
  if (shape->N_pages > 2048)
    return fail(PW_ERR_UNSUPPORTED, "N_pages = %d exceeds 2048 for a pair table", shape->N_pages);
  if (pw::tiled_kv_bytes(*shape) / 2 > 0x7FFFFFFFu)
    return fail(PW_ERR_UNSUPPORTED, "tiled K/V of %zu bytes exceeds 2 GiB",
                pw::tiled_kv_bytes(*shape) / 2);
  const size_t need = pw::dense_union_workspace(*shape);
  if (!ws) return fail(PW_ERR_NULL, "workspace of %zu bytes required", need);
  if (ws_bytes < need) return fail(PW_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (((uintptr_t)ws & 255) != 0) return fail(PW_ERR_DIMS, "workspace must be 256-byte aligned");
  return hip_status(pw::launch_dense_union(*shape, Q, K_fp8, V_fp8, scales, sel_pages, pairs, O,
                                           ws, ws_bytes, (hipStream_t)stream),
                    "pw_dense_union_paired launch");
}

size_t pw_page_pairs_workspace_bytes(const pw_shape* shape) {
  if (check_shape(shape) != PW_OK) return 0;
  return pw::page_pairs_workspace(*shape);
}

pw_status pw_page_pairs(const pw_shape* shape, const int32_t* sel_pages, int32_t* pairs,
                        void* ws, size_t ws_bytes, void* stream) {
  pw_status st = check_shape(shape);
  if (st != PW_OK) return st;
  if (!sel_pages || !pairs) return fail(PW_ERR_NULL, "sel_pages and pairs are required");
  st = check_aligned({{"sel_pages", sel_pages, sel_align(shape)}, {"pairs", pairs, 8}});
  if (st != PW_OK) return st;
  if (shape->N_pages > 2048)
    return fail(PW_ERR_UNSUPPORTED, "N_pages = %d exceeds 2048 for the pairing", shape->N_pages);
  if (shape->T >= (1 << 19))
    return fail(PW_ERR_UNSUPPORTED, "T = %d exceeds the co-selection count range", shape->T);
  if ((size_t)shape->H_kv * shape->N_pages * shape->N_pages >= ((size_t)1 << 31))
    return fail(PW_ERR_UNSUPPORTED, "H_kv * N_pages^2 co-selection counts exceed 2^31");
  const size_t need = pw::page_pairs_workspace(*shape);
  if (!ws) return fail(PW_ERR_NULL, "workspace of %zu bytes required", need);
  if (ws_bytes < need) return fail(PW_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (((uintptr_t)ws & 255) != 0) return fail(PW_ERR_DIMS, "workspace must be 256-byte aligned");
  return hip_status(pw::launch_page_pairs(*shape, sel_pages, pairs, ws, (hipStream_t)stream),
                    "pw_page_pairs launch");
}

size_t pw_select_workspace_bytes(const pw_shape* shape) {
  if (check_shape(shape) != PW_OK) return 0;
  return pw::select_workspace(*shape);
}

pw_status pw_select(const pw_shape* shape, const uint16_t* Q, const uint8_t* K_fp8,
                    const float* scales, int32_t n_local, int32_t* sel_pages, void* ws,
                    size_t ws_bytes, void* stream) {
  pw_status st = check_shape(shape);
  if (st != PW_OK) return st;
  if (!Q || !K_fp8 || !scales || !sel_pages)
    return fail(PW_ERR_NULL, "Q, K_fp8, scales and sel_pages are required");
  st = check_aligned({{"Q", Q, 16}, {"K_fp8", K_fp8, 16}, {"scales", scales, 4},
                      {"sel_pages", sel_pages, sel_align(shape)}});
  if (st != PW_OK) return st;
  if (shape->D != 64 && shape->D != 128)
    return fail(PW_ERR_UNSUPPORTED, "D = %d not in {64, 128}", shape->D);
  if (shape->P != 16 && shape->P != 32 && shape->P != 64)
    return fail(PW_ERR_UNSUPPORTED, "P = %d not in {16, 32, 64}", shape->P);
  if (shape->N_pages > 1024)
    return fail(PW_ERR_UNSUPPORTED, "N_pages = %d exceeds 1024 for the selector", shape->N_pages);
  if (n_local < 1 || n_local + 1 > shape->S)
    return fail(PW_ERR_UNSUPPORTED, "n_local = %d needs 1 <= n_local <= S - 1 (S = %d)", n_local,
                shape->S);
  const size_t need = pw::select_workspace(*shape);
  if (!ws) return fail(PW_ERR_NULL, "workspace of %zu bytes required", need);
  if (ws_bytes < need) return fail(PW_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (((uintptr_t)ws & 255) != 0) return fail(PW_ERR_DIMS, "workspace must be 256-byte aligned");
  return hip_status(pw::launch_select(*shape, Q, K_fp8, scales, n_local, sel_pages, ws,
                                      (hipStream_t)stream),
                    "pw_select launch");
}

}  // extern "C"
