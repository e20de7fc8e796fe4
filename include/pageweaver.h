/*
 * pageweaver.h -- C ABI of the query-union sparse-attention prefill path over
 * a paged FP8 KV cache, for AMD Instinct MI355X (gfx950) only.
 *
 * Sources (cited by title and section):
 *   [abs]   "PageWeaver: KV-Guided Query Unions for Sparse Attention",
 *           arXiv 2610.11201, Abstract.
 *   [radio] AI Radio episode "PageWeaver: KV-Guided Query Unions for Sparse
 *           Attention", sections "Paper summary" and "Conclusion".
 *
 * The path has two calls that together form one complete call [abs: the
 * speedups are quoted on the complete call, search plus attention]:
 *   pw_group            a bounded search that only produces query IDs;
 *   pw_union_attention  an ID-aware attention that reads Q rows by ID, loads
 *                       each group's union of selected pages once and gives
 *                       every query its own full attention over exactly its
 *                       own selected pages (no reordered Q, no cross-page
 *                       partial outputs) [abs].
 * A third call, pw_dense_union_ref, is the direct KV-page union design study
 * [abs; radio "Paper summary": disjoint page pairs, full membership, common
 * and exclusive query lists] and produces the same O through per-pair partial
 * outputs and a merge.
 *
 * Conventions for every call:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library keeps no reference after the call is enqueued.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising.
 *   - The library allocates no device memory; scratch space comes from the
 *     caller's workspace (`ws`, `ws_bytes`), sized by the matching
 *     *_workspace_bytes() query.  A call whose query returns 0 accepts
 *     ws = NULL.
 *   - Problems that can be checked on the host are reported before anything
 *     is enqueued, through the returned status; pw_last_error() then holds a
 *     message for the calling thread.  A HIP launch failure returns
 *     PW_ERR_HIP.  No call aborts, throws or prints.
 *   - Calls are re-entrant: there is no global mutable state besides the
 *     thread-local error message.
 *
 * Shapes (pw_shape):
 *   T        tokens of the prefilled context = number of queries; query t is
 *            at token t and sees key j iff j <= t (whole-context causal
 *            prefill).
 *   H_q,H_kv query and KV heads; G = H_q / H_kv; Q head hq reads KV head
 *            hq / G.
 *   D        head dimension (64 or 128).
 *   P        page size in tokens (16, 32 or 64); key j lives in page j / P,
 *            slot j % P.
 *   N_pages  pages of the cache; T == N_pages * P.
 *   S        selected-page slots per (KV head, query).
 *
 * Tensor layouts (row-major, innermost last):
 *   sel_pages int32 [H_kv][T][S]     selected pages of each (KV head, query).
 *             A slot outside [0, N_pages) is empty; repeated pages count
 *             once (the support is a set); order does not matter.
 *   query_ids int32 [H_kv][T]        per KV head, a permutation of 0..T-1;
 *             group k of that head is entries [k*g, k*g + g).
 *   Q         bf16  [T][H_q][D]      (bit patterns as uint16).
 *   K_fp8     e4m3fn [N_pages][H_kv][P][D]   token-major pages.
 *   V_fp8     e4m3fn [N_pages][H_kv][P][D]   token-major pages (same layout
 *             as K).
 *   scales    fp32  [2][N_pages][H_kv]        K scale then V scale of each
 *             (page, KV head); the value of a code is e4m3fn(code) * scale.
 *             Scales must be positive and finite.
 *   O         bf16  [T][H_q][D]      output, one writer per row.
 *
 * Alignment (else PW_ERR_DIMS): Q, K_fp8, V_fp8 and O 16 bytes (their rows
 * move 16 bytes at a time); sel_pages 16 bytes when S is a multiple of 4,
 * else 4; page pairs 8; every other int32 / fp32 array 4.
 *
 * e4m3fn is the OCP 8-bit E4M3 format with a NaN and no infinities (max 448).
 */
#ifndef PAGEWEAVER_H
#define PAGEWEAVER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pw_status {
  PW_OK = 0,
  PW_ERR_NULL = -1,        /* a required pointer is NULL                     */
  PW_ERR_DIMS = -2,        /* inconsistent or non-positive dimensions        */
  PW_ERR_UNSUPPORTED = -3, /* valid but outside the compiled support set     */
  PW_ERR_WORKSPACE = -4,   /* workspace smaller than *_workspace_bytes()     */
  PW_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed     */
} pw_status;

typedef struct pw_shape {
  int32_t T, H_q, H_kv, D, P, N_pages, S;
} pw_shape;

/* ---------------------------------------------------------------------------
 * pw_group -- bounded-window greedy grouping; produces query IDs only.
 *
 * [abs]: a bounded GPU search produces query IDs.  [radio "Paper summary"]:
 * within a bounded window W the members of a query-owned group are collected
 * greedily, taking queries whose selected sets add few new pages; the group
 * size g is fixed independently of W.
 *
 * For every KV head h and every aligned window of W consecutive query IDs
 * [w*W, min(T, (w+1)*W)): repeatedly, the lowest unassigned ID seeds a group
 * whose union U starts as its support; then, until the group has g members or
 * the window is exhausted, the unassigned query c minimising
 * (|support(c) \ U| in pages, c) joins and U grows by its support.  IDs are
 * written window by window, group by group, members in insertion order.  The
 * result is unique, so it is bit-exact against any correct implementation.
 *
 * In : sel_pages (see layouts), W in [1, 1024], g in [1, 16], W a multiple
 *      of g (otherwise PW_ERR_UNSUPPORTED: the attention reads groups as
 *      fixed runs of g IDs, which would then straddle windows).  T need not be
 *      a multiple of W: the last window is shorter, and its last group may
 *      have fewer than g members.
 * Out: query_ids int32 [H_kv][T] (every entry written).
 * Support set: N_pages <= 1024.  Workspace: none (returns 0).
 * ------------------------------------------------------------------------- */
size_t pw_group_workspace_bytes(const pw_shape* shape, int32_t W, int32_t g);
pw_status pw_group(const pw_shape* shape, const int32_t* sel_pages, int32_t W,
                   int32_t g, int32_t* query_ids, void* ws, size_t ws_bytes,
                   void* stream);

/* ---------------------------------------------------------------------------
 * pw_group_ordered -- pw_group plus an execution order of the groups.
 *
 * [abs]: query unions share page loads.  The groups that the attention runs
 * side by side also share pages through the caches when they sweep their
 * ascending page lists in step, which happens when their unions have similar
 * sizes and come from nearby queries.  The search knows every union it builds,
 * so it also emits an order: per KV head, the group indices 0 .. ceil(T/g) - 1
 * cut into blocks of B consecutive groups, B = 256 / ceil(g * G / 32) (the
 * groups the attention runs at once on one XCD of the MI355X: 256 resident
 * waves, ceil(g * G / 32) waves per group); blocks in increasing index order,
 * and within a block the groups by ascending union size (the number of
 * distinct pages the members select), equal sizes in increasing index.
 * pw_union_attention_tiled_ordered runs the groups listed last first.
 *
 * In : as pw_group.  Out: query_ids int32 [H_kv][T], identical to pw_group's;
 *      group_order int32 [H_kv][ceil(T/g)] (device).
 * Workspace: pw_group_ordered_workspace_bytes() = H_kv * ceil(T/g) * 4 bytes
 * (the union sizes), required; it and group_order must be 4-byte aligned
 * (else PW_ERR_DIMS).  Support set and other errors as pw_group.
 * ------------------------------------------------------------------------- */
size_t pw_group_ordered_workspace_bytes(const pw_shape* shape, int32_t W, int32_t g);
pw_status pw_group_ordered(const pw_shape* shape, const int32_t* sel_pages, int32_t W,
                           int32_t g, int32_t* query_ids, int32_t* group_order, void* ws,
                           size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pw_check_ids -- is every query_ids row a permutation of 0..T-1?
 *
 * pw_union_attention writes exactly the rows listed in query_ids; with a row
 * that is not a permutation, unlisted outputs stay unwritten.  This optional
 * device-side check lets a caller verify IDs that did not come from pw_group
 * without a host round trip of its own.
 *
 * Out: bad_counts int32 [H_kv] (device): per KV head, the number of entries
 * that are outside [0, T) or repeat an earlier entry of the row; every count
 * is 0 exactly when every row is a permutation.  Enqueued on `stream`.
 * Workspace: pw_check_ids_workspace_bytes(shape) = ceil(H_kv * T / 32) * 4
 * bytes, required.
 * ------------------------------------------------------------------------- */
size_t pw_check_ids_workspace_bytes(const pw_shape* shape);
pw_status pw_check_ids(const pw_shape* shape, const int32_t* query_ids, int32_t* bad_counts,
                       void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pw_union_attention -- ID-aware union attention.
 *
 * [abs]: query unions share page loads and fill matrix-core tiles; each query
 * keeps its original support and sole ownership of its output; the kernel
 * consumes the IDs without a reordered Q tensor and without cross-page
 * partial outputs.
 *
 * For each KV head h and group k (entries [k*g, k*g+g) of query_ids[h]), the
 * union of the members' selected pages is loaded once, in ascending page
 * order; every member t and each of its G Q heads hq computes
 *   O[t][hq] = sum_j softmax_j(<Q[t][hq], Khat_j> / sqrt(D)) Vhat_j
 * over exactly the keys j of its own selected pages with j <= t
 * (Khat/Vhat = e4m3fn(code) * scale).  O[t][hq] = 0 when that key set is
 * empty.  Arithmetic:
 *   - Q K^T on the FP8 matrix cores: the e4m3fn K codes as stored, times a
 *     two-part e4m3fn split of each Q row (the row is scaled by a power of two
 *     so that its largest magnitude lies in [128, 256), then hi = e4m3(q) and
 *     lo = e4m3(q - hi)); hi + lo equals the bf16 value for every element of
 *     magnitude >= 2^-2 after scaling (its last bit is then at least the
 *     e4m3 subnormal spacing 2^-9), and differs from it by at most 2^-10 (half
 *     that spacing) below, i.e. at most 2^-17 (7.6e-6) of the row's largest
 *     magnitude; fp32 accumulation;
 *   - fp32 online softmax;
 *   - P V on the bf16 matrix cores: P rounded to bf16 (RNE), the V codes
 *     converted to bf16 exactly; fp32 accumulation;
 *   - bf16 (RNE) output.
 * The result of a row does not depend on which other queries share its group.
 *
 * In : Q, K_fp8, V_fp8, scales, sel_pages, query_ids (see layouts), g in
 *      [1, 16] with g * G <= 64 and g * S <= 1024.  IDs outside [0, T) are skipped; a
 *      query_ids row that is not a permutation leaves unlisted rows of O
 *      unwritten.
 * Out: O.
 * Support set: D in {64, 128}; P in {16, 32, 64}; N_pages <= 32768; the
 * re-tiled K (and V) copy below at most 2 GiB.  Value range: the online
 * softmax works in fp32 base-2 logits, |<Q, Khat>| * log2(e) / sqrt(D) <
 * 2^20 (about 7e5 in natural units), and V scales below 2^60; beyond that an
 * fp32 reference maximum cannot resolve a row (or the unnormalised sums
 * overflow) and the output is unspecified.
 * Workspace: pw_union_attention_workspace_bytes() = 2 * N_pages * H_kv * 64 * D
 * + 16 * N_pages * H_kv (rounded up to 256) bytes, 256-byte aligned, required.
 * Each call first re-tiles the FP8 K and V pages into it in matrix-core operand
 * order (64 key slots per page, keys >= P zero), so that every page load of the
 * attention loop is a contiguous 1 KB wave read, and stores per page its
 * softmax factors (scales, and a bound from its largest key norm that lets the
 * softmax skip row maxima that cannot move); its contents are rebuilt by every
 * call.  pw_union_attention is exactly pw_tile_kv followed by
 * pw_union_attention_tiled on the same workspace and stream.
 * ------------------------------------------------------------------------- */
size_t pw_union_attention_workspace_bytes(const pw_shape* shape, int32_t g);
pw_status pw_union_attention(const pw_shape* shape, const uint16_t* Q,
                             const uint8_t* K_fp8, const uint8_t* V_fp8,
                             const float* scales, const int32_t* sel_pages,
                             const int32_t* query_ids, int32_t g, uint16_t* O,
                             void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pw_union_attention_noalloc -- pw_union_attention without a workspace.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, result and errors as pw_union_attention minus the workspace: the
 * re-tiled K/V copy and page factors live in a device array inside the
 * library, PW_NOALLOC_SCRATCH_BYTES (160 MiB) on each device the library runs
 * on, held until the process ends.  The call allocates nothing; its first call
 * on a device looks up that device's array (hipGetSymbolAddress).
 *
 * Limit: pw_union_attention_workspace_bytes(shape) <= PW_NOALLOC_SCRATCH_BYTES
 * (e.g. 1024 pages x 8 KV heads at D = 128 need 134 MB), else
 * PW_ERR_UNSUPPORTED.  Every call on a device uses that device's one array,
 * which keeps the last call's contents: calls that overlap on one device
 * (concurrent streams or threads) race and give unspecified results; calls on
 * one stream are ordered and safe.  Nothing needs clearing between calls (each
 * call rewrites all it reads).
 * ------------------------------------------------------------------------- */
#define PW_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)
pw_status pw_union_attention_noalloc(const pw_shape* shape, const uint16_t* Q,
                                     const uint8_t* K_fp8, const uint8_t* V_fp8,
                                     const float* scales, const int32_t* sel_pages,
                                     const int32_t* query_ids, int32_t g, uint16_t* O,
                                     void* stream);

/* ---------------------------------------------------------------------------
 * pw_tile_kv / pw_union_attention_tiled -- the two halves of
 * pw_union_attention.
 *
 * [abs]: the kernel loads each group's union of selected pages once; the
 * pages are read in matrix-core operand order from a re-tiled copy of the
 * cache.  pw_tile_kv writes that copy (and the per-page softmax factors) into
 * the workspace; pw_union_attention_tiled runs the attention on it.  A caller
 * that attends to the same K/V several times (other selections or IDs, other
 * Q) re-tiles once; the split also lets a caller time the two kernels apart.
 *
 * pw_tile_kv     In : K_fp8, V_fp8, scales (layouts above).  Out: ws.
 * pw_union_attention_tiled
 *                In : Q, sel_pages, query_ids, g (as pw_union_attention) and a
 *                     workspace that pw_tile_kv filled for the same shape, K,
 *                     V and scales (stream-ordered before this call; the
 *                     library cannot check its contents).  Out: O.
 * Workspace (both): pw_union_attention_workspace_bytes() bytes, 256-byte
 * aligned, required.  Support set and errors as pw_union_attention.
 * ------------------------------------------------------------------------- */
pw_status pw_tile_kv(const pw_shape* shape, const uint8_t* K_fp8, const uint8_t* V_fp8,
                     const float* scales, void* ws, size_t ws_bytes, void* stream);
pw_status pw_union_attention_tiled(const pw_shape* shape, const uint16_t* Q,
                                   const int32_t* sel_pages, const int32_t* query_ids,
                                   int32_t g, uint16_t* O, const void* ws, size_t ws_bytes,
                                   void* stream);

/* ---------------------------------------------------------------------------
 * pw_union_attention_tiled_ordered -- pw_union_attention_tiled with each KV
 * head's groups run in a given order.
 *
 * [abs]: query unions share page loads (see pw_group_ordered for the order).
 * group_order int32 [H_kv][ceil(T/g)] (device): per KV head a permutation of
 * the group indices, e.g. from pw_group_ordered; the entries listed last run
 * first.  An entry outside [0, ceil(T/g)) runs no group, so a row that is not
 * a permutation leaves the output rows of the groups it misses unwritten.
 * The output does not depend on the order: it equals
 * pw_union_attention_tiled's bit for bit.  Other arguments, workspace and
 * errors as pw_union_attention_tiled.
 * ------------------------------------------------------------------------- */
pw_status pw_union_attention_tiled_ordered(const pw_shape* shape, const uint16_t* Q,
                                           const int32_t* sel_pages, const int32_t* query_ids,
                                           const int32_t* group_order, int32_t g, uint16_t* O,
                                           const void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pw_union_attention_tiled_fp8qp -- a lower-precision variant of
 * pw_union_attention_tiled with Q and P in FP8 as well.
 *
 * [abs]: the KV cache is FP8; the pages leave the precision of Q and of the
 * softmax probabilities open, and the exact path keeps both at bf16 accuracy.
 * This variant follows the FP8 mode of FlashAttention-3 ([mls-builds]): each Q
 * row, scaled by a power of two so that its largest magnitude lies in
 * [128, 256), is rounded to e4m3fn (one part, no residual), and each page's
 * probabilities p = 2^(s - m) * phi are rounded to e4m3fn, where m is the
 * row's reference maximum (it moves when a page's largest score passes it by
 * more than 6, log2 units) and v_scale = phi * 2^k with phi in [1, 2); 2^k is
 * applied as the MFMA's scale of P.  Both products then run on the FP8 matrix
 * cores (QK^T at half, PV at about half the matrix cycles of the exact path).
 * The row sums add the rounded p / phi, so every output row is a convex
 * combination of its visible V rows.  The result differs from the method's
 * exact attention by the e4m3 rounding of q and p (measured on the synthetic
 * 64K workload: max-abs 0.12, mean-abs 4e-3; with rows four times as peaked:
 * max-abs 0.37, mean-abs 2e-2); it is NOT within the tolerance the exact path
 * meets.
 *
 * Arguments, layouts, workspace and errors as pw_union_attention_tiled, plus
 * group_order as pw_union_attention_tiled_ordered, here optional (NULL: the
 * groups run in index order).  V scales must lie in [2^-127, 2^127].
 * ------------------------------------------------------------------------- */
pw_status pw_union_attention_tiled_fp8qp(const pw_shape* shape, const uint16_t* Q,
                                         const int32_t* sel_pages, const int32_t* query_ids,
                                         const int32_t* group_order, int32_t g, uint16_t* O,
                                         const void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pw_union_attention_heads -- pw_union_attention for KV heads
 * [h_begin, h_begin + h_count) only.
 *
 * [radio "Conclusion"]: the cost of a call includes building its groups; the
 * search and the attention are independent per KV head, so a caller can run
 * the search of later heads while earlier heads attend: pw_group on a head
 * range (pass sel_pages and query_ids offset by h_begin rows and a shape with
 * H_kv = h_count, H_q = G * h_count: both layouts are head-major), then this
 * call for the same range on another stream once that search is done.
 *
 * Arguments as pw_union_attention (full shape, full tensors); only the rows of
 * O of Q heads [h_begin * G, (h_begin + h_count) * G) are written, and only the
 * range's heads of the workspace's re-tiled K/V copy.  Calls for disjoint head
 * ranges may therefore share one workspace and run concurrently on different
 * streams.  Out-of-range heads: PW_ERR_DIMS.
 * ------------------------------------------------------------------------- */
pw_status pw_union_attention_heads(const pw_shape* shape, const uint16_t* Q,
                                   const uint8_t* K_fp8, const uint8_t* V_fp8,
                                   const float* scales, const int32_t* sel_pages,
                                   const int32_t* query_ids, int32_t g, int32_t h_begin,
                                   int32_t h_count, uint16_t* O, void* ws, size_t ws_bytes,
                                   void* stream);

/* ---------------------------------------------------------------------------
 * pw_dense_union_ref -- direct KV-page union (design-study comparison).
 *
 * [abs]: a direct KV-page union implementation studies non-local reuse
 * against reduction cost.  [radio "Paper summary"]: it uses disjoint page
 * pairs and the full membership of each page to form common or exclusive
 * query lists.
 *
 * Pages are paired as (2k, 2k+1).  Per KV head, the full membership of each
 * pair (every query that selected either page) is built on the device; each
 * (query, pair) computes a partial (running max, sum, unnormalised output)
 * over its own visible keys in the pair (both pages for the common list, one
 * page for an exclusive list), written to the workspace; a second pass merges
 * each query's partials by log-sum-exp into O.  Same O as
 * pw_union_attention up to floating-point order.
 *
 * In/Out/support: as pw_union_attention (no query_ids), plus G <= 8 and
 * N_pages <= 4096; queries are processed in chunks sized so that the partial
 * outputs stay within about 4 GiB of workspace (plus the re-tiled K/V copy).
 * Workspace: pw_dense_union_ref_workspace_bytes(shape) bytes, 256-byte
 * aligned.
 * ------------------------------------------------------------------------- */
size_t pw_dense_union_ref_workspace_bytes(const pw_shape* shape);
pw_status pw_dense_union_ref(const pw_shape* shape, const uint16_t* Q,
                             const uint8_t* K_fp8, const uint8_t* V_fp8,
                             const float* scales, const int32_t* sel_pages,
                             uint16_t* O, void* ws, size_t ws_bytes,
                             void* stream);

/* ---------------------------------------------------------------------------
 * pw_page_pairs -- affinity page pairs for the direct KV-page union.
 *
 * [abs]: the direct KV-page union weighs non-local reuse against the cost of
 * reducing partial outputs; [radio "Paper summary"]: it works on disjoint page
 * pairs with common and exclusive query lists.  Pairing pages that many
 * queries select together moves entries to common lists and cuts the number
 * of (query, pair) partials.
 *
 * Per KV head h: co[u][v] = number of queries t whose support (the valid
 * entries of sel_pages[h][t]) holds both pages u != v.  The pairs are the
 * greedy matching on the edges with co > 0 taken in the order (larger co,
 * then lower first page, then lower second page): an edge is taken when both
 * pages are still free.  Pages left free stay single.  The result is unique,
 * so it is bit-exact against any correct implementation.
 *
 * In : sel_pages (see layouts).
 * Out: pairs int32 [H_kv][N_pages][2] (device): row k = (a, b) with a < b, or
 *      (a, -1) for a single page; rows are ordered by a and every page appears
 *      exactly once; rows past the head's last pair are (-1, -1).
 * Support set: N_pages <= 2048, T < 2^19.
 * Workspace: pw_page_pairs_workspace_bytes(shape) bytes (page columns as
 * query bitsets and the co-selection counts, H_kv * N_pages^2 * 4 bytes),
 * 256-byte aligned.
 * ------------------------------------------------------------------------- */
size_t pw_page_pairs_workspace_bytes(const pw_shape* shape);
pw_status pw_page_pairs(const pw_shape* shape, const int32_t* sel_pages, int32_t* pairs,
                        void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pw_dense_union_paired -- pw_dense_union_ref over a given page pairing.
 *
 * As pw_dense_union_ref, with pairs taken from `pairs` (int32 [H_kv][N_pages]
 * [2], the layout pw_page_pairs writes) instead of (2k, 2k+1).  Each head's
 * rows must partition its pages: every page 0..N_pages-1 in exactly one row,
 * rows (-1, -1) ignored; a page in no row is treated as unselected and a page
 * in two rows gives unspecified results.  Same O as pw_union_attention up to
 * floating-point order, for any partition.
 *
 * Support set: as pw_dense_union_ref, with N_pages <= 2048.
 * Workspace: pw_dense_union_ref_workspace_bytes(shape) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------- */
pw_status pw_dense_union_paired(const pw_shape* shape, const uint16_t* Q, const uint8_t* K_fp8,
                                const uint8_t* V_fp8, const float* scales,
                                const int32_t* sel_pages, const int32_t* pairs, uint16_t* O,
                                void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pw_select -- a synthetic dynamic page selector producing sel_pages.
 *
 * [abs]: dynamic sparse attention gives every query its own set of selected
 * KV pages; the method takes that relation as given.  This call is a
 * stand-in selector (our own rule, in the block-sparse style) that derives
 * the relation from Q and K so the path can run on model-like selections.
 *
 * For KV head h and query t with own page p = t / P:
 *   fixed pages   0 and p, p-1, ..., p-n_local+1 (those >= 0);
 *   candidates    pages 1..p that are not fixed;
 *   score(u)      k_scale[u][h] * sum_d qs[d] * C_u[d], where qs is the sum of
 *                 the query's G head rows of Q and C_u[d] the sum over the
 *                 page's keys of e4m3fn(K[u][h][j][d]);
 *   the min(S - |fixed|, |candidates|) highest-scoring candidates are chosen
 *   (ties to the lower page); sel_pages[h][t] lists fixed and chosen pages in
 *   ascending order, padded with -1.
 * Scores are computed on the matrix cores from bf16 hi/lo parts of qs and C
 * (relative error about 2^-16 of sum_d |qs[d] C_u[d]|) with fp32 accumulation;
 * pages whose scores differ by less than that may be chosen either way.
 *
 * In : Q, K_fp8, scales (layouts above; the V half of scales is unused),
 *      n_local in [1, S - 1].
 * Out: sel_pages int32 [H_kv][T][S] (every entry written).
 * Support set: D in {64, 128}; P in {16, 32, 64}; N_pages <= 1024.
 * Workspace: pw_select_workspace_bytes(shape) = 4 * (T + N_pages) * D bytes of
 * bf16 operands plus T * N_pages * 4 bytes of scores (one KV head at a time),
 * 256-byte aligned, required.
 * ------------------------------------------------------------------------- */
size_t pw_select_workspace_bytes(const pw_shape* shape);
pw_status pw_select(const pw_shape* shape, const uint16_t* Q, const uint8_t* K_fp8,
                    const float* scales, int32_t n_local, int32_t* sel_pages, void* ws,
                    size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* pw_status_string(pw_status status);
/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* pw_last_error(void);
/* ABI version of this header, PW_ABI_VERSION. */
int32_t pw_abi_version(void);

#define PW_ABI_VERSION 4

#ifdef __cplusplus
}
#endif

#endif /* PAGEWEAVER_H */
