/*
 * mla_paged_kv.h -- C ABI of the MI355X (gfx950) MLA decode library.
 *
 * Multi-head latent attention decode over a paged KV cache: for every query
 * row (request r, new token i, head h)
 *
 *     out = softmax(scale * q . K^T) . V,   lse = log(sum_j exp(scale * q . k_j))
 *
 * where all h_q heads share one latent KV head of 576 dims (512 "NoPE" dims
 * followed by 64 RoPE dims) and V is its first 512 dims.  This is the dense MLA
 * decode of "Add SM80 (Ampere/A100) dense MLA decode kernel" (FlashMLA pull
 * request 183: Summary -- dense decode entry point plus combine kernel;
 * Design -- 576-dim Q/K, 512 V columns; Test plan -- causal multi-token
 * queries, split-K via the combine), and the packed top-k FP8 variant of
 * "[SM90] Add packed selected-KV sparse decode" (FlashMLA pull request 200:
 * "SM90 packing kernel", "Packed attention specialization", "Python API",
 * "Supported scope").
 *
 * Conventions for every call below:
 *   - Pointers marked (device) are device pointers on the current HIP device;
 *     the library dereferences none of them on the host.  `stream` is a
 *     hipStream_t (NULL = the default stream); every device-side call is
 *     asynchronous on it.
 *   - The caller allocates and owns every buffer.  The library allocates no
 *     device memory, keeps no per-call state and keeps no pointer after a call
 *     returns.  Inputs are only read.
 *   - Every call returns an mla_status.  Arguments outside the supported scope
 *     are rejected with MLA_ERR_UNSUPPORTED before anything is launched; bad
 *     pointers or sizes give MLA_ERR_INVALID_ARGUMENT or
 *     MLA_ERR_WORKSPACE_TOO_SMALL; a failed HIP call gives MLA_ERR_HIP.
 *     mla_last_error_message() describes the last failure on this thread.
 *   - Data-dependent preconditions (checking them would need a device sync)
 *     are the caller's contract: 0 <= seqlens[r] <= max_pages * 64, page ids of
 *     used blocks in [0, num_pages), top-k ids of the valid prefix in
 *     [0, num_pages * 64).  The kernels bounds-check them anyway, never read
 *     out of range, and record a violation in a device flag that
 *     mla_read_device_errors() returns.
 *   - With MLA_LOG set (and not "0") in the environment, every launch prints
 *     one line to stderr: for the decode its kernel instantiation, grid, block,
 *     split count, resident workgroups per CU, static LDS bytes and VGPRs; for
 *     the other kernels their main sizes.
 *
 * Layouts (all row-major, contiguous):
 *   q            bf16  [batch][s_q][h_q][576]
 *   kcache       bf16  [num_pages][64][h_kv][576]        (MLA_KV_BF16_PAGED; fp16
 *                  for MLA_KV_FP16_PAGED).  Query head h reads KV head
 *                  h / (h_q / h_kv): the h_q heads form h_kv contiguous groups
 *                  (multi-KV-head decode, swept over hk = 1..4 in the dense
 *                  page's Test plan); MLA itself has h_kv = 1.
 *   kcache_fp8   uint8 [num_pages][64][1][656]           656-byte records:
 *                  bytes [0,512) E4M3FN NoPE, [512,528) 4 x fp32 LE scales
 *                  (scale k covers NoPE dims [128k, 128k+128)), [528,656)
 *                  64 x bf16 LE RoPE.  Key = (e4m3 * scale, rope).
 *   block_table  int32 [batch][max_pages]   page id of each 64-token block
 *   seqlens      int32 [batch]   cached tokens per request, including the s_q
 *                                new ones; the s_q new tokens are the last s_q
 *                                positions (causal mask is bottom-right: token
 *                                i sees keys [0, seqlen - s_q + i])
 *   out          bf16  [batch][s_q][h_q][512]
 *   lse          fp32  [batch][s_q][h_q]   natural log; -inf for a row with no
 *                                          visible key (its out is 0)
 *   sched_meta   int32 [num_parts][8]      (see mla_get_decode_metadata)
 *   num_splits   int32 [batch + 1]         exclusive prefix sum of splits
 */
#ifndef MLA_PAGED_KV_H
#define MLA_PAGED_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_D_QK 576
#define MLA_D_V 512
#define MLA_PAGE_TOKENS 64
#define MLA_FP8_RECORD_BYTES 656
#define MLA_SCHED_META_INTS 8
#define MLA_MAX_ROWS 2048      /* s_q * h_q per request */
#define MLA_MAX_BATCH 65536
#define MLA_MAX_PARTS 8192
#define MLA_MAX_KV_HEADS 16    /* h_kv (dense formats; the sparse FP8 formats have 1) */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = -1,
  MLA_ERR_UNSUPPORTED = -2,
  MLA_ERR_WORKSPACE_TOO_SMALL = -3,
  MLA_ERR_HIP = -4
} mla_status;

typedef enum {
  MLA_KV_BF16_PAGED = 0,  /* kcache bf16 pages reached through block_table */
  MLA_KV_FP8_PACKED = 1,  /* the workspace written by mla_pack_selected_kv */
  MLA_KV_FP8_INDEXED = 2, /* the FP8 record pool itself, records gathered by
                             top-k index inside the decode (no pack) */
  MLA_KV_FP16_PAGED = 3   /* as MLA_KV_BF16_PAGED with q, kcache and out in
                             IEEE fp16 (binary16) -- the FP16 instantiation the
                             dense page's Test plan lists */
} mla_kv_format;

/* Text of the last error on the calling host thread ("" if none).  The
 * pointer stays valid until the next library call on that thread. */
const char* mla_last_error_message(void);

/* Recommended split count (partitions of the KV work) for a decode launch on
 * the current device: workgroups that fit per CU (from the compiled kernel's
 * LDS and register footprint, via the HIP occupancy query) times the CU
 * count, divided by the row blocks per request, then capped at an empirical
 * number of pieces per request: 64 for the 16-bit formats (of which
 * mla_get_decode_metadata uses only what the lengths call for) and 32 for the
 * FP8 formats (the partition count is scaled to resident workgroups rather
 * than to the CU count, and gated by measured limits: "How the occupancy work
 * went", FlashMLA PR 183).  Host only; queries the device. */
int mla_decode_num_parts(int batch, int s_q, int h_q, int h_kv, int kv_format, int* num_parts_out);

/* The same policy as a pure function of the device figures (for tests and for
 * callers planning for another device): cus = compute units, wgs_per_cu =
 * decode workgroups resident per CU. */
int mla_plan_num_parts(int batch, int s_q, int h_q, int h_kv, int kv_format, int cus, int wgs_per_cu,
                       int* num_parts_out);

/* Name of the decode kernel instantiation mla_decode_fwd launches for this
 * shape and format, as profilers print it without namespaces and parameters
 * (e.g. "decode_ws_kernel<4, false, false>"), so that a profile or a timing can
 * be attributed to the kernel that ran.  A static string owned by the library;
 * NULL (with mla_last_error_message set) for an unsupported shape.  Host only. */
const char* mla_decode_kernel_name(int s_q, int h_q, int h_kv, int kv_format);

/* Bytes of the caller-owned decode workspace (split partials: fp32 partial
 * outputs and lse for at most batch + num_parts splits).  0 on bad input. */
size_t mla_decode_workspace_size(int batch, int s_q, int h_q, int num_parts);

/* Bytes of the packed top-k workspace: batch * s_q * topk_capacity * 656
 * (one 656-byte record per selected slot; 2048 slots = 1,343,488 B per query
 * row -- "Runtime follow-up", FlashMLA PR 200).  0 on bad input. */
size_t mla_packed_kv_workspace_size(int batch, int s_q, int topk_capacity);

/* Scheduler metadata (device, one workgroup).  The dense page runs a
 * scheduler-metadata kernel ahead of the decode (get_decoding_sched_meta,
 * "Modifications outside csrc/sm80/", "Add SM80 (Ampere/A100) dense MLA decode
 * kernel", FlashMLA PR 183) and scales the partition count to resident
 * workgroups ("How the occupancy work went"); it does not spell out the
 * partition rule, so the rule below is this library's reading.  Splits the KV
 * blocks of all requests into num_parts contiguous partitions.  Definition:
 * request r has
 * ceil(seqlens[r] / 64) blocks (seqlens = topk_length for the packed path),
 * T blocks in total, and P' = min(num_parts, T, L) partitions are used, with
 * the split limit L = max(16 * batch, min(ceil(T / 4), 64 * batch)) (enough
 * pieces to spread long requests over the GPU, not so many that short ones
 * pay for partials they do not need; measured, see mla_decode_num_parts);
 * concatenating all requests' blocks in order, partition p < P' owns global
 * blocks [floor(p*T/P'), floor((p+1)*T/P')) -- at least one -- and
 * partitions p >= P' own none.
 *   sched_meta[p] = { begin_req, begin_block, end_req, end_block_exclusive,
 *                     split index of the first piece within begin_req, 0, 0, 0 }
 *                   or { -1, -1, -1, -1, -1, 0, 0, 0 } for an empty partition;
 *   num_splits[0] = 0, num_splits[r+1] = num_splits[r] + (partitions owning a
 *                   block of request r).
 * seqlens (device) [batch]; sched_meta (device) [num_parts][8]; num_splits
 * (device) [batch + 1].  Call once per decode step; reuse across layers. */
int mla_get_decode_metadata(const int32_t* seqlens, int batch, int s_q, int h_q, int h_kv, int num_parts,
                            int32_t* sched_meta, int32_t* num_splits, void* stream);

/* Scheduler policies of mla_get_packed_decode_metadata. */
typedef enum {
  MLA_SCHED_AUTO = 0,          /* = MLA_SCHED_GLOBAL on this GPU (measured; see below) */
  MLA_SCHED_GLOBAL = 1,        /* the partition of mla_get_decode_metadata */
  MLA_SCHED_REQUEST_LOCAL = 2  /* no partition spans two requests */
} mla_sched_policy;

/* Scheduler metadata for the sparse FP8 paths (device, one workgroup), the
 * get_packed_mla_metadata call of "[SM90] Add packed selected-KV sparse
 * decode" (FlashMLA PR 200, Python API, Scheduler policy).  Same outputs and
 * format as mla_get_decode_metadata, over topk_length.
 *   MLA_SCHED_GLOBAL: mla_get_decode_metadata's partition without the
 *     split limit (P' = min(num_parts, T)).
 *   MLA_SCHED_REQUEST_LOCAL: the page's "compact request-local scheduler",
 *     which it names without defining; here: with b_r = ceil(topk_length[r] /
 *     64) blocks, B = the smallest piece size with sum_r ceil(b_r / B) <=
 *     num_parts; request r is cut into ceil(b_r / B) balanced pieces (piece i =
 *     blocks [floor(i b_r / n_r), floor((i+1) b_r / n_r))), partitions follow in
 *     (request, piece) order and the rest are empty.  If more requests have a
 *     block than there are partitions, the global partition is produced.
 *   MLA_SCHED_AUTO: the page picks request-local for H = 64 outside a
 *     fallback regime on its GPU; on MI355X the global partition measured
 *     faster at every tested shape (h_q 64/128, batch * s_q 1..32), so AUTO
 *     is the global partition.
 * topk_length (device) int32 [batch]; sched_meta (device) [num_parts][8];
 * num_splits (device) [batch + 1]; h_q 64 or 128; topk_capacity a positive
 * multiple of 64. */
int mla_get_packed_decode_metadata(const int32_t* topk_length, int batch, int s_q, int h_q, int topk_capacity,
                                   int num_parts, int policy, int32_t* sched_meta, int32_t* num_splits,
                                   void* stream);

/* Decode (device): the dense decode kernel of "Add SM80 (Ampere/A100) dense MLA
 * decode kernel" (FlashMLA PR 183: Summary -- dense_decode_fwd plus the
 * combine kernel; Design -- 576-dim Q/K shared by all heads, 512 V columns;
 * Test plan -- BF16 and FP16, multi-KV-head, causal multi-token Q, split-K),
 * and for the FP8 formats the packed attention specialization of "[SM90] Add
 * packed selected-KV sparse decode" (FlashMLA PR 200: "Packed attention
 * specialization", partial-tail masking).
 * Launches num_parts x h_kv * ceil(s_q*h_q/h_kv / R) workgroups
 * (R = 16, 32 or 64 query rows of one KV head per workgroup); each walks its
 * partition's pages with an
 * online softmax and writes either the final out/lse rows (request not split)
 * or a split partial into `workspace`.  mla_combine must follow on the same
 * stream to finish split requests.
 *   q (device) bf16 [batch][s_q][h_q][576] (fp16 for MLA_KV_FP16_PAGED)
 *   kv (device): MLA_KV_BF16_PAGED -> kcache bf16 [num_pages][64][h_kv][576];
 *                MLA_KV_FP16_PAGED -> kcache fp16 [num_pages][64][h_kv][576], the
 *                same paging, masks and scope as bf16; P is rounded to fp16
 *                before PV and out is fp16;
 *                MLA_KV_FP8_PACKED -> packed workspace of mla_pack_selected_kv
 *                (then block_table/max_pages/num_pages are ignored, seqlens is
 *                topk_length, h_q must be 64 or 128, no causal; query token s of
 *                request r attends to workspace row r * s_q + s);
 *                MLA_KV_FP8_INDEXED -> kcache_fp8 uint8 [num_pages][64][1][656],
 *                the pool the pack reads: the decode gathers the selected
 *                records itself ("native" sparse decode, the fallback when the
 *                pack cannot be hidden: "[SM90] Add packed selected-KV sparse
 *                decode", FlashMLA PR 200, Motivation and Runtime follow-up).
 *                block_table is then the int32 [batch][s_q][topk_capacity]
 *                top-k physical token ids (page = id / 64, slot = id % 64; only
 *                k < topk_length[r] is read), max_pages is ignored, seqlens is
 *                topk_length, and the same scope as the packed path applies.
 *                Same arithmetic as the packed path: bitwise equal results for
 *                ids inside the pool.  An id outside it is flagged (bit 1) and
 *                read as id 0 (the pack writes a zero record instead); the
 *                output of a flagged call is not meaningful.
 *   block_table (device) int32 [batch][max_pages], seqlens (device) int32 [batch]
 *   softmax_scale: multiplies q.k (e.g. 576^-0.5); must be finite and > 0, else
 *                  MLA_ERR_INVALID_ARGUMENT; causal: 0/1
 *   sched_meta, num_splits (device): from mla_get_decode_metadata with the same
 *     seqlens, batch and num_parts
 *   out (device) bf16 [batch][s_q][h_q][512] (fp16 for MLA_KV_FP16_PAGED), lse
 *     (device) fp32 [batch][s_q][h_q]
 *   workspace (device) of >= mla_decode_workspace_size(batch, s_q, h_q, num_parts)
 * Scope: h_q a multiple of 16 with h_q <= 128; 1 <= h_kv <= 16 dividing h_q
 * (the FP8 formats: h_kv = 1); s_q * h_q <= 2048; gfx950 device. */
int mla_decode_fwd(const void* q, const void* kv, int kv_format, int64_t num_pages, const int32_t* block_table,
                   int max_pages, const int32_t* seqlens, int topk_capacity, int batch, int s_q, int h_q, int h_kv,
                   float softmax_scale, int causal, const int32_t* sched_meta, const int32_t* num_splits,
                   int num_parts, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Combine (device): the combine kernel that merges split-K partials ("Add
 * SM80 (Ampere/A100) dense MLA decode kernel", FlashMLA PR 183: Summary, and
 * "Modifications outside csrc/sm80/" on its split ladder; Test plan: split-K
 * via the combine kernel).  For every request with >= 2 splits, merges its partials
 * from `workspace` by log-sum-exp, L = log(sum_i exp(lse_i)),
 * out = sum_i exp(lse_i - L) * o_i, lse = L (a split with lse -inf has weight
 * 0); a request with 0 splits (no key) gets out = 0, lse = -inf; a request with
 * one split was finished by mla_decode_fwd and is left untouched.  The split
 * count is a runtime value; there is no fixed ladder of supported counts.
 * kv_format is the one the decode ran with: out is fp16 for
 * MLA_KV_FP16_PAGED, bf16 otherwise; the partials are fp32 either way. */
int mla_combine(const int32_t* num_splits, const void* workspace, size_t workspace_bytes, int batch, int s_q,
                int h_q, int num_parts, int kv_format, void* out, float* lse, void* stream);

/* Decode + combine with no caller workspace (device), for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, scope, kernels and results
 * as mla_decode_fwd followed by mla_combine on `stream`, except that the split
 * partials live in a device array the library owns: 128 MiB
 * (MLA_NOALLOC_SCRATCH_BYTES) per device, reserved when the library's device
 * code is loaded on that device and held until the process ends.  The call
 * itself allocates nothing.  mla_decode_workspace_size(batch, s_q, h_q,
 * num_parts) must not exceed that size, else MLA_ERR_WORKSPACE_TOO_SMALL
 * before any launch (use fewer parts or a smaller batch).  Every call on one
 * device shares that device's array and leaves its last contents there (every
 * slot a call reads is first written by that call's decode); calls whose
 * execution overlaps on one device (concurrent streams, or host threads using
 * one device) race on it and must be serialised by the caller. */
#define MLA_NOALLOC_SCRATCH_BYTES (((size_t)128) << 20)
int mla_decode_fwd_noalloc(const void* q, const void* kv, int kv_format, int64_t num_pages,
                           const int32_t* block_table, int max_pages, const int32_t* seqlens, int topk_capacity,
                           int batch, int s_q, int h_q, int h_kv, float softmax_scale, int causal,
                           const int32_t* sched_meta, const int32_t* num_splits, int num_parts, void* out, float* lse,
                           void* stream);

/* Pack (device): the packing kernel of "[SM90] Add packed selected-KV sparse
 * decode" (FlashMLA PR 200, "SM90 packing kernel": selected 656-byte records
 * copied byte for byte into a 64-token tile-major workspace, invalid suffix
 * zero-filled).  Copies the selected 656-byte records byte-for-byte into the
 * tile-major workspace ws[row][tile][slot][656], row = r * s_q + i,
 * tile = k / 64, slot = k % 64, for k < topk_length[r] the record of physical
 * token indices[r][i][k] (page = id / 64, slot = id % 64); slots
 * k >= topk_length[r] are zero-filled.  Tile t of a row is byte-identical to a
 * pool page holding that row's selected records k = 64t .. 64t+63 in order.
 *   kcache_fp8 (device) uint8 [num_pages][64][1][656]; indices (device) int32
 *   [batch][s_q][topk_capacity]; topk_length (device) int32 [batch];
 *   workspace (device) >= mla_packed_kv_workspace_size(batch, s_q, topk_capacity).
 * Scope: topk_capacity a positive multiple of 64. */
int mla_pack_selected_kv(const void* kcache_fp8, int64_t num_pages, const int32_t* indices,
                         const int32_t* topk_length, int batch, int s_q, int topk_capacity, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Current-token patch (device).  Packing ahead of attention (on another
 * stream, during preceding work) reads the pool before the current step's KV
 * is written; afterwards this call overwrites every selected slot that refers
 * to one of the changed tokens: for every row = r * s_q + i and slot
 * k < topk_length[r] with indices[r][i][k] == new_ids[r][j] for some j < n_new,
 * ws[row][k / 64][k % 64] = the record of that id in kcache_fp8.  If only the
 * listed records changed since the pack, the workspace then equals a fresh
 * pack of the current pool byte for byte.  ("Runtime follow-up", FlashMLA PR
 * 200: pack historical records early into caller-managed storage, overwrite
 * any selected current-token record once its KV is available, for example by
 * a scatter, then synchronise the packing stream with attention.)
 *   kcache_fp8, indices, topk_length, workspace: as for mla_pack_selected_kv
 *     (same batch, s_q, topk_capacity; workspace written by that pack);
 *   new_ids (device) int32 [batch][n_new]: the physical token ids whose
 *     records changed, per request; entries < 0 are ignored; a matching id
 *     outside [0, num_pages * 64) is flagged (bit 1) and not copied;
 *   n_new in [1, 64].
 * The pack must have completed (e.g. an event recorded after it on its
 * stream, waited on by `stream`) and the new records must be written before
 * this call runs on `stream`. */
int mla_patch_packed_kv(const void* kcache_fp8, int64_t num_pages, const int32_t* indices,
                        const int32_t* topk_length, int batch, int s_q, int topk_capacity, const int32_t* new_ids,
                        int n_new, void* workspace, size_t workspace_bytes, void* stream);

/* Sparse path choice (host).  *kv_format_out = MLA_KV_FP8_PACKED when the
 * pack can be hidden (pack_hidden != 0: the caller has an overlap window for
 * mla_pack_selected_kv) and mla_packed_kv_workspace_size(batch, s_q,
 * topk_capacity) <= workspace_budget_bytes; otherwise MLA_KV_FP8_INDEXED, the
 * decode that gathers by id and needs no packed workspace.  ("Runtime
 * follow-up", FlashMLA PR 200: choose the native path when the expected
 * overlap is insufficient; enforce a workspace budget, about 1.281 MiB per
 * query row at top-k 2048.)  An unhidden pack costs more than the packed
 * decode saves at every shape measured here. */
int mla_sparse_kv_format(int batch, int s_q, int topk_capacity, size_t workspace_budget_bytes, int pack_hidden,
                         int* kv_format_out);

/* Device-side violation flags accumulated by the kernels on the current
 * device since the last call (bit 0: page id out of range, bit 1: top-k id
 * out of range, bit 2: seqlen above max_pages * 64 or top-k length above the
 * capacity, bit 3: sched_meta / num_splits not produced by
 * mla_get_decode_metadata for this batch and num_parts).  Synchronises `stream`
 * and clears the flags. */
int mla_read_device_errors(int* flags_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_KV_H */
