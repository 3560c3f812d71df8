// C ABI of the MLA decode library (declarations and contracts: include/mla_paged_kv.h).
//
// Host side only: argument validation (fail closed before any launch, as the
// packed path's "Supported scope" on FlashMLA PR 200 asks of unsupported
// shapes), the occupancy-derived split count (FlashMLA PR 183, "How the
// occupancy work went"), workspace sizing and kernel dispatch.
#include <cmath>
#include "../../include/mla_paged_kv.h"

#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "mla_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MLA_OK;
}

// MLA_LOG=1 in the environment: one line per launch on stderr (decode: kernel,
// grid, split count, resident workgroups per CU, LDS bytes, VGPRs).
bool log_on() {
  static const bool on = [] {
    const char* v = getenv("MLA_LOG");
    return v && *v && strcmp(v, "0") != 0;
  }();
  return on;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Empirical partition gates.  Each extra piece re-reads the request's Q rows,
// runs a prologue/epilogue and writes a 128 x 513 fp32 partial that the
// combine re-reads, so splitting finer than the work needs costs bandwidth,
// while too few pieces leave CUs idle on long requests.  The 16-bit paths: the
// plan allows up to 64 pieces per request and the device scheduler, which
// sees the lengths, uses at most max(16 b, min(ceil(T / 4), 64 b)) of them
// (mla_internal.h).  Measured on MI355X (decode + combine, cold KV, h_q 128):
// b = 1 takes 21.7 / 27.6 / 36.6 / 60.5 us at sk = 1024 / 4096 / 16384 / 65536
// with 16 / 16 / 64 / 64 pieces, against 47.8 and 129.0 us for the last two at
// 16; b = 4, sk = 4096 is fastest at 64 (32.0 us against 33.5 at 128).  The
// FP8 kernel is slower per tile and gains from finer pieces (C5, packed decode
// + combine, cold: 35.8 us at 16 per request, 29.8 at 24, 28.8 at 32, 29.0 at
// 48 and 64; b = 64, h_q = 128, top-k 2048 is fastest at the plan's 2 per
// request: 80.4 us against 92.9 at 4).
constexpr int kMaxSplitsPerRequest = mla::kSplitCeilPerRequest;
constexpr int kMaxSplitsPerRequestFp8 = 32;

bool is_gfx950() {
  static int cache[64];  // 0 unknown, 1 gfx950, 2 other (benign race: same value written)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (dev >= 0 && dev < 64 && cache[dev]) return cache[dev] == 1;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return false;
  const bool yes = strncmp(p.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) cache[dev] = yes ? 1 : 2;
  return yes;
}

int check_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n == 0) return fail(MLA_ERR_HIP, "no HIP device: %s", hipGetErrorString(e));
  if (!is_gfx950()) return fail(MLA_ERR_UNSUPPORTED, "device is not gfx950 (MI355X)");
  return MLA_OK;
}

// Scope checks shared by the decode entry points.
int check_shape(int batch, int s_q, int h_q, int h_kv, int kv_format) {
  if (batch < 1 || batch > MLA_MAX_BATCH) return fail(MLA_ERR_INVALID_ARGUMENT, "batch %d out of [1, %d]", batch, MLA_MAX_BATCH);
  if (batch > mla::kSchedMaxBatch)
    return fail(MLA_ERR_UNSUPPORTED, "batch %d above the scheduler limit %d", batch, mla::kSchedMaxBatch);
  if (s_q < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "s_q %d < 1", s_q);
  if (h_q < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "h_q %d < 1", h_q);
  if (h_kv < 1 || h_kv > MLA_MAX_KV_HEADS || h_q % h_kv != 0)
    return fail(MLA_ERR_UNSUPPORTED, "h_kv %d: must divide h_q and be in [1, %d]", h_kv, MLA_MAX_KV_HEADS);
  if (h_q % 16 != 0 || h_q > 128) return fail(MLA_ERR_UNSUPPORTED, "h_q %d: must be a multiple of 16 and <= 128", h_q);
  if ((int64_t)s_q * h_q > MLA_MAX_ROWS) return fail(MLA_ERR_UNSUPPORTED, "s_q * h_q = %d above %d", s_q * h_q, MLA_MAX_ROWS);
  if (kv_format != MLA_KV_BF16_PAGED && kv_format != MLA_KV_FP8_PACKED && kv_format != MLA_KV_FP8_INDEXED &&
      kv_format != MLA_KV_FP16_PAGED)
    return fail(MLA_ERR_UNSUPPORTED, "kv_format %d unknown", kv_format);
  if (kv_format == MLA_KV_FP8_PACKED || kv_format == MLA_KV_FP8_INDEXED) {
    if (h_kv != 1) return fail(MLA_ERR_UNSUPPORTED, "sparse FP8 decode has one KV head (got h_kv %d)", h_kv);
    if (h_q != 64 && h_q != 128) return fail(MLA_ERR_UNSUPPORTED, "sparse FP8 decode supports h_q in {64, 128} (got %d)", h_q);
  }
  return MLA_OK;
}

int slots_for(int batch, int num_parts) { return batch + num_parts; }

// Argument checks of the decode entry points (everything but the workspace).
int check_decode_args(const void* q, const void* kv, int kv_format, int64_t num_pages, const int32_t* block_table,
                      int max_pages, const int32_t* seqlens, int topk_capacity, int batch, int s_q, int h_q, int h_kv,
                      float softmax_scale, const int32_t* sched_meta, const int32_t* num_splits, int num_parts,
                      const void* out, const float* lse, int causal) {
  if (!q || !kv || !seqlens || !sched_meta || !num_splits || !out || !lse)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  int st = check_shape(batch, s_q, h_q, h_kv, kv_format);
  if (st) return st;
  const bool fp8 = kv_format == MLA_KV_FP8_PACKED || kv_format == MLA_KV_FP8_INDEXED;
  if (fp8) {
    if (topk_capacity < mla::kPage || topk_capacity % mla::kPage != 0)
      return fail(MLA_ERR_UNSUPPORTED, "topk_capacity %d must be a positive multiple of 64", topk_capacity);
    if (causal) return fail(MLA_ERR_UNSUPPORTED, "sparse FP8 decode has no causal mask");
    if (kv_format == MLA_KV_FP8_INDEXED) {
      if (!block_table) return fail(MLA_ERR_INVALID_ARGUMENT, "indices (block_table argument) is NULL");
      if (num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages %lld < 1", (long long)num_pages);
      if (num_pages > INT64_MAX / (mla::kPage * mla::kRecBytes)) return fail(MLA_ERR_UNSUPPORTED, "num_pages too large");
    }
  } else {
    if (!block_table) return fail(MLA_ERR_INVALID_ARGUMENT, "block_table is NULL");
    if (max_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "max_pages %d < 1", max_pages);
    if (num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages %lld < 1", (long long)num_pages);
    if ((int64_t)batch * max_pages > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "batch * max_pages above 2^31");
    if ((int64_t)max_pages * mla::kPage > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "max_pages too large");
  }
  if (num_parts < 1 || num_parts > MLA_MAX_PARTS)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts %d out of [1, %d]", num_parts, MLA_MAX_PARTS);
  if (!(softmax_scale > 0.f) || !(softmax_scale < INFINITY))
    return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0 (got %g)", (double)softmax_scale);
  return MLA_OK;
}

// Decode launch on validated arguments; `workspace` holds the split partials
// (at least mla_decode_workspace_size bytes).
int launch_decode_checked(const void* q, const void* kv, int kv_format, int64_t num_pages, const int32_t* block_table,
                          int max_pages, const int32_t* seqlens, int topk_capacity, int batch, int s_q, int h_q,
                          int h_kv, float softmax_scale, int causal, const int32_t* sched_meta,
                          const int32_t* num_splits, int num_parts, void* out, float* lse, void* workspace,
                          hipStream_t stream) {
  mla::DecodeArgs a;
  a.q = (const uint16_t*)q;
  a.kv = (const uint8_t*)kv;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.seqlens = seqlens;
  a.cap = topk_capacity;
  a.batch = batch;
  a.s_q = s_q;
  a.h_q = h_q;
  a.M = s_q * h_q;
  a.h_kv = h_kv;
  a.G = h_q / h_kv;
  a.Mkv = s_q * a.G;
  a.scale_log2 = softmax_scale * 1.44269504088896340736f;
  a.causal = causal ? 1 : 0;
  a.sched_meta = sched_meta;
  a.num_splits = num_splits;
  a.num_parts = num_parts;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.slots = slots_for(batch, num_parts);
  a.part_o = (float*)workspace;
  a.part_lse = a.part_o + (size_t)a.slots * a.M * mla::kDV;
  const int kind = kv_format == MLA_KV_FP8_PACKED    ? mla::kDecodeFp8Packed
                   : kv_format == MLA_KV_FP8_INDEXED ? mla::kDecodeFp8Indexed
                   : kv_format == MLA_KV_FP16_PAGED  ? mla::kDecodeF16
                                                     : mla::kDecodeBf16;
  hipError_t e = mla::launch_decode(a, kind, stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (log_on()) {
    mla::DecodeLaunchInfo info;
    if (mla::decode_launch_info(a, kind, &info) == hipSuccess)
      fprintf(stderr,
              "[mla] decode %s grid=%dx%d block=%d num_parts=%d wgs_per_cu=%d lds=%d vgprs=%d batch=%d s_q=%d "
              "h_q=%d h_kv=%d\n",
              info.name, info.grid_x, info.grid_y, info.block, num_parts, info.wgs_per_cu, info.lds_bytes, info.vgprs,
              batch, s_q, h_q, h_kv);
  }
  return ok();
}

// Combine launch on validated arguments.
int launch_combine_checked(const int32_t* num_splits, const void* workspace, int batch, int s_q, int h_q,
                           int num_parts, int kv_format, void* out, float* lse, hipStream_t stream) {
  const int M = s_q * h_q;
  const float* part_o = (const float*)workspace;
  const float* part_lse = part_o + (size_t)slots_for(batch, num_parts) * M * mla::kDV;
  hipError_t e = mla::launch_combine(num_splits, part_o, part_lse, batch, M, slots_for(batch, num_parts),
                                     kv_format == MLA_KV_FP16_PAGED, (uint16_t*)out, lse, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  if (log_on())
    fprintf(stderr, "[mla] combine batch=%d rows=%d slots=%d num_parts=%d\n", batch, M, slots_for(batch, num_parts),
            num_parts);
  return ok();
}

}  // namespace

extern "C" {

const char* mla_last_error_message(void) { return g_last_error.c_str(); }

int mla_plan_num_parts(int batch, int s_q, int h_q, int h_kv, int kv_format, int cus, int wgs_per_cu,
                       int* num_parts_out) {
  if (!num_parts_out) return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts_out is NULL");
  int st = check_shape(batch, s_q, h_q, h_kv, kv_format);
  if (st) return st;
  if (cus < 1 || wgs_per_cu < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "cus %d / wgs_per_cu %d must be >= 1", cus, wgs_per_cu);
  const int Mkv = s_q * (h_q / h_kv);  // rows per (request, KV head)
  const int kind = kv_format == MLA_KV_FP8_PACKED    ? mla::kDecodeFp8Packed
                   : kv_format == MLA_KV_FP8_INDEXED ? mla::kDecodeFp8Indexed
                   : kv_format == MLA_KV_FP16_PAGED  ? mla::kDecodeF16
                                                     : mla::kDecodeBf16;
  const int rb = mla::decode_rows_per_wg(s_q * h_q, h_kv, kind);
  const int row_blocks = h_kv * ((Mkv + rb - 1) / rb);
  int64_t slots = (int64_t)cus * wgs_per_cu;
  int64_t parts = slots / row_blocks;
  if (parts < 1) parts = 1;
  const bool fp8 = kv_format == MLA_KV_FP8_PACKED || kv_format == MLA_KV_FP8_INDEXED;
  const int64_t cap = (int64_t)batch * (fp8 ? kMaxSplitsPerRequestFp8 : kMaxSplitsPerRequest);
  if (parts > cap) parts = cap;
  if (parts > MLA_MAX_PARTS) parts = MLA_MAX_PARTS;
  *num_parts_out = (int)parts;
  return ok();
}

int mla_decode_num_parts(int batch, int s_q, int h_q, int h_kv, int kv_format, int* num_parts_out) {
  if (!num_parts_out) return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts_out is NULL");
  int st = check_shape(batch, s_q, h_q, h_kv, kv_format);
  if (st) return st;
  st = check_device();
  if (st) return st;
  int dev = 0, cus = 0, wgs = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  e = mla::decode_occupancy(kv_format, s_q * (h_q / h_kv), &wgs);
  if (e != hipSuccess) return hip_fail(e, "occupancy query");
  if (wgs < 1) return fail(MLA_ERR_HIP, "decode kernel does not fit on a CU");
  return mla_plan_num_parts(batch, s_q, h_q, h_kv, kv_format, cus, wgs, num_parts_out);
}

const char* mla_decode_kernel_name(int s_q, int h_q, int h_kv, int kv_format) {
  if (check_shape(1, s_q, h_q, h_kv, kv_format)) return nullptr;
  const int kind = kv_format == MLA_KV_FP8_PACKED    ? mla::kDecodeFp8Packed
                   : kv_format == MLA_KV_FP8_INDEXED ? mla::kDecodeFp8Indexed
                   : kv_format == MLA_KV_FP16_PAGED  ? mla::kDecodeF16
                                                     : mla::kDecodeBf16;
  ok();
  return mla::decode_kernel_name(s_q * h_q, h_kv, kind);
}

size_t mla_decode_workspace_size(int batch, int s_q, int h_q, int num_parts) {
  if (batch < 1 || s_q < 1 || h_q < 1 || num_parts < 1 || num_parts > MLA_MAX_PARTS || batch > MLA_MAX_BATCH) return 0;
  const size_t M = (size_t)s_q * h_q;
  return (size_t)slots_for(batch, num_parts) * M * (mla::kDV + 1) * sizeof(float);
}

size_t mla_packed_kv_workspace_size(int batch, int s_q, int topk_capacity) {
  if (batch < 1 || s_q < 1 || topk_capacity < 1 || topk_capacity % mla::kPage != 0) return 0;
  return (size_t)batch * s_q * topk_capacity * mla::kRecBytes;
}

int mla_get_decode_metadata(const int32_t* seqlens, int batch, int s_q, int h_q, int h_kv, int num_parts,
                            int32_t* sched_meta, int32_t* num_splits, void* stream) {
  if (!seqlens || !sched_meta || !num_splits) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (num_parts < 1 || num_parts > MLA_MAX_PARTS)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts %d out of [1, %d]", num_parts, MLA_MAX_PARTS);
  int st = check_shape(batch, s_q, h_q, h_kv, MLA_KV_BF16_PAGED);
  if (st) return st;
  st = check_device();
  if (st) return st;
  hipError_t e =
      mla::launch_sched(seqlens, batch, num_parts, sched_meta, num_splits, (hipStream_t)stream, false, true);
  if (e != hipSuccess) return hip_fail(e, "scheduler launch");
  if (log_on()) fprintf(stderr, "[mla] metadata global batch=%d num_parts=%d\n", batch, num_parts);
  return ok();
}

int mla_get_packed_decode_metadata(const int32_t* topk_length, int batch, int s_q, int h_q, int topk_capacity,
                                   int num_parts, int policy, int32_t* sched_meta, int32_t* num_splits,
                                   void* stream) {
  if (!topk_length || !sched_meta || !num_splits) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (num_parts < 1 || num_parts > MLA_MAX_PARTS)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts %d out of [1, %d]", num_parts, MLA_MAX_PARTS);
  if (policy != MLA_SCHED_AUTO && policy != MLA_SCHED_GLOBAL && policy != MLA_SCHED_REQUEST_LOCAL)
    return fail(MLA_ERR_INVALID_ARGUMENT, "policy %d unknown", policy);
  int st = check_shape(batch, s_q, h_q, 1, MLA_KV_FP8_PACKED);
  if (st) return st;
  if (topk_capacity < mla::kPage || topk_capacity % mla::kPage != 0)
    return fail(MLA_ERR_UNSUPPORTED, "topk_capacity %d must be a positive multiple of 64", topk_capacity);
  st = check_device();
  if (st) return st;
  // AUTO is the global partition.  The page selects its request-local
  // scheduler for H = 64 outside one fallback regime on its GPU; here (HIP-graph
  // step, metadata + packed decode + combine, h_q 64 and 128, batch * s_q
  // 1..32, full and uneven top-k 2048) the global partition measured 4-16 %
  // faster at every shape: with equal lengths both give the same partition, and
  // the request-local search costs the one-workgroup scheduler several us.
  const bool local = policy == MLA_SCHED_REQUEST_LOCAL;
  hipError_t e = mla::launch_sched(topk_length, batch, num_parts, sched_meta, num_splits, (hipStream_t)stream, local);
  if (e != hipSuccess) return hip_fail(e, "scheduler launch");
  if (log_on())
    fprintf(stderr, "[mla] metadata %s batch=%d num_parts=%d\n", local ? "request-local" : "global", batch, num_parts);
  return ok();
}

int mla_decode_fwd(const void* q, const void* kv, int kv_format, int64_t num_pages, const int32_t* block_table,
                   int max_pages, const int32_t* seqlens, int topk_capacity, int batch, int s_q, int h_q, int h_kv,
                   float softmax_scale, int causal, const int32_t* sched_meta, const int32_t* num_splits,
                   int num_parts, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_decode_args(q, kv, kv_format, num_pages, block_table, max_pages, seqlens, topk_capacity, batch, s_q,
                             h_q, h_kv, softmax_scale, sched_meta, num_splits, num_parts, out, lse, causal);
  if (st) return st;
  const size_t need = mla_decode_workspace_size(batch, s_q, h_q, num_parts);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "decode workspace %zu B < %zu B", workspace_bytes, need);
  st = check_device();
  if (st) return st;
  return launch_decode_checked(q, kv, kv_format, num_pages, block_table, max_pages, seqlens, topk_capacity, batch,
                               s_q, h_q, h_kv, softmax_scale, causal, sched_meta, num_splits, num_parts, out, lse,
                               workspace, (hipStream_t)stream);
}

int mla_combine(const int32_t* num_splits, const void* workspace, size_t workspace_bytes, int batch, int s_q,
                int h_q, int num_parts, int kv_format, void* out, float* lse, void* stream) {
  if (!num_splits || !workspace || !out || !lse) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  int st = check_shape(batch, s_q, h_q, 1, kv_format);
  if (st) return st;
  if (num_parts < 1 || num_parts > MLA_MAX_PARTS)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts %d out of [1, %d]", num_parts, MLA_MAX_PARTS);
  const size_t need = mla_decode_workspace_size(batch, s_q, h_q, num_parts);
  if (workspace_bytes < need) return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "decode workspace %zu B < %zu B", workspace_bytes, need);
  st = check_device();
  if (st) return st;
  return launch_combine_checked(num_splits, workspace, batch, s_q, h_q, num_parts, kv_format, out, lse,
                                (hipStream_t)stream);
}

int mla_decode_fwd_noalloc(const void* q, const void* kv, int kv_format, int64_t num_pages,
                           const int32_t* block_table, int max_pages, const int32_t* seqlens, int topk_capacity,
                           int batch, int s_q, int h_q, int h_kv, float softmax_scale, int causal,
                           const int32_t* sched_meta, const int32_t* num_splits, int num_parts, void* out, float* lse,
                           void* stream) {
  int st = check_decode_args(q, kv, kv_format, num_pages, block_table, max_pages, seqlens, topk_capacity, batch, s_q,
                             h_q, h_kv, softmax_scale, sched_meta, num_splits, num_parts, out, lse, causal);
  if (st) return st;
  const size_t need = mla_decode_workspace_size(batch, s_q, h_q, num_parts);
  if (need > mla::kNoAllocScratchBytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "split partials need %zu B, above the %zu B of library scratch (fewer parts, or a smaller batch)",
                need, mla::kNoAllocScratchBytes);
  st = check_device();
  if (st) return st;
  void* ws = nullptr;
  hipError_t e = mla::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "library scratch lookup");
  st = launch_decode_checked(q, kv, kv_format, num_pages, block_table, max_pages, seqlens, topk_capacity, batch, s_q,
                             h_q, h_kv, softmax_scale, causal, sched_meta, num_splits, num_parts, out, lse, ws,
                             (hipStream_t)stream);
  if (st) return st;
  return launch_combine_checked(num_splits, ws, batch, s_q, h_q, num_parts, kv_format, out, lse,
                                (hipStream_t)stream);
}

int mla_pack_selected_kv(const void* kcache_fp8, int64_t num_pages, const int32_t* indices,
                         const int32_t* topk_length, int batch, int s_q, int topk_capacity, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!kcache_fp8 || !indices || !topk_length || !workspace) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (batch < 1 || batch > MLA_MAX_BATCH) return fail(MLA_ERR_INVALID_ARGUMENT, "batch %d out of [1, %d]", batch, MLA_MAX_BATCH);
  if (s_q < 1 || s_q > MLA_MAX_ROWS) return fail(MLA_ERR_INVALID_ARGUMENT, "s_q %d out of range", s_q);
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages %lld < 1", (long long)num_pages);
  if (topk_capacity < mla::kPage || topk_capacity % mla::kPage != 0)
    return fail(MLA_ERR_UNSUPPORTED, "topk_capacity %d must be a positive multiple of 64", topk_capacity);
  if ((int64_t)batch * s_q > 65535 || topk_capacity / mla::kPage > 65535)
    return fail(MLA_ERR_UNSUPPORTED, "grid too large");
  const size_t need = mla_packed_kv_workspace_size(batch, s_q, topk_capacity);
  if (workspace_bytes < need) return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "packed workspace %zu B < %zu B", workspace_bytes, need);
  int st = check_device();
  if (st) return st;
  hipError_t e = mla::launch_pack((const uint8_t*)kcache_fp8, num_pages, indices, topk_length, batch, s_q,
                                  topk_capacity, (uint8_t*)workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  if (log_on()) fprintf(stderr, "[mla] pack rows=%d topk_capacity=%d\n", batch * s_q, topk_capacity);
  return ok();
}

int mla_patch_packed_kv(const void* kcache_fp8, int64_t num_pages, const int32_t* indices,
                        const int32_t* topk_length, int batch, int s_q, int topk_capacity, const int32_t* new_ids,
                        int n_new, void* workspace, size_t workspace_bytes, void* stream) {
  if (!kcache_fp8 || !indices || !topk_length || !new_ids || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (batch < 1 || batch > MLA_MAX_BATCH) return fail(MLA_ERR_INVALID_ARGUMENT, "batch %d out of [1, %d]", batch, MLA_MAX_BATCH);
  if (s_q < 1 || s_q > MLA_MAX_ROWS) return fail(MLA_ERR_INVALID_ARGUMENT, "s_q %d out of range", s_q);
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages %lld < 1", (long long)num_pages);
  if (num_pages > INT32_MAX / mla::kPage) return fail(MLA_ERR_UNSUPPORTED, "num_pages too large for int32 token ids");
  if (n_new < 1 || n_new > mla::kPatchMaxNewIds)
    return fail(MLA_ERR_INVALID_ARGUMENT, "n_new %d out of [1, %d]", n_new, mla::kPatchMaxNewIds);
  if (topk_capacity < mla::kPage || topk_capacity % mla::kPage != 0)
    return fail(MLA_ERR_UNSUPPORTED, "topk_capacity %d must be a positive multiple of 64", topk_capacity);
  if ((int64_t)batch * s_q > 65535 || topk_capacity / mla::kPage > 65535)
    return fail(MLA_ERR_UNSUPPORTED, "grid too large");
  const size_t need = mla_packed_kv_workspace_size(batch, s_q, topk_capacity);
  if (workspace_bytes < need) return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "packed workspace %zu B < %zu B", workspace_bytes, need);
  int st = check_device();
  if (st) return st;
  hipError_t e = mla::launch_patch((const uint8_t*)kcache_fp8, num_pages, indices, topk_length, new_ids, n_new, batch,
                                   s_q, topk_capacity, (uint8_t*)workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "patch launch");
  if (log_on()) fprintf(stderr, "[mla] patch rows=%d topk_capacity=%d n_new=%d\n", batch * s_q, topk_capacity, n_new);
  return ok();
}

int mla_sparse_kv_format(int batch, int s_q, int topk_capacity, size_t workspace_budget_bytes, int pack_hidden,
                         int* kv_format_out) {
  if (!kv_format_out) return fail(MLA_ERR_INVALID_ARGUMENT, "kv_format_out is NULL");
  if (batch < 1 || batch > MLA_MAX_BATCH) return fail(MLA_ERR_INVALID_ARGUMENT, "batch %d out of [1, %d]", batch, MLA_MAX_BATCH);
  if (s_q < 1 || s_q > MLA_MAX_ROWS) return fail(MLA_ERR_INVALID_ARGUMENT, "s_q %d out of range", s_q);
  if (topk_capacity < mla::kPage || topk_capacity % mla::kPage != 0)
    return fail(MLA_ERR_UNSUPPORTED, "topk_capacity %d must be a positive multiple of 64", topk_capacity);
  const size_t need = mla_packed_kv_workspace_size(batch, s_q, topk_capacity);
  *kv_format_out = (pack_hidden && need <= workspace_budget_bytes) ? MLA_KV_FP8_PACKED : MLA_KV_FP8_INDEXED;
  return ok();
}

int mla_read_device_errors(int* flags_out, void* stream) {
  if (!flags_out) return fail(MLA_ERR_INVALID_ARGUMENT, "flags_out is NULL");
  int st = check_device();
  if (st) return st;
  hipError_t e = mla::read_and_clear_error_flags(flags_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reading device flags");
  return ok();
}

}  // extern "C"
