// Internal interface between the C ABI (mla_api.cpp) and the HIP kernels
// (mla_kernels.hip).  Not installed; callers use include/mla_paged_kv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kPage = 64;
constexpr int kRecBytes = 656;
constexpr int kMaxRowsPerWG = 64;   // query rows (token, head) one decode workgroup covers
constexpr int kSchedMaxBatch = 8192;

// Device-side violation flags (see mla_read_device_errors).
constexpr int kErrPage = 1;
constexpr int kErrIndex = 2;
constexpr int kErrSeqlen = 4;
constexpr int kErrMeta = 8;

struct DecodeArgs {
  const uint16_t* q;          // bf16 (fp16 for kDecodeF16) bits [batch][s_q][h_q][576]
  const uint8_t* kv;          // 16-bit pages [pages][64][h_kv][576], packed FP8 records, or the FP8 record pool
  int64_t num_pages;
  const int32_t* block_table; // [batch][max_pages]; FP8 indexed: top-k token ids [batch][s_q][cap]
  int max_pages;
  const int32_t* seqlens;     // [batch] (packed: topk_length)
  int cap;                    // packed: top-k capacity (multiple of 64)
  int batch, s_q, h_q, M;     // M = s_q * h_q rows per request
  int h_kv, G, Mkv;           // KV heads, query heads per KV head (h_q / h_kv), s_q * G
  float scale_log2;           // softmax_scale * log2(e)
  int causal;
  const int32_t* sched_meta;  // [num_parts][8]
  const int32_t* num_splits;  // [batch + 1]
  int num_parts;
  uint16_t* out;              // bf16 (fp16 for kDecodeF16) bits [batch][M][512]
  float* lse;                 // [batch][M]
  float* part_o;              // [slots][M][512]
  float* part_lse;            // [slots][M]
  int slots;
};

// Rows per workgroup of the 64-row kernel family for M rows per request:
// 16 * RB with RB in {1, 2, 4}.
int decode_row_blocks_per_wg(int M);

// Query rows one decode workgroup covers for this shape.
int decode_rows_per_wg(int M, int h_kv, int kind);
const char* decode_kernel_name(int M, int h_kv, int kind);

// What launch_decode would launch for these arguments (for MLA_LOG).
struct DecodeLaunchInfo {
  const char* name;
  int grid_x, grid_y, block, lds_bytes, vgprs, wgs_per_cu;
};
hipError_t decode_launch_info(const struct DecodeArgs& a, int kind, DecodeLaunchInfo* info);

// Split limit of the dense scheduler: with T blocks over `batch` requests it
// uses at most L = max(16 batch, min(ceil(T / 4), 64 batch)) partitions (see
// mla_get_decode_metadata).
constexpr int kSplitFloorPerRequest = 16;
constexpr int kBlocksPerSplit = 4;
constexpr int kSplitCeilPerRequest = 64;
hipError_t launch_sched(const int32_t* lengths, int batch, int num_parts, int32_t* meta, int32_t* num_splits,
                        hipStream_t stream, bool request_local = false, bool split_limit = false);
// Decode kernel family: bf16 pages, FP8 packed workspace, FP8 pool gathered by
// index, fp16 pages.
enum DecodeKind { kDecodeBf16 = 0, kDecodeFp8Packed = 1, kDecodeFp8Indexed = 2, kDecodeF16 = 3 };
hipError_t launch_decode(const DecodeArgs& a, int kind, hipStream_t stream);
hipError_t launch_combine(const int32_t* num_splits, const float* part_o, const float* part_lse, int batch, int M,
                          int slots, bool out_f16, uint16_t* out, float* lse, hipStream_t stream);
hipError_t launch_pack(const uint8_t* kcache, int64_t num_pages, const int32_t* indices, const int32_t* topk_length,
                       int batch, int s_q, int cap, uint8_t* ws, hipStream_t stream);
hipError_t launch_patch(const uint8_t* kcache, int64_t num_pages, const int32_t* indices, const int32_t* topk_length,
                        const int32_t* new_ids, int n_new, int batch, int s_q, int cap, uint8_t* ws,
                        hipStream_t stream);
constexpr int kPatchMaxNewIds = 64;
hipError_t decode_occupancy(int kind, int M, int* wgs_per_cu);
hipError_t read_and_clear_error_flags(int* flags, hipStream_t stream);

// Device scratch of the entry point that allocates nothing (split partials):
// a file-scope __device__ array of this many bytes per device.  *ptr receives
// the current device's address of it (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace mla
