// HIP kernels for MLA decode over a paged KV cache on MI355X (gfx950, CDNA4).
//
// Method (FlashMLA PR 183 "Add SM80 (Ampere/A100) dense MLA decode kernel",
// Summary/Design; FlashMLA PR 200 "[SM90] Add packed selected-KV sparse
// decode", "SM90 packing kernel" / "Packed attention specialization"):
// softmax(scale * Q K^T) V for s_q*h_q query rows that share one 576-dim latent
// KV head, V = K[:, 0:512], keys in 64-token pages reached through a block
// table, the sequence split over workgroups with an online softmax, and the
// splits merged by a log-sum-exp combine.
//
// gfx950 design (not the pages' SM80/SM90 tiling):
//   * One workgroup = 8 waves, two per SIMD with different jobs, covering up
//     to 64 query rows of one partition: four QK waves (16 rows each, Q in
//     registers) compute scores and the online softmax, four PV waves own 128
//     output columns each for all rows.  Every 32-key tile is fetched once per
//     workgroup and serves all its rows.
//   * Tiles stream HBM -> LDS with global_load_lds (16 B per lane, no VGPR
//     staging) through a 4-slot ring; bf16 key rows are stored with their 16-B
//     chunks XOR-swizzled by (row & 7), which keeps the 16-rows-per-read MFMA
//     operand fetches free of bank conflicts despite the 1152-B row pitch.
//   * QK^T as S^T = K Q^T with v_mfma_f32_16x16x32 (K the A operand from LDS);
//     PV as O^T = V^T P^T with V^T from transposed LDS reads and P^T (bf16)
//     shared through LDS, so each score row is computed once.
//   * Online softmax in the exp2 domain with lazy rescaling: the running max
//     moves (and O is rescaled) only when a tile's max exceeds it by more than
//     kRescaleThreshold (log2 units); final out = O / l is exact either way.
//   * The FP8 paths stream the raw 656-byte records into a ring of their own;
//     the PV waves convert each tile's E4M3 bytes to bf16 (exact) into a tile
//     in the dense layout one iteration before it is used, and each key's fp32
//     block scales multiply the per-block score sums and P.
//   * A launch's parts are mapped so that each XCD runs a contiguous range of
//     them (the pieces of a request share an L2).
#include "mla_internal.h"

#include <mutex>
#include <type_traits>

#include <math.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

__device__ int g_error_flags;

// Read-only kernel inputs that every lane of a wave indexes the same way (page
// table, lengths, scheduler records) are read through the constant address
// space so that they become scalar loads: a vector load here would need a
// vmcnt wait, and vmcnt retires in order, i.e. it would also wait for every
// tile still in flight in the global->LDS ring.
template <class T>
using const_ptr = const __attribute__((address_space(4))) T*;
template <class T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
  return ((const_ptr<T>)(p))[i];
}

// ------------------------------------------------------------------ decode geometry
constexpr int kTK = 32;                             // keys per tile
constexpr int kStages = 4;                          // HBM -> LDS ring depth
constexpr int kRowBytes = kDQK * 2;                 // 1152
constexpr int kTileBytes = kTK * kRowBytes;         // 36864
constexpr int kChunksPerRow = kRowBytes / 16;       // 72
constexpr int kLoadsPerWave = kTileBytes / 1024 / 4;  // 9 wave-wide 16-B loads per tile per wave
// P row pitch (bytes) of the bf16 kernel, from SQ_LDS_BANK_CONFLICT on gfx950
// probes of its exact access patterns: the 16-B reads of 16 rows (+16 B per
// lane group) are conflict-free at a 96-B pitch (2-way at 80), the 8-B writes
// 4-way (2-way at 80); P is read as often as it is written, so both cost the
// same, and the reads are the ones on the PV waves' critical path.
constexpr int kPStride = 96;
constexpr int kRawTileBytes = kTK * kRecBytes;      // FP8 raw tile slot: 32 records, 20992 B
constexpr int kRawChunks = kTK * kRecBytes / 16;    // 1312 16-B chunks = 20.5 wave-wide loads
constexpr float kRescaleThreshold = 8.0f;           // log2 units: p <= 2^8 between rescales

// LDS layout
constexpr int kPBufBytes = kMaxRowsPerWG * kPStride;            // one P buffer (6 KB)
constexpr int kOffKDense = 0;
constexpr int kOffRaw = 2 * kTileBytes;                        // FP8: raw ring, after two bf16 tiles

// ------------------------------------------------------------------ small device helpers
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Barrier that also makes this wave's LDS writes visible.  No vmcnt wait: the
// global->LDS ring is waited for explicitly with wait_vmcnt.
__device__ __forceinline__ void sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// global_load_lds_dwordx4: lane i writes its 16 source bytes to LDS at M0 + 16*i.
// Issued through inline asm on purpose: the compiler then knows of no pending
// LDS DMA, so it inserts no vmcnt(0) in front of later LDS reads (it cannot
// tell they touch other ring slots).  The ring's completion is tracked with the
// explicit wait_vmcnt calls instead.  M0 is a register the compiler reserves
// (it cannot be listed as clobbered), so the asm saves and restores it; the
// s_nop is the one wait state an SALU write of M0 needs before an LDS-DMA load.
__device__ __forceinline__ void load_lds16(const void* gsrc, LDS_AS void* ldst) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)ldst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(m0v)
      : "memory");
}

// Same, with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset
// (saddr form): no per-lane 64-bit address arithmetic.
// `bu` must be wave-uniform and already in SGPRs (see uniform_u64).  NT: the
// nontemporal cache policy (measured: faster where at most two workgroups read
// a tile, slower where four do -- the later readers then miss in L2 -- and on
// records gathered by index).
template <bool NT = false>
__device__ __forceinline__ void load_lds16_s(uint64_t bu, uint32_t voff, LDS_AS void* ldst) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)ldst);
  uint32_t saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(bu), "s"(m0v)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(bu), "s"(m0v)
        : "memory");
}

// A wave-uniform 64-bit value made visible as such (SGPRs).  The builtin returns
// a signed int: each half goes through uint32_t so that the low word is
// zero-extended, not sign-extended.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t b) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

__device__ __forceinline__ bf16x8 lds_read_b128(const LDS_AS uint8_t* p) {
  return *reinterpret_cast<const LDS_AS bf16x8*>(p);
}

// Transposed 4 x 16 read (ds_read_b64_tr_b16): in each 16-lane group, lanes
// 4r..4r+3 address the 16 consecutive bf16 of row r (4 each); lane i receives
// column i of rows 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const LDS_AS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<LDS_AS bf16x4*>(const_cast<LDS_AS uint8_t*>(p)));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


// A score row lives in lanes l, l^16, l^32, l^48.  v_permlane16_swap /
// v_permlane32_swap exchange half-rows between two registers; with both holding
// x, the pair that comes back is {x[l], x[l^16]} (resp. x[l^32]), so two VALU
// ops reduce a row without a trip through LDS.  Inline asm on purpose: with
// both operands equal, the compiler's builtin folds the returned pair to a single
// value (observed: the max of the pair disappeared).  The s_nop covers the
// VALU-write -> permlane-read hazard.
__device__ __forceinline__ void permlane_pair16(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane_pair32(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// One step of the row max: max(v[l], v[l ^ 16]) (resp. l ^ 32) in one asm block,
// so that the compiler adds no NaN-quieting ops around the permlane results.
__device__ __forceinline__ float rowmax16(float v) {
  float b = v;
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_max_f32 %0, %0, %1" : "+v"(v), "+v"(b));
  return v;
}
__device__ __forceinline__ float rowmax32(float v) {
  float b = v;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_max_f32 %0, %0, %1" : "+v"(v), "+v"(b));
  return v;
}
__device__ __forceinline__ float row4_sum(float v) {
  float a = v, b = v;
  permlane_pair16(a, b);
  v = a + b;
  a = v;
  b = v;
  permlane_pair32(a, b);
  return a + b;
}

// byte offset of (key row kr, 16-B chunk c) inside a swizzled bf16 tile
__device__ __forceinline__ uint32_t tile_off(int kr, int c) {
  return (uint32_t)(kr * kRowBytes + ((c ^ (kr & 7)) << 4));
}

// Scheduler part of workgroup column b of a decode grid with P columns.  The
// dispatcher hands workgroups to the 8 XCDs round-robin by linear id (x + P y),
// so with P a multiple of 8 column b runs on XCD b mod 8 for every row block
// y; mapping b to part (b mod 8) * P/8 + b/8 gives each XCD a contiguous range
// of parts, and the pieces of one request (consecutive parts), which read the
// same Q rows, share an L2.
__device__ __forceinline__ int xcd_part(int b, int P) { return (P & 7) ? b : (b & 7) * (P >> 3) + (b >> 3); }

// Lane id in [0, 64), computed where it is used: the asm is never hoisted, so
// values derived from it do not stay live (and spill) across the tile loops.
// Every lane of the wave must be active.
__device__ __forceinline__ int lane_id_here() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

// ------------------------------------------------------------------ scheduler
// One workgroup.  Implements the partition definition in mla_paged_kv.h: request r
// has ceil(len/64) blocks, T in all; with P' = min(P, T) (and, under the split
// limit, min(P', L) with L = max(16 b, min(ceil(T/4), 64 b)) for b requests),
// part p < P' owns global blocks [floor(pT/P'), floor((p+1)T/P')) and parts
// p >= P' own none, so the parts owning one request's blocks are consecutive.
constexpr int kSchedThreads = 256;

__device__ __forceinline__ int64_t part_of_block(int64_t g, int64_t T, int64_t P);

// floor(a / b) for 0 <= a < 2^53, 0 < b < 2^31: exact 32-bit unsigned division
// when a fits in 32 bits (every realistic plan), else a double estimate
// corrected to the exact quotient (64-bit integer division is a long software
// sequence, and the double path costs about 15 double-precision instructions).
__device__ __forceinline__ int64_t floordiv_exact(int64_t a, int64_t b) {
  if (a <= (int64_t)UINT32_MAX && b <= (int64_t)UINT32_MAX) return (int64_t)((uint32_t)a / (uint32_t)b);
  int64_t q = (int64_t)((double)a / (double)b);
  while (q * b > a) --q;
  while ((q + 1) * b <= a) ++q;
  return q;
}

__device__ __forceinline__ int64_t part_of_block(int64_t g, int64_t T, int64_t P) {
  return floordiv_exact((g + 1) * P - 1, T);
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// exclusive prefix of `local` over the workgroup's 256 threads; *total = sum
__device__ __forceinline__ int block_excl_scan(int local, int* total, int32_t* wsum) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int incl = wave_incl_scan(local);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int i = 0; i < kSchedThreads / 64; ++i) base += i < wv ? wsum[i] : 0;
  int tot = 0;
#pragma unroll
  for (int i = 0; i < kSchedThreads / 64; ++i) tot += wsum[i];
  *total = tot;
  __syncthreads();  // wsum is reused by the next scan
  return base + incl - local;
}

// workgroup-wide max of a non-negative int (every thread gets it)
__device__ __forceinline__ int block_max(int v, int32_t* wsum) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  if (lane == 0) wsum[wv] = v;
  __syncthreads();
  int m = 0;
#pragma unroll
  for (int i = 0; i < kSchedThreads / 64; ++i) m = max(m, wsum[i]);
  __syncthreads();  // wsum is reused
  return m;
}

// Request-local partition (no part spans two requests; see mla_paged_kv.h):
// B = the smallest piece size in blocks with sum_r ceil(b_r / B) <= num_parts,
// request r in ceil(b_r / B) balanced pieces, parts in (request, piece) order.
// Returns false, having written nothing, when more requests have a block than
// there are parts.  bl[r] = blocks of request r (LDS), filled by the caller.
__device__ bool request_local_partition(const int32_t* bl, int batch, int num_parts, int32_t* meta,
                                        int32_t* num_splits, int32_t* wsum) {
  const int t = threadIdx.x;
  const int C = (batch + kSchedThreads - 1) / kSchedThreads;
  int nonempty = 0, maxb = 0, tot_local = 0;
  for (int k = 0; k < C; ++k) {
    const int r = t * C + k;
    if (r < batch) {
      nonempty += bl[r] > 0;
      maxb = max(maxb, bl[r]);
      tot_local += bl[r];
    }
  }
  int N = 0, T = 0;
  block_excl_scan(nonempty, &N, wsum);
  block_excl_scan(tot_local, &T, wsum);
  maxb = block_max(maxb, wsum);
  if (N > num_parts) return false;
  int B = maxb;  // sum_r ceil(b_r / maxb) = N <= num_parts
  if (T > 0) {
    int lo = (T + num_parts - 1) / num_parts, hi = maxb;  // smallest B in [lo, hi] that fits
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      int cnt = 0;
      for (int k = 0; k < C; ++k) {
        const int r = t * C + k;
        if (r < batch) cnt += (bl[r] + mid - 1) / mid;
      }
      int total = 0;
      block_excl_scan(cnt, &total, wsum);
      if (total <= num_parts) hi = mid; else lo = mid + 1;
    }
    B = lo;
  }
  int pieces_local = 0;
  for (int k = 0; k < C; ++k) {
    const int r = t * C + k;
    if (r < batch && T > 0) pieces_local += (bl[r] + B - 1) / B;
  }
  int used = 0;
  int off = block_excl_scan(pieces_local, &used, wsum);
  for (int k = 0; k < C; ++k) {
    const int r = t * C + k;
    if (r >= batch) break;
    num_splits[r] = off;
    const int b = bl[r];
    const int n = T > 0 ? (b + B - 1) / B : 0;
    for (int i = 0; i < n; ++i) {
      int32_t* m = meta + (int64_t)(off + i) * 8;
      m[0] = r;
      m[1] = (int32_t)(((int64_t)i * b) / n);
      m[2] = r;
      m[3] = (int32_t)(((int64_t)(i + 1) * b) / n);
      m[4] = i;
      m[5] = m[6] = m[7] = 0;
    }
    off += n;
  }
  if (t == 0) num_splits[batch] = used;
  for (int p = used + t; p < num_parts; p += kSchedThreads) {
    int32_t* m = meta + (int64_t)p * 8;
    m[0] = m[1] = m[2] = m[3] = m[4] = -1;
    m[5] = m[6] = m[7] = 0;
  }
  return true;
}

template <bool LOCAL>
__global__ __launch_bounds__(kSchedThreads) void sched_kernel(const int32_t* __restrict__ lengths, int batch,
                                                              int num_parts, int32_t* __restrict__ meta,
                                                              int32_t* __restrict__ num_splits, int split_limit) {
  __shared__ int32_t cum[kSchedMaxBatch + 1];
  __shared__ int32_t wsum[kSchedThreads / 64];
  const int t = threadIdx.x;
  const int C = (batch + kSchedThreads - 1) / kSchedThreads;  // <= 32 consecutive requests per thread

  if constexpr (LOCAL) {
    for (int k = 0; k < C; ++k) {
      const int r = t * C + k;
      if (r < batch) cum[r] = (max(lengths[r], 0) + kPage - 1) / kPage;  // blocks per request
    }
    __syncthreads();
    if (request_local_partition(cum, batch, num_parts, meta, num_splits, wsum)) return;
    __syncthreads();  // fall back to the global partition below (cum is rebuilt)
  }

  // 1. blocks per request, exclusive prefix -> cum
  int local = 0;
  for (int k = 0; k < C; ++k) {
    const int r = t * C + k;
    if (r < batch) local += (max(lengths[r], 0) + kPage - 1) / kPage;
  }
  int total = 0;
  int run = block_excl_scan(local, &total, wsum);
  for (int k = 0; k < C; ++k) {
    const int r = t * C + k;
    if (r < batch) {
      cum[r] = run;
      run += (max(lengths[r], 0) + kPage - 1) / kPage;
    }
  }
  if (t == 0) cum[batch] = total;
  __syncthreads();
  const int64_t T = total;
  int64_t P = T < num_parts ? T : num_parts;  // P' (0 when there is no block at all)
  if (split_limit) {
    const int64_t L = max((int64_t)kSplitFloorPerRequest * batch,
                          min((T + kBlocksPerSplit - 1) / kBlocksPerSplit, (int64_t)kSplitCeilPerRequest * batch));
    P = min(P, L);
  }

  // 2. partition records
  for (int p = t; p < num_parts; p += kSchedThreads) {
    int32_t* m = meta + (int64_t)p * 8;
    const int64_t G0 = p < P ? floordiv_exact((int64_t)p * T, P) : T;
    const int64_t G1 = p < P ? floordiv_exact((int64_t)(p + 1) * T, P) : T;
    if (G1 <= G0) {
      m[0] = m[1] = m[2] = m[3] = m[4] = -1;
    } else {
      // first request whose block range ends after G0 (resp. after G1 - 1)
      int lo = 0, hi = batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (cum[mid + 1] > G0) hi = mid; else lo = mid + 1;
      }
      const int br = lo;
      lo = br;
      hi = batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (cum[mid + 1] >= G1) hi = mid; else lo = mid + 1;
      }
      const int er = lo;
      m[0] = br;
      m[1] = (int32_t)(G0 - cum[br]);
      m[2] = er;
      m[3] = (int32_t)(G1 - cum[er]);
      m[4] = (int32_t)(p - part_of_block(cum[br], T, P));
    }
    m[5] = m[6] = m[7] = 0;
  }

  // 3. split counts, exclusive prefix -> num_splits
  int splits_local = 0;
  for (int k = 0; k < C; ++k) {
    const int r = t * C + k;
    if (r < batch && cum[r + 1] > cum[r])
      splits_local += (int)(part_of_block(cum[r + 1] - 1, T, P) - part_of_block(cum[r], T, P) + 1);
  }
  int stotal = 0;
  run = block_excl_scan(splits_local, &stotal, wsum);
  for (int k = 0; k < C; ++k) {
    const int r = t * C + k;
    if (r < batch) {
      num_splits[r] = run;
      if (cum[r + 1] > cum[r]) run += (int)(part_of_block(cum[r + 1] - 1, T, P) - part_of_block(cum[r], T, P) + 1);
    }
  }
  if (t == 0) num_splits[batch] = stotal;
}

// ------------------------------------------------------------------ decode
template <bool FP8>
struct TileLoader;

// bf16 pages: tile = 32 consecutive keys of one 64-token page (36,864 contiguous bytes).
template <>
struct TileLoader<false> {
  // Load qi = w + 4k (k < 9) of a tile fills LDS chunks [64qi, 64qi+64); lane
  // l's chunk lies in key row kr = (64qi + l) / 72, and (72 being a multiple of
  // 8) its swizzled source offset in the tile is 1024qi + 16((l & 56) |
  // ((l ^ kr) & 7)).  The three lane-dependent bits of the nine loads share one
  // register; the 1024qi part goes into the wave-uniform base.
  uint32_t bits, l56;
  __device__ void init(int w, int l) {
    bits = 0;
    l56 = 16u * (uint32_t)(l & 56);
#pragma unroll
    for (int k = 0; k < kLoadsPerWave; ++k) {
      const int qi = w + 4 * k;
      const int kr = (qi * 64 + l) / kChunksPerRow;
      bits |= (uint32_t)((l ^ kr) & 7) << (3 * k);
    }
  }
  // Issues this wave's loads of tile `tile` of request r into stage `st`.
  __device__ void issue(const DecodeArgs& a, int r, int key0, LDS_AS uint8_t* smem, int st, int w) {
    issue_page(a, ld_const(a.block_table, (int64_t)r * a.max_pages + (key0 >> 6)), key0, smem, st, w);
  }
  // Same, with the page id already looked up (wave-uniform).
  __device__ void issue_page(const DecodeArgs& a, int64_t page, int key0, LDS_AS uint8_t* smem, int st, int w) {
    const uint64_t src = tile_src(a, page, key0);
#pragma unroll
    for (int k = 0; k < kLoadsPerWave; ++k) issue_one(src, smem, st, w, k);
  }
  // Wave-uniform base address of tile (page, key0) for issue_one, in SGPRs.
  // The page id is made wave-uniform first, so that the bounds check (one
  // unsigned 32-bit compare: a negative id wraps above any pool size) and the
  // address arithmetic run on the scalar unit.
  __device__ uint64_t tile_src(const DecodeArgs& a, int64_t page, int key0) const {
    uint32_t pg = (uint32_t)__builtin_amdgcn_readfirstlane((int)page);
    const uint32_t np = a.num_pages < (int64_t)INT32_MAX ? (uint32_t)a.num_pages : (uint32_t)INT32_MAX;
    if (pg >= np) {
      if ((threadIdx.x & 63) == 0) atomicOr(&g_error_flags, kErrPage);
      pg = 0;  // stay in bounds; the output of this request is undefined
    }
    const uint64_t off = (uint64_t)pg * (uint32_t)(kPage * kRowBytes) + (uint32_t)((key0 & 63) * kRowBytes);
    return uniform_u64((uint64_t)(uintptr_t)a.kv + off);
  }
  // The k-th of this wave's kLoadsPerWave loads of a tile.
  __device__ void issue_one(uint64_t src, LDS_AS uint8_t* smem, int st, int w, int k) const {
    const int qi = w + 4 * k;
    const uint32_t voff = l56 + 16u * ((bits >> (3 * k)) & 7u);
    load_lds16_s(src + (uint64_t)(qi * 1024), voff, smem + kOffKDense + st * kTileBytes + qi * 1024);
  }

  // Several KV heads per token: the cache is [pages][64][h_kv][576], so the key
  // rows of one head are h_kv * 1152 bytes apart.  A lane's chunk of load k lies
  // in key row (64 qi + l) / 72 (kept 5 bits per load); its source offset is the
  // contiguous one plus row * (h_kv - 1) * 1152.
  uint64_t rowbits;
  __device__ void init_rows(int w, int l) {
    rowbits = 0;
#pragma unroll
    for (int k = 0; k < kLoadsPerWave; ++k) {
      const int qi = w + 4 * k;
      rowbits |= (uint64_t)((qi * 64 + l) / kChunksPerRow) << (5 * k);
    }
  }
  __device__ uint64_t tile_src_hkv(const DecodeArgs& a, int64_t page, int key0, int kvh) const {
    if (page < 0 || page >= a.num_pages) {
      if ((threadIdx.x & 63) == 0) atomicOr(&g_error_flags, kErrPage);
      page = 0;
    }
    const uint64_t token = (uint64_t)page * kPage + (uint64_t)(key0 & 63);
    const uint64_t off = (token * (uint64_t)a.h_kv + (uint64_t)kvh) * (uint64_t)kRowBytes;
    return uniform_u64((uint64_t)(uintptr_t)a.kv + off);
  }
  __device__ void issue_page_hkv(const DecodeArgs& a, int64_t page, int key0, int kvh, LDS_AS uint8_t* smem, int st,
                                 int w) const {
    const uint64_t src = tile_src_hkv(a, page, key0, kvh);
    const uint32_t xstride = (uint32_t)(a.h_kv - 1) * (uint32_t)kRowBytes;
#pragma unroll
    for (int k = 0; k < kLoadsPerWave; ++k) {
      const int qi = w + 4 * k;
      const uint32_t row = (uint32_t)(rowbits >> (5 * k)) & 31u;
      const uint32_t voff = l56 + 16u * ((bits >> (3 * k)) & 7u) + row * xstride;
      load_lds16_s(src + (uint64_t)(qi * 1024), voff, smem + kOffKDense + st * kTileBytes + qi * 1024);
    }
  }
};

// FP8 packed workspace: tile = 32 consecutive 656-byte records of one query row
// (1312 16-B chunks).  Wave w moves chunks [64 q, 64 q + 64) for q = w + 4 k,
// k < 5 (the first 1280), and wave 0 also the last 32 (q = 20, lanes 0..31):
// 6 loads for wave 0, 5 for the others (loads_in_flight).
template <>
struct TileLoader<true> {
  static constexpr int kLoads = 6;  // at most, per wave
  __device__ void init(int, int) {}
  __device__ static int loads_of_wave(int w) { return w == 0 ? 6 : 5; }
  __device__ void issue(const DecodeArgs& a, int r, int key0, LDS_AS uint8_t* smem, int st, int w) {
    const uint64_t src = uniform_u64((uint64_t)(uintptr_t)(a.kv + ((int64_t)r * a.cap + key0) * kRecBytes));
    LDS_AS uint8_t* dst = smem + kOffRaw + st * kRawTileBytes;
    const uint32_t l = threadIdx.x & 63;
    // nontemporal: measured 3-4 % faster on the packed workspace (at most two
    // workgroups read a tile there)
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int q = w + 4 * k;
      load_lds16_s<true>(src, (uint32_t)(q * 64 * 16) + 16u * l, dst + q * 1024);
    }
    if (w == 0 && l < (uint32_t)(kRawChunks - 20 * 64))
      load_lds16_s<true>(src, 20u * 64 * 16 + 16u * l, dst + 20 * 1024);
  }
};

// FP8 records gathered by index from the paged pool (no pack): record j of the
// tile of keys [key0, key0 + 32) is kcache_fp8[idx / 64][idx % 64] with
// idx = indices[row][key0 + j] (row = r * s_q + s for query token s of request
// r).  One wave-wide load per record (lanes 0..40 each move one 16-byte chunk
// of the 656 bytes; the others idle), so the record's base address is
// wave-uniform; wave w moves records w, w + 4, ..., w + 28 into the same raw
// tile layout the packed loader produces.  The ids of a request piece's first
// kIdxCache keys are staged in LDS when the piece starts: one LDS read then
// gives lane k the id of the wave's k-th record and the bases are formed on
// the scalar unit (an id read per record on the tile's critical path cost
// about 1.3 us per tile); later keys read their ids with scalar loads.  Keys
// past the request's top-k length `n` (set per request, already clamped to the
// capacity) load record 0 (they are masked); an index of the valid prefix
// outside the pool is flagged and replaced by 0.
constexpr int kIdxLoadsPerWave = kTK / 4;  // 8
constexpr int kIdxCache = 1024;            // top-k ids of a request piece staged in LDS
constexpr int kF8OffIdsLoader = 159040;    // = kF8OffIds (checked below)
struct IndexedLoader {
  static constexpr int kLoads = kIdxLoadsPerWave;
  int n = 0;
  int kc0 = 0, kc1 = 0;  // keys [kc0, kc1) of the current row have their ids staged in LDS
  __device__ void init(int, int) {}
  __device__ static int loads_of_wave(int) { return kIdxLoadsPerWave; }
  __device__ void issue(const DecodeArgs& a, int row, int key0, LDS_AS uint8_t* smem, int st, int w) const {
    const int l = threadIdx.x & 63;
    const int64_t limit = a.num_pages * kPage;
    LDS_AS uint8_t* dst = smem + kOffRaw + st * kRawTileBytes;
    if (key0 >= kc0 && key0 + kTK <= kc1) {
      // ids staged in LDS (one cold round trip per request piece, not per tile):
      // one read gives lane k the id of record w + 4k, and the record bases
      // are then formed on the scalar unit
      const LDS_AS int32_t* ids = reinterpret_cast<const LDS_AS int32_t*>(smem + kF8OffIdsLoader);
      int rec = w + 4 * (l & 7);
      asm volatile("" : "+v"(rec));  // the LDS address is formed here, not hoisted (and spilled)
      const int v = key0 + rec < n ? ids[key0 - kc0 + rec] : 0;
      bool bad = false;
#pragma unroll
      for (int k = 0; k < kIdxLoadsPerWave; ++k) {
        int64_t idx = __builtin_amdgcn_readlane(v, k);
        if (idx < 0 || idx >= limit) {
          bad = true;
          idx = 0;
        }
        const uint64_t base = uniform_u64((uint64_t)(uintptr_t)a.kv + (uint64_t)idx * kRecBytes);
        if (l < kRecBytes / 16) load_lds16_s(base, 16u * (uint32_t)l, dst + (w + 4 * k) * kRecBytes);
      }
      if (bad && l == 0) atomicOr(&g_error_flags, kErrIndex);
      return;
    }
    // keys past the staged range: one scalar id read per record
#pragma unroll
    for (int k = 0; k < kIdxLoadsPerWave; ++k) {
      const int j = w + 4 * k;
      int64_t idx = 0;
      if (key0 + j < n) {
        idx = ld_const(a.block_table, (int64_t)row * a.cap + key0 + j);
        if (idx < 0 || idx >= limit) {
          if (l == 0) atomicOr(&g_error_flags, kErrIndex);
          idx = 0;
        }
      }
      const uint64_t base = uniform_u64((uint64_t)(uintptr_t)a.kv + (uint64_t)idx * kRecBytes);
      if (l < kRecBytes / 16) load_lds16_s(base, 16u * (uint32_t)l, dst + j * kRecBytes);
    }
  }
};

// one v_cvt_pk_bf16_f32 (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// Element type of the dense path: bf16 or IEEE binary16 (fp16).  Tiles,
// fragments and transposed reads move 16-bit patterns either way; only the
// MFMA and the conversions of P and of the output differ.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <bool F16>
__device__ __forceinline__ f32x4 mfma16t(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// two floats -> two 16-bit values (round to nearest even), a in the low half
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
  else
    return pack_bf16x2(a, b);
}

// ------------------------------------------------------------------ dense decode: LDS layout
//
// A ring of kStages 32-key tiles (tile t in slot t & 3), double-buffered P
// (bf16, 64 rows x 32 keys, padded rows), per-row rescale factors and per-row-
// block flags, the row sums handed to the output stage, and the page ids of
// the request piece being processed.
constexpr int kLPW = kLoadsPerWave;
constexpr int kDOffP = kStages * kTileBytes;                  // 147456
constexpr int kDOffAlpha = kDOffP + 2 * kPBufBytes;           // 159744
constexpr int kDOffFlag = kDOffAlpha + 2 * kMaxRowsPerWG * 4; // 160256
constexpr int kDOffL = kDOffFlag + 64;                        // 160320
constexpr int kPageCache = 512;                               // page ids cached per request piece
constexpr int kDOffPages = kDOffL + kMaxRowsPerWG * 4;        // 160576
constexpr int kDLdsBytes = kDOffPages + kPageCache * 4;       // 162624
static_assert(kDLdsBytes <= 160 * 1024, "dense pipelined LDS budget");

// S^T (32 keys x 16 rows) = K Q^T over 576 dims: 18 k-steps x 2 key blocks.
// The K operands come from LDS through a ring of D fragments per key block, so
// the reads of k-step s+D-1 are in flight while the MFMAs of k-step s run.
struct NoHook {
  __device__ void operator()(int) const {}
};

template <int D, bool F16 = false, class Hook = NoHook>
__device__ __forceinline__ void qk_tile(const LDS_AS uint8_t* kt, uint32_t base0, uint32_t base1,
                                        const bf16x8 (&qreg)[18], f32x4 (&acc)[2], const Hook& hook = Hook()) {
  static_assert(D >= 2 && D <= 8, "K operand ring depth");
  auto addr = [&](int s) { return ((s & 1) ? base1 : base0) + (uint32_t)((s >> 1) * 128); };
  bf16x8 k0[D], k1[D];
#pragma unroll
  for (int s = 0; s < D - 1; ++s) {
    k0[s] = lds_read_b128(kt + addr(s));
    k1[s] = lds_read_b128(kt + addr(s) + 16 * kRowBytes);
  }
  // one accumulation chain per key block, kept in the caller's registers: the
  // two chains alternate, and an MFMA whose accumulator comes from the MFMA
  // before the previous one issues at the full rate (measured)
  acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 18; ++s) {
    if (s + D - 1 < 18) {
      k0[(s + D - 1) % D] = lds_read_b128(kt + addr(s + D - 1));
      k1[(s + D - 1) % D] = lds_read_b128(kt + addr(s + D - 1) + 16 * kRowBytes);
    }
    acc[0] = mfma16t<F16>(k0[s % D], qreg[s], acc[0]);
    acc[1] = mfma16t<F16>(k1[s % D], qreg[s], acc[1]);
    hook(s);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ------------------------------------------------------------------ dense decode, wave-specialised
//
// 8 waves, two per SIMD with different jobs, so that one wave's MFMAs fill the
// pipe while the other waits on LDS or runs VALU work:
//   * QK waves 0..3: wave w holds Q for rows [16w, 16w+16) in registers.  In
//     iteration t it computes S(t)^T = K(t) Q^T and, between those MFMAs, the
//     online softmax of S(t-1) (kept in registers from the previous iteration),
//     writing P(t-1) (bf16), the rescale factor and a flag to double-buffered
//     LDS slots.  The VALU softmax thus runs in the shadow of the MFMAs.
//   * PV waves 4..7: wave 4+w owns output columns [128w, 128w+128) for all rows
//     (O in registers).  In iteration t it computes O += V(t-2)^T P(t-2)^T with
//     V(t-2) held in registers and, after each 16-column block, reads the same
//     block of V(t-1) from the ring into the freed registers.  They also stream
//     the ring: at the start of iteration t, tile t+2 goes into the slot of
//     tile t-2 (whose K and V were read in iterations t-2 and t-1).  The QK
//     waves carry the longer instruction stream per tile (softmax VALU next to
//     LDS-fed MFMAs), so the ~36 vector-memory issues of a tile, which stall the
//     issuing wave while the CU's address unit drains them, cost less on the PV
//     waves (measured: decode 5-7 % faster than with the loads in the QK waves).
// One barrier per 32-key tile ends iteration t: after it tile t+1 is resident,
// P(t-1) is visible, and the V(t-1) reads of every PV wave have completed.  The
// loop runs two extra iterations to drain the softmax and PV stages.
constexpr int kWsThreads = 512;
constexpr int kQkDepth = 3;  // K operand reads in flight per key block, + 1 (3 measured 1-2 % faster than 4-5)

// Zero V rows [nvalid, 32) of a bf16 tile; `tid` in [0, 256) strides by 256.
__device__ __forceinline__ void zero_tail_rows_256(LDS_AS uint8_t* kt, int nvalid, int tid) {
  const int n = (kTK - nvalid) * 64;
  for (int idx = tid; idx < n; idx += 256) {
    const int kr = nvalid + (idx >> 6);
    const int c = idx & 63;
    *reinterpret_cast<LDS_AS u32x4*>(kt + tile_off(kr, c)) = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int RB, bool F16, bool MKV>
__global__ __launch_bounds__(kWsThreads, 1) void decode_ws_kernel(DecodeArgs a) {
  constexpr int MB = 16 * RB;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[kDLdsBytes];
  LDS_AS uint8_t* smem = (LDS_AS uint8_t*)(smem_raw);  // C-style: generic -> LDS address space
  LDS_AS float* alpha_s = reinterpret_cast<LDS_AS float*>(smem + kDOffAlpha);  // [2][64]
  LDS_AS uint8_t* flag_s = smem + kDOffFlag;  // [2][4] bytes: one 32-bit word per tile parity
  LDS_AS float* l_s = reinterpret_cast<LDS_AS float*>(smem + kDOffL);
  LDS_AS int* pages_s = reinterpret_cast<LDS_AS int*>(smem + kDOffPages);

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Waves w and w+4 share a SIMD: each SIMD runs one QK and one PV wave.
  const bool is_qk = wv < 4;
  const int w = wv & 3;  // index within the role
  const int l = tid & 63, g = l >> 4, li = l & 15;
  const bool has_rows = is_qk && w < RB;
  const int part = xcd_part(blockIdx.x, gridDim.x);
  // several KV heads: grid.y = h_kv * row blocks per head; the Mkv = s_q * G
  // rows of KV head kvh (G = h_q / h_kv query heads each) are numbered
  // s * G + hh, and are row s * h_q + kvh * G + hh of the request
  const int nrb = MKV ? (a.Mkv + MB - 1) / MB : 1;
  const int kvh = MKV ? (int)blockIdx.y / nrb : 0;
  const int rbk = MKV ? (int)blockIdx.y - kvh * nrb : (int)blockIdx.y;
  const int Mloc = MKV ? a.Mkv : a.M;
  const int Gq = MKV ? a.G : a.h_q;
  auto grow = [&](int rho) -> int {
    if constexpr (MKV) return (rho / a.G) * a.h_q + kvh * a.G + rho % a.G;
    else return rho;
  };
  const int begin_req = ld_const(a.sched_meta, part * 8 + 0);
  if (begin_req < 0) return;
  const int begin_blk = ld_const(a.sched_meta, part * 8 + 1);
  const int end_req = ld_const(a.sched_meta, part * 8 + 2);
  const int end_blk = ld_const(a.sched_meta, part * 8 + 3);
  const int begin_split = ld_const(a.sched_meta, part * 8 + 4);
  if (begin_req >= a.batch || end_req >= a.batch || end_req < begin_req || begin_blk < 0 || end_blk < 0) {
    // not a scheduler record
    if (threadIdx.x == 0) atomicOr(&g_error_flags, kErrMeta);
    return;
  }

  TileLoader<false> loader;
  loader.init(w, l);  // used by the PV waves (4 waves split a tile)
  if constexpr (MKV) loader.init_rows(w, l);
  auto issue_tile = [&](int64_t page, int key0, int st) {
    if constexpr (MKV) loader.issue_page_hkv(a, page, key0, kvh, smem, st, w);
    else loader.issue_page(a, page, key0, smem, st, w);
  };
  const int kx = li & 7;
  const uint32_t kq_base0 = (uint32_t)(li * kRowBytes + 16 * (4 * (0 ^ (kx >> 2)) + (g ^ (kx & 3))));
  const uint32_t kq_base1 = (uint32_t)(li * kRowBytes + 16 * (4 * (1 ^ (kx >> 2)) + (g ^ (kx & 3))));
  // Transposed V reads: lane group g needs keys 8g..8g+7 of the tile, read as two
  // 4-key halves.  Odd groups read the upper half first, so that in each read
  // the 16 rows cover every residue mod 8 twice and the chunk swizzle spreads
  // them over all banks (in natural order two of the four groups collide).  The
  // key order inside the MFMA contraction changes accordingly, and the QK waves
  // store P with the two halves of odd 8-key blocks swapped to match.
  const int kr0 = 8 * g + (li >> 2) + 4 * (g & 1);
  const int kr1 = 8 * g + (li >> 2) + 4 * ((g & 1) ^ 1);
  const int p_off = 8 * (g ^ (g >> 1));  // byte offset of this lane's 4 keys in a P row
  const int tr_j = li & 3;
  const uint32_t tr_within = (tr_j & 1) * 8;
  const int row_local = 16 * w + li;

  for (int r = begin_req; r <= end_req; ++r) {
    int seqlen = ld_const(a.seqlens, r);
    if (seqlen < 0 || seqlen > a.max_pages * kPage) {
      if (tid == 0) atomicOr(&g_error_flags, kErrSeqlen);
      seqlen = seqlen < 0 ? 0 : a.max_pages * kPage;
    }
    const int nblk = (seqlen + kPage - 1) / kPage;
    const int blk0 = (r == begin_req) ? begin_blk : 0;
    const int blk1 = min((r == end_req) ? end_blk : nblk, nblk);
    const int t0 = blk0 * kPage;
    const int t1 = min(blk1 * kPage, seqlen);
    const int ntile = t1 > t0 ? (t1 - t0 + kTK - 1) / kTK : 0;
    const int split = (r == begin_req) ? begin_split : 0;
    const int ns0 = ld_const(a.num_splits, r);
    const int nsplit = ld_const(a.num_splits, r + 1) - ns0;
    const int slot = ns0 + split;
    if (nsplit > 1 && (slot < 0 || slot >= a.slots)) {  // inconsistent metadata: skip, never write out of range
      if (threadIdx.x == 0) atomicOr(&g_error_flags, kErrMeta);
      continue;
    }
    const int rho = rbk * MB + row_local;
    auto uniform = [](int raw) -> int64_t { return __builtin_amdgcn_readfirstlane(raw); };
    // The PV waves start the ring at once: tiles 0 and 1 lie in the piece's
    // first page (t0 is page-aligned), whose id is one scalar load.  Meanwhile
    // the QK waves load Q and copy the page ids of the piece's first
    // kPageCache blocks to LDS (the tile loop then never waits on a scalar
    // load; later blocks, if any, are looked up directly).  Only the QK waves
    // touch the page ids with vector loads: in a PV wave the wait for them
    // would also wait for the tiles already in flight (vmcnt retires in order).
    const int ncache = min(blk1 - blk0, kPageCache);
    // page id of tile t (valid after the barrier below): an LDS read (or, past
    // the cached range, a scalar load) that is made wave-uniform only where it
    // is used
    auto page_raw = [&](int t) -> int {
      const int b = (t0 + t * kTK) / kPage - blk0;
      return b < kPageCache ? pages_s[b] : ld_const(a.block_table, (int64_t)r * a.max_pages + blk0 + b);
    };

    if (is_qk) {
      // ================================================================ QK waves
      const bool live = has_rows && rho < Mloc;
      bf16x8 qreg[18];
      {
        const uint16_t* qrow = a.q + ((int64_t)r * a.M + (live ? grow(rho) : 0)) * kDQK + 8 * g;
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
          qreg[s] = live ? v : bf16x8{};
        }
        static_assert(kPageCache == 2 * 256, "two page ids per QK-wave thread");
        const int32_t* bt = a.block_table + (int64_t)r * a.max_pages + blk0;
        const int pa = tid < ncache ? bt[tid] : 0;
        const int pb = tid + 256 < ncache ? bt[tid + 256] : 0;
        if (tid < ncache) pages_s[tid] = pa;
        if (tid + 256 < ncache) pages_s[tid + 256] = pb;
      }
      sync_lds();  // page ids in LDS (the PV waves' matching barrier follows their first loads)
      int lim = 0;
      if (live) {
        int nvis = seqlen;
        if (a.causal) nvis = min(max(seqlen - a.s_q + rho / Gq + 1, 0), seqlen);
        lim = min(t1, nvis);
      }
      float mrow = -INFINITY, lpart = 0.f;
      int lim_min = live ? lim : INT32_MAX;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) lim_min = min(lim_min, __shfl_xor(lim_min, off, 64));
      lim_min = __builtin_amdgcn_readfirstlane(lim_min);
      // raw scores: tile t's in sacc[t & 1], so that the softmax of tile t-1 reads
      // its scores in place while tile t's are computed (the loop below is
      // unrolled by two to keep the parity a compile-time index)
      f32x4 sacc[2][2];

      // Online softmax of tile ts from its raw scores `sc`, in 18 steps, one per
      // k-step of the next tile's QK^T: the waves issue in order, so a dependent
      // VALU op stalls the MFMAs behind it; one dependency level per k-step lets
      // the two MFMAs of that step cover its latency.  The scale c > 0 (checked at
      // the boundary) is applied as max(c s) = c max(s) and exp2(c s - m) =
      // exp2(fma(s, c, -m)), one op per score.
      float pv[8], mx = 0.f, ma = 0.f, mb = 0.f, alpha = 1.f, nmref = 0.f, s01 = 0.f, s23 = 0.f,
            s45 = 0.f, s67 = 0.f, pw = 0.f;
      uint32_t wp[4] = {0u, 0u, 0u, 0u};
      bool upd = false;
      auto softmax_step = [&](int step, int ts, f32x4 (&sc)[2]) {
        // x(i): score i of this lane's eight (key block i / 4, key 4g + i % 4)
        auto x = [&](int i) -> float { return sc[i >> 2][i & 3]; };
        switch (step) {
          case 0:
          case 1:
            break;
          case 2: {
            // keys past a row's visible range score -inf; skipped when every row
            // of the wave sees the whole tile
            const int key0 = t0 + ts * kTK;
            if (key0 + kTK > lim_min) {
#pragma unroll
              for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (key0 + 16 * kb + 4 * g + i >= lim) sc[kb][i] = -INFINITY;
            }
            break;
          }
          case 3:
            ma = fmaxf(fmaxf(x(0), x(1)), x(2));
            mb = fmaxf(fmaxf(x(3), x(4)), x(5));
            break;
          case 4: ma = fmaxf(fmaxf(x(6), x(7)), ma); break;
          case 5: mx = fmaxf(ma, mb); break;
          case 6: mx = rowmax16(mx); break;
          case 7: mx = rowmax32(mx); break;
          case 8: mx *= a.scale_log2; break;
          case 9: upd = mx > mrow + kRescaleThreshold; break;
          case 10: {
            const float mnew = upd ? mx : mrow;
            pw = mrow - mnew;
            mrow = mnew;
            break;
          }
          case 11:
            alpha = upd ? fast_exp2(pw) : 1.f;  // 0 when the old max was -inf
            nmref = (mrow == -INFINITY) ? 0.f : -mrow;
            break;
          case 12:
#pragma unroll
            for (int k = 0; k < 4; ++k) pv[k] = fast_exp2(__builtin_fmaf(x(k), a.scale_log2, nmref));
            break;
          case 13:
#pragma unroll
            for (int k = 4; k < 8; ++k) pv[k] = fast_exp2(__builtin_fmaf(x(k), a.scale_log2, nmref));
            break;
          case 14:
            s01 = pv[0] + pv[1];
            s23 = pv[2] + pv[3];
            s45 = pv[4] + pv[5];
            s67 = pv[6] + pv[7];
            break;
          case 15:
            wp[0] = pack2<F16>(pv[0], pv[1]);
            wp[1] = pack2<F16>(pv[2], pv[3]);
            wp[2] = pack2<F16>(pv[4], pv[5]);
            wp[3] = pack2<F16>(pv[6], pv[7]);
            s01 += s23;
            s45 += s67;
            break;
          case 16: {
            lpart = lpart * alpha + (s01 + s45);
            LDS_AS uint8_t* prow = smem + kDOffP + (ts & 1) * kPBufBytes + row_local * kPStride + p_off;
            *reinterpret_cast<LDS_AS u32x2*>(prow) = u32x2{wp[0], wp[1]};
            *reinterpret_cast<LDS_AS u32x2*>(prow + 32) = u32x2{wp[2], wp[3]};
            break;
          }
          default: {
            // the factor is read only for row blocks whose flag is set
            const bool any = __any(upd);
            if (any && g == 0) alpha_s[(ts & 1) * kMaxRowsPerWG + row_local] = alpha;
            if (l == 0) flag_s[(ts & 1) * 4 + w] = any ? 1 : 0;
            break;
          }
        }
      };

      sync_lds();  // tile 0 resident (loaded by the PV waves)
      // one iteration; DO_QK: S(t) = QK^T(t), DO_SM: softmax of S(t-1) (in the
      // shadow of the MFMAs when both run); PAR = t & 1.  Instantiated per stage
      // combination and parity.
      auto iter = [&](auto do_qk_c, auto do_sm_c, auto par_c, int t) {
        constexpr bool DO_QK = decltype(do_qk_c)::value;
        constexpr bool DO_SM = decltype(do_sm_c)::value;
        constexpr int PAR = decltype(par_c)::value;
        if (has_rows) {
          if constexpr (DO_QK) {
            const LDS_AS uint8_t* kt = smem + kOffKDense + (t & 3) * kTileBytes;
            if constexpr (DO_SM) {
              // one softmax step after each k-step
              qk_tile<kQkDepth, F16>(kt, kq_base0, kq_base1, qreg, sacc[PAR], [&](int s) {
                softmax_step(s, t - 1, sacc[PAR ^ 1]);
              });
            } else {
              qk_tile<kQkDepth, F16>(kt, kq_base0, kq_base1, qreg, sacc[PAR]);
            }
          } else if constexpr (DO_SM) {
#pragma unroll
            for (int step = 0; step < 18; ++step) softmax_step(step, t - 1, sacc[PAR ^ 1]);
          }
          if (t == ntile) {  // every tile's softmax is done: row sums for the output stage
            const float lt = row4_sum(lpart);
            if (g == 0) {
              l_s[row_local] = lt;
              if (rho < Mloc) {
                const float lse = lt > 0.f ? (mrow + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
                // row index made opaque here: otherwise the compiler hoists the
                // 64-bit store addresses out of the request loop and spills them
                int gr = grow(rho);
                asm volatile("" : "+v"(gr));
                if (nsplit == 1) a.lse[(int64_t)r * a.M + gr] = lse;
                else a.part_lse[(int64_t)slot * a.M + gr] = lse;
              }
            }
          }
        }
        sync_lds();
      };
      using F = std::false_type;
      using T = std::true_type;
      using P0 = std::integral_constant<int, 0>;
      using P1 = std::integral_constant<int, 1>;
      // t = 0: QK only; 1..ntile-1: QK + softmax(t-1); ntile: softmax only;
      // ntile+1: nothing (the PV waves drain)
      if (ntile >= 1) {
        iter(T{}, F{}, P0{}, 0);
        int t = 1;
        for (; t + 1 < ntile; t += 2) {
          iter(T{}, T{}, P1{}, t);
          iter(T{}, T{}, P0{}, t + 1);
        }
        if (t < ntile) iter(T{}, T{}, P1{}, t++);
        if (t & 1) iter(F{}, T{}, P1{}, t);
        else iter(F{}, T{}, P0{}, t);
      } else {
        iter(F{}, F{}, P0{}, 0);
      }
      iter(F{}, F{}, P0{}, ntile + 1);
    } else {
      // ================================================================ PV waves
      f32x4 o[8][RB];
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 v8[8];  // V^T fragments of one tile (this wave's 128 columns, 32 keys)
      // per-lane offsets of the transposed reads: column chunk c = 16w + 2db + (tr_j >> 1)
      // swizzled with the key row; db and db + 4 differ by 8 chunks (bit 3, which
      // the 3-bit swizzle leaves alone), i.e. by 128 bytes
      uint32_t voff0[4], voff1[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int c = 16 * w + 2 * d + (tr_j >> 1);
        voff0[d] = tile_off(kr0, c) + tr_within;
        voff1[d] = tile_off(kr1, c) + tr_within;
      }
      auto vread = [&](int t, int db) {
        const LDS_AS uint8_t* kt = smem + kOffKDense + (t & 3) * kTileBytes + (db >> 2) * 128;
        v8[db] = __builtin_shufflevector(lds_read_tr16(kt + voff0[db & 3]), lds_read_tr16(kt + voff1[db & 3]), 0, 1, 2, 3,
                                         4, 5, 6, 7);
      };

      // The ring: tiles 0 and 1 now, tile t+2 at the start of iteration t.
      if (ntile > 0) {
        const int64_t p0 = uniform(ld_const(a.block_table, (int64_t)r * a.max_pages + blk0));
        issue_tile(p0, t0, 0);
        if (ntile > 1) issue_tile(p0, t0 + kTK, 1);
      }
      sync_lds();  // page ids in LDS (filled by the QK waves)
      // page id of the tile the next iteration loads: read before the barrier that
      // ends an iteration (which waits for it) and made wave-uniform after it
      int pg_next = ntile > 2 ? page_raw(2) : 0;
      if (ntile > 1) wait_vmcnt<kLPW>();
      else wait_vmcnt<0>();
      sync_lds();  // tile 0 resident
      // one iteration; DO_PV: PV(t-2) from registers, DO_VREAD: V(t-1) into
      // registers.  Instantiated per stage combination so that the steady-state
      // loop carries no stage conditions (and no register copies for them).
      auto iter = [&](auto do_pv_c, auto do_vread_c, int t) {
        constexpr bool DO_PV = decltype(do_pv_c)::value;
        constexpr bool DO_VREAD = decltype(do_vread_c)::value;
        if (t < ntile) {
          const int nvalid = min(kTK, t1 - (t0 + t * kTK));
          if (nvalid < kTK) zero_tail_rows_256(smem + kOffKDense + (t & 3) * kTileBytes, nvalid, 64 * w + l);
        }
        const int tp = t - 2, tv = t - 1;
        // loads of tile t+2 into the slot of tile t-2 (its K was read in
        // iteration t-2, its V in iteration t-1), before anything else
        const bool more = t + 2 < ntile;
        if (more) issue_tile(uniform(pg_next), t0 + (t + 2) * kTK, (t + 2) & 3);
        // PV(t-2) operands from LDS first: rescale flags and factors, P^T
        uint32_t fl = 0;
        float al[RB];
        bf16x8 bp[RB];
        if constexpr (DO_PV) {
          const LDS_AS uint8_t* pb = smem + kDOffP + (tp & 1) * kPBufBytes;
          fl = *reinterpret_cast<const LDS_AS uint32_t*>(flag_s + (tp & 1) * 4);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) al[rb] = alpha_s[(tp & 1) * kMaxRowsPerWG + 16 * rb + li];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) bp[rb] = lds_read_b128(pb + (16 * rb + li) * kPStride + 16 * g);
        }
        if constexpr (DO_PV) {
          if (tp > 0) {  // O is still zero before the first tile: nothing to rescale
            const uint32_t fls = __builtin_amdgcn_readfirstlane(fl);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              if ((fls >> (8 * rb)) & 0xffu) {
#pragma unroll
                for (int db = 0; db < 8; ++db) o[db][rb] *= al[rb];
              }
            }
          }
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const bf16x8 av = v8[db];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) o[db][rb] = mfma16t<F16>(av, bp[rb], o[db][rb]);
            if constexpr (DO_VREAD) vread(tv, db);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else if constexpr (DO_VREAD) {
#pragma unroll
          for (int db = 0; db < 8; ++db) vread(tv, db);
        }
        // own loads of tile t+1 done (tile t+2 may stay in flight)
        if (t + 1 < ntile) {
          if (more) wait_vmcnt<kLPW>();
          else wait_vmcnt<0>();
        }
        if (t + 3 < ntile) pg_next = page_raw(t + 3);
        sync_lds();
      };
      using F = std::false_type;
      using T = std::true_type;
      iter(F{}, F{}, 0);
      if (ntile >= 1) {
        iter(F{}, T{}, 1);
        for (int t = 2; t <= ntile; ++t) iter(T{}, T{}, t);
        iter(T{}, F{}, ntile + 1);
      } else {
        iter(F{}, F{}, 1);
      }
      sync_lds();  // l from the QK waves (written in iteration ntile)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int rho_l = rbk * MB + 16 * rb + li;
        if (rho_l >= Mloc) continue;
        int rho_o = grow(rho_l);
        asm volatile("" : "+v"(rho_o));  // keeps the row addresses from being hoisted and spilled
        const float lt = l_s[16 * rb + li];
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        if (nsplit == 1) {
          uint16_t* orow = a.out + ((int64_t)r * a.M + rho_o) * kDV + 128 * w + 4 * g;
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const f32x4 vv = o[db][rb] * inv;
            *reinterpret_cast<u32x2*>(orow + 16 * db) = u32x2{pack2<F16>(vv[0], vv[1]), pack2<F16>(vv[2], vv[3])};
          }
        } else {
          float* prow = a.part_o + ((int64_t)slot * a.M + rho_o) * kDV + 128 * w + 4 * g;
#pragma unroll
          for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(prow + 16 * db) = o[db][rb] * inv;
        }
      }
      wait_vmcnt<0>();  // the next request's loads must not overtake this one's stores in the count
    }
    if (is_qk) sync_lds();  // matches the PV waves' extra barrier before the output stage
    // every LDS buffer is reused by the next request of this partition
    sync_lds();
  }
}

// ------------------------------------------------------------------ FP8 decode, wave-specialised
//
// The sparse FP8 paths with the two-role structure of decode_ws_kernel.  The raw
// 656-byte records stream into a 3-slot ring.  One iteration ahead of their use,
// the PV waves convert each raw tile into a bf16 tile in the dense kernel's
// swizzled layout (E4M3 -> bf16 is exact: every E4M3 value is a bf16 value; the
// RoPE part is copied) and copy the per-key fp32 block scales into two tables.
// The scales are applied in fp32 to the scores and to P, never to a rounded K
// or V.
//   * QK waves 0..3 (16 rows each): S(t)^T = K(t) Q^T from bf16 tile t & 1 with
//     the dense kernel's operand reads.  The four 128-dim NoPE blocks and the
//     RoPE part accumulate apart, and each key's block scales combine them at
//     the end of the tile.  The softmax of tile t-1 runs between the k-steps of
//     tile t and writes P(t-1) once, unnormalised, in fp32.  They also stream
//     the ring: raw tile t+3 at the start of iteration t, into the slot of raw
//     tile t (converted in iteration t-1).
//   * PV waves 4..7: wave 4+w owns output columns [128w, 128w+128) -- NoPE
//     block w -- for all rows.  In iteration t it reads P(t-2), multiplies it by
//     each key's scale of block w and rounds it to bf16 (its P^T operand),
//     computes O += V(t-2)^T P^T from registers while reading V(t-1) into them
//     (transposed reads as in the dense kernel), and then converts block w of
//     raw tile t+1, for all 32 keys, into bf16 tile (t+1) & 1: exactly the
//     region its own V(t-1) reads have just left (a wave's LDS accesses complete
//     in order).  It also copies an eighth of that tile's RoPE and its block-w
//     scales.  Keys past the tile's valid count get zeros (K, V and scales), so
//     no record outside the valid prefix reaches the result (the by-index
//     loader reads record 0 for them).
// One barrier per tile.  (The earlier version converted tile t at the start of
// iteration t in all eight waves, behind a second barrier, and converted V in
// registers after ds_read_b64_tr_b8 reads of the raw records: the conversion
// and that barrier sat on the QK waves' path every tile.)
constexpr int kF8RawSlots = 3;
constexpr int kF8PPitch = kTK * 4 + 16;                          // fp32 P row: 32 keys + 16 B
constexpr int kF8PBuf = kMaxRowsPerWG * kF8PPitch;               // 9216
constexpr int kF8OffP = kOffRaw + kF8RawSlots * kRawTileBytes;   // 136704: fp32 P[2 parities]
constexpr int kF8OffS = kF8OffP + 2 * kF8PBuf;                   // 155136: PV scales [4 tiles][4 blocks][32 keys]
constexpr int kF8OffSq = kF8OffS + 4 * 4 * kTK * 4;              // 157184: QK scales [2 tiles][32 keys][4 blocks]
constexpr int kF8OffAlpha = kF8OffSq + 2 * kTK * 4 * 4;          // 158208
constexpr int kF8OffFlag = kF8OffAlpha + 2 * kMaxRowsPerWG * 4;  // 158720
constexpr int kF8OffL = kF8OffFlag + 64;                         // 158784
constexpr int kF8LdsBytes = kF8OffL + kMaxRowsPerWG * 4;         // 159040
constexpr int kF8OffIds = kF8LdsBytes;                           // by index: top-k ids of the piece
constexpr int kF8LdsBytesIdx = kF8OffIds + kIdxCache * 4;        // 163136
static_assert(kOffRaw == 2 * kTileBytes, "FP8 raw ring after the two bf16 tiles");
static_assert(kF8OffIds == kF8OffIdsLoader, "indexed loader's id cache offset");
static_assert(kF8LdsBytesIdx <= 160 * 1024, "FP8 wave-specialised LDS budget");
static_assert(kF8OffP % 16 == 0 && kF8OffS % 16 == 0 && kF8OffSq % 16 == 0, "16-B aligned LDS regions");

// 8 E4M3 bytes (two dwords, byte k = element k) -> 8 bf16, exactly
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 raw) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// PV wave w's share of converting raw tile `raw` into bf16 tile `kt` (dense
// layout, key row k, 16-B chunk c at tile_off(k, c)):
//   * NoPE block w of all 32 keys: lane l converts the 8 bytes (l & 15) of the
//     block of keys 4i + (l >> 4), i < 8, into chunk 16w + (l & 15);
//   * RoPE chunk (l & 7) of key 8w + (l >> 3), copied;
//   * scale w of key l (l < 32) into the PV table (sp[32w + k]) and the QK
//     table (sq[4k + w]).
// Keys at or past nvalid get zeros.  Eight consecutive lanes write one aligned
// 128-B span of a row (conflict-free 16-B writes).  All reads are issued
// before the first conversion.
template <bool FULL>
__device__ __forceinline__ void convert_block_t(const LDS_AS uint8_t* raw, LDS_AS uint8_t* kt, LDS_AS float* sp,
                                                LDS_AS float* sq, int w, int nvalid) {
  const int l = lane_id_here();  // addresses formed here, not hoisted out of the tile loop (and spilled)
  const int cc = l & 15, kq = l >> 4;
  // key 4i + kq: its raw bytes at src + 4i records, its bf16 chunk at d0 (i even)
  // or d1 (i odd) + (i / 2) * 8 rows (the swizzle depends on the key mod 8 only)
  const LDS_AS uint8_t* src = raw + kq * kRecBytes + 128 * w + 8 * cc;
  LDS_AS uint8_t* const d0 = kt + tile_off(kq, 16 * w + cc);
  LDS_AS uint8_t* const d1 = kt + tile_off(4 + kq, 16 * w + cc);
  u32x2 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const LDS_AS u32x2*>(src + 4 * i * kRecBytes);
  const int rk = 8 * w + (l >> 3);
  const u32x4 rp = *reinterpret_cast<const LDS_AS u32x4*>(raw + rk * kRecBytes + 528 + 16 * (l & 7));
  float s = 0.f;
  if (l < 32) s = *reinterpret_cast<const LDS_AS float*>(raw + l * kRecBytes + 512 + 4 * w);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bf16x8 x = e4m3x8_to_bf16(v[i]);
    if (!FULL && 4 * i + kq >= nvalid) x = bf16x8{};
    *reinterpret_cast<LDS_AS bf16x8*>(((i & 1) ? d1 : d0) + (i >> 1) * 8 * kRowBytes) = x;
  }
  *reinterpret_cast<LDS_AS u32x4*>(kt + tile_off(rk, 64 + (l & 7))) =
      (FULL || rk < nvalid) ? rp : u32x4{0u, 0u, 0u, 0u};
  if (l < 32) {
    if (!FULL && l >= nvalid) s = 0.f;
    sp[32 * w + l] = s;
    sq[4 * l + w] = s;
  }
}
__device__ __forceinline__ void convert_block(const LDS_AS uint8_t* raw, LDS_AS uint8_t* kt, LDS_AS float* sp,
                                              LDS_AS float* sq, int w, int nvalid) {
  if (nvalid >= kTK) convert_block_t<true>(raw, kt, sp, sq, w, nvalid);
  else convert_block_t<false>(raw, kt, sp, sq, w, nvalid);
}

template <bool IDX>
__global__ __launch_bounds__(kWsThreads, 1) void decode_fp8ws_kernel(DecodeArgs a) {
  constexpr int RB = 4, MB = 64;
  using Loader = std::conditional_t<IDX, IndexedLoader, TileLoader<true>>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[IDX ? kF8LdsBytesIdx : kF8LdsBytes];
  LDS_AS uint8_t* smem = (LDS_AS uint8_t*)(smem_raw);
  LDS_AS float* sp_s = reinterpret_cast<LDS_AS float*>(smem + kF8OffS);        // [4 tiles][4 blocks][32 keys]
  LDS_AS float* sq_s = reinterpret_cast<LDS_AS float*>(smem + kF8OffSq);       // [2 tiles][32 keys][4 blocks]
  LDS_AS float* alpha_s = reinterpret_cast<LDS_AS float*>(smem + kF8OffAlpha);  // [2][64]
  LDS_AS uint8_t* flag_s = smem + kF8OffFlag;                                    // [2][4] bytes
  LDS_AS float* l_s = reinterpret_cast<LDS_AS float*>(smem + kF8OffL);

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool is_qk = wv < 4;
  const int w = wv & 3;
  const int l = tid & 63, g = l >> 4, li = l & 15;
  const int part = xcd_part(blockIdx.x, gridDim.x), rbk = blockIdx.y;
  const int begin_req = ld_const(a.sched_meta, part * 8 + 0);
  if (begin_req < 0) return;
  const int begin_blk = ld_const(a.sched_meta, part * 8 + 1);
  const int end_req = ld_const(a.sched_meta, part * 8 + 2);
  const int end_blk = ld_const(a.sched_meta, part * 8 + 3);
  const int begin_split = ld_const(a.sched_meta, part * 8 + 4);
  if (begin_req >= a.batch || end_req >= a.batch || end_req < begin_req || begin_blk < 0 || end_blk < 0) {
    // not a scheduler record
    if (threadIdx.x == 0) atomicOr(&g_error_flags, kErrMeta);
    return;
  }

  Loader loader;
  loader.init(w, l);  // used by the QK waves
  // loads of the newest tile in flight that a QK wave may leave outstanding
  // while it waits for the one before (wave-uniform)
  const bool wave0 = w == 0;
  auto wait_all_but_inflight = [&]() {
    if constexpr (IDX) {
      wait_vmcnt<kIdxLoadsPerWave>();
    } else {
      if (wave0) wait_vmcnt<6>();
      else wait_vmcnt<5>();
    }
  };
  const int row_local = 16 * w + li;
  // the dense kernel's operand reads of a bf16 tile: QK^T (K as the A operand)
  // and the transposed V reads, odd lane groups reading their upper 4-key half
  // first (P^T is built in the same key order)
  const int kx = li & 7;
  const uint32_t kq_base0 = (uint32_t)(li * kRowBytes + 16 * (4 * (0 ^ (kx >> 2)) + (g ^ (kx & 3))));
  const uint32_t kq_base1 = (uint32_t)(li * kRowBytes + 16 * (4 * (1 ^ (kx >> 2)) + (g ^ (kx & 3))));
  const int kh0 = 8 * g + 4 * (g & 1), kh1 = 8 * g + 4 * ((g & 1) ^ 1);  // keys of the two halves
  const int kr0 = kh0 + (li >> 2), kr1 = kh1 + (li >> 2);
  const int tr_j = li & 3;
  const uint32_t tr_within = (tr_j & 1) * 8;

  for (int r = begin_req; r <= end_req; ++r) {
    int seqlen = ld_const(a.seqlens, r);
    if (seqlen < 0 || seqlen > a.cap) {
      if (tid == 0) atomicOr(&g_error_flags, kErrSeqlen);
      seqlen = seqlen < 0 ? 0 : a.cap;
    }
    // the selected keys of query token s of request r are row r * s_q + s
    const int lrow = r * a.s_q + (rbk * MB) / a.h_q;
    if constexpr (IDX) loader.n = seqlen;
    const int nblk = (seqlen + kPage - 1) / kPage;
    const int blk0 = (r == begin_req) ? begin_blk : 0;
    const int blk1 = (r == end_req) ? end_blk : nblk;
    const int t0 = blk0 * kPage;
    const int t1 = min(blk1 * kPage, seqlen);
    const int ntile = t1 > t0 ? (t1 - t0 + kTK - 1) / kTK : 0;
    const int split = (r == begin_req) ? begin_split : 0;
    const int ns0 = ld_const(a.num_splits, r);
    const int nsplit = ld_const(a.num_splits, r + 1) - ns0;
    const int slot = ns0 + split;
    if (nsplit > 1 && (slot < 0 || slot >= a.slots)) {
      if (threadIdx.x == 0) atomicOr(&g_error_flags, kErrMeta);
      continue;
    }
    auto raw_slot = [&](int t) -> LDS_AS uint8_t* { return smem + kOffRaw + (t % kF8RawSlots) * kRawTileBytes; };
    auto bf_tile = [&](int t) -> LDS_AS uint8_t* { return smem + (t & 1) * kTileBytes; };
    auto nvalid_of = [&](int t) { return min(kTK, t1 - (t0 + t * kTK)); };
    if constexpr (IDX) {
      // the piece's first kIdxCache top-k ids -> LDS, read by the ring loads
      // (later ids, if any, are read directly)
      LDS_AS int32_t* ids = reinterpret_cast<LDS_AS int32_t*>(smem + kF8OffIds);
      const int kc1 = max(min(t1, t0 + kIdxCache), t0);
      for (int i = tid; i < kc1 - t0; i += kWsThreads) ids[i] = a.block_table[(int64_t)lrow * a.cap + t0 + i];
      loader.kc0 = t0;
      loader.kc1 = kc1;
      sync_lds();
    }

    if (is_qk) {
      // ================================================================ QK waves
      bool live;
      bf16x8 qreg[18];
      {
        // the Q address is formed here, not hoisted out of the request loop (and spilled)
        const int ln = lane_id_here();
        const int rq = rbk * MB + 16 * w + (ln & 15);
        live = rq < a.M;
        const uint16_t* qrow = a.q + ((int64_t)r * a.M + (live ? rq : 0)) * kDQK + 8 * (ln >> 4);
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
          qreg[s] = live ? v : bf16x8{};
        }
      }
      const int lim = live ? t1 : 0;
      const int lim_min = __all(live) ? t1 : 0;  // every row of the wave sees keys below this
      float mrow = -INFINITY, lpart = 0.f;
      float sx[8];  // scaled scores of the tile whose softmax runs next (keys 16kb + 4g + i)
#pragma unroll
      for (int k = 0; k < 8; ++k) sx[k] = -INFINITY;

      // softmax of tile ts in steps (one dependency level per k-step of the next tile)
      float mx = 0.f, ma = 0.f, mb = 0.f, alpha = 1.f, nmref = 0.f, pw = 0.f, psum = 0.f;
      float pv[8];
      bool upd = false;
      auto softmax_step = [&](int step, int ts) {
        switch (step) {
          case 0: ma = fmaxf(fmaxf(sx[0], sx[1]), fmaxf(sx[2], sx[3])); break;
          case 1: mb = fmaxf(fmaxf(sx[4], sx[5]), fmaxf(sx[6], sx[7])); break;
          case 2: mx = fmaxf(ma, mb); break;
          case 3: mx = rowmax16(mx); break;
          case 4: mx = rowmax32(mx); break;
          case 5: upd = mx > mrow + kRescaleThreshold; break;
          case 6: {
            const float mnew = upd ? mx : mrow;
            pw = mrow - mnew;
            mrow = mnew;
            break;
          }
          case 7:
            alpha = upd ? fast_exp2(pw) : 1.f;
            nmref = (mrow == -INFINITY) ? 0.f : -mrow;
            break;
          case 8:
#pragma unroll
            for (int k = 0; k < 4; ++k) pv[k] = fast_exp2(sx[k] + nmref);
            break;
          case 9:
#pragma unroll
            for (int k = 4; k < 8; ++k) pv[k] = fast_exp2(sx[k] + nmref);
            break;
          case 10:
            psum = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
            lpart = lpart * alpha + psum;
            break;
          case 11: {
            // unnormalised P of tile ts in fp32 (keys 4g + i and 16 + 4g + i); the
            // PV wave of NoPE block b multiplies it by each key's scale b
            LDS_AS uint8_t* prow = smem + kF8OffP + (ts & 1) * kF8PBuf + row_local * kF8PPitch + 16 * g;
            *reinterpret_cast<LDS_AS f32x4*>(prow) = f32x4{pv[0], pv[1], pv[2], pv[3]};
            *reinterpret_cast<LDS_AS f32x4*>(prow + 64) = f32x4{pv[4], pv[5], pv[6], pv[7]};
            break;
          }
          case 12: {
            const bool any = __any(upd);
            if (any && g == 0) alpha_s[(ts & 1) * kMaxRowsPerWG + row_local] = alpha;
            if (l == 0) flag_s[(ts & 1) * 4 + w] = any ? 1 : 0;
            break;
          }
          default: break;
        }
      };

      // QK^T of tile t from bf16 tile t & 1: NoPE k-steps (s < 16) into block
      // s / 4, RoPE k-steps into their own sum; scores combined with the block
      // scales of the QK table -> sx
      auto qk = [&](int t, auto hook) {
        const LDS_AS uint8_t* kt = bf_tile(t);
        const LDS_AS float* sq = sq_s + (t & 1) * kTK * 4;
        auto addr = [&](int s) { return ((s & 1) ? kq_base1 : kq_base0) + (uint32_t)((s >> 1) * 128); };
        auto rd0 = [&](int s) { return lds_read_b128(kt + addr(s)); };
        auto rd1 = [&](int s) { return lds_read_b128(kt + addr(s) + 16 * kRowBytes); };
        constexpr int D = kQkDepth;
        f32x4 acc[2][5];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int gi = 0; gi < 5; ++gi) acc[kb][gi] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 k0[D], k1[D];
#pragma unroll
        for (int s = 0; s < D - 1; ++s) {
          k0[s] = rd0(s);
          k1[s] = rd1(s);
        }
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          if (s + D - 1 < 18) {
            k0[(s + D - 1) % D] = rd0(s + D - 1);
            k1[(s + D - 1) % D] = rd1(s + D - 1);
          }
          const int gi = s < 16 ? (s >> 2) : 4;
          acc[0][gi] = mfma16(k0[s % D], qreg[s], acc[0][gi]);
          acc[1][gi] = mfma16(k1[s % D], qreg[s], acc[1][gi]);
          hook(s);
          __builtin_amdgcn_sched_barrier(0);
        }
        const int key0 = t0 + t * kTK;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kr = 16 * kb + 4 * g + i;
            const f32x4 sc = *reinterpret_cast<const LDS_AS f32x4*>(sq + 4 * kr);  // 0 past the valid count
            float x = acc[kb][4][i] + sc[0] * acc[kb][0][i] + sc[1] * acc[kb][1][i] + sc[2] * acc[kb][2][i] +
                      sc[3] * acc[kb][3][i];
            x *= a.scale_log2;
            sx[kb * 4 + i] = x;
          }
        if (key0 + kTK > lim_min) {  // wave-uniform: some row of the wave does not see the whole tile
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (key0 + 16 * kb + 4 * g + i >= lim) sx[kb * 4 + i] = -INFINITY;
        }
      };

      // the ring: raw tiles 0..2 now; tiles 0 and 1 resident before the PV
      // waves convert tile 0 (and, in iteration 0, tile 1)
      if (ntile > 0) loader.issue(a, lrow, t0, smem, 0, w);
      if (ntile > 1) loader.issue(a, lrow, t0 + kTK, smem, 1, w);
      if (ntile > 2) loader.issue(a, lrow, t0 + 2 * kTK, smem, 2, w);
      if (ntile > 2) wait_all_but_inflight();
      else wait_vmcnt<0>();
      sync_lds();  // raw tiles 0 and 1 resident
      sync_lds();  // bf16 tile 0 converted
      auto iter = [&](auto do_qk_c, auto do_sm_c, int t) {
        constexpr bool DO_QK = decltype(do_qk_c)::value;
        constexpr bool DO_SM = decltype(do_sm_c)::value;
        const bool more = t + 3 < ntile;
        if (more) loader.issue(a, lrow, t0 + (t + 3) * kTK, smem, t % kF8RawSlots, w);
        if constexpr (DO_QK) {
          if constexpr (DO_SM) {
            // the softmax of t-1 reads sx, which qk(t) overwrites only at its end
            qk(t, [&](int s) { softmax_step(s, t - 1); });
          } else {
            qk(t, [](int) {});
          }
        } else if constexpr (DO_SM) {
#pragma unroll
          for (int step = 0; step < 13; ++step) softmax_step(step, t - 1);
        }
        if (t == ntile) {  // every tile's softmax is done: row sums for the output stage
          const float lt = row4_sum(lpart);
          // the row index is formed here: otherwise the compiler hoists the LDS
          // and 64-bit store addresses out of the request loop and spills them
          const int ln = lane_id_here();
          if (ln < 16) {
            const int rl = 16 * w + ln;
            l_s[rl] = lt;
            const int gr = rbk * MB + rl;
            if (gr < a.M) {
              const float lse = lt > 0.f ? (mrow + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
              if (nsplit == 1) a.lse[(int64_t)r * a.M + gr] = lse;
              else a.part_lse[(int64_t)slot * a.M + gr] = lse;
            }
          }
        }
        if (t + 2 < ntile) {  // raw tile t+2 resident before the barrier (converted next iteration)
          if (more) wait_all_but_inflight();
          else wait_vmcnt<0>();
        }
        sync_lds();
      };
      using F = std::false_type;
      using T = std::true_type;
      if (ntile >= 1) {
        iter(T{}, F{}, 0);
        for (int t = 1; t < ntile; ++t) iter(T{}, T{}, t);
        iter(F{}, T{}, ntile);
      } else {
        iter(F{}, F{}, 0);
      }
      iter(F{}, F{}, ntile + 1);
    } else {
      // ================================================================ PV waves
      f32x4 o[8][RB];
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 v8[8];  // V^T fragments of one tile (this wave's 128 columns, 32 keys)
      uint32_t voff0[4], voff1[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int c = 16 * w + 2 * d + (tr_j >> 1);
        voff0[d] = tile_off(kr0, c) + tr_within;
        voff1[d] = tile_off(kr1, c) + tr_within;
      }
      auto vread = [&](int t, int db) {
        const LDS_AS uint8_t* kt = bf_tile(t) + (db >> 2) * 128;
        v8[db] = __builtin_shufflevector(lds_read_tr16(kt + voff0[db & 3]), lds_read_tr16(kt + voff1[db & 3]), 0, 1, 2, 3,
                                         4, 5, 6, 7);
      };
      auto convert = [&](int t) {
        convert_block(raw_slot(t), bf_tile(t), sp_s + (t & 3) * 4 * kTK, sq_s + (t & 1) * kTK * 4, w, nvalid_of(t));
      };
      sync_lds();  // raw tiles 0 and 1 resident
      if (ntile > 0) convert(0);
      sync_lds();  // bf16 tile 0 converted
      // one iteration: PV(t-2) from registers, V(t-1) into registers, then raw
      // tile t+1 converted into the bf16 tile V(t-1) came from
      auto iter = [&](auto do_pv_c, auto do_vread_c, int t) {
        constexpr bool DO_PV = decltype(do_pv_c)::value;
        constexpr bool DO_VREAD = decltype(do_vread_c)::value;
        const int tp = t - 2;
        if constexpr (DO_PV) {
          // P^T operand of row 16 rb + li: the two 4-key halves of keys 8g..8g+7
          // of P(t-2), in the order of the V^T reads, times their scale w.  One
          // row block at a time: forming the operand of row block rb + 1 runs
          // while the MFMAs of row block rb are in the pipe.
          const LDS_AS uint8_t* pb = smem + kF8OffP + (tp & 1) * kF8PBuf + li * kF8PPitch;
          const LDS_AS float* sp = sp_s + (tp & 3) * 4 * kTK + kTK * w;
          const f32x4 s0 = *reinterpret_cast<const LDS_AS f32x4*>(sp + kh0);
          const f32x4 s1 = *reinterpret_cast<const LDS_AS f32x4*>(sp + kh1);
          const uint32_t fls =
              tp > 0 ? __builtin_amdgcn_readfirstlane(*reinterpret_cast<const LDS_AS uint32_t*>(flag_s + (tp & 1) * 4))
                     : 0u;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const f32x4 p0 = *reinterpret_cast<const LDS_AS f32x4*>(pb + 16 * rb * kF8PPitch + 4 * kh0);
            const f32x4 p1 = *reinterpret_cast<const LDS_AS f32x4*>(pb + 16 * rb * kF8PPitch + 4 * kh1);
            const bf16x8 bq = __builtin_bit_cast(
                bf16x8, u32x4{pack_bf16x2(p0[0] * s0[0], p0[1] * s0[1]), pack_bf16x2(p0[2] * s0[2], p0[3] * s0[3]),
                              pack_bf16x2(p1[0] * s1[0], p1[1] * s1[1]), pack_bf16x2(p1[2] * s1[2], p1[3] * s1[3])});
            if ((fls >> (8 * rb)) & 0xffu) {  // the running max of this row block moved
              const float al = alpha_s[(tp & 1) * kMaxRowsPerWG + 16 * rb + li];
#pragma unroll
              for (int db = 0; db < 8; ++db) o[db][rb] *= al;
            }
#pragma unroll
            for (int db = 0; db < 8; ++db) o[db][rb] = mfma16(v8[db], bq, o[db][rb]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // V(t-1) into the registers PV(t-2) has finished with; then raw tile t+1
        // converted into the bf16 tile those reads came from
        if constexpr (DO_VREAD) {
#pragma unroll
          for (int db = 0; db < 8; ++db) vread(t - 1, db);
        }
        if (t + 1 < ntile) convert(t + 1);
        sync_lds();
      };
      using F = std::false_type;
      using T = std::true_type;
      iter(F{}, F{}, 0);
      if (ntile >= 1) {
        iter(F{}, T{}, 1);
        for (int t = 2; t <= ntile; ++t) iter(T{}, T{}, t);
        iter(T{}, F{}, ntile + 1);
      } else {
        iter(F{}, F{}, 1);
      }
      sync_lds();  // l from the QK waves (written in iteration ntile)
      // output rows and addresses formed here from opaque lane indices: the
      // compiler otherwise hoists them out of the request loop and spills them
      int col = 128 * w + 4 * g, lo = li;
      asm volatile("" : "+v"(col), "+v"(lo));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int rho_o = rbk * MB + 16 * rb + lo;
        if (rho_o >= a.M) continue;
        const float lt = l_s[16 * rb + li];
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        if (nsplit == 1) {
          uint16_t* orow = a.out + ((int64_t)r * a.M + rho_o) * kDV + col;
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const f32x4 vv = o[db][rb] * inv;
            *reinterpret_cast<u32x2*>(orow + 16 * db) = u32x2{pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3])};
          }
        } else {
          float* prow = a.part_o + ((int64_t)slot * a.M + rho_o) * kDV + col;
#pragma unroll
          for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(prow + 16 * db) = o[db][rb] * inv;
        }
      }
      wait_vmcnt<0>();
    }
    if (is_qk) sync_lds();  // matches the PV waves' extra barrier before the output stage
    sync_lds();             // every LDS buffer is reused by the next request of this partition
  }
}

// 16-row blocks per workgroup.  Capped at 4 (64 rows): at 128 rows the Q and O
// register tiles alone take ~400 of a wave's 512 registers and the compiler
// spills; an h_q = 128 request is covered by two 64-row workgroups whose
// shared KV tiles meet in L2.
int decode_row_blocks_per_wg(int M) {
  int rb = (M + 15) / 16;
  if (rb <= 1) return 1;
  if (rb <= 2) return 2;
  return 4;
}

template <int RB>
static hipError_t launch_decode_t(const DecodeArgs& a, int kind, hipStream_t stream) {
  const int MB = 16 * RB;
  const bool mkv = a.h_kv > 1;
  dim3 grid(a.num_parts, mkv ? a.h_kv * ((a.Mkv + MB - 1) / MB) : (a.M + MB - 1) / MB);
  if ((kind == kDecodeFp8Packed || kind == kDecodeFp8Indexed) && RB != 4)
    return hipErrorInvalidValue;  // the FP8 kernel covers 64 rows (h_q is 64 or 128 there)
  if (kind == kDecodeFp8Packed)
    hipLaunchKernelGGL((decode_fp8ws_kernel<false>), grid, dim3(kWsThreads), 0, stream, a);
  else if (kind == kDecodeFp8Indexed)
    hipLaunchKernelGGL((decode_fp8ws_kernel<true>), grid, dim3(kWsThreads), 0, stream, a);
  else if (kind == kDecodeF16 && mkv)
    hipLaunchKernelGGL((decode_ws_kernel<RB, true, true>), grid, dim3(kWsThreads), 0, stream, a);
  else if (kind == kDecodeF16)
    hipLaunchKernelGGL((decode_ws_kernel<RB, true, false>), grid, dim3(kWsThreads), 0, stream, a);
  else if (mkv)
    hipLaunchKernelGGL((decode_ws_kernel<RB, false, true>), grid, dim3(kWsThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_ws_kernel<RB, false, false>), grid, dim3(kWsThreads), 0, stream, a);
  return hipGetLastError();
}

int decode_rows_per_wg(int M, int h_kv, int kind) {
  (void)kind;
  return 16 * decode_row_blocks_per_wg(h_kv > 1 ? M / h_kv : M);
}

// Name of the instantiation launch_decode runs for this shape (as profilers
// print it, without namespaces and parameter list).
const char* decode_kernel_name(int M, int h_kv, int kind) {
  if (kind == kDecodeFp8Packed) return "decode_fp8ws_kernel<false>";
  if (kind == kDecodeFp8Indexed) return "decode_fp8ws_kernel<true>";
  static const char* const names[3][2][2] = {
      {{"decode_ws_kernel<1, false, false>", "decode_ws_kernel<1, false, true>"},
       {"decode_ws_kernel<1, true, false>", "decode_ws_kernel<1, true, true>"}},
      {{"decode_ws_kernel<2, false, false>", "decode_ws_kernel<2, false, true>"},
       {"decode_ws_kernel<2, true, false>", "decode_ws_kernel<2, true, true>"}},
      {{"decode_ws_kernel<4, false, false>", "decode_ws_kernel<4, false, true>"},
       {"decode_ws_kernel<4, true, false>", "decode_ws_kernel<4, true, true>"}}};
  const int rb = decode_row_blocks_per_wg(h_kv > 1 ? M / h_kv : M);
  return names[rb == 1 ? 0 : rb == 2 ? 1 : 2][kind == kDecodeF16 ? 1 : 0][h_kv > 1 ? 1 : 0];
}

hipError_t launch_decode(const DecodeArgs& a, int kind, hipStream_t stream) {
  switch (decode_row_blocks_per_wg(a.h_kv > 1 ? a.Mkv : a.M)) {
    case 1: return launch_decode_t<1>(a, kind, stream);
    case 2: return launch_decode_t<2>(a, kind, stream);
    default: return launch_decode_t<4>(a, kind, stream);
  }
}

template <int RB>
static hipError_t occupancy_t(int kind, int* n) {
  if (kind == kDecodeFp8Packed)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, decode_fp8ws_kernel<false>, kWsThreads, 0);
  if (kind == kDecodeFp8Indexed)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, decode_fp8ws_kernel<true>, kWsThreads, 0);
  // (the several-KV-head instantiations use the same registers and LDS)
  if (kind == kDecodeF16)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, decode_ws_kernel<RB, true, false>, kWsThreads, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, decode_ws_kernel<RB, false, false>, kWsThreads, 0);
}

template <int RB>
static const void* decode_fn_t(int kind, bool mkv) {
  if (kind == kDecodeFp8Packed) return reinterpret_cast<const void*>(decode_fp8ws_kernel<false>);
  if (kind == kDecodeFp8Indexed) return reinterpret_cast<const void*>(decode_fp8ws_kernel<true>);
  if (kind == kDecodeF16)
    return mkv ? reinterpret_cast<const void*>(decode_ws_kernel<RB, true, true>)
               : reinterpret_cast<const void*>(decode_ws_kernel<RB, true, false>);
  return mkv ? reinterpret_cast<const void*>(decode_ws_kernel<RB, false, true>)
             : reinterpret_cast<const void*>(decode_ws_kernel<RB, false, false>);
}

hipError_t decode_launch_info(const DecodeArgs& a, int kind, DecodeLaunchInfo* info) {
  const int rb = decode_row_blocks_per_wg(a.h_kv > 1 ? a.Mkv : a.M);
  const int MB = 16 * rb;
  const void* fn = rb == 1 ? decode_fn_t<1>(kind, a.h_kv > 1) : rb == 2 ? decode_fn_t<2>(kind, a.h_kv > 1)
                                                                        : decode_fn_t<4>(kind, a.h_kv > 1);
  info->name = decode_kernel_name(a.M, a.h_kv, kind);
  info->grid_x = a.num_parts;
  info->grid_y = a.h_kv > 1 ? a.h_kv * ((a.Mkv + MB - 1) / MB) : (a.M + MB - 1) / MB;
  info->block = kWsThreads;
  hipFuncAttributes attr;
  hipError_t e = hipFuncGetAttributes(&attr, fn);
  if (e != hipSuccess) return e;
  info->lds_bytes = (int)attr.sharedSizeBytes;
  info->vgprs = attr.numRegs;
  return decode_occupancy(kind, a.h_kv > 1 ? a.Mkv : a.M, &info->wgs_per_cu);
}

hipError_t decode_occupancy(int kind, int M, int* wgs_per_cu) {
  int n = 0;
  hipError_t e;
  switch (decode_row_blocks_per_wg(M)) {
    case 1: e = occupancy_t<1>(kind, &n); break;
    case 2: e = occupancy_t<2>(kind, &n); break;
    default: e = occupancy_t<4>(kind, &n); break;
  }
  *wgs_per_cu = n;
  return e;
}

// ------------------------------------------------------------------ combine
// One wave per (request, row); lane l owns output columns [8l, 8l+8).
template <bool F16>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ num_splits,
                                                      const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse, int M, int slots,
                                                      uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int r = blockIdx.x;
  const int rho = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (rho >= M) return;
  const int s0 = num_splits[r];
  const int S = num_splits[r + 1] - s0;
  if (S == 1) return;
  if (s0 < 0 || S < 0 || s0 + S > slots) {  // not scheduler output: never read out of range
    if (threadIdx.x == 0) atomicOr(&g_error_flags, kErrMeta);
    return;
  }
  uint16_t* orow = out + ((int64_t)r * M + rho) * kDV + 8 * l;
  const float* src0 = part_o + ((int64_t)s0 * M + rho) * kDV + 8 * l;
  const int64_t stride = (int64_t)M * kDV;
  // A split request has at least two pieces: the partial rows of the first two
  // are loaded together with the lse values rather than after the reductions,
  // which takes one dependent memory round trip off every wave.
  f32x4 pa0 = {0.f, 0.f, 0.f, 0.f}, pb0 = pa0, pa1 = pa0, pb1 = pa0;
  if (S >= 2) {
    pa0 = *reinterpret_cast<const f32x4*>(src0);
    pb0 = *reinterpret_cast<const f32x4*>(src0 + 4);
    pa1 = *reinterpret_cast<const f32x4*>(src0 + stride);
    pb1 = *reinterpret_cast<const f32x4*>(src0 + stride + 4);
  }
  // the split lse values, 64 at a time, one per lane: max and sum by wave
  // reductions (the first 64 stay in v0)
  const float v0 = l < S ? part_lse[(int64_t)(s0 + l) * M + rho] : -INFINITY;
  float mx = v0;
  for (int i0 = 64; i0 < S; i0 += 64) {
    const float v = i0 + l < S ? part_lse[(int64_t)(s0 + i0 + l) * M + rho] : -INFINITY;
    mx = fmaxf(mx, v);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (mx == -INFINITY) {  // no split saw a key (or no split at all)
    *reinterpret_cast<u32x4*>(orow) = u32x4{0u, 0u, 0u, 0u};
    if (l == 0) lse[(int64_t)r * M + rho] = -INFINITY;
    return;
  }
  float tot = expf(v0 - mx);
  for (int i0 = 64; i0 < S; i0 += 64) {
    const float v = i0 + l < S ? part_lse[(int64_t)(s0 + i0 + l) * M + rho] : -INFINITY;
    tot += expf(v - mx);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
  const float L = mx + logf(tot);
  // weighted sum of the partial rows in split order; lane l owns columns
  // [8l, 8l+8).  After the first two, four splits per step so that their loads
  // are in flight together.
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  int i = 0;
  if (S >= 2) {
    const float w0 = expf(__shfl(v0, 0, 64) - L), w1 = expf(__shfl(v0, 1, 64) - L);
    acc0 += w0 * pa0;
    acc1 += w0 * pb0;
    acc0 += w1 * pa1;
    acc1 += w1 * pb1;
    i = 2;
  }
  for (; i + 4 <= S; i += 4) {
    f32x4 a[4], b[4];
    float wgt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* src = src0 + (int64_t)(i + u) * stride;
      a[u] = *reinterpret_cast<const f32x4*>(src);
      b[u] = *reinterpret_cast<const f32x4*>(src + 4);
      wgt[u] = expf(part_lse[(int64_t)(s0 + i + u) * M + rho] - L);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc0 += wgt[u] * a[u];
      acc1 += wgt[u] * b[u];
    }
  }
  for (; i < S; ++i) {
    const float* src = src0 + (int64_t)i * stride;
    const float wgt = expf(part_lse[(int64_t)(s0 + i) * M + rho] - L);
    acc0 += wgt * *reinterpret_cast<const f32x4*>(src);
    acc1 += wgt * *reinterpret_cast<const f32x4*>(src + 4);
  }
  u32x4 pk;
  pk.x = pack2<F16>(acc0[0], acc0[1]);
  pk.y = pack2<F16>(acc0[2], acc0[3]);
  pk.z = pack2<F16>(acc1[0], acc1[1]);
  pk.w = pack2<F16>(acc1[2], acc1[3]);
  *reinterpret_cast<u32x4*>(orow) = pk;
  if (l == 0) lse[(int64_t)r * M + rho] = L;
}

// ------------------------------------------------------------------ pack
// One workgroup per (query row, 64-record tile); 16-B chunks, 41 per record.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ kcache, int64_t num_pages,
                                                   const int32_t* __restrict__ indices,
                                                   const int32_t* __restrict__ topk_length, int s_q, int cap,
                                                   uint8_t* __restrict__ ws) {
  constexpr int kChunksPerRec = kRecBytes / 16;  // 41
  const int row = blockIdx.x;                    // r * s_q + i
  const int tile = blockIdx.y;
  const int r = row / s_q;
  int n = topk_length[r];
  if (n < 0 || n > cap) {
    if (threadIdx.x == 0) atomicOr(&g_error_flags, kErrSeqlen);
    n = n < 0 ? 0 : cap;
  }
  const int32_t* idx = indices + (int64_t)row * cap + tile * kPage;
  uint8_t* dst = ws + ((int64_t)row * cap + (int64_t)tile * kPage) * kRecBytes;
  const int64_t limit = num_pages * kPage;
  for (int c = threadIdx.x; c < kPage * kChunksPerRec; c += 256) {
    const int k = c / kChunksPerRec;
    const int piece = c - k * kChunksPerRec;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (tile * kPage + k < n) {
      const int64_t id = idx[k];
      if (id >= 0 && id < limit) {
        v = *reinterpret_cast<const u32x4*>(kcache + id * kRecBytes + piece * 16);
      } else if (piece == 0) {
        atomicOr(&g_error_flags, kErrIndex);
      }
    }
    *reinterpret_cast<u32x4*>(dst + (int64_t)c * 16) = v;
  }
}

// Current-token patch: one wave per (row, 64-slot tile).  Lane l tests slot
// k = 64 tile + l of the row against the request's changed ids; the wave then
// copies each matching record (lanes 0..40 move its 41 16-byte chunks).  Only
// slots whose id matches are written, so the rest of the packed tile stays as
// the pack left it.
__global__ __launch_bounds__(64) void patch_kernel(const uint8_t* __restrict__ kcache, int64_t num_pages,
                                                   const int32_t* __restrict__ indices,
                                                   const int32_t* __restrict__ topk_length,
                                                   const int32_t* __restrict__ new_ids, int n_new, int s_q, int cap,
                                                   uint8_t* __restrict__ ws) {
  constexpr int kChunksPerRec = kRecBytes / 16;  // 41
  const int row = blockIdx.x;                    // r * s_q + i
  const int k = blockIdx.y * kPage + (int)threadIdx.x;
  const int r = row / s_q;
  int n = ld_const(topk_length, r);
  n = n < 0 ? 0 : (n > cap ? cap : n);  // the pack flags out-of-range lengths
  int id = -1;
  if (k < n) id = indices[(int64_t)row * cap + k];
  bool hit = false;
  if (id >= 0) {
    for (int j = 0; j < n_new; ++j) hit |= id == ld_const(new_ids, (int64_t)r * n_new + j);
  }
  uint64_t m = __ballot(hit);
  const int64_t limit = num_pages * kPage;
  while (m) {
    const int src_lane = __builtin_ctzll(m);
    m &= m - 1;
    const int sid = __builtin_amdgcn_readlane(id, src_lane);
    if (sid >= limit) {  // id outside the pool (the pack flagged and zero-filled it)
      if (threadIdx.x == 0) atomicOr(&g_error_flags, kErrIndex);
      continue;
    }
    const int kk = blockIdx.y * kPage + src_lane;
    if (threadIdx.x < kChunksPerRec) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(kcache + (int64_t)sid * kRecBytes + threadIdx.x * 16);
      *reinterpret_cast<u32x4*>(ws + ((int64_t)row * cap + kk) * kRecBytes + threadIdx.x * 16) = v;
    }
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_sched(const int32_t* lengths, int batch, int num_parts, int32_t* meta, int32_t* num_splits,
                        hipStream_t stream, bool request_local, bool split_limit) {
  if (request_local)
    hipLaunchKernelGGL(sched_kernel<true>, dim3(1), dim3(kSchedThreads), 0, stream, lengths, batch, num_parts, meta,
                       num_splits, split_limit ? 1 : 0);
  else
    hipLaunchKernelGGL(sched_kernel<false>, dim3(1), dim3(kSchedThreads), 0, stream, lengths, batch, num_parts, meta,
                       num_splits, split_limit ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_combine(const int32_t* num_splits, const float* part_o, const float* part_lse, int batch, int M,
                          int slots, bool out_f16, uint16_t* out, float* lse, hipStream_t stream) {
  dim3 grid(batch, (M + 3) / 4);
  if (out_f16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, stream, num_splits, part_o, part_lse, M, slots, out,
                       lse);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, stream, num_splits, part_o, part_lse, M, slots, out,
                       lse);
  return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* kcache, int64_t num_pages, const int32_t* indices, const int32_t* topk_length,
                       int batch, int s_q, int cap, uint8_t* ws, hipStream_t stream) {
  dim3 grid(batch * s_q, cap / kPage);
  hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, stream, kcache, num_pages, indices, topk_length, s_q, cap, ws);
  return hipGetLastError();
}

hipError_t launch_patch(const uint8_t* kcache, int64_t num_pages, const int32_t* indices, const int32_t* topk_length,
                        const int32_t* new_ids, int n_new, int batch, int s_q, int cap, uint8_t* ws,
                        hipStream_t stream) {
  dim3 grid(batch * s_q, cap / kPage);
  hipLaunchKernelGGL(patch_kernel, grid, dim3(64), 0, stream, kcache, num_pages, indices, topk_length, new_ids, n_new,
                     s_q, cap, ws);
  return hipGetLastError();
}

// ------------------------------------------------------------------ scratch for the entry point that allocates nothing
// Split partials of mla_decode_fwd_noalloc live here instead of in a caller
// workspace.  Each device holds its own copy of the array (at its own address)
// from the module load until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current and
// kept below; only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t read_and_clear_error_flags(int* flags, hipStream_t stream) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  int v = 0;
  e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_error_flags), sizeof(int), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  int zero = 0;
  e = hipMemcpyToSymbol(HIP_SYMBOL(g_error_flags), &zero, sizeof(int), 0, hipMemcpyHostToDevice);
  if (e != hipSuccess) return e;
  *flags = v;
  return hipSuccess;
}

}  // namespace mla
