// Dense MLA decode for 128 query rows per workgroup on MI355X (gfx950, CDNA4).
//
// Method: as in mla_kernels.hip -- softmax(scale * Q K^T) V over a paged KV
// cache with one 576-dim latent KV head shared by every query head, V = K[:, 0:512],
// split-K over workgroups with an online softmax, partials merged by the combine
// ("Add SM80 (Ampere/A100) dense MLA decode kernel", FlashMLA PR 183: Summary,
// Design, Test plan).  This kernel covers the shapes whose query rows per
// request (s_q * h_q) are 256 or more and a multiple of 128, with one KV head.
//
// Why a separate kernel: with 64 rows per workgroup, an h_q = 128 request is
// covered by two workgroups that each stream every KV tile through their own
// LDS ring, and most of a tile's cost (ring loads, LDS reads, barrier) is paid
// per workgroup, not per row.  Here one workgroup holds all 128 rows: each KV
// tile crosses HBM -> LDS once per request piece.
//
// gfx950 layout:
//   * 4 waves, one per SIMD, 512 registers each.  Wave w owns query rows
//     [32w, 32w + 32): their Q (576 bf16 per row) in 144 VGPRs as the B operand
//     of v_mfma_f32_32x32x16, and their fp32 output (32 rows x 512 columns) in
//     256 accumulation registers.
//   * QK^T as S^T (32 keys x 32 rows) = K Q^T: 36 k-steps of 16 dims, K the A
//     operand read from LDS (ds_read_b128), two accumulation chains.
//   * The MFMA output layout puts row j = lane % 32 of S^T in lanes j and j + 32,
//     16 keys each; that is exactly the B operand layout of the PV product
//     O^T (32 columns x 32 rows) += V^T P^T once the 32 keys are ordered to
//     match, so P stays in registers (rounded to bf16): no LDS round trip and
//     no hand-off between waves.  V^T comes from transposed LDS reads
//     (ds_read_b64_tr_b16) in that key order.
//   * Each lane's 256 output values all belong to its own query row, so the
//     online softmax (exp2 domain, lazy rescale when a tile's maximum exceeds
//     the reference by more than kRescaleThreshold) is per lane with no
//     exchange except the row max and sum across lanes j and j + 32.
//   * KV tiles of 32 keys (36,864 B) stream HBM -> LDS with global_load_lds
//     (no VGPR staging) through a 4-slot ring, 2 tiles in flight, one barrier
//     per tile.  16-B chunk c of key row k is stored at chunk c ^ swz(k), which
//     keeps both the K operand reads (32 rows x 16 B) and the transposed V reads
//     (4 rows x 32 B per 16 lanes) free of bank conflicts.
//   * The workgroups of a request's pieces are placed on one XCD (they read the
//     same Q rows, which then come from that XCD's L2).
#include "mla_internal.h"

#include <math.h>

#include <type_traits>

namespace mla {

// Violation flags raised by this translation unit's kernels (read and cleared
// together with the other kernels' flags; see mla_read_device_errors).
__device__ int g_error_flags_r128;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

// Page table, lengths and scheduler records are read through the constant
// address space so that they become scalar loads (a vector load would need a
// vmcnt wait, which also waits for every ring load in flight).
template <class T>
using const_ptr = const __attribute__((address_space(4))) T*;
template <class T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
  return ((const_ptr<T>)(p))[i];
}

constexpr int kThreads = 256;                         // 4 waves, one per SIMD
constexpr int kRowsPerWG = 128;                       // 32 per wave
constexpr int kTK = 32;                               // keys per tile
constexpr int kStages = 4;                            // ring slots
constexpr int kRowBytes = kDQK * 2;                   // 1152
constexpr int kTileBytes = kTK * kRowBytes;           // 36864
constexpr int kChunksPerRow = kRowBytes / 16;         // 72
constexpr int kLoadsPerWave = kTileBytes / 1024 / 4;  // 9 wave-wide 16-B loads per tile per wave
constexpr int kLdsBytes = kStages * kTileBytes;       // 147456
constexpr int kQkSteps = kDQK / 16;                   // 36
constexpr int kColBlocks = kDV / 32;                  // 16
constexpr float kRescaleThreshold = 8.0f;             // log2 units: p <= 2^8 between rescales
constexpr int kKDepth = 3;                            // K operand reads in flight
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

__device__ __forceinline__ void set_flag(int bit) { atomicOr(&g_error_flags_r128, bit); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Barrier that also makes this wave's LDS writes visible (the ring's loads are
// waited for with wait_vmcnt before it).
__device__ __forceinline__ void sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint64_t uniform_u64(uint64_t b) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// global_load_lds_dwordx4 (saddr form): lane i copies 16 bytes from base + voff
// to LDS at M0 + 16 i.  Inline asm so that the compiler assumes no pending LDS
// DMA (it would otherwise wait for it before every LDS read); the ring is
// waited for explicitly.  M0 is reserved by the compiler, so the asm restores
// it; the s_nop is the wait state an SALU write of M0 needs before LDS DMA.
__device__ __forceinline__ void load_lds16(uint64_t base, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "memory");
}

// Chunk swizzle of key row k: its 16-B chunk c lives at chunk c ^ swz(k).  The
// LDS serves 256 B per cycle (64 banks): 16 lanes of a 16-B read, 32 lanes of an
// 8-B read.  Rows are 1152 B = 72 chunks apart, so without a swizzle 16 rows at
// one chunk hit two bank groups.  The K operand reads (16 consecutive rows, one
// chunk each) need swz to take all 8 values on the even and on the odd rows of
// every 16; the transposed V reads (4 consecutive rows x 4 consecutive chunks
// per 32 lanes) need rows 4a, 4a+2 (and 4a+1, 4a+3) to land in different halves
// of a 128-B line.  swz = 2 b0 ^ 4 b1 ^ b2 ^ 2 b3 (b = key bits) does both,
// and is also conflict-free if only 128 B are served per cycle.
__device__ __forceinline__ uint32_t swz(int k) {
  return (uint32_t)((((k & 3) << 1) | ((k >> 2) & 1)) ^ (((k >> 3) & 1) << 1));
}

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// acc += a^T-layout product into accumulation registers (AGPRs).  The PV
// product is issued through asm so that the output tile (256 registers per
// lane) is pinned to the AGPR file while the QK^T product (compiler builtin,
// VGPR form) keeps its accumulators in VGPRs: the compiler picks one MFMA form
// per function, and either choice alone does not fit.
template <bool F16>
__device__ __forceinline__ void mfma32_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
  if constexpr (F16)
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// the same with a zero accumulator (initialises acc)
template <bool F16>
__device__ __forceinline__ void mfma32_first(f32x16& acc, bf16x8 a, bf16x8 b) {
  if constexpr (F16)
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}

// The compiler does not know that the asm above is an MFMA, so it cannot insert
// the wait states between an MFMA writing the output tile and a VALU reading or
// writing it.  This waits 24 cycles (more than the 32x32x16 product's result
// latency after issue) and, by naming every output register, stays ordered
// between the MFMAs and those VALU accesses.
__device__ __forceinline__ void acc_fence(f32x16 (&o)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]),
                 "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]),
                 "+a"(o[15]));
}

// f(integral_constant<int, I>) for I = B, ..., E - 1, fully unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// One output register read into a VGPR, in program order with the other
// volatile asm: the epilogue drains the tile block by block instead of copying
// all 256 registers out at once.
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// two floats -> two 16-bit values (round to nearest even), a in the low half
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

__device__ __forceinline__ bf16x8 lds_read_b128(const LDS_AS uint8_t* p) {
  return *reinterpret_cast<const LDS_AS bf16x8*>(p);
}

// Transposed 4 x 16 read: in each 16-lane group, lanes 4r..4r+3 address the 16
// consecutive 16-bit values of row r (4 each); lane i receives column i of rows
// 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const LDS_AS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<LDS_AS bf16x4*>(const_cast<LDS_AS uint8_t*>(p)));
}

// max(v[l], v[l ^ 32]) in one asm block (v_permlane32_swap exchanges the two
// halves of the wave; with both operands equal, the pair returned is
// {v[l], v[l ^ 32]}).  The s_nop covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ float rowmax_pair(float v) {
  float b = v;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_max_f32 %0, %0, %1" : "+v"(v), "+v"(b));
  return v;
}
__device__ __forceinline__ float rowsum_pair(float v) {
  float b = v;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_add_f32 %0, %0, %1" : "+v"(v), "+v"(b));
  return v;
}

// The HBM -> LDS ring.  Load qi = w + 4j (j < 9) of a tile fills LDS chunks
// [64 qi, 64 qi + 64), i.e. lane l fills chunk position p = (64 qi + l) % 72 of
// key row k = (64 qi + l) / 72 with logical chunk p ^ swz(k).  As 72 is a
// multiple of 8, its source offset in the tile is 1024 qi + 16 ((l & 56) |
// ((l ^ swz(k)) & 7)): the 1024 qi part goes into the wave-uniform base, the 3
// lane bits of each of the 9 loads share one register.
struct Ring {
  uint32_t bits, l56;
  __device__ void init(int w, int l) {
    bits = 0;
    l56 = 16u * (uint32_t)(l & 56);
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const int qi = w + 4 * j;
      const int k = (qi * 64 + l) / kChunksPerRow;
      bits |= ((uint32_t)(l ^ swz(k)) & 7u) << (3 * j);
    }
  }
  // This wave's 9 loads of the tile of keys [key0, key0 + 32) of page `page`
  // into the ring slot `slot`.
  __device__ void issue(const DecodeArgs& a, int page, int key0, LDS_AS uint8_t* slot, int w) const {
    uint32_t pg = (uint32_t)__builtin_amdgcn_readfirstlane(page);
    const uint32_t np = a.num_pages < (int64_t)INT32_MAX ? (uint32_t)a.num_pages : (uint32_t)INT32_MAX;
    if (pg >= np) {  // a negative id wraps above any pool size
      if ((threadIdx.x & 63) == 0) set_flag(kErrPage);
      pg = 0;  // stay in bounds; the output of this request is undefined
    }
    const uint64_t src = uniform_u64((uint64_t)(uintptr_t)a.kv + (uint64_t)pg * (uint32_t)(kPage * kRowBytes) +
                                     (uint32_t)((key0 & 63) * kRowBytes));
    const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)slot);
    // opaque here: otherwise the compiler keeps all nine offsets live across
    // the tile loop instead of extracting them from one register at each use
    uint32_t b = bits;
    asm volatile("" : "+v"(b));
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const int qi = w + 4 * j;
      const uint32_t voff = l56 + 16u * ((b >> (3 * j)) & 7u);
      load_lds16(src + (uint64_t)(qi * 1024), voff, lds + (uint32_t)(qi * 1024));
    }
  }
};

template <bool F16>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_r128_kernel(
    DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[kLdsBytes];
  LDS_AS uint8_t* smem = (LDS_AS uint8_t*)(smem_raw);  // C-style: generic -> LDS address space

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, h = l >> 5, lr = l & 31;
  // Parts of one request are consecutive; workgroup b runs on XCD b % 8, so
  // part (b % 8) * (G / 8) + b / 8 keeps consecutive parts on one XCD.
  const int G = (int)gridDim.x, bx = (int)blockIdx.x;
  const int part = (G & 7) == 0 ? (bx & 7) * (G >> 3) + (bx >> 3) : bx;
  const int rbk = (int)blockIdx.y;

  const int begin_req = ld_const(a.sched_meta, part * 8 + 0);
  if (begin_req < 0) return;
  const int begin_blk = ld_const(a.sched_meta, part * 8 + 1);
  const int end_req = ld_const(a.sched_meta, part * 8 + 2);
  const int end_blk = ld_const(a.sched_meta, part * 8 + 3);
  const int begin_split = ld_const(a.sched_meta, part * 8 + 4);
  if (begin_req >= a.batch || end_req >= a.batch || end_req < begin_req) {  // not a scheduler record
    if (tid == 0) set_flag(kErrMeta);
    return;
  }

  Ring ring;
  ring.init(w, l);
  // K operand of k-step s: key row lr, dims [16 s + 8 h, +8), i.e. logical chunk
  // 2 s + h = 8 (s >> 2) + (2 (s & 3) + h), stored at 8 (s >> 2) + ((2 (s & 3) + h) ^ swz(lr)).
  uint32_t kb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kb[i] = (uint32_t)(lr * kRowBytes) + 16u * ((uint32_t)(2 * i + h) ^ swz(lr));
  // V^T operand of (column block cb, k-step ks): lane l receives column 32 cb + lr
  // of keys 16 ks + 4 h + {0..3} (read ri = 0) and 16 ks + 8 + 4 h + {0..3} (ri =
  // 1); it addresses row r = (l & 15) >> 2 of its 16-lane group, columns
  // 4 (l & 3) .. +3 of the group's 16-column span 32 cb + 16 ((l >> 4) & 1).
  // Those keys have swz = (2 r | h) ^ 2 ri, so the swizzled chunk is
  // 8 (cb >> 1) + ((4 (cb & 1)) ^ X(ri)) with X below; ks only moves whole rows.
  uint32_t vb[2][2];  // [cb & 1][ri]
  {
    const int gl = (l >> 4) & 1, rr = (l & 15) >> 2, jj = l & 3;
#pragma unroll
    for (int ri = 0; ri < 2; ++ri) {
      const uint32_t X = (uint32_t)((2 * gl + (jj >> 1)) ^ ((rr << 1) | h) ^ (2 * ri));
#pragma unroll
      for (int cp = 0; cp < 2; ++cp)
        vb[cp][ri] = (uint32_t)((4 * h + rr) * kRowBytes) + 16u * ((uint32_t)(4 * cp) ^ X) + 8u * (uint32_t)(jj & 1);
    }
  }

  const int row = rbk * kRowsPerWG + 32 * w + lr;  // this lane's query row in the request (s * h_q + head)
  const int tok = row / a.h_q;

  for (int r = begin_req; r <= end_req; ++r) {
    int seqlen = ld_const(a.seqlens, r);
    if (seqlen < 0 || seqlen > a.max_pages * kPage) {
      if (tid == 0) set_flag(kErrSeqlen);
      seqlen = seqlen < 0 ? 0 : a.max_pages * kPage;
    }
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
    if (nsplit > 1 && (slot < 0 || slot >= a.slots)) {  // inconsistent metadata: never write out of range
      if (tid == 0) set_flag(kErrMeta);
      continue;
    }
    // keys this row may see in the piece: [t0, lim)
    // (the limit grows with the token index, so the wave's smallest one is that
    // of its first row's token: a scalar)
    int lim = t1, lim_min = t1;
    if (a.causal) {
      lim = min(lim, min(max(seqlen - a.s_q + tok + 1, 0), seqlen));
      const int tok0 = (rbk * kRowsPerWG + 32 * w) / a.h_q;
      lim_min = min(lim_min, min(max(seqlen - a.s_q + tok0 + 1, 0), seqlen));
    }

    auto page_of = [&](int t) -> int {
      return ld_const(a.block_table, (int64_t)r * a.max_pages + ((t0 + t * kTK) >> 6));
    };
    auto slot_addr = [&](int t) -> LDS_AS uint8_t* { return smem + (t & 3) * kTileBytes; };
    // rows [nvalid, 32) of a partial tile: zero them (all 1152 bytes) so that
    // 0 * (whatever the page holds past the sequence) cannot reach PV
    auto zero_tail = [&](int t) {
      const int nvalid = min(kTK, t1 - (t0 + t * kTK));
      if (nvalid < kTK) {
        LDS_AS uint8_t* base = slot_addr(t);
        for (int idx = tid; idx < (kTK - nvalid) * kChunksPerRow; idx += kThreads)
          *reinterpret_cast<LDS_AS u32x4*>(base + nvalid * kRowBytes + 16 * idx) = u32x4{0u, 0u, 0u, 0u};
      }
    };

    // ---- prologue: tiles 0..2 into the ring, then Q (its wait covers them all)
    int pg_next = 0;
#pragma unroll
    for (int t = 0; t < 3; ++t)
      if (t < ntile) ring.issue(a, page_of(t), t0 + t * kTK, slot_addr(t), w);
    if (3 < ntile) pg_next = page_of(3);
    bf16x8 q[kQkSteps];
    {
      const uint16_t* qrow = a.q + ((int64_t)r * a.M + row) * kDQK + 8 * h;
#pragma unroll
      for (int s = 0; s < kQkSteps; ++s) q[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
    }
    wait_vmcnt<0>();
    sync_lds();  // tiles 0..2 resident

    f32x16 o[kColBlocks];  // set by the first PV product of the piece (zero accumulator)
    float m = -INFINITY, lsum = 0.f;

    // S^T of tile t into (sa, sb) (even and odd k-steps), with `hook(s)` after
    // the MFMAs of k-step s (the softmax of the previous tile runs there)
    f32x16 sa, sb;
    auto qk = [&](int t, auto hook) {
      const LDS_AS uint8_t* kt = slot_addr(t);
      bf16x8 kf[kKDepth];
      static_for<0, kKDepth - 1>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        kf[s] = lds_read_b128(kt + kb[s & 3] + 128 * (s >> 2));
      });
      static_for<0, kQkSteps>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        constexpr int sn = s + kKDepth - 1;
        if constexpr (sn < kQkSteps) kf[sn % kKDepth] = lds_read_b128(kt + kb[sn & 3] + 128 * (sn >> 2));
        if constexpr (s < 2)  // the first k-step of each chain starts from zero
          (s & 1 ? sb : sa) = mfma32<F16>(kf[s % kKDepth], q[s], f32x16{});
        else if constexpr (s & 1)
          sb = mfma32<F16>(kf[s % kKDepth], q[s], sb);
        else
          sa = mfma32<F16>(kf[s % kKDepth], q[s], sa);
        hook(s_c);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    if (ntile > 0) {
      zero_tail(0);
      qk(0, [](auto) {});
    }

    // ---- main loop: iteration t = softmax(t) in the shadow of QK^T(t+1), then PV(t)
    float sc[16];                        // raw scores of tile t
    uint32_t pk[8];                      // P(t), two 16-bit values per word
    float mx = 0.f, a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, a4 = 0.f, nm = 0.f, ps0 = 0.f, ps1 = 0.f;
    bool upd = false;
    for (int t = 0; t < ntile; ++t) {
      // own loads of tile t+1 done (tile t+2 may still be in flight), then the
      // barrier: tile t+1 resident for every wave, and every wave done with
      // iteration t-1 (whose PV read the slot tile t+3 goes into)
      // (for t = 0 the prologue waited for tiles 0..2; its barrier then also
      // publishes the zeroed tail of tile 0)
      if (t > 0 && t + 1 < ntile) {
        if (t + 2 < ntile) wait_vmcnt<kLoadsPerWave>();
        else wait_vmcnt<0>();
      }
      sync_lds();
      if (t + 3 < ntile) ring.issue(a, pg_next, t0 + (t + 3) * kTK, slot_addr(t + 3), w);
      if (t + 4 < ntile) pg_next = page_of(t + 4);
      if (t + 1 < ntile) zero_tail(t + 1);

      const int key0 = t0 + t * kTK;
      const bool need_mask = key0 + kTK > lim_min;
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[v] = sa[v] + sb[v];
      // Softmax of tile t in steps, one per QK k-step of tile t+1.  Lane l holds
      // scores of row lr for keys 8 (v >> 2) + 4 h + (v & 3), v < 16.
      float alpha = 1.f;
      bool rescale = false;
      auto sm_step = [&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        if constexpr (s == 0) {
          if (need_mask) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (key0 + 8 * (v >> 2) + 4 * h + (v & 3) >= lim) sc[v] = -INFINITY;
          }
        } else if constexpr (s == 1) {
          a0 = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
          a1 = fmaxf(fmaxf(sc[3], sc[4]), sc[5]);
        } else if constexpr (s == 2) {
          a2 = fmaxf(fmaxf(sc[6], sc[7]), sc[8]);
          a3 = fmaxf(fmaxf(sc[9], sc[10]), sc[11]);
        } else if constexpr (s == 3) {
          a4 = fmaxf(fmaxf(sc[12], sc[13]), sc[14]);
          a0 = fmaxf(fmaxf(a0, a1), sc[15]);
        } else if constexpr (s == 4) {
          a2 = fmaxf(fmaxf(a2, a3), a4);
        } else if constexpr (s == 5) {
          mx = fmaxf(a0, a2);
        } else if constexpr (s == 6) {
          mx = rowmax_pair(mx);
        } else if constexpr (s == 7) {
          mx *= a.scale_log2;
        } else if constexpr (s == 8) {
          upd = mx > m + kRescaleThreshold;
        } else if constexpr (s == 9) {
          // the reference maximum moves: the row's sum now, its output after
          // this phase (before PV reads it)
          const float mnew = upd ? mx : m;
          alpha = upd ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;  // 0 when m was -inf
          m = mnew;
          lsum *= alpha;
        } else if constexpr (s == 10) {
          nm = (m == -INFINITY) ? 0.f : -m;
          rescale = __builtin_amdgcn_ballot_w64(upd) != 0;
        } else if constexpr (s >= 11 && s <= 14) {
          constexpr int i = s - 11;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * i + 0], a.scale_log2, nm));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * i + 1], a.scale_log2, nm));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * i + 2], a.scale_log2, nm));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * i + 3], a.scale_log2, nm));
          pk[2 * i] = pack2<F16>(p0, p1);
          pk[2 * i + 1] = pack2<F16>(p2, p3);
          if constexpr (i & 1) ps1 += (p0 + p1) + (p2 + p3);
          else ps0 += (p0 + p1) + (p2 + p3);
        } else if constexpr (s == 15) {
          lsum += ps0 + ps1;
          ps0 = ps1 = 0.f;
        }
      };
      if (t + 1 < ntile) {
        qk(t + 1, sm_step);
      } else {
        static_for<0, 16>(sm_step);
      }
      if (rescale && t > 0) {  // rare: a row's maximum rose by more than the threshold (O is set from tile 0 on)
        acc_fence(o);
        // one 16-register block at a time: each is copied to VGPRs, scaled and
        // pinned back into its AGPRs before the next is touched
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb) {
          o[cb] *= alpha;
          asm volatile("" : "+a"(o[cb]));
        }
        acc_fence(o);
      }

      // PV(t): O^T[cb] += V^T(cb, ks) P^T(ks); k-step ks covers keys 16 ks + {4h..4h+3,
      // 8+4h..8+4h+3} in lane half h, i.e. P values v = 8 ks .. 8 ks + 7 of the lane
      auto pv = [&](auto first_c) {
        constexpr bool kFirst = decltype(first_c)::value;  // tile 0 of the piece: O starts from zero
        const LDS_AS uint8_t* vt = slot_addr(t);
        auto vread = [&](int ks, int cb) -> bf16x8 {
          const LDS_AS uint8_t* base = vt + 128 * (cb >> 1) + ks * 16 * kRowBytes;
          const bf16x4 lo = lds_read_tr16(base + vb[cb & 1][0]);
          const bf16x4 hi = lds_read_tr16(base + vb[cb & 1][1] + 8 * kRowBytes);
          return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        constexpr int kVDepth = 3;
        bf16x8 vf[kVDepth];
#pragma unroll
        for (int i = 0; i < kVDepth - 1; ++i) vf[i] = vread(i / kColBlocks, i % kColBlocks);
#pragma unroll
        for (int i = 0; i < 2 * kColBlocks; ++i) {
          const int ks = i / kColBlocks, cb = i % kColBlocks;
          const int in = i + kVDepth - 1;
          if (in < 2 * kColBlocks) vf[in % kVDepth] = vread(in / kColBlocks, in % kColBlocks);
          const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]});
          if (kFirst && ks == 0) mfma32_first<F16>(o[cb], vf[i % kVDepth], pb);
          else mfma32_acc<F16>(o[cb], vf[i % kVDepth], pb);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (t == 0) pv(std::true_type{});
      else pv(std::false_type{});
    }

    // ---- epilogue: row sums, lse, output (or the split partial)
    acc_fence(o);
    const float lt = rowsum_pair(lsum);
    int gr = row;
    asm volatile("" : "+v"(gr));  // keeps the row addresses from being hoisted out of the request loop
    if (h == 0) {
      const float lse = lt > 0.f ? (m + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
      if (nsplit == 1) a.lse[(int64_t)r * a.M + gr] = lse;
      else a.part_lse[(int64_t)slot * a.M + gr] = lse;
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // lane l holds columns 32 cb + 8 g + 4 h + {0..3} of its row in o[cb][4 g .. 4 g + 3]
    // (nothing attended in the piece: O was never set, write zeros)
    auto val = [&](int cb, int v) -> float { return acc_read(o[cb][v]) * inv; };
    if (ntile == 0) {
      if (nsplit == 1) {
        uint16_t* orow = a.out + ((int64_t)r * a.M + gr) * kDV + 4 * h;
        for (int c = 0; c < kDV / 8; ++c) *reinterpret_cast<u32x2*>(orow + 8 * c) = u32x2{0u, 0u};
      } else {
        float* prow = a.part_o + ((int64_t)slot * a.M + gr) * kDV + 4 * h;
        for (int c = 0; c < kDV / 8; ++c) *reinterpret_cast<u32x4*>(prow + 8 * c) = u32x4{0u, 0u, 0u, 0u};
      }
    } else if (nsplit == 1) {
      uint16_t* orow = a.out + ((int64_t)r * a.M + gr) * kDV + 4 * h;
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int v = 4 * g4;
          const float x0 = val(cb, v), x1 = val(cb, v + 1), x2 = val(cb, v + 2), x3 = val(cb, v + 3);
          *reinterpret_cast<u32x2*>(orow + 32 * cb + 8 * g4) = u32x2{pack2<F16>(x0, x1), pack2<F16>(x2, x3)};
        }
    } else {
      float* prow = a.part_o + ((int64_t)slot * a.M + gr) * kDV + 4 * h;
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int v = 4 * g4;
          const float x0 = val(cb, v), x1 = val(cb, v + 1), x2 = val(cb, v + 2), x3 = val(cb, v + 3);
          *reinterpret_cast<f32x4*>(prow + 32 * cb + 8 * g4) = f32x4{x0, x1, x2, x3};
        }
    }
    wait_vmcnt<0>();  // the next request's ring loads must not overtake these stores in the count
    sync_lds();       // every wave done with the ring before the next request refills it
  }
}

}  // namespace

// Used for 256 or more rows per request (a multiple of 128): there the MFMA work
// per KV byte is high (several query tokens x 128 heads) and sharing each tile
// among 128 rows wins.  Measured against the 64-row kernel, decode + combine on
// one MI355X: b=16, s_q=2, h_q=128, sk=16384 (causal): 161.9 us against 167.9;
// at 128 rows per request it loses (b=64, h_q=128, sk=4096: 105 against 100 us;
// b=1, sk=4096: 39 against 29 us), because covering the chip then takes four
// pieces per request instead of two and the extra partials and prologues cost
// more than the shared tiles save.
bool decode_r128_shape(int M, int h_kv, int kind) {
  return (kind == kDecodeBf16 || kind == kDecodeF16) && h_kv == 1 && M >= 2 * kRowsPerWG && M % kRowsPerWG == 0;
}

hipError_t launch_decode_r128(const DecodeArgs& a, int kind, hipStream_t stream) {
  dim3 grid(a.num_parts, a.M / kRowsPerWG);
  if (kind == kDecodeF16)
    hipLaunchKernelGGL(decode_r128_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_r128_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t decode_r128_occupancy(int kind, int* wgs_per_cu) {
  if (kind == kDecodeF16)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(wgs_per_cu, decode_r128_kernel<true>, kThreads, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(wgs_per_cu, decode_r128_kernel<false>, kThreads, 0);
}

hipError_t read_and_clear_error_flags_r128(int* flags) {
  int v = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_error_flags_r128), sizeof(int), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  int zero = 0;
  e = hipMemcpyToSymbol(HIP_SYMBOL(g_error_flags_r128), &zero, sizeof(int), 0, hipMemcpyHostToDevice);
  *flags = v;
  return e;
}

}  // namespace mla
