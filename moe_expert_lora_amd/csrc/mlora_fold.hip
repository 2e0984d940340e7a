// Device folds of libmlora.so for gfx950 (MI355X): the gather (decode) and
// grouped (prefill) MoE expert-LoRA folds of the "moe_lora_grouped" module
// index page, items moe_lora_gather_bgmv and moe_lora_grouped_down:
//
//     base_out[row] += scale_e * ((x[token(row)] @ A_e^T) @ B_e^T)
//
// Design:
//  * Each call runs as one kernel, or, for large calls given a workspace, as
//    a shrink kernel that writes H (scaled hi/lo bf16 for the grouped fold,
//    fp32 partial sums over k ranges for the gather fold) and an expand
//    kernel that reads it back. The shrink H = X A_e^T and the expand
//    base + s H B_e^T both run on bf16 MFMA (v_mfma_f32_16x16x32_bf16), with
//    fp32 accumulation.
//  * Shrink, transposed: D[rank][row] = A_e[rank,:] . x[row,:]. The 4 waves
//    split k_in; partial sums meet in LDS and are added in a fixed order.
//    A rank permutation makes each lane end up holding 4*NB consecutive ranks
//    of one row, which is exactly the operand layout the expand needs (also
//    the layout H takes in the workspace).
//  * H is scaled by scale_e and split into hi + lo bf16 halves, so the expand
//    MFMA sees H to ~16 mantissa bits (rounding H to one bf16 alone would use
//    most of the error budget that the final bf16 store leaves).
//  * Expand, transposed: D[col][row] = B_e[col,:] . H'[:,row] with
//    K' = 2*max_rank (hi then lo). A column permutation gives each lane a run
//    of 8 consecutive output columns of one row. The grouped expand kernel
//    moves the fp32 deltas through the wave's LDS so that base_out is read
//    and written row-contiguously; the other kernels access base_out in the
//    MFMA layout (16 rows x 64 bytes per instruction).
//  * Every operand moves through raw buffer loads/stores: 32-bit offsets, and
//    a masked lane simply uses an offset past the buffer (its load returns 0,
//    its store is dropped), so no access needs a branch. Loads are issued in
//    batches and consumed after one wait; code that needs an exact wait count
//    stays straight-line.
//  * Gather rows are grouped by expert on the device: each workgroup scans a
//    slice of `indices` for its expert, so each A_e / B_e is streamed from HBM
//    once per workgroup group and reused across that expert's rows.
//  * Grouped rows come in tiles; a tile that straddles expert spans is folded
//    one span (or, in the shrink kernel, two spans) at a time.
//  * Workgroup ids are mapped so that consecutive work units (the splits of
//    one expert, or neighbouring row tiles) run on the same XCD and share its
//    L2. The grouped expand is the exception: its units go to the XCDs in
//    turn (see there).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "mlora.h"
#include "mlora_internal.h"

namespace mlora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileRows = MLORA_MLG_M_TILE;
constexpr int kColStep = 32;     // output columns per expand step of one wave
constexpr int kScanMax = 2048;   // gather rows scanned by one workgroup

// The t-th k step (or column step) of wave `wave` in a workgroup: adjacent
// steps go in pairs, the pairs dealt to the waves in turn (wave w takes 2w,
// 2w+1, 2w+2*kWaves, 2w+2*kWaves+1, ...). Both 64-byte halves of a 128-byte
// line of an A_e row, an x row or a base_out row are then requested by one
// wave back to back: measured 5-9% faster streaming than steps dealt one at
// a time. A bijection from (wave, t) onto the steps; increasing in t.
__device__ __forceinline__ int wave_step(int wave, int t) {
  return 2 * wave + (t & 1) + 2 * kWaves * (t >> 1);
}

// The t-th of `n` column steps of wave `wave`: in pairs (as wave_step) when
// the pairs come out even over the waves, else one at a time (wave w takes w,
// w+kWaves, ...), so that no wave takes two steps more than another. Which
// wave writes a column changes no result.
__device__ __forceinline__ int col_step(int wave, int t, int n) {
  return n % (2 * kWaves) == 0 ? wave_step(wave, t) : wave + kWaves * t;
}
constexpr int kXcds = 8;
// Largest buffer one resource may describe; every offset stays below it.
constexpr uint32_t kMaxBufBytes = 0xFFFFFF00u;
// An offset past every buffer: a load there returns 0, a store is dropped.
constexpr uint32_t kOOB = 0xFFFFFFF0u;

static_assert(kTileRows == 64, "grouped tiles are 64 rows (4 row blocks of 16)");

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 in one word (low half = a), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// bf16 pair word -> its low / high value as fp32 (exact).
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// n / d for 0 <= n < 2^31 and d >= 1, with magic = floor((2^32 - 1) / d): the
// high product is the quotient or one less, and one step corrects it.
__device__ __forceinline__ uint32_t udiv(uint32_t n, uint32_t d, uint32_t magic) {
  uint32_t q = __umulhi(n, magic);
  if ((q + 1) * d <= n) q += 1;
  return q;
}

// buffer resource (gfx9 family descriptor word 3: raw, 32-bit data format)
__device__ __forceinline__ rsrc_t make_buf(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 bld8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t bld4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bld2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ void bst16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, 0);
}

// Non-temporal 16-byte access (base_out is read once and written once).
constexpr int kNT = 2;
__device__ __forceinline__ u32x4 bld16_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT));
}
__device__ __forceinline__ void bst16_nt(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, kNT);
}

__device__ __forceinline__ bf16x8 as_bf(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// A value every lane of the wave holds, moved to scalar registers. Buffer
// descriptors built from scalar values need no per-lane handling, while one
// built from a vector register makes the compiler loop over lanes per access.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
// The 64-bit value (lo, hi) of lane `lane` (wave-uniform) as a scalar. The
// builtin returns int: each half goes back through uint32_t, so the low word
// is never sign-extended into the high one.
__device__ __forceinline__ uint64_t lane_u64(uint32_t lo, uint32_t hi, int lane) {
  const uint32_t l = (uint32_t)__builtin_amdgcn_readlane((int)lo, lane);
  const uint32_t h = (uint32_t)__builtin_amdgcn_readlane((int)hi, lane);
  return ((uint64_t)h << 32) | l;
}
__device__ __forceinline__ float uniform_f32(float v) {
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Appends (v0, v1) of the lanes whose `pred` is set to LDS lists, in one LDS
// atomic per wave. Order across waves is unspecified; nothing downstream
// depends on it (every row is computed independently).
__device__ __forceinline__ void wave_append(bool pred, int v0, int v1, int* cnt, int* l0,
                                            int* l1, int cap) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  const int pop = __popcll(mask);
  int base = 0;
  if (lane == leader) base = atomicAdd(cnt, pop);
  base = __shfl(base, leader);
  const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
  if (pred && base + rank < cap) {
    l0[base + rank] = v0;
    l1[base + rank] = v1;
  }
}

// Workgroup barrier that orders LDS only. Every cross-wave exchange in these
// kernels goes through LDS (each base_out element is read and written by one
// lane), so outstanding global loads, such as prefetches, stay in flight
// across it instead of being drained.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// the per-expert tile engine
// ---------------------------------------------------------------------------

// Buffers of one fold_rows call.
struct Bufs {
  rsrc_t x;    // [n_tokens, K]
  rsrc_t a;    // A_e [R, K]
  rsrc_t b;    // B_e [N, R]
  rsrc_t out;  // base_out rows addressed by this call
};

// Expand operands. After the shrink, lane group g of each row holds the 4*NB
// consecutive ranks g*4NB .. g*4NB+4NB-1 (the rank permutation of the shrink
// puts them there). The expand contracts over ranks in chunks: a chunk is the
// 8 ranks (NB >= 2, one 16x16x32 MFMA) or 4 ranks (NB == 1, one 16x16x16
// MFMA) a lane group holds at one position, so a lane's B_e words load
// straight into an MFMA operand with no rearrangement, and hi and lo of H
// each take one MFMA per chunk.
template <int NB>
struct Chunk {
  static constexpr int kRanks = NB == 1 ? 4 : 8;       // ranks per lane per chunk
  static constexpr int kCount = 4 * NB / kRanks;       // chunks per lane
  static constexpr int kWords = kRanks / 2;            // bf16 pairs per chunk
};

// B_e fragment of one expand step: for each of the 2 column blocks and each
// rank chunk, the lane's kRanks bf16 of one B_e row.
template <int NB>
struct BFrag {
  uint32_t w[2][Chunk<NB>::kCount][Chunk<NB>::kWords];
};

// Output column (relative to the step start) of MFMA row `mi` in column block
// `cb`: lane group g of the result then holds the 8 consecutive columns
// 8g .. 8g+7 of its row (4 from each block).
__device__ __forceinline__ int col_of(int cb, int mi) {
  return (mi >> 2) * 8 + cb * 4 + (mi & 3);
}

// B_e fragments are requested ahead of a block's base_out rows, so that the
// expand's MFMAs wait only for them (waits count loads in issue order).
// FULL_R: the rank is a multiple of the chunk (whole_chunks), so each lane's
// chunk of a B_e row lies wholly inside the row (one 8- or 16-byte load, its
// offset a multiple of the load size) or wholly past the rank (not read, 0).
// Otherwise the words are put together from 16-bit loads, and the compiler
// waits for those right away; there the callers request base_out first.
template <int NB, bool FULL_R>
__device__ __forceinline__ void load_bfrag(BFrag<NB>& f, rsrc_t rb, int R, int c0, int n_hi,
                                           int li, int g) {
  constexpr int CR = Chunk<NB>::kRanks, CC = Chunk<NB>::kCount, CW = Chunk<NB>::kWords;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int col = c0 + col_of(cb, li);
    const bool ok = col < n_hi;
#pragma unroll
    for (int q = 0; q < CC; ++q) {
      const int r0 = g * 4 * NB + q * CR;  // first rank of the chunk
      const uint32_t base = (uint32_t)(col * R + r0) * 2u;
      if constexpr (FULL_R) {
        const bool in = ok && r0 < R;
        if constexpr (CW == 2) {
          const u32x2 v = bld8(rb, in ? base : kOOB);
          f.w[cb][q][0] = v.x;
          f.w[cb][q][1] = v.y;
        } else {
          const u32x4 v = bld16(rb, in ? base : kOOB);
          f.w[cb][q][0] = v.x;
          f.w[cb][q][1] = v.y;
          f.w[cb][q][2] = v.z;
          f.w[cb][q][3] = v.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < CW; ++j) {
          const int r = r0 + 2 * j;
          const uint32_t lo = bld2(rb, (ok && r < R) ? base + 4u * j : kOOB);
          const uint32_t hi = bld2(rb, (ok && r + 1 < R) ? base + 4u * j + 2u : kOOB);
          f.w[cb][q][j] = (lo & 0xffffu) | (hi << 16);
        }
      }
    }
  }
}

// H operands of one row block: hi and lo halves of scale * H, per chunk.
template <int NB>
struct HOp {
  uint32_t hi[Chunk<NB>::kCount][Chunk<NB>::kWords];
  uint32_t lo[Chunk<NB>::kCount][Chunk<NB>::kWords];
};

// One chunk's MFMA: 16x16x32 for 8 ranks, 16x16x16 for 4.
template <int CW>
__device__ __forceinline__ f32x4 mfma_chunk(const uint32_t (&a)[CW], const uint32_t (&b)[CW],
                                            f32x4 c) {
  if constexpr (CW == 4) {
    return mfma16x16x32(as_bf(u32x4{a[0], a[1], a[2], a[3]}),
                        as_bf(u32x4{b[0], b[1], b[2], b[3]}), c);
  } else {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(s16x4, u32x2{a[0], a[1]}), __builtin_bit_cast(s16x4, u32x2{b[0], b[1]}),
        c, 0, 0, 0);
  }
}

// Loads are issued in batches: the k steps of one shrink batch (A_e and x
// fragments) or the column steps of one expand batch (B_e, then base_out
// fragments) are requested together and consumed after a single wait. Two
// batch buffers alternate, so the next batch is in flight while the current
// one is multiplied: a wave always has memory requests outstanding. The batch
// sizes bound the VGPRs a buffer holds.
#ifndef MLORA_BATCH_VGPRS
#define MLORA_BATCH_VGPRS 40
#endif

constexpr int cclamp(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

template <int NB, int MB>
struct Batch {
  static constexpr int US = cclamp(MLORA_BATCH_VGPRS / (4 * (NB + MB)), 1, 8);
  static constexpr int UE = cclamp(MLORA_BATCH_VGPRS / (4 * (NB + MB)), 1, 8);
};

template <int NB, int MB, int US>
struct ShrinkBatch {
  u32x4 a[US][NB];
  u32x4 x[US][MB];
};

template <int NB, int MB, int UE>
struct ExpandBatch {
  BFrag<NB> b[UE];
  u32x4 o[UE][MB];
};

// Per-lane row state of one fold_rows call.
template <int MB>
struct Rows {
  uint32_t xoff[MB];  // byte offset of the row's token in x
  uint32_t ooff[MB];  // byte offset of the row in base_out
  bool valid[MB];
};

template <int NB, int MB, int US>
__device__ __forceinline__ void load_shrink(ShrinkBatch<NB, MB, US>& sb, const Bufs& bf, int K,
                                            int R, const Rows<MB>& rw, int s_base, int wave,
                                            int t0, int nks, int li, int g) {
#pragma unroll
  for (int u = 0; u < US; ++u) {
    const int s = s_base + wave_step(wave, t0 + u);
    const int k0 = s * 32 + g * 8;
    const bool kin = s < nks && k0 < K;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int rank = (li >> 2) * 4 * NB + 4 * b + (li & 3);
      sb.a[u][b] = bld16(bf.a, (kin && rank < R) ? (uint32_t)(rank * K + k0) * 2u : kOOB);
    }
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
      sb.x[u][rb] = bld16(bf.x, (kin && rw.valid[rb]) ? rw.xoff[rb] + 2u * k0 : kOOB);
  }
}

template <int NB, int MB, int US>
__device__ __forceinline__ void mma_shrink(f32x4 (&hacc)[MB][NB],
                                           const ShrinkBatch<NB, MB, US>& sb, int nrb) {
#pragma unroll
  for (int u = 0; u < US; ++u) {
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      if (rb < nrb) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          hacc[rb][b] = mfma16x16x32(as_bf(sb.a[u][b]), as_bf(sb.x[u][rb]), hacc[rb][b]);
      }
    }
  }
}

template <int NB, int MB, int UE, bool FULL_R>
__device__ __forceinline__ void load_expand(ExpandBatch<NB, MB, UE>& eb, const Bufs& bf, int R,
                                            const Rows<MB>& rw, int wave, int t0, int ncs,
                                            int n_lo, int n_hi, int li, int g) {
  auto request_b = [&]() {
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int cs = col_step(wave, t0 + u, ncs);
      load_bfrag<NB, FULL_R>(eb.b[u], bf.b, R, n_lo + cs * kColStep, cs < ncs ? n_hi : 0, li, g);
    }
  };
  auto request_out = [&]() {
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int cs = col_step(wave, t0 + u, ncs);
      const int col = n_lo + cs * kColStep + 8 * g;
      const bool cok = cs < ncs && col < n_hi;
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
        eb.o[u][rb] = bld16_nt(bf.out, (rw.valid[rb] && cok) ? rw.ooff[rb] + 2u * col : kOOB);
    }
  };
  if constexpr (FULL_R) {
    request_b();
    request_out();
  } else {
    request_out();
    request_b();
  }
}

// delta = B_e . (hi + lo) for the batch's columns, added to base_out, stored.
template <int NB, int MB, int UE>
__device__ __forceinline__ void mma_store_expand(const ExpandBatch<NB, MB, UE>& eb,
                                                 const HOp<NB> (&hop)[MB], const Bufs& bf,
                                                 const Rows<MB>& rw, int nrb, int wave, int t0,
                                                 int ncs, int n_lo, int n_hi, int g) {
  constexpr int CC = Chunk<NB>::kCount;
#pragma unroll
  for (int u = 0; u < UE; ++u) {
    const int cs = col_step(wave, t0 + u, ncs);
    const int col = n_lo + cs * kColStep + 8 * g;
    const bool cok = cs < ncs && col < n_hi;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      if (rb < nrb) {
        f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < CC; ++q) {
          d0 = mfma_chunk(eb.b[u].w[0][q], hop[rb].hi[q], d0);
          d1 = mfma_chunk(eb.b[u].w[1][q], hop[rb].hi[q], d1);
          d0 = mfma_chunk(eb.b[u].w[0][q], hop[rb].lo[q], d0);
          d1 = mfma_chunk(eb.b[u].w[1][q], hop[rb].lo[q], d1);
        }
        const u32x4 bq = eb.o[u][rb];
        const uint32_t o0 = pack_bf16(lo_f(bq.x) + d0.x, hi_f(bq.x) + d0.y);
        const uint32_t o1 = pack_bf16(lo_f(bq.y) + d0.z, hi_f(bq.y) + d0.w);
        const uint32_t o2 = pack_bf16(lo_f(bq.z) + d1.x, hi_f(bq.z) + d1.y);
        const uint32_t o3 = pack_bf16(lo_f(bq.w) + d1.z, hi_f(bq.w) + d1.w);
        bst16_nt(bf.out, (rw.valid[rb] && cok) ? rw.ooff[rb] + 2u * col : kOOB,
              u32x4{o0, o1, o2, o3});
      }
    }
  }
}

// Shrink of up to MB row blocks over this wave's k steps in [s_begin, s_end):
// H[rank][row] for the k steps s_begin + wave_step(wave, t), t = 0, 1, ...
// (in increasing order).
template <int NB, int MB>
__device__ __forceinline__ void shrink_k(f32x4 (&hacc)[MB][NB], const Bufs& bf, int K, int R,
                                         const Rows<MB>& rw, int nrb, int wave, int li, int g,
                                         int s_begin = 0, int s_end = 1 << 30) {
  constexpr int US = Batch<NB, MB>::US;
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int b = 0; b < NB; ++b) hacc[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = min((K + 31) >> 5, s_end);
  // The next batch is requested before the current one is used, without a
  // condition: steps past the end load nothing (their offsets are out of
  // range), and straight-line code keeps the wait counts exact.
  // The scheduling barriers keep each batch's loads ahead of the MFMAs of the
  // batch before it (the scheduler would otherwise sink them below, and the
  // loop would wait for every load at its head).
  ShrinkBatch<NB, MB, US> s0b, s1b;
  int t0 = 0;
  load_shrink<NB, MB, US>(s0b, bf, K, R, rw, s_begin, wave, t0, nks, li, g);
  while (s_begin + wave_step(wave, t0) < nks) {
    const int t1 = t0 + US;
    load_shrink<NB, MB, US>(s1b, bf, K, R, rw, s_begin, wave, t1, nks, li, g);
    __builtin_amdgcn_sched_barrier(0);
    mma_shrink<NB, MB, US>(hacc, s0b, nrb);
    __builtin_amdgcn_sched_barrier(0);
    if (s_begin + wave_step(wave, t1) >= nks) break;
    const int t2 = t1 + US;
    load_shrink<NB, MB, US>(s0b, bf, K, R, rw, s_begin, wave, t2, nks, li, g);
    __builtin_amdgcn_sched_barrier(0);
    mma_shrink<NB, MB, US>(hacc, s1b, nrb);
    __builtin_amdgcn_sched_barrier(0);
    t0 = t2;
  }
}

// K-split reduction of the shrink through LDS, the partial sums of the waves
// added in a fixed order, then the hi / lo operands of scale * H for each row
// block. Every wave ends up with the operands of every row block. Contains a
// workgroup barrier: all threads call it with the same arguments.
template <int NB, int MB>
__device__ __forceinline__ void reduce_split(const f32x4 (&hacc)[MB][NB], float* s_part,
                                             float scale, int nrb, int wave, int lane,
                                             HOp<NB> (&hop)[MB]) {
  constexpr int HW = 4 * NB;  // ranks per lane
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    if (rb < nrb) {
      float* dst = s_part + ((size_t)(wave * MB + rb) * 64 + lane) * HW;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        *reinterpret_cast<f32x4*>(dst + 4 * b) = hacc[rb][b];
    }
  }
  lds_barrier();
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    if (rb < nrb) {
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        f32x4 h = *reinterpret_cast<const f32x4*>(
            s_part + ((size_t)(0 * MB + rb) * 64 + lane) * HW + 4 * s);
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
          h += *reinterpret_cast<const f32x4*>(
              s_part + ((size_t)(w * MB + rb) * 64 + lane) * HW + 4 * s);
        const f32x4 v = scale * h;
        const uint32_t hi01 = pack_bf16(v.x, v.y), hi23 = pack_bf16(v.z, v.w);
        const uint32_t lo01 = pack_bf16(v.x - lo_f(hi01), v.y - hi_f(hi01));
        const uint32_t lo23 = pack_bf16(v.z - lo_f(hi23), v.w - hi_f(hi23));
        // ranks 4s .. 4s+3 of this lane: chunk (4s) / kRanks, word offset inside it
        constexpr int CR = Chunk<NB>::kRanks;
        const int q = (4 * s) / CR, w0 = ((4 * s) % CR) / 2;
        hop[rb].hi[q][w0] = hi01;
        hop[rb].hi[q][w0 + 1] = hi23;
        hop[rb].lo[q][w0] = lo01;
        hop[rb].lo[q][w0 + 1] = lo23;
      }
    }
  }
}

// Folds rows 0..nrows-1 (nrows <= 16*MB) of one expert into columns
// [n_lo, n_hi) of base_out. Row m writes base_out row
// (s_row ? s_row[m] : row_base + m) of bf.out, from token s_tok[m]
// (negative: a dead row, neither read nor written).
// All threads of the workgroup must call it with the same arguments.
// Lane state of row blocks 0..MB-1 of a row list: rows 0..nrows-1, row m of
// base_out row (s_row ? s_row[m] : row_base + m), token s_tok[m] (negative:
// a dead row, neither read nor written).
// x_ld / out_ld: elements from one x / base_out row to the next.
template <int MB>
__device__ __forceinline__ Rows<MB> rows_of(int x_ld, int out_ld, const int* s_row, int row_base,
                                            const int* s_tok, int nrows, int li) {
  Rows<MB> rw;
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    const int m = rb * 16 + li;
    int t = -1, r = 0;
    if (m < nrows) {
      t = s_tok[m];
      r = s_row ? s_row[m] : row_base + m;
    }
    rw.valid[rb] = t >= 0;
    rw.xoff[rb] = (uint32_t)(t < 0 ? 0 : t) * (uint32_t)x_ld * 2u;
    rw.ooff[rb] = (uint32_t)r * (uint32_t)out_ld * 2u;
  }
  return rw;
}

// Expand + read-modify-write of this wave's column steps, two batches in
// flight; e0 already holds the wave's first batch.
template <int NB, int MB, bool FULL_R>
__device__ __forceinline__ void expand_rows(const Bufs& bf, int R, const Rows<MB>& rw,
                                            const HOp<NB> (&hop)[MB], int nrb, int n_lo,
                                            int n_hi, int wave, int li, int g,
                                            ExpandBatch<NB, MB, Batch<NB, MB>::UE>& e0) {
  constexpr int UE = Batch<NB, MB>::UE;
  const int ncs = (n_hi - n_lo + kColStep - 1) / kColStep;
  ExpandBatch<NB, MB, UE> e1;
  int t0 = 0;
  while (col_step(wave, t0, ncs) < ncs) {
    const int t1 = t0 + UE;
    load_expand<NB, MB, UE, FULL_R>(e1, bf, R, rw, wave, t1, ncs, n_lo, n_hi, li, g);
    __builtin_amdgcn_sched_barrier(0);
    mma_store_expand<NB, MB, UE>(e0, hop, bf, rw, nrb, wave, t0, ncs, n_lo, n_hi, g);
    __builtin_amdgcn_sched_barrier(0);
    if (col_step(wave, t1, ncs) >= ncs) break;
    const int t2 = t1 + UE;
    load_expand<NB, MB, UE, FULL_R>(e0, bf, R, rw, wave, t2, ncs, n_lo, n_hi, li, g);
    __builtin_amdgcn_sched_barrier(0);
    mma_store_expand<NB, MB, UE>(e1, hop, bf, rw, nrb, wave, t1, ncs, n_lo, n_hi, g);
    __builtin_amdgcn_sched_barrier(0);
    t0 = t2;
  }
}

template <int NB, int MB, bool FULL_R>
__device__ void fold_rows(const Bufs& bf, int K, int R, int x_ld, int out_ld, float scale,
                          const int* s_row, int row_base, const int* s_tok, int nrows, int n_lo,
                          int n_hi, float* s_part) {
  constexpr int UE = Batch<NB, MB>::UE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int nrb = (nrows + 15) >> 4;
  const Rows<MB> rw = rows_of<MB>(x_ld, out_ld, s_row, row_base, s_tok, nrows, li);

  // The first expand batch is requested once the shrink's loads are in and
  // multiplied, so the shrink's loads never queue behind it; the reduction
  // below covers part of its latency.
  const int ncs = (n_hi - n_lo + kColStep - 1) / kColStep;
  ExpandBatch<NB, MB, UE> e0;

  f32x4 hacc[MB][NB];
  shrink_k<NB, MB>(hacc, bf, K, R, rw, nrb, wave, li, g);
  load_expand<NB, MB, UE, FULL_R>(e0, bf, R, rw, wave, 0, ncs, n_lo, n_hi, li, g);
  HOp<NB> hop[MB];
  reduce_split<NB, MB>(hacc, s_part, scale, nrb, wave, lane, hop);
  expand_rows<NB, MB, FULL_R>(bf, R, rw, hop, nrb, n_lo, n_hi, wave, li, g, e0);
  // s_part and the caller's row lists are reused by the next call.
  lds_barrier();
}

// ---------------------------------------------------------------------------
// gather (decode) kernel
// ---------------------------------------------------------------------------

struct GatherArgs {
  const uint16_t* x;
  uint16_t* out;
  const int32_t* indices;
  const int32_t* row_adapter;
  const uint64_t* a_table;
  const uint64_t* b_table;
  const float* scale_table;
  uint32_t x_bytes, out_bytes;
  int32_t n_experts, K, N, R, n_slots, top_k, n_tokens;
  int32_t x_ld, out_ld;  // elements from one x / base_out row to the next
  int32_t x_by_row;      // 1: row r reads x[r] (slot-major x); 0: x[r / top_k]
  uint32_t top_k_magic;  // floor((2^32 - 1) / top_k)
  int32_t rs_count;      // row slices per expert
  int32_t ns_count;      // column slices per expert
  int32_t scan_len;      // rows per row slice (<= kScanMax)
  int32_t ns_cols;       // columns per column slice (multiple of kColStep)
  int32_t units;         // n_experts * rs_count * ns_count (kc_count for the shrink)
  int32_t per_xcd;       // ceil(units / kXcds)
  // two-kernel form only
  float* ws;             // partial H: kc_count x n_slots x RP fp32
  uint32_t ws_bytes;
  int32_t kc_count;      // k ranges of the shrink
  int32_t kc_steps;      // 32-wide k steps per range
};

// The one-kernel gather fold of work unit u (an expert's row slice and column
// slice) of the call `p`; all threads of the workgroup call it with the same
// unit.
template <int NB, int MB, bool FULL_R, bool MULTI = false, int PER = kScanMax / kThreads>
__device__ __forceinline__ void gather_fold_unit(const uint64_t* __restrict__ a_table,
                                                 const uint64_t* __restrict__ b_table,
                                                 const float* __restrict__ scale_table, int u,
                                                 int per_e, int inner, const GatherArgs& p) {
  __shared__ float s_part[kWaves * MB * 64 * 4 * NB];
  __shared__ int s_rows[kScanMax];
  __shared__ int s_toks[kScanMax];
  __shared__ int s_cnt;

  // table cell of the unit: the expert, or with MULTI (tables of
  // n_adapters x n_experts cells) adapter slot * n_experts + expert
  const int cell = u / per_e;
  const int within = u - cell * per_e;
  const int ad = MULTI ? cell / p.n_experts : 0;  // adapter slot
  const int e = cell - ad * p.n_experts;
  const int rs = within / inner, ns = within - rs * inner;

  const uint64_t a_addr = uniform_u64(a_table[cell]), b_addr = uniform_u64(b_table[cell]);
  const float scale = uniform_f32(scale_table[cell]);

  // This slice's routing, requested together with the table cells.
  const rsrc_t r_idx = make_buf(p.indices, (uint32_t)p.n_slots * 4u);
  const rsrc_t r_map = make_buf(p.row_adapter, (uint32_t)p.n_tokens * 4u);
  const int start = rs * p.scan_len;
  const int end = min(start + p.scan_len, p.n_slots);
  constexpr int kPer = PER;  // routing rounds of the slice, rounded up to 4 or 8
  const int rounds = (end - start + kThreads - 1) / kThreads;  // wave-uniform, <= kPer
  int iv[kPer], mv[kPer];
#pragma unroll
  // Loads for every round, those past the slice at an out-of-range offset:
  // straight-line code keeps the wait before the scan exact, so it does not
  // also wait for the weight loads issued after these.
  for (int i = 0; i < kPer; ++i) {
    const int row = start + i * kThreads + (int)threadIdx.x;
    const bool in = i < rounds && row < end;
    const uint32_t tok = udiv((uint32_t)row, (uint32_t)p.top_k, p.top_k_magic);
    iv[i] = (int)bld4(r_idx, in ? (uint32_t)row * 4u : kOOB);
    mv[i] = (int)bld4(r_map, in ? tok * 4u : kOOB);
  }
  if (a_addr == 0 || b_addr == 0) return;

  const int n_lo = ns * p.ns_cols;
  const int n_hi = min(n_lo + p.ns_cols, p.N);
  Bufs bf;
  bf.x = make_buf(p.x, p.x_bytes);
  bf.a = make_buf(reinterpret_cast<const void*>(a_addr), (uint32_t)(p.R * p.K) * 2u);
  bf.b = make_buf(reinterpret_cast<const void*>(b_addr), (uint32_t)(p.N * p.R) * 2u);
  bf.out = make_buf(p.out, p.out_bytes);


  if (threadIdx.x == 0) s_cnt = 0;
  lds_barrier();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (i >= rounds) break;
    const int row = start + i * kThreads + (int)threadIdx.x;
    const bool hit = row < end && iv[i] == e && (MULTI ? mv[i] == ad : mv[i] >= 0);
    const int tok = (int)udiv((uint32_t)row, (uint32_t)p.top_k, p.top_k_magic);
    wave_append(hit, row, p.x_by_row ? row : tok, &s_cnt, s_rows, s_toks, kScanMax);
  }
  lds_barrier();
  const int n = __builtin_amdgcn_readfirstlane(s_cnt);
  // The first row block runs outside the loop (a loop header would make its
  // loads wait for the weight-line requests above).
  if (n > 0)
    fold_rows<NB, MB, FULL_R>(bf, p.K, p.R, p.x_ld, p.out_ld, scale, s_rows, 0, s_toks,
                              min(16 * MB, n),
                              n_lo, n_hi, s_part);
  for (int c = 16 * MB; c < n; c += 16 * MB)
    fold_rows<NB, MB, FULL_R>(bf, p.K, p.R, p.x_ld, p.out_ld, scale, s_rows + c, 0, s_toks + c,
                              min(16 * MB, n - c), n_lo, n_hi, s_part);
}

template <int NB, int MB, bool FULL_R, bool MULTI = false, int PER = kScanMax / kThreads>
__global__ __launch_bounds__(kThreads) void gather_fold_kernel(
    const uint64_t* __restrict__ a_table, const uint64_t* __restrict__ b_table,
    const float* __restrict__ scale_table, int per_xcd, int units, int per_e, int inner,
    GatherArgs p) {
  // XCD-aware unit: consecutive units (the slices of one expert) on one XCD.
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * per_xcd + slot;
  if (u >= units) return;
  gather_fold_unit<NB, MB, FULL_R, MULTI, PER>(a_table, b_table, scale_table, u, per_e, inner, p);
}


// ---------------------------------------------------------------------------
// gather over dense slices: one-entry routes
// ---------------------------------------------------------------------------

// A route with a single expert (the router's fold) folds nearly every row of
// every slice, so its slices are short (at most 16*MB rows) and taken in
// place, without the routing scan's compaction. The x rows of a slice follow
// from its row numbers alone: every x fragment of the wave's k steps is
// requested at once, right after the rows' routing and before the table cell,
// and a row's routing (its expert id and map entry) only gates its base_out
// read and store. A row that folds nothing costs its x loads and
// MFMA columns; its output is neither read nor written. The k steps, their
// order and the reduction are those of fold_rows, so every row comes out bit
// for bit as from the compacting kernel.
constexpr int kDenseSteps = 16;  // k steps per wave: k_in up to 4 * 16 * 32 = 2048

template <int NB, int MB, bool FULL_R>
__global__ __launch_bounds__(kThreads) void gather_dense_kernel(
    const uint64_t* __restrict__ a_table, const uint64_t* __restrict__ b_table,
    const float* __restrict__ scale_table, int per_xcd, int units, int per_e, int inner,
    GatherArgs p) {
  __shared__ float s_part[kWaves * MB * 64 * 4 * NB];
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * per_xcd + slot;
  if (u >= units) return;
  const int e = u / per_e;
  const int within = u - e * per_e;
  const int rs = within / inner, ns = within - rs * inner;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int start = rs * p.scan_len;
  const int nrows = min(p.scan_len, p.n_slots - start);  // <= 16 * MB (the plan)
  const int nrb = (nrows + 15) >> 4;
  const rsrc_t r_idx = make_buf(p.indices, (uint32_t)p.n_slots * 4u);
  const rsrc_t r_map = make_buf(p.row_adapter, (uint32_t)p.n_tokens * 4u);
  const rsrc_t r_x = make_buf(p.x, p.x_bytes);
  // the rows' routing, then their x fragments
  Rows<MB> rw;
  int iv[MB], mv[MB];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    const int m = rb * 16 + li;
    const bool in = m < nrows;
    const int row = start + (in ? m : 0);
    const uint32_t tok = udiv((uint32_t)row, (uint32_t)p.top_k, p.top_k_magic);
    const uint32_t xr = p.x_by_row ? (uint32_t)row : tok;
    iv[rb] = (int)bld4(r_idx, in ? (uint32_t)row * 4u : kOOB);
    mv[rb] = (int)bld4(r_map, in ? tok * 4u : kOOB);
    rw.valid[rb] = in;
    rw.xoff[rb] = xr * (uint32_t)p.x_ld * 2u;
    rw.ooff[rb] = (uint32_t)row * (uint32_t)p.out_ld * 2u;
  }
  // the routing ahead of the x rows: waiting for it later waits for it alone
  __builtin_amdgcn_sched_barrier(0);
  const int K = p.K, R = p.R;
  const int nks = (K + 31) >> 5;
  u32x4 xv[kDenseSteps][MB];
#pragma unroll
  for (int t = 0; t < kDenseSteps; ++t) {
    const int s = wave_step(wave, t);
    const int k0 = s * 32 + g * 8;
    const bool kin = s < nks && k0 < K;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
      xv[t][rb] = bld16(r_x, (kin && rw.valid[rb]) ? rw.xoff[rb] + 2u * k0 : kOOB);
  }
  // The table cell is requested only now: scalar loads return out of order,
  // so any argument fetched after it would wait for it, and the x loads above
  // must not. No early return for an unadapted cell either (the branch would
  // be hoisted above the loads): it gets empty weight buffers and no row
  // that folds.
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t a_addr = uniform_u64(a_table[e]), b_addr = uniform_u64(b_table[e]);
  const float scale = uniform_f32(scale_table[e]);
  const bool cell = a_addr != 0 && b_addr != 0;

  Bufs bf;
  bf.x = r_x;
  bf.a = make_buf(reinterpret_cast<const void*>(a_addr), cell ? (uint32_t)(R * K) * 2u : 0u);
  bf.b = make_buf(reinterpret_cast<const void*>(b_addr), cell ? (uint32_t)(p.N * R) * 2u : 0u);
  bf.out = make_buf(p.out, p.out_bytes);
  u32x4 av[kDenseSteps][NB];
#pragma unroll
  for (int t = 0; t < kDenseSteps; ++t) {
    const int s = wave_step(wave, t);
    const int k0 = s * 32 + g * 8;
    const bool kin = s < nks && k0 < K;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int rank = (li >> 2) * 4 * NB + 4 * b + (li & 3);
      av[t][b] = bld16(bf.a, (kin && rank < R) ? (uint32_t)(rank * K + k0) * 2u : kOOB);
    }
  }
  // every A_e fragment in flight before the first MFMA waits for one
  __builtin_amdgcn_sched_barrier(0);
  // rows that fold (in the slice, routed to this expert, mapped): their
  // base_out and the slice's B_e are requested before the shrink is done
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
    rw.valid[rb] = cell && rw.valid[rb] && iv[rb] == e && mv[rb] >= 0;
  constexpr int UE = Batch<NB, MB>::UE;
  const int n_lo = ns * p.ns_cols;
  const int n_hi = min(n_lo + p.ns_cols, p.N);
  const int ncs = (n_hi - n_lo + kColStep - 1) / kColStep;
  ExpandBatch<NB, MB, UE> e0;
  load_expand<NB, MB, UE, FULL_R>(e0, bf, R, rw, wave, 0, ncs, n_lo, n_hi, li, g);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 hacc[MB][NB];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int b = 0; b < NB; ++b) hacc[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Every MFMA is issued and its result kept only for k steps and row blocks
  // in range (a select, not a branch: a branch would draw the loads it
  // consumes into it), so the sums are fold_rows' sums term for term.
#pragma unroll
  for (int t = 0; t < kDenseSteps; ++t) {
    const bool tin = wave_step(wave, t) < nks;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      const bool use = tin && rb < nrb;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const f32x4 r = mfma16x16x32(as_bf(av[t][b]), as_bf(xv[t][rb]), hacc[rb][b]);
        hacc[rb][b] = use ? r : hacc[rb][b];
      }
    }
  }
  HOp<NB> hop[MB];
  reduce_split<NB, MB>(hacc, s_part, scale, nrb, wave, lane, hop);
  expand_rows<NB, MB, FULL_R>(bf, R, rw, hop, nrb, n_lo, n_hi, wave, li, g, e0);
}

// ---------------------------------------------------------------------------
// gather, two-kernel form: k-split shrink into a workspace, then expand
// ---------------------------------------------------------------------------

// Workspace: kc_count planes of n_slots rows x RP fp32 (RP = 16 * NB), the
// partial H of each folded row over one k range, unscaled, each row in the
// lane order of the shrink (lane group g holds ranks g*4NB .. g*4NB+4NB-1).
// A plane's rows of other experts, or of rows that fold nothing, are not
// written and not read.

// The routing of flat rows [start, end): indices and map entries, requested
// for every round (rounds past the slice at an out-of-range offset), so the
// wait before the scan is exact even with other loads issued after these.
struct ScanLoads {
  static constexpr int kPer = kScanMax / kThreads;
  int iv[kPer], mv[kPer];
  int rounds;
};

__device__ __forceinline__ void request_scan(const GatherArgs& p, int start, int end,
                                             ScanLoads& sl) {
  const rsrc_t r_idx = make_buf(p.indices, (uint32_t)p.n_slots * 4u);
  const rsrc_t r_map = make_buf(p.row_adapter, (uint32_t)p.n_tokens * 4u);
  sl.rounds = (end - start + kThreads - 1) / kThreads;
#pragma unroll
  for (int i = 0; i < ScanLoads::kPer; ++i) {
    const int row = start + i * kThreads + (int)threadIdx.x;
    const bool in = i < sl.rounds && row < end;
    const uint32_t tok = udiv((uint32_t)row, (uint32_t)p.top_k, p.top_k_magic);
    sl.iv[i] = (int)bld4(r_idx, in ? (uint32_t)row * 4u : kOOB);
    sl.mv[i] = (int)bld4(r_map, in ? tok * 4u : kOOB);
  }
}

// Appends the rows of expert e whose token is mapped to s_rows / s_toks and
// returns their number (wave-uniform). Contains workgroup barriers.
__device__ __forceinline__ int finish_scan(const GatherArgs& p, int e, int start, int end,
                                           const ScanLoads& sl, int* s_rows, int* s_toks,
                                           int* s_cnt) {
  if (threadIdx.x == 0) *s_cnt = 0;
  lds_barrier();
#pragma unroll
  for (int i = 0; i < ScanLoads::kPer; ++i) {
    if (i >= sl.rounds) break;
    const int row = start + i * kThreads + (int)threadIdx.x;
    const bool hit = row < end && sl.iv[i] == e && sl.mv[i] >= 0;
    const int tok = (int)udiv((uint32_t)row, (uint32_t)p.top_k, p.top_k_magic);
    wave_append(hit, row, p.x_by_row ? row : tok, s_cnt, s_rows, s_toks, kScanMax);
  }
  lds_barrier();
  return __builtin_amdgcn_readfirstlane(*s_cnt);
}

// k steps (and column steps) one wave of the two-kernel gather holds.
constexpr int kTwoSteps = 4;

// Shrink: one workgroup per (expert, row slice, k range of at most
// kWaves * kTwoSteps k steps). After the routing scan the first row block's
// x fragments are requested, then the range's A_e fragments (loaded once,
// used by every block): the small dependent loads go first, the bulk last.
// The waves split the range's k steps; their sums meet in LDS in a fixed
// order.
template <int NB, int MB>
__global__ __launch_bounds__(kThreads) void gather_shrink_kernel(
    const uint64_t* __restrict__ a_table, const uint64_t* __restrict__ b_table,
    const float* __restrict__ scale_table, int per_xcd, int units, int per_e, int inner,
    GatherArgs p) {
  constexpr int HW = 4 * NB;
  constexpr uint32_t kRowBytes = 64u * NB;  // RP fp32
  __shared__ float s_part[kWaves * MB * 64 * HW];
  __shared__ int s_rows[kScanMax];
  __shared__ int s_toks[kScanMax];
  __shared__ int s_cnt;

  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * per_xcd + slot;
  if (u >= units) return;
  const int e = u / per_e;
  const int within = u - e * per_e;
  const int rs = within / inner, kc = within - rs * inner;
  const uint64_t a_addr = uniform_u64(a_table[e]), b_addr = uniform_u64(b_table[e]);
  (void)scale_table;
  const int start = rs * p.scan_len;
  const int end = min(start + p.scan_len, p.n_slots);
  ScanLoads sl;
  request_scan(p, start, end, sl);
  if (a_addr == 0 || b_addr == 0) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int K = p.K;
  const int s_end = min((K + 31) >> 5, (kc + 1) * p.kc_steps);
  const rsrc_t r_x = make_buf(p.x, p.x_bytes);
  const rsrc_t r_a = make_buf(reinterpret_cast<const void*>(a_addr), (uint32_t)(p.R * K) * 2u);
  const rsrc_t r_ws = make_buf(p.ws, p.ws_bytes);
  // this wave's k steps: kc * kc_steps + wave + kWaves * t (dealt one at a
  // time: the pairs of wave_step measured 3% slower here; the sums of this
  // form are grouped by k range anyway, so no other form has to match them)
  int step[kTwoSteps];
  u32x4 av[kTwoSteps][NB];
  auto request_a = [&]() {
#pragma unroll
    for (int t = 0; t < kTwoSteps; ++t) {
      step[t] = kc * p.kc_steps + wave + kWaves * t;
      const int k0 = step[t] * 32 + g * 8;
      const bool kin = step[t] < s_end && k0 < K;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int rank = (li >> 2) * 4 * NB + 4 * b + (li & 3);
        av[t][b] = bld16(r_a, (kin && rank < p.R) ? (uint32_t)(rank * K + k0) * 2u : kOOB);
      }
    }
  };
  const int n = finish_scan(p, e, start, end, sl, s_rows, s_toks, &s_cnt);
  const uint32_t plane = (uint32_t)kc * (uint32_t)p.n_slots;

  auto block = [&](int c, bool first) {
    const int nrows = min(16 * MB, n - c), nrb = (nrows + 15) >> 4;
    const Rows<MB> rw = rows_of<MB>(p.x_ld, p.out_ld, s_rows + c, 0, s_toks + c, nrows, li);
    u32x4 xv[kTwoSteps][MB];
#pragma unroll
    for (int t = 0; t < kTwoSteps; ++t) {
      const int st = kc * p.kc_steps + wave + kWaves * t;
      const int k0 = st * 32 + g * 8;
      const bool kin = st < s_end && k0 < K;
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
        xv[t][rb] = bld16(r_x, (kin && rw.valid[rb]) ? rw.xoff[rb] + 2u * k0 : kOOB);
    }
    if (first) request_a();
    __builtin_amdgcn_sched_barrier(0);
    f32x4 hacc[MB][NB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
      for (int b = 0; b < NB; ++b) hacc[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kTwoSteps; ++t) {
      if (step[t] < s_end) {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
          if (rb < nrb) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
              hacc[rb][b] = mfma16x16x32(as_bf(av[t][b]), as_bf(xv[t][rb]), hacc[rb][b]);
          }
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      if (rb < nrb) {
        float* dst = s_part + ((size_t)(wave * MB + rb) * 64 + lane) * HW;
#pragma unroll
        for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4*>(dst + 4 * b) = hacc[rb][b];
      }
    }
    lds_barrier();
    // row block rb is reduced and stored by wave rb % kWaves
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      if (rb % kWaves == wave && rb < nrb) {
        const int m = rb * 16 + li;
        const bool ok = rw.valid[rb];
        const uint32_t row = (uint32_t)(m < nrows ? s_rows[c + m] : 0);
        const uint32_t off = (plane + row) * kRowBytes + (uint32_t)g * 4u * HW;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          f32x4 h = *reinterpret_cast<const f32x4*>(s_part + ((size_t)rb * 64 + lane) * HW + 4 * q);
#pragma unroll
          for (int w = 1; w < kWaves; ++w)
            h += *reinterpret_cast<const f32x4*>(
                s_part + ((size_t)(w * MB + rb) * 64 + lane) * HW + 4 * q);
          bst16(r_ws, ok ? off + 16u * q : kOOB, __builtin_bit_cast(u32x4, h));
        }
      }
    }
    lds_barrier();  // s_part is rewritten by the next block
  };
  // the first block runs outside the loop (see the resident gather kernel)
  if (n > 0) block(0, true);
  for (int c = 16 * MB; c < n; c += 16 * MB) block(c, false);
}

// Expand: one workgroup per (expert, row slice, column slice of at most
// kWaves * kTwoSteps column steps). After the routing scan: the rows' partial
// H (summed over the k ranges in order, scaled and split into hi / lo as in
// the one-kernel form), the slice's B_e fragments (loaded once, used by every
// block), then the base_out fragments, needed only by the stores.
constexpr int kMaxKc = 4;

template <int NB, int MB, bool FULL_R>
__global__ __launch_bounds__(kThreads) void gather_expand_kernel(
    const uint64_t* __restrict__ a_table, const uint64_t* __restrict__ b_table,
    const float* __restrict__ scale_table, int per_xcd, int units, int per_e, int inner,
    GatherArgs p) {
  constexpr uint32_t kRowBytes = 64u * NB;
  constexpr int CC = Chunk<NB>::kCount;
  __shared__ int s_rows[kScanMax];
  __shared__ int s_toks[kScanMax];
  __shared__ int s_cnt;

  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * per_xcd + slot;
  if (u >= units) return;
  const int e = u / per_e;
  const int within = u - e * per_e;
  const int rs = within / inner, ns = within - rs * inner;
  const uint64_t a_addr = uniform_u64(a_table[e]), b_addr = uniform_u64(b_table[e]);
  const float scale = uniform_f32(scale_table[e]);
  const int start = rs * p.scan_len;
  const int end = min(start + p.scan_len, p.n_slots);
  ScanLoads sl;
  request_scan(p, start, end, sl);
  if (a_addr == 0 || b_addr == 0) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int n_lo = ns * p.ns_cols;
  const int n_hi = min(n_lo + p.ns_cols, p.N);
  const int ncs = (n_hi - n_lo + kColStep - 1) / kColStep;
  const rsrc_t r_b = make_buf(reinterpret_cast<const void*>(b_addr), (uint32_t)(p.N * p.R) * 2u);
  const rsrc_t r_out = make_buf(p.out, p.out_bytes);
  const rsrc_t r_ws = make_buf(p.ws, p.ws_bytes);
  BFrag<NB> bw[kTwoSteps];
  auto request_b = [&]() {
#pragma unroll
    for (int t = 0; t < kTwoSteps; ++t) {
      const int cs = col_step(wave, t, ncs);
      load_bfrag<NB, FULL_R>(bw[t], r_b, p.R, n_lo + cs * kColStep, cs < ncs ? n_hi : 0, li, g);
    }
  };
  const int n = finish_scan(p, e, start, end, sl, s_rows, s_toks, &s_cnt);
  const int kcs = p.kc_count;

  auto block = [&](int c, bool first) {
    const int nrows = min(16 * MB, n - c), nrb = (nrows + 15) >> 4;
    const Rows<MB> rw = rows_of<MB>(p.x_ld, p.out_ld, s_rows + c, 0, s_toks + c, nrows, li);
    // partial sums of every k range and the base_out fragments, requested together
    u32x4 pv[kMaxKc][MB][NB];
#pragma unroll
    for (int k = 0; k < kMaxKc; ++k)
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) {
        const int m = rb * 16 + li;
        const uint32_t row = (uint32_t)(m < nrows ? s_rows[c + m] : 0);
        const bool ok = k < kcs && rw.valid[rb];
        const uint32_t off = ((uint32_t)k * (uint32_t)p.n_slots + row) * kRowBytes +
                             (uint32_t)g * 16u * NB;
#pragma unroll
        for (int q = 0; q < NB; ++q) pv[k][rb][q] = bld16(r_ws, ok ? off + 16u * q : kOOB);
      }
    u32x4 ov[kTwoSteps][MB];
    auto request_out = [&]() {
#pragma unroll
      for (int t = 0; t < kTwoSteps; ++t) {
        const int cs = col_step(wave, t, ncs);
        const int col = n_lo + cs * kColStep + 8 * g;
        const bool cok = cs < ncs && col < n_hi;
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
          ov[t][rb] = bld16_nt(r_out, (rw.valid[rb] && cok) ? rw.ooff[rb] + 2u * col : kOOB);
      }
    };
    if constexpr (FULL_R) {
      if (first) request_b();
      request_out();
    } else {
      request_out();
      if (first) request_b();
    }
    __builtin_amdgcn_sched_barrier(0);
    HOp<NB> hop[MB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        f32x4 h = __builtin_bit_cast(f32x4, pv[0][rb][q]);
#pragma unroll
        for (int k = 1; k < kMaxKc; ++k)
          if (k < kcs) h += __builtin_bit_cast(f32x4, pv[k][rb][q]);
        const f32x4 v = scale * h;
        const uint32_t hi01 = pack_bf16(v.x, v.y), hi23 = pack_bf16(v.z, v.w);
        const uint32_t lo01 = pack_bf16(v.x - lo_f(hi01), v.y - hi_f(hi01));
        const uint32_t lo23 = pack_bf16(v.z - lo_f(hi23), v.w - hi_f(hi23));
        constexpr int CR = Chunk<NB>::kRanks;
        const int cq = (4 * q) / CR, w0 = ((4 * q) % CR) / 2;
        hop[rb].hi[cq][w0] = hi01;
        hop[rb].hi[cq][w0 + 1] = hi23;
        hop[rb].lo[cq][w0] = lo01;
        hop[rb].lo[cq][w0 + 1] = lo23;
      }
    }
#pragma unroll
    for (int t = 0; t < kTwoSteps; ++t) {
      const int cs = col_step(wave, t, ncs);
      if (cs < ncs) {
        const int col = n_lo + cs * kColStep + 8 * g;
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
          if (rb < nrb) {
            f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < CC; ++q) {
              d0 = mfma_chunk(bw[t].w[0][q], hop[rb].hi[q], d0);
              d1 = mfma_chunk(bw[t].w[1][q], hop[rb].hi[q], d1);
              d0 = mfma_chunk(bw[t].w[0][q], hop[rb].lo[q], d0);
              d1 = mfma_chunk(bw[t].w[1][q], hop[rb].lo[q], d1);
            }
            const u32x4 bq = ov[t][rb];
            const uint32_t o0 = pack_bf16(lo_f(bq.x) + d0.x, hi_f(bq.x) + d0.y);
            const uint32_t o1 = pack_bf16(lo_f(bq.y) + d0.z, hi_f(bq.y) + d0.w);
            const uint32_t o2 = pack_bf16(lo_f(bq.z) + d1.x, hi_f(bq.z) + d1.y);
            const uint32_t o3 = pack_bf16(lo_f(bq.w) + d1.z, hi_f(bq.w) + d1.w);
            bst16_nt(r_out, (rw.valid[rb] && col < n_hi) ? rw.ooff[rb] + 2u * col : kOOB,
                  u32x4{o0, o1, o2, o3});
          }
        }
      }
    }
  };
  if (n > 0) block(0, true);
  for (int c = 16 * MB; c < n; c += 16 * MB) block(c, false);
}

// ---------------------------------------------------------------------------
// gather, decode fast path: resident weights
// ---------------------------------------------------------------------------

// When a wave's whole share of A_e (its k steps) and of B_e (its column steps)
// fits in registers, A_e is requested together with the routing scan, before
// any row is known, and B_e right after the first chunk's x rows, ahead of
// its base_out rows. One 16-row block per chunk; the weights serve every
// chunk of the slice.
constexpr int kResSteps = 8;  // k steps, and column steps, per wave

// The table pointers and the unit arithmetic come first, as plain arguments:
// the library is built with kernel-argument preloading, so they arrive in
// SGPRs and the table-cell loads issue without waiting for the argument
// block (measured 0.3 us per call on the decode down projection).
template <int NB, bool FULL_R, int PER, int KS, bool MULTI = false>
__global__ __launch_bounds__(kThreads) void gather_resident_kernel(
    const uint64_t* __restrict__ a_table, const uint64_t* __restrict__ b_table,
    const float* __restrict__ scale_table, int per_xcd, int units, int per_e, int inner,
    GatherArgs p) {
  constexpr int HW = 4 * NB;
  __shared__ float s_part[kWaves * 64 * HW];
  __shared__ int s_rows[kScanMax];
  __shared__ int s_toks[kScanMax];
  __shared__ int s_cnt;

  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u0 = xcd * per_xcd + slot;
  if (u0 >= units) return;
#include "mlora_resident_body.inc"
}

// ---------------------------------------------------------------------------
// gather, several projections in one launch
// ---------------------------------------------------------------------------

// A set of up to kMaxProj gather calls (projections), each with its own
// tables, x, base_out and routing, run by one launch: the units of call i
// are first[i] .. first[i+1]-1 of one unit range, mapped to XCDs as one
// call's units are, so each call's consecutive units still share an XCD.
constexpr int kMaxProj = 4;

struct GatherSet {
  GatherArgs a[kMaxProj];
  int32_t first[kMaxProj + 1];
  int32_t n;
  int32_t total;  // units of every call (first[n]; kept apart so that no
                  // argument is indexed at run time)
  int32_t per_xcd;
};

// The call that unit u (wave-uniform) belongs to.
__device__ __forceinline__ int set_member(const GatherSet& s, int u) {
  return (s.n > 1 && u >= s.first[1] ? 1 : 0) + (s.n > 2 && u >= s.first[2] ? 1 : 0) +
         (s.n > 3 && u >= s.first[3] ? 1 : 0);
}

// The unit body with member m's arguments read at constant offsets: one
// inlined copy per member. (Picking the arguments field by field with
// selects instead measured 2.2x slower on the same unit; copying the
// picked struct goes through private memory.)
#define MLORA_SET_DISPATCH(BODY)                             \
  switch (set_member(s, u)) {                                \
    case 0: { const GatherArgs& g = s.a[0]; BODY(0); break; } \
    case 1: { const GatherArgs& g = s.a[1]; BODY(1); break; } \
    case 2: { const GatherArgs& g = s.a[2]; BODY(2); break; } \
    default: { const GatherArgs& g = s.a[3]; BODY(3); break; } \
  }

template <int NB, int MB, bool FULL_R, int PER>
__global__ __launch_bounds__(kThreads) void gather_fold_set_kernel(GatherSet s) {
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * s.per_xcd + slot;
  if (u >= s.total) return;
#define MLORA_FOLD_BODY(m)                                                              \
  gather_fold_unit<NB, MB, FULL_R, false, PER>(g.a_table, g.b_table, g.scale_table,  \
                                               u - s.first[m],                          \
                                               g.rs_count * g.ns_count, g.ns_count, g)
  MLORA_SET_DISPATCH(MLORA_FOLD_BODY)
#undef MLORA_FOLD_BODY
}
#undef MLORA_SET_DISPATCH

// The set through the decode kernel's unit (weights in registers), where
// every member's wave share fits there: the decode kernel's body, included
// once per member (its single-call kernel keeps its own code unchanged).
// One rank block may take 16 k steps a wave here (k_in up to 2048).
template <int NB, bool FULL_R, int PER, int KS>
__global__ __launch_bounds__(kThreads) void gather_resident_set_kernel(GatherSet s) {
  constexpr bool MULTI = false;
  constexpr int HW = 4 * NB;
  __shared__ float s_part[kWaves * 64 * HW];
  __shared__ int s_rows[kScanMax];
  __shared__ int s_toks[kScanMax];
  __shared__ int s_cnt;

  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * s.per_xcd + slot;
  if (u >= s.total) return;
  switch (set_member(s, u)) {
    case 0: {
      const GatherArgs& p = s.a[0];
      const uint64_t* __restrict__ a_table = p.a_table;
      const uint64_t* __restrict__ b_table = p.b_table;
      const float* __restrict__ scale_table = p.scale_table;
      const int u0 = u - s.first[0], per_e = p.rs_count * p.ns_count, inner = p.ns_count;
#include "mlora_resident_body.inc"
      break;
    }
    case 1: {
      const GatherArgs& p = s.a[1];
      const uint64_t* __restrict__ a_table = p.a_table;
      const uint64_t* __restrict__ b_table = p.b_table;
      const float* __restrict__ scale_table = p.scale_table;
      const int u0 = u - s.first[1], per_e = p.rs_count * p.ns_count, inner = p.ns_count;
#include "mlora_resident_body.inc"
      break;
    }
    case 2: {
      const GatherArgs& p = s.a[2];
      const uint64_t* __restrict__ a_table = p.a_table;
      const uint64_t* __restrict__ b_table = p.b_table;
      const float* __restrict__ scale_table = p.scale_table;
      const int u0 = u - s.first[2], per_e = p.rs_count * p.ns_count, inner = p.ns_count;
#include "mlora_resident_body.inc"
      break;
    }
    case 3: {
      const GatherArgs& p = s.a[3];
      const uint64_t* __restrict__ a_table = p.a_table;
      const uint64_t* __restrict__ b_table = p.b_table;
      const float* __restrict__ scale_table = p.scale_table;
      const int u0 = u - s.first[3], per_e = p.rs_count * p.ns_count, inner = p.ns_count;
#include "mlora_resident_body.inc"
      break;
    }
  }
}

// ---------------------------------------------------------------------------
// grouped (prefill) kernel
// ---------------------------------------------------------------------------

struct GroupedArgs {
  const uint16_t* x;
  uint16_t* out;  // base_out row row_offset (the window start)
  const int32_t* offsets;
  const int32_t* sorted_ids;
  const int32_t* row_adapter;
  const uint64_t* a_table;
  const uint64_t* b_table;
  const float* scale_table;
  uint32_t x_bytes, out_bytes;
  int64_t row_offset, row_end;
  int32_t n_experts, K, N, R, n_route, top_k, n_tokens;
  uint32_t top_k_magic;
  int32_t n_tiles, ns_count, ns_cols, units, per_xcd;  // units = tiles * sub-tiles * ns
  int32_t expand_xcd;  // expand: 1 each XCD takes a contiguous share of units, 0 block order
  // two-kernel form only: the workspace regions
  uint8_t* ws_h;
  uint64_t* ws_meta;
  uint32_t ws_h_bytes, ws_meta_bytes;
};

// One workgroup folds a sub-tile of 16*MB rows of one MLORA_MLG_M_TILE-row
// tile (4 / MB sub-tiles per tile), over one column slice.
template <int NB, int MB, bool FULL_R>
__global__ __launch_bounds__(kThreads) void grouped_fold_kernel(GroupedArgs p) {
  constexpr int kSub = kTileRows / (16 * MB);  // sub-tiles per tile
  constexpr int kRows = 16 * MB;               // rows per sub-tile
  __shared__ float s_part[kWaves * MB * 64 * 4 * NB];
  __shared__ int s_tok[kRows];
  __shared__ int s_seg_e[kRows], s_seg_lo[kRows], s_seg_hi[kRows];
  __shared__ int s_nseg;

  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * p.per_xcd + slot;
  if (u >= p.units) return;
  const int ns = u % p.ns_count;
  const int ts = u / p.ns_count;  // sub-tile index within the window
  const int64_t r0 = p.row_offset + (int64_t)(ts / kSub) * kTileRows + (ts % kSub) * kRows;
  if (r0 >= p.row_end) return;
  const int64_t r1 = min(r0 + kRows, p.row_end);

  if (threadIdx.x == 0) s_nseg = 0;
  lds_barrier();

  // Expert spans that meet this tile, clipped to it.
  for (int e = threadIdx.x; e < p.n_route; e += kThreads) {
    const int64_t lo = max((int64_t)p.offsets[e], r0);
    const int64_t hi = min((int64_t)p.offsets[e + 1], r1);
    if (lo < hi) {
      const int k = atomicAdd(&s_nseg, 1);
      if (k < kRows) {
        s_seg_e[k] = e;
        s_seg_lo[k] = (int)(lo - r0);
        s_seg_hi[k] = (int)(hi - r0);
      }
    }
  }
  // Token of each sub-tile row, or -1 when the row folds nothing.
  if (threadIdx.x < kRows) {
    const int64_t r = r0 + threadIdx.x;
    int tk = -1;
    if (r < r1) {
      const int id = p.sorted_ids[r];
      if (id >= 0) {
        const int cand = (int)udiv((uint32_t)id, (uint32_t)p.top_k, p.top_k_magic);
        if (cand < p.n_tokens && p.row_adapter[cand] >= 0) tk = cand;
      }
    }
    s_tok[threadIdx.x] = tk;
  }
  lds_barrier();
  const int nseg = min(__builtin_amdgcn_readfirstlane(s_nseg), kRows);

  const int n_lo = ns * p.ns_cols;
  const int n_hi = min(n_lo + p.ns_cols, p.N);
  Bufs bf;
  bf.x = make_buf(p.x, p.x_bytes);
  bf.out = make_buf(p.out, p.out_bytes);
  const int tile_row = (int)(r0 - p.row_offset);
  for (int sg = 0; sg < nseg; ++sg) {
    // LDS values are the same on every lane; say so, so that the expert's
    // table cells and buffer descriptors live in scalar registers.
    const int e = __builtin_amdgcn_readfirstlane(s_seg_e[sg]);
    if (e >= p.n_experts) continue;
    const uint64_t a_addr = uniform_u64(p.a_table[e]), b_addr = uniform_u64(p.b_table[e]);
    if (a_addr == 0 || b_addr == 0) continue;
    const float scale = uniform_f32(p.scale_table[e]);
    bf.a = make_buf(reinterpret_cast<const void*>(a_addr), (uint32_t)(p.R * p.K) * 2u);
    bf.b = make_buf(reinterpret_cast<const void*>(b_addr), (uint32_t)(p.N * p.R) * 2u);
    const int lo = __builtin_amdgcn_readfirstlane(s_seg_lo[sg]);
    const int hi = __builtin_amdgcn_readfirstlane(s_seg_hi[sg]);
    for (int c = lo; c < hi; c += 16 * MB)
      fold_rows<NB, MB, FULL_R>(bf, p.K, p.R, p.K, p.N, scale, nullptr, tile_row + c, s_tok + c,
                                min(16 * MB, hi - c), n_lo, n_hi, s_part);
  }
}

// ---------------------------------------------------------------------------
// grouped (prefill), two-kernel form: shrink into a workspace, then expand
// ---------------------------------------------------------------------------

// Workspace of a window of L rows, RP = 16 * NB (the kernels' rank blocks):
//   h     L rows of 4*RP bytes: RP bf16 of hi(scale_e * H[row]) (the lane
//         order of the shrink: lane group g holds ranks g*4NB .. g*4NB+4NB-1),
//         then RP bf16 of lo;
//   meta  L uint64 at a 256-byte boundary: the B_e address of the row's expert
//         when the row folds, 0 when it folds nothing.
// The shrink kernel writes both for every row of the window; the expand
// kernel reads them. Nothing in it carries over from one call to the next.

__device__ __forceinline__ void bst8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(
      __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), r, off, 0, 0);
}

// The 2*NB words of one half (hi or lo) of a lane's H operands, to / from
// 8*NB consecutive bytes. `ok` false: nothing stored, zeros loaded.
template <int NB>
__device__ __forceinline__ void store_half(rsrc_t r, bool ok, uint32_t off,
                                           const uint32_t (&w)[Chunk<NB>::kCount][Chunk<NB>::kWords]) {
  if constexpr (NB == 1) {
    bst8(r, ok ? off : kOOB, u32x2{w[0][0], w[0][1]});
  } else {
#pragma unroll
    for (int q = 0; q < Chunk<NB>::kCount; ++q)
      bst16(r, ok ? off + 16u * q : kOOB, u32x4{w[q][0], w[q][1], w[q][2], w[q][3]});
  }
}
template <int NB>
__device__ __forceinline__ void load_half(rsrc_t r, bool ok, uint32_t off,
                                          uint32_t (&w)[Chunk<NB>::kCount][Chunk<NB>::kWords]) {
  if constexpr (NB == 1) {
    const u32x2 v = bld8(r, ok ? off : kOOB);
    w[0][0] = v.x;
    w[0][1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < Chunk<NB>::kCount; ++q) {
      const u32x4 v = bld16(r, ok ? off + 16u * q : kOOB);
      w[q][0] = v.x;
      w[q][1] = v.y;
      w[q][2] = v.z;
      w[q][3] = v.w;
    }
  }
}

// Orders one wave's LDS writes before its later LDS reads of other lanes'
// data (the lanes of a wave run in lockstep; this only stops the compiler
// from reordering across it).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Shrink batch of one pass over up to two experts: the A fragments of both and
// the x fragments of the rows, for US k steps. A row's sum runs over the same
// k steps in the same order whichever expert it belongs to.
template <int NB, int MB, int US>
struct ShrinkBatch2 {
  u32x4 a0[US][NB];
  u32x4 a1[US][NB];
  u32x4 x[US][MB];
};

template <int NB, int MB, int US>
__device__ __forceinline__ void load_shrink2(ShrinkBatch2<NB, MB, US>& sb, rsrc_t rx, rsrc_t ra0,
                                             rsrc_t ra1, bool two, int K, int R,
                                             const Rows<MB>& rw, int wave, int t0, int nks, int li,
                                             int g) {
#pragma unroll
  for (int u = 0; u < US; ++u) {
    const int s = wave_step(wave, t0 + u);
    const int k0 = s * 32 + g * 8;
    const bool kin = s < nks && k0 < K;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int rank = (li >> 2) * 4 * NB + 4 * b + (li & 3);
      const uint32_t off = (kin && rank < R) ? (uint32_t)(rank * K + k0) * 2u : kOOB;
      sb.a0[u][b] = bld16(ra0, off);
      sb.a1[u][b] = bld16(ra1, two ? off : kOOB);
    }
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
      sb.x[u][rb] = bld16(rx, (kin && rw.valid[rb]) ? rw.xoff[rb] + 2u * k0 : kOOB);
  }
}

template <int NB, int MB, int US>
__device__ __forceinline__ void mma_shrink2(f32x4 (&h0)[MB][NB], f32x4 (&h1)[MB][NB],
                                            const ShrinkBatch2<NB, MB, US>& sb, int nrb,
                                            bool two) {
#pragma unroll
  for (int u = 0; u < US; ++u) {
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      if (rb < nrb) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          h0[rb][b] = mfma16x16x32(as_bf(sb.a0[u][b]), as_bf(sb.x[u][rb]), h0[rb][b]);
        if (two) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            h1[rb][b] = mfma16x16x32(as_bf(sb.a1[u][b]), as_bf(sb.x[u][rb]), h1[rb][b]);
        }
      }
    }
  }
}

// Batch size of the shrink kernel's passes: about 72 VGPRs per batch buffer.
template <int NB, int MB>
struct ShrinkUS {
  static constexpr int US = cclamp(72 / (4 * (2 * NB + MB)), 1, 8);
};

// Shrink: one workgroup per 16*MB rows of the window. The routing of its rows
// (sorted_ids, the expert spans and the table cells of every expert) is
// requested in one round; the rows' map entries, x rows and A_e fragments in
// the next. The expert spans meeting the rows are taken two per pass, x
// fragments shared. The k-split and the reduction are those of the one-kernel
// form, so H' comes out bit for bit the same.
template <int NB, int MB>
struct ShrinkSmem {
  static constexpr int kRows = 16 * MB;
  static constexpr int kPart = kWaves * MB * 64 * 4 * NB;
  float part[2 * kPart];
  uint64_t seg_a[kRows], seg_b[kRows];
  int tok[kRows], live[kRows], seg_lo[kRows], seg_hi[kRows];
  float seg_s[kRows];
  int nseg;
};

// The shrink of work unit u (16*MB rows of the window); all threads of the
// workgroup call it with the same unit.
template <int NB, int MB, int US = ShrinkUS<NB, MB>::US>
__device__ __forceinline__ void grouped_shrink_unit(const GroupedArgs& p, int u,
                                                    ShrinkSmem<NB, MB>& sm) {
  constexpr int kRows = 16 * MB;
  constexpr uint32_t kRowBytes = 64u * NB;  // 4 * RP
  constexpr int kPart = ShrinkSmem<NB, MB>::kPart;
  float* s_part = sm.part;
  int* s_tok = sm.tok;
  int* s_live = sm.live;
  int* s_seg_lo = sm.seg_lo;
  int* s_seg_hi = sm.seg_hi;
  uint64_t* s_seg_a = sm.seg_a;
  uint64_t* s_seg_b = sm.seg_b;
  float* s_seg_s = sm.seg_s;
  int& s_nseg = sm.nseg;

  const int64_t r0 = p.row_offset + (int64_t)u * kRows;
  const int64_t r1 = min(r0 + kRows, p.row_end);
  const int tid = threadIdx.x;

  // first request round: this thread's row id, and span + table cells of
  // expert e = tid
  int id = -1;
  if (tid < kRows && r0 + tid < r1) id = p.sorted_ids[r0 + tid];
  if (tid == 0) s_nseg = 0;
  lds_barrier();
  for (int e = tid; e < p.n_route; e += kThreads) {
    const int64_t lo = max((int64_t)p.offsets[e], r0);
    const int64_t hi = min((int64_t)p.offsets[e + 1], r1);
    uint64_t a_addr = 0, b_addr = 0;
    float sc = 0.f;
    if (e < p.n_experts) {
      a_addr = p.a_table[e];
      b_addr = p.b_table[e];
      sc = p.scale_table[e];
    }
    // spans of experts without both matrices fold nothing
    if (lo < hi && a_addr != 0 && b_addr != 0) {
      const int k = atomicAdd(&s_nseg, 1);
      if (k < kRows) {
        s_seg_lo[k] = (int)(lo - r0);
        s_seg_hi[k] = (int)(hi - r0);
        s_seg_a[k] = a_addr;
        s_seg_b[k] = b_addr;
        s_seg_s[k] = sc;
      }
    }
  }
  int tok = -1;
  if (id >= 0) {
    const int cand = (int)udiv((uint32_t)id, (uint32_t)p.top_k, p.top_k_magic);
    if (cand < p.n_tokens) tok = cand;
  }
  if (tid < kRows) s_tok[tid] = tok;
  lds_barrier();
  const int nseg = min(__builtin_amdgcn_readfirstlane(s_nseg), kRows);
  if (nseg == 0) {
    // nothing folds here: mark the rows so
    if (tid < kRows && r0 + tid < r1) {
      const rsrc_t r_meta = make_buf(p.ws_meta, p.ws_meta_bytes);
      bst8(r_meta, (uint32_t)(r0 - p.row_offset + tid) * 8u, u32x2{0u, 0u});
    }
    return;
  }

  // second request round: the map entry of this thread's row; consumed after
  // the shrink loads of the first pass are in flight
  int map = -1;
  if (tok >= 0) map = p.row_adapter[tok];

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int tile_row = (int)(r0 - p.row_offset);
  const int nrb = (int)((r1 - r0 + 15) >> 4);
  const rsrc_t r_h = make_buf(p.ws_h, p.ws_h_bytes);
  const rsrc_t r_x = make_buf(p.x, p.x_bytes);
  Rows<MB> rw;
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    const int t = s_tok[rb * 16 + li];
    rw.valid[rb] = t >= 0;
    rw.xoff[rb] = (uint32_t)(t < 0 ? 0 : t) * (uint32_t)p.K * 2u;
    rw.ooff[rb] = 0;
  }
  const int nks = (p.K + 31) >> 5;
  constexpr int HW = 4 * NB;
  uint64_t my_meta = 0;  // thread t < kRows: meta of row t
  for (int sg = 0; sg < nseg; sg += 2) {
    const bool two = sg + 1 < nseg;
    const uint64_t a0 = uniform_u64(s_seg_a[sg]);
    const uint64_t a1 = two ? uniform_u64(s_seg_a[sg + 1]) : a0;
    const rsrc_t ra0 = make_buf(reinterpret_cast<const void*>(a0), (uint32_t)(p.R * p.K) * 2u);
    const rsrc_t ra1 = make_buf(reinterpret_cast<const void*>(a1), (uint32_t)(p.R * p.K) * 2u);
    f32x4 h0[MB][NB], h1[MB][NB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        h0[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        h1[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    {
      ShrinkBatch2<NB, MB, US> b0, b1;
      int t0 = 0;
      load_shrink2<NB, MB, US>(b0, r_x, ra0, ra1, two, p.K, p.R, rw, wave, t0, nks, li, g);
      while (wave_step(wave, t0) < nks) {
        const int t1 = t0 + US;
        load_shrink2<NB, MB, US>(b1, r_x, ra0, ra1, two, p.K, p.R, rw, wave, t1, nks, li, g);
        __builtin_amdgcn_sched_barrier(0);
        mma_shrink2<NB, MB, US>(h0, h1, b0, nrb, two);
        __builtin_amdgcn_sched_barrier(0);
        if (wave_step(wave, t1) >= nks) break;
        const int t2 = t1 + US;
        load_shrink2<NB, MB, US>(b0, r_x, ra0, ra1, two, p.K, p.R, rw, wave, t2, nks, li, g);
        __builtin_amdgcn_sched_barrier(0);
        mma_shrink2<NB, MB, US>(h0, h1, b1, nrb, two);
        __builtin_amdgcn_sched_barrier(0);
        t0 = t2;
      }
    }
    if (sg == 0 && tid < kRows) s_live[tid] = (tok >= 0 && map >= 0) ? 1 : 0;
    // k-split partial sums of both experts through LDS, then hi / lo
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      if (rb < nrb) {
        float* d0 = s_part + ((size_t)(wave * MB + rb) * 64 + lane) * HW;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          *reinterpret_cast<f32x4*>(d0 + 4 * b) = h0[rb][b];
          if (two) *reinterpret_cast<f32x4*>(d0 + kPart + 4 * b) = h1[rb][b];
        }
      }
    }
    lds_barrier();
    const int lo0 = __builtin_amdgcn_readfirstlane(s_seg_lo[sg]);
    const int hi0 = __builtin_amdgcn_readfirstlane(s_seg_hi[sg]);
    const int lo1 = two ? __builtin_amdgcn_readfirstlane(s_seg_lo[sg + 1]) : 0;
    const int hi1 = two ? __builtin_amdgcn_readfirstlane(s_seg_hi[sg + 1]) : 0;
    const float sc0 = uniform_f32(s_seg_s[sg]);
    const float sc1 = two ? uniform_f32(s_seg_s[sg + 1]) : 0.f;
    // row block rb is reduced and written by wave rb % kWaves, live rows only
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      if (rb % kWaves == wave && rb < nrb) {
        const int m = rb * 16 + li;
        const bool in1 = two && m >= lo1 && m < hi1;
        const bool in0 = m >= lo0 && m < hi0;
        const bool ok = (in0 || in1) && s_live[m] != 0;
        const float* src = s_part + (in1 ? kPart : 0);
        const float scale = in1 ? sc1 : sc0;
        HOp<NB> hop;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          f32x4 h = *reinterpret_cast<const f32x4*>(src + ((size_t)rb * 64 + lane) * HW + 4 * q);
#pragma unroll
          for (int w = 1; w < kWaves; ++w)
            h += *reinterpret_cast<const f32x4*>(
                src + ((size_t)(w * MB + rb) * 64 + lane) * HW + 4 * q);
          const f32x4 v = scale * h;
          const uint32_t hi01 = pack_bf16(v.x, v.y), hi23 = pack_bf16(v.z, v.w);
          const uint32_t lo01 = pack_bf16(v.x - lo_f(hi01), v.y - hi_f(hi01));
          const uint32_t lo23 = pack_bf16(v.z - lo_f(hi23), v.w - hi_f(hi23));
          constexpr int CR = Chunk<NB>::kRanks;
          const int cq = (4 * q) / CR, w0 = ((4 * q) % CR) / 2;
          hop.hi[cq][w0] = hi01;
          hop.hi[cq][w0 + 1] = hi23;
          hop.lo[cq][w0] = lo01;
          hop.lo[cq][w0 + 1] = lo23;
        }
        const uint32_t off = (uint32_t)(tile_row + m) * kRowBytes + (uint32_t)g * 8u * NB;
        store_half<NB>(r_h, ok, off, hop.hi);
        store_half<NB>(r_h, ok, off + 32u * NB, hop.lo);
      }
    }
    if (tid < kRows && tok >= 0 && map >= 0) {
      if (tid >= lo0 && tid < hi0) my_meta = uniform_u64(s_seg_b[sg]);
      if (two && tid >= lo1 && tid < hi1) my_meta = uniform_u64(s_seg_b[sg + 1]);
    }
    lds_barrier();  // s_part is rewritten by the next pass
  }
  if (tid < kRows && r0 + tid < r1) {
    const rsrc_t r_meta = make_buf(p.ws_meta, p.ws_meta_bytes);
    bst8(r_meta, (uint32_t)(tile_row + tid) * 8u,
         u32x2{(uint32_t)my_meta, (uint32_t)(my_meta >> 32)});
  }
}

template <int NB, int MB>
__global__ __launch_bounds__(kThreads) void grouped_shrink_kernel(GroupedArgs p) {
  __shared__ ShrinkSmem<NB, MB> sm;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * p.per_xcd + slot;
  if (u >= p.units) return;
  grouped_shrink_unit<NB, MB>(p, u, sm);
}

// Expand: one wave per (16*MB rows, CW column steps). It requests the rows'
// meta and H', then the B_e fragments of the first two runs of rows (rows
// with one B_e) and the rows' base_out, the last in a row-contiguous layout:
// LPR lanes cover one row's CW*32 columns, 16 bytes each. The MFMA deltas
// (fp32, one lane per row) go through the wave's own LDS to that layout; each
// row is then rounded once and stored.
// LDS floats of one expand wave: its fp32 deltas, one padded row per row.
template <int MB, int CW>
struct ExpandSmem {
  static constexpr int kStride = CW * kColStep + 4;  // the pad spreads rows over banks
  static constexpr int kFloats = 16 * MB * kStride;
};

// The expand of work unit u by one wave (no workgroup barriers).
template <int NB, int MB, int CW, bool FULL_R>
__device__ __forceinline__ void grouped_expand_unit(const GroupedArgs& p, int u, float* s_d) {
  constexpr int kRows = 16 * MB;
  constexpr int kCols = CW * kColStep;
  constexpr int kStride = ExpandSmem<MB, CW>::kStride;
  constexpr int LPR = kCols / 8;      // lanes per row in the contiguous layout
  constexpr int RPI = 64 / LPR;       // rows per contiguous access
  constexpr int NI = kRows / RPI;     // contiguous accesses per wave
  constexpr uint32_t kRowBytes = 64u * NB;
  constexpr int CC = Chunk<NB>::kCount;
  static_assert(kRows <= 64 && 64 % LPR == 0 && kRows % RPI == 0, "expand shape");

  const int ns = u % p.ns_count;
  const int r0 = (u / p.ns_count) * kRows;  // window-relative
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;

  const int n_lo = ns * kCols;
  const int n_hi = min(n_lo + kCols, p.N);
  const rsrc_t r_out = make_buf(p.out, p.out_bytes);
  const rsrc_t r_h = make_buf(p.ws_h, p.ws_h_bytes);
  const rsrc_t r_meta = make_buf(p.ws_meta, p.ws_meta_bytes);

  // The meta (which gates the B_e requests) and H' (one lane per row) are
  // requested first; base_out (row-contiguous, needed last) once the meta has
  // told which rows fold, and for those rows only: rows that fold nothing
  // (an unadapted expert's span, a skipped token) cost no base_out traffic.
  // That read measured 7% faster per call where 30% of rows fold nothing and
  // 0.5% slower where all rows fold. Waits count loads in issue order, so the
  // meta's wait covers the meta alone. Rows past the window lie past all
  // three buffers and read as 0.
  const u32x2 mv = bld8(r_meta, lane < kRows ? (uint32_t)(r0 + lane) * 8u : kOOB);
  HOp<NB> hop[MB];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    const uint32_t hoff = (uint32_t)(r0 + rb * 16 + li) * kRowBytes + (uint32_t)g * 8u * NB;
    load_half<NB>(r_h, true, hoff, hop[rb].hi);
    load_half<NB>(r_h, true, hoff + 32u * NB, hop[rb].lo);
  }
  const int cr = lane / LPR, cc = lane % LPR;
  // keep the meta and H' requests ahead of the meta's first use
  __builtin_amdgcn_sched_barrier(0);
  const bool is_live = (mv.x | mv.y) != 0;
  const uint64_t live = __ballot(is_live);
  if (live == 0) return;
  // a run starts at a live row whose previous live row has another B_e
  const uint64_t below = live & ((1ull << lane) - 1ull);
  const int prev = below ? 63 - __clzll((long long)below) : lane;
  const uint32_t plo = (uint32_t)__shfl((int)mv.x, prev), phi = (uint32_t)__shfl((int)mv.y, prev);
  uint64_t starts = __ballot(is_live && (below == 0 || plo != mv.x || phi != mv.y));

  auto request_b = [&](BFrag<NB> (&bw)[CW], int s) {
    const uint64_t b_addr = lane_u64(mv.x, mv.y, s);
    const rsrc_t r_b =
        make_buf(reinterpret_cast<const void*>(b_addr), (uint32_t)(p.N * p.R) * 2u);
#pragma unroll
    for (int c = 0; c < CW; ++c)
      load_bfrag<NB, FULL_R>(bw[c], r_b, p.R, n_lo + c * kColStep, n_hi, li, g);
  };
  auto run = [&](const BFrag<NB> (&bw)[CW], int s, int e_row) {
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      if (rb * 16 < e_row && rb * 16 + 16 > s) {
        const int row = rb * 16 + li;
        const bool in = row >= s && row < e_row;
#pragma unroll
        for (int c = 0; c < CW; ++c) {
          f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < CC; ++q) {
            d0 = mfma_chunk(bw[c].w[0][q], hop[rb].hi[q], d0);
            d1 = mfma_chunk(bw[c].w[1][q], hop[rb].hi[q], d1);
            d0 = mfma_chunk(bw[c].w[0][q], hop[rb].lo[q], d0);
            d1 = mfma_chunk(bw[c].w[1][q], hop[rb].lo[q], d1);
          }
          // lane (g, li) holds columns 8g .. 8g+7 of the step for its row
          if (in) {
            float* dst = s_d + row * kStride + c * kColStep + 8 * g;
            *reinterpret_cast<f32x4*>(dst) = d0;
            *reinterpret_cast<f32x4*>(dst + 4) = d1;
          }
        }
      }
    }
  };
  // The B_e of the first two runs is requested ahead of base_out: waits count
  // loads in issue order, so their MFMAs and LDS writes then run while
  // base_out is still on its way (measured 3% and then another 1.5% faster
  // per call on the 32768-row down projection). Later runs (a wave meeting
  // more than two experts) request theirs as they come.
  BFrag<NB> bw0[CW], bw1[CW];
  const int s0 = __ffsll((unsigned long long)starts) - 1;
  starts &= starts - 1ull;
  const int s1 = starts ? __ffsll((unsigned long long)starts) - 1 : 64;
  if (starts) starts &= starts - 1ull;
  u32x4 bv[NI];
  uint32_t boff[NI];
  auto request_out = [&]() {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int col = n_lo + 8 * cc;
      boff[i] = (uint32_t)(r0 + i * RPI + cr) * (uint32_t)p.N * 2u + 2u * col;
      const bool ok = col < n_hi && ((live >> (i * RPI + cr)) & 1ull) != 0;
      bv[i] = bld16_nt(r_out, ok ? boff[i] : kOOB);
    }
  };
  if constexpr (FULL_R) {
    request_b(bw0, s0);
    if (s1 < 64) request_b(bw1, s1);
    request_out();
  } else {
    request_out();
    request_b(bw0, s0);
    if (s1 < 64) request_b(bw1, s1);
  }
  __builtin_amdgcn_sched_barrier(0);
  run(bw0, s0, s1);
  if (s1 < 64) run(bw1, s1, starts ? __ffsll((unsigned long long)starts) - 1 : 64);
  while (starts) {
    const int s = __ffsll((unsigned long long)starts) - 1;
    starts &= starts - 1ull;
    const int e_row = starts ? __ffsll((unsigned long long)starts) - 1 : 64;
    BFrag<NB> bw[CW];
    request_b(bw, s);
    run(bw, s, e_row);
  }
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const float* src = s_d + (i * RPI + cr) * kStride + 8 * cc;
    const f32x4 d0 = *reinterpret_cast<const f32x4*>(src);
    const f32x4 d1 = *reinterpret_cast<const f32x4*>(src + 4);
    const u32x4 bq = bv[i];
    const uint32_t o0 = pack_bf16(lo_f(bq.x) + d0.x, hi_f(bq.x) + d0.y);
    const uint32_t o1 = pack_bf16(lo_f(bq.y) + d0.z, hi_f(bq.y) + d0.w);
    const uint32_t o2 = pack_bf16(lo_f(bq.z) + d1.x, hi_f(bq.z) + d1.y);
    const uint32_t o3 = pack_bf16(lo_f(bq.w) + d1.z, hi_f(bq.w) + d1.w);
    const bool ok = ((live >> (i * RPI + cr)) & 1ull) != 0 && n_lo + 8 * cc < n_hi;
    bst16_nt(r_out, ok ? boff[i] : kOOB, u32x4{o0, o1, o2, o3});
  }
}

// The expand block that launch block b runs: in block order (the hardware
// deals consecutive blocks to the XCDs in turn, so the column slices of a row
// block run on different XCDs and each XCD reads only its slices of B_e but
// every row's H'), or with each XCD on a contiguous share (H' and B_e read by
// one XCD each). The planner picks (expand_xcd).
__device__ __forceinline__ int expand_block(const GroupedArgs& p, int b) {
  return p.expand_xcd ? (b % kXcds) * p.per_xcd + b / kXcds : b;
}

// Four independent expand waves per workgroup (one wave per workgroup
// measured 3% slower on the mixed batch).
template <int NB, int MB, int CW, bool FULL_R>
__global__ __launch_bounds__(kThreads) void grouped_expand_kernel(GroupedArgs p) {
  __shared__ float s_d[kWaves][ExpandSmem<MB, CW>::kFloats];
  const int wave = threadIdx.x >> 6;
  const int u = expand_block(p, (int)blockIdx.x) * kWaves + wave;
  if (u >= p.units) return;
  grouped_expand_unit<NB, MB, CW, FULL_R>(p, u, s_d[wave]);
}

// One launch that expands one window and shrinks the next: blocks
// 0 .. shrink_blocks-1 run shrink units of `ps`, every later block runs four
// independent expand waves of `pe`. The two halves touch disjoint workspace
// slots, so nothing orders them against each other.
template <int NB, int SMB, int EMB, int CW, bool FULL_R>
__global__ __launch_bounds__(kThreads) void grouped_pipe_kernel(GroupedArgs ps, GroupedArgs pe) {
  __shared__ union {
    ShrinkSmem<NB, SMB> s;
    float d[kWaves][ExpandSmem<EMB, CW>::kFloats];
  } sm;
  const int sblocks = ps.per_xcd * kXcds;
  if ((int)blockIdx.x < sblocks) {
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int u = xcd * ps.per_xcd + slot;
    // a batch of one k step per wave: the shrink half runs beside the
    // expand waves, and the launch's registers are the larger half's
    if (u < ps.units) grouped_shrink_unit<NB, SMB, 1>(ps, u, sm.s);
    return;
  }
  // sblocks is a multiple of kXcds, so b keeps the block's XCD
  const int b = (int)blockIdx.x - sblocks;
  const int wave = threadIdx.x >> 6;
  const int u = expand_block(pe, b) * kWaves + wave;
  if (u < pe.units) grouped_expand_unit<NB, EMB, CW, FULL_R>(pe, u, sm.d[wave]);
}

// ---------------------------------------------------------------------------
// fp32 fold: one workgroup per row (plain VALU; a parity-scale path)
// ---------------------------------------------------------------------------

struct RowwiseArgs {
  const float* x;
  float* out;
  const int32_t* indices;     // gather
  const int32_t* offsets;     // grouped
  const int32_t* sorted_ids;  // grouped
  const int32_t* row_adapter;
  const uint64_t* a_table;
  const uint64_t* b_table;
  const float* scale_table;
  int64_t row_begin;
  int32_t n_experts, K, N, R, top_k, n_tokens, n_route, grouped;
};

__global__ __launch_bounds__(kThreads) void rowwise_f32_kernel(RowwiseArgs p) {
  __shared__ float s_h[128];
  const int64_t row = p.row_begin + blockIdx.x;
  int e, tok;
  if (!p.grouped) {
    e = p.indices[row];
    tok = (int)(row / p.top_k);
  } else {
    // first span whose end lies past the row
    int lo = 0, hi = p.n_route;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.offsets[mid + 1] <= row) lo = mid + 1; else hi = mid;
    }
    if (lo >= p.n_route || p.offsets[lo] > row) return;
    e = lo;
    const int id = p.sorted_ids[row];
    if (id < 0) return;
    tok = id / p.top_k;
    if (tok >= p.n_tokens) return;
  }
  if (p.row_adapter[tok] < 0) return;
  if (e < 0 || e >= p.n_experts) return;
  const uint64_t a_addr = p.a_table[e], b_addr = p.b_table[e];
  if (a_addr == 0 || b_addr == 0) return;
  const float* A = reinterpret_cast<const float*>(a_addr);
  const float* B = reinterpret_cast<const float*>(b_addr);
  const float scale = p.scale_table[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* xr = p.x + (size_t)tok * p.K;
  for (int j = wave; j < p.R; j += kWaves) {
    float acc = 0.f;
    for (int k = lane; k < p.K; k += 64) acc += A[(size_t)j * p.K + k] * xr[k];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) s_h[j] = acc;
  }
  lds_barrier();
  float* orow = p.out + (size_t)row * p.N;
  for (int n = threadIdx.x; n < p.N; n += kThreads) {
    float acc = 0.f;
    for (int j = 0; j < p.R; ++j) acc += B[(size_t)n * p.R + j] * s_h[j];
    orow[n] = orow[n] + scale * acc;
  }
}

// ---------------------------------------------------------------------------
// host side: validation, launch shape, dispatch
// ---------------------------------------------------------------------------

// Launch-shape overrides (MLORA_* environment variables), read once per
// process at the first fold call and again only by
// mlora_reload_launch_overrides: no fold call reads the environment. Every
// value changes which workgroup computes what, never what a call computes
// beyond the rounding differences of the two-kernel gather.
struct Overrides {
  int gather_rs, gather_ns, gather_small, gather_resident, gather_two, gather_two_ns;
  int gather_dense;
  int grouped_mb, grouped_ns, shrink_mb, expand_mb, expand_cw, expand_xcd, all_min_rows;
};
constexpr int kUnset = -0x7fffffff;

int read_env(const char* name) {
  const char* v = std::getenv(name);
  if (!v || !*v) return kUnset;
  return std::atoi(v);
}

Overrides read_overrides() {
  Overrides o;
  o.gather_rs = read_env("MLORA_GATHER_RS");
  o.gather_ns = read_env("MLORA_GATHER_NS");
  o.gather_small = read_env("MLORA_GATHER_SMALL");
  o.gather_resident = read_env("MLORA_GATHER_RESIDENT");
  o.gather_two = read_env("MLORA_GATHER_TWO");
  o.gather_two_ns = read_env("MLORA_GATHER_TWO_NS");
  o.gather_dense = read_env("MLORA_GATHER_DENSE");
  o.grouped_mb = read_env("MLORA_GROUPED_MB");
  o.grouped_ns = read_env("MLORA_GROUPED_NS");
  o.shrink_mb = read_env("MLORA_SHRINK_MB");
  o.expand_mb = read_env("MLORA_EXPAND_MB");
  o.expand_cw = read_env("MLORA_EXPAND_CW");
  o.expand_xcd = read_env("MLORA_EXPAND_XCD");
  o.all_min_rows = read_env("MLORA_ALL_MIN_ROWS");
  return o;
}

Overrides g_overrides;
std::once_flag g_overrides_once;

const Overrides& overrides() {
  std::call_once(g_overrides_once, [] { g_overrides = read_overrides(); });
  return g_overrides;
}

// The override `v` when set, else `dflt`.
int ov(int v, int dflt) { return v == kUnset ? dflt : v; }

uint32_t magic_for(int32_t d) { return (uint32_t)(0xFFFFFFFFu / (uint32_t)d); }

// A rank whose B_e rows load as whole lane chunks (the kernels' FULL_R form):
// a multiple of a lane's chunk of ranks, 4 for ranks up to 16 (one rank
// block), else 8.
bool whole_chunks(int R) { return R % (R <= 16 ? 4 : 8) == 0; }

int32_t check_route(const mlora_expert_route* r, const char* who) {
  if (!r) return fail(MLORA_ERR_INVALID, "%s: NULL route", who);
  if (r->n_experts < 0) return fail(MLORA_ERR_INVALID, "%s: n_experts < 0", who);
  if (r->n_experts > 0 && (!r->a_table || !r->b_table || !r->scale_table))
    return fail(MLORA_ERR_INVALID, "%s: NULL table", who);
  if (r->k_in < 8 || r->k_in % 8 || r->n_out < 8 || r->n_out % 8)
    return fail(MLORA_ERR_INVALID, "%s: k_in=%d and n_out=%d must be positive multiples of 8",
                who, r->k_in, r->n_out);
  if (r->max_rank < 1 || r->max_rank > 128)
    return fail(MLORA_ERR_INVALID, "%s: max_rank=%d outside [1, 128]", who, r->max_rank);
  if (r->dtype != MLORA_BF16 && r->dtype != MLORA_F32)
    return fail(MLORA_ERR_INVALID, "%s: unknown dtype %d", who, r->dtype);
  // one expert's matrices are addressed with 32-bit offsets
  if ((int64_t)r->k_in * r->max_rank * 4 > (int64_t)kMaxBufBytes ||
      (int64_t)r->n_out * r->max_rank * 4 > (int64_t)kMaxBufBytes)
    return fail(MLORA_ERR_INVALID, "%s: an expert matrix exceeds 4 GiB", who);
  return MLORA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t launched(const char* who) {
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(MLORA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(err));
  clear_error();
  return MLORA_OK;
}

// Column slice width: a multiple of the expand step, covering n_out in `ns`.
int ns_cols_for(int N, int ns) {
  const int per = (N + ns - 1) / ns;
  return (per + kColStep - 1) / kColStep * kColStep;
}

// The leading plain arguments of the gather kernels (preloaded into SGPRs):
// the tables and the unit arithmetic, `inner` being the sub-units per row
// slice (column slices, or k ranges for the shrink).
#define LEAD_ARGS(a, inner)                                                              \
  (a).a_table, (a).b_table, (a).scale_table, (a).per_xcd, (a).units,                    \
      (a).rs_count * (inner), (inner), (a)

// Routing rounds a slice of scan_len rows needs, rounded up to 4 or 8: the
// kernels issue every round's loads, those past the slice out of range.
constexpr int scan_rounds(int scan_len) { return scan_len <= 4 * kThreads ? 4 : 8; }

template <int NB, int MB, bool MULTI, int PER>
void launch_gather_per(const GatherArgs& a, int grid, hipStream_t s) {
  if (whole_chunks(a.R))
    hipLaunchKernelGGL((gather_fold_kernel<NB, MB, true, MULTI, PER>), dim3(grid), dim3(kThreads),
                       0, s, LEAD_ARGS(a, a.ns_count));
  else
    hipLaunchKernelGGL((gather_fold_kernel<NB, MB, false, MULTI, PER>), dim3(grid),
                       dim3(kThreads), 0, s, LEAD_ARGS(a, a.ns_count));
}

template <int NB, int MB>
void launch_gather(const GatherArgs& a, int grid, hipStream_t s) {
  if (scan_rounds(a.scan_len) == 4) return launch_gather_per<NB, MB, false, 4>(a, grid, s);
  launch_gather_per<NB, MB, false, 8>(a, grid, s);
}

// Rank blocks of 16 -> (NB, MB) instantiation. `small` picks one 16-row block
// per chunk, for slices that hold few rows of their expert (decode).
// The decode fast path applies when every wave's k steps and column steps fit
// the resident register arrays.
// The set form of the decode kernel also takes one rank block at up to 16 k
// steps a wave (k_in up to 2048).
constexpr int kResStepsWide = 16;

bool resident_set_fits(const GatherArgs& a) {
  const int nb = (a.R + 15) / 16;
  const int nks = (a.K + 31) / 32;
  const int ncs = (a.ns_cols + kColStep - 1) / kColStep;
  return nb <= 2 && nks <= kWaves * (nb <= 1 ? kResStepsWide : kResSteps) &&
         ncs <= kWaves * kResSteps;
}

bool gather_resident_fits(const GatherArgs& a) {
  const int nb = (a.R + 15) / 16;
  const int nks = (a.K + 31) / 32;
  const int ncs = (a.ns_cols + kColStep - 1) / kColStep;
  return nb <= 2 && nks <= kWaves * kResSteps && ncs <= kWaves * kResSteps;
}

// Rank blocks the kernels use for max_rank R: ceil(R / 16) rounded up to 1,
// 2, 4 or 8.
int kernel_nb(int R) {
  const int nb = (R + 15) / 16;
  return nb <= 1 ? 1 : (nb <= 2 ? 2 : (nb <= 4 ? 4 : 8));
}

// Two-kernel gather: k ranges of the shrink (about 16 k steps each, at most
// kMaxKc), and the workspace they need.
int gather_kc(int K) {
  const int nks = (K + 31) / 32;
  const int kc = (nks + kWaves * kTwoSteps - 1) / (kWaves * kTwoSteps);
  return kc < 1 ? 1 : (kc > kMaxKc ? kMaxKc : kc);
}

int64_t gather_ws_bytes(int64_t n_slots, int K, int R) {
  return ((int64_t)gather_kc(K) * n_slots * 64 * kernel_nb(R) + 255) & ~(int64_t)255;
}

// Rows a slice expected to hold `rows` rows may reach: an expert's count in a
// top-k batch spreads about its mean like a Poisson count, so the mean plus
// two standard deviations. Sizing a pass's row blocks by the mean alone sends
// about half the experts through a second pass over their weights (the
// gate/up projection at 16 rows per expert: 24.0 us per call with 16-row
// passes, 22.8 with 32-row ones, in either gather form).
int64_t rows_with_headroom(int64_t rows) {
  int64_t sd = 0;
  while ((sd + 1) * (sd + 1) <= rows) ++sd;
  return rows + 2 * sd;
}

// Row blocks per pass of the two-kernel gather for a slice of `rows` rows.
int gather_two_mb(int R, int64_t rows) {
  const int nb = kernel_nb(R);
  const int cap = nb <= 2 ? 4 : (nb <= 4 ? 2 : 1);
  const int64_t top = rows_with_headroom(rows);
  const int want = top <= 16 ? 1 : (top <= 32 ? 2 : 4);
  return want < cap ? want : cap;
}

template <int NB, int MB>
void launch_gather_two(const GatherArgs& g1, const GatherArgs& g2, hipStream_t s) {
  hipLaunchKernelGGL((gather_shrink_kernel<NB, MB>), dim3(g1.per_xcd * kXcds), dim3(kThreads), 0,
                     s, LEAD_ARGS(g1, g1.kc_count));
  if (whole_chunks(g2.R))
    hipLaunchKernelGGL((gather_expand_kernel<NB, MB, true>), dim3(g2.per_xcd * kXcds),
                       dim3(kThreads), 0, s, LEAD_ARGS(g2, g2.ns_count));
  else
    hipLaunchKernelGGL((gather_expand_kernel<NB, MB, false>), dim3(g2.per_xcd * kXcds),
                       dim3(kThreads), 0, s, LEAD_ARGS(g2, g2.ns_count));
}

template <int NB>
void dispatch_gather_two_mb(const GatherArgs& g1, const GatherArgs& g2, hipStream_t s, int mb) {
  if constexpr (NB <= 2) {
    if (mb >= 4) return launch_gather_two<NB, 4>(g1, g2, s);
  }
  if constexpr (NB <= 4) {
    if (mb >= 2) return launch_gather_two<NB, 2>(g1, g2, s);
  }
  launch_gather_two<NB, 1>(g1, g2, s);
}

void dispatch_gather_two(const GatherArgs& g1, const GatherArgs& g2, hipStream_t s, int mb) {
  switch (kernel_nb(g1.R)) {
    case 1: return dispatch_gather_two_mb<1>(g1, g2, s, mb);
    case 2: return dispatch_gather_two_mb<2>(g1, g2, s, mb);
    case 4: return dispatch_gather_two_mb<4>(g1, g2, s, mb);
    default: return dispatch_gather_two_mb<8>(g1, g2, s, mb);
  }
}

template <int NB, bool FULL_R, int PER, bool MULTI>
void launch_resident_per(const GatherArgs& a, int grid, hipStream_t s) {
  // k steps per wave: 6 cover k_in up to 768 (4 waves x 6 steps of 32),
  // 8 up to 1024, 16 (one rank block, single-adapter calls) up to 2048
  const int nks = (a.K + 31) / 32;
  if (nks <= kWaves * 6)
    hipLaunchKernelGGL((gather_resident_kernel<NB, FULL_R, PER, 6, MULTI>), dim3(grid),
                       dim3(kThreads), 0, s, LEAD_ARGS(a, a.ns_count));
  else if (NB > 1 || MULTI || nks <= kWaves * kResSteps)
    hipLaunchKernelGGL((gather_resident_kernel<NB, FULL_R, PER, kResSteps, MULTI>), dim3(grid),
                       dim3(kThreads), 0, s, LEAD_ARGS(a, a.ns_count));
  else
    hipLaunchKernelGGL((gather_resident_kernel<1, FULL_R, PER, kResStepsWide, false>),
                       dim3(grid), dim3(kThreads), 0, s, LEAD_ARGS(a, a.ns_count));
}

// The routing rounds the slice needs (scan_len rows, kThreads a round),
// rounded up to 1, 2, 3, 4 or 8: rounds past the slice would still issue
// their (out-of-range) loads, and each such load costs issue time (three
// rounds instead of four: 1.5% per call on the decode down projection).
template <int NB, bool FULL_R, bool MULTI = false>
void launch_resident(const GatherArgs& a, int grid, hipStream_t s) {
  const int rounds = (a.scan_len + kThreads - 1) / kThreads;
  if (rounds <= 1) return launch_resident_per<NB, FULL_R, 1, MULTI>(a, grid, s);
  if (rounds <= 2) return launch_resident_per<NB, FULL_R, 2, MULTI>(a, grid, s);
  if (rounds <= 3) return launch_resident_per<NB, FULL_R, 3, MULTI>(a, grid, s);
  if (rounds <= 4) return launch_resident_per<NB, FULL_R, 4, MULTI>(a, grid, s);
  launch_resident_per<NB, FULL_R, kScanMax / kThreads, MULTI>(a, grid, s);
}

template <int NB, int MB>
void launch_dense(const GatherArgs& a, int grid, hipStream_t s) {
  if (whole_chunks(a.R))
    hipLaunchKernelGGL((gather_dense_kernel<NB, MB, true>), dim3(grid), dim3(kThreads), 0, s,
                       LEAD_ARGS(a, a.ns_count));
  else
    hipLaunchKernelGGL((gather_dense_kernel<NB, MB, false>), dim3(grid), dim3(kThreads), 0, s,
                       LEAD_ARGS(a, a.ns_count));
}

void dispatch_gather(const GatherArgs& a, int grid, hipStream_t s, bool small, bool resident,
                     int dense_mb) {
  const int nb = (a.R + 15) / 16;
  if (dense_mb > 0) {
    // the plan's shapes: 32-row slices for one rank block, 16 for two
    if (nb <= 1) launch_dense<1, 2>(a, grid, s);
    else launch_dense<2, 1>(a, grid, s);
    return;
  }
  if (resident && (gather_resident_fits(a) || (nb <= 1 && resident_set_fits(a)))) {
    if (nb <= 1) {
      if (whole_chunks(a.R)) launch_resident<1, true>(a, grid, s);
      else launch_resident<1, false>(a, grid, s);
    } else {
      if (whole_chunks(a.R)) launch_resident<2, true>(a, grid, s);
      else launch_resident<2, false>(a, grid, s);
    }
    return;
  }
  if (nb <= 1) {
    if (small) launch_gather<1, 1>(a, grid, s); else launch_gather<1, 4>(a, grid, s);
  } else if (nb <= 2) {
    if (small) launch_gather<2, 1>(a, grid, s); else launch_gather<2, 4>(a, grid, s);
  } else if (nb <= 4) {
    if (small) launch_gather<4, 1>(a, grid, s); else launch_gather<4, 2>(a, grid, s);
  } else {
    launch_gather<8, 1>(a, grid, s);
  }
}

template <int NB, int MB>
void launch_grouped(const GroupedArgs& a, int grid, hipStream_t s) {
  if (whole_chunks(a.R))
    hipLaunchKernelGGL((grouped_fold_kernel<NB, MB, true>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_fold_kernel<NB, MB, false>), dim3(grid), dim3(kThreads), 0, s, a);
}

// Largest rows-per-workgroup (16 * MB) that each rank width supports.
int grouped_mb_max(int R) {
  const int nb = (R + 15) / 16;
  return nb <= 2 ? 4 : (nb <= 4 ? 2 : 1);
}

template <int NB>
void dispatch_grouped_mb(const GroupedArgs& a, int grid, hipStream_t s, int mb) {
  if (mb >= 4) launch_grouped<NB, 4>(a, grid, s);
  else if (mb == 2) launch_grouped<NB, 2>(a, grid, s);
  else launch_grouped<NB, 1>(a, grid, s);
}

void dispatch_grouped(const GroupedArgs& a, int grid, hipStream_t s, int mb) {
  const int nb = (a.R + 15) / 16;
  if (nb <= 1) dispatch_grouped_mb<1>(a, grid, s, mb);
  else if (nb <= 2) dispatch_grouped_mb<2>(a, grid, s, mb);
  else if (nb <= 4) { if (mb >= 2) launch_grouped<4, 2>(a, grid, s); else launch_grouped<4, 1>(a, grid, s); }
  else launch_grouped<8, 1>(a, grid, s);
}

// The one-kernel launch of a bf16 gather call: its arguments, grid and
// kernel choice. x has x_rows rows of x_ld elements (row r / top_k, or row r
// itself with x_by_row), base_out n_slots rows of out_ld elements, the map
// map_len entries. Validates what the kernels assume; MLORA_OK or an error.
struct GatherPlan {
  GatherArgs a;
  int grid;
  int small, resident;
  bool use_resident;
  int dense_mb;  // > 0: one-entry route in slices of at most 16 * dense_mb rows taken in place
};

int32_t plan_gather(const char* who, const mlora_expert_route* route, const void* x,
                    int64_t x_rows, int64_t x_ld, int32_t x_by_row, void* base_out,
                    int64_t out_ld, const int32_t* indices, const int32_t* row_adapter,
                    int64_t map_len, int64_t n_slots, int32_t top_k, GatherPlan* plan) {
  if (!aligned16(x) || !aligned16(base_out))
    return fail(MLORA_ERR_INVALID, "%s: x and base_out must be 16-byte aligned", who);
  const int E = route->n_experts, K = route->k_in, N = route->n_out, R = route->max_rank;
  if (x_ld < K || x_ld % 8 || out_ld < N || out_ld % 8)
    return fail(MLORA_ERR_INVALID,
                "%s: row strides x_ld=%lld / out_ld=%lld must be multiples of 8 and at least "
                "k_in=%d / n_out=%d", who, (long long)x_ld, (long long)out_ld, K, N);
  const int64_t x_bytes = ((x_rows > 0 ? x_rows - 1 : 0) * x_ld + K) * 2;
  const int64_t out_bytes = ((n_slots - 1) * out_ld + N) * 2;
  if (x_bytes > (int64_t)kMaxBufBytes || out_bytes > (int64_t)kMaxBufBytes)
    return fail(MLORA_ERR_INVALID, "%s: x or base_out exceeds 4 GiB; split the call", who);
  const int ns_max = (N + kColStep - 1) / kColStep;

  // Launch shape. Row slices first (each slice scans at most kScanMax rows),
  // then more row slices while slices keep enough rows, then column slices
  // while the repeated shrink stays cheaper than the expand it splits.
  const int64_t rows_per_e = (n_slots + E - 1) / E;
  int rs = (int)((n_slots + kScanMax - 1) / kScanMax);
  int ns = 1;
  const int64_t target = 256;  // one workgroup per CU; measured better than two
  while ((int64_t)E * rs * ns < target && rows_per_e / (rs * 2) >= 32) rs *= 2;
  // A call with very few experts (a one-entry route over a decode batch)
  // goes on to slices of as few as 4 rows rather than run on a handful of
  // workgroups: the router's fold over 80 decode tokens (k_in 2048) measured
  // 11.3 us at 2 slices, 7.6-8.0 us at 8-16.
  while ((int64_t)E * rs * ns < target / 4 && rows_per_e / (rs * 2) >= 4) rs *= 2;
  // A one-entry route (a router's fold) goes to the dense-slice kernel when
  // its operands fit the kernel's registers: slices of at most 32 rows (16 for
  // ranks above 16), every k step of a wave's x in registers.
  const int dense_mb = kernel_nb(R) == 1 ? 2 : 1;
  bool dense = E == 1 && kernel_nb(R) <= 2 && (K + 31) / 32 <= kWaves * kDenseSteps &&
               ov(overrides().gather_dense, 1) != 0;
  if (dense) {
    const int64_t need = (n_slots + 16 * dense_mb - 1) / (16 * dense_mb);
    if (rs < need) rs = (int)need;
  }
  const double shrink_b = 2.0 * R * K + 2.0 * (double)rows_per_e / rs * K;
  const double expand_b = 2.0 * N * R + 4.0 * (double)rows_per_e / rs * N;
  while ((int64_t)E * rs * ns < target && ns * 2 <= ns_max &&
         (ns * 2) * shrink_b <= 2.0 * (shrink_b + expand_b))
    ns *= 2;
  rs = ov(overrides().gather_rs, rs);
  ns = ov(overrides().gather_ns, ns);
  if (ns < 1) ns = 1;
  if (ns > ns_max) ns = ns_max;
  if (rs < 1) rs = 1;
  int scan = (int)((n_slots + rs - 1) / rs);
  if (scan > kScanMax) {
    rs = (int)((n_slots + kScanMax - 1) / kScanMax);
    scan = (int)((n_slots + rs - 1) / rs);
  }
  // (an override of the row slices can leave them longer than the dense kernel takes)
  if (scan > 16 * dense_mb) dense = false;

  GatherArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.out = static_cast<uint16_t*>(base_out);
  a.indices = indices;
  a.row_adapter = row_adapter;
  a.a_table = route->a_table;
  a.b_table = route->b_table;
  a.scale_table = route->scale_table;
  a.x_bytes = (uint32_t)x_bytes;
  a.out_bytes = (uint32_t)out_bytes;
  a.n_experts = E;
  a.K = K;
  a.N = N;
  a.R = R;
  a.n_slots = (int32_t)n_slots;
  a.top_k = top_k;
  a.n_tokens = (int32_t)map_len;
  a.x_ld = (int32_t)x_ld;
  a.out_ld = (int32_t)out_ld;
  a.x_by_row = x_by_row ? 1 : 0;
  a.top_k_magic = magic_for(top_k);
  a.rs_count = rs;
  a.ns_count = ns;
  a.scan_len = scan;
  a.ns_cols = ns_cols_for(N, ns);
  const int64_t units = (int64_t)E * rs * ns;
  if (units > 0x7fffffffll / 2)
    return fail(MLORA_ERR_INVALID, "%s: launch too large", who);
  a.units = (int32_t)units;
  a.per_xcd = (int32_t)((units + kXcds - 1) / kXcds);
  plan->a = a;
  plan->grid = a.per_xcd * kXcds;
  // one 16-row block per chunk when a slice is expected to hold few rows
  const int64_t rows_per_slice = (n_slots + (int64_t)E * rs - 1) / ((int64_t)E * rs);
  plan->small = ov(overrides().gather_small, rows_with_headroom(rows_per_slice) <= 16 ? 1 : 0);
  // weights held in registers when a slice is expected to hold at most two
  // 16-row blocks (and the wave's share fits)
  // One rank block at k_in 1025..2048 takes the wide form (16 k steps a wave),
  // by default only at up to 6 rows per expert: a decode batch's gate/up call
  // (640 rows, k_in 2048, rank 16) measured 7.35 us against 8.9 for the
  // streaming kernel, while at 16 rows per expert the two-kernel form stays
  // ahead (14.5 against 14.9 us).
  const bool wide = kernel_nb(R) == 1 && !gather_resident_fits(a) && resident_set_fits(a);
  const bool wide_ok = !wide || rows_per_e <= 6;
  plan->resident =
      ov(overrides().gather_resident, (rows_per_slice <= 32 && wide_ok) ? 1 : 0);
  plan->use_resident =
      plan->resident != 0 && (gather_resident_fits(a) || (wide && resident_set_fits(a)));
  plan->dense_mb = dense ? dense_mb : 0;
  return MLORA_OK;
}

}  // namespace
}  // namespace mlora

using namespace mlora;

extern "C" int32_t mlora_gather_bgmv(const mlora_expert_route* route, const void* x,
                                     int64_t n_tokens, void* base_out, const int32_t* indices,
                                     const int32_t* row_adapter, int64_t n_slots, int32_t top_k,
                                     void* workspace, uint64_t workspace_bytes, void* stream) {
  const char* who = "mlora_gather_bgmv";
  if (int32_t rc = check_route(route, who)) return rc;
  if (!workspace && workspace_bytes != 0)
    return fail(MLORA_ERR_INVALID, "%s: NULL workspace with workspace_bytes > 0", who);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLORA_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
  if (top_k <= 0) return fail(MLORA_ERR_INVALID, "%s: top_k=%d must be positive", who, top_k);
  if (n_slots < 0 || n_slots > (int64_t)0x7fffffff - kScanMax)
    return fail(MLORA_ERR_INVALID, "%s: n_slots=%lld out of range", who, (long long)n_slots);
  const int64_t need_tok = (n_slots + top_k - 1) / top_k;
  if (n_tokens < need_tok || n_tokens > 0x3fffffffll)
    return fail(MLORA_ERR_INVALID, "%s: n_tokens=%lld (need >= ceil(n_slots/top_k)=%lld)", who,
                (long long)n_tokens, (long long)need_tok);
  if (n_slots == 0 || route->n_experts == 0) {
    clear_error();
    return MLORA_OK;
  }
  if (!x || !base_out || !indices || !row_adapter)
    return fail(MLORA_ERR_INVALID, "%s: NULL device pointer", who);
  const int64_t ws_need = gather_ws_bytes(n_slots, route->k_in, route->max_rank);
  if (workspace && route->dtype == MLORA_BF16 && (uint64_t)ws_need > workspace_bytes)
    return fail(MLORA_ERR_CAPACITY, "%s: workspace of %llu bytes, %lld needed", who,
                (unsigned long long)workspace_bytes, (long long)ws_need);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();

  if (route->dtype == MLORA_F32) {
    RowwiseArgs a{};
    a.x = static_cast<const float*>(x);
    a.out = static_cast<float*>(base_out);
    a.indices = indices;
    a.row_adapter = row_adapter;
    a.a_table = route->a_table;
    a.b_table = route->b_table;
    a.scale_table = route->scale_table;
    a.row_begin = 0;
    a.n_experts = route->n_experts;
    a.K = route->k_in;
    a.N = route->n_out;
    a.R = route->max_rank;
    a.top_k = top_k;
    a.n_tokens = (int32_t)n_tokens;
    a.grouped = 0;
    hipLaunchKernelGGL(rowwise_f32_kernel, dim3((unsigned)n_slots), dim3(kThreads), 0, s, a);
    return launched(who);
  }

  GatherPlan plan;
  if (int32_t rc = plan_gather(who, route, x, n_tokens, route->k_in, 0, base_out, route->n_out,
                               indices, row_adapter, n_tokens, n_slots, top_k, &plan))
    return rc;
  const GatherArgs& a = plan.a;
  const int grid = plan.grid;
  const int small = plan.small;
  const int resident = plan.resident;
  const bool use_resident = plan.use_resident;
  const int E = a.n_experts, K = a.K, N = a.N, R = a.R;
  const int ns_max = (N + kColStep - 1) / kColStep;
  // The two-kernel form holds at most kWaves * kTwoSteps k steps per range.
  // It pays where an expert's A_e outweighs its rows' x (few rows per expert,
  // k_in split over several ranges); an expert with many rows streams x once
  // per row in one kernel anyway. With few rows per expert the second launch
  // and its routing round cost more than the split saves, until some expert
  // holds more than 16 rows and its one-kernel workgroup takes a second
  // 16-row chunk (measured over 128 experts, top-8, k_in 1536-2048, ranks
  // 16-64: one kernel 3-14% faster at 4-7 rows per expert on average, two
  // kernels 14-36% faster from 8). At 7 the one-kernel form already risks
  // that second chunk, so it is used up to 6.
  const bool two_fits = (K + 31) / 32 <= kMaxKc * kWaves * kTwoSteps;
  const int64_t rows_e_all = (n_slots + E - 1) / E;
  const int two_default = (gather_kc(K) > 1 && rows_e_all > 6 && rows_e_all <= 64) ? 1 : 0;
  if (workspace && !use_resident && plan.dense_mb == 0 && two_fits &&
      ov(overrides().gather_two, two_default) != 0) {
    if (ws_need > (int64_t)kMaxBufBytes)
      return fail(MLORA_ERR_INVALID, "%s: workspace above 4 GiB; split the call", who);
    // k-split shrink, then expand; slices of at most 64 rows of an expert
    const int64_t rows_e = (n_slots + E - 1) / E;
    int64_t rs2 = (n_slots + kScanMax - 1) / kScanMax;
    const int64_t want = (rows_e + 63) / 64;
    if (want > rs2) rs2 = want;
    if (rs2 > n_slots) rs2 = n_slots;
    const int scan2 = (int)((n_slots + rs2 - 1) / rs2);
    const int64_t rows_slice = (rows_e + rs2 - 1) / rs2;
    const int mb = gather_two_mb(R, rows_slice);
    const int kc = gather_kc(K);
    const int nks = (K + 31) / 32;
    // column slices of at most kWaves * kTwoSteps steps, more while short of
    // one workgroup per CU
    int ns2 = (ns_max + kWaves * kTwoSteps - 1) / (kWaves * kTwoSteps);
    while ((int64_t)E * rs2 * ns2 < 256 && ns2 * 2 <= ns_max) ns2 *= 2;
    ns2 = ov(overrides().gather_two_ns, ns2);
    if (ns2 < 1) ns2 = 1;
    if (ns2 > ns_max) ns2 = ns_max;
    if (ns_cols_for(N, ns2) > kWaves * kTwoSteps * kColStep)
      ns2 = (ns_max + kWaves * kTwoSteps - 1) / (kWaves * kTwoSteps);
    GatherArgs g1 = a, g2 = a;
    g1.ws = g2.ws = static_cast<float*>(workspace);
    g1.ws_bytes = g2.ws_bytes = (uint32_t)ws_need;
    g1.kc_count = g2.kc_count = kc;
    g1.kc_steps = g2.kc_steps = (nks + kc - 1) / kc;
    g1.rs_count = g2.rs_count = (int32_t)rs2;
    g1.scan_len = g2.scan_len = scan2;
    const int64_t u1 = (int64_t)E * rs2 * kc, u2 = (int64_t)E * rs2 * ns2;
    if (u1 > 0x3fffffffll || u2 > 0x3fffffffll)
      return fail(MLORA_ERR_INVALID, "%s: launch too large", who);
    g1.units = (int32_t)u1;
    g1.per_xcd = (int32_t)((u1 + kXcds - 1) / kXcds);
    g2.ns_count = ns2;
    g2.ns_cols = ns_cols_for(N, ns2);
    g2.units = (int32_t)u2;
    g2.per_xcd = (int32_t)((u2 + kXcds - 1) / kXcds);
    dispatch_gather_two(g1, g2, s, mb);
    return launched(who);
  }
  dispatch_gather(a, grid, s, small != 0, resident != 0, plan.dense_mb);
  return launched(who);
}

namespace mlora {
namespace {

template <int NB, int MB, bool FULL_R>
void launch_fold_set(const GatherSet& gs, int grid, hipStream_t s) {
  int scan = 0;
  for (int i = 0; i < gs.n; ++i) scan = gs.a[i].scan_len > scan ? gs.a[i].scan_len : scan;
  if (scan_rounds(scan) == 4)
    hipLaunchKernelGGL((gather_fold_set_kernel<NB, MB, FULL_R, 4>), dim3(grid), dim3(kThreads), 0,
                       s, gs);
  else
    hipLaunchKernelGGL((gather_fold_set_kernel<NB, MB, FULL_R, 8>), dim3(grid), dim3(kThreads), 0,
                       s, gs);
}

template <int NB, bool FULL_R, int PER>
void launch_resident_set_per(const GatherSet& gs, int grid, hipStream_t s, int k_max) {
  const int nks = (k_max + 31) / 32;
  if (nks <= kWaves * 6)
    hipLaunchKernelGGL((gather_resident_set_kernel<NB, FULL_R, PER, 6>), dim3(grid),
                       dim3(kThreads), 0, s, gs);
  else if (NB > 1 || nks <= kWaves * kResSteps)
    hipLaunchKernelGGL((gather_resident_set_kernel<NB, FULL_R, PER, kResSteps>), dim3(grid),
                       dim3(kThreads), 0, s, gs);
  else
    hipLaunchKernelGGL((gather_resident_set_kernel<1, FULL_R, PER, kResStepsWide>), dim3(grid),
                       dim3(kThreads), 0, s, gs);
}

// The set through the decode kernel: the routing rounds of the longest
// member's slice (3, 4 or 8) and the k steps of the longest k_in.
template <int NB, bool FULL_R>
void launch_resident_set(const GatherSet& gs, int grid, hipStream_t s, int scan, int k_max) {
  const int rounds = (scan + kThreads - 1) / kThreads;
  if (rounds <= 3) return launch_resident_set_per<NB, FULL_R, 3>(gs, grid, s, k_max);
  if (rounds <= 4) return launch_resident_set_per<NB, FULL_R, 4>(gs, grid, s, k_max);
  launch_resident_set_per<NB, FULL_R, kScanMax / kThreads>(gs, grid, s, k_max);
}

void dispatch_resident_set(const GatherSet& gs, int grid, hipStream_t s, int nb, bool full,
                           int scan, int k_max) {
  if (nb <= 1) {
    if (full) return launch_resident_set<1, true>(gs, grid, s, scan, k_max);
    return launch_resident_set<1, false>(gs, grid, s, scan, k_max);
  }
  if (full) return launch_resident_set<2, true>(gs, grid, s, scan, k_max);
  launch_resident_set<2, false>(gs, grid, s, scan, k_max);
}

template <bool FULL_R>
void dispatch_set(const GatherSet& gs, int grid, hipStream_t s, int nb, bool small) {
  if (nb <= 1) {
    if (small) return launch_fold_set<1, 1, FULL_R>(gs, grid, s);
    return launch_fold_set<1, 4, FULL_R>(gs, grid, s);
  }
  if (nb <= 2) {
    if (small) return launch_fold_set<2, 1, FULL_R>(gs, grid, s);
    return launch_fold_set<2, 4, FULL_R>(gs, grid, s);
  }
  if (nb <= 4) {
    if (small) return launch_fold_set<4, 1, FULL_R>(gs, grid, s);
    return launch_fold_set<4, 2, FULL_R>(gs, grid, s);
  }
  launch_fold_set<8, 1, FULL_R>(gs, grid, s);
}

}  // namespace
}  // namespace mlora

extern "C" int32_t mlora_gather_bgmv_set(const mlora_projection* projs, int32_t n_proj,
                                         void* stream) {
  const char* who = "mlora_gather_bgmv_set";
  if (n_proj < 1 || n_proj > kMaxProj)
    return fail(MLORA_ERR_INVALID, "%s: n_proj=%d outside 1..%d", who, n_proj, kMaxProj);
  if (!projs) return fail(MLORA_ERR_INVALID, "%s: NULL projections", who);
  GatherSet gs{};
  GatherPlan plans[kMaxProj];
  int nb = 0, members = 0, only = -1;
  bool full = true, small = true;
  int64_t total = 0;
  gs.first[0] = 0;
  for (int32_t i = 0; i < n_proj; ++i) {
    const mlora_projection& pj = projs[i];
    if (int32_t rc = check_route(pj.route, who)) return rc;
    const mlora_expert_route* r = pj.route;
    if (r->dtype != MLORA_BF16)
      return fail(MLORA_ERR_INVALID, "%s: projection %d is not bf16", who, i);
    if (pj.top_k <= 0)
      return fail(MLORA_ERR_INVALID, "%s: projection %d: top_k=%d must be positive", who, i,
                  pj.top_k);
    if (pj.n_slots < 0 || pj.n_slots > (int64_t)0x7fffffff - kScanMax)
      return fail(MLORA_ERR_INVALID, "%s: projection %d: n_slots out of range", who, i);
    const int64_t need_tok = (pj.n_slots + pj.top_k - 1) / pj.top_k;
    const int64_t need_x = pj.x_by_row ? pj.n_slots : need_tok;
    if (pj.map_len < need_tok || pj.map_len > 0x3fffffffll || pj.x_rows < need_x ||
        pj.x_rows > 0x3fffffffll)
      return fail(MLORA_ERR_INVALID,
                  "%s: projection %d: %lld map entries and %lld x rows, need >= %lld and %lld",
                  who, i, (long long)pj.map_len, (long long)pj.x_rows, (long long)need_tok,
                  (long long)need_x);
    if (nb == 0) nb = kernel_nb(r->max_rank);
    if (kernel_nb(r->max_rank) != nb)
      return fail(MLORA_ERR_INVALID,
                  "%s: projection %d: max_rank %d and the first one's need different rank "
                  "blocks (ceil(max_rank / 16) rounded to 1, 2, 4, 8 must agree)",
                  who, i, r->max_rank);
    if (pj.n_slots == 0 || r->n_experts == 0) {
      gs.first[i + 1] = (int32_t)total;
      gs.a[i] = GatherArgs{};
      continue;
    }
    if (!pj.x || !pj.base_out || !pj.indices || !pj.row_adapter)
      return fail(MLORA_ERR_INVALID, "%s: projection %d: NULL device pointer", who, i);
    GatherPlan plan;
    if (int32_t rc = plan_gather(who, r, pj.x, pj.x_rows, pj.x_ld, pj.x_by_row, pj.base_out,
                                 pj.out_ld, pj.indices, pj.row_adapter, pj.map_len, pj.n_slots,
                                 pj.top_k, &plan))
      return rc;
    gs.a[i] = plan.a;
    plans[i] = plan;
    ++members;
    only = i;
    full = full && whole_chunks(r->max_rank);
    small = small && plan.small != 0;
    total += plan.a.units;
    if (total > 0x3fffffffll) return fail(MLORA_ERR_INVALID, "%s: launch too large", who);
    gs.first[i + 1] = (int32_t)total;
  }
  for (int32_t i = n_proj; i < kMaxProj; ++i) gs.first[i + 1] = (int32_t)total;
  gs.n = n_proj;
  gs.total = (int32_t)total;
  if (total == 0) {
    clear_error();
    return MLORA_OK;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (members == 1) {
    // one call with rows: the single-call kernels (the decode-resident one
    // where it fits), which take their leading arguments preloaded
    const GatherPlan& pl = plans[only];
    dispatch_gather(pl.a, pl.grid, s, pl.small != 0, pl.resident != 0, pl.dense_mb);
    return launched(who);
  }
  gs.per_xcd = (int32_t)((total + kXcds - 1) / kXcds);
  const int grid = gs.per_xcd * kXcds;
  // the decode kernel's unit where every member with rows asks for it and fits
  bool resident = nb <= 2;
  int scan = 0, k_max = 0;
  for (int32_t i = 0; i < n_proj; ++i) {
    if (gs.a[i].units == 0) continue;
    resident = resident && plans[i].resident != 0 && resident_set_fits(gs.a[i]);
    scan = gs.a[i].scan_len > scan ? gs.a[i].scan_len : scan;
    k_max = gs.a[i].K > k_max ? gs.a[i].K : k_max;
  }
  if (resident) {
    dispatch_resident_set(gs, grid, s, nb, full, scan, k_max);
    return launched(who);
  }
  if (full)
    dispatch_set<true>(gs, grid, s, nb, small);
  else
    dispatch_set<false>(gs, grid, s, nb, small);
  return launched(who);
}

namespace mlora {
namespace {

template <int NB, int MB>
void launch_gather_multi(const GatherArgs& a, int grid, hipStream_t s) {
  if (scan_rounds(a.scan_len) == 4) return launch_gather_per<NB, MB, true, 4>(a, grid, s);
  launch_gather_per<NB, MB, true, 8>(a, grid, s);
}

// The multi-adapter cells through the decode kernel (weights in registers)
// where the plan asks for it and the wave's share fits, else through the
// streaming one-kernel gather.
void dispatch_gather_multi(const GatherArgs& a, int grid, hipStream_t s, bool small,
                           bool resident) {
  const int nb = kernel_nb(a.R);
  if (resident && gather_resident_fits(a)) {
    if (nb <= 1) {
      if (whole_chunks(a.R)) return launch_resident<1, true, true>(a, grid, s);
      return launch_resident<1, false, true>(a, grid, s);
    }
    if (whole_chunks(a.R)) return launch_resident<2, true, true>(a, grid, s);
    return launch_resident<2, false, true>(a, grid, s);
  }
  if (nb <= 1) {
    if (small) return launch_gather_multi<1, 1>(a, grid, s);
    return launch_gather_multi<1, 4>(a, grid, s);
  }
  if (nb <= 2) {
    if (small) return launch_gather_multi<2, 1>(a, grid, s);
    return launch_gather_multi<2, 4>(a, grid, s);
  }
  if (nb <= 4) {
    if (small) return launch_gather_multi<4, 1>(a, grid, s);
    return launch_gather_multi<4, 2>(a, grid, s);
  }
  launch_gather_multi<8, 1>(a, grid, s);
}

}  // namespace
}  // namespace mlora

extern "C" int32_t mlora_gather_bgmv_multi(const mlora_multi_route* route, const void* x,
                                           int64_t n_tokens, void* base_out,
                                           const int32_t* indices, const int32_t* row_adapter,
                                           int64_t n_slots, int32_t top_k, void* stream) {
  const char* who = "mlora_gather_bgmv_multi";
  if (!route) return fail(MLORA_ERR_INVALID, "%s: NULL route", who);
  if (route->n_adapters < 0 || route->n_experts < 0)
    return fail(MLORA_ERR_INVALID, "%s: negative table size", who);
  const int64_t cells = (int64_t)route->n_adapters * route->n_experts;
  if (cells > 0x7fffffffll) return fail(MLORA_ERR_INVALID, "%s: too many table cells", who);
  if (route->dtype != MLORA_BF16) return fail(MLORA_ERR_INVALID, "%s: bf16 only", who);
  // the cell tables as one route over n_adapters * n_experts "experts"
  mlora_expert_route flat{route->a_table, route->b_table, route->scale_table, (int32_t)cells,
                          route->k_in, route->n_out, route->max_rank, route->dtype};
  if (int32_t rc = check_route(&flat, who)) return rc;
  if (top_k <= 0) return fail(MLORA_ERR_INVALID, "%s: top_k=%d must be positive", who, top_k);
  if (n_slots < 0 || n_slots > (int64_t)0x7fffffff - kScanMax)
    return fail(MLORA_ERR_INVALID, "%s: n_slots=%lld out of range", who, (long long)n_slots);
  const int64_t need_tok = (n_slots + top_k - 1) / top_k;
  if (n_tokens < need_tok || n_tokens > 0x3fffffffll)
    return fail(MLORA_ERR_INVALID, "%s: n_tokens=%lld (need >= ceil(n_slots/top_k)=%lld)", who,
                (long long)n_tokens, (long long)need_tok);
  if (n_slots == 0 || cells == 0) {
    clear_error();
    return MLORA_OK;
  }
  if (!x || !base_out || !indices || !row_adapter)
    return fail(MLORA_ERR_INVALID, "%s: NULL device pointer", who);
  GatherPlan plan;
  if (int32_t rc = plan_gather(who, &flat, x, n_tokens, route->k_in, 0, base_out, route->n_out,
                               indices, row_adapter, n_tokens, n_slots, top_k, &plan))
    return rc;
  plan.a.n_experts = route->n_experts;
  GatherArgs& a = plan.a;
  if (plan.resident && kernel_nb(a.R) <= 2 && (a.K + 31) / 32 <= kWaves * kResSteps &&
      !gather_resident_fits(a)) {
    // column slices narrow enough for the decode kernel's registers
    const int ncs = (a.N + kColStep - 1) / kColStep;
    const int ns = (ncs + kWaves * kResSteps - 1) / (kWaves * kResSteps);
    const int64_t units = (int64_t)cells * a.rs_count * ns;
    if (units <= 0x7fffffffll / 2) {
      a.ns_count = ns;
      a.ns_cols = ns_cols_for(a.N, ns);
      a.units = (int32_t)units;
      a.per_xcd = (int32_t)((units + kXcds - 1) / kXcds);
      plan.grid = a.per_xcd * kXcds;
    }
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  dispatch_gather_multi(a, plan.grid, s, plan.small != 0, plan.resident != 0);
  return launched(who);
}

// Workspace layout of the two-kernel grouped form (see the kernels).
struct WsLayout {
  int64_t h_bytes, meta_off, meta_bytes, total;
};

WsLayout grouped_ws_layout(int64_t rows, int R) {
  WsLayout w;
  const int64_t rp = 16 * (int64_t)kernel_nb(R);
  w.h_bytes = rows * 4 * rp;
  w.meta_off = (w.h_bytes + 255) & ~(int64_t)255;
  w.meta_bytes = rows * 8;
  w.total = (w.meta_off + w.meta_bytes + 255) & ~(int64_t)255;
  return w;
}

// Row blocks per expand wave: the largest of `want` (1, 2 or 4) the rank
// width supports.
int expand_mb(int R, int want) {
  const int nb = kernel_nb(R);
  const int cap = nb <= 2 ? 4 : (nb <= 4 ? 2 : 1);
  want = want >= 4 ? 4 : (want >= 2 ? 2 : 1);
  return want < cap ? want : cap;
}

template <int NB>
void launch_shrink(const GroupedArgs& a, int grid, hipStream_t s, int mb) {
  if constexpr (NB <= 2) {
    if (mb >= 4) {
      hipLaunchKernelGGL((grouped_shrink_kernel<NB, 4>), dim3(grid), dim3(kThreads), 0, s, a);
      return;
    }
  }
  if (mb >= 2)
    hipLaunchKernelGGL((grouped_shrink_kernel<NB, 2>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_shrink_kernel<NB, 1>), dim3(grid), dim3(kThreads), 0, s, a);
}

void dispatch_shrink(const GroupedArgs& a, int grid, hipStream_t s, int mb) {
  const int nb = (a.R + 15) / 16;
  if (nb <= 1) launch_shrink<1>(a, grid, s, mb);
  else if (nb <= 2) launch_shrink<2>(a, grid, s, mb);
  else if (nb <= 4) launch_shrink<4>(a, grid, s, mb);
  else launch_shrink<8>(a, grid, s, 1);
}

// Column steps per expand wave: 4 where the operands leave room (ranks of
// whole lane chunks, at most 32), else 2.
int expand_cw(int R, int requested) {
  const int nb = (R + 15) / 16;
  return (whole_chunks(R) && nb <= 2 && requested >= 4) ? 4 : 2;
}

// How expand units meet the XCDs. In block order the column units of a row
// block go to the XCDs in turn: all XCDs work on the same rows at once, and
// every XCD reads the H' (4 * R bytes) of every row. With contiguous shares
// each XCD works through its own eighth of the window and each row's H' is
// read once. Measured on 32768-row prefill batches (all windows, µs per
// call), block order won where a row block splits into more than 16 column
// units (n_out 4096 at ranks 16 and 32, n_out 2048 at rank 64 with its
// 64-column waves: 2-3%) and contiguous shares won at 16 or fewer (n_out 2048
// at ranks 16 and 32, n_out 1024: 1-3.5%).
int expand_xcd(int ns_count) {
  const int v = ov(overrides().expand_xcd, ns_count <= 16 ? 1 : 0);
  return v ? 1 : 0;
}

// Grid of the expand kernel (four waves a block) over a.units units, with
// a.ns_count already set.
int64_t expand_grid(GroupedArgs& a) {
  const int64_t blocks = ((int64_t)a.units + kWaves - 1) / kWaves;
  a.per_xcd = (int32_t)((blocks + kXcds - 1) / kXcds);
  a.expand_xcd = expand_xcd(a.ns_count);
  return (int64_t)a.per_xcd * kXcds;
}

template <int NB, int MB>
void launch_expand(const GroupedArgs& a, int grid, hipStream_t s, int cw) {
  const bool full = whole_chunks(a.R);
  if (!full) {
    hipLaunchKernelGGL((grouped_expand_kernel<NB, MB, 2, false>), dim3(grid), dim3(kThreads), 0, s, a);
  } else if constexpr (NB <= 2) {
    if (cw >= 4)
      hipLaunchKernelGGL((grouped_expand_kernel<NB, MB, 4, true>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((grouped_expand_kernel<NB, MB, 2, true>), dim3(grid), dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((grouped_expand_kernel<NB, MB, 2, true>), dim3(grid), dim3(kThreads), 0, s, a);
  }
}

template <int NB>
void launch_expand_mb(const GroupedArgs& a, int grid, hipStream_t s, int mb, int cw) {
  if constexpr (NB <= 2) {
    if (mb >= 4) return launch_expand<NB, 4>(a, grid, s, cw);
  }
  if constexpr (NB <= 4) {
    if (mb >= 2) return launch_expand<NB, 2>(a, grid, s, cw);
  }
  launch_expand<NB, 1>(a, grid, s, cw);
}

void dispatch_expand(const GroupedArgs& a, int grid, hipStream_t s, int mb, int cw) {
  switch (kernel_nb(a.R)) {
    case 1: return launch_expand_mb<1>(a, grid, s, mb, cw);
    case 2: return launch_expand_mb<2>(a, grid, s, mb, cw);
    case 4: return launch_expand_mb<4>(a, grid, s, mb, cw);
    default: return launch_expand_mb<8>(a, grid, s, mb, cw);
  }
}

// ---- pipelined grouped windows ----

// Launch shape of the two-kernel grouped form on a window of `rows` rows.
struct TwoPlan {
  int smb, emb, cw;
  int64_t sunits, etiles, eslices;
};

// Row blocks of a standalone shrink launch's tile: `want` (1, 2 or 4) within
// what the rank's kernels take (4 up to 32 ranks, 2 up to 64, else 1).
int shrink_tile_mb(int R, int want) {
  return (want >= 4 && kernel_nb(R) <= 2) ? 4 : (want >= 2 && kernel_nb(R) <= 4 ? 2 : 1);
}

TwoPlan two_plan(int R, int N, int64_t rows, bool pipe) {
  TwoPlan t;
  // two expand row blocks per wave share each B_e fragment where the rank
  // has whole lane chunks and is at most 64 (measured 4% faster per window
  // at rank 32)
  const bool small_full = whole_chunks(R) && kernel_nb(R) <= 4;
  // shrink tiles of 64 rows for at most 32 ranks, 32 rows for at most 64: A_e
  // is read once per tile (at rank 32, 64-row tiles measured 3.5% faster per
  // call than 32-row ones and 15% than 16-row ones; at rank 64, 32-row tiles
  // with 32-row expand waves 23% faster than 16-row ones)
  t.smb = kernel_nb(R) <= 2 ? 4 : (kernel_nb(R) <= 4 ? 2 : 1);
  t.emb = expand_mb(R, ov(overrides().expand_mb, small_full ? 2 : 1));
  t.cw = expand_cw(R, ov(overrides().expand_cw, 4));
  if (pipe) {
    // the pipe kernel takes 1 expand row block, or 2 for ranks of whole lane
    // chunks up to 64, and always its default shrink tile
    t.emb = (t.emb >= 2 && small_full) ? 2 : 1;
  } else {
    t.smb = shrink_tile_mb(R, ov(overrides().shrink_mb, t.smb));
  }
  t.sunits = (rows + 16 * t.smb - 1) / (16 * t.smb);
  t.etiles = (rows + 16 * t.emb - 1) / (16 * t.emb);
  t.eslices = (N + t.cw * kColStep - 1) / (t.cw * kColStep);
  return t;
}

template <int NB, int SMB, int EMB, int CW, bool FULL_R>
void launch_pipe(const GroupedArgs& ps, const GroupedArgs& pe, int grid, hipStream_t s) {
  hipLaunchKernelGGL((grouped_pipe_kernel<NB, SMB, EMB, CW, FULL_R>), dim3(grid),
                     dim3(kThreads), 0, s, ps, pe);
}

// The pipelined launches use the shapes of two_plan(pipe = true).
template <int NB>
void dispatch_pipe_nb(const GroupedArgs& ps, const GroupedArgs& pe, int grid, hipStream_t s,
                      int emb, int cw) {
  constexpr int SMB = NB <= 2 ? 4 : (NB <= 4 ? 2 : 1);
  if (!whole_chunks(ps.R)) return launch_pipe<NB, SMB, 1, 2, false>(ps, pe, grid, s);
  if constexpr (NB <= 2) {
    if (emb >= 2) {
      if (cw >= 4) return launch_pipe<NB, SMB, 2, 4, true>(ps, pe, grid, s);
      return launch_pipe<NB, SMB, 2, 2, true>(ps, pe, grid, s);
    }
    if (cw >= 4) return launch_pipe<NB, SMB, 1, 4, true>(ps, pe, grid, s);
  } else if constexpr (NB <= 4) {
    if (emb >= 2) return launch_pipe<NB, SMB, 2, 2, true>(ps, pe, grid, s);
  }
  launch_pipe<NB, SMB, 1, 2, true>(ps, pe, grid, s);
}

void dispatch_pipe(const GroupedArgs& ps, const GroupedArgs& pe, int grid, hipStream_t s,
                   int emb, int cw) {
  switch (kernel_nb(ps.R)) {
    case 1: return dispatch_pipe_nb<1>(ps, pe, grid, s, emb, cw);
    case 2: return dispatch_pipe_nb<2>(ps, pe, grid, s, emb, cw);
    case 4: return dispatch_pipe_nb<4>(ps, pe, grid, s, emb, cw);
    default: return dispatch_pipe_nb<8>(ps, pe, grid, s, emb, cw);
  }
}

// Workspace of one window slot of the pipelined call.
// Rows per launch of the all-windows call: whole windows, at least
// kAllMinRows of them (MLORA_ALL_MIN_ROWS overrides). Fewer, larger launches
// pay less launch and drain time than their shorter pipeline hides (measured
// on 8192-row windows of the prefill down projection: 2 launches of 16384
// rows beat 4 of 8192 by 10%).
constexpr int64_t kAllMinRows = 16384;

// Windows per launch for a launch minimum of `min_rows` rows.
int64_t windows_per_launch(int64_t cap, int64_t min_rows) {
  return cap >= min_rows ? 1 : (min_rows + cap - 1) / cap;
}

// Rows per launch: whole windows, at least the launch minimum (an override
// may only lower it, to between 1 and kAllMinRows rows, so the workspace
// query below covers every value).
int64_t all_chunk_rows(int64_t n_rows, int64_t cap) {
  int64_t min_rows = ov(overrides().all_min_rows, (int)kAllMinRows);
  if (min_rows < 1) min_rows = 1;
  if (min_rows > kAllMinRows) min_rows = kAllMinRows;
  const int64_t chunk = cap * windows_per_launch(cap, min_rows);
  return chunk < n_rows ? chunk : n_rows;
}

int64_t pipe_slot_bytes(int64_t rows, int R) {
  return (grouped_ws_layout(rows, R).total + 255) & ~(int64_t)255;
}

extern "C" uint64_t mlora_gather_bgmv_workspace_bytes(int64_t n_slots, int32_t k_in,
                                                      int32_t max_rank) {
  if (n_slots <= 0 || k_in < 1 || max_rank < 1 || max_rank > 128) return 0;
  return (uint64_t)gather_ws_bytes(n_slots, k_in, max_rank);
}

extern "C" uint64_t mlora_grouped_down_workspace_bytes(int64_t row_offset, int64_t row_end,
                                                       int32_t max_rank) {
  if (row_offset < 0 || row_end < row_offset || max_rank < 1 || max_rank > 128) return 0;
  if (row_end == row_offset) return 0;
  return (uint64_t)grouped_ws_layout(row_end - row_offset, max_rank).total;
}

extern "C" int32_t mlora_grouped_down(const mlora_expert_route* route, const void* x,
                                      int64_t n_tokens, void* base_out, int64_t n_rows,
                                      const int32_t* expert_offsets, int32_t n_route,
                                      const int32_t* sorted_ids, const int32_t* row_adapter,
                                      int32_t top_k, int64_t row_offset, int64_t row_end,
                                      void* workspace, uint64_t workspace_bytes,
                                      void* stream) {
  const char* who = "mlora_grouped_down";
  if (!workspace && workspace_bytes != 0)
    return fail(MLORA_ERR_INVALID, "%s: NULL workspace with workspace_bytes > 0", who);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLORA_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
  if (int32_t rc = check_route(route, who)) return rc;
  if (top_k <= 0) return fail(MLORA_ERR_INVALID, "%s: top_k=%d must be positive", who, top_k);
  if (n_route < 0) return fail(MLORA_ERR_INVALID, "%s: n_route < 0", who);
  if (n_tokens < 0 || n_tokens > 0x3fffffffll)
    return fail(MLORA_ERR_INVALID, "%s: n_tokens out of range", who);
  if (n_rows < 0 || row_offset < 0 || row_end < row_offset || row_end > n_rows)
    return fail(MLORA_ERR_INVALID, "%s: window [%lld, %lld) outside [0, %lld]", who,
                (long long)row_offset, (long long)row_end, (long long)n_rows);
  if (row_end == row_offset || route->n_experts == 0 || n_route == 0) {
    clear_error();
    return MLORA_OK;
  }
  if (!x || !base_out || !expert_offsets || !sorted_ids || !row_adapter)
    return fail(MLORA_ERR_INVALID, "%s: NULL device pointer", who);
  const WsLayout wsl = grouped_ws_layout(row_end - row_offset, route->max_rank);
  if (workspace && route->dtype == MLORA_BF16 && (uint64_t)wsl.total > workspace_bytes)
    return fail(MLORA_ERR_CAPACITY, "%s: workspace of %llu bytes, %lld needed", who,
                (unsigned long long)workspace_bytes, (long long)wsl.total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();

  if (route->dtype == MLORA_F32) {
    RowwiseArgs a{};
    a.x = static_cast<const float*>(x);
    a.out = static_cast<float*>(base_out);
    a.offsets = expert_offsets;
    a.sorted_ids = sorted_ids;
    a.row_adapter = row_adapter;
    a.a_table = route->a_table;
    a.b_table = route->b_table;
    a.scale_table = route->scale_table;
    a.row_begin = row_offset;
    a.n_experts = route->n_experts;
    a.K = route->k_in;
    a.N = route->n_out;
    a.R = route->max_rank;
    a.top_k = top_k;
    a.n_tokens = (int32_t)n_tokens;
    a.n_route = n_route;
    a.grouped = 1;
    const int64_t len = row_end - row_offset;
    if (len > 0x7fffffffll) return fail(MLORA_ERR_INVALID, "%s: window too large", who);
    hipLaunchKernelGGL(rowwise_f32_kernel, dim3((unsigned)len), dim3(kThreads), 0, s, a);
    return launched(who);
  }

  if (!aligned16(x) || !aligned16(base_out))
    return fail(MLORA_ERR_INVALID, "%s: x and base_out must be 16-byte aligned", who);
  const int N = route->n_out, K = route->k_in, R = route->max_rank;
  const int64_t x_bytes = n_tokens * K * 2, out_bytes = (row_end - row_offset) * N * 2;
  if (x_bytes > (int64_t)kMaxBufBytes || out_bytes > (int64_t)kMaxBufBytes)
    return fail(MLORA_ERR_INVALID, "%s: x or the window of base_out exceeds 4 GiB", who);
  GroupedArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.out = static_cast<uint16_t*>(base_out) + row_offset * N;
  a.offsets = expert_offsets;
  a.sorted_ids = sorted_ids;
  a.row_adapter = row_adapter;
  a.a_table = route->a_table;
  a.b_table = route->b_table;
  a.scale_table = route->scale_table;
  a.x_bytes = (uint32_t)x_bytes;
  a.out_bytes = (uint32_t)out_bytes;
  a.row_offset = row_offset;
  a.row_end = row_end;
  a.n_experts = route->n_experts;
  a.K = K;
  a.N = N;
  a.R = R;
  a.n_route = n_route;
  a.top_k = top_k;
  a.n_tokens = (int32_t)n_tokens;
  a.top_k_magic = magic_for(top_k);

  if (workspace) {
    const int64_t rows = row_end - row_offset;
    const WsLayout& w = wsl;
    if (w.h_bytes > (int64_t)kMaxBufBytes || w.meta_bytes > (int64_t)kMaxBufBytes)
      return fail(MLORA_ERR_INVALID, "%s: window too large for one workspace; split it", who);
    a.ws_h = static_cast<uint8_t*>(workspace);
    a.ws_meta = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(workspace) + w.meta_off);
    a.ws_h_bytes = (uint32_t)w.h_bytes;
    a.ws_meta_bytes = (uint32_t)w.meta_bytes;
    // shrink: one workgroup per 16 * smb rows; expand: one wave per
    // (16 * emb rows, cw column steps)
    const TwoPlan t = two_plan(R, N, rows, false);
    if (t.sunits > 0x3fffffffll || t.etiles * t.eslices > 0x3fffffffll)
      return fail(MLORA_ERR_INVALID, "%s: window too large", who);
    a.units = (int32_t)t.sunits;
    a.per_xcd = (int32_t)((t.sunits + kXcds - 1) / kXcds);
    dispatch_shrink(a, a.per_xcd * kXcds, s, t.smb);
    if (int32_t rc = launched(who)) return rc;
    a.ns_count = (int32_t)t.eslices;
    a.units = (int32_t)(t.etiles * t.eslices);
    const int64_t eg = expand_grid(a);
    dispatch_expand(a, (int)eg, s, t.emb, t.cw);
    return launched(who);
  }

  const int64_t tiles = mlora_grouped_down_wc(row_offset, row_end);
  const int ns_max = (N + kColStep - 1) / kColStep;
  // Split a tile's rows over workgroups first (no operand is read twice but
  // A_e / B_e, which L2 serves), then columns while the grid is short of two
  // workgroups per CU and the repeated shrink (x rows + A_e) stays below the
  // expand bytes it splits.
  int mb = grouped_mb_max(R);
  while (mb > 1 && tiles * (4 / mb) < 512) mb /= 2;
  int ns = 1;
  const double shrink_b = 2.0 * 16 * mb * K + 2.0 * R * K;
  const double expand_b = 4.0 * 16 * mb * N + 2.0 * N * R;
  while (tiles * (4 / mb) * ns < 512 && ns * 2 <= ns_max &&
         (ns * 2) * shrink_b <= shrink_b + expand_b)
    ns *= 2;
  mb = ov(overrides().grouped_mb, mb);
  ns = ov(overrides().grouped_ns, ns);
  if (mb != 1 && mb != 2 && mb != 4) mb = 2;
  if (mb > grouped_mb_max(R)) mb = grouped_mb_max(R);
  if (ns < 1) ns = 1;
  if (ns > ns_max) ns = ns_max;
  const int64_t units = tiles * (4 / mb) * ns;
  if (units > 0x7fffffffll / 2) return fail(MLORA_ERR_INVALID, "%s: window too large", who);

  a.n_tiles = (int32_t)tiles;
  a.ns_count = ns;
  a.ns_cols = ns_cols_for(N, ns);
  a.units = (int32_t)units;
  a.per_xcd = (int32_t)((units + kXcds - 1) / kXcds);
  const int grid = a.per_xcd * kXcds;
  dispatch_grouped(a, grid, s, mb);
  return launched(who);
}

extern "C" int32_t mlora_apply_expert_lora_sorted(
    const mlora_expert_route* route, const void* x, int64_t n_tokens, void* base_out,
    int64_t n_rows, const int32_t* expert_offsets, const int32_t* expert_offsets_host,
    int32_t n_route, const uint64_t* a_table_host, const uint64_t* b_table_host,
    const int32_t* sorted_ids, const int32_t* row_adapter, int32_t top_k, void* workspace,
    uint64_t workspace_bytes, void* stream) {
  const char* who = "mlora_apply_expert_lora_sorted";
  if (int32_t rc = check_route(route, who)) return rc;
  if (n_route < 0) return fail(MLORA_ERR_INVALID, "%s: n_route < 0", who);
  if (n_route > 0 && !expert_offsets_host)
    return fail(MLORA_ERR_INVALID, "%s: NULL host offsets", who);
  if (route->n_experts > 0 && (!a_table_host || !b_table_host))
    return fail(MLORA_ERR_INVALID, "%s: NULL host table", who);
  // the spans come from the host copy: check them all before any launch
  for (int32_t e = 0; e < n_route; ++e) {
    const int64_t lo = expert_offsets_host[e], hi = expert_offsets_host[e + 1];
    if (lo < 0 || hi < lo || hi > n_rows)
      return fail(MLORA_ERR_INVALID, "%s: span %d = [%lld, %lld) outside [0, %lld]", who, e,
                  (long long)lo, (long long)hi, (long long)n_rows);
  }
  // one grouped launch per adapted expert with rows: its span is the window
  int64_t launched_rows = 0;
  for (int32_t e = 0; e < n_route && e < route->n_experts; ++e) {
    const int64_t lo = expert_offsets_host[e], hi = expert_offsets_host[e + 1];
    if (hi == lo || a_table_host[e] == 0 || b_table_host[e] == 0) continue;
    if (int32_t rc = mlora_grouped_down(route, x, n_tokens, base_out, n_rows, expert_offsets,
                                        n_route, sorted_ids, row_adapter, top_k, lo, hi,
                                        workspace, workspace_bytes, stream))
      return rc;
    launched_rows += hi - lo;
  }
  (void)launched_rows;
  clear_error();
  return MLORA_OK;
}

extern "C" uint64_t mlora_grouped_down_all_workspace_bytes(int64_t n_rows, int64_t cap,
                                                           int32_t max_rank) {
  if (n_rows <= 0 || cap <= 0 || max_rank < 1 || max_rank > 128) return 0;
  // The call launches m windows at a time, m from 1 (a launch minimum of one
  // row, or the fallback where a group would pass the 4 GiB buffer range,
  // which depends on n_out) up to the default minimum's m_max: the largest
  // need over every such m, without reading any override. Two slots of m
  // windows while they cover fewer than n_rows rows (largest at the largest
  // such m), one slot of every row otherwise.
  const int64_t m_max = windows_per_launch(cap, kAllMinRows);
  const int64_t n_caps = (n_rows + cap - 1) / cap;  // windows
  int64_t need = 0;
  const int64_t m_two = m_max < n_caps - 1 ? m_max : n_caps - 1;  // m with m * cap < n_rows
  if (m_two >= 1) need = 2 * pipe_slot_bytes(cap * m_two, max_rank);
  if (m_max >= n_caps) {
    const int64_t one = pipe_slot_bytes(n_rows, max_rank);
    if (one > need) need = one;
  }
  return (uint64_t)need;
}

extern "C" void mlora_reload_launch_overrides(void) {
  overrides();  // the first read, if it has not happened yet
  g_overrides = read_overrides();
}

// ---- the all-windows call without a caller workspace ----

// Scratch of mlora_grouped_down_all_noalloc: the two launch slots of the
// all-windows call live here instead of in a caller workspace. Each device
// the library runs on holds its own copy until the process ends; host code
// never uses the name itself as an address, only the per-device address
// looked up below.
constexpr uint64_t kScratchBytes = MLORA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept. The caller's stream must belong
// to the current device.
static int32_t scratch_address(hipStream_t s, void** out, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLORA_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MLORA_ERR_INVALID, "%s: device %d outside 0..%d", who, dev, kMaxDevices - 1);
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess)
      return fail(MLORA_ERR_HIP, "%s: hipStreamGetDevice: %s", who, hipGetErrorString(e));
    if (sdev != dev)
      return fail(MLORA_ERR_INVALID, "%s: the stream belongs to device %d, device %d is current",
                  who, (int)sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MLORA_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLORA_OK;
}

static int32_t grouped_down_all_impl(const mlora_expert_route* route, const void* x,
                                     int64_t n_tokens,
                              void* base_out, int64_t n_rows, const int32_t* expert_offsets,
                              int32_t n_route, const int32_t* sorted_ids,
                              const int32_t* row_adapter, int32_t top_k, int64_t cap,
                              void* workspace, uint64_t workspace_bytes, void* stream,
                              bool use_scratch) {
  const char* who = use_scratch ? "mlora_grouped_down_all_noalloc" : "mlora_grouped_down_all";
  if (int32_t rc = check_route(route, who)) return rc;
  if (top_k <= 0) return fail(MLORA_ERR_INVALID, "%s: top_k=%d must be positive", who, top_k);
  if (n_route < 0) return fail(MLORA_ERR_INVALID, "%s: n_route < 0", who);
  if (n_tokens < 0 || n_tokens > 0x3fffffffll)
    return fail(MLORA_ERR_INVALID, "%s: n_tokens out of range", who);
  if (n_rows < 0) return fail(MLORA_ERR_INVALID, "%s: n_rows < 0", who);
  if (cap <= 0) return fail(MLORA_ERR_INVALID, "%s: cap=%lld must be positive", who, (long long)cap);
  if (!workspace && workspace_bytes != 0)
    return fail(MLORA_ERR_INVALID, "%s: NULL workspace with workspace_bytes > 0", who);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLORA_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
  if (n_rows == 0 || route->n_experts == 0 || n_route == 0) {
    clear_error();
    return MLORA_OK;
  }
  if (!x || !base_out || !expert_offsets || !sorted_ids || !row_adapter)
    return fail(MLORA_ERR_INVALID, "%s: NULL device pointer", who);
  const int R = route->max_rank, N = route->n_out, K = route->k_in;
  // launches of whole windows; back to one window per launch where a larger
  // launch would pass the 4 GiB buffer range
  int64_t chunk = all_chunk_rows(n_rows, cap);
  if (chunk > cap && chunk > (int64_t)kMaxBufBytes / (2 * (int64_t)N))
    chunk = cap < n_rows ? cap : n_rows;
  const int64_t n_win = (n_rows + chunk - 1) / chunk;
  const int64_t slot = pipe_slot_bytes(chunk, R);
  const int64_t need = (n_win > 1 ? 2 : 1) * slot;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (use_scratch && route->dtype == MLORA_BF16) {
    if ((uint64_t)need > kScratchBytes)
      return fail(MLORA_ERR_CAPACITY,
                  "%s: needs %lld bytes of scratch, more than the %llu bytes it holds; lower "
                  "cap or max_rank, or pass a workspace to mlora_grouped_down_all",
                  who, (long long)need, (unsigned long long)kScratchBytes);
    if (int32_t rc = scratch_address(s, &workspace, who)) return rc;
    workspace_bytes = kScratchBytes;
  }
  if (route->dtype == MLORA_BF16 && (!workspace || (uint64_t)need > workspace_bytes))
    return fail(MLORA_ERR_CAPACITY, "%s: workspace of %llu bytes, %lld needed", who,
                (unsigned long long)workspace_bytes, (long long)need);
  (void)hipGetLastError();

  if (route->dtype == MLORA_F32) {
    // the plain row-wise kernel has no windows to pipeline: one launch per window
    const int64_t n_cap = (n_rows + cap - 1) / cap;
    for (int64_t w = 0; w < n_cap; ++w) {
      const int64_t r0 = w * cap, r1 = r0 + cap < n_rows ? r0 + cap : n_rows;
      if (int32_t rc = mlora_grouped_down(route, x, n_tokens, base_out, n_rows, expert_offsets,
                                          n_route, sorted_ids, row_adapter, top_k, r0, r1,
                                          nullptr, 0, stream))
        return rc;
    }
    clear_error();
    return MLORA_OK;
  }

  if (!aligned16(x) || !aligned16(base_out))
    return fail(MLORA_ERR_INVALID, "%s: x and base_out must be 16-byte aligned", who);
  const int64_t x_bytes = n_tokens * K * 2;
  const int64_t win_rows = chunk;
  const WsLayout wl = grouped_ws_layout(win_rows, R);
  if (x_bytes > (int64_t)kMaxBufBytes || win_rows * N * 2 > (int64_t)kMaxBufBytes ||
      wl.h_bytes > (int64_t)kMaxBufBytes || wl.meta_bytes > (int64_t)kMaxBufBytes ||
      (win_rows + 63) / 16 * ((N + kColStep - 1) / kColStep) > 0x3fffffffll)
    return fail(MLORA_ERR_INVALID, "%s: window of %lld rows too large; lower cap", who,
                (long long)win_rows);

  // arguments of window w (its rows, its workspace slot), with the shrink or
  // the expand launch fields
  auto window = [&](int64_t w, bool expand, int64_t* blocks) {
    GroupedArgs a{};
    const int64_t r0 = w * chunk, r1 = r0 + chunk < n_rows ? r0 + chunk : n_rows;
    const WsLayout l = grouped_ws_layout(r1 - r0, R);
    uint8_t* base = static_cast<uint8_t*>(workspace) + (w % 2) * slot;
    a.x = static_cast<const uint16_t*>(x);
    a.out = static_cast<uint16_t*>(base_out) + r0 * N;
    a.offsets = expert_offsets;
    a.sorted_ids = sorted_ids;
    a.row_adapter = row_adapter;
    a.a_table = route->a_table;
    a.b_table = route->b_table;
    a.scale_table = route->scale_table;
    a.x_bytes = (uint32_t)x_bytes;
    a.out_bytes = (uint32_t)((r1 - r0) * N * 2);
    a.row_offset = r0;
    a.row_end = r1;
    a.n_experts = route->n_experts;
    a.K = K;
    a.N = N;
    a.R = R;
    a.n_route = n_route;
    a.top_k = top_k;
    a.n_tokens = (int32_t)n_tokens;
    a.top_k_magic = magic_for(top_k);
    a.ws_h = base;
    a.ws_meta = reinterpret_cast<uint64_t*>(base + l.meta_off);
    a.ws_h_bytes = (uint32_t)l.h_bytes;
    a.ws_meta_bytes = (uint32_t)l.meta_bytes;
    const TwoPlan t = two_plan(R, N, r1 - r0, true);
    if (!expand) {
      a.units = (int32_t)t.sunits;
      a.per_xcd = (int32_t)((t.sunits + kXcds - 1) / kXcds);
      *blocks = (int64_t)a.per_xcd * kXcds;
    } else {
      a.ns_count = (int32_t)t.eslices;
      a.units = (int32_t)(t.etiles * t.eslices);
      *blocks = (a.units + kWaves - 1) / kWaves;  // four expand waves per pipe block
    }
    return a;
  };
  const TwoPlan plan = two_plan(R, N, win_rows, true);
  const int cw = plan.cw, emb = plan.emb;
  int64_t nb = 0;
  GroupedArgs first = window(0, false, &nb);
  {
    // the first shrink runs alone: its tile may differ from the pipe kernel's
    const int fmb = shrink_tile_mb(R, ov(overrides().shrink_mb, plan.smb));
    const int64_t rows0 = first.row_end - first.row_offset;
    const int64_t units = (rows0 + 16 * fmb - 1) / (16 * fmb);
    first.units = (int32_t)units;
    first.per_xcd = (int32_t)((units + kXcds - 1) / kXcds);
    nb = (int64_t)first.per_xcd * kXcds;
    dispatch_shrink(first, (int)nb, s, fmb);
  }
  if (int32_t rc = launched(who)) return rc;
  for (int64_t w = 1; w < n_win; ++w) {
    int64_t sb = 0, eb = 0;
    const GroupedArgs ps = window(w, false, &sb);
    GroupedArgs pe = window(w - 1, true, &eb);
    const int64_t grid = sb + expand_grid(pe);  // eb expand blocks, per_xcd * kXcds >= eb
    dispatch_pipe(ps, pe, (int)grid, s, emb, cw);
    if (int32_t rc = launched(who)) return rc;
  }
  int64_t lb = 0;
  GroupedArgs last = window(n_win - 1, true, &lb);
  dispatch_expand(last, (int)expand_grid(last), s, emb, cw);
  return launched(who);
}

extern "C" int32_t mlora_grouped_down_all(const mlora_expert_route* route, const void* x,
                                          int64_t n_tokens, void* base_out, int64_t n_rows,
                                          const int32_t* expert_offsets, int32_t n_route,
                                          const int32_t* sorted_ids, const int32_t* row_adapter,
                                          int32_t top_k, int64_t cap, void* workspace,
                                          uint64_t workspace_bytes, void* stream) {
  return grouped_down_all_impl(route, x, n_tokens, base_out, n_rows, expert_offsets, n_route,
                               sorted_ids, row_adapter, top_k, cap, workspace, workspace_bytes,
                               stream, false);
}

extern "C" int32_t mlora_grouped_down_all_noalloc(const mlora_expert_route* route,
                                                  const void* x, int64_t n_tokens,
                                                  void* base_out, int64_t n_rows,
                                                  const int32_t* expert_offsets, int32_t n_route,
                                                  const int32_t* sorted_ids,
                                                  const int32_t* row_adapter, int32_t top_k,
                                                  int64_t cap, void* stream) {
  return grouped_down_all_impl(route, x, n_tokens, base_out, n_rows, expert_offsets, n_route,
                               sorted_ids, row_adapter, top_k, cap, nullptr, 0, stream, true);
}
