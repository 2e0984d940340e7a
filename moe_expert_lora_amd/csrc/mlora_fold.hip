// Device folds of libmlora.so for gfx950 (MI355X): the gather (decode) and
// grouped (prefill) MoE expert-LoRA folds of the "moe_lora_grouped" module
// index page, items moe_lora_gather_bgmv and moe_lora_grouped_down:
//
//     base_out[row] += scale_e * ((x[token(row)] @ A_e^T) @ B_e^T)
//
// Design (one fused kernel per call, no device scratch):
//  * A work unit is (expert e, up to 16*MB rows of e, a column range of
//    base_out). The shrink H = X A_e^T and the expand base + s H B_e^T both
//    run on bf16 MFMA (v_mfma_f32_16x16x32_bf16), with fp32 accumulation.
//  * Shrink, transposed: D[rank][row] = A_e[rank,:] . x[row,:]. The 4 waves
//    split k_in; partial sums meet in LDS and are added in a fixed order.
//    A rank permutation makes each lane end up holding 4*NB consecutive ranks
//    of one row, which is exactly the operand layout the expand needs.
//  * H is scaled by scale_e and split into hi + lo bf16 halves, so the expand
//    MFMA sees H to ~16 mantissa bits (rounding H to one bf16 alone would use
//    most of the error budget that the final bf16 store leaves).
//  * Expand, transposed: D[col][row] = B_e[col,:] . H'[:,row] with
//    K' = 2*max_rank (hi then lo). A column permutation gives each lane a run
//    of 8 consecutive output columns of one row, so base_out is read and
//    written with 16-byte accesses, 64 contiguous bytes per row per
//    instruction, and never staged through LDS.
//  * Gather rows are grouped by expert on the device: each workgroup scans a
//    slice of `indices` for its expert, so each A_e / B_e is streamed from HBM
//    once per workgroup group and reused across that expert's rows.
//  * Grouped rows come in MLORA_MLG_M_TILE-row tiles; a tile that straddles
//    expert spans is folded one span segment at a time.
//  * Workgroup ids are mapped so that consecutive work units (the splits of
//    one expert, or neighbouring row tiles) run on the same XCD and share its
//    L2.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>

#include "mlora.h"
#include "mlora_internal.h"

namespace mlora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileRows = MLORA_MLG_M_TILE;
constexpr int kColStep = 32;     // output columns per expand step of one wave
constexpr int kScanMax = 2048;   // gather rows scanned by one workgroup
constexpr int kMaxSegs = kTileRows;
constexpr int kXcds = 8;

static_assert(kTileRows == 64, "grouped tiles are 64 rows (4 row blocks of 16)");

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Appends `val` pairs of the lanes whose `pred` is set to LDS lists, in one
// LDS atomic per wave. Order across waves is unspecified; nothing downstream
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

// ---------------------------------------------------------------------------
// the per-expert tile engine
// ---------------------------------------------------------------------------

// B_e fragment of one expand step: for each of the 2 column blocks, the lane's
// 4*NB ranks (rank g*4NB .. g*4NB+4NB-1) of one B_e row, as 2*NB words.
template <int NB>
struct BFrag {
  uint32_t w[2][2 * NB];
};

// Output column (relative to the step start) of MFMA row `mi` in column block
// `cb`: lane group g of the result then holds the 8 consecutive columns
// 8g .. 8g+7 of its row (4 from each block).
__device__ __forceinline__ int col_of(int cb, int mi) {
  return (mi >> 2) * 8 + cb * 4 + (mi & 3);
}

template <int NB, bool FULL_R>
__device__ __forceinline__ void load_bfrag(BFrag<NB>& f, const uint16_t* __restrict__ B, int R,
                                           int c0, int n_hi, int li, int g) {
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int col = c0 + col_of(cb, li);
    if (col < n_hi) {
      const uint16_t* p = B + (size_t)col * R + g * 4 * NB;
      if constexpr (FULL_R) {
        if constexpr (NB == 1) {
          const u32x2 v = ld8(p);
          f.w[cb][0] = v.x;
          f.w[cb][1] = v.y;
        } else {
#pragma unroll
          for (int q = 0; q < NB / 2; ++q) {
            const u32x4 v = ld16(p + 8 * q);
            f.w[cb][4 * q + 0] = v.x;
            f.w[cb][4 * q + 1] = v.y;
            f.w[cb][4 * q + 2] = v.z;
            f.w[cb][4 * q + 3] = v.w;
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 2 * NB; ++q) {
          const int r0 = g * 4 * NB + 2 * q;
          const uint32_t lo = (r0 < R) ? p[2 * q] : 0u;
          const uint32_t hi = (r0 + 1 < R) ? p[2 * q + 1] : 0u;
          f.w[cb][q] = lo | (hi << 16);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2 * NB; ++q) f.w[cb][q] = 0u;
    }
  }
}

// base_out fragment of one expand step: per row block, the lane's run of 8
// columns (16 bytes).
template <int MB>
struct OutFrag {
  u32x4 v[MB];
};

template <int MB>
__device__ __forceinline__ void load_out(OutFrag<MB>& f, const uint16_t* const (&orowp)[MB],
                                         const bool (&valid)[MB], int nrb, int col, int n_hi) {
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    if (rb < nrb) {
      if (valid[rb] && col < n_hi)
        f.v[rb] = ld16(orowp[rb] + col);
      else
        f.v[rb] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Folds rows 0..nrows-1 (nrows <= 16*MB) of expert (A, B, scale) into columns
// [n_lo, n_hi) of base_out. Row m writes base_out row
// (s_row ? s_row[m] : row_base + m) from token s_tok[m] (negative: dead row).
// All threads of the workgroup must call it with the same arguments.
template <int NB, int MB, bool FULL_R>
__device__ void fold_rows(const uint16_t* __restrict__ x, uint16_t* __restrict__ out, int K,
                          int N, int R, const uint16_t* __restrict__ A,
                          const uint16_t* __restrict__ B, float scale,
                          const int* s_row, int64_t row_base, const int* s_tok, int nrows,
                          int n_lo, int n_hi, float* s_part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int nrb = (nrows + 15) >> 4;

  const uint16_t* xrow[MB];
  const uint16_t* orowp[MB];
  bool valid[MB];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb) {
    const int m = rb * 16 + li;
    int t = -1;
    int64_t r = 0;
    if (m < nrows) {
      t = s_tok[m];
      r = s_row ? (int64_t)s_row[m] : row_base + m;
    }
    valid[rb] = t >= 0;
    xrow[rb] = x + (size_t)(t < 0 ? 0 : t) * K;
    orowp[rb] = out + (size_t)r * N;
  }

  // The first expand step's operands do not depend on the shrink: issue them
  // now so their latency hides behind it.
  const int ncs = (n_hi - n_lo + kColStep - 1) / kColStep;
  BFrag<NB> bcur;
  OutFrag<MB> ocur;
  if (wave < ncs) {
    const int c0 = n_lo + wave * kColStep;
    load_bfrag<NB, FULL_R>(bcur, B, R, c0, n_hi, li, g);
    load_out<MB>(ocur, orowp, valid, nrb, c0 + 8 * g, n_hi);
  }

  // ---- shrink: H[rank][row] over this wave's k steps ----------------------
  f32x4 hacc[MB][NB];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int b = 0; b < NB; ++b) hacc[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = (K + 31) >> 5;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int s = wave; s < nks; s += kWaves) {
    const int k0 = s * 32 + g * 8;
    const bool kin = k0 < K;
    bf16x8 af[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int rank = (li >> 2) * 4 * NB + 4 * b + (li & 3);
      af[b] = as_bf((kin && rank < R) ? ld16(A + (size_t)rank * K + k0) : zero4);
    }
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      if (rb < nrb) {
        const bf16x8 xf = as_bf((kin && valid[rb]) ? ld16(xrow[rb] + k0) : zero4);
#pragma unroll
        for (int b = 0; b < NB; ++b) hacc[rb][b] = mfma16x16x32(af[b], xf, hacc[rb][b]);
      }
    }
  }

  // ---- K-split reduction through LDS (fixed order) -----------------------
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
  __syncthreads();

  // H' operands: per row block and k step s, {hi[4s..4s+3], lo[4s..4s+3]}.
  u32x4 hop[MB][NB];
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
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v = scale * h[q];
          hi[q] = f2bf(v);
          lo[q] = f2bf(v - bf2f(hi[q]));
        }
        hop[rb][s] = u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                           lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
      }
    }
  }

  // ---- expand + read-modify-write ------------------------------------------
  for (int cs = wave; cs < ncs; cs += kWaves) {
    const int col = n_lo + cs * kColStep + 8 * g;
    BFrag<NB> bnext;
    OutFrag<MB> onext;
    const bool more = cs + kWaves < ncs;
    if (more) {
      const int c1 = n_lo + (cs + kWaves) * kColStep;
      load_bfrag<NB, FULL_R>(bnext, B, R, c1, n_hi, li, g);
      load_out<MB>(onext, orowp, valid, nrb, c1 + 8 * g, n_hi);
    }
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      if (rb < nrb) {
        f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          const bf16x8 hb = as_bf(hop[rb][s]);
          const uint32_t a0 = bcur.w[0][2 * s], a1 = bcur.w[0][2 * s + 1];
          const uint32_t b0 = bcur.w[1][2 * s], b1 = bcur.w[1][2 * s + 1];
          d0 = mfma16x16x32(as_bf(u32x4{a0, a1, a0, a1}), hb, d0);
          d1 = mfma16x16x32(as_bf(u32x4{b0, b1, b0, b1}), hb, d1);
        }
        if (valid[rb] && col < n_hi) {
          const u32x4 bv = ocur.v[rb];
          const uint32_t o0 = f2bf(bf2f(bv.x & 0xffffu) + d0.x) |
                              (f2bf(bf2f(bv.x >> 16) + d0.y) << 16);
          const uint32_t o1 = f2bf(bf2f(bv.y & 0xffffu) + d0.z) |
                              (f2bf(bf2f(bv.y >> 16) + d0.w) << 16);
          const uint32_t o2 = f2bf(bf2f(bv.z & 0xffffu) + d1.x) |
                              (f2bf(bf2f(bv.z >> 16) + d1.y) << 16);
          const uint32_t o3 = f2bf(bf2f(bv.w & 0xffffu) + d1.z) |
                              (f2bf(bf2f(bv.w >> 16) + d1.w) << 16);
          st16(const_cast<uint16_t*>(orowp[rb]) + col, u32x4{o0, o1, o2, o3});
        }
      }
    }
    if (more) {
      bcur = bnext;
      ocur = onext;
    }
  }
  // s_part and the caller's row lists are reused by the next call.
  __syncthreads();
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
  int32_t n_experts, K, N, R, n_slots, top_k;
  int32_t rs_count;   // row slices per expert
  int32_t ns_count;   // column slices per expert
  int32_t scan_len;   // rows per row slice (<= kScanMax)
  int32_t ns_cols;    // columns per column slice (multiple of kColStep)
  int32_t units;      // n_experts * rs_count * ns_count
  int32_t per_xcd;    // ceil(units / kXcds)
};

template <int NB, int MB, bool FULL_R>
__global__ __launch_bounds__(kThreads) void gather_fold_kernel(GatherArgs p) {
  __shared__ float s_part[kWaves * MB * 64 * 4 * NB];
  __shared__ int s_rows[kScanMax];
  __shared__ int s_toks[kScanMax];
  __shared__ int s_cnt;

  // XCD-aware unit: consecutive units (the slices of one expert) on one XCD.
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * p.per_xcd + slot;
  if (u >= p.units) return;
  const int per_e = p.rs_count * p.ns_count;
  const int e = u / per_e;
  const int within = u - e * per_e;
  const int rs = within / p.ns_count, ns = within - rs * p.ns_count;

  const uint64_t a_addr = p.a_table[e], b_addr = p.b_table[e];
  if (a_addr == 0 || b_addr == 0) return;
  const float scale = p.scale_table[e];

  if (threadIdx.x == 0) s_cnt = 0;
  __syncthreads();

  // Rows of this slice routed to e with a live adapter map entry.
  const int start = rs * p.scan_len;
  const int end = min(start + p.scan_len, p.n_slots);
  constexpr int kPer = kScanMax / kThreads;
  int iv[kPer], mv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int row = start + i * kThreads + (int)threadIdx.x;
    iv[i] = -1;
    mv[i] = -1;
    if (row < end) {
      iv[i] = p.indices[row];
      mv[i] = p.row_adapter[row / p.top_k];
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int row = start + i * kThreads + (int)threadIdx.x;
    const bool hit = row < end && iv[i] == e && mv[i] >= 0;
    wave_append(hit, row, row / p.top_k, &s_cnt, s_rows, s_toks, kScanMax);
  }
  __syncthreads();
  const int n = s_cnt;

  const int n_lo = ns * p.ns_cols;
  const int n_hi = min(n_lo + p.ns_cols, p.N);
  const uint16_t* A = reinterpret_cast<const uint16_t*>(a_addr);
  const uint16_t* B = reinterpret_cast<const uint16_t*>(b_addr);
  for (int c = 0; c < n; c += 16 * MB)
    fold_rows<NB, MB, FULL_R>(p.x, p.out, p.K, p.N, p.R, A, B, scale, s_rows + c, 0,
                              s_toks + c, min(16 * MB, n - c), n_lo, n_hi, s_part);
}

// ---------------------------------------------------------------------------
// grouped (prefill) kernel
// ---------------------------------------------------------------------------

struct GroupedArgs {
  const uint16_t* x;
  uint16_t* out;
  const int32_t* offsets;
  const int32_t* sorted_ids;
  const int32_t* row_adapter;
  const uint64_t* a_table;
  const uint64_t* b_table;
  const float* scale_table;
  int64_t row_offset, row_end;
  int32_t n_experts, K, N, R, n_route, top_k, n_tokens;
  int32_t n_tiles, ns_count, ns_cols, units, per_xcd;
};

template <int NB, int MB, bool FULL_R>
__global__ __launch_bounds__(kThreads) void grouped_fold_kernel(GroupedArgs p) {
  __shared__ float s_part[kWaves * MB * 64 * 4 * NB];
  __shared__ int s_tok[kTileRows];
  __shared__ int s_seg_e[kMaxSegs], s_seg_lo[kMaxSegs], s_seg_hi[kMaxSegs];
  __shared__ int s_nseg;

  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * p.per_xcd + slot;
  if (u >= p.units) return;
  const int t = u / p.ns_count, ns = u - t * p.ns_count;
  const int64_t r0 = p.row_offset + (int64_t)t * kTileRows;
  const int64_t r1 = min(r0 + kTileRows, p.row_end);

  if (threadIdx.x == 0) s_nseg = 0;
  __syncthreads();

  // Expert spans that meet this tile, clipped to it.
  for (int e = threadIdx.x; e < p.n_route; e += kThreads) {
    const int64_t lo = max((int64_t)p.offsets[e], r0);
    const int64_t hi = min((int64_t)p.offsets[e + 1], r1);
    if (lo < hi) {
      const int k = atomicAdd(&s_nseg, 1);
      if (k < kMaxSegs) {
        s_seg_e[k] = e;
        s_seg_lo[k] = (int)(lo - r0);
        s_seg_hi[k] = (int)(hi - r0);
      }
    }
  }
  // Token of each tile row, or -1 when the row folds nothing.
  if (threadIdx.x < kTileRows) {
    const int64_t r = r0 + threadIdx.x;
    int tk = -1;
    if (r < r1) {
      const int id = p.sorted_ids[r];
      if (id >= 0) {
        const int cand = id / p.top_k;
        if (cand < p.n_tokens && p.row_adapter[cand] >= 0) tk = cand;
      }
    }
    s_tok[threadIdx.x] = tk;
  }
  __syncthreads();
  const int nseg = min(s_nseg, kMaxSegs);

  const int n_lo = ns * p.ns_cols;
  const int n_hi = min(n_lo + p.ns_cols, p.N);
  for (int sg = 0; sg < nseg; ++sg) {
    const int e = s_seg_e[sg];
    if (e >= p.n_experts) continue;
    const uint64_t a_addr = p.a_table[e], b_addr = p.b_table[e];
    if (a_addr == 0 || b_addr == 0) continue;
    const float scale = p.scale_table[e];
    const int lo = s_seg_lo[sg], hi = s_seg_hi[sg];
    for (int c = lo; c < hi; c += 16 * MB)
      fold_rows<NB, MB, FULL_R>(p.x, p.out, p.K, p.N, p.R,
                                reinterpret_cast<const uint16_t*>(a_addr),
                                reinterpret_cast<const uint16_t*>(b_addr), scale, nullptr,
                                r0 + c, s_tok + c, min(16 * MB, hi - c), n_lo, n_hi, s_part);
  }
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
  __syncthreads();
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

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

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

template <int NB, int MB, bool FULL_R>
void launch_gather(const GatherArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((gather_fold_kernel<NB, MB, FULL_R>), dim3(grid), dim3(kThreads), 0, s, a);
}

template <int NB, int MB, bool FULL_R>
void launch_grouped(const GroupedArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((grouped_fold_kernel<NB, MB, FULL_R>), dim3(grid), dim3(kThreads), 0, s, a);
}

// Rank blocks of 16 -> (NB, MB) instantiation.
#define MLORA_DISPATCH(FN, ARGS, GRID, STREAM, R)                        \
  do {                                                                   \
    const int nb_ = ((R) + 15) / 16;                                     \
    if (nb_ <= 1) {                                                      \
      if ((R) == 16) FN<1, 4, true>(ARGS, GRID, STREAM);                 \
      else FN<1, 4, false>(ARGS, GRID, STREAM);                          \
    } else if (nb_ <= 2) {                                               \
      if ((R) == 32) FN<2, 4, true>(ARGS, GRID, STREAM);                 \
      else FN<2, 4, false>(ARGS, GRID, STREAM);                          \
    } else if (nb_ <= 4) {                                               \
      if ((R) == 64) FN<4, 2, true>(ARGS, GRID, STREAM);                 \
      else FN<4, 2, false>(ARGS, GRID, STREAM);                          \
    } else {                                                             \
      if ((R) == 128) FN<8, 1, true>(ARGS, GRID, STREAM);                \
      else FN<8, 1, false>(ARGS, GRID, STREAM);                          \
    }                                                                    \
  } while (0)

}  // namespace
}  // namespace mlora

using namespace mlora;

extern "C" int32_t mlora_gather_bgmv(const mlora_expert_route* route, const void* x,
                                     int64_t n_tokens, void* base_out, const int32_t* indices,
                                     const int32_t* row_adapter, int64_t n_slots, int32_t top_k,
                                     void* stream) {
  const char* who = "mlora_gather_bgmv";
  if (int32_t rc = check_route(route, who)) return rc;
  if (top_k <= 0) return fail(MLORA_ERR_INVALID, "%s: top_k=%d must be positive", who, top_k);
  if (n_slots < 0 || n_slots > (int64_t)0x7fffffff - kScanMax)
    return fail(MLORA_ERR_INVALID, "%s: n_slots=%lld out of range", who, (long long)n_slots);
  const int64_t need_tok = (n_slots + top_k - 1) / top_k;
  if (n_tokens < need_tok)
    return fail(MLORA_ERR_INVALID, "%s: n_tokens=%lld < ceil(n_slots/top_k)=%lld", who,
                (long long)n_tokens, (long long)need_tok);
  if (n_slots == 0 || route->n_experts == 0) {
    clear_error();
    return MLORA_OK;
  }
  if (!x || !base_out || !indices || !row_adapter)
    return fail(MLORA_ERR_INVALID, "%s: NULL device pointer", who);
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

  if (!aligned16(x) || !aligned16(base_out))
    return fail(MLORA_ERR_INVALID, "%s: x and base_out must be 16-byte aligned", who);
  const int E = route->n_experts, K = route->k_in, N = route->n_out, R = route->max_rank;
  const int ns_max = (N + kColStep - 1) / kColStep;

  // Launch shape. Row slices first (each slice scans at most kScanMax rows),
  // then more row slices while slices keep enough rows, then column slices
  // while the repeated shrink stays cheaper than the expand it splits.
  const int64_t rows_per_e = (n_slots + E - 1) / E;
  int rs = (int)((n_slots + kScanMax - 1) / kScanMax);
  int ns = 1;
  const int64_t target = 512;
  while ((int64_t)E * rs * ns < target && rows_per_e / (rs * 2) >= 32)
    rs *= 2;
  const double shrink_b = 2.0 * R * K + 2.0 * (double)rows_per_e / rs * K;
  const double expand_b = 2.0 * N * R + 4.0 * (double)rows_per_e / rs * N;
  while ((int64_t)E * rs * ns < target && ns * 2 <= ns_max &&
         (ns * 2) * shrink_b <= shrink_b + expand_b)
    ns *= 2;
  rs = env_int("MLORA_GATHER_RS", rs);
  ns = env_int("MLORA_GATHER_NS", ns);
  if (ns < 1) ns = 1;
  if (ns > ns_max) ns = ns_max;
  if (rs < 1) rs = 1;
  int scan = (int)((n_slots + rs - 1) / rs);
  if (scan > kScanMax) {
    rs = (int)((n_slots + kScanMax - 1) / kScanMax);
    scan = (int)((n_slots + rs - 1) / rs);
  }

  GatherArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.out = static_cast<uint16_t*>(base_out);
  a.indices = indices;
  a.row_adapter = row_adapter;
  a.a_table = route->a_table;
  a.b_table = route->b_table;
  a.scale_table = route->scale_table;
  a.n_experts = E;
  a.K = K;
  a.N = N;
  a.R = R;
  a.n_slots = (int32_t)n_slots;
  a.top_k = top_k;
  a.rs_count = rs;
  a.ns_count = ns;
  a.scan_len = scan;
  a.ns_cols = ns_cols_for(N, ns);
  const int64_t units = (int64_t)E * rs * ns;
  if (units > 0x7fffffffll / 2)
    return fail(MLORA_ERR_INVALID, "%s: launch too large", who);
  a.units = (int32_t)units;
  a.per_xcd = (int32_t)((units + kXcds - 1) / kXcds);
  const int grid = a.per_xcd * kXcds;
  MLORA_DISPATCH(launch_gather, a, grid, s, R);
  return launched(who);
}

extern "C" int32_t mlora_grouped_down(const mlora_expert_route* route, const void* x,
                                      int64_t n_tokens, void* base_out, int64_t n_rows,
                                      const int32_t* expert_offsets, int32_t n_route,
                                      const int32_t* sorted_ids, const int32_t* row_adapter,
                                      int32_t top_k, int64_t row_offset, int64_t row_end,
                                      void* stream) {
  const char* who = "mlora_grouped_down";
  if (int32_t rc = check_route(route, who)) return rc;
  if (top_k <= 0) return fail(MLORA_ERR_INVALID, "%s: top_k=%d must be positive", who, top_k);
  if (n_route < 0) return fail(MLORA_ERR_INVALID, "%s: n_route < 0", who);
  if (n_tokens < 0 || n_tokens > 0x7fffffffll)
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
  const int64_t tiles = mlora_grouped_down_wc(row_offset, row_end);
  const int ns_max = (N + kColStep - 1) / kColStep;
  // Column slices while the grid is short of two workgroups per CU and the
  // repeated shrink (x rows + A_e) stays below the expand bytes it splits.
  int ns = 1;
  const double shrink_b = 2.0 * kTileRows * K + 2.0 * R * K;
  const double expand_b = 4.0 * kTileRows * N + 2.0 * N * R;
  while (tiles * ns < 512 && ns * 2 <= ns_max && (ns * 2) * shrink_b <= shrink_b + expand_b)
    ns *= 2;
  ns = env_int("MLORA_GROUPED_NS", ns);
  if (ns < 1) ns = 1;
  if (ns > ns_max) ns = ns_max;
  const int64_t units = tiles * ns;
  if (units > 0x7fffffffll / 2) return fail(MLORA_ERR_INVALID, "%s: window too large", who);

  GroupedArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.out = static_cast<uint16_t*>(base_out);
  a.offsets = expert_offsets;
  a.sorted_ids = sorted_ids;
  a.row_adapter = row_adapter;
  a.a_table = route->a_table;
  a.b_table = route->b_table;
  a.scale_table = route->scale_table;
  a.row_offset = row_offset;
  a.row_end = row_end;
  a.n_experts = route->n_experts;
  a.K = K;
  a.N = N;
  a.R = R;
  a.n_route = n_route;
  a.top_k = top_k;
  a.n_tokens = (int32_t)n_tokens;
  a.n_tiles = (int32_t)tiles;
  a.ns_count = ns;
  a.ns_cols = ns_cols_for(N, ns);
  a.units = (int32_t)units;
  a.per_xcd = (int32_t)((units + kXcds - 1) / kXcds);
  const int grid = a.per_xcd * kXcds;
  MLORA_DISPATCH(launch_grouped, a, grid, s, R);
  return launched(who);
}
