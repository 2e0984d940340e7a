// Measurement probes for bench.py (not part of the fold's interface): the
// floors that bound what one launch of the fold can do on this part.
//
//   mlora_probe_empty      cost of an empty kernel launch, eager and inside a
//                          HIP graph (the fixed cost every fold launch pays).
//   mlora_probe_read       read bandwidth of 8192 rows of 4096 bytes (the row
//                          of a k_in = 2048 bf16 operand) at a given row
//                          stride, in the access pattern of the folds' MFMA
//                          operands (16 rows x 64 bytes per wave instruction,
//                          step pairs completing 128-byte lines), one row's
//                          1 KB per wave instruction, or one row's 1 KB per
//                          instruction straight into LDS and read back there
//                          in the operand pattern; buffers rotated past L2
//                          and MALL.
//   mlora_probe_rmw        read-modify-write rate of a 16384 x 2048 bf16
//                          buffer (64 MiB, the base_out of one prefill launch
//                          group) in the grouped expand's wave tile (32 rows x
//                          128 columns, 4 rows x 256 bytes per instruction),
//                          one row's 1 KB per instruction, or a workgroup's
//                          contiguous 32 KB; units in the hardware's block
//                          order or each XCD on a contiguous eighth; plain or
//                          non-temporal loads and stores.
//   mlora_probe_stream     a launch shaped like the decode fold with no
//                          dependent load: `units` workgroups, each reading
//                          its own region of weight bytes and
//                          reading-modifying-writing its own region of row
//                          bytes, requested at kernel start; replayed in a
//                          HIP graph over rotated buffers. The floor of what
//                          one launch of those bytes can take.
//
// Each entry point allocates and frees its own buffers, synchronizes the
// device and returns 0, or a HIP error code.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 8192;
constexpr int kRowBytes = 4096;
constexpr int kThreads = 512;  // 8 waves; 256 workgroups of 32 rows

__global__ void empty_kernel() {}

__device__ __forceinline__ u32x4 ld16(const char* p, size_t off) {
  return *reinterpret_cast<const u32x4*>(p + off);
}

// Workgroup b reads rows 32b .. 32b+31. Wave w takes the 64-byte steps
// 2w, 2w+1, 2w+16, 2w+17, ... of each row (the folds' step pairs), lane
// (li, g) the 16 bytes g of row li of a 16-row block.
__global__ __launch_bounds__(kThreads) void read_operand_kernel(const char* x, unsigned* sink,
                                                               int stride) {
  const int b = blockIdx.x, w = threadIdx.x >> 6, l = threadIdx.x & 63, li = l & 15, g = l >> 4;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 v[8][2];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int s = 2 * w + (t & 1) + 16 * (t >> 1);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      v[t][rb] = ld16(x, (size_t)(32 * b + 16 * rb + li) * stride + 64 * s + 16 * g);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc ^= v[t][rb];
  sink[blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Same rows, one row's 1 KB per wave instruction.
__global__ __launch_bounds__(kThreads) void read_rows_kernel(const char* x, unsigned* sink,
                                                            int stride) {
  const int b = blockIdx.x, w = threadIdx.x >> 6, l = threadIdx.x & 63;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int idx = i * 8 + w;  // 128 pieces of 1 KB: (row, quarter)
    const int row = 32 * b + (idx >> 2), q = idx & 3;
    v[i] = ld16(x, (size_t)row * stride + q * 1024 + 16 * l);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) acc ^= v[i];
  sink[blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Same rows and the same per-lane data as read_operand_kernel, but moved in
// 1 KB row pieces straight into LDS (buffer loads with the LDS flag: lane l
// of an instruction lands at the instruction's LDS base + 16 l) and read
// back by every wave in the operand layout. Rows sit 4112 bytes apart in LDS
// so that the 16 rows of an operand read fall on different banks.
constexpr int kLdsPitch = kRowBytes + 16;
constexpr int kLdsBytes = 32 * kLdsPitch;

__global__ __launch_bounds__(kThreads) void read_lds_kernel(const char* x, unsigned* sink,
                                                           int stride) {
  __shared__ __attribute__((aligned(16))) char s_x[kLdsBytes];
  const int b = blockIdx.x, w = threadIdx.x >> 6, l = threadIdx.x & 63, li = l & 15, g = l >> 4;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(x) + (size_t)32 * b * stride, 0, 32 * stride, 0x00020000);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int idx = i * 8 + w;  // 128 pieces of 1 KB: (row, quarter)
    const int row = idx >> 2, q = idx & 3;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(s_x + row * kLdsPitch + q * 1024), 16,
        row * stride + q * 1024 + 16 * l, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int st = 2 * w + (t & 1) + 16 * (t >> 1);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      acc ^= *reinterpret_cast<const u32x4*>(s_x + (16 * rb + li) * kLdsPitch + 64 * st + 16 * g);
  }
  sink[blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Read-modify-write probes: every 16-byte piece of the buffer gets one added
// to each word. 8192 wave units of 32 rows x 128 columns (tile) or 2 rows
// (row), four per 256-thread workgroup, or 2048 workgroups of a contiguous
// 32 KB each (flat): 2048 workgroups in every pattern.
constexpr int kRmwRows = 16384;
constexpr int kRmwRowBytes = 4096;
constexpr uint32_t kRmwBytes = (uint32_t)kRmwRows * kRmwRowBytes;
constexpr int kRmwUnits = 8192;
constexpr int kRmwBlocks = kRmwUnits / 4;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t rmw_buf(char* p) {
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)kRmwBytes, 0x00020000);
}
template <int AUX>
__device__ __forceinline__ u32x4 rmw_ld(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ void rmw_st(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, AUX);
}

// PATTERN 0 tile, 1 row, 2 flat; XCDC: block b's XCD (b % 8) takes units of
// its own contiguous eighth; AUX 0 plain, 2 non-temporal.
template <int PATTERN, bool XCDC, int AUX>
__global__ __launch_bounds__(256) void rmw_kernel(char* buf) {
  const rsrc_t r = rmw_buf(buf);
  const int b = blockIdx.x, w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int blk = XCDC ? (b % 8) * (kRmwBlocks / 8) + b / 8 : b;
  const int u = blk * 4 + w;
  uint32_t off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (PATTERN == 0) {  // rows 32*(u/16) .., columns 128*(u%16) ..
      const int row = (u >> 4) * 32 + i * 4 + (l >> 4);
      off[i] = (uint32_t)row * kRmwRowBytes + (uint32_t)((u & 15) * 128 + 8 * (l & 15)) * 2u;
    } else if constexpr (PATTERN == 1) {  // rows 2u, 2u+1, 1 KB per instruction
      off[i] = (uint32_t)(2 * u + (i >> 2)) * kRmwRowBytes + (uint32_t)(i & 3) * 1024u + 16u * l;
    } else {  // 32 KB from 32 KB * blk, 4 KB per workgroup instruction
      off[i] = (uint32_t)blk * 32768u + (uint32_t)i * 4096u + (uint32_t)threadIdx.x * 16u;
    }
  }
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = rmw_ld<AUX>(r, off[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) rmw_st<AUX>(r, off[i], v[i] + u32x4{1u, 1u, 1u, 1u});
}

// Stream probe: workgroup b reads w16 pieces of 16 bytes per thread of
// weights (its own region, 4 KB per workgroup instruction) and
// reads-modifies-writes r16 pieces per thread of rows (its own region), all
// loads issued before any use; pieces past the counts lie past the buffers
// (the resource's size), so they read 0 and their stores are dropped.
constexpr int kStreamMax = 16;  // pieces per thread of each kind (64 KB a workgroup)
constexpr uint32_t kPastEnd = 0xFFFFFFF0u;

__global__ __launch_bounds__(256) void stream_kernel(const char* w, char* rows, unsigned* sink,
                                                     int w16, int r16, uint32_t wbytes,
                                                     uint32_t rbytes) {
  const uint32_t t16 = threadIdx.x * 16u;
  const rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(w), 0, (int)wbytes,
                                                      0x00020000);
  const rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(rows, 0, (int)rbytes, 0x00020000);
  const uint32_t wb = blockIdx.x * (uint32_t)w16 * 4096u, rb = blockIdx.x * (uint32_t)r16 * 4096u;
  u32x4 wv[kStreamMax], rv[kStreamMax];
#pragma unroll
  for (int i = 0; i < kStreamMax; ++i)
    wv[i] = rmw_ld<0>(rw, i < w16 ? wb + i * 4096u + t16 : kPastEnd);
#pragma unroll
  for (int i = 0; i < kStreamMax; ++i)
    rv[i] = rmw_ld<2>(rr, i < r16 ? rb + i * 4096u + t16 : kPastEnd);
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kStreamMax; ++i) acc ^= wv[i];
#pragma unroll
  for (int i = 0; i < kStreamMax; ++i)
    rmw_st<2>(rr, i < r16 ? rb + i * 4096u + t16 : kPastEnd, rv[i] + acc);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[threadIdx.x] = acc.x;
}

// The first failing call's code is kept; later calls are skipped.
struct Status {
  hipError_t rc = hipSuccess;
  bool ok() const { return rc == hipSuccess; }
  void operator()(hipError_t r) {
    if (rc == hipSuccess) rc = r;
  }
};

}  // namespace

extern "C" int32_t mlora_probe_empty(int32_t launches, float* eager_us, float* graph_us) {
  if (launches < 1 || !eager_us || !graph_us) return (int32_t)hipErrorInvalidValue;
  Status st;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  float ms = 0.f;
  st(hipStreamCreate(&s));
  if (st.ok()) st(hipEventCreate(&e0));
  if (st.ok()) st(hipEventCreate(&e1));
  if (st.ok()) {
    for (int i = 0; i < 16; ++i) hipLaunchKernelGGL(empty_kernel, dim3(256), dim3(64), 0, s);
    st(hipStreamSynchronize(s));
  }
  if (st.ok()) {
    st(hipEventRecord(e0, s));
    for (int i = 0; i < launches; ++i)
      hipLaunchKernelGGL(empty_kernel, dim3(256), dim3(64), 0, s);
    st(hipEventRecord(e1, s));
    st(hipEventSynchronize(e1));
    st(hipEventElapsedTime(&ms, e0, e1));
    *eager_us = ms * 1e3f / (float)launches;
  }
  if (st.ok()) {
    st(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    if (st.ok()) {
      for (int i = 0; i < launches; ++i)
        hipLaunchKernelGGL(empty_kernel, dim3(256), dim3(64), 0, s);
      st(hipStreamEndCapture(s, &graph));
    }
  }
  if (st.ok()) st(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
  if (st.ok()) {
    st(hipGraphLaunch(exec, s));
    st(hipStreamSynchronize(s));
    st(hipEventRecord(e0, s));
    st(hipGraphLaunch(exec, s));
    st(hipEventRecord(e1, s));
    st(hipEventSynchronize(e1));
    st(hipEventElapsedTime(&ms, e0, e1));
    *graph_us = ms * 1e3f / (float)launches;
  }
  st(hipGetLastError());
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (s) (void)hipStreamDestroy(s);
  return (int32_t)st.rc;
}

// pattern 0: operand pattern, 1: row-contiguous, 2: row-contiguous into
// LDS, read back in the operand pattern (checked against pattern 0's
// per-lane values first: hipErrorUnknown if they differ). stride: bytes
// from one row to the next (4096 .. 8192, a multiple of 16). us: mean
// microseconds per launch over `iters` launches rotating over `copies`
// buffers.
extern "C" int32_t mlora_probe_read(int32_t pattern, int32_t stride, int32_t copies,
                                    int32_t iters, float* us) {
  if (pattern < 0 || pattern > 2 || stride < kRowBytes || stride > 8192 || stride % 16 ||
      copies < 1 || copies > 32 || iters < 1 || !us)
    return (int32_t)hipErrorInvalidValue;
  const size_t bytes = (size_t)kRows * stride;
  std::vector<char*> bufs(copies, nullptr);
  unsigned* sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  Status st;
  st(hipMalloc(&sink, (size_t)256 * kThreads * sizeof(unsigned)));
  for (int i = 0; st.ok() && i < copies; ++i) {
    st(hipMalloc(&bufs[i], bytes));
    if (st.ok()) st(hipMemset(bufs[i], i, bytes));
  }
  if (st.ok()) st(hipEventCreate(&e0));
  if (st.ok()) st(hipEventCreate(&e1));
  if (st.ok()) {
    auto launch = [&](int i) {
      if (pattern == 0)
        hipLaunchKernelGGL(read_operand_kernel, dim3(256), dim3(kThreads), 0, 0,
                           bufs[i % copies], sink, stride);
      else if (pattern == 1)
        hipLaunchKernelGGL(read_rows_kernel, dim3(256), dim3(kThreads), 0, 0, bufs[i % copies],
                           sink, stride);
      else
        hipLaunchKernelGGL(read_lds_kernel, dim3(256), dim3(kThreads), 0, 0, bufs[i % copies],
                           sink, stride);
    };
    if (pattern == 2 && st.ok()) {
      // the LDS route must hand every lane pattern 0's values: fill a buffer
      // with distinct words, compare the two kernels' per-lane sinks
      std::vector<uint32_t> words(bytes / 4);
      for (size_t j = 0; j < words.size(); ++j) words[j] = (uint32_t)(j * 2654435761u) ^ (uint32_t)j;
      st(hipMemcpy(bufs[0], words.data(), bytes, hipMemcpyHostToDevice));
      const size_t n_sink = (size_t)256 * kThreads;
      std::vector<unsigned> a(n_sink), c(n_sink);
      if (st.ok()) {
        hipLaunchKernelGGL(read_operand_kernel, dim3(256), dim3(kThreads), 0, 0, bufs[0], sink,
                           stride);
        st(hipMemcpy(a.data(), sink, n_sink * sizeof(unsigned), hipMemcpyDeviceToHost));
      }
      if (st.ok()) {
        hipLaunchKernelGGL(read_lds_kernel, dim3(256), dim3(kThreads), 0, 0, bufs[0], sink,
                           stride);
        st(hipMemcpy(c.data(), sink, n_sink * sizeof(unsigned), hipMemcpyDeviceToHost));
      }
      if (st.ok() && a != c) st(hipErrorUnknown);
    }
    for (int i = 0; st.ok() && i < 2 * copies; ++i) launch(i);
    st(hipDeviceSynchronize());
    float ms = 0.f;
    if (st.ok()) {
      st(hipEventRecord(e0, 0));
      for (int i = 0; i < iters; ++i) launch(i);
      st(hipEventRecord(e1, 0));
      st(hipEventSynchronize(e1));
      st(hipEventElapsedTime(&ms, e0, e1));
      *us = ms * 1e3f / (float)iters;
    }
  }
  st(hipGetLastError());
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  for (char* b : bufs)
    if (b) (void)hipFree(b);
  if (sink) (void)hipFree(sink);
  return (int32_t)st.rc;
}

// pattern 0 tile / 1 row / 2 flat; xcd_contiguous 0 or 1; nt 0 or 1; us: mean
// microseconds per launch over `iters` launches rotating over `copies`
// buffers of 64 MiB (1 .. 16).
extern "C" int32_t mlora_probe_rmw(int32_t pattern, int32_t xcd_contiguous, int32_t nt,
                                   int32_t copies, int32_t iters, float* us) {
  if (pattern < 0 || pattern > 2 || (xcd_contiguous != 0 && xcd_contiguous != 1) ||
      (nt != 0 && nt != 1) || copies < 1 || copies > 16 || iters < 1 || !us)
    return (int32_t)hipErrorInvalidValue;
  std::vector<char*> bufs(copies, nullptr);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  Status st;
  for (int i = 0; st.ok() && i < copies; ++i) {
    st(hipMalloc(&bufs[i], kRmwBytes));
    if (st.ok()) st(hipMemset(bufs[i], 0, kRmwBytes));
  }
  if (st.ok()) st(hipEventCreate(&e0));
  if (st.ok()) st(hipEventCreate(&e1));
  if (st.ok()) {
    using K = void (*)(char*);
    static const K kernels[3][2][2] = {
        {{rmw_kernel<0, false, 0>, rmw_kernel<0, false, 2>},
         {rmw_kernel<0, true, 0>, rmw_kernel<0, true, 2>}},
        {{rmw_kernel<1, false, 0>, rmw_kernel<1, false, 2>},
         {rmw_kernel<1, true, 0>, rmw_kernel<1, true, 2>}},
        {{rmw_kernel<2, false, 0>, rmw_kernel<2, false, 2>},
         {rmw_kernel<2, true, 0>, rmw_kernel<2, true, 2>}}};
    const K k = kernels[pattern][xcd_contiguous][nt];
    auto launch = [&](int i) {
      hipLaunchKernelGGL(k, dim3(kRmwBlocks), dim3(256), 0, 0, bufs[i % copies]);
    };
    for (int i = 0; i < 2 * copies; ++i) launch(i);
    st(hipDeviceSynchronize());
    float ms = 0.f;
    if (st.ok()) {
      st(hipEventRecord(e0, 0));
      for (int i = 0; i < iters; ++i) launch(i);
      st(hipEventRecord(e1, 0));
      st(hipEventSynchronize(e1));
      st(hipEventElapsedTime(&ms, e0, e1));
      *us = ms * 1e3f / (float)iters;
    }
  }
  st(hipGetLastError());
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  for (char* b : bufs)
    if (b) (void)hipFree(b);
  return (int32_t)st.rc;
}

// units: workgroups (1 .. 4096); w_kb / r_kb: weight and row kilobytes per
// workgroup, multiples of 4 up to 64; copies: rotated buffer sets (1 .. 64);
// us: mean microseconds per launch over `iters` launches (1 .. 4096)
// replayed in one HIP graph.
extern "C" int32_t mlora_probe_stream(int32_t units, int32_t w_kb, int32_t r_kb,
                                      int32_t copies, int32_t iters, float* us) {
  if (units < 1 || units > 4096 || w_kb < 0 || w_kb > 4 * kStreamMax || w_kb % 4 || r_kb < 0 ||
      r_kb > 4 * kStreamMax || r_kb % 4 || copies < 1 || copies > 64 || iters < 1 ||
      iters > 4096 || !us)
    return (int32_t)hipErrorInvalidValue;
  const int w16 = w_kb / 4, r16 = r_kb / 4;
  const size_t wbytes = (size_t)units * w_kb * 1024 + 4096;
  const size_t rbytes = (size_t)units * r_kb * 1024 + 4096;
  std::vector<char*> wbuf(copies, nullptr), rbuf(copies, nullptr);
  unsigned* sink = nullptr;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  Status st;
  st(hipMalloc(&sink, 256 * sizeof(unsigned)));
  for (int i = 0; st.ok() && i < copies; ++i) {
    st(hipMalloc(&wbuf[i], wbytes));
    if (st.ok()) st(hipMemset(wbuf[i], i, wbytes));
    if (st.ok()) st(hipMalloc(&rbuf[i], rbytes));
    if (st.ok()) st(hipMemset(rbuf[i], 0, rbytes));
  }
  if (st.ok()) st(hipStreamCreate(&s));
  if (st.ok()) st(hipEventCreate(&e0));
  if (st.ok()) st(hipEventCreate(&e1));
  if (st.ok()) st(hipDeviceSynchronize());
  if (st.ok()) {
    st(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    if (st.ok()) {
      for (int i = 0; i < iters; ++i)
        hipLaunchKernelGGL(stream_kernel, dim3(units), dim3(256), 0, s, wbuf[i % copies],
                           rbuf[i % copies], sink, w16, r16, (uint32_t)wbytes, (uint32_t)rbytes);
      st(hipStreamEndCapture(s, &graph));
    }
  }
  if (st.ok()) st(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
  if (st.ok()) {
    float ms = 0.f;
    st(hipGraphLaunch(exec, s));
    st(hipStreamSynchronize(s));
    st(hipEventRecord(e0, s));
    st(hipGraphLaunch(exec, s));
    st(hipEventRecord(e1, s));
    st(hipEventSynchronize(e1));
    st(hipEventElapsedTime(&ms, e0, e1));
    *us = ms * 1e3f / (float)iters;
  }
  st(hipGetLastError());
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (s) (void)hipStreamDestroy(s);
  for (char* b : wbuf)
    if (b) (void)hipFree(b);
  for (char* b : rbuf)
    if (b) (void)hipFree(b);
  if (sink) (void)hipFree(sink);
  return (int32_t)st.rc;
}
