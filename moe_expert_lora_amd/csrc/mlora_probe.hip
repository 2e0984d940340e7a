// Measurement probes for bench.py (not part of the fold's interface): the
// floors that bound what one launch of the fold can do on this part.
//
//   mlora_probe_empty      cost of an empty kernel launch, eager and inside a
//                          HIP graph (the fixed cost every fold launch pays).
//   mlora_probe_read       read bandwidth of 8192 rows of 4096 bytes (the row
//                          of a k_in = 2048 bf16 operand) at a given row
//                          stride, in the access pattern of the folds' MFMA
//                          operands (16 rows x 64 bytes per wave instruction,
//                          step pairs completing 128-byte lines) or one row's
//                          1 KB per wave instruction, buffers rotated past
//                          L2 and MALL.
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

// pattern 0: operand pattern, 1: row-contiguous. stride: bytes from one row
// to the next (4096 .. 8192, a multiple of 16). us: mean microseconds per
// launch over `iters` launches rotating over `copies` buffers.
extern "C" int32_t mlora_probe_read(int32_t pattern, int32_t stride, int32_t copies,
                                    int32_t iters, float* us) {
  if ((pattern != 0 && pattern != 1) || stride < kRowBytes || stride > 8192 || stride % 16 ||
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
      else
        hipLaunchKernelGGL(read_rows_kernel, dim3(256), dim3(kThreads), 0, 0, bufs[i % copies],
                           sink, stride);
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
  if (sink) (void)hipFree(sink);
  return (int32_t)st.rc;
}
