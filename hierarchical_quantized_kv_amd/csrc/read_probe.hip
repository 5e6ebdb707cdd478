// read_probe.hip -- measurement helper, not part of the cache library: the practical HBM
// ceilings of the device the benchmark runs on, from plain streaming kernels.
//
// stream_read: every lane reads 16-byte words in a grid-stride loop with eight independent
// non-temporal loads in flight and folds them into one register; the result is stored only if it
// equals a value the caller's data cannot produce by accident in practice (so the loads cannot be
// optimized away).
// stream_mix: the same loop reading R 16-byte words (from R consecutive arrays) per 16-byte word
// written, R = 1 (a copy) or 2 (about the read / write ratio of the quantizer kernels).

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kInFlight = 8;

__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ p, size_t n16,
                                                   uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

template <int R>
__global__ __launch_bounds__(256) void stream_mix(const u32x4* __restrict__ src,
                                                  u32x4* __restrict__ dst, size_t n_out) {
  constexpr int U = 4;  // output words in flight per lane (R * U loads)
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n_out; i += U * stride) {
    u32x4 v[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) v[u][r] = __builtin_nontemporal_load(src + r * n_out + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4 w = v[u][0];
#pragma unroll
      for (int r = 1; r < R; ++r) w ^= v[u][r];
      __builtin_nontemporal_store(w, dst + i + u * stride);
    }
  }
  for (; i < n_out; i += stride) {
    u32x4 w = src[i];
#pragma unroll
    for (int r = 1; r < R; ++r) w ^= src[r * n_out + i];
    dst[i] = w;
  }
}

}  // namespace

// Average duration in microseconds of `reps` launches (after two untimed ones) that read the
// first bytes & ~15 bytes of d_buf, with blocks_per_cu 256-thread blocks per compute unit, timed
// with HIP events on `stream`.  d_sink: 4 bytes of device memory.  Returns 0 or a hipError_t.
extern "C" int qs_probe_stream_read(const void* d_buf, size_t bytes, uint32_t* d_sink,
                                    int blocks_per_cu, int reps, void* stream, float* h_avg_us) {
  if (!d_buf || !d_sink || !h_avg_us || blocks_per_cu < 1 || reps < 1 || bytes < 16)
    return (int)hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(cus * blocks_per_cu));
  const size_t n16 = bytes / 16;
  const u32x4* p = static_cast<const u32x4*>(d_buf);
  hipEvent_t a = nullptr, b = nullptr;
  e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  for (int r = 0; e == hipSuccess && r < 2; ++r) {
    hipLaunchKernelGGL(stream_read, grid, dim3(256), 0, st, p, n16, d_sink);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(a, st);
  for (int r = 0; e == hipSuccess && r < reps; ++r) {
    hipLaunchKernelGGL(stream_read, grid, dim3(256), 0, st, p, n16, d_sink);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(b, st);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  if (e != hipSuccess) return (int)e;
  *h_avg_us = ms * 1000.f / (float)reps;
  return 0;
}

// Average duration in microseconds of `reps` launches (after two untimed ones) of stream_mix:
// d_src holds reads_per_write * out_bytes bytes, d_dst out_bytes (rounded down to 16 bytes);
// reads_per_write 1 or 2; blocks_per_cu 256-thread blocks per compute unit; HIP events on
// `stream`.  Bytes moved per launch: (reads_per_write + 1) * out_bytes.  Returns 0 or a
// hipError_t.
extern "C" int qs_probe_stream_mix(const void* d_src, void* d_dst, size_t out_bytes,
                                   int reads_per_write, int blocks_per_cu, int reps, void* stream,
                                   float* h_avg_us) {
  if (!d_src || !d_dst || !h_avg_us || blocks_per_cu < 1 || reps < 1 || out_bytes < 16 ||
      (reads_per_write != 1 && reads_per_write != 2))
    return (int)hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(cus * blocks_per_cu));
  const size_t n_out = out_bytes / 16;
  const u32x4* src = static_cast<const u32x4*>(d_src);
  u32x4* dst = static_cast<u32x4*>(d_dst);
  auto launch = [&]() {
    if (reads_per_write == 1) hipLaunchKernelGGL(stream_mix<1>, grid, dim3(256), 0, st, src, dst, n_out);
    else hipLaunchKernelGGL(stream_mix<2>, grid, dim3(256), 0, st, src, dst, n_out);
    return hipGetLastError();
  };
  hipEvent_t a = nullptr, b = nullptr;
  e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  for (int r = 0; e == hipSuccess && r < 2; ++r) e = launch();
  if (e == hipSuccess) e = hipEventRecord(a, st);
  for (int r = 0; e == hipSuccess && r < reps; ++r) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, st);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  if (e != hipSuccess) return (int)e;
  *h_avg_us = ms * 1000.f / (float)reps;
  return 0;
}
