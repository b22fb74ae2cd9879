// Machine ceilings the roofline fractions are read against: a streaming HBM read and a
// dense MFMA loop. Measurement probes only (libh2o_probes.so); the H2O path never calls
// them.
//
// hbm_read_probe: every thread reads 16-byte chunks, UNROLL loads in flight, and folds
// them into one word that it stores (so no load is dead). Layout 0 strides the whole grid
// between a thread's loads; layout 1 gives each workgroup whole 32 KB tiles (a wave's loads
// fall in one tile); layout 2 is layout 1 with nontemporal loads. The buffer must be a
// whole number of 16 * UNROLL * threads-per-grid chunks: the host call checks that, and
// every load address is below `bytes`.
//
// mfma_probe: every wave runs `iters` rounds of CHAINS independent 16x16x32 fp16 MFMA
// accumulations (independent chains hide the MFMA latency) on register operands, and
// stores its accumulators.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

template <int LAYOUT>
__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const uint4* __restrict__ buf,
                                                           size_t chunks, uint32_t* sink) {
  const size_t threads = (size_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  if constexpr (LAYOUT == 0) {
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i + (kUnroll - 1) * threads < chunks;
         i += kUnroll * threads) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = buf[i + u * threads];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  } else {
    constexpr size_t tile = (size_t)kThreads * kUnroll;          // chunks per tile
    for (size_t t = blockIdx.x; (t + 1) * tile <= chunks; t += gridDim.x) {
      const uint4* p = buf + t * tile + threadIdx.x;
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if constexpr (LAYOUT == 2) {
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + u * kThreads));
          v[u] = make_uint4(x[0], x[1], x[2], x[3]);
        } else {
          v[u] = p[u * kThreads];
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kChains = 8;

__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float* out) {
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(0.001f * (float)((threadIdx.x + e) & 7));
    b[e] = (_Float16)(0.001f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x4 c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) c[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` of `buf` (device memory, 16-byte aligned) with `blocks` workgroups of 256
// threads in the given layout (0, 1 or 2); `sink` holds blocks * 256 words. Returns 0, or
// -1 when an argument is out of range or the sizes do not fit the kernel's unrolled loop
// exactly (then nothing is launched), or the HIP error code.
int hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int blocks, int layout,
                   void* stream) {
  const size_t per_pass = (size_t)16 * kUnroll * kThreads * (size_t)blocks;
  if (!buf || !sink || blocks < 1 || bytes == 0 || bytes % per_pass != 0) return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4* b = static_cast<const uint4*>(buf);
  if (layout == 0) hbm_read_kernel<0><<<dim3(blocks), dim3(kThreads), 0, s>>>(b, bytes / 16, sink);
  else if (layout == 1) hbm_read_kernel<1><<<dim3(blocks), dim3(kThreads), 0, s>>>(b, bytes / 16, sink);
  else if (layout == 2) hbm_read_kernel<2><<<dim3(blocks), dim3(kThreads), 0, s>>>(b, bytes / 16, sink);
  else return -1;
  return (int)hipGetLastError();
}

// Flops executed by one mfma_probe launch.
double mfma_probe_flops(int blocks, int iters) {
  return (double)blocks * (kThreads / 64) * iters * kChains * (16.0 * 16.0 * 32.0 * 2.0);
}

// `out` holds blocks * 256 floats.
int mfma_probe(int blocks, int iters, float* out, void* stream) {
  if (!out || blocks < 1 || iters < 1) return -1;
  mfma_kernel<<<dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return (int)hipGetLastError();
}

}  // extern "C"
