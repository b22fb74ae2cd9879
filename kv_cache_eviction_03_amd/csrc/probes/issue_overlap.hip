// Issue-overlap probe: how far a SIMD runs vector ALU work (v_exp_f32, v_fma_f32) while
// its matrix unit runs MFMAs, within one wave and across the waves that share the SIMD. A
// measurement probe only (libh2o_probes.so); the H2O path never calls it.
//
// One workgroup per CU (each asks for 100 KB of LDS, so no second one fits), 256 threads
// (one wave per SIMD) or 512 (two). Every wave times `iters` iterations of a fixed
// instruction mix with s_memtime and writes its tick count; the host averages waves 0-3
// and waves 4-7 of each workgroup apart, since a SIMD's older wave issues first.
// Modes (per wave and iteration):
//   0  16 v_mfma_f32_16x16x32_f16 (4 independent accumulators)
//   1  16 v_exp_f32 (independent)
//   2  mode 0 and mode 1 interleaved, about one MFMA to one exponential
//   3  mode 0, then mode 1 (two blocks)
//   4  waves 0-3 run mode 1, waves 4-7 mode 0
//   5  16 independent v_fma_f32
//   6  mode 0 and mode 5 interleaved, one MFMA to one FMA
//   7  8 v_mfma_f32_32x32x16_f16 (the same multiply-adds as mode 0)
//   8  mode 7 with 16 exponentials interleaved, one MFMA to two
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kModes = 9;
constexpr size_t kLdsBytes = 100 * 1024;

template <int MODE>
__global__ __launch_bounds__(512) void issue_overlap_kernel(int iters, float* sink,
                                                            unsigned long long* ticks) {
  extern __shared__ char lds_hold[];                // holds the CU's LDS: one workgroup per CU
  const int tid = threadIdx.x, wave = tid >> 6;
  f16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (tid + i));
    b[i] = (_Float16)(0.002f * (tid - i));
  }
  f32x4 c[4];
  for (int j = 0; j < 4; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x16 d[2];
  for (int j = 0; j < 2; ++j)
    for (int i = 0; i < 16; ++i) d[j][i] = 0.f;
  float e[16], g[16];
  for (int j = 0; j < 16; ++j) {
    e[j] = 1e-3f * (tid + j);
    g[j] = 0.5f * j;
  }
  const int mode = MODE == 4 ? ((wave >> 2) & 1 ? 0 : 1) : MODE;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  // The mode is chosen outside the timed loop, so each loop body is one straight block.
#define TIMED for (int it = 0; it < iters; ++it)
  if (mode == 0) {
    TIMED {
#pragma unroll
      for (int j = 0; j < 16; ++j) c[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j & 3], 0, 0, 0);
    }
  } else if (mode == 1) {
    TIMED {
#pragma unroll
      for (int j = 0; j < 16; ++j) e[j] = __builtin_amdgcn_exp2f(e[j]);
    }
  } else if (mode == 2) {
    TIMED {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        c[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j & 3], 0, 0, 0);
        e[j] = __builtin_amdgcn_exp2f(e[j]);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // one VALU
      }
    }
  } else if (mode == 3) {
    TIMED {
#pragma unroll
      for (int j = 0; j < 16; ++j) c[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 16; ++j) e[j] = __builtin_amdgcn_exp2f(e[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if (mode == 5) {
    TIMED {
#pragma unroll
      for (int j = 0; j < 16; ++j) g[j] = g[j] * 0.999f + 0.5f;
    }
  } else if (mode == 6) {
    TIMED {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        c[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j & 3], 0, 0, 0);
        g[j] = g[j] * 0.999f + 0.5f;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
      }
    }
  } else if (mode == 7) {
    TIMED {
#pragma unroll
      for (int j = 0; j < 8; ++j) d[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, d[j & 1], 0, 0, 0);
    }
  } else if (mode == 8) {
    TIMED {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        d[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, d[j & 1], 0, 0, 0);
        e[2 * j] = __builtin_amdgcn_exp2f(e[2 * j]);
        e[2 * j + 1] = __builtin_amdgcn_exp2f(e[2 * j + 1]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
    }
  }
#undef TIMED
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int j = 0; j < 16; ++j) s += e[j] + g[j] + d[0][j] + d[1][j];
  for (int j = 0; j < 4; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  if (tid == 0) s += (float)lds_hold[0];
  const int gid = blockIdx.x * blockDim.x + tid;
  sink[gid] = s;
  if ((tid & 63) == 0) ticks[gid >> 6] = t1 - t0;
}

template <int MODE>
hipError_t launch(int blocks, int threads, int iters, float* sink, unsigned long long* ticks,
                  hipStream_t stream) {
  const void* f = reinterpret_cast<const void*>(&issue_overlap_kernel<MODE>);
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (e != hipSuccess) return e;
  issue_overlap_kernel<MODE><<<blocks, threads, kLdsBytes, stream>>>(iters, sink, ticks);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// blocks workgroups of 64 * 4 * waves_per_simd threads; sink: blocks * 512 device floats;
// ticks: blocks * 8 device uint64 (one per wave, s_memtime ticks over the timed loop).
// Returns 0, -1 for an argument out of range (nothing launched), or a HIP error code.
int issue_overlap_probe(int mode, int waves_per_simd, int blocks, int iters, float* sink,
                        unsigned long long* ticks, hipStream_t stream) {
  if (mode < 0 || mode >= kModes || waves_per_simd < 1 || waves_per_simd > 2 || blocks < 1 ||
      iters < 1)
    return -1;
  const int threads = 256 * waves_per_simd;
  switch (mode) {
    case 0: return (int)launch<0>(blocks, threads, iters, sink, ticks, stream);
    case 1: return (int)launch<1>(blocks, threads, iters, sink, ticks, stream);
    case 2: return (int)launch<2>(blocks, threads, iters, sink, ticks, stream);
    case 3: return (int)launch<3>(blocks, threads, iters, sink, ticks, stream);
    case 4: return (int)launch<4>(blocks, threads, iters, sink, ticks, stream);
    case 5: return (int)launch<5>(blocks, threads, iters, sink, ticks, stream);
    case 6: return (int)launch<6>(blocks, threads, iters, sink, ticks, stream);
    case 7: return (int)launch<7>(blocks, threads, iters, sink, ticks, stream);
    default: return (int)launch<8>(blocks, threads, iters, sink, ticks, stream);
  }
}

}  // extern "C"
