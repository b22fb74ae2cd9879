// LDS access-pattern probe: the LDS cycles and bank-conflict cycles one wave instruction
// costs for a given set of per-lane byte offsets, read with rocprofv3 --pmc
// SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS (one dispatch per pattern). A
// measurement probe only (libh2o_probes.so); the H2O path never calls it.
//
// One 256-thread workgroup; every wave repeats `iters` times a batch of four identical
// LDS instructions at offs[lane] (lanes with offset -1 stay idle), waiting for the batch
// inside the same asm block. Modes: 0 ds_read_b128, 1 ds_write_b64, 2 ds_read_b64,
// 3 ds_read_b64_tr_b16. The host call checks every offset: -1, or aligned to the access
// size and inside the 64 KB array.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
constexpr int kLdsBytes = 65536;

__global__ __launch_bounds__(256) void lds_bank_kernel(const int* __restrict__ offs, int mode,
                                                       int iters, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += 256) reinterpret_cast<uint32_t*>(lds)[i] = i;
  __syncthreads();
  const int off = offs[threadIdx.x & 63];
  u4 acc = {0, 0, 0, 0};
  if (off >= 0) {
    for (int it = 0; it < iters; ++it) {
      if (mode == 0) {
        u4 a, b, c, d;
        asm volatile(
            "ds_read_b128 %0, %4\n ds_read_b128 %1, %4\n ds_read_b128 %2, %4\n ds_read_b128 %3, %4\n"
            "s_waitcnt lgkmcnt(0)\n"
            : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d) : "v"(off) : "memory");
        acc ^= a ^ b ^ c ^ d;
      } else if (mode == 1) {
        const u2 v = {(uint32_t)it, (uint32_t)threadIdx.x};
        asm volatile(
            "ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n"
            "s_waitcnt lgkmcnt(0)\n" :: "v"(off), "v"(v) : "memory");
      } else {
        u2 a, b, c, d;
        if (mode == 2) {
          asm volatile(
              "ds_read_b64 %0, %4\n ds_read_b64 %1, %4\n ds_read_b64 %2, %4\n ds_read_b64 %3, %4\n"
              "s_waitcnt lgkmcnt(0)\n"
              : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d) : "v"(off) : "memory");
        } else {
          asm volatile(
              "ds_read_b64_tr_b16 %0, %4\n ds_read_b64_tr_b16 %1, %4\n"
              "ds_read_b64_tr_b16 %2, %4\n ds_read_b64_tr_b16 %3, %4\n"
              "s_waitcnt lgkmcnt(0)\n"
              : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d) : "v"(off) : "memory");
        }
        const u2 x = a ^ b ^ c ^ d;
        acc.x ^= x.x;
        acc.y ^= x.y;
      }
    }
  }
  // A plain read of the array keeps it (and its 64 KB allocation) alive: the asm accesses
  // alone would let the compiler drop it.
  acc.x ^= reinterpret_cast<volatile uint32_t*>(lds)[threadIdx.x];
  sink[threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// offs: 64 host int32 (one per lane), copied to `offs_dev` (64 device int32) before the
// launch; sink: 256 device uint32. Returns 0, -1 for an offset or mode out of range, -2 if
// the kernel does not hold its 64 KB LDS array (nothing launched in either case), or a HIP
// error code.
int lds_bank_probe(const int* offs, int* offs_dev, int mode, int iters, uint32_t* sink,
                   hipStream_t stream) {
  if (mode < 0 || mode > 3 || iters < 1) return -1;
  const int size = mode == 0 ? 16 : 8;
  for (int l = 0; l < 64; ++l) {
    const int o = offs[l];
    if (o != -1 && (o < 0 || o % size != 0 || o + size > kLdsBytes)) return -1;
  }
  hipFuncAttributes attr;
  hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&lds_bank_kernel));
  if (e != hipSuccess) return (int)e;
  if (attr.sharedSizeBytes < (size_t)kLdsBytes) return -2;
  e = hipMemcpyAsync(offs_dev, offs, 64 * sizeof(int), hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return (int)e;
  lds_bank_kernel<<<1, 256, 0, stream>>>(offs_dev, mode, iters, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
