// Cache seeding after the prompt, and the reset of a layer's slots.
//
// seed: per unit, keep the last k_local prompt positions (the recent tokens of
// the H2O blog, ttsmallhot.github.io, §2.2) plus the k_heavy positions of
// [0, T - k_local) with the highest fp32 column sum, i.e. the top-k of the
// cumulative attention ("H2O Heavy-Hitter Oracle 分析", §3.1). Ties rank the
// newer position higher, so the older one is dropped. The k_heavy-th largest
// 64-bit key (float bits of c_j << 32 | j; c_j >= 0 so the bits order like the
// values) is found by an 8-pass MSB radix select over LDS histograms, which
// needs O(1) LDS for any prompt length; kept positions are then compacted in
// ascending order with a ballot scan and their K/V rows copied into slots.
// If T <= k every position is kept. Slots past the kept count are marked free.
//
// reset: slot_pos = -1, acc = 0 (blog §2.3: freeing a slot only marks it).
#include "h2o_device.hpp"
#include "h2o_kernels.hpp"

namespace h2o {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint64_t seed_key(const float* c, int j) {
  return ((uint64_t)__float_as_uint(c[j]) << 32) | (uint32_t)j;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void seed_kernel(SeedParams p) {
  extern __shared__ int slot_of[];               // [k] position held by each kept slot
  __shared__ unsigned hist[256];
  __shared__ unsigned suf[256];
  __shared__ unsigned s_sel, s_above;
  __shared__ int wcount[kThreads / kWave];

  const int unit = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int T_ = p.T, k = p.k_heavy + p.k_local;
  const float* c = p.colsum + (size_t)unit * T_;

  int n_keep;
  if (T_ <= k) {
    n_keep = T_;
    for (int s = tid; s < T_; s += kThreads) slot_of[s] = s;
  } else {
    const int ncand = T_ - p.k_local;
    uint64_t thr = ~0ull;                         // no heavy hitter passes ~0
    if (p.k_heavy > 0) {
      uint64_t prefix = 0, mask = 0;
      unsigned want = (unsigned)p.k_heavy;        // rank from the top, 1-based
      for (int pass = 7; pass >= 0; --pass) {
        const int sh = pass * 8;
        hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < ncand; j += kThreads) {
          const uint64_t key = seed_key(c, j);
          if ((key & mask) == prefix) atomicAdd(&hist[(key >> sh) & 255u], 1u);
        }
        __syncthreads();
        suf[tid] = hist[tid];
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
          const unsigned add = tid + off < 256 ? suf[tid + off] : 0u;
          __syncthreads();
          suf[tid] += add;
          __syncthreads();
        }
        const unsigned here = suf[tid], next = tid < 255 ? suf[tid + 1] : 0u;
        if (here >= want && next < want) { s_sel = (unsigned)tid; s_above = next; }
        __syncthreads();
        prefix |= (uint64_t)s_sel << sh;
        mask |= 255ull << sh;
        want -= s_above;
        __syncthreads();
      }
      thr = prefix;                              // exactly k_heavy keys are >= thr
    }
    int running = 0;
    for (int base = 0; base < T_; base += kThreads) {
      const int j = base + tid;
      const bool keep = j < T_ && (j >= ncand || seed_key(c, j) >= thr);
      const uint64_t b = __ballot(keep);
      const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
      if (lane == 0) wcount[wave] = __popcll(b);
      __syncthreads();
      int off = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kThreads / kWave; ++w) {
        off += w < wave ? wcount[w] : 0;
        total += wcount[w];
      }
      if (keep && running + off + in_wave < k) slot_of[running + off + in_wave] = j;
      running += total;
      __syncthreads();
    }
    n_keep = running < k ? running : k;
  }
  __syncthreads();

  int32_t* pos = p.slot_pos + (size_t)unit * k;
  float* acc = p.acc + (size_t)unit * k;
  for (int s = tid; s < k; s += kThreads) {
    if (s < n_keep) {
      const int j = slot_of[s];
      pos[s] = j;
      acc[s] = c[j];
    } else {
      pos[s] = -1;
      acc[s] = 0.f;
    }
  }
  constexpr int CPR = D * (int)sizeof(T) / 16;   // 16-byte chunks per row
  constexpr int VEC = 16 / (int)sizeof(T);
  const T* K = static_cast<const T*>(p.k) + (size_t)unit * T_ * D;
  const T* V = static_cast<const T*>(p.v) + (size_t)unit * T_ * D;
  T* ks = static_cast<T*>(p.k_slots) + (size_t)unit * k * D;
  T* vs = static_cast<T*>(p.v_slots) + (size_t)unit * k * D;
  for (int idx = tid; idx < n_keep * CPR; idx += kThreads) {
    const int s = idx / CPR, ch = idx - s * CPR;
    const size_t src = (size_t)slot_of[s] * D + ch * VEC, dst = (size_t)s * D + ch * VEC;
    st16(ks + dst, ld16(K + src));
    st16(vs + dst, ld16(V + src));
  }
}

__global__ void reset_kernel(ResetParams p) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < p.n; i += stride) {
    p.slot_pos[i] = -1;
    p.acc[i] = 0.f;
  }
}

template <typename T, int D>
hipError_t seed(const SeedParams& p, hipStream_t s) {
  const size_t lds = (size_t)(p.k_heavy + p.k_local) * sizeof(int);
  seed_kernel<T, D><<<dim3((unsigned)p.units), dim3(kThreads), lds, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_seed(DType dt, int D, const SeedParams& p, hipStream_t s) {
  switch (dt) {
    case DType::F32: return D == 64 ? seed<float, 64>(p, s) : seed<float, 128>(p, s);
    case DType::F16: return D == 64 ? seed<_Float16, 64>(p, s) : seed<_Float16, 128>(p, s);
    default: return D == 64 ? seed<__bf16, 64>(p, s) : seed<__bf16, 128>(p, s);
  }
}

hipError_t launch_reset(const ResetParams& p, hipStream_t s) {
  const int64_t blocks64 = (p.n + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 4096 ? (blocks64 > 0 ? blocks64 : 1) : 4096);
  reset_kernel<<<dim3(blocks), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace h2o
