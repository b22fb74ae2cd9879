// Fused H2O decode step: one workgroup per unit (sequence, head).
//
// Per unit, with n = min(k, t) valid slots (a prefix of the unit's slots):
//   1. logits s_j = q . key_j / sqrt(d) over the n slots and the new token
//      (the scaled softmax attention of the H2O blog, ttsmallhot.github.io,
//      §2.1.1), softmax, out = sum_j p_j value_j;
//   2. acc[j] += p_j, one fp32 add per valid slot (the running score of blog
//      §2.2; score = sum over steps in "H2O Heavy-Hitter Oracle 分析", §3.2);
//   3. if the cache is full, the victim is the lexicographic minimum of
//      (acc, position) over slots with position <= t - k_local (blog §2.2
//      greedy eviction outside the recent tokens; analysis page §3.2 argmin),
//      and the new token's K/V, position and score (its own p) overwrite that
//      slot in place (blog §2.3, no compaction). Otherwise the new token takes
//      slot n.
//
// Memory plan: a slot row is D*sizeof(T) bytes, read as 16-byte chunks by
// LANES consecutive lanes, so one pass of 256 threads covers ROWS slots and
// each wave's loads are fully coalesced. Up to U passes of K and V chunks are
// issued before any is consumed; when the whole cache fits in one batch
// (k + 1 <= ROWS * U, e.g. 104 fp16 d=128 slots) every K and V byte of the
// unit is in flight at once and V needs no second trip. Logits and then
// probabilities sit in LDS; reductions use lane butterflies plus a
// four-entry LDS stage, in a fixed order, so results are bit-reproducible.
// The victim is chosen with 64-bit keys (fp32 score bits << 32 | position):
// scores are >= 0, so the integer order is the (score, position) order.
#include "h2o_device.hpp"
#include "h2o_kernels.hpp"

namespace h2o {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int U = 8;          // passes per load batch
constexpr int kPrefetch = 2;  // slots per thread whose (acc, pos) are loaded up front

template <typename T, int D> struct Shape {
  static constexpr int VEC = Chunk<T>::N;
  static constexpr int LANES = D / VEC;
  static constexpr int ROWS = kThreads / LANES;
};

__device__ __forceinline__ float block_max(float v, float* stage) {
  v = group_max<kWave>(v);
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) stage[tid >> 6] = v;
  __syncthreads();
  float r = stage[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, stage[w]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* stage) {
  v = group_sum<kWave>(v);
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) stage[tid >> 6] = v;
  __syncthreads();
  float r = stage[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r += stage[w];
  return r;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  using S = Shape<T, D>;
  constexpr int VEC = S::VEC, LANES = S::LANES, ROWS = S::ROWS;
  extern __shared__ float lds[];
  __shared__ float s_stage[kWaves];
  __shared__ uint64_t s_key[kWaves];
  __shared__ int s_victim;

  const int k = p.k;
  float* prob = lds;                              // [k + 1]
  float* red = lds + ((k + 1 + 3) & ~3);          // [ROWS][D]

  const int unit = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = tid % LANES, g = tid / LANES;
  const int t = p.t;
  const int n = min(k, t);
  const bool full = n == k;
  const int limit = t - p.k_local;

  const T* ks = static_cast<const T*>(p.k_slots) + (size_t)unit * k * D;
  const T* vs = static_cast<const T*>(p.v_slots) + (size_t)unit * k * D;
  const T* kn = static_cast<const T*>(p.k_new) + (size_t)unit * D;
  const T* vn = static_cast<const T*>(p.v_new) + (size_t)unit * D;
  int32_t* pos = p.slot_pos + (size_t)unit * k;
  float* acc = p.acc + (size_t)unit * k;

  // Scores and positions of this thread's first slots, fetched with the rows.
  float acc_r[kPrefetch];
  int pos_r[kPrefetch];
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) {
    const int j = tid + i * kThreads;
    acc_r[i] = j < n ? acc[j] : 0.f;
    pos_r[i] = j < n ? pos[j] : 0;
  }

  if (tid == 0) s_victim = k - 1;   // in-bounds default; a full cache always has a candidate

  float qf[VEC];
  load_f32(static_cast<const T*>(p.q) + (size_t)unit * D + rl * VEC, qf);
#pragma unroll
  for (int i = 0; i < VEC; ++i) qf[i] *= p.qk_scale;

  const bool one_batch = n + 1 <= ROWS * U;
  uint4 vr[U];

  // 1. logits (log2 domain)
  for (int base = 0; base <= n; base += ROWS * U) {
    uint4 kr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * ROWS + g;
      kr[u] = make_uint4(0, 0, 0, 0);
      if (j <= n) kr[u] = ld16((j < n ? ks + (size_t)j * D : kn) + rl * VEC);
      if (one_batch) {
        vr[u] = make_uint4(0, 0, 0, 0);
        if (j <= n) vr[u] = ld16((j < n ? vs + (size_t)j * D : vn) + rl * VEC);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC];
      unpack(kr[u], kf, T{});
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) s = fmaf(qf[i], kf[i], s);
      s = group_sum<LANES>(s);
      const int j = base + u * ROWS + g;
      if (rl == 0 && j <= n) prob[j] = s;
    }
  }
  __syncthreads();

  // 2. softmax statistics
  float m = -INFINITY;
  for (int j = tid; j <= n; j += kThreads) m = fmaxf(m, prob[j]);
  m = block_max(m, s_stage);
  float l = 0.f;
  for (int j = tid; j <= n; j += kThreads) l += exp2f(prob[j] - m);
  l = block_sum(l, s_stage);
  const float inv = 1.0f / l;
  const float p_new = exp2f(prob[n] - m) * inv;

  // 3. probabilities, score accumulation, candidate minimum
  uint64_t best = ~0ull;
  int best_slot = -1;
  auto visit = [&](int j, float a_old, int ps) {
    const float pj = exp2f(prob[j] - m) * inv;
    prob[j] = pj;
    const float a = a_old + pj;
    acc[j] = a;
    if (full && ps <= limit) {
      const uint64_t key = ((uint64_t)__float_as_uint(a) << 32) | (uint32_t)ps;
      if (key < best) { best = key; best_slot = j; }
    }
  };
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) {
    const int j = tid + i * kThreads;
    if (j < n) visit(j, acc_r[i], pos_r[i]);
  }
  for (int j = tid + kPrefetch * kThreads; j < n; j += kThreads) visit(j, acc[j], pos[j]);
  const uint64_t wbest = wave_min_u64(best);
  if (lane == 0) s_key[wave] = wbest;
  __syncthreads();
  uint64_t gbest = s_key[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) gbest = s_key[w] < gbest ? s_key[w] : gbest;
  if (full && best == gbest && best_slot >= 0) s_victim = best_slot;

  // 4. out = sum_j p_j value_j
  float o[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) o[i] = 0.f;
  if (one_batch) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = u * ROWS + g;
      if (j <= n) {
        const float pj = j < n ? prob[j] : p_new;
        float vf[VEC];
        unpack(vr[u], vf, T{});
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = fmaf(pj, vf[i], o[i]);
      }
    }
  } else {
    for (int base = 0; base <= n; base += ROWS * U) {
      uint4 vb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = base + u * ROWS + g;
        vb[u] = make_uint4(0, 0, 0, 0);
        if (j <= n) vb[u] = ld16((j < n ? vs + (size_t)j * D : vn) + rl * VEC);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = base + u * ROWS + g;
        if (j <= n) {
          const float pj = j < n ? prob[j] : p_new;
          float vf[VEC];
          unpack(vb[u], vf, T{});
#pragma unroll
          for (int i = 0; i < VEC; ++i) o[i] = fmaf(pj, vf[i], o[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) red[g * D + rl * VEC + i] = o[i];
  __syncthreads();   // every K/V read of this unit has been consumed past this point
  for (int c = tid; c < D; c += kThreads) {
    float sum = 0.f;
#pragma unroll 4
    for (int r = 0; r < ROWS; ++r) sum += red[r * D + c];
    p.out[(size_t)unit * D + c] = sum;
  }

  // 5. place the new token
  const int dst = full ? s_victim : n;
  T* ksw = static_cast<T*>(p.k_slots) + ((size_t)unit * k + dst) * D;
  T* vsw = static_cast<T*>(p.v_slots) + ((size_t)unit * k + dst) * D;
  if (tid < LANES) st16(ksw + tid * VEC, ld16(kn + tid * VEC));
  else if (tid < 2 * LANES) st16(vsw + (tid - LANES) * VEC, ld16(vn + (tid - LANES) * VEC));
  // The thread that owned slot dst in step 3 (j = tid + 256 i) writes its metadata,
  // so the score written there is overwritten in program order.
  if (tid == (dst & (kThreads - 1))) {
    pos[dst] = t;
    acc[dst] = p_new;
  }
  if (tid == 0) {
    if (p.victim_slot) p.victim_slot[unit] = full ? dst : -1;
    if (p.evicted_pos) p.evicted_pos[unit] = full ? (int32_t)(uint32_t)(gbest & 0xffffffffu) : -1;
    if (p.evicted_acc) p.evicted_acc[unit] = full ? __uint_as_float((uint32_t)(gbest >> 32)) : 0.f;
  }
}

template <typename T, int D>
hipError_t run(DType dt, const DecodeParams& p, hipStream_t s) {
  decode_kernel<T, D><<<dim3((unsigned)p.units), dim3(kThreads), decode_lds_bytes(dt, D, p.k), s>>>(p);
  return hipGetLastError();
}

}  // namespace

size_t decode_lds_bytes(DType dt, int D, int k) {
  const int vec = dt == DType::F32 ? 4 : 8;
  const int rows = kThreads / (D / vec);
  return (size_t)((k + 1 + 3) & ~3) * 4 + (size_t)rows * D * 4;
}

hipError_t launch_decode(DType dt, int D, const DecodeParams& p, hipStream_t s) {
  switch (dt) {
    case DType::F32: return D == 64 ? run<float, 64>(dt, p, s) : run<float, 128>(dt, p, s);
    case DType::F16: return D == 64 ? run<_Float16, 64>(dt, p, s) : run<_Float16, 128>(dt, p, s);
    default: return D == 64 ? run<__bf16, 64>(dt, p, s) : run<__bf16, 128>(dt, p, s);
  }
}

}  // namespace h2o
