// Fused H2O decode step.
//
// Per unit (sequence, head), with n = min(k, t) valid slots (always a prefix):
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
// Memory plan. A slot row is D*sizeof(T) bytes, read as 16-byte chunks by LANES
// consecutive lanes (a "row group"); a 256-thread workgroup has ROWS row
// groups and covers ROWS slots per pass, every wave load fully coalesced.
// Row group g owns slots j = u*ROWS + g, u < U, and issues all of their K and
// V loads (plus q, the scores and the positions) before consuming any, so the
// whole unit is in flight at once. Rows past the new token are clamped to the
// new token's row (always valid memory) and masked, so the load stream has no
// branches. Logit sums over a row group use DPP lane moves.
//
// Two kernels:
//   * resident: one workgroup per unit when k + 1 <= ROWS * U (U = 8 or 16):
//     two barriers, everything else in registers.
//   * split: S workgroups per unit, one slot chunk each, for large k or few
//     units. Each writes (max, sum, unnormalised out) and its logits to the
//     workspace, then bumps a per-unit counter with agent-scope acq_rel
//     ordering; the last arrival combines the partials, updates the scores,
//     takes the argmin and overwrites the victim (every other workgroup has
//     finished reading it), then puts the counter back to zero.
// The victim is chosen with 64-bit keys (fp32 score bits << 32 | position):
// scores are >= 0, so the integer order is the (score, position) order.
// All reductions run in a fixed order: results are bit-reproducible.
#include "h2o_device.hpp"
#include "h2o_kernels.hpp"

namespace h2o {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <typename T, int D> struct Shape {
  static constexpr int VEC = Chunk<T>::N;       // elements per 16-byte chunk
  static constexpr int LANES = D / VEC;         // lanes per slot row
  static constexpr int ROWS = kThreads / LANES; // row groups per workgroup
  static constexpr int GPW = kWave / LANES;     // row groups per wave
};

// DPP lane move inside a 16-lane row (all lanes active).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over each group of WIDTH consecutive lanes; every lane gets the group's sum
// (the pairings are symmetric, so all lanes of a group hold the same bits).
template <int WIDTH>
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0xb1>(v);                                    // quad_perm [1,0,3,2]
  v += dpp<0x4e>(v);                                    // quad_perm [2,3,0,1]
  if constexpr (WIDTH >= 8) v += dpp<0x141>(v);         // row_half_mirror
  if constexpr (WIDTH >= 16) v += dpp<0x140>(v);        // row_mirror
  if constexpr (WIDTH >= 32) v += __shfl_xor(v, 16, kWave);
  return v;
}

// Loads of one row group: K and V chunks of its U slots (clamped to the new token row).
template <typename T, int D, int U>
__device__ __forceinline__ void load_rows(const T* ks, const T* vs, const T* kn, const T* vn,
                                          int first, int n, int rl, uint4 (&kr)[U],
                                          uint4 (&vr)[U]) {
  using S = Shape<T, D>;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = first + u * S::ROWS;
    const bool slot = j < n;
    const size_t off = (size_t)(slot ? j : 0) * D + rl * S::VEC;
    kr[u] = ld16(slot ? ks + off : kn + rl * S::VEC);
    vr[u] = ld16(slot ? vs + off : vn + rl * S::VEC);
  }
}

// Logits (log2 domain) of a row group's U slots; slots past `last` are -inf.
// Returns the group max, its sum of 2^(s - max) and the unnormalised out chunk.
template <typename T, int D, int U>
__device__ __forceinline__ void group_softmax(const uint4& qr, float qk_scale, const uint4 (&kr)[U],
                                              const uint4 (&vr)[U], int first, int last,
                                              float (&s)[U], float& mg, float& lg,
                                              float (&o)[Shape<T, D>::VEC]) {
  using S = Shape<T, D>;
  constexpr int VEC = S::VEC;
  float qf[VEC];
  unpack(qr, qf, T{});
#pragma unroll
  for (int i = 0; i < VEC; ++i) qf[i] *= qk_scale;
  mg = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float kf[VEC];
    unpack(kr[u], kf, T{});
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) d = fmaf(qf[i], kf[i], d);
    d = row_sum<S::LANES>(d);
    s[u] = first + u * S::ROWS <= last ? d : -INFINITY;
    mg = fmaxf(mg, s[u]);
  }
  const float mref = mg == -INFINITY ? 0.f : mg;
  lg = 0.f;
#pragma unroll
  for (int i = 0; i < VEC; ++i) o[i] = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float e = fast_exp2(s[u] - mref);
    lg += e;
    float vf[VEC];
    unpack(vr[u], vf, T{});
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = fmaf(e, vf[i], o[i]);
  }
}

__device__ __forceinline__ uint64_t score_key(float a, int pos) {
  return ((uint64_t)__float_as_uint(a) << 32) | (uint32_t)pos;
}

// ------------------------------------------------------------------ resident --

template <typename T, int D, int U>
__global__ __launch_bounds__(kThreads) void decode_resident_kernel(DecodeParams p) {
  using S = Shape<T, D>;
  constexpr int VEC = S::VEC, LANES = S::LANES, ROWS = S::ROWS;
  __shared__ __attribute__((aligned(16))) float s_red[ROWS * D];
  __shared__ float s_m[ROWS], s_l[ROWS];
  __shared__ float s_logit[ROWS * U];
  __shared__ uint64_t s_key[kWaves];

  const int unit = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = tid % LANES, g = tid / LANES;
  const int k = p.k, t = p.t;
  const int n = min(k, t);
  const bool full = n == k;
  const int limit = t - p.k_local;

  T* ks = static_cast<T*>(p.k_slots) + (size_t)unit * k * D;
  T* vs = static_cast<T*>(p.v_slots) + (size_t)unit * k * D;
  const T* kn = static_cast<const T*>(p.k_new) + (size_t)unit * D;
  const T* vn = static_cast<const T*>(p.v_new) + (size_t)unit * D;
  int32_t* pos = p.slot_pos + (size_t)unit * k;
  float* acc = p.acc + (size_t)unit * k;

  // Every load of the unit, issued before any is consumed.
  const uint4 qr = ld16(static_cast<const T*>(p.q) + (size_t)unit * D + rl * VEC);
  uint4 kr[U], vr[U];
  load_rows<T, D, U>(ks, vs, kn, vn, g, n, rl, kr, vr);
  const int jo = rl * ROWS + g;                 // slot whose score this lane owns
  const bool own = rl < U && jo < n;
  const int jc = own ? jo : 0;
  const float acc_old = acc[jc];
  const int pos_old = pos[jc];
  __builtin_amdgcn_sched_barrier(0);            // keep every load ahead of the math

  float s[U], mg, lg, o[VEC];
  group_softmax<T, D, U>(qr, p.qk_scale, kr, vr, g, n, s, mg, lg, o);

#pragma unroll
  for (int i = 0; i < VEC; ++i) s_red[g * D + rl * VEC + i] = o[i];
  if (rl == 0) {
    s_m[g] = mg;
    s_l[g] = lg;
#pragma unroll
    for (int u = 0; u < U; ++u) s_logit[u * ROWS + g] = s[u];
  }
  __syncthreads();                              // (1) every K/V read is consumed

  float M = -INFINITY;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) M = fmaxf(M, s_m[r]);
  float sc[ROWS], L = 0.f;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const float mr = s_m[r];
    sc[r] = mr == -INFINITY ? 0.f : fast_exp2(mr - M);
    L = fmaf(s_l[r], sc[r], L);
  }
  const float inv = 1.0f / L;
  const float p_new = fast_exp2(s_logit[n] - M) * inv;

  for (int c = tid; c < D; c += kThreads) {
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) v = fmaf(s_red[r * D + c], sc[r], v);
    p.out[(size_t)unit * D + c] = v * inv;
  }

  uint64_t key = ~0ull;
  float a = 0.f;
  if (own) {
    a = acc_old + fast_exp2(s_logit[jo] - M) * inv;
    acc[jo] = a;
    if (full && pos_old <= limit) key = score_key(a, pos_old);
  }
  const uint64_t wmin = wave_min_u64(key);
  if (lane == 0) s_key[wave] = wmin;
  __syncthreads();                              // (2)
  uint64_t best = s_key[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) best = s_key[w] < best ? s_key[w] : best;

  int dst = -1;
  bool meta = false;
  if (full) {
    const uint64_t hit = __ballot(key == best && best != ~0ull);
    const uint64_t grp = (hit >> ((lane / LANES) * LANES)) & ((1ull << LANES) - 1ull);
    if (grp) dst = (__ffsll((unsigned long long)grp) - 1) * ROWS + g;
    meta = key == best && best != ~0ull;
  } else {
    if (g == n % ROWS) dst = n;
    meta = jo == n;
  }
  if (dst >= 0) {
    st16(ks + (size_t)dst * D + rl * VEC, ld16(kn + rl * VEC));
    st16(vs + (size_t)dst * D + rl * VEC, ld16(vn + rl * VEC));
  }
  if (meta) {                                   // the lane that wrote acc[dst] above, if any
    pos[dst] = t;
    acc[dst] = p_new;
    if (p.victim_slot) p.victim_slot[unit] = full ? dst : -1;
    if (p.evicted_pos) p.evicted_pos[unit] = full ? pos_old : -1;
    if (p.evicted_acc) p.evicted_acc[unit] = full ? a : 0.f;
  }
}

// --------------------------------------------------------------------- split --

template <typename T, int D, int U>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p, SplitScratch w) {
  using S = Shape<T, D>;
  constexpr int VEC = S::VEC, LANES = S::LANES, ROWS = S::ROWS;
  constexpr int C = ROWS * U;                   // slots per workgroup
  __shared__ __attribute__((aligned(16))) float s_red[ROWS * D];
  __shared__ float s_m[ROWS], s_l[ROWS];
  __shared__ uint64_t s_key[kWaves];
  __shared__ int s_last, s_dst;

  const int nsplit = w.splits;
  const int unit = blockIdx.x / nsplit, sp = blockIdx.x - unit * nsplit;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = tid % LANES, g = tid / LANES;
  const int k = p.k, t = p.t;
  const int n = min(k, t);
  const bool full = n == k;
  const int limit = t - p.k_local;

  T* ks = static_cast<T*>(p.k_slots) + (size_t)unit * k * D;
  T* vs = static_cast<T*>(p.v_slots) + (size_t)unit * k * D;
  const T* kn = static_cast<const T*>(p.k_new) + (size_t)unit * D;
  const T* vn = static_cast<const T*>(p.v_new) + (size_t)unit * D;
  int32_t* pos = p.slot_pos + (size_t)unit * k;
  float* acc = p.acc + (size_t)unit * k;
  float* logit = w.logits + (size_t)unit * (k + 1);
  float* pml = w.part_ml + ((size_t)unit * nsplit + sp) * 2;
  float* po = w.part_o + ((size_t)unit * nsplit + sp) * D;

  // Phase A: this workgroup's chunk [sp*C, sp*C + C) of the n + 1 keys.
  const int first = sp * C + g;
  const uint4 qr = ld16(static_cast<const T*>(p.q) + (size_t)unit * D + rl * VEC);
  uint4 kr[U], vr[U];
  load_rows<T, D, U>(ks, vs, kn, vn, first, n, rl, kr, vr);
  __builtin_amdgcn_sched_barrier(0);            // keep every load ahead of the math
  float s[U], mg, lg, o[VEC];
  group_softmax<T, D, U>(qr, p.qk_scale, kr, vr, first, n, s, mg, lg, o);
  if (rl == 0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (first + u * ROWS <= n) logit[first + u * ROWS] = s[u];
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) s_red[g * D + rl * VEC + i] = o[i];
  if (rl == 0) { s_m[g] = mg; s_l[g] = lg; }
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) m = fmaxf(m, s_m[r]);
  float sc[ROWS], l = 0.f;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    sc[r] = s_m[r] == -INFINITY ? 0.f : fast_exp2(s_m[r] - m);
    l = fmaf(s_l[r], sc[r], l);
  }
  for (int c = tid; c < D; c += kThreads) {
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) v = fmaf(s_red[r * D + c], sc[r], v);
    po[c] = v;
  }
  if (tid == 0) { pml[0] = m; pml[1] = l; }

  // Arrival: all of this workgroup's stores are ordered before the counter bump.
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(w.counters + unit, 1, __ATOMIC_ACQ_REL,
                                            __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == nsplit - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // other workgroups' partials are visible

  // Phase B (last arrival only): combine, score, choose, overwrite.
  const float* ml = w.part_ml + (size_t)unit * nsplit * 2;
  float M = -INFINITY;
  for (int q = 0; q < nsplit; ++q) M = fmaxf(M, ml[2 * q]);
  float L = 0.f;
  for (int q = 0; q < nsplit; ++q) {
    const float mq = ml[2 * q];
    if (mq != -INFINITY) L = fmaf(ml[2 * q + 1], fast_exp2(mq - M), L);
  }
  const float inv = 1.0f / L;
  for (int c = tid; c < D; c += kThreads) {
    float v = 0.f;
    for (int q = 0; q < nsplit; ++q) {
      const float mq = ml[2 * q];
      if (mq != -INFINITY)
        v = fmaf(w.part_o[((size_t)unit * nsplit + q) * D + c],
                 fast_exp2(mq - M), v);
    }
    p.out[(size_t)unit * D + c] = v * inv;
  }
  const float p_new = fast_exp2(logit[n] - M) * inv;
  if (tid == 0) s_dst = full ? -1 : n;

  uint64_t best = ~0ull;
  int best_slot = -1;
  for (int j = tid; j < n; j += kThreads) {
    const float a = acc[j] + fast_exp2(logit[j] - M) * inv;
    acc[j] = a;
    const int ps = pos[j];
    if (full && ps <= limit) {
      const uint64_t key = score_key(a, ps);
      if (key < best) { best = key; best_slot = j; }
    }
  }
  const uint64_t wmin = wave_min_u64(best);
  if (lane == 0) s_key[wave] = wmin;
  __syncthreads();
  uint64_t gbest = s_key[0];
#pragma unroll
  for (int q = 1; q < kWaves; ++q) gbest = s_key[q] < gbest ? s_key[q] : gbest;
  const bool mine = full && best_slot >= 0 && best == gbest;
  if (mine) s_dst = best_slot;
  __syncthreads();
  const int dst = s_dst;
  if (dst >= 0) {
    for (int c = tid; c < 2 * LANES; c += kThreads) {
      const int ch = c % LANES;
      T* row = (c < LANES ? ks : vs) + (size_t)dst * D + ch * VEC;
      st16(row, ld16((c < LANES ? kn : vn) + ch * VEC));
    }
    // The metadata is written by the thread that updated acc[dst] in the loop above
    // (j = dst is visited by thread dst % 256), so its two writes are in program order.
    if (tid == (dst & (kThreads - 1))) {
      pos[dst] = t;
      acc[dst] = p_new;
    }
  }
  if (tid == 0) {
    if (p.victim_slot) p.victim_slot[unit] = full ? dst : -1;
    if (p.evicted_pos) p.evicted_pos[unit] = full && dst >= 0 ? (int32_t)(uint32_t)gbest : -1;
    if (p.evicted_acc)
      p.evicted_acc[unit] = full && dst >= 0 ? __uint_as_float((uint32_t)(gbest >> 32)) : 0.f;
    w.counters[unit] = 0;                       // ready for the next step
  }
}

// ------------------------------------------------------------------ dispatch --

template <typename T, int D>
hipError_t run(const DecodeParams& p, const SplitScratch& w, hipStream_t s) {
  const DecodePlan plan = plan_decode(sizeof(T), D, p.k, p.units);
  if (plan.splits == 0) {
    if constexpr (Shape<T, D>::LANES >= 16) {
      if (plan.u == 16) {
        decode_resident_kernel<T, D, 16><<<dim3(p.units), dim3(kThreads), 0, s>>>(p);
        return hipGetLastError();
      }
    }
    decode_resident_kernel<T, D, 8><<<dim3(p.units), dim3(kThreads), 0, s>>>(p);
  } else {
    decode_split_kernel<T, D, kSplitU><<<dim3((unsigned)(p.units * plan.splits)), dim3(kThreads),
                                         0, s>>>(p, w);
  }
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int elem_bytes, int D, int k, int units) {
  const int rows = kThreads / (D * elem_bytes / 16);
  DecodePlan plan{0, 0};
  // One resident workgroup per unit while the whole cache fits one load batch and the
  // units alone fill most of the chip; otherwise split the slots over workgroups.
  const int lanes = kThreads / rows;             // a lane owns one slot score: u <= lanes
  if (units >= 128 || k + 1 <= rows * 8) {
    if (k + 1 <= rows * 8) { plan.u = 8; return plan; }
    if (k + 1 <= rows * 16 && lanes >= 16) { plan.u = 16; return plan; }
  }
  plan.u = kSplitU;
  plan.splits = (k + 1 + rows * kSplitU - 1) / (rows * kSplitU);
  return plan;
}

size_t decode_scratch_bytes(int elem_bytes, int D, int k, int units, size_t* counter_bytes) {
  const DecodePlan plan = plan_decode(elem_bytes, D, k, units);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  *counter_bytes = plan.splits ? up((size_t)units * 4) : 0;
  if (!plan.splits) return 0;
  return up((size_t)units * plan.splits * 2 * 4) + up((size_t)units * plan.splits * D * 4) +
         up((size_t)units * (k + 1) * 4);
}

SplitScratch carve_decode_scratch(int elem_bytes, int D, int k, int units, void* counters,
                                  void* scratch) {
  const DecodePlan plan = plan_decode(elem_bytes, D, k, units);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* b = static_cast<char*>(scratch);
  SplitScratch w{};
  w.splits = plan.splits;
  w.counters = static_cast<int*>(counters);
  w.part_ml = reinterpret_cast<float*>(b);
  b += up((size_t)units * plan.splits * 2 * 4);
  w.part_o = reinterpret_cast<float*>(b);
  b += up((size_t)units * plan.splits * D * 4);
  w.logits = reinterpret_cast<float*>(b);
  return w;
}

hipError_t launch_decode(DType dt, int D, const DecodeParams& p, const SplitScratch& w,
                         hipStream_t s) {
  switch (dt) {
    case DType::F32: return D == 64 ? run<float, 64>(p, w, s) : run<float, 128>(p, w, s);
    case DType::F16: return D == 64 ? run<_Float16, 64>(p, w, s) : run<_Float16, 128>(p, w, s);
    default: return D == 64 ? run<__bf16, 64>(p, w, s) : run<__bf16, 128>(p, w, s);
  }
}

}  // namespace h2o
