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
// consecutive lanes (a "row group"); a workgroup of THREADS threads has ROWS row
// groups and covers ROWS slots per pass, every wave load fully coalesced.
// Row group g owns slots j = u*ROWS + g, u < U, and issues all of their K and
// V loads (plus q, the scores and the positions) before consuming any, so the
// whole unit is in flight at once. Rows past the new token are clamped to the
// new token's row (always valid memory) and masked, so the load stream has no
// branches. Logit sums over a row group use DPP lane moves.
//
// Kernels:
//   * resident: one workgroup per unit (256 or 1024 threads) when the unit fits
//     one load batch (k + 1 <= ROWS * 8). Row groups publish (max, sum,
//     unnormalised out) in LDS; every wave folds them into scale factors with
//     wave-uniform DPP reductions (the factors reach the output loop as scalars);
//     owners update their scores and the (acc, pos) minimum is a wave fold plus
//     an LDS stage. Two barriers, no global scratch. Launches of many units take
//     its two-phase form (TP below): K rows first, then V rows into the same
//     registers, so that a lane holds half as many chunks and every workgroup of
//     the launch is resident at once.
//   * split: for larger k, two launches. split_partial gives S workgroups per
//     unit one slot chunk each and writes (max, sum, unnormalised out) plus the
//     chunk's logits to the workspace; split_combine (one 512-thread workgroup
//     per unit) merges the partials, updates every score, takes the argmin and
//     overwrites the victim. The kernel boundary orders the two, so no
//     workgroup ever waits on another and no device-scope fence is needed.
// The victim is chosen with 64-bit keys (fp32 score bits << 32 | position):
// scores are >= 0, so the integer order is the (score, position) order.
// All reductions run in a fixed order: results are bit-reproducible.
#include "../../include/h2o.h"
#include "h2o_device.hpp"
#include "h2o_kernels.hpp"

namespace h2o {
namespace {

constexpr int kBatch = 8;         // slot rows per row group in one load batch
// Slot rows (16-bit input slots) are read with nontemporal loads: each is read once per
// step, and a deep model visits every other layer before it comes back to this one.
constexpr bool kSlotNT = true;
__device__ __forceinline__ uint4 ld_slot(const void* p) { return kSlotNT ? ld16_nt(p) : ld16(p); }
// 256-thread launches with more units than this take the two-phase resident kernel. The
// one-phase kernel (76-90 VGPRs: five or six workgroups per CU, 1280-1536 on 256 CUs) runs
// a launch it holds at once faster (OPT-6.7B layer, 256 units: 4.24 against 4.47 us), the
// two-phase kernel one it does not (LLaMA-7B layer, 2048 units: 19.7 -> 19.4 us).
constexpr int kTwoPhaseUnits = 1024;
// The split partial kernel's: 7 makes 37 chunks of 112 slots for the 4096-slot stream
// instead of 33 of 128 (the last holding one slot), 17.4 -> 17.1 us per step.
constexpr int kPartBatch = 7;

template <typename T, int D, int THREADS = 256> struct Shape {
  static constexpr int VEC = Chunk<T>::N;       // elements per 16-byte chunk
  static constexpr int LANES = D / VEC;         // lanes per slot row
  static constexpr int ROWS = THREADS / LANES;  // row groups per workgroup
  static constexpr int WAVES = THREADS / kWave;
};

// Sum over each group of WIDTH consecutive lanes; every lane gets the group's sum
// (the pairings are symmetric, so all lanes of a group hold the same bits).
template <int WIDTH>
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_mov<0xb1>(v);                                    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4e>(v);                                    // quad_perm [2,3,0,1]
  if constexpr (WIDTH >= 8) v += dpp_mov<0x141>(v);         // row_half_mirror
  if constexpr (WIDTH >= 16) v += dpp_mov<0x140>(v);        // row_mirror
  if constexpr (WIDTH >= 32) v += __shfl_xor(v, 16, kWave);
  return v;
}

// Loads of one row group: K and V chunks of its U slots. Rows past the valid slots are
// clamped to the new token's row (slots stored in T) or to slot 0 (E4M3 slots, whose rows
// are replaced by the new token's codes once those are formed). E4M3: every K chunk is
// issued before any V chunk, so that (the loads complete in order) the logits can be
// formed while the V rows are still arriving.
template <typename T, int D, int U, int THREADS, bool F8>
__device__ __forceinline__ void load_rows(const typename SlotChunk<T, F8>::elem* ks,
                                          const typename SlotChunk<T, F8>::elem* vs,
                                          const T* kn, const T* vn, int first, int n, int rl,
                                          typename SlotChunk<T, F8>::type (&kr)[U],
                                          typename SlotChunk<T, F8>::type (&vr)[U]) {
  using S = Shape<T, D, THREADS>;
  using SC = SlotChunk<T, F8>;
  if constexpr (F8) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = first + u * S::ROWS;
      kr[u] = SC::load(ks + (size_t)(j < n ? j : 0) * D + rl * S::VEC);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = first + u * S::ROWS;
      vr[u] = SC::load(vs + (size_t)(j < n ? j : 0) * D + rl * S::VEC);
    }
  } else {
    // One base address per lane and a constant step per slot (row u is a valid slot when
    // first < n - u * ROWS, a compare against a uniform value): fewer live address
    // registers than one offset per slot (OPT-6.7B and LLaMA-7B shapes: 84 -> 77 VGPRs).
    const size_t off = (size_t)first * D + rl * S::VEC;
    const T* kb = ks + off;
    const T* vb = vs + off;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool slot = first < n - u * S::ROWS;
      kr[u] = ld_slot(slot ? kb + u * S::ROWS * D : kn + rl * S::VEC);
      vr[u] = ld_slot(slot ? vb + u * S::ROWS * D : vn + rl * S::VEC);
    }
  }
}

// E4M3 slots: the new token's K/V join as codes before attention reads them, so rows at
// and past the valid slots take the new token's codes.
template <typename T, int D, int U, int THREADS>
__device__ __forceinline__ void fill_new_rows(int first, int n, const uint2& knq, const uint2& vnq,
                                              uint2 (&kr)[U], uint2 (&vr)[U]) {
  using S = Shape<T, D, THREADS>;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool slot = first + u * S::ROWS < n;
    kr[u] = slot ? kr[u] : knq;
    vr[u] = slot ? vr[u] : vnq;
  }
}

// Dot product of two 16-byte chunks of T, accumulated into c in fp32: v_dot2 on fp16 /
// bf16 pairs (the products are exact in fp32), fma for fp32.
__device__ __forceinline__ float chunk_dot(const uint4& a, const uint4& b, float c, float) {
  c = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), c);
  c = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), c);
  c = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), c);
  return fmaf(__uint_as_float(a.w), __uint_as_float(b.w), c);
}
__device__ __forceinline__ float chunk_dot(const uint4& a, const uint4& b, float c, _Float16) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, x[i]), __builtin_bit_cast(h2, y[i]), c, false);
  return c;
}
__device__ __forceinline__ float chunk_dot(const uint4& a, const uint4& b, float c, __bf16) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, x[i]), __builtin_bit_cast(b2, y[i]),
                                        c, false);
  return c;
}
// q chunk (8 elements of T) against 8 E4M3 codes: each code pair is widened to a T pair
// (exact: E4M3 values are fp16 and bf16 values) and fed to v_dot2.
__device__ __forceinline__ float chunk_dot(const uint4& a, const uint2& b, float c, _Float16) {
  const f16x2 k0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)b.x, 1.0f, false);
  const f16x2 k1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)b.x, 1.0f, true);
  const f16x2 k2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)b.y, 1.0f, false);
  const f16x2 k3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)b.y, 1.0f, true);
  c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a.x), k0, c, false);
  c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a.y), k1, c, false);
  c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a.z), k2, c, false);
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a.w), k3, c, false);
}
__device__ __forceinline__ float chunk_dot(const uint4& a, const uint2& b, float c, __bf16) {
  const bf16x2 k0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)b.x, 1.0f, false);
  const bf16x2 k1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)b.x, 1.0f, true);
  const bf16x2 k2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)b.y, 1.0f, false);
  const bf16x2 k3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)b.y, 1.0f, true);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), k0, c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), k1, c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), k2, c, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), k3, c, false);
}

// Logits (log2 domain) of a row group's U slots; slots past `last` are -inf.
// Returns the group max, its sum of 2^(s - max) and the unnormalised out chunk.
// FILLV (E4M3 slots): rows at and past `last` take the V codes `vnew` of the new token, so
// that the V rows need not have landed before the logits are formed.
template <typename T, int D, int U, int THREADS, typename C, bool FILLV = false>
__device__ __forceinline__ void group_softmax(const uint4& qr, float qk_scale, const C (&kr)[U],
                                              const C (&vr)[U], int first, int last,
                                              float (&s)[U], float& mg, float& lg,
                                              float (&o)[Shape<T, D>::VEC], const C& vnew = C{}) {
  using S = Shape<T, D, THREADS>;
  constexpr int VEC = S::VEC;
  mg = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float d = row_sum<S::LANES>(chunk_dot(qr, kr[u], 0.f, T{})) * qk_scale;
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
    if constexpr (FILLV) unpack(first + u * S::ROWS < last ? vr[u] : vnew, vf, T{});
    else unpack(vr[u], vf, T{});
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = fmaf(e, vf[i], o[i]);
  }
}

__device__ __forceinline__ uint64_t score_key(float a, int pos) {
  return ((uint64_t)__float_as_uint(a) << 32) | (uint32_t)pos;
}


// ------------------------------------------------------------------ resident --

// Workgroup barrier that orders LDS only: vector memory operations in flight stay in flight
// (a __syncthreads first waits for every outstanding load and store of the wave).
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Component-wise select of 16-byte chunks (a select of whole vectors can be lowered
// through private memory).
__device__ __forceinline__ uint4 sel16(bool c, const uint4& a, const uint4& b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

template <typename T, int D, int THREADS, bool F8, int UB = kBatch, bool TP = false>
// TP (two phases, 16-bit input slots only): the K rows are loaded and turned into logits
// before the V rows are loaded into the same registers, and the new token's row reaches
// the store through LDS, so a lane holds one set of slot chunks instead of two (at most 64
// VGPRs: eight waves per SIMD, the LLaMA-7B layer's 2048 workgroups all resident at once).
// With 256 threads, the scores, the argmin and the bookkeeping stores are done while the
// V rows are in flight, so that only the PV product, one fold and the stores follow them.
// UB slots per row group: kBatch, or 7 for 16-bit inputs when k + 1 <= 7 row groups' worth
// (the k = 104 caches of the OPT-6.7B and LLaMA-7B layers need 105 of the 112 slots; the
// OPT-30B layer's 411 need 7 of 8 at 1024 threads): one load and one logit fewer per lane.
// Register budget: at most 128 VGPRs for the 256-thread shape, so that at least four
// workgroups share a CU (three per CU measured 3.5% slower on the 32-layer LLaMA-7B-shaped
// stack); fp16 / bf16 need 84-90 with eight slots and 76-80 with seven (at 64 they spill);
// the 1024-thread fp16 shape with seven ran the OPT-30B layer in 38.5 us against 38.9.
// The E4M3 shapes with seven slots are held to 64 VGPRs (eight waves per SIMD) and fit
// without spilling: the 256-thread one then runs eight workgroups per CU (the LLaMA-7B
// layer's 2048 all at once; 12.7 -> 12.3 us), the 1024-thread one two per CU (OPT-30B layer
// 29.1 us uncapped, 27.2 us capped with eight slots and four spilled VGPRs, 20.7 us capped
// with seven). The cap with eight slots spilled and measured slower on the 256-thread
// shape (12.5 -> 15.8 us on the LLaMA-7B layer).
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(
    TP ? 8 : (THREADS == 256 ? (UB == 7 && F8 ? 8 : 4) : (UB == 7 && F8 ? 8 : 1)), 8)))
void decode_resident_kernel(DecodeParams p) {
  using S = Shape<T, D, THREADS>;
  using SC = SlotChunk<T, F8>;
  using SE = typename SC::elem;
  constexpr int VEC = S::VEC, LANES = S::LANES, ROWS = S::ROWS, U = UB;
  static_assert(U <= LANES, "a lane owns one slot score");
  static_assert(!(TP && (F8 || sizeof(T) != 2)), "two-phase loads take 16-bit input slots");
  __shared__ uint4 s_new[2][TP ? LANES : 1];     // TP: the new token's K and V rows
  __shared__ __attribute__((aligned(16))) float s_red[ROWS * D];
  __shared__ float s_m[ROWS], s_l[ROWS];
  __shared__ float s_logit[ROWS * U];
  __shared__ uint64_t s_key[S::WAVES];
  __shared__ float s_scw[S::WAVES][ROWS];       // each wave's copy of the scale factors

  const int unit = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = tid % LANES, g = tid / LANES;
  const int k = p.k, t = unit_bound(p.tpos, unit, p.heads, p.t, 0x7ffffffe);
  const int n = min(k, t);
  const bool full = n == k;
  const int limit = t - p.k_local;

  SE* ks = static_cast<SE*>(p.k_slots) + (size_t)unit * k * D;
  SE* vs = static_cast<SE*>(p.v_slots) + (size_t)unit * k * D;
  const T* kn = static_cast<const T*>(p.k_new) + (size_t)unit * D;
  const T* vn = static_cast<const T*>(p.v_new) + (size_t)unit * D;
  int32_t* pos = p.slot_pos + (size_t)unit * k;
  float* acc = p.acc + (size_t)unit * k;

  // Every load of the unit (with TP: every K load), issued before any is consumed.
  const uint4 qr = ld16(static_cast<const T*>(p.q) + (size_t)unit * D + rl * VEC);
  typename SC::type kr[U], vr[U];
  // TP: one base address per lane and a constant step per slot, row u valid when
  // g < n - u * ROWS (a compare against a uniform value), rows past the valid slots read
  // the new token's row.
  const size_t lane_off = (size_t)g * D + rl * VEC;
  uint4 knr, vnr;
  if constexpr (F8) {                           // first, so its codes are formed early
    knr = ld16(kn + rl * VEC);
    vnr = ld16(vn + rl * VEC);
  }
  if constexpr (TP) {
    const SE* kb = ks + lane_off;
#pragma unroll
    for (int u = 0; u < U; ++u)
      kr[u] = ld_slot(g < n - u * ROWS ? kb + u * ROWS * D : kn + rl * VEC);
  } else {
    load_rows<T, D, U, THREADS, F8>(ks, vs, kn, vn, g, n, rl, kr, vr);
  }
  const int jo = rl * ROWS + g;                 // slot whose score this lane owns
  const bool own = rl < U && jo < n;
  const int jc = own ? jo : 0;
  const float acc_old = acc[jc];
  const int pos_old = pos[jc];
  if constexpr (!TP && !F8) {
    knr = ld16(kn + rl * VEC);
    vnr = ld16(vn + rl * VEC);
  }
  __builtin_amdgcn_sched_barrier(0);            // keep every load ahead of the math

  // The new token's row as it will be stored (TP: read back from LDS at the store).
  typename SC::type kst, vst;
  if constexpr (F8) {
    kst = quant_e4m3<T>(knr, p.k_inv);
    vst = quant_e4m3<T>(vnr, p.v_inv);
    // The new token's K codes join the rows now, its V codes at the PV product.
#pragma unroll
    for (int u = 0; u < U; ++u) kr[u] = g + u * ROWS < n ? kr[u] : kst;
  } else if constexpr (!TP) {
    kst = knr;
    vst = vnr;
  }
  float s[U], mg, lg, o[VEC];

  // Once every row group's maximum, sum and logits are in LDS. fold(): the row groups'
  // scale factors 2^(m_g - M), formed by every wave for itself with wave-uniform folds
  // (lane r holds groups r and r + 64, one exp2 per lane) into the wave's own LDS copy, and
  // the normaliser. choose(): every slot's new score, the masked argmin and the bookkeeping
  // stores; it gives the victim's slot to the lanes that store its row. Neither needs a V
  // row.
  struct Fold {
    float M, inv, p_new, lg_own;
  };
  auto fold = [&]() -> Fold {
    static_assert(ROWS <= 2 * kWave, "at most two row groups per lane");
    // Every LDS read of this stretch is issued here (clamped indices), one round trip.
    const bool in_a = lane < ROWS, in_b = lane + kWave < ROWS;
    const float m_a0 = s_m[in_a ? lane : 0], m_b0 = s_m[in_b ? lane + kWave : 0];
    const float l_a0 = s_l[in_a ? lane : 0], l_b0 = s_l[in_b ? lane + kWave : 0];
    const float lg_new = s_logit[n], lg_own = s_logit[own ? jo : 0];
    const float m_a = in_a ? m_a0 : -INFINITY;
    const float m_b = in_b ? m_b0 : -INFINITY;
    const float M = wave_max_uniform(fmaxf(m_a, m_b));
    const float sc_a = m_a == -INFINITY ? 0.f : fast_exp2(m_a - M);
    const float sc_b = m_b == -INFINITY ? 0.f : fast_exp2(m_b - M);
    const float l_ab = (in_a ? l_a0 * sc_a : 0.f) + (in_b ? l_b0 * sc_b : 0.f);
    const float inv = __builtin_amdgcn_rcpf(wave_sum_uniform(l_ab));
    if (lane < ROWS) s_scw[wave][lane] = sc_a;
    if (lane + kWave < ROWS) s_scw[wave][lane + kWave] = sc_b;
    return {M, inv, fast_exp2(lg_new - M) * inv, lg_own};
  };
  auto choose = [&](const Fold& f) -> int {
    uint64_t key = ~0ull;
    float a = 0.f;
    if (own) {
      const float pj = fast_exp2(f.lg_own - f.M) * f.inv;
      a = acc_old + pj;
      acc[jo] = a;
      if (full && pos_old <= limit)
        key = score_key(policy_key(p.policy, p.policy_param, a, pj, pos_old), pos_old);
    }
    const uint64_t wmin = wave_min_u64_uniform(key);
    if (lane == 0) s_key[wave] = wmin;
    // The waves' minima. Taken while V rows are in flight (two phases, 256 threads) this
    // barrier must not wait for them; elsewhere a __syncthreads measured slightly faster.
    if constexpr (TP && THREADS == 256) lds_barrier();
    else __syncthreads();
    uint64_t best = s_key[0];
#pragma unroll
    for (int w = 1; w < S::WAVES; ++w) best = s_key[w] < best ? s_key[w] : best;

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
    if (meta) {                                 // the lane that wrote acc[dst] above, if any
      pos[dst] = t;
      acc[dst] = f.p_new;
      if (p.victim_slot) p.victim_slot[unit] = full ? dst : -1;
      if (p.evicted_pos) p.evicted_pos[unit] = full ? pos_old : -1;
      if (p.evicted_acc) p.evicted_acc[unit] = full ? a : 0.f;
    }
    return dst;
  };
  // Output, once s_red holds every row group's partial: every wave takes CW columns; the
  // SL lanes of one column (lanes c, c + CW, ...) each sum RS of the row groups, then fold
  // their partial sums with lane swaps.
  auto write_out = [&](float scale) {
    constexpr int SL = THREADS / D, CW = kWave / SL, RS = ROWS / SL;
    static_assert(SL * CW == kWave && RS * SL == ROWS, "output split");
    const int c = wave * CW + lane % CW, sl = lane / CW;
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < RS; ++j) {
      const int r = sl * RS + j;
      v = fmaf(s_red[r * D + c], s_scw[wave][r], v);
    }
#pragma unroll
    for (int w = CW; w < kWave; w *= 2) v += __shfl_xor(v, w, kWave);
    if (sl == 0) p.out[(size_t)unit * D + c] = v * scale;
  };
  if constexpr (TP) {
    // Row n (the new token) sits in row group n % ROWS at u = n / ROWS (k + 1 <= U * ROWS).
    const int un = n / ROWS;
    const bool gn = g == n % ROWS;
    mg = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float d = row_sum<LANES>(chunk_dot(qr, kr[u], 0.f, T{})) * p.qk_scale;
      s[u] = g <= n - u * ROWS ? d : -INFINITY;
      mg = fmaxf(mg, s[u]);
    }
    if (gn) {
      uint4 x = kr[0];
#pragma unroll
      for (int u = 1; u < U; ++u) x = sel16(u == un, kr[u], x);
      s_new[0][rl] = x;
    }
    if (rl == 0) {                              // the logits are staged now: s[] turns into
#pragma unroll                                  // the weights below
      for (int u = 0; u < U; ++u) s_logit[u * ROWS + g] = s[u];
    }
    __builtin_amdgcn_sched_barrier(0);          // the V loads reuse the K registers
    const SE* vb = vs + lane_off;
#pragma unroll
    for (int u = 0; u < U; ++u)
      vr[u] = ld_slot(g < n - u * ROWS ? vb + u * ROWS * D : vn + rl * VEC);
    const float mref = mg == -INFINITY ? 0.f : mg;
    lg = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {               // the weights, while the V rows are in flight
      s[u] = fast_exp2(s[u] - mref);
      lg += s[u];
    }
    // The V rows of the slots, weighted, and the new token's V row (for the store).
    auto weigh_v = [&]() {
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[i] = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[VEC];
        unpack(vr[u], vf, T{});
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = fmaf(s[u], vf[i], o[i]);
      }
      __builtin_amdgcn_sched_barrier(0);          // the copy below waits for every V row
      if (gn) {
        uint4 x = vr[0];
#pragma unroll
        for (int u = 1; u < U; ++u) x = sel16(u == un, vr[u], x);
        s_new[1][rl] = x;
      }
    };
    if constexpr (THREADS == 256) {
      // The decision needs only the logits, so it is taken while the V rows are in
      // flight; once they land, the PV product, one fold and the stores remain. The
      // barriers before that wait on LDS only: a __syncthreads would first wait for every
      // load in flight. (The 1024-thread shape would need more than the 64 VGPRs that keep
      // two of its workgroups on a CU; it decides after the V rows.)
      if (rl == 0) {
        s_m[g] = mg;
        s_l[g] = lg;
      }
      lds_barrier();                            // group maxima, sums and logits staged
      const Fold f = fold();
      const int dst = choose(f);
      weigh_v();
#pragma unroll
      for (int i = 0; i < VEC; ++i) s_red[g * D + rl * VEC + i] = o[i];
      __syncthreads();                          // every V read is consumed
      write_out(f.inv);
      if (dst >= 0) {
        SC::store(ks + (size_t)dst * D + rl * VEC, s_new[0][rl]);
        SC::store(vs + (size_t)dst * D + rl * VEC, s_new[1][rl]);
      }
      return;
    }
    weigh_v();
  } else {
    if constexpr (F8)
      group_softmax<T, D, U, THREADS, typename SC::type, true>(qr, p.qk_scale, kr, vr, g, n, s, mg,
                                                               lg, o, vst);
    else
      group_softmax<T, D, U, THREADS>(qr, p.qk_scale, kr, vr, g, n, s, mg, lg, o);
  }

#pragma unroll
  for (int i = 0; i < VEC; ++i) s_red[g * D + rl * VEC + i] = o[i];
  if (rl == 0) {
    s_m[g] = mg;
    s_l[g] = lg;
    if constexpr (!TP) {
#pragma unroll
      for (int u = 0; u < U; ++u) s_logit[u * ROWS + g] = s[u];
    }
  }
  __syncthreads();                              // every K/V read is consumed
  const Fold f = fold();
  write_out(F8 ? f.inv * p.v_scale : f.inv);    // E4M3: values in code units until here
  const int dst = choose(f);
  if (dst >= 0) {
    if constexpr (TP) {
      kst = s_new[0][rl];
      vst = s_new[1][rl];
    }
    SC::store(ks + (size_t)dst * D + rl * VEC, kst);
    SC::store(vs + (size_t)dst * D + rl * VEC, vst);
  }
}

// --------------------------------------------------------------------- split --

constexpr int kPartThreads = 256;
// The largest cache (H2O_MAX_SLOTS, fp32 at d = 128: 32 lanes per row, the smallest chunk)
// must split into no more chunks than the combine's tables hold.
constexpr int kMinChunk = (kPartThreads / 32) * kPartBatch;
static_assert((H2O_MAX_SLOTS + kMinChunk) / kMinChunk <= kMaxSplits,
              "split count of the largest cache exceeds kMaxSplits");
// 512 threads with 8 slots each per load batch: 1024 threads with 4 measured 5% slower on
// the 4096-slot stream (fewer waves to launch on the unit's CU, the same one round trip).
constexpr int kCombThreads = 512;

template <typename T, int D, bool F8>
__global__ __launch_bounds__(kPartThreads) void decode_split_partial_kernel(DecodeParams p,
                                                                            SplitScratch w) {
  using S = Shape<T, D, kPartThreads>;
  using SC = SlotChunk<T, F8>;
  using SE = typename SC::elem;
  constexpr int VEC = S::VEC, LANES = S::LANES, ROWS = S::ROWS, U = kPartBatch;
  constexpr int C = ROWS * U;                   // slots per workgroup
  __shared__ __attribute__((aligned(16))) float s_red[ROWS * D];
  __shared__ float s_m[ROWS], s_l[ROWS], s_sc[ROWS];

  const int nsplit = w.splits;
  const int unit = blockIdx.x / nsplit, sp = blockIdx.x - unit * nsplit;
  const int tid = threadIdx.x;
  const int rl = tid % LANES, g = tid / LANES;
  const int k = p.k, n = min(k, unit_bound(p.tpos, unit, p.heads, p.t, 0x7ffffffe));
  const SE* ks = static_cast<const SE*>(p.k_slots) + (size_t)unit * k * D;
  const SE* vs = static_cast<const SE*>(p.v_slots) + (size_t)unit * k * D;
  const T* kn = static_cast<const T*>(p.k_new) + (size_t)unit * D;
  const T* vn = static_cast<const T*>(p.v_new) + (size_t)unit * D;
  float* logit = w.logits + (size_t)unit * (k + 1);

  // This workgroup's chunk [sp*C, sp*C + C) of the n + 1 keys.
  const int first = sp * C + g;
  const uint4 qr = ld16(static_cast<const T*>(p.q) + (size_t)unit * D + rl * VEC);
  typename SC::type kr[U], vr[U];
  load_rows<T, D, U, kPartThreads, F8>(ks, vs, kn, vn, first, n, rl, kr, vr);
  uint4 knr, vnr;
  if constexpr (F8) {
    knr = ld16(kn + rl * VEC);
    vnr = ld16(vn + rl * VEC);
  }
  __builtin_amdgcn_sched_barrier(0);            // keep every load ahead of the math
  if constexpr (F8)
    fill_new_rows<T, D, U, kPartThreads>(first, n, quant_e4m3<T>(knr, p.k_inv),
                                         quant_e4m3<T>(vnr, p.v_inv), kr, vr);
  float s[U], mg, lg, o[VEC];
  group_softmax<T, D, U, kPartThreads>(qr, p.qk_scale, kr, vr, first, n, s, mg, lg, o);
  if (rl == 0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (first + u * ROWS <= n) logit[first + u * ROWS] = s[u];
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) s_red[g * D + rl * VEC + i] = o[i];
  if (rl == 0) { s_m[g] = mg; s_l[g] = lg; }
  __syncthreads();
  // Chunk partial: max m, sum l and out relative to m (1 / l is not applied).
  if (tid < kWave) {
    float m = -INFINITY;
#pragma unroll
    for (int r = tid; r < ROWS; r += kWave) m = fmaxf(m, s_m[r]);
    m = group_max<kWave>(m);
    float l = 0.f;
#pragma unroll
    for (int r = tid; r < ROWS; r += kWave) {
      const float sc = s_m[r] == -INFINITY ? 0.f : fast_exp2(s_m[r] - m);
      s_sc[r] = sc;
      l = fmaf(s_l[r], sc, l);
    }
    l = group_sum<kWave>(l);
    if (tid == 0) {
      float* pml = w.part_ml + ((size_t)unit * nsplit + sp) * 2;
      pml[0] = m;
      pml[1] = l;
    }
  }
  __syncthreads();
  float* po = w.part_o + ((size_t)unit * nsplit + sp) * D;
  for (int c = tid; c < D; c += kPartThreads) {
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) v = fmaf(s_red[r * D + c], s_sc[r], v);
    po[c] = v;
  }
}

// One memory round trip: the first batch of every load the unit needs (the partial
// statistics, which every wave folds for itself; the partial outs; the slots' logits,
// scores and positions; the new token's logit and K/V) is issued before any is
// consumed. Further batches (more than QB * G splits or R * kCombThreads slots) follow
// in loops.
template <typename T, int D, bool F8>
__global__ __launch_bounds__(kCombThreads) void decode_split_combine_kernel(DecodeParams p,
                                                                            SplitScratch w) {
  using SC = SlotChunk<T, F8>;
  using SE = typename SC::elem;
  constexpr int VEC = Chunk<T>::N, LANES = D / VEC;
  constexpr int WAVES = kCombThreads / kWave;
  constexpr int G = kCombThreads / D;           // groups that share the partial-out sums
  constexpr int QB = 16;                        // partial outs per thread per load batch
  constexpr int R = 8;                          // slots per thread per load batch
  constexpr int MQ = (kMaxSplits + kWave - 1) / kWave;   // partial statistics per lane
  static_assert(QB * G <= kMaxSplits, "first batch of partial outs");
  __shared__ float s_scw[WAVES][kMaxSplits];    // each wave's copy of the split scale factors
  __shared__ float s_o[G * D];
  __shared__ uint64_t s_key[WAVES];
  __shared__ int s_dst;

  const int unit = blockIdx.x, nsplit = w.splits;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = p.k, t = unit_bound(p.tpos, unit, p.heads, p.t, 0x7ffffffe);
  const int n = min(k, t);
  const bool full = n == k;
  const int limit = t - p.k_local;
  SE* ks = static_cast<SE*>(p.k_slots) + (size_t)unit * k * D;
  SE* vs = static_cast<SE*>(p.v_slots) + (size_t)unit * k * D;
  const T* kn = static_cast<const T*>(p.k_new) + (size_t)unit * D;
  const T* vn = static_cast<const T*>(p.v_new) + (size_t)unit * D;
  int32_t* pos = p.slot_pos + (size_t)unit * k;
  float* acc = p.acc + (size_t)unit * k;
  const float* logit = w.logits + (size_t)unit * (k + 1);
  const float* pml = w.part_ml + (size_t)unit * nsplit * 2;
  const float* po = w.part_o + (size_t)unit * nsplit * D;
  const int c = tid % D, grp = tid / D;

  float pm[MQ], pl[MQ];
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    const int q = lane + i * kWave, qc = q < nsplit ? q : 0;
    pm[i] = pml[2 * qc];
    pl[i] = pml[2 * qc + 1];
  }
  float pov[QB];
#pragma unroll
  for (int i = 0; i < QB; ++i) {
    const int q = grp + i * G;
    pov[i] = po[(size_t)(q < nsplit ? q : 0) * D + c];
  }
  float lg[R], ac[R];
  int ps[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int j = i * kCombThreads + tid, jc = j < n ? j : 0;
    lg[i] = logit[jc];
    ac[i] = acc[jc];
    ps[i] = pos[jc];
  }
  const float lg_new = logit[n];
  const uint4 kvn = ld16((tid < LANES ? kn : vn) + (tid % LANES) * VEC);
  if (tid == 0) s_dst = full ? -1 : n;
  __builtin_amdgcn_sched_barrier(0);            // keep every load ahead of the math

  // Global max M and 1 / sum over the splits, wave-uniform in every wave.
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < MQ; ++i)
    if (lane + i * kWave < nsplit) mx = fmaxf(mx, pm[i]);
  const float M = wave_max_uniform(mx);
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    const int q = lane + i * kWave;
    const float sc = q < nsplit && pm[i] != -INFINITY ? fast_exp2(pm[i] - M) : 0.f;
    if (q < kMaxSplits) s_scw[wave][q] = sc;
    l = fmaf(pl[i], sc, l);
  }
  const float inv = 1.0f / wave_sum_uniform(l);
  const float out_scale = F8 ? inv * p.v_scale : inv;   // E4M3: values in code units until here

  // out: G groups of D threads each sum every G-th partial, then a fixed-order merge.
  {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < QB; ++i) v = fmaf(pov[i], s_scw[wave][grp + i * G], v);
    for (int q = grp + QB * G; q < nsplit; q += G)
      v = fmaf(po[(size_t)q * D + c], s_scw[wave][q], v);
    s_o[grp * D + c] = v;
  }
  // scores: slot j = tid + i * kCombThreads
  uint64_t best = ~0ull;
  int best_slot = -1;
  float best_acc = 0.f;
  auto score = [&](int j, float lgv, float acv, int psv) {
    if (j < n) {
      const float pj = fast_exp2(lgv - M) * inv;
      const float a = acv + pj;
      acc[j] = a;
      if (full && psv <= limit) {
        const uint64_t key = score_key(policy_key(p.policy, p.policy_param, a, pj, psv), psv);
        if (key < best) { best = key; best_slot = j; best_acc = a; }
      }
    }
  };
#pragma unroll
  for (int i = 0; i < R; ++i) score(i * kCombThreads + tid, lg[i], ac[i], ps[i]);
  for (int base = R * kCombThreads; base < n; base += R * kCombThreads) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int j = base + i * kCombThreads + tid, jc = j < n ? j : 0;
      lg[i] = logit[jc];
      ac[i] = acc[jc];
      ps[i] = pos[jc];
    }
#pragma unroll
    for (int i = 0; i < R; ++i) score(base + i * kCombThreads + tid, lg[i], ac[i], ps[i]);
  }
  const uint64_t wmin = wave_min_u64(best);
  if (lane == 0) s_key[wave] = wmin;
  __syncthreads();
  if (tid < D) {
    float v = 0.f;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) v += s_o[gi * D + tid];
    p.out[(size_t)unit * D + tid] = v * out_scale;
  }
  uint64_t gbest = s_key[0];
#pragma unroll
  for (int q = 1; q < WAVES; ++q) gbest = s_key[q] < gbest ? s_key[q] : gbest;
  // The victim is the slot whose key is gbest (keys are unique: positions are); the thread
  // that wrote its score publishes it and later writes its metadata, keeping them in order.
  if (full && best_slot >= 0 && best == gbest) s_dst = best_slot;
  __syncthreads();
  const int dst = s_dst;
  if (dst >= 0) {
    if (tid < 2 * LANES) {
      SE* row = (tid < LANES ? ks : vs) + (size_t)dst * D + (tid % LANES) * VEC;
      if constexpr (F8)
        SC::store(row, quant_e4m3<T>(kvn, tid < LANES ? p.k_inv : p.v_inv));
      else
        SC::store(row, kvn);
    }
    if (tid == dst % kCombThreads) {            // visited slot dst in the score loop
      pos[dst] = t;
      acc[dst] = fast_exp2(lg_new - M) * inv;
      if (full && p.evicted_acc) p.evicted_acc[unit] = best_acc;   // the victim's final score
    }
  }
  if (tid == 0) {
    if (p.victim_slot) p.victim_slot[unit] = full ? dst : -1;
    if (p.evicted_pos) p.evicted_pos[unit] = full && dst >= 0 ? (int32_t)(uint32_t)gbest : -1;
    if (p.evicted_acc && !(full && dst >= 0)) p.evicted_acc[unit] = 0.f;
  }
}

// ------------------------------------------------------------------ dispatch --

template <typename T, int D, bool F8 = false>
hipError_t run(const DecodeParams& p, const SplitScratch& w, hipStream_t s) {
  const DecodePlan plan = plan_decode(sizeof(T), D, p.k, p.units);
  if (plan.splits == 0) {
    if (plan.threads == 256) {
      if constexpr (sizeof(T) == 2) {
        if (p.k + 1 <= Shape<T, D, 256>::ROWS * 7) {
          // Two phases only where the one-phase kernel (five workgroups per CU) cannot hold
          // every unit at once: with fewer units the extra round trip costs more than it
          // saves (OPT-6.7B layer, 256 units: 4.32 -> 4.57 us; LLaMA-7B layer, 2048 units:
          // 19.7 -> 19.4 us, and 23.3 -> 22.5 us per launch in the 32-layer stack).
          if (!F8 && p.units > kTwoPhaseUnits)
            decode_resident_kernel<T, D, 256, F8, 7, !F8><<<dim3(p.units), dim3(256), 0, s>>>(p);
          else
            decode_resident_kernel<T, D, 256, F8, 7><<<dim3(p.units), dim3(256), 0, s>>>(p);
          return hipGetLastError();
        }
      }
      decode_resident_kernel<T, D, 256, F8><<<dim3(p.units), dim3(256), 0, s>>>(p);
    }
    else {
      if constexpr (sizeof(T) == 2) {
        if (p.k + 1 <= Shape<T, D, 1024>::ROWS * 7) {
          // Two phases at 1024 threads: two workgroups per CU instead of one (OPT-30B layer,
          // 896 units: 38.2 -> 31.0 us warm, 49.5 -> 41.3 us MALL-cold).
          decode_resident_kernel<T, D, 1024, F8, 7, !F8><<<dim3(p.units), dim3(1024), 0, s>>>(p);
          return hipGetLastError();
        }
      }
      decode_resident_kernel<T, D, 1024, F8><<<dim3(p.units), dim3(1024), 0, s>>>(p);
    }
    return hipGetLastError();
  }
  decode_split_partial_kernel<T, D, F8>
      <<<dim3((unsigned)(p.units * plan.splits)), dim3(kPartThreads), 0, s>>>(p, w);
  if (hipError_t e = hipGetLastError()) return e;
  decode_split_combine_kernel<T, D, F8><<<dim3(p.units), dim3(kCombThreads), 0, s>>>(p, w);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int elem_bytes, int D, int k, int units) {
  (void)units;
  const int lanes = D * elem_bytes / 16;
  DecodePlan plan{256, 0};
  if (k + 1 <= (256 / lanes) * kBatch) return plan;
  if (k + 1 <= (1024 / lanes) * kBatch) { plan.threads = 1024; return plan; }
  const int chunk = (kPartThreads / lanes) * kPartBatch;
  plan.splits = (k + 1 + chunk - 1) / chunk;
  return plan;
}

size_t decode_scratch_bytes(int elem_bytes, int D, int k, int units) {
  const DecodePlan plan = plan_decode(elem_bytes, D, k, units);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  if (!plan.splits) return 0;
  return up((size_t)units * plan.splits * 2 * 4) + up((size_t)units * plan.splits * D * 4) +
         up((size_t)units * (k + 1) * 4);
}

SplitScratch carve_decode_scratch(int elem_bytes, int D, int k, int units, void* scratch) {
  const DecodePlan plan = plan_decode(elem_bytes, D, k, units);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* b = static_cast<char*>(scratch);
  SplitScratch w{};
  w.splits = plan.splits;
  w.part_ml = reinterpret_cast<float*>(b);
  b += up((size_t)units * plan.splits * 2 * 4);
  w.part_o = reinterpret_cast<float*>(b);
  b += up((size_t)units * plan.splits * D * 4);
  w.logits = reinterpret_cast<float*>(b);
  return w;
}

hipError_t launch_decode(DType dt, bool f8, int D, const DecodeParams& p, const SplitScratch& w,
                         hipStream_t s) {
  if (f8) {
    if (dt == DType::F16) return D == 64 ? run<_Float16, 64, true>(p, w, s) : run<_Float16, 128, true>(p, w, s);
    return D == 64 ? run<__bf16, 64, true>(p, w, s) : run<__bf16, 128, true>(p, w, s);
  }
  switch (dt) {
    case DType::F32: return D == 64 ? run<float, 64>(p, w, s) : run<float, 128>(p, w, s);
    case DType::F16: return D == 64 ? run<_Float16, 64>(p, w, s) : run<_Float16, 128>(p, w, s);
    default: return D == 64 ? run<__bf16, 64>(p, w, s) : run<__bf16, 128>(p, w, s);
  }
}

}  // namespace h2o
