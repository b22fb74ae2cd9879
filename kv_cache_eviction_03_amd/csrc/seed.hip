// Cache seeding after the prompt, and the reset of a layer's slots.
//
// seed: per unit, keep the last k_local prompt positions (the recent tokens of
// the H2O blog, ttsmallhot.github.io, §2.2) plus the k_heavy positions of
// [0, T - k_local) with the highest fp32 column sum, i.e. the top-k of the
// cumulative attention ("H2O Heavy-Hitter Oracle 分析", §3.1) — or, under Top-K
// (blog §3.1.1: the highest current attention), the highest probability in the
// prompt's last attention row, or, under a position policy (blog §3.1.1, §3.3 Q1),
// the highest 0/1 position class. Ties rank the newer position higher, so the older
// one is dropped. If T <= k every position is kept. Kept positions fill slots 0.. in
// ascending order; the other slots are marked free. The seeded running score is the
// column sum under every policy.
//
// last_row (Top-K only, before the seed): per unit, the logits of the last prompt
// query against every prompt key, then their softmax, written as the seed scores.
//
// Selection: column sums are >= 0, so their fp32 bit patterns order like the
// values. Four MSB-first radix passes (8-bit digits, 256-bin LDS histogram, a
// wave-level scan of the bins) find the k_heavy-th largest bit pattern v* and
// how many positions equal to v* must be kept. One ordered ballot sweep over
// the positions then keeps every candidate above v*, the newest of those equal
// to v*, and the recent window, writing kept positions to slots in order.
// Copies: the recent window's K/V rows (every row when T <= k) go to slots known
// in advance, so they are issued first and overlap the column-sum reads and the
// selection; the heavy rows follow the selection.
// The column sums arrive as partial rows (one per block of part_rows query rows);
// the kernel adds them in row order, writes the sums out, and stages them in LDS
// when they fit (T + k <= 15872 words); the seeded scores are then read back
// from LDS.
//
// E4M3 slots (F8): each copied row is quantised on the way (x * 1/scale, clamped to +-448,
// nearest-even E4M3 codes), 8 codes per 16-byte chunk of the prompt row.
//
// reset: slot_pos = -1, acc = 0 (blog §2.3: freeing a slot only marks it).
#include <type_traits>

#include "h2o_device.hpp"
#include "h2o_kernels.hpp"

namespace h2o {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// Column sums are staged in LDS when slot table + sums fit in 62 KB of dynamic LDS.
constexpr int kStageWords = 62 * 1024 / 4;
// Ts = rows stored per unit (sizes the LDS), Tb = this unit's prompt length.
__host__ __device__ inline bool stage_alloc(int Ts, int k) { return Ts + k <= kStageWords; }
__host__ __device__ inline bool stage_bits(int Ts, int Tb, int k) { return Tb > k && stage_alloc(Ts, k); }

// Inclusive prefix sum over the 64 lanes of a wave, with DPP lane moves only: shifts by
// 1, 2, 4 and 8 inside each 16-lane row (lanes shifted in from outside the row read 0),
// then row_bcast:15 adds the last lane of rows 0 and 2 to rows 1 and 3, and row_bcast:31
// the last lane of row 1 to rows 2 and 3.
__device__ __forceinline__ unsigned wave_prefix(unsigned v) {
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

template <typename T, int D, bool F8>
__global__ __launch_bounds__(kThreads) void seed_kernel(SeedParams p) {
  using SC = SlotChunk<T, F8>;
  using SE = typename SC::elem;
  extern __shared__ int lds_dyn[];               // [k] slot -> position, then [T] staged bits
  __shared__ unsigned hist[2][256];             // radix passes alternate between the two
  __shared__ unsigned wsum[kWaves];
  __shared__ unsigned s_sel, s_above;
  __shared__ int wcnt[2][kWaves];

  const int unit = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int Ts = p.T, k = p.k_heavy + p.k_local;
  const int T_ = unit_bound(p.lens, unit, p.heads, Ts, Ts);   // this unit's prompt length
  float* c = p.colsum + (size_t)unit * Ts;
  int* slot_of = lds_dyn;
  unsigned* bits = reinterpret_cast<unsigned*>(lds_dyn + k);
  const bool staged = stage_bits(Ts, T_, k);

  constexpr int CPR = D * (int)sizeof(T) / 16;   // 16-byte chunks per row
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int B = 4;                           // copies in flight per thread (more measured slower)
  const T* K = static_cast<const T*>(p.k) + (size_t)unit * Ts * D;
  const T* V = static_cast<const T*>(p.v) + (size_t)unit * Ts * D;
  SE* ks = static_cast<SE*>(p.k_slots) + (size_t)unit * k * D;
  SE* vs = static_cast<SE*>(p.v_slots) + (size_t)unit * k * D;
  // A prompt chunk as the slot stores it.
  auto put = [&](SE* dst_k, SE* dst_v, const uint4& kx, const uint4& vx) {
    if constexpr (F8) {
      SC::store(dst_k, quant_e4m3<T>(kx, p.k_inv));
      SC::store(dst_v, quant_e4m3<T>(vx, p.v_inv));
    } else {
      SC::store(dst_k, kx);
      SC::store(dst_v, vx);
    }
  };
  // Rows whose slot is known before the selection: every row when T <= k (slot = position),
  // else the recent window (positions T - k_local.., slots k_heavy..). Their first batch
  // of loads is issued now and lands while the column sums are formed.
  const int nfix = T_ <= k ? T_ : p.k_local;
  const int fsrc = T_ <= k ? 0 : T_ - p.k_local, fdst = T_ <= k ? 0 : p.k_heavy;
  const int ftotal = nfix * CPR;
  uint4 kf[B], vf[B];
  auto load_fix = [&](int base) {
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int idx = base + i * kThreads + tid;
      const int r = idx < ftotal ? idx / CPR : 0, ch = idx < ftotal ? idx - r * CPR : 0;
      const size_t src = (size_t)(fsrc + r) * D + ch * VEC;
      kf[i] = ld16(K + src);
      vf[i] = ld16(V + src);
    }
  };
  auto store_fix = [&](int base) {
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int idx = base + i * kThreads + tid;
      if (idx < ftotal) {
        const int r = idx / CPR, ch = idx - r * CPR;
        const size_t dst = (size_t)(fdst + r) * D + ch * VEC;
        put(ks + dst, vs + dst, kf[i], vf[i]);
      }
    }
  };
  load_fix(0);

  // c_j = sum of the partial rows r >= j / part_rows, in row order. JB positions per thread
  // and RR rows per batch, all loads of a batch in flight together (branch-free: loads
  // outside the triangle read the stretch's first word and are dropped).
  {
    constexpr int JB = 2, RR = 8;
    const int pb = p.part_rows, nr = (T_ + pb - 1) / pb;
    const float* part = p.colpart + (size_t)unit * colpart_stride(Ts, pb);
    for (int j0 = 0; j0 < T_; j0 += JB * kThreads) {
      float sum[JB];
#pragma unroll
      for (int a = 0; a < JB; ++a) sum[a] = 0.f;
      for (int r0 = j0 / pb; r0 < nr; r0 += RR) {   // rows below j0 / pb cover none of them
        float x[JB][RR];
#pragma unroll
        for (int a = 0; a < JB; ++a)
#pragma unroll
          for (int rr = 0; rr < RR; ++rr) {
            const int j = j0 + a * kThreads + tid, r = r0 + rr;
            const bool in = j < T_ && r < nr && j < (r + 1) * pb;   // row r covers key j
            x[a][rr] = part[in ? colpart_row_offset(r, pb) + j : 0];
            if (!in) x[a][rr] = 0.f;
          }
#pragma unroll
        for (int a = 0; a < JB; ++a)
#pragma unroll
          for (int rr = 0; rr < RR; ++rr) sum[a] += x[a][rr];
      }
#pragma unroll
      for (int a = 0; a < JB; ++a) {
        const int j = j0 + a * kThreads + tid;
        if (j < T_) {
          c[j] = sum[a];
          if (staged) bits[j] = __float_as_uint(sum[a]);
        }
      }
    }
  }
  store_fix(0);
  for (int base = B * kThreads; base < ftotal; base += B * kThreads) {
    load_fix(base);
    store_fix(base);
  }
  __syncthreads();                              // the sums are visible to the whole workgroup

  int n_keep;
  if (T_ <= k) {
    n_keep = T_;
    for (int s = tid; s < T_; s += kThreads) slot_of[s] = s;
  } else {
    // The selection reads its scores from the LDS stage (SRC 0), the column sums in global
    // memory (SRC 1) or, under Top-K, the last-row kernel's array (SRC 2); each source is
    // an instantiation of its own, so every read is a plain LDS or global load (a runtime
    // choice between the pointers would make them generic-address loads).
    auto select = [&](auto src_c) -> int {
    constexpr int SRC = decltype(src_c)::value;
    const int ncand = T_ - p.k_local;
    const float* rank = SRC == 2 ? p.rank + (size_t)unit * Ts : nullptr;
    // The ranking score of position j (a 0/1 position class under the position policies).
    auto key = [&](int j) -> unsigned {
      float cj;
      if constexpr (SRC == 0) cj = __uint_as_float(bits[j]);
      else if constexpr (SRC == 1) cj = c[j];
      else cj = rank[j];
      return __float_as_uint(policy_seed(p.policy, p.policy_param, cj, j));
    };

    unsigned prefix = 0, mask = 0, want = (unsigned)p.k_heavy, eq_total = 0;
    if (p.k_heavy > 0) {
      hist[1][tid] = 0;                          // the first pass counts into hist[1]
      for (int pass = 3; pass >= 0; --pass) {
        const int sh = pass * 8;
        unsigned* h = hist[pass & 1];
        // h was cleared during the previous pass (or above), and every read of it by the
        // pass that used it last came before the barrier that ended its counting loop.
        __syncthreads();
        for (int j0 = 0; j0 < ncand; j0 += kThreads) {
          const int j = j0 + tid;
          unsigned bin = 256u;                    // 256: no count from this lane
          if (j < ncand) {
            const unsigned b = key(j);
            if ((b & mask) == prefix) bin = (b >> sh) & 255u;
          }
          // Column sums of one prompt share a few exponents, so the high digits pile
          // into a few bins: the wave counts up to four distinct bins with one ballot
          // each, and only the lanes left over add one by one.
          uint64_t pend = __ballot(bin < 256u);
#pragma unroll
          for (int it = 0; it < 4 && pend; ++it) {
            const int leader = __builtin_ctzll(pend);
            const unsigned lb = (unsigned)__builtin_amdgcn_readlane((int)bin, leader);
            const uint64_t same = __ballot(bin == lb) & pend;
            if (lane == leader) atomicAdd(&h[lb], (unsigned)__popcll(same));
            pend &= ~same;
          }
          if ((pend >> lane) & 1ull) atomicAdd(&h[bin], 1u);
        }
        __syncthreads();
        // Thread i holds bin 255 - i, so a prefix over threads is a suffix over bins.
        const unsigned cnt = h[255 - tid];
        const unsigned incl_w = wave_prefix(cnt);
        if (lane == 63) wsum[wave] = incl_w;
        hist[(pass & 1) ^ 1][tid] = 0;           // the next pass's histogram
        __syncthreads();
        unsigned before = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) before += w < wave ? wsum[w] : 0u;
        const unsigned incl = before + incl_w, excl = incl - cnt;
        if (excl < want && want <= incl) {       // exactly one bin qualifies
          s_sel = 255u - (unsigned)tid;
          s_above = excl;
        }
        __syncthreads();
        prefix |= s_sel << sh;
        mask |= 255u << sh;
        want -= s_above;
        if (pass == 0) eq_total = h[s_sel];
        // No barrier here: the next pass writes s_sel, s_above and wsum only after two
        // barriers that every thread reaches after these reads.
      }
      __syncthreads();                           // s_sel / s_above reads done before reuse
    }
    // Keep: j >= ncand (recent window); bits > v*; bits == v* and among the `want`
    // newest such positions (want = how many equal ones are still needed).
    const unsigned vstar = prefix;
    const bool any_heavy = p.k_heavy > 0;
    int running = 0, eq_seen = 0;
    for (int base = 0; base < T_; base += kThreads) {
      const int j = base + tid;
      bool keep = false, eq = false;
      if (j < T_) {
        if (j >= ncand) {
          keep = true;
        } else if (any_heavy) {
          const unsigned b = key(j);
          eq = b == vstar;
          keep = b > vstar;
        }
      }
      const uint64_t beq = __ballot(eq);
      const int eq_in_wave = __popcll(beq & ((1ull << lane) - 1ull));
      if (lane == 0) wcnt[1][wave] = __popcll(beq);
      // Position index among equal keys decides whether this one is among the newest.
      __syncthreads();
      int eq_off = 0, eq_tot = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        eq_off += w < wave ? wcnt[1][w] : 0;
        eq_tot += wcnt[1][w];
      }
      if (eq && eq_seen + eq_off + eq_in_wave >= (int)eq_total - (int)want) keep = true;
      eq_seen += eq_tot;
      const uint64_t bk = __ballot(keep);
      const int in_wave = __popcll(bk & ((1ull << lane) - 1ull));
      if (lane == 0) wcnt[0][wave] = __popcll(bk);
      __syncthreads();
      int off = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        off += w < wave ? wcnt[0][w] : 0;
        total += wcnt[0][w];
      }
      if (keep && running + off + in_wave < k) slot_of[running + off + in_wave] = j;
      running += total;
      __syncthreads();
    }
    return running < k ? running : k;
    };
    n_keep = p.rank ? select(std::integral_constant<int, 2>{})
             : staged ? select(std::integral_constant<int, 0>{})
                      : select(std::integral_constant<int, 1>{});
  }
  __syncthreads();

  int32_t* pos = p.slot_pos + (size_t)unit * k;
  float* acc = p.acc + (size_t)unit * k;
  auto write_meta = [&](auto from_lds) {
    for (int s = tid; s < k; s += kThreads) {
      if (s < n_keep) {
        const int j = slot_of[s];
        pos[s] = j;
        if constexpr (decltype(from_lds)::value) acc[s] = __uint_as_float(bits[j]);
        else acc[s] = c[j];
      } else {
        pos[s] = -1;
        acc[s] = 0.f;
      }
    }
  };
  if (staged) write_meta(std::true_type{}); else write_meta(std::false_type{});
  // The heavy rows (slots [0, k_heavy) when T > k), gathered by the selection.
  const int total = (T_ > k ? p.k_heavy : 0) * CPR;
  for (int base = 0; base < total; base += B * kThreads) {
    uint4 kr[B], vr[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int idx = base + i * kThreads + tid;
      const int s = idx < total ? idx / CPR : 0, ch = idx < total ? idx - s * CPR : 0;
      const size_t src = (size_t)slot_of[s] * D + ch * VEC;
      kr[i] = ld16(K + src);
      vr[i] = ld16(V + src);
    }
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int idx = base + i * kThreads + tid;
      if (idx < total) {
        const int s = idx / CPR, ch = idx - s * CPR;
        const size_t dst = (size_t)s * D + ch * VEC;
        put(ks + dst, vs + dst, kr[i], vr[i]);
      }
    }
  }
}

// One workgroup per unit: s_j = q_{T-1} . k_j * log2(e) / sqrt(D) for every prompt key
// (row groups of LANES lanes read one key row as 16-byte chunks), then M = max s,
// L = sum 2^(s_j - M), P[T-1][j] = 2^(s_j - M) / L. The logits go through the rank array
// itself; every sum runs in a fixed order.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void last_row_kernel(LastRowParams p) {
  constexpr int VEC = Chunk<T>::N, LANES = D / VEC, ROWS = kThreads / LANES;
  __shared__ float s_red[kWaves];
  const int unit = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = tid % LANES, g = tid / LANES;
  const int Ts = p.T, T_ = unit_bound(p.lens, unit, p.heads, Ts, Ts);
  if (T_ <= p.k_slots) return;                  // every position is kept: nothing to rank
  const T* K = static_cast<const T*>(p.k) + (size_t)unit * Ts * D;
  const T* Q = static_cast<const T*>(p.q) + ((size_t)unit * Ts + (T_ - 1)) * D;
  float* rank = p.rank + (size_t)unit * Ts;
  float qf[VEC];
  load_f32(Q + rl * VEC, qf);

  float m = -INFINITY;
  for (int j0 = 0; j0 < T_; j0 += ROWS) {
    const int j = j0 + g, jc = j < T_ ? j : 0;
    float kf[VEC];
    load_f32(K + (size_t)jc * D + rl * VEC, kf);
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) d = fmaf(qf[i], kf[i], d);
    const float s = group_sum<LANES>(d) * p.qk_scale;
    if (j < T_) {
      if (rl == 0) rank[j] = s;
      m = fmaxf(m, s);
    }
  }
  auto block_fold = [&](float v, bool is_max) {
    v = is_max ? group_max<kWave>(v) : group_sum<kWave>(v);
    if (lane == 0) s_red[wave] = v;
    __syncthreads();                            // also publishes the rank writes above
    float r = s_red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = is_max ? fmaxf(r, s_red[w]) : r + s_red[w];
    __syncthreads();                            // s_red is reused by the next fold
    return r;
  };
  const float M = block_fold(m, true);
  float l = 0.f;
  for (int j = tid; j < T_; j += kThreads) l += fast_exp2(rank[j] - M);
  const float L = block_fold(l, false);
  for (int j = tid; j < T_; j += kThreads) rank[j] = fast_exp2(rank[j] - M) / L;
}

__global__ void reset_kernel(ResetParams p) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < p.n; i += stride) {
    p.slot_pos[i] = -1;
    p.acc[i] = 0.f;
  }
}

template <typename T, int D, bool F8 = false>
hipError_t seed(const SeedParams& p, hipStream_t s) {
  const int k = p.k_heavy + p.k_local;
  const size_t lds = (size_t)k * sizeof(int) + (stage_alloc(p.T, k) ? (size_t)p.T * 4 : 0);
  seed_kernel<T, D, F8><<<dim3((unsigned)p.units), dim3(kThreads), lds, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_seed(DType dt, bool f8, int D, const SeedParams& p, hipStream_t s) {
  if (f8) {
    if (dt == DType::F16) return D == 64 ? seed<_Float16, 64, true>(p, s) : seed<_Float16, 128, true>(p, s);
    return D == 64 ? seed<__bf16, 64, true>(p, s) : seed<__bf16, 128, true>(p, s);
  }
  switch (dt) {
    case DType::F32: return D == 64 ? seed<float, 64>(p, s) : seed<float, 128>(p, s);
    case DType::F16: return D == 64 ? seed<_Float16, 64>(p, s) : seed<_Float16, 128>(p, s);
    default: return D == 64 ? seed<__bf16, 64>(p, s) : seed<__bf16, 128>(p, s);
  }
}

hipError_t launch_last_row(DType dt, int D, const LastRowParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.units), block(kThreads);
  switch (dt) {
    case DType::F32:
      if (D == 64) last_row_kernel<float, 64><<<grid, block, 0, s>>>(p);
      else last_row_kernel<float, 128><<<grid, block, 0, s>>>(p);
      break;
    case DType::F16:
      if (D == 64) last_row_kernel<_Float16, 64><<<grid, block, 0, s>>>(p);
      else last_row_kernel<_Float16, 128><<<grid, block, 0, s>>>(p);
      break;
    default:
      if (D == 64) last_row_kernel<__bf16, 64><<<grid, block, 0, s>>>(p);
      else last_row_kernel<__bf16, 128><<<grid, block, 0, s>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_reset(const ResetParams& p, hipStream_t s) {
  const int64_t blocks64 = (p.n + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 4096 ? (blocks64 > 0 ? blocks64 : 1) : 4096);
  reset_kernel<<<dim3(blocks), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace h2o
