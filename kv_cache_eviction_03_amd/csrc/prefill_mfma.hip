// Prefill kernels for fp16 / bf16 storage on gfx950 MFMA.
//
// prefill_attn: causal attention over the prompt, O = softmax(Q K^T / sqrt(d)) V
//   with the row max/sum kept online (flash style), plus each row's
//   log-sum-exp. The scaled row softmax is the attention of the H2O blog
//   (ttsmallhot.github.io), §2.1.1.
// prefill_colsum: c_j = sum_{i >= j} P_ij, the cumulative attention of each
//   prompt token ("H2O Heavy-Hitter Oracle 分析", §3.1). The softmax of a row
//   is only final once the whole row is seen, so this kernel re-forms P from
//   the stored log-sum-exp, one key block per workgroup, and sums it over the
//   query rows in a fixed order (no float atomics, bit-reproducible).
//
// Both kernels compute S^T = K Q^T with v_mfma_f32_16x16x32_{f16,bf16}: lane l
// then holds the logits of query l%16 against keys 4*(l/16)+i of each 16-key
// block, so a query's softmax statistics live in the four lanes l%16 + 16*g.
// The PV product is computed as O^T = V^T P^T: P leaves the S^T accumulators
// directly as the B operand (no LDS round trip), and the output accumulators
// again belong to query l%16, so the online rescale is lane-local.
//
// Tiling: each wave holds RB blocks of 16 rows, so every operand read from LDS
// feeds RB MFMAs; the next key (or query) tile is loaded into registers while
// the current one is consumed from LDS. K and V tiles sit row-major in LDS
// (rows padded by 16 bytes); the V operand of the PV product is fetched with
// gfx950's transposing LDS read, so V needs no register transpose.
//
// bf16: P rounded to bf16 alone gives up to ~3e-3 abs error on O for N(0,1)
// data, so P is split into a bf16 high part and a bf16 residual, two MFMAs.
#include "h2o_device.hpp"
#include "h2o_kernels.hpp"

namespace h2o {
namespace {

constexpr int BN = 64;    // keys per tile (attention) / queries per tile (column sums)
constexpr float kLazy = 8.f;  // log2-domain slack before the running max is moved
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <typename T> __device__ __forceinline__ typename Vec8<T>::type ld8(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::type*>(p);
}

// LDS row strides. K/Q tiles are read 16 bytes per lane, one row per lane: a stride of
// D + 8 elements (4 dwords past a multiple of 32 banks) spreads consecutive rows over
// distinct banks. The V tile is read with the transposing 8-byte read, four 32-byte row
// segments per 16-lane group: a stride of D + 16 (8 dwords past a multiple of 32) puts
// those four segments in disjoint banks.
#ifndef H2O_KPAD
#define H2O_KPAD 8
#endif
#ifndef H2O_VPAD
#define H2O_VPAD 16
#endif
template <int D> struct Tile {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int KS = D + H2O_KPAD;            // K / Q tile stride (elements)
  static constexpr int VS = D + H2O_VPAD;            // V tile stride (elements)
  static constexpr int KCH = BN * CPR / kThreads;    // row chunks per thread
};

// One BN-row tile of a [T][D] matrix, held in registers between the global load
// and the LDS store. Rows past T are loaded from row T-1 and zeroed.
template <typename T, int D>
struct RowTile {
  uint4 c[Tile<D>::KCH];
  __device__ __forceinline__ void load(const T* src, int row0, int T_, int tid) {
    if (row0 + BN <= T_) {                       // whole tile in range
#pragma unroll
      for (int i = 0; i < Tile<D>::KCH; ++i) {
        const int ch = tid + i * kThreads, row = ch / Tile<D>::CPR, cc = ch % Tile<D>::CPR;
        c[i] = ld16(src + (size_t)(row0 + row) * D + cc * 8);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < Tile<D>::KCH; ++i) {
      const int ch = tid + i * kThreads, row = ch / Tile<D>::CPR, cc = ch % Tile<D>::CPR;
      const int r = row0 + row;
      uint4 v = ld16(src + (size_t)(r < T_ ? r : T_ - 1) * D + cc * 8);
      if (r >= T_) v = make_uint4(0, 0, 0, 0);
      c[i] = v;
    }
  }
  template <int STRIDE>
  __device__ __forceinline__ void store(T* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < Tile<D>::KCH; ++i) {
      const int ch = tid + i * kThreads, row = ch / Tile<D>::CPR, cc = ch % Tile<D>::CPR;
      st16(tile + row * STRIDE + cc * 8, c[i]);
    }
  }
};

// Transposed LDS read (gfx950 ds_read_b64_tr_b16). Within each 16-lane group the 16
// lanes' 4-element reads form 4 rows of 16 elements (row r = lanes 4r..4r+3 in
// order); lane i receives element i of each row. Pointing lane 4r + q at
// V[key_r][d0 + 4q] therefore hands lane i the values V[key_0..3][d0 + i]: four
// consecutive keys of one dim, the k-contiguous layout an MFMA A operand needs.
template <typename T> struct TrRead;
template <> struct TrRead<_Float16> {
  typedef short s4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f16x4 read(const _Float16* p) {
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4*)(p));
    return __builtin_bit_cast(f16x4, v);
  }
};
template <> struct TrRead<__bf16> {
  typedef short s4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ bf16x4 read(const __bf16* p) {
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4*)(p));
    return __builtin_bit_cast(bf16x4, v);
  }
};

template <typename T, int D, int RB, bool PREFETCH>
__global__ __launch_bounds__(kThreads) void prefill_attn_kernel(PrefillParams p) {
  using V8 = typename Vec8<T>::type;
  using V4 = typename Vec8<T>::half;
  constexpr bool kSplit = !__is_same(T, _Float16);
  constexpr int BM = kWaves * 16 * RB;
  constexpr int KS = Tile<D>::KS, VS = Tile<D>::VS;
  __shared__ __attribute__((aligned(16))) T k_tile[BN * KS];
  __shared__ __attribute__((aligned(16))) T v_tile[BN * VS];

  const int T_ = p.T;
  const int nqb = (T_ + BM - 1) / BM;
  const int r = blockIdx.x / p.units;          // longest rows first
  const int unit = blockIdx.x - r * p.units;
  const int qb = nqb - 1 - r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)unit * T_ * D;
  const T* Q = static_cast<const T*>(p.q) + base;
  const T* K = static_cast<const T*>(p.k) + base;
  const T* V = static_cast<const T*>(p.v) + base;
  const int row0 = qb * BM + wave * 16 * RB;    // this wave's first row

  V8 qa[RB][D / 32];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qr = row0 + rb * 16 + l16;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      V8 v = ld8(Q + (size_t)(qr < T_ ? qr : T_ - 1) * D + kk * 32 + 8 * g);
      if (qr >= T_) v = V8{};
      qa[rb][kk] = v;
    }
  }

  f32x4 o[RB][D / 16];
  float m[RB], ls[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    ls[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int kend = min(T_, (qb + 1) * BM);
  const int nkt = (kend + BN - 1) / BN;
  RowTile<T, D> kreg, vreg;
  if constexpr (PREFETCH) {
    kreg.load(K, 0, T_, tid);
    vreg.load(V, 0, T_, tid);
  }

  for (int kt = 0; kt < nkt; ++kt) {
    const int key0 = kt * BN;
    if constexpr (PREFETCH) {
      kreg.template store<KS>(k_tile, tid);
      vreg.template store<VS>(v_tile, tid);
      __syncthreads();
      if (kt + 1 < nkt) {
        kreg.load(K, key0 + BN, T_, tid);
        vreg.load(V, key0 + BN, T_, tid);
      }
      __builtin_amdgcn_sched_barrier(0);        // next tile's loads go out first
    } else {
      kreg.load(K, key0, T_, tid);
      vreg.load(V, key0, T_, tid);
      kreg.template store<KS>(k_tile, tid);
      vreg.template store<VS>(v_tile, tid);
      __syncthreads();
    }
    // Only tiles that reach past the wave's first row need the causal mask.
    const bool diag = key0 + BN - 1 > row0 || key0 + BN > T_;

    f32x4 s[RB][BN / 16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) s[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {       // consecutive MFMAs use different accumulators
      V8 a[BN / 16];
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) a[kb] = ld8(k_tile + (kb * 16 + l16) * KS + kk * 32 + 8 * g);
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb][kb] = mfma16x16x32(a[kb], qa[rb][kk], s[rb][kb]);
    }

    // Online softmax in the log2 domain with the 1/sqrt(d) scale folded into one FMA
    // per logit. The running max only moves when a row's new max exceeds it by more
    // than kLazy (checked per wave), so most tiles skip the output rescale; P then
    // stays <= 2^kLazy, well inside fp16/bf16 range.
    V8 pb[RB][BN / 32], pl[RB][BN / 32];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int qrow = row0 + rb * 16 + l16;
      float mx = -INFINITY;
      if (diag) {
#pragma unroll
        for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = key0 + kb * 16 + 4 * g + i;
            if (key > qrow || key >= T_) s[rb][kb][i] = -INFINITY;
            mx = fmaxf(mx, s[rb][kb][i]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[rb][kb][i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mt = mx * p.qk_scale;
      const bool grow = mt > m[rb] + kLazy;
      if (__any(grow)) {
        const float mnew = grow ? mt : m[rb];
        const float alpha = fast_exp2(m[rb] - mnew);
        m[rb] = mnew;
        ls[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) o[rb][db] *= alpha;
      }
      const float nm = -m[rb];
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = fast_exp2(fmaf(s[rb][kb][i], p.qk_scale, nm));
          s[rb][kb][i] = x;
          ps += x;
        }
      ls[rb] += ps;
#pragma unroll
      for (int ks = 0; ks < BN / 32; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[rb][ks][i] = (T)s[rb][2 * ks][i];
          pb[rb][ks][4 + i] = (T)s[rb][2 * ks + 1][i];
          if constexpr (kSplit) {
            pl[rb][ks][i] = (T)(s[rb][2 * ks][i] - (float)pb[rb][ks][i]);
            pl[rb][ks][4 + i] = (T)(s[rb][2 * ks + 1][i] - (float)pb[rb][ks][4 + i]);
          }
        }
    }

#pragma unroll
    for (int ks = 0; ks < BN / 32; ++ks)
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        // keys ks*32 + 4g + r (then + 16) of dim db*16 + l16: lane 4r + q of each
        // 16-lane group points at V[key][db*16 + 4q]
        const T* vr = v_tile + (ks * 32 + 4 * g + (l16 >> 2)) * VS + db * 16 + 4 * (l16 & 3);
        const V4 lo = TrRead<T>::read(vr);
        const V4 hi = TrRead<T>::read(vr + 16 * VS);
        const V8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          o[rb][db] = mfma16x16x32(a, pb[rb][ks], o[rb][db]);
          if constexpr (kSplit) o[rb][db] = mfma16x16x32(a, pl[rb][ks], o[rb][db]);
        }
      }
    __syncthreads();
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qrow = row0 + rb * 16 + l16;
    float lt = ls[rb] + __shfl_xor(ls[rb], 16, kWave);
    lt = lt + __shfl_xor(lt, 32, kWave);
    if (qrow < T_) {
      const float inv = 1.0f / lt;
      float* orow = p.out + ((size_t)unit * T_ + qrow) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const f32x4 v = o[rb][db] * inv;
        *reinterpret_cast<f32x4*>(orow + db * 16 + 4 * g) = v;
      }
      if (g == 0) p.lse2[(size_t)unit * T_ + qrow] = m[rb] + log2f(lt);
    }
  }
}

template <typename T, int D, int RB, bool PREFETCH>
__global__ __launch_bounds__(kThreads) void prefill_colsum_kernel(PrefillParams p) {
  using V8 = typename Vec8<T>::type;
  constexpr int BK = kWaves * 16 * RB;          // keys per workgroup
  constexpr int KS = Tile<D>::KS;
  __shared__ __attribute__((aligned(16))) T q_tile[BN * KS];
  __shared__ float lse_tile[BN];

  const int T_ = p.T;
  const int nq = (T_ + BN - 1) / BN;
  const int kb = blockIdx.x / p.units;          // early keys (most rows) first
  const int unit = blockIdx.x - kb * p.units;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)unit * T_ * D;
  const T* Q = static_cast<const T*>(p.q) + base;
  const T* K = static_cast<const T*>(p.k) + base;
  const float* lse = p.lse2 + (size_t)unit * T_;
  const int key0 = kb * BK + wave * 16 * RB;    // this wave's first key

  V8 ka[RB][D / 32];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int kr = key0 + rb * 16 + l16;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      V8 v = ld8(K + (size_t)(kr < T_ ? kr : T_ - 1) * D + kk * 32 + 8 * g);
      if (kr >= T_) v = V8{};
      ka[rb][kk] = v;
    }
  }
  float cs[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) cs[rb][i] = 0.f;

  const int qt0 = (kb * BK) / BN;
  RowTile<T, D> qreg;
  float lreg = 0.f;
  if constexpr (PREFETCH) {
    qreg.load(Q, qt0 * BN, T_, tid);
    if (tid < BN) lreg = qt0 * BN + tid < T_ ? lse[qt0 * BN + tid] : 0.f;
  }

  for (int qt = qt0; qt < nq; ++qt) {
    const int q0 = qt * BN;
    if constexpr (PREFETCH) {
      qreg.template store<KS>(q_tile, tid);
      if (tid < BN) lse_tile[tid] = lreg;
      __syncthreads();
      if (qt + 1 < nq) {
        qreg.load(Q, q0 + BN, T_, tid);
        if (tid < BN) lreg = q0 + BN + tid < T_ ? lse[q0 + BN + tid] : 0.f;
      }
      __builtin_amdgcn_sched_barrier(0);        // next tile's loads go out first
    } else {
      qreg.load(Q, q0, T_, tid);
      if (tid < BN) lreg = q0 + tid < T_ ? lse[q0 + tid] : 0.f;
      qreg.template store<KS>(q_tile, tid);
      if (tid < BN) lse_tile[tid] = lreg;
      __syncthreads();
    }
    const bool diag = q0 < key0 + 16 * RB;      // some queries of the tile precede some keys
    f32x4 s[BN / 16][RB];
#pragma unroll
    for (int qb = 0; qb < BN / 16; ++qb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[qb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {       // consecutive MFMAs use different accumulators
      V8 b[BN / 16];
#pragma unroll
      for (int qb = 0; qb < BN / 16; ++qb) b[qb] = ld8(q_tile + (qb * 16 + l16) * KS + kk * 32 + 8 * g);
#pragma unroll
      for (int qb = 0; qb < BN / 16; ++qb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[qb][rb] = mfma16x16x32(ka[rb][kk], b[qb], s[qb][rb]);
    }
    const bool masked = diag || q0 + BN > T_;
#pragma unroll
    for (int qb = 0; qb < BN / 16; ++qb) {
      const int q = q0 + qb * 16 + l16;
      const float nl = -lse_tile[qb * 16 + l16];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(fmaf(s[qb][rb][i], p.qk_scale, nl));
          if (masked) {
            const int key = key0 + rb * 16 + 4 * g + i;
            cs[rb][i] += (q < T_ && q >= key) ? e : 0.f;
          } else {
            cs[rb][i] += e;
          }
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = group_sum<16>(cs[rb][i]);
      const int key = key0 + rb * 16 + 4 * g + i;
      if (l16 == 0 && key < T_) p.colsum[(size_t)unit * T_ + key] = v;
    }
}

// Tuning knobs (compile-time): 16-row blocks per wave and register prefetch of the
// next tile, for the attention and the column-sum kernels.
// Defaults from a sweep on MI355X (OPT-30B-shaped prompt, T = 2048): attention
// 2.06 ms with RB = 2 + prefetch vs 3.2 ms with RB = 1; column sums 1.11 ms with
// RB = 2 and no prefetch.
#ifndef H2O_ATTN_RB
#define H2O_ATTN_RB 2
#endif
#ifndef H2O_ATTN_PREFETCH
#define H2O_ATTN_PREFETCH 1
#endif
#ifndef H2O_COLSUM_RB
#define H2O_COLSUM_RB 2
#endif
#ifndef H2O_COLSUM_PREFETCH
#define H2O_COLSUM_PREFETCH 0
#endif

template <typename T, int D>
hipError_t attn(const PrefillParams& p, hipStream_t s) {
  constexpr int BM = kWaves * 16 * H2O_ATTN_RB;
  const int nqb = (p.T + BM - 1) / BM;
  prefill_attn_kernel<T, D, H2O_ATTN_RB, H2O_ATTN_PREFETCH != 0>
      <<<dim3((unsigned)(nqb * p.units)), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}
template <typename T, int D>
hipError_t colsum(const PrefillParams& p, hipStream_t s) {
  constexpr int BK = kWaves * 16 * H2O_COLSUM_RB;
  const int nb = (p.T + BK - 1) / BK;
  prefill_colsum_kernel<T, D, H2O_COLSUM_RB, H2O_COLSUM_PREFETCH != 0>
      <<<dim3((unsigned)(nb * p.units)), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_attn_mfma(DType dt, int D, const PrefillParams& p, hipStream_t s) {
  if (dt == DType::F16) return D == 64 ? attn<_Float16, 64>(p, s) : attn<_Float16, 128>(p, s);
  return D == 64 ? attn<__bf16, 64>(p, s) : attn<__bf16, 128>(p, s);
}
hipError_t launch_prefill_colsum_mfma(DType dt, int D, const PrefillParams& p, hipStream_t s) {
  if (dt == DType::F16) return D == 64 ? colsum<_Float16, 64>(p, s) : colsum<_Float16, 128>(p, s);
  return D == 64 ? colsum<__bf16, 64>(p, s) : colsum<__bf16, 128>(p, s);
}

}  // namespace h2o
