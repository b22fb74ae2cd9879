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
// bf16: P rounded to bf16 alone gives up to ~3e-3 abs error on O for N(0,1)
// data, so P is split into a bf16 high part and a bf16 residual, two MFMAs.
#include "h2o_device.hpp"
#include "h2o_kernels.hpp"

namespace h2o {
namespace {

constexpr int BM = 64;    // query rows per workgroup (16 per wave)
constexpr int BN = 64;    // keys per tile
constexpr int kThreads = 256;

template <typename T> __device__ __forceinline__ typename Vec8<T>::type ld8(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::type*>(p);
}

// Cooperative K tile load: BN rows x D into LDS rows of stride D + 8.
template <typename T, int D>
__device__ __forceinline__ void load_rows(T* tile, const T* src, int row0, int T_, int tid) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int KS = D + 8;
#pragma unroll
  for (int c = tid; c < BN * CPR; c += kThreads) {
    const int row = c / CPR, cc = c % CPR;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row0 + row < T_) v = ld16(src + (size_t)(row0 + row) * D + cc * 8);
    st16(tile + row * KS + cc * 8, v);
  }
}

// Cooperative V tile load, transposed: LDS holds V^T [D][BN + 8].
template <typename T, int D>
__device__ __forceinline__ void load_vt(T* tile, const T* src, int row0, int T_, int tid) {
  constexpr int CPR = D / 8;
  constexpr int VS = BN + 8;
  for (int c = tid; c < (BN / 4) * CPR; c += kThreads) {
    const int kg = c / CPR, dc = c % CPR;
    uint4 r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = row0 + 4 * kg + e;
      r[e] = key < T_ ? ld16(src + (size_t)key * D + dc * 8) : make_uint4(0, 0, 0, 0);
    }
    const uint32_t w[4][4] = {{r[0].x, r[0].y, r[0].z, r[0].w}, {r[1].x, r[1].y, r[1].z, r[1].w},
                              {r[2].x, r[2].y, r[2].z, r[2].w}, {r[3].x, r[3].y, r[3].z, r[3].w}};
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const int word = e8 >> 1, sh = (e8 & 1) * 16;
      uint2 o;
      o.x = ((w[0][word] >> sh) & 0xffffu) | (((w[1][word] >> sh) & 0xffffu) << 16);
      o.y = ((w[2][word] >> sh) & 0xffffu) | (((w[3][word] >> sh) & 0xffffu) << 16);
      *reinterpret_cast<uint2*>(tile + (dc * 8 + e8) * VS + 4 * kg) = o;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void prefill_attn_kernel(PrefillParams p) {
  using V8 = typename Vec8<T>::type;
  using V4 = typename Vec8<T>::half;
  constexpr bool kSplit = sizeof(T) == 2 && !__is_same(T, _Float16);
  constexpr int KS = D + 8, VS = BN + 8;
  __shared__ __attribute__((aligned(16))) T k_tile[BN * KS];
  __shared__ __attribute__((aligned(16))) T v_tile[D * VS];

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
  const int qrow = qb * BM + wave * 16 + l16;

  V8 qa[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    V8 z = {};
    qa[kk] = qrow < T_ ? ld8(Q + (size_t)qrow * D + kk * 32 + 8 * g) : z;
  }

  f32x4 o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  for (int kt = 0; kt <= qb; ++kt) {
    const int key0 = kt * BN;
    load_rows<T, D>(k_tile, K, key0, T_, tid);
    load_vt<T, D>(v_tile, V, key0, T_, tid);
    __syncthreads();

    f32x4 s[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 16; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        s[kb] = mfma16x16x32(ld8(k_tile + (kb * 16 + l16) * KS + kk * 32 + 8 * g), qa[kk], s[kb]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + kb * 16 + 4 * g + i;
        float x = s[kb][i] * p.qk_scale;
        if (key > qrow || key >= T_) x = -INFINITY;
        s[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mnew = fmaxf(m, mx);
    const float alpha = exp2f(m - mnew);
    m = mnew;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = exp2f(s[kb][i] - mnew);
        s[kb][i] = x;
        ps += x;
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db] *= alpha;

    V8 pb[BN / 32], pl[BN / 32];
#pragma unroll
    for (int ks = 0; ks < BN / 32; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[ks][i] = (T)s[2 * ks][i];
        pb[ks][4 + i] = (T)s[2 * ks + 1][i];
        if constexpr (kSplit) {
          pl[ks][i] = (T)(s[2 * ks][i] - (float)pb[ks][i]);
          pl[ks][4 + i] = (T)(s[2 * ks + 1][i] - (float)pb[ks][4 + i]);
        }
      }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int ks = 0; ks < BN / 32; ++ks) {
        const T* vr = v_tile + (db * 16 + l16) * VS + ks * 32 + 4 * g;
        const V4 lo = *reinterpret_cast<const V4*>(vr);
        const V4 hi = *reinterpret_cast<const V4*>(vr + 16);
        const V8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = mfma16x16x32(a, pb[ks], o[db]);
        if constexpr (kSplit) o[db] = mfma16x16x32(a, pl[ks], o[db]);
      }
    __syncthreads();
  }

  float lt = lsum + __shfl_xor(lsum, 16, kWave);
  lt = lt + __shfl_xor(lt, 32, kWave);
  if (qrow < T_) {
    const float inv = 1.0f / lt;
    float* orow = p.out + ((size_t)unit * T_ + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const f32x4 v = o[db] * inv;
      *reinterpret_cast<f32x4*>(orow + db * 16 + 4 * g) = v;
    }
    if (g == 0) p.lse2[(size_t)unit * T_ + qrow] = m + log2f(lt);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void prefill_colsum_kernel(PrefillParams p) {
  using V8 = typename Vec8<T>::type;
  constexpr int KS = D + 8;
  __shared__ __attribute__((aligned(16))) T q_tile[BM * KS];
  __shared__ float lse_tile[BM];

  const int T_ = p.T;
  const int nb = (T_ + BN - 1) / BN;
  const int kb = blockIdx.x / p.units;         // early keys (most rows) first
  const int unit = blockIdx.x - kb * p.units;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)unit * T_ * D;
  const T* Q = static_cast<const T*>(p.q) + base;
  const T* K = static_cast<const T*>(p.k) + base;
  const float* lse = p.lse2 + (size_t)unit * T_;
  const int key0 = kb * BN + wave * 16;        // this wave's 16 keys

  V8 ka[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    V8 z = {};
    ka[kk] = key0 + l16 < T_ ? ld8(K + (size_t)(key0 + l16) * D + kk * 32 + 8 * g) : z;
  }
  float cs[4] = {0.f, 0.f, 0.f, 0.f};

  for (int qt = kb; qt < nb; ++qt) {
    const int q0 = qt * BM;
    load_rows<T, D>(q_tile, Q, q0, T_, tid);
    if (tid < BM) lse_tile[tid] = q0 + tid < T_ ? lse[q0 + tid] : 0.f;
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < BM / 16; ++qb) {
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        s = mfma16x16x32(ka[kk], ld8(q_tile + (qb * 16 + l16) * KS + kk * 32 + 8 * g), s);
      const int q = q0 + qb * 16 + l16;
      const float l2 = lse_tile[qb * 16 + l16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 4 * g + i;
        if (q < T_ && q >= key) cs[i] += exp2f(s[i] * p.qk_scale - l2);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) cs[i] = group_sum<16>(cs[i]);
  if (l16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + 4 * g + i;
      if (key < T_) p.colsum[(size_t)unit * T_ + key] = cs[i];
    }
  }
}

template <typename T, int D>
hipError_t attn(const PrefillParams& p, hipStream_t s) {
  const int nqb = (p.T + BM - 1) / BM;
  prefill_attn_kernel<T, D><<<dim3((unsigned)(nqb * p.units)), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}
template <typename T, int D>
hipError_t colsum(const PrefillParams& p, hipStream_t s) {
  const int nb = (p.T + BN - 1) / BN;
  prefill_colsum_kernel<T, D><<<dim3((unsigned)(nb * p.units)), dim3(kThreads), 0, s>>>(p);
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
