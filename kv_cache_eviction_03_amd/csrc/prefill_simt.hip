// Prefill kernels for fp32 storage (vector ALU, no MFMA).
//
// Same two outputs as the MFMA kernels: causal attention with each row's
// log-sum-exp (H2O blog, ttsmallhot.github.io, §2.1.1), then the softmax
// column sums c_j = sum_{i >= j} P_ij ("H2O Heavy-Hitter Oracle 分析", §3.1)
// re-formed from the stored log-sum-exp in a fixed order. The column sums are
// written as a single partial row per unit (partial-row block = T).
//
// Layout: 16 rows per workgroup, 16 lanes per row, each lane owning D/16
// consecutive dims; a logit is a 16-lane butterfly sum, so both kernels form
// bit-identical logits for the same (query, key) pair.
#include "h2o_device.hpp"
#include "h2o_kernels.hpp"

namespace h2o {
namespace {

constexpr int kThreads = 256;
constexpr int RB = 16;  // rows per workgroup

template <int D>
__device__ __forceinline__ void load_part(const float* row, int part, float (&x)[D / 16]) {
#pragma unroll
  for (int c = 0; c < D / 64; ++c) {
    float f[4];
    load_f32(row + part * (D / 16) + 4 * c, f);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * c + i] = f[i];
  }
}

template <int D>
__device__ __forceinline__ float dot16(const float (&a)[D / 16], const float (&b)[D / 16]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) s = fmaf(a[i], b[i], s);
  return group_sum<16>(s);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(PrefillParams p) {
  constexpr int DP = D / 16;
  const int Ts = p.T;
  const int nqb = (Ts + RB - 1) / RB;
  const UnitBlock ub = xcd_unit_block(blockIdx.x, p.units, nqb);
  if (ub.unit >= p.units) return;
  const int unit = ub.unit;
  const int T_ = unit_bound(p.lens, unit, p.heads, Ts, Ts);   // this unit's prompt length
  const int qb = nqb - 1 - ub.r;
  if (qb * RB >= T_) return;                   // past this prompt
  const int qi = threadIdx.x / 16, part = threadIdx.x % 16;
  const int q = qb * RB + qi;
  const int qc = q < T_ ? q : T_ - 1;   // rows past T compute a copy, never stored
  const size_t base = (size_t)unit * Ts * D;
  const float* Q = static_cast<const float*>(p.q) + base;
  const float* K = static_cast<const float*>(p.k) + base;
  const float* V = static_cast<const float*>(p.v) + base;

  float qv[DP];
  load_part<D>(Q + (size_t)qc * D, part, qv);
  // The running sum and output are kept in fp64: over a prompt of T keys an fp32 running
  // sum drifts by up to T half-ulps, which with a thousand keys and a few dominant ones
  // reached 1.7e-5 of the output; the logits and weights stay fp32.
  double o[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) o[i] = 0.0;
  float m = -INFINITY;
  double l = 0.0;
  const int jmax = min(qb * RB + RB - 1, T_ - 1);   // uniform over the workgroup
  for (int j = 0; j <= jmax; ++j) {
    float kv[DP], vv[DP];
    load_part<D>(K + (size_t)j * D, part, kv);
    load_part<D>(V + (size_t)j * D, part, vv);
    float s = dot16<D>(qv, kv) * p.qk_scale;
    if (j > qc) s = -INFINITY;
    const float mn = fmaxf(m, s);
    const float alpha = fast_exp2(m - mn);
    const float pj = fast_exp2(s - mn);
    l = fma(l, (double)alpha, (double)pj);
#pragma unroll
    for (int i = 0; i < DP; ++i) o[i] = fma((double)pj, (double)vv[i], o[i] * (double)alpha);
    m = mn;
  }
  if (q < T_) {
    const double inv = 1.0 / l;
    float* orow = p.out + ((size_t)unit * Ts + q) * D + part * DP;
#pragma unroll
    for (int i = 0; i < DP; ++i) orow[i] = (float)(o[i] * inv);
    if (part == 0) p.lse2[(size_t)unit * Ts + q] = m + log2f((float)l);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void colsum_f32_kernel(PrefillParams p) {
  constexpr int DP = D / 16;
  const int Ts = p.T;
  const UnitBlock ub = xcd_unit_block(blockIdx.x, p.units, (Ts + RB - 1) / RB);
  if (ub.unit >= p.units) return;
  const int unit = ub.unit;
  const int T_ = unit_bound(p.lens, unit, p.heads, Ts, Ts);   // this unit's prompt length
  const int kb = ub.r;
  if (kb * RB >= T_) return;                   // past this prompt
  const int kj = kb * RB + threadIdx.x / 16, part = threadIdx.x % 16;
  const int kc = kj < T_ ? kj : T_ - 1;
  const size_t base = (size_t)unit * Ts * D;
  const float* Q = static_cast<const float*>(p.q) + base;
  const float* K = static_cast<const float*>(p.k) + base;
  const float* lse = p.lse2 + (size_t)unit * Ts;

  float kv[DP];
  load_part<D>(K + (size_t)kc * D, part, kv);
  float cs = 0.f;
  for (int i = kb * RB; i < T_; ++i) {
    float qv[DP];
    load_part<D>(Q + (size_t)i * D, part, qv);
    const float s = dot16<D>(qv, kv) * p.qk_scale;
    if (i >= kj) cs += fast_exp2(s - lse[i]);
  }
  if (part == 0 && kj < T_) p.colpart[(size_t)unit * Ts + kj] = cs;
}

}  // namespace

hipError_t launch_prefill_attn_f32(int D, const PrefillParams& p, hipStream_t s) {
  const int nqb = (p.T + RB - 1) / RB;
  const dim3 grid((unsigned)xcd_grid_blocks(p.units, nqb));
  if (D == 64) attn_f32_kernel<64><<<grid, dim3(kThreads), 0, s>>>(p);
  else attn_f32_kernel<128><<<grid, dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_prefill_colsum_f32(int D, const PrefillParams& p, hipStream_t s) {
  const int nb = (p.T + RB - 1) / RB;
  const dim3 grid((unsigned)xcd_grid_blocks(p.units, nb));
  if (D == 64) colsum_f32_kernel<64><<<grid, dim3(kThreads), 0, s>>>(p);
  else colsum_f32_kernel<128><<<grid, dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace h2o
