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
// feeds RB MFMAs. Tiles are copied straight from global memory into
// double-buffered LDS (buffer_load ... lds), so the next tile's loads are in
// flight while the current one is consumed and one barrier per tile suffices.
// Tile rows are unpadded with XOR-swizzled 16-byte chunks; the V operand of the
// PV product is fetched with gfx950's transposing LDS read, so V needs no
// register transpose.
//
// bf16: P rounded to bf16 alone gives up to ~3e-3 abs error on O for N(0,1)
// data, so P is split into a bf16 high part and a bf16 residual, two MFMAs.
#include "h2o_device.hpp"
#include "h2o_kernels.hpp"

#include <type_traits>

namespace h2o {
namespace {

constexpr int BN = 64;    // queries per column-sum tile
constexpr float kLazy = 8.f;  // log2-domain slack before the running max is moved
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <typename T> __device__ __forceinline__ typename Vec8<T>::type ld8(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::type*>(p);
}

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

// ---------------------------------------------------------------------------------
// Direct-to-LDS tiles. buffer_load_dwordx4 ... lds (gfx950) writes each lane's 16 bytes
// to LDS at M0 + 16 * lane, so one wave instruction fills 1 KB of LDS with no register
// staging. Tile rows are unpadded; instead the 16-byte chunks of a row are XOR-swizzled
// so that the MFMA operand reads stay conflict-free. Rows at or past T fall outside the
// buffer descriptor's range and read as zero.
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 untyped buffer access (32-bit data format)
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int BNA = 32;   // keys per attention tile (one PV MFMA deep)

template <typename T, int D, int ROWS> struct DTile {
  static constexpr int ROW = D * (int)sizeof(T);             // bytes per row
  static constexpr int CPR = ROW / 16;                        // 16-byte chunks per row
  static constexpr int BYTES = ROWS * ROW;                    // bytes per tile
  static constexpr int NI = BYTES / (kThreads * 16);          // loads per thread per tile
  static_assert(NI >= 1 && BYTES % (kThreads * 16) == 0, "tile must be whole 16-byte loads per thread");
};
// K tiles feed the A operand of S^T = K Q^T: 16 lanes read one chunk of 16 consecutive
// rows, so chunk c of row r is stored at c ^ (r % CPR).
template <int CPR> __device__ __forceinline__ int swz_k(int row, int c) { return c ^ (row & (CPR - 1)); }
// V tiles feed the transposing 8-byte reads: 16 lanes read 32 bytes of 4 consecutive
// rows, so chunk c of row r is stored at c ^ 2 * (r % (CPR / 2)).
template <int CPR> __device__ __forceinline__ int swz_v(int row, int c) { return c ^ ((row & (CPR / 2 - 1)) << 1); }

template <typename T, int D, int ROWS, bool V_LAYOUT>
struct TileDma {
  using G = DTile<T, D, ROWS>;
  uint32_t voff[G::NI];   // byte offset in the source rows of each of this lane's loads
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
      const int L = (wave * G::NI + i) * kWave + lane;        // LDS chunk this lane fills
      const int row = L / G::CPR, c = L % G::CPR;
      const int src_c = V_LAYOUT ? swz_v<G::CPR>(row, c) : swz_k<G::CPR>(row, c);
      voff[i] = (uint32_t)(row * G::ROW + src_c * 16);
    }
  }
  // Rows [row0, row0 + ROWS) of a [T][D] matrix into `tile`.
  __device__ __forceinline__ void issue(const T* src, int row0, int T_, char* tile, int wave) const {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(src + (size_t)row0 * D), (short)0, (T_ - row0) * G::ROW, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < G::NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_ptr)(tile + (wave * G::NI + i) * (kWave * 16)), 16, voff[i], 0, 0, 0);
  }
};

// Max of a value over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes that hold one query
// row of an S^T accumulator), with the gfx950 lane-swap instructions.
__device__ __forceinline__ float quad_row_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Causal attention of query block qb (BM rows) of one unit over all keys up to the block's
// last row, software-pipelined over 32-key tiles. The wave's logits of tile kt come from
// the previous step; after the row maxima (and the rare output rescale, in its own
// branch) one straight stretch of code holds the QK product of tile kt + 1, the
// exponentials, sums and conversions of tile kt, then its PV product, so the matrix unit
// runs while the vector ALU forms P. K and V tiles are double-buffered in LDS with K one
// tile ahead of V: in step kt the wave reads K(kt + 1) and V(kt), then starts the loads
// of K(kt + 2) and V(kt + 1) into the buffers the previous barrier freed.
template <typename T, int D, int RB>
__device__ __forceinline__ void attn_block(const PrefillParams& p, int unit, int qb,
                                                char* kbuf, char* vbuf) {
  using V8 = typename Vec8<T>::type;
  using V4 = typename Vec8<T>::half;
  using G = DTile<T, D, BNA>;
  constexpr bool kSplit = !__is_same(T, _Float16);
  constexpr int BM = kWaves * 16 * RB;
  typedef f32x4 STile[RB][BNA / 16];
  typedef V8 KOps[D / 32][BNA / 16];
  typedef V8 VOps[BNA / 32][D / 16];
  const int T_ = p.T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)unit * T_ * D;
  const T* Q = static_cast<const T*>(p.q) + base;
  const T* K = static_cast<const T*>(p.k) + base;
  const T* V = static_cast<const T*>(p.v) + base;
  const int row0 = qb * BM + wave * 16 * RB;    // this wave's first row

  TileDma<T, D, BNA, false> kdma;
  TileDma<T, D, BNA, true> vdma;
  kdma.init(wave, lane);
  vdma.init(wave, lane);
  const int kend = min(T_, (qb + 1) * BM);
  const int nkt = (kend + BNA - 1) / BNA;
  kdma.issue(K, 0, T_, kbuf, wave);
  vdma.issue(V, 0, T_, vbuf, wave);
  if (nkt > 1) kdma.issue(K, BNA, T_, kbuf + G::BYTES, wave);

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
  // This wave computes tiles 0..wlast. Its rows start on a tile boundary, so every tile
  // before wlast lies wholly below the diagonal and below T: only tile wlast is masked.
  static_assert((16 * RB) % BNA == 0, "a wave's rows must start on a key-tile boundary");
  const int wlast = (min(row0 + 16 * RB, kend) - 1) / BNA;

  auto read_k = [&](int kt, KOps& ak) {
    const char* t = kbuf + (kt & 1) * G::BYTES;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
      for (int kb = 0; kb < BNA / 16; ++kb) {
        const int row = kb * 16 + l16;
        ak[kk][kb] = *reinterpret_cast<const V8*>(t + row * G::ROW + swz_k<G::CPR>(row, kk * 4 + g) * 16);
      }
  };
  auto read_v = [&](int kt, VOps& av) {
    const char* t = vbuf + (kt & 1) * G::BYTES;
#pragma unroll
    for (int ks = 0; ks < BNA / 32; ++ks)
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        // keys ks*32 + 4g + r (then + 16) of dims db*16 + 4q .. + 3, lane 4r + q of each
        // 16-lane group; both rows share one swizzle (they differ by 16)
        const int row = ks * 32 + 4 * g + (l16 >> 2), q = l16 & 3;
        const char* vr = t + row * G::ROW + swz_v<G::CPR>(row, 2 * db + (q >> 1)) * 16 + (q & 1) * 8;
        const V4 lo = TrRead<T>::read(reinterpret_cast<const T*>(vr));
        const V4 hi = TrRead<T>::read(reinterpret_cast<const T*>(vr + 16 * G::ROW));
        av[ks][db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  };
  auto qk = [&](const KOps& ak, STile& s) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < BNA / 16; ++kb) s[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)         // consecutive MFMAs use different accumulators
#pragma unroll
      for (int kb = 0; kb < BNA / 16; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb][kb] = mfma16x16x32(ak[kk][kb], qa[rb][kk], s[rb][kb]);
  };
  // Start the loads of K(kt + 2) and V(kt + 1).
  auto loads = [&](int kt) {
    if (kt + 2 < nkt) kdma.issue(K, (kt + 2) * BNA, T_, kbuf + (kt & 1) * G::BYTES, wave);
    if (kt + 1 < nkt) vdma.issue(V, (kt + 1) * BNA, T_, vbuf + ((kt + 1) & 1) * G::BYTES, wave);
  };

  // Tile kt: softmax of s (its logits), PV; with NEXT the QK product of tile kt + 1 into sn.
  auto tile = [&](auto mask_c, auto next_c, int kt, STile& s, STile& sn) {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    KOps ak;
    VOps av;
    if constexpr (NEXT) read_k(kt + 1, ak);
    read_v(kt, av);
    loads(kt);
    __builtin_amdgcn_sched_barrier(0);          // reads and loads go out before the math
    const int key0 = kt * BNA;
    constexpr int NE = BNA / 16 * 4;            // logits per lane per row block
    float mnew[RB];
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float e[NE];
      if constexpr (MASK) {
        const int qrow = row0 + rb * 16 + l16;
#pragma unroll
        for (int kb = 0; kb < BNA / 16; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = key0 + kb * 16 + 4 * g + i;
            if (key > qrow || key >= T_) s[rb][kb][i] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < BNA / 16; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) e[kb * 4 + i] = s[rb][kb][i];
#pragma unroll
      for (int w = NE / 2; w >= 1; w /= 2)
#pragma unroll
        for (int j = 0; j < w; ++j) e[j] = fmaxf(e[j], e[j + w]);
      const float mt = quad_row_max(e[0]) * p.qk_scale;
      const bool gr = mt > m[rb] + kLazy;       // the running max moves only by > kLazy
      mnew[rb] = gr ? mt : m[rb];
      grow |= gr;
    }
    if (__any(grow)) {                          // rare: rescale what was accumulated so far
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float alpha = fast_exp2(m[rb] - mnew[rb]);
        m[rb] = mnew[rb];
        ls[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) o[rb][db] *= alpha;
      }
    }
    // One straight stretch from here to the barrier: the next tile's QK MFMAs, this
    // tile's exponentials and conversions, then its PV MFMAs.
    if constexpr (NEXT) qk(ak, sn);
    V8 pb[RB][BNA / 32], pl[RB][BNA / 32];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float nm = -m[rb];
      float e[NE];
#pragma unroll
      for (int kb = 0; kb < BNA / 16; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = fast_exp2(fmaf(s[rb][kb][i], p.qk_scale, nm));
          s[rb][kb][i] = x;
          e[kb * 4 + i] = x;
        }
#pragma unroll
      for (int w = NE / 2; w >= 1; w /= 2)
#pragma unroll
        for (int j = 0; j < w; ++j) e[j] += e[j + w];
      ls[rb] += e[0];
#pragma unroll
      for (int ks = 0; ks < BNA / 32; ++ks)
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
    for (int ks = 0; ks < BNA / 32; ++ks)
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          o[rb][db] = mfma16x16x32(av[ks][db], pb[rb][ks], o[rb][db]);
          if constexpr (kSplit) o[rb][db] = mfma16x16x32(av[ks][db], pl[rb][ks], o[rb][db]);
        }
    __builtin_amdgcn_sched_barrier(0);          // the math stays ahead of the barrier
    __syncthreads();                            // K(kt + 2), V(kt + 1) landed; old buffers free
  };
  using Yes = std::true_type;
  using No = std::false_type;
  // Tile kt < wlast: unmasked, and the next tile is this wave's too.
  auto mid = [&](int kt, STile& s, STile& sn) { tile(No{}, Yes{}, kt, s, sn); };

  STile s0, s1;
  __syncthreads();                              // K(0), V(0), K(1) landed
  {
    KOps ak;
    read_k(0, ak);
    qk(ak, s0);
  }
  __syncthreads();                              // K(0) read by every wave: tile 0 reloads its buffer
  int kt = 0;
  for (; kt + 1 < wlast; kt += 2) {
    mid(kt, s0, s1);
    mid(kt + 1, s1, s0);
  }
  if (kt < wlast) {
    mid(kt, s0, s1);
    tile(Yes{}, No{}, wlast, s1, s0);           // the wave's last tile reaches the diagonal
  } else {
    tile(Yes{}, No{}, wlast, s0, s1);
  }
  for (kt = wlast + 1; kt < nkt; ++kt) {        // tiles past this wave's rows: loads only
    loads(kt);
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

// Workgroups are numbered XCD-grouped (see xcd_grid_blocks), so the query blocks of a
// unit run side by side on one XCD and read its K/V through that XCD's L2.
// Register budget: two waves per SIMD (256 VGPRs), so waves of two workgroups overlap.
template <typename T, int D, int RB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_attn_kernel(PrefillParams p) {
  constexpr int BM = kWaves * 16 * RB;
  __shared__ __attribute__((aligned(1024))) char kbuf[2 * DTile<T, D, BNA>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf[2 * DTile<T, D, BNA>::BYTES];
  const int nqb = (p.T + BM - 1) / BM;
  const UnitBlock ub = xcd_unit_block(blockIdx.x, p.units, nqb);
  if (ub.unit >= p.units) return;
  attn_block<T, D, RB>(p, ub.unit, nqb - 1 - ub.r, kbuf, vbuf);  // longest first
}

// Column sums of key block kb (BK keys) of one unit over all query rows at or after it.
// The wave's keys stay in registers as the A operand; 64-query tiles of Q stream through
// double-buffered LDS (loaded straight to LDS, one barrier per tile) and each lane keeps
// the log-sum-exps of its four queries one tile ahead in registers.
template <typename T, int D, int RB>
__device__ __forceinline__ void colsum_block(const PrefillParams& p, int unit, int kb, char* qbuf) {
  using V8 = typename Vec8<T>::type;
  using G = DTile<T, D, BN>;
  constexpr int BK = kWaves * 16 * RB;          // keys per workgroup
  constexpr int QB = BN / 16;                   // 16-query blocks per tile
  const int T_ = p.T;
  const int nq = (T_ + BN - 1) / BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)unit * T_ * D;
  const T* Q = static_cast<const T*>(p.q) + base;
  const T* K = static_cast<const T*>(p.k) + base;
  const float* lse = p.lse2 + (size_t)unit * T_;
  const int key0 = kb * BK + wave * 16 * RB;    // this wave's first key
  const int qt0 = (kb * BK) / BN;

  TileDma<T, D, BN, false> qdma;
  qdma.init(wave, lane);
  qdma.issue(Q, qt0 * BN, T_, qbuf, wave);
  auto load_lse = [&](int q0, float (&l)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)             // rows past T only meet masked tiles
      l[qb] = lse[min(q0 + qb * 16 + l16, T_ - 1)];
  };
  float lcur[QB], lnext[QB];
  load_lse(qt0 * BN, lcur);

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
  __syncthreads();                              // first tile landed

  for (int qt = qt0; qt < nq; ++qt) {
    const int q0 = qt * BN;
    const char* qt_lds = qbuf + ((qt - qt0) & 1) * G::BYTES;
    // Every operand of the tile is read into registers before the next tile's loads are
    // issued: the compiler cannot tell which buffer an in-flight LDS load writes, and
    // would otherwise wait for it before these reads.
    V8 b[D / 32][QB];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = qb * 16 + l16;
        b[kk][qb] = *reinterpret_cast<const V8*>(qt_lds + row * G::ROW + swz_k<G::CPR>(row, kk * 4 + g) * 16);
      }
    if (qt + 1 < nq) {                          // its buffer was freed by the last barrier
      load_lse(q0 + BN, lnext);                 // first: waiting for these leaves the tile loads in flight
      qdma.issue(Q, q0 + BN, T_, qbuf + ((qt - qt0 + 1) & 1) * G::BYTES, wave);
    }
    __builtin_amdgcn_sched_barrier(0);          // reads and loads go out before the math
    // Tile math; MASK for the tiles that reach the diagonal or run past T (a separate
    // instantiation, so the unmasked tiles carry no selects).
    auto math = [&](auto mask_c) {
      constexpr bool MASK = decltype(mask_c)::value;
      f32x4 s[QB][RB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[qb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // Raised issue priority while this wave feeds the matrix unit, so a wave of another
      // workgroup in its exponential stretch fills the vector ALU meanwhile.
      __builtin_amdgcn_s_setprio(3);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)       // consecutive MFMAs use different accumulators
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) s[qb][rb] = mfma16x16x32(ka[rb][kk], b[kk][qb], s[qb][rb]);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int q = q0 + qb * 16 + l16;
        const float nl = -lcur[qb];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = fast_exp2(fmaf(s[qb][rb][i], p.qk_scale, nl));
            if constexpr (MASK) {
              const int key = key0 + rb * 16 + 4 * g + i;
              cs[rb][i] += (q < T_ && q >= key) ? e : 0.f;
            } else {
              cs[rb][i] += e;
            }
          }
      }
    };
    if (q0 < key0 + 16 * RB || q0 + BN > T_) math(std::true_type{});
    else math(std::false_type{});
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lcur[qb] = lnext[qb];
    __builtin_amdgcn_sched_barrier(0);          // the math stays ahead of the barrier
    __syncthreads();                            // next tile landed; this tile's buffer free
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

// Numbered XCD-grouped like the attention blocks; early keys (the most query rows) first.
template <typename T, int D, int RB>
__global__ __launch_bounds__(kThreads) void prefill_colsum_kernel(PrefillParams p) {
  constexpr int BK = kWaves * 16 * RB;
  __shared__ __attribute__((aligned(1024))) char qbuf[2 * DTile<T, D, BN>::BYTES];
  const int nb = (p.T + BK - 1) / BK;
  const UnitBlock ub = xcd_unit_block(blockIdx.x, p.units, nb);
  if (ub.unit >= p.units) return;
  colsum_block<T, D, RB>(p, ub.unit, ub.r, qbuf);
}

// Tuning knobs (compile-time): 16-row blocks per wave. Defaults from sweeps on MI355X
// (OPT-30B-shaped prompt, T = 2048).
#ifndef H2O_ATTN_RB
#define H2O_ATTN_RB 2
#endif
#ifndef H2O_COLSUM_RB
#define H2O_COLSUM_RB 2
#endif

template <typename T, int D>
hipError_t attn(const PrefillParams& p, hipStream_t s) {
  constexpr int BM = kWaves * 16 * H2O_ATTN_RB;
  const int nqb = (p.T + BM - 1) / BM;
  prefill_attn_kernel<T, D, H2O_ATTN_RB>
      <<<dim3((unsigned)xcd_grid_blocks(p.units, nqb)), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}
template <typename T, int D>
hipError_t colsum(const PrefillParams& p, hipStream_t s) {
  constexpr int BK = kWaves * 16 * H2O_COLSUM_RB;
  const int nb = (p.T + BK - 1) / BK;
  prefill_colsum_kernel<T, D, H2O_COLSUM_RB>
      <<<dim3((unsigned)xcd_grid_blocks(p.units, nb)), dim3(kThreads), 0, s>>>(p);
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
