// Prefill kernel for fp16 / bf16 storage on gfx950 MFMA.
//
// prefill_attn: causal attention over the prompt, O = softmax(Q K^T / sqrt(d)) V
//   (the scaled row softmax of the H2O blog, ttsmallhot.github.io, §2.1.1), and
//   the column sums c_j = sum_{i >= j} P_ij, the cumulative attention of each
//   prompt token ("H2O Heavy-Hitter Oracle 分析", §3.1). A row's softmax is
//   only final once the whole row is seen, so each workgroup (one block of
//   query rows) makes two passes: the first finds every row's log-sum-exp, the
//   second forms the final P, accumulates O and sums P over the block's rows
//   into one partial column-sum row. The seed kernel adds the partial rows in
//   a fixed order (no float atomics, bit-reproducible).
//
// S^T = K Q^T is computed with v_mfma_f32_16x16x32_{f16,bf16}: lane l then
// holds the logits of query l%16 against keys 4*(l/16)+i of each 16-key block,
// so a query's softmax statistics live in the four lanes l%16 + 16*g. The PV
// product is computed as O^T = V^T P^T: P leaves the S^T accumulators directly
// as the B operand (no LDS round trip), and the output accumulators again
// belong to query l%16.
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

constexpr int BNA = 32;   // keys per pass-2 attention tile (one PV MFMA deep)
constexpr int BN1 = 64;   // keys per pass-1 (statistics) tile
// Pass 1 keeps its reference max until a lane's tile sum exceeds this (2^8: some logit of
// the tile lies more than ~4 above the reference in the log2 domain).
constexpr float kLazySum = 256.f;

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

// Causal attention of query block qb (BM rows) of one unit, with the block's share of the
// column sums, in two passes over the keys up to the block's last row.
//   Pass 1 streams the K tiles and keeps each row's running max and sum, which give the
//   row's log-sum-exp.
//   Pass 2 streams K and V again and forms the final P = 2^(s - lse) directly: O = P V
//   needs no rescaling, and P summed over the block's rows gives one partial column-sum
//   row (a DPP reduction over a wave's 16 query lanes, then the four waves through LDS).
// Both passes are software-pipelined over 32-key tiles: the QK product of tile kt + 1 is
// issued before tile kt's exponentials, so the matrix unit runs while the vector ALU
// forms P. Tiles are double-buffered in LDS; in pass 2 K runs one tile ahead of V: in
// step kt the wave reads K(kt + 1) and V(kt), then starts the loads of K(kt + 2) and
// V(kt + 1) into the buffers the previous barrier freed.
template <typename T, int D, int RB>
__device__ __forceinline__ void attn_block(const PrefillParams& p, int unit, int qb, char* lds,
                                           float (*cbuf)[kWaves][BNA]) {
  using V8 = typename Vec8<T>::type;
  using V4 = typename Vec8<T>::half;
  using G = DTile<T, D, BNA>;
  using G1 = DTile<T, D, BN1>;
  constexpr bool kSplit = !__is_same(T, _Float16);
  constexpr int BM = kWaves * 16 * RB;
  static_assert(BM == kPrefillPartRows, "one partial column-sum row per query block");
  static_assert(BNA == 32, "the column reduction covers two 16-key blocks");
  typedef f32x4 STile[RB][BNA / 16];
  typedef V8 KOps[D / 32][BNA / 16];
  typedef V8 VOps[BNA / 32][D / 16];
  const int Ts = p.T;                           // rows stored per unit
  const int T_ = unit_bound(p.lens, unit, p.heads, Ts, Ts);   // this unit's prompt length
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = (size_t)unit * Ts * D;
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
  // Wave w computes tiles 0..wlast(w). Its rows start on a tile boundary, so every tile
  // before wlast lies wholly below the diagonal and below T: only tile wlast is masked.
  static_assert((16 * RB) % BNA == 0, "a wave's rows must start on a key-tile boundary");
  auto wlast_of = [&](int w) { return (min(qb * BM + (w + 1) * 16 * RB, kend) - 1) / BNA; };
  const int wlast = wlast_of(wave);

  auto read_k = [&](int kt, KOps& ak) {
    const char* t = lds + (kt & 1) * G::BYTES;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
      for (int kb = 0; kb < BNA / 16; ++kb) {
        const int row = kb * 16 + l16;
        ak[kk][kb] = *reinterpret_cast<const V8*>(t + row * G::ROW + swz_k<G::CPR>(row, kk * 4 + g) * 16);
      }
  };
  // LDS stretch: pass 1 double-buffers its 64-key K tiles in [0, 2 G1::BYTES). In pass 2 K
  // tile kt sits at (kt & 1) * G::BYTES (K(0), K(1) are pass 1's last tile), and V tile kt
  // at 2 G1::BYTES for even kt (a buffer pass 1 never touches, so V(0) loads during pass 1)
  // and at 2 G1::BYTES - G::BYTES for odd kt.
  auto vtile = [&](int kt) { return lds + 2 * G1::BYTES - (kt & 1) * G::BYTES; };
  auto read_v = [&](int kt, VOps& av) {
    const char* t = vtile(kt);
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
  // Logits past the diagonal or past T become -inf (tile wlast only).
  auto mask = [&](int kt, STile& s) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int qrow = row0 + rb * 16 + l16;
#pragma unroll
      for (int kb = 0; kb < BNA / 16; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kt * BNA + kb * 16 + 4 * g + i;
          if (key > qrow || key >= T_) s[rb][kb][i] = -INFINITY;
        }
    }
  };
  using Yes = std::true_type;
  using No = std::false_type;

  // ---------------------------------------------------------------- pass 1 --
  // 64-key tiles (no output accumulators are live, so the larger logit tile fits),
  // double-buffered in the first two G1::BYTES of the LDS stretch (even tiles first).
  static_assert(G1::BYTES == 2 * G::BYTES, "a pass-1 tile holds two pass-2 tiles");
  typedef f32x4 STile1[RB][BN1 / 16];
  typedef V8 KOps1[D / 32][BN1 / 16];
  TileDma<T, D, BN1, false> k1dma;
  k1dma.init(wave, lane);
  const int nkt1 = (kend + BN1 - 1) / BN1;
  const int wlast1 = (min(row0 + 16 * RB, kend) - 1) / BN1;
  auto buf1 = [&](int kt) { return lds + (kt & 1) * G1::BYTES; };
  auto read_k1 = [&](int kt, KOps1& ak) {
    const char* t = buf1(kt);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
      for (int kb = 0; kb < BN1 / 16; ++kb) {
        const int row = kb * 16 + l16;
        ak[kk][kb] = *reinterpret_cast<const V8*>(t + row * G1::ROW + swz_k<G1::CPR>(row, kk * 4 + g) * 16);
      }
  };
  auto qk1 = [&](const KOps1& ak, STile1& s) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < BN1 / 16; ++kb) s[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
      for (int kb = 0; kb < BN1 / 16; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb][kb] = mfma16x16x32(ak[kk][kb], qa[rb][kk], s[rb][kb]);
  };
  float m[RB], ls[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    ls[rb] = 0.f;
  }
  // Pass 1 walks the tiles from the last down to tile 0, so that tile 0 (keys 0..63, at
  // the start of the stretch) is in LDS at the end: it holds pass 2's first two K tiles in their layout. Step t
  // issues tile t - 2 into the buffer of tile t (read by every wave in step t + 1), reads
  // tile t - 1 and, with NEXT, starts its QK product into sn; with COMP it takes tile t's
  // statistics from s (MASK: tile wlast1, the wave's first, which reaches the diagonal;
  // the tiles after it lie wholly below the diagonal and below T, since 64 * wlast1 <= row0).
  auto step1 = [&](auto comp_c, auto mask_c, auto next_c, int t, STile1& s, STile1& sn) {
    constexpr bool COMP = decltype(comp_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    constexpr int NE1 = BN1 / 16 * 4;
    KOps1 ak;
    if constexpr (NEXT) read_k1(t - 1, ak);
    if (t >= 2) k1dma.issue(K, (t - 2) * BN1, T_, buf1(t - 2), wave);
    __builtin_amdgcn_sched_barrier(0);          // reads and loads go out before the math
    if constexpr (COMP && MASK) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int qrow = row0 + rb * 16 + l16;
#pragma unroll
        for (int kb = 0; kb < BN1 / 16; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t * BN1 + kb * 16 + 4 * g + i;
            if (key > qrow || key >= T_) s[rb][kb][i] = -INFINITY;
          }
      }
    }
    if constexpr (NEXT) {
      __builtin_amdgcn_s_setprio(3);            // feed the matrix unit first
      qk1(ak, sn);
      __builtin_amdgcn_s_setprio(0);
    }
    // Row statistics. The reference m[rb] is the exact row max only after the wave's first
    // tile (MASK): later tiles are exponentiated against the current m directly, and only
    // if a lane's sum shows a logit more than about kLazy above m (rare) is the tile max
    // taken and the running sum rescaled to it. m + log2(l) is exact for any reference
    // that keeps the terms in range.
    auto full = [&](int rb, float& tsum) {
      float e[NE1];
#pragma unroll
      for (int kb = 0; kb < BN1 / 16; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) e[kb * 4 + i] = s[rb][kb][i];
#pragma unroll
      for (int w = NE1 / 2; w >= 1; w /= 2)
#pragma unroll
        for (int j = 0; j < w; ++j) e[j] = fmaxf(e[j], e[j + w]);
      // Every row has an unmasked key in each tile it computes; mref guards -inf anyway.
      const float mn = fmaxf(m[rb], quad_row_max(e[0]) * p.qk_scale);
      const float mref = mn == -INFINITY ? 0.f : mn;
      ls[rb] *= fast_exp2(m[rb] - mref);
      m[rb] = mn;
#pragma unroll
      for (int kb = 0; kb < BN1 / 16; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) e[kb * 4 + i] = fast_exp2(fmaf(s[rb][kb][i], p.qk_scale, -mref));
#pragma unroll
      for (int w = NE1 / 2; w >= 1; w /= 2)
#pragma unroll
        for (int j = 0; j < w; ++j) e[j] += e[j + w];
      tsum = e[0];
    };
    if constexpr (COMP && MASK) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float tsum;
        full(rb, tsum);
        ls[rb] += tsum;
      }
    } else if constexpr (COMP) {
      float tsum[RB];
      bool grow = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float e[NE1];
        const float nm = -m[rb];
#pragma unroll
        for (int kb = 0; kb < BN1 / 16; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) e[kb * 4 + i] = fast_exp2(fmaf(s[rb][kb][i], p.qk_scale, nm));
#pragma unroll
        for (int w = NE1 / 2; w >= 1; w /= 2)
#pragma unroll
          for (int j = 0; j < w; ++j) e[j] += e[j + w];
        tsum[rb] = e[0];
        grow |= !(e[0] <= kLazySum);            // also catches inf / NaN
      }
      if (__any(grow)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) full(rb, tsum[rb]);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) ls[rb] += tsum[rb];
    }
    __builtin_amdgcn_sched_barrier(0);          // the math stays ahead of the barrier
    __syncthreads();                            // tile t - 2 landed; tile t - 1 read by all
  };

  k1dma.issue(K, (nkt1 - 1) * BN1, T_, buf1(nkt1 - 1), wave);
  if (nkt1 > 1) k1dma.issue(K, (nkt1 - 2) * BN1, T_, buf1(nkt1 - 2), wave);
  vdma.issue(V, 0, T_, vtile(0), wave);        // pass 2's first V tile, in a buffer of its own
  {
    STile1 s0, s1;
    int t = nkt1 - 1;
    __syncthreads();                            // tiles t and t - 1 (and V(0)) landed
    if (wlast1 == t) {
      KOps1 ak;
      read_k1(t, ak);
      qk1(ak, s0);
    }
    __syncthreads();                            // tile t read by every wave
    if (wlast1 < t) {
      for (; t > wlast1 + 1; --t) step1(No{}, No{}, No{}, t, s1, s0);   // loads only
      step1(No{}, No{}, Yes{}, t, s1, s0);      // starts the QK product of tile wlast1
      --t;
    }
    // t == wlast1 and s0 holds its logits.
    if (t >= 1) step1(Yes{}, Yes{}, Yes{}, t, s0, s1);
    else step1(Yes{}, Yes{}, No{}, t, s0, s1);
    for (t -= 1; t >= 2; t -= 2) {
      step1(Yes{}, No{}, Yes{}, t, s1, s0);
      step1(Yes{}, No{}, Yes{}, t - 1, s0, s1);
    }
    if (t == 1) {
      step1(Yes{}, No{}, Yes{}, 1, s1, s0);
      step1(Yes{}, No{}, No{}, 0, s0, s1);
    } else if (t == 0) {
      step1(Yes{}, No{}, No{}, 0, s1, s0);
    }
  }
  // Row log-sum-exp (log2 domain); rows past T get +inf, so their P is 0 in pass 2.
  float lse[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lt = ls[rb] + __shfl_xor(ls[rb], 16, kWave);
    lt = lt + __shfl_xor(lt, 32, kWave);
    lse[rb] = row0 + rb * 16 + l16 < T_ ? m[rb] + log2f(lt) : INFINITY;
  }

  // ---------------------------------------------------------------- pass 2 --
  // K(0), K(1) (pass 1's last tile) and V(0) are already in LDS.
  f32x4 o[RB][D / 16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float* cpart = p.colpart + (size_t)unit * colpart_stride(Ts, BM) + colpart_row_offset(qb, BM);
  // Wave 0 adds the four waves' column partials of tile kt (in wave order, skipping waves
  // that did not compute it) and stores them.
  auto flush = [&](int kt) {
    float x[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) x[w] = cbuf[kt & 1][w][lane & (BNA - 1)];
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += kt <= wlast_of(w) ? x[w] : 0.f;
    const int key = kt * BNA + lane;
    if (lane < BNA && key < kend) cpart[key] = v;
  };
  // Sum of a lane's column values c[kb][i] (key kb*16 + 4g + i) over the 16 query lanes of
  // its row: each step keeps half of the values and adds the partner's copy of that half
  // (partners lane ^ 8, lane ^ 7, lane ^ 2, lane ^ 1 inside the 16-lane row). Afterwards
  // lanes l and l ^ 1 hold the sum for key kb*16 + 4g + i, kb = bit 3 of l16 and
  // i = 2 * bit 2 + bit 1.
  auto colred = [&](const float (&c)[BNA / 16][4]) {
    const bool b3 = l16 & 8, b2 = l16 & 4, b1 = l16 & 2;
    float v1[4], v2[2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v1[j] = (b3 ? c[1][j] : c[0][j]) + dpp_mov<0x128>(b3 ? c[0][j] : c[1][j]);   // row_ror:8
#pragma unroll
    for (int j = 0; j < 2; ++j)
      v2[j] = (b2 ? v1[2 + j] : v1[j]) + dpp_mov<0x141>(b2 ? v1[j] : v1[2 + j]);   // row_half_mirror
    const float v3 = (b1 ? v2[1] : v2[0]) + dpp_mov<0x4e>(b1 ? v2[0] : v2[1]);     // quad_perm [2,3,0,1]
    return v3 + dpp_mov<0xb1>(v3);                                                 // quad_perm [1,0,3,2]
  };
  const int ckey = (l16 & 8 ? 16 : 0) + 4 * g + (l16 & 4 ? 2 : 0) + (l16 & 2 ? 1 : 0);
  // Start the loads of K(kt + 2) and V(kt + 1).
  auto loads = [&](int kt) {
    if (kt + 2 < nkt) kdma.issue(K, (kt + 2) * BNA, T_, lds + (kt & 1) * G::BYTES, wave);
    if (kt + 1 < nkt) vdma.issue(V, (kt + 1) * BNA, T_, vtile(kt + 1), wave);
  };

  // Tile kt: P from its logits s, PV and the column partial; with NEXT the QK product of
  // tile kt + 1 into sn.
  auto step2 = [&](auto mask_c, auto next_c, int kt, STile& s, STile& sn) {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    if (wave == 0 && kt > 0) flush(kt - 1);
    KOps ak;
    VOps av;
    if constexpr (NEXT) read_k(kt + 1, ak);
    read_v(kt, av);
    loads(kt);
    __builtin_amdgcn_sched_barrier(0);          // reads and loads go out before the math
    if constexpr (MASK) mask(kt, s);
    // One straight stretch from here to the barrier: the next tile's QK MFMAs, this
    // tile's exponentials and conversions, then its PV MFMAs.
    if constexpr (NEXT) qk(ak, sn);
    V8 pb[RB][BNA / 32], pl[RB][BNA / 32];
    float c[BNA / 16][4];
#pragma unroll
    for (int kb = 0; kb < BNA / 16; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) c[kb][i] = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float nl = -lse[rb];
#pragma unroll
      for (int kb = 0; kb < BNA / 16; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = fast_exp2(fmaf(s[rb][kb][i], p.qk_scale, nl));
          s[rb][kb][i] = x;
          c[kb][i] += x;
        }
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
    const float cv = colred(c);
    if ((l16 & 1) == 0) cbuf[kt & 1][wave][ckey] = cv;
    __builtin_amdgcn_sched_barrier(0);          // the math stays ahead of the barrier
    __syncthreads();                            // K(kt + 2), V(kt + 1) landed; old buffers free
  };

  STile s0, s1;
  {
    KOps ak;
    read_k(0, ak);
    qk(ak, s0);
  }
  __syncthreads();                              // K(0) read by every wave: step 0 reloads its buffer
  int kt = 0;
  for (; kt + 1 < wlast; kt += 2) {
    step2(No{}, Yes{}, kt, s0, s1);
    step2(No{}, Yes{}, kt + 1, s1, s0);
  }
  if (kt < wlast) {
    step2(No{}, Yes{}, kt, s0, s1);
    step2(Yes{}, No{}, wlast, s1, s0);          // the wave's last tile reaches the diagonal
  } else {
    step2(Yes{}, No{}, wlast, s0, s1);
  }
  for (kt = wlast + 1; kt < nkt; ++kt) {        // tiles past this wave's rows: loads only
    if (wave == 0) flush(kt - 1);
    loads(kt);
    __syncthreads();
  }
  if (wave == 0) flush(nkt - 1);

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qrow = row0 + rb * 16 + l16;
    if (qrow < T_) {
      // Plain stores: a wave writes 64 bytes of each of 16 rows per instruction, and the
      // next instruction the other half of those 128-byte lines, which L2 merges (streaming
      // stores measured 15% more HBM writes for no gain in time).
      float* orow = p.out + ((size_t)unit * Ts + qrow) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<f32x4*>(orow + db * 16 + 4 * g) = o[rb][db];
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
  __shared__ __attribute__((aligned(1024))) char lds[2 * DTile<T, D, BN1>::BYTES + DTile<T, D, BNA>::BYTES];
  __shared__ float cbuf[2][kWaves][BNA];
  const int nqb = (p.T + BM - 1) / BM;
  const UnitBlock ub = xcd_unit_block(blockIdx.x, p.units, nqb);
  if (ub.unit >= p.units) return;
  const int qb = nqb - 1 - ub.r;                // longest first
  if (qb * BM >= unit_bound(p.lens, ub.unit, p.heads, p.T, p.T)) return;   // past this prompt
  attn_block<T, D, RB>(p, ub.unit, qb, lds, cbuf);
}

// 16-row blocks per wave: BM = 4 waves x 16 x RB query rows per workgroup.
constexpr int kAttnRB = kPrefillPartRows / (kWaves * 16);

template <typename T, int D>
hipError_t attn(const PrefillParams& p, hipStream_t s) {
  constexpr int BM = kWaves * 16 * kAttnRB;
  const int nqb = (p.T + BM - 1) / BM;
  prefill_attn_kernel<T, D, kAttnRB>
      <<<dim3((unsigned)xcd_grid_blocks(p.units, nqb)), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_attn_mfma(DType dt, int D, const PrefillParams& p, hipStream_t s) {
  if (dt == DType::F16) return D == 64 ? attn<_Float16, 64>(p, s) : attn<_Float16, 128>(p, s);
  return D == 64 ? attn<__bf16, 64>(p, s) : attn<__bf16, 128>(p, s);
}

}  // namespace h2o
