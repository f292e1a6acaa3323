// Prefill scoring on the matrix cores (bf16 / fp16 inputs, d = 64 or 128).
//
// The H2O review page (proposed method) ranks tokens by accumulated attention;
// at the prompt that is the column sum of the causal softmax,
//   c_j = sum_{i >= j} exp(scale q_i.k_j - lse_i),  lse_i = log sum_{j <= i} exp(scale q_i.k_j),
// a dense contraction (Q K^T) followed by elementwise exponentials.  Two passes:
//
//   rowstats: workgroup = (unit, 128 queries); waves hold 32 queries each as
//             MFMA B fragments in registers; 64-key tiles of K are staged in
//             LDS and read as A fragments; S^T = K Q^T per 16x16 block with
//             v_mfma_f32_16x16x32_{bf16,f16}; online maximum per query; the
//             per-tile sums are added in float64.
//   colsum:   workgroup = (unit, 128 keys); waves hold 32 keys each as A
//             fragments; 64-query tiles of Q (and their lse) are staged in LDS;
//             weights exp2(s * scale * log2e - lse2) are summed per key in
//             float32 within a tile and in float64 across tiles; after a
//             wave's first tile the row pass keeps its running offset unless
//             a weight could overflow.  No atomics:
//             each workgroup owns its columns.
//   persist:  the colsum structure over only the last `window` queries,
//             collecting for each key the bits "weight >= 1 / (i + 1)" of
//             rows i (the persistence reading of the Scissorhands page) by
//             one wave ballot per 16 x 16 block instead of summing weights.
//   attend:   rowstats plus the causal attention output o_i = sum_j p_ij v_j
//             (the optional prompt output), as O^T = V^T P^T on the matrix
//             cores: the weights a lane forms for its query are already a B
//             fragment, and the accumulator lane that receives O^T[dim][query]
//             owns that same query, so the online rescaling and the final
//             normalisation stay within the lane.  V tiles are staged
//             transposed in LDS; each weight enters as a 16-bit pair (hi, lo)
//             so the output keeps about 16 significant bits of every weight.
//
// MFMA 16x16x32 lane layout: lane l supplies row (l % 16) of A and column
// (l % 16) of B, each with 8 consecutive k values chosen by l / 16; it
// receives D[4 (l / 16) + r][l % 16], r = 0..3.  With A = keys and B =
// queries, lane l therefore holds s(query = l % 16, keys 4 (l / 16) + r).
//
// Exponents use base 2 with the factor scale * log2(e) split into a float
// pair (hi + lo) applied by two fused multiply-adds, so the only rounding of
// the argument is relative to its (small) result.  lse is exchanged in
// natural-log units as a float pair (hi, lo) whose sum is the float64 value.
#include "common.hpp"

namespace kve {
namespace {

// Register budget as resident waves per SIMD (3 keeps both kernels free of
// spills at d = 128).
#ifndef KVE_PREFILL_WAVES_PER_EU
#define KVE_PREFILL_WAVES_PER_EU 3
#endif
// The output pass keeps a D x 32 float accumulator per wave as well.
#ifndef KVE_ATTEND_WAVES_PER_EU
#define KVE_ATTEND_WAVES_PER_EU 2
#endif

constexpr int kNT = 256;
constexpr int kBlk = 128;          // queries (rowstats) / keys (colsum) per workgroup
constexpr int kTile = 64;          // keys (rowstats) / queries (colsum) per LDS tile
constexpr double kLog2e = 1.4426950408889634;
constexpr double kLn2 = 0.6931471805599453;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Mfma;
template <> struct Mfma<BF16> {
  __device__ static inline f32x4 run(const uint4& a, const uint4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};
template <> struct Mfma<F16> {
  __device__ static inline f32x4 run(const uint4& a, const uint4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  }
};

// LDS tile of kTile rows x D 16-bit elements, rows padded by 16 bytes so that
// the 16 rows read by one 16-lane group fall on distinct banks.
template <int D> struct Tile {
  static constexpr int kRowBytes = D * 2 + 16;
  static constexpr int kBytes = kTile * kRowBytes;
};

// A tile of kTile rows x D 16-bit elements moves global -> registers ->
// LDS: each thread carries kChunks 16-byte chunks, so the next tile's global
// loads are in flight while the current tile is consumed from LDS.
template <int D> struct TileRegs {
  static constexpr int CPR = D * 2 / 16;                 // 16-byte chunks per row
  static constexpr int kChunks = kTile * CPR / kNT;
  static_assert(kTile * CPR % kNT == 0, "tile chunks");
  uint4 v[kChunks];
};

// Buffer resource over rows [r0, P) of a unit's [P][D] 16-bit matrix: raw
// buffer loads check their (per-lane) offset against the byte count, so
// rows at or past P read as zero with no compare, select or 64-bit address
// arithmetic per load.  The third descriptor word is the gfx9-family raw
// buffer format (32-bit data, no swizzle).
template <int D>
__device__ inline __amdgpu_buffer_rsrc_t rows_rsrc(const char* src, int r0, int P) {
  const uint32_t bytes = r0 < P ? (uint32_t)(P - r0) * D * 2 : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + (size_t)r0 * D * 2, (short)0, (int)bytes,
                                           0x00020000);
}

// Rows at or past P read as zero.
template <int D>
__device__ inline void load_tile(TileRegs<D>& t, const char* src, int r0, int P) {
  constexpr int CPR = TileRegs<D>::CPR;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc<D>(src, r0, P);
#pragma unroll
  for (int j = 0; j < TileRegs<D>::kChunks; ++j) {
    const int i = threadIdx.x + j * kNT;
    const int r = i / CPR, c = i % CPR;
    t.v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, r * D * 2 + c * 16, 0, 0));
  }
}

template <int D>
__device__ inline void store_tile(const TileRegs<D>& t, char* lds) {
  constexpr int CPR = TileRegs<D>::CPR;
#pragma unroll
  for (int j = 0; j < TileRegs<D>::kChunks; ++j) {
    const int i = threadIdx.x + j * kNT;
    const int r = i / CPR, c = i % CPR;
    *reinterpret_cast<uint4*>(lds + r * Tile<D>::kRowBytes + c * 16) = t.v[j];
  }
}

// V tile transposed for the A operand of O^T = V^T P^T: D rows (one per head
// dimension) of kTile keys in 16 groups of 4, rows padded by 8 bytes.  The
// group index is XOR-swizzled by bits 5..6 of the row: the transposing stores
// (16 rows 8 apart per wave) then fall on distinct banks up to 2-way, and the
// fragment reads need one address per swizzle value, with the block of 16
// rows, the k-step and the half as immediate offsets.
template <int D> struct VtTile {
  static constexpr int kRowBytes = kTile * 2 + 8;
  static constexpr int kBytes = D * kRowBytes;
};

__device__ inline int vt_offset(int row, int key) {
  return row * (kTile * 2 + 8) + (((key >> 2) ^ ((row >> 5) & 3)) << 3) + ((key & 3) << 1);
}

// Global -> registers -> LDS for a V tile: thread t carries the 16-byte chunk
// t % CPR (8 head dimensions) of pairs of consecutive keys, so each LDS store
// is one 32-bit word holding the same dimension of two keys.
template <int D> struct VtRegs {
  static constexpr int CPR = D * 2 / 16;
  static constexpr int kPairs = kNT / CPR;               // key pairs per pass
  static constexpr int kPasses = kTile / 2 / kPairs;
  static_assert(kTile / 2 % kPairs == 0, "V tile pairs");
  uint4 v[kPasses][2];
};

template <int D>
__device__ inline void load_vtile(VtRegs<D>& t, const char* src, int r0, int P) {
  constexpr int CPR = VtRegs<D>::CPR;
  const int c = threadIdx.x % CPR, m = threadIdx.x / CPR;
#pragma unroll
  for (int ps = 0; ps < VtRegs<D>::kPasses; ++ps)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = r0 + 2 * (m + ps * VtRegs<D>::kPairs) + e;
      t.v[ps][e] = r < P ? ld16(src + ((size_t)r * D) * 2 + c * 16) : make_uint4(0, 0, 0, 0);
    }
}

template <int D>
__device__ inline void store_vtile(const VtRegs<D>& t, char* lds) {
  constexpr int CPR = VtRegs<D>::CPR;
  const int c = threadIdx.x % CPR, m = threadIdx.x / CPR;
#pragma unroll
  for (int ps = 0; ps < VtRegs<D>::kPasses; ++ps) {
    const int key = 2 * (m + ps * VtRegs<D>::kPairs);
    const uint32_t a[4] = {t.v[ps][0].x, t.v[ps][0].y, t.v[ps][0].z, t.v[ps][0].w};
    const uint32_t b[4] = {t.v[ps][1].x, t.v[ps][1].y, t.v[ps][1].z, t.v[ps][1].w};
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int sh = (x & 1) * 16;
      const uint32_t wd = ((a[x >> 1] >> sh) & 0xFFFFu) | (((b[x >> 1] >> sh) & 0xFFFFu) << 16);
      *reinterpret_cast<uint32_t*>(lds + vt_offset(8 * c + x, key)) = wd;
    }
  }
}

// A fragment of V^T for rows (dims) d0 + lane % 16 and the 8 keys that the
// weight fragments of k-step kp carry: 32 kp + 4 g + {0..3} and
// 32 kp + 16 + 4 g + {0..3}, g = lane / 16.
__device__ inline uint4 vt_fragment(const char* lds, int d0, int kp, int g, int c16) {
  const int row = d0 + c16;
  const uint2 x = *reinterpret_cast<const uint2*>(lds + vt_offset(row, 32 * kp + 4 * g));
  const uint2 y = *reinterpret_cast<const uint2*>(lds + vt_offset(row, 32 * kp + 16 + 4 * g));
  return make_uint4(x.x, x.y, y.x, y.y);
}

// Splits 8 float weights into 16-bit (hi, lo) halves of the input dtype,
// hi = round(w), lo = round(w - hi).
template <int DT> struct Split16;
template <> struct Split16<BF16> {
  __device__ static inline void run(const float (&w)[8], uint4& hi, uint4& lo) {
    bf16x8 h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 t = (__bf16)w[e];
      h[e] = t;
      l[e] = (__bf16)(w[e] - (float)t);
    }
    hi = __builtin_bit_cast(uint4, h);
    lo = __builtin_bit_cast(uint4, l);
  }
};
template <> struct Split16<F16> {
  __device__ static inline void run(const float (&w)[8], uint4& hi, uint4& lo) {
    f16x8 h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const _Float16 t = (_Float16)w[e];
      h[e] = t;
      l[e] = (_Float16)(w[e] - (float)t);
    }
    hi = __builtin_bit_cast(uint4, h);
    lo = __builtin_bit_cast(uint4, l);
  }
};

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// c2 = fl32(scale * log2(e)): every pass forms a weight's exponent as one
// fused multiply-add s * c2 - offset, so the weights are the exact softmax
// at the temperature c2, which differs from scale * log2(e) by at most 2^-24
// relative (9.0e-9 at d = 128, 1.3e-8 at d = 64): a weight's relative error
// from it is that times the deviation of its logit from the row's mean.
__device__ inline float make_scale2(float scale) { return (float)((double)scale * kLog2e); }

// Logit given to masked pairs: its weight exp2(x c - m) underflows to 0 and
// it never sets a maximum; x c stays finite for any positive scale.
__device__ inline float masked_logit(float c2) { return -1e30f / fmaxf(c2, 1.f); }

// ------------------------------------------------------------------ rowstats
// Diagonal and last tiles: pairs whose key follows the query or lies at or
// past P get the masked logit.  Every query of a processed tile keeps at
// least its first key (a tile starts at or before the wave's first query).
__device__ inline void rowstats_mask(f32x4 (&acc)[4][2], int k0, int q0, int P, int g, int c16, float msk) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int lim = min(q0 + nb * 16 + c16, P - 1) - k0 - 4 * g;   // largest valid mb 16 + r
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (mb * 16 + r > lim) acc[mb][nb][r] = msk;
  }
}

// Folds one 64-key tile (already in acc, edge tiles masked) into the online
// statistics of this lane's two queries: raises the offset to the tile's
// maximum where it is larger, then adds the tile's weights.
__device__ inline void rowstats_fold(const f32x4 (&acc)[4][2], float c2, float (&mc)[2], double (&l)[2]) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, acc[mb][nb][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(mc[nb], tmax * c2);
    if (mn > mc[nb]) {
      l[nb] *= (double)exp2_fast(mc[nb] - mn);
      mc[nb] = mn;
    }
    float sum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = acc[mb][nb][r];
        sum += exp2_fast(fmaf(s, c2, -mn));
      }
    l[nb] += (double)sum;
  }
}

// Interior tile after a wave's first: weights against the running offset mc,
// with no new maximum (one vector operation less per pair).  The offset only
// has to keep every weight finite; if any lane's tile sum reaches 2^100 the
// wave keeps its state unchanged and returns false, and the caller folds the
// tile with rowstats_fold, which raises the offset.
__device__ inline bool rowstats_fold_lazy(const f32x4 (&acc)[4][2], float c2, const float (&mc)[2],
                                          double (&l)[2]) {
  float sums[2];
  bool big = false;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float sum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = acc[mb][nb][r];
        sum += exp2_fast(fmaf(s, c2, -mc[nb]));
      }
    sums[nb] = sum;
    big |= !(sum < 0x1p100f);                  // also catches inf / NaN
  }
  if (__ballot(big) != 0) return false;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) l[nb] += (double)sums[nb];
  return true;
}

template <int DT, int D>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(KVE_PREFILL_WAVES_PER_EU)))
void rowstats_mfma_kernel(Shape sh, int P, UnitList ul, const void* q, const void* k, float* lse) {
  constexpr int KS = D / 32;                    // MFMA k-steps over the head dimension
  __shared__ __attribute__((aligned(16))) char Ks[2][Tile<D>::kBytes];
  const int u = ul.ids ? ul.ids[blockIdx.x] : blockIdx.x;
  const int nqb = (P + kBlk - 1) / kBlk;
  const int qb = nqb - 1 - (int)blockIdx.y;     // heaviest (last) query block first
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const size_t base = (size_t)u * P * D * 2;
  const char* qbase = (const char*)q + base;
  const char* kbase = (const char*)k + base;
  const int q0 = qb * kBlk + w * 32;            // this wave's first query
  const float c2 = make_scale2(sh.scale);
  const float msk = masked_logit(c2);

  // B fragments: the wave's 32 queries
  uint4 qf[2][KS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int qi = q0 + nb * 16 + c16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[nb][ks] = qi < P ? ld16(qbase + ((size_t)qi * D + ks * 32 + g * 8) * 2) : make_uint4(0, 0, 0, 0);
  }
  // mc: running offset = (max raw logit) * c2, per query of this lane;
  // weights are exp2(s * c2 - mc), one fused multiply-add and the exponential
  float mc[2] = {-INFINITY, -INFINITY};
  double l[2] = {0.0, 0.0};
  const int kend = min(P, qb * kBlk + kBlk);    // keys needed by the block
  TileRegs<D> nxt;
  load_tile<D>(nxt, kbase, 0, P);
  store_tile<D>(nxt, Ks[0]);
  __syncthreads();
  for (int it = 0, k0 = 0; k0 < kend; ++it, k0 += kTile) {
    const char* cur = Ks[it & 1];
    const bool more = k0 + kTile < kend;
    if (more) load_tile<D>(nxt, kbase, k0 + kTile, P);   // in flight during the compute below
    if (k0 <= q0 + 31) {                        // some key of the tile precedes a query of the wave
      f32x4 acc[4][2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 a = *reinterpret_cast<const uint4*>(cur + (mb * 16 + c16) * Tile<D>::kRowBytes + (ks * 32 + g * 8) * 2);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = Mfma<DT>::run(a, qf[nb][ks], acc[mb][nb]);
        }
      }
      if (k0 + kTile > q0 || k0 + kTile > P) {
        rowstats_mask(acc, k0, q0, P, g, c16, msk);
        rowstats_fold(acc, c2, mc, l);
      } else if (k0 == 0 || !rowstats_fold_lazy(acc, c2, mc, l)) {
        rowstats_fold(acc, c2, mc, l);
      }
    }
    if (more) store_tile<D>(nxt, Ks[(it + 1) & 1]);   // that buffer was last read before the previous barrier
    __syncthreads();
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    double lt = l[nb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int qi = q0 + nb * 16 + c16;
    if (g == 0 && qi < P) {
      const double L = ((double)mc[nb] + log2(lt)) * kLn2;  // natural-log units
      const float hi = (float)L;
      lse[((size_t)u * P + qi) * 2] = hi;
      lse[((size_t)u * P + qi) * 2 + 1] = (float)(L - (double)hi);
    }
  }
}

// ------------------------------------------------------------------ colsum
// Adds one 64-query tile's weights exp2(s * c2 - lse2) into part (this lane's
// keys; edge tiles masked).  The low word of lse2 enters as the factor
// fl = 2^-ll on the weight, taken by the accumulating fused multiply-add.
__device__ inline void colsum_fold(const f32x4 (&acc)[2], float c2, float lh, float fl,
                                   float (&part)[2][4]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s = acc[mb][r];
      const float p = exp2_fast(fmaf(s, c2, -lh));
      part[mb][r] = fmaf(p, fl, part[mb][r]);
    }
}

// Diagonal and last tiles: pairs whose query precedes the key or lies at or
// past P get the masked logit (weight 0).
__device__ inline void colsum_mask(f32x4 (&acc)[2], int i0, int nb, int j0, int P, int g, int c16, float msk) {
  const int qi = i0 + nb * 16 + c16;
  const int lim = qi < P ? qi - j0 - 4 * g : -1;   // largest valid mb 16 + r
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (mb * 16 + r > lim) acc[mb][r] = msk;
}

// colsum_fold with masks, also adding the weights of rows >= wlo into pm.
__device__ inline void mass_fold(const f32x4 (&acc)[2], int i0, int nb, int j0, int P, int wlo, int g, int c16,
                                 float c2, float lh, float fl, float (&part)[2][4], float (&pm)[2][4]) {
  const int qi = i0 + nb * 16 + c16;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s = acc[mb][r];
      const float p = exp2_fast(fmaf(s, c2, -lh)) * fl;
      const int kj = j0 + mb * 16 + g * 4 + r;
      const bool ok = qi < P && qi >= kj;
      part[mb][r] += ok ? p : 0.f;
      pm[mb][r] += (ok && qi >= wlo) ? p : 0.f;
    }
}

// Bits of one 16 x 16 block: for this lane's key (mb, r) and the 16 queries
// i0 + nb * 16 + 0..15, the history bits at ages P - 1 - query.  Every lane
// takes part in the ballots.
__device__ inline void persist_fold(const f32x4 (&acc)[2], int i0, int nb, int j0, int P, int wlo, int g,
                                    int c16, float c2, float lh, float ll, float th,
                                    uint64_t (&bits)[2][4]) {
  const int qi = i0 + nb * 16 + c16;
  const int age15 = P - 1 - (i0 + nb * 16 + 15);   // age of the block's last query
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s = acc[mb][r];
      const float x = fmaf(s, c2, -lh) - ll;
      const int kj = j0 + mb * 16 + g * 4 + r;
      const bool piv = qi < P && qi >= kj && qi >= wlo && x >= th;
      const uint64_t b = __ballot(piv);
      // lanes 16 g .. 16 g + 15 voted for this key; bit c <-> query c of the block
      const uint32_t q16 = (uint32_t)(b >> (16 * g)) & 0xFFFFu;
      const uint64_t rev = (uint64_t)(__builtin_bitreverse32(q16) >> 16);   // bit 15 - c
      if (age15 >= 64 || age15 <= -16) continue;
      bits[mb][r] |= age15 >= 0 ? rev << age15 : rev >> (-age15);
    }
}

// MODE 0: column sums; 1: persistence bits; 2: column sums plus, per key, the
// mass of the last `rows` prompt rows (into mass).
template <int DT, int D, int MODE>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(KVE_PREFILL_WAVES_PER_EU)))
void colsum_mfma_kernel(Shape sh, int P, UnitList ul, const void* q, const void* k, const float* lse,
                        double* colsum, const HeadMeta* meta, float* mass, int rows) {
  constexpr bool BITS = MODE == 1;
  constexpr int KS = D / 32;
  __shared__ __attribute__((aligned(16))) char Qs[2][Tile<D>::kBytes];
  __shared__ float Lh[2][kTile], Ll[2][kTile];  // lse in log2 units, float pair
  __shared__ float Lf[2][kTile];                // 2^-Ll
  __shared__ float Th[2][kTile];                // BITS: -log2(i + 1)
  const int u = ul.ids ? ul.ids[blockIdx.x] : blockIdx.x;
  const int kb = blockIdx.y;                    // key block 0 (the heaviest) first
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const size_t base = (size_t)u * P * D * 2;
  const char* qbase = (const char*)q + base;
  const char* kbase = (const char*)k + base;
  const int j0 = kb * kBlk + w * 32;            // this wave's first key
  const float c2 = make_scale2(sh.scale);
  const float msk = masked_logit(c2);

  uint4 kf[2][KS];                              // A fragments: the wave's 32 keys
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int kj = j0 + mb * 16 + c16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[mb][ks] = kj < P ? ld16(kbase + ((size_t)kj * D + ks * 32 + g * 8) * 2) : make_uint4(0, 0, 0, 0);
  }
  double cs[2][4], ms[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) cs[mb][r] = ms[mb][r] = 0.0;

  // lse of one query as loaded (natural-log float pair), then in log2 units
  // as a float pair; the loads for the next tile are issued before the
  // current tile is computed and converted only after it
  auto lse_load = [&](int i, float& a, float& b) {
    const int qi = min(i, P - 1);
    a = lse[((size_t)u * P + qi) * 2];
    b = lse[((size_t)u * P + qi) * 2 + 1];
  };
  auto lse2 = [&](float a, float b, float& hi, float& lo) {
    const double L2 = ((double)a + (double)b) * kLog2e;
    hi = (float)L2;
    lo = (float)(L2 - (double)hi);
  };
  // BITS: only rows i >= wlo count, starting from the 64-aligned tile that holds the first
  const int wlo = BITS ? P - meta[u].window : (MODE == 2 ? P - rows : 0);
  const int i_first = BITS ? max(kb * kBlk, wlo) & ~(kTile - 1) : kb * kBlk;
  auto thr = [&](int i) { return (float)(-log2((double)(i + 1))); };
  uint64_t bits[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  // float32 sums of this lane's weights over two tiles at a time (8 terms),
  // then added into the float64 column sums
  float part[2][4], pm[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[mb][r] = pm[mb][r] = 0.f;
  int held = 0;                                 // tiles summed in part since the last flush
  auto flush = [&]() {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        cs[mb][r] += (double)part[mb][r];
        if (MODE == 2) ms[mb][r] += (double)pm[mb][r];
        part[mb][r] = pm[mb][r] = 0.f;
      }
    held = 0;
  };
  TileRegs<D> nxt;
  float la = 0.f, lb = 0.f;                     // the next tile's lse pair, as loaded
  load_tile<D>(nxt, qbase, i_first, P);
  store_tile<D>(nxt, Qs[0]);
  if (threadIdx.x < kTile) {
    float a, b, nh, nl;
    lse_load(i_first + threadIdx.x, a, b);
    lse2(a, b, nh, nl);
    Lh[0][threadIdx.x] = nh;
    Ll[0][threadIdx.x] = nl;
    Lf[0][threadIdx.x] = exp2f(-nl);
    if (BITS) Th[0][threadIdx.x] = thr(i_first + threadIdx.x);
  }
  __syncthreads();
  for (int it = 0, i0 = i_first; i0 < P; ++it, i0 += kTile) {
    const int buf = it & 1;
    const bool more = i0 + kTile < P;
    if (more) {
      load_tile<D>(nxt, qbase, i0 + kTile, P);
      if (threadIdx.x < kTile) lse_load(i0 + kTile + threadIdx.x, la, lb);   // in flight during the tile
    }
    if (i0 + kTile - 1 >= j0) {                 // some query of the tile follows a key of the wave
      const bool edge = i0 < j0 + 32 || i0 + kTile > P;
      const bool in_rows = MODE == 2 && i0 + kTile > wlo;   // the tile reaches the profiled rows
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 b = *reinterpret_cast<const uint4*>(Qs[buf] + (nb * 16 + c16) * Tile<D>::kRowBytes + (ks * 32 + g * 8) * 2);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) acc[mb] = Mfma<DT>::run(kf[mb][ks], b, acc[mb]);
        }
        const float lh = Lh[buf][nb * 16 + c16];
        if (BITS) persist_fold(acc, i0, nb, j0, P, wlo, g, c16, c2, lh, Ll[buf][nb * 16 + c16], Th[buf][nb * 16 + c16], bits);
        else if (in_rows) mass_fold(acc, i0, nb, j0, P, wlo, g, c16, c2, lh, Lf[buf][nb * 16 + c16], part, pm);
        else {
          if (edge) colsum_mask(acc, i0, nb, j0, P, g, c16, msk);
          colsum_fold(acc, c2, lh, Lf[buf][nb * 16 + c16], part);
        }
      }
      if constexpr (!BITS) {
        held = __builtin_amdgcn_readfirstlane(held + 1);   // the same in every lane of the wave
        if (held == 2) flush();
      }
    }
    if (more) {
      store_tile<D>(nxt, Qs[buf ^ 1]);          // that buffer was last read before the previous barrier
      if (threadIdx.x < kTile) {
        float nh, nl;
        lse2(la, lb, nh, nl);
        Lh[buf ^ 1][threadIdx.x] = nh;
        Ll[buf ^ 1][threadIdx.x] = nl;
        Lf[buf ^ 1][threadIdx.x] = exp2f(-nl);
        if (BITS) Th[buf ^ 1][threadIdx.x] = thr(i0 + kTile + threadIdx.x);
      }
    }
    __syncthreads();
  }
  if (!BITS && held) flush();
  if (BITS) {
    // the 16 lanes that share a key hold the same bits
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kj = j0 + mb * 16 + g * 4 + r;
        if (c16 == 0 && kj < P) reinterpret_cast<uint64_t*>(colsum)[(size_t)u * P + kj] = bits[mb][r];
      }
    return;
  }
  // sum over the 16 lanes (queries) that share each key
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      double v = cs[mb][r];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
      const int kj = j0 + mb * 16 + g * 4 + r;
      if (c16 == 0 && kj < P) colsum[(size_t)u * P + kj] = v;
      if (MODE == 2) {
        double w = ms[mb][r];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) w += __shfl_xor(w, o);
        if (c16 == 0 && kj < P) mass[(size_t)u * P + kj] = (float)w;
      }
    }
}

// ------------------------------------------------------------------ attend
// rowstats_fold plus the output: rescales this lane's output accumulators
// when a query's offset grows, and returns the tile's weights (zero where
// masked) as (hi, lo) B fragments, pw[nb][kp][0 = hi, 1 = lo].
template <int DT, int DB, bool EDGE>
__device__ inline void attend_fold(const f32x4 (&acc)[4][2], int k0, int q0, int P, int g, int c16,
                                   float c2, float (&mc)[2], double (&l)[2], f32x4 (&o)[DB][2],
                                   uint4 (&pw)[2][2][2]) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int qi = q0 + nb * 16 + c16;
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kj = k0 + mb * 16 + g * 4 + r;
        const bool ok = !EDGE || (kj <= qi && kj < P);
        tmax = fmaxf(tmax, ok ? acc[mb][nb][r] : -INFINITY);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(mc[nb], tmax * c2);
    if (mn > mc[nb]) {
      const float a = exp2_fast(mc[nb] - mn);
      l[nb] *= (double)a;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db][nb] *= a;
      mc[nb] = mn;
    }
    float p[4][4];
    float sum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = acc[mb][nb][r];
        float x = exp2_fast(fmaf(s, c2, -mn));
        if (EDGE) {
          const int kj = k0 + mb * 16 + g * 4 + r;
          x = (kj <= qi && kj < P) ? x : 0.f;
        }
        p[mb][r] = x;
        sum += x;
      }
    l[nb] += (double)sum;
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const float w[8] = {p[2 * kp][0], p[2 * kp][1], p[2 * kp][2], p[2 * kp][3],
                          p[2 * kp + 1][0], p[2 * kp + 1][1], p[2 * kp + 1][2], p[2 * kp + 1][3]};
      Split16<DT>::run(w, pw[nb][kp][0], pw[nb][kp][1]);
    }
  }
}

template <int D>
constexpr size_t attend_lds_bytes() {
  return 2 * (size_t)Tile<D>::kBytes + 2 * (size_t)VtTile<D>::kBytes;
}

// Workgroup = (unit, 128 queries) as in rowstats; LDS holds double-buffered K
// tiles and transposed V tiles.  Writes lse (as rowstats) and out[u][i][:].
template <int DT, int D>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(KVE_ATTEND_WAVES_PER_EU)))
void attend_mfma_kernel(Shape sh, int P, UnitList ul, const void* q, const void* k, const void* v, float* lse,
                        float* out) {
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;                    // 16-row blocks of V^T (head dimensions)
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const Ks = smem;                        // [2][Tile]
  char* const Vt = smem + 2 * Tile<D>::kBytes;  // [2][VtTile]
  const int u = ul.ids ? ul.ids[blockIdx.x] : blockIdx.x;
  const int nqb = (P + kBlk - 1) / kBlk;
  const int qb = nqb - 1 - (int)blockIdx.y;     // heaviest (last) query block first
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const size_t base = (size_t)u * P * D * 2;
  const char* qbase = (const char*)q + base;
  const char* kbase = (const char*)k + base;
  const char* vbase = (const char*)v + base;
  const int q0 = qb * kBlk + w * 32;
  const float c2 = make_scale2(sh.scale);

  uint4 qf[2][KS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int qi = q0 + nb * 16 + c16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[nb][ks] = qi < P ? ld16(qbase + ((size_t)qi * D + ks * 32 + g * 8) * 2) : make_uint4(0, 0, 0, 0);
  }
  float mc[2] = {-INFINITY, -INFINITY};
  double l[2] = {0.0, 0.0};
  f32x4 o[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) o[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int kend = min(P, qb * kBlk + kBlk);
  TileRegs<D> nk;
  VtRegs<D> nv;
  load_tile<D>(nk, kbase, 0, P);
  load_vtile<D>(nv, vbase, 0, P);
  store_tile<D>(nk, Ks);
  store_vtile<D>(nv, Vt);
  __syncthreads();
  for (int it = 0, k0 = 0; k0 < kend; ++it, k0 += kTile) {
    const int buf = it & 1;
    const char* ck = Ks + buf * Tile<D>::kBytes;
    const char* cv = Vt + buf * VtTile<D>::kBytes;
    const bool more = k0 + kTile < kend;
    if (more) {
      load_tile<D>(nk, kbase, k0 + kTile, P);
      load_vtile<D>(nv, vbase, k0 + kTile, P);
    }
    if (k0 <= q0 + 31) {
      f32x4 acc[4][2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 a = *reinterpret_cast<const uint4*>(ck + (mb * 16 + c16) * Tile<D>::kRowBytes + (ks * 32 + g * 8) * 2);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = Mfma<DT>::run(a, qf[nb][ks], acc[mb][nb]);
        }
      }
      if (more) {                               // those buffers were last read before the previous barrier
        store_tile<D>(nk, Ks + (buf ^ 1) * Tile<D>::kBytes);
        store_vtile<D>(nv, Vt + (buf ^ 1) * VtTile<D>::kBytes);
      }
      uint4 pw[2][2][2];
      if (k0 + kTile > q0 || k0 + kTile > P) attend_fold<DT, DB, true>(acc, k0, q0, P, g, c16, c2, mc, l, o, pw);
      else attend_fold<DT, DB, false>(acc, k0, q0, P, g, c16, c2, mc, l, o, pw);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const uint4 a = vt_fragment(cv, db * 16, kp, g, c16);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            o[db][nb] = Mfma<DT>::run(a, pw[nb][kp][0], o[db][nb]);
            o[db][nb] = Mfma<DT>::run(a, pw[nb][kp][1], o[db][nb]);
          }
        }
    } else if (more) {
      store_tile<D>(nk, Ks + (buf ^ 1) * Tile<D>::kBytes);
      store_vtile<D>(nv, Vt + (buf ^ 1) * VtTile<D>::kBytes);
    }
    __syncthreads();
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    double lt = l[nb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int qi = q0 + nb * 16 + c16;
    if (qi < P) {
      if (g == 0) {
        const double L = ((double)mc[nb] + log2(lt)) * kLn2;
        const float hi = (float)L;
        lse[((size_t)u * P + qi) * 2] = hi;
        lse[((size_t)u * P + qi) * 2 + 1] = (float)(L - (double)hi);
      }
      // this lane holds O^T[db * 16 + 4 g + r][qi], r = 0..3
      const float inv = (float)(1.0 / lt);
      float* orow = out + ((size_t)u * P + qi) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(orow + db * 16) = o[db][nb] * inv;
    }
  }
}

template <int DT, int D>
hipError_t attend_t(const Shape& sh, int P, UnitList ul, const void* q, const void* k, const void* v, float* lse,
                    float* out, hipStream_t st) {
  const size_t lds = attend_lds_bytes<D>();
  hipError_t e = hipFuncSetAttribute((const void*)attend_mfma_kernel<DT, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid(ul.n, (P + kBlk - 1) / kBlk);
  hipLaunchKernelGGL((attend_mfma_kernel<DT, D>), grid, dim3(kNT), lds, st, sh, P, ul, q, k, v, lse, out);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t rowstats_t(const Shape& sh, int P, UnitList ul, const void* q, const void* k, float* lse, int q_from,
                      hipStream_t st) {
  // blockIdx.y = 0 is the last query block, so the first nqb - q_from / kBlk blocks cover rows >= q_from
  dim3 grid(ul.n, (P + kBlk - 1) / kBlk - q_from / kBlk);
  hipLaunchKernelGGL((rowstats_mfma_kernel<DT, D>), grid, dim3(kNT), 0, st, sh, P, ul, q, k, lse);
  return hipGetLastError();
}

template <int DT, int D, int MODE>
hipError_t colsum_t(const Shape& sh, int P, UnitList ul, const void* q, const void* k, const float* lse,
                    double* colsum, const HeadMeta* meta, float* mass, int rows, hipStream_t st) {
  dim3 grid(ul.n, (P + kBlk - 1) / kBlk);
  hipLaunchKernelGGL((colsum_mfma_kernel<DT, D, MODE>), grid, dim3(kNT), 0, st, sh, P, ul, q, k, lse, colsum,
                     meta, mass, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_rowstats_mfma(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                        float* lse, int q_from, hipStream_t st) {
  if (ul.n <= 0) return hipSuccess;
  if (q_from < 0 || q_from >= P) return hipErrorInvalidValue;
  switch (sh.dtype * 1000 + sh.d) {
    case F16 * 1000 + 64: return rowstats_t<F16, 64>(sh, P, ul, q, k, lse, q_from, st);
    case F16 * 1000 + 128: return rowstats_t<F16, 128>(sh, P, ul, q, k, lse, q_from, st);
    case BF16 * 1000 + 64: return rowstats_t<BF16, 64>(sh, P, ul, q, k, lse, q_from, st);
    case BF16 * 1000 + 128: return rowstats_t<BF16, 128>(sh, P, ul, q, k, lse, q_from, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_attend_mfma(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                      const void* v, float* lse, float* out, hipStream_t st) {
  if (ul.n <= 0) return hipSuccess;
  switch (sh.dtype * 1000 + sh.d) {
    case F16 * 1000 + 64: return attend_t<F16, 64>(sh, P, ul, q, k, v, lse, out, st);
    case F16 * 1000 + 128: return attend_t<F16, 128>(sh, P, ul, q, k, v, lse, out, st);
    case BF16 * 1000 + 64: return attend_t<BF16, 64>(sh, P, ul, q, k, v, lse, out, st);
    case BF16 * 1000 + 128: return attend_t<BF16, 128>(sh, P, ul, q, k, v, lse, out, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_colsum_mfma(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                      const float* lse, double* colsum, hipStream_t st) {
  if (ul.n <= 0) return hipSuccess;
  switch (sh.dtype * 1000 + sh.d) {
    case F16 * 1000 + 64: return colsum_t<F16, 64, 0>(sh, P, ul, q, k, lse, colsum, nullptr, nullptr, 0, st);
    case F16 * 1000 + 128: return colsum_t<F16, 128, 0>(sh, P, ul, q, k, lse, colsum, nullptr, nullptr, 0, st);
    case BF16 * 1000 + 64: return colsum_t<BF16, 64, 0>(sh, P, ul, q, k, lse, colsum, nullptr, nullptr, 0, st);
    case BF16 * 1000 + 128: return colsum_t<BF16, 128, 0>(sh, P, ul, q, k, lse, colsum, nullptr, nullptr, 0, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_persist_mfma(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                       const float* lse, const HeadMeta* meta, double* bits, hipStream_t st) {
  if (ul.n <= 0) return hipSuccess;
  if (!meta) return hipErrorInvalidValue;
  switch (sh.dtype * 1000 + sh.d) {
    case F16 * 1000 + 64: return colsum_t<F16, 64, 1>(sh, P, ul, q, k, lse, bits, meta, nullptr, 0, st);
    case F16 * 1000 + 128: return colsum_t<F16, 128, 1>(sh, P, ul, q, k, lse, bits, meta, nullptr, 0, st);
    case BF16 * 1000 + 64: return colsum_t<BF16, 64, 1>(sh, P, ul, q, k, lse, bits, meta, nullptr, 0, st);
    case BF16 * 1000 + 128: return colsum_t<BF16, 128, 1>(sh, P, ul, q, k, lse, bits, meta, nullptr, 0, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve

namespace kve {

hipError_t launch_prefill_colsum_mass_mfma(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                           const float* lse, double* colsum, float* mass, int rows,
                                           hipStream_t st) {
  if (ul.n <= 0) return hipSuccess;
  if (!mass || rows < 1) return hipErrorInvalidValue;
  switch (sh.dtype * 1000 + sh.d) {
    case F16 * 1000 + 64: return colsum_t<F16, 64, 2>(sh, P, ul, q, k, lse, colsum, nullptr, mass, rows, st);
    case F16 * 1000 + 128: return colsum_t<F16, 128, 2>(sh, P, ul, q, k, lse, colsum, nullptr, mass, rows, st);
    case BF16 * 1000 + 64: return colsum_t<BF16, 64, 2>(sh, P, ul, q, k, lse, colsum, nullptr, mass, rows, st);
    case BF16 * 1000 + 128: return colsum_t<BF16, 128, 2>(sh, P, ul, q, k, lse, colsum, nullptr, mass, rows, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve
