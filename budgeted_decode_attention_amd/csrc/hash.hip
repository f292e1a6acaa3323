// HashEvict (summary page, original abstract): keys are tracked by sign
// sketches of a Gaussian projection far narrower than the head dimension,
// kept as a small binary structure in GPU memory; before attention, the new
// token replaces the cached token whose sketch is farthest (Hamming distance)
// from the query's sketch -- the one expected to receive the least attention.
//
// Sketch bit b of x is set iff the exact sum_i W[i][b] x[i] is positive.  The
// products of bf16 W with bf16/fp16/fp32 inputs are exact in float64; their
// float64 sum is within gamma_d * sum|terms| of the exact value, so the sign
// is taken from it unless |sum| is inside that bound, in which case the terms
// are re-added exactly as a non-overlapping expansion (two-sum chains).
//
// Ties in distance go to the oldest position.  The prompt is replayed: the
// cache starts as positions [0, B) and each prompt position i >= B replaces
// the farthest key from sketch(q_i).
//
// Sketch widths of 16, 32 and 64 bits (the page only asks for a projection
// far narrower than the head dimension): one lane per bit, 32-bit words for
// 16 and 32 bits, 64-bit words for 64.
//
// With 4-bit slots the rows entering the cache (the replay's gather, the
// replacement at each step) are quantised; sketches always come from the
// inputs.
#include "hash.hpp"

namespace kve {
namespace {

constexpr int kNT = 256;

constexpr int kSketchRows = 64;   // rows per workgroup in sketch_rows_kernel

// Sketches of rows [row0, row0 + nrows) of each listed unit: a workgroup
// stages the projection once and then covers kSketchRows rows, kNT / BITS at
// a time (BITS lanes per row; the lane index within the row is the bit).
template <int DT, int D, int BITS>
__global__ __launch_bounds__(kNT) void sketch_rows_kernel(Shape sh, UnitList ul, const void* x, int P, int row0,
                                                          int nrows, const uint16_t* proj,
                                                          typename SkWord<BITS>::T* out) {
  constexpr int RPP = kNT / BITS;                            // rows per pass
  __shared__ __attribute__((aligned(16))) uint16_t Ws[D * BITS];
  __shared__ float xs[RPP][D];
  __shared__ double ebuf[kNT / kWave][D + 1];                // the exact fallback, per wave
  constexpr int ES = elem_bytes<DT>();
  const int u = ul.ids ? ul.ids[blockIdx.y] : blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int b = lane % BITS;
  const int slot = threadIdx.x / BITS;                       // row slot within a pass
  stage_proj<D, BITS>(Ws, proj);
  for (int pass = 0; pass < kSketchRows / RPP; ++pass) {
    const int r = blockIdx.x * kSketchRows + pass * RPP + slot;   // row index within [0, nrows)
    const bool ok = r < nrows;
    const char* row = (const char*)x + ((size_t)u * P + row0 + (ok ? r : 0)) * D * ES;
    __syncthreads();                                        // previous pass done with xs; Ws staged
    for (int i = b; i < D; i += BITS) xs[slot][i] = ok ? load_elem<DT>(row, i) : 0.f;
    __syncthreads();
    const int bit = sketch_bit<DT, D>(ok, xs[slot], Ws, row, proj, BITS, b, ebuf[threadIdx.x / kWave]);
    const uint64_t m = __ballot(bit != 0);
    if (ok && b == 0) out[(size_t)u * P + row0 + r] = ballot_field<BITS>(m, lane);
  }
}

// ---------------------------------------------------------------- matrix-core sketches (bf16 rows)
//
// For bf16 rows the projections run on the matrix cores: v_mfma_f32_16x16x32_bf16
// with A = 16 rows x 32 features and B = 32 features x 16 sketch bits gives
// every (row, bit) sum s in float32, and a second product of |rows| and |W|
// gives a = sum |x_i w_ib|.  Products of two bf16 values are exact in float32;
// the accumulation of D of them errs by at most gamma_D = D u / (1 - D u)
// times a with u = 2^-23 (one unit in the last place per addition: this also
// covers truncating or multi-operand adders), plus an absolute D 2^-126
// (max|W| + 2) for products, inputs and partial sums flushed below the
// float32 normal range.  The sign of s is the exact sign when |s| exceeds
// twice that relative bound times a plus twice the absolute one; every other
// (row, bit) -- tiny or cancelling sums, non-finite or overflowing rows -- is
// settled as before (float64 with its own bound, then the exact expansion).

typedef __bf16 sk_bf16x8 __attribute__((ext_vector_type(8)));
typedef float sk_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaTiles = 4;                                 // 16-row tiles per wave and pass
constexpr int kMfmaPasses = 2;                                // passes per workgroup
constexpr int kMfmaRows = kNT / kWave * kMfmaTiles * 16 * kMfmaPasses;   // 512 rows per workgroup

__device__ inline sk_f32x4 mfma_bf16(const uint4& a, const uint4& b, sk_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sk_bf16x8, a), __builtin_bit_cast(sk_bf16x8, b),
                                                 c, 0, 0, 0);
}
__device__ inline uint4 abs_bf16x8(uint4 v) {
  return make_uint4(v.x & 0x7fff7fffu, v.y & 0x7fff7fffu, v.z & 0x7fff7fffu, v.w & 0x7fff7fffu);
}

// Relative threshold factor 2 gamma_D / (1 - gamma_D) with u = 2^-23, rounded up.
template <int D> __host__ __device__ constexpr float mfma_sign_threshold() {
  constexpr double u = 1.0 / 8388608.0;
  constexpr double g = D * u / (1.0 - D * u);
  return (float)(2.0 * g / (1.0 - g) * 1.0001);
}

// Sketches of rows [row0, row0 + nrows) of each listed unit from bf16 rows.
// Wave w of a workgroup takes kMfmaTiles tiles of 16 consecutive rows per
// pass; lane l supplies row l % 16 of a tile and features 8 (l / 16) + 0..7
// of each 32-feature step, and receives rows 4 (l / 16) + 0..3, bit l % 16
// of each 16-bit block of the sketch.
template <int D, int BITS>
__global__ __launch_bounds__(kNT) void sketch_rows_mfma_kernel(UnitList ul, const void* x, int P, int row0,
                                                               int nrows, const uint16_t* proj,
                                                               typename SkWord<BITS>::T* out) {
  using SW = typename SkWord<BITS>::T;
  constexpr int NB = BITS / 16;                              // 16-bit blocks of a sketch
  constexpr int KS = D / 32;                                 // 32-feature steps
  static_assert(NB * 4 <= 32, "one flag bit per (block, row) of a lane");
  __shared__ __attribute__((aligned(16))) uint16_t Ws[D * BITS];
  __shared__ double ebuf[kNT / kWave][D + 1];                // the exact fallback, per wave
  __shared__ float wred[kNT / kWave];
  const int u = ul.ids ? ul.ids[blockIdx.y] : blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const char* base = (const char*)x + ((size_t)u * P + row0) * D * 2;

  stage_proj<D, BITS>(Ws, proj);
  __syncthreads();
  float wm = 0.f;
  for (int i = tid; i < D * BITS; i += kNT) wm = fmaxf(wm, fabsf(__uint_as_float((uint32_t)Ws[i] << 16)));
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) wm = fmaxf(wm, __shfl_xor(wm, o));
  if (lane == 0) wred[wv] = wm;
  // B fragments: lane (g, c16) holds W[32 kk + 8 g + 0..7][16 nb + c16]
  uint4 wf[KS][NB], wa[KS][NB];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint32_t h[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i0 = kk * 32 + 8 * g + 2 * t;
        h[t] = (uint32_t)Ws[i0 * BITS + nb * 16 + c16] | ((uint32_t)Ws[(i0 + 1) * BITS + nb * 16 + c16] << 16);
      }
      wf[kk][nb] = make_uint4(h[0], h[1], h[2], h[3]);
      wa[kk][nb] = abs_bf16x8(wf[kk][nb]);
    }
  __syncthreads();
  float wmax = wred[0];
#pragma unroll
  for (int i = 1; i < kNT / kWave; ++i) wmax = fmaxf(wmax, wred[i]);
  const float thr = mfma_sign_threshold<D>();
  const float tau = 2.f * (float)D * 0x1p-126f * (wmax + 2.f);   // inf (everything falls back) if W is huge

  for (int pass = 0; pass < kMfmaPasses; ++pass) {
    const int rw = blockIdx.x * kMfmaRows + (pass * (kNT / kWave) + wv) * (kMfmaTiles * 16);
    // rows at or past nrows read as zero (range-checked buffer loads)
    const uint32_t bytes = rw < nrows ? (uint32_t)(nrows - rw) * D * 2 : 0u;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base) + (size_t)rw * D * 2, (short)0, (int)bytes,
                                          0x00020000);
    uint4 xt[kMfmaTiles][KS];
#pragma unroll
    for (int t = 0; t < kMfmaTiles; ++t)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        xt[t][kk] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (t * 16 + c16) * D * 2 + kk * 64 + g * 16, 0, 0));
#pragma unroll
    for (int t = 0; t < kMfmaTiles; ++t) {
      const int rt = rw + t * 16;                            // the tile's first row
      if (rt >= nrows) break;                                // uniform
      sk_f32x4 sv[NB], av[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sv[nb] = sk_f32x4{0.f, 0.f, 0.f, 0.f};
        av[nb] = sk_f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint4 xa = abs_bf16x8(xt[t][kk]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          sv[nb] = mfma_bf16(xt[t][kk], wf[kk][nb], sv[nb]);
          av[nb] = mfma_bf16(xa, wa[kk][nb], av[nb]);
        }
      }
      // flag bit nb * 4 + r: row rt + 4 g + r, sketch bit 16 nb + c16
      uint32_t bitm = 0, ambm = 0;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = sv[nb][r], a = av[nb][r];
          if (s > 0.f) bitm |= 1u << (nb * 4 + r);
          if (rt + 4 * g + r < nrows && !(fabsf(s) > fmaf(thr, a, tau))) ambm |= 1u << (nb * 4 + r);
        }
      if (__ballot(ambm != 0)) {                             // rare: float64, then exact
#pragma unroll
        for (int f = 0; f < NB * 4; ++f) {
          const bool mine = (ambm >> f) & 1u;
          if (!__ballot(mine)) continue;
          const int r = f & 3, b = (f >> 2) * 16 + c16;
          const char* row = base + (size_t)(rt + 4 * g + r) * D * 2;
          int v = mine ? sketch_bit_fast<D>([&](int i) { return load_elem<BF16>(row, i); }, Ws, BITS, b) : 0;
          uint64_t fr = __ballot(v < 0);
          while (fr) {                                       // uniform over the wave
            if (lane == __builtin_ctzll(fr)) v = exact_sign<BF16, D>(row, proj, BITS, b, ebuf[wv]);
            fr &= fr - 1;
          }
          if (mine) bitm = (bitm & ~(1u << f)) | ((uint32_t)v << f);
        }
      }
      uint64_t m[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) m[nb][r] = __ballot((bitm >> (nb * 4 + r)) & 1u);
      // lane L < 16 assembles row rt + L = rt + 4 (L / 4) + (L % 4)
      if (lane < 16 && rt + lane < nrows) {
        const int gg = lane >> 2, rr = lane & 3;
        SW word = 0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint64_t mm = rr == 0 ? m[nb][0] : rr == 1 ? m[nb][1] : rr == 2 ? m[nb][2] : m[nb][3];
          word |= (SW)((mm >> (16 * gg)) & 0xFFFFu) << (16 * nb);
        }
        out[(size_t)u * P + row0 + rt + lane] = word;
      }
    }
  }
}

// Copies the kept prompt rows (positions spos[0, n0)) into the unit's slots,
// quantised with 4-bit slots.  All threads of the workgroup.
template <int DT, int D>
__device__ inline void replay_gather(const LayerCache& c, int u, int P, int n0, const int32_t* spos,
                                     const void* k, const void* v) {
  constexpr int EPL = St<DT>::EPL;
  constexpr int ES = elem_bytes<DT>();
  constexpr int LPR = D / EPL;
  constexpr int RPI = kNT / LPR;
  const int tid = threadIdx.x;
  const size_t slot0 = (size_t)u * c.cap;
  const size_t src0 = (size_t)u * P * D * ES;
  if (c.q4) {
    constexpr int G = D / kQGroup;
    char* Kq = (char*)c.K + slot0 * (D / 2);
    char* Vq = (char*)c.V + slot0 * (D / 2);
    const int g = tid % G;
    for (int s = tid / G; s < n0; s += kNT / G) {
      const size_t so = src0 + (size_t)spos[s] * D * ES;
      q4_store_group<DT, D>((const char*)k + so, Kq + (size_t)s * (D / 2), c.Ksc + (slot0 + s) * G, g);
      q4_store_group<DT, D>((const char*)v + so, Vq + (size_t)s * (D / 2), c.Vsc + (slot0 + s) * G, g);
    }
    return;
  }
  char* Kd = (char*)c.K + slot0 * D * ES;
  char* Vd = (char*)c.V + slot0 * D * ES;
  const int col = tid % LPR;
  for (int s = tid / LPR; s < n0; s += RPI) {
    const size_t so = ((size_t)spos[s] * D + col * EPL) * ES;
    const size_t dof = ((size_t)s * D + col * EPL) * ES;
    st16(Kd + dof, ld16((const char*)k + src0 + so));
    st16(Vd + dof, ld16((const char*)v + src0 + so));
  }
}

// Prompt replay for one HASH unit per workgroup; slot state in LDS.
template <int DT, int D, int BITS>
__global__ __launch_bounds__(kNT) void hash_replay_kernel(Shape sh, LayerCache c, UnitList ul, int P,
                                                          const typename SkWord<BITS>::T* qsk,
                                                          const typename SkWord<BITS>::T* ksk,
                                                          const void* k, const void* v) {
  using SW = typename SkWord<BITS>::T;
  extern __shared__ __attribute__((aligned(16))) char lds[];   // sk[B] then pos[B]
  __shared__ uint64_t kscr[2][kNT / kWave];
  const int u = ul.ids[blockIdx.x];
  const int tid = threadIdx.x;
  const HeadMeta m = c.meta[u];
  const int B = m.heavy;
  const int n0 = min(P, B);
  SW* ssk = reinterpret_cast<SW*>(lds);
  int32_t* spos = reinterpret_cast<int32_t*>(lds + (size_t)B * sizeof(SW));
  const SW* kq = ksk + (size_t)u * P;
  const SW* qq = qsk + (size_t)u * P;
  for (int s = tid; s < n0; s += kNT) {
    ssk[s] = kq[s];
    spos[s] = s;
  }
  __syncthreads();
  const int lane = tid & (kWave - 1);
  for (int i = B; i < P; ++i) {
    const SW qs = qq[i];
    uint32_t best = 0;
    int bslot = 0;
    // four slots per thread per round: their LDS reads are issued together;
    // past the budget a thread re-reads its own slot s0, so it reads only
    // slots it owns (their owner alone rewrites them)
    for (int s0 = tid; s0 < B; s0 += 4 * kNT) {
      SW sk[4];
      int ps[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = s0 + j * kNT < B ? s0 + j * kNT : s0;
        sk[j] = ssk[s];
        ps[j] = spos[s];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t key = evict_key(popcnt(qs ^ sk[j]), ps[j]);
        if (s0 + j * kNT < B && key > best) {
          best = key;
          bslot = s0 + j * kNT;
        }
      }
    }
    const uint64_t wb = wave_best(best, bslot);
    // one barrier per step: the wave maxima alternate between two buffers,
    // every thread reduces them, and the replaced slot is rewritten by the
    // thread whose scan owns it (slot % NT), which alone reads it later
    if (lane == 0) kscr[i & 1][tid / kWave] = wb;
    __syncthreads();
    uint64_t bb = kscr[i & 1][0];
#pragma unroll
    for (int w = 1; w < kNT / kWave; ++w) bb = kscr[i & 1][w] > bb ? kscr[i & 1][w] : bb;
    const int slot = (int)(bb & 0xFFFFFFFFu);
    if (slot % kNT == tid) {
      ssk[slot] = kq[i];
      spos[slot] = i;
    }
  }
  __syncthreads();                              // every slot's last write is visible
  const size_t slot0 = (size_t)u * c.cap;
  for (int s = tid; s < c.cap; s += kNT) {
    int32_t p = -1;
    SW sk = 0;
    if (s < n0) {
      p = spos[s];
      sk = ssk[s];
    }
    c.pos[slot0 + s] = p;
    reinterpret_cast<SW*>(c.sk)[slot0 + s] = sk;
    c.S[slot0 + s] = 0.0;
  }
  if (tid == 0) c.count[u] = n0;
  replay_gather<DT, D>(c, u, P, n0, spos, k, v);
}

// Lane d's value of x, as a wave-uniform value.
__device__ inline uint32_t lane_read(uint32_t x, int d) { return (uint32_t)__builtin_amdgcn_readlane((int)x, d); }
__device__ inline uint64_t lane_read(uint64_t x, int d) {
  return ((uint64_t)lane_read((uint32_t)(x >> 32), d) << 32) | lane_read((uint32_t)x, d);
}

// Prompt replay with every slot's state in registers, for budgets up to
// JR * kNT slots: thread tid owns slots j * kNT + tid (j < JR), keeping each
// one's sketch and its eviction key's low part, ((65535 - position) << 7) | j,
// so a decision costs four vector operations per slot (xor, population count,
// shift-or, signed maximum) and no LDS traffic.  Slots at or past the budget
// carry a low part with the sign bit set, so their keys are negative and never
// win: the scan needs no masks.  The workgroup's maximum key names the
// winner's position and j; the winning lane's thread index travels with it,
// and the owner rewrites its registers j.  Positions below 65,536 are
// distinct, so the maximum is unique.
template <int DT, int D, int BITS, int JR>
__global__ __launch_bounds__(kNT) void hash_replay_reg_kernel(Shape sh, LayerCache c, UnitList ul, int P,
                                                              const typename SkWord<BITS>::T* qsk,
                                                              const typename SkWord<BITS>::T* ksk,
                                                              const void* k, const void* v) {
  using SW = typename SkWord<BITS>::T;
  static_assert(JR <= 128, "j takes 7 bits of the key");
  constexpr uint32_t kDead = 0x80000000u;
  extern __shared__ __attribute__((aligned(16))) char lds[];   // pos[B] for the gather
  __shared__ uint64_t kscr[2][kNT / kWave];
  const int u = ul.ids[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int B = c.meta[u].heavy;
  const int n0 = min(P, B);
  const SW* kq = ksk + (size_t)u * P;
  const SW* qq = qsk + (size_t)u * P;
  SW sk[JR];
  uint32_t lo[JR];
#pragma unroll
  for (int j = 0; j < JR; ++j) {
    const int s = j * kNT + tid;
    sk[j] = s < n0 ? kq[s] : (SW)0;
    lo[j] = s < B ? ((uint32_t)(0xFFFF - s) << 7) | (uint32_t)j : kDead;
  }
  // the decisions' query and key sketches come in windows of 64, lane l of
  // every wave holding decision w0 + l's, in two register pairs used in turn:
  // each window is loaded while the one before it is decided, and a decision
  // reads its own with two lane reads
  const int nd = P - B;                         // decisions (none if P <= B)
  auto window = [&](const SW* x, int w0) -> SW { return x[min(B + w0 + lane, P - 1)]; };
  auto decide = [&](SW qw, SW kw, int w0) {
    const int m = min(kWave, nd - w0);
    for (int d = 0; d < m; ++d) {
      const int i = B + w0 + d;
      const SW qs = lane_read(qw, d), ks = lane_read(kw, d);
      int best = INT32_MIN;
#pragma unroll
      for (int j = 0; j < JR; ++j)
        best = max(best, (int)(((uint32_t)popcnt(qs ^ sk[j]) << 23) | lo[j]));
      const uint32_t kb = (uint32_t)max(best, 0);   // a thread with no slot offers 0
      const uint32_t wm = wave_max_key(kb);
      const int wl = __builtin_ctzll(__ballot(kb == wm));
      if (lane == 0) kscr[i & 1][tid / kWave] = ((uint64_t)wm << 32) | (uint32_t)(tid + wl);
      __syncthreads();
      uint64_t bb = kscr[i & 1][0];
#pragma unroll
      for (int w = 1; w < kNT / kWave; ++w) bb = kscr[i & 1][w] > bb ? kscr[i & 1][w] : bb;
      const int owner = __builtin_amdgcn_readfirstlane((int)(bb & 0xFFFFFFFFu));
      const int jw = __builtin_amdgcn_readfirstlane((int)((bb >> 32) & 0x7F));
      if (tid == owner) {                         // jw is uniform: an indexed register write
        sk[jw] = ks;
        lo[jw] = ((uint32_t)(0xFFFF - i) << 7) | (uint32_t)jw;
      }
    }
  };
  if (nd > 0) {
    SW qa = window(qq, 0), ka = window(kq, 0);
    SW qb = window(qq, kWave), kb = window(kq, kWave);
    for (int w0 = 0;; w0 += 2 * kWave) {
      decide(qa, ka, w0);
      if (w0 + kWave >= nd) break;
      qa = window(qq, w0 + 2 * kWave);
      ka = window(kq, w0 + 2 * kWave);
      decide(qb, kb, w0 + kWave);
      if (w0 + 2 * kWave >= nd) break;
      qb = window(qq, w0 + 3 * kWave);
      kb = window(kq, w0 + 3 * kWave);
    }
  }
  int32_t* spos = reinterpret_cast<int32_t*>(lds);
  const size_t slot0 = (size_t)u * c.cap;
#pragma unroll
  for (int j = 0; j < JR; ++j) {
    const int s = j * kNT + tid;
    if (s < B) {
      const bool full = s < n0;
      const int p = 0xFFFF - (int)(lo[j] >> 7);
      if (full) spos[s] = p;
      c.pos[slot0 + s] = full ? p : -1;
      reinterpret_cast<SW*>(c.sk)[slot0 + s] = full ? sk[j] : (SW)0;
      c.S[slot0 + s] = 0.0;
    }
  }
  for (int s = B + tid; s < c.cap; s += kNT) {
    c.pos[slot0 + s] = -1;
    reinterpret_cast<SW*>(c.sk)[slot0 + s] = 0;
    c.S[slot0 + s] = 0.0;
  }
  if (tid == 0) c.count[u] = n0;
  __syncthreads();                              // spos complete
  replay_gather<DT, D>(c, u, P, n0, spos, k, v);
}

// Decode-time replacement for one HASH unit per workgroup (layers that take
// the split decode; the fused decode runs the same replacement itself).
template <int DT, int D, int BITS>
__global__ __launch_bounds__(kNT) void hash_evict_kernel(Shape sh, LayerCache c, UnitList ul, int t,
                                                         const void* q, const void* k, const void* v,
                                                         int32_t* evicted) {
  static_assert(kNT == kHashNT, "workgroup size");
  __shared__ __attribute__((aligned(16))) char lds[hash_replace_lds<D, BITS>()];
  const int u = ul.ids[blockIdx.x];
  hash_replace<DT, D, BITS>(c, u, t, c.meta[u].heavy, c.count[u], q, k, v, evicted, lds);
}

#define KVE_DISPATCH_D(FN, BITS, ...)                                           \
  switch (sh.dtype * 1000 + sh.d) {                                              \
    case F32 * 1000 + 64: return FN<F32, 64, BITS>(__VA_ARGS__);                 \
    case F32 * 1000 + 128: return FN<F32, 128, BITS>(__VA_ARGS__);               \
    case F16 * 1000 + 64: return FN<F16, 64, BITS>(__VA_ARGS__);                 \
    case F16 * 1000 + 128: return FN<F16, 128, BITS>(__VA_ARGS__);               \
    case BF16 * 1000 + 64: return FN<BF16, 64, BITS>(__VA_ARGS__);               \
    case BF16 * 1000 + 128: return FN<BF16, 128, BITS>(__VA_ARGS__);             \
  }                                                                              \
  return hipErrorInvalidValue;

#define KVE_DISPATCH(FN, BITS_RT, ...)                                          \
  switch (BITS_RT) {                                                             \
    case 16: { KVE_DISPATCH_D(FN, 16, __VA_ARGS__) }                             \
    case 32: { KVE_DISPATCH_D(FN, 32, __VA_ARGS__) }                             \
    case 64: { KVE_DISPATCH_D(FN, 64, __VA_ARGS__) }                             \
  }                                                                              \
  return hipErrorInvalidValue;

template <int DT, int D, int BITS>
hipError_t sketch_t(const Shape& sh, UnitList ul, const void* x, int P, int row0, int nrows,
                    const uint16_t* proj, void* out, hipStream_t st) {
  if (nrows <= 0 || ul.n <= 0) return hipSuccess;
  if constexpr (DT == BF16) {
    dim3 grid((nrows + kMfmaRows - 1) / kMfmaRows, ul.n);
    hipLaunchKernelGGL((sketch_rows_mfma_kernel<D, BITS>), grid, dim3(kNT), 0, st, ul, x, P, row0, nrows, proj,
                       reinterpret_cast<typename SkWord<BITS>::T*>(out));
    return hipGetLastError();
  }
  dim3 grid((nrows + kSketchRows - 1) / kSketchRows, ul.n);
  hipLaunchKernelGGL((sketch_rows_kernel<DT, D, BITS>), grid, dim3(kNT), 0, st, sh, ul, x, P, row0, nrows, proj,
                     reinterpret_cast<typename SkWord<BITS>::T*>(out));
  return hipGetLastError();
}

template <int DT, int D, int BITS>
hipError_t replay_t(const Shape& sh, const LayerCache& c, UnitList ul, int P, const void* qsk, const void* ksk,
                    const void* k, const void* v, int B, hipStream_t st) {
  using SW = typename SkWord<BITS>::T;
  if (ul.n <= 0) return hipSuccess;
  if (B <= 16 * kNT) {
    auto fn = B <= 4 * kNT ? hash_replay_reg_kernel<DT, D, BITS, 4> : hash_replay_reg_kernel<DT, D, BITS, 16>;
    hipLaunchKernelGGL(fn, dim3(ul.n), dim3(kNT), (size_t)B * 4, st, sh, c, ul, P,
                       reinterpret_cast<const SW*>(qsk), reinterpret_cast<const SW*>(ksk), k, v);
    return hipGetLastError();
  }
  const size_t lds = (size_t)B * (sizeof(SW) + 4);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)hash_replay_kernel<DT, D, BITS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((hash_replay_kernel<DT, D, BITS>), dim3(ul.n), dim3(kNT), lds, st, sh, c, ul, P,
                     reinterpret_cast<const SW*>(qsk), reinterpret_cast<const SW*>(ksk), k, v);
  return hipGetLastError();
}

template <int DT, int D, int BITS>
hipError_t evict_t(const Shape& sh, const LayerCache& c, UnitList ul, int t, const void* q, const void* k,
                   const void* v, int32_t* evicted, hipStream_t st) {
  if (ul.n <= 0) return hipSuccess;
  hipLaunchKernelGGL((hash_evict_kernel<DT, D, BITS>), dim3(ul.n), dim3(kNT), 0, st, sh, c, ul, t, q, k, v,
                     evicted);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sketch_rows(const Shape& sh, UnitList units, const void* x, int P, int row0, int nrows,
                              const uint16_t* proj, int bits, void* out, hipStream_t st) {
  KVE_DISPATCH(sketch_t, bits, sh, units, x, P, row0, nrows, proj, out, st)
}

hipError_t launch_hash_prefill(const Shape& sh, const LayerCache& c, UnitList units, int P, int max_budget,
                               const void* qsk, const void* ksk, const void* k, const void* v, hipStream_t st) {
  KVE_DISPATCH(replay_t, c.sk_bits, sh, c, units, P, qsk, ksk, k, v, max_budget, st)
}

hipError_t launch_hash_evict(const Shape& sh, const LayerCache& c, UnitList units, int t, const void* q,
                             const void* k, const void* v, int32_t* evicted, hipStream_t st) {
  KVE_DISPATCH(evict_t, c.sk_bits, sh, c, units, t, q, k, v, evicted, st)
}

}  // namespace kve
