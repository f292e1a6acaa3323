// Decode step: attention over a unit's kept slots, score accumulation and
// the cache policy's replacement.
//
// H2O review page, proposed method: each decode step's attention weights are
// the statistics that drive a greedy eviction; the lowest-scoring token
// outside the recent window leaves and the new token takes its slot.  FastGen
// review page: the same step under per-head positional policies.
// Scissorhands summary page (persistence of importance), as read here: the
// same step with the score replaced by the number of recent steps at which a
// token's weight reached the uniform weight 1 / |A|.
//
// Layout: slot rows of d elements, 16 bytes per lane; LPR lanes cover one row
// (a row group) and the workgroup covers NT / LPR rows per load wave.  Logits
// are formed by DPP sums inside each row group.
//
// Two launch shapes, chosen per layer by the slot stride:
//   fused     one workgroup per unit: logits to LDS, exact softmax (maximum,
//             float64 sum), P.V, then the policy step;
//   split     `partials` over (unit, chunk of slots) writes each chunk's
//             maximum, sum and unnormalised output plus the raw logits;
//             `combine`, one workgroup per unit, merges the chunks under the
//             global maximum and runs the same policy step, recomputing the
//             exact weights from the logits for the float64 score update.
//
// 4-bit slots (Q4 instantiations): one lane owns half a group, 16 elements of
// a row (d / 16 lanes per row, one 8-byte code load and its group's scale per
// lane, the register budget of the 16-bit kernels, so every workgroup of a
// layer stays resident); the dot uses the stored nibbles c + 8 and subtracts
// 8 * (sum of the lane's query elements) once per row, the value pass
// accumulates w * scale * (c + 8) and subtracts 8 * sum(w * scale) at the end.  Token t's own key and
// value are read from the inputs at full precision and quantised into its slot.
#include "common.hpp"
#include "hash.hpp"
#include "q4.hpp"

namespace kve {
namespace {

// Compile-time tuning: rows loaded per thread before use; the register budget
// as resident waves per SIMD (0 = compiler's choice; 8 lets every workgroup of
// a 1,792-unit layer be resident at once); non-temporal K/V loads.
#ifndef KVE_DECODE_UNROLL
#define KVE_DECODE_UNROLL 2
#endif
#ifndef KVE_DECODE_WAVES_PER_EU
#define KVE_DECODE_WAVES_PER_EU 8
#endif
#ifndef KVE_DECODE_NT_LOADS
#define KVE_DECODE_NT_LOADS 1
#endif

constexpr int kNT = 256;
constexpr int kUnroll = KVE_DECODE_UNROLL;
// Caches of at most kSmallCache slots load kUnrollSmall rows per thread at a
// time (4 x 16 rows of 16-bit elements per round trip: a 102-slot unit in
// two), still within the register budget of 8 waves per SIMD.
#ifndef KVE_DECODE_SMALL_CACHE
#define KVE_DECODE_SMALL_CACHE 256
#endif
constexpr int kSmallCache = KVE_DECODE_SMALL_CACHE;
constexpr int kUnrollSmall = 4;
// Small caches take the policy's decision before the value pass.
#ifndef KVE_DECODE_DECIDE_EARLY
#define KVE_DECODE_DECIDE_EARLY 1
#endif
// Wave priority by phase for small caches: a workgroup starts at the
// highest and lowers it after the key pass and after the value pass, so waves
// still streaming keys win issue over those further on (the youngest
// workgroups on a CU otherwise finish their key pass last).
#ifndef KVE_DECODE_PRIO
#define KVE_DECODE_PRIO 1
#endif

#ifndef KVE_DECODE_WAVES_PER_EU_Q4
#define KVE_DECODE_WAVES_PER_EU_Q4 8
#endif
#if KVE_DECODE_WAVES_PER_EU > 0
#define KVE_DECODE_ATTR                  \
  __launch_bounds__(kNT) __attribute__( \
      (amdgpu_waves_per_eu(Q4 ? KVE_DECODE_WAVES_PER_EU_Q4 : KVE_DECODE_WAVES_PER_EU)))
#else
#define KVE_DECODE_ATTR __launch_bounds__(kNT)
#endif

// Cached K/V rows are read once per step: mark them streaming.
__device__ inline uint4 ld_kv(const void* p) {
#if KVE_DECODE_NT_LOADS
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return ld16(p);
#endif
}

template <int DT, int D> struct Rows {
  static constexpr int EPL = St<DT>::EPL;
  static constexpr int ES = elem_bytes<DT>();
  static constexpr int LPR = D / EPL;
  static constexpr int RPI = kNT / LPR;
  static_assert(LPR >= 4 && LPR <= 32 && kNT % LPR == 0, "row layout");
};

// 4-bit rows: half a group (16 elements, 8 code bytes) per lane; lanes 2g
// and 2g + 1 of a row share group g's scale.
template <int D> struct Q4Rows {
  static constexpr int EPL = kQGroup / 2;
  static constexpr int LPR = D / EPL;         // 4 (d 64) or 8 (d 128)
  static constexpr int RPI = kNT / LPR;
  static constexpr int CB = D / 2;            // code bytes per row
  static constexpr int G = D / kQGroup;       // scales per row
  static constexpr int RED = kNT / 16;        // row groups left after the in-row fold
  static_assert(LPR == 4 || LPR == 8, "row layout");
};

// Lane layout of the query and of the output columns for one slot format.
template <int DT, int D, bool Q4> struct Lay {
  static constexpr int EPL = Q4 ? Q4Rows<D>::EPL : Rows<DT, D>::EPL;
  static constexpr int LPR = D / EPL;
  static constexpr int NRED = Q4 ? Q4Rows<D>::RED : Rows<DT, D>::RPI;   // partial-output rows in LDS
};

// Logits scale * q.k_r for rows [r0, r1) into lg[r - r0] (LDS) and, when
// lgg is non-null, lgg[r] (global).  qf holds this lane's q elements.
template <int DT, int D, int UNR = kUnroll>
__device__ inline void row_logits(const char* Kb, const float* qf, float scale, int r0, int r1, float* lg,
                                  float* lgg) {
  using R = Rows<DT, D>;
  const int col = threadIdx.x % R::LPR, rg = threadIdx.x / R::LPR;
  for (int b = r0; b < r1; b += R::RPI * UNR) {
    uint4 raw[UNR];
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int r = b + i * R::RPI + rg;
      raw[i] = r < r1 ? ld_kv(Kb + ((size_t)r * D + col * R::EPL) * R::ES) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int r = b + i * R::RPI + rg;
      float f[R::EPL];
      St<DT>::unpack(raw[i], f);
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < R::EPL; ++j) s = fmaf(qf[j], f[j], s);
      s = group_sum<R::LPR>(s) * scale;
      if (col == 0 && r < r1) {
        lg[r - r0] = s;
        if (lgg) lgg[r] = s;
      }
    }
  }
}

// One tile of value rows b + i RPI + rg (i < UNR), zero past r1.
template <int DT, int D, int UNR>
__device__ inline void value_tile_load(const char* Vb, int b, int r1, uint4 (&raw)[UNR]) {
  using R = Rows<DT, D>;
  const int col = threadIdx.x % R::LPR, rg = threadIdx.x / R::LPR;
#pragma unroll
  for (int i = 0; i < UNR; ++i) {
    const int r = b + i * R::RPI + rg;
    raw[i] = r < r1 ? ld_kv(Vb + ((size_t)r * D + col * R::EPL) * R::ES) : make_uint4(0, 0, 0, 0);
  }
}

template <int DT, int D, int UNR>
__device__ inline void value_tile_fma(const uint4 (&raw)[UNR], const float* w, int b, int r0, int r1, float* acc) {
  using R = Rows<DT, D>;
  const int rg = threadIdx.x / R::LPR;
#pragma unroll
  for (int i = 0; i < UNR; ++i) {
    const int r = b + i * R::RPI + rg;
    const float wr = r < r1 ? w[r - r0] : 0.f;
    float f[R::EPL];
    St<DT>::unpack(raw[i], f);
#pragma unroll
    for (int j = 0; j < R::EPL; ++j) acc[j] = fmaf(wr, f[j], acc[j]);
  }
}

// acc (this lane's EPL columns) += sum over rows [r0, r1) of w[r - r0] * v_r.
// With `first`, the tile of rows from r0 is already in registers.
template <int DT, int D, int UNR = kUnroll>
__device__ inline void row_values(const char* Vb, const float* w, int r0, int r1, float* acc,
                                  const uint4 (*first)[UNR] = nullptr) {
  using R = Rows<DT, D>;
  int b = r0;
  if (first && b < r1) {
    value_tile_fma<DT, D, UNR>(*first, w, b, r0, r1, acc);
    b += R::RPI * UNR;
  }
  for (; b < r1; b += R::RPI * UNR) {
    uint4 raw[UNR];
    value_tile_load<DT, D, UNR>(Vb, b, r1, raw);
    value_tile_fma<DT, D, UNR>(raw, w, b, r0, r1, acc);
  }
}

// Dot of q with one input row of unit u, held by row group 0 (threads
// [0, D / EPL)), each lane holding EPL elements; every lane of the group
// receives the value.
template <int DT, int D, int EPL = St<DT>::EPL>
__device__ inline float group0_dot(const float* qf, const void* rows, int u) {
  constexpr int LPR = D / EPL;
  const int col = threadIdx.x % LPR;
  float f[EPL];
  load_elems<DT, EPL>((const char*)rows + ((size_t)u * D + col * EPL) * elem_bytes<DT>(), f);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) s = fmaf(qf[j], f[j], s);
  return group_sum<LPR>(s);
}

// ---------------------------------------------------------------- 4-bit rows
#ifndef KVE_DECODE_UNROLL_Q4
#define KVE_DECODE_UNROLL_Q4 1
#endif
constexpr int kUnrollQ4 = KVE_DECODE_UNROLL_Q4;

// One load tile of 4-bit rows: kUnrollQ4 rows per thread (rows b + i RPI +
// rg), their 8 code bytes and group scale, by raw buffer loads whose range
// check covers rows [0, rlast]: rows past it read as zero, so every load is
// issued unconditionally with a 32-bit offset and the compiler waits only
// for the tile being used, not for the one in flight behind it; callers
// mask those rows.  Loads carry the non-temporal hint, as the 16-bit rows'.
struct Q4Tile {
  uint2 raw[kUnrollQ4];
  float sc[kUnrollQ4];
};

__device__ inline __amdgpu_buffer_rsrc_t q4_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

template <int D>
__device__ inline void q4_load(const char* Xq, const float* Xs, int b, int rlast, Q4Tile& t) {
  using Q = Q4Rows<D>;
  constexpr int kNtAux = KVE_DECODE_NT_LOADS ? 2 : 0;   // cache policy: non-temporal
  const int col = threadIdx.x % Q::LPR, rg = threadIdx.x / Q::LPR;
  const __amdgpu_buffer_rsrc_t rq = q4_rsrc(Xq, (uint32_t)(rlast + 1) * Q::CB);
  const __amdgpu_buffer_rsrc_t rs = q4_rsrc(Xs, (uint32_t)(rlast + 1) * Q::G * 4);
#pragma unroll
  for (int i = 0; i < kUnrollQ4; ++i) {
    const int r = b + i * Q::RPI + rg;
    t.raw[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, r * Q::CB + col * 8, 0, kNtAux));
    t.sc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (r * Q::G + col / 2) * 4, 0, kNtAux));
  }
}

// Logits of one loaded tile (rows b + i RPI + rg) into lg[r - r0] and, when
// lgg is non-null, lgg[r], for r < r1.
template <int D>
__device__ inline void q4_tile_logits(const Q4Tile& t, const float* qf, float qsum, float scale, int b, int r0,
                                      int r1, float* lg, float* lgg) {
  using Q = Q4Rows<D>;
  const int col = threadIdx.x % Q::LPR, rg = threadIdx.x / Q::LPR;
#pragma unroll
  for (int i = 0; i < kUnrollQ4; ++i) {
    const int r = b + i * Q::RPI + rg;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float f[8];
      q4_nibbles(w == 0 ? t.raw[i].x : t.raw[i].y, f);
#pragma unroll
      for (int j = 0; j < 8; ++j) s = fmaf(qf[w * 8 + j], f[j], s);
    }
    s = group_sum<Q::LPR>(t.sc[i] * fmaf(-8.f, qsum, s)) * scale;
    if (col == 0 && r < r1) {
      lg[r - r0] = s;
      if (lgg) lgg[r] = s;
    }
  }
}

// Logits of 4-bit rows [r0, r1): Kq = the unit's code bytes, Ks its scales;
// qf = this lane's 16 query elements, qsum their sum.  Two register tiles in
// ping-pong: the next tile's loads are in flight while the current one is
// reduced, and every pass of the loop issues both tiles' loads, so the state
// at its back edge is the one at its entry.
template <int D>
__device__ inline void row_logits_q4(const char* Kq, const float* Ks, const float* qf, float qsum, float scale,
                                     int r0, int r1, float* lg, float* lgg) {
  constexpr int STEP = Q4Rows<D>::RPI * kUnrollQ4;
  const int rlast = max(r1 - 1, 0);
  const int ntile = r1 > r0 ? (r1 - r0 + STEP - 1) / STEP : 0;
  Q4Tile ta, tb;
  q4_load<D>(Kq, Ks, r0, rlast, ta);
  int k = 0;
  for (; k + 1 < ntile; k += 2) {
    const int b = r0 + k * STEP;
    q4_load<D>(Kq, Ks, b + STEP, rlast, tb);
    q4_tile_logits<D>(ta, qf, qsum, scale, b, r0, r1, lg, lgg);
    q4_load<D>(Kq, Ks, b + 2 * STEP, rlast, ta);   // past the range: reads as zero
    q4_tile_logits<D>(tb, qf, qsum, scale, b + STEP, r0, r1, lg, lgg);
  }
  if (k < ntile) q4_tile_logits<D>(ta, qf, qsum, scale, r0 + k * STEP, r0, r1, lg, lgg);
}

// acc += w[r - r0] * scale_r * (c + 8) over one loaded tile's rows r < r1;
// off += w[r - r0] * scale_r.
template <int D>
__device__ inline void q4_tile_values(const Q4Tile& t, const float* w, int b, int r0, int r1, float* acc,
                                      float& off) {
  using Q = Q4Rows<D>;
  const int rg = threadIdx.x / Q::LPR;
#pragma unroll
  for (int i = 0; i < kUnrollQ4; ++i) {
    const int r = b + i * Q::RPI + rg;
    const float ws = r < r1 ? w[r - r0] * t.sc[i] : 0.f;
    off += ws;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float f[8];
      q4_nibbles(k == 0 ? t.raw[i].x : t.raw[i].y, f);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[k * 8 + j] = fmaf(ws, f[j], acc[k * 8 + j]);
    }
  }
}

// acc (this lane's 16 columns) += sum over rows [r0, r1) of w[r - r0] * scale_r
// * (c + 8); off += sum of w[r - r0] * scale_r (the caller subtracts 8 * off).
// `first` is the tile of rows from r0, already loaded by the caller with
// q4_load(.., r0, max(r1 - 1, 0), ..); pipelined like row_logits_q4.
template <int D>
__device__ inline void row_values_q4(const char* Vq, const float* Vs, const float* w, int r0, int r1, float* acc,
                                     float& off, const Q4Tile& first) {
  constexpr int STEP = Q4Rows<D>::RPI * kUnrollQ4;
  const int rlast = max(r1 - 1, 0);
  const int ntile = r1 > r0 ? (r1 - r0 + STEP - 1) / STEP : 0;
  Q4Tile ta = first, tb;
  int k = 0;
  for (; k + 1 < ntile; k += 2) {
    const int b = r0 + k * STEP;
    q4_load<D>(Vq, Vs, b + STEP, rlast, tb);
    q4_tile_values<D>(ta, w, b, r0, r1, acc, off);
    q4_load<D>(Vq, Vs, b + 2 * STEP, rlast, ta);   // past the range: reads as zero
    q4_tile_values<D>(tb, w, b + STEP, r0, r1, acc, off);
  }
  if (k < ntile) q4_tile_values<D>(ta, w, r0 + k * STEP, r0, r1, acc, off);
}

// Folds the row groups of each 16-lane row (lanes with equal column, LPR
// apart) by DPP rotations, then lanes [0, LPR) of each 16-lane row store
// their 16 columns: red[tid / 16][d].
template <int D>
__device__ inline void stash_q4(float* acc, float* red) {
  using Q = Q4Rows<D>;
#pragma unroll
  for (int j = 0; j < Q::EPL; ++j) {
    float v = acc[j];
    if constexpr (Q::LPR <= 4) v = dpp_add<0x124>(v);   // row_ror:4
    v = dpp_add<0x128>(v);                               // row_ror:8
    acc[j] = v;
  }
  const int l16 = threadIdx.x % 16;
  if (l16 < Q::LPR) {
#pragma unroll
    for (int j = 0; j < Q::EPL; ++j) red[(threadIdx.x / 16) * D + l16 * Q::EPL + j] = acc[j];
  }
}

// Per-lane partial outputs -> red[rg][d]; after a barrier column i's total is
// the sum over row groups of red[g][i].
template <int DT, int D>
__device__ inline void stash_groups(const float* acc, float* red) {
  using R = Rows<DT, D>;
  const int col = threadIdx.x % R::LPR, rg = threadIdx.x / R::LPR;
#pragma unroll
  for (int j = 0; j < R::EPL; ++j) red[rg * D + col * R::EPL + j] = acc[j];
}

// What a policy step decided: the slot that receives token t (-1: none), the
// position it evicts (-1: none) and token t's score word.
struct PolicyDecision {
  int wslot;
  int evicted;
  double s_new;
};

// The policy's decision for one unit (every thread of the workgroup calls
// it): the kept slots' scores (or histories) are updated in place and the
// victim chosen.  It reads the step's weights and the slots' metadata, never
// their key or value rows, so it may run while the value pass is still to
// come; policy_write then moves token t into the chosen slot.
template <int DT, int D, bool Q4, int RND = 4>
__device__ inline PolicyDecision policy_decide(const Shape& sh, const LayerCache& c, const DecodeIO& io,
                                               const HeadMeta& m, int u, int n, const float* wts, float e_new,
                                               double L, double invL, MinKey* kscr) {
  const int tid = threadIdx.x;
  const int t = io.t;
  const size_t slot0 = (size_t)u * c.cap;
  int wslot = -1;        // slot that receives token t
  int evicted = -1;
  double s_new = 0.0;
  if (m.policy == H2O) {
    // With protected ids (a profiled composite) protected tokens carry score
    // +inf, so they are never the minimum, and only unprotected tokens count
    // against heavy + recent (npcount[u]).
    const int lim = t - m.recent;              // candidates: position <= t - recent
    const bool prot_new = m.ids != IDS_NONE && id_protected(m.ids, io.sets, io.ids[u / sh.heads]);
    // unprotected tokens kept before t: read by every thread before the
    // argmin's barriers, so thread 0's update below cannot race with it
    const int held = m.ids == IDS_NONE ? n : c.npcount[u];
    MinKey best{INFINITY, INT32_MAX, INT32_MAX};
    // RND slots per thread per round: their score/position loads are issued
    // together, so a large cache costs n / (RND NT) load latencies, not n / NT
    for (int r0 = tid; r0 < n; r0 += RND * kNT) {
      double sv[RND];
      int pv[RND];
#pragma unroll
      for (int i = 0; i < RND; ++i) {
        const int r = r0 + i * kNT;
        sv[i] = r < n ? c.S[slot0 + r] : 0.0;
        pv[i] = r < n ? c.pos[slot0 + r] : 0;
      }
#pragma unroll
      for (int i = 0; i < RND; ++i) {
        const int r = r0 + i * kNT;
        if (r < n) {
          const double s = sv[i] + (double)wts[r] * invL;
          c.S[slot0 + r] = s;
          if (pv[i] <= lim) {
            const MinKey k{s, pv[i], r};
            if (key_less(k, best)) best = k;
          }
        }
      }
    }
    s_new = prot_new ? (double)INFINITY : (double)e_new * invL;
    if (tid == 0 && t <= lim && !prot_new) {
      const MinKey k{s_new, t, n};
      if (key_less(k, best)) best = k;
    }
    best = block_argmin<kNT>(best, kscr);      // barriers inside: S[] updates done
    if (prot_new) {
      wslot = n;
    } else if (held >= m.heavy + m.recent && best.s < INFINITY) {
      if (best.slot == n) {
        evicted = t;                           // the new token itself scores lowest
      } else {
        wslot = best.slot;
        evicted = best.pos;
      }
    } else {
      wslot = n;
      if (tid == 0 && m.ids != IDS_NONE) c.npcount[u] = held + 1;
    }
  } else if (m.policy == PERSIST) {
    // history bit k = pivotal k steps ago; pivotal: weight / L >= 1 / (n + 1),
    // tested as w (n + 1) >= L in float64 (exact for equal weights)
    const int lim = t - m.recent;
    const unsigned long long wm = m.window >= 64 ? ~0ull : ((1ull << m.window) - 1ull);
    const double nA = (double)(n + 1);
    unsigned long long* Hs = reinterpret_cast<unsigned long long*>(c.S) + slot0;
    MinKey best{INFINITY, INT32_MAX, INT32_MAX};
    for (int r0 = tid; r0 < n; r0 += RND * kNT) {
      unsigned long long hv[RND];
      int pv[RND];
#pragma unroll
      for (int i = 0; i < RND; ++i) {
        const int r = r0 + i * kNT;
        hv[i] = r < n ? Hs[r] : 0ull;
        pv[i] = r < n ? c.pos[slot0 + r] : 0;
      }
#pragma unroll
      for (int i = 0; i < RND; ++i) {
        const int r = r0 + i * kNT;
        if (r < n) {
          const unsigned long long piv = (double)wts[r] * nA >= L ? 1ull : 0ull;
          const unsigned long long h = ((hv[i] << 1) | piv) & wm;
          Hs[r] = h;
          if (pv[i] <= lim) {
            const MinKey k{(double)__popcll(h), pv[i], r};
            if (key_less(k, best)) best = k;
          }
        }
      }
    }
    const unsigned long long h_new = (double)e_new * nA >= L ? 1ull : 0ull;
    s_new = __longlong_as_double((long long)h_new);
    if (tid == 0 && t <= lim) {
      const MinKey k{(double)h_new, t, n};
      if (key_less(k, best)) best = k;
    }
    best = block_argmin<kNT>(best, kscr);      // barriers inside: history updates done
    if (n >= m.heavy + m.recent) {
      if (best.slot == n) {
        evicted = t;
      } else {
        wslot = best.slot;
        evicted = best.pos;
      }
    } else {
      wslot = n;
    }
  } else if (m.policy == LOCAL) {
    if (n >= m.recent) {
      wslot = t % m.recent;                    // ring: slot of position t - W
      if (tid == 0) evicted = c.pos[slot0 + wslot];
    } else {
      wslot = n;
    }
  } else if (m.policy == FULL) {
    wslot = n;
  } else if (m.policy == SPECIAL) {
    if (id_protected(m.ids, io.sets, io.ids[u / sh.heads])) wslot = n;
    else evicted = t;
  }
  return PolicyDecision{wslot, evicted, s_new};
}

// Token t's key and value rows written into the decided slot with its score
// word, position and the unit's count; the eviction log.  Ends the step.
template <int DT, int D, bool Q4>
__device__ inline void policy_write(const Shape& sh, const LayerCache& c, const DecodeIO& io, const HeadMeta& m,
                                    int u, int n, const PolicyDecision& pd) {
  using R = Rows<DT, D>;
  const int tid = threadIdx.x;
  const int t = io.t;
  const size_t slot0 = (size_t)u * c.cap;
  const int wslot = pd.wslot;
  if (wslot >= 0) {
    __syncthreads();                           // every read of the slot is done
    if constexpr (Q4) {
      // one element per thread: threads [0, D) the key row, [D, 2D) the value
      // row (whole waves; with D = 64 the upper two waves have no element)
      constexpr int G = D / kQGroup;
      if (tid < 2 * D) {
        const bool val = tid >= D;
        const int e = tid - (val ? D : 0);
        const size_t row = slot0 + wslot;
        const float x = load_elem<DT>((const char*)(val ? io.v : io.k) + (size_t)u * D * R::ES, e);
        q4_quantize_lane(x, e, (char*)(val ? c.V : c.K) + row * (D / 2), (val ? c.Vsc : c.Ksc) + row * G);
      }
    } else {
      char* Kb = (char*)c.K + slot0 * D * R::ES;
      char* Vb = (char*)c.V + slot0 * D * R::ES;
      if (tid < R::LPR) {
        const size_t src = ((size_t)u * D + tid * R::EPL) * R::ES;
        const size_t dst = ((size_t)wslot * D + tid * R::EPL) * R::ES;
        st16(Kb + dst, ld16((const char*)io.k + src));
        st16(Vb + dst, ld16((const char*)io.v + src));
      }
    }
    if (tid == 0) {
      c.S[slot0 + wslot] = pd.s_new;
      c.pos[slot0 + wslot] = t;
      if (wslot == n) c.count[u] = n + 1;
    }
  }
  // HASH units log their replacement in the pre-attention kernel
  if (tid == 0 && io.evicted && m.policy != HASH) io.evicted[u] = pd.evicted;
}

// The head's policy after attention: H2O score update and victim, the
// persistence-count update and victim, or the positional rule; writes token
// t's key/value/score/position into its slot.  wts[r] = exp(l_r - M) for the
// n kept slots (read for H2O and PERSIST heads only), e_new = exp(l_t - M),
// L = the sum of every weight, invL = 1 / L.  Control flow is uniform over
// the workgroup; contains barriers.
template <int DT, int D, bool Q4, int RND = 4>
__device__ inline void policy_step(const Shape& sh, const LayerCache& c, const DecodeIO& io, const HeadMeta& m,
                                   int u, int n, const float* wts, float e_new, double L, double invL,
                                   MinKey* kscr) {
  const PolicyDecision pd = policy_decide<DT, D, Q4, RND>(sh, c, io, m, u, n, wts, e_new, L, invL, kscr);
  policy_write<DT, D, Q4>(sh, c, io, m, u, n, pd);
}

// ------------------------------------------------------------------ fused
// Dynamic LDS of the fused kernel: the [cap + 1] weights, then (layers with
// HASH units) the replacement's projection and rows.
__host__ __device__ constexpr size_t fused_wts_bytes(int cap) { return ((size_t)cap + 1 + 3) / 4 * 16; }

// One workgroup per unit.  HASH units first run HashEvict's pre-attention
// replacement in the same workgroup (token t takes the farthest key's slot,
// or is appended), so a step is one launch and the passes below read token t
// from its slot like every kept token.
template <int DT, int D, bool Q4, int UNR = kUnroll>
__global__ KVE_DECODE_ATTR void decode_fused_kernel(Shape sh, LayerCache c, DecodeIO io) {
  using R = Rows<DT, D>;
  using Y = Lay<DT, D, Q4>;
  extern __shared__ __attribute__((aligned(16))) float wts[];   // [cap + 1], then the replacement's LDS
  __shared__ float red[Y::NRED * D];
  __shared__ float fscr[kNT / kWave];
  __shared__ double dscr[kNT / kWave];
  __shared__ MinKey kscr[kNT / kWave];

  constexpr bool kPrio = KVE_DECODE_PRIO && !Q4 && UNR == kUnrollSmall;
  if constexpr (kPrio) __builtin_amdgcn_s_setprio(3);
  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int col = tid % Y::LPR;
  const int rg = tid / Y::LPR;
  const HeadMeta m = c.meta[u];
  int n = c.count[u];
  if (m.policy == HASH) {                        // uniform over the workgroup
    char* hl = reinterpret_cast<char*>(wts) + fused_wts_bytes(c.cap);
    switch (c.sk_bits) {
      case 16: n = hash_replace<DT, D, 16>(c, u, io.t, m.heavy, n, io.q, io.k, io.v, io.evicted, hl); break;
      case 64: n = hash_replace<DT, D, 64>(c, u, io.t, m.heavy, n, io.q, io.k, io.v, io.evicted, hl); break;
      default: n = hash_replace<DT, D, 32>(c, u, io.t, m.heavy, n, io.q, io.k, io.v, io.evicted, hl); break;
    }
  }
  const int with_new = m.policy == HASH ? 0 : 1;  // HASH: token t is now in a slot
  const size_t slot0 = (size_t)u * c.cap;
  const char* Kb = (const char*)c.K + slot0 * (Q4 ? D / 2 : D * R::ES);
  const char* Vb = (const char*)c.V + slot0 * (Q4 ? D / 2 : D * R::ES);

  float qf[Y::EPL];
  load_elems<DT, Y::EPL>((const char*)io.q + ((size_t)u * D + col * Y::EPL) * R::ES, qf);

  if constexpr (Q4) {
    float qsum = 0.f;
#pragma unroll
    for (int j = 0; j < Y::EPL; ++j) qsum += qf[j];
    row_logits_q4<D>(Kb, c.Ksc + slot0 * Q4Rows<D>::G, qf, qsum, sh.scale, 0, n, wts, nullptr);
  } else {
    row_logits<DT, D, UNR>(Kb, qf, sh.scale, 0, n, wts, nullptr);
  }
  if (with_new && rg == 0) {
    const float s = group0_dot<DT, D, Y::EPL>(qf, io.k, u) * sh.scale;
    if (col == 0) wts[n] = s;
  }
  // 4-bit rows and small caches: the value pass's first tile loads while
  // the softmax runs (a small cache's unit streams in one or two tiles, so
  // this takes a whole round trip off its chain)
  constexpr bool kVFirst = !Q4 && UNR == kUnrollSmall;
  Q4Tile vfirst;
  uint4 vraw[UNR];
  if constexpr (Q4) {
    q4_load<D>(Vb, c.Vsc + slot0 * Q4Rows<D>::G, 0, max(n - 1, 0), vfirst);
  } else if constexpr (kVFirst) {
    value_tile_load<DT, D, UNR>(Vb, 0, n, vraw);
  }
  __syncthreads();
  if constexpr (kPrio) __builtin_amdgcn_s_setprio(2);

  // softmax over the n kept slots (+ the new token)
  const int nt = n + with_new;
  float mx = -INFINITY;
  for (int r = tid; r < nt; r += kNT) mx = fmaxf(mx, wts[r]);
  mx = block_max<kNT>(mx, fscr);
  double ls = 0.0;
  for (int r = tid; r < nt; r += kNT) {
    const float w = expf(wts[r] - mx);
    wts[r] = w;
    ls += (double)w;
  }
  const double L = block_sum<kNT>(ls, dscr);     // barriers inside: wts[] complete
  const double invL = 1.0 / L;

  // The policy's decision needs only the weights and the slots' metadata.
  // A small cache takes it here, while its first value tile is still in
  // flight (at most one slot per thread: one score per round); token t's
  // rows go into their slot once the output is formed.  Larger caches
  // decide after the value pass, which measured faster for them.
  constexpr bool kDecideEarly = kVFirst && KVE_DECODE_DECIDE_EARLY;
  constexpr int kRnd = kVFirst && kSmallCache <= kNT ? 1 : 4;
  PolicyDecision pd{-1, -1, 0.0};
  if constexpr (kDecideEarly)
    pd = policy_decide<DT, D, Q4, kRnd>(sh, c, io, m, u, n, wts, with_new ? wts[n] : 0.f, L, invL, kscr);

  // output o = sum_j w_j v_j / L
  float acc[Y::EPL];
#pragma unroll
  for (int j = 0; j < Y::EPL; ++j) acc[j] = 0.f;
  if constexpr (Q4) {
    float off = 0.f;
    row_values_q4<D>(Vb, c.Vsc + slot0 * Q4Rows<D>::G, wts, 0, n, acc, off, vfirst);
#pragma unroll
    for (int j = 0; j < Y::EPL; ++j) acc[j] = fmaf(-8.f, off, acc[j]);
  } else {
    row_values<DT, D, UNR>(Vb, wts, 0, n, acc, kVFirst ? &vraw : nullptr);
  }
  if (with_new && rg == 0) {
    const float w = wts[n];
    float f[Y::EPL];
    load_elems<DT, Y::EPL>((const char*)io.v + ((size_t)u * D + col * Y::EPL) * R::ES, f);
#pragma unroll
    for (int j = 0; j < Y::EPL; ++j) acc[j] = fmaf(w, f[j], acc[j]);
  }
  if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
  if constexpr (Q4) stash_q4<D>(acc, red);
  else stash_groups<DT, D>(acc, red);
  __syncthreads();
  for (int i = tid; i < D; i += kNT) {
    float s = 0.f;
#pragma unroll 4
    for (int g = 0; g < Y::NRED; ++g) s += red[g * D + i];
    io.out[(size_t)u * D + i] = (float)((double)s * invL);
  }
  if constexpr (!kDecideEarly)
    pd = policy_decide<DT, D, Q4, kRnd>(sh, c, io, m, u, n, wts, with_new ? wts[n] : 0.f, L, invL, kscr);
  policy_write<DT, D, Q4>(sh, c, io, m, u, n, pd);
}

// ------------------------------------------------------------------ split
// One chunk [c0, c0 + chunk) of one unit's kept slots:
// part = (unnormalised output[d], chunk maximum, chunk sum of exp(l - max)).
template <int DT, int D, bool Q4>
__global__ KVE_DECODE_ATTR void decode_partial_kernel(Shape sh, LayerCache c, DecodeIO io, SplitScratch sp) {
  using R = Rows<DT, D>;
  using Y = Lay<DT, D, Q4>;
  extern __shared__ float lg[];                  // [chunk]
  __shared__ float red[Y::NRED * D];
  __shared__ float fscr[kNT / kWave];
  __shared__ double dscr[kNT / kWave];
  const int u = blockIdx.y;
  const int ch = blockIdx.x;
  const int n = c.count[u];
  const int c0 = ch * sp.chunk;
  if (c0 >= n) return;                           // uniform: the whole workgroup leaves
  const int c1 = min(n, c0 + sp.chunk);
  const int tid = threadIdx.x;
  const int col = tid % Y::LPR;
  const HeadMeta m = c.meta[u];
  const size_t slot0 = (size_t)u * c.cap;
  const char* Kb = (const char*)c.K + slot0 * (Q4 ? D / 2 : D * R::ES);
  const char* Vb = (const char*)c.V + slot0 * (Q4 ? D / 2 : D * R::ES);
  float qf[Y::EPL];
  load_elems<DT, Y::EPL>((const char*)io.q + ((size_t)u * D + col * Y::EPL) * R::ES, qf);

  const bool keep_logits = m.policy == H2O || m.policy == PERSIST;   // the combine needs every weight
  if constexpr (Q4) {
    float qsum = 0.f;
#pragma unroll
    for (int j = 0; j < Y::EPL; ++j) qsum += qf[j];
    row_logits_q4<D>(Kb, c.Ksc + slot0 * Q4Rows<D>::G, qf, qsum, sh.scale, c0, c1, lg,
                     keep_logits ? sp.logits + slot0 : nullptr);
  } else {
    row_logits<DT, D>(Kb, qf, sh.scale, c0, c1, lg, keep_logits ? sp.logits + slot0 : nullptr);
  }
  Q4Tile vfirst;
  if constexpr (Q4) q4_load<D>(Vb, c.Vsc + slot0 * Q4Rows<D>::G, c0, max(c1 - 1, 0), vfirst);
  __syncthreads();
  const int len = c1 - c0;
  float mx = -INFINITY;
  for (int r = tid; r < len; r += kNT) mx = fmaxf(mx, lg[r]);
  mx = block_max<kNT>(mx, fscr);
  double ls = 0.0;
  for (int r = tid; r < len; r += kNT) {
    const float w = expf(lg[r] - mx);
    lg[r] = w;
    ls += (double)w;
  }
  const double L = block_sum<kNT>(ls, dscr);     // barriers inside: lg[] complete
  float acc[Y::EPL];
#pragma unroll
  for (int j = 0; j < Y::EPL; ++j) acc[j] = 0.f;
  if constexpr (Q4) {
    float off = 0.f;
    row_values_q4<D>(Vb, c.Vsc + slot0 * Q4Rows<D>::G, lg, c0, c1, acc, off, vfirst);
#pragma unroll
    for (int j = 0; j < Y::EPL; ++j) acc[j] = fmaf(-8.f, off, acc[j]);
    stash_q4<D>(acc, red);
  } else {
    row_values<DT, D>(Vb, lg, c0, c1, acc);
    stash_groups<DT, D>(acc, red);
  }
  __syncthreads();
  float* part = sp.part + ((size_t)u * sp.max_chunks + ch) * (D + 2);
  for (int i = tid; i < D; i += kNT) {
    float s = 0.f;
#pragma unroll 4
    for (int g = 0; g < Y::NRED; ++g) s += red[g * D + i];
    part[i] = s;
  }
  if (tid == 0) {
    part[D] = mx;
    part[D + 1] = (float)L;
  }
}

// Merges a unit's chunks, normalises the output and runs the policy step.
// The unit's chunk partials are staged in LDS with coalesced loads first.
template <int DT, int D, bool Q4>
__global__ KVE_DECODE_ATTR void decode_combine_kernel(Shape sh, LayerCache c, DecodeIO io, SplitScratch sp) {
  using R = Rows<DT, D>;
  extern __shared__ float lds[];                 // [max_chunks * (D + 2)] partials, then [cap] weights
  __shared__ float gf[kMaxChunks];
  __shared__ double dscr[kNT / kWave];
  __shared__ MinKey kscr[kNT / kWave];
  __shared__ float snew_s;
  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int col = tid % R::LPR;
  const int rg = tid / R::LPR;
  const HeadMeta m = c.meta[u];
  const int n = c.count[u];
  const int with_new = m.policy == HASH ? 0 : 1;
  const int nch = (n + sp.chunk - 1) / sp.chunk;
  const size_t slot0 = (size_t)u * c.cap;
  float* part = lds;
  float* wts = lds + (size_t)sp.max_chunks * (D + 2);
  const float* gpart = sp.part + (size_t)u * sp.max_chunks * (D + 2);
  const int total = nch * (D + 2);
  for (int i0 = tid; i0 < total; i0 += 8 * kNT) {   // eight loads in flight per thread
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = i0 + j * kNT < total ? gpart[i0 + j * kNT] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (i0 + j * kNT < total) part[i0 + j * kNT] = v[j];
  }

  if (with_new && rg == 0) {
    float qf[R::EPL];
    St<DT>::unpack(ld16((const char*)io.q + ((size_t)u * D + col * R::EPL) * R::ES), qf);
    const float s = group0_dot<DT, D>(qf, io.k, u) * sh.scale;
    if (col == 0) snew_s = s;
  }
  __syncthreads();
  const float s_new = with_new ? snew_s : -INFINITY;
  float M = s_new;
  for (int ch = 0; ch < nch; ++ch) M = fmaxf(M, part[ch * (D + 2) + D]);
  const float e_new = with_new ? expf(s_new - M) : 0.f;
  for (int ch = tid; ch < nch; ch += kNT) gf[ch] = expf(part[ch * (D + 2) + D] - M);
  double ls = 0.0;
  if (m.policy == H2O || m.policy == PERSIST) {
    // exact weights of every kept slot, recomputed from the stored logits
    const float* lgs = sp.logits + slot0;
    // eight slots per thread per round: a 2,048-slot cache in one load latency
    for (int r0 = tid; r0 < n; r0 += 8 * kNT) {
      float lv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) lv[i] = r0 + i * kNT < n ? lgs[r0 + i * kNT] : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = r0 + i * kNT;
        if (r < n) {
          const float w = expf(lv[i] - M);
          wts[r] = w;
          ls += (double)w;
        }
      }
    }
  } else {
    for (int ch = tid; ch < nch; ch += kNT)
      ls += (double)part[ch * (D + 2) + D + 1] * (double)expf(part[ch * (D + 2) + D] - M);
  }
  const double L = block_sum<kNT>(ls, dscr) + (double)e_new;  // barriers inside: wts[], gf[] complete
  const double invL = 1.0 / L;
  for (int i = tid; i < D; i += kNT) {
    float s = 0.f;
    for (int ch = 0; ch < nch; ++ch) s = fmaf(part[ch * (D + 2) + i], gf[ch], s);
    if (with_new) {
      float f[R::EPL];
      St<DT>::unpack(ld16((const char*)io.v + ((size_t)u * D + (i / R::EPL) * R::EPL) * R::ES), f);
      s = fmaf(e_new, f[i % R::EPL], s);
    }
    io.out[(size_t)u * D + i] = (float)((double)s * invL);
  }
  policy_step<DT, D, Q4, 8>(sh, c, io, m, u, n, wts, e_new, L, invL, kscr);
}

hipError_t set_lds(const void* fn, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <int DT, int D, bool Q4>
hipError_t launch_f(const Shape& sh, const LayerCache& c, const DecodeIO& io, const SplitScratch* sp,
                    hipStream_t st) {
  if (!sp) {
    size_t lds = fused_wts_bytes(c.cap);
    if (c.sk) lds += c.sk_bits == 64 ? hash_replace_lds<D, 64>() : hash_replace_lds<D, 32>();
    // small caches: a unit's rows in fewer dependent round trips
    if (!Q4 && c.cap <= kSmallCache) {
      hipError_t e = set_lds((const void*)decode_fused_kernel<DT, D, Q4, kUnrollSmall>, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((decode_fused_kernel<DT, D, Q4, kUnrollSmall>), dim3(sh.units()), dim3(kNT), lds, st, sh,
                         c, io);
      return hipGetLastError();
    }
    hipError_t e = set_lds((const void*)decode_fused_kernel<DT, D, Q4>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_fused_kernel<DT, D, Q4>), dim3(sh.units()), dim3(kNT), lds, st, sh, c, io);
    return hipGetLastError();
  }
  const size_t lds_p = (size_t)sp->chunk * sizeof(float);
  const size_t lds_c = ((size_t)sp->max_chunks * (D + 2) + c.cap) * sizeof(float);
  hipError_t e = set_lds((const void*)decode_partial_kernel<DT, D, Q4>, lds_p);
  if (e == hipSuccess) e = set_lds((const void*)decode_combine_kernel<DT, D, Q4>, lds_c);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_partial_kernel<DT, D, Q4>), dim3(sp->max_chunks, sh.units()), dim3(kNT), lds_p, st, sh,
                     c, io, *sp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<DT, D, Q4>), dim3(sh.units()), dim3(kNT), lds_c, st, sh, c, io, *sp);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_t(const Shape& sh, const LayerCache& c, const DecodeIO& io, const SplitScratch* sp,
                    hipStream_t st) {
  return c.q4 ? launch_f<DT, D, true>(sh, c, io, sp, st) : launch_f<DT, D, false>(sh, c, io, sp, st);
}

}  // namespace

hipError_t launch_decode(const Shape& sh, const LayerCache& c, const DecodeIO& io, const SplitScratch* sp,
                         hipStream_t st) {
  if (sp && (sp->max_chunks < 1 || sp->max_chunks > kMaxChunks || sp->chunk < 1 ||
             (long long)sp->max_chunks * sp->chunk < c.cap))
    return hipErrorInvalidValue;
  switch (sh.dtype * 1000 + sh.d) {
    case F32 * 1000 + 64: return launch_t<F32, 64>(sh, c, io, sp, st);
    case F32 * 1000 + 128: return launch_t<F32, 128>(sh, c, io, sp, st);
    case F16 * 1000 + 64: return launch_t<F16, 64>(sh, c, io, sp, st);
    case F16 * 1000 + 128: return launch_t<F16, 128>(sh, c, io, sp, st);
    case BF16 * 1000 + 64: return launch_t<BF16, 64>(sh, c, io, sp, st);
    case BF16 * 1000 + 128: return launch_t<BF16, 128>(sh, c, io, sp, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve
