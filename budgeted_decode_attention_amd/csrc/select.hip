// Prefill selection: which prompt positions each unit keeps, and the gather
// of their keys/values into the unit's slots.  One workgroup per unit.
//
//   H2O      [P - r, P) plus the `heavy` positions of [0, P - r) with the
//            largest column score; on equal scores the newer position wins
//            (H2O review page, proposed method: greedy on accumulated
//            attention; motivation: recency balanced against relevance).
//   LOCAL    [P - W, P), position j in slot j mod W (FastGen review page).
//   FULL     [0, P).
//   SPECIAL  positions whose token id is in the keep bitmap (FastGen page).
//   PERSIST  as H2O with the rank key = the persistence count (set bits of
//            the token's 64-bit pivotal history, Scissorhands persistence
//            reading); the slot keeps the history bits themselves.
//   HASH     skipped here (prompt replay kernel).
//   profiled units (ADAPTIVE heads): adaptive_kernel below.
//
// The heavy threshold is found by a radix select over the float64 score bit
// patterns (scores are >= 0, so unsigned order is numeric order): eight
// 8-bit passes with an LDS histogram give the exact k-th largest value T and
// how many positions equal to T are still needed; those are taken newest
// first.  Occupied slots are [0, count) in increasing position order (LOCAL:
// ring order); the rest of the stride holds position -1 and score 0.
#include "common.hpp"
#include "q4.hpp"

namespace kve {
namespace {

constexpr int kNT = 256;

// Exclusive prefix of a 0/1 flag over the workgroup in thread order; *total
// receives the number of set flags.  Contains barriers.
__device__ inline int block_flag_scan(bool flag, int* total, int* scratch) {
  const uint64_t b = __ballot(flag);
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) scratch[w] = __popcll(b);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kNT / kWave; ++i) {
    if (i < w) before += scratch[i];
    all += scratch[i];
  }
  __syncthreads();
  *total = all;
  return before + in_wave;
}

// Rank key of prompt position j: the float64 score bits (H2O) or the number
// of set history bits (PERSIST); larger keys rank higher either way.
__device__ inline uint64_t score_key(const double* c, int j, bool count) {
  const uint64_t b = (uint64_t)__double_as_longlong(c[j]);
  return count ? (uint64_t)__popcll(b) : b;
}

// LDS state of one radix selection.
struct RadixLds {
  uint32_t hist[256];
  int iscr[kNT / kWave];
  uint64_t prefix;
  int want;
  int cut;
};

// The `want` largest keys among positions j in [0, nc) with cand(j), the
// newer first on equal keys: on return j is selected iff cand(j) and
// (key > T or (key == T and j >= cut)).  want must not exceed the number of
// candidates.  Eight 8-bit passes over the key bits (first_pass > 0 when
// the higher bytes are known to be zero); uniform control flow, barriers.
template <class Key, class Cand>
__device__ inline void radix_top(int nc, int want, int first_pass, Key key, Cand cand, RadixLds& r, uint64_t& T,
                                 int& cut) {
  const int tid = threadIdx.x;
  if (tid == 0) { r.prefix = 0; r.want = want; }
  for (int pass = first_pass; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    r.hist[tid] = 0;
    __syncthreads();
    const uint64_t prefix = r.prefix;
    const uint64_t hmask = pass == 0 ? 0ull : (~0ull << (shift + 8));   // bytes already fixed (zero when skipped)
    for (int j = tid; j < nc; j += kNT) {
      if (!cand(j)) continue;
      const uint64_t kv = key(j);
      if ((kv & hmask) == (prefix & hmask)) atomicAdd(&r.hist[(kv >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int w = r.want;
      int b = 255;
      for (; b > 0; --b) {
        if ((int)r.hist[b] >= w) break;
        w -= r.hist[b];
      }
      r.want = w;
      r.prefix = prefix | ((uint64_t)b << shift);
    }
    __syncthreads();
  }
  T = r.prefix;
  // the `want` newest candidates with key == T
  const int w = r.want;
  if (tid == 0) r.cut = 0;
  int seen = 0;
  for (int base = nc - 1; base >= 0 && seen < w; base -= kNT) {
    const int j = base - tid;
    const bool eq = j >= 0 && cand(j) && key(j) == T;
    int total;
    const int before = block_flag_scan(eq, &total, r.iscr);
    if (eq && seen + before + 1 == w) r.cut = j;
    seen += total;
  }
  __syncthreads();
  cut = r.cut;
}

// Gathers the K/V rows of kept_pos[0, count) into the unit's slots; a layer
// of 4-bit slots quantises them on the way (one lane per group of 32).
template <int DT, int D>
__device__ inline void gather_rows(const LayerCache& c, int u, int P, const int32_t* kept_pos, int count,
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
    char* Kd = (char*)c.K + slot0 * (D / 2);
    char* Vd = (char*)c.V + slot0 * (D / 2);
    const int g = tid % G;
    for (int s = tid / G; s < count; s += kNT / G) {
      const size_t so = src0 + (size_t)kept_pos[s] * D * ES;
      q4_store_group<DT, D>((const char*)k + so, Kd + (size_t)s * (D / 2), c.Ksc + (slot0 + s) * G, g);
      q4_store_group<DT, D>((const char*)v + so, Vd + (size_t)s * (D / 2), c.Vsc + (slot0 + s) * G, g);
    }
    return;
  }
  char* Kd = (char*)c.K + slot0 * D * ES;
  char* Vd = (char*)c.V + slot0 * D * ES;
  const int col = tid % LPR;
  for (int s = tid / LPR; s < count; s += RPI) {
    const size_t so = ((size_t)kept_pos[s] * D + col * EPL) * ES;
    const size_t dof = ((size_t)s * D + col * EPL) * ES;
    st16(Kd + dof, ld16((const char*)k + src0 + so));
    st16(Vd + dof, ld16((const char*)v + src0 + so));
  }
}

template <int DT, int D>
__global__ __launch_bounds__(kNT) void select_kernel(Shape sh, LayerCache c, int P, const double* colsum,
                                                     const void* k, const void* v, const int32_t* ids,
                                                     IdSets sets) {
  extern __shared__ int32_t kept_pos[];     // [cap]
  __shared__ RadixLds rl;
  __shared__ int iscr[kNT / kWave];

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const HeadMeta m = c.meta[u];
  if (m.policy == HASH || m.policy == ADAPTIVE || m.choice != 0) return;   // replay / profiled units
  const size_t slot0 = (size_t)u * c.cap;
  const double* cu = colsum ? colsum + (size_t)u * P : nullptr;

  // ---- heavy threshold (H2O and PERSIST heads)
  const bool persist = m.policy == PERSIST;
  const bool h2o = m.policy == H2O || persist;
  const int B = m.heavy + m.recent;
  const bool select_heavy = h2o && P > B && m.heavy > 0;
  const int nc = h2o ? P - m.recent : 0;    // candidate positions [0, nc)
  uint64_t T = 0;
  int cut = 0;                              // ties with key == T kept iff position >= cut
  if (select_heavy) {
    // persistence counts are at most 64: only the lowest byte can differ
    radix_top(nc, m.heavy, persist ? 7 : 0, [&](int j) { return score_key(cu, j, persist); },
              [](int) { return true; }, rl, T, cut);
  }

  // ---- kept flags and compaction into slots [0, count)
  int count = 0;
  for (int j0 = 0; j0 < P; j0 += kNT) {
    const int j = j0 + tid;
    bool keep = false;
    if (j < P) {
      if (m.policy == FULL) {
        keep = true;
      } else if (m.policy == LOCAL) {
        keep = j >= P - m.recent;
      } else if (m.policy == SPECIAL) {
        keep = id_protected(m.ids, sets, ids[(size_t)(u / sh.heads) * P + j]);
      } else if (h2o) {
        if (P <= B || j >= nc) {
          keep = true;
        } else if (select_heavy) {
          const uint64_t key = score_key(cu, j, persist);
          keep = key > T || (key == T && j >= cut);
        }
      }
    }
    int total;
    const int before = block_flag_scan(keep, &total, iscr);
    if (keep) {
      const int slot = (m.policy == LOCAL) ? (j % m.recent) : count + before;
      kept_pos[slot] = j;
      c.pos[slot0 + slot] = j;
      c.S[slot0 + slot] = h2o ? cu[j] : 0.0;
    }
    count += total;
  }
  for (int s = count + tid; s < c.cap; s += kNT) {
    c.pos[slot0 + s] = -1;
    c.S[slot0 + s] = 0.0;
  }
  if (tid == 0) c.count[u] = count;
  __syncthreads();

  // ---- gather K/V rows of the kept positions
  gather_rows<DT, D>(c, u, P, kept_pos, count, k, v);
}

// ------------------------------------------------------------------ profiled units
// FastGen review page, proposed method: a lightweight profile of the prompt's
// attention picks each head's policy, the composites being tried greedily in
// the order special -> punctuation -> frequent -> local, with the full cache
// last.  Per unit: the share a composite recovers is the mass the last R
// prompt rows give to its end-of-prompt kept set (mass[u][j] holds that mass
// per key, so a share is a sum over the set divided by R); the first share
// reaching the threshold picks the composite, which then fills the cache and
// becomes the unit's policy.  Protected tokens (special or punctuation ids)
// carry score +inf in the frequent composites, so they are never evicted.
template <int DT, int D>
__global__ __launch_bounds__(kNT) void adaptive_kernel(Shape sh, LayerCache c, UnitList ul, int P,
                                                       const double* colsum, const float* mass, Profile pf,
                                                       const void* k, const void* v, const int32_t* ids,
                                                       IdSets sets) {
  extern __shared__ int32_t kept_pos[];     // [cap]
  __shared__ RadixLds rl;
  __shared__ int iscr[kNT / kWave];
  __shared__ double dscr[kNT / kWave];
  const int u = ul.ids ? ul.ids[blockIdx.x] : blockIdx.x;
  const int tid = threadIdx.x;
  const size_t slot0 = (size_t)u * c.cap;
  const double* cu = colsum + (size_t)u * P;
  const float* mu = mass + (size_t)u * P;
  const int32_t* idu = ids + (size_t)(u / sh.heads) * P;
  const int R = min(pf.rows, P);
  const int hh = pf.heavy, W = pf.recent;
  const double thr = (double)pf.threshold;
  auto special = [&](int j) { return token_kept(sets.special, sets.vocab, idu[j]); };
  auto prot = [&](int j) { return special(j) || token_kept(sets.punct, sets.vocab, idu[j]); };
  auto key = [&](int j) { return (uint64_t)__double_as_longlong(cu[j]); };
  auto free_ = [&](int j) { return !prot(j); };

  // masses of the id sets, of the whole prompt and of the unprotected window
  double m1 = 0.0, m2 = 0.0, mall = 0.0, mwin = 0.0, nfree = 0.0, wfree = 0.0;
  for (int j = tid; j < P; j += kNT) {
    const double x = (double)mu[j];
    const bool s1 = special(j), s2 = s1 || token_kept(sets.punct, sets.vocab, idu[j]);
    mall += x;
    if (s1) m1 += x;
    if (s2) {
      m2 += x;
    } else {
      nfree += 1.0;
      if (j >= P - W) {
        wfree += 1.0;
        mwin += x;
      }
    }
  }
  m1 = block_sum<kNT>(m1, dscr);
  m2 = block_sum<kNT>(m2, dscr);
  mall = block_sum<kNT>(mall, dscr);
  mwin = block_sum<kNT>(mwin, dscr);
  const int nf = (int)block_sum<kNT>(nfree, dscr);
  const int wf = (int)block_sum<kNT>(wfree, dscr);

  const double inv = 1.0 / R;
  int choice = 5;
  uint64_t T3 = 0, T4 = 0;
  int cut3 = 0, cut4 = 0;
  const bool all3 = nf <= hh, all4 = nf <= hh + W;   // the prompt fits the unprotected budget
  const int quota4 = hh + W - wf;                    // older unprotected slots of the local composite
  if (m1 * inv >= thr) {
    choice = 1;
  } else if (m2 * inv >= thr) {
    choice = 2;
  } else {
    double rec3 = mall * inv;
    if (!all3) {
      if (hh > 0) radix_top(P, hh, 0, key, free_, rl, T3, cut3);
      double sel = 0.0;
      for (int j = tid; j < P; j += kNT)
        if (hh > 0 && free_(j) && (key(j) > T3 || (key(j) == T3 && j >= cut3))) sel += (double)mu[j];
      rec3 = (m2 + block_sum<kNT>(sel, dscr)) * inv;
    }
    if (rec3 >= thr) {
      choice = 3;
    } else {
      double rec4 = mall * inv;
      if (!all4) {
        const int nc = P - W;
        if (quota4 > 0) radix_top(nc, quota4, 0, key, free_, rl, T4, cut4);
        double sel = 0.0;
        for (int j = tid; j < nc; j += kNT)
          if (quota4 > 0 && free_(j) && (key(j) > T4 || (key(j) == T4 && j >= cut4))) sel += (double)mu[j];
        rec4 = (m2 + mwin + block_sum<kNT>(sel, dscr)) * inv;
      }
      if (rec4 >= thr) choice = 4;
    }
  }

  // ---- the chosen composite's kept set, compacted into slots [0, count)
  int count = 0;
  double nfk = 0.0;                                  // unprotected tokens kept (frequent composites)
  for (int j0 = 0; j0 < P; j0 += kNT) {
    const int j = j0 + tid;
    bool keep = false, pj = false;
    if (j < P) {
      pj = prot(j);
      switch (choice) {
        case 1: keep = special(j); break;
        case 2: keep = pj; break;
        case 3: keep = pj || all3 || (hh > 0 && (key(j) > T3 || (key(j) == T3 && j >= cut3))); break;
        case 4:
          keep = pj || all4 || j >= P - W ||
                 (quota4 > 0 && (key(j) > T4 || (key(j) == T4 && j >= cut4)));
          break;
        default: keep = true;
      }
    }
    int total;
    const int before = block_flag_scan(keep, &total, iscr);
    if (keep) {
      const int slot = count + before;
      kept_pos[slot] = j;
      c.pos[slot0 + slot] = j;
      c.S[slot0 + slot] = (choice == 3 || choice == 4) ? (pj ? (double)INFINITY : cu[j]) : 0.0;
      if (!pj) nfk += 1.0;
    }
    count += total;
  }
  nfk = block_sum<kNT>(nfk, dscr);
  for (int s = count + tid; s < c.cap; s += kNT) {
    c.pos[slot0 + s] = -1;
    c.S[slot0 + s] = 0.0;
  }
  if (tid == 0) {
    c.count[u] = count;
    c.npcount[u] = (int)nfk;
    HeadMeta m{FULL, 0, 0, c.cap, 0, IDS_NONE, choice};
    if (choice == 1) { m.policy = SPECIAL; m.ids = IDS_SPECIAL; }
    if (choice == 2) { m.policy = SPECIAL; m.ids = IDS_SPECIAL_PUNCT; }
    if (choice == 3) { m.policy = H2O; m.ids = IDS_SPECIAL_PUNCT; m.heavy = hh; }
    if (choice == 4) { m.policy = H2O; m.ids = IDS_SPECIAL_PUNCT; m.heavy = hh; m.recent = W; }
    c.meta[u] = m;
  }
  __syncthreads();
  gather_rows<DT, D>(c, u, P, kept_pos, count, k, v);
}

template <int DT, int D>
hipError_t adaptive_t(const Shape& sh, const LayerCache& c, UnitList ul, int P, const double* colsum,
                      const float* mass, const Profile& pf, const void* k, const void* v, const int32_t* ids,
                      const IdSets& sets, hipStream_t st) {
  const size_t lds = (size_t)c.cap * sizeof(int32_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)adaptive_kernel<DT, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((adaptive_kernel<DT, D>), dim3(ul.n), dim3(kNT), lds, st, sh, c, ul, P, colsum, mass, pf, k, v,
                     ids, sets);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t select_t(const Shape& sh, const LayerCache& c, int P, const double* colsum, const void* k,
                    const void* v, const int32_t* ids, const IdSets& sets, hipStream_t st) {
  const size_t lds = (size_t)c.cap * sizeof(int32_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel<DT, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((select_kernel<DT, D>), dim3(sh.units()), dim3(kNT), lds, st, sh, c, P, colsum, k, v, ids,
                     sets);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_select(const Shape& sh, const LayerCache& c, int P, const double* colsum,
                                 const void* k, const void* v, const int32_t* ids, const IdSets& sets,
                                 hipStream_t st) {
  switch (sh.dtype * 1000 + sh.d) {
    case F32 * 1000 + 64: return select_t<F32, 64>(sh, c, P, colsum, k, v, ids, sets, st);
    case F32 * 1000 + 128: return select_t<F32, 128>(sh, c, P, colsum, k, v, ids, sets, st);
    case F16 * 1000 + 64: return select_t<F16, 64>(sh, c, P, colsum, k, v, ids, sets, st);
    case F16 * 1000 + 128: return select_t<F16, 128>(sh, c, P, colsum, k, v, ids, sets, st);
    case BF16 * 1000 + 64: return select_t<BF16, 64>(sh, c, P, colsum, k, v, ids, sets, st);
    case BF16 * 1000 + 128: return select_t<BF16, 128>(sh, c, P, colsum, k, v, ids, sets, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve

namespace kve {

hipError_t launch_prefill_adaptive(const Shape& sh, const LayerCache& c, UnitList ul, int P, const double* colsum,
                                   const float* mass, const Profile& pf, const void* k, const void* v,
                                   const int32_t* ids, const IdSets& sets, hipStream_t st) {
  if (ul.n <= 0) return hipSuccess;
  if (!colsum || !mass || !ids || pf.rows < 1) return hipErrorInvalidValue;
  switch (sh.dtype * 1000 + sh.d) {
    case F32 * 1000 + 64: return adaptive_t<F32, 64>(sh, c, ul, P, colsum, mass, pf, k, v, ids, sets, st);
    case F32 * 1000 + 128: return adaptive_t<F32, 128>(sh, c, ul, P, colsum, mass, pf, k, v, ids, sets, st);
    case F16 * 1000 + 64: return adaptive_t<F16, 64>(sh, c, ul, P, colsum, mass, pf, k, v, ids, sets, st);
    case F16 * 1000 + 128: return adaptive_t<F16, 128>(sh, c, ul, P, colsum, mass, pf, k, v, ids, sets, st);
    case BF16 * 1000 + 64: return adaptive_t<BF16, 64>(sh, c, ul, P, colsum, mass, pf, k, v, ids, sets, st);
    case BF16 * 1000 + 128: return adaptive_t<BF16, 128>(sh, c, ul, P, colsum, mass, pf, k, v, ids, sets, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve
