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
//
// The heavy threshold is found by a radix select over the float64 score bit
// patterns (scores are >= 0, so unsigned order is numeric order): eight
// 8-bit passes with an LDS histogram give the exact k-th largest value T and
// how many positions equal to T are still needed; those are taken newest
// first.  Occupied slots are [0, count) in increasing position order (LOCAL:
// ring order); the rest of the stride holds position -1 and score 0.
#include "common.hpp"

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

template <int DT, int D>
__global__ __launch_bounds__(kNT) void select_kernel(Shape sh, LayerCache c, int P, const double* colsum,
                                                     const void* k, const void* v, const int32_t* ids,
                                                     const uint32_t* keep_bitmap, int32_t vocab) {
  constexpr int EPL = St<DT>::EPL;
  constexpr int ES = elem_bytes<DT>();
  constexpr int LPR = D / EPL;
  constexpr int RPI = kNT / LPR;
  extern __shared__ int32_t kept_pos[];     // [cap]
  __shared__ uint32_t hist[256];
  __shared__ int iscr[kNT / kWave];
  __shared__ uint64_t sh_prefix;
  __shared__ int sh_want;
  __shared__ int sh_cut;

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const HeadMeta m = c.meta[u % sh.heads];
  if (m.policy == HASH) return;
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
    if (tid == 0) { sh_prefix = 0; sh_want = m.heavy; }
    // persistence counts are at most 64: only the lowest byte can differ
    for (int pass = persist ? 7 : 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      const uint64_t prefix = sh_prefix;
      const uint64_t hmask = pass == 0 ? 0ull : (~0ull << (shift + 8));   // bytes already fixed (zero when skipped)
      for (int j = tid; j < nc; j += kNT) {
        const uint64_t key = score_key(cu, j, persist);
        const bool match = (key & hmask) == (prefix & hmask);
        if (match) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int want = sh_want;
        int b = 255;
        for (; b > 0; --b) {
          if ((int)hist[b] >= want) break;
          want -= hist[b];
        }
        sh_want = want;
        sh_prefix = prefix | ((uint64_t)b << shift);
      }
      __syncthreads();
    }
    T = sh_prefix;
    // the `want` newest positions with key == T
    const int want = sh_want;
    if (tid == 0) sh_cut = 0;
    int seen = 0;
    for (int base = nc - 1; base >= 0 && seen < want; base -= kNT) {
      const int j = base - tid;
      const bool eq = j >= 0 && score_key(cu, j, persist) == T;
      int total;
      const int before = block_flag_scan(eq, &total, iscr);
      if (eq && seen + before + 1 == want) sh_cut = j;
      seen += total;
    }
    __syncthreads();
    cut = sh_cut;
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
        keep = token_kept(keep_bitmap, vocab, ids[(size_t)(u / sh.heads) * P + j]);
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
  const size_t src0 = (size_t)u * P * D * ES;
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
hipError_t select_t(const Shape& sh, const LayerCache& c, int P, const double* colsum, const void* k,
                    const void* v, const int32_t* ids, const uint32_t* keep_bitmap, int32_t vocab,
                    hipStream_t st) {
  const size_t lds = (size_t)c.cap * sizeof(int32_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel<DT, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((select_kernel<DT, D>), dim3(sh.units()), dim3(kNT), lds, st, sh, c, P, colsum, k, v, ids,
                     keep_bitmap, vocab);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_select(const Shape& sh, const LayerCache& c, int P, const double* colsum,
                                 const void* k, const void* v, const int32_t* ids,
                                 const uint32_t* keep_bitmap, int32_t vocab, hipStream_t st) {
  switch (sh.dtype * 1000 + sh.d) {
    case F32 * 1000 + 64: return select_t<F32, 64>(sh, c, P, colsum, k, v, ids, keep_bitmap, vocab, st);
    case F32 * 1000 + 128: return select_t<F32, 128>(sh, c, P, colsum, k, v, ids, keep_bitmap, vocab, st);
    case F16 * 1000 + 64: return select_t<F16, 64>(sh, c, P, colsum, k, v, ids, keep_bitmap, vocab, st);
    case F16 * 1000 + 128: return select_t<F16, 128>(sh, c, P, colsum, k, v, ids, keep_bitmap, vocab, st);
    case BF16 * 1000 + 64: return select_t<BF16, 64>(sh, c, P, colsum, k, v, ids, keep_bitmap, vocab, st);
    case BF16 * 1000 + 128: return select_t<BF16, 128>(sh, c, P, colsum, k, v, ids, keep_bitmap, vocab, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve
