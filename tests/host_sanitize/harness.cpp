// Host-side check of libkvevict's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with g++, no GPU code): the real
// kvevict.cpp (validation, workspace layout and carving, table copies, state
// machine) linked against
//   - HIP runtime stand-ins that treat "device" memory as host memory, and
//   - kernel-launcher stand-ins that check every pointer a kernel would touch
//     against the registered allocations, over the extent the kernel indexes,
//     and that a layer's arrays do not overlap.
// Prints "ok" and exits 0 when every scenario passes; any violation prints a
// message and aborts.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "kvevict.h"
#include "launch.hpp"

// ------------------------------------------------------------------ allocation registry
namespace {

struct Alloc {
  std::string name;
  const char* lo;
  const char* hi;
};
std::vector<Alloc> g_allocs;
int g_launches = 0;

void reg(const char* name, const void* p, size_t bytes) {
  g_allocs.push_back({name, (const char*)p, (const char*)p + bytes});
}
void unreg_all() { g_allocs.clear(); }

[[noreturn]] void die(const std::string& what) {
  std::fprintf(stderr, "harness: %s\n", what.c_str());
  std::fflush(stderr);
  std::abort();
}

// [p, p + bytes) lies inside one registered allocation
void in_bounds(const char* what, const void* p, size_t bytes) {
  if (bytes == 0) return;
  if (!p) die(std::string(what) + ": null pointer");
  const char* c = (const char*)p;
  for (const Alloc& a : g_allocs)
    if (c >= a.lo && c + bytes <= a.hi) return;
  die(std::string(what) + ": " + std::to_string(bytes) + " bytes outside every allocation");
}

struct Span {
  const char* name;
  const char* lo;
  const char* hi;
};

void disjoint(const std::vector<Span>& v) {
  for (size_t i = 0; i < v.size(); ++i)
    for (size_t j = i + 1; j < v.size(); ++j)
      if (v[i].lo < v[j].hi && v[j].lo < v[i].hi && v[i].lo != v[i].hi && v[j].lo != v[j].hi)
        die(std::string("overlap: ") + v[i].name + " and " + v[j].name);
}

size_t es(const kve::Shape& sh) { return sh.dtype == kve::F32 ? 4 : 2; }

// Every array of one layer's cache, at the extents the kernels index.
void check_cache(const kve::Shape& sh, const kve::LayerCache& c) {
  const size_t U = sh.units(), cap = c.cap, d = sh.d;
  if (cap < 1) die("layer stride < 1");
  const size_t row = c.q4 ? d / 2 : d * es(sh);
  std::vector<Span> s;
  auto add = [&](const char* n, const void* p, size_t b) {
    in_bounds(n, p, b);
    s.push_back({n, (const char*)p, (const char*)p + b});
  };
  add("K", c.K, U * cap * row);
  add("V", c.V, U * cap * row);
  if (c.q4) {
    add("Ksc", c.Ksc, U * cap * (d / 32) * 4);
    add("Vsc", c.Vsc, U * cap * (d / 32) * 4);
  }
  add("S", c.S, U * cap * 8);
  add("pos", c.pos, U * cap * 4);
  if (c.sk) add("sk", c.sk, U * cap * (c.sk_bits == 64 ? 8 : 4));
  add("count", c.count, U * 4);
  add("npcount", c.npcount, U * 4);
  add("meta", c.meta, U * sizeof(kve::HeadMeta));
  disjoint(s);
  if (c.proj) in_bounds("proj", c.proj, d * (size_t)c.sk_bits * 2);
}

void check_units(kve::UnitList ul, int U) {
  if (ul.n < 0 || ul.n > U) die("unit list size");
  if (ul.ids) in_bounds("unit list", ul.ids, (size_t)ul.n * 4);
}

}  // namespace

// ------------------------------------------------------------------ HIP runtime stand-ins
extern "C" {
hipError_t hipMemcpy(void* dst, const void* src, size_t bytes, hipMemcpyKind) {
  in_bounds("hipMemcpy dst", dst, bytes);
  if (bytes) std::memcpy(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  in_bounds("hipMemcpyAsync dst", dst, bytes);
  in_bounds("hipMemcpyAsync src", src, bytes);
  if (bytes) std::memmove(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipMemcpy2DAsync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                            hipMemcpyKind, hipStream_t) {
  for (size_t r = 0; r < height; ++r) {
    in_bounds("hipMemcpy2DAsync dst", (char*)dst + r * dpitch, width);
    in_bounds("hipMemcpy2DAsync src", (const char*)src + r * spitch, width);
    std::memmove((char*)dst + r * dpitch, (const char*)src + r * spitch, width);
  }
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipGetLastError() { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stand-in"; }
}

// ------------------------------------------------------------------ kernel-launcher stand-ins
namespace kve {

static char g_static_scratch[1 << 20];
size_t static_scratch_bytes() { return sizeof g_static_scratch; }
hipError_t static_scratch_address(void** out) {
  *out = g_static_scratch;
  return hipSuccess;
}

hipError_t launch_prefill_rowstats_valu(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                        const void* v, float* lse, float* out, hipStream_t) {
  const size_t U = sh.units(), b = U * P * sh.d * es(sh);
  check_units(ul, (int)U);
  in_bounds("q", q, b);
  in_bounds("k", k, b);
  in_bounds("lse", lse, U * P * 8);
  if (out) {
    in_bounds("v", v, b);
    in_bounds("out", out, U * P * sh.d * 4);
  }
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefill_colsum_valu(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                      const float* lse, double* colsum, hipStream_t) {
  const size_t U = sh.units(), b = U * P * sh.d * es(sh);
  check_units(ul, (int)U);
  in_bounds("q", q, b);
  in_bounds("k", k, b);
  in_bounds("lse", lse, U * P * 8);
  in_bounds("colsum", colsum, U * P * 8);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefill_rowstats_mfma(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                        float* lse, int q_from, hipStream_t) {
  if (q_from < 0 || q_from >= P) die("rowstats q_from");
  return launch_prefill_rowstats_valu(sh, P, ul, q, k, nullptr, lse, nullptr, nullptr);
}
hipError_t launch_prefill_attend_mfma(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                      const void* v, float* lse, float* out, hipStream_t) {
  return launch_prefill_rowstats_valu(sh, P, ul, q, k, v, lse, out, nullptr);
}
hipError_t launch_prefill_colsum_mfma(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                      const float* lse, double* colsum, hipStream_t st) {
  return launch_prefill_colsum_valu(sh, P, ul, q, k, lse, colsum, st);
}
hipError_t launch_prefill_persist_mfma(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                       const float* lse, const HeadMeta* meta, double* bits, hipStream_t st) {
  in_bounds("meta", meta, sh.units() * sizeof(HeadMeta));
  return launch_prefill_colsum_valu(sh, P, ul, q, k, lse, bits, st);
}
hipError_t launch_prefill_persist_valu(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                       const float* lse, const HeadMeta* meta, double* bits, hipStream_t st) {
  return launch_prefill_persist_mfma(sh, P, ul, q, k, lse, meta, bits, st);
}
hipError_t launch_prefill_colsum_mass_mfma(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                           const float* lse, double* colsum, float* mass, int rows,
                                           hipStream_t st) {
  if (rows < 1 || rows > P) die("profiled rows");
  in_bounds("mass", mass, sh.units() * P * 4);
  return launch_prefill_colsum_valu(sh, P, ul, q, k, lse, colsum, st);
}
hipError_t launch_prefill_colsum_mass_valu(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                           const float* lse, double* colsum, float* mass, int rows,
                                           hipStream_t st) {
  return launch_prefill_colsum_mass_mfma(sh, P, ul, q, k, lse, colsum, mass, rows, st);
}
hipError_t launch_prefill_select(const Shape& sh, const LayerCache& c, int P, const double* colsum, const void* k,
                                 const void* v, const int32_t* ids, const IdSets& sets, hipStream_t) {
  const size_t U = sh.units();
  check_cache(sh, c);
  in_bounds("colsum", colsum, U * P * 8);
  in_bounds("k", k, U * P * sh.d * es(sh));
  in_bounds("v", v, U * P * sh.d * es(sh));
  if (ids) in_bounds("ids", ids, (size_t)sh.batch * P * 4);
  const size_t words = ((size_t)sets.vocab + 31) / 32 * 4;
  if (sets.keep) in_bounds("keep bitmap", sets.keep, words);
  if (sets.special) in_bounds("special bitmap", sets.special, words);
  if (sets.punct) in_bounds("punct bitmap", sets.punct, words);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefill_adaptive(const Shape& sh, const LayerCache& c, UnitList ul, int P, const double* colsum,
                                   const float* mass, const Profile& pf, const void* k, const void* v,
                                   const int32_t* ids, const IdSets& sets, hipStream_t st) {
  check_units(ul, sh.units());
  in_bounds("mass", mass, sh.units() * P * 4);
  if (pf.rows < 1 || pf.rows > P) die("profile rows");
  return launch_prefill_select(sh, c, P, colsum, k, v, ids, sets, st);
}
hipError_t launch_sketch_rows(const Shape& sh, UnitList ul, const void* x, int P, int row0, int nrows,
                              const uint16_t* proj, int bits, void* out, hipStream_t) {
  const size_t U = sh.units();
  check_units(ul, (int)U);
  if (row0 < 0 || nrows < 0 || row0 + nrows > P) die("sketch rows");
  in_bounds("x", x, U * P * sh.d * es(sh));
  in_bounds("proj", proj, (size_t)sh.d * bits * 2);
  in_bounds("sketches", out, U * P * (bits == 64 ? 8 : 4));
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_hash_prefill(const Shape& sh, const LayerCache& c, UnitList ul, int P, int max_budget,
                               const void* qsk, const void* ksk, const void* k, const void* v, hipStream_t) {
  const size_t U = sh.units(), w = c.sk_bits == 64 ? 8 : 4;
  check_cache(sh, c);
  check_units(ul, (int)U);
  if (max_budget < 1 || max_budget > c.cap) die("hash budget");
  in_bounds("qsk", qsk, U * P * w);
  in_bounds("ksk", ksk, U * P * w);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_hash_evict(const Shape& sh, const LayerCache& c, UnitList ul, int, const void* q, const void* k,
                             const void* v, int32_t* evicted, hipStream_t) {
  const size_t U = sh.units();
  check_cache(sh, c);
  check_units(ul, (int)U);
  in_bounds("q", q, U * sh.d * es(sh));
  in_bounds("k", k, U * sh.d * es(sh));
  in_bounds("v", v, U * sh.d * es(sh));
  if (evicted) in_bounds("evicted", evicted, U * 4);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode(const Shape& sh, const LayerCache& c, const DecodeIO& io, const SplitScratch* sp,
                         hipStream_t) {
  const size_t U = sh.units();
  check_cache(sh, c);
  in_bounds("q", io.q, U * sh.d * es(sh));
  in_bounds("k", io.k, U * sh.d * es(sh));
  in_bounds("v", io.v, U * sh.d * es(sh));
  in_bounds("out", io.out, U * sh.d * 4);
  if (io.evicted) in_bounds("evicted", io.evicted, U * 4);
  if (io.ids) in_bounds("token id", io.ids, (size_t)sh.batch * 4);
  if (sp) {
    if (sp->max_chunks < 1 || sp->max_chunks > kMaxChunks || (long long)sp->max_chunks * sp->chunk < c.cap)
      die("split shape");
    in_bounds("partials", sp->part, U * sp->max_chunks * (sh.d + 2) * 4);
    in_bounds("logits", sp->logits, U * (size_t)c.cap * 4);
  }
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t) {
  in_bounds("stream_read src", src, bytes);
  in_bounds("stream_read sink", sink, 4);
  ++g_launches;
  return hipSuccess;
}

}  // namespace kve

// ------------------------------------------------------------------ scenarios
namespace {

void expect(bool ok, const char* what) {
  if (!ok) die(std::string("expectation failed: ") + what);
}

// --short-input: the prompt's q buffer is registered 16 bytes short, so the
// checks must stop the run (the harness's own self-check).
bool g_short_input = false;

struct Buf {
  std::vector<char> v;
  Buf(const char* name, size_t bytes) : v(bytes ? bytes : 1, 0) {
    reg(name, v.data(), g_short_input && std::strcmp(name, "q") == 0 && bytes > 16 ? bytes - 16 : bytes);
  }
  void* p() { return v.data(); }
};

struct Scenario {
  const char* name;
  int layers, batch, heads, d, N, dtype, P, steps;
  std::vector<int32_t> policy, heavy, recent, history;
  int bits, cache_bits;
};

void run(const Scenario& s) {
  unreg_all();
  {
    void* ss = nullptr;
    (void)kve::static_scratch_address(&ss);
    reg("static scratch", ss, kve::static_scratch_bytes());
  }
  const int H = s.heads, L = s.layers, U = s.batch * H;
  const int vocab = 64;
  std::vector<uint32_t> keep((vocab + 31) / 32, 0x0000000Fu), special((vocab + 31) / 32, 0x3u),
      punct((vocab + 31) / 32, 0xCu);
  std::vector<uint16_t> proj((size_t)L * s.d * (s.bits ? s.bits : 32), 0x3f80);
  kve_config c{};
  c.layers = L;
  c.batch = s.batch;
  c.heads = H;
  c.head_dim = s.d;
  c.max_context = s.N;
  c.dtype = s.dtype;
  c.policy = s.policy.data();
  c.heavy = s.heavy.data();
  c.recent = s.recent.data();
  c.vocab = vocab;
  c.keep_token_bitmap = keep.data();
  c.sketch_bits = s.bits;
  c.lsh_proj_bf16 = s.bits ? proj.data() : nullptr;
  c.history = s.history.empty() ? nullptr : s.history.data();
  c.special_token_bitmap = special.data();
  c.punct_token_bitmap = punct.data();
  c.profile_rows = 8;
  c.profile_threshold = 0.95f;
  c.cache_bits = s.cache_bits;
  size_t bytes = 0;
  expect(kvevict_workspace_size(&c, &bytes) == KVE_OK, s.name);
  // a 256-byte aligned "device" workspace, exactly the size asked for
  std::vector<char> raw(bytes + 256);
  char* ws = raw.data() + (256 - (uintptr_t)raw.data() % 256) % 256;
  reg("workspace", ws, bytes);
  kve_handle h = nullptr;
  expect(kvevict_create(&c, ws, bytes - 256, &h) == KVE_ENOMEM || bytes < 256, "short workspace rejected");
  expect(kvevict_create(&c, ws, bytes, &h) == KVE_OK && h, s.name);
  const size_t E = s.dtype == KVE_F32 ? 4 : 2;
  Buf q("q", (size_t)U * s.P * s.d * E), k("k", (size_t)U * s.P * s.d * E), v("v", (size_t)U * s.P * s.d * E);
  Buf ids("ids", (size_t)s.batch * s.P * 4), out("prompt out", (size_t)U * s.P * s.d * 4);
  Buf dq("dq", (size_t)U * s.d * E), dk("dk", (size_t)U * s.d * E), dv("dv", (size_t)U * s.d * E);
  Buf did("decode ids", (size_t)s.batch * 4), dout("decode out", (size_t)U * s.d * 4), ev("evicted", (size_t)U * 4);
  for (int l = 0; l < L; ++l) {
    const int cap = kvevict_capacity(h, l);
    expect(cap >= 1, "capacity");
    expect(kvevict_decode_step(h, l, dq.p(), dk.p(), dv.p(), (int32_t*)did.p(), (float*)dout.p(), nullptr, nullptr) ==
               KVE_ESTATE, "decode before prefill");
    expect(kvevict_prefill(h, l, s.P, q.p(), k.p(), v.p(), (int32_t*)ids.p(), nullptr, nullptr) == KVE_OK, "prefill");
    expect(kvevict_prefill(h, l, s.P, q.p(), k.p(), v.p(), (int32_t*)ids.p(), (float*)out.p(), nullptr) == KVE_OK,
           "prefill with output");
    expect(kvevict_position(h, l) == s.P, "position after prefill");
    for (int t = 0; t < s.steps; ++t) {
      const bool na = t % 2 == 1;
      kve_status st = na ? kvevict_decode_step_noalloc(h, l, dq.p(), dk.p(), dv.p(), (int32_t*)did.p(),
                                                       (float*)dout.p(), (int32_t*)ev.p(), nullptr)
                         : kvevict_decode_step(h, l, dq.p(), dk.p(), dv.p(), (int32_t*)did.p(), (float*)dout.p(),
                                               (int32_t*)ev.p(), nullptr);
      expect(st == KVE_OK || (na && st == KVE_EUNSUPPORTED), "decode step");
    }
    Buf pos("pos out", (size_t)U * cap * 4), cnt("count out", (size_t)U * 4), sc("scores out", (size_t)U * cap * 8);
    expect(kvevict_kept_indices(h, l, (int32_t*)pos.p(), (int32_t*)cnt.p(), (double*)sc.p(), nullptr) == KVE_OK,
           "kept indices");
    const size_t row = s.cache_bits == 4 ? s.d / 2 : s.d * E;
    Buf ko("k rows", (size_t)U * cap * row), vo("v rows", (size_t)U * cap * row);
    Buf kso("k scales", (size_t)U * cap * (s.d / 32) * 4), vso("v scales", (size_t)U * cap * (s.d / 32) * 4);
    expect(kvevict_cache_rows(h, l, ko.p(), vo.p(), (float*)kso.p(), (float*)vso.p(), nullptr) == KVE_OK,
           "cache rows");
    Buf ch("choices", (size_t)U * 4);
    expect(kvevict_unit_policies(h, l, (int32_t*)ch.p(), nullptr) == KVE_OK, "unit policies");
  }
  // out-of-range and null arguments are rejected before anything is touched
  expect(kvevict_prefill(h, L, s.P, q.p(), k.p(), v.p(), nullptr, nullptr, nullptr) == KVE_EINVAL, "layer range");
  expect(kvevict_prefill(h, 0, s.N + 1, q.p(), k.p(), v.p(), nullptr, nullptr, nullptr) == KVE_EINVAL, "prompt range");
  expect(kvevict_decode_step(h, 0, nullptr, dk.p(), dv.p(), nullptr, (float*)dout.p(), nullptr, nullptr) ==
             KVE_EINVAL, "null q");
  expect(kvevict_kept_indices(h, 0, nullptr, nullptr, nullptr, nullptr) == KVE_EINVAL, "null outputs");
  expect(kvevict_capacity(h, -1) == -1 && kvevict_position(h, L) == -1, "bookkeeping range");
  expect(kvevict_destroy(h) == KVE_OK, "destroy");
  std::printf("scenario %-28s workspace %10zu B, launches so far %d\n", s.name, bytes, g_launches);
}

std::vector<int32_t> rep(std::vector<int32_t> v, int layers) {
  std::vector<int32_t> r;
  for (int l = 0; l < layers; ++l) r.insert(r.end(), v.begin(), v.end());
  return r;
}

}  // namespace

int main(int argc, char** argv) {
  g_short_input = argc > 1 && std::strcmp(argv[1], "--short-input") == 0;
  const int F32 = KVE_F32, F16 = KVE_F16, BF16 = KVE_BF16;
  std::vector<Scenario> all = {
      {"h2o bf16 fused", 2, 2, 3, 128, 300, BF16, 200, 5, rep({1, 1, 1}, 2), rep({30, 20, 10}, 2), rep({20, 20, 5}, 2),
       {}, 0, 0},
      {"h2o fp32 d64 split", 1, 1, 2, 64, 2600, F32, 1500, 4, {1, 1}, {1100, 900}, {200, 150}, {}, 0, 0},
      {"fastgen mixed split", 1, 2, 4, 128, 1400, BF16, 1300, 4, {0, 1, 2, 3}, {0, 50, 0, 0}, {0, 100, 120, 0}, {}, 0,
       0},
      {"hash 16 fused", 1, 2, 2, 128, 400, BF16, 300, 3, {4, 4}, {100, 120}, {0, 0}, {}, 16, 0},
      {"hash 32 split", 1, 1, 3, 128, 2400, F16, 2100, 3, {4, 4, 4}, {2048, 1500, 1100}, {0, 0, 0}, {}, 32, 0},
      {"hash 64 q4 fused", 1, 2, 2, 128, 600, BF16, 500, 3, {4, 4}, {256, 300}, {0, 0}, {}, 64, 4},
      {"persist + h2o", 2, 1, 2, 128, 300, BF16, 250, 3, rep({5, 1}, 2), rep({40, 30}, 2), rep({20, 10}, 2),
       rep({16, 0}, 2), 0, 0},
      {"profiled split", 1, 2, 2, 128, 1200, BF16, 1100, 3, {6, 6}, {40, 40}, {60, 60}, {}, 0, 0},
      {"h2o q4", 1, 1, 4, 128, 500, BF16, 400, 3, {1, 1, 1, 1}, {50, 40, 30, 20}, {10, 10, 10, 10}, {}, 0, 4},
  };
  for (const Scenario& s : all) run(s);
  // invalid configurations: validation returns an error and reads nothing it should not
  kve_config c{};
  size_t b = 0;
  expect(kvevict_workspace_size(nullptr, &b) == KVE_EINVAL, "null config");
  expect(kvevict_workspace_size(&c, &b) == KVE_EINVAL, "zero sizes");
  std::vector<int32_t> pol = {1, 9}, hv = {3, 3}, rc = {2, 2};
  c.layers = 1;
  c.batch = 1;
  c.heads = 2;
  c.head_dim = 128;
  c.max_context = 100;
  c.dtype = BF16;
  c.policy = pol.data();
  c.heavy = hv.data();
  c.recent = rc.data();
  expect(kvevict_workspace_size(&c, &b) == KVE_EINVAL, "unknown policy");
  pol[1] = 4;
  expect(kvevict_workspace_size(&c, &b) != KVE_OK, "hash without projection");
  pol[1] = 1;
  c.head_dim = 96;
  expect(kvevict_workspace_size(&c, &b) == KVE_EUNSUPPORTED, "head_dim");
  c.head_dim = 128;
  c.cache_bits = 3;
  expect(kvevict_workspace_size(&c, &b) == KVE_EUNSUPPORTED, "cache bits");
  std::printf("ok\n");
  return 0;
}
