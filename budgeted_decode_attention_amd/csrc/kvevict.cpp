// libkvevict host side: argument validation, workspace layout, per-layer
// state and kernel dispatch behind the C ABI declared in include/kvevict.h.
//
// The library allocates no device memory.  Everything lives in the caller's
// workspace, carved in a fixed order by Plan below; kvevict_workspace_size and
// kvevict_create run the same plan so their layouts always agree.
#include "kvevict.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

kve_status fail(kve_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kve_status fail(kve_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

constexpr int kMaxContext = 32768;     // LDS-resident per-unit slot lists
// Layers whose slot stride exceeds kSplitAbove use the split decode.  Chunk
// size: a layer whose heads all share one capacity splits each unit in about
// two (half the capacity rounded up to 256, at least 512: fewer partials to
// merge), in about four with 4-bit slots; a layer with mixed capacities, or
// whose units fill the stride to different counts (profiled and special-id
// heads), uses 256-slot chunks so units of very different sizes balance
// across the GPU.  Both can be overridden at create
// time through the environment (KVEVICT_SPLIT_ABOVE, KVEVICT_SPLIT_CHUNK) to
// exercise either path at any size.
constexpr int kSplitAbove = 1024;
constexpr int kSplitChunkMixed = 256;
constexpr size_t kMaxSplitLds = 150 * 1024;
// The replay keeps every slot's sketch and position in LDS: 8 bytes per slot
// with 16- and 32-bit sketches, 12 with 64-bit ones.
constexpr int kMaxHashBudget = 16384;
constexpr int kMaxHashBudget64 = 12288;

int sketch_word_bytes(int bits) { return bits == 64 ? 8 : 4; }
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  char* end = nullptr;
  const long x = std::strtol(v, &end, 10);
  return (end && *end == 0 && x >= 0 && x <= (1 << 30)) ? (int)x : dflt;
}

struct SplitPolicy {
  int above;
  int chunk;   // 0: chosen per layer
};

SplitPolicy split_policy() {
  SplitPolicy p{env_int("KVEVICT_SPLIT_ABOVE", kSplitAbove), env_int("KVEVICT_SPLIT_CHUNK", 0)};
  if (p.chunk != 0 && p.chunk < 16) p.chunk = 0;
  return p;
}

int layer_chunk(const SplitPolicy& sp, int cap, int head_dim, bool uniform, bool q4) {
  if (sp.chunk) return sp.chunk;
  // 4-bit slots carry a third of the bytes: four chunks per unit fill the GPU
  int chunk = uniform ? std::max(512, (cap / (q4 ? 4 : 2) + 255) / 256 * 256) : kSplitChunkMixed;
  // grow it (256 slots at a time) until a unit's chunks fit the combine
  // kernel: at most kMaxChunks partials, and the partials plus one weight per
  // slot within kMaxSplitLds.  Growth stops at a single chunk, which fits
  // every capacity up to kMaxContext; the caller rejects whatever does not fit.
  auto fits = [&](int ch) {
    const size_t nch = (size_t)(cap + ch - 1) / ch;
    return nch <= (size_t)kve::kMaxChunks && (nch * (head_dim + 2) + cap) * 4 <= kMaxSplitLds;
  };
  while (chunk < cap && !fits(chunk)) chunk += 256;
  return chunk;
}


int elem_size(int dtype) { return dtype == KVE_F32 ? 4 : 2; }

int head_capacity(int policy, int heavy, int recent, int max_context) {
  switch (policy) {
    case KVE_H2O:
    case KVE_PERSIST: return heavy + recent;
    case KVE_LOCAL: return recent;
    case KVE_HASH: return heavy;
    default: return max_context;       // FULL, SPECIAL, ADAPTIVE (protected tokens accumulate)
  }
}

// Per-layer summary of the head table.
struct LayerInfo {
  int cap = 0;
  bool split = false;
  bool uniform = true;   // every head of the layer has the same capacity
  int chunk = 0;         // split-decode chunk (slots)
  int nch = 0;           // chunks per unit
  bool any_h2o = false, any_hash = false, any_special = false, any_persist = false, any_adaptive = false;
  int max_hash_budget = 0;
  int min_hash_budget = 0;   // smallest HASH budget of the layer (0: none)
  int max_window = 0;    // largest history window of the layer's PERSIST heads
  int ad_heavy = -1, ad_recent = -1;   // the layer's ADAPTIVE heads' frequent slots and local window
  std::vector<int32_t> h2o_units, hash_units, persist_units, adaptive_units;
};

kve_status validate(const kve_config* c, std::vector<LayerInfo>* info) {
  if (!c) return fail(KVE_EINVAL, "config is null");
  if (c->layers < 1 || c->batch < 1 || c->heads < 1)
    return fail(KVE_EINVAL, "layers, batch and heads must be >= 1");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(KVE_EUNSUPPORTED, "head_dim %d not built (64 or 128)", c->head_dim);
  if (c->dtype != KVE_F32 && c->dtype != KVE_F16 && c->dtype != KVE_BF16)
    return fail(KVE_EINVAL, "dtype %d unknown", c->dtype);
  if (c->max_context < 1 || c->max_context > kMaxContext)
    return fail(KVE_EUNSUPPORTED, "max_context %d outside [1, %d]", c->max_context, kMaxContext);
  if (!(c->softmax_scale >= 0.f) || !std::isfinite(c->softmax_scale))
    return fail(KVE_EINVAL, "softmax_scale must be finite and >= 0");
  if (!c->policy || !c->heavy || !c->recent) return fail(KVE_EINVAL, "policy/heavy/recent tables are null");
  const long long units = (long long)c->batch * c->heads;
  if (units > (1 << 24)) return fail(KVE_EUNSUPPORTED, "more than 2^24 units per layer");
  info->assign(c->layers, LayerInfo());
  bool need_bitmap = false, need_proj = false, need_ids_tables = false;
  for (int l = 0; l < c->layers; ++l) {
    LayerInfo& li = (*info)[l];
    for (int h = 0; h < c->heads; ++h) {
      const int i = l * c->heads + h;
      const int p = c->policy[i], hv = c->heavy[i], rc = c->recent[i];
      switch (p) {
        case KVE_H2O:
          if (hv < 0 || rc < 0 || hv + rc < 1)
            return fail(KVE_EINVAL, "layer %d head %d: H2O needs heavy, recent >= 0 and heavy + recent >= 1", l, h);
          if (hv + rc > c->max_context)
            return fail(KVE_EINVAL, "layer %d head %d: heavy + recent exceeds max_context", l, h);
          li.any_h2o = true;
          break;
        case KVE_PERSIST: {
          if (hv < 0 || rc < 0 || hv + rc < 1)
            return fail(KVE_EINVAL, "layer %d head %d: PERSIST needs heavy, recent >= 0 and heavy + recent >= 1", l,
                        h);
          if (hv + rc > c->max_context)
            return fail(KVE_EINVAL, "layer %d head %d: heavy + recent exceeds max_context", l, h);
          if (!c->history) return fail(KVE_EINVAL, "PERSIST heads need the history table");
          const int w = c->history[i];
          if (w < 1 || w > 64)
            return fail(KVE_EINVAL, "layer %d head %d: history window %d outside [1, 64]", l, h, w);
          li.any_persist = true;
          li.max_window = std::max(li.max_window, w);
          break;
        }
        case KVE_LOCAL:
          if (hv != 0 || rc < 1 || rc > c->max_context)
            return fail(KVE_EINVAL, "layer %d head %d: LOCAL needs heavy = 0 and 1 <= recent <= max_context", l, h);
          break;
        case KVE_HASH:
          if (rc != 0 || hv < 1 ||
              hv > std::min(c->max_context, c->sketch_bits == 64 ? kMaxHashBudget64 : kMaxHashBudget))
            return fail(KVE_EINVAL, "layer %d head %d: HASH needs recent = 0 and 1 <= budget <= %d", l, h,
                        std::min(c->max_context, c->sketch_bits == 64 ? kMaxHashBudget64 : kMaxHashBudget));
          li.any_hash = true;
          li.max_hash_budget = std::max(li.max_hash_budget, hv);
          li.min_hash_budget = li.min_hash_budget ? std::min(li.min_hash_budget, hv) : hv;
          need_proj = true;
          break;
        case KVE_ADAPTIVE:
          if (hv < 0 || rc < 0 || hv + rc > c->max_context)
            return fail(KVE_EINVAL, "layer %d head %d: ADAPTIVE needs 0 <= heavy, recent and heavy + recent <= "
                        "max_context", l, h);
          if (li.ad_heavy >= 0 && (hv != li.ad_heavy || rc != li.ad_recent))
            return fail(KVE_EUNSUPPORTED, "layer %d: ADAPTIVE heads of one layer must share heavy and recent", l);
          li.ad_heavy = hv;
          li.ad_recent = rc;
          li.any_adaptive = true;
          need_ids_tables = true;
          break;
        case KVE_FULL:
        case KVE_SPECIAL:
          if (hv != 0 || rc != 0)
            return fail(KVE_EINVAL, "layer %d head %d: FULL/SPECIAL take heavy = recent = 0", l, h);
          if (p == KVE_SPECIAL) {
            li.any_special = true;
            need_bitmap = true;
          }
          break;
        default:
          return fail(KVE_EINVAL, "layer %d head %d: policy %d unknown", l, h, p);
      }
      const int hc = head_capacity(p, hv, rc, c->max_context);
      if (h > 0 && hc != li.cap) li.uniform = false;
      // profiled and special-id units fill their common stride to very
      // different counts (chosen composite, token ids): balance them as a
      // layer of mixed capacities
      if (p == KVE_ADAPTIVE || p == KVE_SPECIAL) li.uniform = false;
      li.cap = std::max(li.cap, hc);
    }
    for (int b = 0; b < c->batch; ++b)
      for (int h = 0; h < c->heads; ++h) {
        const int p = c->policy[l * c->heads + h];
        if (p == KVE_H2O) li.h2o_units.push_back(b * c->heads + h);
        if (p == KVE_HASH) li.hash_units.push_back(b * c->heads + h);
        if (p == KVE_PERSIST) li.persist_units.push_back(b * c->heads + h);
        if (p == KVE_ADAPTIVE) li.adaptive_units.push_back(b * c->heads + h);
      }
  }
  const SplitPolicy sp = split_policy();
  for (int l = 0; l < c->layers; ++l) {
    LayerInfo& li = (*info)[l];
    li.split = li.cap > sp.above;
    if (!li.split) continue;
    li.chunk = layer_chunk(sp, li.cap, c->head_dim, li.uniform, c->cache_bits == 4);
    li.nch = (li.cap + li.chunk - 1) / li.chunk;
    if (li.nch > kve::kMaxChunks)
      return fail(KVE_EUNSUPPORTED, "layer %d: %d slots need more than %d chunks of %d", l, li.cap,
                  kve::kMaxChunks, li.chunk);
    // the combine kernel holds a unit's chunk partials and weights in LDS
    if (((size_t)li.nch * (c->head_dim + 2) + li.cap) * 4 > kMaxSplitLds)
      return fail(KVE_EUNSUPPORTED, "layer %d: %d slots exceed the split decode's LDS", l, li.cap);
  }
  if (need_bitmap && (!c->keep_token_bitmap || c->vocab < 1))
    return fail(KVE_EINVAL, "SPECIAL heads need keep_token_bitmap and vocab >= 1");
  if (need_proj && (!c->lsh_proj_bf16 || (c->sketch_bits != 16 && c->sketch_bits != 32 && c->sketch_bits != 64)))
    return fail(KVE_EUNSUPPORTED, "HASH heads need lsh_proj_bf16 and sketch_bits of 16, 32 or 64");
  if (c->cache_bits != 0 && c->cache_bits != 4)
    return fail(KVE_EUNSUPPORTED, "cache_bits %d not built (0 or 4)", c->cache_bits);
  if (c->cache_bits == 4)
    for (int i = 0; i < c->layers * c->heads; ++i)
      if (c->policy[i] != KVE_H2O && c->policy[i] != KVE_PERSIST && c->policy[i] != KVE_HASH)
        return fail(KVE_EUNSUPPORTED, "layer %d head %d: 4-bit slots are built for H2O, PERSIST and HASH heads only",
                    i / c->heads, i % c->heads);
  if (need_ids_tables) {
    if (!c->special_token_bitmap || !c->punct_token_bitmap || c->vocab < 1)
      return fail(KVE_EINVAL, "ADAPTIVE heads need special_token_bitmap, punct_token_bitmap and vocab >= 1");
    if (c->profile_rows < 1 || !std::isfinite(c->profile_threshold))
      return fail(KVE_EINVAL, "ADAPTIVE heads need profile_rows >= 1 and a finite profile_threshold");
  }
  return KVE_OK;
}

// Workspace layout.  With base == nullptr only sizes are accumulated.
struct Plan {
  char* base;
  size_t off = 0;
  explicit Plan(void* b) : base((char*)b) {}
  template <class T> T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + count * sizeof(T));
    return p;
  }
};

struct Layer {
  kve::LayerCache cache{};
  kve::SplitScratch split{};   // chunk == 0: fused path
  LayerInfo info;
  kve::UnitList h2o{nullptr, 0}, hash{nullptr, 0}, persist{nullptr, 0}, adaptive{nullptr, 0};
  int position = -1;   // next decode position; -1 before prefill
};

}  // namespace

struct kve_ctx {
  kve_config cfg{};
  kve::Shape shape{};
  std::vector<Layer> layers;
  kve::HeadMeta* meta = nullptr;       // device [layers][U]
  uint32_t* bitmap = nullptr;          // device keep set (SPECIAL heads)
  uint32_t* special = nullptr;         // device special / punctuation sets (ADAPTIVE heads)
  uint32_t* punct = nullptr;
  float* mass = nullptr;               // device [U][max_context] (ADAPTIVE layers): the profile
  uint16_t* proj = nullptr;            // device [layers][d][32]
  float* lse = nullptr;                // device [U][max_context][2]
  double* colsum = nullptr;            // device [U][max_context]
  void* qsk = nullptr;                 // device [U][max_context] sketch words
  void* ksk = nullptr;
  void* static_scratch = nullptr;      // device address of the per-GPU static scratch (null: unavailable)
  bool sync_check = false;

  kve::IdSets sets() const { return {bitmap, special, punct, cfg.vocab}; }
};


namespace {

size_t layout(const kve_config* c, const std::vector<LayerInfo>& info, void* base, kve_ctx* ctx) {
  Plan pl(base);
    const size_t U = (size_t)c->batch * c->heads;
  const size_t d = c->head_dim, es = elem_size(c->dtype);
  const size_t N = c->max_context;
  bool any_hash = false, any_special = false, any_adaptive = false;
  for (const auto& li : info) {
    any_hash |= li.any_hash;
    any_special |= li.any_special;
    any_adaptive |= li.any_adaptive;
  }
  const size_t words = ((size_t)c->vocab + 31) / 32;
  auto* meta = pl.take<kve::HeadMeta>((size_t)c->layers * U);
  auto* bitmap = any_special ? pl.take<uint32_t>(words) : nullptr;
  auto* special = any_adaptive ? pl.take<uint32_t>(words) : nullptr;
  auto* punct = any_adaptive ? pl.take<uint32_t>(words) : nullptr;
  auto* mass = any_adaptive ? pl.take<float>(U * N) : nullptr;
  const size_t bits = c->sketch_bits, swb = sketch_word_bytes(c->sketch_bits);
  auto* proj = any_hash ? pl.take<uint16_t>((size_t)c->layers * d * bits) : nullptr;
  auto* lse = pl.take<float>(U * N * 2);
  auto* colsum = pl.take<double>(U * N);
  void* qsk = any_hash ? (void*)pl.take<char>(U * N * swb) : nullptr;
  void* ksk = any_hash ? (void*)pl.take<char>(U * N * swb) : nullptr;
  // split-decode scratch, sized for the largest split layer
  size_t split_cap = 0, split_nch = 0;
  for (const auto& li : info)
    if (li.split) {
      split_cap = std::max(split_cap, (size_t)li.cap);
      split_nch = std::max(split_nch, (size_t)li.nch);
    }
  float* part = split_cap ? pl.take<float>(U * split_nch * (d + 2)) : nullptr;
  float* logits = split_cap ? pl.take<float>(U * split_cap) : nullptr;
  if (ctx) {
    ctx->meta = meta;
    ctx->bitmap = bitmap;
    ctx->special = special;
    ctx->punct = punct;
    ctx->mass = mass;
    ctx->proj = proj;
    ctx->lse = lse;
    ctx->colsum = colsum;
    ctx->qsk = qsk;
    ctx->ksk = ksk;
  }
  for (int l = 0; l < c->layers; ++l) {
    const LayerInfo& li = info[l];
    const size_t cap = li.cap;
    kve::LayerCache lc{};
    const bool q4 = c->cache_bits == 4;
    const size_t row_bytes = q4 ? d / 2 : d * es;   // 4-bit slots: two codes per byte
    lc.K = pl.take<char>(U * cap * row_bytes);
    lc.V = pl.take<char>(U * cap * row_bytes);
    lc.Ksc = q4 ? pl.take<float>(U * cap * (d / 32)) : nullptr;
    lc.Vsc = q4 ? pl.take<float>(U * cap * (d / 32)) : nullptr;
    lc.q4 = q4 ? 1 : 0;
    lc.S = pl.take<double>(U * cap);
    lc.pos = pl.take<int32_t>(U * cap);
    lc.sk = li.any_hash ? (void*)pl.take<char>(U * cap * swb) : nullptr;
    lc.sk_bits = c->sketch_bits;
    lc.count = pl.take<int32_t>(U);
    lc.npcount = pl.take<int32_t>(U);
    lc.meta = meta ? meta + (size_t)l * U : nullptr;
    lc.proj = proj ? proj + (size_t)l * d * bits : nullptr;
    lc.cap = (int32_t)cap;
    int32_t* h2o_ids = li.h2o_units.empty() ? nullptr : pl.take<int32_t>(li.h2o_units.size());
    int32_t* hash_ids = li.hash_units.empty() ? nullptr : pl.take<int32_t>(li.hash_units.size());
    int32_t* persist_ids = li.persist_units.empty() ? nullptr : pl.take<int32_t>(li.persist_units.size());
    int32_t* adaptive_ids = li.adaptive_units.empty() ? nullptr : pl.take<int32_t>(li.adaptive_units.size());
    if (ctx) {
      Layer& L = ctx->layers[l];
      L.cache = lc;
      if (li.split) L.split = {part, logits, li.chunk, li.nch};
      L.info = li;
      L.h2o = {h2o_ids, (int32_t)li.h2o_units.size()};
      L.hash = {hash_ids, (int32_t)li.hash_units.size()};
      L.persist = {persist_ids, (int32_t)li.persist_units.size()};
      L.adaptive = {adaptive_ids, (int32_t)li.adaptive_units.size()};
    }
  }
  return pl.off;
}

kve_status dev(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVE_OK;
  return fail(KVE_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

kve_status check_layer(kve_handle h, int32_t layer) {
  if (!h) return fail(KVE_EINVAL, "handle is null");
  if (layer < 0 || layer >= h->cfg.layers) return fail(KVE_EINVAL, "layer %d out of range", layer);
  return KVE_OK;
}

kve_status finish(kve_handle h, hipStream_t st, const char* what) {
  kve_status s = dev(hipGetLastError(), what);
  if (s != KVE_OK) return s;
  if (h->sync_check) {
    s = dev(hipStreamSynchronize(st), what);
    if (s != KVE_OK) return s;
    s = dev(hipGetLastError(), what);
  }
  return s;
}

// One decode step; `scratch` overrides where the split decode keeps its
// partials and logits (null: the workspace's region).
kve_status decode_step_impl(kve_handle h, int32_t layer, const void* q, const void* k, const void* v,
                            const int32_t* token_ids, float* out, int32_t* evicted_pos, void* stream,
                            const kve::SplitScratch* scratch, const char* what) {
  kve_status s = check_layer(h, layer);
  if (s != KVE_OK) return s;
  Layer& L = h->layers[layer];
  if (L.position < 0) return fail(KVE_ESTATE, "layer %d: decode before prefill", layer);
  if (L.position >= h->cfg.max_context)
    return fail(KVE_ESTATE, "layer %d: position %d reached max_context", layer, L.position);
  if (!q || !k || !v || !out) return fail(KVE_EINVAL, "q, k, v and out are required");
  if ((L.info.any_special || L.info.any_adaptive) && !token_ids)
    return fail(KVE_EINVAL, "token_ids required (layer has SPECIAL or ADAPTIVE heads)");
  hipStream_t st = (hipStream_t)stream;
  const kve::Shape& sh = h->shape;
  hipError_t e = hipSuccess;
  // HASH units: the pre-attention replacement runs as its own launch before
  // the split decode; the fused decode runs it inside each unit's workgroup
  if (L.hash.n && L.split.chunk) e = kve::launch_hash_evict(sh, L.cache, L.hash, L.position, q, k, v, evicted_pos, st);
  if (e == hipSuccess) {
    const kve::DecodeIO io{q, k, v, token_ids, h->sets(), out, evicted_pos, L.position};
    const kve::SplitScratch* sp = L.split.chunk ? (scratch ? scratch : &L.split) : nullptr;
    e = kve::launch_decode(sh, L.cache, io, sp, st);
  }
  if (e != hipSuccess) return dev(e, "decode launch");
  s = finish(h, st, what);
  if (s == KVE_OK) L.position += 1;
  return s;
}

}  // namespace

extern "C" {

kve_status kvevict_workspace_size(const kve_config* cfg, size_t* bytes) {
  if (!bytes) return fail(KVE_EINVAL, "bytes is null");
  std::vector<LayerInfo> info;
  kve_status s = validate(cfg, &info);
  if (s != KVE_OK) return s;
  *bytes = layout(cfg, info, nullptr, nullptr);
  return KVE_OK;
}

kve_status kvevict_create(const kve_config* cfg, void* d_workspace, size_t bytes, kve_handle* out) {
  if (!out) return fail(KVE_EINVAL, "out is null");
  *out = nullptr;
  std::vector<LayerInfo> info;
  kve_status s = validate(cfg, &info);
  if (s != KVE_OK) return s;
  if (!d_workspace) return fail(KVE_EINVAL, "workspace is null");
  if ((uintptr_t)d_workspace % kAlign) return fail(KVE_EINVAL, "workspace is not 256-byte aligned");
  const size_t need = layout(cfg, info, nullptr, nullptr);
  if (bytes < need) return fail(KVE_ENOMEM, "workspace has %zu bytes, needs %zu", bytes, need);

  kve_ctx* ctx = new (std::nothrow) kve_ctx();
  if (!ctx) return fail(KVE_ENOMEM, "host allocation failed");
  ctx->cfg = *cfg;
  ctx->cfg.policy = ctx->cfg.heavy = ctx->cfg.recent = nullptr;
  ctx->cfg.keep_token_bitmap = nullptr;
  ctx->cfg.lsh_proj_bf16 = nullptr;
  ctx->cfg.history = nullptr;
  ctx->cfg.special_token_bitmap = ctx->cfg.punct_token_bitmap = nullptr;
  const float scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / std::sqrt((float)cfg->head_dim);
  ctx->shape = {cfg->batch, cfg->heads, cfg->head_dim, cfg->dtype, scale};
  ctx->layers.resize(cfg->layers);
  layout(cfg, info, d_workspace, ctx);
  const char* env = std::getenv("KVEVICT_SYNC_CHECK");
  ctx->sync_check = env && env[0] == '1';

  // tables to the device
  // one record per unit: units of a head share the head's entry (profiled
  // units get theirs at prefill)
  const size_t U = (size_t)cfg->batch * cfg->heads;
  std::vector<kve::HeadMeta> meta((size_t)cfg->layers * U);
  for (int l = 0; l < cfg->layers; ++l)
    for (size_t u = 0; u < U; ++u) {
      const size_t i = (size_t)l * cfg->heads + u % cfg->heads;
      const int p = cfg->policy[i], hv = cfg->heavy[i], rc = cfg->recent[i];
      const int w = p == KVE_PERSIST ? cfg->history[i] : 0;
      const int ids = p == KVE_SPECIAL ? kve::IDS_KEEP : kve::IDS_NONE;
      meta[(size_t)l * U + u] = {p, hv, rc, head_capacity(p, hv, rc, cfg->max_context), w, ids, 0};
    }
  s = dev(hipMemcpy(ctx->meta, meta.data(), meta.size() * sizeof(kve::HeadMeta), hipMemcpyHostToDevice),
          "copy head table");
  if (s == KVE_OK && ctx->bitmap)
    s = dev(hipMemcpy(ctx->bitmap, cfg->keep_token_bitmap, ((size_t)cfg->vocab + 31) / 32 * 4,
                      hipMemcpyHostToDevice), "copy keep bitmap");
  if (s == KVE_OK && ctx->special)
    s = dev(hipMemcpy(ctx->special, cfg->special_token_bitmap, ((size_t)cfg->vocab + 31) / 32 * 4,
                      hipMemcpyHostToDevice), "copy special bitmap");
  if (s == KVE_OK && ctx->punct)
    s = dev(hipMemcpy(ctx->punct, cfg->punct_token_bitmap, ((size_t)cfg->vocab + 31) / 32 * 4,
                      hipMemcpyHostToDevice), "copy punctuation bitmap");
  if (s == KVE_OK && ctx->proj)
    s = dev(hipMemcpy(ctx->proj, cfg->lsh_proj_bf16, (size_t)cfg->layers * cfg->head_dim * cfg->sketch_bits * 2,
                      hipMemcpyHostToDevice), "copy projection");
  for (int l = 0; l < cfg->layers && s == KVE_OK; ++l) {
    Layer& L = ctx->layers[l];
    if (L.h2o.n)
      s = dev(hipMemcpy((void*)L.h2o.ids, L.info.h2o_units.data(), L.h2o.n * 4, hipMemcpyHostToDevice),
              "copy unit list");
    if (s == KVE_OK && L.hash.n)
      s = dev(hipMemcpy((void*)L.hash.ids, L.info.hash_units.data(), L.hash.n * 4, hipMemcpyHostToDevice),
              "copy unit list");
    if (s == KVE_OK && L.persist.n)
      s = dev(hipMemcpy((void*)L.persist.ids, L.info.persist_units.data(), L.persist.n * 4,
                        hipMemcpyHostToDevice), "copy unit list");
    if (s == KVE_OK && L.adaptive.n)
      s = dev(hipMemcpy((void*)L.adaptive.ids, L.info.adaptive_units.data(), L.adaptive.n * 4,
                        hipMemcpyHostToDevice), "copy unit list");
  }
  if (s != KVE_OK) {
    delete ctx;
    return s;
  }
  // the static scratch of the allocation-free decode entry point, on the
  // device current at create (where the workspace lives); looked up once per
  // device.  A failure only disables that entry point, so the error state it
  // leaves is cleared here rather than reported by a later call.
  if (kve::static_scratch_address(&ctx->static_scratch) != hipSuccess) {
    ctx->static_scratch = nullptr;
    (void)hipGetLastError();
  }
  *out = ctx;
  return KVE_OK;
}

kve_status kvevict_destroy(kve_handle h) {
  if (!h) return fail(KVE_EINVAL, "handle is null");
  delete h;
  return KVE_OK;
}

kve_status kvevict_prefill(kve_handle h, int32_t layer, int32_t P, const void* q, const void* k, const void* v,
                           const int32_t* token_ids, float* out, void* stream) {
  kve_status s = check_layer(h, layer);
  if (s != KVE_OK) return s;
  if (P < 1 || P > h->cfg.max_context)
    return fail(KVE_EINVAL, "prompt_len %d outside [1, %d]", P, h->cfg.max_context);
  if (!q || !k || !v) return fail(KVE_EINVAL, "q, k and v are required");
  Layer& L = h->layers[layer];
  if ((L.info.any_special || L.info.any_adaptive) && !token_ids)
    return fail(KVE_EINVAL, "token_ids required (layer has SPECIAL or ADAPTIVE heads)");
  hipStream_t st = (hipStream_t)stream;
  const kve::Shape& sh = h->shape;
  hipError_t e = hipSuccess;
  // Scores (H2O heads): row statistics, then column sums.  Pivotal histories
  // (PERSIST heads): row statistics of the last `window` rows, then their
  // bits.  16-bit inputs use the matrix-core kernels, fp32 inputs the
  // vector-ALU ones.  The optional prompt output covers every unit and writes
  // the row statistics with it.
  const kve::UnitList all{nullptr, sh.units()};
  const bool mfma = sh.dtype != KVE_F32;
  if (out) {
    e = mfma ? kve::launch_prefill_attend_mfma(sh, P, all, q, k, v, h->lse, out, st)
             : kve::launch_prefill_rowstats_valu(sh, P, all, q, k, v, h->lse, out, st);
  } else {
    if (L.h2o.n)
      e = mfma ? kve::launch_prefill_rowstats_mfma(sh, P, L.h2o, q, k, h->lse, 0, st)
               : kve::launch_prefill_rowstats_valu(sh, P, L.h2o, q, k, v, h->lse, nullptr, st);
    if (e == hipSuccess && L.persist.n)
      e = mfma ? kve::launch_prefill_rowstats_mfma(sh, P, L.persist, q, k, h->lse,
                                                   std::max(0, P - L.info.max_window), st)
               : kve::launch_prefill_rowstats_valu(sh, P, L.persist, q, k, v, h->lse, nullptr, st);
    if (e == hipSuccess && L.adaptive.n)
      e = mfma ? kve::launch_prefill_rowstats_mfma(sh, P, L.adaptive, q, k, h->lse, 0, st)
               : kve::launch_prefill_rowstats_valu(sh, P, L.adaptive, q, k, v, h->lse, nullptr, st);
  }
  if (e == hipSuccess && L.h2o.n)
    e = mfma ? kve::launch_prefill_colsum_mfma(sh, P, L.h2o, q, k, h->lse, h->colsum, st)
             : kve::launch_prefill_colsum_valu(sh, P, L.h2o, q, k, h->lse, h->colsum, st);
  if (e == hipSuccess && L.persist.n)
    e = mfma ? kve::launch_prefill_persist_mfma(sh, P, L.persist, q, k, h->lse, L.cache.meta, h->colsum, st)
             : kve::launch_prefill_persist_valu(sh, P, L.persist, q, k, h->lse, L.cache.meta, h->colsum, st);
  // Profiled units: column sums with the profiled rows' mass, then the choice
  if (e == hipSuccess && L.adaptive.n) {
    const int rows = std::min(P, h->cfg.profile_rows);
    e = mfma ? kve::launch_prefill_colsum_mass_mfma(sh, P, L.adaptive, q, k, h->lse, h->colsum, h->mass, rows, st)
             : kve::launch_prefill_colsum_mass_valu(sh, P, L.adaptive, q, k, h->lse, h->colsum, h->mass, rows, st);
    const kve::Profile pf{rows, h->cfg.profile_threshold, L.info.ad_heavy, L.info.ad_recent};
    if (e == hipSuccess)
      e = kve::launch_prefill_adaptive(sh, L.cache, L.adaptive, P, h->colsum, h->mass, pf, k, v, token_ids,
                                       h->sets(), st);
  }
  if (e == hipSuccess)
    e = kve::launch_prefill_select(sh, L.cache, P, h->colsum, k, v, token_ids, h->sets(), st);
  if (e == hipSuccess && L.hash.n) {
    const int bits = h->cfg.sketch_bits;
    // the replay ranks with the queries of positions [B, P) only (B the
    // unit's budget), and every prompt key's sketch
    const int q0 = std::min(P, L.info.min_hash_budget);
    e = kve::launch_sketch_rows(sh, L.hash, q, P, q0, P - q0, L.cache.proj, bits, h->qsk, st);
    if (e == hipSuccess) e = kve::launch_sketch_rows(sh, L.hash, k, P, 0, P, L.cache.proj, bits, h->ksk, st);
    if (e == hipSuccess)
      e = kve::launch_hash_prefill(sh, L.cache, L.hash, P, L.info.max_hash_budget, h->qsk, h->ksk, k, v, st);
  }
  if (e != hipSuccess) return dev(e, "prefill launch");
  s = finish(h, st, "prefill");
  if (s == KVE_OK) L.position = P;
  return s;
}

kve_status kvevict_decode_step(kve_handle h, int32_t layer, const void* q, const void* k, const void* v,
                               const int32_t* token_ids, float* out, int32_t* evicted_pos, void* stream) {
  return decode_step_impl(h, layer, q, k, v, token_ids, out, evicted_pos, stream, nullptr, "decode_step");
}

kve_status kvevict_decode_step_noalloc(kve_handle h, int32_t layer, const void* q, const void* k, const void* v,
                                       const int32_t* token_ids, float* out, int32_t* evicted_pos,
                                       void* stream) {
  kve_status s = check_layer(h, layer);
  if (s != KVE_OK) return s;
  const Layer& L = h->layers[layer];
  if (!L.split.chunk)          // fused layers use no scratch at all
    return decode_step_impl(h, layer, q, k, v, token_ids, out, evicted_pos, stream, nullptr, "decode_step_noalloc");
  // partials [U][nch][d + 2] float, then logits [U][cap] float, 256-byte aligned
  const size_t U = h->shape.units(), d = h->shape.d;
  const size_t part_bytes = align_up(U * (size_t)L.split.max_chunks * (d + 2) * sizeof(float));
  const size_t need = part_bytes + align_up(U * (size_t)L.cache.cap * sizeof(float));
  if (need > kve::static_scratch_bytes())
    return fail(KVE_EUNSUPPORTED, "layer %d: the split decode needs %zu bytes of scratch; the static scratch holds %zu",
                layer, need, kve::static_scratch_bytes());
  if (!h->static_scratch)
    return fail(KVE_EDEVICE, "the static scratch's device address could not be looked up at create");
  char* base = static_cast<char*>(h->static_scratch);
  const kve::SplitScratch sp{reinterpret_cast<float*>(base), reinterpret_cast<float*>(base + part_bytes),
                             L.split.chunk, L.split.max_chunks};
  return decode_step_impl(h, layer, q, k, v, token_ids, out, evicted_pos, stream, &sp, "decode_step_noalloc");
}

kve_status kvevict_kept_indices(kve_handle h, int32_t layer, int32_t* pos_out, int32_t* count_out,
                                double* scores_out, void* stream) {
  kve_status s = check_layer(h, layer);
  if (s != KVE_OK) return s;
  if (!pos_out || !count_out) return fail(KVE_EINVAL, "pos_out and count_out are required");
  const Layer& L = h->layers[layer];
  if (L.position < 0) return fail(KVE_ESTATE, "layer %d has no cache yet", layer);
  hipStream_t st = (hipStream_t)stream;
  const size_t U = h->shape.units(), cap = L.cache.cap;
  hipError_t e = hipMemcpyAsync(pos_out, L.cache.pos, U * cap * 4, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(count_out, L.cache.count, U * 4, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && scores_out)
    e = hipMemcpyAsync(scores_out, L.cache.S, U * cap * 8, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return dev(e, "kept_indices copy");
  return finish(h, st, "kept_indices");
}

kve_status kvevict_cache_rows(kve_handle h, int32_t layer, void* k_out, void* v_out, float* k_scale_out,
                              float* v_scale_out, void* stream) {
  kve_status s = check_layer(h, layer);
  if (s != KVE_OK) return s;
  const Layer& L = h->layers[layer];
  const bool q4 = L.cache.q4 != 0;
  if (!k_out || !v_out || (q4 && (!k_scale_out || !v_scale_out)))
    return fail(KVE_EINVAL, "k_out and v_out (and, for 4-bit slots, the scale outputs) are required");
  if (L.position < 0) return fail(KVE_ESTATE, "layer %d has no cache yet", layer);
  hipStream_t st = (hipStream_t)stream;
  const size_t U = h->shape.units(), cap = L.cache.cap, d = h->shape.d;
  const size_t rows = U * cap * (q4 ? d / 2 : d * elem_size(h->cfg.dtype));
  hipError_t e = hipMemcpyAsync(k_out, L.cache.K, rows, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(v_out, L.cache.V, rows, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && q4)
    e = hipMemcpyAsync(k_scale_out, L.cache.Ksc, U * cap * (d / 32) * 4, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && q4)
    e = hipMemcpyAsync(v_scale_out, L.cache.Vsc, U * cap * (d / 32) * 4, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return dev(e, "cache_rows copy");
  return finish(h, st, "cache_rows");
}

kve_status kvevict_unit_policies(kve_handle h, int32_t layer, int32_t* choice_out, void* stream) {
  kve_status s = check_layer(h, layer);
  if (s != KVE_OK) return s;
  if (!choice_out) return fail(KVE_EINVAL, "choice_out is required");
  const Layer& L = h->layers[layer];
  if (L.position < 0) return fail(KVE_ESTATE, "layer %d has no cache yet", layer);
  hipStream_t st = (hipStream_t)stream;
  const size_t U = h->shape.units();
  // the `choice` field of each unit record, strided copy
  hipError_t e = hipMemcpy2DAsync(choice_out, sizeof(int32_t), &L.cache.meta[0].choice, sizeof(kve::HeadMeta),
                                  sizeof(int32_t), U, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return dev(e, "unit_policies copy");
  return finish(h, st, "unit_policies");
}

int32_t kvevict_capacity(kve_handle h, int32_t layer) {
  if (!h || layer < 0 || layer >= h->cfg.layers) return -1;
  return h->layers[layer].cache.cap;
}

int32_t kvevict_position(kve_handle h, int32_t layer) {
  if (!h || layer < 0 || layer >= h->cfg.layers) return -1;
  return h->layers[layer].position;
}

kve_status kvevict_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return fail(KVE_EINVAL, "src and sink are required");
  if (bytes < 16 || bytes % 16 || (uintptr_t)src % 16)
    return fail(KVE_EINVAL, "bytes must be a positive multiple of 16 and src 16-byte aligned");
  hipError_t e = kve::launch_stream_read(src, bytes, sink, (hipStream_t)stream);
  if (e != hipSuccess) return dev(e, "stream_read launch");
  const char* env = std::getenv("KVEVICT_SYNC_CHECK");
  if (env && env[0] == '1') {
    kve_status s = dev(hipStreamSynchronize((hipStream_t)stream), "stream_read");
    if (s != KVE_OK) return s;
  }
  return KVE_OK;
}

const char* kvevict_status_string(kve_status s) {
  switch (s) {
    case KVE_OK: return "ok";
    case KVE_EINVAL: return "invalid argument";
    case KVE_ESTATE: return "invalid state";
    case KVE_ENOMEM: return "workspace too small";
    case KVE_EDEVICE: return "device error";
    case KVE_EUNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

const char* kvevict_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
