// C ABI: argument validation, workspace layout and kernel dispatch.
// Validation runs entirely on the host before any HIP call, so every error
// path is exercised without a GPU.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gemma_attn.h"
#include "kernels.h"

namespace {

thread_local std::string g_error;

ga_status fail(ga_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

ga_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return GA_OK;
  return fail(GA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- kernel timing hooks -----------------------------------------------------
// When enabled, a pair of HIP events brackets every attention / decode kernel
// launch on the caller's stream; gemma_attn_profile_read() resolves them.
struct Timed {
  int kernel;   // 0 prefill attention, 1 prefill prep, 2 decode split-K, 3 decode merge, 4 kv_append
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<Timed> g_prof;

struct ProfScope {
  hipStream_t s;
  int kernel;
  hipEvent_t start = nullptr, stop = nullptr;
  ProfScope(hipStream_t st, int k) : s(st), kernel(k) {
    if (!g_prof_on) return;
    if (hipEventCreate(&start) != hipSuccess || hipEventCreate(&stop) != hipSuccess) {
      start = stop = nullptr;
      return;
    }
    hipEventRecord(start, s);
  }
  ~ProfScope() {
    if (!start) return;
    hipEventRecord(stop, s);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back({kernel, start, stop});
  }
};

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
// Query columns (token x head of the group) of one column group, of one decode
// launch (two groups), and of one call (as several launches).
constexpr int kDecodeColumns = 16;
constexpr int kDecodeLaunchColumns = 32;
constexpr int kDecodeMaxColumns = 64;

struct Derived {
  int group;
  int n_rot;
  int elem;
  bool q8;                 // int8 K=V cache
  bool pre;                // pre-rotated K=V cache (rows, then rotated heads)
  float scale;
  double log2_theta;
};

// Validity first (GA_EINVAL), then what the built kernels cover (GA_EUNSUPPORTED).
ga_status check_layer(const ga_layer* L, Derived* out) {
  if (!L) return fail(GA_EINVAL, "layer is NULL");
  if (L->n_q_heads <= 0 || L->n_kv_heads <= 0 || L->head_dim <= 0)
    return fail(GA_EINVAL, "head counts and head_dim must be positive");
  if (L->n_q_heads % L->n_kv_heads)
    return fail(GA_EINVAL, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", L->n_q_heads, L->n_kv_heads);
  if (L->head_dim % 2) return fail(GA_EINVAL, "head_dim must be even");
  if (L->window < 0) return fail(GA_EINVAL, "window must be >= 0");
  if (L->kv_shared != 0 && L->kv_shared != 1) return fail(GA_EINVAL, "kv_shared must be 0 or 1");
  if (!(L->rope_theta > 0.f) || !std::isfinite(L->rope_theta)) return fail(GA_EINVAL, "rope_theta must be > 0");
  if (!(L->rope_fraction >= 0.f && L->rope_fraction <= 1.f))
    return fail(GA_EINVAL, "rope_fraction must lie in [0, 1]");
  const double pairs = static_cast<double>(L->rope_fraction) * L->head_dim / 2.0;
  const double rounded = std::nearbyint(pairs);
  if (std::fabs(pairs - rounded) > 1e-6)
    return fail(GA_EINVAL, "rope_fraction * head_dim / 2 = %g is not a whole number of pairs", pairs);
  if (!(L->norm_eps > 0.f)) return fail(GA_EINVAL, "norm_eps must be > 0");
  if (!std::isfinite(L->softmax_scale)) return fail(GA_EINVAL, "softmax_scale must be finite");
  if (L->dtype != GA_BF16 && L->dtype != GA_F32) return fail(GA_EINVAL, "dtype must be GA_BF16 or GA_F32");
  if (L->cache_format != GA_CACHE_NATIVE && L->cache_format != GA_CACHE_INT8 &&
      L->cache_format != GA_CACHE_PREROTATED)
    return fail(GA_EINVAL, "cache_format must be GA_CACHE_NATIVE, GA_CACHE_INT8 or GA_CACHE_PREROTATED");

  const int G = L->n_q_heads / L->n_kv_heads;
  const int n_rot = static_cast<int>(rounded);
  if (L->head_dim != 256 && L->head_dim != 512)
    return fail(GA_EUNSUPPORTED, "head_dim %d: kernels are built for 256 and 512", L->head_dim);
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(GA_EUNSUPPORTED, "n_q_heads / n_kv_heads = %d: kernels are built for 1, 2, 4, 8", G);
  if (L->kv_shared && L->window > 0)
    return fail(GA_EUNSUPPORTED, "K=V layers are supported with window 0 only");
  if (L->kv_shared && n_rot != 64)
    return fail(GA_EUNSUPPORTED, "K=V layers rotate exactly 64 pairs on the fly (got %d)", n_rot);
  if (L->cache_format == GA_CACHE_INT8 &&
      (!L->kv_shared || L->dtype != GA_BF16 || L->head_dim != 512 || (G != 4 && G != 8)))
    return fail(GA_EUNSUPPORTED, "the int8 cache is built for bf16 K=V layers with head_dim 512 and 4 or 8 "
                                 "query heads per KV head");
  if (L->cache_format == GA_CACHE_PREROTATED &&
      (!L->kv_shared || L->dtype != GA_BF16 || L->head_dim != 512 || (G != 4 && G != 8)))
    return fail(GA_EUNSUPPORTED, "the pre-rotated cache is built for bf16 K=V layers with head_dim 512 and 4 or "
                                 "8 query heads per KV head");
  if (out) {
    out->group = G;
    out->n_rot = n_rot;
    out->elem = L->dtype == GA_BF16 ? 2 : 4;
    out->q8 = L->cache_format == GA_CACHE_INT8;
    out->pre = L->cache_format == GA_CACHE_PREROTATED;
    out->scale = L->softmax_scale > 0.f ? L->softmax_scale : 1.0f / std::sqrt(static_cast<float>(L->head_dim));
    out->log2_theta = std::log2(static_cast<double>(L->rope_theta));
  }
  return GA_OK;
}

// Cache arguments shared by prefill and kv_append.
ga_status check_caches(const ga_layer* L, const void* k_cache, const void* v_cache, int32_t cache_cap,
                       bool optional, int32_t min_cap) {
  if (!k_cache) {
    if (!optional) return fail(GA_EINVAL, "k_cache is NULL");
    if (v_cache) return fail(GA_EINVAL, "v_cache given without k_cache");
    return GA_OK;
  }
  if (cache_cap <= 0) return fail(GA_EINVAL, "cache_cap must be > 0");
  if (L->kv_shared) {
    if (v_cache) return fail(GA_EINVAL, "K=V layer: v_cache must be NULL (one cache tensor)");
  } else if (!v_cache) {
    return fail(GA_EINVAL, "layer with a separate V needs v_cache");
  }
  if (L->window > 0) {
    if (cache_cap < L->window)
      return fail(GA_EINVAL, "windowed layer: cache_cap (%d) must be at least the window (%d)", cache_cap,
                  L->window);
  } else if (cache_cap < min_cap) {
    return fail(GA_EINVAL, "cache_cap (%d) is smaller than the sequence (%d)", cache_cap, min_cap);
  }
  return GA_OK;
}

// int8 cache: codes [B][Hkv][cap][d] bytes, then the fp32 scales [B][Hkv][cap].
size_t q8_scale_offset(const ga_layer* L, int batch, int cap) {
  return align_up(static_cast<size_t>(batch) * L->n_kv_heads * cap * L->head_dim);
}
// pre-rotated cache: rows [B][Hkv][cap][d] as the native K=V cache, then the
// rotated heads [B][Hkv][cap][2 n_rot].
size_t pre_heads_offset(const ga_layer* L, const Derived& dv, int batch, int cap) {
  return align_up(static_cast<size_t>(batch) * L->n_kv_heads * cap * L->head_dim * dv.elem);
}
size_t cache_bytes(const ga_layer* L, const Derived& dv, int batch, int cap) {
  const size_t rows = static_cast<size_t>(batch) * L->n_kv_heads * cap;
  if (dv.q8) return q8_scale_offset(L, batch, cap) + rows * 4;
  if (dv.pre) return pre_heads_offset(L, dv, batch, cap) + rows * 2 * dv.n_rot * dv.elem;
  return rows * L->head_dim * dv.elem;
}
void* pre_heads(const ga_layer* L, const Derived& dv, void* cache, int batch, int cap) {
  if (!dv.pre || !cache) return nullptr;
  return static_cast<char*>(cache) + pre_heads_offset(L, dv, batch, cap);
}
float* q8_scales(const ga_layer* L, const Derived& dv, void* cache, int batch, int cap) {
  if (!dv.q8 || !cache) return nullptr;
  return reinterpret_cast<float*>(static_cast<char*>(cache) + q8_scale_offset(L, batch, cap));
}

struct PrefillLayout {
  size_t table, table16, ws_k, ws_v, ws_kn, total;
  int seq_pad, kw;
};

// Workspace: RoPE table [seq_pad][n_rot] (cos, sin) fp32, the same table in
// fp16 (read by the local-layer query prologue), key rows [B][Hkv][seq_pad][kw],
// value rows [B][Hkv][seq_pad][d], the largest squared key length of each tile
// of key rows [B][Hkv][seq_pad / kPrepTile] fp32; each 256-byte aligned.
PrefillLayout prefill_layout(const ga_layer* L, const Derived& dv, int batch, int seq_len) {
  PrefillLayout p;
  p.seq_pad = (seq_len + ga::kPrepTile - 1) / ga::kPrepTile * ga::kPrepTile;
  p.kw = L->kv_shared ? 2 * dv.n_rot : L->head_dim;
  const size_t rows = static_cast<size_t>(batch) * L->n_kv_heads * p.seq_pad;
  p.table = 0;
  p.table16 = align_up(static_cast<size_t>(p.seq_pad) * dv.n_rot * 8);
  p.ws_k = p.table16 + align_up(static_cast<size_t>(p.seq_pad) * dv.n_rot * 4);
  p.ws_v = p.ws_k + align_up(rows * p.kw * dv.elem);
  p.ws_kn = p.ws_v + align_up(rows * L->head_dim * dv.elem);
  p.total = p.ws_kn + align_up(rows / ga::kPrepTile * sizeof(float));
  return p;
}

// Tiles of one (sequence, KV head) segment at most: windowed layers read the
// min(L, cache_cap) filled ring slots; cache_cap = 0 (the size queries, which
// do not take it) bounds them by max_seq_len.
int decode_tiles_per_seq(const ga_layer* L, int max_seq_len, int cache_cap) {
  const int keys = (L->window > 0 && cache_cap > 0) ? std::min(max_seq_len, cache_cap) : max_seq_len;
  return (keys + ga::kDecodeTile - 1) / ga::kDecodeTile;
}

// Decode scratch is sized for the largest grid the launch can pick (at most
// 1024 waves' partial slots plus one per wave and segment), so it does not
// depend on the device; the launch then uses one workgroup per CU at most.
constexpr int kMaxDecodeCUs = 1 << 20;

// The query tokens of one column group fill the 16 columns of its QK^T MFMAs
// (G heads per token).  A launch takes one group, or two for 17..32 columns
// (both streaming the same tiles); more tokens take several launches.
int decode_pass_tokens(const Derived& dv, int q_len) { return std::min(q_len, kDecodeLaunchColumns / dv.group); }
int decode_groups(const Derived& dv, int n_tok) { return n_tok * dv.group > kDecodeColumns ? 2 : 1; }

bool decode_plan(const ga_layer* L, const Derived& dv, int batch, int n_tok, int max_seq_len, int cache_cap,
                 int n_cus, ga::DecodePlan* plan) {
  return ga::plan_decode(L->dtype, L->head_dim, dv.group, L->kv_shared, batch, L->n_kv_heads,
                         decode_tiles_per_seq(L, max_seq_len, cache_cap), n_cus, n_tok, decode_groups(dv, n_tok),
                         plan);
}

// Scratch of a call: the largest of its launches' plans (a full launch, and
// a last one with fewer tokens).
size_t decode_bytes(const ga_layer* L, const Derived& dv, int batch, int q_len, int max_seq_len) {
  const int per = decode_pass_tokens(dv, q_len);
  size_t need = 0;
  for (int n : {per, q_len % per}) {
    if (n == 0) continue;
    ga::DecodePlan plan;
    if (!decode_plan(L, dv, batch, n, max_seq_len, 0, kMaxDecodeCUs, &plan)) return 0;
    need = std::max(need, plan.bytes());
  }
  return align_up(need);
}

// Query tokens of one decode call: q_len tokens x G heads, at most
// kDecodeMaxColumns (launched kDecodeLaunchColumns at a time).
ga_status check_q_len(const ga_layer* L, const Derived& dv, int q_len) {
  (void)L;
  if (q_len < 1) return fail(GA_EINVAL, "q_len must be >= 1");
  if (q_len * dv.group > kDecodeMaxColumns)
    return fail(GA_EUNSUPPORTED, "q_len %d x %d query heads per KV head exceeds %d query columns (%d passes of %d)",
                q_len, dv.group, kDecodeMaxColumns, kDecodeMaxColumns / kDecodeColumns, kDecodeColumns);
  return GA_OK;
}

ga_status check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return GA_OK;
  if (!ws) return fail(GA_EWORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(GA_EINVAL, "workspace must be 256-byte aligned");
  if (have < need) return fail(GA_EWORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return GA_OK;
}

// ---- scratch for the decode that allocates nothing ------------------------------
// One static device array per GPU, reached through its address on that device
// (hipGetSymbolAddress); the array's name in host code is only a stand-in.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;

__global__ void zero_fill_kernel(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device: the scratch array's device address

// The current device's scratch address, found (and the array cleared, by a
// fill kernel on `s`) on the first call on that device.
ga_status device_scratch(int dev, hipStream_t s, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (dev < 0) return fail(GA_EINVAL, "bad device index %d", dev);
  if (static_cast<size_t>(dev) >= g_scratch_ptr.size()) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "decode scratch: hipGetSymbolAddress");
    hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, s, static_cast<uint4*>(p),
                       kNoAllocScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "decode scratch: clearing launch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GA_OK;
}

}  // namespace

// Decode launches two kernels; the launcher reports each to this callback.
void record_decode(hipStream_t s, int which, bool before) {
  static thread_local hipEvent_t pending = nullptr;
  if (before) {
    if (hipEventCreate(&pending) == hipSuccess) hipEventRecord(pending, s);
    else pending = nullptr;
    return;
  }
  if (!pending) return;
  hipEvent_t stop;
  if (hipEventCreate(&stop) != hipSuccess) return;
  hipEventRecord(stop, s);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back({which, pending, stop});
  pending = nullptr;
}

namespace {

// Decode of the last q_len positions of each sequence.  `noalloc`: the
// split-K scratch is this device's static scratch array instead of
// `workspace`, and a plan that needs more than it holds is rejected.
ga_status decode_impl(const ga_layer* layer, int32_t batch, int32_t q_len, const void* q, const void* q_gain,
                      const void* k_cache, const void* v_cache, int32_t cache_cap, const int32_t* seq_lens,
                      int32_t max_seq_len, void* out, void* workspace, size_t workspace_bytes, bool noalloc,
                      void* stream) {
  Derived dv;
  ga_status st = check_layer(layer, &dv);
  if (st != GA_OK) return st;
  if (batch < 0) return fail(GA_EINVAL, "batch must be >= 0");
  st = check_q_len(layer, dv, q_len);
  if (st != GA_OK) return st;
  if (batch == 0) return GA_OK;
  if (max_seq_len < 1) return fail(GA_EINVAL, "max_seq_len must be >= 1");
  if (static_cast<int64_t>(batch) * layer->n_kv_heads * decode_tiles_per_seq(layer, max_seq_len, 0) > INT32_MAX)
    return fail(GA_EUNSUPPORTED, "batch %d x max_seq_len %d: too many cached positions for one decode call", batch,
                max_seq_len);
  if (!q || !q_gain || !seq_lens || !out) return fail(GA_EINVAL, "q, q_gain, seq_lens and out must be non-NULL");
  if (layer->dtype == GA_F32 && layer->head_dim == 512 && !layer->kv_shared)
    return fail(GA_EUNSUPPORTED, "fp32 decode with head_dim 512 and a separate V cache is not built");
  st = check_caches(layer, k_cache, v_cache, cache_cap, false, 1);
  if (st != GA_OK) return st;
  if (layer->window > 0 && q_len > 1 && cache_cap < layer->window + q_len - 1)
    return fail(GA_EINVAL, "windowed layer: %d new tokens at once need a ring of window + %d = %d slots (cache_cap "
                "%d); the earliest of them still sees keys the later ones push out of a smaller ring", q_len,
                q_len - 1, layer->window + q_len - 1, cache_cap);
  if (static_cast<int64_t>(cache_cap) * layer->head_dim * (dv.q8 ? 1 : dv.elem) > INT32_MAX)
    return fail(GA_EUNSUPPORTED, "cache_cap %d: one head's cache must stay under 2 GiB for decode", cache_cap);
  if (reinterpret_cast<uintptr_t>(k_cache) % 16 || reinterpret_cast<uintptr_t>(v_cache) % 16)
    return fail(GA_EINVAL, "the caches must be 16-byte aligned");
  if (!noalloc) {
    st = check_workspace(workspace, workspace_bytes, decode_bytes(layer, dv, batch, q_len, max_seq_len));
    if (st != GA_OK) return st;
  }
  int dev = 0, cus = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he == hipSuccess) he = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (he != hipSuccess) return hip_status(he, "decode: device query");
  const int per = decode_pass_tokens(dv, q_len);
  ga::DecodePlan plan, last;   // a full launch, and the last one when it has fewer tokens
  if (!decode_plan(layer, dv, batch, per, max_seq_len, cache_cap, cus, &plan) ||
      !decode_plan(layer, dv, batch, q_len % per ? q_len % per : per, max_seq_len, cache_cap, cus, &last))
    return fail(GA_EUNSUPPORTED, "no decode kernel for this layer configuration");
  if (noalloc) {
    const size_t need = std::max(plan.bytes(), last.bytes());
    if (need > kNoAllocScratchBytes)
      return fail(GA_EWORKSPACE, "decode needs %zu bytes of scratch for batch %d, max_seq_len %d; the static "
                  "scratch holds %zu (use gemma_attn_decode with a workspace)", need, batch, max_seq_len,
                  kNoAllocScratchBytes);
    st = device_scratch(dev, static_cast<hipStream_t>(stream), &workspace);
    if (st != GA_OK) return st;
  }
  ga::DecodeArgs da{};
  da.q = q; da.q_gain = q_gain; da.k_cache = k_cache; da.v_cache = v_cache; da.seq_lens = seq_lens;
  da.out = out;
  da.tile_prefix = static_cast<int32_t*>(workspace);
  da.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.prefix_bytes);
  da.batch = batch; da.n_q_heads = layer->n_q_heads; da.n_kv_heads = layer->n_kv_heads; da.n_rot = dv.n_rot;
  da.window = layer->window; da.cache_cap = cache_cap; da.max_seq_len = max_seq_len;
  da.q_len = q_len;
  da.k_scales = q8_scales(layer, dv, const_cast<void*>(k_cache), batch, cache_cap);
  da.k_heads = pre_heads(layer, dv, const_cast<void*>(k_cache), batch, cache_cap);
  da.eps = layer->norm_eps; da.qk_scale_log2 = dv.scale * 1.4426950408889634f; da.log2_theta = dv.log2_theta;
  // One launch (split-K and merge) per 32 query columns; the launches reuse
  // the scratch in stream order.
  for (int tok0 = 0; tok0 < q_len; tok0 += per) {
    da.tok0 = tok0;
    da.n_tok = std::min(per, q_len - tok0);
    const ga::DecodePlan& pl = da.n_tok == per ? plan : last;
    da.n_wgs = pl.n_wgs;
    da.n_groups = pl.groups;
    da.slot_floats = static_cast<int>(pl.slot_floats);
    da.group_floats = static_cast<int64_t>(pl.slots * pl.slot_floats);
    st = hip_status(ga::launch_decode(da, layer->dtype, layer->head_dim, dv.group, layer->kv_shared, batch,
                                      static_cast<hipStream_t>(stream), g_prof_on ? &record_decode : nullptr),
                    "decode launch");
    if (st != GA_OK) return st;
  }
  return GA_OK;
}

}  // namespace

extern "C" {

void gemma_attn_profile_enable(int on) { g_prof_on = on != 0; }

int gemma_attn_profile_read(int kernel, double* total_ms, int* count) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double t = 0.0;
  int n = 0;
  for (const Timed& e : g_prof) {
    if (e.kernel != kernel) continue;
    if (hipEventSynchronize(e.stop) != hipSuccess) return -1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e.start, e.stop) != hipSuccess) return -1;
    t += ms;
    ++n;
  }
  if (total_ms) *total_ms = t;
  if (count) *count = n;
  return 0;
}

void gemma_attn_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const Timed& e : g_prof) {
    hipEventDestroy(e.start);
    hipEventDestroy(e.stop);
  }
  g_prof.clear();
}

const char* gemma_attn_last_error(void) { return g_error.c_str(); }

ga_status gemma_attn_calibrate_mfma(const void* ops, int32_t n_ops, int32_t iters, int32_t n_wgs, float* sink,
                                    void* stream) {
  if (!ops || !sink || n_ops <= 0 || iters <= 0 || n_wgs <= 0)
    return fail(GA_EINVAL, "calibrate_mfma: NULL pointer or non-positive size");
  return hip_status(ga::launch_calib_mfma(ops, n_ops, iters, n_wgs, sink, static_cast<hipStream_t>(stream)),
                    "calibrate_mfma launch");
}

ga_status gemma_attn_calibrate_stream(const void* buf, size_t bytes, int32_t n_wgs, unsigned* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || n_wgs <= 0)
    return fail(GA_EINVAL, "calibrate_stream: NULL pointer, or bytes not a positive multiple of 16");
  return hip_status(ga::launch_calib_stream(buf, bytes, n_wgs, sink, static_cast<hipStream_t>(stream)),
                    "calibrate_stream launch");
}

const char* gemma_attn_version(void) { return "gemma_attn 0.1 (gfx950)"; }

size_t gemma_attn_cache_bytes(const ga_layer* layer, int32_t batch, int32_t cache_cap) {
  Derived dv;
  if (check_layer(layer, &dv) != GA_OK || batch < 0 || cache_cap < 0) return 0;
  return cache_bytes(layer, dv, batch, cache_cap);
}

size_t gemma_attn_prefill_workspace_size(const ga_layer* layer, int32_t batch, int32_t seq_len) {
  Derived dv;
  if (check_layer(layer, &dv) != GA_OK || batch < 0 || seq_len < 0) return 0;
  return prefill_layout(layer, dv, batch, seq_len).total;
}

size_t gemma_attn_decode_workspace_size(const ga_layer* layer, int32_t batch, int32_t max_seq_len) {
  return gemma_attn_decode_multi_workspace_size(layer, batch, 1, max_seq_len);
}

size_t gemma_attn_decode_multi_workspace_size(const ga_layer* layer, int32_t batch, int32_t q_len,
                                              int32_t max_seq_len) {
  Derived dv;
  if (check_layer(layer, &dv) != GA_OK || batch < 0 || max_seq_len < 1) return 0;
  if (check_q_len(layer, dv, q_len) != GA_OK) return 0;
  return decode_bytes(layer, dv, batch, q_len, max_seq_len);
}

// Prefill of positions start .. start + seq_len - 1 of every sequence.  start
// > 0: positions before start are in the caches already (K=V and separate-V
// global layers: slot = position; windowed layers: their ring) and are read
// back into the workspace rows.
static ga_status prefill_impl(const ga_layer* layer, int32_t batch, int32_t start, int32_t seq_len, const void* q,
                              const void* k, const void* v, const void* q_gain, const void* k_gain, void* k_cache,
                              void* v_cache, int32_t cache_cap, void* out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Derived dv;
  ga_status st = check_layer(layer, &dv);
  if (st != GA_OK) return st;
  if (batch < 0 || seq_len < 0 || start < 0) return fail(GA_EINVAL, "batch, start and seq_len must be >= 0");
  const int64_t total = static_cast<int64_t>(start) + seq_len;
  if (total > (1 << 22)) return fail(GA_EUNSUPPORTED, "seq_len above 4M positions");
  if ((total + ga::kPrepTile) * layer->head_dim * dv.elem > INT32_MAX)
    return fail(GA_EUNSUPPORTED, "seq_len %lld: one head's key tiles must stay under 2 GiB",
                static_cast<long long>(total));
  if (start > 0 && !k_cache)
    return fail(GA_EINVAL, "a prefill chunk after cached positions needs the caches holding them");
  if (batch == 0 || seq_len == 0) return GA_OK;
  if (!q || !k || !q_gain || !k_gain || !out) return fail(GA_EINVAL, "q, k, q_gain, k_gain and out must be non-NULL");
  if (layer->kv_shared && v) return fail(GA_EINVAL, "K=V layer: v must be NULL (keys are the values)");
  if (!layer->kv_shared && !v) return fail(GA_EINVAL, "layer with a separate V needs v");
  // the kernels move rows, gains and cache rows in 16-byte pieces
  for (const void* t : {q, k, v, q_gain, k_gain, static_cast<const void*>(k_cache), static_cast<const void*>(v_cache),
                        static_cast<const void*>(out)})
    if (reinterpret_cast<uintptr_t>(t) % 16)
      return fail(GA_EINVAL, "q, k, v, the gains, the caches and out must be 16-byte aligned");
  st = check_caches(layer, k_cache, v_cache, cache_cap, true, static_cast<int32_t>(total));
  if (st != GA_OK) return st;
  const PrefillLayout lay = prefill_layout(layer, dv, batch, static_cast<int32_t>(total));
  st = check_workspace(workspace, workspace_bytes, lay.total);
  if (st != GA_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  // Separate-V layers: the attention kernel reads v in place when the prompt
  // is whole and one head's rows (Hkv d elements apart) span less than 2^31
  // bytes; else prep copies v (and the cached values) into the workspace rows.
  const bool v_in_place = !layer->kv_shared && start == 0 &&
      static_cast<int64_t>(seq_len) * layer->n_kv_heads * layer->head_dim * dv.elem < (int64_t{1} << 31);
  // Windowed layers read only the window before the chunk's first position.
  const int tile0 = layer->window > 0 ? std::max(0, start - layer->window + 1) / ga::kPrepTile : 0;
  // A windowed chunk reads ring slots that its own rows overwrite: the ring
  // is written by a second pass, after every read.
  const bool ring_after = layer->window > 0 && start > 0;
  {
    ProfScope ps(s, 1);
    st = hip_status(ga::launch_rope_table(ws + lay.table, ws + lay.table16, tile0 * ga::kPrepTile, lay.seq_pad, dv.n_rot,
                                          layer->head_dim, dv.log2_theta, s),
                    "rope table launch");
    ga::PrepArgs pa{};
    pa.k = k; pa.v = v; pa.k_gain = k_gain; pa.rope_table = ws + lay.table;
    pa.k_cache = k_cache; pa.v_cache = v_cache; pa.ws_k = ws + lay.ws_k; pa.ws_v = ws + lay.ws_v; pa.kw = lay.kw;
    pa.seq_len = seq_len; pa.seq_pad = lay.seq_pad; pa.n_kv_heads = layer->n_kv_heads; pa.n_rot = dv.n_rot;
    pa.window = layer->window; pa.kv_shared = layer->kv_shared; pa.cache_cap = cache_cap; pa.eps = layer->norm_eps;
    pa.pos0 = start;
    pa.tile0 = tile0;
    pa.write_v = !layer->kv_shared && !v_in_place;
    pa.write_ws = 1;
    pa.write_cache = !ring_after;
    pa.k_scales = q8_scales(layer, dv, k_cache, batch, cache_cap);
    pa.k_heads = pre_heads(layer, dv, k_cache, batch, cache_cap);
    pa.ws_kn = reinterpret_cast<float*>(ws + lay.ws_kn);
    if (st == GA_OK)
      st = hip_status(ga::launch_prefill_prep(pa, layer->dtype, layer->head_dim, batch, s), "prefill prep launch");
    if (st == GA_OK && ring_after && k_cache) {
      // the chunk's last cache_cap positions into the ring
      pa.write_ws = 0;
      pa.write_cache = 1;
      pa.tile0 = static_cast<int>(std::max<int64_t>(start, total - cache_cap) / ga::kPrepTile);
      st = hip_status(ga::launch_prefill_prep(pa, layer->dtype, layer->head_dim, batch, s), "ring write launch");
    }
  }
  if (st != GA_OK) return st;

  ga::PrefillArgs fa{};
  fa.q = q; fa.q_gain = q_gain; fa.rope_table = ws + lay.table; fa.rope_table16 = ws + lay.table16;
  fa.table_rows = lay.seq_pad; fa.ws_k = ws + lay.ws_k; fa.ws_v = ws + lay.ws_v;
  fa.out = out; fa.seq_len = seq_len; fa.seq_pad = lay.seq_pad; fa.n_q_heads = layer->n_q_heads;
  fa.n_kv_heads = layer->n_kv_heads; fa.n_rot = dv.n_rot; fa.window = layer->window; fa.eps = layer->norm_eps;
  fa.q_pos0 = start;
  fa.v = v_in_place ? v : nullptr;
  fa.ws_kn = reinterpret_cast<const float*>(ws + lay.ws_kn);
  fa.qk_scale_log2 = dv.scale * 1.4426950408889634f;
  ProfScope ps(s, 0);
  return hip_status(ga::launch_prefill_attn(fa, layer->dtype, layer->head_dim, dv.group, layer->kv_shared, batch, s),
                    "prefill attention launch");
}

ga_status gemma_attn_prefill(const ga_layer* layer, int32_t batch, int32_t seq_len, const void* q,
                             const void* k, const void* v, const void* q_gain, const void* k_gain,
                             void* k_cache, void* v_cache, int32_t cache_cap, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(layer, batch, 0, seq_len, q, k, v, q_gain, k_gain, k_cache, v_cache, cache_cap, out, workspace,
                      workspace_bytes, stream);
}

size_t gemma_attn_prefill_chunk_workspace_size(const ga_layer* layer, int32_t batch, int32_t start, int32_t chunk) {
  Derived dv;
  if (check_layer(layer, &dv) != GA_OK || batch < 0 || start < 0 || chunk < 0) return 0;
  const int64_t total = static_cast<int64_t>(start) + chunk;
  if (total > (1 << 22)) return 0;
  return prefill_layout(layer, dv, batch, static_cast<int32_t>(total)).total;
}

ga_status gemma_attn_prefill_chunk(const ga_layer* layer, int32_t batch, int32_t start, int32_t chunk,
                                   const void* q, const void* k, const void* v, const void* q_gain,
                                   const void* k_gain, void* k_cache, void* v_cache, int32_t cache_cap, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(layer, batch, start, chunk, q, k, v, q_gain, k_gain, k_cache, v_cache, cache_cap, out,
                      workspace, workspace_bytes, stream);
}

ga_status kv_append(const ga_layer* layer, int32_t batch, const void* k_new, const void* v_new,
                    const void* k_gain, const int32_t* positions, void* k_cache, void* v_cache,
                    int32_t cache_cap, void* stream) {
  Derived dv;
  ga_status st = check_layer(layer, &dv);
  if (st != GA_OK) return st;
  if (batch < 0) return fail(GA_EINVAL, "batch must be >= 0");
  if (batch == 0) return GA_OK;
  if (!k_new || !k_gain || !positions) return fail(GA_EINVAL, "k_new, k_gain and positions must be non-NULL");
  if (layer->kv_shared && v_new) return fail(GA_EINVAL, "K=V layer: v_new must be NULL");
  if (!layer->kv_shared && !v_new) return fail(GA_EINVAL, "layer with a separate V needs v_new");
  st = check_caches(layer, k_cache, v_cache, cache_cap, false, 1);
  if (st != GA_OK) return st;
  if (reinterpret_cast<uintptr_t>(k_cache) % 16 || reinterpret_cast<uintptr_t>(v_cache) % 16)
    return fail(GA_EINVAL, "the caches must be 16-byte aligned");
  ga::AppendArgs aa{};
  aa.k_new = k_new; aa.v_new = v_new; aa.k_gain = k_gain; aa.positions = positions;
  aa.k_cache = k_cache; aa.v_cache = v_cache; aa.n_kv_heads = layer->n_kv_heads; aa.n_rot = dv.n_rot;
  aa.window = layer->window; aa.kv_shared = layer->kv_shared; aa.cache_cap = cache_cap; aa.eps = layer->norm_eps;
  aa.log2_theta = dv.log2_theta;
  aa.k_scales = q8_scales(layer, dv, k_cache, batch, cache_cap);
  aa.k_heads = pre_heads(layer, dv, k_cache, batch, cache_cap);
  ProfScope ps(static_cast<hipStream_t>(stream), 4);
  return hip_status(ga::launch_kv_append(aa, layer->dtype, layer->head_dim, batch, static_cast<hipStream_t>(stream)),
                    "kv_append launch");
}

ga_status gemma_attn_decode(const ga_layer* layer, int32_t batch, const void* q, const void* q_gain,
                            const void* k_cache, const void* v_cache, int32_t cache_cap,
                            const int32_t* seq_lens, int32_t max_seq_len, void* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return gemma_attn_decode_multi(layer, batch, 1, q, q_gain, k_cache, v_cache, cache_cap, seq_lens, max_seq_len,
                                 out, workspace, workspace_bytes, stream);
}

ga_status gemma_attn_decode_multi(const ga_layer* layer, int32_t batch, int32_t q_len, const void* q,
                                  const void* q_gain, const void* k_cache, const void* v_cache, int32_t cache_cap,
                                  const int32_t* seq_lens, int32_t max_seq_len, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_impl(layer, batch, q_len, q, q_gain, k_cache, v_cache, cache_cap, seq_lens, max_seq_len, out,
                     workspace, workspace_bytes, false, stream);
}

ga_status gemma_attn_decode_noalloc(const ga_layer* layer, int32_t batch, const void* q, const void* q_gain,
                                    const void* k_cache, const void* v_cache, int32_t cache_cap,
                                    const int32_t* seq_lens, int32_t max_seq_len, void* out, void* stream) {
  return decode_impl(layer, batch, 1, q, q_gain, k_cache, v_cache, cache_cap, seq_lens, max_seq_len, out, nullptr, 0,
                     true, stream);
}

}  // extern "C"
