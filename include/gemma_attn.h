/*
 * gemma_attn.h -- C ABI of the MI355X (gfx950) attention block of a
 * Gemma-4-style decoder: local sliding-window GQA layers and global K=V GQA
 * layers with QKNorm and (p-)RoPE.
 *
 * Source of the method (all pages are about the "Gemma 4 Technical Report"):
 *   - QKNorm (per-head RMSNorm of q and k): "Gemma 4 Technical Report" notes,
 *     §2 Model Architecture; "Gemma 4 技术报告摘要", table "1. 预训练 Recipe".
 *   - RoPE base 10k on local layers, p-RoPE p = 0.25 base 1M on global layers:
 *     "Gemma 4 Technical Report" notes, §2 "Long-context efficiency";
 *     "Gemma 4多模态大模型架构详解", section "p-RoPE（低频剪枝旋转位置编码）".
 *   - keys reused as values on global layers: same notes §2; "Gemma 4多模态大模型
 *     架构详解", section "K=V".
 *   - GQA 2:1 local, 8:1 global, head dim 256 -> 512: "Gemma 4多模态大模型架构详解",
 *     section "分组查询注意力"; "Gemma 4 架構與多模態拆解" talk notes, chapter
 *     "Grouped query attention".
 *   - sliding window (512 / 1024) and full causal attention: "Gemma 4多模态大模型
 *     架构详解", section "交错层（局部与全局注意力）".
 *
 * Conventions fixed here (the pages leave them open):
 *   - rotary pairs are adjacent dims (2i, 2i+1); pair i < n_rot = p*d/2 turns
 *     counter-clockwise by pos * theta^(-2i/d); pairs >= n_rot are untouched;
 *   - positions are 0-based; QKNorm is x / sqrt(mean(x^2) + eps) * gain;
 *   - query head h reads KV head h / (n_q_heads / n_kv_heads);
 *   - a window W keeps keys j with i - W < j <= i;
 *   - K=V layers: the cache is ONE tensor of normalised, UNROTATED keys, slot j
 *     = position j; p-RoPE is applied on the fly when scores are formed and the
 *     unrotated tensor is the value;
 *   - layers with a separate V: the K cache holds normalised and ROTATED keys and
 *     the V cache the raw values; windowed layers keep a ring of cache_cap >= W
 *     slots (slot = position mod cache_cap).  W slots hold every key the newest
 *     token sees; checking q_len new tokens at once needs W + q_len - 1.
 *
 * Ownership and execution:
 *   - every pointer argument is caller-owned DEVICE memory except `layer`
 *     (host).  Tensors are dense, row-major, in the layer's dtype unless stated.
 *   - the library never allocates or frees device memory, never synchronises,
 *     and keeps no pointer past a call.  Work is enqueued on `stream` (a
 *     hipStream_t; NULL = the null stream) and runs asynchronously.
 *   - all argument validation happens on the host before any launch; a failed
 *     validation launches nothing.  Device-resident values (positions, lengths)
 *     are range-checked by the kernels, which then skip the write or write NaN
 *     as documented per call.
 *   - on any status other than GA_OK, gemma_attn_last_error() returns a message
 *     for the calling thread.
 *
 * Supported on the GPU: head_dim 256 or 512; n_q_heads / n_kv_heads in
 * {1, 2, 4, 8}; n_rot = rope_fraction * head_dim / 2 a whole multiple of 4 (any
 * for separate-V layers, exactly 64 for K=V layers, e.g. d = 512 with
 * p = 0.25); K=V only with window 0.  Other shapes return GA_EUNSUPPORTED.
 */
#ifndef GEMMA_ATTN_H
#define GEMMA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GA_BF16 = 0, GA_F32 = 1 } ga_dtype;

typedef enum {
  GA_OK = 0,
  GA_EINVAL = 1,        /* bad argument (null pointer, shape, size)         */
  GA_EUNSUPPORTED = 2,  /* valid, but no kernel is built for this shape     */
  GA_EWORKSPACE = 3,    /* workspace smaller than *_workspace_size() says   */
  GA_EHIP = 4           /* a HIP launch failed; message holds the HIP error */
} ga_status;

/* One attention layer.  window = 0 is a global (full causal) layer. */
typedef struct {
  int32_t n_q_heads;      /* Hq                                               */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0                               */
  int32_t head_dim;       /* d                                                */
  int32_t window;         /* 0 = full causal; W > 0 = keys i-W < j <= i       */
  int32_t kv_shared;      /* 1 = keys are the values (one cache tensor)       */
  float rope_theta;       /* 1e4 on local layers, 1e6 on global layers        */
  float rope_fraction;    /* p: 1.0 local, 0.25 global                        */
  float norm_eps;         /* QKNorm epsilon, > 0 (1e-6)                       */
  float softmax_scale;    /* <= 0 selects 1/sqrt(d)                           */
  int32_t dtype;          /* ga_dtype of every tensor; accumulation is fp32   */
  int32_t cache_format;   /* ga_cache_format of k_cache (0: dtype elements)   */
} ga_layer;

/*
 * Cache formats.  GA_CACHE_INT8 (global K=V layers with dtype GA_BF16,
 * head_dim 512 and 4 or 8 query heads per KV head; others: GA_EUNSUPPORTED)
 * keeps each cached row (one position of one KV head) as d int8 codes and one
 * fp32 scale s = max_i |k_i| / 127, codes c_i = round-half-even(k_i / s), the
 * row standing for c_i * s: the int8 KV cache of the pages' 32K memory table
 * ("Gemma 4 技术报告：开源全模态密集 + MoE 模型家族，长上下文与端侧高效是本代核心",
 * table "显存占用（32k 上下文，文本 only，int8 KV cache）"), which leaves the int8
 * mapping open.  One k_cache buffer holds, for B sequences of cache_cap slots:
 *   int8  [B][Hkv][cache_cap][d]   c_i (two's complement, -127 .. 127)
 *   then, at byte offset round_up(B * Hkv * cache_cap * d, 256),
 *   float [B][Hkv][cache_cap]      s
 * Every call that takes k_cache and batch finds the scales there; a cache is
 * filled and read with the same batch.  An all-zero row has s = 0 and codes 0.
 * Prefill attends over the prompt's own keys at full precision and only
 * writes the cache; decode and a later prefill chunk read cached rows back as
 * c_i * s.  Decode streams about half the bytes of a bf16 cache.
 */
/*
 * GA_CACHE_PREROTATED (the same layers as GA_CACHE_INT8) is the "1.25 d"
 * layout the pages' 37.5% reduction describes ("解读 Gemma 4 的架构创新",
 * "关键架构创新" ② Keys as Values; "Gemma 4 Technical Report" notes, §2): per
 * cached row, the normalised unrotated key, which is also the value, plus its
 * leading 2 n_rot dims already rotated to the row's position.  One k_cache
 * buffer holds, in dtype elements:
 *   [B][Hkv][cache_cap][d]         the rows, laid out as a GA_CACHE_NATIVE K=V cache
 *   then, at byte offset round_up(B * Hkv * cache_cap * d * sizeof(dtype), 256),
 *   [B][Hkv][cache_cap][2 n_rot]   the rotated heads
 * Decode takes the rotated dims of each key from the heads instead of rotating
 * them; it reads 1.25 d values per cached row instead of d.
 */
typedef enum { GA_CACHE_NATIVE = 0, GA_CACHE_INT8 = 1, GA_CACHE_PREROTATED = 2 } ga_cache_format;

/* Bytes of one cache tensor (k_cache; v_cache alike) of this layer. */
size_t gemma_attn_cache_bytes(const ga_layer* layer, int32_t batch, int32_t cache_cap);

/* Bytes of scratch gemma_attn_prefill needs for this batch and length. */
size_t gemma_attn_prefill_workspace_size(const ga_layer* layer, int32_t batch,
                                         int32_t seq_len);

/*
 * Prefill: causal attention over a whole prompt of seq_len tokens per sequence,
 * and the cache fill.  Implements the attention of each layer type as stated
 * above: QKNorm on q and k, (p-)RoPE at positions 0..S-1, GQA softmax attention
 * with V = normalised unrotated K on K=V layers and V = v otherwise.
 *
 *   q       [B, S, Hq, d]   raw (post-projection, pre-norm, unrotated)
 *   k       [B, S, Hkv, d]  raw
 *   v       [B, S, Hkv, d]  raw; must be NULL when kv_shared = 1
 *   q_gain, k_gain [d]      QKNorm gains
 *   k_cache [B, Hkv, cache_cap, d] or NULL (no cache write).
 *           K=V: slots 0..S-1 receive the normalised unrotated keys; needs
 *           cache_cap >= S.  Windowed: ring of cache_cap >= W slots receiving
 *           the normalised rotated keys of positions max(0, S-cache_cap)..S-1.
 *   v_cache like k_cache; windowed separate-V layers only (else NULL); gets v.
 *   out     [B, S, Hq, d]
 *   q, k, v, the gains, the caches and out are read and written in 16-byte
 *   pieces and must be 16-byte aligned (GA_EINVAL otherwise).
 *   workspace  >= gemma_attn_prefill_workspace_size() bytes, 256-byte aligned.
 * Errors: GA_EINVAL / GA_EUNSUPPORTED / GA_EWORKSPACE before any launch,
 * GA_EHIP if a launch fails.  seq_len = 0 or batch = 0 is a no-op (GA_OK).
 */
ga_status gemma_attn_prefill(const ga_layer* layer, int32_t batch, int32_t seq_len,
                             const void* q, const void* k, const void* v,
                             const void* q_gain, const void* k_gain,
                             void* k_cache, void* v_cache, int32_t cache_cap,
                             void* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Append one new token per sequence to the caches (decode step, before
 * gemma_attn_decode).  The cache grows by one position per generated token
 * as the context lengthens ("Gemma 4 技术报告：开源全模态密集 + MoE 模型家族，长上下文与
 * 端侧高效是本代核心", section "解决的真问题": the KV cache grows linearly with the
 * context; "Gemma 4 Technical Report" notes, §2 "Long-context efficiency").
 * On global K=V layers the row written is the one tensor that later serves as
 * both key and value ("Gemma 4多模态大模型架构详解", section "K=V"), so one
 * row per KV head is stored and no v_new is taken; on windowed layers only the
 * last W positions are kept ("交错层（局部与全局注意力）" of the same page).
 * The stored form follows the cache conventions above.
 *
 *   k_new   [B, Hkv, d] raw key of the new token;  v_new [B, Hkv, d] raw value
 *           (NULL when kv_shared = 1)
 *   k_gain  [d]
 *   positions  device int32 [B]: position of the new token of each sequence.
 *           K=V: slot = position; a position outside [0, cache_cap) writes
 *           nothing.  Windowed: slot = position mod W; a negative position
 *           writes nothing.
 *   k_cache, v_cache, cache_cap as for gemma_attn_prefill.
 */
ga_status kv_append(const ga_layer* layer, int32_t batch,
                    const void* k_new, const void* v_new, const void* k_gain,
                    const int32_t* positions, void* k_cache, void* v_cache,
                    int32_t cache_cap, void* stream);

/*
 * Prefill of a later chunk of a prompt against the positions already cached:
 * positions start .. start + chunk - 1 of each sequence attend causally (and
 * within the window on windowed layers) to positions 0 .. their own.  The
 * earlier positions come from the caches as a prefill, an earlier chunk or
 * kv_append wrote them: K=V and separate-V global layers from slots
 * 0 .. start - 1, windowed layers from their ring (which holds the last
 * cache_cap >= W positions before start, so every key the chunk sees).  The
 * chunk's keys (and values) are then written as gemma_attn_prefill writes
 * them: slots start .. start + chunk - 1, or the ring's slots of the last
 * cache_cap positions of the chunk.  Each output row is the row a prefill of
 * the whole prompt would give; this is also the longer form of checking many
 * new tokens at once (see gemma_attn_decode_multi).
 *
 *   q [B, chunk, Hq, d], k [B, chunk, Hkv, d] raw; v [B, chunk, Hkv, d] raw on
 *   layers with a separate V (NULL on K=V layers); out [B, chunk, Hq, d]
 *   k_cache, v_cache [B, Hkv, cache_cap, d]: global layers cache_cap >= start +
 *   chunk, windowed layers cache_cap >= W; v_cache NULL on K=V layers
 *   workspace >= gemma_attn_prefill_chunk_workspace_size() bytes, 256-byte
 *   aligned (the workspace of a prefill of start + chunk positions).
 * start = 0 is gemma_attn_prefill with the caches.  GA_EINVAL for start > 0
 * without k_cache; other errors as for gemma_attn_prefill.
 */
size_t gemma_attn_prefill_chunk_workspace_size(const ga_layer* layer, int32_t batch,
                                               int32_t start, int32_t chunk);
ga_status gemma_attn_prefill_chunk(const ga_layer* layer, int32_t batch, int32_t start,
                                   int32_t chunk, const void* q, const void* k, const void* v,
                                   const void* q_gain, const void* k_gain, void* k_cache,
                                   void* v_cache, int32_t cache_cap, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Bytes of scratch gemma_attn_decode needs: per-sequence tile offsets and the
 * split-K partial results (one per wave and visited segment).  Depends on the
 * layer, batch and max_seq_len only, never on the device.
 */
size_t gemma_attn_decode_workspace_size(const ga_layer* layer, int32_t batch,
                                        int32_t max_seq_len);

/*
 * Decode: one query token per sequence against its cache.  The query of the
 * newest position attends to every cached position of a global layer (full
 * causal) or to the last W of a windowed one ("Gemma 4多模态大模型架构详解",
 * section "交错层（局部与全局注意力）"), with the G query heads of a group reading
 * their one KV head (section "分组查询注意力").  On K=V layers the single cached
 * tensor is read once and used as keys, p-RoPE applied on the fly to its
 * leading 2 n_rot dims, and, unrotated, as values (section "K=V"; "Gemma 4
 * Technical Report" notes, §2 "Long-context efficiency", where key = value
 * on global layers cuts the KV cache).  The cache read grows with the context
 * ("Gemma 4 技术报告：开源全模态密集 + MoE 模型家族，长上下文与端侧高效是本代核心",
 * section "解决的真问题"), so this call is bound by HBM bandwidth.  A persistent
 * split-K pass (one workgroup per CU, each streaming an equal share of all
 * cached positions of all sequences and KV heads) is followed by a
 * log-sum-exp merge of the partial results.
 *
 *   q        [B, Hq, d] raw query of the new token, at position seq_lens[b]-1
 *   q_gain   [d]
 *   k_cache, v_cache, cache_cap: as written by prefill / kv_append (v_cache
 *            NULL when kv_shared = 1)
 *   seq_lens device int32 [B]: valid keys including the new token (L_b >= 1).
 *            Global layers read slots 0..L_b-1; windowed layers the
 *            min(L_b, cache_cap) filled ring slots, of which those inside the
 *            window are seen.
 *   max_seq_len host bound on every seq_lens[b], sizes the workspace.  A
 *            sequence with L_b < 1, L_b > max_seq_len or (K=V) L_b > cache_cap
 *            gets a NaN output row instead of reading out of bounds.
 *   out      [B, Hq, d]
 *   workspace >= gemma_attn_decode_workspace_size() bytes, 256-byte aligned.
 * GA_EUNSUPPORTED if one head's cache (cache_cap * d * element size) reaches
 * 2 GiB, if B * Hkv * ceil(max_seq_len / 16) exceeds 2^31 - 1, or for fp32
 * with d = 512 and a separate V cache.
 */
ga_status gemma_attn_decode(const ga_layer* layer, int32_t batch,
                            const void* q, const void* q_gain,
                            const void* k_cache, const void* v_cache,
                            int32_t cache_cap, const int32_t* seq_lens,
                            int32_t max_seq_len, void* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Multi-token decode: the last q_len positions of each sequence attend to its
 * cache in one pass, each causally (token j at position seq_lens[b] - q_len + j
 * sees keys 0 .. its own position).  This is the step in which the main model
 * checks the tokens its multi-token-prediction drafter proposed ("Gemma 4
 * Technical Report (translated notes)", section 2.6, MTP drafter); the cache
 * is streamed once for all q_len tokens.  The new tokens' keys must already be
 * in the cache (kv_append for each, or a prefill).
 *
 *   q        [B, q_len, Hq, d] raw queries of the new tokens
 *   out      [B, q_len, Hq, d]
 *   seq_lens device int32 [B]: valid keys including the q_len new tokens; a
 *            sequence with L_b < q_len gets NaN rows like an invalid length.
 *   other arguments as for gemma_attn_decode, with the workspace from
 *   gemma_attn_decode_multi_workspace_size().
 * Every layer type: global layers read slots 0 .. L_b - 1, windowed layers
 * their ring, token j seeing the positions inside its own window.  A
 * windowed layer needs a ring of cache_cap >= W + q_len - 1 slots (GA_EINVAL
 * otherwise): with W slots the later new tokens would have pushed out keys
 * the earlier ones still see.
 * One pass over the cache serves up to 32 query columns (q_len tokens x
 * Hq / Hkv heads; two groups of 16 that share the tiles): more tokens take
 * ceil(q_len (Hq / Hkv) / 32) passes, one after another on the stream,
 * sharing the workspace.
 * q_len = 1 is gemma_attn_decode.  GA_EINVAL for q_len < 1; GA_EUNSUPPORTED
 * when q_len * (Hq / Hkv) > 64.
 */
size_t gemma_attn_decode_multi_workspace_size(const ga_layer* layer, int32_t batch,
                                              int32_t q_len, int32_t max_seq_len);
ga_status gemma_attn_decode_multi(const ga_layer* layer, int32_t batch, int32_t q_len,
                                  const void* q, const void* q_gain,
                                  const void* k_cache, const void* v_cache,
                                  int32_t cache_cap, const int32_t* seq_lens,
                                  int32_t max_seq_len, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * gemma_attn_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace: the split-K scratch (per-sequence tile
 * offsets and partial results) is a static 32 MiB device array of the
 * library, one copy per GPU, held until the process ends.  On the first call
 * on a device the library looks up that copy's address and clears it with a
 * fill kernel on `stream`.  Nothing is allocated, by this call or the library.
 *
 * Arguments, layouts and results are those of gemma_attn_decode (the same
 * kernels and launch shape; the output matches it bit for bit).
 * GA_EWORKSPACE if the call would need more than 32 MiB of scratch (about
 * 4 * (CUs + batch * Hkv) * (G * d + 64) * 4 bytes, e.g. batch 64 with 4 KV
 * heads of G = 8, d = 512 on 256 CUs needs 32.5 MiB); use gemma_attn_decode
 * with a workspace then.  Every call on one GPU shares that GPU's array and
 * finds the previous call's contents there: calls that overlap on one GPU
 * (several streams, or several threads) race and must be serialised by the
 * caller.
 */
ga_status gemma_attn_decode_noalloc(const ga_layer* layer, int32_t batch,
                                    const void* q, const void* q_gain,
                                    const void* k_cache, const void* v_cache,
                                    int32_t cache_cap, const int32_t* seq_lens,
                                    int32_t max_seq_len, void* out, void* stream);

/*
 * Measurement hooks (not part of the computation).  While enabled, every
 * launch of the kernels below is bracketed by a pair of HIP events recorded
 * on the caller's stream; gemma_attn_profile_read() waits for the recorded
 * events and returns the summed elapsed milliseconds and the launch count of
 * one kernel: 0 prefill attention, 1 prefill prep (RoPE table + key/value
 * preparation), 2 decode split-K, 3 decode merge, 4 kv_append.  Returns 0, or
 * -1 if a HIP event call failed.  gemma_attn_profile_reset() destroys the
 * recorded events.  Host-side bookkeeping only; thread-safe.
 */
void gemma_attn_profile_enable(int on);
int gemma_attn_profile_read(int kernel, double* total_ms, int* count);
void gemma_attn_profile_reset(void);

/*
 * Calibration probes (measurement only, not part of the computation): the
 * rates this GPU reaches on the two resources the kernels above are bound by.
 * gemma_attn_calibrate_mfma: n_wgs workgroups of 4 waves, each wave running 4
 *   independent chains of `iters` 32x32x16 bf16 MFMAs (32768 flops each) on
 *   operands taken from `ops` (n_ops 16-byte pieces of bf16, device); `sink`
 *   (device, n_wgs * 256 floats) is written only to keep the chains alive.
 * gemma_attn_calibrate_stream: n_wgs workgroups read `bytes` (a multiple of
 *   16) of device memory at `buf` once, in 16-byte loads; `sink` (device,
 *   n_wgs unsigned ints) as above.
 * Both enqueue one kernel on `stream`; the caller times it.  GA_EINVAL for
 * NULL pointers or non-positive sizes, GA_EHIP if the launch fails.
 */
ga_status gemma_attn_calibrate_mfma(const void* ops, int32_t n_ops, int32_t iters, int32_t n_wgs,
                                    float* sink, void* stream);
ga_status gemma_attn_calibrate_stream(const void* buf, size_t bytes, int32_t n_wgs, unsigned* sink,
                                      void* stream);

/* Message for the last non-OK status returned to the calling thread. */
const char* gemma_attn_last_error(void);

/* Library version string. */
const char* gemma_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMMA_ATTN_H */
