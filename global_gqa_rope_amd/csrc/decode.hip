// Split-K decode: one query token per sequence against its cache, gfx950.
//
// Work item = (chunk of kDecodeChunk cached positions, KV head, sequence).  Each
// wave of the workgroup streams a quarter of the chunk in tiles of 16 keys:
//   global loads (128-bit where the layout allows) -> registers, the next tile
//   already in flight while the current one is processed;
//   K=V layers: pairs 0..63 of every key are rotated on the fly (p-RoPE of the
//   "Gemma 4多模态大模型架构详解" section "p-RoPE（低频剪枝旋转位置编码）"), the raw
//   key is kept as the value ("K=V" section of the same page);
//   S^T[key][head] = K~ Q~^T   (16x16x32 MFMA, the G heads padded to 16 columns)
//   online softmax per head (wave shuffles, exp2 domain)
//   O^T[d][head] += V^T P^T     (16x16x16 MFMA, P straight from the S^T registers)
// The waves then merge through LDS into one partial (max, sum, o) per item, or
// the final row when the item is the sequence's only chunk; a second kernel
// merges the partials of longer sequences by log-sum-exp.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ga {

template <typename T, int D, int G, bool SHARED>
struct DecodeCfg {
  static constexpr int KT = 16;                       // keys per wave tile
  static constexpr int kSz = int(sizeof(T));
  static constexpr int kRot = SHARED ? 64 : 0;        // pairs rotated on the fly
  static constexpr int kHeadElems = 2 * kRot;         // dims 0..127 for K=V
  static constexpr int kRowBytes = D * kSz + 16;      // padded key row in LDS
  static constexpr int kVRowBytes = SHARED ? kHeadElems * kSz + 16 : kRowBytes;
  static constexpr int kWaveLds = KT * (kRowBytes + kVRowBytes);
  static constexpr int kWaves = (4 * kWaveLds <= 96 * 1024) ? 4 : 2;
  static constexpr int kPerWave = kDecodeChunk / kWaves;
  static constexpr int kTiles = kPerWave / KT;
  static constexpr int kQSteps = D / 32;              // QK^T reduction steps
  static constexpr int kDBlocks = D / 16;             // PV output blocks of 16 dims
  // register-staged tile: rotated head pairs (SHARED) + 16-byte chunks
  static constexpr int kTailChunks = SHARED ? (D - kHeadElems) * kSz / 16 : D * kSz / 16;  // per key
  static constexpr int kChunkLoads = KT * kTailChunks / 64 * (SHARED ? 1 : 2);  // per lane
  static constexpr int kCombineBytes = kWaves * (G * D + 32) * 4;
  static constexpr int kLdsBytes = (kWaves * kWaveLds > kCombineBytes) ? kWaves * kWaveLds : kCombineBytes;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Orders this wave's LDS accesses (compiler and hardware) around a tile reuse.
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <typename T, int D, int G, bool SHARED>
struct TileRegs {
  using C = DecodeCfg<T, D, G, SHARED>;
  using PairT = typename std::conditional<sizeof(T) == 2, uint32_t, uint64_t>::type;
  u32x4 chunk[C::kChunkLoads];
  PairT pair[SHARED ? C::KT : 1];   // K=V: the lane's rotary pair of each of the 16 keys
};

// Sequence b's number of readable keys, or -1 if its length is out of range.
__device__ __forceinline__ int decode_keys(const DecodeArgs& a, int b, bool shared) {
  const int L = a.seq_lens[b];
  if (L < 1 || L > a.max_seq_len) return -1;
  if (a.window == 0 && L > a.cache_cap) return -1;
  return a.window > 0 ? min(L, a.window) : L;
}

template <typename T, int D, int G, bool SHARED>
__device__ __forceinline__ void load_tile(TileRegs<T, D, G, SHARED>& r, const char* kbase, const char* vbase,
                                          int key0, int nkeys, int lane) {
  using C = DecodeCfg<T, D, G, SHARED>;
  constexpr int kGlobRow = D * C::kSz;
  if constexpr (SHARED) {
#pragma unroll
    for (int j = 0; j < C::KT; ++j) {
      const int key = min(key0 + j, nkeys - 1);
      const char* p = kbase + static_cast<int64_t>(key) * kGlobRow + lane * 2 * C::kSz;
      r.pair[j] = *reinterpret_cast<const typename TileRegs<T, D, G, SHARED>::PairT*>(p);
    }
#pragma unroll
    for (int i = 0; i < C::kChunkLoads; ++i) {
      const int q = i * 64 + lane;
      const int j = q / C::kTailChunks, c = q % C::kTailChunks;
      const int key = min(key0 + j, nkeys - 1);
      const char* p = kbase + static_cast<int64_t>(key) * kGlobRow + C::kHeadElems * C::kSz + c * 16;
      r.chunk[i] = *reinterpret_cast<const u32x4*>(p);
    }
  } else {
    constexpr int kHalf = C::kChunkLoads / 2;
#pragma unroll
    for (int i = 0; i < C::kChunkLoads; ++i) {
      const int q = (i % kHalf) * 64 + lane;
      const int j = q / C::kTailChunks, c = q % C::kTailChunks;
      const int key = min(key0 + j, nkeys - 1);
      const char* base = i < kHalf ? kbase : vbase;
      r.chunk[i] = *reinterpret_cast<const u32x4*>(base + static_cast<int64_t>(key) * kGlobRow + c * 16);
    }
  }
}

template <typename T>
__device__ __forceinline__ void unpack_pair(uint32_t w, float& x0, float& x1) {
  x0 = __uint_as_float(w << 16);
  x1 = __uint_as_float(w & 0xffff0000u);
}
__device__ __forceinline__ void unpack_pair_f(uint64_t w, float& x0, float& x1) {
  x0 = __uint_as_float(static_cast<uint32_t>(w));
  x1 = __uint_as_float(static_cast<uint32_t>(w >> 32));
}

template <typename T, int D, int G, bool SHARED>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeArgs a) {
  using C = DecodeCfg<T, D, G, SHARED>;
  __shared__ __attribute__((aligned(16))) char smem[C::kLdsBytes];
  __shared__ float q_s[G][D];          // normalised, rotated, pre-scaled queries
  __shared__ f32x2 qcs[D / 2];         // (cos, sin) at the query position
  __shared__ f32x2 fine[SHARED ? C::KT : 1][64];  // (cos, sin)(j * omega_pair)
  __shared__ float rstd_s[G];

  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nthreads = C::kWaves * 64;
  if (threadIdx.x >= nthreads) return;
  const int nkeys = decode_keys(a, b, SHARED);
  T* __restrict__ out = static_cast<T*>(a.out) + (static_cast<int64_t>(b) * a.n_q_heads + kvh * G) * D;
  if (nkeys < 0) {
    if (chunk == 0)
      for (int i = threadIdx.x; i < G * D; i += nthreads) out[i] = from_f32<T>(NAN);
    return;
  }
  const int c0 = chunk * kDecodeChunk;
  if (c0 >= nkeys) return;
  const int n_chunks = (nkeys + kDecodeChunk - 1) / kDecodeChunk;
  const int qpos = a.seq_lens[b] - 1;

  // ---- query prep: QKNorm + rotation at qpos, into LDS --------------------------
  {
    const T* __restrict__ q = static_cast<const T*>(a.q) + (static_cast<int64_t>(b) * a.n_q_heads + kvh * G) * D;
    const T* __restrict__ gq = static_cast<const T*>(a.q_gain);
    for (int i = threadIdx.x; i < a.n_rot; i += nthreads)
      qcs[i] = rope_cos_sin(static_cast<double>(qpos) * rope_omega(i, D, a.log2_theta));
    if constexpr (SHARED) {
      for (int i = threadIdx.x; i < C::KT * 64; i += nthreads) {
        const int j = i >> 6, pr = i & 63;
        fine[j][pr] = rope_cos_sin(static_cast<double>(j) * rope_omega(pr, D, a.log2_theta));
      }
    }
    for (int h = wave; h < G; h += C::kWaves) {
      float ss = 0.f;
      for (int d = lane; d < D; d += 64) {
        const float x = to_f32(q[h * D + d]);
        ss += x * x;
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) ss += wave_xor(ss, m);
      if (lane == 0) rstd_s[h] = 1.0f / sqrtf(ss / D + a.eps);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < G * D / 2; i += nthreads) {
      const int h = i / (D / 2), pr = i % (D / 2);
      float x0 = to_f32(q[h * D + 2 * pr]) * rstd_s[h] * to_f32(gq[2 * pr]);
      float x1 = to_f32(q[h * D + 2 * pr + 1]) * rstd_s[h] * to_f32(gq[2 * pr + 1]);
      if (pr < a.n_rot) rotate_pair(x0, x1, qcs[pr]);
      q_s[h][2 * pr] = x0 * a.qk_scale_log2;
      q_s[h][2 * pr + 1] = x1 * a.qk_scale_log2;
    }
    __syncthreads();
  }
  const int hcol = lane & 15, kg = lane >> 4;
  Frag8<T> qf[C::kQSteps];
#pragma unroll
  for (int u = 0; u < C::kQSteps; ++u)
#pragma unroll
    for (int j = 0; j < 8; ++j) frag_set(qf[u], j, hcol < G ? q_s[hcol][32 * u + 8 * kg + j] : 0.f);

  // ---- stream this wave's keys ---------------------------------------------------
  const int64_t head = static_cast<int64_t>(b) * a.n_kv_heads + kvh;
  constexpr int kGlobRow = D * C::kSz;
  const char* kbase = static_cast<const char*>(a.k_cache) + head * a.cache_cap * static_cast<int64_t>(kGlobRow);
  const char* vbase = SHARED ? nullptr
                             : static_cast<const char*>(a.v_cache) + head * a.cache_cap * static_cast<int64_t>(kGlobRow);
  char* kt_lds = smem + wave * C::kWaveLds;                 // [16][kRowBytes]
  char* vt_lds = kt_lds + C::KT * C::kRowBytes;             // [16][kVRowBytes]

  const int w0 = c0 + wave * C::kPerWave;
  const int w1 = min(w0 + C::kPerWave, nkeys);
  const int ntiles = w1 > w0 ? (w1 - w0 + C::KT - 1) / C::KT : 0;

  f32x4 o[C::kDBlocks];
#pragma unroll
  for (int t = 0; t < C::kDBlocks; ++t) o[t] = f32x4{};
  float m_run = -INFINITY, l_part = 0.f;
  constexpr float kTau = 8.0f;

  // One register tile: tile `it` is moved to LDS (rotating the K=V head pairs on
  // the way), then the same registers take the loads of tile it+1, which stay
  // in flight while tile `it` is computed from LDS.
  TileRegs<T, D, G, SHARED> buf;
  if (ntiles > 0) load_tile<T, D, G, SHARED>(buf, kbase, vbase, w0, nkeys, lane);
  for (int it = 0; it < ntiles; ++it) {
    const int key0 = w0 + it * C::KT;

    if constexpr (SHARED) {
      const double omega = rope_omega(lane, D, a.log2_theta);
      const f32x2 base = rope_cos_sin(static_cast<double>(key0) * omega);
#pragma unroll
      for (int j = 0; j < C::KT; ++j) {
        const f32x2 fj = fine[j][lane];
        f32x2 cs;
        cs[0] = base[0] * fj[0] - base[1] * fj[1];
        cs[1] = base[1] * fj[0] + base[0] * fj[1];
        float x0, x1;
        if constexpr (sizeof(T) == 2) unpack_pair<T>(buf.pair[j], x0, x1);
        else unpack_pair_f(buf.pair[j], x0, x1);
        *reinterpret_cast<typename TileRegs<T, D, G, SHARED>::PairT*>(vt_lds + j * C::kVRowBytes + lane * 2 * C::kSz) = buf.pair[j];
        rotate_pair(x0, x1, cs);
        T* dst = reinterpret_cast<T*>(kt_lds + j * C::kRowBytes + lane * 2 * C::kSz);
        dst[0] = from_f32<T>(x0);
        dst[1] = from_f32<T>(x1);
      }
#pragma unroll
      for (int i = 0; i < C::kChunkLoads; ++i) {
        const int q = i * 64 + lane;
        const int j = q / C::kTailChunks, c = q % C::kTailChunks;
        *reinterpret_cast<u32x4*>(kt_lds + j * C::kRowBytes + C::kHeadElems * C::kSz + c * 16) = buf.chunk[i];
      }
    } else {
      constexpr int kHalf = C::kChunkLoads / 2;
#pragma unroll
      for (int i = 0; i < C::kChunkLoads; ++i) {
        const int q = (i % kHalf) * 64 + lane;
        const int j = q / C::kTailChunks, c = q % C::kTailChunks;
        char* base = i < kHalf ? kt_lds : vt_lds;
        *reinterpret_cast<u32x4*>(base + j * C::kRowBytes + c * 16) = buf.chunk[i];
      }
    }
    lds_fence();   // this wave's LDS writes are complete before any lane reads them
    if (it + 1 < ntiles) load_tile<T, D, G, SHARED>(buf, kbase, vbase, key0 + C::KT, nkeys, lane);

    // S^T = K~ Q~^T
    f32x4 s = f32x4{};
    {
      const char* krow = kt_lds + hcol * C::kRowBytes;
#pragma unroll
      for (int u = 0; u < C::kQSteps; ++u) {
        Frag8<T> kf;
        load_frag(kf, reinterpret_cast<const T*>(krow + (32 * u + 8 * kg) * C::kSz));
        mma16(s, kf, qf[u]);
      }
    }
    // online softmax; lane holds keys 4*kg + v of head column hcol
    float mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (key0 + 4 * kg + v >= w1) s[v] = -INFINITY;
      mt = fmaxf(mt, s[v]);
    }
    mt = fmaxf(mt, wave_xor(mt, 16));
    mt = fmaxf(mt, wave_xor(mt, 32));
    if (__any(mt > m_run + kTau)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int t = 0; t < C::kDBlocks; ++t) o[t] *= alpha;
      l_part *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    Frag4<T> pf;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float p = __builtin_amdgcn_exp2f(s[v] - m_use);
      l_part += p;
      frag_set(pf, v, p);
    }
    // O^T += V^T P^T: lane reads V[4*kg + j][16 t + hcol]
#pragma unroll
    for (int t = 0; t < C::kDBlocks; ++t) {
      const int d = 16 * t + hcol;
      const char* col;
      int stride;
      if (SHARED && d < C::kHeadElems) {
        col = vt_lds + d * C::kSz;
        stride = C::kVRowBytes;
      } else {
        col = (SHARED ? kt_lds : vt_lds) + d * C::kSz;
        stride = C::kRowBytes;
      }
      Frag4<T> vf;
#pragma unroll
      for (int j = 0; j < 4; ++j) vf.v[j] = *reinterpret_cast<const T*>(col + (4 * kg + j) * stride);
      mma16k16(o[t], vf, pf);
    }
    lds_fence();   // reads of this tile finish before the next tile overwrites it
  }

  // ---- merge the waves of this item ------------------------------------------------
  float l = l_part + wave_xor(l_part, 16);
  l += wave_xor(l, 32);
  __syncthreads();
  float* comb = reinterpret_cast<float*>(smem);          // [wave][G*D + 32]
  float* mine = comb + wave * (G * D + 32);
  if (hcol < G) {
#pragma unroll
    for (int t = 0; t < C::kDBlocks; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) mine[hcol * D + 16 * t + 4 * kg + v] = o[t][v];
    if (kg == 0) {
      mine[G * D + hcol] = m_run;
      mine[G * D + 16 + hcol] = l;
    }
  }
  __syncthreads();
  float* part = a.partials + ((head * a.n_chunks + chunk) * G) * (D + 2);
  for (int i = threadIdx.x; i < G * D; i += nthreads) {
    const int h = i / D, d = i % D;
    float M = -INFINITY;
    for (int w = 0; w < C::kWaves; ++w) M = fmaxf(M, comb[w * (G * D + 32) + G * D + h]);
    float L = 0.f, O = 0.f;
    for (int w = 0; w < C::kWaves; ++w) {
      const float* cw = comb + w * (G * D + 32);
      const float mw = cw[G * D + h];
      const float e = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += e * cw[G * D + 16 + h];
      O += e * cw[h * D + d];
    }
    if (n_chunks == 1) {
      out[h * D + d] = from_f32<T>(O / L);
    } else {
      part[h * (D + 2) + 2 + d] = O;
      if (d == 0) {
        part[h * (D + 2)] = M;
        part[h * (D + 2) + 1] = L;
      }
    }
  }
}

// Log-sum-exp merge of the chunk partials of one (sequence, query head): the
// chunk weights exp2(m_c - M) are computed once into LDS, then each thread
// accumulates whole head dims across chunks (consecutive threads, consecutive
// dims).
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float wgt[1024];
  __shared__ float red[256];
  const int h = blockIdx.x % G, kvh = blockIdx.x / G, b = blockIdx.y;
  const int nkeys = decode_keys(a, b, false);
  if (nkeys < 0) return;
  const int n_chunks = (nkeys + kDecodeChunk - 1) / kDecodeChunk;
  if (n_chunks <= 1) return;
  const int64_t head = static_cast<int64_t>(b) * a.n_kv_heads + kvh;
  const float* part = a.partials + head * a.n_chunks * G * (D + 2) + h * (D + 2);
  constexpr int kStride = G * (D + 2);          // floats between chunks
  const int t = threadIdx.x;

  float mx = -INFINITY;
  for (int c = t; c < n_chunks; c += 256) mx = fmaxf(mx, part[c * kStride]);
  red[t] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] = fmaxf(red[t], red[t + s]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float lsum = 0.f;
  for (int c = t; c < n_chunks; c += 256) {
    const float w = __builtin_amdgcn_exp2f(part[c * kStride] - M);
    wgt[c] = w;
    lsum += w * part[c * kStride + 1];
  }
  red[t] = lsum;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  const float inv = 1.0f / red[0];
  T* __restrict__ out = static_cast<T*>(a.out) + (static_cast<int64_t>(b) * a.n_q_heads + kvh * G + h) * D;
  for (int d = t; d < D; d += 256) {
    float o = 0.f;
    for (int c = 0; c < n_chunks; ++c) o += wgt[c] * part[c * kStride + 2 + d];
    out[d] = from_f32<T>(o * inv);
  }
}

template <typename T, int D, int G, bool SHARED>
static hipError_t launch_one(const DecodeArgs& a, int batch, hipStream_t s, LaunchTimer timer) {
  using C = DecodeCfg<T, D, G, SHARED>;
  if (timer) timer(s, 2, true);
  hipLaunchKernelGGL((decode_kernel<T, D, G, SHARED>), dim3(a.n_chunks, a.n_kv_heads, batch),
                     dim3(C::kWaves * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (timer) timer(s, 2, false);
  if (e != hipSuccess || a.n_chunks <= 1) return e;
  if (timer) timer(s, 3, true);
  hipLaunchKernelGGL((decode_merge_kernel<T, D, G>), dim3(a.n_kv_heads * G, batch), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (timer) timer(s, 3, false);
  return e;
}

template <typename T, int D, bool SHARED>
static hipError_t launch_g(const DecodeArgs& a, int group, int batch, hipStream_t s, LaunchTimer tm) {
  switch (group) {
    case 1: return launch_one<T, D, 1, SHARED>(a, batch, s, tm);
    case 2: return launch_one<T, D, 2, SHARED>(a, batch, s, tm);
    case 4: return launch_one<T, D, 4, SHARED>(a, batch, s, tm);
    case 8: return launch_one<T, D, 8, SHARED>(a, batch, s, tm);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group, int kv_shared,
                         int batch, hipStream_t s, LaunchTimer tm) {
  if (dtype == 0 && head_dim == 512) return kv_shared ? launch_g<bf16, 512, true>(a, group, batch, s, tm)
                                                      : launch_g<bf16, 512, false>(a, group, batch, s, tm);
  if (dtype == 0 && head_dim == 256) return kv_shared ? launch_g<bf16, 256, true>(a, group, batch, s, tm)
                                                      : launch_g<bf16, 256, false>(a, group, batch, s, tm);
  if (dtype == 1 && head_dim == 512) return kv_shared ? launch_g<float, 512, true>(a, group, batch, s, tm)
                                                      : launch_g<float, 512, false>(a, group, batch, s, tm);
  if (dtype == 1 && head_dim == 256) return kv_shared ? launch_g<float, 256, true>(a, group, batch, s, tm)
                                                      : launch_g<float, 256, false>(a, group, batch, s, tm);
  return hipErrorInvalidValue;
}

}  // namespace ga
