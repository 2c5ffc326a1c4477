// Split-K decode: one query token per sequence against its cache, gfx950.
//
// Work item = (chunk of kDecodeChunk cached positions, KV head, sequence).  Each
// wave of the workgroup streams its share of the chunk in tiles of 16 keys:
//   global -> LDS by direct-to-LDS copies, two tiles per wave, the next tile
//   already in flight while the current one is computed (no register staging);
//   K=V layers: pairs 0..63 of every key are rotated on the fly as they are
//   loaded into the QK^T operand (p-RoPE of the "Gemma 4多模态大模型架构详解"
//   section "p-RoPE（低频剪枝旋转位置编码）"); the raw rows in LDS are the values
//   ("K=V" section of the same page);
//   S^T[key][head] = K~ Q~^T   (16x16x32 MFMA, the G heads padded to 16 columns)
//   online softmax per head (wave shuffles, exp2 domain)
//   O^T[d][head] += V^T P^T     (16x16x16 MFMA; V^T by LDS transpose reads, P
//                               straight from the S^T registers)
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
  static constexpr int kRotSteps = 2 * kRot / 32;     // QK^T steps that cover rotated dims
  static constexpr int kRowBytes = D * kSz;           // one key row
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kKBytes = KT * kRowBytes;      // key tile (the values too for K=V)
  static constexpr int kTileBytes = SHARED ? kKBytes : 2 * kKBytes;   // + value tile
  static constexpr int kBufs = 2;                     // tiles in LDS per wave
  static constexpr int kWaves = (4 * kBufs * kTileBytes <= 128 * 1024) ? 4 : 2;
  static constexpr int kPerWave = kDecodeChunk / kWaves;
  static constexpr int kQSteps = D / 32;              // QK^T reduction steps
  static constexpr int kDBlocks = D / 16;             // PV output blocks of 16 dims
  static constexpr int kDmaPerTile = kTileBytes / 1024;
  static constexpr int kWaveLds = kBufs * kTileBytes + 64 * 8;   // tiles + coarse angles
  static constexpr int kCombineBytes = kWaves * (G * D + 32) * 4;
  static constexpr int kLdsBytes = (kWaves * kWaveLds > kCombineBytes) ? kWaves * kWaveLds : kCombineBytes;
  static_assert(kChunksPerRow >= 16, "row swizzle needs 16 chunks per row");
  static_assert(kTileBytes % 1024 == 0 && kDmaPerTile < 64, "tile copy");
};

// Orders this wave's LDS accesses (compiler and hardware) around a tile reuse.
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vm_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Sequence b's number of readable keys, or -1 if its length is out of range.
__device__ __forceinline__ int decode_keys(const DecodeArgs& a, int b) {
  const int L = a.seq_lens[b];
  if (L < 1 || L > a.max_seq_len) return -1;
  if (a.window == 0 && L > a.cache_cap) return -1;
  return a.window > 0 ? min(L, a.window) : L;
}

// Key rows sit in LDS in natural order [key][d]; 16-byte chunk c of row r is
// stored at chunk c ^ (r & 15), so the 16 rows one QK^T operand read touches
// fall in distinct banks.
__device__ __forceinline__ int row_chunk(int r, int c) { return c ^ (r & 15); }

// Copy one tile (16 key rows, plus 16 value rows for separate-V layers) from
// global memory straight into LDS.  Each instruction moves 1 KiB: the lane
// fetches the global chunk that the swizzle places at its LDS slot.  Rows
// past the sequence read its last row (their scores are masked).
template <typename T, int D, int G, bool SHARED>
__device__ __forceinline__ void issue_tile(char* dst, const char* kbase, const char* vbase, int key0,
                                           int nkeys, int lane) {
  using C = DecodeCfg<T, D, G, SHARED>;
#pragma unroll
  for (int i = 0; i < C::kDmaPerTile; ++i) {
    const int off = (i % (C::kKBytes / 1024)) * 1024 + lane * 16;
    const int r = off / C::kRowBytes;
    const int pc = (off % C::kRowBytes) >> 4;
    const int key = min(key0 + r, nkeys - 1);
    const char* base = (SHARED || i < C::kKBytes / 1024) ? kbase : vbase;
    const char* src = base + static_cast<int64_t>(key) * C::kRowBytes + (row_chunk(r, pc) << 4);
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
  }
}

// The 8 elements of key row r starting at logical chunk c (QK^T A operand):
// one chunk for bf16, two for fp32.
__device__ __forceinline__ void row_frag(Frag8<bf16>& f, const char* row, int r, int c) {
  f.v = *reinterpret_cast<const bf16x8*>(row + (row_chunk(r, c) << 4));
}
__device__ __forceinline__ void row_frag(Frag8<float>& f, const char* row, int r, int c) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(row + (row_chunk(r, c) << 4));
  const f32x4 hi = *reinterpret_cast<const f32x4*>(row + (row_chunk(r, c + 1) << 4));
  f.v[0] = lo[0]; f.v[1] = lo[1]; f.v[2] = lo[2]; f.v[3] = lo[3];
  f.v[4] = hi[0]; f.v[5] = hi[1]; f.v[6] = hi[2]; f.v[7] = hi[3];
}

// V^T fragment for a 16x16x16 MFMA: lane l needs V[key 4(l/16) + j][d0 + l%16],
// j = 0..3.  bf16: one transpose read (within each 16-lane group, lane i gets
// element i%4 of the 8-byte pieces addressed by lanes i/4 + 4j); each lane
// addresses key 4(l/16) + (l%16)/4, dims d0 + 4 (l%4) .. +3.  fp32: four reads.
template <int kRowBytes>
__device__ __forceinline__ void vt_frag(Frag4<bf16>& f, const char* vt, int d0, int lane) {
  const int r = 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int byte = (d0 + 4 * (lane & 3)) * 2;
  const char* p = vt + r * kRowBytes + (row_chunk(r, byte >> 4) << 4) + (byte & 15);
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  f.v = __builtin_bit_cast(bf16x4, v);
}
template <int kRowBytes>
__device__ __forceinline__ void vt_frag(Frag4<float>& f, const char* vt, int d0, int lane) {
  const int d = d0 + (lane & 15);
  const int byte = d * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * (lane >> 4) + j;
    f.v[j] = *reinterpret_cast<const float*>(vt + r * kRowBytes + (row_chunk(r, byte >> 4) << 4) + (byte & 15));
  }
}

template <typename T, int D, int G, bool SHARED>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeArgs a) {
  using C = DecodeCfg<T, D, G, SHARED>;
  __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes];
  __shared__ float q_s[G][D];          // normalised, rotated, pre-scaled queries
  __shared__ f32x2 qcs[D / 2];         // (cos, sin) at the query position
  __shared__ float rstd_s[G];

  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int kThreads = C::kWaves * 64;
  const int nkeys = decode_keys(a, b);
  T* __restrict__ out = static_cast<T*>(a.out) + (static_cast<int64_t>(b) * a.n_q_heads + kvh * G) * D;
  if (nkeys < 0) {
    if (chunk == 0)
      for (int i = threadIdx.x; i < G * D; i += kThreads) out[i] = from_f32<T>(NAN);
    return;
  }
  const int c0 = chunk * kDecodeChunk;
  if (c0 >= nkeys) return;
  const int n_chunks = (nkeys + kDecodeChunk - 1) / kDecodeChunk;
  const int qpos = a.seq_lens[b] - 1;

  // ---- stream setup: start this wave's first two tile copies right away -----
  const int64_t head = static_cast<int64_t>(b) * a.n_kv_heads + kvh;
  const char* kbase = static_cast<const char*>(a.k_cache) + head * a.cache_cap * static_cast<int64_t>(C::kRowBytes);
  const char* vbase = SHARED ? kbase
                             : static_cast<const char*>(a.v_cache) + head * a.cache_cap * static_cast<int64_t>(C::kRowBytes);
  char* wlds = smem + wave * C::kWaveLds;
  f32x2* coarse_s = reinterpret_cast<f32x2*>(wlds + C::kBufs * C::kTileBytes);
  const int w0 = c0 + wave * C::kPerWave;
  const int w1 = min(w0 + C::kPerWave, nkeys);
  const int ntiles = w1 > w0 ? (w1 - w0 + C::KT - 1) / C::KT : 0;
  if (ntiles > 0) issue_tile<T, D, G, SHARED>(wlds, kbase, vbase, w0, nkeys, lane);
  if (ntiles > 1) issue_tile<T, D, G, SHARED>(wlds + C::kTileBytes, kbase, vbase, w0 + C::KT, nkeys, lane);

  // ---- query prep: QKNorm + rotation at qpos, into LDS --------------------------
  {
    const T* __restrict__ q = static_cast<const T*>(a.q) + (static_cast<int64_t>(b) * a.n_q_heads + kvh * G) * D;
    const T* __restrict__ gq = static_cast<const T*>(a.q_gain);
    for (int i = threadIdx.x; i < a.n_rot; i += kThreads)
      qcs[i] = rope_cos_sin(static_cast<double>(qpos) * rope_omega(i, D, a.log2_theta));
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
    for (int i = threadIdx.x; i < G * D / 2; i += kThreads) {
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

  // ---- K=V rotation factors ------------------------------------------------------
  // The lane's rotated QK^T fragments hold key (key0 + hcol) at pairs
  // i = 16u + 4kg + p (u < kRotSteps, p < 4).  cos/sin((key0 + hcol) w_i) =
  // coarse(key0 w_i) (x) fine(hcol w_i): fine stays in registers; coarse is
  // kept per pair (lane = pair), stepped by 16 w_i each tile and shared
  // through LDS.
  f32x2 fine[SHARED ? C::kRotSteps * 4 : 1];
  f32x2 coarse_l{}, step_l{};
  if constexpr (SHARED) {
#pragma unroll
    for (int u = 0; u < C::kRotSteps; ++u)
#pragma unroll
      for (int p = 0; p < 4; ++p)
        fine[4 * u + p] = rope_cos_sin(static_cast<double>(hcol) * rope_omega(16 * u + 4 * kg + p, D, a.log2_theta));
    const double w = rope_omega(lane, D, a.log2_theta);
    coarse_l = rope_cos_sin(static_cast<double>(w0) * w);
    step_l = rope_cos_sin(16.0 * w);
  }

  // ---- stream this wave's keys -----------------------------------------------------
  f32x4 o[C::kDBlocks];
#pragma unroll
  for (int t = 0; t < C::kDBlocks; ++t) o[t] = f32x4{};
  float m_run = -INFINITY, l_part = 0.f;
  constexpr float kTau = 8.0f;

  for (int it = 0; it < ntiles; ++it) {
    const int key0 = w0 + it * C::KT;
    const char* kt_lds = wlds + (it & 1) * C::kTileBytes;
    const char* vt_lds = SHARED ? kt_lds : kt_lds + C::kKBytes;
    // tile `it` has landed once at most the next tile's copies are in flight
    if (it + 1 < ntiles) wait_vm_le<C::kDmaPerTile>();
    else wait_vm_le<0>();

    // S^T = K~ Q~^T; the lane's A operand is key row hcol, dims 32u + 8kg .. +7
    f32x4 s = f32x4{};
    const char* krow = kt_lds + hcol * C::kRowBytes;
    if constexpr (SHARED) {
      coarse_s[lane] = coarse_l;
      lds_fence();
#pragma unroll
      for (int u = 0; u < C::kRotSteps; ++u) {
        Frag8<T> kf;
        row_frag(kf, krow, hcol, (32 * u + 8 * kg) * C::kSz / 16);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const f32x2 cb = coarse_s[16 * u + 4 * kg + p];
          const f32x2 fj = fine[4 * u + p];
          f32x2 cs;
          cs[0] = cb[0] * fj[0] - cb[1] * fj[1];
          cs[1] = cb[1] * fj[0] + cb[0] * fj[1];
          float x0 = to_f32(kf.v[2 * p]), x1 = to_f32(kf.v[2 * p + 1]);
          rotate_pair(x0, x1, cs);
          frag_set(kf, 2 * p, x0);
          frag_set(kf, 2 * p + 1, x1);
        }
        mma16(s, kf, qf[u]);
      }
      // next tile's coarse angle: advance by 16 positions
      const f32x2 c = coarse_l;
      coarse_l[0] = c[0] * step_l[0] - c[1] * step_l[1];
      coarse_l[1] = c[1] * step_l[0] + c[0] * step_l[1];
    }
#pragma unroll
    for (int u = C::kRotSteps; u < C::kQSteps; ++u) {
      Frag8<T> kf;
      row_frag(kf, krow, hcol, (32 * u + 8 * kg) * C::kSz / 16);
      mma16(s, kf, qf[u]);
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
    const bool rescale = __any(mt > m_run + kTau);
    const float m_new = rescale ? fmaxf(m_run, mt) : m_run;
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    m_run = m_new;
    Frag4<T> pf;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float p = __builtin_amdgcn_exp2f(s[v] - m_use);
      psum += p;
      frag_set(pf, v, p);
    }
    if (rescale) {
#pragma unroll
      for (int t = 0; t < C::kDBlocks; ++t) o[t] *= alpha;
      l_part *= alpha;
    }
    l_part += psum;

    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < C::kDBlocks; ++t) {
      Frag4<T> vf;
      vt_frag<C::kRowBytes>(vf, vt_lds, 16 * t, lane);
      mma16k16(o[t], vf, pf);
    }
    lds_fence();   // this tile's LDS reads are done before its buffer is refilled
    if (it + 2 < ntiles)
      issue_tile<T, D, G, SHARED>(wlds + (it & 1) * C::kTileBytes, kbase, vbase, key0 + 2 * C::KT, nkeys, lane);
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
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
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
  const int nkeys = decode_keys(a, b);
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
                                                      : hipErrorInvalidValue;   // not built (host rejects it)
  if (dtype == 1 && head_dim == 256) return kv_shared ? launch_g<float, 256, true>(a, group, batch, s, tm)
                                                      : launch_g<float, 256, false>(a, group, batch, s, tm);
  return hipErrorInvalidValue;
}

}  // namespace ga
