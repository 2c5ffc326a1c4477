// Flash-style causal prefill for one layer type, gfx950.
//
// A workgroup owns one KV head of one sequence and QB consecutive query
// positions: all G query heads of the group at those positions share every key
// tile it stages in LDS (the grouped-query sharing of "Gemma 4多模态大模型架构详解",
// section "分组查询注意力").  Its 128 query rows (QB positions x G heads) are
// split over eight waves of 16 rows, two waves per SIMD.  Per key tile of 32
// positions each wave computes, over the full head dim:
//   S^T[key][row] = K~ Q~^T      16x16x32 bf16 MFMAs, A = key fragments read
//                                from LDS, B = the wave's normalised, rotated
//                                queries held in registers
//   online softmax per row        in registers, exp2 domain
//   O^T[d][row] += V^T P^T        16x16x32 MFMAs; P goes from the score
//                                registers into the B operand unchanged
// Each wave keeps 16 rows x d fp32 accumulators (128 registers at d = 512).
//
// Key tiles (rotated normalised keys) and value tiles come from the prep pass
// already laid out in MFMA operand order, so each is copied global -> LDS by
// linear direct-to-LDS loads (two stages) and every operand read is 1 KiB of
// consecutive LDS bytes.  K=V layers get the normalised unrotated key as the
// value tile, so one cached tensor feeds both products ("Gemma 4多模态大模型架构
// 详解", section "K=V").  Windowed layers start at the first tile that can hold
// a visible key and mask keys with j <= i - W (section "交错层（局部与全局注意力）").
#include "common.h"
#include "kernels.h"

namespace ga {

template <typename T, int D, int G>
struct PrefillCfg {
  static constexpr int KT = kPrepTile;              // keys per tile
  static constexpr int kWaves = 8;
  static constexpr int kRows = 16;                  // query rows per wave
  static constexpr int PW = kRows / G;              // positions per wave
  static constexpr int QB = kWaves * PW;            // positions per workgroup
  static constexpr int kQSteps = D / 32;            // QK^T reduction steps
  static constexpr int kDBlocks = D / 16;           // 16-dim output blocks
  static constexpr int kSz = int(sizeof(T));
  static constexpr int kFrag = frag_bytes<T>();
  static constexpr int kKTileBytes = KT * D * kSz;
  static constexpr int kVTileBytes = KT * D * kSz;
  static constexpr int kStageBytes = kKTileBytes + kVTileBytes;
  static constexpr int kLdsCap = 160 * 1024;
  static constexpr int kStages = (2 * kStageBytes <= kLdsCap) ? 2 : 1;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static_assert(kLdsBytes <= kLdsCap, "LDS budget");
  static_assert(kKTileBytes % (1024 * kWaves) == 0, "tile split");
};

// This lane's 8 elements of an operand-ordered fragment (see frag_elem_off):
// one (bf16) or two (fp32) 16-byte reads, consecutive lanes at consecutive
// addresses.
__device__ __forceinline__ void frag_read(Frag8<bf16>& f, const char* frag, int lane) {
  f.v = *reinterpret_cast<const bf16x8*>(frag + lane * 16);
}
__device__ __forceinline__ void frag_read(Frag8<float>& f, const char* frag, int lane) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(frag + lane * 16);
  const f32x4 b = *reinterpret_cast<const f32x4*>(frag + 1024 + lane * 16);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Direct-to-LDS copy of one key tile and one value tile (both already in
// operand order, so the copy is linear).  Each instruction moves 64 lanes x
// 16 B into 1 KiB of consecutive LDS bytes.
template <typename T, int D, int G>
__device__ __forceinline__ void issue_tile(const char* __restrict__ ksrc, const char* __restrict__ vsrc,
                                           char* kdst, char* vdst, int wave, int lane) {
  using C = PrefillCfg<T, D, G>;
  const char* ks = ksrc + wave * 1024 + lane * 16;
  const char* vs = vsrc + wave * 1024 + lane * 16;
#pragma unroll
  for (int k = 0; k < C::kKTileBytes / 1024 / C::kWaves; ++k) {
    const int i = k * C::kWaves + wave;
    __builtin_amdgcn_global_load_lds(ks + k * C::kWaves * 1024,
                                     (__attribute__((address_space(3))) void*)(kdst + i * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < C::kVTileBytes / 1024 / C::kWaves; ++k) {
    const int i = k * C::kWaves + wave;
    __builtin_amdgcn_global_load_lds(vs + k * C::kWaves * 1024,
                                     (__attribute__((address_space(3))) void*)(vdst + i * 1024), 16, 0, 0);
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(512, 1) void prefill_attn_kernel(PrefillArgs a) {
  using C = PrefillCfg<T, D, G>;
  __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes];

  const int n_qb = (a.seq_len + C::QB - 1) / C::QB;
  const int qb = n_qb - 1 - static_cast<int>(blockIdx.x);   // longest causal rows first
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;                     // row of this lane, reduction group
  const int p0 = qb * C::QB;
  const int pos = p0 + wave * C::PW + m / G;                  // query position of row m
  const int qh = kvh * G + (m % G);                           // query head of row m
  const bool row_valid = pos < a.seq_len;

  // ---- prologue: QKNorm + rotation of query row m (this lane's quarter) ------
  Frag8<T> qf[C::kQSteps];
  {
    const T* __restrict__ q = static_cast<const T*>(a.q) +
        ((static_cast<int64_t>(b) * a.seq_len + (row_valid ? pos : 0)) * a.n_q_heads + qh) * D;
    const T* __restrict__ gq = static_cast<const T*>(a.q_gain);
    const f32x2* __restrict__ table = static_cast<const f32x2*>(a.rope_table) +
                                      static_cast<int64_t>(row_valid ? pos : 0) * a.n_rot;
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < C::kQSteps; ++u) {
      load_frag(qf[u], q + 32 * u + 8 * g);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += to_f32(qf[u].v[j]) * to_f32(qf[u].v[j]);
    }
    ss += wave_xor(ss, 16);
    ss += wave_xor(ss, 32);
    const float rs = row_valid ? (1.0f / sqrtf(ss / D + a.eps)) * a.qk_scale_log2 : 0.f;
#pragma unroll
    for (int u = 0; u < C::kQSteps; ++u) {
      const int d0 = 32 * u + 8 * g;
      Frag8<T> gain;
      load_frag(gain, gq + d0);
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = to_f32(qf[u].v[j]) * rs * to_f32(gain.v[j]);
      if (d0 < 2 * a.n_rot) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x2 cs = table[min(d0 / 2 + j, a.n_rot - 1)];
          if (d0 / 2 + j < a.n_rot) rotate_pair(x[2 * j], x[2 * j + 1], cs);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) frag_set(qf[u], j, x[j]);
    }
  }

  // ---- key tile range ----------------------------------------------------------
  const int p_last = min(p0 + C::QB, a.seq_len) - 1;
  const int kt_lo = a.window > 0 ? max(0, p0 - a.window + 1) / C::KT : 0;
  const int kt_hi = p_last / C::KT + 1;
  const int64_t head = static_cast<int64_t>(b) * a.n_kv_heads + kvh;
  const int64_t n_tiles = a.seq_pad / C::KT;
  const char* kbase = static_cast<const char*>(a.ws_k) + head * n_tiles * C::kKTileBytes;
  const char* vbase = static_cast<const char*>(a.ws_vt) + head * n_tiles * C::kVTileBytes;
  const int w_first = p0 + wave * C::PW;            // this wave's first and last query position
  const int w_last = w_first + C::PW - 1;

  f32x4 o[C::kDBlocks];
#pragma unroll
  for (int t = 0; t < C::kDBlocks; ++t) o[t] = f32x4{};
  float m_run = -INFINITY, l_part = 0.f;
  constexpr float kTau = 8.0f;   // rescale only when the running max grows by > 2^8

  issue_tile<T, D, G>(kbase + static_cast<int64_t>(kt_lo) * C::kKTileBytes,
                      vbase + static_cast<int64_t>(kt_lo) * C::kVTileBytes,
                      smem, smem + C::kKTileBytes, wave, lane);

  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int stage = C::kStages == 2 ? ((kt - kt_lo) & 1) : 0;
    const char* ks = smem + stage * C::kStageBytes;
    const char* vs = ks + C::kKTileBytes;
    wait_vm_all();
    __syncthreads();   // tile kt visible; every wave is past iteration kt-1
    if (C::kStages == 2 && kt + 1 < kt_hi) {
      char* kn = smem + (stage ^ 1) * C::kStageBytes;
      issue_tile<T, D, G>(kbase + static_cast<int64_t>(kt + 1) * C::kKTileBytes,
                          vbase + static_cast<int64_t>(kt + 1) * C::kVTileBytes,
                          kn, kn + C::kKTileBytes, wave, lane);
    }
    const int key0 = kt * C::KT;
    if (key0 > w_last) continue;   // tile entirely above this wave's diagonal

    // S^T for key blocks 0 (keys 0..15) and 1 (keys 16..31)
    f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
    for (int u = 0; u < C::kQSteps; ++u) {
      Frag8<T> k0, k1;
      frag_read(k0, ks + (2 * u) * C::kFrag, lane);
      frag_read(k1, ks + (2 * u + 1) * C::kFrag, lane);
      mma16(s0, k0, qf[u]);
      mma16(s1, k1, qf[u]);
    }

    // mask + online softmax (column m of S^T is query row m); this lane holds
    // keys 4g + v (s0) and 16 + 4g + v (s1)
    const bool need_mask = (key0 + C::KT - 1 > w_first) ||
                           (a.window > 0 && key0 <= w_last - a.window);
    if (need_mask) {
      const int lo = a.window > 0 ? pos - a.window : -1;   // visible keys: lo < key <= pos
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int k_a = key0 + 4 * g + v, k_b = k_a + 16;
        s0[v] = (k_a <= pos && k_a > lo) ? s0[v] : -INFINITY;
        s1[v] = (k_b <= pos && k_b > lo) ? s1[v] : -INFINITY;
      }
    }
    float mt = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
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
    Frag8<T> pf;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float pa = __builtin_amdgcn_exp2f(s0[v] - m_use);
      const float pb = __builtin_amdgcn_exp2f(s1[v] - m_use);
      l_part += pa + pb;
      frag_set(pf, v, pa);
      frag_set(pf, 4 + v, pb);
    }

    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < C::kDBlocks; ++t) {
      Frag8<T> vf;
      frag_read(vf, vs + t * C::kFrag, lane);
      mma16(o[t], vf, pf);
    }

    if (C::kStages == 1 && kt + 1 < kt_hi) {
      __syncthreads();
      issue_tile<T, D, G>(kbase + static_cast<int64_t>(kt + 1) * C::kKTileBytes,
                          vbase + static_cast<int64_t>(kt + 1) * C::kVTileBytes,
                          smem, smem + C::kKTileBytes, wave, lane);
    }
  }

  // ---- epilogue ------------------------------------------------------------------
  float l = l_part + wave_xor(l_part, 16);
  l += wave_xor(l, 32);
  if (!row_valid) return;
  const float inv = 1.0f / l;
  T* __restrict__ out = static_cast<T*>(a.out) +
      ((static_cast<int64_t>(b) * a.seq_len + pos) * a.n_q_heads + qh) * D + 4 * g;
#pragma unroll
  for (int t = 0; t < C::kDBlocks; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) out[16 * t + v] = from_f32<T>(o[t][v] * inv);
}

template <typename T, int D, int G>
static hipError_t launch_one(const PrefillArgs& a, int batch, hipStream_t s) {
  using C = PrefillCfg<T, D, G>;
  const int n_qb = (a.seq_len + C::QB - 1) / C::QB;
  hipLaunchKernelGGL((prefill_attn_kernel<T, D, G>), dim3(n_qb, a.n_kv_heads, batch), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_d(const PrefillArgs& a, int group, int batch, hipStream_t s) {
  switch (group) {
    case 1: return launch_one<T, D, 1>(a, batch, s);
    case 2: return launch_one<T, D, 2>(a, batch, s);
    case 4: return launch_one<T, D, 4>(a, batch, s);
    case 8: return launch_one<T, D, 8>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_attn(const PrefillArgs& a, int dtype, int head_dim, int group, int batch,
                               hipStream_t s) {
  if (dtype == 0 && head_dim == 512) return launch_d<bf16, 512>(a, group, batch, s);
  if (dtype == 0 && head_dim == 256) return launch_d<bf16, 256>(a, group, batch, s);
  if (dtype == 1 && head_dim == 512) return launch_d<float, 512>(a, group, batch, s);
  if (dtype == 1 && head_dim == 256) return launch_d<float, 256>(a, group, batch, s);
  return hipErrorInvalidValue;
}

}  // namespace ga
