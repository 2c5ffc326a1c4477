// Flash-style causal prefill for one layer type, gfx950.
//
// A workgroup owns one KV head of one sequence and QB consecutive query
// positions: all G query heads of the group at those positions share every key
// tile it stages in LDS (the grouped-query sharing of "Gemma 4多模态大模型架构详解",
// section "分组查询注意力").  The 128 query rows (QB positions x G heads) form 4
// row groups of 32; eight waves run as 4 row groups x 2 halves of the head
// dim, two waves per SIMD:
//   S^T[key][row] (partial over this wave's half of d) = K~ Q~^T
//                                 32x32x16 MFMAs, A = key rows from LDS,
//                                 B = the wave's normalised, rotated queries
//   partner waves add their partial scores through LDS
//   online softmax per row          in registers, exp2 domain (both partners
//                                   compute it identically)
//   O^T[d][row] += V^T P^T          32x32x16 MFMAs over this wave's half of d
// Splitting d keeps the output accumulator at 128 registers for d = 512, so it
// and the score accumulator fit the accumulation registers together.
//
// Key tiles (rotated normalised keys) and value tiles come from the prep pass
// already laid out in MFMA operand order, so each is copied global -> LDS by
// linear direct-to-LDS loads (two stages when they fit) and every operand read
// is 1 KiB of consecutive LDS bytes.  K=V layers get the normalised unrotated key as the value
// tile, so one cached tensor feeds both products ("Gemma 4多模态大模型架构详解",
// section "K=V").  Windowed layers start at the first tile that can hold a
// visible key and mask keys with j <= i - W (section "交错层（局部与全局注意力）").
#include "common.h"
#include "kernels.h"

namespace ga {

template <typename T, int D, int G>
struct PrefillCfg {
  static constexpr int KT = kPrepTile;              // keys per tile
  static constexpr int kWaves = 8;
  static constexpr int kRows = 32;                  // query rows per row group
  static constexpr int PW = kRows / G;              // positions per row group
  static constexpr int QB = 4 * PW;                 // positions per workgroup
  static constexpr int kDHalf = D / 2;              // head dims per wave
  static constexpr int kSteps = kDHalf / 16;        // QK^T reduction steps per wave
  static constexpr int kDBlocks = kDHalf / 32;      // 32-dim output blocks per wave
  static constexpr int kSz = int(sizeof(T));
  static constexpr int kRowBytes = D * kSz;         // key row
  static constexpr int kKTileBytes = KT * kRowBytes;
  static constexpr int kVtRowBytes = KT * kSz;      // value tile row: 32 keys of one dim
  static constexpr int kVTileBytes = D * kVtRowBytes;
  static constexpr int kStageBytes = kKTileBytes + kVTileBytes;
  static constexpr int kXBytes = kWaves * 16 * 64 * 4;   // partial score exchange
  static constexpr int kLdsCap = 160 * 1024;
  static constexpr int kStages = (2 * kStageBytes + kXBytes <= kLdsCap) ? 2 : 1;
  static constexpr int kLdsBytes = kStages * kStageBytes + kXBytes;
  static_assert(kLdsBytes <= kLdsCap, "LDS budget");
  static_assert(kKTileBytes % (1024 * kWaves) == 0 && kVTileBytes % (1024 * kWaves) == 0, "tile split");
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
#pragma unroll
  for (int k = 0; k < C::kKTileBytes / 1024 / C::kWaves; ++k) {
    const int i = k * C::kWaves + wave;
    __builtin_amdgcn_global_load_lds(ksrc + i * 1024 + lane * 16,
                                     (__attribute__((address_space(3))) void*)(kdst + i * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < C::kVTileBytes / 1024 / C::kWaves; ++k) {
    const int i = k * C::kWaves + wave;
    __builtin_amdgcn_global_load_lds(vsrc + i * 1024 + lane * 16,
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
  const int rg = wave & 3, dh = wave >> 2;                    // row group, half of d
  const int m = lane & 31, g = lane >> 5;
  const int p0 = qb * C::QB;
  const int pos = p0 + rg * C::PW + m / G;                    // query position of row m
  const int qh = kvh * G + (m % G);                           // query head of row m
  const bool row_valid = pos < a.seq_len;
  const int dbase = dh * C::kDHalf;

  // ---- prologue: QKNorm + rotation of query row m, this wave's half of d ----
  // Pass 1 sums squares over the whole row, pass 2 forms the B operand.
  Frag8<T> qf[C::kSteps];
  {
    const T* __restrict__ q = static_cast<const T*>(a.q) +
        ((static_cast<int64_t>(b) * a.seq_len + (row_valid ? pos : 0)) * a.n_q_heads + qh) * D;
    const T* __restrict__ gq = static_cast<const T*>(a.q_gain);
    const f32x2* __restrict__ table = static_cast<const f32x2*>(a.rope_table) +
                                      static_cast<int64_t>(row_valid ? pos : 0) * a.n_rot;
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < 2 * C::kSteps; ++u) {
      Frag8<T> raw;
      load_frag(raw, q + 16 * u + 8 * g);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += to_f32(raw.v[j]) * to_f32(raw.v[j]);
    }
    ss += wave_xor(ss, 32);
    const float rs = row_valid ? (1.0f / sqrtf(ss / D + a.eps)) * a.qk_scale_log2 : 0.f;
#pragma unroll
    for (int u = 0; u < C::kSteps; ++u) {
      const int d0 = dbase + 16 * u + 8 * g;
      Frag8<T> raw, gain;
      load_frag(raw, q + d0);
      load_frag(gain, gq + d0);
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = to_f32(raw.v[j]) * rs * to_f32(gain.v[j]);
      if (d0 < 2 * a.n_rot) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (d0 / 2 + j < a.n_rot) rotate_pair(x[2 * j], x[2 * j + 1], table[d0 / 2 + j]);
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
  const char* kbase = static_cast<const char*>(a.ws_k) +
                      head * (a.seq_pad / C::KT) * static_cast<int64_t>(C::kKTileBytes);
  const char* vbase = static_cast<const char*>(a.ws_vt) +
                      head * (a.seq_pad / C::KT) * static_cast<int64_t>(C::kVTileBytes);
  float* xs = reinterpret_cast<float*>(smem + C::kStages * C::kStageBytes);   // [wave][16][64]

  f32x16 o[C::kDBlocks];
#pragma unroll
  for (int t = 0; t < C::kDBlocks; ++t) o[t] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;
  constexpr float kTau = 8.0f;   // rescale only when the running max grows by > 2^8

  constexpr int kFrag = frag_bytes<T>();
  const int kfrag0 = (dbase / 16) * kFrag;          // first key fragment of this half
  const int vfrag0 = (dbase / 32) * 2 * kFrag;      // first value fragment of this half

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

    // partial S^T over this wave's half of d
    f32x16 s = f32x16{};
#pragma unroll
    for (int u = 0; u < C::kSteps; ++u) {
      Frag8<T> kf;
      frag_read(kf, ks + kfrag0 + u * kFrag, lane);
      mma32(s, kf, qf[u]);
    }
    // add the partner wave's half
#pragma unroll
    for (int v = 0; v < 16; ++v) xs[(wave * 16 + v) * 64 + lane] = s[v];
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float mine = s[v];
      const float other = xs[((wave ^ 4) * 16 + v) * 64 + lane];
      s[v] = dh == 0 ? mine + other : other + mine;   // same order in both waves
    }

    // mask + online softmax (column m of S^T is query row m)
    const int key0 = kt * C::KT;
    const bool need_mask = (key0 + C::KT - 1 > p0 + rg * C::PW) ||
                           (a.window > 0 && key0 <= p0 + (rg + 1) * C::PW - 1 - a.window);
    if (need_mask) {
      const int lo = a.window > 0 ? pos - a.window : -1;   // visible keys: lo < key <= pos
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + 8 * (v >> 2) + 4 * g + (v & 3);
        s[v] = (key <= pos && key > lo) ? s[v] : -INFINITY;
      }
    }
    float mt = s[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mt = fmaxf(mt, s[v]);
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
    Frag8<T> pf[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = __builtin_amdgcn_exp2f(s[v] - m_use);
      l_part += p;
      frag_set(pf[v >> 3], v & 7, p);
    }

    // O^T += V^T P^T over this wave's half of d
#pragma unroll
    for (int t = 0; t < C::kDBlocks; ++t) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        Frag8<T> vf;
        frag_read(vf, vs + vfrag0 + (2 * t + st) * kFrag, lane);
        mma32(o[t], vf, pf[st]);
      }
    }

    if (C::kStages == 1 && kt + 1 < kt_hi) {
      __syncthreads();
      issue_tile<T, D, G>(kbase + static_cast<int64_t>(kt + 1) * C::kKTileBytes,
                          vbase + static_cast<int64_t>(kt + 1) * C::kVTileBytes,
                          smem, smem + C::kKTileBytes, wave, lane);
    }
  }

  // ---- epilogue ------------------------------------------------------------------
  const float l = l_part + wave_xor(l_part, 32);
  if (!row_valid) return;
  const float inv = 1.0f / l;
  T* __restrict__ out = static_cast<T*>(a.out) +
      ((static_cast<int64_t>(b) * a.seq_len + pos) * a.n_q_heads + qh) * D + dbase;
#pragma unroll
  for (int t = 0; t < C::kDBlocks; ++t) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int d = 32 * t + 8 * v4 + 4 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[d + j] = from_f32<T>(o[t][4 * v4 + j] * inv);
    }
  }
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
