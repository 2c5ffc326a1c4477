// Key/value preparation kernels: the RoPE angle table, the prefill K/V pass
// (QKNorm, rotation, transposed value tiles, cache fill) and kv_append.
#include "common.h"
#include "kernels.h"

namespace ga {

// table[pos][pair] = (cos, sin)(pos * theta^(-2 pair / d)), fp64 math.
// Rows pos_begin .. n_pos - 1 (earlier rows are not read).
__global__ void rope_table_kernel(f32x2* __restrict__ table, uint32_t* __restrict__ table16, int pos_begin,
                                  int n_pos, int n_rot, int head_dim, double log2_theta) {
  const int64_t first = static_cast<int64_t>(pos_begin) * n_rot;
  const int64_t total = static_cast<int64_t>(n_pos) * n_rot;
  for (int64_t i = first + blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int pos = static_cast<int>(i / n_rot);
    const int pair = static_cast<int>(i % n_rot);
    const f32x2 cs = rope_cos_sin(static_cast<double>(pos) * rope_omega(pair, head_dim, log2_theta));
    table[i] = cs;
    if (table16) {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const h2 v = {static_cast<_Float16>(cs[0]), static_cast<_Float16>(cs[1])};
      table16[i] = __builtin_bit_cast(uint32_t, v);
    }
  }
}

// int8 K=V cache rows: codes round-half-even(x / s), s = max |x| / 127, kept
// as two's-complement bytes.  The division is the correctly rounded float32
// one, so equal inputs give equal codes.
__device__ __forceinline__ uint2 q8_pack8(const float (&x)[8], float s) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float c = s > 0.f ? fminf(fmaxf(rintf(x[j] / s), -127.f), 127.f) : 0.f;
    w[j / 4] |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xffu) << (8 * (j % 4));
  }
  return uint2{w[0], w[1]};
}
__device__ __forceinline__ void q8_unpack8(float (&x)[8], uint2 u, float s) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    x[j] = static_cast<float>(static_cast<int8_t>((j < 4 ? u.x : u.y) >> (8 * (j % 4)))) * s;
}

// One workgroup per (tile of kPrepTile key positions, kv head, batch), for the
// tiles tile0 .. seq_pad / kPrepTile - 1 (earlier rows are never read).
// Thread t owns key row r = t / 8 of the tile and the 8-element chunks
// i * 8 + t % 8 of that row, so eight neighbouring lanes cover 64 contiguous
// elements of one row.  Every global access is a 16-byte vector, and all
// loads of a thread are issued before the first use.  A row is one of:
//  - new (positions pos0 .. pos0 + seq_len - 1, k's rows): normalised; the key
//    row is rotated, the value row is the normalised key (K=V) or v;
//  - cached (a position below pos0, a later chunk of a prompt), read back from
//    the caches: on K=V layers the stored normalised, unrotated key (int8:
//    codes times the row scale), rotated for the key row and as stored for the
//    value row; on separate-V layers the stored key, already normalised and
//    rotated, and the stored value.  A windowed layer's ring holds the last
//    cache_cap positions before pos0; older rows lie outside every new row's
//    window and are zeros;
//  - padding (past the sequence): zeros.
// write_ws: write the key and value rows of the workspace.  write_cache:
// write the new rows into the caches (windowed layers: those among the last
// cache_cap positions, at slot position mod cache_cap; others: slot =
// position).
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_prep_kernel(PrepArgs a) {
  constexpr int kChunks = D / 8;             // 8-element chunks per row
  constexpr int kMine = kChunks / 8;         // chunks per thread
  typedef T vec8 __attribute__((ext_vector_type(8)));

  // Workgroup order: the KV heads of every sequence for one tile of positions
  // run together, so the tile's rows of the cos/sin table are read once into
  // L2 and then hit there, instead of once per head and sequence.
  const int n_tiles = a.seq_pad / kPrepTile - a.tile0;
  const int n_seq = static_cast<int>(gridDim.x) / (a.n_kv_heads * n_tiles);
  const int h = static_cast<int>(blockIdx.x) % a.n_kv_heads;
  const int b = (static_cast<int>(blockIdx.x) / a.n_kv_heads) % n_seq;
  const int tile = a.tile0 + static_cast<int>(blockIdx.x) / (a.n_kv_heads * n_seq);
  const int t = threadIdx.x;
  const int r = t >> 3, c8 = t & 7;
  const int pos = tile * kPrepTile + r;
  const int total = a.pos0 + a.seq_len;
  const bool has_v = !a.kv_shared;
  const bool valid = pos >= a.pos0 && pos < total;                 // one of k's rows
  const bool cached = pos < a.pos0 && (a.window == 0 || pos >= a.pos0 - a.cache_cap);
  const bool cached_sep = cached && has_v;                          // stored rotated, value in v_cache
  const int slot = a.window > 0 ? pos % a.cache_cap : pos;
  // other positions read k's last row (then zeroed) so no load leaves the tensor
  const int src_pos = valid ? pos - a.pos0 : a.seq_len - 1;
  const int64_t src_row = ((static_cast<int64_t>(b) * a.seq_len + src_pos) * a.n_kv_heads + h) * D;
  const int64_t head_base = (static_cast<int64_t>(b) * a.n_kv_heads + h);
  const bool to_cache = a.write_cache && a.k_cache && valid && (a.window == 0 || pos >= total - a.cache_cap);
  const bool v_to_ws = has_v && a.write_ws && a.write_v;

  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const T* __restrict__ gk = static_cast<const T*>(a.k_gain);
  const f32x2* __restrict__ table = static_cast<const f32x2*>(a.rope_table) + static_cast<int64_t>(pos) * a.n_rot;

  vec8 kin[kMine], vin[kMine], gin[kMine];
  f32x2 cs[kMine][4];
  const T* __restrict__ cache_row = static_cast<const T*>(a.k_cache) + (head_base * a.cache_cap + slot) * D;
  const T* __restrict__ vcache_row = static_cast<const T*>(a.v_cache) + (head_base * a.cache_cap + slot) * D;
  const bool q8 = a.k_scales != nullptr;                  // int8 K=V cache
  const uint8_t* __restrict__ code_row = static_cast<const uint8_t*>(a.k_cache) + (head_base * a.cache_cap + pos) * D;
  uint2 qin[kMine];
  float q_scale = 0.f;
#pragma unroll
  for (int i = 0; i < kMine; ++i) {
    const int d0 = (i * 8 + c8) * 8;
    if (cached && q8) qin[i] = *reinterpret_cast<const uint2*>(code_row + d0);
    else kin[i] = *reinterpret_cast<const vec8*>((cached ? cache_row : k + src_row) + d0);
    gin[i] = *reinterpret_cast<const vec8*>(gk + d0);
    if (has_v) {
      if (cached_sep) vin[i] = *reinterpret_cast<const vec8*>(vcache_row + d0);
      else if (valid && (v_to_ws || to_cache)) vin[i] = *reinterpret_cast<const vec8*>(v + src_row + d0);
    }
  }
  if (cached && q8) q_scale = a.k_scales[head_base * a.cache_cap + pos];
  // (cos, sin) of the chunk's four pairs; pairs >= n_rot read a clamped entry
  // of the same row and are not used
  if (a.n_rot > 0) {
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int d0 = (i * 8 + c8) * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) cs[i][j] = table[min(d0 / 2 + j, a.n_rot - 1)];
    }
  }

  float x[kMine][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMine; ++i) {
    if (cached && q8) {
      q8_unpack8(x[i], qin[i], q_scale);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[i][j] = (valid || cached) ? to_f32(kin[i][j]) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[i][j] * x[i][j];
  }
  ss += wave_xor(ss, 1);
  ss += wave_xor(ss, 2);
  ss += wave_xor(ss, 4);
  const float rstd = 1.0f / sqrtf(ss / D + a.eps);
  if (!cached) {   // cached rows are normalised already
#pragma unroll
    for (int i = 0; i < kMine; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[i][j] = x[i][j] * rstd * to_f32(gin[i][j]);
  }

  const int64_t row = head_base * a.seq_pad + pos;          // row in ws_k / ws_v
  T* __restrict__ kc = static_cast<T*>(a.k_cache);
  T* __restrict__ vc = static_cast<T*>(a.v_cache);
  T* __restrict__ wv = static_cast<T*>(a.ws_v) + row * D;

  // Value row.  K=V: the normalised, unrotated key, which is also what the
  // cache keeps (int8 caches: its codes and the row's scale).  Otherwise v
  // (the stored value for cached rows, zeros for padding).
  if (!has_v && q8 && to_cache) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kMine; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[i][j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
    const float sc = amax / 127.0f;
    uint8_t* codes = static_cast<uint8_t*>(a.k_cache) + (head_base * a.cache_cap + pos) * D;
#pragma unroll
    for (int i = 0; i < kMine; ++i) *reinterpret_cast<uint2*>(codes + (i * 8 + c8) * 8) = q8_pack8(x[i], sc);
    if (c8 == 0) a.k_scales[head_base * a.cache_cap + pos] = sc;
  }
  vec8 vout[kMine];
#pragma unroll
  for (int i = 0; i < kMine; ++i) {
    const int d0 = (i * 8 + c8) * 8;
    if (has_v) {
#pragma unroll
      for (int j = 0; j < 8; ++j) vout[i][j] = (valid || cached) ? vin[i][j] : from_f32<T>(0.f);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) vout[i][j] = from_f32<T>(x[i][j]);
      if (to_cache && !q8) *reinterpret_cast<vec8*>(kc + (head_base * a.cache_cap + pos) * D + d0) = vout[i];
    }
    if (a.write_ws && (!has_v || a.write_v)) *reinterpret_cast<vec8*>(wv + d0) = vout[i];
  }

  // Rotate the first 2*n_rot dims (cached separate-V keys are stored rotated).
  if (!cached_sep) {
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int d0 = (i * 8 + c8) * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (d0 / 2 + j < a.n_rot) rotate_pair(x[i][2 * j], x[i][2 * j + 1], cs[i][j]);
      }
    }
  }
  vec8 kout[kMine];
#pragma unroll
  for (int i = 0; i < kMine; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) kout[i][j] = cached_sep ? kin[i][j] : from_f32<T>(x[i][j]);

  // Largest squared length of the tile's key rows, as the attention kernel
  // reads them (the rounded rotated key; on K=V layers its dims past kw are
  // the value row's, which the rotation left unchanged).  The attention
  // kernel bounds its scores with it.
  if (a.write_ws && a.ws_kn) {
    __shared__ float wave_max[4];
    float n2 = 0.f;
#pragma unroll
    for (int i = 0; i < kMine; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) n2 += to_f32(kout[i][j]) * to_f32(kout[i][j]);
    n2 += wave_xor(n2, 1);
    n2 += wave_xor(n2, 2);
    n2 += wave_xor(n2, 4);
    n2 = fmaxf(n2, wave_xor(n2, 8));
    n2 = fmaxf(n2, wave_xor(n2, 16));
    n2 = fmaxf(n2, wave_xor(n2, 32));
    static_assert(kPrepTile * 8 == 256, "four waves of eight rows");
    if ((t & (kWave - 1)) == 0) wave_max[t / kWave] = n2;
    __syncthreads();
    if (t == 0)
      a.ws_kn[head_base * (a.seq_pad / kPrepTile) + tile] =
          fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  }

  // Key row: dims 0..kw-1 of the rotated normalised key.
  if (a.write_ws) {
    T* __restrict__ wk = static_cast<T*>(a.ws_k) + row * a.kw;
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int d0 = (i * 8 + c8) * 8;
      if (d0 < a.kw) *reinterpret_cast<vec8*>(wk + d0) = kout[i];
    }
  }

  // Pre-rotated K=V caches also keep each new row's rotated head
  // (dims 0 .. 2 n_rot - 1, as the key row above).
  if (a.k_heads && to_cache) {
    T* __restrict__ hk = static_cast<T*>(a.k_heads) + (head_base * a.cache_cap + pos) * (2 * a.n_rot);
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int d0 = (i * 8 + c8) * 8;
      if (d0 < 2 * a.n_rot) *reinterpret_cast<vec8*>(hk + d0) = kout[i];
    }
  }

  // Separate-V layers: windowed ones keep the last cache_cap positions in a
  // ring (slot = position mod cache_cap), global ones every position (slot =
  // position); keys rotated.
  if (has_v && to_cache) {
    T* dk = kc + (head_base * a.cache_cap + slot) * D;
    T* dv = vc + (head_base * a.cache_cap + slot) * D;
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int d0 = (i * 8 + c8) * 8;
      *reinterpret_cast<vec8*>(dk + d0) = kout[i];
      *reinterpret_cast<vec8*>(dv + d0) = vin[i];
    }
  }
}

// One wave per (kv head, batch).  Lane l owns dims [l*D/64, (l+1)*D/64).
template <typename T, int D>
__global__ __launch_bounds__(64) void kv_append_kernel(AppendArgs a) {
  constexpr int kPer = D / 64;
  const int h = blockIdx.x, b = blockIdx.y;
  const int l = threadIdx.x;
  const int pos = a.positions[b];
  const int64_t head_base = static_cast<int64_t>(b) * a.n_kv_heads + h;
  if (pos < 0) return;
  if (a.kv_shared && pos >= a.cache_cap) return;
  const int slot = a.window > 0 ? pos % a.cache_cap : pos;
  if (slot >= a.cache_cap) return;

  const T* __restrict__ kn = static_cast<const T*>(a.k_new) + head_base * D + l * kPer;
  const T* __restrict__ gk = static_cast<const T*>(a.k_gain) + l * kPer;
  float x[kPer];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    x[j] = to_f32(kn[j]);
    ss += x[j] * x[j];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) ss += wave_xor(ss, m);
  const float rstd = 1.0f / sqrtf(ss / D + a.eps);
#pragma unroll
  for (int j = 0; j < kPer; ++j) x[j] = x[j] * rstd * to_f32(gk[j]);

  if (a.k_scales) {   // int8 K=V cache: codes and the row's scale
    static_assert(kPer == 8 || kPer == 4, "8 or 4 elements per lane");
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
    const float sc = amax / 127.0f;
    uint8_t* codes = static_cast<uint8_t*>(a.k_cache) + (head_base * a.cache_cap + slot) * D + l * kPer;
    float x8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x8[j] = j < kPer ? x[j] : 0.f;
    const uint2 u = q8_pack8(x8, sc);
    if constexpr (kPer == 8) *reinterpret_cast<uint2*>(codes) = u;
    else *reinterpret_cast<uint32_t*>(codes) = u.x;
    if (l == 0) a.k_scales[head_base * a.cache_cap + slot] = sc;
    return;
  }
  if (a.k_heads && l * kPer < 2 * a.n_rot) {   // pre-rotated K=V cache: the row's rotated head too
    float r[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) r[j] = x[j];
#pragma unroll
    for (int j = 0; j < kPer / 2; ++j) {
      const int pair = l * kPer / 2 + j;
      if (pair < a.n_rot)
        rotate_pair(r[2 * j], r[2 * j + 1], rope_cos_sin(static_cast<double>(pos) * rope_omega(pair, D, a.log2_theta)));
    }
    T* __restrict__ hk = static_cast<T*>(a.k_heads) + (head_base * a.cache_cap + slot) * (2 * a.n_rot) + l * kPer;
#pragma unroll
    for (int j = 0; j < kPer; ++j) hk[j] = from_f32<T>(r[j]);
  }
  T* __restrict__ kc = static_cast<T*>(a.k_cache) + (head_base * a.cache_cap + slot) * D + l * kPer;
  if (!a.kv_shared) {
#pragma unroll
    for (int j = 0; j < kPer / 2; ++j) {
      const int pair = l * kPer / 2 + j;
      if (pair < a.n_rot)
        rotate_pair(x[2 * j], x[2 * j + 1],
                    rope_cos_sin(static_cast<double>(pos) * rope_omega(pair, D, a.log2_theta)));
    }
    const T* __restrict__ vn = static_cast<const T*>(a.v_new) + head_base * D + l * kPer;
    T* __restrict__ vcp = static_cast<T*>(a.v_cache) + (head_base * a.cache_cap + slot) * D + l * kPer;
#pragma unroll
    for (int j = 0; j < kPer; ++j) vcp[j] = vn[j];
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) kc[j] = from_f32<T>(x[j]);
}

// ---- launchers ---------------------------------------------------------------

hipError_t launch_rope_table(void* table, void* table16, int pos_begin, int n_pos, int n_rot, int head_dim, double log2_theta,
                             hipStream_t s) {
  if (n_rot == 0 || n_pos <= pos_begin) return hipSuccess;
  const int64_t total = static_cast<int64_t>(n_pos - pos_begin) * n_rot;
  const int blocks = static_cast<int>(std::min<int64_t>((total + 255) / 256, 4096));
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, s, static_cast<f32x2*>(table),
                     static_cast<uint32_t*>(table16), pos_begin, n_pos, n_rot, head_dim, log2_theta);
  return hipGetLastError();
}

hipError_t launch_prefill_prep(const PrepArgs& a, int dtype, int head_dim, int batch, hipStream_t s) {
  const int tiles = a.seq_pad / kPrepTile - a.tile0;
  if (tiles <= 0 || batch == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tiles) * a.n_kv_heads * batch);
  if (dtype == 0 && head_dim == 512) hipLaunchKernelGGL((prefill_prep_kernel<bf16, 512>), grid, dim3(256), 0, s, a);
  else if (dtype == 0 && head_dim == 256) hipLaunchKernelGGL((prefill_prep_kernel<bf16, 256>), grid, dim3(256), 0, s, a);
  else if (dtype == 1 && head_dim == 512) hipLaunchKernelGGL((prefill_prep_kernel<float, 512>), grid, dim3(256), 0, s, a);
  else if (dtype == 1 && head_dim == 256) hipLaunchKernelGGL((prefill_prep_kernel<float, 256>), grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, int dtype, int head_dim, int batch, hipStream_t s) {
  const dim3 grid(a.n_kv_heads, batch);
  if (dtype == 0 && head_dim == 512) hipLaunchKernelGGL((kv_append_kernel<bf16, 512>), grid, dim3(64), 0, s, a);
  else if (dtype == 0 && head_dim == 256) hipLaunchKernelGGL((kv_append_kernel<bf16, 256>), grid, dim3(64), 0, s, a);
  else if (dtype == 1 && head_dim == 512) hipLaunchKernelGGL((kv_append_kernel<float, 512>), grid, dim3(64), 0, s, a);
  else if (dtype == 1 && head_dim == 256) hipLaunchKernelGGL((kv_append_kernel<float, 256>), grid, dim3(64), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ga
