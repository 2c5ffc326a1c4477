// Launch interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace ga {

constexpr int kPrepTile = 32;      // key positions per prefill tile (prep and attention)
constexpr int kDecodeChunk = 1024; // cached positions per decode workgroup

// Prefill tiles in MFMA operand order.  A tile of kPrepTile keys is a sequence
// of fragments; fragment f holds, for each of the 64 lanes of a wave, the 8
// elements that lane feeds to one 32x32 MFMA.  Inside a fragment, element j of
// lane l sits at byte ((j * sizeof(T)) / 16) * 1024 + l * 16 + (j * sizeof(T)) % 16,
// so every operand read is 1 KiB of consecutive LDS bytes (lane order).
//   key tile, fragment u (u < D/16):   lane l, element j = K~[key l%32][16u + 8(l/32) + j]
//   value tile, fragment 2t+s (t < D/32, s < 2):
//     lane l, element j = V[key perm(16s + 8(l/32) + j)][32t + l%32]
//   perm swaps bits 2 and 3 of the key index (the order in which the score
//   accumulator lanes hold keys).
template <typename T>
__host__ __device__ constexpr int frag_bytes() { return 64 * 8 * int(sizeof(T)); }
template <typename T>
__host__ __device__ inline int frag_elem_off(int lane, int j) {
  return (j * int(sizeof(T)) / 16) * 1024 + lane * 16 + (j * int(sizeof(T))) % 16;
}
__host__ __device__ constexpr int key_perm(int q) { return (q & ~12) | ((q & 4) << 1) | ((q & 8) >> 1); }

struct PrepArgs {
  const void* k;
  const void* v;
  const void* k_gain;
  const void* rope_table;  // [seq_pad][n_rot] (cos, sin) fp32
  void* k_cache;
  void* v_cache;
  void* ws_k;              // [B][Hkv][seq_pad/32] key tiles (rotated, normalised), operand order
  void* ws_vt;             // [B][Hkv][seq_pad/32] value tiles, operand order
  int seq_len, seq_pad, n_kv_heads, n_rot, window, kv_shared, cache_cap;
  float eps;
};

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const void* k_gain;
  const int32_t* positions;
  void* k_cache;
  void* v_cache;
  int n_kv_heads, n_rot, window, kv_shared, cache_cap;
  float eps;
  double log2_theta;
};

struct PrefillArgs {
  const void* q;
  const void* q_gain;
  const void* rope_table;
  const void* ws_k;
  const void* ws_vt;
  void* out;
  int seq_len, seq_pad, n_q_heads, n_kv_heads, n_rot, window;
  float eps;
  float qk_scale_log2;     // softmax scale * log2(e), folded into q
};

struct DecodeArgs {
  const void* q;
  const void* q_gain;
  const void* k_cache;
  const void* v_cache;
  const int32_t* seq_lens;
  void* out;
  float* partials;         // [B][Hkv][n_chunks][G][D + 2] fp32
  int n_q_heads, n_kv_heads, n_rot, window, cache_cap, max_seq_len, n_chunks;
  float eps;
  float qk_scale_log2;
  double log2_theta;
};

hipError_t launch_rope_table(void* table, int n_pos, int n_rot, int head_dim, double log2_theta,
                             hipStream_t s);
hipError_t launch_prefill_prep(const PrepArgs& a, int dtype, int head_dim, int batch, hipStream_t s);
hipError_t launch_kv_append(const AppendArgs& a, int dtype, int head_dim, int batch, hipStream_t s);
hipError_t launch_prefill_attn(const PrefillArgs& a, int dtype, int head_dim, int group, int batch,
                               hipStream_t s);
// `timer` (optional) is called before and after each of the decode kernels:
// (stream, 2 = split-K kernel / 3 = merge kernel, before?).
typedef void (*LaunchTimer)(hipStream_t, int, bool);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group, int kv_shared,
                         int batch, hipStream_t s, LaunchTimer timer);

}  // namespace ga
