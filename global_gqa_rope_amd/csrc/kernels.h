// Launch interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace ga {

constexpr int kPrepTile = 32;      // key positions per prefill tile (prep and attention)
constexpr int kDecodeTile = 16;     // cached positions per decode tile

// Prefill keys and values, as the prep pass writes them for the attention
// kernel: row-major rows per (sequence, KV head), seq_pad = S rounded up to
// kPrepTile positions, padded rows zero.
//   ws_v [B][Hkv][seq_pad][d]   the value row: the normalised unrotated key on
//                               K=V layers, the raw v otherwise
//   ws_k [B][Hkv][seq_pad][kw]  the normalised rotated key, dims 0..kw-1:
//                               kw = 2 n_rot (the rotated head) on K=V layers,
//                               whose remaining key dims are the value row's;
//                               kw = d on layers with a separate V
// The attention kernel copies 32-row tiles of both into LDS and reads them as
// MFMA operands there (the value operand by transposing LDS reads).
struct PrepArgs {
  const void* k;
  const void* v;
  const void* k_gain;
  const void* rope_table;  // [seq_pad][n_rot] (cos, sin) fp32
  void* k_cache;
  void* v_cache;
  void* ws_k;              // [B][Hkv][seq_pad][kw] rotated normalised keys
  void* ws_v;              // [B][Hkv][seq_pad][d] value rows
  int seq_len, seq_pad, n_kv_heads, n_rot, window, kv_shared, cache_cap, kw;
  int pos0;                // position of k's first row; rows 0 .. pos0-1 come from the caches
  int tile0;               // first tile of kPrepTile positions to prepare (earlier rows are not read)
  int write_v;             // separate-V layers: copy v into ws_v (the attention kernel reads it there)
  int write_ws;            // write the key and value rows of the workspace
  int write_cache;         // write the new rows into the caches
  float* k_scales;         // int8 K=V cache: per-row scales [B][Hkv][cache_cap] (else null)
  void* k_heads;           // pre-rotated K=V cache: heads [B][Hkv][cache_cap][2 n_rot] (else null)
  float* ws_kn;            // [B][Hkv][seq_pad / kPrepTile] largest squared norm of a tile's key rows (with write_ws)
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
  float* k_scales;         // int8 K=V cache: per-row scales (else null)
  void* k_heads;           // pre-rotated K=V cache: heads (else null)
  float eps;
  double log2_theta;
};

struct PrefillArgs {
  const void* q;
  const void* q_gain;
  const void* rope_table;
  const void* rope_table16;   // the same (cos, sin) pairs in fp16, [rows][n_rot]
  int table_rows;
  const void* ws_k;        // see PrepArgs
  const void* ws_v;        // K=V layers' value rows (separate-V layers read v)
  const void* v;           // separate-V layers: v [B][S][Hkv][d] read in place (null: ws_v holds it)
  const float* ws_kn;      // see PrepArgs
  void* out;
  int seq_len, seq_pad, n_q_heads, n_kv_heads, n_rot, window;
  int q_pos0;              // position of q's (and out's) first row; keys from position 0
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
  int32_t* tile_prefix;    // [B + 1] tiles of the sequences before b (written by the split-K kernel)
  float* partials;         // [slots][slot_floats] fp32: o per column, then (m, l) per column
  int batch, n_q_heads, n_kv_heads, n_rot, window, cache_cap, max_seq_len;
  int q_len;               // query tokens per sequence: the last q_len positions (1 = one token)
  int tok0, n_tok;         // this launch's tokens tok0 .. tok0 + n_tok - 1 (G n_tok <= 16 n_groups columns)
  int n_groups;            // column groups of 16 query columns, each with its own workgroups and partials
  int64_t group_floats;    // partials of one column group (slots x slot_floats)
  const float* k_scales;   // int8 K=V cache: per-row scales [B][Hkv][cache_cap] (else null)
  const void* k_heads;     // pre-rotated K=V cache: heads [B][Hkv][cache_cap][2 n_rot] (else null)
  int slot_floats;         // q_len * G * D + 64
  int n_wgs;               // split-K workgroups per column group (the grid is n_groups n_wgs)
  float eps;
  float qk_scale_log2;
  double log2_theta;
};

// Launch shape and scratch of one decode call: per column group, n_wgs
// workgroups of `waves` waves split the tiles evenly and `slots` partial
// results of slot_floats each.
struct DecodePlan {
  int waves, n_wgs, groups;
  size_t prefix_bytes;     // tile_prefix, padded to 256 bytes
  size_t slots, slot_floats;
  size_t bytes() const { return prefix_bytes + groups * slots * slot_floats * 4; }
};
// Returns false if the configuration has no decode kernel.
// groups: column groups per launch (1, or 2 for 17..32 query columns).
bool plan_decode(int dtype, int head_dim, int group, int kv_shared, int batch, int n_kv_heads,
                 int max_tiles_per_seq, int n_cus, int q_len, int groups, DecodePlan* plan);

hipError_t launch_rope_table(void* table, void* table16, int pos_begin, int n_pos, int n_rot, int head_dim, double log2_theta,
                             hipStream_t s);
hipError_t launch_prefill_prep(const PrepArgs& a, int dtype, int head_dim, int batch, hipStream_t s);
hipError_t launch_kv_append(const AppendArgs& a, int dtype, int head_dim, int batch, hipStream_t s);
hipError_t launch_prefill_attn(const PrefillArgs& a, int dtype, int head_dim, int group, int kv_shared,
                               int batch, hipStream_t s);
// `timer` (optional) is called before and after each of the decode kernels:
// (stream, 2 = split-K kernel / 3 = merge kernel, before?).
typedef void (*LaunchTimer)(hipStream_t, int, bool);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group, int kv_shared,
                         int batch, hipStream_t s, LaunchTimer timer);

hipError_t launch_calib_mfma(const void* ops, int n_ops, int iters, int n_wgs, float* sink, hipStream_t s);
hipError_t launch_calib_stream(const void* buf, size_t bytes, int n_wgs, unsigned* sink, hipStream_t s);

}  // namespace ga
