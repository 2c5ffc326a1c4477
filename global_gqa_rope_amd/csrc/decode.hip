// Split-K decode: one query token per sequence against its cache, gfx950.
//
// A persistent grid: one workgroup per CU takes an equal, contiguous share of
// all 16-key tiles of all (sequence, KV head) segments, so every CU streams
// the same number of bytes and keeps streaming across segment boundaries.
// Each wave of the workgroup takes every kWaves-th tile of that share:
//   global -> LDS by buffer loads that write LDS directly, two tiles per wave,
//   the next tile in flight while the current one is computed;
//   K=V layers: pairs 0..63 of every key are rotated on the fly as they are
//   loaded into the QK^T operand (p-RoPE of the "Gemma 4多模态大模型架构详解"
//   section "p-RoPE（低频剪枝旋转位置编码）"); the raw rows in LDS are the values
//   ("K=V" section of the same page);
//   S^T[key][head] = K~ Q~^T   (16x16x32 MFMA, the G heads padded to 16 columns;
//                               the query operand is read from LDS, where the
//                               workgroup writes it once per segment in operand
//                               order)
//   online softmax per head (exp2 domain, lazy rescale)
//   O^T[d][head] += V^T P^T     (16x16x16 MFMA; V^T by LDS transpose reads, P
//                               straight from the S^T registers)
// Every wave leaves one partial (o, max, sum) per segment it took part in; a
// second kernel merges the partials of each (sequence, query head) by
// log-sum-exp.
//
// All LDS addressing inside the loop is one XOR per read: tiles sit at
// multiples of their size and rows at multiples of the row size, and a
// fragment's 16-byte chunk index splits into a lane part and a per-step part
// with disjoint bits, so the row swizzle (chunk c of row r at c ^ row_swz(r))
// turns into lane_base ^ (step part << 4).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ga {

constexpr int kLdsLimit = 160 * 1024;

// Q8: the K=V cache holds int8 rows (codes c and one fp32 scale s per row,
// standing for c s).  Each tile's codes and scales are copied into a staging
// buffer; the codes, exact in bf16, are expanded into the bf16 tile the native
// cache is copied into, so the score and value products are the same code for
// both formats, and the row scales are applied in fp32: to each score
// (q . c s = (q . c) s) and to each softmax weight before it meets the codes
// as values (p (c s) = (p s) c).
// PRE: the pre-rotated ("1.25 d") K=V cache: the rows as in the native K=V
// cache, plus per row its leading 2 n_rot dims already rotated to the row's
// position (the heads).  The QK^T steps over those dims take the key operand
// from the heads, loaded into registers a tile ahead, instead of rotating the
// row's dims; nothing else changes.
template <typename T, int D, int G, bool SHARED, bool Q8 = false, bool PRE = false>
struct DecodeCfg {
  static constexpr int KT = 16;                       // keys per wave tile
  static constexpr int kD = D;
  static constexpr int kSz = int(sizeof(T));
  static constexpr int kRot = (SHARED && !PRE) ? 64 : 0;   // pairs rotated on the fly
  static constexpr int kHeadSteps = PRE ? 2 * 64 / 32 : 0;  // QK^T steps whose keys come from the heads
  static constexpr int kRotSteps = 2 * kRot / 32;     // QK^T steps that cover rotated dims
  static constexpr int kRowBytes = D * kSz;           // one key row
  static constexpr int kKBytes = KT * kRowBytes;      // key tile (the values too for K=V)
  static constexpr int kTileBytes = SHARED ? kKBytes : 2 * kKBytes;   // + value tile
  static constexpr int kBufs = Q8 ? 1 : 2;            // tiles in LDS per wave
  static constexpr int kCodeBytes = KT * D;           // Q8: one tile's codes
  static constexpr int kStageBytes = Q8 ? kCodeBytes + 256 : 0;   // codes, then 64 scale slots
  static constexpr int kQSteps = D / 32;              // QK^T reduction steps
  static constexpr int kDBlocks = D / 16;             // PV output blocks of 16 dims
  static constexpr int kFragBytes = 64 * 8 * kSz;     // one query operand fragment
  static constexpr int kQBytes = kQSteps * kFragBytes;
  // cos/sin(j w_i), j < 16, i < kRot: row j (one key offset) padded by 16 B, so
  // the 16 rows one rotated QK^T step reads start 4 banks apart instead of all
  // in the same 4 banks (a 16-way conflict without the pad).
  static constexpr int kFineRow = kRot > 0 ? kRot * 8 + 16 : 0;
  static constexpr int kFineBytes = 16 * kFineRow;
  static constexpr int kCoarseBytes = kRot * 8;       // per wave: cos/sin(key0 w_i)
  static constexpr int kPerWaveBytes = kBufs * kTileBytes + 2 * kStageBytes + kCoarseBytes;
  static constexpr int kMiscBytes = 64;               // partition scratch
  static constexpr int kCommonBytes = kQBytes + kFineBytes + kMiscBytes;
  static constexpr int kWaves = (4 * kPerWaveBytes + kCommonBytes <= kLdsLimit)   ? 4
                                : (2 * kPerWaveBytes + kCommonBytes <= kLdsLimit) ? 2
                                                                                  : 1;
  static constexpr int kDmaPerTile = kTileBytes / 1024;
  static constexpr int kQ8Copies = kCodeBytes / 1024 + 1;   // Q8: copy instructions of one tile
  static constexpr int kKDma = kKBytes / 1024;
  // LDS map: [wave][buf] tiles | [wave][2] staging (Q8) | [wave] coarse angles |
  // query operand | fine angles | misc
  static constexpr int kStageOff = kWaves * kBufs * kTileBytes;
  static constexpr int kCoarseOff = kStageOff + kWaves * 2 * kStageBytes;
  static constexpr int kQOff = kCoarseOff + kWaves * kCoarseBytes;
  static constexpr int kFineOff = kQOff + kQBytes;
  static constexpr int kMiscOff = kFineOff + kFineBytes;
  static constexpr int kLdsBytes = kMiscOff + kMiscBytes;
  static_assert(kLdsBytes <= kLdsLimit, "LDS budget");
  static_assert(kRowBytes / 16 >= 16, "row swizzle needs 16 chunks per row");
  static_assert(kTileBytes % 1024 == 0 && kDmaPerTile < 64, "tile copy");
  static_assert(!Q8 || (SHARED && sizeof(T) == 2 && kCodeBytes % 1024 == 0), "int8 tiles: bf16 K=V");
  static_assert(!PRE || (SHARED && !Q8 && sizeof(T) == 2 && D == 512), "pre-rotated heads: bf16 K=V, d = 512");
};

typedef __attribute__((address_space(3))) char lds_char;
typedef __amdgpu_buffer_rsrc_t BufRsrc;

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char*)p));
}
__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
template <typename V>
__device__ __forceinline__ V lds_ld(uint32_t addr) {
  return *(const __attribute__((address_space(3))) V*)(static_cast<uintptr_t>(addr));
}
template <typename V>
__device__ __forceinline__ void lds_st(uint32_t addr, V v) {
  *(__attribute__((address_space(3))) V*)(static_cast<uintptr_t>(addr)) = v;
}

// Raw buffer over `bytes` bytes: loads past the end return zeros instead of
// touching memory (dword 3: 32-bit data format, as untyped buffer loads need).
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// Orders this wave's LDS accesses (compiler and hardware) around a tile reuse.
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vm_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Sequence b's number of readable keys, or -1 if its length is out of range.
// Global layers read slots 0 .. L-1 (slot = position); windowed layers the
// min(L, cache_cap) filled slots of their ring (slot = position mod cache_cap).
__device__ __forceinline__ int decode_keys(const DecodeArgs& a, int b) {
  const int L = a.seq_lens[b];
  if (L < a.q_len || L < 1 || L > a.max_seq_len) return -1;
  if (a.window == 0 && L > a.cache_cap) return -1;
  return a.window > 0 ? min(L, a.cache_cap) : L;
}

// Key rows sit in LDS in natural order [key][d]; 16-byte chunk c of row r is
// stored at chunk c ^ row_swz(r).  Rows are a multiple of 512 B apart, so
// without the swizzle every row starts in the same bank.  Measured on this
// chip with SQ_LDS_BANK_CONFLICT: a ds_read_b128 resolves banks over 8
// consecutive lanes within 128 B, and a ds_read_b64_tr_b16 over 32 lanes
// within 256 B.  The QK^T key read puts rows 0..7 (or 8..15) on 8 consecutive
// lanes, one chunk each, so row_swz(r) & 7 must differ across them.  The PV
// transposing read puts rows 0..7 (or 8..15) on 32 lanes, each row a 32-byte
// run of chunks 2t, 2t + 1, so row_swz(r) >> 1 must differ across them.
// row_swz(r) = (r & 7) + 8 (r & 1) satisfies both (c ^ r met only the first:
// 2-way conflicts on every PV read).
__device__ __forceinline__ int row_swz(int r) { return (r & 7) | ((r & 1) << 3); }
__device__ __forceinline__ int row_chunk(int r, int c) { return c ^ row_swz(r); }

// Copy one tile (16 key rows, plus 16 value rows for separate-V layers) from
// the cache straight into LDS at `dst`.  Each instruction moves 1 KiB: lane l
// writes LDS slot dst + 16 l and fetches the cache chunk that the swizzle
// places there.  Rows past the sequence read its last row (their scores are
// masked); the buffer's range check backs this up.
template <typename C>
__device__ __forceinline__ void issue_tile(lds_char* dst, BufRsrc rk, BufRsrc rv, int key0, int nkeys, int lane) {
#pragma unroll
  for (int i = 0; i < C::kDmaPerTile; ++i) {
    const int ik = i % C::kKDma;                   // 1 KiB piece within the K (or V) tile
    const BufRsrc& rs = (i < C::kKDma) ? rk : rv;
    lds_char* slot = dst + i * 1024;
    if constexpr (C::kRowBytes >= 1024) {          // piece inside one row: the key is wave-uniform
      constexpr int kPiecesPerRow = C::kRowBytes / 1024;
      const int r = ik / kPiecesPerRow;
      const int s = (ik % kPiecesPerRow) * 64 + lane;
      const int key = min(key0 + r, nkeys - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, slot, 16, row_chunk(r, s) << 4, key * C::kRowBytes, 0, 0);
    } else {                                       // several rows per piece
      constexpr int kChunksPerRow = C::kRowBytes / 16;
      const int r = ik * (1024 / C::kRowBytes) + lane / kChunksPerRow;
      const int s = lane % kChunksPerRow;
      const int key = min(key0 + r, nkeys - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, slot, 16, key * C::kRowBytes + (row_chunk(r, s) << 4), 0, 0, 0);
    }
  }
}

// Q8: copy one tile's codes (16 rows of D bytes, natural order) and the 16
// row scales into a staging buffer.  Lane l of the scale copy fetches the
// scale of row l (clamped to the sequence); slots 16..63 are not read.
template <typename C>
__device__ __forceinline__ void issue_q8(lds_char* dst, BufRsrc rc, BufRsrc rs, int key0, int nkeys, int lane) {
  constexpr int kRowsPerPiece = 1024 / C::kD;     // D-byte code rows per 1 KiB
  constexpr int kChunksPerRow = C::kD / 16;
#pragma unroll
  for (int i = 0; i < C::kCodeBytes / 1024; ++i) {
    const int r = i * kRowsPerPiece + lane / kChunksPerRow;
    const int key = min(key0 + r, nkeys - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, dst + i * 1024, 16, key * C::kD + (lane % kChunksPerRow) * 16,
                                             0, 0, 0);
  }
  const int key = min(key0 + lane, nkeys - 1);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + C::kCodeBytes, 4, key * 4, 0, 0, 0);
}

// Q8: expand the staged codes into the bf16 tile (|c| <= 127: exact in bf16).
// Lane l writes the 16-byte chunk l of every row at the row swizzle.
template <typename C>
__device__ __forceinline__ void expand_q8(const lds_char* __restrict__ stage, lds_char* __restrict__ tile, int lane) {
  constexpr int kD = C::kD;
  static_assert(kD == 64 * 8, "one 8-code piece per lane and row");
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  // all the tile's code reads first, so their latencies overlap
  u32x2 w[C::KT];
#pragma unroll
  for (int r = 0; r < C::KT; ++r) w[r] = *(const __attribute__((address_space(3))) u32x2*)(stage + r * kD + 8 * lane);
#pragma unroll
  for (int r = 0; r < C::KT; ++r) {
    u32x4 packed;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {   // sign-extend and convert each byte, pack pairs
      const f32x2 x{static_cast<float>(static_cast<int8_t>(w[r][j / 4] >> (8 * (j % 4)))),
                    static_cast<float>(static_cast<int8_t>(w[r][j / 4] >> (8 * (j % 4 + 1))))};
      packed[j / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
    }
    const bf16x8 v = __builtin_bit_cast(bf16x8, packed);
    *(__attribute__((address_space(3))) bf16x8*)(tile + r * C::kRowBytes + (row_chunk(r, lane) << 4)) = v;
  }
}

// QK^T A operand: the 8 elements of the lane's key row at dims 32u + 8kg .. +7.
// `a` = lane base (row hcol, lane chunk part); the step part is XORed in.
template <typename C>
__device__ __forceinline__ void key_frag(Frag8<bf16>& f, uint32_t a, int u) {
  f.v = lds_ld<bf16x8>(a ^ ((4 * u) << 4));
}
template <typename C>
__device__ __forceinline__ void key_frag(Frag8<float>& f, uint32_t a, int u) {
  const f32x4 lo = lds_ld<f32x4>(a ^ ((8 * u) << 4));
  const f32x4 hi = lds_ld<f32x4>(a ^ ((8 * u) << 4) ^ 16);
  f.v[0] = lo[0]; f.v[1] = lo[1]; f.v[2] = lo[2]; f.v[3] = lo[3];
  f.v[4] = hi[0]; f.v[5] = hi[1]; f.v[6] = hi[2]; f.v[7] = hi[3];
}

// PV A operand V^T for dims 16t .. +15: lane l needs V[key 4(l/16) + j][16t + l%16],
// j = 0..3.  bf16: one transpose read (within each 16-lane group, lane i gets
// element i%4 of the 8-byte pieces addressed by lanes i/4 + 4j); lane l
// addresses key 4(l/16) + (l%16)/4, dims 16t + 4(l%4) .. +3, whose chunk is
// 2t + (l%4)/2.  fp32: four plain reads (rows 4(l/16) + j, dim 16t + l%16).
// `buf` is the tile buffer, `off` the lane's offset in it (buffers are aligned
// to their size, so the XOR stays inside the offset).
template <typename C>
__device__ __forceinline__ void value_frag(Frag4<bf16>& f, const lds_char* buf, uint32_t off, int t) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(buf + (off ^ ((2 * t) << 4))));
  f.v = __builtin_bit_cast(bf16x4, v);
}
template <typename C>
__device__ __forceinline__ void value_frag(Frag4<float>& f, const lds_char* buf, uint32_t off, int t) {
  const uint32_t vtile = lds_addr(buf) + off;
  const int lane = threadIdx.x & 63;
  const int cvar = (lane & 15) >> 2;              // chunk of dim 16t + l%16 is 4t + cvar
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * (lane >> 4) + j;
    const uint32_t at = vtile + r * C::kRowBytes + (row_chunk(r, cvar) << 4) + 4 * (lane & 3);
    f.v[j] = lds_ld<float>(at ^ ((4 * t) << 4));
  }
}

// Per-lane base addresses (tile buffer 0) of the two operand reads.
template <typename C, typename T>
__device__ __forceinline__ uint32_t key_lane_base(uint32_t tile, int lane) {
  const int hcol = lane & 15, kg = lane >> 4;
  const int cvar = kg * C::kSz / 2;               // lane part of chunk (32u + 8kg) * size / 16
  return tile + hcol * C::kRowBytes + (row_chunk(hcol, cvar) << 4);
}
template <typename C, typename T>
__device__ __forceinline__ uint32_t value_lane_base(uint32_t vtile, int lane) {
  if constexpr (std::is_same<T, bf16>::value) {
    const int r = 4 * (lane >> 4) + ((lane & 15) >> 2);
    const int cvar = (lane & 3) >> 1;
    return vtile + r * C::kRowBytes + (row_chunk(r, cvar) << 4) + 8 * (lane & 1);
  } else {
    return vtile;                                 // the fp32 reads form their own lane addresses
  }
}

// Query operand fragment u of this lane (written once per workgroup).
__device__ __forceinline__ void load_qfrag(Frag8<bf16>& f, uint32_t a) { f.v = lds_ld<bf16x8>(a); }
__device__ __forceinline__ void load_qfrag(Frag8<float>& f, uint32_t a) {
  const f32x4 lo = lds_ld<f32x4>(a), hi = lds_ld<f32x4>(a + 16);
  f.v[0] = lo[0]; f.v[1] = lo[1]; f.v[2] = lo[2]; f.v[3] = lo[3];
  f.v[4] = hi[0]; f.v[5] = hi[1]; f.v[6] = hi[2]; f.v[7] = hi[3];
}

// One QK^T step's operands: key fragment, query fragment and, for the
// rotated steps, the coarse and fine angle factors of the lane's 4 pairs.
template <typename T>
struct QkStep {
  Frag8<T> kf, qf;
  f32x4 cb[2], fj[2];   // (cos, sin) of pairs p = 0, 1 and p = 2, 3
};
template <typename C, typename T>
__device__ __forceinline__ void load_step(QkStep<T>& st, int u, uint32_t k_lane, uint32_t q_lane,
                                          uint32_t coarse_lane, uint32_t fine_lane) {
  if (u >= C::kHeadSteps) key_frag<C>(st.kf, k_lane, u);
  load_qfrag(st.qf, q_lane + u * C::kFragBytes);
  if (u < C::kRotSteps) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      st.cb[h] = lds_ld<f32x4>(coarse_lane + (16 * u + 2 * h) * 8);
      st.fj[h] = lds_ld<f32x4>(fine_lane + (16 * u + 2 * h) * 8);
    }
  }
}
// Rotate the 4 pairs of a key fragment by cos/sin = coarse (x) fine.
template <typename T>
__device__ __forceinline__ void rotate_step(QkStep<T>& st) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f32x4& cb4 = st.cb[p >> 1];
    const f32x4& fj4 = st.fj[p >> 1];
    const int o = 2 * (p & 1);
    f32x2 cs;
    cs[0] = cb4[o] * fj4[o] - cb4[o + 1] * fj4[o + 1];
    cs[1] = cb4[o + 1] * fj4[o] + cb4[o] * fj4[o + 1];
    float x0 = to_f32(st.kf.v[2 * p]), x1 = to_f32(st.kf.v[2 * p + 1]);
    rotate_pair(x0, x1, cs);
    frag_set(st.kf, 2 * p, x0);
    frag_set(st.kf, 2 * p + 1, x1);
  }
}

// Sum over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float sum_across_kg(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const unsigned v = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Max over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48),
// with the gfx950 row-swap moves instead of LDS permutes.
__device__ __forceinline__ float max_across_kg(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const unsigned v = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// ---- work partition ---------------------------------------------------------------
// Segment s = b * Hkv + kvh holds sequence b's readable keys for KV head kvh,
// n_b = ceil(keys_b / 16) tiles (none for an invalid length).  Segments sit end
// to end in tile order, segment s starting at tile T_s = Hkv * prefix_b + kvh * n_b.
// Workgroup w of P takes tiles [floor(T w / P), floor(T (w + 1) / P)) of the T
// in total, so every workgroup streams the same number of tiles (+-1).
__device__ __forceinline__ int seq_tiles(const DecodeArgs& a, int b) {
  const int keys = decode_keys(a, b);
  return keys > 0 ? (keys + kDecodeTile - 1) / kDecodeTile : 0;
}

// Wave-uniform cursor over segments, moved forward only.
struct Seg {
  int b, kvh, T, n, keys;
};
__device__ __forceinline__ void seg_next(Seg& g, const DecodeArgs& a) {
  g.T += g.n;
  if (++g.kvh == a.n_kv_heads) {
    g.kvh = 0;
    ++g.b;
    g.keys = g.b < a.batch ? decode_keys(a, g.b) : 0;
    g.n = g.keys > 0 ? (g.keys + kDecodeTile - 1) / kDecodeTile : 0;
  }
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}
__device__ __forceinline__ int wave_incl_scan_i(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

template <typename T, int D, int G, bool SHARED, bool Q8, bool PRE>
__global__ __launch_bounds__((DecodeCfg<T, D, G, SHARED, Q8, PRE>::kWaves * 64), 1) void decode_kernel(DecodeArgs a) {
  using C = DecodeCfg<T, D, G, SHARED, Q8, PRE>;
  static_assert(C::KT == kDecodeTile, "tile size");
  const int kSlot = a.slot_floats;
  __shared__ __attribute__((aligned(4096))) char smem[C::kLdsBytes];

  // Column groups: with two, group g takes query columns 16g .. 16g + 15 (its
  // tokens), with its own workgroups and partials; workgroup w of each group
  // streams the same tiles.  Workgroups are dealt to the XCDs in turn, so the
  // two groups' workgroup w run as w' and w' + 8 of the grid: on one XCD, at
  // about the same time, and the second reads the tiles from its L2.
  const int P = static_cast<int>(gridDim.x) / a.n_groups;   // workgroups per group
  int wg = static_cast<int>(blockIdx.x), grp = 0;
  if (a.n_groups == 2) {
    if (P % 8 == 0) {
      const int x = wg % 8, i = wg / 8;
      grp = i % 2;
      wg = x + 8 * (i / 2);
    } else {
      grp = wg / P;
      wg %= P;
    }
  }
  constexpr int kGroupTokens = 16 / G;
  const int tok0 = a.tok0 + grp * kGroupTokens;   // the group's tokens tok0 .. tok0 + n_tok - 1
  const int n_tok = min(kGroupTokens, a.n_tok - grp * kGroupTokens);
  if (n_tok <= 0) return;
  float* const partials = a.partials + grp * a.group_floats;
  const int ncol = G * n_tok;   // query columns: column c is token tok0 + c / G, head c % G (<= 16)
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  constexpr int kThreads = C::kWaves * 64;
  int* misc = reinterpret_cast<int*>(smem + C::kMiscOff);

  // ---- partition: total tiles, then this workgroup's first segment -----------------
  int total = 0;
  for (int b0 = 0; b0 < a.batch; b0 += kThreads) {
    const int bb = b0 + static_cast<int>(threadIdx.x);
    const int n = wave_sum_i(bb < a.batch ? seq_tiles(a, bb) : 0);
    if (lane == 0) misc[wave] = n;
    __syncthreads();
    for (int i = 0; i < C::kWaves; ++i) total += misc[i];
    __syncthreads();
  }
  const int t_all = a.n_kv_heads * total;
  const int t_begin = static_cast<int>(static_cast<int64_t>(t_all) * wg / P);
  const int t_end = static_cast<int>(static_cast<int64_t>(t_all) * (wg + 1) / P);
  int run = 0;
  for (int b0 = 0; b0 < a.batch; b0 += kThreads) {
    const int bb = b0 + static_cast<int>(threadIdx.x);
    const int n = bb < a.batch ? seq_tiles(a, bb) : 0;
    const int incl = wave_incl_scan_i(n, lane);
    if (lane == 63) misc[wave] = incl;
    __syncthreads();
    int before = run, block = 0;
    for (int i = 0; i < C::kWaves; ++i) {
      before += (i < wave) ? misc[i] : 0;
      block += misc[i];
    }
    if (bb < a.batch) {
      const int excl = before + incl - n;
      if (wg == 0 && grp == 0) a.tile_prefix[bb] = excl;
      const int lo = a.n_kv_heads * excl;
      if (n > 0 && t_begin >= lo && t_begin < lo + a.n_kv_heads * n) {
        misc[8] = bb;
        misc[9] = (t_begin - lo) / n;
        misc[10] = lo;
      }
    }
    run += block;
    __syncthreads();
  }
  if (wg == 0 && grp == 0 && threadIdx.x == 0) a.tile_prefix[a.batch] = run;
  if (t_begin >= t_end) return;
  Seg cur;
  cur.b = misc[8];
  cur.kvh = misc[9];
  cur.keys = decode_keys(a, cur.b);
  cur.n = (cur.keys + C::KT - 1) / C::KT;
  cur.T = misc[10] + cur.kvh * cur.n;

  // ---- tile stream: the wave's k-th tile is global tile t_begin + wave + kWaves k,
  // copied into buffer k & 1; the copy of tile k + 1 starts as tile k is
  // computed, across segments ------------------------------------------------------
  const uint32_t smem0 = lds_addr(smem);
  const uint32_t tiles = smem0 + wave * C::kBufs * C::kTileBytes;
  lds_char* const tile_buf = (lds_char*)smem + wave * C::kBufs * C::kTileBytes;
  lds_char* const stage_buf = (lds_char*)smem + C::kStageOff + wave * 2 * C::kStageBytes;   // Q8
  // bytes of one head's cache rows: < 2^31 (checked on the host)
  const uint32_t span = static_cast<uint32_t>(a.cache_cap) * (Q8 ? C::kD : C::kRowBytes);
  Seg pf = cur;
  // PRE: the lane's head fragments (row hcol, dims 32u + 8kg .. +7, u < 4) of
  // the tile whose copy was issued last
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 head_next[C::kHeadSteps > 0 ? C::kHeadSteps : 1];
  auto issue = [&](lds_char* dst, int k) {
    const int g = t_begin + wave + C::kWaves * k;
    if (g >= t_end) return;
    while (g >= pf.T + pf.n) seg_next(pf, a);
    const int64_t head = static_cast<int64_t>(pf.b) * a.n_kv_heads + pf.kvh;
    const BufRsrc rk = make_rsrc(static_cast<const char*>(a.k_cache) + head * span, span);
    if constexpr (Q8) {
      const BufRsrc rs = make_rsrc(a.k_scales + head * a.cache_cap, static_cast<uint32_t>(a.cache_cap) * 4);
      issue_q8<C>(dst, rk, rs, (g - pf.T) * C::KT, pf.keys, lane);
    } else {
      const BufRsrc rv = SHARED ? rk : make_rsrc(static_cast<const char*>(a.v_cache) + head * span, span);
      issue_tile<C>(dst, rk, rv, (g - pf.T) * C::KT, pf.keys, lane);
    }
    if constexpr (PRE) {   // rows past the sequence read its last row, like the tile
      constexpr uint32_t kHeadRow = 2 * 64 * sizeof(T);
      const BufRsrc rh = make_rsrc(static_cast<const char*>(a.k_heads) + head * a.cache_cap * kHeadRow,
                                   static_cast<uint32_t>(a.cache_cap) * kHeadRow);
      const int key = min((g - pf.T) * C::KT + (lane & 15), pf.keys - 1);
#pragma unroll
      for (int u = 0; u < C::kHeadSteps; ++u)
        head_next[u] = __builtin_amdgcn_raw_buffer_load_b128(rh, key * kHeadRow + (32 * u + 8 * (lane >> 4)) * 2, 0, 0);
    }
  };
  issue(Q8 ? stage_buf : tile_buf, 0);
  // Q8: the tile after it too; the staging buffer of tile k is refilled with
  // tile k + 2 as soon as tile k is expanded, so two copies are in flight
  // while a tile is computed (a tile's codes are half the bytes of a bf16 tile).
  if constexpr (Q8) issue(stage_buf + C::kStageBytes, 1);

  // ---- rotation rates of the lane's pairs lane + 64 m (fp64, one exp2 each) ------
  constexpr int kPairsPerLane = D / 128;
  double w_pair[kPairsPerLane];
#pragma unroll
  for (int m = 0; m < kPairsPerLane; ++m)
    w_pair[m] = (lane + 64 * m < a.n_rot) ? rope_omega(lane + 64 * m, D, a.log2_theta) : 0.0;

  // ---- K=V rotation factors ------------------------------------------------------
  // The lane's rotated QK^T fragments hold key (key0 + hcol) at pairs
  // i = 16u + 4kg + p (u < kRotSteps, p < 4).  cos/sin((key0 + hcol) w_i) =
  // coarse(key0 w_i) (x) fine(hcol w_i): fine is a table shared by the
  // workgroup; coarse is kept per pair (lane = pair) and published to the wave
  // through LDS.  Every factor comes from an fp64 angle with fp64 sine and
  // cosine, rounded to fp32 once.  Between two tiles of the wave the coarse
  // factor is stepped by the rotation of the wave's tile stride (kWaves * 16
  // positions), a complex product that adds a few fp32 roundings per step; so
  // that those never add up over a long segment, every kAnchor-th tile takes
  // its coarse factor straight from the fp64 angle again.
  constexpr int kAnchor = 8;
  f32x2 coarse_l{}, step_l{};
  const uint32_t coarse_s = smem0 + C::kCoarseOff + wave * C::kCoarseBytes;
  if constexpr (C::kRot > 0) {
    static_assert(kThreads % 64 == 0 && C::kRot == 64, "fine table: thread t fills pair t % 64");
    for (int i = threadIdx.x; i < 16 * C::kRot; i += kThreads)
      lds_st<f32x2>(smem0 + C::kFineOff + (i / C::kRot) * C::kFineRow + (i % C::kRot) * 8,
                    rope_cos_sin(static_cast<double>(i / C::kRot) * w_pair[0]));
    step_l = rope_cos_sin(static_cast<double>(C::kWaves * C::KT) * w_pair[0]);
  }

  const int hcol = lane & 15, kg = lane >> 4;
  const uint32_t k_lane = key_lane_base<C, T>(tiles, lane);
  const uint32_t v_off = value_lane_base<C, T>(SHARED ? 0 : C::kKBytes, lane);   // within a buffer
  const uint32_t q_lane = smem0 + C::kQOff + lane * 8 * C::kSz;
  const uint32_t fine_lane = smem0 + C::kFineOff + hcol * C::kFineRow + 4 * kg * 8;
  const uint32_t coarse_lane = coarse_s + 4 * kg * 8;
  constexpr float kTau = 8.0f;
  constexpr int kQAhead = 2;   // QK^T steps whose LDS reads are in flight
  constexpr int kVAhead = 8;   // PV blocks whose LDS reads are in flight
  const T* __restrict__ gq = static_cast<const T*>(a.q_gain);

  int k = 0;   // the wave's next tile
  for (;;) {
    const int seg = cur.b * a.n_kv_heads + cur.kvh;
    const int p_end = min(cur.T + cur.n, t_end);
    __syncthreads();   // the previous segment's reads of the query operand are done

    // ---- query prep: QKNorm + rotation at each token's position, written in
    // operand order.  Operand fragment u, lane hcol + 16 kg, element j =
    // q~[hcol][32u + 8kg + j]; column c is token tok0 + c / G (position
    // L - q_len + tok0 + c / G) and head c % G of the group; columns >= G n_tok
    // are zeros.  One wave per column: lane owns pairs lane + 64 m.
    {
      const int L = a.seq_lens[cur.b];
      for (int h = wave; h < 16; h += C::kWaves) {
        const int tok = tok0 + h / G;
        const T* __restrict__ q = static_cast<const T*>(a.q) +
            ((static_cast<int64_t>(cur.b) * a.q_len + (h < ncol ? tok : 0)) * a.n_q_heads + cur.kvh * G + h % G) * D;
        float x[kPairsPerLane][2];
        f32x2 qcs[kPairsPerLane];
        float rstd = 0.f;
        if (h < ncol) {
          const int qpos = L - a.q_len + tok;
#pragma unroll
          for (int m = 0; m < kPairsPerLane; ++m)
            qcs[m] = (lane + 64 * m < a.n_rot) ? rope_cos_sin(static_cast<double>(qpos) * w_pair[m])
                                               : f32x2{1.f, 0.f};
          float ss = 0.f;
#pragma unroll
          for (int m = 0; m < kPairsPerLane; ++m) {
            const int pr = lane + 64 * m;
            x[m][0] = to_f32(q[2 * pr]);
            x[m][1] = to_f32(q[2 * pr + 1]);
            ss += x[m][0] * x[m][0] + x[m][1] * x[m][1];
          }
#pragma unroll
          for (int sh = 1; sh < 64; sh <<= 1) ss += wave_xor(ss, sh);
          rstd = 1.0f / sqrtf(ss / D + a.eps) * a.qk_scale_log2;
        }
#pragma unroll
        for (int m = 0; m < kPairsPerLane; ++m) {
          const int pr = lane + 64 * m;
          float x0 = 0.f, x1 = 0.f;
          if (h < ncol) {
            x0 = x[m][0] * rstd * to_f32(gq[2 * pr]);
            x1 = x[m][1] * rstd * to_f32(gq[2 * pr + 1]);
            rotate_pair(x0, x1, qcs[m]);
          }
          const int u = pr / 16, g4 = (pr % 16) / 4, j = 2 * (pr % 4);
          const uint32_t at = smem0 + C::kQOff + u * C::kFragBytes + ((h + 16 * g4) * 8 + j) * C::kSz;
          if constexpr (std::is_same<T, bf16>::value) {
            typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
            bf16x2 v;
            v[0] = from_f32<bf16>(x0);
            v[1] = from_f32<bf16>(x1);
            lds_st<bf16x2>(at, v);
          } else {
            lds_st<f32x2>(at, f32x2{x0, x1});
          }
        }
      }
    }
    if constexpr (C::kRot > 0) {   // coarse angles of the wave's first tile in this segment
      const int g = t_begin + wave + C::kWaves * k;
      coarse_l = rope_cos_sin(static_cast<double>((g - cur.T) * C::KT) * w_pair[0]);
      lds_st<f32x2>(coarse_s + lane * 8, coarse_l);
    }
    __syncthreads();   // query operand (and on the first pass the fine table) ready

    f32x4 o[C::kDBlocks];
#pragma unroll
    for (int t = 0; t < C::kDBlocks; ++t) o[t] = f32x4{};
    float m_run = -INFINITY, l_part = 0.f;
    // Keys the lane's column sees: token j of q_len sits at position
    // P = L - q_len + j.  Global layers (slot = position): slots below
    // key_lim = P + 1.  Windowed layers: slot s of the ring holds position
    // base + s, or base + s - cache_cap past the newest slot h = (L - 1) mod
    // cache_cap, and is seen when P - W < position <= P.
    const int key_lim = cur.keys - ((hcol < ncol) ? a.q_len - 1 - (tok0 + hcol / G) : 0);
    const int L_cur = a.seq_lens[cur.b];
    const int col_pos = L_cur - a.q_len + ((hcol < ncol) ? tok0 + hcol / G : a.q_len - 1);
    const int ring_h = a.window > 0 ? (L_cur - 1) % a.cache_cap : 0;
    const int ring_base = L_cur - 1 - ring_h;

    for (;; ++k) {
      const int g = t_begin + wave + C::kWaves * k;
      if (g >= p_end) break;
      const int key0 = (g - cur.T) * C::KT;
      const uint32_t buf = Q8 ? 0u : (k & 1) * C::kTileBytes;
      if constexpr (Q8) {
        // tile k has landed once at most the copy of tile k + 1 (if there is
        // one) is in flight
        if (g + C::kWaves < t_end) wait_vm_le<C::kQ8Copies>();
        else wait_vm_le<0>();
      } else {
        wait_vm_le<0>();   // tile k has landed: it is the wave's only copy in flight
      }
      // The step runs in a function whose buffers are restrict pointers: the
      // compiler then knows the copy of tile k + 1 into `nxt` does not feed
      // the reads of `cur_buf` (or of `stage`), and adds no wait for it before
      // them.
      auto step = [&](lds_char* __restrict__ cur_buf, lds_char* __restrict__ nxt,
                      lds_char* __restrict__ stage) {
        u32x4 head_cur[C::kHeadSteps > 0 ? C::kHeadSteps : 1];   // PRE: tile k's heads (landed with it)
        if constexpr (PRE) {
  #pragma unroll
          for (int u = 0; u < C::kHeadSteps; ++u) head_cur[u] = head_next[u];
        }
        f32x4 row_scale;   // Q8: scales of the lane's keys 4 kg .. 4 kg + 3
        if constexpr (Q8) {
          expand_q8<C>(stage, cur_buf, lane);
          row_scale = *(const __attribute__((address_space(3))) f32x4*)(stage + C::kCodeBytes + 16 * kg);
          lds_fence();   // the codes and scales are read before tile k + 2 lands on them
          issue(stage, k + 2);
        } else {
          issue(nxt, k + 1);
        }

        // S^T = K~ Q~^T; the lane's A operand is key row hcol, dims 32u + 8kg .. +7.
        // Reads run kQAhead steps ahead of the MFMAs.
        QkStep<T> st[kQAhead + 1];
  #pragma unroll
        for (int u = 0; u < kQAhead; ++u) load_step<C>(st[u], u, k_lane + buf, q_lane, coarse_lane, fine_lane);
        f32x4 sa = f32x4{}, sb = f32x4{};
  #pragma unroll
        for (int u = 0; u < C::kQSteps; ++u) {
          if (u + kQAhead < C::kQSteps)
            load_step<C>(st[(u + kQAhead) % (kQAhead + 1)], u + kQAhead, k_lane + buf, q_lane, coarse_lane, fine_lane);
          QkStep<T>& cs = st[u % (kQAhead + 1)];
          if constexpr (PRE) {
            if (u < C::kHeadSteps) cs.kf.v = __builtin_bit_cast(bf16x8, head_cur[u]);
          }
          if (u < C::kRotSteps) rotate_step(cs);
          mma16((u & 1) ? sb : sa, cs.kf, cs.qf);
          __builtin_amdgcn_sched_barrier(0);
        }
        f32x4 s = sa + sb;
        if constexpr (Q8) s *= row_scale;
        if constexpr (C::kRot > 0) {   // publish the wave's next tile's coarse angles
          if ((k + 1) % kAnchor == 0) {
            coarse_l = rope_cos_sin(static_cast<double>(key0 + C::kWaves * C::KT) * w_pair[0]);
          } else {
            const f32x2 c = coarse_l;
            coarse_l[0] = c[0] * step_l[0] - c[1] * step_l[1];
            coarse_l[1] = c[1] * step_l[0] + c[0] * step_l[1];
          }
          lds_st<f32x2>(coarse_s + lane * 8, coarse_l);   // read next tile, after the fence below
        }

        // online softmax; lane holds keys 4*kg + v of head column hcol
        float mt = -INFINITY;
        if (a.window > 0) {
  #pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int slot = key0 + 4 * kg + v;
            const int p = ring_base + slot - (slot > ring_h ? a.cache_cap : 0);
            if (slot >= cur.keys || p > col_pos || p <= col_pos - a.window) s[v] = -INFINITY;
          }
        } else {
  #pragma unroll
          for (int v = 0; v < 4; ++v)
            if (key0 + 4 * kg + v >= key_lim) s[v] = -INFINITY;
        }
  #pragma unroll
        for (int v = 0; v < 4; ++v) mt = fmaxf(mt, s[v]);
        mt = max_across_kg(mt);
        const bool rescale = __any(mt > m_run + kTau);
        const float m_new = rescale ? fmaxf(m_run, mt) : m_run;
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        m_run = m_new;
        Frag4<T> pf4;
        float psum = 0.f;
  #pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = __builtin_amdgcn_exp2f(s[v] - m_use);
          psum += p;
          frag_set(pf4, v, Q8 ? p * row_scale[v] : p);
        }
        if (rescale) {
  #pragma unroll
          for (int t = 0; t < C::kDBlocks; ++t) o[t] *= alpha;
          l_part *= alpha;
        }
        l_part += psum;

        // O^T += V^T P^T, reads kVAhead blocks ahead
        Frag4<T> vf[kVAhead];
  #pragma unroll
        for (int t = 0; t < kVAhead; ++t) value_frag<C>(vf[t], cur_buf, v_off, t);
  #pragma unroll
        for (int t = 0; t < C::kDBlocks; ++t) {
          const Frag4<T> vc = vf[t % kVAhead];
          if (t + kVAhead < C::kDBlocks) value_frag<C>(vf[t % kVAhead], cur_buf, v_off, t + kVAhead);
          mma16k16(o[t], vc, pf4);
          __builtin_amdgcn_sched_barrier(0);
        }
        lds_fence();   // this tile's LDS reads are done before its buffer is refilled
      };
      if constexpr (Q8) {
        step(tile_buf, stage_buf + ((k + 1) & 1) * C::kStageBytes, stage_buf + (k & 1) * C::kStageBytes);
      } else {
        step(tile_buf + buf, tile_buf + (buf ^ C::kTileBytes), nullptr);
      }
    }

    // ---- this wave's partial result for the segment --------------------------------
    // Slot kWaves * (wg + seg) + wave: wg + seg is distinct for every (workgroup,
    // segment) pair that exists, as a workgroup's segments begin where the
    // previous workgroup's end.  A wave without tiles here leaves m = -inf.
    const float l = sum_across_kg(l_part);
    float* slot = partials + static_cast<size_t>(C::kWaves * (wg + seg) + wave) * kSlot;
    if (hcol < ncol) {
#pragma unroll
      for (int t = 0; t < C::kDBlocks; ++t) *reinterpret_cast<f32x4*>(slot + hcol * D + 16 * t + 4 * kg) = o[t];
      if (kg == 0) *reinterpret_cast<f32x2*>(slot + ncol * D + 2 * hcol) = f32x2{m_run, l};
    }
    wait_vm_le<0>();   // stores retired: later tile waits count copies only
    if (p_end >= t_end) break;
    do seg_next(cur, a); while (cur.n == 0);
  }
}

// Log-sum-exp merge of one (sequence, query column): the partials of the waves of
// every workgroup that streamed the segment.  Their weights exp2(m_i - M) go to
// LDS once; then each thread accumulates whole head dims (consecutive threads,
// consecutive dims).  Invalid lengths get a NaN row.
template <typename T, int D, int G, bool SHARED>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  using C = DecodeCfg<T, D, G, SHARED>;
  const int kSlot = a.slot_floats;
  const int ncol_all = G * a.n_tok;   // the launch's columns, 16 per column group
  __shared__ float wgt[1024];
  __shared__ float red[8];
  const int seg = blockIdx.x / ncol_all, hc = blockIdx.x % ncol_all;
  constexpr int kGroupTokens = 16 / G;
  const int grp = hc / 16, h = hc % 16;   // h: column of group grp (token h / G of the group, head h % G)
  const int ncol = G * min(kGroupTokens, a.n_tok - grp * kGroupTokens);
  const float* __restrict__ partials = a.partials + grp * a.group_floats;
  const int b = seg / a.n_kv_heads, kvh = seg % a.n_kv_heads;
  const int t = threadIdx.x;
  T* __restrict__ out = static_cast<T*>(a.out) +
      ((static_cast<int64_t>(b) * a.q_len + a.tok0 + grp * kGroupTokens + h / G) * a.n_q_heads + kvh * G + h % G) *
          D;
  const int keys = decode_keys(a, b);
  if (keys < 0) {
    for (int d = t; d < D; d += 256) out[d] = from_f32<T>(NAN);
    return;
  }
  const int n = (keys + C::KT - 1) / C::KT;
  const int t_all = a.n_kv_heads * a.tile_prefix[a.batch];
  const int t_seg = a.n_kv_heads * a.tile_prefix[b] + kvh * n;
  const int64_t P = a.n_wgs;
  const int w_lo = static_cast<int>((static_cast<int64_t>(t_seg + 1) * P - 1) / t_all);
  const int w_hi = static_cast<int>((static_cast<int64_t>(t_seg + n) * P - 1) / t_all);
  const int count = (w_hi - w_lo + 1) * C::kWaves;    // <= kWaves * P <= 1024
  auto slot = [&](int i) {
    return partials + static_cast<size_t>(C::kWaves * (w_lo + i / C::kWaves + seg) + i % C::kWaves) * kSlot;
  };
  // A workgroup with an empty share (fewer tiles than workgroups) wrote nothing.
  auto written = [&](int i) {
    const int64_t w = w_lo + i / C::kWaves;
    return (t_all * w) / P < (t_all * (w + 1)) / P;
  };

  // Each thread keeps the (m, l) of its slots (at most 4: count <= 1024) in
  // registers; the max and the sum go across the wave by row-swap moves and
  // across the 4 waves through LDS, one barrier each.
  constexpr int kPer = 1024 / 256;
  float mi[kPer], li[kPer];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = t + 256 * k;
    mi[k] = -INFINITY;
    li[k] = 0.f;
    if (i < count && written(i)) {
      const f32x2 ml = *reinterpret_cast<const f32x2*>(slot(i) + ncol * D + 2 * h);
      mi[k] = ml[0];
      li[k] = ml[1];
    }
    mx = fmaxf(mx, mi[k]);
  }
  const int wave = t >> 6;
#pragma unroll
  for (int x = 1; x < kWave; x <<= 1) mx = fmaxf(mx, wave_xor(mx, x));
  if ((t & (kWave - 1)) == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float lsum = 0.f;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = t + 256 * k;
    const float w = (mi[k] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mi[k] - M);
    lsum += w * li[k];
    if (i < count) wgt[i] = w;
  }
#pragma unroll
  for (int x = 1; x < kWave; x <<= 1) lsum += wave_xor(lsum, x);
  if ((t & (kWave - 1)) == 0) red[4 + wave] = lsum;
  __syncthreads();
  const float inv = 1.0f / ((red[4] + red[5]) + (red[6] + red[7]));
  // Every slot below `count` lies in the partials buffer, so its load needs no
  // guard and several can be in flight; a zero weight (a share that wrote
  // nothing, whose slot may hold anything) selects 0 instead of the product.
  // Thread t owns D / 256 consecutive dims (one 8-byte load per slot at
  // d = 512); eight slots' loads go out together.
  constexpr int kDims = D / 256;
  static_assert(kDims == 1 || kDims == 2, "head dim 256 or 512");
  typedef float fvec __attribute__((ext_vector_type(kDims)));
  const int d0 = t * kDims;
  fvec acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = fvec(0.f);
  int i = 0;
  for (; i + 8 <= count; i += 8) {
    fvec v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const fvec*>(slot(i + k) + h * D + d0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float wk = wgt[i + k];
      acc[k % 4] += wk != 0.f ? wk * v[k] : fvec(0.f);
    }
  }
  for (; i < count; ++i) {
    const fvec v = *reinterpret_cast<const fvec*>(slot(i) + h * D + d0);
    const float wk = wgt[i];
    acc[0] += wk != 0.f ? wk * v : fvec(0.f);
  }
  const fvec o = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * inv;
#pragma unroll
  for (int k = 0; k < kDims; ++k) out[d0 + k] = from_f32<T>(o[k]);
}

template <typename T, int D, int G, bool SHARED, bool Q8 = false, bool PRE = false>
static hipError_t launch_one(const DecodeArgs& a, hipStream_t s, LaunchTimer timer) {
  using C = DecodeCfg<T, D, G, SHARED, Q8, PRE>;
  if (timer) timer(s, 2, true);
  hipLaunchKernelGGL((decode_kernel<T, D, G, SHARED, Q8, PRE>), dim3(a.n_wgs * a.n_groups), dim3(C::kWaves * 64), 0,
                     s, a);
  hipError_t e = hipGetLastError();
  if (timer) timer(s, 2, false);
  if (e != hipSuccess) return e;
  if (timer) timer(s, 3, true);
  hipLaunchKernelGGL((decode_merge_kernel<T, D, G, SHARED>), dim3(a.batch * a.n_kv_heads * G * a.n_tok), dim3(256),
                     0, s, a);
  e = hipGetLastError();
  if (timer) timer(s, 3, false);
  return e;
}

template <typename T, int D, bool SHARED>
static hipError_t launch_g(const DecodeArgs& a, int group, hipStream_t s, LaunchTimer tm) {
  if constexpr (SHARED && D == 512 && sizeof(T) == 2) {
    static_assert(DecodeCfg<T, D, 8, SHARED, true>::kWaves == DecodeCfg<T, D, 8, SHARED>::kWaves &&
                      DecodeCfg<T, D, 8, SHARED, false, true>::kWaves == DecodeCfg<T, D, 8, SHARED>::kWaves,
                  "the plan and the merge assume one wave count for every cache format");
    if (a.k_heads) {   // pre-rotated K=V cache
      if (a.k_scales) return hipErrorInvalidValue;
      switch (group) {
        case 8: return launch_one<T, D, 8, SHARED, false, true>(a, s, tm);
        case 4: return launch_one<T, D, 4, SHARED, false, true>(a, s, tm);
        default: return hipErrorInvalidValue;
      }
    }
    if (a.k_scales) {   // int8 K=V cache
      switch (group) {
        case 8: return launch_one<T, D, 8, SHARED, true>(a, s, tm);
        case 4: return launch_one<T, D, 4, SHARED, true>(a, s, tm);
        default: return hipErrorInvalidValue;
      }
    }
  }
  if (a.k_scales || a.k_heads) return hipErrorInvalidValue;
  switch (group) {
    case 1: return launch_one<T, D, 1, SHARED>(a, s, tm);
    case 2: return launch_one<T, D, 2, SHARED>(a, s, tm);
    case 4: return launch_one<T, D, 4, SHARED>(a, s, tm);
    case 8: return launch_one<T, D, 8, SHARED>(a, s, tm);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group, int kv_shared,
                         int batch, hipStream_t s, LaunchTimer tm) {
  (void)batch;
  if (dtype == 0 && head_dim == 512) return kv_shared ? launch_g<bf16, 512, true>(a, group, s, tm)
                                                      : launch_g<bf16, 512, false>(a, group, s, tm);
  if (dtype == 0 && head_dim == 256) return kv_shared ? launch_g<bf16, 256, true>(a, group, s, tm)
                                                      : launch_g<bf16, 256, false>(a, group, s, tm);
  if (dtype == 1 && head_dim == 512) return kv_shared ? launch_g<float, 512, true>(a, group, s, tm)
                                                      : hipErrorInvalidValue;   // not built (host rejects it)
  if (dtype == 1 && head_dim == 256) return kv_shared ? launch_g<float, 256, true>(a, group, s, tm)
                                                      : launch_g<float, 256, false>(a, group, s, tm);
  return hipErrorInvalidValue;
}

template <typename T, int D, bool SHARED>
static int waves_of() {
  return DecodeCfg<T, D, 8, SHARED>::kWaves;   // independent of the group size
}

bool plan_decode(int dtype, int head_dim, int group, int kv_shared, int batch, int n_kv_heads,
                 int max_tiles_per_seq, int n_cus, int q_len, int groups, DecodePlan* plan) {
  int waves = 0;
  if (dtype == 0 && head_dim == 512) waves = kv_shared ? waves_of<bf16, 512, true>() : waves_of<bf16, 512, false>();
  if (dtype == 0 && head_dim == 256) waves = kv_shared ? waves_of<bf16, 256, true>() : waves_of<bf16, 256, false>();
  if (dtype == 1 && head_dim == 512) waves = kv_shared ? waves_of<float, 512, true>() : 0;
  if (dtype == 1 && head_dim == 256) waves = kv_shared ? waves_of<float, 256, true>() : waves_of<float, 256, false>();
  if (waves == 0) return false;
  // One workgroup per CU (at most 1024 partials per segment in the merge), but
  // no more workgroups than give each wave two tiles of the largest possible
  // total.
  const int64_t tiles_ub = static_cast<int64_t>(batch) * n_kv_heads * max_tiles_per_seq;
  const int64_t by_work = (tiles_ub + 2 * waves - 1) / (2 * waves);
  // With two column groups each group gets half the CUs (a multiple of 8, so
  // that the groups' workgroups pair up on the XCDs).
  int64_t wgs = n_cus < 1 ? 1 : n_cus;
  if (groups == 2) wgs = wgs >= 16 ? wgs / 16 * 8 : (wgs + 1) / 2;
  wgs = wgs > 1024 / waves ? 1024 / waves : wgs;
  wgs = wgs > by_work ? by_work : wgs;
  plan->waves = waves;
  plan->groups = groups;
  plan->n_wgs = static_cast<int>(wgs < 1 ? 1 : wgs);
  plan->prefix_bytes = (static_cast<size_t>(batch + 1) * 4 + 255) / 256 * 256;
  plan->slots = static_cast<size_t>(waves) * (plan->n_wgs + static_cast<size_t>(batch) * n_kv_heads);
  plan->slot_floats = static_cast<size_t>(q_len < 16 / group ? q_len : 16 / group) * group * head_dim + 64;
  return true;
}

}  // namespace ga
