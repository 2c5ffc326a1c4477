// Flash-style causal prefill for one layer type, gfx950.
//
// A workgroup owns one KV head of one sequence and QB consecutive query
// positions: all G query heads of the group at those positions share every key
// tile it stages in LDS (the grouped-query sharing of "Gemma 4多模态大模型架构详解",
// section "分组查询注意力").  Its query rows (QB positions x G heads) are
// split over four waves, one wave per SIMD, each with kRB blocks of 32 rows
// (one block at d = 512, two at d = 256, so that every key and value
// fragment read from LDS feeds kRB MFMAs).  Per key tile of 32 positions each
// wave computes, for each row block, over the full head dim:
//   S^T[key][row] = K~ Q~^T      32x32x16 bf16 MFMAs, A = key rows read from
//                                LDS, B = the wave's normalised, rotated queries
//                                held in registers
//   softmax per row               in registers, exp2 domain (a lane holds 16
//                                of the 32 keys of its row, the lane 32 apart
//                                the rest): P = 2^S directly where QKNorm
//                                bounds the wave's scores (score_bound_ok),
//                                else with a running max
//   O^T[d][row] += V^T P^T       32x32x16 MFMAs; V^T by transposing LDS reads of
//                                the value rows, P straight from the score
//                                registers
// Each wave keeps 32 kRB rows x d fp32 accumulators (256 registers at d = 512
// and at d = 256, in the accumulation register file, AGPRs); the scores of a
// tile stay in VGPRs
// (MFMAs in VGPR form for QK^T, the PV MFMAs written out with AGPR
// accumulators).
//
// With three or more stages (every bf16 layer) the tile loop is software
// pipelined: step i takes the row max of tile i's scores, then runs the QK^T
// MFMAs of tile i + 1 with tile i's exponentials under them, then the PV
// MFMAs of tile i.  With one wave per SIMD nothing else would feed the matrix
// unit while a wave computes its softmax.  Edge tiles (the causal diagonal,
// the window's lower edge) run a masked copy of the step; all other tiles
// skip the mask.
//
// Tiles are 32 row-major rows (16-byte chunk c of row r stored at
// c ^ swz(r), see row_swizzle),
// copied global -> LDS by buffer loads that write LDS directly, kStages tiles
// deep.  K=V layers ("Gemma 4多模态大模型架构详解", section "K=V") stage the
// value rows (the normalised unrotated keys) plus only the rotated head of the
// keys (dims 0..127, p-RoPE section "p-RoPE（低频剪枝旋转位置编码）"): the
// other key dims are read from the value rows, so a tile takes 40 KiB instead
// of 64 and four fit in LDS.  Windowed layers start at the first tile that
// can hold a visible key and mask keys with j <= i - W (section
// "交错层（局部与全局注意力）").
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ga {

template <typename T, int D, int G, bool SHARED>
struct PrefillCfg {
  static constexpr int KT = kPrepTile;              // keys per tile
  static constexpr int kWaves = 4;
  static constexpr int kRows = 32;                  // query rows of one row block
  // Row blocks per wave: local (d = 256) bf16 layers take two, so that each
  // key and value fragment read from LDS feeds two MFMAs and the wave's
  // 64 x 256 fp32 outputs fill the accumulation registers as the global
  // layers' 32 x 512 do.
  static constexpr int kRB = (D == 256 && sizeof(T) == 2) ? 2 : 1;
  static constexpr int PW = kRB * kRows / G;        // positions per wave
  static constexpr int QB = kWaves * PW;            // positions per workgroup
  static constexpr int kQSteps = D / 16;            // QK^T reduction steps
  static constexpr int kDBlocks = D / 32;           // 32-dim output blocks
  static constexpr int kSz = int(sizeof(T));
  static constexpr bool kShared = SHARED;
  static constexpr int kKW = SHARED ? 128 : D;      // key dims staged from the key rows
  static constexpr int kKSteps = kKW / 16;          // QK^T steps reading the key rows
  static constexpr int kKRowBytes = kKW * kSz;
  static constexpr int kVRowBytes = D * kSz;
  static constexpr int kKBytes = KT * kKRowBytes;   // key region of a stage
  static constexpr int kVBytes = KT * kVRowBytes;   // value region (after the key region)
  static constexpr int kStageBytes = kKBytes + kVBytes;
  static constexpr int kLdsCap = 160 * 1024;
  static constexpr int kMaxStages = 4;
  static constexpr int kStages = (kMaxStages * kStageBytes <= kLdsCap)       ? kMaxStages
                                 : (3 * kStageBytes <= kLdsCap && kMaxStages >= 3) ? 3
                                 : (2 * kStageBytes <= kLdsCap)                    ? 2
                                                                                   : 1;
  // Local layers stage the (cos, sin) rows of their query positions in fp16 in
  // the LDS the prologue does not use yet (the last stage and past it): each
  // wave copies its PW positions' rows with whole-row loads, and each lane
  // then reads its pairs from LDS instead of 32 scattered rows from memory.
  static constexpr bool kTabLds = sizeof(T) == 2 && kRB == 2 && !SHARED && kStages == 4 &&
                                  (kStages - 1) * kStageBytes + kWaves * PW * (D / 2 * 4) <= kLdsCap;
  static constexpr int kTabRow = D / 2 * 4;                     // one position's pairs (full rotation)
  static constexpr int kTabOff = (kStages - 1) * kStageBytes;
  static constexpr int kTabBytes = kTabLds ? kWaves * PW * kTabRow : 0;
  static constexpr int kLdsBytes = kTabLds && kTabOff + kTabBytes > kStages * kStageBytes ? kTabOff + kTabBytes
                                                                                          : kStages * kStageBytes;
  static constexpr int kDmaK = kKBytes / 1024, kDmaV = kVBytes / 1024;
  static constexpr int kDmaPerWave = (kDmaK + kDmaV) / kWaves;
  // Key fragment reads in flight and value fragments (two reads each) in
  // flight: fewer with two row blocks, whose second query block takes the
  // registers (four and four spilled inside the tile loop; two and two do
  // not, 1% faster).
  static constexpr int kKAhead = kRB == 2 ? 2 : 6;
  static constexpr int kVAhead = kRB == 2 ? 2 : 4;
  static_assert(kLdsBytes <= kLdsCap, "LDS budget");
  static_assert(!kTabLds || (kTabRow % 512 == 0 && PW % 2 == 0), "table rows: two per copy instruction");
  static_assert((kDmaK + kDmaV) % kWaves == 0 && kKBytes % 1024 == 0, "tile copy split");
  static_assert(kKBytes % kVRowBytes == 0 && kStageBytes % kVRowBytes == 0, "row alignment for the swizzle");
  static_assert(kKRowBytes >= 256 && kVRowBytes >= 256, "row swizzle needs 16 chunks per row");
  static_assert(kStages <= 4 && (kStages - 2) * kDmaPerWave < 64, "copy counter range");
};

// Accelerator complex dies (each with its own L2) that workgroups are dealt
// to in turn.
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) char lds_char;
typedef __amdgpu_buffer_rsrc_t BufRsrc;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char*)p));
}
template <typename V>
__device__ __forceinline__ V lds_ld(uint32_t addr) {
  return *(const __attribute__((address_space(3))) V*)(static_cast<uintptr_t>(addr));
}

// Raw buffer over one head's rows (dword 3: 32-bit data format, as untyped
// buffer loads need); loads past `bytes` return zeros.
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

template <int N>
__device__ __forceinline__ void wait_vm_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Wait until at most `later` tiles' copies of this wave are still in flight.
template <typename C>
__device__ __forceinline__ void wait_tiles(int later) {
  if (later >= 2 && C::kStages >= 4) wait_vm_le<(C::kStages >= 4 ? 2 * C::kDmaPerWave : 0)>();
  else if (later >= 1 && C::kStages >= 3) wait_vm_le<(C::kStages >= 3 ? C::kDmaPerWave : 0)>();
  else wait_vm_le<0>();
}

// Max / sum with the other half of the wave (lane l ^ 32), by the gfx950
// row-swap move.
__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc *= alpha for an accumulator that lives in the accumulation registers
// (AGPRs): read, multiply and write back in place, so the accumulator never
// needs a copy in the vector registers.
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\ts_nop 1\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(acc[r]), "=&v"(tmp)
                 : "v"(alpha));
  }
}
// Two floats as a pair of bf16 (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_f32<bf16>(lo))) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_f32<bf16>(hi))) << 16);
}
// O += A B for an output block held in the accumulation registers (AGPRs).
// This file is built with MFMAs in VGPR form, so the QK^T scores stay in
// VGPRs and all 256 AGPRs hold the 32 x 512 output block of a wave (with the
// scores' 16 registers also in AGPRs, one output block would not fit and the
// compiler moved it between the two register files twice per tile: 64 moves
// per step).  This MFMA is written out so that its accumulator stays in AGPRs.
// The compiler adds no wait states around it: the s_nop gives the two a
// VALU write of A or B needs before an MFMA reads it (here the softmax
// weights, converted by VALU ops); readers of the accumulator wait on their
// own (update_max, the epilogue).
__device__ __forceinline__ void mma32_acc(f32x16& c, const Frag8<bf16>& a, const Frag8<bf16>& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a.v), "v"(b.v));
}
__device__ __forceinline__ void mma32_acc(f32x16& c, const Frag8<float>& a, const Frag8<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x2_f32 %0, %1, %2, %0" : "+a"(c) : "v"(a.v[j]), "v"(b.v[j]));
}
__device__ __forceinline__ float read_acc(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Scheduling pattern for a pipelined operand stream of N steps of M MFMAs
// sharing R LDS reads, whose reads run A steps ahead: the first A*R reads
// (when PRE; else they were issued before this region), then M MFMAs and R
// reads alternately, then the last A steps; NV global->LDS copies go one
// after every SV-th step.  Keeps the reads in flight where the scheduler would
// otherwise trade prefetch depth for registers, and spreads the copies so the
// wave never queues many of them at once.  Other work (the exponentials) is
// left to the scheduler: fixed vector-ALU slots between the MFMAs measured
// slower.
template <int A, int N, int R, int NV = 0, int SV = 1, bool PRE = true, int M = 1>
__device__ __forceinline__ void interleave_reads_mfma() {
  if constexpr (PRE) __builtin_amdgcn_sched_group_barrier(0x100, A * R, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    if (i < N - A) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    if (NV > 0 && i % SV == 0 && i / SV < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

// Row swizzle: 16-byte chunk c of row r sits at chunk c ^ row_swizzle(r), the
// two low bit pairs of r swapped.  The 16 rows of one key-operand read (lanes
// 0..15 or 16..31, same chunk) land on 16 different chunks, and the 4
// consecutive rows a transposing value read touches per half-wave land in 4
// different 64-byte bank groups, so neither read has bank conflicts.
__device__ __forceinline__ int row_swizzle(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Copy of a tile (32 rows of each region) into a stage: copy instruction i of
// the stage moves 1 KiB, lane l writing LDS slot stage + 1024 i + 16 l with
// the row chunk the swizzle places there.  Wave w issues instructions
// w, w + kWaves, ...; copy_piece gives the k-th of them.
struct CopyPiece {
  bool is_k;     // key region (else value region)
  int rb;        // row bytes of that region in LDS
  int gs;        // bytes between consecutive rows of that region in global memory
  int lds;       // LDS offset of the instruction within the stage
  int voff;      // byte offset within the tile's rows in global memory
};
// vstride: bytes between consecutive value rows in global memory.  K=V layers
// stage the workspace's value rows (kVRowBytes apart, a compile-time
// constant); layers with a separate V read v where it lies, token-major.
template <typename C>
__device__ __forceinline__ CopyPiece copy_piece(int k, int wave, int lane, uint32_t vstride) {
  static_assert(C::kDmaK % C::kWaves == 0, "key-region instructions split evenly over the waves");
  constexpr int kPerWaveK = C::kDmaK / C::kWaves;
  CopyPiece cp;
  cp.is_k = k < kPerWaveK;                                  // known at compile time with k
  const int j = (cp.is_k ? k : k - kPerWaveK) * C::kWaves + wave;   // piece within its region
  const int i = (cp.is_k ? 0 : C::kDmaK) + j;               // = k kWaves + wave
  cp.rb = cp.is_k ? C::kKRowBytes : C::kVRowBytes;
  cp.gs = cp.is_k ? C::kKRowBytes : (C::kShared ? C::kVRowBytes : static_cast<int>(vstride));
  int r, slot;
  if (cp.rb >= 1024) {
    r = j / (cp.rb / 1024);
    slot = (j % (cp.rb / 1024)) * 64 + lane;
  } else {
    r = j * (1024 / cp.rb) + lane / (cp.rb / 16);
    slot = lane % (cp.rb / 16);
  }
  cp.lds = i * 1024;
  cp.voff = r * cp.gs + ((slot ^ row_swizzle(r)) << 4);
  return cp;
}
// One copy instruction of a tile.  The tile's first row goes into the scalar
// offset, which the buffer's range check does not cover, except for values
// read in place (separate-V layers): there the whole offset is in the checked
// per-lane offset, so the rows past the sequence in its last tile read zeros
// instead of memory past v.
template <typename C>
__device__ __forceinline__ void copy_load(const CopyPiece& cp, BufRsrc rk, BufRsrc rv, lds_char* dst, int tile) {
  const uint32_t tile_off = static_cast<uint32_t>(tile) * C::KT * cp.gs;
  if (!C::kShared && !cp.is_k)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst + cp.lds, 16, cp.voff + tile_off, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(cp.is_k ? rk : rv, dst + cp.lds, 16, cp.voff, tile_off, 0, 0);
}
template <typename C>
__device__ __forceinline__ void issue_tile(BufRsrc rk, BufRsrc rv, uint32_t vstride, int tile, lds_char* dst, int wave,
                                           int lane) {
#pragma unroll
  for (int k = 0; k < C::kDmaPerWave; ++k) {
    const CopyPiece cp = copy_piece<C>(k, wave, lane, vstride);
    copy_load<C>(cp, rk, rv, dst, tile);
  }
}

// off ^ x, where off is a lane's offset into a row-aligned region (row base,
// plus a swizzled chunk in bits 4..7, plus bits below 4) and x < the row size
// is a per-step chunk offset.  Bits 8 and up of x meet only zero bits of off
// below the row base, so they add without carry: only the low byte needs a
// VALU XOR, and the rest becomes the read's immediate offset.
__device__ __forceinline__ int chunk_xor(int off, int x) { return (off ^ (x & 0xff)) + (x & ~0xff); }

// QK^T A operand of step u: the 8 elements of key row l%32 at dims 16u + 8h ..,
// at stage `st`, from the lane's row offset `off` (lane part of the chunk
// already swizzled; the step part enters as an XOR).
template <typename V>
__device__ __forceinline__ V st_ld(const lds_char* st, int off) {
  return *(const __attribute__((address_space(3))) V*)(st + off);
}
__device__ __forceinline__ void key_frag(Frag8<bf16>& f, const lds_char* st, int off, int u) {
  f.v = st_ld<bf16x8>(st, chunk_xor(off, (2 * u) << 4));
}
__device__ __forceinline__ void key_frag(Frag8<float>& f, const lds_char* st, int off, int u) {
  const int o = chunk_xor(off, (4 * u) << 4);
  const f32x4 a = st_ld<f32x4>(st, o);
  const f32x4 b = st_ld<f32x4>(st, o ^ 16);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}

// PV A operand for dims 32t .. 32t+31 and key step c: lane l needs
// V[tile_key(c, h, j)][32t + l%32], j = 0..7, tile_key(c, h, j) =
// 16c + 8(j/4) + 4h + j%4 (the keys the lane's score registers 8c .. 8c+7
// hold).  bf16: two transposing reads (j < 4 and j >= 4); within a 16-lane
// group, lane i receives element i%4 of the 8-byte pieces addressed by lanes
// i/4 + 4j', so lane p of group g addresses key 16c + 4(g/2) + p/4 (+8), dims
// 32t + 16(g%2) + 4(p%4) .. +3.  `vt[s]` are those lane offsets for t = 0,
// c = 0; t enters as an XOR of the chunk, c as 16 rows further on.
template <typename C>
__device__ __forceinline__ void value_frag(Frag8<bf16>& f, const lds_char* st, const int (&vt)[2], int t, int c) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int off = chunk_xor(vt[s], (4 * t) << 4) + c * 16 * C::kVRowBytes;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(st + off));
    const bf16x4 w = __builtin_bit_cast(bf16x4, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.v[4 * s + j] = w[j];
  }
}
// fp32: eight plain reads (slow path for exact tests).
template <typename C>
__device__ __forceinline__ void value_frag_f32(Frag8<float>& f, const lds_char* st, int t, int c, int lane) {
  const int h = lane >> 5, d = 32 * t + (lane & 31);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int key = 16 * c + 8 * (j / 4) + 4 * h + (j % 4);
    const int byte = d * 4;
    f.v[j] = st_ld<float>(st, C::kKBytes + key * C::kVRowBytes + (((byte >> 4) ^ row_swizzle(key)) << 4) + (byte & 15));
  }
}

// Where query fragment u of this lane comes from: registers (bf16), or the raw
// query row normalised, rotated and scaled again at each use (fp32).
template <typename T, int D>
struct QSource {
  const Frag8<T>* regs;
  const T* row;
  const T* gain;
  const f32x2* table;    // (cos, sin) of the row's position, n_rot pairs
  float rs;              // 1 / rms(q) * softmax scale * log2(e)
  int n_rot;
};
template <typename T, int D>
__device__ __forceinline__ void make_qfrag(Frag8<T>& f, const QSource<T, D>& q, int u, int h) {
  const int d0 = 16 * u + 8 * h;
  Frag8<T> gain;
  load_frag(gain, q.gain + d0);
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = to_f32(f.v[j]) * q.rs * to_f32(gain.v[j]);
  if (d0 < 2 * q.n_rot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x2 cs = q.table[min(d0 / 2 + j, q.n_rot - 1)];
      if (d0 / 2 + j < q.n_rot) rotate_pair(x[2 * j], x[2 * j + 1], cs);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) frag_set(f, j, x[j]);
}
template <typename T, int D>
__device__ __forceinline__ Frag8<T> query_frag(const QSource<T, D>& q, int u, int h) {
  if constexpr (sizeof(T) == 2) {
    return q.regs[u];
  } else {
    Frag8<T> f;
    load_frag(f, q.row + 16 * u + 8 * h);
    make_qfrag(f, q, u, h);
    return f;
  }
}

// acc + the sum of squares of a bf16 fragment, by paired dot products on the
// packed values (the squares are exact in fp32).  Working on the packed
// words also keeps the compiler from holding fp32 copies of the query.
__device__ __forceinline__ float sum_squares(const Frag8<bf16>& f, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 p = {f.v[2 * i], f.v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
  }
  return acc;
}

// Per-lane operand offsets within a stage.
struct LaneOffsets {
  int kq, vq;      // QK^T key rows: key region, value region (K=V dims >= 128)
  int vt[2];       // PV transposing reads
};

// Running softmax state of the wave's 32 rows.
template <int NB>
struct RowState {
  f32x16 o[NB];
  float m_run, l_part;
};

// ---- pieces of a tile step ----------------------------------------------------

// First kKAhead key fragments of the S^T of the tile at `cur`.
template <typename C, typename T, int D>
__device__ __forceinline__ void qk_prefetch(Frag8<T> (&kf)[C::kKAhead], const lds_char* cur, const LaneOffsets& lo) {
#pragma unroll
  for (int u = 0; u < C::kKAhead; ++u) key_frag(kf[u], cur, u < C::kKSteps ? lo.kq : lo.vq, u);
}
// S^T[key][row] of the tile at `cur` from prefetched fragments `kf`, later
// fragments read kKAhead steps ahead of the MFMAs.  `copy(k)`, k < NC, goes
// after every (kQSteps / NC)-th MFMA, and `work(u)` (other, independent work)
// after MFMA u in program order.
// PRE: the kKAhead prefetch reads are in the same scheduling region (no
// branch between them and this run), so the pattern places them first.
template <typename C, typename T, int D, int NC, bool PRE = false, typename CopyFn, typename WorkFn>
__device__ __forceinline__ void qk_run(f32x16 (&s)[C::kRB], Frag8<T> (&kf)[C::kKAhead], const lds_char* cur,
                                       const LaneOffsets& lo, const QSource<T, D> (&qs)[C::kRB], int h,
                                       CopyFn&& copy, WorkFn&& work) {
  constexpr int kStride = NC > 0 ? C::kQSteps / NC : 1;
  static_assert(NC <= C::kQSteps, "one copy per QK^T step at most");
#pragma unroll
  for (int rb = 0; rb < C::kRB; ++rb) s[rb] = f32x16{};
#pragma unroll
  for (int u = 0; u < C::kQSteps; ++u) {
    const Frag8<T> k = kf[u % C::kKAhead];
    if (u + C::kKAhead < C::kQSteps)
      key_frag(kf[u % C::kKAhead], cur, u + C::kKAhead < C::kKSteps ? lo.kq : lo.vq, u + C::kKAhead);
#pragma unroll
    for (int rb = 0; rb < C::kRB; ++rb) mma32(s[rb], k, query_frag(qs[rb], u, h));   // one key read, kRB MFMAs
    if (NC > 0 && u % kStride == 0 && u / kStride < NC) copy(u / kStride);
    work(u);
  }
  if constexpr (sizeof(T) == 2)
    interleave_reads_mfma<C::kKAhead, C::kQSteps, 1, NC, kStride, PRE, C::kRB>();
}

// Scores of an edge tile masked: register r of this lane is key
// key0 + 8(r/4) + 4h + r%4 of the lane's query row; visible keys satisfy
// pos - W < key <= pos, that is diff - W < c_r <= diff with
// diff = pos - key0 - 4h and c_r = 8(r/4) + r%4.
__device__ __forceinline__ void mask_scores(float (&sv)[16], int key0, int pos, int window, int h) {
  const int diff = pos - key0 - 4 * h;
  const int low = window > 0 ? diff - window : -(1 << 30);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int c = 8 * (r / 4) + (r % 4);
    sv[r] = (c <= diff && c > low) ? sv[r] : -INFINITY;
  }
}

// Row max of the tile's scores and the lazy rescale of the running state: O
// and the partial sum are rescaled only when the row max grows by more than
// 2^kTau (scores are bounded after QKNorm, so this is rare past the first
// tiles).  Returns the max the exponentials subtract.
template <int NB>
__device__ __forceinline__ float update_max(const float (&sv)[16], RowState<NB>& rs) {
  float mt = sv[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sv[r]);
  mt = max_halves(mt);
  constexpr float kTau = 8.0f;
  if (__any(mt > rs.m_run + kTau)) {
    const float m_new = fmaxf(rs.m_run, mt);
    if (rs.m_run != -INFINITY) {   // nothing accumulated yet otherwise
      const float alpha = __builtin_amdgcn_exp2f(rs.m_run - m_new);
      // the last output MFMA has retired before its accumulators are read,
      // and the writes land before the next one reads them
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int t = 0; t < NB; ++t) scale_acc(rs.o[t], alpha);
      asm volatile("s_nop 4" ::: "memory");
      rs.l_part *= alpha;
    }
    rs.m_run = m_new;
  }
  return rs.m_run == -INFINITY ? 0.f : rs.m_run;
}

// Softmax weight r (of the lane's 16) into the B operands of the PV MFMAs
// (score registers 8c .. 8c+7 form operand c), and into the lane's part of
// the row sum.  bf16: the row sum adds the rounded weights the MFMAs use, a
// pair at a time (paired dot product with ones), so the weights of a row sum
// to one after the division; a row with one visible key returns its value
// row exactly.
__device__ __forceinline__ void put_weight(Frag8<bf16> (&pf)[2], int r, float p, float& l) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  frag_set(pf[r / 8], r % 8, p);
  if (r % 2 == 1) {
    const bf16x2 w = {pf[r / 8].v[r % 8 - 1], pf[r / 8].v[r % 8]};
    const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    l = __builtin_amdgcn_fdot2_f32_bf16(w, one, l, false);
  }
}
__device__ __forceinline__ void put_weight(Frag8<float> (&pf)[2], int r, float p, float& l) {
  frag_set(pf[r / 8], r % 8, p);
  l += p;
}

// P = exp2(S - m) into the two B operands of the PV MFMAs, and the lane's
// part of the row sum.
template <typename T>
__device__ __forceinline__ void tile_exps(Frag8<T> (&pf)[2], const float (&sv)[16], float m_use, float& l) {
#pragma unroll
  for (int r = 0; r < 16; ++r) put_weight(pf, r, __builtin_amdgcn_exp2f(sv[r] - m_use), l);
}

// O^T += V^T P^T from the value rows of the stage at `st`: step f = 2t + c
// pairs value block t with keys 16c .. 16c+15 (score registers 8c .. 8c+7).
template <typename C, typename T, int NB>
__device__ __forceinline__ void pv_tile(const lds_char* st, const LaneOffsets& lo, const Frag8<T> (&pf)[C::kRB][2],
                                        RowState<NB> (&rs)[C::kRB], int lane) {
  if constexpr (sizeof(T) == 2) {
    Frag8<T> vf[C::kVAhead];
#pragma unroll
    for (int f = 0; f < C::kVAhead; ++f) value_frag<C>(vf[f], st + C::kKBytes, lo.vt, f >> 1, f & 1);
#pragma unroll
    for (int f = 0; f < 2 * C::kDBlocks; ++f) {
      const Frag8<T> v = vf[f % C::kVAhead];
      if (f + C::kVAhead < 2 * C::kDBlocks)
        value_frag<C>(vf[f % C::kVAhead], st + C::kKBytes, lo.vt, (f + C::kVAhead) >> 1, (f + C::kVAhead) & 1);
#pragma unroll
      for (int rb = 0; rb < C::kRB; ++rb) mma32_acc(rs[rb].o[f >> 1], v, pf[rb][f & 1]);   // one value read
    }
  } else {
#pragma unroll
    for (int f = 0; f < 2 * C::kDBlocks; ++f) {
      Frag8<T> vf;
      value_frag_f32<C>(vf, st, f >> 1, f & 1, lane);
#pragma unroll
      for (int rb = 0; rb < C::kRB; ++rb) mma32_acc(rs[rb].o[f >> 1], vf, pf[rb][f & 1]);
    }
  }
}

// Copy instruction k of this wave for tile `tile` into stage `nxt`.  Tiles
// past the sequence's padded end read zeros (the buffer's range check); past
// this workgroup's last tile they are never used.  The per-lane offsets do
// not depend on the tile, so the compiler keeps them in registers across the
// loop (measured faster than recomputing them at each use).
template <typename C>
struct TileCopier {
  BufRsrc rk, rv;
  uint32_t vstride;
  lds_char* nxt;
  int tile, wave, ln;
  __device__ __forceinline__ void operator()(int k) const {
    const CopyPiece cp = copy_piece<C>(k, wave, ln, vstride);
    copy_load<C>(cp, rk, rv, nxt, tile);
  }
};
template <typename C>
__device__ __forceinline__ TileCopier<C> make_copier(const char* kbase, const char* vbase, uint32_t kspan,
                                                     uint32_t vspan, uint32_t vstride, lds_char* nxt, int tile,
                                                     int wave, int lane) {
  return TileCopier<C>{make_rsrc(kbase, kspan), make_rsrc(vbase, vspan), vstride, nxt, tile, wave, lane};
}

// One whole tile (fewer than three stages): QK^T, softmax and PV from `cur`,
// with the copy of tile next_tile into `nxt` spread over the QK^T MFMAs.
// `cur` and `nxt` are distinct stages: with them as restrict pointers the
// compiler knows the copy does not feed this tile's reads (the kernel's own
// waits order the copies), and adds no waits for the copies before the LDS
// reads.
template <typename C, typename T, int D, bool MASK>
__device__ __forceinline__ void tile_step(const lds_char* __restrict__ cur, lds_char* __restrict__ nxt,
                                          const char* kbase, const char* vbase, uint32_t kspan, uint32_t vspan,
                                          uint32_t vstride, int next_tile, int wave, int lane, const LaneOffsets& lo,
                                          const QSource<T, D> (&qs)[C::kRB], int key0, const int (&pos)[C::kRB],
                                          int window, RowState<C::kDBlocks> (&rs)[C::kRB]) {
  const int h = lane >> 5;
  const TileCopier<C> copy = make_copier<C>(kbase, vbase, kspan, vspan, vstride, nxt, next_tile, wave, lane);
  f32x16 s[C::kRB];
  Frag8<T> kf[C::kKAhead];
  qk_prefetch<C, T, D>(kf, cur, lo);
  qk_run<C, T, D, (C::kStages > 1 ? C::kDmaPerWave : 0)>(s, kf, cur, lo, qs, h, copy, [](int) {});
  Frag8<T> pf[C::kRB][2];
#pragma unroll
  for (int rb = 0; rb < C::kRB; ++rb) {
    float sv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = s[rb][r];
    if constexpr (MASK) mask_scores(sv, key0, pos[rb], window, h);
    const float m_use = update_max(sv, rs[rb]);
    tile_exps(pf[rb], sv, m_use, rs[rb].l_part);
  }
  pv_tile<C, T>(cur, lo, pf, rs, lane);
}

// One pipelined step (three or more stages): the softmax and PV of tile i
// (its scores in `s`, from the step before; its values at `vcur`), with the
// QK^T of tile i + 1 (keys at `kcur`, scores into `s`) between the row max and
// PV, so that the exponentials of tile i run under the QK^T MFMAs of tile
// i + 1 instead of stalling the matrix unit.  The copy of tile next_tile into
// `nxt` spreads over those MFMAs.  NEXT = false: the last tile, no QK^T and no
// copy.  All three stages are distinct (restrict, as for tile_step).  s_in
// (tile i's scores) and s_out (tile i + 1's) may be one array: the scores are
// copied first.
// FIXED: the wave's scores are known to lie within +-kScoreBound (see
// score_bound_ok), so P = 2^S needs no running max: no row max, no rescale
// test and no subtraction.
template <typename C, typename T, int D, bool MASK, bool NEXT, bool FIXED>
__device__ __forceinline__ void pipe_step(const lds_char* __restrict__ kcur, const lds_char* __restrict__ vcur,
                                          lds_char* __restrict__ nxt, const char* kbase, const char* vbase,
                                          uint32_t kspan, uint32_t vspan, uint32_t vstride, int next_tile, int wave,
                                          int lane,
                                          const LaneOffsets& lo, const QSource<T, D> (&qs)[C::kRB], int key0,
                                          const int (&pos)[C::kRB], int window, RowState<C::kDBlocks> (&rs)[C::kRB],
                                          const f32x16 (&s_in)[C::kRB], f32x16 (&s_out)[C::kRB]) {
  const int h = lane >> 5;
  Frag8<T> kf[C::kKAhead];
  if constexpr (NEXT) qk_prefetch<C, T, D>(kf, kcur, lo);
  float sv[C::kRB][16];
  float m_use[C::kRB];
#pragma unroll
  for (int rb = 0; rb < C::kRB; ++rb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[rb][r] = s_in[rb][r];
    if constexpr (MASK) mask_scores(sv[rb], key0, pos[rb], window, h);
    if constexpr (FIXED) m_use[rb] = 0.f;
    else m_use[rb] = update_max(sv[rb], rs[rb]);
  }
  Frag8<T> pf[C::kRB][2];
  if constexpr (NEXT) {
    // exponential r of every row block after QK^T step r
    const TileCopier<C> copy = make_copier<C>(kbase, vbase, kspan, vspan, vstride, nxt, next_tile, wave, lane);
    // without the rescale test's branch the prefetch reads share the region
    qk_run<C, T, D, C::kDmaPerWave, FIXED>(s_out, kf, kcur, lo, qs, h, copy, [&](int u) {
      if (u < 16) {
#pragma unroll
        for (int rb = 0; rb < C::kRB; ++rb)
          put_weight(pf[rb], u, __builtin_amdgcn_exp2f(FIXED ? sv[rb][u] : sv[rb][u] - m_use[rb]), rs[rb].l_part);
      }
    });
  } else {
#pragma unroll
    for (int rb = 0; rb < C::kRB; ++rb) tile_exps(pf[rb], sv[rb], m_use[rb], rs[rb].l_part);
  }
  pv_tile<C, T>(vcur, lo, pf, rs, lane);
}

// Scores S = q~ . k~ (q~ already scaled by softmax scale * log2(e)) satisfy
// |S| <= |q~| max |k~| (Cauchy-Schwarz).  QKNorm makes both lengths about
// sqrt(d) times the gains' rms, so with moderate gains and the 1/sqrt(d)
// scale the bound is a few tens: then P = 2^S lies in [2^-kScoreBound,
// 2^kScoreBound] and needs no running max (a constant shift of the
// exponent does not change the softmax).  Row sums stay below 2^(kScoreBound
// + 22) for 4M keys, far inside fp32.  Rows whose bound is larger keep the
// online max.
constexpr float kScoreBound = 40.f;
// True when every row of the wave is within the bound: qn2 its squared query
// length, kn2 the largest squared key length of the tiles it reads.  2% of
// margin covers the rounding of the sums of squares; NaN gives false.
__device__ __forceinline__ bool score_bound_ok(float qn2, float kn2) {
  const float b2 = qn2 * kn2 * 1.0404f;
  return !__any(!(b2 <= kScoreBound * kScoreBound));
}

template <typename T, int D, int G, bool SHARED>
__global__ __launch_bounds__(256, 1) void prefill_attn_kernel(PrefillArgs a) {
  using C = PrefillCfg<T, D, G, SHARED>;
  __shared__ __attribute__((aligned(4096))) char smem[C::kLdsBytes];

  const int n_qb = (a.seq_len + C::QB - 1) / C::QB;
  int qb, kvh, b;
  if (a.window > 0) {
    // Windowed layers: every workgroup has about the same work, and the
    // windows of neighbouring query blocks share all but two key tiles.
    // Workgroups are dispatched round-robin over the XCDs (each with its own
    // L2), so the linear workgroup index is remapped to give each XCD a
    // contiguous run of (head, query block): the blocks an XCD runs together
    // are neighbours, and their tiles are read from its L2.
    const int n = static_cast<int>(gridDim.x * gridDim.y * gridDim.z);
    const int w = static_cast<int>(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    const int per = n / kXcds, extra = n % kXcds;
    const int x = w % kXcds, i = w / kXcds;
    const int lin = x * per + min(x, extra) + i;              // a bijection of [0, n)
    qb = lin % n_qb;
    kvh = (lin / n_qb) % a.n_kv_heads;
    b = lin / (n_qb * a.n_kv_heads);
  } else {
    // Causal layers: longest rows first, and each (sequence, KV head) on a
    // fixed set of XCDs (a head per XCD and several in turn, or one head over
    // 8 / H XCDs taking its query blocks in turn), so the workgroups an XCD
    // runs together stream the same head's key/value tiles through its L2.
    // Shapes where that is no bijection keep the plain longest-first order.
    const int H = a.n_kv_heads * static_cast<int>(gridDim.z);
    const int w = static_cast<int>(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    const int x = w % kXcds, i = w / kXcds;
    int hh = -1, rank = 0;   // (sequence, KV head) and query block rank from the longest
    if (H % kXcds == 0) {
      const int hp = H / kXcds;
      hh = x + kXcds * (i % hp);
      rank = i / hp;
    } else if (kXcds % H == 0 && n_qb % (kXcds / H) == 0) {
      const int k = kXcds / H;
      hh = x % H;
      rank = i * k + x / H;
    }
    if (hh >= 0) {
      qb = n_qb - 1 - rank;
      kvh = hh % a.n_kv_heads;
      b = hh / a.n_kv_heads;
    } else {
      qb = n_qb - 1 - static_cast<int>(blockIdx.x);
      kvh = blockIdx.y;
      b = blockIdx.z;
    }
  }
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, h = lane >> 5;                     // row of this lane, half of the slice
  // Query rows are positions q_pos0 .. q_pos0 + seq_len - 1 (q_pos0 > 0: a
  // later chunk of a prompt whose earlier keys are in the workspace rows too).
  // Row block rb of the wave holds its rows 32 rb .. 32 rb + 31; row r of
  // the wave is query head r % G at position p0 + wave PW + r / G.  32 is a
  // multiple of G, so the lane's rows in all blocks share one head.
  const int p0 = a.q_pos0 + qb * C::QB;
  const int qh = kvh * G + (m % G);                           // query head of row m
  int pos[C::kRB], lpos[C::kRB];                              // query position of row m, its row in q and out
  bool row_valid[C::kRB];
#pragma unroll
  for (int rb = 0; rb < C::kRB; ++rb) {
    pos[rb] = p0 + wave * C::PW + (C::kRows * rb + m) / G;
    lpos[rb] = pos[rb] - a.q_pos0;
    row_valid[rb] = lpos[rb] < a.seq_len;
  }

  // ---- tile stream setup (the first kStages - 1 copies start in the prologue) -----
  const int p_last = min(p0 + C::QB, a.q_pos0 + a.seq_len) - 1;
  const int kt_lo = a.window > 0 ? max(0, p0 - a.window + 1) / C::KT : 0;
  const int kt_hi = p_last / C::KT + 1;
  const int64_t head = static_cast<int64_t>(b) * a.n_kv_heads + kvh;
  const char* kbase = static_cast<const char*>(a.ws_k) + head * a.seq_pad * C::kKRowBytes;
  // Value rows: the workspace's (K=V layers, and separate-V layers whose
  // rows of one head span 2^31 bytes or more), or v itself, token-major, rows
  // Hkv d apart (the other separate-V layers).  Rows past the sequence read
  // zeros (the buffer's range check; see copy_load).
  const char* vbase;
  uint32_t vspan, vstride;
  if (C::kShared || a.v == nullptr) {
    vbase = static_cast<const char*>(a.ws_v) + head * a.seq_pad * C::kVRowBytes;
    vspan = static_cast<uint32_t>(a.seq_pad) * C::kVRowBytes;
    vstride = C::kVRowBytes;
  } else {
    vstride = static_cast<uint32_t>(a.n_kv_heads) * C::kVRowBytes;
    vbase = static_cast<const char*>(a.v) + (static_cast<int64_t>(b) * a.seq_len * a.n_kv_heads + kvh) * C::kVRowBytes;
    vspan = static_cast<uint32_t>(a.seq_len - 1) * vstride + C::kVRowBytes;
  }
  const uint32_t kspan = static_cast<uint32_t>(a.seq_pad) * C::kKRowBytes;   // < 2^31 (host check)
  const BufRsrc rk = make_rsrc(kbase, kspan);
  const BufRsrc rv = make_rsrc(vbase, vspan);
  // ---- prologue: QKNorm + rotation of query row m (this lane's half) ---------
  // bf16: the query fragments stay in registers.  fp32 would need 256
  // registers for them, so the fp32 build rebuilds each fragment from the raw
  // query when it is used (a slow path that exists for exact tests).
  constexpr bool kQRegs = sizeof(T) == 2;
  constexpr int kRB = C::kRB;
  lds_char* const tab = (lds_char*)smem + C::kTabOff + wave * C::PW * C::kTabRow;   // this wave's table rows
  static_assert(kQRegs || kRB == 1, "the fp32 build keeps one row block");
  Frag8<T> qf[kRB][kQRegs ? C::kQSteps : 1];
  const T* __restrict__ qrow[kRB];
  const f32x2* __restrict__ qtable[kRB];
  const T* __restrict__ gq = static_cast<const T*>(a.q_gain);
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    qrow[rb] = static_cast<const T*>(a.q) +
               ((static_cast<int64_t>(b) * a.seq_len + (row_valid[rb] ? lpos[rb] : 0)) * a.n_q_heads + qh) * D;
    qtable[rb] = static_cast<const f32x2*>(a.rope_table) + static_cast<int64_t>(row_valid[rb] ? pos[rb] : 0) * a.n_rot;
  }
  float rs[kRB];
  // Largest squared key length over the tiles this workgroup reads.
  const int n_kt = kt_hi - kt_lo;
  const float* __restrict__ kn_tiles = a.ws_kn + head * (a.seq_pad / C::KT) + kt_lo;
  float kn2 = 0.f;
  {
    float ss[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) ss[rb] = 0.f;
    if constexpr (kQRegs) {
      // The query loads go out before the first tiles' copies: loads
      // complete in order, so waiting for the queries does not wait for the
      // copies.
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int u = 0; u < C::kQSteps; ++u) load_frag(qf[rb][u], qrow[rb] + 16 * u + 8 * h);
      if constexpr (C::kTabLds) {
        // rows p0 + wave PW .. + PW - 1, two per instruction; chunk c (pairs
        // 4c .. 4c + 3) of row r lands in slot c ^ (r & 15) so the lanes'
        // reads below spread over the banks.  With n_rot < d / 2 the chunks
        // past n_rot hold the next row's pairs and are not used; rows past
        // the table read zeros.  At most 4M positions of 128 pairs: the byte
        // offsets stay below 2^32.
        const uint32_t row_bytes = static_cast<uint32_t>(a.n_rot) * 4;
        const BufRsrc rt = make_rsrc(a.rope_table16, static_cast<uint32_t>(a.table_rows) * row_bytes);
        constexpr int kSlots = C::kTabRow / 16;
#pragma unroll
        for (int i = 0; i < C::PW / 2; ++i) {
          const int r = 2 * i + lane / kSlots, slot = lane % kSlots;
          const uint32_t pos_r = static_cast<uint32_t>(p0 + wave * C::PW + r);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, tab + i * 1024, 16,
                                                   pos_r * row_bytes + ((slot ^ (r & 15)) << 4), 0, 0, 0);
        }
      }
      // the key-length maxima of the first 64 tiles (the rest after the copies)
      kn2 = lane < n_kt ? kn_tiles[lane] : 0.f;
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < C::kStages - 1; ++i)
        issue_tile<C>(rk, rv, vstride, kt_lo + i, (lds_char*)smem + i * C::kStageBytes, wave, lane);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int u = 0; u < C::kQSteps; ++u) ss[rb] = sum_squares(qf[rb][u], ss[rb]);
    } else {
#pragma unroll
      for (int i = 0; i < C::kStages - 1; ++i)
        issue_tile<C>(rk, rv, vstride, kt_lo + i, (lds_char*)smem + i * C::kStageBytes, wave, lane);
#pragma unroll
      for (int u = 0; u < C::kQSteps; ++u) {
        Frag8<T> f;
        load_frag(f, qrow[0] + 16 * u + 8 * h);
#pragma unroll
        for (int j = 0; j < 8; ++j) ss[0] += to_f32(f.v[j]) * to_f32(f.v[j]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      ss[rb] = sum_halves(ss[rb]);
      rs[rb] = row_valid[rb] ? (1.0f / sqrtf(ss[rb] / D + a.eps)) * a.qk_scale_log2 : 0.f;
    }
  }
  QSource<T, D> qs[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) qs[rb] = QSource<T, D>{qf[rb], qrow[rb], gq, qtable[rb], rs[rb], a.n_rot};
  if constexpr (C::kTabLds) {
    // the table rows have landed once at most the first tiles' copies (issued
    // after them) are in flight; each wave reads only the rows it copied
    wait_vm_le<(C::kStages - 1) * C::kDmaPerWave>();
  }
  if constexpr (kQRegs) {
    // Gain and rotation of the register fragments.  The gains and (cos, sin)
    // pairs of kBatch steps are all loaded before any is used, so their round
    // trips overlap instead of queuing one after another behind the tile
    // copies in flight.  Pair p of the row sits at table[p]; reads for
    // p >= n_rot fall on later rows or the key rows after the table, inside
    // the workspace, and are not used.
    constexpr int kBatch = 4;
    constexpr int kRotSteps = SHARED ? 8 : C::kQSteps;   // K=V layers rotate pairs 0..63, dims 0..127
#pragma unroll
    for (int u0 = 0; u0 < C::kQSteps; u0 += kBatch) {
      Frag8<T> g[kBatch];
      f32x2 cs[kRB][kBatch][4];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) load_frag(g[i], gq + 16 * (u0 + i) + 8 * h);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (u0 + i < kRotSteps) {
            if constexpr (C::kTabLds) {
              // row r of the wave's block: pairs 8u + 4h .. +3 are chunk 2u + h
              const int r = C::kRows * rb / G + m / G;
              typedef _Float16 h8 __attribute__((ext_vector_type(8)));
              const h8 v = *(const __attribute__((address_space(3))) h8*)(
                  tab + r * C::kTabRow + (((2 * (u0 + i) + h) ^ (r & 15)) << 4));
#pragma unroll
              for (int j = 0; j < 4; ++j)
                cs[rb][i][j] = f32x2{static_cast<float>(v[2 * j]), static_cast<float>(v[2 * j + 1])};
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) cs[rb][i][j] = qtable[rb][8 * (u0 + i) + 4 * h + j];
            }
          }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int u = u0 + i;
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = to_f32(qf[rb][u].v[j]) * rs[rb] * to_f32(g[i].v[j]);
          if (u < kRotSteps) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float r0 = x[2 * j], r1 = x[2 * j + 1];
              rotate_pair(r0, r1, cs[rb][i][j]);
              const bool on = 8 * u + 4 * h + j < a.n_rot;
              x[2 * j] = on ? r0 : x[2 * j];
              x[2 * j + 1] = on ? r1 : x[2 * j + 1];
            }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) frag_set(qf[rb][u], j, x[j]);
        }
    }
  }

  // ---- lane operand offsets within a stage --------------------------------------
  LaneOffsets lo;
  {
    const int cl = h * C::kSz / 2;                      // lane part of the key chunk (16u + 8h) * size / 16
    lo.kq = m * C::kKRowBytes + ((cl ^ row_swizzle(m)) << 4);
    lo.vq = C::kKBytes + m * C::kVRowBytes + ((cl ^ row_swizzle(m)) << 4);
    const int g = lane >> 4, p = lane & 15;
    const int x = 2 * (g & 1) + ((p & 3) >> 1);         // lane part of the value chunk
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int r = 4 * (g >> 1) + (p >> 2) + 8 * s;
      lo.vt[s] = r * C::kVRowBytes + ((x ^ row_swizzle(r)) << 4) + 8 * (p & 1);
    }
  }

  RowState<C::kDBlocks> st[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
    for (int t = 0; t < C::kDBlocks; ++t) st[rb].o[t] = f32x16{};
    st[rb].m_run = -INFINITY;
    st[rb].l_part = 0.f;
  }
  lds_char* const lds = (lds_char*)smem;

  // Edge tiles take the masked step: tiles [kt_lo, lo_end) reach below some
  // row's window (key0 <= p0 + QB - 1 - W), tiles [hi_begin, kt_hi) above
  // some row's position (key0 + KT - 1 > p0).  The tiles between are inside
  // every row's range and skip the mask.  One loop per kind keeps a single
  // copy of each step in the code.
  const int lo_end = a.window > 0 ? min(kt_hi, max(kt_lo, (p0 + C::QB - 1 - a.window) / C::KT + 1)) : kt_lo;
  const int hi_begin = max(lo_end, min(kt_hi, (p0 + 1) / C::KT));
  auto stage_of = [&](int t) { return lds + (static_cast<unsigned>(t - kt_lo) % C::kStages) * C::kStageBytes; };

  // Scores within +-kScoreBound for all of the wave's rows: no running max.
  bool fixed = false;
  if constexpr (kQRegs && C::kStages >= 3) {
    for (int i = lane + kWave; i < n_kt; i += kWave) kn2 = fmaxf(kn2, kn_tiles[i]);
#pragma unroll
    for (int x = 1; x < kWave; x <<= 1) kn2 = fmaxf(kn2, wave_xor(kn2, x));
    float qn2 = 0.f;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float q2 = 0.f;
#pragma unroll
      for (int u = 0; u < C::kQSteps; ++u) q2 = sum_squares(qf[rb][u], q2);
      qn2 = fmaxf(qn2, sum_halves(q2));
    }
    // Rows that see fewer than 64 keys keep the online max: with P = 2^S
    // every weight is rounded to bf16, where the max-subtracted weight of a
    // row's largest score is exactly 1, and on rows of a few keys that
    // difference shows in the outputs (on longer rows the roundings average
    // out).
    const bool long_rows = p0 + wave * C::PW >= 63 && (a.window == 0 || a.window >= 64);
    fixed = long_rows && __builtin_amdgcn_readfirstlane(static_cast<int>(score_bound_ok(qn2, kn2))) != 0;
  }

  if constexpr (C::kStages >= 3) {
   auto pipeline = [&](auto fx) {
    constexpr bool FX = decltype(fx)::value;
    // Pipelined: step i runs the softmax and PV of tile i and the QK^T of
    // tile i + 1.  It reads the keys of tile i + 1 and the values of tile i,
    // and copies tile i + kStages - 1 into the stage of tile i - 1, which
    // every wave has left once it passes the step's barrier.
    f32x16 s[kRB];
    {
      wait_tiles<C>(C::kStages - 2);   // tile kt_lo landed; the next kStages - 2 may be in flight
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      Frag8<T> kf[C::kKAhead];
      qk_prefetch<C, T, D>(kf, stage_of(kt_lo), lo);
      qk_run<C, T, D, 0>(s, kf, stage_of(kt_lo), lo, qs, h, [](int) {}, [](int) {});
    }
    auto step = [&](int kt, auto masked, const f32x16 (&s_in)[kRB], f32x16 (&s_out)[kRB]) {
      // tile kt + 1 landed (one later tile may be in flight) and is visible
      // to all waves; all waves are past step kt - 1.  A bare barrier: the
      // wait above already covers the copies.
      wait_tiles<C>(C::kStages - 3);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // copies of tiles past the workgroup's last one read nothing (an empty range)
      const bool live = kt + C::kStages - 1 < kt_hi;
      pipe_step<C, T, D, decltype(masked)::value, true, FX>(
          stage_of(kt + 1), stage_of(kt), stage_of(kt + C::kStages - 1), kbase, vbase, live ? kspan : 0u,
          live ? vspan : 0u, vstride, kt + C::kStages - 1, wave, lane, lo, qs, kt * C::KT, pos, a.window, st, s_in,
          s_out);
    };
    const int last = kt_hi - 1;
    const int m1 = min(lo_end, last), m2 = max(m1, min(hi_begin, last));
    int kt = kt_lo;
#pragma nounroll
    for (int phase = 0; phase < 2; ++phase) {
      const int masked_end = phase == 0 ? m1 : last;
      for (; kt < masked_end; ++kt) step(kt, std::true_type{}, s, s);
      if (phase == 0) {
        for (; kt < m2; ++kt) step(kt, std::false_type{}, s, s);
      }
    }
    // The last tile (always an edge): its values landed with its keys, and
    // nothing is copied, so neither a wait nor a barrier.
    pipe_step<C, T, D, true, false, FX>(stage_of(last + 1), stage_of(last), stage_of(last + C::kStages - 1), kbase,
                                        vbase, kspan, vspan, vstride, 0, wave, lane, lo, qs, last * C::KT, pos, a.window,
                                        st, s, s);
   };
    if (fixed) pipeline(std::true_type{});
    else pipeline(std::false_type{});
  } else {
    // One tile per step: wait for it, barrier, then the (masked or plain) step.
    auto run_tile = [&](int kt, auto masked) {
      // tile kt has landed once at most the later tiles' copies are in flight
      // (every step copies one tile, kStages - 1 ahead)
      wait_tiles<C>(C::kStages - 2);
      // Tile kt visible to all waves; all waves are past tile kt - 1 (whose
      // reads all fed MFMAs, so they have returned).
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      tile_step<C, T, D, decltype(masked)::value>(stage_of(kt), stage_of(kt + C::kStages - 1), kbase, vbase, kspan,
                                                  vspan, vstride, kt + C::kStages - 1, wave, lane, lo, qs, kt * C::KT, pos,
                                                  a.window, st);
      if (C::kStages == 1 && kt + 1 < kt_hi) {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_tile<C>(rk, rv, vstride, kt + 1, lds, wave, lane);
      }
    };
    int kt = kt_lo;
#pragma nounroll
    for (int phase = 0; phase < 2; ++phase) {
      const int masked_end = phase == 0 ? lo_end : kt_hi;
      for (; kt < masked_end; ++kt) run_tile(kt, std::true_type{});
      if (phase == 0)
        for (; kt < hi_begin; ++kt) run_tile(kt, std::false_type{});
    }
  }

  // ---- epilogue: register r of block t is dim 32t + 8(r/4) + 4h + r%4 of row m -------
  wait_vm_le<0>();   // copies of tiles past the last one have landed before the workgroup ends
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // last PV MFMA retired
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float inv = 1.0f / sum_halves(st[rb].l_part);
    T* __restrict__ out = static_cast<T*>(a.out) +
        ((static_cast<int64_t>(b) * a.seq_len + (row_valid[rb] ? lpos[rb] : 0)) * a.n_q_heads + qh) * D;
    if constexpr (sizeof(T) == 2) {
      // Lanes m and m + 32 hold the two 4-dim halves of each 8-dim run of row
      // m.  One row swap per pair of runs hands each lane a whole run (lane m
      // the even run, lane m + 32 the odd one), so every store is 16 bytes.
#pragma unroll
      for (int t = 0; t < C::kDBlocks; ++t) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t lo[2], hi[2];   // runs 2j (registers 8j..8j+3) and 2j+1 (8j+4..8j+7)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            lo[e] = pack_bf16x2(read_acc(st[rb].o[t][8 * j + 2 * e]) * inv,
                                read_acc(st[rb].o[t][8 * j + 2 * e + 1]) * inv);
            hi[e] = pack_bf16x2(read_acc(st[rb].o[t][8 * j + 4 + 2 * e]) * inv,
                                read_acc(st[rb].o[t][8 * j + 4 + 2 * e + 1]) * inv);
            const auto r = __builtin_amdgcn_permlane32_swap(lo[e], hi[e], false, false);
            lo[e] = r[0];
            hi[e] = r[1];
          }
          if (row_valid[rb])
            *reinterpret_cast<uint4*>(out + 32 * t + 16 * j + 8 * h) = uint4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
    } else {
      // fp32: each 4-dim half is 16 bytes already
      if (row_valid[rb]) {
#pragma unroll
        for (int t = 0; t < C::kDBlocks; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float4 v;
            v.x = read_acc(st[rb].o[t][4 * q]) * inv;
            v.y = read_acc(st[rb].o[t][4 * q + 1]) * inv;
            v.z = read_acc(st[rb].o[t][4 * q + 2]) * inv;
            v.w = read_acc(st[rb].o[t][4 * q + 3]) * inv;
            *reinterpret_cast<float4*>(out + 32 * t + 8 * q + 4 * h) = v;
          }
      }
    }
  }
}

template <typename T, int D, int G, bool SHARED>
static hipError_t launch_one(const PrefillArgs& a, int batch, hipStream_t s) {
  using C = PrefillCfg<T, D, G, SHARED>;
  const int n_qb = (a.seq_len + C::QB - 1) / C::QB;
  hipLaunchKernelGGL((prefill_attn_kernel<T, D, G, SHARED>), dim3(n_qb, a.n_kv_heads, batch), dim3(C::kWaves * 64),
                     0, s, a);
  return hipGetLastError();
}

template <typename T, int D, bool SHARED>
static hipError_t launch_d(const PrefillArgs& a, int group, int batch, hipStream_t s) {
  switch (group) {
    case 1: return launch_one<T, D, 1, SHARED>(a, batch, s);
    case 2: return launch_one<T, D, 2, SHARED>(a, batch, s);
    case 4: return launch_one<T, D, 4, SHARED>(a, batch, s);
    case 8: return launch_one<T, D, 8, SHARED>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
static hipError_t launch_s(const PrefillArgs& a, int group, int kv_shared, int batch, hipStream_t s) {
  return kv_shared ? launch_d<T, D, true>(a, group, batch, s) : launch_d<T, D, false>(a, group, batch, s);
}

hipError_t launch_prefill_attn(const PrefillArgs& a, int dtype, int head_dim, int group, int kv_shared,
                               int batch, hipStream_t s) {
  if (dtype == 0 && head_dim == 512) return launch_s<bf16, 512>(a, group, kv_shared, batch, s);
  if (dtype == 0 && head_dim == 256) return launch_s<bf16, 256>(a, group, kv_shared, batch, s);
  if (dtype == 1 && head_dim == 512) return launch_s<float, 512>(a, group, kv_shared, batch, s);
  if (dtype == 1 && head_dim == 256) return launch_s<float, 256>(a, group, kv_shared, batch, s);
  return hipErrorInvalidValue;
}

}  // namespace ga
