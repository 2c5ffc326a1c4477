// Flash-style causal prefill for one layer type, gfx950.
//
// A workgroup owns one KV head of one sequence and QB consecutive query
// positions: all G query heads of the group at those positions share every key
// tile it stages in LDS (the grouped-query sharing of "Gemma 4多模态大模型架构详解",
// section "分组查询注意力").  Its 128 query rows (QB positions x G heads) are
// split over four waves of 32 rows, one wave per SIMD.  Per key tile of 32
// positions each wave computes, over the full head dim:
//   S^T[key][row] = K~ Q~^T      32x32x16 bf16 MFMAs, A = key rows read from
//                                LDS, B = the wave's normalised, rotated queries
//                                held in registers
//   online softmax per row        in registers, exp2 domain (a lane holds 16
//                                of the 32 keys of its row, the lane 32 apart
//                                the rest)
//   O^T[d][row] += V^T P^T       32x32x16 MFMAs; V^T by transposing LDS reads of
//                                the value rows, P straight from the score
//                                registers
// Each wave keeps 32 rows x d fp32 accumulators (256 registers at d = 512, in
// the accumulation register file).
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
  static constexpr int kRows = 32;                  // query rows per wave
  static constexpr int PW = kRows / G;              // positions per wave
  static constexpr int QB = kWaves * PW;            // positions per workgroup
  static constexpr int kQSteps = D / 16;            // QK^T reduction steps
  static constexpr int kDBlocks = D / 32;           // 32-dim output blocks
  static constexpr int kSz = int(sizeof(T));
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
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kDmaK = kKBytes / 1024, kDmaV = kVBytes / 1024;
  static constexpr int kDmaPerWave = (kDmaK + kDmaV) / kWaves;
  static constexpr int kKAhead = 6;                 // key fragment reads in flight
  static constexpr int kVAhead = 4;                 // value fragments (two reads each) in flight
  static_assert(kLdsBytes <= kLdsCap, "LDS budget");
  static_assert((kDmaK + kDmaV) % kWaves == 0 && kKBytes % 1024 == 0, "tile copy split");
  static_assert(kKBytes % kVRowBytes == 0 && kStageBytes % kVRowBytes == 0, "row alignment for the swizzle");
  static_assert(kKRowBytes >= 256 && kVRowBytes >= 256, "row swizzle needs 16 chunks per row");
  static_assert(kStages <= 4 && (kStages - 2) * kDmaPerWave < 64, "copy counter range");
};

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
__device__ __forceinline__ float read_acc(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Scheduling pattern for a pipelined operand stream of N MFMAs, R LDS reads
// each, whose reads run A MFMAs ahead: the first A*R reads, then one MFMA and
// R reads alternately, then the last A MFMAs; NV global->LDS copies go one
// after every SV-th MFMA.  Keeps the reads in flight where the scheduler would
// otherwise trade prefetch depth for registers, and spreads the copies so the
// wave never queues many of them at once.
template <int A, int N, int R, int NV = 0, int SV = 1>
__device__ __forceinline__ void interleave_reads_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, A * R, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
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
  int rb;        // row bytes of that region
  int lds;       // LDS offset of the instruction within the stage
  int voff;      // byte offset within the tile's rows in global memory
};
template <typename C>
__device__ __forceinline__ CopyPiece copy_piece(int k, int wave, int lane) {
  CopyPiece cp;
  const int i = k * C::kWaves + wave;
  cp.is_k = i < C::kDmaK;
  const int j = cp.is_k ? i : i - C::kDmaK;                 // piece within its region
  cp.rb = cp.is_k ? C::kKRowBytes : C::kVRowBytes;          // uniform per (k, wave)
  int r, slot;
  if (cp.rb >= 1024) {
    r = j / (cp.rb / 1024);
    slot = (j % (cp.rb / 1024)) * 64 + lane;
  } else {
    r = j * (1024 / cp.rb) + lane / (cp.rb / 16);
    slot = lane % (cp.rb / 16);
  }
  cp.lds = i * 1024;
  cp.voff = r * cp.rb + ((slot ^ row_swizzle(r)) << 4);
  return cp;
}
template <typename C>
__device__ __forceinline__ void issue_tile(BufRsrc rk, BufRsrc rv, int tile, lds_char* dst, int wave, int lane) {
#pragma unroll
  for (int k = 0; k < C::kDmaPerWave; ++k) {
    const CopyPiece cp = copy_piece<C>(k, wave, lane);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(cp.is_k ? rk : rv, dst + cp.lds, 16, cp.voff, tile * C::KT * cp.rb, 0, 0);
  }
}

// QK^T A operand of step u: the 8 elements of key row l%32 at dims 16u + 8h ..,
// at stage `st`, from the lane's row offset `off` (lane part of the chunk
// already swizzled; the step part enters as an XOR).
template <typename V>
__device__ __forceinline__ V st_ld(const lds_char* st, int off) {
  return *(const __attribute__((address_space(3))) V*)(st + off);
}
__device__ __forceinline__ void key_frag(Frag8<bf16>& f, const lds_char* st, int off, int u) {
  f.v = st_ld<bf16x8>(st, off ^ ((2 * u) << 4));
}
__device__ __forceinline__ void key_frag(Frag8<float>& f, const lds_char* st, int off, int u) {
  const f32x4 a = st_ld<f32x4>(st, off ^ ((4 * u) << 4));
  const f32x4 b = st_ld<f32x4>(st, off ^ ((4 * u) << 4) ^ 16);
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
    const int off = (vt[s] ^ ((4 * t) << 4)) + c * 16 * C::kVRowBytes;
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

// One key tile: copy tile `next_tile` into `nxt` (spread over the QK^T steps), S^T,
// online softmax and O^T += V^T P^T from `cur`.  `cur` and `nxt` are distinct
// stages: with them as restrict pointers the compiler knows the copy does not
// feed this tile's reads (the kernel's own waits order the copies), and adds
// no waits for the copies before the LDS reads.
template <typename C, typename T, int D>
__device__ __forceinline__ void tile_step(const lds_char* __restrict__ cur, lds_char* __restrict__ nxt,
                                          const char* kbase, const char* vbase, uint32_t kspan, uint32_t vspan,
                                          int next_tile, int wave, int lane,
                                          const LaneOffsets& lo, const QSource<T, D>& qs, int key0, int pos, int w_first,
                                          int window, RowState<C::kDBlocks>& rs) {
  constexpr bool kQRegs = sizeof(T) == 2;
  const int h = lane >> 5;
  // Copies of tile next_tile into `nxt` go between the QK^T MFMAs, one per
  // kDmaStride steps.  Tiles past the sequence's padded end read zeros (the
  // buffer's range check); past this workgroup's last tile they are never used.
  const BufRsrc rk = make_rsrc(kbase, kspan), rv = make_rsrc(vbase, vspan);
  // The copy offsets are recomputed each tile (two VALU ops each) instead of
  // being kept live across the loop in registers the MFMA operands need.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  constexpr int kDmaStride = C::kQSteps / C::kDmaPerWave > 0 ? C::kQSteps / C::kDmaPerWave : 1;
  static_assert(C::kDmaPerWave <= C::kQSteps, "one copy per QK^T step at most");
  auto copy = [&](int k) {
    const CopyPiece cp = copy_piece<C>(k, wave, ln);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(cp.is_k ? rk : rv, nxt + cp.lds, 16, cp.voff, next_tile * C::KT * cp.rb,
                                             0, 0);
  };

  // S^T[key][row]: reads kKAhead fragments ahead of the MFMAs
  f32x16 s = f32x16{};
  {
    auto kfrag = [&](Frag8<T>& f, int u) { key_frag(f, cur, u < C::kKSteps ? lo.kq : lo.vq, u); };
    Frag8<T> kf[C::kKAhead];
#pragma unroll
    for (int u = 0; u < C::kKAhead; ++u) kfrag(kf[u], u);
#pragma unroll
    for (int u = 0; u < C::kQSteps; ++u) {
      const Frag8<T> k = kf[u % C::kKAhead];
      if (u + C::kKAhead < C::kQSteps) kfrag(kf[u % C::kKAhead], u + C::kKAhead);
      mma32(s, k, query_frag(qs, u, h));
      if (C::kStages > 1 && u % kDmaStride == 0 && u / kDmaStride < C::kDmaPerWave) copy(u / kDmaStride);
    }
    if constexpr (kQRegs) interleave_reads_mfma<C::kKAhead, C::kQSteps, 1, (C::kStages > 1 ? C::kDmaPerWave : 0), kDmaStride>();
  }

  // mask + online softmax: register r of this lane is key key0 + 8(r/4) + 4h + r%4
  // of query row m
  const bool need_mask = (key0 + C::KT - 1 > w_first) || (window > 0 && key0 <= w_first + C::PW - 1 - window);
  if (need_mask) {
    // visible keys: pos - W < key <= pos; with key = key0 + 4h + c_r,
    // c_r = 8(r/4) + r%4, that is diff - W < c_r <= diff
    const int diff = pos - key0 - 4 * h;
    const int low = window > 0 ? diff - window : -(1 << 30);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 8 * (r / 4) + (r % 4);
      s[r] = (c <= diff && c > low) ? s[r] : -INFINITY;
    }
  }
  float mt = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
  mt = max_halves(mt);
  constexpr float kTau = 8.0f;   // rescale only when the running max grows by > 2^8
  if (__any(mt > rs.m_run + kTau)) {
    const float m_new = fmaxf(rs.m_run, mt);
    if (rs.m_run != -INFINITY) {   // nothing accumulated yet otherwise
      const float alpha = __builtin_amdgcn_exp2f(rs.m_run - m_new);
#pragma unroll
      for (int t = 0; t < C::kDBlocks; ++t) scale_acc(rs.o[t], alpha);
      rs.l_part *= alpha;
    }
    rs.m_run = m_new;
  }
  const float m_use = (rs.m_run == -INFINITY) ? 0.f : rs.m_run;
  Frag8<T> pf[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = __builtin_amdgcn_exp2f(s[r] - m_use);
    rs.l_part += p;
    frag_set(pf[r / 8], r % 8, p);
  }

  // O^T += V^T P^T: step f = 2t + c pairs value block t, keys 16c .. with
  // score registers 8c .. 8c+7
  if constexpr (kQRegs) {
    Frag8<T> vf[C::kVAhead];
#pragma unroll
    for (int f = 0; f < C::kVAhead; ++f) value_frag<C>(vf[f], cur + C::kKBytes, lo.vt, f >> 1, f & 1);
#pragma unroll
    for (int f = 0; f < 2 * C::kDBlocks; ++f) {
      const Frag8<T> v = vf[f % C::kVAhead];
      if (f + C::kVAhead < 2 * C::kDBlocks)
        value_frag<C>(vf[f % C::kVAhead], cur + C::kKBytes, lo.vt, (f + C::kVAhead) >> 1, (f + C::kVAhead) & 1);
      mma32(rs.o[f >> 1], v, pf[f & 1]);
    }
    interleave_reads_mfma<C::kVAhead, 2 * C::kDBlocks, 2>();
  } else {
#pragma unroll
    for (int f = 0; f < 2 * C::kDBlocks; ++f) {
      Frag8<T> vf;
      value_frag_f32<C>(vf, cur, f >> 1, f & 1, lane);
      mma32(rs.o[f >> 1], vf, pf[f & 1]);
    }
  }
}

template <typename T, int D, int G, bool SHARED>
__global__ __launch_bounds__(256, 1) void prefill_attn_kernel(PrefillArgs a) {
  using C = PrefillCfg<T, D, G, SHARED>;
  __shared__ __attribute__((aligned(4096))) char smem[C::kLdsBytes];

  const int n_qb = (a.seq_len + C::QB - 1) / C::QB;
  const int qb = n_qb - 1 - static_cast<int>(blockIdx.x);   // longest causal rows first
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, h = lane >> 5;                     // row of this lane, half of the slice
  const int p0 = qb * C::QB;
  const int pos = p0 + wave * C::PW + m / G;                  // query position of row m
  const int qh = kvh * G + (m % G);                           // query head of row m
  const bool row_valid = pos < a.seq_len;

  // ---- tile stream setup: start the first kStages - 1 copies -------------------
  const int p_last = min(p0 + C::QB, a.seq_len) - 1;
  const int kt_lo = a.window > 0 ? max(0, p0 - a.window + 1) / C::KT : 0;
  const int kt_hi = p_last / C::KT + 1;
  const int64_t head = static_cast<int64_t>(b) * a.n_kv_heads + kvh;
  const char* kbase = static_cast<const char*>(a.ws_k) + head * a.seq_pad * C::kKRowBytes;
  const char* vbase = static_cast<const char*>(a.ws_v) + head * a.seq_pad * C::kVRowBytes;
  const uint32_t kspan = static_cast<uint32_t>(a.seq_pad) * C::kKRowBytes;   // < 2^31 (host check)
  const uint32_t vspan = static_cast<uint32_t>(a.seq_pad) * C::kVRowBytes;
  const BufRsrc rk = make_rsrc(kbase, kspan);
  const BufRsrc rv = make_rsrc(vbase, vspan);
#pragma unroll
  for (int i = 0; i < C::kStages - 1; ++i)
    issue_tile<C>(rk, rv, kt_lo + i, (lds_char*)smem + i * C::kStageBytes, wave, lane);

  // ---- prologue: QKNorm + rotation of query row m (this lane's half) ---------
  // bf16: the query fragments stay in registers.  fp32 would need 256
  // registers for them, so the fp32 build rebuilds each fragment from the raw
  // query when it is used (a slow path that exists for exact tests).
  constexpr bool kQRegs = sizeof(T) == 2;
  Frag8<T> qf[kQRegs ? C::kQSteps : 1];
  const T* __restrict__ qrow = static_cast<const T*>(a.q) +
      ((static_cast<int64_t>(b) * a.seq_len + (row_valid ? pos : 0)) * a.n_q_heads + qh) * D;
  const T* __restrict__ gq = static_cast<const T*>(a.q_gain);
  const f32x2* __restrict__ qtable = static_cast<const f32x2*>(a.rope_table) +
                                     static_cast<int64_t>(row_valid ? pos : 0) * a.n_rot;
  float rs;
  {
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < C::kQSteps; ++u) {
      Frag8<T> f;
      load_frag(f, qrow + 16 * u + 8 * h);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += to_f32(f.v[j]) * to_f32(f.v[j]);
      if constexpr (kQRegs) qf[u] = f;
    }
    ss = sum_halves(ss);
    rs = row_valid ? (1.0f / sqrtf(ss / D + a.eps)) * a.qk_scale_log2 : 0.f;
  }
  QSource<T, D> qs{qf, qrow, gq, qtable, rs, a.n_rot};
  if constexpr (kQRegs) {
#pragma unroll
    for (int u = 0; u < C::kQSteps; ++u) make_qfrag(qf[u], qs, u, h);
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
  const int w_first = p0 + wave * C::PW;            // this wave's first query position

  RowState<C::kDBlocks> st;
#pragma unroll
  for (int t = 0; t < C::kDBlocks; ++t) st.o[t] = f32x16{};
  st.m_run = -INFINITY;
  st.l_part = 0.f;
  lds_char* const lds = (lds_char*)smem;

  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int stage = (kt - kt_lo) % C::kStages;
    // tile kt has landed once at most the later tiles' copies are in flight
    // (every iteration copies one tile, kStages - 1 ahead)
    wait_tiles<C>(C::kStages - 2);
    // Tile kt visible to all waves; all waves are past tile kt - 1 (whose
    // reads all fed MFMAs, so they have returned).  A bare barrier: the
    // waits above already cover the copies.
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int nstage = (kt - kt_lo + C::kStages - 1) % C::kStages;
    tile_step<C, T, D>(lds + stage * C::kStageBytes, lds + nstage * C::kStageBytes, kbase, vbase, kspan,
                    vspan, kt + C::kStages - 1, wave, lane, lo, qs, kt * C::KT, pos, w_first, a.window, st);
    if (C::kStages == 1 && kt + 1 < kt_hi) {
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue_tile<C>(rk, rv, kt + 1, lds, wave, lane);
    }
  }

  // ---- epilogue: register r of block t is dim 32t + 8(r/4) + 4h + r%4 -------------
  wait_vm_le<0>();   // copies of tiles past the last one have landed before the workgroup ends
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // last PV MFMA retired
  const float l = sum_halves(st.l_part);
  if (!row_valid) return;
  const float inv = 1.0f / l;
  T* __restrict__ out = static_cast<T*>(a.out) +
      ((static_cast<int64_t>(b) * a.seq_len + pos) * a.n_q_heads + qh) * D + 4 * h;
#pragma unroll
  for (int t = 0; t < C::kDBlocks; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) out[32 * t + 8 * (r / 4) + (r % 4)] = from_f32<T>(read_acc(st.o[t][r]) * inv);
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
