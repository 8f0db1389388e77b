// Split-K decode attention over the packed cache (MFMA path).
//
// One work-group of four waves owns one (sequence, kv head, context chunk)
// and all query rows of that kv group: up to 16 rows = query tokens x query
// heads, so grouped query heads (and the verify step's query tokens) share
// every K/V byte loaded.  Waves take 32-token tiles of the chunk in turn.
//
// Memory: each wave streams its tiles through a ring of LDS slots with
// direct global->LDS loads (16 bytes per lane), up to two tiles ahead of the
// one it is working on, so every CU keeps ~100 KB of K/V in flight without
// holding it in registers.  Chunks are XOR-swizzled on their way into LDS so
// the 8-byte operand reads below spread over the banks.
//
//   QK^T   v_mfma_i32_16x16x32_i8, one MFMA per 32-block and 16 tokens, so
//          each block keeps its own int32 dot sum (page 1: int8 K and Q go
//          straight into the integer dot); the sums are rescaled in fp32 by
//          d_q * d_k and summed over blocks, in the log2 domain.
//   softmax running maximum per row, updated once per tile; the
//          accumulators are rescaled only when it grows.
//   P.V    v_mfma_f32_16x16x32_f16.  V tiles are stored token-interleaved
//          (32 tokens per tile, "BitLLM" page 3: the layout follows the
//          reduction axis, which is T for S.V), so one 8-byte read per lane is
//          8 tokens of one nibble pair = one MFMA B operand.  Nibbles become
//          exact fp16 integers (n - 8) with a byte permute and one packed f16
//          add; A = p * d_v is split into fp16 hi + lo so the weights keep
//          about 22 bits.
//
// The four waves merge through LDS and the group writes one unnormalized
// partial (m, l, o) per row.  The last group to finish a (sequence, kv head)
// -- counted with a device-scope atomic in the workspace -- merges all of
// its partials and writes the output rows, then resets the counter.

#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_qk.h"

namespace kvq {

constexpr int kWaves = 4;

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

struct AttnParams {
  const uint32_t* k_qs;
  const uint16_t* k_d;
  const uint8_t* v_qs;
  const uint16_t* v_d;
  const float* q;
  float* out;
  float* part_o;          // [n_seq][n_kv][n_split][rows][D]
  float* part_ml;         // [n_seq][n_kv][n_split][rows][2]
  unsigned* counters;     // [n_seq][n_kv]
  const int32_t* seg_table;
  const int32_t* seq_len;
  int n_kv_heads;
  int n_q_heads;
  int n_qtok;
  int group;
  int rows;               // n_qtok * group, at most 16
  int seg_tokens;
  int max_segs;
  int chunk;              // tokens per work-group, a multiple of kWaves * kTile
  int n_split;
  int causal;
  float scale_log2;       // sm_scale * log2(e)
};

// Geometry of one LDS ring slot for head_dim D and V format VF.
template <int D, int VF>
struct Slot {
  static constexpr int NB = D / kBlock;
  static constexpr int VROW = VF == 0 ? D / 2 : D;   // V payload bytes per token
  static constexpr int KBYTES = kTile * D;           // K codes of the tile
  static constexpr int VBYTES = kTile * VROW;        // V payload of the tile
  static constexpr int SBYTES = kTile * NB * 2;      // one scale plane of the tile
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = KBYTES;
  static constexpr int DK_OFF = KBYTES + VBYTES;
  static constexpr int DV_OFF = DK_OFF + SBYTES;
  static constexpr int BYTES = DV_OFF + SBYTES;
  static constexpr int CPR = D / 16;                 // 16-byte chunks per K row
  static constexpr int PBYTES = kRows * (kTile + 4) * 4;   // padded P staging tile
  static constexpr bool P_IN_K = PBYTES <= KBYTES;   // P can reuse the K area
  // three slots per wave where two groups of four waves still fit in a CU
  static constexpr int NSLOT = (3 * BYTES * kWaves <= 81920) ? 3 : 2;
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "whole 1 KB load steps");
};

// Direct global->LDS loads (lane l's bytes land at lds + size * l for the
// 16- and 4-byte forms used here; the sub-dword forms keep a 4-byte lane
// stride, so they are not used) issued
// from inline assembly: the compiler cannot tell which LDS bytes such a load
// writes and would wait for all of them before every LDS read, which undoes
// the ring.  The kernel counts these loads itself with vmcnt.  The address
// is a uniform base plus a per-lane 32-bit offset.
template <int SIZE>
__device__ __forceinline__ void dma(const void* sbase, uint32_t voff, uint32_t lds) {
  if constexpr (SIZE == 16) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 ::"v"(voff), "s"(sbase), "s"(lds) : "memory");
  } else if constexpr (SIZE == 4) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 ::"v"(voff), "s"(sbase), "s"(lds) : "memory");
  } else {
    static_assert(SIZE == 16 || SIZE == 4, "16 or 4 bytes per lane");
  }
}
// The same with a full per-lane 64-bit address.
__device__ __forceinline__ void dma16_v(const void* vaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(vaddr), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4_v(const void* vaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               ::"v"(vaddr), "s"(lds) : "memory");
}

// A uniform 32-bit load on the scalar path (waits only for itself).
__device__ __forceinline__ int load_uniform(const int32_t* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// Per-lane byte offsets of one tile's loads inside its global rows; the
// swizzle repeats every 1 KB, so every 1 KB step of a tile uses the same.
struct TileLane {
  uint32_t k, v, s;
};
template <int D, int VF>
__device__ __forceinline__ TileLane tile_lane_offsets(int lane) {
  using S = Slot<D, VF>;
  const int r = lane / S::CPR;
  const int q = (lane % S::CPR) ^ (r % S::CPR);
  const int R = lane >> 1;
  const int c = (lane & 1) ^ ((R >> 2) & 1);
  return {(uint32_t)(r * D + 16 * q), (uint32_t)(R * 32 + 16 * c), (uint32_t)(4 * (lane % (S::SBYTES / 4)))};
}

// Issue the loads of one tile (32 tokens starting at t0) into a ring slot.
// K rows (CPR chunks) land at chunk r*CPR + (q ^ (r % CPR)); V rows (two
// chunks) at R*2 + (c ^ ((R >> 2) & 1)); scales as they are.
template <int D, int VF>
__device__ __forceinline__ void issue_tile(const AttnParams& p, int seq, int kvh, int t0,
                                           uint32_t slot, const TileLane& tl) {
  using S = Slot<D, VF>;
  const int segj = __builtin_amdgcn_readfirstlane(t0 / p.seg_tokens);
  const int seg = p.seg_table ? load_uniform(p.seg_table + (seq * p.max_segs + segj))
                              : seq * p.max_segs + segj;
  const size_t row0 = ((size_t)seg * p.n_kv_heads + kvh) * p.seg_tokens + (t0 - segj * p.seg_tokens);
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k_qs) + row0 * D;
#pragma unroll
  for (int n = 0; n < S::KBYTES / 1024; ++n) dma<16>(kg + 1024 * n, tl.k, slot + S::K_OFF + 1024 * n);
  const uint8_t* vg = p.v_qs + row0 * S::VROW;
#pragma unroll
  for (int n = 0; n < S::VBYTES / 1024; ++n) dma<16>(vg + 1024 * n, tl.v, slot + S::V_OFF + 1024 * n);
  const uint8_t* kdg = reinterpret_cast<const uint8_t*>(p.k_d) + row0 * S::NB * 2;
  const uint8_t* vdg = reinterpret_cast<const uint8_t*>(p.v_d) + row0 * S::NB * 2;
  if constexpr (S::SBYTES == 256) {
    dma<4>(kdg, tl.s, slot + S::DK_OFF);
    dma<4>(vdg, tl.s, slot + S::DV_OFF);
  } else {
    // 128-byte planes: one load, lanes 0-31 K scales, lanes 32-63 V scales
    // (DV_OFF directly follows DK_OFF)
    static_assert(S::SBYTES == 128 && S::DV_OFF == S::DK_OFF + 128, "scale planes");
    dma4_v((__lane_id() < 32 ? kdg : vdg) + tl.s, slot + S::DK_OFF);
  }
}

// VMEM instructions issue_tile emits per tile.
template <int D, int VF>
constexpr int loads_per_tile() {
  return Slot<D, VF>::KBYTES / 1024 + Slot<D, VF>::VBYTES / 1024 + (Slot<D, VF>::SBYTES == 256 ? 2 : 1);
}

// Four bytes -> two fp16 pairs (1024 + byte) placed as [b0, b1] and [b2, b3].
__device__ __forceinline__ uint32_t bytes01_f16(uint32_t x) {
  return __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
}
__device__ __forceinline__ uint32_t bytes23_f16(uint32_t x) {
  return __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
}
__device__ __forceinline__ uint32_t sub_f16x2(uint32_t x, _Float16 c) {
  const v2h r = __builtin_bit_cast(v2h, x) - (v2h){c, c};
  return __builtin_bit_cast(uint32_t, r);
}
// 8 bytes (two words, byte k = token k) with values in [0, 255] -> 8 exact
// fp16 values byte - off.
__device__ __forceinline__ v8h bytes_to_f16x8(uint32_t w0, uint32_t w1, _Float16 off) {
  uint32_t r[4];
  r[0] = sub_f16x2(bytes01_f16(w0), off);
  r[1] = sub_f16x2(bytes23_f16(w0), off);
  r[2] = sub_f16x2(bytes01_f16(w1), off);
  r[3] = sub_f16x2(bytes23_f16(w1), off);
  return __builtin_bit_cast(v8h, r);
}

// p * d as an fp16 pair sum, for two tokens at once: hi = fp16(p*d),
// lo = fp16(p*d - hi), each from one fused multiply-add in fp32 with a single
// rounding (d is an fp16 pair, p two fp32 values); hi + lo keeps ~22 bits.
__device__ __forceinline__ void split_f16_pair(float p0, float p1, uint32_t dpair, uint32_t& hi,
                                               uint32_t& lo) {
  asm("v_fma_mixlo_f16 %0, %2, %4, 0 op_sel_hi:[0,1,0]\n\t"
      "v_fma_mixhi_f16 %0, %3, %4, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]\n\t"
      "v_fma_mixlo_f16 %1, %2, %4, -%0 op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixhi_f16 %1, %3, %4, -%0 op_sel:[0,1,1] op_sel_hi:[0,1,1]"
      : "=&v"(hi), "=&v"(lo)
      : "v"(p0), "v"(p1), "v"(dpair));
}

// Running state of one wave: output tiles (rows 4*(lane/16)+i, dims
// 16n + lane%16) and the per-row running maximum and sum of weights.
template <int D>
struct WaveState {
  v4f acc[D / 16];
  float mrow[4];
  float lrow[4];
};

// One 32-token tile from its LDS slot: scores, online softmax update, P.V.
// P is staged in the slot's K area when it fits, else in `pbuf`.
template <int D, int VF>
__device__ __forceinline__ void process_tile(uint8_t* slot, float* pbuf, int t0, int c1,
                                             const long (&qa)[D / kBlock],
                                             const float (&dqs)[4][D / kBlock], const int (&vis)[4],
                                             WaveState<D>& st) {
  using S = Slot<D, VF>;
  constexpr int NB = D / kBlock;
  constexpr int PSTRIDE = kTile + 4;   // padded row of the P staging tile (floats)
  const int lane = __lane_id();
  const int col = lane & 15, grp = lane >> 4;
  v4f(&acc)[D / 16] = st.acc;
  float(&mrow)[4] = st.mrow;
  float(&lrow)[4] = st.lrow;

  // ---- scores (log2 domain) of rows 4*grp+i, tokens t0 + 16*h + col
  float s[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 16 * h + col;
    long kb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int q = 2 * b + (grp >> 1);
      kb[b] = *reinterpret_cast<const long*>(slot + S::K_OFF + (r * S::CPR + (q ^ (r % S::CPR))) * 16 +
                                             8 * (grp & 1));
    }
    _Float16 dk[NB];
    if constexpr (NB == 4) {
      const uint2 w = *reinterpret_cast<const uint2*>(slot + S::DK_OFF + r * 8);
      dk[0] = __builtin_bit_cast(_Float16, (uint16_t)w.x);
      dk[1] = __builtin_bit_cast(_Float16, (uint16_t)(w.x >> 16));
      dk[2] = __builtin_bit_cast(_Float16, (uint16_t)w.y);
      dk[3] = __builtin_bit_cast(_Float16, (uint16_t)(w.y >> 16));
    } else {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(slot + S::DK_OFF + r * 4);
      dk[0] = __builtin_bit_cast(_Float16, (uint16_t)w);
      dk[1] = __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s[h][i] = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const v4i c = qk_block_mfma(qa[b], kb[b]);
      const float dkf = (float)dk[b];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[h][i] = fmaf((float)c[i], dqs[i][b] * dkf, s[h][i]);
    }
    const int t = t0 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[h][i] = t < vis[i] ? s[h][i] : -INFINITY;
  }

  // ---- online softmax: row maxima over the tile, rescale when they grow
  float mnew[4];
  bool grow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mnew[i] = fmaxf(mrow[i], max_row16(fmaxf(s[0][i], s[1][i])));
    grow |= mnew[i] > mrow[i];
  }
  if (__any(grow)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __builtin_amdgcn_exp2f(mrow[i] - mnew[i]);
      lrow[i] *= a;
#pragma unroll
      for (int n = 0; n < D / 16; ++n) acc[n][i] *= a;
      mrow[i] = mnew[i];
    }
  }
  // P goes through the slot's K area (every K read of this tile is done)
  float* sP = S::P_IN_K ? reinterpret_cast<float*>(slot + S::K_OFF) : pbuf;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(s[h][i] - mrow[i]);
      lrow[i] += e;
      sP[(4 * grp + i) * PSTRIDE + 16 * h + col] = e;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- A operands: row col, tokens 8*grp .. +8, times the V block scale
  float pr[8];
  {
    const float4 a0 = *reinterpret_cast<const float4*>(sP + col * PSTRIDE + 8 * grp);
    const float4 a1 = *reinterpret_cast<const float4*>(sP + col * PSTRIDE + 8 * grp + 4);
    pr[0] = a0.x; pr[1] = a0.y; pr[2] = a0.z; pr[3] = a0.w;
    pr[4] = a1.x; pr[5] = a1.y; pr[6] = a1.z; pr[7] = a1.w;
  }
  v8h dv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    dv[b] = *reinterpret_cast<const v8h*>(slot + S::DV_OFF + b * 64 + 16 * grp);
  if (t0 + kTile > c1) {
    // tokens past the chunk end may hold anything (even non-finite scales)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (t0 + 8 * grp + j >= c1) {
#pragma unroll
        for (int b = 0; b < NB; ++b) dv[b][j] = (_Float16)0.0f;
      }
  }

#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint32_t* dvw = reinterpret_cast<const uint32_t*>(&dv[b]);
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) split_f16_pair(pr[2 * k], pr[2 * k + 1], dvw[k], hw[k], lw[k]);
    const v8h ahi = __builtin_bit_cast(v8h, hw);
    const v8h alo = __builtin_bit_cast(v8h, lw);
    if constexpr (VF == 0) {
      // byte = nibble(dim 32b + col) | nibble(dim 32b + 16 + col) << 4, 8 tokens
      const int R = 16 * b + col;
      const uint2 w = *reinterpret_cast<const uint2*>(
          slot + S::V_OFF + (R * 2 + ((grp >> 1) ^ ((R >> 2) & 1))) * 16 + 8 * (grp & 1));
      const v8h blo = bytes_to_f16x8(w.x & 0x0F0F0F0Fu, w.y & 0x0F0F0F0Fu, (_Float16)1032.0f);
      const v8h bhi =
          bytes_to_f16x8((w.x >> 4) & 0x0F0F0F0Fu, (w.y >> 4) & 0x0F0F0F0Fu, (_Float16)1032.0f);
      acc[2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, blo, acc[2 * b], 0, 0, 0);
      acc[2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, blo, acc[2 * b], 0, 0, 0);
      acc[2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bhi, acc[2 * b + 1], 0, 0, 0);
      acc[2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bhi, acc[2 * b + 1], 0, 0, 0);
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int n = 2 * b + hh;
        const int R = 16 * n + col;
        const uint2 w = *reinterpret_cast<const uint2*>(
            slot + S::V_OFF + (R * 2 + ((grp >> 1) ^ ((R >> 2) & 1))) * 16 + 8 * (grp & 1));
        // int8 code c -> byte c ^ 0x80 = c + 128 -> fp16 (1024 + c + 128) - 1152
        const v8h bv = bytes_to_f16x8(w.x ^ 0x80808080u, w.y ^ 0x80808080u, (_Float16)1152.0f);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bv, acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bv, acc[n], 0, 0, 0);
      }
    }
  }
  // every LDS read of this slot is done before the slot is refilled
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Wait until at most `pending` tiles' loads of this wave are still in flight
// (vmcnt counts the wave's outstanding loads; each tile issues L of them).
template <int L>
__device__ __forceinline__ void wait_tiles(int pending) {
  if (pending >= 2) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * L) : "memory");
  } else if (pending == 1) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

template <int D, int VF>
__global__ __launch_bounds__(256) void k_attn_split(AttnParams p) {
  using S = Slot<D, VF>;
  constexpr int NB = D / kBlock;
  constexpr int NT = D / 16;
  constexpr int NSLOT = S::NSLOT;
  constexpr int LPT = loads_per_tile<D, VF>();
  constexpr int RING = kWaves * NSLOT * S::BYTES + (S::P_IN_K ? 0 : kWaves * S::PBYTES);
  constexpr int MERGE = kWaves * kRows * D * 4 + 2 * kWaves * kRows * 4;
  constexpr int LDS_BYTES = RING > MERGE ? RING : MERGE;
  static_assert(2 * kMaxSplits * kRows * 4 + 16 * (kRows * D / 4 > 256 ? kRows * D / 4 : 256) <=
                    LDS_BYTES, "split merge does not fit the LDS buffer");
  static_assert(kRows / kWaves * D * 4 + kRows * D + kRows * NB * 4 <= S::BYTES,
                "Q staging does not fit a slot");

  __shared__ __attribute__((aligned(16))) uint8_t s_lds[LDS_BYTES];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int L = p.seq_len[seq];
  const int n_split_seq = (L + p.chunk - 1) / p.chunk;
  if (split >= n_split_seq) return;               // nothing of this sequence here
  const int c0 = split * p.chunk;
  const int c1 = min(c0 + p.chunk, L);
  const int R = p.rows;
  const int G = p.group;

  uint8_t* ring = s_lds + wave * NSLOT * S::BYTES;
  const uint32_t ring_lds = lds_addr(ring);
  float* pbuf = reinterpret_cast<float*>(s_lds + kWaves * NSLOT * S::BYTES + wave * S::PBYTES);
  constexpr int kStride = kTile * kWaves;
  const int t_first = c0 + kTile * wave;
  const TileLane tl = tile_lane_offsets<D, VF>(lane);

  // Q: this wave's rows (wave, wave + 4, ...) go to its last slot as fp32,
  // ahead of the first tiles, so the wait for them leaves the tiles in flight.
  // Rows past R load row 0 and quantize as zeros.
  constexpr int QLANES = D / 4;   // 16-byte pieces per fp32 row
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    const int k = (64 * j + lane) / QLANES;
    const int r = wave + kWaves * k;
    const int rr = r < R ? r : 0;
    const float* src = p.q + (((size_t)seq * p.n_qtok + rr / G) * p.n_q_heads + kvh * G + rr % G) * D +
                       4 * ((64 * j + lane) % QLANES);
    dma16_v(src, ring_lds + (NSLOT - 1) * S::BYTES + 1024 * j);
  }
  // the first tiles go to slots 0 and 1 while Q is quantized
  const int n_pro = t_first >= c1 ? 0 : (NSLOT == 3 && t_first + kStride < c1 ? 2 : 1);
  if (n_pro >= 1) issue_tile<D, VF>(p, seq, kvh, t_first, ring_lds, tl);
  if (n_pro >= 2) issue_tile<D, VF>(p, seq, kvh, t_first + kStride, ring_lds + S::BYTES, tl);
  wait_tiles<LPT>(n_pro);

  // Q codes and scales are shared through wave 0's last slot, after its fp32
  // staging; that slot is only refilled once every wave has read them.
  const float* s_qf = reinterpret_cast<const float*>(ring + (NSLOT - 1) * S::BYTES);
  int8_t* s_qc = reinterpret_cast<int8_t*>(s_lds + (NSLOT - 1) * S::BYTES + kRows / kWaves * D * 4);
  float* s_qd = reinterpret_cast<float*>(s_lds + (NSLOT - 1) * S::BYTES + kRows / kWaves * D * 4 + kRows * D);
  float qv[kRows / kWaves][D / 64];
#pragma unroll
  for (int k = 0; k < kRows / kWaves; ++k)
#pragma unroll
    for (int e = 0; e < D / 64; ++e)
      qv[k][e] = wave + kWaves * k < R ? s_qf[k * D + 64 * e + lane] : 0.0f;
#pragma unroll
  for (int k = 0; k < kRows / kWaves; ++k) {
    const int r = wave + kWaves * k;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) quantize_q_lane(qv[k][e], 64 * e + lane, s_qc + r * D, s_qd + r * NB);
  }
  __syncthreads();
  long qa[NB];
  load_q_operands<D>(s_qc, qa);
  float dqs[4][NB];
  int vis[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * grp + i;
#pragma unroll
    for (int b = 0; b < NB; ++b) dqs[i][b] = s_qd[r * NB + b] * p.scale_log2;
    const int v = p.causal ? L - p.n_qtok + r / G + 1 : L;
    vis[i] = min(r < R ? v : 0, c1);
  }
  __syncthreads();
  if (NSLOT == 2 && t_first + kStride < c1)
    issue_tile<D, VF>(p, seq, kvh, t_first + kStride, ring_lds + S::BYTES, tl);

  WaveState<D> st;
#pragma unroll
  for (int n = 0; n < NT; ++n) st.acc[n] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.mrow[i] = -1e30f;
    st.lrow[i] = 0.0f;
  }

  int slot = 0;
  for (int t0 = t_first; t0 < c1; t0 += kStride) {
    int pending;
    if constexpr (NSLOT == 3) {
      // issue the tile after next into the slot freed last step, then wait
      // for this one (at most two younger tiles stay in flight)
      const bool more = t0 + 2 * kStride < c1;
      if (more) issue_tile<D, VF>(p, seq, kvh, t0 + 2 * kStride, ring_lds + ((slot + 2) % 3) * S::BYTES, tl);
      pending = more ? 2 : (t0 + kStride < c1 ? 1 : 0);
    } else {
      pending = t0 + kStride < c1 ? 1 : 0;
    }
    wait_tiles<LPT>(pending);
    process_tile<D, VF>(ring + slot * S::BYTES, pbuf, t0, c1, qa, dqs, vis, st);
    if constexpr (NSLOT == 2) {
      if (t0 + 2 * kStride < c1)
        issue_tile<D, VF>(p, seq, kvh, t0 + 2 * kStride, ring_lds + slot * S::BYTES, tl);
    }
    slot = (slot + 1 == NSLOT) ? 0 : slot + 1;
  }
  v4f(&acc)[NT] = st.acc;
  float(&mrow)[4] = st.mrow;
  float(&lrow)[4] = st.lrow;

  // ---- merge the four waves through LDS; one partial per work-group
  float* s_buf = reinterpret_cast<float*>(s_lds);
  float* s_m = s_buf + kWaves * kRows * D;
  float* s_l = s_m + kWaves * kRows;
#pragma unroll
  for (int i = 0; i < 4; ++i) lrow[i] = sum_row16(lrow[i]);
  __syncthreads();   // every wave is done with its ring
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_buf[(wave * kRows + 4 * grp + i) * D + 16 * n + col] = acc[n][i];
  if (col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s_m[wave * kRows + 4 * grp + i] = mrow[i];
      s_l[wave * kRows + 4 * grp + i] = lrow[i];
    }
  }
  __syncthreads();

  // Partials go out with agent-scope stores (write-through, coherent across
  // XCDs once complete), so publishing needs only a wait for the stores and
  // the counter increment, not a write-back of the whole L2.
  const size_t pbase = ((size_t)seq * p.n_kv_heads + kvh) * p.n_split;
  for (int e = tid; e < R * D; e += 256) {
    const int r = e / D;
    float M = s_m[r];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w * kRows + r]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float a = __builtin_amdgcn_exp2f(s_m[w * kRows + r] - M);
      o = fmaf(a, s_buf[(w * kRows + r) * D + (e - r * D)], o);
      l = fmaf(a, s_l[w * kRows + r], l);
    }
    __hip_atomic_store(&p.part_o[((pbase + split) * R) * D + e], o, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (e - r * D == 0) {
      __hip_atomic_store(&p.part_ml[((pbase + split) * R + r) * 2], M, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.part_ml[((pbase + split) * R + r) * 2 + 1], l, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const unsigned done = __hip_atomic_fetch_add(&p.counters[(size_t)seq * p.n_kv_heads + kvh], 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (done == (unsigned)(n_split_seq - 1));
  }
  __syncthreads();
  if (!s_last) return;
  // The last group of this (sequence, kv head): drop stale cached lines, then
  // merge the partials of every split.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  const int nsp = n_split_seq;
  float* sw = s_buf;                      // [nsp][R] split maxima, then weights
  float* sl = s_buf + nsp * R;            // [nsp][R] split sums
  float4* red = reinterpret_cast<float4*>(s_buf + 2 * kMaxSplits * kRows);
  for (int i = tid; i < nsp * R; i += 256) {
    const int sp = i / R, r = i - sp * R;
    const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + ((pbase + sp) * R + r) * 2);
    sw[i] = ml.x;
    sl[i] = ml.y;
  }
  __syncthreads();
  if (tid < R) {
    float M = -INFINITY;
    for (int sp = 0; sp < nsp; ++sp) M = fmaxf(M, sw[sp * R + tid]);
    float den = 0.0f;
    for (int sp = 0; sp < nsp; ++sp)
      den = fmaf(__builtin_amdgcn_exp2f(sw[sp * R + tid] - M), sl[sp * R + tid], den);
    s_m[tid] = M;
    s_l[tid] = 1.0f / den;
  }
  __syncthreads();
  for (int i = tid; i < nsp * R; i += 256) {
    const int r = i % R;
    sw[i] = __builtin_amdgcn_exp2f(sw[i] - s_m[r]) * s_l[r];
  }
  __syncthreads();

  // Outputs as float4 columns; 256 / cols threads share a column, each summing
  // every tpc-th split with eight loads in flight.
  const int cols = R * D / 4;
  const int tpc = cols >= 256 ? 1 : 256 / cols;
  for (int c = tid; c < cols * tpc; c += 256) {
    const int cc = c % cols, part = c / cols;
    const int r = (4 * cc) / D;
    const float* ob = p.part_o + (pbase * R) * D + 4 * cc;
    float4 a = {0.0f, 0.0f, 0.0f, 0.0f};
    int sp = part;
    for (; sp + 7 * tpc < nsp; sp += 8 * tpc) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const float4*>(ob + (size_t)(sp + u * tpc) * R * D);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = sw[(sp + u * tpc) * R + r];
        a.x = fmaf(w, v[u].x, a.x);
        a.y = fmaf(w, v[u].y, a.y);
        a.z = fmaf(w, v[u].z, a.z);
        a.w = fmaf(w, v[u].w, a.w);
      }
    }
    for (; sp < nsp; sp += tpc) {
      const float4 v = *reinterpret_cast<const float4*>(ob + (size_t)sp * R * D);
      const float w = sw[sp * R + r];
      a.x = fmaf(w, v.x, a.x);
      a.y = fmaf(w, v.y, a.y);
      a.z = fmaf(w, v.z, a.z);
      a.w = fmaf(w, v.w, a.w);
    }
    red[c] = a;
  }
  __syncthreads();
  for (int cc = tid; cc < cols; cc += 256) {
    float4 a = red[cc];
    for (int part = 1; part < tpc; ++part) {
      const float4 b = red[part * cols + cc];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    const int r = (4 * cc) / D;
    const int d = 4 * cc - r * D;
    const int j = r / G;
    const int h = kvh * G + r % G;
    *reinterpret_cast<float4*>(p.out + (((size_t)seq * p.n_qtok + j) * p.n_q_heads + h) * D + d) = a;
  }
  if (tid == 0)
    __hip_atomic_store(&p.counters[(size_t)seq * p.n_kv_heads + kvh], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

bool attn_supported(int head_dim, int v_format) {
  return (head_dim == 64 || head_dim == 128) && (v_format == 0 || v_format == 1);
}

int launch_attn(const kvq_cache& c, const float* q, float* out, int n_seq, int n_qtok, int n_q_heads,
                const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                const SplitPlan& plan, float sm_scale, int causal, void* workspace,
                hipStream_t stream) {
  AttnParams p;
  const WorkspaceLayout ws = workspace_layout(c, n_seq, n_qtok, n_q_heads, plan);
  char* base = static_cast<char*>(workspace);
  p.k_qs = c.k_qs;
  p.k_d = c.k_d;
  p.v_qs = c.v_qs;
  p.v_d = c.v_d;
  p.q = q;
  p.out = out;
  p.counters = reinterpret_cast<unsigned*>(base + ws.counters);
  p.part_o = reinterpret_cast<float*>(base + ws.part_o);
  p.part_ml = reinterpret_cast<float*>(base + ws.part_ml);
  p.seg_table = seg_table;
  p.seq_len = seq_len;
  p.n_kv_heads = c.n_kv_heads;
  p.n_q_heads = n_q_heads;
  p.n_qtok = n_qtok;
  p.group = n_q_heads / c.n_kv_heads;
  p.rows = n_qtok * p.group;
  p.seg_tokens = c.seg_tokens;
  p.max_segs = max_segs;
  p.chunk = plan.chunk;
  p.n_split = plan.n_split;
  p.causal = causal;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  const dim3 grid(plan.n_split, c.n_kv_heads, n_seq);
  if (c.head_dim == 128) {
    if (c.v_format == 0)
      hipLaunchKernelGGL((k_attn_split<128, 0>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((k_attn_split<128, 1>), grid, dim3(256), 0, stream, p);
  } else {
    if (c.v_format == 0)
      hipLaunchKernelGGL((k_attn_split<64, 0>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((k_attn_split<64, 1>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvq
