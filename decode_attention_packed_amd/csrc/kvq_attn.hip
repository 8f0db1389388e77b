// Split-K decode attention over the packed cache (MFMA path).
//
// One work-group of eight waves (twelve in the w12 build below; one
// work-group per CU) owns one (sequence, kv head, context chunk) and all
// query rows of that kv group (query tokens x query heads, at most 16), so
// grouped query heads and the verify step's query tokens share every K/V
// byte loaded.  The chunk's 32-token tiles are dealt to the waves
// round-robin, so every run accumulates the same tiles in the same order.
//
// Memory: each wave streams its tiles through a ring of LDS slots with
// direct global->LDS loads (16 bytes per lane), up to two tiles ahead of the
// one it is working on, so a CU keeps 100-160 KB of K/V in flight without
// holding it in registers.  K rows are XOR-swizzled on their way into LDS so
// the 8-byte operand reads spread over the banks.
//
// Two tile bodies share that machinery.
//
// Column layout (rows x blocks <= 16: single-token decode with up to 4
// grouped heads at head_dim 128, 8 at 64).  The 16 MFMA columns are the
// (query row, quant block) pairs.
//   QK^T   v_mfma_i32_16x16x32_i8 with A = K rows (16 tokens) and B = the Q
//          codes of block b placed only in the columns of block b, so one
//          accumulator collects every block's int32 dot in its own column
//          (page 1: int8 K and Q go straight into the integer dot).  Each
//          column scales its dots by d_q * d_k and a DPP butterfly over the
//          block columns of a row adds them up: every lane then holds the
//          scores of 8 consecutive tokens of one row, with no padding rows.
//   softmax the row's reference (up to kRefHead above its running
//          maximum) is checked lane by lane; the cross-lane reduction and
//          the rescale of the accumulators only run when a score passes it.
//   P.V    computed transposed, v_mfma_f32_16x16x32_f16 with A = 16 dims of
//          V codes (exact fp16 integers from a byte permute and one packed
//          f16 add) and B = p * d_v of the column's block rounded to fp16
//          (fp32 accumulation).  V tiles are stored token-interleaved
//          ("BitLLM" page 3: the layout follows the reduction axis, T for
//          S.V), so one 8-byte read is 8 tokens of one dim.
//
// Row layout (larger groups, e.g. 4 query tokens x 4 heads): the 16 MFMA
// columns are query rows; the per-block dots come from one MFMA per block
// (S^T = K Q^T, the tile's tokens dealt to the MFMA rows so that each lane
// receives its row's weights in the order the P.V operand takes them), and
// P.V runs transposed as in the column layout, P straight from registers.
//
// The waves merge through LDS and the work-group writes one unnormalized
// partial (m, l, o) per row.  Column layout: the last work-group to finish a
// (sequence, kv head) -- counted with a device-scope atomic in the workspace
// -- merges all of its partials and writes the output rows, then resets the
// counter.  Row layout: a second launch (k_split_merge) merges them.

#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_qk.h"

#include <type_traits>

// This file is compiled three times.  The plain build (8 waves per
// work-group) serves every call.  KVQ_NS names the namespace of the other two:
//  - kvq::f16k (kvq_attn_f16k.hip): KVQ_KFMT 1 keeps K as fp16 rows, the
//    unpacked baseline page 1 compares against (A/B reference only, column
//    layout and head_dim 128 only).  Its K tiles are twice as large, so that
//    build runs 6 waves with 2 ring slots each.
//  - kvq::w12 (kvq_attn_w12.hip): KVQ_Q4_128_ONLY builds only the kernels
//    for q4_0 V at head_dim 128 (both layouts, single calls and batched
//    launches), with 12 waves (3 per SIMD) and 2 ring slots each; the plain
//    build hands those calls to it when their chunks reach 1536 tokens.
#ifndef KVQ_KFMT
#define KVQ_KFMT 0
#endif
#ifndef KVQ_Q4_128_ONLY
#define KVQ_Q4_128_ONLY 0
#endif

namespace kvq {
#ifdef KVQ_NS
namespace KVQ_NS {
#endif

#ifndef KVQ_WAVES
#define KVQ_WAVES 8
#endif
constexpr bool kF16K = KVQ_KFMT == 1;
constexpr int kWaves = KVQ_WAVES;          // one work-group fills a CU
constexpr int kThreads = kWaves * 64;
constexpr int kLdsBudget = 163840 - 512;   // LDS of one work-group, less the small shared words
constexpr int kMaxAppend = KVQ_MAX_APPEND;  // appended tokens per sequence in one call

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

struct AttnParams {
  uint32_t* k_qs;
  uint16_t* k_d;
  uint8_t* v_qs;
  uint16_t* v_d;
  const float* q;
  const float* k_new;     // rows appended at the end of each sequence, [n_seq][n_new][n_kv][D]
  const float* v_new;
  int n_new;              // 0: attention only
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
  float rcp_group;        // 1 / group, for small_div
  float rcp_cols;         // 1 / (rows * head_dim / 4), for small_div
  int seg_tokens;
  int max_segs;
  int chunk;              // tokens per work-group, a multiple of kTile
  int n_split;
  int causal;
  float scale_log2;       // sm_scale * log2(e)
  int merge_launch;       // 1: the split merge runs as a second launch (k_split_merge)
  int n_seq_groups;       // n_seq * n_kv_heads
  int xcd_local;          // all splits of a group on one XCD (see block_coords)
  int n_groups_pad;       // groups in the grid: n_seq_groups, rounded up to 8 when xcd_local
  int lpt_seqs;           // > 0: unsplit batch of that many sequences, groups dealt by length
  int max_len;            // the call's bound on seq_len (host argument)
  // test hook (kvq_debug_attn_isum): the kernels built with DBG store every
  // per-block int32 Q.K sum of their tiles to
  // dbg_isum[seq][qtok][q_head][dbg_max_len][D/32]
  int32_t* dbg_isum;
  int dbg_max_len;
  // measurement hook (kvq_debug_attn_timeline): the kernels built with the
  // timeline mode store stamps per work-group (stamp_row)
  unsigned long long* dbg_stamps;
};

// The timeline mode's stamps, per work-group ([sequence][kv head][split, up
// to kMaxSplits][kStamps]), in the device's constant 100 MHz clock
// (s_memrealtime): entry, Q codes ready (after the prologue's barrier), wave
// 0's first tile ready, the first and the last wave's ring done, partial
// published (split counter returned; stores issued for the row layout, whose
// merge is a second launch), merge or direct output done, and flags (bit 0:
// this work-group merged the splits, bit 1: a single split wrote its rows
// directly).  They are kept in LDS while the work-group runs and written out
// at its end: a stamp stored to memory mid-kernel would sit in the next wait
// on the memory counter and lengthen the phase it measures.
enum { kStStart, kStQ, kStTile, kStRing0, kStRing1, kStPub, kStDone, kStFlags, kStamps };
__device__ __forceinline__ unsigned long long* stamp_row(const AttnParams& p, int seq, int kvh, int split) {
  return p.dbg_stamps + (((size_t)seq * p.n_kv_heads + kvh) * kMaxSplits + split) * kStamps;
}
__device__ __forceinline__ unsigned long long now_stamp() { return __builtin_amdgcn_s_memrealtime(); }

// Where the debug build stores query row r's block sums (row r of a kv
// group is query token r / group, head kv_head * group + r % group).
__device__ __forceinline__ int32_t* dbg_row(const AttnParams& p, int seq, int kvh, int r, int nb) {
  return p.dbg_isum +
         (((size_t)seq * p.n_qtok + r / p.group) * p.n_q_heads + kvh * p.group + r % p.group) *
             (size_t)p.dbg_max_len * nb;
}

// Chunks from which single calls run the 12-wave build (12 waves x 4 tiles).
constexpr int kW12MinChunk = 12 * 4 * kTile;

// Several calls in one launch (attn_decode_packed_batch): call i runs
// work-groups start[i] .. start[i] + count[i] - 1 of the grid; start[i] is a
// multiple of 8, so a call's work-groups keep the XCD placement below, and
// the work-groups that pad a call's range to a multiple of 8 do nothing.
// mstart gives the same ranges for the split-merge launch (row layout).
constexpr int kMaxBatch = KVQ_MAX_BATCH;
struct AttnBatch {
  AttnParams p[kMaxBatch];
  int start[kMaxBatch + 1];
  int count[kMaxBatch];
  int mstart[kMaxBatch + 1];
  int n;
};
__device__ __forceinline__ int batch_call(const int* start, int n, int blk) {
  int i = 0;
#pragma unroll
  for (int k = 1; k < kMaxBatch; ++k)
    if (k < n && blk >= start[k]) i = k;
  return i;
}

// Work-groups go to the 8 XCDs round-robin by linear index.  With xcd_local
// the grid holds n_groups_pad (a multiple of 8) groups of n_split
// work-groups: linear index b runs group (b % 8) + 8 * ((b / 8) / n_split),
// split (b / 8) % n_split, so all splits of a group land on one XCD and the
// fused split merge reads partials that passed through its own L2 (groups
// past n_seq_groups only pad the grid and do nothing).  That placement is
// used when the group count is a multiple of 8 or the grid is small, where
// padding costs no parallelism; otherwise a group's splits are consecutive
// work-groups spread over all XCDs, and the merge reads their write-through
// partials after an agent-scope acquire.
constexpr int kXcds = 8;
struct BlockCoords {
  int seq, kvh, split;
  bool pad;       // a padding work-group: returns at once
  bool off_xcd;   // this work-group does not sit on the XCD its group expects
  int len;        // the sequence's length when block_coords read it, else -1
};
__device__ __forceinline__ BlockCoords block_coords(const AttnParams& p, int b) {
  int g, split;
  if (p.xcd_local) {
    const int k = b / kXcds;
    g = b % kXcds + kXcds * (k / p.n_split);
    split = k % p.n_split;
  } else {
    g = b / p.n_split;
    split = b % p.n_split;
  }
  int len = -1;
  if (p.lpt_seqs > 0) {
    // Unsplit batches: work-group b < N/2 takes the b-th longest group and
    // work-group N/2 + b the b-th shortest, so the two work-groups that
    // share a CU carry about the same total.  Every work-group ranks the
    // sequences by length (longest first, ties by index) itself.
    const int N = p.n_seq_groups, half = (N + 1) / 2;
    const int idx = b < half ? b : N - 1 - (b - half);
    const int lane = __lane_id();
    const int n = p.lpt_seqs;
    const int my = lane < n ? p.seq_len[lane] : -1;
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const int lj = __builtin_amdgcn_readlane(my, j);
      rank += (lj > my) || (lj == my && j < lane);
    }
    const unsigned long long hit = __ballot(lane < n && rank == idx / p.n_kv_heads);
    const int s = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
    g = __builtin_amdgcn_readfirstlane(s * p.n_kv_heads + idx % p.n_kv_heads);
    len = __builtin_amdgcn_readlane(my, s);
  }
  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  BlockCoords c;
  c.pad = g >= p.n_seq_groups;
  c.seq = c.pad ? 0 : g / p.n_kv_heads;
  c.kvh = c.pad ? 0 : g - c.seq * p.n_kv_heads;
  c.split = split;
  c.off_xcd = !p.xcd_local || (int)(xcc & 0xF) != b % kXcds;
  c.len = len;
  return c;
}

// Geometry of one LDS ring slot for head_dim D and V format VF.
template <int D, int VF>
struct Slot {
  static constexpr int NB = D / kBlock;
  static constexpr int VROW = VF == 0 ? D / 2 : D;   // V payload bytes per token
  static constexpr int KROW = kF16K ? 2 * D : D;     // K bytes per token
  static constexpr int KBYTES = kTile * KROW;        // K of the tile
  static constexpr int VBYTES = kTile * VROW;        // V payload of the tile
  static constexpr int SBYTES = kTile * NB * 2;      // one scale plane of the tile
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = KBYTES;
  static constexpr int DK_OFF = KBYTES + VBYTES;     // (fp16 K has no scale plane)
  static constexpr int DV_OFF = DK_OFF + (kF16K ? 0 : SBYTES);
  static constexpr int BYTES = DV_OFF + SBYTES;
  static constexpr int CPR = KROW / 16;              // 16-byte chunks per K row
  // packed bytes of one appended token in the patch buffer: K row, K scales,
  // V row, V scales
  static constexpr int PK = 0, PKS = D, PV = D + 2 * NB, PVS = D + 2 * NB + VROW;
  static constexpr int PTOK = (PVS + 2 * NB + 15) & ~15;
  static constexpr int PATCH = kMaxAppend * PTOK;   // patch buffer, after the ring
  // three slots per wave where they fit in the CU's LDS, else two; head_dim
  // 64 takes two so that two work-groups share a CU (see kOccupancy)
  static constexpr int NSLOT = (D != 64 && 3 * BYTES * kWaves + PATCH <= kLdsBudget) ? 3 : 2;
  static constexpr int RPW = (kRows + kWaves - 1) / kWaves;   // Q rows per wave
  static constexpr int QSTAGE = RPW * D * 4;         // fp32 Q rows of one wave
  // Q operands shared through wave 0's last slot: int8 codes and fp32 block
  // scales, or fp16 values for fp16 K
  static constexpr int QOPS = kF16K ? kRows * D * 2 : kRows * D + kRows * NB * 4;
  // fp32 appended rows staged in a wave's last slot, behind the Q staging
  // (and, in wave 0, the Q operands)
  static constexpr int STAGE = (QSTAGE + QOPS + 15) & ~15;
  static constexpr int STAGE_UNITS = (2 * kMaxAppend + kWaves - 1) / kWaves;   // rows per wave
  // loads per tile: K, V, and the scale planes (one load when they are 128 B)
  static constexpr int LPT = KBYTES / 1024 + VBYTES / 1024 + (kF16K || SBYTES != 256 ? 1 : 2);
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "whole 1 KB load steps");
  static_assert(!kF16K || SBYTES == 256, "fp16 K: the V scale plane is one 256-byte load");
  static_assert(QSTAGE + QOPS <= BYTES, "Q staging does not fit a slot");
  static_assert(NSLOT * BYTES * kWaves + PATCH <= kLdsBudget, "ring does not fit the LDS");
  static_assert(STAGE + STAGE_UNITS * D * 4 <= BYTES, "appended rows do not fit a slot");
};

// Direct global->LDS loads (lane l's bytes land at lds + size * l for the
// 16- and 4-byte forms used here; the sub-dword forms keep a 4-byte lane
// stride, so they are not used) issued from inline assembly: the compiler
// cannot tell which LDS bytes such a load writes and would wait for all of
// them before every LDS read, which undoes the ring.  The kernels count these
// loads themselves with vmcnt.  The address is a uniform base plus a
// per-lane 32-bit offset, or a per-lane 64-bit address.
//
// The K/V stream is read once per call, so its loads carry the nontemporal
// hint: they do not displace other lines in the caches, and on MI355X a
// plain streaming read issued this way sustains ~6.9 TB/s against ~6.0 TB/s
// without it.
template <int SIZE>
__device__ __forceinline__ void dma(const void* sbase, uint32_t voff, uint32_t lds) {
  static_assert(SIZE == 16 || SIZE == 4, "16 or 4 bytes per lane");
  if constexpr (SIZE == 16) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 ::"v"(voff), "s"(sbase), "s"(lds) : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1 nt"
                 ::"v"(voff), "s"(sbase), "s"(lds) : "memory");
  }
}
__device__ __forceinline__ void dma16_v(const void* vaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(vaddr), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4_v(const void* vaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt"
               ::"v"(vaddr), "s"(lds) : "memory");
}

// A uniform 32-bit load on the scalar path (waits only for itself).
__device__ __forceinline__ int load_uniform(const int32_t* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// n / d (0 <= n < 2^20, d >= 1) from r = 1 / d as a float (correctly
// rounded, or v_rcp_f32's 1 ulp): (n + 0.5) * r is off by at most
// (n + 0.5) / d * 2^-22, below the 0.5 / d between (n + 0.5) / d and the
// integers on either side, so the truncation gives floor(n / d) exactly.
// Three VALU instructions in place of an integer division's ~20.
__device__ __forceinline__ int small_div(int n, float r) { return (int)(((float)n + 0.5f) * r); }

// K rows are stored in LDS with their 16-byte chunks permuted: chunk q of
// token row t sits at chunk q ^ kswz(t) of the row.  The column layout reads
// 8 bytes per lane from 16 rows (tokens 8a + 4h + c for a, c < 4) and two
// chunks at once; folding both a and c into the permutation spreads those
// reads evenly over the LDS banks (XOR with t % 8 alone left half of them
// idle and doubled the cycles of every K read).
template <int CPR>
__device__ __forceinline__ int kswz(int t) {
  if constexpr (CPR == 16) return t & 15;   // fp16 K rows: chunk 4b + g read by 16 rows at once
  else if constexpr (CPR == 8) return (2 * ((t ^ (t >> 3)) & 3)) | ((t >> 2) & 1);
  else return (t ^ (t >> 3)) & 3;
}

// Per-lane byte offsets of one tile's loads inside its global rows (lane l
// of load n fills LDS chunk l of that load's 1 KB).  The V chunk order
// repeats every 1 KB.
template <int D, int VF>
struct TileLane {
  uint32_t k[Slot<D, VF>::KBYTES / 1024];
  uint32_t v[Slot<D, VF>::VBYTES / 1024];
  uint32_t s;
};
template <int D, int VF>
__device__ __forceinline__ TileLane<D, VF> tile_lane_offsets(int lane) {
  using S = Slot<D, VF>;
  TileLane<D, VF> t;
  const int r = lane / S::CPR;
  const int R = lane >> 1;
  const int c = (lane & 1) ^ ((R >> 2) & 1);
  constexpr int ROWS_PER_KB = 1024 / S::KROW;
#pragma unroll
  for (int n = 0; n < S::KBYTES / 1024; ++n) {
    const int q = (lane % S::CPR) ^ kswz<S::CPR>(r + ROWS_PER_KB * n);
    t.k[n] = (uint32_t)(r * S::KROW + 16 * q + 1024 * n);
  }
#pragma unroll
  for (int n = 0; n < S::VBYTES / 1024; ++n) t.v[n] = (uint32_t)(R * 32 + 16 * c + 1024 * n);
  t.s = (uint32_t)(4 * (lane % (S::SBYTES / 4)));
  return t;
}

// Segment of the tiles a wave is loading: looked up again only when a tile
// leaves the cached segment (tiles of one wave only move forward).
struct TileCursor {
  int seg_hi;       // first token past the cached segment
  long long base;   // global row of token t is base + t inside it
};

// Issue the loads of one tile (32 tokens starting at t0) into a ring slot.
// K rows (CPR chunks) land at chunk r*CPR + (q ^ kswz(r)); V rows (two
// chunks) at R*2 + (c ^ ((R >> 2) & 1)); scale planes as they are.
template <int D, int VF>
__device__ __forceinline__ void issue_tile(const AttnParams& p, int seq, int kvh, int t0,
                                           uint32_t slot, const TileLane<D, VF>& tl,
                                           TileCursor& cur) {
  using S = Slot<D, VF>;
  if (t0 >= cur.seg_hi) {
    const int segj = __builtin_amdgcn_readfirstlane(t0 / p.seg_tokens);
    const int seg = p.seg_table ? load_uniform(p.seg_table + (seq * p.max_segs + segj))
                                : seq * p.max_segs + segj;
    const int lo = segj * p.seg_tokens;
    cur.seg_hi = lo + p.seg_tokens;
    cur.base = ((long long)seg * p.n_kv_heads + kvh) * p.seg_tokens - lo;
  }
  const long long row0 = cur.base + t0;
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k_qs) + row0 * S::KROW;
#pragma unroll
  for (int n = 0; n < S::KBYTES / 1024; ++n) dma<16>(kg, tl.k[n], slot + S::K_OFF + 1024 * n);
  const uint8_t* vg = p.v_qs + row0 * S::VROW;
#pragma unroll
  for (int n = 0; n < S::VBYTES / 1024; ++n) dma<16>(vg, tl.v[n], slot + S::V_OFF + 1024 * n);
  const uint8_t* kdg = reinterpret_cast<const uint8_t*>(p.k_d) + row0 * S::NB * 2;
  const uint8_t* vdg = reinterpret_cast<const uint8_t*>(p.v_d) + row0 * S::NB * 2;
  if constexpr (kF16K) {
    dma<4>(vdg, tl.s, slot + S::DV_OFF);
  } else if constexpr (S::SBYTES == 256) {
    dma<4>(kdg, tl.s, slot + S::DK_OFF);
    dma<4>(vdg, tl.s, slot + S::DV_OFF);
  } else {
    // 128-byte planes: one load, lanes 0-31 K scales, lanes 32-63 V scales
    static_assert(S::SBYTES == 128 && S::DV_OFF == S::DK_OFF + 128, "scale planes");
    dma4_v((__lane_id() < 32 ? kdg : vdg) + tl.s, slot + S::DK_OFF);
  }
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

// Tiles of a work-group's chunk are dealt to its waves round-robin: wave w
// takes tiles w, w + kWaves, w + 2 kWaves, ...  Every wave accumulates the
// same tiles in the same order on every run, so for a fixed split plan the
// output is bit-for-bit reproducible.  (Handing tiles out from an LDS counter
// let a wave that runs ahead take more, 1-2 us faster on the verify step,
// but then which tiles share a wave's running maximum, and with it the fp16
// rounding of the P.V operand, changed from run to run.)
//
// The SIMDs issue their oldest wave first, so with an even deal the first
// wave on each SIMD (waves 0-3) finishes well ahead of the others: by ~7 us
// in 128-tile chunks of the 8-wave row layout (4 query tokens x 4 heads)
// and ~6 us in the ragged batch (column layout, head_dim 64), leaving one
// wave per SIMD for the rest of the chunk.  Those kernels therefore deal the last tiles
// of a chunk of at least kSkewMin tiles round-robin to waves 0-3 only (a
// fraction SF/64 of the chunk, at most a cap: kSkewF, kSkewCap), still a
// fixed map: half of the row layout's chunk up to 32 tiles (the gap is
// about the same in 64- and 128-tile chunks), 5/64 of the column layout's
// at head_dim 64.  In the 12-wave
// build of the long single-query step the three waves per SIMD finish ~5
// and ~9 us apart as well, but a CU's remaining waves still keep enough
// tiles in flight, and skewed deals measured slower there; chunks shorter
// than kSkewMin (where the deal decides the end) keep the even one.
#ifndef KVQ_SKEW_ROWS_CAP
#define KVQ_SKEW_ROWS_CAP 32  // row layout: half the chunk, at most 32 tiles
#endif
constexpr int kWaveStride = kTile * kWaves;
constexpr int kFastWaves = 4;                       // the first wave on each SIMD
constexpr int kSkewMin = 64;                        // tiles
constexpr int kNoTile = 0x3fffffff;                 // past every chunk
template <bool ROWS, int D>
constexpr int kSkewF = kWaves != 8 ? 0 : ROWS ? 32 : D == 64 ? 5 : 0;
template <bool ROWS>
constexpr int kSkewCap = ROWS ? KVQ_SKEW_ROWS_CAP : 1 << 20;

// A wave's tiles in flight: `cur` is the next one to process, `n1` was
// issued after it, `g` is the one after `n1`, not issued yet.  Tile starts
// only grow, so once one is past the chunk end all later ones are.  Tiles
// from `tail` on are the skewed tail (tail is the chunk end when there is
// none).
struct TileQueue {
  int cur, n1, g;
  int tail, wave;
};
template <int SF>
__device__ __forceinline__ int next_tile(const TileQueue& q, int t) {
  if constexpr (SF == 0) {
    return t + kWaveStride;
  } else {
    if (t >= q.tail) return t >= kNoTile ? kNoTile : t + kTile * kFastWaves;
    const int t2 = t + kWaveStride;
    if (t2 < q.tail) return t2;
    return q.wave < kFastWaves ? q.tail + kTile * q.wave : kNoTile;
  }
}
template <int SF, int CAP>
__device__ __forceinline__ TileQueue first_tiles(int c0, int wave, int chunk) {
  TileQueue q;
  const int ct = chunk / kTile;
  q.tail = c0 + (SF > 0 && ct >= kSkewMin ? chunk - kTile * min((ct * SF) >> 6, CAP) : chunk);
  q.wave = wave;
  int t = c0 + kTile * wave;
  if (SF > 0 && t >= q.tail) t = wave < kFastWaves ? q.tail + kTile * wave : kNoTile;
  q.cur = t;
  q.n1 = next_tile<SF>(q, t);
  q.g = next_tile<SF>(q, q.n1);
  return q;
}

// One step of a wave's ring: refill and wait as the slot count allows, then
// run `body` on the tile in slot SLOT (a compile-time slot, so LDS offsets
// become immediates).  Returns false once the wave's tiles are done.
template <int D, int VF, int SLOT, int SF, class Body>
__device__ __forceinline__ bool ring_step(const AttnParams& p, int seq, int kvh, int c1,
                                          uint32_t ring_lds, const TileLane<D, VF>& tl,
                                          TileCursor& cur, TileQueue& q, Body& body) {
  using S = Slot<D, VF>;
  if (q.cur >= c1) return false;
  if constexpr (S::NSLOT == 3) {
    // the next tile goes into the slot freed last step
    const int n2 = q.g;
    if (n2 < c1) issue_tile<D, VF>(p, seq, kvh, n2, ring_lds + ((SLOT + 2) % 3) * S::BYTES, tl, cur);
    q.g = next_tile<SF>(q, n2);
    wait_tiles<S::LPT>((q.n1 < c1) + (n2 < c1));
    body(std::integral_constant<int, SLOT>{}, q.cur);
    q.cur = q.n1;
    q.n1 = n2;
  } else {
    wait_tiles<S::LPT>(q.n1 < c1);
    body(std::integral_constant<int, SLOT>{}, q.cur);
    if (q.g < c1) issue_tile<D, VF>(p, seq, kvh, q.g, ring_lds + SLOT * S::BYTES, tl, cur);
    q.cur = q.n1;
    q.n1 = q.g;
    q.g = next_tile<SF>(q, q.g);
  }
  return true;
}

// Run a wave's ring to the end.  On entry tile q.cur sits in slot 0 and
// q.n1 in slot 1 (both issued or past the end).
template <int D, int VF, int SF, class Body>
__device__ __forceinline__ void run_ring(const AttnParams& p, int seq, int kvh, int c1,
                                         uint32_t ring_lds, const TileLane<D, VF>& tl,
                                         TileCursor& cur, TileQueue& q, Body& body) {
  if constexpr (Slot<D, VF>::NSLOT == 3) {
    while (ring_step<D, VF, 0, SF>(p, seq, kvh, c1, ring_lds, tl, cur, q, body) &&
           ring_step<D, VF, 1, SF>(p, seq, kvh, c1, ring_lds, tl, cur, q, body) &&
           ring_step<D, VF, 2, SF>(p, seq, kvh, c1, ring_lds, tl, cur, q, body)) {
    }
  } else {
    while (ring_step<D, VF, 0, SF>(p, seq, kvh, c1, ring_lds, tl, cur, q, body) &&
           ring_step<D, VF, 1, SF>(p, seq, kvh, c1, ring_lds, tl, cur, q, body)) {
    }
  }
}

// ---------------------------------------------------------------------------
// Rows appended in the same call
// ---------------------------------------------------------------------------
//
// With n_new > 0 the call first appends the rows k_new / v_new at tokens
// L - n_new .. L - 1 of each sequence, exactly as kv_append_quant does, and
// then attends over all L tokens.  The work-group whose chunk holds such a
// token stages the fp32 rows in its prologue (ahead of its tiles), quantizes
// them with the append kernel's block quantizers into a patch buffer in LDS,
// writes the packed rows to the cache right after its prologue, and patches
// every tile it loads that holds one of them.  Its tile loads may see the old
// or the new rows; the patch makes the LDS copy right either way, and no
// other work-group reads these rows.

// Appended tokens [lo, hi) that fall into this work-group's chunk [c0, c1).
struct AppendRange {
  int lo, hi;
};
__device__ __forceinline__ AppendRange append_range(const AttnParams& p, int L, int c0, int c1) {
  AppendRange a;
  a.lo = max(c0, L - p.n_new);
  a.hi = p.n_new > 0 ? c1 : c0;
  if (a.lo > a.hi) a.lo = a.hi;
  return a;
}

// Stage this wave's appended rows (unit u = 2 * token + {0: K, 1: V}, units
// wave, wave + kWaves, ...) as fp32 in its last slot, one dword per lane.
template <int D, int VF>
__device__ __forceinline__ void stage_appended(const AttnParams& p, int seq, int kvh, int L, int wave,
                                               const AppendRange& a, uint32_t stage_lds) {
  using S = Slot<D, VF>;
  const int units = 2 * (a.hi - a.lo);
#pragma unroll
  for (int i = 0; i < S::STAGE_UNITS; ++i) {
    const int u = wave + kWaves * i;
    if (u >= units) break;
    const int j = a.lo + (u >> 1) - (L - p.n_new);   // row of k_new / v_new
    const float* src = ((u & 1) ? p.v_new : p.k_new) +
                       (((size_t)seq * p.n_new + j) * p.n_kv_heads + kvh) * D;
#pragma unroll
    for (int n = 0; n < D / 64; ++n) dma4_v(src + 64 * n + __lane_id(), stage_lds + i * D * 4 + 256 * n);
  }
}

// Quantize this wave's staged rows into the patch buffer (per token: K row,
// K scales, V row, V scales, as the append kernel computes them).
template <int D, int VF>
__device__ __forceinline__ void quantize_appended(const AppendRange& a, int wave, const float* stage,
                                                  uint8_t* patch) {
  using S = Slot<D, VF>;
  const int lane = __lane_id();
  const int e = lane & 31;
  const int units = 2 * (a.hi - a.lo);
#pragma unroll
  for (int i = 0; i < S::STAGE_UNITS; ++i) {
    const int u = wave + kWaves * i;
    if (u >= units) break;
    uint8_t* pt = patch + (u >> 1) * S::PTOK;
#pragma unroll
    for (int e0 = 0; e0 < D; e0 += 64) {
      const float x = stage[i * D + e0 + lane];
      const int b = (e0 + lane) / kBlock;
      int code;
      uint32_t byte;
      if (!(u & 1)) {
        const uint16_t dbits = quant_sym8(x, code);
        pt[S::PK + e0 + lane] = (uint8_t)code;
        if (e == 0) reinterpret_cast<uint16_t*>(pt + S::PKS)[b] = dbits;
      } else if (VF == 0) {
        const uint16_t dbits = quant_q4_0(x, e, byte);
        if (e < 16) pt[S::PV + b * 16 + e] = (uint8_t)byte;
        if (e == 0) reinterpret_cast<uint16_t*>(pt + S::PVS)[b] = dbits;
      } else {
        const uint16_t dbits = quant_sym8(x, code);
        pt[S::PV + e0 + lane] = (uint8_t)code;
        if (e == 0) reinterpret_cast<uint16_t*>(pt + S::PVS)[b] = dbits;
      }
    }
  }
}

// Overwrite the appended tokens of tile t0 in its ring slot with their
// packed rows, in the slot's layout (K rows swizzled in 16-byte chunks, V
// and both scale planes token-interleaved).
template <int D, int VF>
__device__ __forceinline__ void patch_tile(uint8_t* slot, const uint8_t* patch, int t0,
                                           const AppendRange& a) {
  using S = Slot<D, VF>;
  constexpr int NB = D / kBlock;
  const int lane = __lane_id();
  const int lo = max(t0, a.lo), hi = min(t0 + kTile, a.hi);
  for (int pos = lo; pos < hi; ++pos) {
    const int r = pos - t0;
    const uint8_t* pt = patch + (pos - a.lo) * S::PTOK;
    if (lane < D / 4) {
      const int q = lane >> 2;
      *reinterpret_cast<uint32_t*>(slot + S::K_OFF + (r * S::CPR + (q ^ kswz<S::CPR>(r))) * 16 + 4 * (lane & 3)) =
          reinterpret_cast<const uint32_t*>(pt + S::PK)[lane];
    }
#pragma unroll
    for (int k0 = 0; k0 < S::VROW; k0 += 64) {
      const int k = k0 + lane;
      if (k < S::VROW) slot[S::V_OFF + (2 * k + ((r >> 4) ^ ((k >> 2) & 1))) * 16 + (r & 15)] = pt[S::PV + k];
    }
    if (lane < NB) {
      reinterpret_cast<uint16_t*>(slot + S::DK_OFF)[lane * kTile + r] =
          reinterpret_cast<const uint16_t*>(pt + S::PKS)[lane];
      reinterpret_cast<uint16_t*>(slot + S::DV_OFF)[lane * kTile + r] =
          reinterpret_cast<const uint16_t*>(pt + S::PVS)[lane];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Write the packed appended rows of this work-group to the cache (the
// layout kv_append_quant writes).  Runs after the prologue, before the
// wave's second tile is issued: the stores then sit behind the first tile in
// the wave's hand-counted vmcnt sequence, where an older outstanding
// operation can only make a wait stricter, and they are acknowledged long
// before the partial is published (0.4 us per 128k step against writing
// them after the loop).  The segment id comes through the scalar cache so
// that the compiler adds no vmcnt wait of its own here.
template <int D, int VF>
__device__ __forceinline__ void write_appended(const AttnParams& p, int seq, int kvh,
                                               const AppendRange& a, const uint8_t* patch) {
  using S = Slot<D, VF>;
  constexpr int NB = D / kBlock;
  const int tid = threadIdx.x;
  for (int pos = a.lo; pos < a.hi; ++pos) {
    const uint8_t* pt = patch + (pos - a.lo) * S::PTOK;
    const int segj = pos / p.seg_tokens;
    const int seg = p.seg_table ? load_uniform(p.seg_table + (seq * p.max_segs + segj)) : seq * p.max_segs + segj;
    const size_t prow = ((size_t)seg * p.n_kv_heads + kvh) * p.seg_tokens + (pos - segj * p.seg_tokens);
    const size_t tile0 = prow & ~(size_t)(kTile - 1);
    const int t = (int)(prow - tile0);
    uint8_t* kq = reinterpret_cast<uint8_t*>(p.k_qs);
    if (tid < D / 4)
      reinterpret_cast<uint32_t*>(kq + prow * D)[tid] = reinterpret_cast<const uint32_t*>(pt + S::PK)[tid];
    for (int k = tid; k < S::VROW; k += kThreads) p.v_qs[tile0 * S::VROW + (size_t)k * kTile + t] = pt[S::PV + k];
    if (tid < NB) {
      p.k_d[tile0 * NB + tid * kTile + t] = reinterpret_cast<const uint16_t*>(pt + S::PKS)[tid];
      p.v_d[tile0 * NB + tid * kTile + t] = reinterpret_cast<const uint16_t*>(pt + S::PVS)[tid];
    }
  }
}

// Common prologue, in two parts around the load of the sequence's length.
//
// prologue_issue: this wave's Q rows (wave, wave + kWaves) go to its last
// slot as fp32 ahead of its first tiles, so waiting for them leaves the tiles
// in flight; the appended rows (if any) for the length `Ls`, then the wave's
// static first tiles (q.cur, and q.n1 when three slots allow it) that start
// below `cs1`.  Rows past `rows` load row 0.  Returns the tiles issued.
// Without a segment table these loads need not wait for the length: `Ls`
// and `cs1` may come from the call's max_seq_len, every token below it lies
// inside the cache, and tiles past the real end are masked or never used.
template <int D, int VF>
__device__ __forceinline__ int prologue_issue(const AttnParams& p, uint8_t* s_lds, int seq, int kvh,
                                              int wave, int Ls, int cs1, const AppendRange& app_s,
                                              const TileLane<D, VF>& tl, TileCursor& cur,
                                              const TileQueue& q) {
  using S = Slot<D, VF>;
  constexpr int NSLOT = S::NSLOT;
  constexpr int RPW = S::RPW;            // Q rows per wave
  constexpr int PIECES = RPW * D / 4;   // 16-byte pieces of them
  const int lane = __lane_id();
  const int R = p.rows, G = p.group;
  uint8_t* ring = s_lds + wave * NSLOT * S::BYTES;
  const uint32_t ring_lds = lds_addr(ring);
  // Q rows first.  When a chunk is at most one tile per wave, only the waves
  // that own a row (row wave, wave + kWaves, ...) load Q and then every wave
  // meets at a bare barrier (no wait), so all the Q loads reach the CU's
  // memory pipeline ahead of any wave's tile loads: issued in any order, the
  // last wave's Q row queued behind the other waves' tiles and held up every
  // wave at the barrier after the quantization (gqa8k 10.13 -> 9.93 us).
  // Longer chunks are better served without the barrier (128k step +0.1 us
  // with it).
  const bool q_first = p.chunk <= kWaveStride;   // at most one tile per wave
  if (!q_first || wave < R) {
#pragma unroll
    for (int base = 0; base < PIECES; base += 64) {
      // one piece per lane; lanes past PIECES stay idle (their bytes would
      // land on the Q operands other waves write into wave 0's slot)
      const int pc = base + lane;
      if (base + 64 <= PIECES || pc < PIECES) {
        const int r = wave + kWaves * (pc / (D / 4));
        const int rr = r < R ? r : 0;
        const int tq = small_div(rr, p.rcp_group);
        const float* src = p.q + (((size_t)seq * p.n_qtok + tq) * p.n_q_heads + kvh * G + rr - tq * G) * D +
                           4 * (pc % (D / 4));
        dma16_v(src, ring_lds + (NSLOT - 1) * S::BYTES + 16 * base);
      }
    }
  }
  if (q_first) asm volatile("s_barrier" ::: "memory");
  // appended rows, ahead of the tiles so that waiting for them leaves the
  // tiles in flight
  if (app_s.hi > app_s.lo)
    stage_appended<D, VF>(p, seq, kvh, Ls, wave, app_s, ring_lds + (NSLOT - 1) * S::BYTES + S::STAGE);
  const int n = (q.cur < cs1) + (NSLOT == 3 && q.n1 < cs1);
  if (q.cur < cs1) issue_tile<D, VF>(p, seq, kvh, q.cur, ring_lds, tl, cur);
  if (NSLOT == 3 && q.n1 < cs1) issue_tile<D, VF>(p, seq, kvh, q.n1, ring_lds + S::BYTES, tl, cur);
  return n;
}

// prologue_finish: with the length L known, stages the appended rows again
// if the guess `Ls` staged other ones (after the tiles, so it then waits for
// everything), waits for the Q rows, quantizes them (a = max|q|, d = a / 127
// in fp32) into codes and scales shared through wave 0's last slot, quantizes
// the appended rows into the patch buffer, and returns after the barrier that
// publishes the codes.
template <int D, int VF>
__device__ __forceinline__ void prologue_finish(const AttnParams& p, uint8_t* s_lds, int seq, int kvh,
                                                int wave, int L, int Ls, const AppendRange& app,
                                                const AppendRange& app_s, int n_issued,
                                                uint8_t* s_patch, int8_t*& s_qc, float*& s_qd) {
  using S = Slot<D, VF>;
  constexpr int NB = D / kBlock;
  constexpr int NSLOT = S::NSLOT;
  constexpr int RPW = S::RPW;
  const int lane = __lane_id();
  const int R = p.rows;
  uint8_t* ring = s_lds + wave * NSLOT * S::BYTES;
  const bool restage = app.hi > app.lo && (L != Ls || app.lo != app_s.lo || app.hi != app_s.hi);
  if (restage) {
    stage_appended<D, VF>(p, seq, kvh, L, wave, app, lds_addr(ring) + (NSLOT - 1) * S::BYTES + S::STAGE);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    wait_tiles<S::LPT>(n_issued);
  }

  const float* s_qf = reinterpret_cast<const float*>(ring + (NSLOT - 1) * S::BYTES);
  s_qc = reinterpret_cast<int8_t*>(s_lds + (NSLOT - 1) * S::BYTES + S::QSTAGE);
  s_qd = reinterpret_cast<float*>(s_lds + (NSLOT - 1) * S::BYTES + S::QSTAGE + kRows * D);
  float qv[RPW][D / 64];
#pragma unroll
  for (int k = 0; k < RPW; ++k)
#pragma unroll
    for (int e = 0; e < D / 64; ++e)
      qv[k][e] = wave + kWaves * k < R ? s_qf[k * D + 64 * e + lane] : 0.0f;
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int r = wave + kWaves * k;
    if (r >= kRows) break;
    if constexpr (kF16K) {
      // fp16 K: Q enters the f16 dot as fp16 values
      _Float16* s_qh = reinterpret_cast<_Float16*>(s_qc);
#pragma unroll
      for (int e = 0; e < D / 64; ++e) s_qh[r * D + 64 * e + lane] = (_Float16)qv[k][e];
    } else {
#pragma unroll
      for (int e = 0; e < D / 64; ++e) quantize_q_lane(qv[k][e], 64 * e + lane, s_qc + r * D, s_qd + r * NB);
    }
  }
  if (app.hi > app.lo)
    quantize_appended<D, VF>(app, wave, reinterpret_cast<const float*>(ring + (NSLOT - 1) * S::BYTES + S::STAGE),
                             s_patch);
  __syncthreads();
}

// The start of a work-group: coordinates, the first loads and the length.
// Without a segment table (and without length-ordered dealing, which reads
// every length first) Q, the first tiles and the appended rows go out
// before the length is known, taking the call's max_seq_len for it: the
// length's load is a memory round trip at the head of every work-group's
// critical path.  A work-group whose split turns out to lie past the end
// waits for those loads before it leaves (its LDS must not be written after
// it is freed).  Returns false for such a work-group.
struct WgStart {
  int seq, kvh, split, L, n_split_seq, c0, c1;
  bool off_xcd;
  AppendRange app;
};
template <int D, int VF, int SF, int CAP>
__device__ __forceinline__ bool wg_start(const AttnParams& p, int blk, uint8_t* s_lds, int wave,
                                         uint8_t* s_patch, const TileLane<D, VF>& tl,
                                         TileCursor& cur, TileQueue& tq, int8_t*& s_qc,
                                         float*& s_qd, WgStart& w) {
  const BlockCoords bc = block_coords(p, blk);
  if (bc.pad) return false;
  w.split = bc.split;
  w.kvh = bc.kvh;
  w.seq = bc.seq;
  w.off_xcd = bc.off_xcd;
  w.c0 = w.split * p.chunk;
  const bool guess = bc.len < 0 && p.seg_table == nullptr;
  const int Ls = bc.len >= 0 ? bc.len : (guess ? p.max_len : load_uniform(p.seq_len + w.seq));
  if (w.c0 >= Ls) return false;   // no tokens here even at the bound
  tq = first_tiles<SF, CAP>(w.c0, wave, p.chunk);
  const int cs1 = min(w.c0 + p.chunk, Ls);
  const AppendRange app_s = append_range(p, Ls, w.c0, cs1);
  const int n_issued = prologue_issue<D, VF>(p, s_lds, w.seq, w.kvh, wave, Ls, cs1, app_s, tl, cur, tq);
  w.L = guess ? load_uniform(p.seq_len + w.seq) : Ls;
  w.n_split_seq = min((w.L + p.chunk - 1) / p.chunk, p.n_split);   // clamp: see k_split_merge
  if (w.split >= w.n_split_seq) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return false;
  }
  w.c1 = min(w.c0 + p.chunk, w.L);
  w.app = append_range(p, w.L, w.c0, w.c1);
  prologue_finish<D, VF>(p, s_lds, w.seq, w.kvh, wave, w.L, Ls, w.app, app_s, n_issued, s_patch, s_qc,
                         s_qd);
  return true;
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

// p * d as fp16, for two tokens at once (d is an fp16 pair, p two fp32
// values): the P.V operand of both layouts, 11 significant bits, with the
// weighted sum accumulated in fp32 by the MFMA.  Each product is formed in
// fp32 by v_fma_mix_f32 and the pair rounded to fp16 by v_cvt_pk_f16_f32.
// Written as plain arithmetic rather than inline assembly on purpose: the
// compiler inserts the wait states an MFMA needs before a VALU instruction
// overwrites a register the MFMA still reads as its accumulator input only
// for instructions it emits itself, and it reuses such a dead accumulator
// register for the next value right after the MFMA issues.
// The softmax weights enter P.V scaled by 2^kPvShift (p <= 2^kPvShift
// instead of p <= 1; the running sum l carries the same factor, so o / l and
// the split merge are unchanged).  It keeps p * d_v out of the fp16
// subnormal range for small V: with d_v about max|V| / 8 (q4_0) or
// max|V| / 127 (q8_0), a 1e-2 V scale at 128k tokens put most weights below
// 6.1e-5 and gave ~7e-3 relative error in the output (q8_0).  The bound it
// sets: p * d_v <= 2^kPvShift * d_v must stay below the fp16 maximum, i.e.
// max|V| of a block up to ~32000 for either format (the two shifts differ by
// the formats' step ratio, 16).
template <int VF>
constexpr float kPvShift = VF == 0 ? 4.0f : 8.0f;

// Headroom of the softmax reference above a row's maximum (log2 domain),
// both layouts.  The reference only moves when a score passes it, and then
// to kRefHead above the row's new maximum: right after such a rescale the
// largest weight is 2^(kPvShift - kRefHead), and later scores up to
// kRefHead higher need no rescale.  Every weight and sum of a row stays
// relative to the same reference, so o / l and the split merge are
// unchanged, and no weight exceeds 2^kPvShift.  A wave sees ~10-20 tiles
// of a chunk, and without headroom some row's maximum grew in a third (4
// rows) to most (16 rows) of them, each time rescaling every accumulator.
constexpr float kRefHead = 2.0f;

__device__ __forceinline__ uint32_t round_f16_pair(float p0, float p1, uint32_t dpair) {
  const v2h d = __builtin_bit_cast(v2h, dpair);
  const v2h r = {(_Float16)__builtin_fmaf(p0, (float)d.x, 0.0f), (_Float16)__builtin_fmaf(p1, (float)d.y, 0.0f)};
  return __builtin_bit_cast(uint32_t, r);
}

// One wave's merge block: its unnormalized rows ([16][DP] floats, rows
// padded to DP >= D so that the writes spread over the LDS banks), then
// their maxima and sums ([16] each).  A wave writes its block into its own
// ring slots as soon as its ring ends (its loads have all landed and no
// other wave reads those slots), so the waves meet at a single barrier.
template <int D, int DP>
struct MergeBlock {
  static constexpr int FLOATS = kRows * DP + 2 * kRows;
  __device__ static float* at(uint8_t* s_lds, int wave, int wave_bytes) {
    return reinterpret_cast<float*>(s_lds + wave * wave_bytes);
  }
};

// Publish this work-group's partial and, in the last work-group of the
// (sequence, kv head), merge every split into the output rows.  On entry
// every wave's merge block (MergeBlock<D, DP>, wave w's at s_lds + w *
// WAVE_BYTES) is written and the work-group is synchronized.  A sequence
// with a single split writes its rows directly.
template <int D, int LDS_BYTES, int WAVE_BYTES, int DP>
__device__ __forceinline__ void finish_split(const AttnParams& p, uint8_t* s_lds, int* s_last, int seq,
                                             int kvh, int split, int n_split_seq, bool off_xcd,
                                             unsigned long long* ts = nullptr) {
  constexpr int kBatch = 16;                              // partial loads in flight per lane
  // The column layout (the only one merging here) has rows * D / 32 <= 16,
  // so at most 8 rows (head_dim 64, 8-wave build) or 4 (head_dim 128): one
  // wave per row.
  static_assert(D == 128 || kWaves >= 8, "one wave per row of the column layout");
  static_assert(MergeBlock<D, DP>::FLOATS * 4 <= WAVE_BYTES, "a merge block does not fit a wave's slots");
  using MB = MergeBlock<D, DP>;
  const int tid = threadIdx.x;
  const int R = p.rows, G = p.group;
  auto out_row = [&](int r) {
    const int t = small_div(r, p.rcp_group);
    return p.out + (((size_t)seq * p.n_qtok + t) * p.n_q_heads + kvh * G + r - t * G) * D;
  };

  // ---- merge the waves: one (m, l, o) per row
  // A wave takes 64 consecutive elements of one row (D is a multiple of 64),
  // so the row's per-wave weights are one exponential in each of the first
  // kWaves lanes, broadcast with readlane; every lane then folds the waves'
  // partial values in wave order.
  // Partials go out with agent-scope stores (write-through, coherent across
  // XCDs once complete), so publishing needs only a wait for the stores and
  // the counter increment, not a write-back of the whole L2.
  static_assert(D % 64 == 0 && kWaves <= 16, "one row per wave, the waves' weights in one DPP row");
  const bool single = n_split_seq == 1;
  const size_t pbase = ((size_t)seq * p.n_kv_heads + kvh) * p.n_split;
  float* const po = p.part_o + ((pbase + split) * R) * D;      // this split's rows
  float* const pml = p.part_ml + ((pbase + split) * R) * 2;
  {
    const int lane = tid & 63;
    for (int e0 = __builtin_amdgcn_readfirstlane(tid - lane); e0 < R * D; e0 += kThreads) {
      const int r = e0 / D;
      const int d = e0 - r * D + lane;
      const float mw = lane < kWaves ? MB::at(s_lds, lane, WAVE_BYTES)[kRows * DP + r] : -INFINITY;
      const float lw = lane < kWaves ? MB::at(s_lds, lane, WAVE_BYTES)[kRows * DP + kRows + r] : 0.0f;
      const float M = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, max_row16(mw)), 0));
      const float a = __builtin_amdgcn_exp2f(mw - M);             // wave `lane`'s weight (0 past kWaves)
      const float l = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum_row16(a * lw)), 0));
      float o = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float aw = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a), w));
        o = fmaf(aw, MB::at(s_lds, w, WAVE_BYTES)[r * DP + d], o);
      }
      if (single) {
        out_row(r)[d] = o / l;
        continue;
      }
      __hip_atomic_store(po + r * D + d, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(pml + 2 * r, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pml + 2 * r + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // with the merge as its own launch, the kernel boundary publishes the partials
  if (single || p.merge_launch) {
    if (ts && tid == 0) {
      ts[single ? kStDone : kStPub] = now_stamp();
      ts[kStFlags] = single ? 2u : 0u;
    }
    return;
  }
  // The split merge's addressing, formed by every work-group while its
  // partial's stores are being acknowledged (off the merging work-group's
  // critical path).  Wave w merges output row w on its own (the column
  // layout has at most kWaves rows): lane (g, c) adds float4 column c of
  // splits g, g + SG, g + 2 SG, ..., so batch k's loads are a uniform base
  // plus the lane's fixed offset; the SG lane groups are summed by lane
  // swaps at the end, and no LDS or barrier is involved.  In the last batch
  // the lanes without a split reload split nsp - 1 (a finite partial) with
  // weight 0, which keeps the loads and adds free of lane masks.
  static_assert(kMaxSplits <= 64, "one lane per split");
  constexpr int CR = D / 4;                              // float4 columns of a row
  constexpr int SG = 64 / CR;                            // split groups per wave
  const int nsp = n_split_seq;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane / CR, c = lane % CR;
  const int nb = (nsp + SG - 1) / SG;                    // batches
  const int gx = min(g, nsp - 1 - SG * (nb - 1));        // the split group loaded in the last batch
  const int wr = wave < R ? wave : 0;
  const float* const ob = p.part_o + (pbase * R + wr) * D;   // row wr of split 0
  const uint32_t boff = (uint32_t)((g * R * D + 4 * c) * 4);
  const uint32_t boffx = (uint32_t)((gx * R * D + 4 * c) * 4);
  const float* const pmlw = p.part_ml + ((pbase + lane) * R + wr) * 2;   // split `lane`, row wr
  float* const dst = out_row(wr) + 4 * c;
  asm volatile("" ::"v"(boff), "v"(boffx), "v"(pmlw), "v"(dst), "s"(nb));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // The counter's low 16 bits count finished splits; each work-group that is
  // not on its group's XCD also adds 1 << 16.
  if (tid == 0) {
    const unsigned inc = 1u + (off_xcd ? (1u << 16) : 0u);
    const unsigned done = __hip_atomic_fetch_add(&p.counters[((size_t)seq * p.n_kv_heads + kvh) * kCounterStride], inc,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = (done & 0xFFFFu) == (unsigned)(n_split_seq - 1);
    const int code = last ? (((done + inc) >> 16) == 0 ? 2 : 1) : 0;
    // The last group of this (sequence, kv head) merges the partials of
    // every split.  When every split ran on this XCD, their stores went
    // through this L2 and only the CU's own cache needs dropping: done here,
    // once for all waves (they load only after the barrier below), not by
    // each wave.
    if (code == 2) asm volatile("buffer_inv sc0\n\ts_waitcnt vmcnt(0)" ::: "memory");
    *s_last = code;
    if (ts) {
      ts[kStPub] = now_stamp();
      ts[kStFlags] = last ? 1u : 0u;
    }
  }
  __syncthreads();
  if (!*s_last) return;
  // Some split ran on another XCD: stale lines of the whole L2 are dropped.
  if (*s_last == 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (wave >= R) return;
  // this row's split maxima and sums (lane = split), then the first batch of
  // partial outputs, all in flight at once
  float2 ml = {-INFINITY, 0.0f};
  if (lane < nsp) ml = *reinterpret_cast<const float2*>(pmlw);
  // Every batch issues all kBatch loads (those past the last batch repeat
  // its addresses, with weight 0 below): with a fixed count and no branch
  // between them, the weights wait for the maxima alone, not for the rows.
  float4 v[kBatch];
  auto load_batch = [&](int k0) {
    const char* pk = reinterpret_cast<const char*>(ob + (size_t)min(k0, nb - 1) * SG * R * D);   // uniform
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const bool inner = k0 + k < nb - 1;
      v[k] = *reinterpret_cast<const float4*>(pk + (inner ? boff : boffx));
      if (inner) pk += (size_t)SG * R * D * 4;
    }
  };
  load_batch(0);
  // weights exp2(m_s - M) / sum_s exp2(m_s - M) l_s, in lane s (0 past nsp)
  const float M = wave_max(ml.x);
  const float e = lane < nsp ? __builtin_amdgcn_exp2f(ml.x - M) : 0.0f;
  const float w = e / wave_sum(e * ml.y);
  float4 a = {0.0f, 0.0f, 0.0f, 0.0f};
  auto add_batch = [&](int k0) {
    float wk[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (k0 + k >= nb) break;
      wk[k] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((g + SG * (k0 + k)) << 2,
                                                                     __builtin_bit_cast(int, w)));
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (k0 + k >= nb) break;
      a.x = fmaf(wk[k], v[k].x, a.x);
      a.y = fmaf(wk[k], v[k].y, a.y);
      a.z = fmaf(wk[k], v[k].z, a.z);
      a.w = fmaf(wk[k], v[k].w, a.w);
    }
  };
  add_batch(0);
  // more splits than one batch covers: further batches
  for (int k0 = kBatch; k0 < nb; k0 += kBatch) {
    load_batch(k0);
    add_batch(k0);
  }
  // the split groups: lanes c + CR * g, summed in a fixed order
  auto fold = [&](auto swap) {
    a.x = swap(a.x);
    a.y = swap(a.y);
    a.z = swap(a.z);
    a.w = swap(a.w);
  };
  if constexpr (SG == 4) fold([](float x) { return across16(x, fadd); });
  fold([](float x) { return across32(x, fadd); });
  if (g == 0) *reinterpret_cast<float4*>(dst) = a;
  if (tid == 0) {
    if (ts) ts[kStDone] = now_stamp();
    __hip_atomic_store(&p.counters[((size_t)seq * p.n_kv_heads + kvh) * kCounterStride], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Row layout
// ---------------------------------------------------------------------------

// wq * fp16 half (0 = low, 1 = high) of `pair`, in fp32 with one rounding
// (one v_fma_mix_f32; plain arithmetic for the reason given at round_f16_pair).
template <int HI>
__device__ __forceinline__ float mul_f32_f16(float wq, uint32_t pair) {
  const v2h d = __builtin_bit_cast(v2h, pair);
  return __builtin_fmaf(wq, (float)(HI ? d.y : d.x), 0.0f);
}

// Running state of one wave: output tiles acc[n][i] = row l%16, dim
// 16n + 4(l/16) + i; the reference of row l%16 (at least its running
// maximum, log2 domain) and the sum of the weights of this lane's tokens
// (the four lanes of a row are summed once, at the end of the ring).
template <int D>
struct WaveState {
  v4f acc[D / 16];
  float mrow;
  float lrow;
};

// One 32-token tile from its LDS slot: scores, online softmax update, P.V.
// Both products run transposed, S^T = K Q^T and O^T += V^T P^T.  Score MFMA
// h takes token 8(m/4) + 4h + m%4 as its row m, so lane l receives the
// scores of row l%16 for tokens 8(l/16) + 4h + i: over h and i, the 8 tokens
// 8(l/16) .. +8, which is the k-range of lane l's B operand in the P.V MFMA.
// P thus stays in registers, and the softmax check is an in-lane maximum
// against the row's reference (kRefHead), with the two exchanges between
// the lanes of a row only when a score passes it.  `full`: every token of
// the tile is visible to every query row (no mask).
template <int D, int VF, int DBG = 0>
__device__ __forceinline__ void process_tile(uint8_t* slot, int t0, int c1, bool full,
                                             const long (&qa)[D / kBlock], const float (&dq)[D / kBlock],
                                             int vis, WaveState<D>& st, int32_t* dbg) {
  using S = Slot<D, VF>;
  constexpr int NB = D / kBlock;
  const int lane = __lane_id();
  const int col = lane & 15, grp = lane >> 4;
  v4f(&acc)[D / 16] = st.acc;

  // ---- scores (log2 domain) of row col, tokens t0 + 8*grp + 4h + i
  float s[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * (col >> 2) + 4 * h + (col & 3);   // this lane's K row in MFMA h
    long kb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int q = 2 * b + (grp >> 1);
      kb[b] = *reinterpret_cast<const long*>(slot + S::K_OFF + (r * S::CPR + (q ^ kswz<S::CPR>(r))) * 16 +
                                             8 * (grp & 1));
    }
    // K scales of the 4 output tokens (scale b of token t sits at b*32 + t)
    uint2 dk[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
      dk[b] = *reinterpret_cast<const uint2*>(slot + S::DK_OFF + (b * kTile + 8 * grp + 4 * h) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[h][i] = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const v4i c = qk_block_mfma(kb[b], qa[b]);
      if constexpr (DBG == 1) {
        // the test hook: row col, token t0 + 8*grp + 4h + i, block b
        if (dbg)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = t0 + 8 * grp + 4 * h + i;
            if (t < c1) dbg[(size_t)t * NB + b] = c[i];
          }
      }
      const float w[4] = {mul_f32_f16<0>(dq[b], dk[b].x), mul_f32_f16<1>(dq[b], dk[b].x),
                          mul_f32_f16<0>(dq[b], dk[b].y), mul_f32_f16<1>(dq[b], dk[b].y)};
#pragma unroll
      for (int i = 0; i < 4; ++i) s[h][i] = fmaf((float)c[i], w[i], s[h][i]);
    }
    if (!full) {
      const int lim = vis - t0 - 8 * grp - 4 * h;   // tokens i >= lim are not visible to row col
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i >= lim) s[h][i] = -INFINITY;
    }
  }

  // ---- online softmax against the row's reference (kRefHead): the row
  // maximum and the rescale only when a score passes it
  float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                   fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  if (__any(mx > st.mrow)) {
    mx = across32(across16(mx, fmax2), fmax2);   // the row maximum, in every lane of the row
    const float mnew = mx > st.mrow ? mx + kRefHead : st.mrow;
    const float a = __builtin_amdgcn_exp2f(st.mrow - mnew);
    st.lrow *= a;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[n] *= a;
    st.mrow = mnew;
  }
  const float mshift = st.mrow - kPvShift<VF>;   // the reference less the P.V shift
  float pr[8];   // weights of row col, tokens t0 + 8*grp + j
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[4 * h + i] = __builtin_amdgcn_exp2f(s[h][i] - mshift);
      st.lrow += pr[4 * h + i];
    }

  // ---- B operands: row col, tokens 8*grp .. +8, times the V block scale
  v8h dv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    dv[b] = *reinterpret_cast<const v8h*>(slot + S::DV_OFF + b * 64 + 16 * grp);
  if (t0 + kTile > c1) {
    // tokens past the chunk end may hold anything (even non-finite scales)
    const int lim = c1 - t0 - 8 * grp;   // tokens j >= lim are past it
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j >= lim) {
#pragma unroll
        for (int b = 0; b < NB; ++b) dv[b][j] = (_Float16)0.0f;
      }
  }

#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint32_t* dvw = reinterpret_cast<const uint32_t*>(&dv[b]);
    uint32_t hw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) hw[k] = round_f16_pair(pr[2 * k], pr[2 * k + 1], dvw[k]);
    const v8h pb = __builtin_bit_cast(v8h, hw);
    if constexpr (VF == 0) {
      // A: byte = nibble(dim 32b + col) | nibble(dim 32b + 16 + col) << 4, 8
      // tokens; the high nibble is used in place, as 16 * (n - 8) (exact), and
      // the factor 16 is taken out of those accumulators at the end
      const int R = 16 * b + col;
      const uint2 w = *reinterpret_cast<const uint2*>(
          slot + S::V_OFF + (R * 2 + ((grp >> 1) ^ ((R >> 2) & 1))) * 16 + 8 * (grp & 1));
      const v8h alo = bytes_to_f16x8(w.x & 0x0F0F0F0Fu, w.y & 0x0F0F0F0Fu, (_Float16)1032.0f);
      const v8h ahi = bytes_to_f16x8(w.x & 0xF0F0F0F0u, w.y & 0xF0F0F0F0u, (_Float16)1152.0f);
      acc[2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, pb, acc[2 * b], 0, 0, 0);
      acc[2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, pb, acc[2 * b + 1], 0, 0, 0);
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int n = 2 * b + hh;
        const int R = 16 * n + col;
        const uint2 w = *reinterpret_cast<const uint2*>(
            slot + S::V_OFF + (R * 2 + ((grp >> 1) ^ ((R >> 2) & 1))) * 16 + 8 * (grp & 1));
        // int8 code c -> byte c ^ 0x80 = c + 128 -> fp16 (1024 + c + 128) - 1152
        const v8h av = bytes_to_f16x8(w.x ^ 0x80808080u, w.y ^ 0x80808080u, (_Float16)1152.0f);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb, acc[n], 0, 0, 0);
      }
    }
  }
  // every LDS read of this slot is done before the slot is refilled
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The first and the last wave's ring end, from the per-wave stamps (after a
// barrier; thread 0 writes them).
__device__ __forceinline__ void ring_end_stamps(const unsigned long long* s_ring_end,
                                                unsigned long long* ts) {
  if (threadIdx.x != 0) return;
  unsigned long long lo = s_ring_end[0], hi = s_ring_end[0];
  for (int w = 1; w < kWaves; ++w) {
    lo = s_ring_end[w] < lo ? s_ring_end[w] : lo;
    hi = s_ring_end[w] > hi ? s_ring_end[w] : hi;
  }
  ts[kStRing0] = lo;
  ts[kStRing1] = hi;
}

template <int D, int VF, int DBG = 0>
__device__ __forceinline__ void attn_rows_body(const AttnParams& p, int blk) {
  using S = Slot<D, VF>;
  constexpr int NB = D / kBlock;
  constexpr int NT = D / 16;
  constexpr int RING = kWaves * S::NSLOT * S::BYTES;
  constexpr int LDS_BYTES = RING + S::PATCH;
  constexpr int WAVE_BYTES = S::NSLOT * S::BYTES;   // one wave's ring slots, later its merge block
  constexpr int DP = D + 4;                         // merge rows: a lane's 4 rows on distinct banks

  __shared__ __attribute__((aligned(16))) uint8_t s_lds[LDS_BYTES];
  __shared__ int s_last;
  __shared__ unsigned long long s_ring_end[DBG == 2 ? kWaves : 1];
  __shared__ unsigned long long s_tl[DBG == 2 ? kStamps : 1];   // this work-group's stamps

  const unsigned long long t_entry = DBG == 2 ? now_stamp() : 0ull;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const TileLane<D, VF> tl = tile_lane_offsets<D, VF>(lane);
  TileCursor cur = {-1, 0};
  TileQueue tq;
  const uint32_t ring_lds = lds_addr(s_lds + wave * WAVE_BYTES);
  int8_t* s_qc;
  float* s_qd;
  uint8_t* s_patch = s_lds + RING;
  WgStart ws;
  constexpr int SF = kSkewF<true, D>;
  if (!wg_start<D, VF, SF, kSkewCap<true>>(p, blk, s_lds, wave, s_patch, tl, cur, tq, s_qc, s_qd, ws)) return;
  const int split = ws.split, kvh = ws.kvh, seq = ws.seq, L = ws.L, n_split_seq = ws.n_split_seq;
  const int c1 = ws.c1;
  const AppendRange app = ws.app;
  const int R = p.rows, G = p.group;
  unsigned long long* ts = nullptr;
  if constexpr (DBG == 2) {
    ts = s_tl;
    if (tid == 0) {
      for (int k = 0; k < kStamps; ++k) s_tl[k] = 0;
      s_tl[kStStart] = t_entry;
      s_tl[kStQ] = now_stamp();
    }
  }
  bool first_tile = true;
  // Q operands and block scales of row col (zero codes and scales on padding
  // rows), and the tokens it sees: tokens below `vis`; below `vis_lo` every
  // row sees them
  long qa[NB];
  load_q_operands<D>(s_qc, qa);
  float dq[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) dq[b] = s_qd[col * NB + b] * p.scale_log2;
  const int vis = min(col < R ? (p.causal ? L - p.n_qtok + col / G + 1 : L) : 0, c1);
  const int vis_lo = min(p.causal ? L - p.n_qtok + 1 : L, c1);
  __syncthreads();   // every wave has its operands; wave 0's last slot is free
  // the packed appended rows go out now, ahead of this wave's next tile, so
  // their stores are acknowledged long before the partial is published
  if (app.hi > app.lo) write_appended<D, VF>(p, seq, kvh, app, s_patch);
  if (S::NSLOT == 2 && tq.n1 < c1) issue_tile<D, VF>(p, seq, kvh, tq.n1, ring_lds + S::BYTES, tl, cur);

  WaveState<D> st;
#pragma unroll
  for (int n = 0; n < NT; ++n) st.acc[n] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  st.mrow = -1e30f;
  st.lrow = 0.0f;
  uint8_t* ring = s_lds + wave * S::NSLOT * S::BYTES;
  int32_t* dbg = nullptr;
  if constexpr (DBG == 1) {
    if (col < R) dbg = dbg_row(p, seq, kvh, col, NB);
  }
  auto body = [&](auto slot_c, int t0) {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (DBG == 2) {
      if (first_tile && wave == 0 && lane == 0) ts[kStTile] = now_stamp();
      first_tile = false;
    }
    if (t0 + kTile > app.lo && t0 < app.hi) patch_tile<D, VF>(ring + SL * S::BYTES, s_patch, t0, app);
    // (wave-uniform by construction; readfirstlane lets the compiler branch
    // around the mask instead of masking lanes through it)
    const bool full = __builtin_amdgcn_readfirstlane(t0 + kTile - vis_lo) <= 0;
    process_tile<D, VF, DBG>(ring + SL * S::BYTES, t0, c1, full, qa, dq, vis, st, dbg);
  };
  run_ring<D, VF, SF>(p, seq, kvh, c1, ring_lds, tl, cur, tq, body);
  // a tile issued before the length was known and past it may still land
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (DBG == 2) {
    if (lane == 0) s_ring_end[wave] = now_stamp();
  }

  // ---- this wave's rows into its merge block (its own ring slots)
  st.lrow = across32(across16(st.lrow, fadd), fadd);   // the four lanes of row col
  {
    float* mb = MergeBlock<D, DP>::at(s_lds, wave, WAVE_BYTES);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      // q4_0: the high-nibble dims (odd n) accumulated 16 x their value
      const float sc = (VF == 0 && (n & 1)) ? 0.0625f : 1.0f;
      *reinterpret_cast<v4f*>(mb + col * DP + 16 * n + 4 * grp) = st.acc[n] * sc;
    }
    if (grp == 0) {
      mb[kRows * DP + col] = st.mrow;
      mb[kRows * DP + kRows + col] = st.lrow;
    }
  }
  __syncthreads();   // every wave's merge block is written
  if constexpr (DBG == 2) ring_end_stamps(s_ring_end, ts);
  finish_split<D, LDS_BYTES, WAVE_BYTES, DP>(p, s_lds, &s_last, seq, kvh, split, n_split_seq, ws.off_xcd,
                                             ts);
  if constexpr (DBG == 2) {
    // every stamp was taken by thread 0, which copies them out last
    if (tid == 0) {
      unsigned long long* row = stamp_row(p, seq, kvh, split);
      for (int k = 0; k < kStamps; ++k) row[k] = s_tl[k];
    }
  }
}

// ---------------------------------------------------------------------------
// Column layout
// ---------------------------------------------------------------------------

// Per-lane state: acc[g][i] = sum over tokens of p * V for dim 16g + 4*(l/16)
// + i of this lane's column; m is the row's softmax reference (at least its
// running maximum, log2 domain; kRefHead), c0 = kPvShift - m on the block-0
// lane of a live row (so the block sum yields score - m + kPvShift) and
// -1e30 on the block-0 lane of a padding column; l sums this lane's weights
// (each 2^kPvShift times p).
template <int D>
struct ColState {
  v4f acc[D / 16];
  float m;
  float c0;
  float l;
};

// Lanes of one row (its NB block columns) sit next to each other; the
// butterfly adds their values.
template <int NB>
__device__ __forceinline__ float sum_blocks(float x) {
  x += dpp_f<0xB1>(x);
  if constexpr (NB == 4) x += dpp_f<0x4E>(x);
  return x;
}

// The Q operand of one block for this lane: 8 int8 codes, or 8 fp16 values
// for fp16 K.
using QOp = std::conditional_t<kF16K, v8h, long>;

template <int D, int VF, int DBG = 0>
__device__ __forceinline__ void process_tile_cols(const uint8_t* slot, int t0, int c1, bool full,
                                                  bool first, int vis, bool valid,
                                                  const QOp (&qb)[D / kBlock], float wq,
                                                  ColState<D>& st, int32_t* dbg = nullptr) {
  using S = Slot<D, VF>;
  constexpr int NB = D / kBlock;
  constexpr int NG = D / 16;
  const int lane = __lane_id();
  const int col = lane & 15, grp = lane >> 4;
  const int b = col % NB;

  // ---- int32 block dots.  Half h feeds row m of A with the K row of token
  // 8*(m/4) + 4h + m%4, so output row 4*grp + i of half h is token
  // 8*grp + 4h + i: this lane ends up with tokens 8*grp .. +8 in order.
  float s[8];   // scores minus the running maximum, log2 domain, tokens t0 + 8*grp + j
  if constexpr (kF16K) {
    // fp16 K: the block dots come out of the f16 MFMA in fp32, and only the
    // softmax scale (wq) applies
    v4f cf[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      cf[h] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
      const int tau = 8 * (col >> 2) + 4 * h + (col & 3);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const int q = 4 * bb + grp;   // dims 32bb + 8grp .. +8
        const v8h ka = *reinterpret_cast<const v8h*>(slot + S::K_OFF +
                                                     (tau * S::CPR + (q ^ kswz<S::CPR>(tau))) * 16);
        cf[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[bb], cf[h], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = fmaf(cf[j >> 2][j & 3], wq, st.c0);
  } else {
    v4i cq[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      cq[h] = (v4i){0, 0, 0, 0};
      const int tau = 8 * (col >> 2) + 4 * h + (col & 3);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const int q = 2 * bb + (grp >> 1);
        const long ka = *reinterpret_cast<const long*>(
            slot + S::K_OFF + (tau * S::CPR + (q ^ kswz<S::CPR>(tau))) * 16 + 8 * (grp & 1));
        cq[h] = __builtin_amdgcn_mfma_i32_16x16x32_i8(ka, qb[bb], cq[h], 0, 0, 0);
      }
    }
    if constexpr (DBG == 1) {
      // the test hook: column (row r, block b) holds that block's sums of
      // tokens t0 + 8*grp + 4h + i (dbg points at row r's block b)
      if (valid)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = t0 + 8 * grp + 4 * h + i;
            if (t < c1) dbg[(size_t)t * NB] = cq[h][i];
          }
    }
    const uint4 dkw = *reinterpret_cast<const uint4*>(slot + S::DK_OFF + b * 64 + 16 * grp);
    const uint32_t dkv[4] = {dkw.x, dkw.y, dkw.z, dkw.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = (j & 1) ? mul_f32_f16<1>(wq, dkv[j >> 1]) : mul_f32_f16<0>(wq, dkv[j >> 1]);
      s[j] = fmaf((float)cq[j >> 2][j & 3], w, st.c0);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = sum_blocks<NB>(s[j]);
  if (!full) {
    const int lim = vis - t0 - 8 * grp;   // tokens j >= lim are not visible
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j >= lim) s[j] = -INFINITY;
  }
  float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  if (!valid) mx = -INFINITY;
  constexpr float kShift = kPvShift<VF>;
  if (first || __any(mx > kShift)) {
    // row maximum over the four lane groups (the block lanes agree already)
    const float rm = across32(across16(mx, fmax2), fmax2);
    float delta;
    // the reference moves kRefHead above the new maximum of the rows that
    // passed it
    if (first) {
      delta = rm == -INFINITY ? 0.0f : rm - kShift + kRefHead;   // nothing accumulated yet
    } else {
      delta = rm > kShift ? rm - kShift + kRefHead : 0.0f;
      const float a = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
      for (int g = 0; g < NG; ++g) st.acc[g] *= a;
      st.l *= a;
    }
    st.m += delta;
    if (b == 0 && valid) st.c0 -= delta;
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] -= delta;
  }
  float pj[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pj[j] = __builtin_amdgcn_exp2f(s[j]);
    st.l += pj[j];
  }

  // ---- B operand: p * d_v of this column's block, rounded to fp16
  const uint4 dvw = *reinterpret_cast<const uint4*>(slot + S::DV_OFF + b * 64 + 16 * grp);
  uint32_t dv[4] = {dvw.x, dvw.y, dvw.z, dvw.w};
  if (!full) {
    // tokens past the chunk end may hold anything (even non-finite scales)
    const int lim = c1 - t0 - 8 * grp;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j >= lim) dv[j >> 1] &= (j & 1) ? 0x0000FFFFu : 0xFFFF0000u;
  }
  uint32_t hw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) hw[k] = round_f16_pair(pj[2 * k], pj[2 * k + 1], dv[k]);
  const v8h bpv = __builtin_bit_cast(v8h, hw);

  // ---- (P.V)^T: A = V codes of dims 16g + col, tokens 8*grp .. +8
  if constexpr (VF == 0) {
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      // byte = nibble(dim 32bb + col) | nibble(dim 32bb + 16 + col) << 4; the
      // high nibble is used in place, as 16 * (n - 8) (exact), and the factor
      // 16 is taken out of those accumulators at the end
      const int R = 16 * bb + col;
      const uint2 w = *reinterpret_cast<const uint2*>(
          slot + S::V_OFF + (R * 2 + ((grp >> 1) ^ ((R >> 2) & 1))) * 16 + 8 * (grp & 1));
      const v8h alo = bytes_to_f16x8(w.x & 0x0F0F0F0Fu, w.y & 0x0F0F0F0Fu, (_Float16)1032.0f);
      const v8h ahi = bytes_to_f16x8(w.x & 0xF0F0F0F0u, w.y & 0xF0F0F0F0u, (_Float16)1152.0f);
      st.acc[2 * bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bpv, st.acc[2 * bb], 0, 0, 0);
      st.acc[2 * bb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bpv, st.acc[2 * bb + 1], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int R = 16 * g + col;
      const uint2 w = *reinterpret_cast<const uint2*>(
          slot + S::V_OFF + (R * 2 + ((grp >> 1) ^ ((R >> 2) & 1))) * 16 + 8 * (grp & 1));
      // int8 code c -> byte c ^ 0x80 = c + 128 -> fp16 (1024 + c + 128) - 1152
      const v8h av = bytes_to_f16x8(w.x ^ 0x80808080u, w.y ^ 0x80808080u, (_Float16)1152.0f);
      st.acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bpv, st.acc[g], 0, 0, 0);
    }
  }
}

template <int D, int VF, int DBG = 0>
__device__ __forceinline__ void attn_cols_body(const AttnParams& p, int blk) {
  using S = Slot<D, VF>;
  constexpr int NB = D / kBlock;
  constexpr int NG = D / 16;
  constexpr int RING = kWaves * S::NSLOT * S::BYTES;
  constexpr int LDS_BYTES = RING + S::PATCH;
  constexpr int WAVE_BYTES = S::NSLOT * S::BYTES;   // one wave's ring slots, later its merge block
  constexpr int DP = D + 16;                        // merge rows: 16-byte writes spread over all banks

  __shared__ __attribute__((aligned(16))) uint8_t s_lds[LDS_BYTES];
  __shared__ int s_last;
  __shared__ unsigned long long s_ring_end[DBG == 2 ? kWaves : 1];
  __shared__ unsigned long long s_tl[DBG == 2 ? kStamps : 1];   // this work-group's stamps

  const unsigned long long t_entry = DBG == 2 ? now_stamp() : 0ull;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const TileLane<D, VF> tl = tile_lane_offsets<D, VF>(lane);
  TileCursor cur = {-1, 0};
  TileQueue tq;
  const uint32_t ring_lds = lds_addr(s_lds + wave * WAVE_BYTES);
  int8_t* s_qc;
  float* s_qd;
  uint8_t* s_patch = s_lds + RING;
  WgStart ws;
  constexpr int SF = kSkewF<false, D>;
  if (!wg_start<D, VF, SF, kSkewCap<false>>(p, blk, s_lds, wave, s_patch, tl, cur, tq, s_qc, s_qd, ws)) return;
  const int split = ws.split, kvh = ws.kvh, seq = ws.seq, L = ws.L, n_split_seq = ws.n_split_seq;
  const int c1 = ws.c1;
  const AppendRange app = ws.app;
  const int R = p.rows, G = p.group;
  unsigned long long* ts = nullptr;
  if constexpr (DBG == 2) {
    ts = s_tl;
    if (tid == 0) {
      for (int k = 0; k < kStamps; ++k) s_tl[k] = 0;
      s_tl[kStStart] = t_entry;
      s_tl[kStQ] = now_stamp();
    }
  }

  // column (row r, block b); B operands hold row r's Q codes of block bb in
  // the columns of block bb only
  const int r = col / NB, b = col % NB;
  const bool valid = r < R;
  QOp qb[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    if constexpr (kF16K) {
      const _Float16* s_qh = reinterpret_cast<const _Float16*>(s_qc);
      qb[bb] = (valid && bb == b) ? *reinterpret_cast<const v8h*>(s_qh + r * D + kBlock * bb + 8 * grp)
                                  : (v8h){};
    } else {
      qb[bb] = (valid && bb == b) ? *reinterpret_cast<const long*>(s_qc + r * D + kBlock * bb + 8 * grp) : 0;
    }
  }
  float wq;
  if constexpr (kF16K) wq = valid ? p.scale_log2 : 0.0f;
  else wq = valid ? s_qd[r * NB + b] * p.scale_log2 : 0.0f;
  const int vis = valid ? min(p.causal ? L - p.n_qtok + r / G + 1 : L, c1) : 0;
  const int vis_min = min(p.causal ? L - p.n_qtok + 1 : L, c1);   // the first query token's
  __syncthreads();   // every wave has its operands; wave 0's last slot is free
  // the packed appended rows go out now, ahead of this wave's next tile, so
  // their stores are acknowledged long before the partial is published
  if (app.hi > app.lo) write_appended<D, VF>(p, seq, kvh, app, s_patch);
  if (S::NSLOT == 2 && tq.n1 < c1) issue_tile<D, VF>(p, seq, kvh, tq.n1, ring_lds + S::BYTES, tl, cur);

  ColState<D> st;
#pragma unroll
  for (int g = 0; g < NG; ++g) st.acc[g] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  st.m = 0.0f;
  st.c0 = b != 0 ? 0.0f : (valid ? kPvShift<VF> : -1e30f);
  st.l = 0.0f;

  uint8_t* ring = s_lds + wave * S::NSLOT * S::BYTES;
  int32_t* dbg = nullptr;
  if constexpr (DBG == 1) {
    if (valid) dbg = dbg_row(p, seq, kvh, r, NB) + b;
  }
  bool first = true;
  auto body = [&](auto slot_c, int t0) {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (DBG == 2) {
      if (first && wave == 0 && lane == 0) ts[kStTile] = now_stamp();
    }
    if (t0 + kTile > app.lo && t0 < app.hi) patch_tile<D, VF>(ring + SL * S::BYTES, s_patch, t0, app);
    process_tile_cols<D, VF, DBG>(ring + SL * S::BYTES, t0, c1, t0 + kTile <= vis_min, first, vis,
                                  valid, qb, wq, st, dbg);
    first = false;
  };
  run_ring<D, VF, SF>(p, seq, kvh, c1, ring_lds, tl, cur, tq, body);
  // a tile issued before the length was known and past it may still land
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (DBG == 2) {
    if (lane == 0) s_ring_end[wave] = now_stamp();
  }

  // ---- this wave's rows into its merge block (its own ring slots).  The
  // lane's useful accumulators are the two of its block b (dims 32b +
  // 4grp .. +4 and 32b + 16 + 4grp .. +4 of row r): picked by selects, then
  // written with two 16-byte stores.
  const float l = across32(across16(st.l, fadd), fadd);
  if (valid) {
    // q4_0 high-nibble dims (odd groups) were accumulated 16 times too large
    constexpr float kHi = VF == 0 ? 0.0625f : 1.0f;
    v4f lo = st.acc[0], hi = st.acc[1];
#pragma unroll
    for (int bb = 1; bb < NB; ++bb) {
      lo = b == bb ? st.acc[2 * bb] : lo;
      hi = b == bb ? st.acc[2 * bb + 1] : hi;
    }
    float* mb = MergeBlock<D, DP>::at(s_lds, wave, WAVE_BYTES);
    float* dst = mb + r * DP + 32 * b + 4 * grp;
    *reinterpret_cast<v4f*>(dst) = lo;
    *reinterpret_cast<v4f*>(dst + 16) = hi * kHi;
    if (b == 0 && grp == 0) {
      mb[kRows * DP + r] = l > 0.0f ? st.m : -1e30f;
      mb[kRows * DP + kRows + r] = l;
    }
  }
  __syncthreads();   // every wave's merge block is written
  if constexpr (DBG == 2) ring_end_stamps(s_ring_end, ts);
  finish_split<D, LDS_BYTES, WAVE_BYTES, DP>(p, s_lds, &s_last, seq, kvh, split, n_split_seq, ws.off_xcd,
                                             ts);
  if constexpr (DBG == 2) {
    // every stamp was taken by thread 0, which copies them out last
    if (tid == 0) {
      unsigned long long* row = stamp_row(p, seq, kvh, split);
      for (int k = 0; k < kStamps; ++k) row[k] = s_tl[k];
    }
  }
}

// ---------------------------------------------------------------------------
// Split merge as its own launch
// ---------------------------------------------------------------------------
//
// For the row layout (up to 16 query rows) a split's partial is 16 rows of D
// floats, and one work-group reading every split's partial would be limited
// by its own CU's bandwidth (hundreds of KB for 32-64 splits).  There the
// attention kernel only stores the partials, and this kernel combines them
// with one 64-lane work-group per (sequence, kv head, row): lane s holds
// split s's maximum and sum and forms its weight exp2(m_s - M) / sum_s
// exp2(m_s - M) l_s, which the lanes read back one split at a time
// (readlane), and each lane combines D/64 columns of the row in split order.
template <int D>
__device__ __forceinline__ void split_merge_body(const AttnParams& p, int blk) {
  constexpr int C = D / 64;      // columns per lane
  constexpr int kPre = 32;       // splits whose partials are loaded up front
  const int lane = threadIdx.x;
  const int R = p.rows, G = p.group;
  const int r = blk % R;
  const int grp = blk / R;   // sequence * n_kv_heads + kv head
  const int seq = grp / p.n_kv_heads, kvh = grp - seq * p.n_kv_heads;
  // Every slot of the group's partials (n_split of them) lies inside the
  // workspace, so the maxima, sums and the first kPre partial rows are all
  // loaded before the length says how many splits ran: one memory round
  // trip.  Slots past that count hold stale values and are never used.  All
  // kPre loads are issued (slots past n_split repeat the last one): with a
  // fixed count and no branch between them the compiler keeps them ahead of
  // the weights, which then wait for the maxima alone (loads under a
  // per-slot condition were moved below the weights, a second round trip).
  const size_t pbase = (size_t)grp * p.n_split;
  const int nmax = min(p.n_split, kPre);
  // (lanes past n_split load slot 0's pair; the weights below mask them)
  const float2 ml = *reinterpret_cast<const float2*>(
      p.part_ml + ((pbase + (lane < p.n_split ? lane : 0)) * R + r) * 2);
  // row r of split 0 (uniform) and this lane's byte offset in a row
  const char* const ob = reinterpret_cast<const char*>(p.part_o + (pbase * R + r) * D);
  const uint32_t lo = (uint32_t)(C * lane * 4);
  auto load_slot = [&](int k, float (&x)[C]) {
    const char* row = ob + (size_t)k * R * D * 4;   // uniform
    if constexpr (C == 2) {
      const float2 t = *reinterpret_cast<const float2*>(row + lo);
      x[0] = t.x;
      x[1] = t.y;
    } else {
      x[0] = *reinterpret_cast<const float*>(row + lo);
    }
  };
  float v[kPre][C];
#pragma unroll
  for (int k = 0; k < kPre; ++k) load_slot(min(k, nmax - 1), v[k]);
  const int L = p.seq_len[seq];
  // (seq_len above max_seq_len breaks the call's contract; the clamp keeps
  // the reads inside this group's partials even then)
  const int nsp = min((L + p.chunk - 1) / p.chunk, p.n_split);
  if (nsp <= 1) return;   // a single split wrote its rows itself
  const float m = lane < nsp ? ml.x : -INFINITY;
  const float M = wave_max(m);
  const float e = lane < nsp ? __builtin_amdgcn_exp2f(m - M) : 0.0f;
  const float den = wave_sum(e * (lane < nsp ? ml.y : 0.0f));
  const float w = e / den;
  float acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) acc[c] = 0.0f;
  // Every slot's sum is formed and kept only below nsp (a select, not a
  // branch: under a branch the compiler moved each slot's load into it,
  // after the weights, one round trip per slot).
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float t = fmaf(wk, v[k][c], acc[c]);
      acc[c] = k < nsp ? t : acc[c];
    }
  }
  // more than kPre splits: the rest in batches of kPre, each batch's loads
  // all in flight before its sums
  for (int k0 = kPre; k0 < nsp; k0 += kPre) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) load_slot(min(k0 + k, nsp - 1), v[k]);
    // (these slots all ran: the repeats of slot nsp - 1 are finite and
    // carry weight 0)
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const float wk = k0 + k < nsp ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                     __builtin_bit_cast(int, w), (k0 + k) & 63))
                                    : 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = fmaf(wk, v[k][c], acc[c]);
    }
  }
  const int t = small_div(r, p.rcp_group);
  float* dst = p.out + (((size_t)seq * p.n_qtok + t) * p.n_q_heads + kvh * G + r - t * G) * D + C * lane;
#pragma unroll
  for (int c = 0; c < C; ++c) dst[c] = acc[c];
}

// Work-groups per CU the column-layout kernels are built for.  At head_dim
// 64 two fit (2 ring slots, <= 128 VGPRs), so one work-group's start-up (its
// Q and first tiles in flight) overlaps another's stream: the wide batches
// that run several work-groups per CU gain ~5% (ragged: 93.7 -> 89 us).
template <int D>
constexpr int kOccupancy = (D == 64 && !kF16K) ? 2 : 1;

template <int D, int VF>
__global__ __launch_bounds__(kThreads) void k_attn_rows(AttnParams p) {
  attn_rows_body<D, VF>(p, blockIdx.x);
}
template <int D, int VF>
__global__ __launch_bounds__(kThreads, kOccupancy<D>) void k_attn_cols(AttnParams p) {
  attn_cols_body<D, VF>(p, blockIdx.x);
}
// The same kernels with the block-sum store of the test hook, and with the
// timeline stamps of the measurement hook.
template <int D, int VF>
__global__ __launch_bounds__(kThreads) void k_attn_rows_dbg(AttnParams p) {
  attn_rows_body<D, VF, 1>(p, blockIdx.x);
}
template <int D, int VF>
__global__ __launch_bounds__(kThreads, kOccupancy<D>) void k_attn_cols_dbg(AttnParams p) {
  attn_cols_body<D, VF, 1>(p, blockIdx.x);
}
template <int D, int VF>
__global__ __launch_bounds__(kThreads) void k_attn_rows_tl(AttnParams p) {
  attn_rows_body<D, VF, 2>(p, blockIdx.x);
}
template <int D, int VF>
__global__ __launch_bounds__(kThreads, kOccupancy<D>) void k_attn_cols_tl(AttnParams p) {
  attn_cols_body<D, VF, 2>(p, blockIdx.x);
}
template <int D>
__global__ __launch_bounds__(64) void k_split_merge(AttnParams p) {
  split_merge_body<D>(p, blockIdx.x);
}
template <int D, int VF>
__global__ __launch_bounds__(kThreads) void k_attn_rows_batch(AttnBatch b) {
  const int i = batch_call(b.start, b.n, blockIdx.x);
  const int blk = blockIdx.x - b.start[i];
  if (blk < b.count[i]) attn_rows_body<D, VF>(b.p[i], blk);
}
template <int D, int VF>
__global__ __launch_bounds__(kThreads, kOccupancy<D>) void k_attn_cols_batch(AttnBatch b) {
  const int i = batch_call(b.start, b.n, blockIdx.x);
  const int blk = blockIdx.x - b.start[i];
  if (blk < b.count[i]) attn_cols_body<D, VF>(b.p[i], blk);
}
template <int D>
__global__ __launch_bounds__(64) void k_split_merge_batch(AttnBatch b) {
  const int i = batch_call(b.mstart, b.n, blockIdx.x);
  const int blk = blockIdx.x - b.mstart[i];
  if (blk < b.p[i].n_seq_groups * b.p[i].rows) split_merge_body<D>(b.p[i], blk);
}

bool attn_supported(int head_dim, int v_format) {
  return (head_dim == 128 || (!kF16K && head_dim == 64)) && (v_format == 0 || v_format == 1);
}

template <int D, int VF>
static void launch_attn_kernel(AttnParams p, dim3 grid, hipStream_t stream) {
  const dim3 merge_grid((unsigned)((long long)p.n_seq_groups * p.rows));
  if (kF16K || p.rows * (D / kBlock) <= 16) {
    // column layout (the fp16-K build has no other): the split merge runs in
    // the last work-group of each group
    p.merge_launch = 0;
    if (p.dbg_isum)
      hipLaunchKernelGGL((k_attn_cols_dbg<D, VF>), grid, dim3(kThreads), 0, stream, p);
    else if (p.dbg_stamps)
      hipLaunchKernelGGL((k_attn_cols_tl<D, VF>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((k_attn_cols<D, VF>), grid, dim3(kThreads), 0, stream, p);
  } else {
    p.merge_launch = p.n_split > 1;
    if (p.dbg_isum)
      hipLaunchKernelGGL((k_attn_rows_dbg<D, VF>), grid, dim3(kThreads), 0, stream, p);
    else if (p.dbg_stamps)
      hipLaunchKernelGGL((k_attn_rows_tl<D, VF>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((k_attn_rows<D, VF>), grid, dim3(kThreads), 0, stream, p);
  }
  if (p.merge_launch) hipLaunchKernelGGL((k_split_merge<D>), merge_grid, dim3(64), 0, stream, p);
}

static AttnParams make_params(const kvq_cache& c, const float* q, float* out, int n_seq, int n_qtok,
                              int n_q_heads, const int32_t* seg_table, int max_segs,
                              const int32_t* seq_len, int max_seq_len, const SplitPlan& plan,
                              float sm_scale, int causal, void* workspace, const float* k_new,
                              const float* v_new, int n_new) {
  AttnParams p;
  const WorkspaceLayout ws = workspace_layout(c, n_seq, n_qtok, n_q_heads, plan);
  char* base = static_cast<char*>(workspace);
  p.k_qs = c.k_qs;
  p.k_d = c.k_d;
  p.v_qs = c.v_qs;
  p.v_d = c.v_d;
  p.q = q;
  p.k_new = k_new;
  p.v_new = v_new;
  p.n_new = n_new;
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
  p.rcp_group = 1.0f / (float)p.group;
  p.rcp_cols = 4.0f / (float)(p.rows * c.head_dim);
  p.n_seq_groups = n_seq * c.n_kv_heads;
  // XCD-local placement when it costs no parallelism (see block_coords)
  p.xcd_local = p.n_seq_groups % kXcds == 0 || (long long)p.n_seq_groups * plan.n_split <= 64;
  p.n_groups_pad = p.xcd_local ? (p.n_seq_groups + kXcds - 1) / kXcds * kXcds : p.n_seq_groups;
  p.merge_launch = 0;
  p.dbg_isum = nullptr;
  p.dbg_max_len = 0;
  p.dbg_stamps = nullptr;
  p.max_len = max_seq_len;
  // unsplit batches of up to 64 sequences (one lane per sequence when the
  // work-groups rank them; see block_coords): ragged batch 85.5 -> 75.7 us
  p.lpt_seqs = (plan.n_split == 1 && n_seq >= 2 && n_seq <= 64 && p.n_groups_pad == p.n_seq_groups) ? n_seq : 0;
  return p;
}

int launch_attn(const kvq_cache& c, const float* q, float* out, int n_seq, int n_qtok, int n_q_heads,
                const int32_t* seg_table, int max_segs, const int32_t* seq_len, int max_seq_len,
                const SplitPlan& plan, float sm_scale, int causal, void* workspace,
                const float* k_new, const float* v_new, int n_new, hipStream_t stream,
                int32_t* dbg_isum, int dbg_max_len, unsigned long long* dbg_stamps) {
#if KVQ_KFMT == 0 && !KVQ_Q4_128_ONLY
  // q4_0 V at head_dim 128 runs the 12-wave build when its chunks give
  // every wave at least 4 tiles
  if (c.head_dim == 128 && c.v_format == 0 && plan.chunk >= kW12MinChunk)
    return w12::launch_attn(c, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                            max_seq_len, plan, sm_scale, causal, workspace, k_new, v_new, n_new,
                            stream, dbg_isum, dbg_max_len, dbg_stamps);
#endif
  AttnParams p = make_params(c, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                             max_seq_len, plan, sm_scale, causal, workspace, k_new, v_new, n_new);
  p.dbg_isum = dbg_isum;
  p.dbg_max_len = dbg_max_len;
  p.dbg_stamps = dbg_stamps;
  const dim3 grid((unsigned)((long long)p.n_groups_pad * plan.n_split));
  if constexpr (KVQ_Q4_128_ONLY) {
    if (c.head_dim != 128 || c.v_format != 0) return -4;   // not reached: only those calls come here
    launch_attn_kernel<128, 0>(p, grid, stream);
  } else if (c.head_dim == 128) {
    if (c.v_format == 0)
      launch_attn_kernel<128, 0>(p, grid, stream);
    else
      launch_attn_kernel<128, 1>(p, grid, stream);
  } else if constexpr (!kF16K) {
    if (c.v_format == 0)
      launch_attn_kernel<64, 0>(p, grid, stream);
    else
      launch_attn_kernel<64, 1>(p, grid, stream);
  } else {
    return -4;   // not reached: the entry point checks head_dim
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

#if KVQ_KFMT == 0
template <int D, int VF>
static void launch_batch_kernels(AttnBatch& b, bool rows, hipStream_t stream) {
  // the column layout merges in the last work-group of each group, the row
  // layout in a second launch (launch_attn_kernel)
  bool merge = false;
  for (int i = 0; i < b.n; ++i) {
    b.p[i].merge_launch = rows && b.p[i].n_split > 1;
    merge = merge || b.p[i].merge_launch;
  }
  if (!rows)
    hipLaunchKernelGGL((k_attn_cols_batch<D, VF>), dim3((unsigned)b.start[b.n]), dim3(kThreads), 0, stream, b);
  else
    hipLaunchKernelGGL((k_attn_rows_batch<D, VF>), dim3((unsigned)b.start[b.n]), dim3(kThreads), 0, stream, b);
  if (merge)
    hipLaunchKernelGGL((k_split_merge_batch<D>), dim3((unsigned)b.mstart[b.n]), dim3(64), 0, stream, b);
}

int launch_attn_batch(const AttnCall* calls, const SplitPlan* plans, int n_calls, void* workspace,
                      hipStream_t stream) {
  AttnBatch b;
  b.n = n_calls;
  b.start[0] = 0;
  b.mstart[0] = 0;
  char* base = static_cast<char*>(workspace);
  for (int i = 0; i < n_calls; ++i) {
    const AttnCall& a = calls[i];
    b.p[i] = make_params(*a.cache, a.q, a.out, a.n_seq, a.n_qtok, a.n_q_heads, a.seg_table, a.max_segs,
                         a.seq_len, a.max_seq_len, plans[i], a.sm_scale, a.causal, base, nullptr,
                         nullptr, 0);
    base += workspace_layout(*a.cache, a.n_seq, a.n_qtok, a.n_q_heads, plans[i]).total;
    b.count[i] = b.p[i].n_groups_pad * plans[i].n_split;
    b.start[i + 1] = b.start[i] + (b.count[i] + kXcds - 1) / kXcds * kXcds;
    b.mstart[i + 1] = b.mstart[i] + b.p[i].n_seq_groups * b.p[i].rows;
  }
  const kvq_cache& c = *calls[0].cache;
  const bool rows = b.p[0].rows * (c.head_dim / kBlock) > 16;
#if KVQ_Q4_128_ONLY
  if (c.head_dim != 128 || c.v_format != 0) return -4;   // not reached: only those calls come here
  launch_batch_kernels<128, 0>(b, rows, stream);
#else
  // q4_0 V at head_dim 128 in the row layout runs the 12-wave build when
  // every call's chunks give every wave at least 4 tiles
  bool w12_rows = rows && c.head_dim == 128 && c.v_format == 0;
  for (int i = 0; i < n_calls; ++i) w12_rows = w12_rows && plans[i].chunk >= kW12MinChunk;
  if (w12_rows) return w12::launch_attn_batch(calls, plans, n_calls, workspace, stream);
  if (c.head_dim == 128) {
    if (c.v_format == 0)
      launch_batch_kernels<128, 0>(b, rows, stream);
    else
      launch_batch_kernels<128, 1>(b, rows, stream);
  } else {
    if (c.v_format == 0)
      launch_batch_kernels<64, 0>(b, rows, stream);
    else
      launch_batch_kernels<64, 1>(b, rows, stream);
  }
#endif
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
#endif

#ifdef KVQ_NS
}  // namespace KVQ_NS
#endif
}  // namespace kvq
