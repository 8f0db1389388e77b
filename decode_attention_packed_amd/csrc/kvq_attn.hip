// Split-K decode attention over the packed cache (MFMA path).
//
// One work-group of four waves owns one (sequence, kv head, context chunk)
// and all query rows of that kv group: up to 16 rows = query tokens x query
// heads, so grouped query heads (and the verify step's query tokens) share
// every K/V byte loaded.  Waves take 32-token tiles of the chunk in turn:
//
//   QK^T   v_mfma_i32_16x16x32_i8, one MFMA per 32-block and 16 tokens, so
//          each block keeps its own int32 dot sum (page 1: int8 K and Q go
//          straight into the integer dot); the sums are rescaled in fp32 by
//          d_q * d_k and summed over blocks, in the log2 domain.
//   softmax running maximum per row, updated once per tile; the
//          accumulators are rescaled only when it grows.
//   P.V    v_mfma_f32_16x16x32_f16.  V tiles are stored token-interleaved
//          (32 tokens per tile, "BitLLM" page 3: the layout follows the
//          reduction axis, which is T for S.V), so one 8-byte load per lane is
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
// 8 bytes (two words, byte k = token k) with values in [0, 255] after `xor`
// -> 8 exact fp16 values (byte ^ xr) - off.
__device__ __forceinline__ v8h bytes_to_f16x8(uint32_t w0, uint32_t w1, _Float16 off) {
  uint32_t r[4];
  r[0] = sub_f16x2(bytes01_f16(w0), off);
  r[1] = sub_f16x2(bytes23_f16(w0), off);
  r[2] = sub_f16x2(bytes01_f16(w1), off);
  r[3] = sub_f16x2(bytes23_f16(w1), off);
  return __builtin_bit_cast(v8h, r);
}

// Everything one wave loads for a 32-token tile: K codes and scales of
// tokens t0 + 16h + (lane % 16), and the lane's slices of the V tile.
template <int D, int VF>
struct TileData {
  static constexpr int NB = D / kBlock;
  static constexpr int NVL = VF == 0 ? NB : D / 16;
  long kb[2][NB];
  _Float16 dk[2][NB];
  long vb[NVL];
  v8h dv[NB];
};

template <int D, int VF>
__device__ __forceinline__ void load_tile(const AttnParams& p, int seq, int kvh, int t0,
                                          TileData<D, VF>& td) {
  constexpr int NB = D / kBlock;
  constexpr int VROW = VF == 0 ? D / 2 : D;
  constexpr int NVL = TileData<D, VF>::NVL;
  const int lane = __lane_id();
  const int col = lane & 15, grp = lane >> 4;
  const int segj = t0 / p.seg_tokens;
  const int seg = segment_of(p.seg_table, seq, p.max_segs, segj);
  const size_t row0 = ((size_t)seg * p.n_kv_heads + kvh) * p.seg_tokens + (t0 - segj * p.seg_tokens);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const size_t r = row0 + 16 * h + col;
    load_k_operands<D>(reinterpret_cast<const uint8_t*>(p.k_qs) + r * D, td.kb[h]);
    const _Float16* kd = reinterpret_cast<const _Float16*>(p.k_d) + r * NB;
#pragma unroll
    for (int b = 0; b < NB; ++b) td.dk[h][b] = kd[b];
  }
  const uint8_t* vt = p.v_qs + row0 * VROW;
  const _Float16* dvt = reinterpret_cast<const _Float16*>(p.v_d) + row0 * NB;
#pragma unroll
  for (int n = 0; n < NVL; ++n)
    td.vb[n] = *reinterpret_cast<const long*>(vt + (16 * n + col) * kTile + 8 * grp);
#pragma unroll
  for (int b = 0; b < NB; ++b) td.dv[b] = *reinterpret_cast<const v8h*>(dvt + b * kTile + 8 * grp);
}

template <int D, int VF>
__global__ __launch_bounds__(256) void k_attn_split(AttnParams p) {
  constexpr int NB = D / kBlock;
  constexpr int NT = D / 16;                    // 16-column output tiles
  constexpr int PSTRIDE = kTile + 4;            // padded row of the P staging tile
  static_assert(2 * kMaxSplits * kRows + 4 * (kRows * D / 4 > 256 ? kRows * D / 4 : 256) <=
                    kWaves * kRows * D, "split merge does not fit the LDS buffer");

  __shared__ __attribute__((aligned(16))) int8_t s_qc[kRows * D];
  __shared__ float s_qd[kRows * NB];
  __shared__ __attribute__((aligned(16))) float s_buf[kWaves * kRows * D];
  __shared__ float s_m[kWaves * kRows];
  __shared__ float s_l[kWaves * kRows];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  quantize_group_rows<D>(p.q, seq, p.n_qtok, p.n_q_heads, kvh, G, R, wave, kWaves, s_qc, s_qd);
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

  v4f acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  float mrow[4] = {-1e30f, -1e30f, -1e30f, -1e30f};
  float lrow[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float* sP = s_buf + wave * kRows * PSTRIDE;

  const int t_first = c0 + kTile * wave;
  constexpr int kStride = kTile * kWaves;
  constexpr int NVL = VF == 0 ? NB : NT;       // 8-byte V loads per lane
  TileData<D, VF> cur;
  if (t_first < c1) load_tile<D, VF>(p, seq, kvh, t_first, cur);
  for (int t0 = t_first; t0 < c1; t0 += kStride) {
    // issue the next tile's loads before working on this one
    TileData<D, VF> nxt;
    if (t0 + kStride < c1) load_tile<D, VF>(p, seq, kvh, t0 + kStride, nxt);
    const long(&kb)[2][NB] = cur.kb;
    const _Float16(&dk)[2][NB] = cur.dk;
    const long(&vb)[NVL] = cur.vb;
    v8h dv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) dv[b] = cur.dv[b];

    // ---- scores (log2 domain) of rows 4*grp+i, tokens t0 + 16*h + col
    float s[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[h][i] = 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const v4i c = qk_block_mfma(qa[b], kb[h][b]);
        const float dkf = (float)dk[h][b];
#pragma unroll
        for (int i = 0; i < 4; ++i) s[h][i] = fmaf((float)c[i], dqs[i][b] * dkf, s[h][i]);
      }
      const int t = t0 + 16 * h + col;
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
        for (int n = 0; n < NT; ++n) acc[n][i] *= a;
        mrow[i] = mnew[i];
      }
    }
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
      v8h ahi, alo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = pr[j] * (float)dv[b][j];
        const _Float16 hi = (_Float16)x;
        ahi[j] = hi;
        alo[j] = (_Float16)(pr[j] * (float)dv[b][j] - (float)hi);
      }
      if constexpr (VF == 0) {
        // byte = nibble(dim 32b + col) | nibble(dim 32b + 16 + col) << 4, 8 tokens
        const uint32_t w0 = (uint32_t)vb[b], w1 = (uint32_t)((unsigned long)vb[b] >> 32);
        const v8h blo = bytes_to_f16x8(w0 & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (_Float16)1032.0f);
        const v8h bhi =
            bytes_to_f16x8((w0 >> 4) & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu, (_Float16)1032.0f);
        acc[2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, blo, acc[2 * b], 0, 0, 0);
        acc[2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, blo, acc[2 * b], 0, 0, 0);
        acc[2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bhi, acc[2 * b + 1], 0, 0, 0);
        acc[2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bhi, acc[2 * b + 1], 0, 0, 0);
      } else {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int n = 2 * b + hh;
          // int8 code c -> byte c ^ 0x80 = c + 128 -> fp16 (1024 + c + 128) - 1152
          const uint32_t w0 = (uint32_t)vb[n] ^ 0x80808080u;
          const uint32_t w1 = (uint32_t)((unsigned long)vb[n] >> 32) ^ 0x80808080u;
          const v8h bv = bytes_to_f16x8(w0, w1, (_Float16)1152.0f);
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bv, acc[n], 0, 0, 0);
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bv, acc[n], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
  }

  // ---- merge the four waves through LDS; one partial per work-group
#pragma unroll
  for (int i = 0; i < 4; ++i) lrow[i] = sum_row16(lrow[i]);
  __syncthreads();   // every wave is done with its P staging tile
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
