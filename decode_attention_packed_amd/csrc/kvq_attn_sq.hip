// Single-query split-K decode attention over the packed cache (VALU path).
//
// One wave owns one (sequence, kv head, context chunk).  It quantizes the G
// query heads of the group to int8 blocks (page 1: the packed dot needs int8
// on both sides), then walks the chunk in tiles:
//   QK^T:  each token's 16-byte K slices are spread over PARTS = D/16 lanes;
//          v_dot4_i32_i8 gives a half-block int32 sum per head, rescaled in
//          fp32 by d_q * d_k and summed over the PARTS lanes with DPP.
//   softmax: scores live in the log2 domain; the running maximum is shared
//          by the whole wave and updated once per tile, so the accumulators
//          are rescaled only when the maximum grows.
//   P.V:   the same lanes read the token's V slice (16 values of one block),
//          convert codes to fp32 and accumulate p * d_v * code for every head
//          of the group, so each K/V byte is loaded once for all G heads.
// The wave writes unnormalized (m, l, o) partials; k_combine merges them.

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

struct SqParams {
  const uint32_t* k_qs;
  const uint16_t* k_d;
  const uint8_t* v_qs;
  const uint16_t* v_d;
  const float* q;
  float* part_o;
  float* part_ml;
  const int32_t* seg_table;
  const int32_t* seq_len;
  int n_kv_heads;
  int n_q_heads;
  int seg_tokens;
  int max_segs;
  int chunk;
  int n_split;
  float scale_log2;   // sm_scale * log2(e)
};

// Signed byte k of w as fp32 (one SDWA conversion on gfx950).
__device__ __forceinline__ float sbyte(uint32_t w, int k) { return (float)(int8_t)(w >> (8 * k)); }

template <int D, int G, int VF>
__global__ __launch_bounds__(64) void k_attn_split_sq(SqParams p) {
  constexpr int PARTS = D / 16;        // lanes per token (16 K bytes each)
  constexpr int SLOTS = 64 / PARTS;    // tokens per wave step
  constexpr int U = 4;                 // steps per tile
  constexpr int TILE = SLOTS * U;
  constexpr int NB = D / kBlock;
  constexpr int KW4 = D / 16;          // uint4 per K row
  constexpr int VROW = VF == 0 ? D / 2 : D;

  __shared__ __attribute__((aligned(16))) int8_t s_qc[G * D];
  __shared__ float s_qd[G * NB];

  const int lane = threadIdx.x;
  const int part = lane % PARTS;
  const int slot = lane / PARTS;
  const int bk = part >> 1;            // block index of this lane's K/V dims
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int L = p.seq_len[seq];
  const int c0 = split * p.chunk;
  const int c1 = min(c0 + p.chunk, L);
  const size_t prow0 = ((size_t)seq * p.n_q_heads + (size_t)kvh * G) * p.n_split + split;

  if (c0 >= c1) {
    for (int i = lane; i < G * D; i += 64) {
      const int g = i / D;
      p.part_o[(prow0 + (size_t)g * p.n_split) * D + (i - g * D)] = 0.0f;
    }
    if (lane < G) {
      p.part_ml[(prow0 + (size_t)lane * p.n_split) * 2] = -INFINITY;
      p.part_ml[(prow0 + (size_t)lane * p.n_split) * 2 + 1] = 0.0f;
    }
    return;
  }

  quantize_q_wave(p.q + ((size_t)seq * p.n_q_heads + (size_t)kvh * G) * D, G * D, s_qc, s_qd);
  __syncthreads();

  uint32_t qw[G][4];
  float dqs[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 t = *reinterpret_cast<const uint4*>(s_qc + g * D + 16 * part);
    qw[g][0] = t.x; qw[g][1] = t.y; qw[g][2] = t.z; qw[g][3] = t.w;
    dqs[g] = s_qd[g * NB + bk] * p.scale_log2;
  }

  float acc[G][16];
  float m[G], l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[g][i] = 0.0f;
  }

  for (int t0 = c0; t0 < c1; t0 += TILE) {
    const int segj = t0 / p.seg_tokens;
    const int seg = segment_of(p.seg_table, seq, p.max_segs, segj);
    const size_t rbase = ((size_t)seg * p.n_kv_heads + kvh) * p.seg_tokens + (t0 - segj * p.seg_tokens);
    const int nvalid = c1 - t0;

    // ---- scores of the tile (log2 domain)
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tt = u * SLOTS + slot;
      const bool valid = tt < nvalid;
      const size_t r = rbase + (valid ? tt : 0);
      const uint4 kv = reinterpret_cast<const uint4*>(p.k_qs)[r * KW4 + part];
      const float dk = half_bits_to_f32(p.k_d[r * NB + bk]);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        int is = dot4(qw[g][0], kv.x, 0);
        is = dot4(qw[g][1], kv.y, is);
        is = dot4(qw[g][2], kv.z, is);
        is = dot4(qw[g][3], kv.w, is);
        const float ps = sum_parts<PARTS>((float)is * (dqs[g] * dk));
        s[u][g] = valid ? ps : -INFINITY;
      }
    }

    // ---- wave-wide tile maximum; rescale only when it grows
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][g]);
      mx = max_slots<PARTS>(mx);
      const float mn = fmaxf(m[g], mx);
      if (mn > m[g]) {
        const float sc = __builtin_amdgcn_exp2f(m[g] - mn);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] *= sc;
        l[g] *= sc;
        m[g] = mn;
      }
    }

    // ---- P.V with in-loop dequantization
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tt = u * SLOTS + slot;
      const bool valid = tt < nvalid;
      const size_t r = rbase + (valid ? tt : 0);
      float vals[16];
      float dv;
      if constexpr (VF == 0) {
        // q4_0: nibble n -> (n ^ 8) is the 4-bit two's complement of n - 8;
        // moved to the top of its byte it reads as the int8 16 * (n - 8).
        const uint2 vv = *reinterpret_cast<const uint2*>(p.v_qs + r * VROW + 8 * part);
        const uint32_t w2[2] = {vv.x, vv.y};
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
          const uint32_t x = w2[wi] ^ 0x88888888u;
          const uint32_t lo = (x << 4) & 0xF0F0F0F0u;
          const uint32_t hi = x & 0xF0F0F0F0u;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            vals[8 * wi + k] = sbyte(lo, k);
            vals[8 * wi + 4 + k] = sbyte(hi, k);
          }
        }
        dv = half_bits_to_f32(p.v_d[r * NB + bk]) * 0.0625f;
      } else {
        const uint4 vv = *reinterpret_cast<const uint4*>(p.v_qs + r * VROW + 16 * part);
        const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int wi = 0; wi < 4; ++wi)
#pragma unroll
          for (int k = 0; k < 4; ++k) vals[4 * wi + k] = sbyte(w4[wi], k);
        dv = half_bits_to_f32(p.v_d[r * NB + bk]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pe = valid ? __builtin_amdgcn_exp2f(s[u][g] - m[g]) : 0.0f;
        l[g] += pe;
        const float pv = pe * dv;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] = fmaf(pv, vals[i], acc[g][i]);
      }
    }
  }

  // ---- merge the token slots of the wave and write the partials
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = sum_slots<PARTS>(l[g]);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[g][i] = sum_slots<PARTS>(acc[g][i]);
  }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* o = p.part_o + (prow0 + (size_t)g * p.n_split) * D;
      if constexpr (VF == 0) {
        const int base = 32 * bk + 8 * (part & 1);
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
          *reinterpret_cast<float4*>(o + base + 4 * wi) =
              make_float4(acc[g][8 * wi], acc[g][8 * wi + 1], acc[g][8 * wi + 2], acc[g][8 * wi + 3]);
          *reinterpret_cast<float4*>(o + base + 16 + 4 * wi) =
              make_float4(acc[g][8 * wi + 4], acc[g][8 * wi + 5], acc[g][8 * wi + 6], acc[g][8 * wi + 7]);
        }
      } else {
#pragma unroll
        for (int wi = 0; wi < 4; ++wi)
          *reinterpret_cast<float4*>(o + 16 * part + 4 * wi) =
              make_float4(acc[g][4 * wi], acc[g][4 * wi + 1], acc[g][4 * wi + 2], acc[g][4 * wi + 3]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (lane == g) {
      p.part_ml[(prow0 + (size_t)g * p.n_split) * 2] = m[g];
      p.part_ml[(prow0 + (size_t)g * p.n_split) * 2 + 1] = l[g];
    }
  }
}

template <int D, int G, int VF>
static void launch_sq_t(const SqParams& p, int n_seq, hipStream_t stream) {
  hipLaunchKernelGGL((k_attn_split_sq<D, G, VF>), dim3(p.n_split, p.n_kv_heads, n_seq), dim3(64), 0,
                     stream, p);
}

template <int D, int VF>
static bool dispatch_g(int g, const SqParams& p, int n_seq, hipStream_t s) {
  switch (g) {
    case 1: launch_sq_t<D, 1, VF>(p, n_seq, s); return true;
    case 2: launch_sq_t<D, 2, VF>(p, n_seq, s); return true;
    case 4: launch_sq_t<D, 4, VF>(p, n_seq, s); return true;
    case 8: launch_sq_t<D, 8, VF>(p, n_seq, s); return true;
    default: return false;
  }
}

bool attn_sq_supported(int head_dim, int group, int v_format) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8) &&
         (v_format == 0 || v_format == 1);
}

int launch_attn_sq(const kvq_cache& c, const float* q, float* out, int n_seq, int n_q_heads,
                   const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                   const SplitPlan& plan, float sm_scale, void* workspace, hipStream_t stream) {
  const int D = c.head_dim;
  const int G = n_q_heads / c.n_kv_heads;
  const size_t n_rows = (size_t)n_seq * n_q_heads;
  SqParams p;
  p.k_qs = c.k_qs;
  p.k_d = c.k_d;
  p.v_qs = c.v_qs;
  p.v_d = c.v_d;
  p.q = q;
  p.part_o = static_cast<float*>(workspace);
  p.part_ml = p.part_o + n_rows * plan.n_split * D;
  p.seg_table = seg_table;
  p.seq_len = seq_len;
  p.n_kv_heads = c.n_kv_heads;
  p.n_q_heads = n_q_heads;
  p.seg_tokens = c.seg_tokens;
  p.max_segs = max_segs;
  p.chunk = plan.chunk;
  p.n_split = plan.n_split;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  bool ok;
  if (D == 128)
    ok = c.v_format == 0 ? dispatch_g<128, 0>(G, p, n_seq, stream) : dispatch_g<128, 1>(G, p, n_seq, stream);
  else
    ok = c.v_format == 0 ? dispatch_g<64, 0>(G, p, n_seq, stream) : dispatch_g<64, 1>(G, p, n_seq, stream);
  if (!ok) return -2;
  if (hipGetLastError() != hipSuccess) return -4;
  return launch_combine(p.part_o, p.part_ml, out, (int)n_rows, plan.n_split, D, stream);
}

}  // namespace kvq
