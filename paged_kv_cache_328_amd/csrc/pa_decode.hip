// Paged decode attention for gfx950: pass 1 (per-partition attention over the
// block table) and pass 2 (log-sum-exp merge of the partitions).
//
// What is computed: for sequence s and query head h, the softmax attention of
// q[s,h] over the sequence's cached keys/values, which sit in fixed-size
// physical blocks reached through the block table (wiblog "PagedAttention"
// page, sections on the block mapping and on the dedicated kernel; the
// attention formula itself is the ordinary one).  Long contexts are split
// into partitions (the PARTITION_SIZE split of the intelliparadigm page,
// sections 3.1-3.2); each partition writes (max, sum, unnormalised output)
// and pass 2 merges them exactly: M = max_p m_p, out = sum_p 2^(m_p-M) acc_p /
// sum_p 2^(m_p-M) l_p (logits are kept in base 2: x * scale * log2(e)).
//
// Pool layout (intelliparadigm page, section 2.2), 16-bit types, x = 8:
//   K [NB, Hkv, D/8, BS, 8]: for a fixed 8-channel chunk, the BS tokens of a
//     block are consecutive 16-byte vectors;
//   V [NB, Hkv, D, BS]:      for a fixed channel, the BS tokens are consecutive.
// These are exactly the operand layouts of the gfx950 matrix instruction
// v_mfma_f32_16x16x32_{f16,bf16}, where each lane feeds 8 consecutive
// reduction-dimension elements of one row:
//   QK:  S[token][head]  = K[token][d]   x Q^T[d][head]   (reduction over d:
//        a lane loads one token's 8-channel chunk = one 16-byte vector of K)
//   PV:  O^T[d][head]   += V^T[d][token] x P^T[token][head] (reduction over
//        tokens: a lane loads 8 consecutive tokens of one channel = one
//        16-byte vector of V)
// The S accumulator leaves lane l holding 8 logits of head l%16, which is
// exactly the P^T operand lane l must feed to the PV product, so the softmax
// weights never move between lanes; the running max / sum per head is
// lane-local too, because O^T keeps head l%16 in lane l.
//
// Work decomposition: one wave (64 lanes) per (partition, KV head, group of
// up to 16 query heads sharing that KV head, sequence).  The group of G
// query heads that read one KV head is the N = 16 dimension of both products,
// so K/V bytes are read once per KV head whatever G is.  A wave walks its
// partition in chunks of 32 tokens (two 16-token MFMA tiles).
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 32;          // tokens per step of the 16-bit kernel
constexpr int kMaxF32Part = 1024;   // largest partition of the fp32 kernel

// ----------------------------------------------------------------------------
// 16-bit pass 1 (matrix cores).
// grid: x = partition, y = KV head * groups + group, z = sequence; block = 64.
// ----------------------------------------------------------------------------
template <typename Ty, int D, int BS>
__global__ __launch_bounds__(64) void decode_mfma_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, int Hq, int Hkv, int G, int n_groups, int NB,
    int max_blocks, int max_ctx, float scale_log2, int P, int max_parts,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
  static_assert(BS == 16 || BS == 32, "block size 16 or 32");
  static_assert(D % 32 == 0, "head_dim multiple of 32");
  using V8 = typename Ty::vec8;
  constexpr int KK = D / 32;     // QK products along head_dim (32 channels each)
  constexpr int MM = D / 16;     // PV products along head_dim (16 channels each)
  constexpr int TILE = D * BS;   // elements of one (block, KV head) tile

  const int lane = threadIdx.x;
  const int i = lane & 15;       // row (A operand) / column (B operand, output)
  const int g4 = lane >> 4;      // which 8-element slice of the reduction dim
  const int p = blockIdx.x;
  const int hk = blockIdx.y / n_groups;
  const int grp = blockIdx.y - hk * n_groups;
  const int s = blockIdx.z;

  const int c = clampi(lens[s], 0, min(max_ctx, max_blocks * BS));
  const int n_p = (c + P - 1) / P;
  if (p >= max(n_p, 1)) return;
  const int t_begin = p * P;
  const int t_end = min(c, t_begin + P);

  const int hl = grp * 16 + i;   // query head within the KV head's group
  const bool head_ok = hl < G;
  const int qh = hk * G + (head_ok ? hl : 0);

  // Q^T operand of the QK product: lane feeds head i, channels 8*(4*kk+g4)..+8.
  V8 qop[KK];
  {
    const uint16_t* qrow = q + ((int64_t)s * Hq + qh) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 raw = head_ok ? load16(qrow + 8 * (4 * kk + g4)) : u32x4{0u, 0u, 0u, 0u};
      qop[kk] = __builtin_bit_cast(V8, raw);
    }
  }

  f32x4 acc[MM];
#pragma unroll
  for (int mm = 0; mm < MM; ++mm) acc[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of the base-2 logits (per head i)
  float l_run = 0.f;        // this lane's share of the running sum

  const int32_t* trow = tables + (int64_t)s * max_blocks;
  const int64_t blk_stride = (int64_t)Hkv * TILE;
  const int64_t head_off = (int64_t)hk * TILE;
  // Token (within the 32-token chunk) fed by A-operand row i of tile 0; tile 1
  // adds 4.  With this order the S accumulator of lane l holds tokens
  // 8*g4 .. 8*g4+7, the same 8 tokens lane l feeds to the PV product.
  const int tok_row = 8 * (i >> 2) + (i & 3);

  for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int bA = uniform(clampi(trow[t0 / BS], 0, NB - 1));
    int bB = bA;
    if (BS == 16 && t0 + 16 < c) bB = uniform(clampi(trow[t0 / BS + 1], 0, NB - 1));
    const uint16_t* kA = kc + bA * blk_stride + head_off;
    const uint16_t* kB = kc + bB * blk_stride + head_off;
    const uint16_t* vA = vc + bA * blk_stride + head_off;
    const uint16_t* vB = vc + bB * blk_stride + head_off;

    // K operands: row i of tile `tl` is token tok_row + 4*tl, chunk 4*kk+g4.
    u32x4 kraw[2][KK];
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      const int tok = tok_row + 4 * tl;
      const uint16_t* kb = (BS == 16 && tok >= 16) ? kB : kA;
      const int o = BS == 16 ? (tok & 15) : tok;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kraw[tl][kk] = load16(kb + ((4 * kk + g4) * BS + o) * 8);
    }
    // V operands: channel 16*mm + i, tokens 8*g4 .. 8*g4+7.
    u32x4 vraw[MM];
    {
      const uint16_t* vb = (BS == 16 && g4 >= 2) ? vB : vA;
      const int o0 = BS == 16 ? 8 * (g4 & 1) : 8 * g4;
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) vraw[mm] = load16(vb + (16 * mm + i) * BS + o0);
    }

    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s0 = Ty::mma(__builtin_bit_cast(V8, kraw[0][kk]), qop[kk], s0);
      s1 = Ty::mma(__builtin_bit_cast(V8, kraw[1][kk]), qop[kk], s1);
    }
    // x[e]: base-2 logit of token t0 + 8*g4 + e for head i.
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = s0[j] * scale_log2;
      x[4 + j] = s1[j] * scale_log2;
    }
    if (t0 + kChunk > c) {  // last chunk: drop tokens past the context by select
      const int first = t0 + 8 * g4;
      uint32_t keep[4];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (first + e >= c) x[e] = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        keep[w] = (first + 2 * w < c ? 0x0000FFFFu : 0u) | (first + 2 * w + 1 < c ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int mm = 0; mm < MM; ++mm)
#pragma unroll
        for (int w = 0; w < 4; ++w) vraw[mm][w] &= keep[w];
    }

    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2_fast(m_run - m_new);  // 0 on the first chunk
    m_run = m_new;

    uint32_t pw[4];
    float psum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint16_t lo = Ty::from_f32(exp2_fast(x[2 * w] - m_new));
      const uint16_t hi = Ty::from_f32(exp2_fast(x[2 * w + 1] - m_new));
      psum += Ty::to_f32(lo) + Ty::to_f32(hi);  // the sum uses the weights the PV product sees
      pw[w] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    l_run = l_run * alpha + psum;
    const V8 pop = __builtin_bit_cast(V8, u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) {
      acc[mm] *= alpha;
      acc[mm] = Ty::mma(__builtin_bit_cast(V8, vraw[mm]), pop, acc[mm]);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!head_ok) return;

  // Lane holds O^T[d = 16*mm + 4*g4 + j][head i], j = 0..3.
  if (n_p <= 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = out + ((int64_t)s * Hq + qh) * D;
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) {
      const f32x4 a = acc[mm] * inv;
      const u32x2 packed = {(uint32_t)Ty::from_f32(a[0]) | ((uint32_t)Ty::from_f32(a[1]) << 16),
                            (uint32_t)Ty::from_f32(a[2]) | ((uint32_t)Ty::from_f32(a[3]) << 16)};
      *reinterpret_cast<u32x2*>(orow + 16 * mm + 4 * g4) = packed;
    }
  } else {
    const int64_t idx = ((int64_t)s * Hq + qh) * max_parts + p;
    float* a = ws_acc + idx * D;
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) *reinterpret_cast<f32x4*>(a + 16 * mm + 4 * g4) = acc[mm];
    if (g4 == 0) {
      ws_ml[2 * idx] = m_run;
      ws_ml[2 * idx + 1] = l_tot;
    }
  }
}

// ----------------------------------------------------------------------------
// fp32 pass 1 (vector ALU).  One wave per (partition, query head, sequence).
// Logits of the partition go to LDS, then the weights, then each lane
// accumulates whole channels.  K layout for fp32: [NB, Hkv, D/4, BS, 4].
// ----------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(64) void decode_f32_kernel(
    float* __restrict__ out, const float* __restrict__ q, const float* __restrict__ kc,
    const float* __restrict__ vc, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, int Hq, int Hkv, int G, int NB, int max_blocks,
    int max_ctx, float scale_log2, int P, int max_parts, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml) {
  __shared__ float xs[kMaxF32Part];
  __shared__ float qs[D];
  const int lane = threadIdx.x;
  const int p = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int hk = h / G;
  const int c = clampi(lens[s], 0, min(max_ctx, max_blocks * BS));
  const int n_p = (c + P - 1) / P;
  if (p >= max(n_p, 1)) return;
  const int t_begin = p * P;
  const int n = max(0, min(c, t_begin + P) - t_begin);
  const int32_t* trow = tables + (int64_t)s * max_blocks;
  const int64_t tile = (int64_t)D * BS;

  for (int d = lane; d < D; d += kWave) qs[d] = q[((int64_t)s * Hq + h) * D + d];
  __syncthreads();

  float mloc = -INFINITY;
  for (int t = lane; t < n; t += kWave) {
    const int tok = t_begin + t;
    const int64_t b = clampi(trow[tok / BS], 0, NB - 1);
    const float* kb = kc + (b * Hkv + hk) * tile + (tok % BS) * 4;
    float dot = 0.f;
#pragma unroll 4
    for (int cc = 0; cc < D / 4; ++cc) {
      const f32x4 k4 = *reinterpret_cast<const f32x4*>(kb + cc * BS * 4);
      dot = fmaf(qs[4 * cc], k4[0], dot);
      dot = fmaf(qs[4 * cc + 1], k4[1], dot);
      dot = fmaf(qs[4 * cc + 2], k4[2], dot);
      dot = fmaf(qs[4 * cc + 3], k4[3], dot);
    }
    const float x = dot * scale_log2;
    xs[t] = x;
    mloc = fmaxf(mloc, x);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
  float lloc = 0.f;
  for (int t = lane; t < n; t += kWave) {
    const float w = exp2_fast(xs[t] - mloc);
    xs[t] = w;
    lloc += w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lloc += __shfl_xor(lloc, off);
  __syncthreads();

  for (int d = lane; d < D; d += kWave) {
    float a = 0.f;
    for (int t = 0; t < n; ++t) {
      const int tok = t_begin + t;
      const int64_t b = clampi(trow[tok / BS], 0, NB - 1);
      a = fmaf(xs[t], vc[((b * Hkv + hk) * D + d) * BS + tok % BS], a);
    }
    if (n_p <= 1) {
      out[((int64_t)s * Hq + h) * D + d] = lloc > 0.f ? a / lloc : 0.f;
    } else {
      const int64_t idx = ((int64_t)s * Hq + h) * max_parts + p;
      ws_acc[idx * D + d] = a;
      if (d == 0) {
        ws_ml[2 * idx] = mloc;
        ws_ml[2 * idx + 1] = lloc;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Pass 2: merge the partitions of every (sequence, query head) that has more
// than one.  grid: x = query head, y = sequence; block = D threads.
// ----------------------------------------------------------------------------
template <typename OutT>
__global__ __launch_bounds__(256) void merge_kernel(
    OutT* __restrict__ out, const int32_t* __restrict__ lens, const float* __restrict__ ws_acc,
    const float* __restrict__ ws_ml, int Hq, int D, int max_ctx, int max_blocks, int BS, int P,
    int max_parts) {
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int c = clampi(lens[s], 0, min(max_ctx, max_blocks * BS));
  const int n_p = (c + P - 1) / P;
  if (n_p <= 1 || d >= D) return;
  const int64_t base = ((int64_t)s * Hq + h) * max_parts;
  float M = -INFINITY;
  for (int p = 0; p < n_p; ++p) M = fmaxf(M, ws_ml[2 * (base + p)]);
  float L = 0.f, o = 0.f;
  for (int p = 0; p < n_p; ++p) {
    const float w = exp2_fast(ws_ml[2 * (base + p)] - M);
    L = fmaf(w, ws_ml[2 * (base + p) + 1], L);
    o = fmaf(w, ws_acc[(base + p) * D + d], o);
  }
  const float r = o / L;
  if constexpr (sizeof(OutT) == 4) {
    out[((int64_t)s * Hq + h) * D + d] = r;
  } else {
    out[((int64_t)s * Hq + h) * D + d] = OutT::from_f32(r);
  }
}

// Output adaptor for 16-bit merges (stores the rounded bit pattern).
template <typename Ty>
struct Out16 {
  uint16_t bits;
  static __device__ __forceinline__ Out16 from_f32(float f) { return Out16{Ty::from_f32(f)}; }
};

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
struct Plan {
  int P = 0;          // partition size in tokens
  int max_parts = 0;  // partitions of the longest context
  int groups = 1;     // query-head groups of 16 per KV head (16-bit kernel)
  size_t ws_bytes = 0;
};

pa_status validate(const pa_decode_args* a) {
  if (!a) return PA_ERR_INVALID;
  if (!elem_bytes(a->dtype)) return PA_ERR_INVALID;
  if (a->num_seqs < 0 || a->num_q_heads <= 0 || a->num_kv_heads <= 0 || a->head_dim <= 0 ||
      a->block_size <= 0 || a->num_blocks <= 0 || a->max_blocks_per_seq <= 0 ||
      a->max_context_len < 0)
    return PA_ERR_INVALID;
  if (a->num_q_heads % a->num_kv_heads != 0) return PA_ERR_INVALID;
  if ((int64_t)a->max_context_len > (int64_t)a->max_blocks_per_seq * a->block_size)
    return PA_ERR_INVALID;
  if (a->partition_size < 0) return PA_ERR_INVALID;
  if (a->partition_size > 0 && (a->partition_size % kChunk || a->partition_size % a->block_size))
    return PA_ERR_INVALID;
  if (!isfinite(a->scale)) return PA_ERR_INVALID;
  if (a->head_dim != 64 && a->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (a->block_size != 16 && a->block_size != 32) return PA_ERR_UNSUPPORTED;
  if (a->dtype == PA_F32 && a->partition_size > kMaxF32Part) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Partition size when the caller leaves it to the library: the smallest of
// 512/256/128 tokens that still yields enough waves to cover the chip
// (256 CUs x 16 waves), judged from the longest context.
int choose_partition(const pa_decode_args* a, int waves_per_part) {
  if (a->dtype == PA_F32) return 512;
  const int64_t base = (int64_t)a->num_seqs * waves_per_part;
  const int64_t target = 256 * 16;
  for (int P : {512, 256, 128}) {
    const int64_t parts = (a->max_context_len + P - 1) / P;
    if (base * parts >= target) return P;
  }
  return 128;
}

Plan make_plan(const pa_decode_args* a) {
  Plan pl;
  const int G = a->num_q_heads / a->num_kv_heads;
  pl.groups = a->dtype == PA_F32 ? 1 : (G + 15) / 16;
  const int waves_per_part = a->dtype == PA_F32 ? a->num_q_heads : a->num_kv_heads * pl.groups;
  pl.P = a->partition_size > 0 ? a->partition_size : choose_partition(a, waves_per_part);
  pl.max_parts = (a->max_context_len + pl.P - 1) / pl.P;
  if (pl.max_parts > 1)
    pl.ws_bytes = (size_t)a->num_seqs * a->num_q_heads * pl.max_parts * (a->head_dim + 2) * 4;
  return pl;
}

template <typename Ty, int D, int BS>
void launch_mfma(const pa_decode_args* a, const Plan& pl, float* ws_acc, float* ws_ml,
                 hipStream_t st) {
  const int G = a->num_q_heads / a->num_kv_heads;
  dim3 grid((unsigned)max(pl.max_parts, 1), (unsigned)(a->num_kv_heads * pl.groups),
            (unsigned)a->num_seqs);
  decode_mfma_kernel<Ty, D, BS><<<grid, 64, 0, st>>>(
      (uint16_t*)a->out, (const uint16_t*)a->q, (const uint16_t*)a->k_cache,
      (const uint16_t*)a->v_cache, a->block_tables, a->context_lens, a->num_q_heads,
      a->num_kv_heads, G, pl.groups, a->num_blocks, a->max_blocks_per_seq, a->max_context_len,
      a->scale * kLog2e, pl.P, pl.max_parts, ws_acc, ws_ml);
}

template <int D, int BS>
void launch_f32(const pa_decode_args* a, const Plan& pl, float* ws_acc, float* ws_ml,
                hipStream_t st) {
  const int G = a->num_q_heads / a->num_kv_heads;
  dim3 grid((unsigned)max(pl.max_parts, 1), (unsigned)a->num_q_heads, (unsigned)a->num_seqs);
  decode_f32_kernel<D, BS><<<grid, 64, 0, st>>>(
      (float*)a->out, (const float*)a->q, (const float*)a->k_cache, (const float*)a->v_cache,
      a->block_tables, a->context_lens, a->num_q_heads, a->num_kv_heads, G, a->num_blocks,
      a->max_blocks_per_seq, a->max_context_len, a->scale * kLog2e, pl.P, pl.max_parts, ws_acc,
      ws_ml);
}

template <typename Ty>
void launch_mfma_dims(const pa_decode_args* a, const Plan& pl, float* wa, float* wm,
                      hipStream_t st) {
  if (a->head_dim == 128) {
    if (a->block_size == 16) launch_mfma<Ty, 128, 16>(a, pl, wa, wm, st);
    else launch_mfma<Ty, 128, 32>(a, pl, wa, wm, st);
  } else {
    if (a->block_size == 16) launch_mfma<Ty, 64, 16>(a, pl, wa, wm, st);
    else launch_mfma<Ty, 64, 32>(a, pl, wa, wm, st);
  }
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" {

PA_API size_t pa_decode_workspace_bytes(const pa_decode_args* args) {
  if (validate(args) != PA_OK) return 0;
  return make_plan(args).ws_bytes;
}

PA_API int32_t pa_decode_partition_size(const pa_decode_args* args) {
  if (validate(args) != PA_OK) return -1;
  return make_plan(args).P;
}

PA_API pa_status pa_decode(const pa_decode_args* a, void* stream) {
  pa_status st = validate(a);
  if (st != PA_OK) return st;
  if (a->num_seqs == 0) return PA_OK;
  if (!aligned16(a->out) || !aligned16(a->q) || !aligned16(a->k_cache) ||
      !aligned16(a->v_cache) || !a->block_tables || !a->context_lens)
    return PA_ERR_INVALID;
  const Plan pl = make_plan(a);
  if (a->num_seqs > 65535 || (int64_t)a->num_kv_heads * pl.groups > 65535 ||
      a->num_q_heads > 65535)
    return PA_ERR_UNSUPPORTED;
  float* ws_acc = nullptr;
  float* ws_ml = nullptr;
  if (pl.ws_bytes) {
    if (!a->workspace || a->workspace_bytes < pl.ws_bytes || !aligned16(a->workspace))
      return PA_ERR_WORKSPACE;
    ws_acc = (float*)a->workspace;
    ws_ml = ws_acc + (size_t)a->num_seqs * a->num_q_heads * pl.max_parts * a->head_dim;
  }
  hipStream_t hs = (hipStream_t)stream;
  switch (a->dtype) {
    case PA_F16: launch_mfma_dims<F16>(a, pl, ws_acc, ws_ml, hs); break;
    case PA_BF16: launch_mfma_dims<BF16>(a, pl, ws_acc, ws_ml, hs); break;
    default:
      if (a->head_dim == 128) {
        if (a->block_size == 16) launch_f32<128, 16>(a, pl, ws_acc, ws_ml, hs);
        else launch_f32<128, 32>(a, pl, ws_acc, ws_ml, hs);
      } else {
        if (a->block_size == 16) launch_f32<64, 16>(a, pl, ws_acc, ws_ml, hs);
        else launch_f32<64, 32>(a, pl, ws_acc, ws_ml, hs);
      }
  }
  if ((st = launch_status()) != PA_OK) return st;
  if (pl.max_parts > 1) {
    dim3 grid((unsigned)a->num_q_heads, (unsigned)a->num_seqs);
    switch (a->dtype) {
      case PA_F16:
        merge_kernel<Out16<F16>><<<grid, a->head_dim, 0, hs>>>(
            (Out16<F16>*)a->out, a->context_lens, ws_acc, ws_ml, a->num_q_heads, a->head_dim,
            a->max_context_len, a->max_blocks_per_seq, a->block_size, pl.P, pl.max_parts);
        break;
      case PA_BF16:
        merge_kernel<Out16<BF16>><<<grid, a->head_dim, 0, hs>>>(
            (Out16<BF16>*)a->out, a->context_lens, ws_acc, ws_ml, a->num_q_heads, a->head_dim,
            a->max_context_len, a->max_blocks_per_seq, a->block_size, pl.P, pl.max_parts);
        break;
      default:
        merge_kernel<float><<<grid, a->head_dim, 0, hs>>>(
            (float*)a->out, a->context_lens, ws_acc, ws_ml, a->num_q_heads, a->head_dim,
            a->max_context_len, a->max_blocks_per_seq, a->block_size, pl.P, pl.max_parts);
    }
    if ((st = launch_status()) != PA_OK) return st;
  }
  return PA_OK;
}

}  // extern "C"
