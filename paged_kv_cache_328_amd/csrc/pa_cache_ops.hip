// Cache-maintenance kernels of libpagedattn: the slot-mapped cache write,
// copy-on-write block copies and the gather test hook, which are plain bit
// copies moved in 16-byte vectors, and the quantising write into INT8 pools.
//
// Pool layout (intelliparadigm.com, "vLLM的Paged Attention技术", section
// "2.2 内存布局优化"), x = 16 B / element size:
//   k_cache [NB, Hkv, D/x, BS, x]   -> a token's x-element chunk cc of head h in
//                                      block b starts at ((b*Hkv+h)*(D/x)+cc)*BS*x + o*x
//   v_cache [NB, Hkv, D, BS]         -> element d of that token at ((b*Hkv+h)*D+d)*BS + o
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

// One thread per (token, KV head, 16-byte chunk of the head's channels).
template <int ESIZE>
__global__ __launch_bounds__(256) void write_kv_kernel(const uint8_t* __restrict__ k_new,
                                                       const uint8_t* __restrict__ v_new,
                                                       uint8_t* __restrict__ k_cache,
                                                       uint8_t* __restrict__ v_cache,
                                                       const int64_t* __restrict__ slots, int T,
                                                       int Hkv, int D, int BS, int NB) {
  constexpr int X = 16 / ESIZE;
  const int chunks = D / X;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= (int64_t)T * Hkv * chunks) return;
  const int cc = (int)(item % chunks);
  const int h = (int)((item / chunks) % Hkv);
  const int t = (int)(item / chunks / Hkv);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= (int64_t)NB * BS) return;  // padding or out of the pool
  const int64_t b = slot / BS;
  const int o = (int)(slot % BS);
  const int64_t src = ((int64_t)t * Hkv + h) * D + (int64_t)cc * X;  // element offset
  const u32x4 kv = load16(k_new + src * ESIZE);
  const u32x4 vv = load16(v_new + src * ESIZE);
  const int64_t kdst = (((b * Hkv + h) * chunks + cc) * BS + o) * X;
  store16(k_cache + kdst * ESIZE, kv);
  const int64_t vrow = ((b * Hkv + h) * D + (int64_t)cc * X) * BS + o;
  if constexpr (ESIZE == 2) {
    uint16_t* vd = reinterpret_cast<uint16_t*>(v_cache);
#pragma unroll
    for (int e = 0; e < 8; ++e) vd[vrow + (int64_t)e * BS] = (uint16_t)(vv[e / 2] >> (16 * (e % 2)));
  } else {
    uint32_t* vd = reinterpret_cast<uint32_t*>(v_cache);
#pragma unroll
    for (int e = 0; e < 4; ++e) vd[vrow + (int64_t)e * BS] = vv[e];
  }
}

// grid: (16-byte vectors of one block's slab / 256, pairs, 2 pools)
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ k_cache,
                                                          uint8_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t slab_vec16, int NB) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= slab_vec16) return;
  const int src = pairs[2 * blockIdx.y], dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= NB || dst < 0 || dst >= NB) return;
  uint8_t* pool = blockIdx.z == 0 ? k_cache : v_cache;
  const int64_t slab = slab_vec16 * 16;
  store16(pool + dst * slab + i * 16, load16(pool + src * slab + i * 16));
}

// One thread per (seq, token, KV head, 16-byte chunk).
template <int ESIZE>
__global__ __launch_bounds__(256) void gather_kv_kernel(
    const uint8_t* __restrict__ k_cache, const uint8_t* __restrict__ v_cache,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
    uint8_t* __restrict__ k_out, uint8_t* __restrict__ v_out, int S, int Hkv, int D, int BS,
    int NB, int max_blocks, int max_ctx) {
  constexpr int X = 16 / ESIZE;
  const int chunks = D / X;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= (int64_t)S * max_ctx * Hkv * chunks) return;
  const int cc = (int)(item % chunks);
  const int h = (int)((item / chunks) % Hkv);
  const int t = (int)((item / chunks / Hkv) % max_ctx);
  const int s = (int)(item / chunks / Hkv / max_ctx);
  const int c = clampi(lens[s], 0, min(max_ctx, max_blocks * BS));
  if (t >= c) return;
  const int64_t b = clampi(tables[(int64_t)s * max_blocks + t / BS], 0, NB - 1);
  const int o = t % BS;
  const int64_t dst = (((int64_t)s * max_ctx + t) * Hkv + h) * D + (int64_t)cc * X;
  store16(k_out + dst * ESIZE, load16(k_cache + ((((b * Hkv + h) * chunks + cc) * BS + o) * X) * ESIZE));
  const int64_t vrow = ((b * Hkv + h) * D + (int64_t)cc * X) * BS + o;
  u32x4 v;
  if constexpr (ESIZE == 2) {
    const uint16_t* vs = reinterpret_cast<const uint16_t*>(v_cache);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (uint32_t)vs[vrow + (int64_t)(2 * e) * BS] | ((uint32_t)vs[vrow + (int64_t)(2 * e + 1) * BS] << 16);
  } else {
    const uint32_t* vs = reinterpret_cast<const uint32_t*>(v_cache);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = vs[vrow + (int64_t)e * BS];
  }
  store16(v_out + dst * ESIZE, v);
}

// Quantising cache write into 8-bit pools: one wave per (token, KV head); the
// wave quantises the K row, then the V row.  A row x (widened exactly to
// fp32) gets scale = max|x| / Code::kMax and codes Code::encode(x / scale)
// (INT8: rint clamped to [-127, 127]; FP8: nearest E4M3, ties to even,
// saturating), all in fp32 with correctly rounded division; a zero row gets
// scale 0 and zero codes.  Per (block, KV head) tile: K codes
// [D/16][BS][16], or V codes [D][BS], then BS fp32 scales.
template <typename Src>
__device__ inline float load_src(const void* p, int64_t i) {
  if constexpr (std::is_same<Src, float>::value) return reinterpret_cast<const float*>(p)[i];
  else return Src::to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

template <typename Src, typename Code>
__global__ __launch_bounds__(256) void write_kv_q8_kernel(const void* __restrict__ k_new,
                                                          const void* __restrict__ v_new,
                                                          uint8_t* __restrict__ k_cache,
                                                          uint8_t* __restrict__ v_cache,
                                                          const int64_t* __restrict__ slots,
                                                          int T, int Hkv, int D, int BS, int NB) {
  const int64_t item = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (item >= (int64_t)T * Hkv) return;
  const int h = (int)(item % Hkv);
  const int t = (int)(item / Hkv);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= (int64_t)NB * BS) return;  // padding or out of the pool
  const int64_t b = slot / BS;
  const int o = (int)(slot % BS);
  const int64_t tile = (int64_t)D * BS + 4 * BS;
  const int64_t src = ((int64_t)t * Hkv + h) * D;
  for (int kv = 0; kv < 2; ++kv) {
    const void* x = kv == 0 ? k_new : v_new;
    uint8_t* dst = (kv == 0 ? k_cache : v_cache) + (b * Hkv + h) * tile;
    float am = 0.f;
    for (int d = lane; d < D; d += 64) {
      const float a = fabsf(load_src<Src>(x, src + d));
      am = a > am ? a : am;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float other = __shfl_xor(am, off);
      am = other > am ? other : am;
    }
    const float sc = am / Code::kMax;
    for (int d = lane; d < D; d += 64) {
      const uint32_t code = sc != 0.f ? Code::encode(load_src<Src>(x, src + d) / sc) : 0u;
      const int64_t off = kv == 0 ? ((int64_t)(d / 16) * BS + o) * 16 + d % 16 : (int64_t)d * BS + o;
      dst[off] = (uint8_t)code;
    }
    if (lane == 0) *reinterpret_cast<float*>(dst + (int64_t)D * BS + 4 * o) = sc;
  }
}

inline unsigned grid1d(int64_t n) { return (unsigned)((n + 255) / 256); }
// whether n items at 256 per workgroup fit a 1-D grid
inline bool fits1d(int64_t n) { return (n + 255) / 256 <= 0x7FFFFFFF; }

}  // namespace
}  // namespace pa

using namespace pa;

// The quantising write for 8-bit pools of code format Code.
template <typename Code>
pa_status write_kv_q8(const void* k_new, const void* v_new, int32_t src_dtype, void* k_cache,
                      void* v_cache, const int64_t* slot_mapping, int32_t num_tokens,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, void* stream) {
  if (!elem_bytes(src_dtype)) return PA_ERR_INVALID;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID;
  if (head_dim % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !slot_mapping)
    return PA_ERR_INVALID;
  const int64_t waves = (int64_t)num_tokens * num_kv_heads;
  if ((waves + 3) / 4 > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  hipStream_t st = (hipStream_t)stream;
  uint8_t* kc = (uint8_t*)k_cache;
  uint8_t* vc = (uint8_t*)v_cache;
  switch (src_dtype) {
    case PA_F16:
      write_kv_q8_kernel<F16, Code><<<grid, 256, 0, st>>>(k_new, v_new, kc, vc, slot_mapping,
                                                          num_tokens, num_kv_heads, head_dim,
                                                          block_size, num_blocks);
      break;
    case PA_BF16:
      write_kv_q8_kernel<BF16, Code><<<grid, 256, 0, st>>>(k_new, v_new, kc, vc, slot_mapping,
                                                           num_tokens, num_kv_heads, head_dim,
                                                           block_size, num_blocks);
      break;
    default:
      write_kv_q8_kernel<float, Code><<<grid, 256, 0, st>>>(k_new, v_new, kc, vc, slot_mapping,
                                                            num_tokens, num_kv_heads, head_dim,
                                                            block_size, num_blocks);
      break;
  }
  return launch_status();
}

extern "C" {

PA_API pa_status pa_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t dtype, void* stream) {
  const int es = elem_bytes(dtype);
  if (!es) return PA_ERR_INVALID;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID;
  if (head_dim % (16 / es) != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !slot_mapping)
    return PA_ERR_INVALID;
  const int64_t items = (int64_t)num_tokens * num_kv_heads * (head_dim / (16 / es));
  if (!fits1d(items)) return PA_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  if (es == 2)
    write_kv_kernel<2><<<grid1d(items), 256, 0, st>>>(
        (const uint8_t*)k_new, (const uint8_t*)v_new, (uint8_t*)k_cache, (uint8_t*)v_cache,
        slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, num_blocks);
  else
    write_kv_kernel<4><<<grid1d(items), 256, 0, st>>>(
        (const uint8_t*)k_new, (const uint8_t*)v_new, (uint8_t*)k_cache, (uint8_t*)v_cache,
        slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, num_blocks);
  return launch_status();
}

PA_API pa_status pa_write_kv_i8(const void* k_new, const void* v_new, int32_t src_dtype,
                                void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t num_blocks, void* stream) {
  return write_kv_q8<I8Code>(k_new, v_new, src_dtype, k_cache, v_cache, slot_mapping, num_tokens,
                             num_kv_heads, head_dim, block_size, num_blocks, stream);
}

PA_API pa_status pa_write_kv_fp8(const void* k_new, const void* v_new, int32_t src_dtype,
                                 void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, void* stream) {
  return write_kv_q8<Fp8Code>(k_new, v_new, src_dtype, k_cache, v_cache, slot_mapping, num_tokens,
                              num_kv_heads, head_dim, block_size, num_blocks, stream);
}

PA_API pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                                int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t num_blocks, int32_t dtype,
                                void* stream) {
  const bool i8 = dtype == PA_I8 || dtype == PA_FP8;  // 8-bit tiles: codes, then scales
  const int es = elem_bytes(dtype);
  if (!es && !i8) return PA_ERR_INVALID;
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID;
  if (head_dim % (i8 ? 16 : 16 / es) != 0) return PA_ERR_UNSUPPORTED;
  if (i8 && block_size % 4 != 0) return PA_ERR_UNSUPPORTED;  // whole 16-byte vectors per tile
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > 65535) return PA_ERR_UNSUPPORTED;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !block_mapping) return PA_ERR_INVALID;
  // bytes of one block of one pool: every KV head's tile (INT8: codes, then scales)
  const int64_t slab = i8 ? (int64_t)num_kv_heads * ((int64_t)head_dim * block_size + 4 * block_size)
                          : (int64_t)num_kv_heads * head_dim * block_size * es;
  const int64_t slab_vec16 = slab / 16;
  dim3 grid(grid1d(slab_vec16), (unsigned)num_pairs, 2);
  copy_blocks_kernel<<<grid, 256, 0, (hipStream_t)stream>>>((uint8_t*)k_cache, (uint8_t*)v_cache,
                                                            block_mapping, slab_vec16, num_blocks);
  return launch_status();
}

PA_API pa_status pa_gather_kv(const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              void* k_out, void* v_out, int32_t num_seqs, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_context_len, int32_t dtype,
                              void* stream) {
  if (dtype == PA_I8 || dtype == PA_FP8) return PA_ERR_UNSUPPORTED;
  const int es = elem_bytes(dtype);
  if (!es) return PA_ERR_INVALID;
  if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return PA_ERR_INVALID;
  if (head_dim % (16 / es) != 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_context_len == 0) return PA_OK;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_out) || !aligned16(v_out) ||
      !block_tables || !context_lens)
    return PA_ERR_INVALID;
  const int64_t items = (int64_t)num_seqs * max_context_len * num_kv_heads * (head_dim / (16 / es));
  if (!fits1d(items)) return PA_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  if (es == 2)
    gather_kv_kernel<2><<<grid1d(items), 256, 0, st>>>(
        (const uint8_t*)k_cache, (const uint8_t*)v_cache, block_tables, context_lens,
        (uint8_t*)k_out, (uint8_t*)v_out, num_seqs, num_kv_heads, head_dim, block_size,
        num_blocks, max_blocks_per_seq, max_context_len);
  else
    gather_kv_kernel<4><<<grid1d(items), 256, 0, st>>>(
        (const uint8_t*)k_cache, (const uint8_t*)v_cache, block_tables, context_lens,
        (uint8_t*)k_out, (uint8_t*)v_out, num_seqs, num_kv_heads, head_dim, block_size,
        num_blocks, max_blocks_per_seq, max_context_len);
  return launch_status();
}

}  // extern "C"
