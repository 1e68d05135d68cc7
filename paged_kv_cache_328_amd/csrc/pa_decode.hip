// Paged attention for gfx950: decode pass 1 (per-partition attention over the
// block table), pass 2 (log-sum-exp merge of the partitions), and paged
// (chunked) prefill.  pa_decode_prefix runs the prefill body (as a
// shared-prefix pass) and the decode body in one launch, then the merge.
//
// What is computed: for sequence s and query head h, the softmax attention of
// q[s,h] over the sequence's cached keys/values, which sit in fixed-size
// physical blocks reached through the block table (wiblog.cn, "AI 推理系列
// （十六）：PagedAttention", sections "PagedAttention 如何把连续序列映射到离散显存块"
// and "非连续 KV 为什么需要专门的 Attention Kernel"; the attention formula itself
// is the ordinary one).  Long contexts are split into partitions (the
// PARTITION_SIZE split of intelliparadigm.com, "vLLM的Paged Attention技术",
// sections 3.1 and 3.2); each partition writes (max, sum, unnormalised
// output) and pass 2 merges them exactly: M = max_p m_p, out = sum_p
// 2^(m_p-M) acc_p / sum_p 2^(m_p-M) l_p (logits are kept in base 2:
// x * scale * log2(e)).
//
// Pool layout (intelliparadigm.com, section "2.2 内存布局优化"), 16-bit types,
// x = 8:
//   K [NB, Hkv, D/8, BS, 8]: for a fixed 8-channel chunk, the BS tokens of a
//     block are consecutive 16-byte vectors;
//   V [NB, Hkv, D, BS]:      for a fixed channel, the BS tokens are consecutive.
// Both products run on the gfx950 matrix instruction
// v_mfma_f32_16x16x32_{f16,bf16} (lane l feeds row/column l%16 and 8
// consecutive reduction-dimension elements 8*(l/16)..+7; the 16x16 result
// leaves rows 4*(l/16)..+3 of column l%16 in lane l):
//   QK:  S[token][head] = K[token][d] x Q^T[d][head], reduction over d.  Row i
//        of a 16-token tile is token i, so for one 8-channel chunk the 16
//        lanes of a row group read 16 consecutive 16-byte vectors: 256
//        contiguous bytes, whole cache lines.  A 32-token chunk is two tiles.
//   PV:  O^T[d][head] += V^T[d][k] x P^T[k][head], reduction over the 32
//        tokens of a chunk, k = token.  Lane l's V operand is tokens
//        8*(l/16)..+7 of channel l%16 (one 16-byte load).  The QK result
//        leaves lane row g = l/16 with tokens 4g..4g+3 and 16+4g..16+4g+3;
//        two lane-row swaps (v_permlane32_swap, then v_permlane16_swap) of
//        the packed weights regroup them to tokens 8g..8g+7.
// The running max / sum of head l%16 stays lane-local apart from one
// reduction over the 4 row groups of the wave.
//
// Decode work decomposition: one workgroup of NW waves per (KV head, group
// of up to 16 query heads sharing that KV head, partition, sequence).  The
// group's query heads are the N = 16 dimension of both products, so K/V
// bytes are read once per KV head whatever the group size G is.  The
// partition is cut into chunks of 32 tokens dealt round-robin to the waves
// (the warp-to-block assignment of intelliparadigm.com, section "4.2
// 动态负载均衡"); each wave keeps its own running (max, sum, output) and the
// waves are merged through LDS at the end.
//
// Prefill: one workgroup per (tile of 64 NC (row, head) slots, KV head,
// sequence) walks the keys in 32-token chunks staged through LDS; every wave
// computes its own slots' columns against each staged chunk.
//
// INT8 caches (codes plus one fp32 scale per token and KV head, in the block
// tile): the codes are widened exactly to the query type for the same
// products, the K scale multiplies the logit and the V scale the weight.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 32;          // tokens per step of the 16-bit kernel
constexpr int kMaxF32Part = 1024;   // largest partition of the fp32 kernel
constexpr float kSlack = 8.f;       // base-2 headroom of the 16-bit kernel's running max
constexpr int kXcds = 8;            // accelerator dies (each with its own L2) of an MI355X

__device__ __forceinline__ u32x2 load8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// Work unit `u` of a flat (sequence, partition) list in which sequence s owns
// max(1, ceil(c_s / P)) consecutive units (an empty context still gets one,
// which writes its zero output).  Each lane reads one context length per
// round of 64 sequences; an inclusive wave prefix sum finds the owner.
// Returns false when u is past the last unit.  All results (s, p and the
// clamped context length c_s) are wave-uniform.
__device__ __forceinline__ bool flat_unit(const int32_t* __restrict__ lens, int S, int cmax,
                                         int P, int u, int lane, int& s, int& p, int& c_s) {
  int base = 0;
  for (int s0 = 0; s0 < S; s0 += kWave) {
    const int sl = s0 + lane;
    const int c = sl < S ? clampi(lens[sl], 0, cmax) : 0;
    const int own = sl < S ? max((c + P - 1) / P, 1) : 0;
    int incl = own;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const int total = __shfl(incl, kWave - 1);
    if (u < base + total) {
      const uint64_t hit = __ballot(incl > u - base);
      const int first = __ffsll((unsigned long long)hit) - 1;  // lowest lane holding unit u
      s = uniform(s0 + first);
      p = uniform(u - base - (__shfl(incl, first) - __shfl(own, first)));
      c_s = uniform(__shfl(c, first));
      return true;
    }
    base += total;
  }
  return false;
}

// The flat work list in an order the host chose from its copy of the context
// lengths: entry j (packed s | p << 16) is the (sequence, partition) unit of
// grid row j.  Passed by value as a kernel argument; n = 0 means no list (the
// kernel finds its unit with flat_unit, in sequence order).
constexpr int kMaxUnits = 512;
struct UnitList {
  int32_t n;
  uint32_t e[kMaxUnits];
};

// Running state of a log-sum-exp merge: max m, sum l, unnormalised output o
// (4 channels).  Adding partition (m', l', o') with M = max(m, m'):
// l <- l 2^(m-M) + l' 2^(m'-M), o likewise, m <- M.
struct Lse {
  float m, l;
  f32x4 o;
};

// Adds a partition (m, l, o) to a running state (online log-sum-exp).
__device__ __forceinline__ void lse_add(Lse& st, float m, float l, f32x4 o) {
  const float mn = fmaxf(st.m, m);
  const float a = exp2_fast(st.m - mn);  // 0 while the state is empty
  const float b = exp2_fast(m - mn);
  st.l = st.l * a + l * b;
  st.o = st.o * a + o * b;
  st.m = mn;
}

// K/V are streamed: every byte is read once per step, so the loads are
// non-temporal (they do not displace reusable lines in the caches); this is
// worth several percent of HBM bandwidth on these scattered 4-8 KiB tiles.
__device__ __forceinline__ u32x4 stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 stream8(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// V rows of a 64-token block are longer than one 32-token chunk: a chunk
// reads half of each row (64 of 128 bytes for 16-bit values, 32 of 64 for
// INT8 codes) and the sibling chunk, on another wave at about the same time,
// reads the other half.  Those loads are kept ordinary so the line stays in
// L2 for the sibling: measured on MI355X (LLaMA-13B-shaped step at block
// size 64), non-temporal V loads fetched 1.23x the algorithmic bytes and
// took 82.9 us, ordinary ones 74.4 us.  Other block sizes read whole lines.
template <int BS>
__device__ __forceinline__ u32x4 v_row16(const void* p) {
  if constexpr (BS > kChunk) return load16(p);
  else return stream16(p);
}
template <int BS>
__device__ __forceinline__ u32x2 v_row8(const void* p) {
  if constexpr (BS > kChunk) return load8(p);
  else return stream8(p);
}

__device__ __forceinline__ uint32_t stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ float stream_f1(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const float*>(p));
}

// 8-bit codes (INT8, or FP8 with an Fp8Elem type) -> 16-bit operand values
// (8 codes, exact: Ty::codes4).
template <typename Ty>
__device__ __forceinline__ u32x4 codes_to_operand(u32x2 c) {
  const u32x2 a = Ty::codes4(c[0]), b = Ty::codes4(c[1]);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// INT8 tile of one (block, KV head): D*BS codes (K: [D/16][BS][16], V:
// [D][BS]), then BS fp32 scales, one per token.
template <int D, int BS>
struct I8Tile {
  static constexpr int kBytes = D * BS + 4 * BS;
  static constexpr int kScales = D * BS;  // byte offset of the scales
};

// ----------------------------------------------------------------------------
// 16-bit pass 1 (matrix cores).
// grid: x = KV head * n_groups + group, y = partition, z = sequence;
// block = 64 * NW threads; dynamic LDS = merge_lds_bytes(NW, G, D).
// Partitions beyond a sequence's context exit at once.  Neighbouring
// workgroups are the KV heads of one (sequence, partition): they read the
// adjacent head tiles of the same physical blocks.
// ----------------------------------------------------------------------------
// Raw K / V operand registers of one 32-token chunk: 16-bit elements, or
// (KV8) INT8 codes plus the scales of the lane's 8 tokens.
// Tokens of a chunk are numbered 0..31; tile 0 is tokens 0..15, tile 1 tokens
// 16..31.  K operands hold token i of each tile; V operands hold tokens
// 8*g4..8*g4+7 of one channel.
template <int KK, int MM, bool KV8>
struct Raw {
  u32x4 k[2][KK];  // channels 8*(4*kk+g4)..+8 of tile-0 / tile-1 token i
  u32x4 v[MM];     // channel 16*mm + i, tokens 8*g4..+8
};
template <int KK, int MM>
struct Raw<KK, MM, true> {
  u32x2 k[2][KK];  // 8 codes of tile-0 / tile-1 token i, channels 8*m..+8 with
                   // m = 8*(kk/2) + 2*g4 + kk%2 (half kk%2 of one 16-byte x-vector)
  u32x2 v[MM];     // 8 codes: channel 16*mm + i, tokens 8*g4..+8
  float sc;        // lane L < 32: K scale of the chunk's token L; else V scale of token L - 32
};

// Block id j (0 <= j < N) of a chunk's N wave-uniform block ids, for a
// lane-dependent j.  The ids are taken as values (readfirstlane of a uniform
// value is the value): written as a lookup in the array, the compiler turned
// the selects into an indexed load, which left the array in scratch memory.
template <int N>
__device__ __forceinline__ int pick_block(const int (&b)[N], int j) {
  int id = b[0];
#pragma unroll
  for (int t = 1; t < N; ++t) id = j == t ? __builtin_amdgcn_readfirstlane(b[t]) : id;
  return id;
}

// The block-table side of one wave's walk over 32-token chunks, shared by
// the decoders below (Derived supplies RawT, issue and consume): the block
// ids of the coming chunks are held one per lane, a batch fetched by one
// vector load before the first K/V load is issued, so no chunk waits on a
// table read (a chunk whose block ids came from a load in the loop would
// also wait for every K/V load issued before that read).
template <typename Derived, int BS>
struct ChunkWalker {
  static constexpr int BPC = BS >= kChunk ? 1 : kChunk / BS;  // blocks per chunk
  static constexpr int CPB = 64 / BPC;                         // chunks per batch of block ids
  int tbl = 0;  // block ids of the current batch (lane e: entry e)

  // Loads the table entries of the chunks ch(k0), ch(k0 + 1), ... (ch(k) =
  // c0 + stride * k), one block id per lane: lane e holds block e % BPC of
  // the chunk k0 + e / BPC.  Entries past the cached range [0, cc) or past
  // n_chunks are not read (id 0 stands in; those tokens are dropped).
  __device__ __forceinline__ void load_batch(const int32_t* __restrict__ trow, int t_begin,
                                             int n_chunks, int cc, int NB, int c0, int stride,
                                             int k0) {
    const int lane = threadIdx.x & 63;
    const int ch = c0 + stride * (k0 + lane / BPC);
    const int t = t_begin + ch * kChunk + (lane % BPC) * BS;
    tbl = ch < n_chunks && t < cc ? clampi(trow[t / BS], 0, NB - 1) : 0;
  }

  // Physical blocks of the k-th chunk of the current walk, in token order
  // (one block when BS >= 32); a new batch is loaded every CPB chunks.
  __device__ __forceinline__ void block_ids(int k, int (&b)[BPC], const int32_t* __restrict__ trow,
                                            int t_begin, int n_chunks, int cc, int NB, int c0,
                                            int stride) {
    if (k > 0 && k % CPB == 0) load_batch(trow, t_begin, n_chunks, cc, NB, c0, stride, k);
    const int e = (k % CPB) * BPC;
#pragma unroll
    for (int j = 0; j < BPC; ++j) b[j] = __builtin_amdgcn_readlane(tbl, e + j);
  }

  // Streams the chunks k = 0 .. n - 1 of a walk (chunk k starts at token
  // t0_of(k); ids(k, b) gives its block ids, reading the table in batches).
  // All loads of a chunk are issued before any of them is used: the
  // scheduling barrier keeps the compiler from interleaving the products
  // with the loads.  AHEAD: the loads of chunk k + 1 are issued before chunk
  // k is consumed.  The compiler turns `cur = nxt` into register copies,
  // which wait for those loads at the end of the iteration, so in effect one
  // chunk is in flight while the previous one is computed.  Measured on
  // MI355X, this form at 218 VGPRs (two waves per SIMD) beat two register
  // sets used in turn (no copies, two chunks really in flight): 264 VGPRs
  // and one wave per SIMD, 70.0 against 63.8 us on the LLaMA-13B-shaped
  // step; capped at 256 VGPRs that form spills and took 76 us.
  template <bool AHEAD, typename T0, typename Ids>
  __device__ __forceinline__ void walk(int n, T0 t0_of, Ids ids, int cc, int skip) {
    Derived& d = static_cast<Derived&>(*this);
    using RawT = typename Derived::RawT;
    if (n <= 0) return;
    int nb[BPC] = {};
    ids(0, nb);
    if constexpr (AHEAD) {
      RawT cur, nxt;
      d.issue(nb, t0_of(0), cur);
      if (n > 1) ids(1, nb);
      for (int k = 0; k < n; ++k) {
        if (k + 1 < n) {
          d.issue(nb, t0_of(k + 1), nxt);
          if (k + 2 < n) ids(k + 2, nb);
        }
        __builtin_amdgcn_sched_barrier(0);
        d.consume(t0_of(k), cur, cc, skip);
        cur = nxt;
      }
    } else {
      for (int k = 0; k < n; ++k) {
        RawT one;
        d.issue(nb, t0_of(k), one);
        if (k + 1 < n) ids(k + 1, nb);
        __builtin_amdgcn_sched_barrier(0);
        d.consume(t0_of(k), one, cc, skip);
      }
    }
  }

  // The same walk with one register set and the loads of chunk k + 1 split
  // around chunk k's products: its K loads go out as soon as chunk k's QK
  // product has read the K registers, its V loads once the PV product has
  // read the V registers.  Loads are then in flight while the wave computes,
  // without the second register set of walk<true> (Derived supplies
  // issue_k / issue_v and consume_k / consume_v).
  template <typename T0, typename Ids>
  __device__ __forceinline__ void walk_skew(int n, T0 t0_of, Ids ids, int cc, int skip) {
    Derived& d = static_cast<Derived&>(*this);
    using RawT = typename Derived::RawT;
    if (n <= 0) return;
    int nb[BPC] = {};
    ids(0, nb);
    RawT r;
    d.issue_k(nb, t0_of(0), r);
    d.issue_v(nb, t0_of(0), r);
    for (int k = 0; k < n; ++k) {
      const bool more = k + 1 < n;
      if (more) ids(k + 1, nb);
      float x[8], sv[8];
      __builtin_amdgcn_sched_barrier(0);
      d.consume_k(t0_of(k), r, cc, skip, x, sv);
      __builtin_amdgcn_sched_barrier(0);
      if (more) d.issue_k(nb, t0_of(k + 1), r);
      __builtin_amdgcn_sched_barrier(0);
      d.consume_v(t0_of(k), r, cc, x, sv);
      __builtin_amdgcn_sched_barrier(0);
      if (more) d.issue_v(nb, t0_of(k + 1), r);
    }
  }
};

// One wave's share of the decode pass: q held as the B operand of both
// products, the running (max, sum, output) of the 16 columns (query heads
// i = lane % 16 of a group), the block ids of its coming chunks, and the
// per-chunk steps:
//   issue    -- every K and V load of one 32-token chunk (per lane: 2 x KK
//               16-byte K vectors and MM 16-byte V rows, or for INT8 codes
//               2 x KK/2 16-byte K vectors, MM 8-byte V rows and one scale);
//   consume  -- both products and the online-softmax update for that chunk;
//   add_token -- the fused append's new token, on the vector ALU.
// Token tau of a chunk (0..31) sits in block tau / BS of the chunk at row
// tau % BS; a block of 64 tokens holds the whole chunk from row t0 % 64.
template <typename Ty, int D, int BS, bool KV8>
struct WaveDecoder : ChunkWalker<WaveDecoder<Ty, D, BS, KV8>, BS> {
  static_assert(BS == 8 || BS == 16 || BS == 32 || BS == 64, "block size 8, 16, 32 or 64");
  static_assert(D % 32 == 0, "head_dim multiple of 32");
  using V8 = typename Ty::vec8;
  static constexpr int KK = D / 32;  // QK products along head_dim (32 channels each)
  static constexpr int MM = D / 16;  // PV products along head_dim (16 channels each)
  // one (block, KV head) tile: D*BS 16-bit elements, or an INT8 tile (bytes)
  static constexpr int TILE = KV8 ? I8Tile<D, BS>::kBytes : D * BS;
  static constexpr int BPC = BS >= kChunk ? 1 : kChunk / BS;  // blocks per chunk
  static constexpr int CPB = 64 / BPC;                         // chunks per batch of block ids
  using Elem = typename std::conditional<KV8, uint8_t, uint16_t>::type;
  using RawT = Raw<KK, MM, KV8>;

  const Elem* kc;
  const Elem* vc;
  int lane, i, g4;     // lane; row (A operand) / column (B operand, output); reduction slice
  int64_t blk_stride;  // elements (bytes for INT8) from one block to the next
  int64_t head_off;    // offset of the KV head's tile inside a block
  float scale_log2;
  V8 qop[KK];          // Q^T operand: head i, channels 8*qchunk(kk)..+8
  f32x4 acc[MM];       // O^T[d = 16*mm + 4*g4 + j][head i]
  float m_run;         // running max of the base-2 logits (head i)
  float l_run;         // this lane's share of the running sum

  __device__ __forceinline__ WaveDecoder(const void* kcv, const void* vcv, int Hkv, float sl2)
      : kc(reinterpret_cast<const Elem*>(kcv)), vc(reinterpret_cast<const Elem*>(vcv)),
        lane(threadIdx.x & 63), i(threadIdx.x & 15), g4((threadIdx.x & 63) >> 4),
        blk_stride((int64_t)Hkv * TILE), head_off(0), scale_log2(sl2) {}

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) acc[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  }

  // Channels 8*m..+8 of the K operand that product kk meets (m = 4*kk + g4;
  // INT8: 8*(kk/2) + 2*g4 + kk%2, so that one 16-byte load of codes feeds
  // two products).
  __device__ __forceinline__ int qchunk(int kk) const {
    return KV8 ? 8 * (kk >> 1) + 2 * g4 + (kk & 1) : 4 * kk + g4;
  }

  // q row of this lane's column (zeros for a column past the group).
  __device__ __forceinline__ void load_q(const uint16_t* __restrict__ qrow, bool head_ok) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 raw = head_ok ? load16(qrow + 8 * qchunk(kk)) : u32x4{0u, 0u, 0u, 0u};
      qop[kk] = __builtin_bit_cast(V8, raw);
    }
  }

  // Tile offset and row of token tau (0..31) of the chunk at token t0.
  __device__ __forceinline__ void token_at(const int (&b)[BPC], int t0, int tau, int64_t& off,
                                           int& row) const {
    const int id = pick_block<BPC>(b, tau / BS);
    off = (int64_t)id * blk_stride + head_off;
    row = BS >= kChunk ? (BS > kChunk ? t0 % BS : 0) + tau : tau % BS;
  }

  // The chunk's K loads (INT8: and its K and V scales).
  __device__ __forceinline__ void issue_k(const int (&b)[BPC], int t0, RawT& r) const {
    int64_t ok0, ok1;
    int rk0, rk1;
    token_at(b, t0, i, ok0, rk0);       // K operand of tile 0: token i
    token_at(b, t0, 16 + i, ok1, rk1);  // tile 1: token 16 + i
    if constexpr (!KV8) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        r.k[0][kk] = stream16(kc + ok0 + ((4 * kk + g4) * BS + rk0) * 8);
        r.k[1][kk] = stream16(kc + ok1 + ((4 * kk + g4) * BS + rk1) * 8);
      }
    } else {
      // K codes: one 16-byte x-vector 4*k2 + g4 (channels 16*(4*k2+g4)..+16)
      // of the token's row feeds products 2*k2 and 2*k2 + 1.
#pragma unroll
      for (int k2 = 0; k2 < KK / 2; ++k2) {
        const u32x4 a = stream16(kc + ok0 + ((4 * k2 + g4) * BS + rk0) * 16);
        const u32x4 c = stream16(kc + ok1 + ((4 * k2 + g4) * BS + rk1) * 16);
        r.k[0][2 * k2] = u32x2{a[0], a[1]};
        r.k[0][2 * k2 + 1] = u32x2{a[2], a[3]};
        r.k[1][2 * k2] = u32x2{c[0], c[1]};
        r.k[1][2 * k2 + 1] = u32x2{c[2], c[3]};
      }
      // Scales: one per lane (the chunk's 32 K scales, then its 32 V
      // scales); consume hands each lane the ones it needs by lane shuffles,
      // which keeps one register per chunk in flight instead of sixteen.
      constexpr int SC = I8Tile<D, BS>::kScales;
      int64_t osc;
      int rsc;
      token_at(b, t0, lane & 31, osc, rsc);
      r.sc = stream_f1((lane < 32 ? kc : vc) + osc + SC + 4 * rsc);
    }
  }

  // The chunk's V loads: the V^T operand, tokens 8*g4..+8 (one block row).
  __device__ __forceinline__ void issue_v(const int (&b)[BPC], int t0, RawT& r) const {
    int64_t ov;
    int rv;
    token_at(b, t0, 8 * g4, ov, rv);
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) {
      if constexpr (!KV8) r.v[mm] = v_row16<BS>(vc + ov + (16 * mm + i) * BS + rv);
      else r.v[mm] = v_row8<BS>(vc + ov + (16 * mm + i) * BS + rv);
    }
  }

  __device__ __forceinline__ void issue(const int (&b)[BPC], int t0, RawT& r) const {
    issue_k(b, t0, r);
    issue_v(b, t0, r);
  }

  // Both products and the online-softmax update for the chunk at token t0;
  // tokens outside [skip, cc) are dropped.  In two halves: consume_k (the QK
  // product, which reads r.k and r.sc) and consume_v (softmax update and PV
  // product, which reads r.v), so that a walk may reload r.k between them.
  __device__ __forceinline__ void consume(int t0, RawT& r, int cc, int skip) {
    float x[8], sv[8];
    consume_k(t0, r, cc, skip, x, sv);
    consume_v(t0, r, cc, x, sv);
  }

  // x[e]: base-2 logit for head i of token t0 + 4*g4 + e (e < 4) or
  // t0 + 16 + 4*g4 + e - 4 (e >= 4), the reduction index 8*g4 + e of the PV
  // product; -inf for a dropped token.  INT8: sv[e] is that token's V scale
  // (0 for a dropped token).
  __device__ __forceinline__ void consume_k(int t0, const RawT& r, int cc, int skip, float (&x)[8],
                                            float (&sv)[8]) const {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if constexpr (!KV8) {
        s0 = Ty::mma(__builtin_bit_cast(V8, r.k[0][kk]), qop[kk], s0);
        s1 = Ty::mma(__builtin_bit_cast(V8, r.k[1][kk]), qop[kk], s1);
      } else {
        s0 = Ty::mma(__builtin_bit_cast(V8, codes_to_operand<Ty>(r.k[0][kk])), qop[kk], s0);
        s1 = Ty::mma(__builtin_bit_cast(V8, codes_to_operand<Ty>(r.k[1][kk])), qop[kk], s1);
      }
    }
    // INT8: V scales of this lane's tokens 4*g4 + (e & 3) + 16 * (e >> 2)
    if constexpr (KV8) {  // logits of INT8 keys: code dot q times the token's scale
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s0[j] *= __shfl(r.sc, 4 * g4 + j);
        s1[j] *= __shfl(r.sc, 16 + 4 * g4 + j);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = __shfl(r.sc, 32 + 16 * (e >> 2) + 4 * g4 + (e & 3));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = s0[j] * scale_log2;
      x[4 + j] = s1[j] * scale_log2;
    }
    if (t0 + kChunk > cc || t0 < skip) {  // drop tokens outside [skip, cc) by select
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = t0 + 4 * g4 + (e & 3) + 16 * (e >> 2);
        if (tok >= cc || tok < skip) x[e] = -INFINITY;
      }
      if constexpr (KV8) {  // and their V scales (codes are finite; a scale may be NaN)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (x[e] == -INFINITY) sv[e] = 0.f;
      }
    }
  }

  // The online-softmax update with the logits x (and INT8 V scales sv) of
  // consume_k, and the PV product over r.v.
  __device__ __forceinline__ void consume_v(int t0, RawT& r, int cc, const float (&x)[8],
                                            const float (&sv)[8]) {
    if constexpr (!KV8) {
      if (t0 + kChunk > cc) {  // zero the V bits of tokens past cc (they may hold NaN)
        uint32_t keep[4];      // V word wd holds tokens t0 + 8*g4 + 2*wd, +1
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
          keep[wd] = (t0 + 8 * g4 + 2 * wd < cc ? 0x0000FFFFu : 0u) |
                     (t0 + 8 * g4 + 2 * wd + 1 < cc ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int mm = 0; mm < MM; ++mm)
#pragma unroll
          for (int wd = 0; wd < 4; ++wd) r.v[mm][wd] &= keep[wd];
      }
    } else if constexpr (kFp8Codes<Ty>) {
      if (t0 + kChunk > cc) {  // zero the codes of tokens past cc (an unwritten slot may hold NaN)
        const uint32_t keep0 = bytes_before(t0 + 8 * g4, cc), keep1 = bytes_before(t0 + 8 * g4 + 4, cc);
#pragma unroll
        for (int mm = 0; mm < MM; ++mm) {
          r.v[mm][0] &= keep0;
          r.v[mm][1] &= keep1;
        }
      }
    }

    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // The reference m_run moves only when some head's chunk maximum passes it
    // by more than kSlack: the weights then stay below 2^kSlack, and on most
    // chunks the rescaling of the sums and accumulators is skipped.  The
    // branch is wave-uniform.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      // 0 on the column's first kept key; 1 while the column has none yet
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) acc[mm] *= alpha;
    }

    // A column whose keys were all dropped so far keeps m_run = -inf; its
    // weights must come out 0, not 2^(-inf + inf).
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    uint32_t pw[4];
    float psum = 0.f;
    if constexpr (!KV8) {
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        pw[wd] = Ty::pack2(exp2_fast(x[2 * wd] - m_use), exp2_fast(x[2 * wd + 1] - m_use));
        psum += Ty::lo_f32(pw[wd]) + Ty::hi_f32(pw[wd]);  // the weights the PV product sees
      }
    } else {
      // INT8 values: the PV product sees weight * V scale per token (the
      // scale varies along the reduction, so it rides on the weight).  The
      // sum takes the weights the product sees, rounded(p * s) / s, so that
      // the output stays a convex combination of the cached values (a token
      // with scale 0 has values 0 and counts with its weight p).
      float pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pr[e] = exp2_fast(x[e] - m_use);
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const float sa = sv[2 * wd], sb = sv[2 * wd + 1];
        pw[wd] = Ty::pack2(pr[2 * wd] * sa, pr[2 * wd + 1] * sb);
        psum += sa != 0.f ? Ty::lo_f32(pw[wd]) * __builtin_amdgcn_rcpf(sa) : pr[2 * wd];
        psum += sb != 0.f ? Ty::hi_f32(pw[wd]) * __builtin_amdgcn_rcpf(sb) : pr[2 * wd + 1];
      }
    }
    l_run += psum;
    // Row g4 holds the weights of tokens 4*g4..+3 (pw[0], pw[1]) and
    // 16 + 4*g4..+3 (pw[2], pw[3]); the PV product wants tokens 8*g4..+8 in
    // row g4.  Swapping rows between the two word pairs (upper half with lower
    // half, then odd rows with even rows) regroups them.
    const auto a32 = __builtin_amdgcn_permlane32_swap(pw[0], pw[2], false, false);
    const auto b32 = __builtin_amdgcn_permlane32_swap(pw[1], pw[3], false, false);
    const auto a16 = __builtin_amdgcn_permlane16_swap(a32[0], a32[1], false, false);
    const auto b16 = __builtin_amdgcn_permlane16_swap(b32[0], b32[1], false, false);
    const V8 pop = __builtin_bit_cast(V8, u32x4{a16[0], b16[0], a16[1], b16[1]});
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) {
      if constexpr (!KV8)
        acc[mm] = Ty::mma(__builtin_bit_cast(V8, r.v[mm]), pop, acc[mm]);
      else
        acc[mm] = Ty::mma(__builtin_bit_cast(V8, codes_to_operand<Ty>(r.v[mm])), pop, acc[mm]);
    }
  }

  // Fused append: the new token's K row and V row, 8 bytes per lane (lanes
  // [0, D/4) hold K elements 4*lane..+3, lanes [D/4, D/2) hold V elements
  // 4*(lane - D/4)..+3), fetched early so the data is in registers when the
  // token is added.
  using Token = u32x2;
  __device__ __forceinline__ Token fetch_token(const uint16_t* __restrict__ krow,
                                               const uint16_t* __restrict__ vrow) const {
    Token nv = {0u, 0u};
    if (lane < D / 2) nv = lane < D / 4 ? load8(krow + 4 * lane) : load8(vrow + 4 * (lane - D / 4));
    return nv;
  }

  // LDS merge of a workgroup's waves, in the layout the body reads: the
  // wave's running max of column c at m_row[c]; then its sum and output
  // rescaled by 2^(m_w - M), M the max over the NW waves of m_sh (row v at
  // m_sh + 16 v), at l_row[c] and a_base[c * DP + d].  A wave that saw no
  // token has m_w = -inf and weight 0.
  __device__ __forceinline__ void stash_max(float* m_row) const {
    if (g4 == 0) m_row[i] = m_run;
  }
  template <int NW>
  __device__ __forceinline__ void stash_scaled(const float* m_sh, float* l_row, float* a_base, int Gv,
                                               int DP) const {
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, m_sh[v * 16 + i]);
    const float f = m_run > -INFINITY ? exp2_fast(m_run - M) : 0.f;
    if (i < Gv) {
      if (g4 == 0) l_row[i] = l_tot * f;
      // lane holds O^T[d = 16*mm + 4*g4 + j][head i], j = 0..3
      float* arow = a_base + i * DP + 4 * g4;
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) *reinterpret_cast<f32x4*>(arow + 16 * mm) = acc[mm] * f;
    }
  }

  // Fused append: adds the token fetched into nv (fetch_token) to the
  // running state on the vector ALU (one logit per head: each lane of a head
  // takes 32 channels and the 4 row groups are added), rounding the weight
  // to the element type as the matrix-core path does.  With `store` the
  // token also goes bit for bit (INT8: quantised) into the cache slot at row
  // o of block b.
  __device__ __forceinline__ void add_token(u32x2 nv, bool store, int64_t b, int o) {
    if constexpr (!KV8) {
      // operands gathered from the lanes holding them: K chunk 4*kk+g4 (16 B)
      // sits in lanes 2*chunk, 2*chunk+1; V channels 16*mm+4*g4..+3 (8 B) in
      // lane D/4 + 4*mm + g4.
      u32x4 kx[KK];
      u32x2 vx[MM];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int src = 2 * (4 * kk + g4);
        kx[kk] = u32x4{(uint32_t)__shfl((int)nv[0], src), (uint32_t)__shfl((int)nv[1], src),
                       (uint32_t)__shfl((int)nv[0], src + 1), (uint32_t)__shfl((int)nv[1], src + 1)};
      }
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) {
        const int src = D / 4 + 4 * mm + g4;
        vx[mm] = u32x2{(uint32_t)__shfl((int)nv[0], src), (uint32_t)__shfl((int)nv[1], src)};
      }
      float dot = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 qw = __builtin_bit_cast(u32x4, qop[kk]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dot = fmaf(Ty::to_f32((uint16_t)(qw[e / 2] >> (16 * (e & 1)))),
                     Ty::to_f32((uint16_t)(kx[kk][e / 2] >> (16 * (e & 1)))), dot);
      }
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      const float xn = dot * scale_log2;
      const float m_new = fmaxf(m_run, xn);
      const float alpha = exp2_fast(m_run - m_new);  // 0 when the wave saw no cached token
      const float pn = Ty::to_f32(Ty::from_f32(exp2_fast(xn - m_new)));
      m_run = m_new;
      l_run = l_run * alpha + (g4 == 0 ? pn : 0.f);
      // lane holds O^T[d = 16*mm + 4*g4 + j][head i]; vx[mm] holds v_new[16*mm + 4*g4 + j]
#pragma unroll
      for (int mm = 0; mm < MM; ++mm)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[mm][j] = fmaf(pn, Ty::to_f32((uint16_t)(vx[mm][j / 2] >> (16 * (j & 1)))),
                            acc[mm][j] * alpha);
      if (store && lane < D / 2) {
        if (lane < D / 4) {  // K elements 4*lane..+3: half of chunk lane/2's 16-byte row piece
          uint16_t* kd = const_cast<Elem*>(kc) + b * blk_stride + head_off;
          *reinterpret_cast<u32x2*>(kd + ((lane / 2) * BS + o) * 8 + 4 * (lane & 1)) = nv;
        } else {             // V channels 4*(lane - D/4)..+3 of row o
          uint16_t* vd = const_cast<Elem*>(vc) + b * blk_stride + head_off;
          const int d0 = 4 * (lane - D / 4);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            vd[(d0 + j) * BS + o] = (uint16_t)(nv[j / 2] >> (16 * (j & 1)));
        }
      }
    } else {
      // 8-bit caches: quantise the token's K and V rows in fp32 (scale =
      // max|x| / Code::kMax, codes Code::encode(x / scale): INT8 or FP8),
      // then add the token with the values value(code) * scale, as a cache
      // write followed by a read would.  Each half of the lanes finds its
      // row maximum.
      float xv[4];
      float am = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[j] = lane < D / 2 ? Ty::to_f32((uint16_t)(nv[j / 2] >> (16 * (j & 1)))) : 0.f;
        am = fmaxf(am, fabsf(xv[j]));
      }
#pragma unroll
      for (int off = D / 8; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
      using Code = typename Ty::Code;
      const float qsc = am / Code::kMax;
      uint32_t cw = 0;  // this lane's 4 codes
#pragma unroll
      for (int j = 0; j < 4; ++j) cw |= (qsc > 0.f ? Code::encode(xv[j] / qsc) : 0u) << (8 * j);
      const float sk_new = __shfl(qsc, 0);
      const float sv_new = __shfl(qsc, D / 4);
      float dot = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {  // K codes of the channels qop[kk] holds
        const int src = 2 * qchunk(kk);
        const u32x2 kq = {(uint32_t)__shfl((int)cw, src), (uint32_t)__shfl((int)cw, src + 1)};
        const u32x4 qw = __builtin_bit_cast(u32x4, qop[kk]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dot = fmaf(Ty::to_f32((uint16_t)(qw[e / 2] >> (16 * (e & 1)))),
                     Code::value((kq[e / 4] >> (8 * (e % 4))) & 0xFFu), dot);
      }
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      const float xn = dot * sk_new * scale_log2;
      const float m_new = fmaxf(m_run, xn);
      const float alpha = exp2_fast(m_run - m_new);
      const float pn = exp2_fast(xn - m_new);
      m_run = m_new;
      l_run = l_run * alpha + (g4 == 0 ? pn : 0.f);
      const float pv = pn * sv_new;
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) {  // V codes of channels 16*mm + 4*g4..+3
        const uint32_t vq = (uint32_t)__shfl((int)cw, D / 4 + 4 * mm + g4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[mm][j] = fmaf(pv, Code::value((vq >> (8 * j)) & 0xFFu), acc[mm][j] * alpha);
      }
      if (store && lane < D / 2) {
        constexpr int SC = I8Tile<D, BS>::kScales;
        if (lane < D / 4) {  // K codes of channels 4*lane..+3: bytes 4*(lane%4).. of x-vector lane/4
          uint8_t* kd = const_cast<Elem*>(kc) + b * blk_stride + head_off;
          *reinterpret_cast<uint32_t*>(kd + ((lane / 4) * BS + o) * 16 + 4 * (lane & 3)) = cw;
          if (lane == 0) *reinterpret_cast<float*>(kd + SC + 4 * o) = qsc;
        } else {             // V codes of channels 4*(lane - D/4)..+3 of row o
          uint8_t* vd = const_cast<Elem*>(vc) + b * blk_stride + head_off;
          const int d0 = 4 * (lane - D / 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) vd[(d0 + j) * BS + o] = (uint8_t)(cw >> (8 * j));
          if (lane == D / 4) *reinterpret_cast<float*>(vd + SC + 4 * o) = qsc;
        }
      }
    }
  }
};

// One wave's share of the decode pass on the vector ALU, for a KV head read
// by a single query head (G = 1: the matrix-core path would leave 15 of its
// 16 columns empty).  Same interface as WaveDecoder; per 32-token chunk:
//   QK -- lane l takes token l % 32 and half l / 32 of head_dim: its K
//         x-vectors (16 bytes each, 16 lanes on 16 consecutive tokens read
//         256 contiguous bytes) meet q in packed dot products (v_dot2, fp32
//         accumulation), and the two halves are added across lanes;
//   PV -- each 16-byte V load is 8 consecutive tokens of one channel row;
//         lane l takes piece pc = l % PPB of a row (PPB pieces per row of the
//         chunk) for channels CPI * n + l / PPB, so one load instruction reads
//         whole rows, contiguous.  The lane keeps partial sums per channel
//         over its own tokens; the PPB lanes of a channel are added at the end.
//         The chunk's weights (rounded to the element type, packed in pairs)
//         reach each lane's piece by lane shuffles.
// Same arithmetic contract as the matrix-core path: fp32 logits from exact
// products, base-2 online softmax with the lazy reference maximum, weights
// rounded to the element type for PV and for the running sum.
template <typename Ty, int D, int BS>
struct VaWaveDecoder : ChunkWalker<VaWaveDecoder<Ty, D, BS>, BS> {
  static_assert(BS == 8 || BS == 16 || BS == 32 || BS == 64, "block size 8, 16, 32 or 64");
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static constexpr int XH = D / 16;   // 16-byte K x-vectors per half of a row
  static constexpr int TILE = D * BS;
  static constexpr int BPC = BS >= kChunk ? 1 : kChunk / BS;  // blocks per chunk
  static constexpr int RT = BS >= kChunk ? kChunk : BS;       // tokens of a row in one chunk
  static constexpr int PPB = RT / 8;                          // 16-byte pieces of such a row
  static constexpr int CPI = 64 / PPB;                        // channel rows per load instruction
  static constexpr int NCH = D / CPI;                         // channels per lane
  struct RawT {
    u32x4 k[XH];         // token t's x-vectors h2*XH .. h2*XH + XH - 1
    u32x4 v[BPC][NCH];   // block bb of the chunk, channel CPI*n + lane/PPB, piece lane % PPB
  };
  struct Token {         // fused append: q, k, v of the lane's channels (piece 0 lanes)
    uint16_t q[NCH], k[NCH], v[NCH];
  };

  const uint16_t* kc;
  const uint16_t* vc;
  int lane, i, g4;     // lane; the column (always 0: one query head); unused
  int t, h2;           // the lane's token of a chunk and its half of head_dim
  int pc, ch0;         // the lane's piece of a row and its first channel
  int64_t blk_stride, head_off;
  float scale_log2;
  u32x4 qh[XH];        // q channels 8*(h2*XH) .. of the query head
  const uint16_t* qrow;
  float acc[NCH];      // unnormalised output over the lane's tokens, channels ch0 + CPI*n
  float m_run;         // running max of the base-2 logits (wave-uniform)
  float l_run;         // running sum over this lane's tokens (lanes of half 0)

  __device__ __forceinline__ VaWaveDecoder(const void* kcv, const void* vcv, int Hkv, float sl2)
      : kc(reinterpret_cast<const uint16_t*>(kcv)), vc(reinterpret_cast<const uint16_t*>(vcv)),
        lane(threadIdx.x & 63), i(0), g4(0), t(threadIdx.x & 31), h2((threadIdx.x & 63) >> 5),
        pc((threadIdx.x & 63) % PPB), ch0((threadIdx.x & 63) / PPB),
        blk_stride((int64_t)Hkv * TILE), head_off(0), scale_log2(sl2) {}

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int n = 0; n < NCH; ++n) acc[n] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
  }

  __device__ __forceinline__ void load_q(const uint16_t* __restrict__ q_row, bool) {
    qrow = q_row;
#pragma unroll
    for (int j = 0; j < XH; ++j) qh[j] = load16(q_row + 8 * (h2 * XH + j));
  }

  __device__ __forceinline__ void issue(const int (&b)[BPC], int t0, RawT& r) const {
    const int r0 = BS > kChunk ? t0 % BS : 0;  // the chunk's first row of a 64-token block
    {  // K row of token t
      const int id = pick_block<BPC>(b, t / BS);
      const int row = BS >= kChunk ? r0 + t : t % BS;
      const uint16_t* base = kc + (int64_t)id * blk_stride + head_off;
#pragma unroll
      for (int j = 0; j < XH; ++j) r.k[j] = stream16(base + ((h2 * XH + j) * BS + row) * 8);
    }
#pragma unroll
    for (int bb = 0; bb < BPC; ++bb) {  // V rows: piece pc of channel ch0 + CPI*n
      const uint16_t* base = vc + (int64_t)b[bb] * blk_stride + head_off + r0 + 8 * pc;
#pragma unroll
      for (int n = 0; n < NCH; ++n) r.v[bb][n] = v_row16<BS>(base + (ch0 + CPI * n) * BS);
    }
  }

  __device__ __forceinline__ void consume(int t0, RawT& r, int cc, int skip) {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < XH; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) part = Ty::dot2(r.k[j][w], qh[j][w], part);
    float x = (part + __shfl_xor(part, 32)) * scale_log2;
    if (t0 + kChunk > cc || t0 < skip) {  // drop tokens outside [skip, cc) (wave-uniform test)
      const int tok = t0 + t;
      if (tok >= cc || tok < skip) x = -INFINITY;
#pragma unroll
      for (int bb = 0; bb < BPC; ++bb)
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {  // zero the V bits of tokens past cc (they may hold NaN)
          const int tk = t0 + bb * RT + 8 * pc + 2 * wd;
          const uint32_t keep = (tk < cc ? 0x0000FFFFu : 0u) | (tk + 1 < cc ? 0xFFFF0000u : 0u);
#pragma unroll
          for (int n = 0; n < NCH; ++n) r.v[bb][n][wd] &= keep;
        }
    }
    float mx = x;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mx)));  // both halves agree
    if (mx > m_run + kSlack) {  // as in WaveDecoder: rescale only when the max moves far
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NCH; ++n) acc[n] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    const float p = Ty::to_f32(Ty::from_f32(exp2_fast(x - m_use)));  // the weight PV sees
    l_run += h2 == 0 ? p : 0.f;
    // lane 2k holds the packed weights of tokens 2k, 2k + 1
    const int pp = (int)Ty::pack2(p, __shfl_xor(p, 1));
#pragma unroll
    for (int bb = 0; bb < BPC; ++bb)
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t wv = (uint32_t)__shfl(pp, bb * RT + 8 * pc + 2 * wd);
#pragma unroll
        for (int n = 0; n < NCH; ++n) acc[n] = Ty::dot2(r.v[bb][n][wd], wv, acc[n]);
      }
  }

  __device__ __forceinline__ Token fetch_token(const uint16_t* __restrict__ krow,
                                               const uint16_t* __restrict__ vrow) const {
    Token tk{};
    if (pc == 0) {
#pragma unroll
      for (int n = 0; n < NCH; ++n) {
        const int d = ch0 + CPI * n;
        tk.q[n] = qrow[d];
        tk.k[n] = krow[d];
        tk.v[n] = vrow[d];
      }
    }
    return tk;
  }

  // Fused append on the vector ALU: the lanes of piece 0 hold every channel
  // once; their dot products add up to the logit, and they add the token's
  // value to their partial sums.
  __device__ __forceinline__ void add_token(const Token& tk, bool store, int64_t b, int o) {
    float dot = 0.f;
    if (pc == 0) {
#pragma unroll
      for (int n = 0; n < NCH; ++n) dot = fmaf(Ty::to_f32(tk.q[n]), Ty::to_f32(tk.k[n]), dot);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
    const float xn = dot * scale_log2;
    const float m_new = fmaxf(m_run, xn);
    const float alpha = exp2_fast(m_run - m_new);  // 0 when the wave saw no cached token
    const float pn = Ty::to_f32(Ty::from_f32(exp2_fast(xn - m_new)));
    m_run = m_new;
    l_run = l_run * alpha + (lane == 0 ? pn : 0.f);
#pragma unroll
    for (int n = 0; n < NCH; ++n)
      acc[n] = pc == 0 ? fmaf(pn, Ty::to_f32(tk.v[n]), acc[n] * alpha) : acc[n] * alpha;
    if (store && pc == 0) {
      uint16_t* kd = const_cast<uint16_t*>(kc) + b * blk_stride + head_off;
      uint16_t* vd = const_cast<uint16_t*>(vc) + b * blk_stride + head_off;
#pragma unroll
      for (int n = 0; n < NCH; ++n) {  // channel d: x-vector d / 8, element d % 8; V row d
        const int d = ch0 + CPI * n;
        kd[((d / 8) * BS + o) * 8 + d % 8] = tk.k[n];
        vd[d * BS + o] = tk.v[n];
      }
    }
  }

  __device__ __forceinline__ void stash_max(float* m_row) const {
    if (lane == 0) m_row[0] = m_run;
  }
  template <int NW>
  __device__ __forceinline__ void stash_scaled(const float* m_sh, float* l_row, float* a_base, int,
                                               int) const {
    float l_tot = l_run;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l_tot += __shfl_xor(l_tot, off);
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, m_sh[v * 16]);
    const float f = m_run > -INFINITY ? exp2_fast(m_run - M) : 0.f;
    if (lane == 0) l_row[0] = l_tot * f;
#pragma unroll
    for (int n = 0; n < NCH; ++n) {  // add the PPB pieces of each channel
      float a = acc[n];
#pragma unroll
      for (int off = 1; off < PPB; off <<= 1) a += __shfl_xor(a, off);
      if (pc == 0) a_base[ch0 + CPI * n] = a * f;
    }
  }
};

// Chunk walk of the matrix-core decoders.  INT8 caches take walk_skew (one
// register set, the next chunk's loads split around the products); 16-bit
// caches take walk<true>.  Measured on MI355X, 300 steps each against the
// one-chunk walk<false> for INT8 and walk<true> for 16-bit:
//   INT8: LLaMA-13B-shaped 43.2 -> 42.4 us, mixed lengths 43.4 -> 43.0, long
//         context (P = 512) 112.4 -> 111.8 (168 VGPRs, still 3 waves per SIMD);
//   16-bit: LLaMA-13B-shaped 64.1 -> 64.7 us, mixed lengths 60.8 -> 60.9, long
//         context 183.8 -> 181.8; at block size 32 the 3-wave budget spilled
//         (65.3 -> 77.9 us).
// INT8 at block size 64 keeps walk<false>: walk_skew spilled there (f16).
template <bool KV8, bool VALU, int BS>
constexpr bool kSkewWalk = KV8 && !VALU && BS <= 32;

// Body of the decode pass for the workgroup at grid position (bx, by, bz);
// `lds` holds merge_lds_bytes(NW, G, D) bytes.  With prefix groups
// (pa_decode_prefix, through prefix_suffix_kernel) it takes each member's
// keys after its group's shared prefix; the prefix itself is attended by the
// shared-prefix pass of the prefill body, in pre_parts partitions of pre_P
// tokens that fill the first partial slots of every member.
template <typename Ty, int D, int BS, int NW, bool KV8, bool VALU = false>
__device__ __forceinline__ void decode_mfma_body(int bx, int by, int bz, float* lds,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const void* __restrict__ kcv,
    const void* __restrict__ vcv, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, int Hq, int Hkv, int G, int n_groups, int NB,
    int max_blocks, int max_ctx, float scale_log2, int P, int max_parts,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, int num_seqs, int pre_parts, int pre_P,
    const int32_t* __restrict__ grp_start, const int32_t* __restrict__ grp_len, int n_grp) {
  static_assert(!VALU || !KV8, "the vector-ALU decoder reads 16-bit caches");
  using W = typename std::conditional<VALU, VaWaveDecoder<Ty, D, BS>, WaveDecoder<Ty, D, BS, KV8>>::type;
  constexpr int BPC = W::BPC;
  constexpr int DP = D + 4;      // padded LDS row of the merge buffer

  W wd(kcv, vcv, Hkv, scale_log2);
  const int lane = wd.lane, i = wd.i;
  const int w = uniform(threadIdx.x >> 6);
  int hk, grp = 0, p = 0, s, c;
  if (num_seqs > 0) {
    hk = bx / n_groups;
    grp = bx - hk * n_groups;
    // Flat work list: y enumerates the (sequence, partition) units that exist,
    // sequence by sequence; each wave finds its unit from a prefix sum of the
    // sequences' partition counts, so grid slots past the real work sit at
    // the end of the grid instead of between sequences.
    if (!flat_unit(lens, num_seqs, min(max_ctx, max_blocks * BS), P, by, lane, s, p,
                   c))
      return;
  } else {
    hk = bx / n_groups;
    grp = bx - hk * n_groups;
    p = by;
    s = bz;
    c = clampi(lens[s], 0, min(max_ctx, max_blocks * BS));
  }
  // With prefix groups: tokens [0, skip) of sequence s belong to its group's
  // shared prefix, attended by the prefix pass (partial slots 0 .. pb - 1);
  // this launch covers [skip, c) in the slots after them.
  int skip = 0;
  if (n_grp > 0) {
    int lo = 0, hi = n_grp - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (grp_start[mid] <= s) lo = mid;
      else hi = mid - 1;
    }
    skip = uniform(clampi(grp_len[lo], 0, min(c, pre_parts * pre_P)));
  }
  const int pb = n_grp > 0 ? (skip + pre_P - 1) / pre_P : 0;  // partial slots of the prefix
  // Chunks start on 32-token boundaries: the partitions run from the boundary
  // at or below skip, and tokens below skip are dropped.
  const int a_skip = skip & ~(kChunk - 1);
  const int n_p = (c - a_skip + P - 1) / P;
  if (p < 0 || p >= max(n_p, 1)) return;
  const int t_begin = a_skip + p * P;
  // With a fused append the token at c - 1 comes from k_new / v_new, not from
  // the cache: the chunk loop reads [t_begin, cc) and the new token is added
  // afterwards by the workgroup whose partition holds it.
  const bool append = k_new != nullptr;
  const int cc = append ? max(c - 1, 0) : c;  // keys [0, cc) come from the cache
  const bool has_new = append && c > 0 && c - 1 >= t_begin && c - 1 < t_begin + P;
  const int t_end = min(cc, t_begin + P);
  const int n_chunks = max(0, t_end - t_begin + kChunk - 1) / kChunk;

  // Columns: query heads qh0 + i of the group of 16.
  const int Gv = min(16, G - grp * 16);  // valid columns
  const bool head_ok = i < Gv;
  const int qh0 = hk * G + grp * 16;     // first query head of the group
  // q / out row (times Hq, plus head) of column `col`
  auto out_row = [&](int col) -> int64_t { return (int64_t)s * Hq + qh0 + col; };

  wd.load_q(q + out_row(head_ok ? i : 0) * D, head_ok);

  // Fused append: wave 0 of the workgroup whose partition holds token c - 1
  // fetches the new K row and V row up front, so the data is in registers
  // when the token is added.
  const bool new_here = has_new && w == 0;
  typename W::Token nv{};
  if (new_here) {
    const int64_t row = ((int64_t)s * Hkv + hk) * D;
    nv = wd.fetch_token(k_new + row, v_new + row);
  }

  wd.reset();
  const int32_t* trow = tables + (int64_t)s * max_blocks;
  wd.head_off = (int64_t)hk * W::TILE;

  // Block ids of this wave's chunks (w, w + NW, ...), held in registers: one
  // vector load fetches a batch of table entries before the first K/V load is
  // issued, so no chunk waits on a table read (a chunk whose block ids came
  // from a load in the loop would also wait for every K/V load issued before
  // that read).  Chunks are dealt to the waves round-robin (the
  // intelliparadigm page's warp-to-block assignment, section 4.2, with a wave
  // taking 32 tokens).
  auto chunk_of = [&](int k) { return w + NW * k; };  // the wave's k-th chunk
  if (chunk_of(0) < n_chunks) wd.load_batch(trow, t_begin, n_chunks, cc, NB, w, NW, 0);
  auto block_ids = [&](int k, int (&b)[BPC]) {
    wd.block_ids(k, b, trow, t_begin, n_chunks, cc, NB, w, NW);
  };

  // Chunk loop over the wave's chunks w, w + NW, ... of the partition.
  // 16-bit caches keep the next chunk in flight in a second register set;
  // INT8 caches (block sizes up to 32) keep one register set and load the
  // next chunk's K and V halves as the products free them (measured on
  // MI355X: with half the bytes per chunk, a second register set made the
  // INT8 step slower; with one the kernel fits 3 waves per SIMD).
  const int n_mine = w < n_chunks ? (n_chunks - w + NW - 1) / NW : 0;
  auto t0_of = [&](int k) { return t_begin + chunk_of(k) * kChunk; };
  if constexpr (kSkewWalk<KV8, VALU, BS>) wd.walk_skew(n_mine, t0_of, block_ids, cc, skip);
  else wd.template walk<!KV8>(n_mine, t0_of, block_ids, cc, skip);

  // Fused append: that wave adds token c - 1 to its running state; the
  // group-0 workgroup also stores the token into the cache slot of position
  // c - 1.
  if (new_here) {
    const int tn = c - 1;
    wd.add_token(nv, grp == 0, clampi(trow[tn / BS], 0, NB - 1), tn % BS);
  }

  // Merge the NW waves: M = max_w m_w per head, then every wave rescales its
  // sum and output by 2^(m_w - M) into LDS and the workgroup adds them up in
  // wave order.
  float* m_sh = lds;                  // [NW][16]
  float* l_sh = lds + NW * 16;        // [NW][16]
  float* a_sh = lds + 2 * NW * 16;    // [NW][Gv][DP]
  wd.stash_max(m_sh + w * 16);
  __syncthreads();
  wd.template stash_scaled<NW>(m_sh, l_sh + w * 16, a_sh + w * Gv * DP, Gv, DP);
  __syncthreads();

  const bool split = pb > 0 || n_p > 1;
  for (int e = threadIdx.x; e < Gv * (D / 4); e += 64 * NW) {
    const int hh = e / (D / 4);
    const int d = 4 * (e - hh * (D / 4));
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      sum += *reinterpret_cast<const f32x4*>(a_sh + (v * Gv + hh) * DP + d);
      L += l_sh[v * 16 + hh];
    }
    const int64_t row = out_row(hh);
    if (!split) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      const f32x4 r = sum * inv;
      const u32x2 packed = {(uint32_t)Ty::from_f32(r[0]) | ((uint32_t)Ty::from_f32(r[1]) << 16),
                            (uint32_t)Ty::from_f32(r[2]) | ((uint32_t)Ty::from_f32(r[3]) << 16)};
      *reinterpret_cast<u32x2*>(out + row * D + d) = packed;
    } else {
      const int64_t idx = row * max_parts + pb + p;
      *reinterpret_cast<f32x4*>(ws_acc + idx * D + d) = sum;
      if (d == 0) {
        float Mh = -INFINITY;
#pragma unroll
        for (int v = 0; v < NW; ++v) Mh = fmaxf(Mh, m_sh[v * 16 + hh]);
        ws_ml[2 * idx] = Mh;
        ws_ml[2 * idx + 1] = L;
      }
    }
  }
}

template <typename Ty, int D, int BS, int NW, bool KV8, bool VALU>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(KV8 ? 3 : 1))) void decode_mfma_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const void* __restrict__ kcv,
    const void* __restrict__ vcv, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, int Hq, int Hkv, int G, int n_groups, int NB,
    int max_blocks, int max_ctx, float scale_log2, int P, int max_parts,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, int num_seqs, int pre_parts, int pre_P,
    const int32_t* __restrict__ grp_start, const int32_t* __restrict__ grp_len, int n_grp,
    int xcd_order, UnitList ul) {
  extern __shared__ float lds[];
  // Workgroups are dealt to the XCDs round-robin (linear id L goes to XCD
  // L % kXcds).  With xcd_order the grid is renumbered so that each XCD
  // takes one contiguous range of the (head, partition, sequence) order: the
  // workgroups of a sequence then run on one XCD, and each XCD touches the
  // blocks of its own sequences only.  The host sets it for 16-bit caches
  // on the (head, partition, sequence) grid; measured on MI355X, the
  // LLaMA-13B-shaped step went from 65.6 to 64.0 us.  It stays off:
  //   - for INT8 caches: all of their workgroups fit at once (3 waves per
  //     SIMD), and contiguous ranges made the LLaMA-13B-shaped INT8 step
  //     2.7% slower (uneven work per XCD);
  //   - for the flat work list.  In hardware order, with 8 KV heads, each
  //     XCD takes one head of every sequence, so blocks shared by many
  //     sequences (a common prefix) are re-read from that XCD's L2.
  //     Renumbered, a 32-sequence batch sharing 2048 tokens decoded in
  //     63.3 us instead of 45.7 (long context gained 2%, mixed lengths
  //     nothing).  Without host context lengths the flat list's surplus
  //     workgroups also sit at its end and would idle the last XCDs.
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if (!KV8 && xcd_order) {
    const int64_t X = gridDim.x, Y = gridDim.y;
    const int64_t T = X * Y * gridDim.z;
    const int64_t L = blockIdx.x + X * (blockIdx.y + Y * blockIdx.z);
    const int64_t xcd = L % kXcds, per = T / kXcds, rem = T % kXcds;
    const int64_t lam = xcd * per + (xcd < rem ? xcd : rem) + L / kXcds;
    bx = (int)(lam % X);
    by = (int)((lam / X) % Y);
    bz = (int)(lam / (X * Y));
  }
  if (ul.n > 0) {  // the host's unit order: row by is unit (s, p) of its list
    const uint32_t e = ul.e[by];
    bz = (int)(e & 0xFFFFu);
    by = (int)(e >> 16);
    num_seqs = 0;  // the body then takes p = by, s = bz
  }
  decode_mfma_body<Ty, D, BS, NW, KV8, VALU>(bx, by, bz, lds, out, q, kcv, vcv, tables, lens, k_new,
                                       v_new, Hq, Hkv, G, n_groups, NB, max_blocks, max_ctx,
                                       scale_log2, P, max_parts, ws_acc, ws_ml, num_seqs, pre_parts,
                                       pre_P, grp_start, grp_len, n_grp);
}

// LDS of the prefill pass: two chunk buffers, each a 32-token chunk's K and
// V (16-bit), or its K codes, V codes and 64 scales (INT8).
// With DMA (the prefill pass proper) the chunks go from global memory
// straight to LDS, into four buffers; INT8 chunks are then widened into two
// more buffers of 16-bit K and V.
template <int D, bool KV8, bool DMA = false>
struct PrefillLds {
  static constexpr int kBuf = KV8 ? kChunk * (D / 16) * 16 + D * 4 * 8 + 64 * 4 : 2 * kChunk * (D / 8) * 16;
  static constexpr int kBufs = DMA ? 4 : 2;
  // INT8 chunks loaded straight to LDS are widened once per workgroup into
  // one of two buffers of 16-bit K and V
  static constexpr int kConvBuf = KV8 && DMA ? 2 * kChunk * (D / 8) * 16 : 0;
  static constexpr int kBytes = kBufs * kBuf + 2 * kConvBuf;
};

// Direct global-to-LDS loads for the prefill pass (not the shared-prefix
// pass, which shares its launch with decode workgroups).
template <bool KV8, bool PFX>
constexpr bool kPrefillDma = !PFX;

// s_waitcnt immediate that waits until at most n vector memory operations
// of this wave are outstanding (n <= 15), leaving the other counters free.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 15, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// 16 bytes from global address g to LDS: lane l of the wave writes
// lds_wave + 16 l (lds_wave must be the same in every lane).
__device__ __forceinline__ void load_to_lds16(const void* g, void* lds_wave) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)(g), (lds_void_ptr)(lds_wave), 16, 0, 0);
}

// 4 bytes from global address g to LDS: lane l writes lds_wave + 4 l.
__device__ __forceinline__ void load_to_lds4(const void* g, void* lds_wave) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)(g), (lds_void_ptr)(lds_wave), 4, 0, 0);
}

// wait_vmcnt for a wave-uniform count n (0 <= n <= 15).
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<15>(); break;
  }
}

// A thread's share of one prefill chunk on its way to LDS.
template <int PER>
struct Stage16 {
  u32x4 k[PER], v[PER];
};
template <int PV8>
struct StageI8 {
  u32x4 k = {0u, 0u, 0u, 0u};
  u32x2 v[PV8];
  float sc = 0.f;
};

// ----------------------------------------------------------------------------
// Paged prefill with K/V staged through LDS.  A workgroup of
// NW waves takes 16 * NC * NW (row, head) slots of one sequence and KV head;
// wave w owns slots sb .. sb + 16*NC - 1 (NC column groups of 16).  The
// workgroup walks the keys in 32-token chunks, stages each chunk's K and V
// in LDS, and every wave reads its matrix-core operands from there, so each
// K/V byte crosses L1 once per workgroup rather than once per wave.  Staging:
//   - the prefill pass proper (DMA): the chunk goes from global memory
//     straight into one of four LDS buffers (global_load_lds), three chunks
//     in flight while one is computed;
//   - the shared-prefix pass: all threads load a chunk (16-byte vectors in
//     the pool's order, coalesced) into registers and store it into one of
//     two LDS buffers; two chunks in flight while one is computed.
// The LDS order makes the operand reads (16 bytes per lane, 16 lanes on 16
// tokens or channels) hit distinct banks:
//   K vector (token tau, x-vector j) at j * 32 + tau (DMA) or
//     tau * XV + (j ^ (tau % XV)) (register staging),
//   V vector (channel d, tokens 8*qd..+8) at d * 4 + (qd ^ ((d / 2) % 4)).
// INT8 caches (KV8): a chunk is its K codes (16-byte x-vectors, 4 KiB at
// D = 128), its V codes (8-byte runs of 8 tokens, 4 KiB) and its 64 scales;
//   K vector (token tau, x-vector j) at j * 32 + tau (DMA) or
//     tau * XV8 + (j ^ (tau % XV8)) (register staging),
//   V run (channel d, tokens 8*qd..+8) at d * 4 + (qd ^ ((d / 4) % 4)),
// and the codes are widened to the query type as the operands are read.
// Arithmetic per column as in decode_mfma_kernel: base-2 online softmax with
// the lazy reference maximum, fp32 accumulation, weights rounded to the
// element type for the PV product.
// ----------------------------------------------------------------------------
// Body of the prefill pass for the workgroup at grid position (bx, by, bz) of
// a (gx, gy, gz) grid; `lds_raw` holds PrefillLds<D, KV8, DMA>::kBytes bytes.
// PFX: the shared-prefix pass of pa_decode_prefix instead (run by
// prefix_suffix_kernel).  Grid x = slot tiles of a group's (member, head)
// slots, y = partition of the prefix (P tokens), z = group * Hkv + KV head;
// members are rows qstart[g] .. qstart[g+1] - 1 (query rows of the decode),
// the keys [p*P, (p+1)*P) of the prefix (grp_len[g] tokens) come through the
// first member's table, no causal limit, and each column's partial (max,
// sum, unnormalised output) goes to partial slot p of its row in the split-K
// workspace.
template <typename Ty, int D, int BS, int NW, int NC, bool KV8, bool PFX>
__device__ __forceinline__ void prefill_lds_body(int bx, int by, int bz, int gx, int gy, int gz,
    uint8_t* lds_raw, uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const void* __restrict__ kcv,
    const void* __restrict__ vcv, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ qstart, int Hq, int Hkv, int G,
    int NB, int max_blocks, int max_ctx, int max_q, int num_rows, float scale_log2,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, int P, int max_parts,
    const int32_t* __restrict__ grp_len) {
  static_assert(BS == 8 || BS == 16 || BS == 32 || BS == 64, "block size 8, 16, 32 or 64");
  using V8 = typename Ty::vec8;
  constexpr int KK = D / 32;           // QK products along head_dim
  constexpr int MM = D / 16;           // PV products along head_dim
  constexpr int XV = D / 8;            // 16-byte vectors per K row (one token)
  constexpr int CV = kChunk * XV;      // 16-byte vectors of a chunk's K (and of its V)
  constexpr int PER = CV / (64 * NW);  // K (and V) vectors each thread moves per chunk
  static_assert(PER * 64 * NW == CV, "chunk vectors split evenly over the threads");
  constexpr int XV8 = D / 16;          // INT8: 16-byte code vectors per K row
  constexpr int CK8 = kChunk * XV8;    // INT8: K code vectors of a chunk
  constexpr int CV8 = D * 4;           // INT8: 8-byte V runs of a chunk
  static_assert(!KV8 || (CK8 <= 64 * NW && CV8 % (64 * NW) == 0), "INT8 chunk split over the threads");
  constexpr int PV8 = CV8 / (64 * NW);  // INT8: V runs each thread moves per chunk
  constexpr int RV8 = 2 * CV8 / (64 * NW);  // INT8: 4-byte V loads per thread and chunk (straight to LDS)
  static_assert(!KV8 || (CK8 % 64 == 0 && 2 * CV8 == RV8 * 64 * NW), "INT8 LDS loads");
  constexpr int TILE = KV8 ? I8Tile<D, BS>::kBytes : D * BS;  // elements (16-bit) or bytes (INT8)
  using Elem = typename std::conditional<KV8, uint8_t, uint16_t>::type;
  const Elem* kc = reinterpret_cast<const Elem*>(kcv);
  const Elem* vc = reinterpret_cast<const Elem*>(vcv);
  constexpr int BPC = BS >= kChunk ? 1 : kChunk / BS;  // blocks per chunk
  constexpr int CPB = 64 / BPC;                         // chunks per batch of table entries
  // one LDS buffer: K then V (16-bit), or K codes, V codes and 64 scales (INT8)
  constexpr int BUF = KV8 ? CK8 * 16 + CV8 * 8 + 64 * 4 : 2 * CV * 16;
  constexpr bool DMA = kPrefillDma<KV8, PFX>;
  // INT8 chunks loaded straight to LDS: widened once per workgroup (each
  // thread a share of the chunk) into conversion buffer k % 2, in the 16-bit
  // LDS order, from which every wave reads 16-bit operands
  constexpr bool CONV = KV8 && DMA;
  constexpr int CBUF = PrefillLds<D, KV8, DMA>::kConvBuf;
  static_assert(PrefillLds<D, KV8, DMA>::kBufs * BUF + 2 * CBUF == PrefillLds<D, KV8, DMA>::kBytes,
                "LDS size of the prefill pass");
  auto lck = [&](int c) {
    return reinterpret_cast<u32x4*>(lds_raw + PrefillLds<D, KV8, DMA>::kBufs * BUF + c * CBUF);
  };
  auto lcv = [&](int c) {
    return reinterpret_cast<u32x4*>(lds_raw + PrefillLds<D, KV8, DMA>::kBufs * BUF + c * CBUF + CV * 16);
  };
  auto lk = [&](int buf) { return reinterpret_cast<u32x4*>(lds_raw + buf * BUF); };
  auto lv = [&](int buf) { return reinterpret_cast<u32x4*>(lds_raw + buf * BUF + CV * 16); };
  auto lk8 = [&](int buf) { return reinterpret_cast<u32x4*>(lds_raw + buf * BUF); };
  auto lv8 = [&](int buf) { return reinterpret_cast<u32x2*>(lds_raw + buf * BUF + CK8 * 16); };
  auto lsc = [&](int buf) { return reinterpret_cast<float*>(lds_raw + buf * BUF + CK8 * 16 + CV8 * 8); };
  using Stage = typename std::conditional<KV8, StageI8<(PV8 > 0 ? PV8 : 1)>, Stage16<PER>>::type;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int i = lane & 15;
  const int g4 = lane >> 4;
  // Workgroups are dealt to the 8 XCDs round-robin, and each XCD has its own
  // L2.  The linear id is remapped so that the consecutive workgroups of one
  // XCD are the slot tiles of one (sequence, KV head) -- they read the same
  // K/V lines at about the same time, through one L2 -- while the (sequence,
  // KV head) pairs are dealt to the XCDs round-robin (balanced work).  (The
  // prefill pass over at most 64 (sequence, slot tile) pairs orders its
  // workgroups by work instead, below.)
  int tile, ya, za;  // grid position after the reordering
  {
    const int X = gx, Y = gy;
    const int L = bx + X * (by + Y * bz);
    int grp = L / X;
    tile = L % X;
    if ((Y * gz) % kXcds == 0) {
      const int n = L / kXcds;  // the workgroup's place on its XCD
      tile = n % X;
      grp = (n / X) * kXcds + L % kXcds;
    }
    ya = grp % Y;
    za = grp / Y;
  }
  // Rows q0 .. q0 + nq - 1; keys from t_begin on, up to c.
  int hk, s, c, q0, nq, p = 0, t_begin = 0;
  if constexpr (!PFX) {
    hk = ya;
    // Longest work first, so that the workgroups that start last are short
    // ones and fewer CUs idle while the grid drains.  With at most 64
    // (sequence, slot tile) pairs the whole grid is ordered by each pair's
    // work (measured on MI355X, chunked prefill at LLaMA-13B shape: f16
    // 174.9 / 172.0 -> 171.1 / 169.0 us, INT8 251 / 248 -> 234 / 229 us, FP8
    // 248 -> 229 us, against the order below; a makespan model of the 960
    // workgroups on 512 slots gave 93 -> 87 chunk-times, bound 79).  Larger
    // grids: the grid position za is a rank, and the sequence of rank za is
    // the za-th longest context (ties in sequence order), its slot tiles
    // last row first, since later rows see more keys (ranks need every
    // length in one wave: at most 64 sequences; larger batches keep their
    // order).
    s = za;
    const int cmax = min(max_ctx, max_blocks * BS);
    if (gz * gx <= kWave) {
      // At most 64 (sequence, slot tile) pairs: the grid runs them longest
      // first across the whole batch, each pair's KV heads together (and
      // thus spread over the XCDs).  Lane m weighs pair m (sequence m / gx,
      // tile m % gx) by the keys its last slot sees; the workgroup takes the
      // pair of rank L / gy (ties in pair order) and KV head L % gy.
      constexpr int TS = NW * NC * 16;  // slots per tile
      const int L = bx + gx * (by + gy * bz);
      const int r = L / gy;
      hk = L - r * gy;
      const int npair = gz * gx;
      int wl = -1;
      if (lane < npair) {
        const int sm = lane / gx, jm = lane - sm * gx;
        const int cm = clampi(lens[sm], 0, cmax);
        const int q0m = clampi(qstart[sm], 0, num_rows);
        const int nqm = clampi(qstart[sm + 1] - q0m, 0, min(min(max_q, cm), num_rows - q0m));
        const int first = jm * TS;
        wl = first < nqm * G ? cm - nqm + (min(first + TS, nqm * G) - 1) / G + 1 : 0;
      }
      int rank = 0;  // pairs ahead of this lane's
      for (int m = 0; m < npair; ++m) {
        const int wm = __builtin_amdgcn_readlane(wl, m);
        rank += (wm > wl || (wm == wl && m < lane)) ? 1 : 0;
      }
      const uint64_t hit = __ballot(lane < npair && rank == r);
      const int pick = uniform(__ffsll((unsigned long long)hit) - 1);
      s = pick / gx;
      tile = pick - s * gx;
    } else {
      if (gz <= kWave) {
        const int lane_c = lane < gz ? clampi(lens[lane], 0, cmax) : -1;
        int rank = 0;  // sequences ahead of this lane's
        for (int m = 0; m < gz; ++m) {
          const int cm = __builtin_amdgcn_readlane(lane_c, m);
          rank += (cm > lane_c || (cm == lane_c && m < lane)) ? 1 : 0;
        }
        const uint64_t hit = __ballot(lane < gz && rank == za);
        s = uniform(__ffsll((unsigned long long)hit) - 1);
      }
      tile = gx - 1 - tile;
    }
    c = clampi(lens[s], 0, min(max_ctx, max_blocks * BS));
    q0 = clampi(qstart[s], 0, num_rows);
    nq = clampi(qstart[s + 1] - q0, 0, min(min(max_q, c), num_rows - q0));
  } else {
    p = ya;
    const int g = za / Hkv;
    hk = za - g * Hkv;
    q0 = clampi(qstart[g], 0, num_rows);
    nq = clampi(qstart[g + 1] - q0, 0, num_rows - q0);
    s = q0;  // the first member's table holds the shared blocks
    c = clampi(grp_len[g], 0, min(min(max_ctx, max_blocks * BS), gy * P));
    t_begin = p * P;
    if (t_begin >= c) return;  // the whole workgroup: no barrier reached yet
    c = min(c, t_begin + P);
  }
  const int swg = tile * NW * NC * 16;  // first slot of the workgroup
  if (swg >= nq * G) return;            // the whole workgroup: no barrier reached yet
  // Slot u is row q0 + u / G, query head hk*G + u % G; in prefill it sits at
  // position c - nq + u / G and sees keys up to there, in the shared-prefix
  // pass it sees all keys [t_begin, c).
  auto key_end = [&](int u) { return PFX ? c : c - nq + u / G + 1; };
  const int last = min(nq * G, swg + NW * NC * 16) - 1;  // last slot of the workgroup
  const int c_load = key_end(last);                      // tokens the workgroup loads
  const int n_chunks = (c_load - t_begin + kChunk - 1) / kChunk;
  const int sb = swg + w * NC * 16;                // the wave's first slot
  const int slots = nq * G - sb;                   // may be <= 0: the wave only loads
  const int cc = slots > 0 ? key_end(sb + min(slots, 16 * NC) - 1) : t_begin;  // keys it needs
  const int lim_min = slots > 0 ? key_end(sb) : t_begin;
  const int n_mine = (cc - t_begin + kChunk - 1) / kChunk;  // chunks this wave computes

  int Gv[NC], lim[NC];
  bool head_ok[NC];
#pragma unroll
  for (int nc = 0; nc < NC; ++nc) {
    Gv[nc] = clampi(slots - 16 * nc, 0, 16);
    head_ok[nc] = i < Gv[nc];
    lim[nc] = head_ok[nc] ? key_end(sb + 16 * nc + i) : cc;
  }
  auto out_row = [&](int col) -> int64_t {
    const int u = sb + col;
    return (int64_t)(q0 + u / G) * Hq + hk * G + u % G;
  };
  // Q^T operand: lane feeds column i, channels 8*m..+8 with m = 4*kk + g4
  // (INT8: 8*(kk/2) + 2*g4 + kk%2, so that one 16-byte code vector feeds two
  // products)
  auto qchunk = [&](int kk) { return KV8 && !CONV ? 8 * (kk >> 1) + 2 * g4 + (kk & 1) : 4 * kk + g4; };
  // The softmax step takes its maximum over the raw products and scales it
  // once, which needs a scale >= 0: a negative scale is moved onto q by
  // flipping its sign bits (exact; every product and sum is negated exactly).
  // A zero scale is taken as the smallest normal float, so that a dropped
  // token's -inf logit never meets a zero factor; every kept weight is then
  // 1 up to rounding, as scale 0 means.
  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const float sc = fmaxf(fabsf(scale_log2), 1.17549435e-38f);
  const float inv_sc = 1.f / sc;
  V8 qop[NC][KK];
#pragma unroll
  for (int nc = 0; nc < NC; ++nc) {
    const uint16_t* qrow = q + out_row(head_ok[nc] ? 16 * nc + i : 0) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 raw = head_ok[nc] ? load16(qrow + 8 * qchunk(kk)) : u32x4{0u, 0u, 0u, 0u};
      qop[nc][kk] = __builtin_bit_cast(V8, raw ^ qsign);
    }
  }
  f32x4 acc[NC][MM];
  float m_run[NC], l_run[NC];
  // thr: unscaled logit above which a chunk moves the reference maximum,
  // (m_run + kSlack) / scale, kept up to date with m_run
  float thr[NC];
#pragma unroll
  for (int nc = 0; nc < NC; ++nc) {
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) acc[nc][mm] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[nc] = -INFINITY;
    l_run[nc] = 0.f;
    thr[nc] = -INFINITY;
  }

  // Block ids in registers, as in decode: lane j holds block j % BPC of chunk
  // (batch start) + j / BPC; entries past the loaded range read as block 0.
  const int32_t* trow = tables + (int64_t)s * max_blocks;
  const int64_t blk_stride = (int64_t)Hkv * TILE;
  const int64_t head_off = (int64_t)hk * TILE;
  int tbl = 0;
  auto load_batch = [&](int k0) {
    const int ch = k0 + lane / BPC;
    const int t = t_begin + ch * kChunk + (lane % BPC) * BS;
    tbl = ch < n_chunks && t < c_load ? clampi(trow[t / BS], 0, NB - 1) : 0;
  };
  load_batch(0);

  // This thread's share of chunk k (16-bit): vector g = tid + 64*NW*r of K (x-vector
  // g / 32, token g % 32: 16 consecutive lanes read 16 consecutive tokens of
  // one x-vector, 256 contiguous bytes) and of V (channel g / 4, tokens
  // 8*(g % 4)..+8: consecutive lanes read consecutive bytes of a block row).
  // The wave issues the chunk's loads at raised priority, so that they leave
  // ahead of the other waves' softmax arithmetic (measured on MI355X:
  // f16 chunked prefill at LLaMA-13B shape 183.5 -> 180.6 us).
  auto gload = [&](int k, Stage& st) {
    __builtin_amdgcn_s_setprio(2);
    if (k > 0 && k % CPB == 0) load_batch(k);
    const int e = (k % CPB) * BPC;
    int b[BPC];
#pragma unroll
    for (int j = 0; j < BPC; ++j) b[j] = __builtin_amdgcn_readlane(tbl, e + j);
    const int r0 = BS > kChunk ? (t_begin + k * kChunk) % BS : 0;
    auto at = [&](int tau, int64_t& off, int& row) {  // tile offset and row of token tau
      const int id = pick_block<BPC>(b, tau / BS);
      off = (int64_t)id * blk_stride + head_off;
      row = BS >= kChunk ? r0 + tau : tau % BS;
    };
    if constexpr (!KV8) {
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        const int g = tid + 64 * NW * r;
        int64_t off;
        int row;
        at(g % kChunk, off, row);
        st.k[r] = load16(kc + off + ((g / kChunk) * BS + row) * 8);
        at(8 * (g & 3), off, row);
        st.v[r] = load16(vc + off + (g >> 2) * BS + row);
      }
    } else {
      int64_t off;
      int row;
      if (tid < CK8) {  // K code vector: x-vector tid / 32, token tid % 32
        at(tid % kChunk, off, row);
        st.k = load16(kc + off + ((tid / kChunk) * BS + row) * 16);
      }
#pragma unroll
      for (int r = 0; r < PV8; ++r) {  // V run: channel g / 4, tokens 8*(g % 4)..+8
        const int g = tid + 64 * NW * r;
        at(8 * (g & 3), off, row);
        st.v[r] = load8(vc + off + (g >> 2) * BS + row);
      }
      if (tid < 64) {  // scales: K of token tid (tid < 32), V of token tid - 32
        at(tid & 31, off, row);
        st.sc = *reinterpret_cast<const float*>((tid < 32 ? kc : vc) + off + I8Tile<D, BS>::kScales + 4 * row);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto swrite = [&](int buf, const Stage& st) {
    if constexpr (!KV8) {
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        const int g = tid + 64 * NW * r;
        const int tau = g % kChunk, j = g / kChunk;
        lk(buf)[tau * XV + (j ^ (tau % XV))] = st.k[r];
        const int d = g >> 2, qd = g & 3;
        lv(buf)[d * 4 + (qd ^ ((d >> 1) & 3))] = st.v[r];
      }
    } else {
      if (tid < CK8) {
        const int tau = tid % kChunk, j = tid / kChunk;
        lk8(buf)[tau * XV8 + (j ^ (tau % XV8))] = st.k;
      }
#pragma unroll
      for (int r = 0; r < PV8; ++r) {
        const int g = tid + 64 * NW * r;
        const int d = g >> 2, qd = g & 3;
        lv8(buf)[d * 4 + (qd ^ ((d >> 2) & 3))] = st.v[r];
      }
      if (tid < 64) lsc(buf)[tid] = st.sc;
    }
  };

  // The wave's products and online-softmax update for chunk k (in buf).
  auto compute = [&](int k, int buf) {
    const int t0 = t_begin + k * kChunk;
    const bool edge = t0 + kChunk > lim_min;
    // operands: 16-bit K rows / V runs, or INT8 code vectors and scales
    u32x4 kop[2][KK], vop[MM];
    u32x4 kv8[2][KK / 2 > 0 ? KK / 2 : 1];
    u32x2 vv8[MM];
    f32x4 sk[2], sv[2];
    if constexpr (CONV) {  // widened INT8 codes (finite), scales of the chunk
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kop[t][kk] = lck(buf & 1)[(4 * kk + g4) * kChunk + 16 * t + i];
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) {
        const int d = 16 * mm + i;
        vop[mm] = lcv(buf & 1)[d * 4 + (g4 ^ ((d >> 1) & 3))];
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sk[t] = *reinterpret_cast<const f32x4*>(lsc(buf) + 16 * t + 4 * g4);
        sv[t] = *reinterpret_cast<const f32x4*>(lsc(buf) + 32 + 16 * t + 4 * g4);
      }
    } else if constexpr (!KV8) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const int tau = 16 * t + i, j = 4 * kk + g4;
          kop[t][kk] = DMA ? lk(buf)[j * kChunk + tau] : lk(buf)[tau * XV + (j ^ (tau % XV))];
        }
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) {
        const int d = 16 * mm + i;
        vop[mm] = lv(buf)[d * 4 + (g4 ^ ((d >> 1) & 3))];
      }
      if (edge) {  // zero the V bits of tokens past the wave's keys (they may hold NaN)
        uint32_t keep[4];  // V word wd holds tokens t0 + 8*g4 + 2*wd, +1
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
          keep[wd] = (t0 + 8 * g4 + 2 * wd < cc ? 0x0000FFFFu : 0u) |
                     (t0 + 8 * g4 + 2 * wd + 1 < cc ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int mm = 0; mm < MM; ++mm)
#pragma unroll
          for (int wd = 0; wd < 4; ++wd) vop[mm][wd] &= keep[wd];
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int k2 = 0; k2 < KK / 2; ++k2) {
          const int tau = 16 * t + i, j = 4 * k2 + g4;
          kv8[t][k2] = DMA ? lk8(buf)[j * kChunk + tau] : lk8(buf)[tau * XV8 + (j ^ (tau % XV8))];
        }
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) {
        const int d = 16 * mm + i;
        vv8[mm] = lv8(buf)[d * 4 + (g4 ^ ((d >> 2) & 3))];
      }
      if constexpr (kFp8Codes<Ty>) {
        if (edge) {  // zero the codes of tokens past the wave's keys (an unwritten slot may hold NaN)
          const uint32_t keep0 = bytes_before(t0 + 8 * g4, cc), keep1 = bytes_before(t0 + 8 * g4 + 4, cc);
#pragma unroll
          for (int mm = 0; mm < MM; ++mm) {
            vv8[mm][0] &= keep0;
            vv8[mm][1] &= keep1;
          }
        }
      }
      // scales of tokens 16*t + 4*g4 .. +3 (K, then V)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sk[t] = *reinterpret_cast<const f32x4*>(lsc(buf) + 16 * t + 4 * g4);
        sv[t] = *reinterpret_cast<const f32x4*>(lsc(buf) + 32 + 16 * t + 4 * g4);
      }
    }
#pragma unroll
    for (int nc = 0; nc < NC; ++nc) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if constexpr (!KV8 || CONV) {
          s0 = Ty::mma(__builtin_bit_cast(V8, kop[0][kk]), qop[nc][kk], s0);
          s1 = Ty::mma(__builtin_bit_cast(V8, kop[1][kk]), qop[nc][kk], s1);
        } else {  // product kk takes half kk % 2 of code vector kk / 2
          const u32x4 a = kv8[0][kk >> 1], b = kv8[1][kk >> 1];
          const u32x2 ha = (kk & 1) ? u32x2{a[2], a[3]} : u32x2{a[0], a[1]};
          const u32x2 hb = (kk & 1) ? u32x2{b[2], b[3]} : u32x2{b[0], b[1]};
          s0 = Ty::mma(__builtin_bit_cast(V8, codes_to_operand<Ty>(ha)), qop[nc][kk], s0);
          s1 = Ty::mma(__builtin_bit_cast(V8, codes_to_operand<Ty>(hb)), qop[nc][kk], s1);
        }
      }
      if constexpr (KV8) {  // logits of INT8 keys: code dot q times the token's scale
        s0 *= sk[0];
        s1 *= sk[1];
      }
      // y[e]: unscaled logit of token t0 + 4*g4 + e (e < 4) or t0 + 16 + 4*g4
      // + e - 4 (e >= 4); its base-2 logit is y[e] * sc.
      float y[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[j] = s0[j];
        y[4 + j] = s1[j];
      }
      float svc[8];  // INT8: V scales, 0 for dropped tokens (a scale may be NaN)
#pragma unroll
      for (int e = 0; e < 8; ++e) svc[e] = KV8 ? sv[e >> 2][e & 3] : 0.f;
      if (edge) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (t0 + 4 * g4 + (e & 3) + 16 * (e >> 2) >= lim[nc]) {
            y[e] = -INFINITY;
            svc[e] = 0.f;
          }
      }
      // The reference maximum moves only when some column's chunk maximum
      // passes it by more than kSlack, that is when some unscaled logit
      // exceeds the column's threshold; only then is the chunk maximum formed.
      bool above = false;
#pragma unroll
      for (int e = 0; e < 8; ++e) above |= y[e] > thr[nc];
      if (__builtin_amdgcn_ballot_w64(above) != 0) {
        float my = fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])),
                         fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
        // maximum over the 4 row groups (lanes i, i+16, i+32, i+48 hold
        // column i): each lane-row swap of two copies leaves a lane's
        // partner value in one of the pair
        const auto h32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(my), __float_as_uint(my),
                                                          false, false);
        my = fmaxf(__uint_as_float(h32[0]), __uint_as_float(h32[1]));
        const auto h16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(my), __float_as_uint(my),
                                                          false, false);
        my = fmaxf(__uint_as_float(h16[0]), __uint_as_float(h16[1]));
        const float m_new = fmaxf(m_run[nc], my * sc);
        if (m_new > m_run[nc]) {
          const float alpha = m_run[nc] == -INFINITY ? 0.f : exp2_fast(m_run[nc] - m_new);
          m_run[nc] = m_new;
          thr[nc] = (m_new + kSlack) * inv_sc;
          l_run[nc] *= alpha;
#pragma unroll
          for (int mm = 0; mm < MM; ++mm) acc[nc][mm] *= alpha;
        }
      }
      const float neg_m = m_run[nc] == -INFINITY ? 0.f : -m_run[nc];
      uint32_t pw[4];
      if constexpr (!KV8) {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
          pw[wd] = Ty::pack2(exp2_fast(fmaf(y[2 * wd], sc, neg_m)),
                             exp2_fast(fmaf(y[2 * wd + 1], sc, neg_m)));
      } else {
        // INT8 values: the PV product sees weight * V scale per token; the sum
        // takes rounded(p * s) / s, as in decode (a token with scale 0 counts
        // with its weight p).
        float pr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = exp2_fast(fmaf(y[e], sc, neg_m));
        float psum = l_run[nc];
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const float s0w = svc[2 * wd], s1w = svc[2 * wd + 1];
          pw[wd] = Ty::pack2(pr[2 * wd] * s0w, pr[2 * wd + 1] * s1w);
          psum += s0w != 0.f ? Ty::lo_f32(pw[wd]) * __builtin_amdgcn_rcpf(s0w) : pr[2 * wd];
          psum += s1w != 0.f ? Ty::hi_f32(pw[wd]) * __builtin_amdgcn_rcpf(s1w) : pr[2 * wd + 1];
        }
        l_run[nc] = psum;
      }
      const auto a32 = __builtin_amdgcn_permlane32_swap(pw[0], pw[2], false, false);
      const auto b32 = __builtin_amdgcn_permlane32_swap(pw[1], pw[3], false, false);
      const auto a16 = __builtin_amdgcn_permlane16_swap(a32[0], a32[1], false, false);
      const auto b16 = __builtin_amdgcn_permlane16_swap(b32[0], b32[1], false, false);
      const u32x4 pwords = {a16[0], b16[0], a16[1], b16[1]};
      if constexpr (!KV8) {
        // the weights the PV product sees, summed after the swaps: the four
        // lanes of a column hold the same weights in another order
        float psum = l_run[nc];
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) psum = Ty::sum2(pwords[wd], psum);
        l_run[nc] = psum;
      }
      const V8 pop = __builtin_bit_cast(V8, pwords);
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) {
        if constexpr (!KV8 || CONV)
          acc[nc][mm] = Ty::mma(__builtin_bit_cast(V8, vop[mm]), pop, acc[nc][mm]);
        else
          acc[nc][mm] = Ty::mma(__builtin_bit_cast(V8, codes_to_operand<Ty>(vv8[mm])), pop, acc[nc][mm]);
      }
    }
  };

  if constexpr (DMA) {
    // Chunk k goes from global memory straight into LDS buffer k % 4, each
    // lane's 16-byte vector to its own place: instruction r of wave w fills
    // vectors 64 (NW r + w) .. +63 of the buffer's K part and of its V part.
    // K is stored x-vector major (vector (token tau, x-vector j) at j * 32 +
    // tau): 16 lanes of an operand read take 16 consecutive vectors, and the
    // lanes of a load instruction read 32 consecutive tokens of an x-vector
    // (256 contiguous bytes per block).  V keeps the swizzled order of the
    // register-staged path.
    auto dma = [&](int k, int buf) {
      __builtin_amdgcn_s_setprio(2);
      if (k > 0 && k % CPB == 0) load_batch(k);
      const int e = (k % CPB) * BPC;
      int b[BPC];
#pragma unroll
      for (int j = 0; j < BPC; ++j) b[j] = __builtin_amdgcn_readlane(tbl, e + j);
      const int r0 = BS > kChunk ? (t_begin + k * kChunk) % BS : 0;
      auto at = [&](int tau, int64_t& off, int& row) {
        const int id = pick_block<BPC>(b, tau / BS);
        off = (int64_t)id * blk_stride + head_off;
        row = BS >= kChunk ? r0 + tau : tau % BS;
      };
      if constexpr (!KV8) {
        // Vector u = 64 (NW r + w) + lane of instruction r: K x-vector u / 32
        // of token u % 32 = lane % 32; V channel d = u / 4 and token group qd
        // = (u % 4) ^ ((d / 2) % 4), which is (lane % 4) ^ ((lane / 8) % 4)
        // for every r.  So a lane's K token and V token group, and their
        // blocks, are the same in all its instructions of a chunk.
        int64_t ok, ov;
        int rk, rv;
        at(lane & (kChunk - 1), ok, rk);
        at(8 * ((lane & 3) ^ ((lane >> 3) & 3)), ov, rv);
        const Elem* ksrc = kc + ok + rk * 8 + (lane >> 5) * BS * 8;
        const Elem* vsrc = vc + ov + rv + (lane >> 2) * BS;
#pragma unroll
        for (int r = 0; r < PER; ++r) {
          const int base = 64 * (NW * r + w);  // first vector of the instruction
          load_to_lds16(ksrc + (int64_t)(2 * (NW * r + w)) * BS * 8, lk(buf) + base);
          load_to_lds16(vsrc + (int64_t)(16 * (NW * r + w)) * BS, lv(buf) + base);
        }
      } else {
        // K codes: vector u = 64 w + lane (waves w < CK8 / 64), x-vector u / 32
        // of token lane % 32, stored x-vector major like the 16-bit K.
        int64_t off;
        int row;
        if (w < CK8 / 64) {
          at(lane & (kChunk - 1), off, row);
          load_to_lds16(kc + off + (((64 * w + lane) >> 5) * BS + row) * 16, lk8(buf) + 64 * w);
        }
        // V codes in 4-byte halves of the 8-byte runs: dword v = 64 X + lane
        // (X = NW r + w) of the buffer's V part is half v % 2 of run v / 2,
        // which is channel d = run / 4, token group (run % 4) ^ ((d / 4) % 4)
        // (the swizzled order the operand reads expect).
#pragma unroll
        for (int r = 0; r < RV8; ++r) {
          const int X = NW * r + w;
          const int run = 32 * X + (lane >> 1);
          const int d = run >> 2, qd = (run & 3) ^ ((d >> 2) & 3);
          at(8 * qd, off, row);
          load_to_lds4(vc + off + d * BS + row + 4 * (lane & 1),
                       reinterpret_cast<uint8_t*>(lv8(buf)) + 256 * X);
        }
        // scales (wave 0): lane l < 32 the K scale of token l, else the V
        // scale of token l - 32
        if (w == 0) {
          at(lane & (kChunk - 1), off, row);
          load_to_lds4((lane < 32 ? kc : vc) + off + I8Tile<D, BS>::kScales + 4 * row, lsc(buf));
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // Three chunks in flight while one is computed.  At step k the wave
    // waits for its own loads of chunk k (in-order completion: the loads of
    // chunks k + 1 and k + 2, 2 PER each, may stay outstanding), the barrier
    // then covers every wave's loads of chunk k and every wave's reads of
    // buffer (k - 1) % 4 in step k - 1, which chunk k + 3 then overwrites.
    // Every wave takes every barrier (n_chunks is the workgroup's).
    // The first three chunks are issued unconditionally (a chunk past
    // n_chunks reads block 0 into a buffer no step reads), so that the
    // compiler knows how many loads follow q's and does not wait for them
    // all before the first step.
    // load instructions per chunk of this wave
    const int pc = KV8 ? (w < CK8 / 64 ? 1 : 0) + RV8 + (w == 0 ? 1 : 0) : 2 * PER;
#pragma unroll
    for (int j = 0; j < 3; ++j) dma(j, j);
    if constexpr (!CONV) {
      for (int k = 0; k < n_chunks; ++k) {
        if (k + 2 < n_chunks) wait_vmcnt_upto(2 * pc);
        else if (k + 1 < n_chunks) wait_vmcnt_upto(pc);
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        if (k + 3 < n_chunks) dma(k + 3, (k + 3) & 3);
        if (k < n_mine) compute(k, k & 3);
      }
    } else {
      // Chunk j's codes (buffer j % 4) widened to 16-bit operands in
      // conversion buffer j % 2, each thread a share: K code vector g (token
      // g % 32, channels 16 (g / 32) ..) becomes 16-bit x-vectors 2 (g / 32)
      // and 2 (g / 32) + 1, V code run g (channel g / 4, token group g % 4)
      // one 16-bit vector.  The exact small integers feed the matrix cores
      // as in the per-wave widening; the scales stay in the code buffer.
      // FP8 codes of tokens past the workgroup's keys are zeroed first (an
      // unwritten slot may hold a NaN code, which would meet a zero weight).
      auto convert = [&](int j) {
        const int cb = j & 3, ob = j & 1;
        const int t0 = t_begin + j * kChunk;
        const bool tail = kFp8Codes<Ty> && t0 + kChunk > c_load;
        // static trip counts (one K vector and two V runs per thread at D = 128):
        // measured on MI355X, FP8 253 -> 244 us, INT8 at block size 32 254 -> 235
        // us (no spill), INT8 at block size 16 248 -> 251 us
        constexpr int RK = (CK8 + 64 * NW - 1) / (64 * NW), RV = (CV8 + 64 * NW - 1) / (64 * NW);
#pragma unroll
        for (int r = 0; r < RK; ++r) {
          const int g = tid + 64 * NW * r;
          if (CK8 % (64 * NW) != 0 && g >= CK8) break;
          const int tau = g & (kChunk - 1), j8 = g / kChunk;
          u32x4 c = lk8(cb)[j8 * kChunk + tau];
          if (tail && t0 + tau >= c_load) c = u32x4{0u, 0u, 0u, 0u};
          lck(ob)[2 * j8 * kChunk + tau] = codes_to_operand<Ty>(u32x2{c[0], c[1]});
          lck(ob)[(2 * j8 + 1) * kChunk + tau] = codes_to_operand<Ty>(u32x2{c[2], c[3]});
        }
#pragma unroll
        for (int r = 0; r < RV; ++r) {
          const int g = tid + 64 * NW * r;
          if (CV8 % (64 * NW) != 0 && g >= CV8) break;
          const int d = g >> 2, qd = g & 3;
          u32x2 c = lv8(cb)[d * 4 + (qd ^ ((d >> 2) & 3))];
          if (tail) c = u32x2{c[0] & bytes_before(t0 + 8 * qd, c_load), c[1] & bytes_before(t0 + 8 * qd + 4, c_load)};
          lcv(ob)[d * 4 + (qd ^ ((d >> 1) & 3))] = codes_to_operand<Ty>(c);
        }
      };
      // Step k: the wave's own loads of chunk k + 1 are done (chunk k + 2's
      // may stay outstanding) and so are its LDS writes of conversion k;
      // after the barrier chunk k + 1's codes and chunk k's 16-bit operands
      // are in LDS for every wave, and nobody reads code buffer (k - 1) % 4
      // (converted in step k - 2, its scales read in step k - 1) or
      // conversion buffer (k + 1) % 2 (read in step k - 1) any more.  Every
      // wave takes every barrier.
      if (1 < n_chunks) wait_vmcnt_upto(2 * pc);
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      convert(0);
      for (int k = 0; k < n_chunks; ++k) {
        if (k + 2 < n_chunks) wait_vmcnt_upto(pc);
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));  // lgkmcnt(0): the conversion's LDS writes
        __builtin_amdgcn_s_barrier();
        if (k + 3 < n_chunks) dma(k + 3, (k + 3) & 3);
        if (k + 1 < n_chunks) convert(k + 1);
        if (k < n_mine) compute(k, k & 3);
      }
    }
    wait_vmcnt<0>();  // no load may still write this workgroup's LDS when it ends
  } else {
  // Chunk k is computed from buffer k % 2 while chunks k + 1 (in registers)
  // and k + 2 (being loaded) are in flight; the barrier after each step makes
  // the next chunk visible and frees the buffer just read.  Every wave takes
  // every barrier (n_chunks is the workgroup's).
  Stage st_a, st_b;
  gload(0, st_a);
  if (1 < n_chunks) gload(1, st_b);
  swrite(0, st_a);
  __syncthreads();
  for (int k = 0; k < n_chunks; k += 2) {
    if (k + 2 < n_chunks) gload(k + 2, st_a);
    if (k < n_mine) compute(k, 0);
    if (k + 1 < n_chunks) swrite(1, st_b);
    __syncthreads();
    if (k + 1 >= n_chunks) break;
    if (k + 3 < n_chunks) gload(k + 3, st_b);
    if (k + 1 < n_mine) compute(k + 1, 1);
    if (k + 2 < n_chunks) swrite(0, st_a);
    __syncthreads();
  }
  }

#pragma unroll
  for (int nc = 0; nc < NC; ++nc) {
    float l_tot = l_run[nc] + __shfl_xor(l_run[nc], 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!head_ok[nc]) continue;
    if constexpr (!PFX) {  // the row's output
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* orow = out + out_row(16 * nc + i) * D + 4 * g4;
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) {
        const f32x4 r = acc[nc][mm] * inv;
        *reinterpret_cast<u32x2*>(orow + 16 * mm) = u32x2{Ty::pack2(r[0], r[1]), Ty::pack2(r[2], r[3])};
      }
    } else {  // partial slot p of the row: max, sum, unnormalised output
      const int64_t idx = out_row(16 * nc + i) * max_parts + p;
      float* arow = ws_acc + idx * D + 4 * g4;
#pragma unroll
      for (int mm = 0; mm < MM; ++mm) *reinterpret_cast<f32x4*>(arow + 16 * mm) = acc[nc][mm];
      if (g4 == 0) {
        ws_ml[2 * idx] = m_run[nc];
        ws_ml[2 * idx + 1] = l_tot;
      }
    }
  }
}

// Two waves per SIMD at least (at most 256 registers): the INT8 kernels at
// block size 32 would otherwise take 260 and run one wave per SIMD (measured
// on MI355X: 367 us against 250 us with 12 bytes of spill; with the widening
// loops unrolled they now fit, and only the FP8 f16 / bf16 ones at block size
// 32 spill, 12 bytes).
template <typename Ty, int D, int BS, int NW, int NC, bool KV8, bool PFX>
__global__ __launch_bounds__(64 * NW, 2) void prefill_lds_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const void* __restrict__ kcv,
    const void* __restrict__ vcv, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ qstart, int Hq, int Hkv, int G,
    int NB, int max_blocks, int max_ctx, int max_q, int num_rows, float scale_log2,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, int P, int max_parts,
    const int32_t* __restrict__ grp_len) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[PrefillLds<D, KV8, kPrefillDma<KV8, PFX>>::kBytes];
  prefill_lds_body<Ty, D, BS, NW, NC, KV8, PFX>(blockIdx.x, blockIdx.y, blockIdx.z, gridDim.x,
                                                gridDim.y, gridDim.z, lds_raw, out, q, kcv, vcv, tables, lens, qstart, Hq, Hkv, G, NB, max_blocks, max_ctx, max_q,
      num_rows, scale_log2, ws_acc, ws_ml, P, max_parts, grp_len);
}

// Waves per workgroup of the 16-bit kernel (measured best on MI355X among 1,
// 2, 4 and 8 for the workloads of the tests and the benchmark).
constexpr int kWaves = 4;
// Column groups of 16 slots per wave in the shared-prefix pass, which stages
// its chunks through registers (INT8 caches take one, so that the widened
// operands fit 3 waves per SIMD).
constexpr int kLdsGroups = 2;
// Column groups per wave of the prefill pass proper, whose chunks go straight
// to LDS.  Measured on MI355X (chunked prefill at LLaMA-13B shape): 16-bit
// caches 176.9 -> 171.6 us with three groups (256 VGPRs, still 2 waves per
// SIMD, although 512-row chunks then fill 3 tiles of 192 slots); INT8 caches
// 264 -> 359 us with three (314 registers, 1 wave per SIMD), so they keep two.
template <bool KV8>
constexpr int kPrefillGroups = KV8 ? 2 : 3;

// ----------------------------------------------------------------------------
// pa_decode_prefix in one launch.  The shared-prefix pass and the members'
// own tokens are independent (they fill different partial slots), so one
// grid holds both: workgroups 0 .. n_pre - 1 are the prefix pass over a
// (px, py, pz) grid (prefill_lds_body with PFX), the rest the decode pass
// over a (dx, dy, dz) grid (decode_mfma_body).  The short prefix
// workgroups then run beside the decode ones instead of before them.  The
// LDS is the larger of the two passes' needs.
// ----------------------------------------------------------------------------
template <int NW, int D>
struct FusedLds {
  static constexpr int kMerge = (2 * NW * 16 + NW * 16 * (D + 4)) * 4;  // merge_lds_bytes at G >= 16
  static constexpr int kBytes = kMerge > PrefillLds<D, false>::kBytes ? kMerge : PrefillLds<D, false>::kBytes;
};

template <typename Ty, int D, int BS, int NW, bool KV8>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(KV8 ? 3 : 1))) void prefix_suffix_kernel(
    int n_pre, int px, int py, int pz, int dx, int dy,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const void* __restrict__ kcv,
    const void* __restrict__ vcv, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, int Hq, int Hkv, int G, int n_groups, int NB,
    int max_blocks, int max_ctx, float scale_log2, int P, int max_parts,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, int num_seqs, int pre_parts, int pre_P,
    const int32_t* __restrict__ grp_start, const int32_t* __restrict__ grp_len, int n_grp) {
  static_assert(PrefillLds<D, KV8>::kBytes <= FusedLds<NW, D>::kBytes, "LDS of the fused launch");
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[FusedLds<NW, D>::kBytes];
  const int L = blockIdx.x;
  if (L < n_pre) {
    constexpr int NC = KV8 ? 1 : kLdsGroups;
    prefill_lds_body<Ty, D, BS, NW, NC, KV8, true>(
        L % px, (L / px) % py, L / (px * py), px, py, pz, lds_raw, nullptr, q, kcv, vcv, tables,
        nullptr, grp_start, Hq, Hkv, G, NB, max_blocks, max_ctx, 0, num_seqs, scale_log2, ws_acc,
        ws_ml, pre_P, max_parts, grp_len);
  } else {
    const int M = L - n_pre;
    decode_mfma_body<Ty, D, BS, NW, KV8>(M % dx, (M / dx) % dy, M / (dx * dy),
                                         reinterpret_cast<float*>(lds_raw), out, q, kcv, vcv, tables, lens, k_new, v_new, Hq, Hkv, G, n_groups, NB, max_blocks,
        max_ctx, scale_log2, P, max_parts, ws_acc, ws_ml, 0, pre_parts, pre_P, grp_start,
        grp_len, n_grp);
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
    const int32_t* __restrict__ lens, const float* __restrict__ k_new,
    const float* __restrict__ v_new, int Hq, int Hkv, int G, int NB, int max_blocks,
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
  // fused append: token c - 1 is read from k_new / v_new ([S, Hkv, D])
  const int t_new = k_new != nullptr ? c - 1 : -1;
  const float* kn = k_new != nullptr ? k_new + ((int64_t)s * Hkv + hk) * D : nullptr;
  const float* vn = v_new != nullptr ? v_new + ((int64_t)s * Hkv + hk) * D : nullptr;

  for (int d = lane; d < D; d += kWave) qs[d] = q[((int64_t)s * Hq + h) * D + d];
  __syncthreads();

  float mloc = -INFINITY;
  for (int t = lane; t < n; t += kWave) {
    const int tok = t_begin + t;
    const int64_t b = clampi(trow[tok / BS], 0, NB - 1);
    const bool fresh = tok == t_new;
    const float* kb = fresh ? kn : kc + (b * Hkv + hk) * tile + (tok % BS) * 4;
    const int kstride = fresh ? 4 : BS * 4;
    float dot = 0.f;
#pragma unroll 4
    for (int cc = 0; cc < D / 4; ++cc) {
      const f32x4 k4 = *reinterpret_cast<const f32x4*>(kb + cc * kstride);
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
      const float v = tok == t_new ? vn[d] : vc[((b * Hkv + hk) * D + d) * BS + tok % BS];
      a = fmaf(xs[t], v, a);
    }
    // the cache write of the step: one workgroup per (sequence, KV head)
    if (t_new >= t_begin && t_new < t_begin + P && h == hk * G) {
      const int64_t b = clampi(trow[t_new / BS], 0, NB - 1);
      const int o = t_new % BS;
      const_cast<float*>(kc)[((b * Hkv + hk) * (D / 4) + d / 4) * BS * 4 + o * 4 + d % 4] = kn[d];
      const_cast<float*>(vc)[((b * Hkv + hk) * D + d) * BS + o] = vn[d];
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
// than one.  grid: x = query head, y = sequence; block = NT threads (128
// when every row has at most 32 partials, else 512).
// Thread (r, c4) walks partitions r, r + ROWS, ... keeping its own running
// (max, sum, output for channels 4*c4..+3) with the log-sum-exp rule, so one
// pass reads every live partial once and all loads of a batch are independent
// (they are issued once the context length gives the row's partition count).
// The ROWS states
// are then combined in LDS in row order, so the result depends only on the
// partition contents, never on where the blocks sit.
// ----------------------------------------------------------------------------
// The rows a merge launch covers, from the host copy of the context lengths:
// the sequences with more than one partition, one packed entry s | parts << 16
// each.  Passed by value as a kernel argument; n = 0 means no list (the grid
// covers every sequence, and each workgroup reads its length).
constexpr int kMaxSplit = 512;
struct SplitList {
  int32_t n;
  uint32_t e[kMaxSplit];
};

template <typename Store, int D, int NT>
__global__ __launch_bounds__(NT) void merge_kernel(
    typename Store::T* __restrict__ out, const int32_t* __restrict__ lens,
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml, int Hq, int max_ctx,
    int max_blocks, int BS, int P, int max_parts, const int32_t* __restrict__ grp_start,
    const int32_t* __restrict__ grp_len, int n_grp, int pre_parts, int pre_P, SplitList split) {
  constexpr int C4 = D / 4;                   // threads per partition row
  constexpr int ROWS = NT / C4;               // partitions read at once
  constexpr int U = 8;                        // partitions per thread per batch
  __shared__ float sm[ROWS][C4], sl[ROWS][C4];
  __shared__ f32x4 so[ROWS][C4];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int r = tid / C4, c4 = tid - r * C4;
  int s, n_p, skip = 0;
  if (split.n > 0) {  // a split sequence of the host's list: no length to read
    s = (int)(split.e[blockIdx.y] & 0xFFFFu);
    n_p = min((int)(split.e[blockIdx.y] >> 16), max_parts);
  } else {
    s = blockIdx.y;
    const int c = clampi(lens[s], 0, min(max_ctx, max_blocks * BS));
    // With prefix groups, partial 0 is the shared prefix (when the
    // sequence's group has one) and the decode partitions follow.
    if (n_grp > 0) {
      int lo = 0, hi = n_grp - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (grp_start[mid] <= s) lo = mid;
        else hi = mid - 1;
      }
      skip = clampi(grp_len[lo], 0, min(c, pre_parts * pre_P));
    }
    n_p = min((n_grp > 0 ? (skip + pre_P - 1) / pre_P : 0) +
                  (c - (skip & ~(kChunk - 1)) + P - 1) / P,
              max_parts);
    if (n_p <= 1 && skip == 0) return;  // pass 1 stored the output itself
  }
  const int64_t base = ((int64_t)s * Hq + h) * max_parts;
  // Only the row's own partials are read (the length is known first): a
  // speculative batch over max_parts slots read several times the live
  // bytes on mixed-length batches.
  Lse st = {-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
  float bm[U], bl[U];
  f32x4 bo[U];
  for (int p0 = r; p0 < n_p; p0 += U * ROWS) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int pp = min(p0 + k * ROWS, n_p - 1);
      bm[k] = ws_ml[2 * (base + pp)];
      bl[k] = ws_ml[2 * (base + pp) + 1];
      bo[k] = *reinterpret_cast<const f32x4*>(ws_acc + (base + pp) * D + 4 * c4);
    }
#pragma unroll
    for (int k = 0; k < U; ++k)
      if (p0 + k * ROWS < n_p) lse_add(st, bm[k], bl[k], bo[k]);
  }
  sm[r][c4] = st.m;
  sl[r][c4] = st.l;
  so[r][c4] = st.o;
  __syncthreads();
  if (r == 0) {
    Lse tot = {sm[0][c4], sl[0][c4], so[0][c4]};
#pragma unroll
    for (int rr = 1; rr < ROWS; ++rr)
      if (rr < n_p) lse_add(tot, sm[rr][c4], sl[rr][c4], so[rr][c4]);
    Store::put(out + ((int64_t)s * Hq + h) * D + 4 * c4, tot.o * (tot.l > 0.f ? 1.f / tot.l : 0.f));
  }
}

struct StoreF32 {
  using T = float;
  static __device__ __forceinline__ void put(float* dst, f32x4 v) {
    *reinterpret_cast<f32x4*>(dst) = v;
  }
};

template <typename Ty>
struct Store16 {
  using T = uint16_t;
  static __device__ __forceinline__ void put(uint16_t* dst, f32x4 v) {
    *reinterpret_cast<u32x2*>(dst) =
        u32x2{(uint32_t)Ty::from_f32(v[0]) | ((uint32_t)Ty::from_f32(v[1]) << 16),
              (uint32_t)Ty::from_f32(v[2]) | ((uint32_t)Ty::from_f32(v[3]) << 16)};
  }
};

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
struct Plan {
  int P = 0;          // partition size in tokens
  int max_parts = 0;  // partitions of the longest context
  int groups = 1;     // query-head groups of 16 per KV head (16-bit kernel)
  bool flat = true;   // flat (sequence, partition) work list (16-bit kernel)
  size_t ws_bytes = 0;
  // shared-prefix groups (pa_decode_prefix): partial 0 of a member is its
  // group's prefix, computed by the prefix pass
  const int32_t* grp_start = nullptr;
  const int32_t* grp_len = nullptr;
  int n_grp = 0;
  int max_group = 0;
  int pre_parts = 0;  // partitions of the longest shared prefix
  int pre_P = 0;      // tokens per partition of the shared prefixes
  int own_parts = 0;  // partitions of the longest run of a member's own tokens
  // (sequence, partition) units of the flat work list, from the host copy of
  // the context lengths (0 = unknown: the grid covers num_seqs * max_parts)
  int64_t units = 0;
  // the flat list's units longest first (n = 0: sequence order, in-kernel)
  UnitList order;
  Plan() { order.n = 0; }
  // both products on the vector ALU (decode_mfma_kernel with VaWaveDecoder)
  bool valu = false;
};

pa_status validate(const pa_decode_args* a) {
  if (!a) return PA_ERR_INVALID;
  if (!elem_bytes(a->dtype)) return PA_ERR_INVALID;
  // the caches hold q's type, or 8-bit codes with scales under 16-bit queries
  if (a->kv_dtype != a->dtype && !(is_q8(a->kv_dtype) && a->dtype != PA_F32))
    return PA_ERR_INVALID;
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
  if (a->block_size != 8 && a->block_size != 16 && a->block_size != 32 && a->block_size != 64)
    return PA_ERR_UNSUPPORTED;
  if (a->dtype == PA_F32 && a->partition_size > kMaxF32Part) return PA_ERR_UNSUPPORTED;
  if (a->products < PA_PRODUCTS_AUTO || a->products > PA_PRODUCTS_VALU) return PA_ERR_INVALID;
  if (a->products == PA_PRODUCTS_VALU &&
      (a->num_q_heads != a->num_kv_heads || is_q8(a->kv_dtype) || a->dtype == PA_F32))
    return PA_ERR_UNSUPPORTED;
  if (a->context_lens_host)
    for (int s = 0; s < a->num_seqs; ++s)
      if (a->context_lens_host[s] < 0 || a->context_lens_host[s] > a->max_context_len)
        return PA_ERR_INVALID;
  return PA_OK;
}

// Partition size when the caller leaves it to the library.
// Measured on MI355X (non-temporal loads, 4 waves per workgroup): a
// workgroup streams best when it walks a long run of tokens, but splits must
// leave enough workgroups to keep every CU's loads in flight, and with mixed
// lengths long runs leave a tail of late-starting long workgroups.  So:
//   - contexts up to 2048 tokens are not split when the (sequence, KV head,
//     head group) workgroups alone fill the chip (>= 512 of them);
//   - otherwise P = max_context / 16 rounded up to a power of two within
//     [256, 4096] tokens, halved (down to one 32-token chunk) while fewer
//     than 1024 workgroups would exist even if every context were maximal.
// Measured on MI355X (4 sequences of 16k..128k tokens, 8 KV heads): P = 512
// 185 us, 1024 171 us, 2048 162 us, 4096 156 us.  8-bit caches move half the
// bytes per token, so a split pays for its merge at twice the tokens: P starts
// from max_context / 8 (measured, mixed-length batch of 64 sequences up to
// 7.6k tokens: INT8 P = 512 43.0 us, 768 40.6, 1024 40.8, 2048 40.5; FP8
// 41.8, 39.9, 39.9, 39.9).
int choose_partition(const pa_decode_args* a, int wg_per_part) {
  if (a->dtype == PA_F32) return 512;
  const int64_t base = (int64_t)a->num_seqs * wg_per_part;
  const int64_t max_ctx = a->max_context_len;
  if (max_ctx <= 2048 && base >= 512) return 2048;
  const int per = is_q8(a->kv_dtype) ? 8 : 16;
  int P = 256;
  while (P < 4096 && (int64_t)P * per < max_ctx) P *= 2;
  while (P > kChunk && base * ((max_ctx + P - 1) / P) < 1024) P /= 2;
  return max(P, a->block_size);  // a power of two >= 32: a multiple of the block size
}

// Products of the G = 1 case when the caller leaves the choice to the library.
constexpr bool kValuForMha = false;

Plan make_plan(const pa_decode_args* a) {
  Plan pl;
  const int G = a->num_q_heads / a->num_kv_heads;
  pl.groups = a->dtype == PA_F32 ? 1 : (G + 15) / 16;
  const int wg_per_part = a->dtype == PA_F32 ? a->num_q_heads : a->num_kv_heads * pl.groups;
  pl.P = a->partition_size > 0 ? a->partition_size : choose_partition(a, wg_per_part);
  pl.max_parts = (a->max_context_len + pl.P - 1) / pl.P;
  // The flat work list pays off when contexts of different lengths leave
  // many of the S x max_parts slots empty (measured: mixed-length batch at
  // 1024-token partitions 108 -> 80 us); with one to three partitions per
  // sequence its prefix-sum prologue costs more than the few empty slots.
  // It walks the context lengths 64 at a time and needs one grid row per
  // (sequence, partition) slot.
  pl.flat = pl.max_parts >= 4 && a->num_seqs <= 1024 &&
            (int64_t)a->num_seqs * pl.max_parts <= 65535;
  if (pl.flat && a->context_lens_host) {
    // the kernel's own count: every sequence has max(ceil(c / P), 1) units
    for (int s = 0; s < a->num_seqs; ++s)
      pl.units += max((a->context_lens_host[s] + pl.P - 1) / pl.P, 1);
    // Longest unit first (ties in sequence order): the last units to start
    // are the short tails of the sequences, so the workgroups still running
    // when the grid drains are short ones.
    if (pl.units <= kMaxUnits) {
      int n = 0;
      for (int s = 0; s < a->num_seqs; ++s) {
        const int c = a->context_lens_host[s];
        const int parts = max((c + pl.P - 1) / pl.P, 1);
        for (int p = 0; p < parts; ++p) pl.order.e[n++] = (uint32_t)s | ((uint32_t)p << 16);
      }
      auto tokens = [&](uint32_t e) {
        const int c = a->context_lens_host[e & 0xFFFFu];
        return min(pl.P, c - (int)(e >> 16) * pl.P);
      };
      std::stable_sort(pl.order.e, pl.order.e + n,
                       [&](uint32_t x, uint32_t y) { return tokens(x) > tokens(y); });
      pl.order.n = n;
    }
  }
  if (pl.max_parts > 1)
    pl.ws_bytes = (size_t)a->num_seqs * a->num_q_heads * pl.max_parts * (a->head_dim + 2) * 4;
  pl.valu = G == 1 && !is_q8(a->kv_dtype) && a->dtype != PA_F32 &&
            (a->products == PA_PRODUCTS_VALU || (a->products == PA_PRODUCTS_AUTO && kValuForMha));
  return pl;
}

size_t merge_lds_bytes(int NW, int G, int D) {
  return (size_t)(2 * NW * 16 + NW * min(G, 16) * (D + 4)) * sizeof(float);
}


template <typename Ty, int D, int BS, int NW, bool KV8, bool VALU = false>
void launch_mfma(const pa_decode_args* a, const Plan& pl, float* ws_acc, float* ws_ml,
                 hipStream_t st) {
  const int G = a->num_q_heads / a->num_kv_heads;
  const bool flat = pl.flat;
  // partitions of the longest context (with prefix groups, the partial
  // slots also hold the prefix partitions, which this launch does not cover)
  const int dec_parts = max((a->max_context_len + pl.P - 1) / pl.P, 1);
  dim3 grid((unsigned)(a->num_kv_heads * pl.groups),
            flat ? (unsigned)(pl.units > 0 ? pl.units : (int64_t)a->num_seqs * dec_parts)
                 : (unsigned)dec_parts,
            flat ? 1u : (unsigned)a->num_seqs);
  decode_mfma_kernel<Ty, D, BS, NW, KV8, VALU><<<grid, 64 * NW, merge_lds_bytes(NW, G, D), st>>>(
      (uint16_t*)a->out, (const uint16_t*)a->q, a->k_cache, a->v_cache, a->block_tables,
      a->context_lens, (const uint16_t*)a->k_new, (const uint16_t*)a->v_new, a->num_q_heads,
      a->num_kv_heads, G, pl.groups, a->num_blocks, a->max_blocks_per_seq, a->max_context_len,
      a->scale * kLog2e, pl.P, max(pl.max_parts, 1), ws_acc, ws_ml, flat ? a->num_seqs : 0,
      pl.pre_parts, pl.pre_P, pl.grp_start, pl.grp_len, pl.n_grp, (int)!flat, pl.order);
}

// pa_decode_prefix: prefix_suffix_kernel, one launch of the shared-prefix
// pass (grid: slot tiles of the largest group x prefix partitions x group *
// Hkv + KV head; it writes partial slots 0 .. pre_parts - 1 of every member)
// followed in the same grid by the decode pass over each member's own tokens
// (KV head * head group x partitions x sequences).
int64_t fused_prefix_wgs(const pa_decode_args* a, const Plan& pl, int* px, int* py, int* pz) {
  const int G = a->num_q_heads / a->num_kv_heads;
  const int NC = is_q8(a->kv_dtype) ? 1 : kLdsGroups;
  const int64_t tiles = ((int64_t)pl.max_group * G + 16 * NC * kWaves - 1) / (16 * NC * kWaves);
  *px = (int)tiles;
  *py = pl.pre_parts;
  *pz = pl.n_grp * a->num_kv_heads;
  return tiles * pl.pre_parts * pz[0];
}

int64_t fused_decode_wgs(const pa_decode_args* a, const Plan& pl, int* dx, int* dy) {
  *dx = a->num_kv_heads * pl.groups;
  *dy = pl.own_parts;
  return (int64_t)dx[0] * dy[0] * a->num_seqs;
}

template <typename Ty, int D, int BS, int NW, bool KV8>
void launch_fused(const pa_decode_args* a, const Plan& pl, float* ws_acc, float* ws_ml,
                  hipStream_t st) {
  const int G = a->num_q_heads / a->num_kv_heads;
  int px, py, pz, dx, dy;
  const int64_t n_pre = fused_prefix_wgs(a, pl, &px, &py, &pz);
  const int64_t n_dec = fused_decode_wgs(a, pl, &dx, &dy);
  prefix_suffix_kernel<Ty, D, BS, NW, KV8><<<dim3((unsigned)(n_pre + n_dec)), 64 * NW, 0, st>>>(
      (int)n_pre, px, py, pz, dx, dy, (uint16_t*)a->out, (const uint16_t*)a->q, a->k_cache,
      a->v_cache, a->block_tables, a->context_lens, (const uint16_t*)a->k_new,
      (const uint16_t*)a->v_new, a->num_q_heads, a->num_kv_heads, G, pl.groups, a->num_blocks,
      a->max_blocks_per_seq, a->max_context_len, a->scale * kLog2e, pl.P, max(pl.max_parts, 1),
      ws_acc, ws_ml, a->num_seqs, pl.pre_parts, pl.pre_P, pl.grp_start, pl.grp_len, pl.n_grp);
}

template <typename Ty, bool KV8, int D>
void launch_fused_bs(const pa_decode_args* a, const Plan& pl, float* wa, float* wm,
                     hipStream_t st) {
  switch (a->block_size) {
    case 8: launch_fused<Ty, D, 8, kWaves, KV8>(a, pl, wa, wm, st); break;
    case 16: launch_fused<Ty, D, 16, kWaves, KV8>(a, pl, wa, wm, st); break;
    case 32: launch_fused<Ty, D, 32, kWaves, KV8>(a, pl, wa, wm, st); break;
    default: launch_fused<Ty, D, 64, kWaves, KV8>(a, pl, wa, wm, st); break;
  }
}

template <typename Ty, bool KV8>
void launch_fused_dims(const pa_decode_args* a, const Plan& pl, float* wa, float* wm,
                       hipStream_t st) {
  if (a->head_dim == 128) launch_fused_bs<Ty, KV8, 128>(a, pl, wa, wm, st);
  else launch_fused_bs<Ty, KV8, 64>(a, pl, wa, wm, st);
}

// Prefill: grid x = tiles of 16 (row, head) slots of the longest chunk, y =
// KV head, z = sequence; no split-K (each tile's key range is its own).

template <typename Ty, int D, int BS, int NW, bool KV8>
void launch_prefill(const pa_prefill_args* a, hipStream_t st) {
  const int G = a->num_q_heads / a->num_kv_heads;
  // K/V (or INT8 codes and scales) loaded straight into LDS, 16 * NC slots
  // per wave.  INT8 takes two column groups: without the register staging
  // they fit in 238 VGPRs with no spill (measured on MI355X, chunked prefill
  // at LLaMA-13B shape: 299 -> 262 us against one column group).
  constexpr int NC = kPrefillGroups<KV8>;
  const int64_t tiles = ((int64_t)a->max_query_len * G + 16 * NC * NW - 1) / (16 * NC * NW);
  dim3 grid((unsigned)tiles, (unsigned)a->num_kv_heads, (unsigned)a->num_seqs);
  prefill_lds_kernel<Ty, D, BS, NW, NC, KV8, false><<<grid, 64 * NW, 0, st>>>(
      (uint16_t*)a->out, (const uint16_t*)a->q, a->k_cache, a->v_cache, a->block_tables,
      a->context_lens, a->query_start, a->num_q_heads, a->num_kv_heads, G, a->num_blocks,
      a->max_blocks_per_seq, a->max_context_len, a->max_query_len, a->num_tokens,
      a->scale * kLog2e, nullptr, nullptr, 0, 0, nullptr);
}

template <typename Ty, bool KV8, int D>
void launch_prefill_bs(const pa_prefill_args* a, hipStream_t st) {
  switch (a->block_size) {
    case 8: launch_prefill<Ty, D, 8, kWaves, KV8>(a, st); break;
    case 16: launch_prefill<Ty, D, 16, kWaves, KV8>(a, st); break;
    case 32: launch_prefill<Ty, D, 32, kWaves, KV8>(a, st); break;
    default: launch_prefill<Ty, D, 64, kWaves, KV8>(a, st); break;
  }
}

template <typename Ty, bool KV8>
void launch_prefill_dims(const pa_prefill_args* a, hipStream_t st) {
  if (a->head_dim == 128) launch_prefill_bs<Ty, KV8, 128>(a, st);
  else launch_prefill_bs<Ty, KV8, 64>(a, st);
}

template <typename Ty, bool KV8, int D>
void launch_mfma_bs(const pa_decode_args* a, const Plan& pl, float* wa, float* wm,
                    hipStream_t st) {
  // INT8 caches on the flat work list with partitions of at most 512 tokens:
  // two waves per workgroup, 8 chunks each (INT8 waves keep one chunk in
  // flight, so four waves over 16 chunks spent much of their life in the
  // prologue and the LDS merge).  Measured on MI355X: mixed-length INT8 step
  // 47.4 -> 44.4 us, long context at P = 512 121.0 -> 118.1 us; at P = 4096
  // two waves over 128 chunks took 145 us instead of 102, hence the limit.
  if (KV8 && pl.flat && pl.P <= 512) {
    switch (a->block_size) {
      case 8: launch_mfma<Ty, D, 8, 2, KV8>(a, pl, wa, wm, st); break;
      case 16: launch_mfma<Ty, D, 16, 2, KV8>(a, pl, wa, wm, st); break;
      case 32: launch_mfma<Ty, D, 32, 2, KV8>(a, pl, wa, wm, st); break;
      default: launch_mfma<Ty, D, 64, 2, KV8>(a, pl, wa, wm, st); break;
    }
    return;
  }
  if constexpr (!KV8) {
    if (pl.valu) {  // one query head per KV head: both products on the vector ALU
      switch (a->block_size) {
        case 8: launch_mfma<Ty, D, 8, kWaves, false, true>(a, pl, wa, wm, st); break;
        case 16: launch_mfma<Ty, D, 16, kWaves, false, true>(a, pl, wa, wm, st); break;
        case 32: launch_mfma<Ty, D, 32, kWaves, false, true>(a, pl, wa, wm, st); break;
        default: launch_mfma<Ty, D, 64, kWaves, false, true>(a, pl, wa, wm, st); break;
      }
      return;
    }
  }
  switch (a->block_size) {
    case 8: launch_mfma<Ty, D, 8, kWaves, KV8>(a, pl, wa, wm, st); break;
    case 16: launch_mfma<Ty, D, 16, kWaves, KV8>(a, pl, wa, wm, st); break;
    case 32: launch_mfma<Ty, D, 32, kWaves, KV8>(a, pl, wa, wm, st); break;
    default: launch_mfma<Ty, D, 64, kWaves, KV8>(a, pl, wa, wm, st); break;
  }
}

template <typename Ty, bool KV8>
void launch_mfma_dims(const pa_decode_args* a, const Plan& pl, float* wa, float* wm,
                      hipStream_t st) {
  if (a->head_dim == 128) launch_mfma_bs<Ty, KV8, 128>(a, pl, wa, wm, st);
  else launch_mfma_bs<Ty, KV8, 64>(a, pl, wa, wm, st);
}

template <int D, int BS>
void launch_f32(const pa_decode_args* a, const Plan& pl, float* ws_acc, float* ws_ml,
                hipStream_t st) {
  const int G = a->num_q_heads / a->num_kv_heads;
  dim3 grid((unsigned)max(pl.max_parts, 1), (unsigned)a->num_q_heads, (unsigned)a->num_seqs);
  decode_f32_kernel<D, BS><<<grid, 64, 0, st>>>(
      (float*)a->out, (const float*)a->q, (const float*)a->k_cache, (const float*)a->v_cache,
      a->block_tables, a->context_lens, (const float*)a->k_new, (const float*)a->v_new,
      a->num_q_heads, a->num_kv_heads, G, a->num_blocks,
      a->max_blocks_per_seq, a->max_context_len, a->scale * kLog2e, pl.P, pl.max_parts, ws_acc,
      ws_ml);
}

template <int D>
void launch_f32_bs(const pa_decode_args* a, const Plan& pl, float* wa, float* wm, hipStream_t st) {
  switch (a->block_size) {
    case 8: launch_f32<D, 8>(a, pl, wa, wm, st); break;
    case 16: launch_f32<D, 16>(a, pl, wa, wm, st); break;
    case 32: launch_f32<D, 32>(a, pl, wa, wm, st); break;
    default: launch_f32<D, 64>(a, pl, wa, wm, st); break;
  }
}

template <typename Store, int D>
void launch_merge(const pa_decode_args* a, const Plan& pl, const float* wa, const float* wm,
                  hipStream_t st) {
  // With the host copy of the context lengths (and no prefix groups) the
  // grid covers only the split sequences; when none is split there is no
  // merge launch at all.  Measured on MI355X: mixed-length step 66.1 to
  // 65.7 us, with INT8 caches 47.6 to 47.1 us.
  SplitList sl;
  sl.n = 0;
  unsigned rows = (unsigned)a->num_seqs;
  if (a->context_lens_host && pl.n_grp == 0) {
    int n = 0;
    for (int s = 0; s < a->num_seqs && n >= 0; ++s) {
      const int parts = (a->context_lens_host[s] + pl.P - 1) / pl.P;
      if (parts <= 1) continue;
      if (n == kMaxSplit) {
        n = -1;  // too many for the list: every sequence reads its length
        break;
      }
      sl.e[n] = (uint32_t)s | ((uint32_t)parts << 16);
      ++n;
    }
    if (n == 0) return;
    if (n > 0) {
      sl.n = n;
      rows = (unsigned)n;
    }
  }
  dim3 grid((unsigned)a->num_q_heads, rows);
  if (pl.max_parts <= 32)  // one batch of loads per thread at D = 128
    merge_kernel<Store, D, 128><<<grid, 128, 0, st>>>(
        (typename Store::T*)a->out, a->context_lens, wa, wm, a->num_q_heads, a->max_context_len,
        a->max_blocks_per_seq, a->block_size, pl.P, pl.max_parts, pl.grp_start, pl.grp_len,
        pl.n_grp, pl.pre_parts, pl.pre_P, sl);
  else
    merge_kernel<Store, D, 512><<<grid, 512, 0, st>>>(
        (typename Store::T*)a->out, a->context_lens, wa, wm, a->num_q_heads, a->max_context_len,
        a->max_blocks_per_seq, a->block_size, pl.P, pl.max_parts, pl.grp_start, pl.grp_len,
        pl.n_grp, pl.pre_parts, pl.pre_P, sl);
}

template <typename Store>
void launch_merge_dims(const pa_decode_args* a, const Plan& pl, const float* wa,
                       const float* wm, hipStream_t st) {
  if (a->head_dim == 128) launch_merge<Store, 128>(a, pl, wa, wm, st);
  else launch_merge<Store, 64>(a, pl, wa, wm, st);
}

// Launches pass 1 and, when some context spans several partitions, pass 2.
pa_status run_plan(const pa_decode_args* a, const Plan& pl, hipStream_t hs) {
  float* ws_acc = nullptr;
  float* ws_ml = nullptr;
  if (pl.ws_bytes) {
    ws_acc = (float*)a->workspace;
    ws_ml = ws_acc + (size_t)a->num_seqs * a->num_q_heads * pl.max_parts * a->head_dim;
  }
  // 8-bit caches: the element type carries the code format (F16 / BF16:
  // INT8 codes; Fp8Elem: FP8)
  const bool kv8 = is_q8(a->kv_dtype), fp8 = a->kv_dtype == PA_FP8;
  if (pl.n_grp > 0) {  // shared prefixes and own tokens in one launch (16-bit queries only)
    if (a->dtype == PA_F16) {
      if (fp8) launch_fused_dims<Fp8Elem<F16>, true>(a, pl, ws_acc, ws_ml, hs);
      else if (kv8) launch_fused_dims<F16, true>(a, pl, ws_acc, ws_ml, hs);
      else launch_fused_dims<F16, false>(a, pl, ws_acc, ws_ml, hs);
    } else {
      if (fp8) launch_fused_dims<Fp8Elem<BF16>, true>(a, pl, ws_acc, ws_ml, hs);
      else if (kv8) launch_fused_dims<BF16, true>(a, pl, ws_acc, ws_ml, hs);
      else launch_fused_dims<BF16, false>(a, pl, ws_acc, ws_ml, hs);
    }
  } else switch (a->dtype) {
    case PA_F16:
      if (fp8) launch_mfma_dims<Fp8Elem<F16>, true>(a, pl, ws_acc, ws_ml, hs);
      else if (kv8) launch_mfma_dims<F16, true>(a, pl, ws_acc, ws_ml, hs);
      else launch_mfma_dims<F16, false>(a, pl, ws_acc, ws_ml, hs);
      break;
    case PA_BF16:
      if (fp8) launch_mfma_dims<Fp8Elem<BF16>, true>(a, pl, ws_acc, ws_ml, hs);
      else if (kv8) launch_mfma_dims<BF16, true>(a, pl, ws_acc, ws_ml, hs);
      else launch_mfma_dims<BF16, false>(a, pl, ws_acc, ws_ml, hs);
      break;
    default:
      if (a->head_dim == 128) launch_f32_bs<128>(a, pl, ws_acc, ws_ml, hs);
      else launch_f32_bs<64>(a, pl, ws_acc, ws_ml, hs);
  }
  pa_status st = launch_status();
  if (st != PA_OK) return st;
  if (pl.max_parts > 1 || pl.n_grp > 0) {
    switch (a->dtype) {
      case PA_F16: launch_merge_dims<Store16<F16>>(a, pl, ws_acc, ws_ml, hs); break;
      case PA_BF16: launch_merge_dims<Store16<BF16>>(a, pl, ws_acc, ws_ml, hs); break;
      default: launch_merge_dims<StoreF32>(a, pl, ws_acc, ws_ml, hs);
    }
    st = launch_status();
  }
  return st;
}

}  // namespace
}  // namespace pa

// ----------------------------------------------------------------------------
// Allocation-free decode (pa_decode_static): the split-K partials go to a
// file-scope device array instead of a caller workspace.  In host code the
// array's name is only a host-side stand-in; its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is passed to the kernels.
// ----------------------------------------------------------------------------
namespace pa {
namespace {

constexpr size_t kScratchBytes = PA_DECODE_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call per device).
pa_status scratch_on_current_device(hipStream_t stream, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return PA_ERR_HIP;
    if (sdev != dev) return PA_ERR_INVALID;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return PA_ERR_HIP;
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
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

PA_API int32_t pa_decode_products(const pa_decode_args* args) {
  if (validate(args) != PA_OK) return -1;
  return make_plan(args).valu ? PA_PRODUCTS_VALU : PA_PRODUCTS_MATRIX;
}

// Plan of a decode with shared-prefix groups: one partial slot for the
// prefix plus the decode partitions; always merged; no flat work list.
static pa_status prefix_plan(const pa_decode_args* a, const pa_prefix_groups* g, Plan& pl) {
  pa_status st = validate(a);
  if (st != PA_OK) return st;
  if (!g || g->num_groups < 0 || g->max_group_size < 0) return PA_ERR_INVALID;
  if (a->dtype == PA_F32) return PA_ERR_UNSUPPORTED;
  pl = make_plan(a);
  if (g->num_groups == 0) return PA_OK;  // plain decode
  if (!g->group_start || !g->prefix_len || g->max_group_size == 0 ||
      g->max_group_size > a->num_seqs || g->max_prefix_len < 0 ||
      g->max_prefix_len > a->max_context_len || g->min_prefix_len < 0 ||
      g->min_prefix_len > g->max_prefix_len)
    return PA_ERR_INVALID;
  if ((int64_t)g->num_groups * a->num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  pl.grp_start = g->group_start;
  pl.grp_len = g->prefix_len;
  pl.n_grp = g->num_groups;
  pl.max_group = g->max_group_size;
  pl.flat = false;
  // Prefix partitions of 256 tokens, doubled (up to 2048) while a long
  // prefix would leave more than 64 partials per row for the merge.  The
  // prefix workgroups run in the same launch as the members' own tokens, so
  // they need not fill the chip by themselves; a workgroup over 256 tokens
  // of 128 columns takes about as long as a decode workgroup.  Measured on
  // MI355X (32 members sharing 2048 tokens, 8 KV heads, G = 4): prefix
  // partitions of 64 tokens 31.9 us per step, 128 28.8, 256 25.2, 512 29.6,
  // 1024 44.9.
  {
    int pp = 256;
    while (pp < 2048 && (g->max_prefix_len + pp - 1) / pp > 64) pp *= 2;
    pl.pre_P = pp;
  }
  pl.pre_parts = max(1, (g->max_prefix_len + pl.pre_P - 1) / pl.pre_P);
  // A member's own tokens start at the 32-token boundary at or below its
  // prefix length, so with a host lower bound of the prefixes they span at
  // most max_context_len - floor32(min_prefix_len) tokens.
  pl.own_parts = max(1, (a->max_context_len - (g->min_prefix_len & ~(kChunk - 1)) + pl.P - 1) / pl.P);
  pl.max_parts = pl.pre_parts + (a->max_context_len + pl.P - 1) / pl.P;
  pl.ws_bytes = (size_t)a->num_seqs * a->num_q_heads * pl.max_parts * (a->head_dim + 2) * 4;
  return PA_OK;
}

PA_API pa_status pa_prefill(const pa_prefill_args* a, void* stream) {
  if (!a) return PA_ERR_INVALID;
  if (a->dtype != PA_F16 && a->dtype != PA_BF16) {
    return a->dtype == PA_F32 ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID;
  }
  if (a->kv_dtype != a->dtype && !is_q8(a->kv_dtype)) return PA_ERR_INVALID;
  if (a->num_seqs < 0 || a->num_tokens < 0 || a->num_q_heads <= 0 || a->num_kv_heads <= 0 ||
      a->head_dim <= 0 || a->block_size <= 0 || a->num_blocks <= 0 ||
      a->max_blocks_per_seq <= 0 || a->max_query_len < 0 || a->max_context_len < 0)
    return PA_ERR_INVALID;
  if (a->num_q_heads % a->num_kv_heads != 0) return PA_ERR_INVALID;
  if ((int64_t)a->max_context_len > (int64_t)a->max_blocks_per_seq * a->block_size)
    return PA_ERR_INVALID;
  if (!isfinite(a->scale)) return PA_ERR_INVALID;
  if (a->head_dim != 64 && a->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (a->block_size != 8 && a->block_size != 16 && a->block_size != 32 && a->block_size != 64)
    return PA_ERR_UNSUPPORTED;
  if (a->num_seqs == 0 || a->num_tokens == 0 || a->max_query_len == 0) return PA_OK;
  if (!aligned16(a->out) || !aligned16(a->q) || !aligned16(a->k_cache) ||
      !aligned16(a->v_cache) || !a->block_tables || !a->context_lens || !a->query_start)
    return PA_ERR_INVALID;
  // grid: slot tiles (at least 64 slots each) x KV heads x sequences; the
  // kernel numbers its workgroups with 32-bit ints
  const int64_t tiles =
      ((int64_t)a->max_query_len * (a->num_q_heads / a->num_kv_heads) + 16 * kWaves - 1) /
      (16 * kWaves);
  if (a->num_seqs > 65535 || a->num_kv_heads > 65535 ||
      tiles * a->num_kv_heads * a->num_seqs > 0x7FFFFFFF)
    return PA_ERR_UNSUPPORTED;
  hipStream_t hs = (hipStream_t)stream;
  const bool kv8 = is_q8(a->kv_dtype), fp8 = a->kv_dtype == PA_FP8;
  if (a->dtype == PA_F16) {
    if (fp8) launch_prefill_dims<Fp8Elem<F16>, true>(a, hs);
    else if (kv8) launch_prefill_dims<F16, true>(a, hs);
    else launch_prefill_dims<F16, false>(a, hs);
  } else {
    if (fp8) launch_prefill_dims<Fp8Elem<BF16>, true>(a, hs);
    else if (kv8) launch_prefill_dims<BF16, true>(a, hs);
    else launch_prefill_dims<BF16, false>(a, hs);
  }
  return launch_status();
}

PA_API size_t pa_decode_prefix_workspace_bytes(const pa_decode_args* a,
                                               const pa_prefix_groups* g) {
  Plan pl;
  return prefix_plan(a, g, pl) == PA_OK ? pl.ws_bytes : 0;
}

PA_API pa_status pa_decode_prefix(const pa_decode_args* a, const pa_prefix_groups* g,
                                  void* stream) {
  Plan pl;
  pa_status st = prefix_plan(a, g, pl);
  if (st != PA_OK) return st;
  if (a->num_seqs == 0) return PA_OK;
  if (!aligned16(a->out) || !aligned16(a->q) || !aligned16(a->k_cache) ||
      !aligned16(a->v_cache) || !a->block_tables || !a->context_lens)
    return PA_ERR_INVALID;
  if (a->num_seqs > 65535 || pl.max_parts > 65535 || a->num_q_heads > 65535)
    return PA_ERR_UNSUPPORTED;
  if (pl.n_grp > 0) {  // one 1-D grid of both passes; the kernel numbers it with 32-bit ints
    int px, py, pz, dx, dy;
    const int64_t wgs = fused_prefix_wgs(a, pl, &px, &py, &pz) + fused_decode_wgs(a, pl, &dx, &dy);
    if (wgs * 64 * kWaves > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
  }
  if ((a->k_new == nullptr) != (a->v_new == nullptr)) return PA_ERR_INVALID;
  if (a->k_new && (!aligned16(a->k_new) || !aligned16(a->v_new))) return PA_ERR_INVALID;
  if (pl.ws_bytes &&
      (!a->workspace || a->workspace_bytes < pl.ws_bytes || !aligned16(a->workspace)))
    return PA_ERR_WORKSPACE;
  return run_plan(a, pl, (hipStream_t)stream);
}

PA_API pa_status pa_decode(const pa_decode_args* a, void* stream) {
  pa_status st = validate(a);
  if (st != PA_OK) return st;
  if (a->num_seqs == 0) return PA_OK;
  if (!aligned16(a->out) || !aligned16(a->q) || !aligned16(a->k_cache) ||
      !aligned16(a->v_cache) || !a->block_tables || !a->context_lens)
    return PA_ERR_INVALID;
  const Plan pl = make_plan(a);
  if (a->num_seqs > 65535 || pl.max_parts > 65535 || a->num_q_heads > 65535)
    return PA_ERR_UNSUPPORTED;
  if ((a->k_new == nullptr) != (a->v_new == nullptr)) return PA_ERR_INVALID;
  if (a->k_new && (!aligned16(a->k_new) || !aligned16(a->v_new))) return PA_ERR_INVALID;
  if (pl.ws_bytes &&
      (!a->workspace || a->workspace_bytes < pl.ws_bytes || !aligned16(a->workspace)))
    return PA_ERR_WORKSPACE;
  return run_plan(a, pl, (hipStream_t)stream);
}

PA_API pa_status pa_decode_static(const pa_decode_args* a, void* stream) {
  pa_status st = validate(a);
  if (st != PA_OK) return st;
  if (a->num_seqs == 0) return PA_OK;
  if (!aligned16(a->out) || !aligned16(a->q) || !aligned16(a->k_cache) ||
      !aligned16(a->v_cache) || !a->block_tables || !a->context_lens)
    return PA_ERR_INVALID;
  const Plan pl = make_plan(a);
  if (a->num_seqs > 65535 || pl.max_parts > 65535 || a->num_q_heads > 65535)
    return PA_ERR_UNSUPPORTED;
  if ((a->k_new == nullptr) != (a->v_new == nullptr)) return PA_ERR_INVALID;
  if (a->k_new && (!aligned16(a->k_new) || !aligned16(a->v_new))) return PA_ERR_INVALID;
  if (pl.ws_bytes > kScratchBytes) return PA_ERR_WORKSPACE;
  pa_decode_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (pl.ws_bytes) {
    st = scratch_on_current_device((hipStream_t)stream, &b.workspace);
    if (st != PA_OK) return st;
    b.workspace_bytes = kScratchBytes;
  }
  return run_plan(&b, pl, (hipStream_t)stream);
}

}  // extern "C"
