// gfx950 (CDNA4) kernels for paged KV-cache attention.
//
// Decode computes softmax(q . K^T * scale) V for one new token per sequence, with K
// and V read through the sequence's block table ("LLM inference optimization: KV
// cache & PagedAttention", carlstack.gravito.dev, section 二 attention formula and
// section 三.1 block table; "vLLM explained", jackchen890311.github.io, two
// implementation layers: the kernel jumps through the page table, the math is
// unchanged).  Decode streams the whole cached K/V of every sequence from HBM for one
// token of work, so it is bandwidth-bound (carlstack page, section 一.2) and is built
// on the vector ALUs, not on MFMA.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "kernels.hpp"

namespace pa {
namespace {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// A score may exceed the running reference maximum by this much (base-2 units)
// before the accumulators are rescaled: probabilities stay below 2^8, far from fp32
// overflow, and the common path skips the rescale entirely.
constexpr float kRescaleSlack = 8.0f;

// s_waitcnt immediate for "vmcnt(0)" with expcnt and lgkmcnt left at their maxima.

// ------------------------------------------------------------------ element formats
// Each format says how a lane's chunk of a K/V row is loaded (Chunk: the lane's kElems
// elements), how one dword of q meets one dword of k (fp32-accumulated dot product;
// k_operand turns a K chunk into those dwords) and how a V chunk widens to fp32.  The
// query is stored with kQBytes per element.
struct ElemF32 {
  using Chunk = u32x4;
  static constexpr int kBytes = 4, kQBytes = 4, kElems = 4;
  __device__ static float dot(uint32_t q, uint32_t k, float acc) {
    return fmaf(__uint_as_float(q), __uint_as_float(k), acc);
  }
  __device__ static float dot0(uint32_t q, uint32_t k) { return __uint_as_float(q) * __uint_as_float(k); }
  __device__ static u32x4 k_operand(Chunk c) { return c; }
  __device__ static void widen(Chunk c, float (&v)[kElems]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = __uint_as_float(c[w]);
  }
};

struct ElemF16 {
  using Chunk = u32x4;
  static constexpr int kBytes = 2, kQBytes = 2, kElems = 8;
  __device__ static float dot(uint32_t q, uint32_t k, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q), __builtin_bit_cast(f16x2, k),
                                  acc, false);
  }
  // First product of a chain, with the zero accumulator as an inline constant (the
  // two-operand form the compiler prefers would need a register cleared first).
  __device__ static float dot0(uint32_t q, uint32_t k) {
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(q), "v"(k));
    return r;
  }
  __device__ static u32x4 k_operand(Chunk c) { return c; }
  // 16 tokens x 16 heads of scores from 32 dims (A = K rows, B = query columns).
  __device__ static f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static void widen(Chunk c, float (&v)[kElems]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // Copy the element out first: a bit cast of the vector-element lvalue c[w] reads
      // element 0 whatever w is (seen in the generated code).
      const uint32_t x = c[w];
      const f16x2 h = __builtin_bit_cast(f16x2, x);
      v[2 * w] = static_cast<float>(h[0]);
      v[2 * w + 1] = static_cast<float>(h[1]);
    }
  }
};

struct ElemBF16 {
  using Chunk = u32x4;
  static constexpr int kBytes = 2, kQBytes = 2, kElems = 8;
  __device__ static float dot(uint32_t q, uint32_t k, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q),
                                           __builtin_bit_cast(bf16x2, k), acc, false);
  }
  __device__ static float dot0(uint32_t q, uint32_t k) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(q), "v"(k));
    return r;
  }
  __device__ static u32x4 k_operand(Chunk c) { return c; }
  __device__ static f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static void widen(Chunk c, float (&v)[kElems]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      v[2 * w] = __uint_as_float(c[w] << 16);
      v[2 * w + 1] = __uint_as_float(c[w] & 0xffff0000u);
    }
  }
};

// FP8 (e4m3) cache, bf16 queries: a lane loads 8 bytes (8 elements) of a row, so a
// 128-element row is still 16 lanes and the decode layout is the 16-bit one.  e4m3
// values are exact in bf16 and in fp32, so K goes through the bf16 dot product and V
// through fp32 FMAs without rounding; the per-tensor scales are applied outside.
struct ElemFP8 {
  using Chunk = u32x2;
  static constexpr int kBytes = 1, kQBytes = 2, kElems = 8;
  __device__ static float dot(uint32_t q, uint32_t k, float acc) { return ElemBF16::dot(q, k, acc); }
  __device__ static float dot0(uint32_t q, uint32_t k) { return ElemBF16::dot0(q, k); }
  __device__ static f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) { return ElemBF16::mma16(a, b, c); }
  template <bool HI>
  __device__ static uint32_t to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
  __device__ static u32x4 k_operand(Chunk c) {
    return u32x4{to_bf16x2<false>(c.x), to_bf16x2<true>(c.x), to_bf16x2<false>(c.y),
                 to_bf16x2<true>(c.y)};
  }
  __device__ static void widen(Chunk c, float (&v)[kElems]) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(c[w], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(c[w], true);
      v[4 * w] = lo.x;
      v[4 * w + 1] = lo.y;
      v[4 * w + 2] = hi.x;
      v[4 * w + 3] = hi.y;
    }
  }
};

// Materializes x here: keeps the compiler from sinking the computation of x into
// a branch when x feeds a lane-dependent select (which would split the scheduling
// region of the surrounding loop).
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// ------------------------------------------------------------------ decode partitions
// One workgroup of kDecodeWaves waves per (sequence, KV head, partition of
// partition_tokens tokens).  The waves take the partition's 16-token tiles in turn
// (wave w: tiles w, w+4, ...); each tile of one KV head is a contiguous
// 16 x 128-element run inside one physical block, read as kLoads 1 KiB wave-wide loads
// (lane l takes the 16-byte chunk l of each KiB, so a token row is NCH consecutive
// lanes).  K never passes through LDS:
//   * QK: each lane dots its own 8 (fp32: 4) K elements with the same elements of all
//     G query heads of the group, then a butterfly over the 16 lanes of its DPP row
//     sums the partial dot products.  The first log2(G) steps are a reduce-scatter
//     (each step keeps half the heads and adds the partner's other half), the rest
//     an all-reduce; the lane's q registers hold the heads in the order that makes
//     every step a single DPP add.  Lane a of a row ends with the full score of
//     head (a >> (4 - log2 G)) for its token.
//   * Online softmax in base 2 against a per-head reference maximum that is raised
//     (and the accumulators rescaled) only when a score passes it by kRescaleSlack.
//   * PV: the lane that loaded 16 bytes of a V row takes the G probabilities of that
//     token from its own DPP row (row broadcasts) and accumulates o[G][chunk].
//   * Each wave keeps the loads of its next tile or two in flight while it computes.
// At the end the waves' (max, sum, o) are merged through LDS; a sequence with one
// partition writes `out`, otherwise the partition writes its normalized o and its
// base-2 log-sum-exp for the reduce kernel.
template <class E, int GW>
struct DecodeLds {
  static constexpr int NCH = kHeadDim / E::kElems;  // lane chunks per K/V row
  static constexpr int TG = kWave / NCH;            // rows per wave-wide load
  // Each row of o is padded by 4 floats, and dims are stored permuted (see o_pos) so
  // that the lanes of a row write 16 consecutive 16-byte pieces: no bank conflicts.
  static constexpr int kRow = kHeadDim + 4;
  // Rows of partial sums per head: one per DPP row for the row-broadcast PV, one for the
  // MFMA PV of e4m3 caches at groups of 4 or 8, which sums all of a wave's tokens.
  static constexpr int kRows = (E::kBytes == 1 && GW >= 4) ? 1 : TG;
  float o[kDecodeWaves][GW][kRows][kRow];
  float m[kDecodeWaves][GW];
  float l[kDecodeWaves][GW];
  // Position of dims d .. d + 3 (d a multiple of 4) within a row: the piece (d % VD) / 4
  // of every chunk first, chunks in order.
  __device__ static constexpr int o_pos(int d) {
    return ((d % E::kElems) / 4) * (4 * NCH) + (d / E::kElems) * 4;
  }
};

// DPP controls (16-lane rows): partner lane a ^ 8, a ^ 7, a ^ 2, a ^ 1 and broadcast of
// lane k of the row.
constexpr int kDppRor8 = 0x128;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppXor1 = 0xB1;
constexpr int kDppRowBcast0 = 0x150;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int G>
struct GroupLayout {
  static constexpr int kLog2 = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  static_assert((1 << kLog2) == G, "group size must be 1, 2, 4 or 8");
  // Head whose full score lane position a (0..15) of a DPP row holds after the butterfly.
  __device__ static int head_of_lane(int a) { return G == 1 ? 0 : (a >> (4 - kLog2)) & (G - 1); }
  // First lane position of a row holding head h.
  static constexpr int lane_of_head(int h) { return G == 1 ? 0 : h << (4 - kLog2); }
  // Head held in q slot p by a lane whose final head is hs.
  __device__ static int slot_head(int hs, int p) { return hs ^ (G == 8 ? (p ^ ((p >> 1) & 1)) : p); }
};

// s[i][0..G) holds the partial dot products of load i in slot order; on return
// s[i][0] is the full 16-lane sum for head_of_lane(lane & 15).  The loads go through
// each level together, so consecutive DPP instructions are independent.
template <int G, int N>
__device__ __forceinline__ void row_butterfly(float (&s)[N][G]) {
  if constexpr (G >= 2) {
#pragma unroll
    for (int k = 0; k < G / 2; ++k)
#pragma unroll
      for (int i = 0; i < N; ++i) s[i][k] += dpp<kDppRor8>(s[i][G / 2 + k]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) s[i][0] += dpp<kDppRor8>(s[i][0]);
  }
  if constexpr (G >= 4) {
#pragma unroll
    for (int k = 0; k < G / 4; ++k)
#pragma unroll
      for (int i = 0; i < N; ++i) s[i][k] += dpp<kDppHalfMirror>(s[i][G / 4 + k]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) s[i][0] += dpp<kDppHalfMirror>(s[i][0]);
  }
  if constexpr (G >= 8) {
#pragma unroll
    for (int i = 0; i < N; ++i) s[i][0] += dpp<kDppXor2>(s[i][1]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) s[i][0] += dpp<kDppXor2>(s[i][0]);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) s[i][0] += dpp<kDppXor1>(s[i][0]);
}

// Lane h of each 16-lane row, broadcast to the row (every lane is written, so no old
// value is needed).
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(x), kDppRowBcast0 + H, 0xF, 0xF, true));
}

// acc += (p of lane LANE of this 16-lane row) * v, as one DPP FMA.  Volatile keeps the
// FMAs after the s_nop that precedes them (the compiler cannot see the DPP read).
template <int LANE>
__device__ __forceinline__ void fma_row_bcast(float& acc, float p, float v) {
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
               : "+v"(acc)
               : "v"(p), "v"(v), "i"(LANE));
}

// Lane position (0..15) of the row that holds head h's probability: after the DPP
// butterfly (GroupLayout), or lane h itself when the scores come from MFMA.
template <int GW, bool MF>
constexpr int prob_lane(int h) { return MF ? h : GroupLayout<GW>::lane_of_head(h); }

template <int GW, int VD, int H, bool MF>
__device__ __forceinline__ void pv_row(float (&o)[GW][VD], float pr, const float (&v)[VD]) {
  if constexpr (H < GW) {
#pragma unroll
    for (int e = 0; e < VD; ++e) fma_row_bcast<prob_lane<GW, MF>(H)>(o[H][e], pr, v[e]);
    pv_row<GW, VD, H + 1, MF>(o, pr, v);
  }
}

// Loads through the scalar data cache: for data that no kernel writes while this one
// runs (the work list), at a wave-uniform address.
template <class T>
__device__ __forceinline__ T ld_uniform(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)(p))[i];
}

// First token a sequence of length L attends to (a sliding window of `window` tokens;
// 0 = no window), and the tile-aligned token its first partition starts at.
__device__ __forceinline__ int window_start(int L, int window) {
  return window > 0 && L > window ? L - window : 0;
}
__device__ __forceinline__ int window_base(int L, int window) {
  return window_start(L, window) / kTileTokens * kTileTokens;
}

// Log-sum-exp merge of one query row's n partitions, dims d4 .. d4 + 3:
//   M = max_p lse_p,  w_p = 2^(lse_p - M),  out = sum_p w_p o_p / sum_p w_p,
// where o_p is partition p's normalized output and lse_p its base-2 log-sum-exp (the
// identity of the softmax over a union of token sets).  Partitions are taken in order,
// so every caller gets the same bits.
__device__ __forceinline__ f32x4 merge_partitions(const DecodeArgs& a, int64_t row, int n, int d4) {
  const float* lse = a.part_lse + row * a.pmax;
  float M = -INFINITY;
  bool has_nan = false;
#pragma unroll 4
  for (int i = 0; i < n; ++i) {
    const float x = lse[i];
    has_nan |= x != x;
    M = fmaxf(M, x);
  }
  const float* po = a.part_o + row * a.pmax * kHeadDim + d4;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float wsum = 0.0f;
#pragma unroll 4
  for (int i = 0; i < n; ++i) {
    const float w = __builtin_amdgcn_exp2f(lse[i] - M);
    wsum += w;
    acc += w * *reinterpret_cast<const f32x4*>(po + static_cast<size_t>(i) * kHeadDim);
  }
  const f32x4 res = acc / wsum;
  return has_nan ? f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")} : res;
}

// PV on the matrix cores for an e4m3 cache (one step of two 16-token tiles).  w[m][d][k]
// holds, for token pair m (token slots 2m, 2m + 1) and dword d of the lane's V chunks
// (dims 4d .. 4d + 3 of the chunk), the bytes of dims 4d + 2k and 4d + 2k + 1 of the two
// tokens, paired by token: [t0 dim, t1 dim, t0 dim', t1 dim'].  MFMA J takes dim J of the
// chunk (its A row is the lane's chunk, its K index the token slot): 8 e4m3 values
// converted exactly to bf16; the B operands are the probabilities of the same token slots,
// as bf16 plus the bf16 rounding of the remainder.
template <int J>
__device__ __forceinline__ void pv_mfma_e4m3(f32x4 (&po)[8], const uint32_t (&w)[4][2][2], u32x4 bh,
                                             u32x4 bl) {
  if constexpr (J < 8) {
    constexpr int d = J / 4, k = (J % 4) / 2;
    constexpr bool hi = (J % 2) != 0;
    const u32x4 a = {ElemFP8::to_bf16x2<hi>(w[0][d][k]), ElemFP8::to_bf16x2<hi>(w[1][d][k]),
                     ElemFP8::to_bf16x2<hi>(w[2][d][k]), ElemFP8::to_bf16x2<hi>(w[3][d][k])};
    po[J] = ElemBF16::mma16(a, bh, po[J]);
    po[J] = ElemBF16::mma16(a, bl, po[J]);
    pv_mfma_e4m3<J + 1>(po, w, bh, bl);
  }
}

// One work unit: (sequence, KV head, partition) and the sequence's context length,
// wave-uniform.  Everything else is derived from these four numbers when needed.
struct Unit {
  int seq, kvh, part, L;
};

// Persistent decode workgroups.  Each claims work numbers (item, KV head) from the
// counter the plan kernel zeroed until they run out.  The next unit is claimed late in
// the current one, a few steps before its end (wave 0 takes the number and hands it to
// the other waves through LDS), so that no workgroup holds work that an idle one could
// run: the list ends on its smallest items, and those go to whichever workgroups free
// up first.  The claim still comes early enough for the next unit to be made ready
// while the current one runs: its descriptor (scalar loads), the row offsets of its
// tiles, its query rows (staged through LDS) and its first K/V step (issued by the
// last step of the current tile loop), so consecutive units run back to back.
// Workgroups per CU the register budget is sized for: the more query heads a wave
// carries (query and output registers), the fewer workgroups fit.
template <class E, int GW>
constexpr int decode_blocks_per_cu() {
  // GW >= 4 with 16-bit queries runs the MFMA path; its LDS (g = 8) or, at g = 4, the
  // memory system allows two workgroups (a third or fourth measured no faster or slower).
  // With an e4m3 cache PV is on MFMA too: its merge needs a quarter of the LDS and its
  // registers leave room for a third workgroup (0.648 / 0.658 of peak at g = 8 / 4
  // against 0.642 / 0.653 with two, within the spread between boxes).
  return E::kBytes == 4 ? 2 : E::kBytes == 1 && GW >= 4 ? 3 : (GW >= 4 ? 2 : 4);
}

template <class E, int GW, int HS>
__global__ __launch_bounds__(kWave * kDecodeWaves, (decode_blocks_per_cu<E, GW>())) void decode_partition_kernel(const DecodeArgs a) {
  constexpr int G = GW * HS;            // query heads per KV head
  constexpr int NS = kDecodeWaves / HS;  // tile streams per workgroup
  static_assert(NS * kWave * kTileTokens >= kMaxPartition, "a wave's tiles of a unit fit its lanes");
  using GL = GroupLayout<GW>;
  using Lds = DecodeLds<E, GW>;
  constexpr int NCH = Lds::NCH;
  constexpr int TG = Lds::TG;
  constexpr int LOADS = kTileTokens / TG;  // wave-wide loads per tile (K, and again V)
  constexpr int VD = E::kElems;            // elements per lane chunk
  constexpr int QDW = G * kHeadDim * E::kQBytes / 4;  // dwords of one group's query rows
  using Chunk = typename E::Chunk;
  constexpr int QPT = (QDW + kWave * kDecodeWaves - 1) / (kWave * kDecodeWaves);
  // With 16-bit queries and groups of 4 or 8, QK runs on MFMA (16x16x32): the A operand
  // is 16 tokens x 32 dims of K (lane l: token l % 16, dims 8 (l / 16) .. + 7 of the
  // slice), the B operand 32 dims x 16 query heads (heads past G are zero), and the
  // result gives lane l the scores of head l % 16 for tokens 4 (l / 16) + i, i = 0..3.
  // V load i then reads tokens 4r + i into row r, so each row's probabilities sit in
  // the row that holds the V values they weight, and PV is the same row-broadcast FMA.
  constexpr bool MF = E::kQBytes == 2 && GW >= 4 && HS == 1;
  static_assert(!MF || (NCH == 16 && LOADS == 4), "MFMA scores assume 16-lane rows, 4 loads");
  // With an e4m3 cache on the MFMA path, PV runs on MFMA too (16x16x32 over two tiles,
  // pv_mfma_e4m3): per 32 tokens a lane's V chunks, byte-transposed in registers and
  // converted exactly to bf16, are the A operands of 8 MFMAs (one per dim of the chunk)
  // and its own probabilities the B operand, instead of 512 row-broadcast FMAs and the
  // widening of every V element, which bound this path's vector unit.
  constexpr bool PVM = MF && E::kBytes == 1;
  // Tiles per step (each wave keeps one step's K and V in flight).  The MFMA path has the
  // registers for two, but with 16-bit K/V the chip then has about 32 MiB of reads in
  // flight, more than the memory system serves best: one tile per step measured 4% faster
  // at g = 8.  An e4m3 tile is half the bytes, and its PV MFMAs take two tiles.
  constexpr int TS = PVM ? 2 : 1;
  // Rows of partial sums per head in the LDS merge: the row-broadcast PV leaves one per
  // DPP row (tokens of other rows), the MFMA PV sums all of a wave's tokens in one.
  constexpr int MR = PVM ? 1 : TG;
  static_assert(Lds::kRows == MR, "the LDS merge rows follow the PV path");
  // K of an e4m3 cache on the MFMA path: a lane's part of its token's 128-byte row (the A
  // operand's row is the token l % 16) is read as two 16-byte pieces, bytes 32 (l / 16)
  // + 16 h .. + 15, so each row's line is touched by two loads instead of four 8-byte
  // ones (the line lookups per byte were the bound: twice those of 16-bit K).  The
  // MFMA's K index then runs over dims 32 (l / 16) + 8 s + e for slice s, and the query
  // operand takes the same dims.
  using KChunk = typename std::conditional<PVM, u32x4, Chunk>::type;
  constexpr int KL = PVM ? 2 : LOADS;  // K loads per tile
  constexpr int NKL = TS * KL;
  constexpr int NL = TS * LOADS;  // K (and V) loads per step
  constexpr int64_t kRowBytes = kHeadDim * E::kBytes;

  __shared__ Lds lds;
  __shared__ u32x4 s_q[G * NCH];  // query rows of the next unit
  __shared__ int s_claim;       // the first unit's work number
  __shared__ int s_next_work;   // the next unit's work number, published by wave 0 ...
  __shared__ int s_next_epoch;  // ... for the unit with this count (units started so far)

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int stream = wave % NS;  // takes the unit's tiles stream, stream + NS, ...
  const int half = wave / NS;    // takes query heads half * GW .. half * GW + GW - 1
  const int rr = lane / NCH;  // token row of the lane within each 1 KiB load
  const int ch = lane % NCH;  // 16-byte chunk of that row
  const int hsel = MF ? (lane & 15) : GL::head_of_lane(lane & 15);
  const int P = a.partition_tokens;

  auto unit_of = [&](int work) -> Unit {
    Unit u;
    const int item = work / a.num_kv_heads;
    u.kvh = work - item * a.num_kv_heads;
    u.seq = ld_uniform(a.work_items, 4 * static_cast<int64_t>(item));
    u.part = ld_uniform(a.work_items, 4 * static_cast<int64_t>(item) + 1);
    u.L = ld_uniform(a.work_items, 4 * static_cast<int64_t>(item) + 2);
    return u;
  };
  // Empty (zeros) or invalid (NaNs) sequences have no tiles.
  auto is_bad = [&](const Unit& u) {
    return u.L < 0 || u.L > a.max_context ||
           static_cast<int64_t>(u.L) > static_cast<int64_t>(a.max_blocks) * a.block_size;
  };
  // Partition `part` covers tokens [t_begin, t_end): partitions start at the window's
  // tile-aligned first token.
  auto t_begin_of = [&](const Unit& u) { return window_base(u.L, a.window) + u.part * P; };
  auto t_end_of = [&](const Unit& u) {
    return (is_bad(u) || u.L == 0) ? t_begin_of(u) : min(u.L, t_begin_of(u) + P);
  };
  // Number of tiles this wave takes in a unit (tiles stream, stream + NS, ...).
  auto wave_tiles_of_stream = [&](const Unit& u, int st) {
    const int n_tiles = (t_end_of(u) - t_begin_of(u) + kTileTokens - 1) / kTileTokens;
    return st < n_tiles ? (n_tiles - st + NS - 1) / NS : 0;
  };
  auto wave_tiles = [&](const Unit& u) { return wave_tiles_of_stream(u, stream); };
  // Row offset (rows of head_dim elements from the layer's K base) of the wave's tile
  // `lane`, or -1 if its block id lies outside the pool; 0 for lanes past the wave's
  // tiles.  partition_tokens <= kMaxPartition keeps a wave's tiles within 64 lanes.
  auto tile_rows = [&](const Unit& u, int nt) -> int {
    if (lane >= nt) return 0;
    const int t0 = t_begin_of(u) + (stream + NS * lane) * kTileTokens;
    const int phys = a.tables[static_cast<int64_t>(u.seq) * a.max_blocks + t0 / a.block_size];
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(a.num_blocks)) return -1;
    return (phys * a.num_kv_heads + u.kvh) * a.block_size + t0 % a.block_size;
  };
  auto load_q = [&](const Unit& u, uint32_t (&qd)[QPT]) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.q) +
                          (static_cast<int64_t>(u.seq) * a.num_q_heads + u.kvh * G) * (QDW / G);
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int d = tid + i * kWave * kDecodeWaves;
      qd[i] = d < QDW ? src[d] : 0u;
    }
  };
  auto stage_q = [&](const uint32_t (&qd)[QPT]) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(s_q);
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int d = tid + i * kWave * kDecodeWaves;
      if (d < QDW) dst[d] = qd[i];
    }
  };

  if (tid == 0) {
    s_claim = atomicAdd(a.work_header, 1);
    s_next_epoch = 0;
  }
  __syncthreads();
  const int n_work = ld_uniform(a.work_header, 1);
  const int first = __builtin_amdgcn_readfirstlane(s_claim);
  if (first >= n_work) return;
  int epoch = 0;  // units started so far

  Unit it = unit_of(first);
  int nt = wave_tiles(it);
  int rows_cur = tile_rows(it, nt);
  {
    uint32_t qd[QPT];
    load_q(it, qd);
    stage_q(qd);
  }
  bool prefetched = false;  // kr / vr already hold (or are receiving) the unit's step 0
  KChunk kr[NKL];
  Chunk vr[NL];
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);

  while (true) {
    __syncthreads();  // s_q is staged; every wave has read s_next_*; the LDS is free
    ++epoch;
    const int t_begin = t_begin_of(it);
    const int t_end = t_end_of(it);
    const int t_lo = window_start(it.L, a.window);  // tokens before it are outside the window

    u32x4 qv[MF ? 4 : GW];
    {
      // Recomputed per unit on purpose: hoisted out of the loop, the G addresses would
      // stay live through the tile loop and spill.
      int hs = hsel;
      asm volatile("" : "+v"(hs));
      if constexpr (PVM) {
        // B operand of slice s: head hs, dims 32 rr + 8 s .. + 7 (chunk 4 rr + s).
#pragma unroll
        for (int k = 0; k < 4; ++k)
          qv[k] = hs < G ? s_q[hs * NCH + 4 * rr + k] : u32x4{0u, 0u, 0u, 0u};
      } else if constexpr (MF) {
        // B operand of slice s: head hs, dims 32 s + 8 rr .. + 7 (chunk 4 s + rr).
#pragma unroll
        for (int k = 0; k < 4; ++k)
          qv[k] = hs < G ? s_q[hs * NCH + 4 * k + rr] : u32x4{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int p = 0; p < GW; ++p) qv[p] = s_q[(half * GW + GL::slot_head(hs, p)) * NCH + ch];
      }
    }

    // The next unit, known from the step at which this wave loads it (load_next).
    bool has_next = false;
    Unit nx = it;
    int nt_nx = 0;
    bool cross = false;  // the next unit has tiles on this wave: its first step is prefetched
    int rows_next = 0;
    // A block id outside the pool (row offset -1) makes the unit's result NaN; such
    // tiles are read from block 0 instead, so nothing outside the pool is touched.
    const bool bad_blk = __builtin_amdgcn_ballot_w64(lane < nt && rows_cur < 0) != 0;
    // Lane chunk offsets within the tile: K load i (e4m3 on MFMA: token ch, 16-byte piece
    // 2 rr + i; other MFMA: token ch, dim chunk 4 i + rr; else token 4 i + rr, chunk ch)
    // and V load i (MFMA: token 4 rr + i, chunk ch).
    const int k_off = PVM ? ch * (kHeadDim / 16) + 2 * rr : MF ? ch * NCH + rr : lane;
    const int v_off = MF ? 4 * rr * NCH + ch : lane;
    constexpr int k_step = PVM ? 1 : MF ? 4 : kWave;
    constexpr int v_step = MF ? NCH : kWave;
    // Step n covers the wave's tiles TS n .. TS n + TS - 1.  Past the unit's steps it
    // fetches the next unit's first step (when the next unit has tiles on this wave),
    // else this unit's last tile again (a cache hit), so every pass has the same loads
    // in flight and the same waits; tiles past the wave's last one repeat the last
    // tile's rows and are masked out by their tokens.
    const int ns = (nt + TS - 1) / TS;
    auto rows_of = [&](int n, int u) -> int {
      const int rows = n >= ns ? (cross ? __builtin_amdgcn_readlane(rows_next, min(u, nt_nx - 1))
                                        : __builtin_amdgcn_readlane(rows_cur, nt - 1))
                               : __builtin_amdgcn_readlane(rows_cur, min(TS * n + u, nt - 1));
      return max(rows, 0);
    };
    // K and V are read once per decode step: streaming loads keep them from displacing
    // reusable lines (measured 3-6% faster than plain loads).
    auto load_one = [&](const char* base, int rows, int off, int idx) -> Chunk {
      const Chunk* src = reinterpret_cast<const Chunk*>(base + static_cast<int64_t>(rows) * kRowBytes) + off;
      return __builtin_nontemporal_load(src + idx);
    };
    auto issue_k = [&](int n) {
#pragma unroll
      for (int u = 0; u < TS; ++u) {
        const int rows = rows_of(n, u);
        const KChunk* src =
            reinterpret_cast<const KChunk*>(kbase + static_cast<int64_t>(rows) * kRowBytes) + k_off;
#pragma unroll
        for (int i = 0; i < KL; ++i) kr[u * KL + i] = __builtin_nontemporal_load(src + i * k_step);
      }
    };
    auto issue = [&](int n, const char* base, Chunk (&r)[NL], int off, int step) {
#pragma unroll
      for (int u = 0; u < TS; ++u) {
        const int rows = rows_of(n, u);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) r[u * LOADS + i] = load_one(base, rows, off, i * step);
      }
    };

    // Wave 0 claims the next unit at step claim_step of its stream and publishes the
    // number at its load step; every wave loads the next unit (descriptor, row offsets,
    // query rows) at its own load step, waiting for the publication if it gets there
    // first.  Both steps sit a few steps before the end, so that the next unit's first
    // step can be issued by this unit's last one; short units do both at step 0.  With
    // 16-bit K/V at groups of 8 (the longest units) two more steps of lead let the next
    // unit's loads land before the switch (+0.3% at the Llama-3-70B layer, +0.8% with a
    // 1024-token window); the same lead costs 0.5% at groups of 4 and 2% on the vector
    // path, whose units are shorter.
    constexpr bool kLongLead = MF && GW == 8 && !PVM;
    constexpr int kClaimLead = (kLongLead ? 8 : 6) / TS, kLoadLead = (kLongLead ? 6 : 4) / TS;
    const int ns0 = (wave_tiles_of_stream(it, 0) + TS - 1) / TS;  // wave 0's steps
    const int claim_step = max(0, ns0 - kClaimLead);
    const int load_step = max(0, ns - kLoadLead);
    int claimed = 0;
    bool claim_done = false;
    auto claim = [&]() {
      if (tid == 0) claimed = atomicAdd(a.work_header, 1);
      claim_done = true;
    };
    uint32_t qn[QPT];
    bool next_loaded = false;
    auto load_next = [&]() {
      if (wave == 0) {
        if (!claim_done) claim();
        if (tid == 0) {
          s_next_work = claimed;
          __hip_atomic_store(&s_next_epoch, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      while (__hip_atomic_load(&s_next_epoch, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != epoch)
        __builtin_amdgcn_s_sleep(1);
      const int nxt = __builtin_amdgcn_readfirstlane(s_next_work);
      has_next = nxt < n_work;
      if (has_next) {
        nx = unit_of(nxt);
        nt_nx = wave_tiles(nx);
        cross = nt_nx > 0;
        rows_next = tile_rows(nx, nt_nx);
        load_q(nx, qn);
      }
      next_loaded = true;
    };

    if (nt > 0 && !prefetched) {
      issue_k(0);
      issue(0, vbase, vr, v_off, v_step);
    }

    float o[PVM ? 1 : GW][PVM ? 1 : VD];  // row-broadcast PV: o[head][element of the chunk]
    f32x4 po[PVM ? 8 : 1];                // MFMA PV: po[J][r] = dim 32 (l / 16) + 8 r + J, head l % 16
#pragma unroll
    for (int h = 0; h < (PVM ? 1 : GW); ++h)
#pragma unroll
      for (int e = 0; e < (PVM ? 1 : VD); ++e) o[h][e] = 0.0f;
#pragma unroll
    for (int j = 0; j < (PVM ? 8 : 1); ++j) po[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_ref = -INFINITY;  // reference maximum of head hsel (same on all its lanes)
    float l_acc = 0.0f;       // sum of this lane's probabilities (head hsel, its rows)

    // Tile n's K and V are in kr / vr on entry; tile n + 1's are on their way into the
    // same registers on exit, each issued as soon as tile n has consumed the registers.
    auto process = [&](int n) {
      // First token of tile u of this step, and the token of a lane's value i in it
      // (score i, and V load i's row).
      if (wave == 0 && n == claim_step) claim();
      auto tile_t0 = [&](int u) { return t_begin + (stream + NS * (TS * n + u)) * kTileTokens; };
      auto token = [&](int u, int i) {
        return MF ? tile_t0(u) + 4 * rr + i : tile_t0(u) + i * TG + rr;
      };
      float z[NL];
      if constexpr (MF) {
        f32x4 acc[TS];
#pragma unroll
        for (int u = 0; u < TS; ++u) {
          acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if constexpr (PVM) {
              // Slice k: bytes 8 (k % 2) .. + 7 of piece k / 2.
              const KChunk& piece = kr[u * KL + k / 2];
              const u32x2 half8 = {piece[2 * (k % 2)], piece[2 * (k % 2) + 1]};
              acc[u] = E::mma16(ElemFP8::k_operand(half8), qv[k], acc[u]);
            } else {
              acc[u] = E::mma16(E::k_operand(kr[u * LOADS + k]), qv[k], acc[u]);
            }
          }
        }
        if (n == load_step) load_next();
        issue_k(n + 1);
#pragma unroll
        for (int u = 0; u < TS; ++u)
#pragma unroll
          for (int i = 0; i < LOADS; ++i) {
            const int t = token(u, i);
            z[u * LOADS + i] = (t < t_end && t >= t_lo) ? acc[u][i] * a.scale_log2 : -INFINITY;
          }
      } else {
        // Partial dot products of every load first, then the butterflies of all loads
        // level by level, so that no DPP step waits on the instruction just before it.
        float s[LOADS][GW];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const u32x4 kk = E::k_operand(kr[i]);
#pragma unroll
          for (int p = 0; p < GW; ++p) {
            float acc = E::dot0(qv[p].x, kk.x);
            acc = E::dot(qv[p].y, kk.y, acc);
            acc = E::dot(qv[p].z, kk.z, acc);
            s[i][p] = E::dot(qv[p].w, kk.w, acc);
          }
        }
        if (n == load_step) load_next();
        issue_k(n + 1);
        if constexpr (NCH == 32) {
          // A row spans two DPP rows: add the other half of the row first.
#pragma unroll
          for (int i = 0; i < LOADS; ++i)
#pragma unroll
            for (int p = 0; p < GW; ++p) s[i][p] += __shfl_xor(s[i][p], 16);
        }
        row_butterfly<GW, LOADS>(s);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          pin(s[i][0]);
          const int t = token(0, i);
          z[i] = (t < t_end && t >= t_lo) ? s[i][0] * a.scale_log2 : -INFINITY;
        }
      }
      __builtin_amdgcn_sched_barrier(0);

      bool over = false;
#pragma unroll
      for (int i = 0; i < NL; ++i) over |= z[i] > m_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
        // Raise each head's reference maximum to the tile's maximum and rescale.  Lanes
        // of one head within a row hold the same scores; rows of other tokens are other
        // lanes 16 (or 32) apart.
        float tmax = z[0];
#pragma unroll
        for (int i = 1; i < NL; ++i) tmax = fmaxf(tmax, z[i]);
#pragma unroll
        for (int m = NCH; m < kWave; m <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, m));
        const float m_new = fmaxf(m_ref, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        l_acc *= alpha;
        m_ref = m_new;
        if constexpr (PVM) {
          // The lane's accumulators are its own head's.
#pragma unroll
          for (int j = 0; j < 8; ++j) po[j] *= alpha;
        } else {
#pragma unroll
          for (int h = 0; h < GW; ++h) {
            const float ah =
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), prob_lane<GW, MF>(h)));
#pragma unroll
            for (int e = 0; e < VD; ++e) o[h][e] *= ah;
          }
        }
      }

      if constexpr (PVM) {
        // Token slot 4u + i of this lane is token 4 (l / 16) + i of tile u, the token of
        // its score z[4u + i] and of its V chunk vr[4u + i].  Rows past the context (or
        // before the window) may hold anything, even NaN: their chunks are zeroed by
        // select (their probabilities are 0).
        u32x2 vv[NL];
#pragma unroll
        for (int u = 0; u < TS; ++u) {
          const bool partial_tile = tile_t0(u) + kTileTokens > t_end || tile_t0(u) < t_lo;
#pragma unroll
          for (int i = 0; i < LOADS; ++i) {
            vv[u * LOADS + i] = vr[u * LOADS + i];
            if (partial_tile) {
              const bool keep = token(u, i) < t_end && token(u, i) >= t_lo;
              vv[u * LOADS + i] = keep ? vv[u * LOADS + i] : u32x2{0u, 0u};
            }
          }
        }
        // The next step's V loads leave now, before this step's PV.
#pragma unroll
        for (int u = 0; u < TS; ++u) {
          const int vrows = rows_of(n + 1, u);
#pragma unroll
          for (int i = 0; i < LOADS; ++i) vr[u * LOADS + i] = load_one(vbase, vrows, v_off, i * v_step);
        }
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        uint32_t ph[NL / 2], pl[NL / 2];
#pragma unroll
        for (int m = 0; m < NL / 2; ++m) {
          const f32x2 p = f32x2{__builtin_amdgcn_exp2f(z[2 * m] - m_ref),
                                __builtin_amdgcn_exp2f(z[2 * m + 1] - m_ref)};
          l_acc += p.x + p.y;
          const bf16x2_t h = __builtin_convertvector(p, bf16x2_t);
          const f32x2 hf = __builtin_convertvector(h, f32x2);
          const bf16x2_t e = __builtin_convertvector(f32x2{p.x - hf.x, p.y - hf.y}, bf16x2_t);
          ph[m] = __builtin_bit_cast(uint32_t, h);
          pl[m] = __builtin_bit_cast(uint32_t, e);
        }
        uint32_t w[4][2][2];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const uint32_t x0 = vv[2 * m][d], x1 = vv[2 * m + 1][d];
            w[m][d][0] = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // [x0.b0 x1.b0 x0.b1 x1.b1]
            w[m][d][1] = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // [x0.b2 x1.b2 x0.b3 x1.b3]
          }
        pv_mfma_e4m3<0>(po, w, u32x4{ph[0], ph[1], ph[2], ph[3]}, u32x4{pl[0], pl[1], pl[2], pl[3]});
      } else {
      // Each V register is reloaded with the next step's value as soon as PV has used
      // it, so the next step's V loads leave during this step's PV rather than after it.
#pragma unroll
      for (int u = 0; u < TS; ++u) {
        const bool partial_tile = tile_t0(u) + kTileTokens > t_end || tile_t0(u) < t_lo;
        const int vrows = rows_of(n + 1, u);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const float pr = __builtin_amdgcn_exp2f(z[u * LOADS + i] - m_ref);
          l_acc += pr;
          float v[VD];
          E::widen(vr[u * LOADS + i], v);
          if (partial_tile) {
            // Rows past the context (or before the window) may hold anything, even NaN:
            // drop them by select.
            const bool keep = token(u, i) < t_end && token(u, i) >= t_lo;
#pragma unroll
            for (int e = 0; e < VD; ++e) {
              pin(v[e]);
              v[e] = keep ? v[e] : 0.0f;
            }
          }
          if constexpr (GW == 1) {
#pragma unroll
            for (int e = 0; e < VD; ++e) o[0][e] = fmaf(pr, v[e], o[0][e]);
          } else {
            // o[h] += p(head h, this row) * v: the probability comes straight from the
            // lane holding head h through the FMA's row broadcast.  Two wait states
            // separate the write of pr from its first DPP read.
            // (pr is an operand of the s_nop so that its computation cannot be scheduled
            // between the s_nop and the FMAs.)
            asm volatile("s_nop 1" ::"v"(pr));
            pv_row<GW, VD, 0, MF>(o, pr, v);
          }
          vr[u * LOADS + i] = load_one(vbase, vrows, v_off, i * v_step);
          // One load's probabilities and V values at a time: interleaving the loads
          // would keep all of them live and spill.
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      }
    };

    for (int n = 0; n < ns; ++n) process(n);
    if (!next_loaded) load_next();
    prefetched = nt > 0 && cross;

    // ---- merge the waves and write the unit's result
    const size_t group_row = static_cast<size_t>(it.seq) * a.num_q_heads + static_cast<size_t>(it.kvh) * G;
    if (t_end == t_begin) {
      // Empty sequence (zeros) or invalid one (NaNs); a unit with tiles is never empty.
      const float fill = is_bad(it) ? __builtin_nanf("") : 0.0f;
      for (int i = tid; i < G * kHeadDim; i += blockDim.x) a.out[group_row * kHeadDim + i] = fill;
      __syncthreads();  // every wave has read s_q before it is restaged
    } else {
      if (bad_blk) l_acc = __builtin_nanf("");
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < TG; ++r)
          sum += __int_as_float(
              __builtin_amdgcn_readlane(__float_as_int(l_acc), r * NCH + prob_lane<GW, MF>(h)));
        const float mh =
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_ref), prob_lane<GW, MF>(h)));
        if (lane == 0) {
          lds.m[wave][h] = mh;
          lds.l[wave][h] = sum;
        }
      }
      if constexpr (PVM) {
        const int h = lane & 15;
        if (h < GW) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = 32 * rr + 8 * r;
            *reinterpret_cast<f32x4*>(&lds.o[wave][h][0][Lds::o_pos(d)]) =
                f32x4{po[0][r], po[1][r], po[2][r], po[3][r]};
            *reinterpret_cast<f32x4*>(&lds.o[wave][h][0][Lds::o_pos(d + 4)]) =
                f32x4{po[4][r], po[5][r], po[6][r], po[7][r]};
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < GW; ++h)
#pragma unroll
          for (int e4 = 0; e4 < VD; e4 += 4)
            *reinterpret_cast<f32x4*>(&lds.o[wave][h][rr][Lds::o_pos(ch * VD + e4)]) =
                f32x4{o[h][e4], o[h][e4 + 1], o[h][e4 + 2], o[h][e4 + 3]};
      }
      __syncthreads();

      const int n_parts = (it.L - window_base(it.L, a.window) + P - 1) / P;
      for (int idx = tid; idx < G * (kHeadDim / 4); idx += blockDim.x) {
        const int h = idx / (kHeadDim / 4);
        const int d4 = (idx % (kHeadDim / 4)) * 4;
        const int hw = h % GW;        // head within its wave
        const int w0 = (h / GW) * NS;  // first wave holding head h (one per stream)
        float M = -INFINITY;
#pragma unroll
        for (int j = 0; j < NS; ++j) M = fmaxf(M, lds.m[w0 + j][hw]);
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        float lt = 0.0f;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const int w = w0 + j;
          const float W = __builtin_amdgcn_exp2f(lds.m[w][hw] - M);
          lt += W * lds.l[w][hw];
          const int pos = Lds::o_pos(d4);
          f32x4 sum = *reinterpret_cast<const f32x4*>(&lds.o[w][hw][0][pos]);
#pragma unroll
          for (int r = 1; r < MR; ++r) sum += *reinterpret_cast<const f32x4*>(&lds.o[w][hw][r][pos]);
          acc += W * sum;
        }
        const f32x4 res = acc / lt * a.v_scale;
        const size_t row = group_row + h;
        if (n_parts == 1) {
          *reinterpret_cast<f32x4*>(a.out + row * kHeadDim + d4) = res;
        } else {
          const size_t prow = row * a.pmax + it.part;
          *reinterpret_cast<f32x4*>(a.part_o + prow * kHeadDim + d4) = res;
          if (d4 == 0) a.part_lse[prow] = M + __log2f(lt);
        }
      }
    }
    if (!has_next) break;
    stage_q(qn);  // s_q was last read at this unit's start, before a barrier
    __syncthreads();  // the merge is done with lds
    it = nx;
    nt = nt_nx;
    rows_cur = rows_next;
  }
}

// ------------------------------------------------------------------ decode plan
// One workgroup lists the work: every full partition of every sequence, then each
// sequence's last partial partition (so that the smallest items are taken last),
// and a single item for an empty or invalid sequence (it writes the zeros or NaNs).
// It also zeroes the work counter the persistent decode kernel draws from.
__device__ __forceinline__ int block_exclusive_scan(int x, int* s_tmp, int* total) {
  // s_tmp: kPlanThreads / 64 ints
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_tmp[wv] = incl;
  __syncthreads();
  int base = 0, sum = 0;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) {
    const int t = s_tmp[w];
    if (w < wv) base += t;
    sum += t;
  }
  __syncthreads();
  *total = sum;
  return base + incl - x;
}

// The plan's body: one workgroup of kPlanThreads threads runs it, alone in
// decode_plan_kernel or beside the cache writes in cache_write_plan_kernel.
__device__ __forceinline__ void plan_work(const DecodeArgs& a) {
  // Partial items are listed largest first (bucketed by their length in steps of
  // kBucketTokens: 32 tokens, two tiles, so that the serial pass over the buckets below
  // stays at 129), so that the smallest units are the last ones claimed and the
  // persistent workgroups finish together.  The order of items within a bucket is
  // whatever the LDS counters give: a unit's result does not depend on which workgroup
  // runs it or when.
  constexpr int kBucketTokens = kMaxPartition / 128;
  constexpr int kBuckets = kMaxPartition / kBucketTokens + 1;  // 0: empty or invalid
  __shared__ int s_tmp[kPlanThreads / 64];
  __shared__ int s_count[kBuckets];
  __shared__ int s_next[kBuckets];
  const int P = a.partition_tokens;
  auto classify = [&](int s, int* full, int* bucket) {
    const int L = a.ctx[s];
    const bool bad = L < 0 || L > a.max_context ||
                     static_cast<int64_t>(L) > static_cast<int64_t>(a.max_blocks) * a.block_size;
    if (bad || L == 0) {
      *full = 0;
      *bucket = 0;
    } else {
      const int span = L - window_base(L, a.window);  // tokens from the first partition on
      const int rem = span % P;
      *full = span / P;
      *bucket = rem == 0 ? -1 : (rem + kBucketTokens - 1) / kBucketTokens;  // -1: no partial item
    }
  };
  for (int b = threadIdx.x; b < kBuckets; b += blockDim.x) s_count[b] = 0;
  __syncthreads();
  // Pass 1: the number of full items, and the partial items per bucket.
  int full_total = 0;
  for (int s0 = 0; s0 < a.num_seqs; s0 += blockDim.x) {
    const int s = s0 + threadIdx.x;
    int f = 0, b = -1;
    if (s < a.num_seqs) classify(s, &f, &b);
    if (b >= 0) atomicAdd(&s_count[b], 1);
    int t;
    block_exclusive_scan(f, s_tmp, &t);
    full_total += t;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int at = full_total;
    for (int b = kBuckets - 1; b >= 0; --b) {
      s_next[b] = at;
      at += s_count[b];
    }
    s_tmp[0] = at;  // total items
  }
  __syncthreads();
  const int n_items = s_tmp[0];
  __syncthreads();
  // Pass 2: the items themselves.
  int full_base = 0;
  for (int s0 = 0; s0 < a.num_seqs; s0 += blockDim.x) {
    const int s = s0 + threadIdx.x;
    int f = 0, b = -1;
    if (s < a.num_seqs) classify(s, &f, &b);
    int tf;
    const int fo = block_exclusive_scan(f, s_tmp, &tf) + full_base;
    const int L = s < a.num_seqs ? a.ctx[s] : 0;
    for (int k = 0; k < f; ++k) {
      int32_t* d = a.work_items + 4 * (fo + k);
      d[0] = s;
      d[1] = k;
      d[2] = L;
      d[3] = 0;
    }
    if (b >= 0) {
      int32_t* d = a.work_items + 4 * atomicAdd(&s_next[b], 1);
      d[0] = s;
      d[1] = f;
      d[2] = L;
      d[3] = 0;
    }
    full_base += tf;
  }
  if (threadIdx.x == 0) {
    a.work_header[0] = 0;
    a.work_header[1] = n_items * a.num_kv_heads;
  }
}

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(const DecodeArgs a) { plan_work(a); }

// ------------------------------------------------------------------ decode reduce
// Merges every multi-partition row from the partials the partition kernel left in the
// workspace.  32 threads per (sequence, query head), four dims each.  (A merge inside the
// partition kernel by the last workgroup to finish a sequence would need a device-scope
// release and acquire per unit, i.e. an L2 write-back and invalidate on each XCD: measured
// several times slower than this separate launch.)
__global__ __launch_bounds__(256) void decode_reduce_kernel(const DecodeArgs a) {
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 8 + threadIdx.x / 32;
  if (row >= rows) return;
  const int seq = static_cast<int>(row / a.num_q_heads);
  const int L = a.ctx[seq];
  if (L <= 0 || L > a.max_context ||
      static_cast<int64_t>(L) > static_cast<int64_t>(a.max_blocks) * a.block_size)
    return;  // written (zeros or NaN) by the partition kernel
  const int n = (L - window_base(L, a.window) + a.partition_tokens - 1) / a.partition_tokens;
  if (n <= 1) return;  // written by the partition kernel
  const int d4 = (threadIdx.x % 32) * 4;
  *reinterpret_cast<f32x4*>(a.out + row * kHeadDim + d4) = merge_partitions(a, row, n, d4);
}

// ------------------------------------------------------------------ cache writes
// One thread per 16-byte chunk of the new rows: token t, KV head h, chunk c goes to
// block slot / bs, offset slot % bs of head h ("vLLM explained", PagedAttention
// section, item 4: blocks fill on demand).
__device__ __forceinline__ void write_row_chunk(const CacheWrite& w, int64_t i) {
  if (i >= w.total_chunks) return;
  const int64_t row = i / w.row_chunks;
  const int c = static_cast<int>(i - row * w.row_chunks);
  const int64_t t = row / w.num_kv_heads;
  const int h = static_cast<int>(row - t * w.num_kv_heads);
  const int64_t slot = w.slots[t];
  if (slot < 0 || slot >= w.num_slots) return;
  const int64_t blk = slot / w.block_size;
  const int64_t off = slot - blk * w.block_size;
  const int64_t dst = ((blk * w.num_kv_heads + h) * w.block_size + off) * w.row_chunks + c;
  const u32x4* k = static_cast<const u32x4*>(w.k);
  const u32x4* v = static_cast<const u32x4*>(w.v);
  static_cast<u32x4*>(w.k_cache)[dst] = k[i];
  static_cast<u32x4*>(w.v_cache)[dst] = v[i];
}

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(const CacheWrite w) {
  write_row_chunk(w, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
}

// FP8 cache writes: one thread per 16 stored bytes (16 elements) of a new row, read as
// 32 bytes of bf16 input.  Each value is multiplied by the float32 reciprocal of the
// layer's scale, clamped to the largest e4m3 magnitude (448; NaN stays NaN) and rounded
// to nearest even by the hardware conversion.
__device__ __forceinline__ float fp8_clamp(float y) {
  return y != y ? y : fminf(fmaxf(y, -448.0f), 448.0f);
}

__device__ __forceinline__ void write_row_chunk_fp8(const CacheWrite& w, int64_t i) {
  constexpr int kRowChunks = kHeadDim / 16;  // 16-byte chunks of a stored row
  if (i >= w.total_chunks) return;
  const int64_t row = i / kRowChunks;
  const int c = static_cast<int>(i - row * kRowChunks);
  const int64_t t = row / w.num_kv_heads;
  const int h = static_cast<int>(row - t * w.num_kv_heads);
  const int64_t slot = w.slots[t];
  if (slot < 0 || slot >= w.num_slots) return;
  const int64_t blk = slot / w.block_size;
  const int64_t off = slot - blk * w.block_size;
  const int64_t dst = ((blk * w.num_kv_heads + h) * w.block_size + off) * kRowChunks + c;
  auto quantize16 = [](u32x4 a0, u32x4 a1, float inv) -> u32x4 {
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4& a = q < 2 ? a0 : a1;
      const uint32_t x0 = a[2 * (q % 2)], x1 = a[2 * (q % 2) + 1];
      const float e0 = fp8_clamp(__uint_as_float(x0 << 16) * inv);
      const float e1 = fp8_clamp(__uint_as_float(x0 & 0xffff0000u) * inv);
      const float e2 = fp8_clamp(__uint_as_float(x1 << 16) * inv);
      const float e3 = fp8_clamp(__uint_as_float(x1 & 0xffff0000u) * inv);
      int d = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
      d = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, d, true);
      out[q] = static_cast<uint32_t>(d);
    }
    return out;
  };
  const u32x4* k = static_cast<const u32x4*>(w.k);
  const u32x4* v = static_cast<const u32x4*>(w.v);
  static_cast<u32x4*>(w.k_cache)[dst] = quantize16(k[2 * i], k[2 * i + 1], w.inv_k);
  static_cast<u32x4*>(w.v_cache)[dst] = quantize16(v[2 * i], v[2 * i + 1], w.inv_v);
}

__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(const CacheWrite w) {
  write_row_chunk_fp8(w, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
}

// One launch for a decode step's first two stages: workgroup 0 lists the decode work
// (plan_work), the others write the new rows into their slots.  The plan reads only the
// context lengths, which the writes leave alone, and the partition kernel after this
// launch sees both.
template <bool FP8>
__global__ __launch_bounds__(kPlanThreads) void cache_write_plan_kernel(const CacheWrite w,
                                                                        const DecodeArgs a) {
  if (blockIdx.x == 0) {
    plan_work(a);
    return;
  }
  const int64_t i = static_cast<int64_t>(blockIdx.x - 1) * blockDim.x + threadIdx.x;
  if constexpr (FP8)
    write_row_chunk_fp8(w, i);
  else
    write_row_chunk(w, i);
}

// ------------------------------------------------------------------ block copies
// blockIdx.x = pair, blockIdx.y = array (layer * 2 + {K, V}); the workgroup copies one
// whole block of that array (carlstack page, section 三.2: copy-on-write).
__global__ __launch_bounds__(256) void copy_blocks_kernel(const int32_t* __restrict__ pairs,
                                                          u32x4* base, int64_t array_chunks,
                                                          int64_t block_chunks, int32_t num_blocks) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (static_cast<unsigned>(src) >= static_cast<unsigned>(num_blocks) ||
      static_cast<unsigned>(dst) >= static_cast<unsigned>(num_blocks))
    return;
  u32x4* arr = base + static_cast<int64_t>(blockIdx.y) * array_chunks;
  const u32x4* s = arr + src * block_chunks;
  u32x4* d = arr + dst * block_chunks;
  constexpr int kUnroll = 4;
  int64_t c = threadIdx.x;
  for (; c + (kUnroll - 1) * 256 < block_chunks; c += kUnroll * 256) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = s[c + u * 256];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) d[c + u * 256] = x[u];
  }
  for (; c < block_chunks; c += 256) d[c] = s[c];
}

// blockIdx.x = pair, blockIdx.y = array: block pairs[2x] of the source side to block
// pairs[2x + 1] of the destination side, where the two sides are the device pool and
// the host swap space (same layout, their own block counts).  The host side is pinned
// host memory read or written through its device mapping, so one launch moves every
// block over the host link ("vLLM explained", table on when KV may be overwritten:
// preemption by swapping to CPU memory).
__global__ __launch_bounds__(256) void swap_blocks_kernel(const int32_t* __restrict__ pairs,
                                                          const u32x4* src_base, int32_t src_blocks,
                                                          u32x4* dst_base, int32_t dst_blocks,
                                                          int64_t block_chunks) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (static_cast<unsigned>(src) >= static_cast<unsigned>(src_blocks) ||
      static_cast<unsigned>(dst) >= static_cast<unsigned>(dst_blocks))
    return;
  const u32x4* s = src_base + (static_cast<int64_t>(blockIdx.y) * src_blocks + src) * block_chunks;
  u32x4* d = dst_base + (static_cast<int64_t>(blockIdx.y) * dst_blocks + dst) * block_chunks;
  constexpr int kUnroll = 4;
  int64_t c = threadIdx.x;
  for (; c + (kUnroll - 1) * 256 < block_chunks; c += kUnroll * 256) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = s[c + u * 256];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) d[c + u * 256] = x[u];
  }
  for (; c < block_chunks; c += 256) d[c] = s[c];
}

template <class E, int GW, int HS>
hipError_t launch_persistent(const DecodeArgs& a, hipStream_t s) {
  // Workgroups resident at once on the current device (cached per device).
  static int cached[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_partition_kernel<E, GW, HS>,
                                                     kWave * kDecodeWaves, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached[dev] = std::max(1, per_cu) * std::max(1, cus);
  }
  const int64_t upper = static_cast<int64_t>(a.num_seqs) * a.pmax * a.num_kv_heads;
  const int grid = static_cast<int>(std::min<int64_t>(cached[dev], upper));
  hipLaunchKernelGGL(HIP_KERNEL_NAME(decode_partition_kernel<E, GW, HS>), dim3(grid),
                     dim3(kWave * kDecodeWaves), 0, s, a);
  return hipGetLastError();
}

template <class E>
hipError_t launch_decode_typed(const DecodeArgs& a, int group, hipStream_t s) {
  switch (group) {
    // One wave carries the whole group (HS = 1).  HS = 2 would split a group over two
    // waves that read the same K/V tiles; measured slower for groups of 8 (the
    // duplicated loads and conversions outweigh the register savings).
    case 1: return launch_persistent<E, 1, 1>(a, s);
    case 2: return launch_persistent<E, 2, 1>(a, s);
    case 4: return launch_persistent<E, 4, 1>(a, s);
    case 8: return launch_persistent<E, 8, 1>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Decode workspace for callers that cannot allocate (pa_cache_and_decode_static): the
// library's own device memory, one copy per GPU, held until the process ends.  In host
// code this name is not a device address; only the address hipGetSymbolAddress returns
// for the current device is (static_scratch below).
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

}  // namespace

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_decode_partitions(const DecodeArgs& a, int dtype, int group, hipStream_t s) {
  (void)hipGetLastError();
  switch (dtype) {
    case 0: return launch_decode_typed<ElemF32>(a, group, s);
    case 1: return launch_decode_typed<ElemF16>(a, group, s);
    case 2: return launch_decode_typed<ElemBF16>(a, group, s);
    case 3: return launch_decode_typed<ElemFP8>(a, group, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_plan(const DecodeArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  const dim3 grid(static_cast<unsigned>((rows + 7) / 8));
  hipLaunchKernelGGL(decode_reduce_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const CacheWrite& w, hipStream_t s) {
  (void)hipGetLastError();
  if (w.total_chunks == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((w.total_chunks + 255) / 256));
  if (w.fp8)
    hipLaunchKernelGGL(reshape_and_cache_fp8_kernel, grid, dim3(256), 0, s, w);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel, grid, dim3(256), 0, s, w);
  return hipGetLastError();
}

hipError_t launch_cache_write_plan(const CacheWrite& w, const DecodeArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>(1 + (w.total_chunks + kPlanThreads - 1) / kPlanThreads));
  if (w.fp8)
    hipLaunchKernelGGL(cache_write_plan_kernel<true>, grid, dim3(kPlanThreads), 0, s, w, a);
  else
    hipLaunchKernelGGL(cache_write_plan_kernel<false>, grid, dim3(kPlanThreads), 0, s, w, a);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const int32_t* pairs, int32_t n_pairs, const void* src_base,
                              int32_t src_blocks, void* dst_base, int32_t dst_blocks, int32_t arrays,
                              int64_t block_bytes, hipStream_t s) {
  (void)hipGetLastError();
  if (n_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(n_pairs, arrays), dim3(256), 0, s, pairs,
                     static_cast<const u32x4*>(src_base), src_blocks, static_cast<u32x4*>(dst_base),
                     dst_blocks, block_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const int32_t* pairs, int32_t n_pairs, void* base, int32_t arrays,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t s) {
  (void)hipGetLastError();
  if (n_pairs == 0) return hipSuccess;
  const int64_t block_chunks = block_bytes / 16;
  const int64_t array_chunks = block_chunks * num_blocks;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n_pairs, arrays), dim3(256), 0, s, pairs,
                     static_cast<u32x4*>(base), array_chunks, block_chunks, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
