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

#include "kernels.hpp"

namespace pa {
namespace {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// A score may exceed the running reference maximum by this much (base-2 units)
// before the accumulators are rescaled: probabilities stay below 2^8, far from fp32
// overflow, and the common path skips the rescale entirely.
constexpr float kRescaleSlack = 8.0f;

// s_waitcnt immediate for "vmcnt(0)" with expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

// ------------------------------------------------------------------ element formats
// Each format says how one dword of q meets one dword of k (fp32-accumulated dot
// product) and how a dword of v widens to fp32.
struct ElemF32 {
  static constexpr int kBytes = 4;
  __device__ static float dot(uint32_t q, uint32_t k, float acc) {
    return fmaf(__uint_as_float(q), __uint_as_float(k), acc);
  }
  __device__ static void widen(uint32_t w, float* out) { out[0] = __uint_as_float(w); }
};

struct ElemF16 {
  static constexpr int kBytes = 2;
  __device__ static float dot(uint32_t q, uint32_t k, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q), __builtin_bit_cast(f16x2, k),
                                  acc, false);
  }
  __device__ static void widen(uint32_t w, float* out) {
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    out[0] = static_cast<float>(h[0]);
    out[1] = static_cast<float>(h[1]);
  }
};

struct ElemBF16 {
  static constexpr int kBytes = 2;
  __device__ static float dot(uint32_t q, uint32_t k, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q),
                                           __builtin_bit_cast(bf16x2, k), acc, false);
  }
  __device__ static void widen(uint32_t w, float* out) {
    out[0] = __uint_as_float(w << 16);
    out[1] = __uint_as_float(w & 0xffff0000u);
  }
};

// Orders this wave's LDS accesses around the call (LDS operations of one wave
// execute in issue order, so only the compiler has to be held back).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Materializes x here: keeps the compiler from sinking the computation of x into
// a branch when x feeds a lane-dependent select (which would split the scheduling
// region of the surrounding loop).
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

template <int kXor>
__device__ __forceinline__ float dpp_xor_add(float x) {
  // quad_perm patterns: [1,0,3,2] swaps neighbours, [2,3,0,1] swaps pairs.
  constexpr int ctrl = kXor == 1 ? 0xB1 : 0x4E;
  const int y = __builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false);
  return x + __int_as_float(y);
}

// ------------------------------------------------------------------ decode partitions
// One workgroup of kDecodeWaves waves per (sequence, KV head, partition of
// partition_tokens tokens).  The waves take the partition's 16-token tiles in turn
// (wave w: tiles w, w+4, ...); each tile of one KV head is a contiguous
// 16 x 128-element run inside one physical block.
//
// Per tile and wave:
//   * K and V rows arrive with 16-byte loads, a quarter-wave covering 256
//     contiguous bytes; the next tile's loads are issued before this tile's math.
//   * K goes to LDS with rows padded by 16 bytes, so lanes reading the same chunk of
//     different rows hit different banks and every chunk is a constant offset from
//     the lane's row address.
//   * QK: lane (head hq, token t) takes whole-row dot products of its query head with
//     K rows read back from LDS, so all G query heads of the group share one read of
//     K from memory; for G < 4 a dot product is split over LPP lanes and summed with
//     DPP.
//   * Online softmax in base 2 against a per-head reference maximum that is raised
//     (and the accumulators rescaled) only when a score passes it by kRescaleSlack.
//   * Probabilities go through LDS to the PV layout: lane (token group, 16-byte
//     chunk) keeps o[G][chunk] for the tokens it loaded from V.
// At the end the waves' (max, sum, o) are merged through LDS; a sequence with one
// partition writes `out`, otherwise the partition writes its normalized o and its
// base-2 log-sum-exp for the reduce kernel.
template <class E, int G>
struct DecodeLds {
  static constexpr int NCH = kHeadDim * E::kBytes / 16;  // 16-byte chunks per K/V row
  static constexpr int TG = kWave / NCH;                 // rows per wave-wide 16-byte load
  struct Main {
    u32x4 k[kDecodeWaves][kTileTokens][NCH + 1];  // +1: row padding against bank conflicts
    float p[kDecodeWaves][kTileTokens][G];
  };
  struct Merge {
    float o[kDecodeWaves][TG][G][kHeadDim];
  };
  union {
    Main main;
    Merge merge;
  };
  float m[kDecodeWaves][G];
  float l[kDecodeWaves][G];
};

// One work item: (sequence, KV head, partition).  Every thread of the workgroup calls
// this with the same item.
template <class E, int G>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, DecodeLds<E, G>& lds, int seq,
                                            int kvh, int part) {
  constexpr int NCH = DecodeLds<E, G>::NCH;
  constexpr int TG = DecodeLds<E, G>::TG;
  constexpr int LOADS = kTileTokens / TG;         // 16-byte loads per lane per tile (K, and V)
  constexpr int VD = 16 / E::kBytes;              // elements per 16-byte chunk
  constexpr int LPP = G >= 4 ? 1 : 4 / G;         // lanes sharing one (head, token) dot product
  constexpr int NPL = G >= 4 ? G / 4 : 1;         // (head, token) pairs per lane
  constexpr int TSTRIDE = kWave / (LPP * G);      // token distance between a lane's pairs
  constexpr int QCH = NCH / LPP;                  // 16-byte chunks of q per lane

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Hq = a.num_q_heads;
  const int L = a.ctx[seq];
  const bool bad_len = L < 0 || L > a.max_context ||
                       static_cast<int64_t>(L) > static_cast<int64_t>(a.max_blocks) * a.block_size;
  const size_t group_row = static_cast<size_t>(seq) * Hq + static_cast<size_t>(kvh) * G;
  if (bad_len || L == 0) {
    const float fill = bad_len ? __builtin_nanf("") : 0.0f;
    for (int i = threadIdx.x; i < G * kHeadDim; i += blockDim.x) a.out[group_row * kHeadDim + i] = fill;
    return;
  }
  const int t_begin = part * a.partition_tokens;
  const int t_end = min(L, t_begin + a.partition_tokens);
  const int n_tiles = (t_end - t_begin + kTileTokens - 1) / kTileTokens;
  const int n_parts = (L + a.partition_tokens - 1) / a.partition_tokens;

  // QK role of this lane.
  const int sub = lane % LPP;
  const int hq = (lane / LPP) % G;
  const int tq = (lane / LPP) / G;
  // PV (and load) role of this lane.
  const int tg = lane / NCH;
  const int ch = lane % NCH;

  u32x4 qv[QCH];
  {
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(a.q) + (group_row + hq) * NCH + sub * QCH;
#pragma unroll
    for (int c = 0; c < QCH; ++c) qv[c] = qsrc[c];
  }

  float o[G][VD];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < VD; ++e) o[h][e] = 0.0f;
  float m_mine = -INFINITY;  // reference maximum of head hq (same on all its lanes)
  float l_acc = 0.0f;
  bool bad_blk = false;

  const int32_t* tbl = a.tables + static_cast<size_t>(seq) * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  const int64_t row_bytes = kHeadDim * E::kBytes;
  const int64_t run_bytes = static_cast<int64_t>(a.block_size) * row_bytes;

  // Block ids of this wave's tiles (wave, wave + 4, ...), one per lane, loaded once
  // per partition; each tile takes its id with readlane, so no memory wait stands
  // between one tile's loads and the next.  Entries past the sequence's last block
  // are not read.  (partition_tokens <= 4096 keeps a wave's tiles within 64 lanes.)
  int tbl_lane = 0;
  {
    const int j = wave + kDecodeWaves * lane;
    if (j < n_tiles) tbl_lane = tbl[(t_begin + j * kTileTokens) / a.block_size];
  }
  // Wait for it here, before any K/V load is in flight: otherwise the compiler
  // cannot prove inside the tile loop that it has landed and drains every
  // outstanding load on each tile.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  auto tile_offset = [&](int j) -> int64_t {
    const int t0 = t_begin + j * kTileTokens;
    const int off = t0 % a.block_size;
    int phys = __builtin_amdgcn_readlane(tbl_lane, (j - wave) / kDecodeWaves);
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(a.num_blocks)) {
      bad_blk = true;
      phys = 0;
    }
    return (static_cast<int64_t>(phys) * a.num_kv_heads + kvh) * run_bytes + off * row_bytes;
  };

  auto load_rows = [&](const char* base, int64_t off, u32x4 (&r)[LOADS]) {
    const u32x4* src = reinterpret_cast<const u32x4*>(base + off) + lane;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) r[i] = src[i * kWave];
  };

  // Tile j's K and V rows are in kr / vr on entry; tile jn's are on their way into
  // the same registers on exit: K as soon as tile j's K is in LDS, V as soon as tile
  // j's PV has consumed it.  Past the last tile the loads repeat tile j (cache hits)
  // so that the count of loads in flight, and with it every wait, is the same on
  // each pass.
  auto process = [&](int j, int jn, int64_t cur_off, u32x4 (&kr)[LOADS], u32x4 (&vr)[LOADS]) {
    const int t0 = t_begin + j * kTileTokens;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = i * TG + tg;
      lds.main.k[wave][r][ch] = kr[i];
    }
    const int64_t next_off = jn < n_tiles ? tile_offset(jn) : cur_off;
    load_rows(kbase, next_off, kr);
    wave_sync();

    // QK, software-pipelined by hand: the K chunks of all NPL rows are read
    // kAhead chunks before they are used; the scheduling fences keep the compiler
    // from hoisting every read of the row at once (which would need 64 registers
    // per row).
    constexpr int kAhead = 2;
    float acc[NPL][2];
    u32x4 kk[kAhead + 1][NPL];
#pragma unroll
    for (int jj = 0; jj < NPL; ++jj) acc[jj][0] = acc[jj][1] = 0.0f;
#pragma unroll
    for (int c = 0; c < kAhead && c < QCH; ++c)
#pragma unroll
      for (int jj = 0; jj < NPL; ++jj) kk[c][jj] = lds.main.k[wave][tq + jj * TSTRIDE][sub * QCH + c];
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      if (c + kAhead < QCH) {
#pragma unroll
        for (int jj = 0; jj < NPL; ++jj)
          kk[(c + kAhead) % (kAhead + 1)][jj] =
              lds.main.k[wave][tq + jj * TSTRIDE][sub * QCH + c + kAhead];
      }
#pragma unroll
      for (int jj = 0; jj < NPL; ++jj) {
        const u32x4 x = kk[c % (kAhead + 1)][jj];
        acc[jj][0] = E::dot(qv[c].x, x.x, acc[jj][0]);
        acc[jj][1] = E::dot(qv[c].y, x.y, acc[jj][1]);
        acc[jj][0] = E::dot(qv[c].z, x.z, acc[jj][0]);
        acc[jj][1] = E::dot(qv[c].w, x.w, acc[jj][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float z[NPL];
#pragma unroll
    for (int jj = 0; jj < NPL; ++jj) {
      z[jj] = acc[jj][0] + acc[jj][1];
      pin(z[jj]);
    }
    if constexpr (LPP >= 2) {
#pragma unroll
      for (int jj = 0; jj < NPL; ++jj) z[jj] = dpp_xor_add<1>(z[jj]);
    }
    if constexpr (LPP >= 4) {
#pragma unroll
      for (int jj = 0; jj < NPL; ++jj) z[jj] = dpp_xor_add<2>(z[jj]);
    }
    bool over = false;
#pragma unroll
    for (int jj = 0; jj < NPL; ++jj) {
      const int t = tq + jj * TSTRIDE;
      z[jj] = (t0 + t < t_end) ? z[jj] * a.scale_log2 : -INFINITY;
      over |= z[jj] > m_mine + kRescaleSlack;
    }

    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      // Raise each head's reference maximum to the tile's maximum and rescale: the
      // lanes of one head (same hq) reduce their scores, then every lane fetches the
      // G rescale factors from the first lane of each head.
      float tmax = z[0];
#pragma unroll
      for (int jj = 1; jj < NPL; ++jj) tmax = fmaxf(tmax, z[jj]);
#pragma unroll
      for (int m = LPP * G; m < kWave; m <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, m));
      const float m_new = fmaxf(m_mine, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_mine - m_new);
      l_acc *= alpha;
      m_mine = m_new;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h * LPP));
#pragma unroll
        for (int e = 0; e < VD; ++e) o[h][e] *= ah;
      }
    }

#pragma unroll
    for (int jj = 0; jj < NPL; ++jj) {
      const float pr = __builtin_amdgcn_exp2f(z[jj] - m_mine);
      l_acc += pr;
      if (sub == 0) lds.main.p[wave][tq + jj * TSTRIDE][hq] = pr;
    }
    wave_sync();

    const bool partial_tile = t0 + kTileTokens > t_end;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = i * TG + tg;
      float pv[G];
      if constexpr (G % 4 == 0) {
#pragma unroll
        for (int h4 = 0; h4 < G / 4; ++h4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&lds.main.p[wave][r][h4 * 4]);
          pv[h4 * 4 + 0] = x.x;
          pv[h4 * 4 + 1] = x.y;
          pv[h4 * 4 + 2] = x.z;
          pv[h4 * 4 + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) pv[h] = lds.main.p[wave][r][h];
      }
      float v[VD];
#pragma unroll
      for (int w = 0; w < 4; ++w) E::widen(vr[i][w], &v[w * (VD / 4)]);
      if (partial_tile) {
        // Rows past the context may hold anything (even NaN): drop them by select.
        const bool keep = t0 + r < t_end;
#pragma unroll
        for (int e = 0; e < VD; ++e) {
          pin(v[e]);
          v[e] = keep ? v[e] : 0.0f;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VD; ++e) o[h][e] = fmaf(pv[h], v[e], o[h][e]);
    }
    load_rows(vbase, next_off, vr);
    wave_sync();
    return next_off;
  };

  {
    u32x4 kr[LOADS], vr[LOADS];
    if (wave < n_tiles) {
      int64_t off = tile_offset(wave);
      load_rows(kbase, off, kr);
      load_rows(vbase, off, vr);
      for (int j = wave; j < n_tiles; j += kDecodeWaves) off = process(j, j + kDecodeWaves, off, kr, vr);
    }
  }

  // ---- merge the waves
  if (bad_blk) l_acc = __builtin_nanf("");
#pragma unroll
  for (int m = LPP * G; m < kWave; m <<= 1) l_acc += __shfl_xor(l_acc, m);
  __syncthreads();  // every wave is done with lds.main before lds.merge overwrites it
  if (tq == 0 && sub == 0) {
    lds.l[wave][hq] = l_acc;
    lds.m[wave][hq] = m_mine;
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e4 = 0; e4 < VD; e4 += 4)
      *reinterpret_cast<f32x4*>(&lds.merge.o[wave][tg][h][ch * VD + e4]) =
          f32x4{o[h][e4], o[h][e4 + 1], o[h][e4 + 2], o[h][e4 + 3]};
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * (kHeadDim / 4); idx += blockDim.x) {
    const int h = idx / (kHeadDim / 4);
    const int d4 = (idx % (kHeadDim / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, lds.m[w][h]);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float lt = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float W = __builtin_amdgcn_exp2f(lds.m[w][h] - M);
      lt += W * lds.l[w][h];
      f32x4 sum = *reinterpret_cast<const f32x4*>(&lds.merge.o[w][0][h][d4]);
#pragma unroll
      for (int g = 1; g < TG; ++g) sum += *reinterpret_cast<const f32x4*>(&lds.merge.o[w][g][h][d4]);
      acc += W * sum;
    }
    const f32x4 res = acc / lt;
    const size_t row = group_row + h;
    if (n_parts == 1) {
      *reinterpret_cast<f32x4*>(a.out + row * kHeadDim + d4) = res;
    } else {
      const size_t prow = row * a.pmax + part;
      *reinterpret_cast<f32x4*>(a.part_o + prow * kHeadDim + d4) = res;
      if (d4 == 0) a.part_lse[prow] = M + __log2f(lt);
    }
  }
}

// Persistent decode workgroups: each takes (item, KV head) work numbers from the
// counter the plan kernel zeroed, until the numbers run out; the next number is
// fetched while the current item runs.
template <class E, int G>
__global__ __launch_bounds__(kWave * kDecodeWaves, 2) void decode_partition_kernel(const DecodeArgs a) {
  __shared__ DecodeLds<E, G> lds;
  __shared__ int s_next;
  int* counter = a.work_header;
  const int n_work = a.work_header[1];
  if (threadIdx.x == 0) s_next = atomicAdd(counter, 1);
  __syncthreads();
  int work = s_next;
  while (work < n_work) {
    __syncthreads();  // s_next has been read and the previous item's LDS is free
    if (threadIdx.x == 0) s_next = atomicAdd(counter, 1);
    const int item = work / a.num_kv_heads;
    decode_item<E, G>(a, lds, a.work_items[2 * item], work - item * a.num_kv_heads,
                      a.work_items[2 * item + 1]);
    __syncthreads();
    work = s_next;
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

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(const DecodeArgs a) {
  __shared__ int s_tmp[kPlanThreads / 64];
  const int P = a.partition_tokens;
  auto classify = [&](int s, int* full, int* partial) {
    const int L = a.ctx[s];
    const bool bad = L < 0 || L > a.max_context ||
                     static_cast<int64_t>(L) > static_cast<int64_t>(a.max_blocks) * a.block_size;
    if (bad || L == 0) {
      *full = 0;
      *partial = 1;
    } else {
      *full = L / P;
      *partial = (L % P) != 0;
    }
  };
  // Pass 1: the number of full items (the partial items are listed after them).
  int full_total = 0;
  for (int s0 = 0; s0 < a.num_seqs; s0 += blockDim.x) {
    const int s = s0 + threadIdx.x;
    int f = 0, pp = 0;
    if (s < a.num_seqs) classify(s, &f, &pp);
    int t;
    block_exclusive_scan(f, s_tmp, &t);
    full_total += t;
  }
  // Pass 2: positions, then the items themselves.
  int full_base = 0, part_base = full_total;
  for (int s0 = 0; s0 < a.num_seqs; s0 += blockDim.x) {
    const int s = s0 + threadIdx.x;
    int f = 0, pp = 0;
    if (s < a.num_seqs) classify(s, &f, &pp);
    int tf, tp;
    const int fo = block_exclusive_scan(f, s_tmp, &tf) + full_base;
    const int po = block_exclusive_scan(pp, s_tmp, &tp) + part_base;
    for (int k = 0; k < f; ++k) {
      a.work_items[2 * (fo + k)] = s;
      a.work_items[2 * (fo + k) + 1] = k;
    }
    if (pp) {
      a.work_items[2 * po] = s;
      a.work_items[2 * po + 1] = f;
    }
    full_base += tf;
    part_base += tp;
  }
  if (threadIdx.x == 0) {
    a.work_header[0] = 0;
    a.work_header[1] = part_base * a.num_kv_heads;
  }
}

// ------------------------------------------------------------------ decode reduce
// One wave per (sequence, query head) whose sequence spans several partitions:
//   M = max_p lse_p,  w_p = 2^(lse_p - M),  out = sum_p w_p o_p / sum_p w_p,
// where o_p is partition p's normalized output and lse_p its base-2 log-sum-exp.
__global__ __launch_bounds__(256) void decode_reduce_kernel(const DecodeArgs a) {
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int seq = static_cast<int>(row / a.num_q_heads);
  const int L = a.ctx[seq];
  if (L <= 0 || L > a.max_context ||
      static_cast<int64_t>(L) > static_cast<int64_t>(a.max_blocks) * a.block_size)
    return;  // written (zeros or NaN) by the partition kernel
  const int n = (L + a.partition_tokens - 1) / a.partition_tokens;
  if (n <= 1) return;  // written by the partition kernel
  const float* lse = a.part_lse + row * a.pmax;
  float M = -INFINITY;
  bool has_nan = false;
  for (int i = 0; i < n; ++i) {
    const float x = lse[i];
    has_nan |= x != x;
    M = fmaxf(M, x);
  }
  const float* po = a.part_o + row * a.pmax * kHeadDim + lane * 2;
  f32x2 acc = {0.0f, 0.0f};
  float wsum = 0.0f;
  for (int i = 0; i < n; ++i) {
    const float w = __builtin_amdgcn_exp2f(lse[i] - M);
    wsum += w;
    acc += w * *reinterpret_cast<const f32x2*>(po + static_cast<size_t>(i) * kHeadDim);
  }
  f32x2 res = acc / wsum;
  if (has_nan) res = f32x2{__builtin_nanf(""), __builtin_nanf("")};
  *reinterpret_cast<f32x2*>(a.out + row * kHeadDim + lane * 2) = res;
}

// ------------------------------------------------------------------ cache writes
// One thread per 16-byte chunk of the new rows: token t, KV head h, chunk c goes to
// block slot / bs, offset slot % bs of head h ("vLLM explained", PagedAttention
// section, item 4: blocks fill on demand).
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, const int64_t* __restrict__ slots,
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache, int64_t total_chunks,
    int32_t num_kv_heads, int32_t block_size, int64_t num_slots, int32_t row_chunks) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total_chunks) return;
  const int64_t row = i / row_chunks;
  const int c = static_cast<int>(i - row * row_chunks);
  const int64_t t = row / num_kv_heads;
  const int h = static_cast<int>(row - t * num_kv_heads);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_chunks + c;
  k_cache[dst] = k[i];
  v_cache[dst] = v[i];
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

template <class E, int G>
hipError_t launch_persistent(const DecodeArgs& a, hipStream_t s) {
  // Workgroups resident at once on the current device (cached per device).
  static int cached[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_partition_kernel<E, G>,
                                                     kWave * kDecodeWaves, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached[dev] = std::max(1, per_cu) * std::max(1, cus);
  }
  const int64_t upper = static_cast<int64_t>(a.num_seqs) * a.pmax * a.num_kv_heads;
  const int grid = static_cast<int>(std::min<int64_t>(cached[dev], upper));
  hipLaunchKernelGGL(HIP_KERNEL_NAME(decode_partition_kernel<E, G>), dim3(grid),
                     dim3(kWave * kDecodeWaves), 0, s, a);
  return hipGetLastError();
}

template <class E>
hipError_t launch_decode_typed(const DecodeArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_persistent<E, 1>(a, s);
    case 2: return launch_persistent<E, 2>(a, s);
    case 4: return launch_persistent<E, 4>(a, s);
    case 8: return launch_persistent<E, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_partitions(const DecodeArgs& a, int dtype, int group, hipStream_t s) {
  (void)hipGetLastError();
  switch (dtype) {
    case 0: return launch_decode_typed<ElemF32>(a, group, s);
    case 1: return launch_decode_typed<ElemF16>(a, group, s);
    case 2: return launch_decode_typed<ElemBF16>(a, group, s);
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
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  hipLaunchKernelGGL(decode_reduce_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* k, const void* v, const int64_t* slots,
                                    void* k_cache, void* v_cache, int32_t n_tokens,
                                    int32_t num_kv_heads, int32_t block_size, int64_t num_slots,
                                    int32_t row_bytes, hipStream_t s) {
  (void)hipGetLastError();
  const int32_t row_chunks = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(n_tokens) * num_kv_heads * row_chunks;
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  hipLaunchKernelGGL(reshape_and_cache_kernel, grid, dim3(256), 0, s,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slots,
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), total,
                     num_kv_heads, block_size, num_slots, row_chunks);
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
