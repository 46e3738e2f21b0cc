// gfx950 (CDNA4) kernel for chunked prefill over a paged KV cache.
//
// A long prompt is processed in chunks that are batched with decode work ("LLM inference
// optimization: KV cache & PagedAttention", carlstack.gravito.dev, section 六 item 2;
// "vLLM explained", jackchen890311.github.io, appendix).  The chunk's own K/V rows are
// written into the cache first; then each query row of the chunk attends, causally, to
// every cached token of its sequence up to and including its own position, reading
// K/V through the block table.  Unlike decode, the query rows of a chunk form a real
// dense contraction (prefill is a matrix product on the matrix units: carlstack page,
// section 一.1), so QK^T and PV run on MFMA.
//
// Scheduling.  The work is cut into units: TR = 128 / G consecutive query rows of one
// sequence with all G query heads of one KV head (128 (row, head) columns, 32 per wave),
// over one part of their keys (parts of part_keys keys; a merge kernel combines the parts
// of rows that span several).  A plan kernel lists the units longest first in one queue per
// XCD, every unit of a (sequence, KV head) in the same queue, so that the row blocks that
// read the same keys run on one XCD at about the same time and share its L2.  The prefill
// kernel is persistent: as many workgroups as fit on the device, each claiming units from
// its own XCD's queue and, once that is empty, from the queue with the most units left.
//
// Tiling of a unit.  Keys go in tiles of 32:
//   * S^T = K Q^T with v_mfma_f32_32x32x16 (A = 32 keys x 16 dims of K from LDS, B = 16
//     dims x 32 columns of Q held in registers).  The accumulator layout (lane l holds
//     keys 8j + 4(l/32) + i of column l % 32) is already the B-operand layout PV needs,
//     so probabilities never move between lanes.
//   * Online softmax per column (the two lanes l, l ^ 32 of a column share its maximum),
//     base 2, with the accumulators rescaled only when a score passes the reference
//     maximum by kRescaleSlack.
//   * O^T += V^T P^T with the same MFMA, V^T read from the (untransposed) V tile by
//     transposing LDS reads.  P goes in as two MFMA operands, its bf16 (or fp16) rounding
//     and the rounding of the remainder, so the only error left is the fp32 accumulation
//     (a single rounding of P could move an output by several 1e-3 on rows that see only
//     a few keys).
//   * K and V tiles go from the cache straight into LDS (direct-to-LDS loads, three tiles
//     in LDS: the one being read and two in flight), one barrier per tile.
//   * Causal and length masks by select; V rows past the context are zeroed in LDS (a
//     zero probability times a NaN from unused cache memory would still be NaN).
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "prefill.hpp"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr int kHead = 128;    // head_dim
constexpr int kKeys = 32;     // keys per tile
constexpr int kCols = kPrefillColumns;  // (row, head) columns per workgroup
constexpr float kRescaleSlack = 8.0f;
// Workgroups of the prefill kernel per CU (its register budget: 512 / 3 -> 168 VGPRs).
constexpr int kPrefillBlocksPerCu = 3;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct MmaBF16 {
  typedef __bf16 elem;
  __device__ static f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
struct MmaF16 {
  typedef _Float16 elem;
  __device__ static f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// Per-sequence facts the plan and the prefill kernel both derive from the arguments.
struct SeqInfo {
  int qs, n_rows, L;
  bool bad;        // metadata the kernel cannot attend over: its rows get NaN
  bool rows_ok;    // its rows lie within [0, num_rows)
};
__device__ __forceinline__ SeqInfo seq_info(const PrefillArgs& a, int seq) {
  SeqInfo i;
  const int64_t qs = a.query_start[seq];
  const int64_t n_rows = a.query_start[seq + 1] - qs;
  i.qs = static_cast<int>(qs);
  i.n_rows = static_cast<int>(max<int64_t>(-1, min<int64_t>(n_rows, 0x7fffffff)));
  i.L = a.ctx[seq];
  i.rows_ok = qs >= 0 && n_rows >= 0 && qs + n_rows <= a.num_rows;
  i.bad = i.L < 0 || i.L > a.max_context ||
          static_cast<int64_t>(i.L) > static_cast<int64_t>(a.max_blocks) * a.block_size ||
          n_rows > i.L || !i.rows_ok;
  return i;
}

// The work list.  A unit is one (sequence, KV head, row block, key part); every part but
// a row block's last holds part_keys / 32 tiles.  Units go to queue (sequence * H_kv +
// KV head) mod 8, so with 8 KV heads (or a multiple) queue j holds KV head j's units of
// every sequence, and within a queue in buckets of kBucketTiles tiles, longest first: the
// shortest units are the last ones claimed, and the workgroups finish close together.  A
// sequence with bad metadata gets one unit per (KV head, row block), in the last bucket,
// which writes its NaN rows.
constexpr int kBucketTiles = 4;
constexpr int kBuckets = kPrefillPartKeys / kKeys / kBucketTiles + 1;
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(const PrefillArgs a, int tr) {
  __shared__ int s_count[kPrefillQueues][kBuckets];
  __shared__ int s_next[kPrefillQueues][kBuckets];
  const int tid = threadIdx.x;
  const int tiles_per_part = a.part_keys / kKeys;
  const int H = a.num_kv_heads;
  // Units of item i = (sequence, row block) per KV head: `full` whole parts, then one
  // unit in bucket `last` (-1: no unit at all).
  auto classify = [&](int i, int* seq, int* rb, int* full, int* last) {
    *seq = i / a.row_blocks;
    *rb = i % a.row_blocks;
    *full = 0;
    *last = -1;
    const SeqInfo si = seq_info(a, *seq);
    const int r0 = *rb * tr;
    if (r0 >= si.n_rows) return;
    if (si.bad) {
      if (si.rows_ok) *last = kBuckets - 1;
      return;
    }
    const int kmax = si.L - si.n_rows + min(r0 + tr, si.n_rows) - 1;
    const int n_parts = kmax / a.part_keys + 1;
    const int tiles_last = kmax / kKeys - (n_parts - 1) * tiles_per_part + 1;
    *full = n_parts - 1;
    *last = (tiles_per_part - tiles_last) / kBucketTiles;
  };
  // KV heads of sequence s that go to queue x: kvh = k0, k0 + 8, ... below H.
  auto heads_in = [&](int s, int x, int* k0) {
    *k0 = (x - (s % kPrefillQueues) * (H % kPrefillQueues) % kPrefillQueues + kPrefillQueues) % kPrefillQueues;
    return *k0 < H ? (H - 1 - *k0) / kPrefillQueues + 1 : 0;
  };
  for (int j = tid; j < kPrefillQueues * kBuckets; j += kPlanThreads) (&s_count[0][0])[j] = 0;
  __syncthreads();
  const int items = a.num_seqs * a.row_blocks;
  for (int i = tid; i < items; i += kPlanThreads) {
    int seq, rb, full, last;
    classify(i, &seq, &rb, &full, &last);
    if (last < 0) continue;
    for (int x = 0; x < kPrefillQueues; ++x) {
      int k0;
      const int n = heads_in(seq, x, &k0);
      if (n == 0) continue;
      if (full > 0) atomicAdd(&s_count[x][0], full * n);
      atomicAdd(&s_count[x][last], n);
    }
  }
  __syncthreads();
  if (tid < kPrefillQueues) {
    int start = 0;
    for (int y = 0; y < tid; ++y)
      for (int b = 0; b < kBuckets; ++b) start += s_count[y][b];
    int at = start;
    for (int b = 0; b < kBuckets; ++b) {
      s_next[tid][b] = at;
      at += s_count[tid][b];
    }
    // Units past the list's capacity are dropped (only a query_start that decreases can
    // list more units than the capacity, which counts one per query row; counts that
    // wrap around are clamped too: such a batch's output is undefined, its accesses are
    // not).
    const int cap = a.work_cap;
    const int lo = min(max(start, 0), cap), hi = min(max(at, lo), cap);
    a.work_header[tid] = lo;
    a.work_header[kPrefillQueues + tid] = hi - lo;
    a.work_header[kPrefillClaimStride * (tid + 1)] = 0;
  }
  __syncthreads();
  for (int i = tid; i < items; i += kPlanThreads) {
    int seq, rb, full, last;
    classify(i, &seq, &rb, &full, &last);
    if (last < 0) continue;
    for (int x = 0; x < kPrefillQueues; ++x) {
      int k0;
      const int n = heads_in(seq, x, &k0);
      if (n == 0) continue;
      if (full > 0) {
        int at = atomicAdd(&s_next[x][0], full * n);
        for (int k = 0; k < n; ++k)
          for (int p = 0; p < full; ++p, ++at)
            if (static_cast<unsigned>(at) < static_cast<unsigned>(a.work_cap))
              *reinterpret_cast<int4*>(a.work_units + 4 * static_cast<int64_t>(at)) =
                  make_int4(seq, k0 + k * kPrefillQueues, rb, p);
      }
      int at = atomicAdd(&s_next[x][last], n);
      for (int k = 0; k < n; ++k, ++at)
        if (static_cast<unsigned>(at) < static_cast<unsigned>(a.work_cap))
          *reinterpret_cast<int4*>(a.work_units + 4 * static_cast<int64_t>(at)) =
              make_int4(seq, k0 + k * kPrefillQueues, rb, full);
    }
  }
}

// LDS tiles.  A tile holds 32 keys x 128 dims of K (or V) as 32 rows of 256 bytes, filled
// by direct-to-LDS loads: lane i of a load instruction writes the 16 bytes at 16 i of the
// instruction's 1 KiB destination, so one instruction fills 4 rows.  Within a row the
// sixteen 16-byte chunks are permuted, so that the MFMA operand reads spread over the
// banks: chunk c of key k sits at position c ^ (k % 8) in a K tile (an S operand read
// takes one chunk of each of 32 consecutive keys, and any 8 consecutive keys then use 8
// different 16-byte bank groups) and at position c ^ 2 (k % 4) in a V tile (a transposing
// read takes 2 chunks of each of 4 consecutive keys, which then use 8 different bank
// groups).  The permutation costs nothing: each lane simply loads the chunk that belongs
// at its position.
constexpr int kRowBytes = kHead * 2;
constexpr int kTileBytes = kKeys * kRowBytes;  // 8 KiB
constexpr int kStages = 3;                     // tiles in LDS: the one read, two in flight

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0, expcnt 6:4, lgkmcnt 11:8): every
// LDS access of this wave done, and all but the last n vector-memory operations.
constexpr int wait_vm_lds(int n) { return (n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14); }

// LDS byte address of a __shared__ object.
template <class X>
__device__ __forceinline__ uint32_t lds_addr(X* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) X*)(p)));
}

// One tile's four direct-to-LDS loads of this lane: 16 bytes at k_base + k_off[j] into
// the K tile's rows filled by instruction j (LDS k_dst[j] + 16 lane), the same for V.  A
// load writes the LDS at M0 + its instruction offset + 16 lane, so the instructions carry
// no offset: every address is in the operands.  Written out, not through the compiler's
// intrinsic, so that the compiler, which tracks these loads as pending LDS writes, does
// not wait for every load in flight (the next tiles' included) before each LDS read: the
// kernel's own waits (tile_barrier) order these loads against the reads.  The loads write
// no register.  Each M0 write is one wait state ahead of the load that reads it, and the
// s_nop covers a scalar base that a VALU instruction (readlane) wrote.
__device__ __forceinline__ void dma_tile(const void* k_base, const void* v_base, uint32_t k_off0,
                                         uint32_t k_off1, uint32_t v_off0, uint32_t v_off1,
                                         uint32_t k_dst0, uint32_t k_dst1, uint32_t v_dst0,
                                         uint32_t v_dst1) {
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %0\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %0\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %1\n\t"
      "s_mov_b32 m0, %9\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %1"
      :
      : "s"(k_base), "s"(v_base), "v"(k_off0), "v"(k_off1), "v"(v_off0), "v"(v_off1),
        "s"(k_dst0), "s"(k_dst1), "s"(v_dst0), "s"(v_dst1)
      : "memory", "m0");
}

template <class M, int G>
__global__ __launch_bounds__(256, kPrefillBlocksPerCu) void prefill_kernel(const PrefillArgs a) {
  using T = typename M::elem;
  typedef T T2 __attribute__((ext_vector_type(2)));
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  constexpr int TR = kCols / G;  // query rows per unit

  __shared__ __align__(16) unsigned char s_k[kStages][kTileBytes];
  __shared__ __align__(16) unsigned char s_v[kStages][kTileBytes];
  __shared__ int4 s_unit;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int half = lane / 32;  // which 8 of a 16-dim slice, which 4 keys of 8

  // Per-lane LDS and global offsets, the same for every tile.
  //  Loads: instruction j (0, 1) of wave w fills rows 4 (2 w + j) .. + 3 of a tile; lane l
  //  of it takes key kl = 4 (2 w + j) + l / 16 at position p = l % 16.  Waves 0 and 1 load
  //  keys 0 .. 15 of a tile, waves 2 and 3 keys 16 .. 31 (the two halves' blocks differ
  //  when blocks hold 16 keys), so every instruction reads one block.
  //  Byte offsets within the 16 rows of the wave's half, of instruction 0; instruction 1
  //  reads 4 rows further on, whose K chunk is permuted by key % 8 + 4: chunk c ^ 4, i.e.
  //  byte (k_src ^ 64) + 1024 (bit 6 of k_src holds bit 2 of c); V's permutation repeats
  //  every 4 keys: byte v_src + 1024.
  int k_src, v_src;
  {
    const int kl = 4 * (2 * wave) + lane / 16, p = lane % 16;  // kl % 8 < 4
    k_src = kRowBytes * (kl & 15) + 16 * (p ^ (kl % 8));
    v_src = kRowBytes * (kl & 15) + 16 * (p ^ (2 * (kl % 4)));
  }
  //  S operand (K rows): lane l reads key l % 32, chunk 2 sl + half, at byte
  //  256 key + 16 ((2 sl + half) ^ (key % 8)) = 128 (sl / 4) + (k_rd ^ 32 (sl % 4)) with
  //  k_rd = 256 key + 32 ka + 16 kb, ka = (key % 8) / 2, kb = half ^ (key % 2) (the XOR
  //  only touches the bits that hold ka).
  const int k_rd = kRowBytes * (lane % 32) + 32 * ((lane % 8) / 2) + 16 * (half ^ (lane % 2));
  //  PV operand (V^T by transposing reads): for dims 32 dt .. + 31 and keys 16 q + 8 j +
  //  4 half .. + 3, lane L = l % 16 of 16-lane group g = l / 16 supplies the address of the
  //  4 dims 32 dt + 16 (g % 2) + 4 (L % 4) .. + 3 of key 16 q + 8 j + 4 half + L / 4; lane
  //  i of the group then receives, for e = 0 .. 3, dim 32 dt + 16 (g % 2) + i of key
  //  16 q + 8 j + 4 half + e, i.e. its own dim's four keys.  With x = 2 (g % 2) + (L % 4) / 2
  //  the chunk is 4 dt + x, at position (4 dt + x) ^ 2 (L / 4) = 4 (dt ^ (L / 8)) + (x ^
  //  (2 (L / 4) % 4)): byte 256 (16 q + 8 j) + 128 (dt / 2) + (v_rd0 ^ 64 (dt % 2))
  //  (bit 6 of v_rd[0] holds L / 8, so v_rd[1] = v_rd[0] ^ 64).
  int v_rd0;
  {
    const int L = lane % 16, g = lane / 16, x = 2 * (g % 2) + (L % 4) / 2;
    v_rd0 = kRowBytes * (4 * half + L / 4) + 16 * (x ^ (2 * (L / 4) % 4)) + 8 * (L % 2) + 64 * (L / 8);
  }

  // Persistent: claim units from this XCD's queue, then, once it is empty, from the queue
  // with the most units left.  Only thread 0 claims; the unit reaches the others through
  // the LDS.  The queues' starts and lengths are read once.
  __shared__ int s_hdr[2 * kPrefillQueues];
  if (tid < 2 * kPrefillQueues) s_hdr[tid] = a.work_header[tid];
  int queue = static_cast<int>(__builtin_amdgcn_s_getreg((3 << 11) | 20)) & (kPrefillQueues - 1);  // XCC_ID
  unsigned live = 0xffffffffu;  // queues not known to be empty (thread 0's view)
  auto counter = [&](int x) { return a.work_header + kPrefillClaimStride * (x + 1); };

  while (true) {
    // Every wave has read the previous unit from s_unit (a unit that writes only NaN rows
    // passes no other barrier) and is done with the LDS tiles; s_hdr is in place.
    __syncthreads();
    if (tid == 0) {
      int4 u = make_int4(-1, 0, 0, 0);
      if (live == 0xffffffffu) {
        live = 0;
        for (int x = 0; x < kPrefillQueues; ++x) live |= (s_hdr[kPrefillQueues + x] > 0 ? 1u : 0u) << x;
      }
      // Every pass takes an index of a queue or drops a queue from `live`.
      while (live != 0) {
        if ((live >> queue & 1u) != 0) {
          const int idx = atomicAdd(counter(queue), 1);
          if (idx < s_hdr[kPrefillQueues + queue]) {
            u = *reinterpret_cast<const int4*>(a.work_units + 4 * static_cast<int64_t>(s_hdr[queue] + idx));
            // A well-formed batch lists only valid units; the check keeps a garbled list
            // (a query_start that decreases) from reaching outside the arguments.
            if (u.x >= 0 && u.x < a.num_seqs && u.y >= 0 && u.y < a.num_kv_heads && u.z >= 0 &&
                u.z < a.row_blocks && u.w >= 0 && u.w < a.pmax)
              break;
            u = make_int4(-1, 0, 0, 0);
            continue;
          }
          live &= ~(1u << queue);
        }
        // Another queue: every counter read at once (coherently, past this XCD's L2).
        int left[kPrefillQueues];
#pragma unroll
        for (int x = 0; x < kPrefillQueues; ++x)
          left[x] = s_hdr[kPrefillQueues + x] -
                    __hip_atomic_load(counter(x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int best = -1, most = 0;
#pragma unroll
        for (int x = 0; x < kPrefillQueues; ++x) {
          if (left[x] <= 0) live &= ~(1u << x);
          if ((live >> x & 1u) != 0 && left[x] > most) {
            most = left[x];
            best = x;
          }
        }
        if (best >= 0) queue = best;
      }
      s_unit = u;
    }
    // Every wave sees the new unit.
    __syncthreads();
    const int4 unit = s_unit;
    if (unit.x < 0) break;  // uniform: the queues are empty
    const int seq = __builtin_amdgcn_readfirstlane(unit.x);
    const int kvh = __builtin_amdgcn_readfirstlane(unit.y);
    const int r0 = __builtin_amdgcn_readfirstlane(unit.z) * TR;
    const int part = __builtin_amdgcn_readfirstlane(unit.w);

    const SeqInfo si = seq_info(a, seq);
    const int qs = si.qs, n_rows = si.n_rows, L = si.L;
    if (r0 >= n_rows) continue;  // uniform (the plan lists no such unit)

    // This lane's column: wave w holds columns 32w .. 32w + 31; column n is query head
    // n / TR of the group, row r0 + n % TR of the sequence's chunk.
    const int col = wave * 32 + (lane % 32);
    const int hh = col / TR;
    const int row = r0 + col % TR;
    const bool col_ok = row < n_rows;
    const int pos = L - n_rows + row;  // the row's position; it sees keys 0 .. pos
    // The wave's first row: no column of the wave sees fewer keys than it.
    const int pos_min = L - n_rows + r0 + (TR >= 32 ? (32 * wave) % TR : 0);
    const int64_t out_row = (static_cast<int64_t>(qs) + row) * a.num_q_heads + kvh * G + hh;

    // A sequence with bad metadata runs no tile: its part-0 unit writes NaN rows (where
    // its rows lie inside the query rows) through the common epilogue.
    if (si.bad && (part != 0 || !si.rows_ok)) continue;
    // Largest key any column of the unit sees, and this part's tiles of 0 .. kmax.
    const int kmax = si.bad ? -1 : L - n_rows + min(r0 + TR, n_rows) - 1;
    const int n_parts = si.bad ? 1 : kmax / a.part_keys + 1;
    if (part >= n_parts) continue;  // uniform (the plan lists no such unit)
    const int t_first = part * (a.part_keys / kKeys);
    const int n_tiles = si.bad ? 0 : min(kmax, (part + 1) * a.part_keys - 1) / kKeys - t_first + 1;  // <= 64

    // Block ids of the unit's tiles, lane i holding tile t_first + i's: keys t0 .. t0 + 15
    // lie in the block of key t0 and keys t0 + 16 .. t0 + 31 in that of key t0 + 16 (the
    // same block once blocks hold 32 keys or more), each clamped to kmax, so that every
    // load stays inside blocks of the sequence.  An id outside the pool makes every output
    // of the unit NaN (and is read as block 0).
    const int32_t* tbl = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
    const int sh = a.block_shift;
    const int bmask = a.block_size - 1;
    const bool upper = wave >= 2;  // this wave loads keys 16 .. 31 of every tile
    int id = 0;
    if (lane < n_tiles) id = tbl[min((t_first + lane) * kKeys + (upper ? kKeys / 2 : 0), kmax) >> sh];
    const bool out_of_pool = static_cast<unsigned>(id) >= static_cast<unsigned>(a.num_blocks);
    // Known to every wave at the end of the unit (__syncthreads_or there).
    const bool wave_bad = si.bad || __builtin_amdgcn_ballot_w64(out_of_pool) != 0;
    if (out_of_pool) id = 0;

    // Q^T operands: slice s covers dims 16s .. 16s + 15; lane l holds dims 16s + 8 half ..
    // + 7 of its column.
    u32x4 qb[8];
    {
      const u32x4* qrow = reinterpret_cast<const u32x4*>(static_cast<const T*>(a.q) + out_row * kHead);
#pragma unroll
      for (int s = 0; s < 8; ++s) qb[s] = col_ok ? (qrow[2 * s + half] & a.q_and) ^ a.q_xor : u32x4{0u, 0u, 0u, 0u};
    }

    // The K and V rows of tile r go into stage st: four direct loads per thread, whatever
    // the keys (rows past kmax are read from the clamped blocks, inside the sequence), so
    // that every tile's loads number the same and the waits on them stay exact.
    const int64_t run_elems = static_cast<int64_t>(a.block_size) * kHead;
    const int64_t blk_elems = static_cast<int64_t>(a.num_kv_heads) * run_elems;
    auto issue_tile = [&](int r, int st) {
      const int t0 = (t_first + r) * kKeys;
      const int blk = __builtin_amdgcn_readlane(id, r);
      const int row0 = (t0 + (upper ? kKeys / 2 : 0)) & bmask;
      const int64_t base = blk * blk_elems + kvh * run_elems + static_cast<int64_t>(row0) * kHead;
      const T* kc = static_cast<const T*>(a.k_cache) + base;
      const T* vc = static_cast<const T*>(a.v_cache) + base;
      dma_tile(kc, vc, k_src, (k_src ^ 64) + 1024, v_src, v_src + 1024,
               __builtin_amdgcn_readfirstlane(lds_addr(&s_k[st][1024 * (2 * wave)])),
               __builtin_amdgcn_readfirstlane(lds_addr(&s_k[st][1024 * (2 * wave + 1)])),
               __builtin_amdgcn_readfirstlane(lds_addr(&s_v[st][1024 * (2 * wave)])),
               __builtin_amdgcn_readfirstlane(lds_addr(&s_v[st][1024 * (2 * wave + 1)])));
    };
    // Wait for this thread's loads of the tile about to be read (all but the `newer` tiles'
    // loads issued after it) and its LDS accesses, then for every wave.
    auto tile_barrier = [&](bool newer) {
      asm volatile("" ::: "memory");
      if (newer)
        __builtin_amdgcn_s_waitcnt(wait_vm_lds(4));
      else
        __builtin_amdgcn_s_waitcnt(wait_vm_lds(0));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m_ref = -INFINITY;  // reference maximum of this lane's column (base 2)
    float l_part = 0.0f;      // sum of this lane's probabilities (its 16 keys of each tile)

    // One tile: scores, softmax and PV from stage ST.
    auto step = [&](int r, auto stage) {
      constexpr int ST = decltype(stage)::value;
      const unsigned char* kb = s_k[ST];
      const unsigned char* vb = s_v[ST];
      const int t0 = (t_first + r) * kKeys;
      // V rows past kmax (only in a unit's last tile) are zeroed: a zero probability times
      // a NaN from unused cache memory would still be NaN.  Each thread clears the rows it
      // loaded, after its loads landed, before every wave reads them.
      if (t0 + kKeys - 1 > kmax) {
        // The zeros are made here (not kept in registers through the loop).
        u32x4 z;
        asm volatile("v_mov_b32 %0, 0\n\tv_mov_b32 %1, 0\n\tv_mov_b32 %2, 0\n\tv_mov_b32 %3, 0"
                     : "=v"(z.x), "=v"(z.y), "=v"(z.z), "=v"(z.w));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kl = 4 * (2 * wave + j) + lane / 16;
          if (t0 + kl > kmax) *reinterpret_cast<u32x4*>(&s_v[ST][1024 * (2 * wave + j) + 16 * lane]) = z;
        }
        tile_barrier(false);
      }
      // S^T (32 keys x this wave's 32 columns).
      f32x16 s = f32x16{};
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(kb + (k_rd ^ (32 * (sl % 4))) + 128 * (sl / 4));
        s = M::mma(ka, qb[sl], s);
      }
      // Causal mask, only on tiles that reach past the wave's first position; lane holds
      // keys t0 + 8j + 4 half + i, j, i = 0..3.  (Columns past the chunk have pos >= L and
      // zero queries: they compute finite values that are never stored.)
      if (t0 + kKeys - 1 > pos_min) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = t0 + 8 * (rr / 4) + 4 * half + (rr % 4);
          s[rr] = key <= pos ? s[rr] : -INFINITY;
        }
      }
      // Maximum of the raw scores (the score scale is positive: the sign of the caller's
      // scale went into the queries), then base 2.
      float tmax = s[0];
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) tmax = fmaxf(tmax, s[rr]);
      {
        // The column's other 16 keys sit in lane l ^ 32: swapping the wave's two halves in
        // registers (no LDS round trip) gives each lane its own value and its partner's.
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                                         false, false);
        tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float c = a.scale_log2;
      const float tm = tmax * c;
      // Rescale when any column of the wave needs it (rare after the first tiles); a branch
      // the whole wave takes or skips, so that the 64 products are not paid on every tile.
      const bool need = tm > m_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - tm) : 1.0f;  // 0 on the first tile
        m_ref = need ? tm : m_ref;
        l_part *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      }
      // Probabilities exp2(s c - m), split into a 16-bit value and the 16-bit rounding of
      // the rest.  A column that has seen no key yet (possible in a later part of a split
      // range) keeps m = -inf: its masked scores must give 0, not -inf - -inf.
      const float mr = m_ref == -INFINITY ? 0.0f : m_ref;
      uint32_t ph[8], pl[8];
#pragma unroll
      for (int rr = 0; rr < 16; rr += 2) {
        const f32x2 p = f32x2{__builtin_amdgcn_exp2f(fmaf(s[rr], c, -mr)),
                              __builtin_amdgcn_exp2f(fmaf(s[rr + 1], c, -mr))};
        l_part += p.x + p.y;
        // Two probabilities per conversion (round to nearest even), then the remainders.
        const T2 h = __builtin_convertvector(p, T2);
        const f32x2 hf = __builtin_convertvector(h, f32x2);
        const T2 e = __builtin_convertvector(f32x2{p.x - hf.x, p.y - hf.y}, T2);
        ph[rr / 2] = __builtin_bit_cast(uint32_t, h);
        pl[rr / 2] = __builtin_bit_cast(uint32_t, e);
      }
      // O^T += V^T P^T: MFMA q covers keys 16q .. 16q + 15; its B operand is this lane's
      // probabilities 8q .. 8q + 7, whose keys (in operand order) are 16q + 4 half + i and
      // 16q + 8 + 4 half + i, i = 0..3; the A operand (V^T) takes the same keys, in the same
      // order, from two transposing reads.
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32x4 bh = u32x4{ph[4 * q], ph[4 * q + 1], ph[4 * q + 2], ph[4 * q + 3]};
        const u32x4 bl = u32x4{pl[4 * q], pl[4 * q + 1], pl[4 * q + 2], pl[4 * q + 3]};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const unsigned char* vr = vb + (v_rd0 ^ (64 * (dt % 2))) + 128 * (dt / 2) + kRowBytes * 16 * q;
          typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vr));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vr + kRowBytes * 8));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          const u32x4 va = u32x4{lo2.x, lo2.y, hi2.x, hi2.y};
          o[dt] = M::mma(va, bh, o[dt]);
          o[dt] = M::mma(va, bl, o[dt]);
        }
      }
    };

    // Pipeline: at step r the LDS holds tile r (stage r % 3, read now) and tiles r + 1 and
    // r + 2 are in flight or landed (stages (r + 1) % 3, (r + 2) % 3).  Step r begins by
    // waiting for tile r's loads (all but tile r + 1's four loads, issued after them) and a
    // barrier, which also ends every wave's reads of stage (r + 2) % 3 = (r - 1) % 3 in
    // step r - 1; it then issues tile r + 2's loads into that stage.
    if (n_tiles > 0) issue_tile(0, 0);
    asm volatile("" ::: "memory");  // tile 0's loads strictly before tile 1's
    if (n_tiles > 1) issue_tile(1, 1);
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    for (int r = 0; r < n_tiles; r += kStages) {
      tile_barrier(r + 1 < n_tiles);
      if (r + 2 < n_tiles) issue_tile(r + 2, 2);
      step(r, S0{});
      if (r + 1 >= n_tiles) break;
      tile_barrier(r + 2 < n_tiles);
      if (r + 3 < n_tiles) issue_tile(r + 3, 0);
      step(r + 1, S1{});
      if (r + 2 >= n_tiles) break;
      tile_barrier(r + 3 < n_tiles);
      if (r + 4 < n_tiles) issue_tile(r + 4, 1);
      step(r + 2, S2{});
    }

    // A block id outside the pool anywhere in the unit's keys makes every output NaN.
    const bool bad_blk = __syncthreads_or(wave_bad);
    // Columns past the chunk (their partner lane l ^ 32 is the same column) write nothing.
    if (col_ok) {
      const float l_col = l_part + __shfl_xor(l_part, 32);
      // A column may see no key of a later part (its row ends before the part): it then
      // weighs nothing in the merge (lse -inf, o 0).
      const float inv = bad_blk ? __builtin_nanf("") : (l_col > 0.0f ? 1.0f / l_col : 0.0f);
      float* dst = a.out + out_row * kHead;
      if (n_parts > 1) {
        const int64_t prow = out_row * a.pmax + part;
        dst = a.part_o + prow * kHead;
        if (half == 0)
          a.part_lse[prow] = bad_blk ? __builtin_nanf("") : (l_col > 0.0f ? m_ref + __log2f(l_col) : -INFINITY);
      }
      // Lane holds dims 32 dt + 8 j + 4 half + i of its column.
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = f32x4{o[dt][4 * j], o[dt][4 * j + 1], o[dt][4 * j + 2], o[dt][4 * j + 3]} * inv;
          *reinterpret_cast<f32x4*>(dst + 32 * dt + 8 * j + 4 * half) = v;
        }
    }
  }
}

// Log-sum-exp merge of a row block's parts, for row blocks with more than one: the same
// (row block, sequence, KV head) grid with each row block's kMergeSlices workgroups side by
// side, one thread per (column, 4 dims) item, so every thread's loads are independent.
//   M = max_p lse_p,  w_p = 2^(lse_p - M),  out = sum_p w_p o_p / sum_p w_p
// (the identity of the softmax over a union of key sets; o_p is part p's normalized
// output, lse_p its base-2 log-sum-exp).  A NaN in any part makes the output NaN.
constexpr int kMergeSlices = kCols * (kHead / 4) / 256;

template <int G>
__global__ __launch_bounds__(256) void prefill_merge_kernel(const PrefillArgs a) {
  constexpr int TR = kCols / G;
  const int seq = blockIdx.y;
  const int kvh = blockIdx.z;
  const int r0 = (blockIdx.x / kMergeSlices) * TR;
  const SeqInfo si = seq_info(a, seq);
  const int qs = si.qs, n_rows = si.n_rows, L = si.L;
  if (r0 >= n_rows) return;
  if (si.bad) return;  // the prefill kernel wrote its NaNs straight to out
  const int kmax = L - n_rows + min(r0 + TR, n_rows) - 1;
  const int n_parts = kmax / a.part_keys + 1;
  if (n_parts == 1) return;
  {
    const int item = (blockIdx.x % kMergeSlices) * 256 + threadIdx.x;
    const int col = item / (kHead / 4);
    const int d4 = (item % (kHead / 4)) * 4;
    const int row = r0 + col % TR;
    if (row >= n_rows) return;
    const int64_t out_row = (static_cast<int64_t>(qs) + row) * a.num_q_heads + kvh * G + col / TR;
    const float* lse = a.part_lse + out_row * a.pmax;
    const float* po = a.part_o + out_row * a.pmax * kHead + d4;
    // Parts four at a time, every load of a group issued before its arithmetic (parts past
    // n_parts read as lse -inf, weight 0).  Part 0 holds key 0, which every row sees, so M
    // is finite unless a part is NaN.
    float M = -INFINITY;
    bool has_nan = false;
    for (int p0 = 0; p0 < n_parts; p0 += 4) {
      float l[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) l[i] = p0 + i < n_parts ? lse[p0 + i] : -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        has_nan |= l[i] != l[i];
        M = fmaxf(M, l[i]);
      }
    }
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float wsum = 0.0f;
    for (int p0 = 0; p0 < n_parts; p0 += 4) {
      float l[4];
      f32x4 o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = p0 + i < n_parts;
        l[i] = ok ? lse[p0 + i] : -INFINITY;
        o[i] = ok ? *reinterpret_cast<const f32x4*>(po + (p0 + i) * kHead) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float w = __builtin_amdgcn_exp2f(l[i] - M);
        wsum += w;
        acc += w * o[i];
      }
    }
    const float nan = __builtin_nanf("");
    *reinterpret_cast<f32x4*>(a.out + out_row * kHead + d4) =
        has_nan ? f32x4{nan, nan, nan, nan} : acc / wsum;
  }
}

template <class M, int G>
hipError_t launch_persistent(const PrefillArgs& a, hipStream_t s) {
  // Workgroups resident at once on the current device (cached per device).
  static int cached[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prefill_kernel<M, G>, 256, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached[dev] = std::max(1, per_cu) * std::max(1, cus);
  }
  // No more workgroups than units can exist.
  const int64_t upper = static_cast<int64_t>(a.num_seqs) * a.row_blocks * a.pmax * a.num_kv_heads;
  const int grid = static_cast<int>(std::min<int64_t>(cached[dev], std::min<int64_t>(upper, a.work_cap)));
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_kernel<M, G>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class M>
hipError_t launch_typed(const PrefillArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_persistent<M, 1>(a, s);
    case 2: return launch_persistent<M, 2>(a, s);
    case 4: return launch_persistent<M, 4>(a, s);
    case 8: return launch_persistent<M, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill_plan(const PrefillArgs& a, int group, hipStream_t s) {
  (void)hipGetLastError();
  if (group != 1 && group != 2 && group != 4 && group != 8) return hipErrorInvalidValue;
  if (a.num_seqs == 0 || a.row_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a, kCols / group);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int group, hipStream_t s) {
  (void)hipGetLastError();
  if (a.num_seqs == 0 || a.row_blocks == 0) return hipSuccess;
  switch (dtype) {
    case 1: return launch_typed<MmaF16>(a, group, s);
    case 2: return launch_typed<MmaBF16>(a, group, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_merge(const PrefillArgs& a, int group, int max_query_len, hipStream_t s) {
  (void)hipGetLastError();
  if (a.pmax <= 1) return hipSuccess;
  const int tr = kCols / group;
  const dim3 grid(static_cast<unsigned>((max_query_len + tr - 1) / tr * kMergeSlices),
                  static_cast<unsigned>(a.num_seqs), static_cast<unsigned>(a.num_kv_heads));
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  switch (group) {
    case 1: hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_merge_kernel<1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_merge_kernel<2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_merge_kernel<4>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_merge_kernel<8>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
