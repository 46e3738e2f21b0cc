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
//   * O^T += V^T P^T with the same MFMA, V staged transposed in LDS.  P goes in as two
//     MFMA operands, its bf16 (or fp16) rounding and the rounding of the remainder, so
//     the only error left is the fp32 accumulation (a single rounding of P could move an
//     output by several 1e-3 on rows that see only a few keys).
//   * Causal and length masks by select; V rows past the context are zeroed when staged
//     (a zero probability times a NaN from unused cache memory would still be NaN).
#include <math.h>

#include <algorithm>

#include "prefill.hpp"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr int kHead = 128;    // head_dim
constexpr int kKeys = 32;     // keys per tile
constexpr int kCols = kPrefillColumns;  // (row, head) columns per workgroup
constexpr int kKRow = kHead + 8;   // K tile row stride in LDS (elements), against bank conflicts
// Transposed V tile row stride (elements): 18 dwords.  A staging store of a wave writes
// 16 key pairs of 8 dims rows apart for each of its four 8-dim groups, 144 dwords apart:
// 16 banks apart, so the 64 stores fill the banks twice over (at 20 dwords they were 160
// apart and four-way conflicted).  The PV operand reads (8 bytes, 16 rows per pass) land
// 18 dwords apart, on distinct bank pairs.
constexpr int kVRow = kKeys + 4;
constexpr float kRescaleSlack = 8.0f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// A load the compiler makes a scalar load: the address is the same for every lane and
// the data is not written while the kernel runs.
template <class X>
__device__ __forceinline__ X ld_uniform(const X* p, int64_t i) {
  return ((const __attribute__((address_space(4))) X*)(p))[i];
}

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

template <class M, int G>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const PrefillArgs a) {
  using T = typename M::elem;
  typedef T T2 __attribute__((ext_vector_type(2)));
  constexpr int TR = kCols / G;  // query rows per workgroup
  constexpr int kTileK = kKeys * kKRow;
  constexpr int kTileV = kHead * kVRow;

  // Two buffers of each tile: while one is read, the next tile is stored into the other,
  // so a tile costs one barrier.
  __shared__ __align__(16) T s_k[2 * kTileK];   // K tile, [key][dim]
  __shared__ __align__(16) T s_vt[2 * kTileV];  // V tile transposed, [dim][key]
  __shared__ int4 s_unit;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int half = lane / 32;  // which 8 of a 16-dim slice, which 4 keys of 8
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
    // passes no other barrier); s_hdr is in place.
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
    // Every wave sees the new unit (and is past the previous unit's LDS reads).
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

    if (si.bad) {
      if (part == 0 && col_ok && si.rows_ok) {
#pragma unroll
        for (int d4 = 0; d4 < kHead; d4 += 8)
          *reinterpret_cast<f32x4*>(a.out + out_row * kHead + d4 + 4 * half) =
              f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      }
      continue;
    }

    // Q^T operands: slice s covers dims 16s .. 16s + 15; lane l holds dims 16s + 8 half ..
    // + 7 of its column.
    u32x4 qb[8];
    {
      const u32x4* qrow = reinterpret_cast<const u32x4*>(static_cast<const T*>(a.q) + out_row * kHead);
#pragma unroll
      for (int s = 0; s < 8; ++s) qb[s] = col_ok ? (qrow[2 * s + half] & a.q_and) ^ a.q_xor : u32x4{0u, 0u, 0u, 0u};
    }

    // Largest key any column of the workgroup sees, and this part's tiles of 0 .. kmax.
    const int kmax = L - n_rows + min(r0 + TR, n_rows) - 1;
    const int n_parts = kmax / a.part_keys + 1;
    if (part >= n_parts) continue;  // uniform (the plan lists no such unit)
    const int t_first = part * (a.part_keys / kKeys);
    const int n_tiles = min(kmax, (part + 1) * a.part_keys - 1) / kKeys - t_first + 1;

    // Staging: thread t moves 16-byte chunk t / 16 of keys 2 (t % 16) and 2 (t % 16) + 1
    // (one block: block sizes are powers of two >= 16).  The 16 threads of a chunk hold 16
    // key pairs, so their stores into the transposed V tile are 16 consecutive dwords of
    // one row (distinct banks), and each global load still reads 64 contiguous bytes of
    // every key it touches.  Every load below is issued whatever the key: keys past kmax
    // read an in-bounds row and are zeroed when staged, so the loads of a tile always
    // number the same and the waits before using them stay exact.
    const int sk = 2 * (tid % 16);
    const int sc = tid / 16;
    const int32_t* tbl = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
    const int64_t run_elems = static_cast<int64_t>(a.block_size) * kHead;
    const int64_t blk_elems = static_cast<int64_t>(a.num_kv_heads) * run_elems;  // one block of the array
    const int sh = a.block_shift;
    const int bmask = a.block_size - 1;
    // The block ids of a tile are the same for the whole workgroup: keys t0 .. t0 + 15 lie
    // in the block of key t0 and keys t0 + 16 .. t0 + 31 in that of key t0 + 16 (the same
    // block once blocks hold 32 keys or more), each clamped to kmax.  They are read with
    // scalar loads, and a thread's element offset is one of the two scalar bases (its keys'
    // half of the tile) plus a part that does not change from tile to tile.
    const int64_t lane_off = sc * 8 + static_cast<int64_t>(sk & bmask) * kHead;
    const bool upper_keys = sk >= kKeys / 2;
    bool bad_blk = false;  // a block id outside the pool (wave-uniform)
    struct TileBase {
      int64_t lo, hi;  // element offsets of keys t0 .. t0 + 15 and t0 + 16 .. t0 + 31
    };
    auto tile_block = [&](int t) -> TileBase {
      const int t0 = t * kKeys;
      int id0 = ld_uniform(tbl, min(t0, kmax) >> sh);
      int id1 = ld_uniform(tbl, min(t0 + kKeys / 2, kmax) >> sh);
      // Both keys are at most kmax, so both blocks hold keys this workgroup attends to.
      if (static_cast<unsigned>(id0) >= static_cast<unsigned>(a.num_blocks)) {
        bad_blk = true;
        id0 = 0;
      }
      if (static_cast<unsigned>(id1) >= static_cast<unsigned>(a.num_blocks)) {
        bad_blk = true;
        id1 = 0;
      }
      const int64_t in_blk = static_cast<int64_t>(kvh) * run_elems + static_cast<int64_t>(t0 & bmask) * kHead;
      return TileBase{id0 * blk_elems + in_blk, id1 * blk_elems + in_blk};
    };
    // Global address (elements) of this thread's first row of tile t.  The bases are
    // copied to values first: a lane-dependent choice between two members of one object
    // becomes a lane-dependent address into a private array (scratch memory).
    auto tile_rows = [&](const TileBase b) -> int64_t {
      const int64_t lo = b.lo, hi = b.hi;
      return (upper_keys ? hi : lo) + lane_off;
    };
    auto issue_k = [&](const TileBase b, u32x4 (&kr)[2]) {
      const int64_t off = tile_rows(b);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        kr[j] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.k_cache) + off + j * kHead);
    };
    auto issue_v = [&](int t, const TileBase b, u32x4 (&vr)[2], int& valid) {
      const int key = t * kKeys + sk;
      valid = (key <= kmax ? 1 : 0) | (key + 1 <= kmax ? 2 : 0);
      const int64_t off = tile_rows(b);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        vr[j] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.v_cache) + off + j * kHead);
    };
    auto store_k = [&](int buf, const u32x4 (&kr)[2]) {
      T* sk_buf = s_k + buf * kTileK;
      *reinterpret_cast<u32x4*>(&sk_buf[sk * kKRow + sc * 8]) = kr[0];
      *reinterpret_cast<u32x4*>(&sk_buf[(sk + 1) * kKRow + sc * 8]) = kr[1];
    };
    auto store_v = [&](int buf, const u32x4 (&vr)[2], int valid) {
      T* sv_buf = s_vt + buf * kTileV;
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      const u32x4 v0 = (valid & 1) ? vr[0] : z, v1 = (valid & 2) ? vr[1] : z;
      // V transposed: dims sc * 8 .. + 7, keys sk and sk + 1 side by side.
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // Byte permutes: low halves of the two keys' dwords, then high halves.
        const int d = sc * 8 + 2 * w;
        *reinterpret_cast<uint32_t*>(&sv_buf[d * kVRow + sk]) = __builtin_amdgcn_perm(v1[w], v0[w], 0x05040100u);
        *reinterpret_cast<uint32_t*>(&sv_buf[(d + 1) * kVRow + sk]) = __builtin_amdgcn_perm(v1[w], v0[w], 0x07060302u);
      }
    };

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m_ref = -INFINITY;  // reference maximum of this lane's column (base 2)
    float l_part = 0.0f;      // sum of this lane's probabilities (its 16 keys of each tile)

    // S^T of a tile (32 keys x this wave's 32 columns) from the K buffer kb.
    auto scores = [&](const T* kb) -> f32x16 {
      f32x16 s = f32x16{};
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(&kb[(lane % 32) * kKRow + 16 * sl + 8 * half]);
        s = M::mma(ka, qb[sl], s);
      }
      return s;
    };

    // Softmax and PV of tile t, whose scores are in s, with V from the buffer vb.  The next
    // tile's scores are computed meanwhile from the K buffer kb_next and left in s: their
    // MFMAs do not depend on this tile's vector work, so the two interleave in the wave's
    // instruction stream and the matrix cores run while the softmax does.
    auto step = [&](int t, f32x16& s, const T* kb_next, const T* vb) {
      const int t0 = t * kKeys;
      // Causal mask, only on tiles that reach past the wave's first position; lane holds
      // keys t0 + 8j + 4 half + i, j, i = 0..3.  (Columns past the chunk have pos >= L and
      // zero queries: they compute finite values that are never stored.)
      if (t0 + kKeys - 1 > pos_min) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t0 + 8 * (r / 4) + 4 * half + (r % 4);
          s[r] = key <= pos ? s[r] : -INFINITY;
        }
      }
      // Maximum of the raw scores (the score scale is positive: the sign of the caller's
      // scale went into the queries), then base 2.
      float tmax = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
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
      const f32x16 s_next = scores(kb_next);
      // Probabilities exp2(s c - m), split into a 16-bit value and the 16-bit rounding of
      // the rest.  A column that has seen no key yet (possible in a later part of a split
      // range) keeps m = -inf: its masked scores must give 0, not -inf - -inf.
      const float mr = m_ref == -INFINITY ? 0.0f : m_ref;
      uint32_t ph[8], pl[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const f32x2 p = f32x2{__builtin_amdgcn_exp2f(fmaf(s[r], c, -mr)),
                              __builtin_amdgcn_exp2f(fmaf(s[r + 1], c, -mr))};
        l_part += p.x + p.y;
        // Two probabilities per conversion (round to nearest even), then the remainders.
        const T2 h = __builtin_convertvector(p, T2);
        const f32x2 hf = __builtin_convertvector(h, f32x2);
        const T2 e = __builtin_convertvector(f32x2{p.x - hf.x, p.y - hf.y}, T2);
        ph[r / 2] = __builtin_bit_cast(uint32_t, h);
        pl[r / 2] = __builtin_bit_cast(uint32_t, e);
      }
      // O^T += V^T P^T: MFMA q covers keys 16q .. 16q + 15; its B operand is this lane's
      // probabilities 8q .. 8q + 7, whose keys (in operand order) are 16q + 4 half + i and
      // 16q + 8 + 4 half + i, i = 0..3.
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32x4 bh = u32x4{ph[4 * q], ph[4 * q + 1], ph[4 * q + 2], ph[4 * q + 3]};
        const u32x4 bl = u32x4{pl[4 * q], pl[4 * q + 1], pl[4 * q + 2], pl[4 * q + 3]};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const T* vrow = &vb[(32 * dt + lane % 32) * kVRow + 16 * q + 4 * half];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
          const u32x4 va = u32x4{lo.x, lo.y, hi.x, hi.y};
          o[dt] = M::mma(va, bh, o[dt]);
          o[dt] = M::mma(va, bl, o[dt]);
        }
      }
      s = s_next;
    };

    // Pipeline.  K runs one tile ahead of V: during step r (tile r of the part) the LDS
    // holds K of tile r + 1 (buffer (r + 1) % 2, for the next scores) and V of tile r
    // (buffer r % 2); the stores at the end of the step put K of tile r + 2 into buffer r % 2
    // and V of tile r + 1 into buffer (r + 1) % 2, both last read in the step before.  The
    // loads of a step's stores were issued at the top of the step before, into the other of
    // two register sets, and block ids run one tile ahead of the K loads.  Every load is
    // issued whatever the key: keys past kmax read an in-bounds row (K rows past it are
    // masked through their scores, V rows zeroed when staged), so the loads in flight always
    // number the same and the waits before the stores stay exact.
    const T* kbuf0 = s_k;
    const T* kbuf1 = s_k + kTileK;
    const T* vbuf0 = s_vt;
    const T* vbuf1 = s_vt + kTileV;
    u32x4 kA[2], vA[2], kB[2], vB[2];
    int mA, mB;
    const TileBase id0 = tile_block(t_first);
    const TileBase id1 = tile_block(t_first + 1);
    issue_k(id0, kA);
    issue_v(t_first, id0, vA, mA);
    issue_k(id1, kB);
    store_k(0, kA);
    store_v(0, vA, mA);
    store_k(1, kB);
    __syncthreads();
    f32x16 s = scores(kbuf0);
    // Every wave has read K buffer 0 before the first step's stores overwrite it.
    __syncthreads();
    // The loads of the first step's stores, and the block ids of the two tiles after them.
    TileBase id_v = tile_block(t_first + 2);  // blocks of the next V issue (tile r + 2)
    TileBase id_k = tile_block(t_first + 3);  // blocks of the next K issue (tile r + 3)
    issue_k(id_v, kA);
    issue_v(t_first + 1, id1, vA, mA);
    TileBase id_n = tile_block(t_first + 4);  // blocks of the K issue after next (tile r + 4)
    // Pairs of steps per trip with one exit test, so that the loop header is reached only
    // from the prologue and from the end of a pair; the scheduling barriers keep the loads
    // ahead of the step and the stores after it.  The block ids (scalar loads) are read
    // after a step's stores: scalar and LDS results share one wait counter, so a scalar
    // load in flight during the step would hold up its first LDS wait, while the stores'
    // wait before the barrier is there anyway.
    int r = 0;
    for (; r + 1 < n_tiles; r += 2) {
      issue_k(id_k, kB);
      issue_v(t_first + r + 2, id_v, vB, mB);
      id_v = id_k;
      id_k = id_n;
      __builtin_amdgcn_sched_barrier(0);
      step(t_first + r, s, kbuf1, vbuf0);
      __builtin_amdgcn_sched_barrier(0);
      store_k(0, kA);
      store_v(1, vA, mA);
      id_n = tile_block(t_first + r + 5);
      __syncthreads();
      issue_k(id_k, kA);
      issue_v(t_first + r + 3, id_v, vA, mA);
      id_v = id_k;
      id_k = id_n;
      __builtin_amdgcn_sched_barrier(0);
      step(t_first + r + 1, s, kbuf0, vbuf1);
      __builtin_amdgcn_sched_barrier(0);
      store_k(1, kB);
      store_v(0, vB, mB);
      id_n = tile_block(t_first + r + 6);
      __syncthreads();
    }
    // An odd tile count: the last step (its next scores, of a tile past the part, go unused).
    if (r < n_tiles) step(t_first + r, s, kbuf1, vbuf0);

    // A block id outside the pool anywhere in the workgroup's keys makes every output NaN.
    bad_blk = __syncthreads_or(bad_blk);
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
    float M = -INFINITY;
    bool has_nan = false;
    for (int p = 0; p < n_parts; ++p) {
      has_nan |= lse[p] != lse[p];
      M = fmaxf(M, lse[p]);
    }
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float wsum = 0.0f;
    for (int p = 0; p < n_parts; ++p) {
      const float w = __builtin_amdgcn_exp2f(lse[p] - M);
      wsum += w;
      acc += w * *reinterpret_cast<const f32x4*>(a.part_o + (out_row * a.pmax + p) * kHead + d4);
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
