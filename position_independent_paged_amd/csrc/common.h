// Shared device code for the position-free paged attention kernels (gfx950).
//
// One call runs three kernels on the caller's stream:
//
//   plan_tiles  one work-group per (request r, q tile): the tile's query rows
//               (context index, span id, PDep bit per token) and the compacted
//               list of the key blocks at least one of its rows may see.
//   plan_items  one work-group: splits long key lists into pieces, assigns
//               partial-result slots to split tiles, and writes the work items
//               (tile, KV head, piece of the key list) sorted longest first.
//   attention   a persistent grid (about one work-group per CU) that takes
//               items from an atomic counter; a piece of a split tile writes
//               its fp32 partial result (O, m, l) to its slot.
//   merge       one work-group per split (tile, KV head): log-sum-exp merge
//               of the pieces, in piece order. A separate launch: a fence
//               inside the attention kernel would write back and invalidate
//               the L2 of the XCD, evicting the K/V tiles the other
//               work-groups there are reusing.
//
// The visibility rule follows "MiniPIC: Flexible Position-Independent Caching
// in <100LOC", §3.1.1 (SSep / PDep) and §3.3.1 (documents and the system
// prompt prefilled as separate requests), for a query at context index c and
// a key at context index j:
//     visible(c, j) = j <= c and (PDEP(c's block) or GLOBAL(j's block)
//                                 or span(j's block) == span(c's block))
// The span test compares runs, not bare ids: a span id names one contiguous
// run of blocks (the caller's contract), and a block with the row's span id
// that lies before the start of the row's own run is a different, invisible
// span. plan_tiles records each row's run start, sets MINIPIC_EW_SPAN in the
// error word when such an earlier block exists (the contract is broken), and
// the attention kernels evaluate the same run-based rule, so the result never
// depends on how rows are grouped into tiles.
// The key blocks a tile may see are then the GLOBAL blocks below `lo` plus
// blocks of [lo, hi], where hi is the block of the tile's last query and lo
// is 0 if a row is PDep, else the earliest run start of its rows. plan_tiles
// keeps the blocks of that range some row really sees.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/minipic.h"

namespace minipic {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kBlock = 16;        // tokens per cache block
constexpr int kMaxSplits = 64;    // key-list pieces per tile at most
constexpr int kCostBins = 1024;   // item sort buckets (cost in key blocks, clipped)
constexpr int kItemCostBlocks = 16;  // fixed cost of starting a work item, in key blocks
constexpr int kPlanThreads = 1024;// plan_tiles work-group size
constexpr int kPlanBlocksPerThread = 2;  // key blocks per plan_tiles thread and pass
constexpr int kTileCache = 4096;  // tiles whose list lengths plan_items keeps in LDS
constexpr int kItemThreads = 1024;// plan_items work-group size

// Work items are kept in kQueues queues, one per XCD of the GPU. The
// dispatcher places work-group b on XCD b % 8, so work-group b drains queue
// b % kQueues first; items that read the same K/V blocks share a queue, so
// the work-groups reading them share one L2. An empty queue is left for the
// next one (work stealing).
constexpr int kQueues = 8;
constexpr int kDecodeMaxSplits = 4096;   // key splits per (request, KV head) in decode at most

// Header of the workspace (first 256 bytes).
struct WsHeader {
  uint32_t err;                 // MINIPIC_EW_* bits of calls that take the workspace from the caller
  uint32_t num_items;           // written by plan_items
  uint32_t chunk;               // key blocks per piece chosen by plan_items
  uint32_t num_groups;          // split (tile, KV head) groups listed for the merge
  uint32_t next[kQueues];       // per-queue ticket counters (plan_items starts each past the
                                // work-groups' own first tickets)
  uint32_t qstart[kQueues];     // first item of each queue
  uint32_t qcount[kQueues];     // items in each queue
  uint64_t plan_key;            // configuration the plan was built for (written by plan_items;
                                // the attention and merge kernels run only on a matching plan;
                                // never 0)
  uint32_t pad[2];
  // Measurement: the attention kernel's work-group 0 stores the shader clock
  // counter and the 100 MHz real-time counter when it starts and when it has
  // drained the queues (the ratio of the differences is the shader clock).
  uint64_t clk_start, rt_start, clk_end, rt_end;
};
static_assert(sizeof(WsHeader) <= 256, "workspace header");
static_assert(offsetof(WsHeader, clk_start) == 128, "clock stamps at byte 128 of the workspace");
static_assert(offsetof(WsHeader, plan_key) % 8 == 0, "aligned plan key");

// One split (tile, KV head): its pieces occupy slots slot0 .. slot0+nsplit-1.
struct Group {
  int32_t tile;
  int32_t g;
  int32_t nsplit;
  int32_t slot0;
};

// One q tile (written by plan_tiles; nsplit / slot0 completed by plan_items).
struct TileDesc {
  int32_t r;       // request
  int32_t row0;    // first packed query row
  int32_t nq;      // query tokens in the tile (0: no tile)
  int32_t nlist;   // visible key blocks listed for the tile
  int32_t nsplit;  // pieces the list is cut into
  int32_t slot0;   // first partial-result slot (split tiles only)
  int32_t item0;   // first of the tile's items, numbered in tile order (plan_items)
  int32_t pad1;
};

// One query token of a tile.
struct TokDesc {
  int32_t c;       // context index, -1 for a row past the end of the tile
  int32_t span;    // span id of its block
  int32_t pdep;    // PDEP bit of its block
  int32_t lo;      // first block of the run of its span id that holds its block (0 for PDep rows)
};

// One visible key block of a tile.
struct BlkDesc {
  int32_t kb;      // logical block index in the request
  int32_t phys;    // physical cache block, -1 if the block table entry was invalid
  int32_t span;    // span id
  int32_t flags;   // MINIPIC_BLK_* bits
  int32_t pos0;    // if >= 0: the block's logical positions are pos0 .. pos0+15, all
                   // inside the cos/sin table (key offset k sits at pos0 + k); -1: look
                   // each key's position up in logical_pos
  int32_t full;    // 1: every query row of the tile sees every key of the block (the
                   // block lies below each row's own block and is visible to each row)
  int32_t nvalid;  // keys of the block inside the context (16 except in a ragged last block);
                   // keys past it hold no token: their values are never read into a result
  int32_t pad2;
};

// One unit of attention work: KV head g of tile `tile`, list entries [p0, p1),
// with the fields of the tile the attention kernel needs (copied here so an
// item is one load).
struct Item {
  int32_t tile;
  int32_t p0;
  int32_t p1;
  uint32_t gsn;    // g | split << 8 | nsplit << 20
  int32_t r;       // request
  int32_t row0;    // first packed query row of the tile
  int32_t nq;      // query tokens in the tile
  int32_t slot0;   // first partial-result slot of the tile (split tiles only)
};

__host__ __device__ inline uint32_t pack_gsn(int g, int s, int ns) {
  return (uint32_t)g | ((uint32_t)s << 8) | ((uint32_t)ns << 20);
}

// Parameters of the two planning kernels.
struct PlanParams {
  const int32_t* q_indptr;
  const int32_t* q_ctx_idx;
  const int32_t* ctx_len;
  const int32_t* block_table;
  const int32_t* span_id;
  const uint8_t* blk_flags;
  WsHeader* hdr;
  uint32_t* err;       // MINIPIC_EW_* bits (the workspace's first word, or the caller's word)
  TileDesc* tiles;
  TokDesc* toks;       // [num_tiles][bq]
  BlkDesc* blist;      // [num_tiles][max_blocks]
  Item* items;         // [max_items]
  Group* groups;       // [max_slots / 2]
  int64_t num_blocks;
  int32_t num_reqs;
  int32_t nqt;         // q tiles per request (host upper bound)
  int32_t num_tiles;   // num_reqs * nqt
  int32_t bq;          // query tokens per tile
  int32_t hkv;
  int32_t max_blocks;
  int32_t num_wg;      // persistent attention work-groups
  int32_t max_slots;   // partial-result slots available
  int32_t max_items;
  int32_t min_chunk;   // smallest piece (key blocks)
  const int32_t* logical_pos;
  int32_t max_pos;     // rows of the cos/sin table (1 when no table is used)
  uint64_t plan_key;   // configuration key stored with the plan
};

// Parameters of the attention kernels.
struct AttnParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* out;
  const float* cos_sin;
  const int32_t* logical_pos;
  WsHeader* hdr;
  uint32_t* err;       // MINIPIC_EW_* bits (the workspace's first word, or the caller's word)
  const TileDesc* tiles;
  const TokDesc* toks;
  const BlkDesc* blist;
  const Item* items;
  const Group* groups;
  float2* part_ml;     // [slots][rows] (m in log2 units, l)
  float* part_o;       // [slots][rows][D]; the bf16 kernel orders each 32-row block by lane (see its epilogue)
  int32_t hq;
  int32_t hkv;
  int32_t max_blocks;
  int32_t max_pos;
  int32_t max_groups;  // capacity of the group list
  float scale_log2;    // softmax_scale * log2(e)
  uint32_t flags;
  uint64_t plan_key;   // configuration key the plan in the workspace must carry
  int32_t num_wg;      // persistent attention work-groups
};

// Tickets a queue's counter starts past: work-group b takes ticket b / kQueues
// of queue b % kQueues as its first item without an atomic.
__device__ __forceinline__ uint32_t first_tickets(int num_wg, int q) {
  return num_wg > q ? (uint32_t)((num_wg - q + kQueues - 1) / kQueues) : 0u;
}

// Parameters of the decode kernels (one query row per request).
struct DecodeParams {
  const void* q;              // [R][Hq][D] bf16, row r = request r's query
  const void* k_cache;        // [num_blocks][Hkv][16][D]
  const void* v_cache;        // [num_blocks][Hkv][D][16]
  void* out;                  // [R][Hq][D]
  const float* cos_sin;       // [max_pos][D]
  const int32_t* q_ctx_idx;   // [R] context index of the query
  const int32_t* ctx_len;     // [R]
  const int32_t* block_table; // [R][MB]
  const int32_t* logical_pos; // [R][MB*16]
  const int32_t* span_id;     // [R][MB]
  const uint8_t* blk_flags;   // [R][MB]
  uint32_t* err;              // error word (MINIPIC_EW_* bits)
  float2* part_ml;            // [R*Hkv*nsplit*G] (m, l)
  float* part_o;              // [R*Hkv*nsplit*G][D]
  int64_t num_blocks;
  int32_t num_reqs, hq, hkv, max_blocks, max_pos, nsplit, split_blocks;
  float scale_log2;
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 p = {(__bf16)a, (__bf16)b};  // round-to-nearest-even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint32_t, p);
}

// Exclusive prefix count of integer contributions over the work-group.
// Every thread must call it. `tmp` holds NT/64 ints of LDS.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    int c = tmp[i];
    off += (i < w) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

template <int NT>
__device__ __forceinline__ int block_excl_scan_pred(bool pred, int* tmp, int* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint64_t b = __ballot(pred);
  const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) tmp[w] = __popcll(b);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    int c = tmp[i];
    off += (i < w) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + in_wave;
}

// Block-level visibility of key block (kb, span, flags) for a query row in
// block bq with (span_row, pdep_row) whose span run starts at block lo_row;
// the causal test inside the diagonal block is element-wise and done by the
// caller.
__device__ __forceinline__ bool block_visible(int kb, int span, int flags, int bq, int span_row, bool pdep_row,
                                              int lo_row) {
  return kb <= bq && (pdep_row || (flags & MINIPIC_BLK_GLOBAL) || (span == span_row && kb >= lo_row));
}

// Work items are claimed with one atomic add on the counter of the queue the
// work-group is draining, issued when the work-group starts an item; the
// ticket is checked against the queue's size later in that item, so the
// claim's latency hides behind the item's work. A ticket past the end means
// the queue is drained: the work-group moves on to the other queues (queues
// never refill), and returns -1 when every queue is drained. The counters
// only grow, so a queue whose counter already reads at or past its size is
// empty for good: the counters of all queues are read in one round trip and
// only a queue that may still hold items is claimed from. `qs`, `qc` hold the
// queues' first items and sizes (copied to LDS). Thread 0 only.
__device__ __forceinline__ int resolve_ticket(WsHeader* hdr, const uint32_t* qs, const uint32_t* qc, int& q,
                                              uint32_t ticket) {
  if (ticket < qc[q]) return (int)(qs[q] + ticket);
  uint32_t seen[kQueues];
#pragma unroll
  for (int k = 0; k < kQueues; ++k) seen[k] = __hip_atomic_load(&hdr->next[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int k = 1; k < kQueues; ++k) {
    const int q2 = (q + k) % kQueues;
    if (seen[q2] >= qc[q2]) continue;
    const uint32_t t = atomicAdd(&hdr->next[q2], 1u);
    if (t < qc[q2]) {
      q = q2;
      return (int)(qs[q2] + t);
    }
  }
  return -1;
}

}  // namespace minipic
