// Shared device code for the position-free paged attention kernels (gfx950).
//
// Work decomposition: one work-group owns (request r, q tile of BQ query
// tokens, KV head g, key split s) and all Hq/Hkv query heads of that KV head.
// Before its flash loop it derives the set of key blocks any of its rows may
// see from the per-block descriptors, following the visibility rule of
// "MiniPIC: Flexible Position-Independent Caching in <100LOC", §3.1.1 (SSep /
// PDep) and §3.3.1 (spans prefilled as separate requests):
//     visible(c, j) = j <= c and (PDEP(c's block) or GLOBAL(j's block)
//                                 or span(j's block) == span(c's block))
// Under the contract that one span id names one contiguous run of blocks, the
// blocks a tile may see are the GLOBAL blocks below `lo` plus the range
// [lo, hi], where hi is the block of the tile's last query and lo is 0 if a
// row is PDep, else the start of the run holding the tile's first query block.
// That "visit sequence" is split across key splits, and each split compacts
// the blocks some row really sees into an LDS list (block id, physical block,
// span id, flags) that the flash loop walks four blocks (64 keys) at a time.
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

constexpr int kBlock = 16;          // tokens per cache block
constexpr int kGlobalMax = 256;     // GLOBAL blocks listed per tile before falling back to a full scan
constexpr int kListMax = 256;       // blocks compacted per pass of the flash loop

// Kernel parameters shared by the attention kernels.
struct AttnParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* out;
  const float* cos_sin;
  const int32_t* q_indptr;
  const int32_t* q_ctx_idx;
  const int32_t* ctx_len;
  const int32_t* block_table;
  const int32_t* logical_pos;
  const int32_t* span_id;
  const uint8_t* blk_flags;
  uint32_t* err;            // workspace error word
  int32_t* tile_nsplit;     // [num_reqs][num_q_tiles][Hkv]
  float2* part_ml;          // [splits][total_q][Hq] (m in log2 units, l)
  float* part_o;            // [splits][total_q][Hq][D]
  int64_t num_blocks;
  int64_t total_q;
  int32_t num_reqs;
  int32_t hq;
  int32_t hkv;
  int32_t max_blocks;       // max_blocks_per_req
  int32_t max_pos;
  int32_t num_q_tiles;
  int32_t num_splits;
  int32_t split_blocks;
  float scale_log2;         // softmax_scale * log2(e)
  uint32_t flags;
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

// LDS state of the tile planner.
template <int BQ>
struct PlanSmem {
  int qctx[BQ];          // context index per tile token (-1 past the end)
  int qent[BQ];          // distinct-query-block entry of each token
  int e_bq[BQ];          // entry: query block
  int e_span[BQ];        // entry: its span id
  int e_pdep[BQ];        // entry: PDEP bit
  int g_list[kGlobalMax];
  int l_kb[kListMax];    // compacted visible key blocks of the current pass
  int l_phys[kListMax];
  int l_span[kListMax];
  int l_flags[kListMax];
  int tmp[16];
  int n_e, lo, hi, n_g, any_pdep, pdep_hi, min_bq, n_l;
};

struct TileInfo {
  int r, qt, g, s;
  int row0;      // first packed query row of the tile
  int nq;        // query tokens in the tile
  int L;         // context length (clamped)
  int nsplit;    // splits holding part of this tile's keys
  int p0, p1;    // this split's range of the visit sequence
};

// Decode the 1-D grid: heaviest q tiles (largest context) first, splits of a
// tile adjacent.
__device__ __forceinline__ void decode_block(const AttnParams& P, int64_t bid, TileInfo& t) {
  const int S = P.num_splits;
  t.s = (int)(bid % S);
  int64_t rest = bid / S;
  t.g = (int)(rest % P.hkv);
  rest /= P.hkv;
  const int qt_rev = (int)(rest % P.num_q_tiles);
  t.r = (int)(rest / P.num_q_tiles);
  t.qt = P.num_q_tiles - 1 - qt_rev;
}

// Phase 1 of the planner: query rows, distinct query blocks, key range and the
// GLOBAL list. Returns false (uniformly) when the tile has no rows or this
// split has no keys. Work-group-wide; contains barriers.
template <int NT, int BQ>
__device__ bool plan_tile(const AttnParams& P, TileInfo& t, PlanSmem<BQ>& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int qb = P.q_indptr[t.r];
  const int qe = P.q_indptr[t.r + 1];
  t.row0 = qb + t.qt * BQ;
  if (t.row0 >= qe) return false;
  t.nq = min(BQ, qe - t.row0);
  int L = P.ctx_len[t.r];
  const int Lmax = P.max_blocks * kBlock;
  if (L > Lmax || L < 0) {
    if (tid == 0) atomicOr(P.err, (uint32_t)MINIPIC_EW_CTX);
    L = L < 0 ? 0 : Lmax;
  }
  t.L = L;
  const int* span = P.span_id + (int64_t)t.r * P.max_blocks;
  const uint8_t* flg = P.blk_flags + (int64_t)t.r * P.max_blocks;

  // --- query rows
  static_assert(BQ <= NT, "one token per thread");
  bool valid = tid < t.nq;
  int c = -1;
  if (valid) {
    c = P.q_ctx_idx[t.row0 + tid];
    if (c < 0 || c >= L) {
      atomicOr(P.err, (uint32_t)MINIPIC_EW_QCTX);
      c = c < 0 ? 0 : L - 1;
      if (c < 0) valid = false;  // empty context: nothing to attend
    }
  }
  if (tid < BQ) sm.qctx[tid] = valid ? c : -1;
  __syncthreads();
  const int bq = valid ? (c >> 4) : -1;
  const bool first = valid && (tid == 0 || (sm.qctx[tid - 1] >> 4) != bq || sm.qctx[tid - 1] < 0);
  int n_e;
  const int idx = block_excl_scan_pred<NT>(first, sm.tmp, &n_e);
  if (first) {
    sm.e_bq[idx] = bq;
    sm.e_span[idx] = span[bq];
    sm.e_pdep[idx] = flg[bq] & MINIPIC_BLK_PDEP;
  }
  if (tid < BQ) sm.qent[tid] = valid ? idx + (first ? 1 : 0) - 1 : 0;
  __syncthreads();

  // --- summary over entries (wave 0)
  if (tid < 64) {
    int hi = -1, mn = 0x7fffffff, anyp = 0, phi = -1;
    for (int e = lane; e < n_e; e += 64) {
      const int b = sm.e_bq[e];
      hi = max(hi, b);
      mn = min(mn, b);
      if (sm.e_pdep[e]) { anyp = 1; phi = max(phi, b); }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      hi = max(hi, __shfl_xor(hi, o, 64));
      mn = min(mn, __shfl_xor(mn, o, 64));
      anyp |= __shfl_xor(anyp, o, 64);
      phi = max(phi, __shfl_xor(phi, o, 64));
    }
    // run start of the smallest query block (seg start is monotone in the block)
    int lo = 0;
    if (!anyp && mn != 0x7fffffff) {
      const int sp = span[mn];
      int base = mn;
      while (true) {
        const int b = base - 1 - lane;
        const bool stop = (b < 0) || (span[b] != sp);
        const uint64_t m = __ballot(stop);
        if (m) {
          lo = base - (__ffsll((unsigned long long)m) - 1);
          break;
        }
        base -= 64;
      }
    }
    if (lane == 0) {
      sm.n_e = n_e;
      sm.hi = hi;
      sm.min_bq = mn;
      sm.any_pdep = anyp;
      sm.pdep_hi = phi;
      sm.lo = lo;
    }
  }
  __syncthreads();
  const int lo = sm.lo;
  const int hi = sm.hi;

  // --- GLOBAL blocks below lo (16 descriptor bytes per thread per round)
  int n_g = 0;
  for (int base = 0; base < lo; base += 16 * NT) {
    const int b0 = base + tid * 16;
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int b = b0 + i;
      if (b < lo && (flg[b] & MINIPIC_BLK_GLOBAL)) bits |= 1u << i;
    }
    int tot;
    int off = block_excl_scan<NT>(__popc(bits), sm.tmp, &tot);
    while (bits) {
      const int i = __ffs(bits) - 1;
      bits &= bits - 1;
      const int slot = n_g + off++;
      if (slot < kGlobalMax) sm.g_list[slot] = b0 + i;
    }
    n_g += tot;
  }
  int lo_eff = lo;
  if (n_g > kGlobalMax) {  // too many to list: visit every block below hi instead
    n_g = 0;
    lo_eff = 0;
  }
  __syncthreads();
  if (tid == 0) {
    sm.n_g = n_g;
    sm.lo = lo_eff;
  }

  // --- split of the visit sequence
  const int V = n_g + (hi - lo_eff + 1);
  const int chunk = P.split_blocks;
  int ns = (V + chunk - 1) / chunk;
  if (ns > P.num_splits) ns = P.num_splits;
  if (ns < 1) ns = 1;
  t.nsplit = ns;
  if (t.s == 0 && tid == 0 && P.num_splits > 1)
    P.tile_nsplit[((int64_t)t.r * P.num_q_tiles + t.qt) * P.hkv + t.g] = ns;
  __syncthreads();
  if (t.s >= ns) return false;
  t.p0 = t.s * chunk;
  t.p1 = (t.s == ns - 1) ? V : min(V, (t.s + 1) * chunk);
  return true;
}

// Phase 2: compact the blocks of visit positions [c0, c1) that some row sees.
// Returns the list length (uniform). Work-group-wide; contains barriers.
template <int NT, int BQ>
__device__ int build_list(const AttnParams& P, const TileInfo& t, PlanSmem<BQ>& sm, int c0, int c1) {
  const int tid = threadIdx.x;
  const int* span = P.span_id + (int64_t)t.r * P.max_blocks;
  const uint8_t* flg = P.blk_flags + (int64_t)t.r * P.max_blocks;
  const int* btab = P.block_table + (int64_t)t.r * P.max_blocks;
  const int n_g = sm.n_g, lo = sm.lo, n_e = sm.n_e, anyp = sm.any_pdep, phi = sm.pdep_hi;
  int n_l = 0;
  for (int base = c0; base < c1; base += NT) {
    const int p = base + tid;
    bool vis = false;
    int kb = 0, sp = 0, fl = 0, ph = 0;
    if (p < c1) {
      kb = p < n_g ? sm.g_list[p] : lo + (p - n_g);
      sp = span[kb];
      fl = flg[kb];
      if (anyp && kb <= phi) {
        vis = true;
      } else {
        const bool glob = (fl & MINIPIC_BLK_GLOBAL) != 0;
        for (int e = 0; e < n_e; ++e) {
          const int eb = sm.e_bq[e];
          if (kb <= eb && (sm.e_pdep[e] || glob || sm.e_span[e] == sp)) {
            vis = true;
            break;
          }
        }
      }
      if (vis) {
        ph = btab[kb];
        if (ph < 0 || (int64_t)ph >= P.num_blocks) {
          atomicOr(P.err, (uint32_t)MINIPIC_EW_BLOCK);
          ph = -1;  // read as zeros
        }
      }
    }
    int tot;
    const int idx = block_excl_scan_pred<NT>(vis, sm.tmp, &tot);
    if (vis && n_l + idx < kListMax) {
      sm.l_kb[n_l + idx] = kb;
      sm.l_phys[n_l + idx] = ph;
      sm.l_span[n_l + idx] = sp;
      sm.l_flags[n_l + idx] = fl;
    }
    n_l += tot;
  }
  __syncthreads();
  return n_l;
}

}  // namespace minipic
