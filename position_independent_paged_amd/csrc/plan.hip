// Planning kernels of the position-free paged attention (gfx950).
//
// plan_tiles: one work-group per (request, q tile). It records every query
// token of the tile (context index, span id, PDEP bit) and compacts the key
// blocks at least one of its rows may see, following the block visibility of
// "MiniPIC: Flexible Position-Independent Caching in <100LOC", §3.1.1 and
// §3.3.1 (rule restated in common.h), into a per-tile list.
//
// plan_items: one work-group. It picks the piece length from the total work
// and the number of persistent attention work-groups, cuts long tile lists
// into pieces, assigns partial-result slots, and writes the work items
// (tile, KV head, piece) into per-XCD queues, longest first, and the list of
// split (tile, KV head) groups for the merge. It also starts the scheduler's
// queue counters (so the attention kernel needs no host-side memset) and
// records the configuration key the attention and merge kernels check.
#include <climits>

#include "common.h"

namespace minipic {

// Descriptor of one listed key block. `lpos` is the request's row of logical
// positions, `L` its context length. Only the block's keys below L hold
// tokens (nvalid of them): pos0 is set when their positions run pos0, pos0+1,
// ... and all of them lie inside the cos/sin table; positions past L are
// never read for a result.
__device__ __forceinline__ BlkDesc blk_from(const PlanParams& P, int ph, const int4 (&pp)[kBlock / 4], int L, int kb,
                                            int span, int flags, int full) {
  if (ph < 0 || (int64_t)ph >= P.num_blocks) {
    atomicOr(P.err, (uint32_t)MINIPIC_EW_BLOCK);
    ph = -1;  // read as zeros by the attention kernels
  }
  int p[kBlock];
#pragma unroll
  for (int i = 0; i < kBlock / 4; ++i) {
    p[4 * i] = pp[i].x;
    p[4 * i + 1] = pp[i].y;
    p[4 * i + 2] = pp[i].z;
    p[4 * i + 3] = pp[i].w;
  }
  const int nvalid = max(0, min(kBlock, L - kb * kBlock));
  bool cons = p[0] >= 0 && p[0] <= P.max_pos - nvalid;
#pragma unroll
  for (int k = 1; k < kBlock; ++k) cons = cons && (k >= nvalid || p[k] == p[0] + k);
  return BlkDesc{kb, ph, span, flags, cons ? p[0] : -1, full, nvalid, 0};
}

__device__ __forceinline__ BlkDesc make_blk(const PlanParams& P, int ph, const int32_t* lpos, int L, int kb, int span,
                                            int flags, int full) {
  const int4* src = (const int4*)(lpos + (int64_t)kb * kBlock);
  int4 pp[kBlock / 4];
#pragma unroll
  for (int i = 0; i < kBlock / 4; ++i) pp[i] = src[i];
  return blk_from(P, ph, pp, L, kb, span, flags, full);
}

template <int BQ, int NT>
__global__ void __launch_bounds__(NT) plan_tiles_kernel(PlanParams P) {
  static_assert(BQ <= NT, "one query token per thread");
  constexpr int BPT = kPlanBlocksPerThread;
  constexpr int PASS = NT * BPT;   // key blocks per pass, each thread owning BPT consecutive ones
  __shared__ int qblk[BQ];
  __shared__ int e_bq[BQ], e_span[BQ], e_pdep[BQ], e_lo[BQ];
  __shared__ int tmp[NT / 64];
  __shared__ int s_hi, s_lo, s_anyp, s_phi;
  __shared__ int s_span[PASS];     // span ids and flags of the first pass's blocks
  __shared__ uint8_t s_flg[PASS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int t = blockIdx.x;
  const int r = t / P.nqt;
  const int qt = t % P.nqt;
  TileDesc* td = P.tiles + t;
  const int32_t* span = P.span_id + (int64_t)r * P.max_blocks;
  const uint8_t* flg = P.blk_flags + (int64_t)r * P.max_blocks;
  const int32_t* btab = P.block_table + (int64_t)r * P.max_blocks;
  const int32_t* lpos = P.logical_pos + (int64_t)r * P.max_blocks * kBlock;

  // The span ids, flags and physical blocks of the first pass's blocks depend
  // only on the request: they are loaded before anything else, together with
  // the request's offsets, so the tile's dependent round trips are the
  // offsets, the query contexts and the positions of its visible blocks.
  const int nb0 = P.max_blocks < PASS ? P.max_blocks : PASS;
  int f0[BPT], s0[BPT], ph0[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int kb = tid * BPT + j;
    const bool in = kb < nb0;
    f0[j] = in ? flg[kb] : 0;
    s0[j] = in ? span[kb] : 0;
    ph0[j] = in ? btab[kb] : -1;
  }
  const int qb = P.q_indptr[r];
  const int qe = P.q_indptr[r + 1];
  const int row0 = qb + qt * BQ;
  if (row0 >= qe) {
    if (tid == 0) *td = TileDesc{r, row0, 0, 0, 0, -1, 0, 0};
    return;
  }
  const int nq = min(BQ, qe - row0);
  int L = P.ctx_len[r];
  const int Lmax = P.max_blocks * kBlock;
  if (L > Lmax || L < 0) {
    if (tid == 0) atomicOr(P.err, (uint32_t)MINIPIC_EW_CTX);
    L = L < 0 ? 0 : Lmax;
  }
  const int cq = tid < nq ? P.q_ctx_idx[row0 + tid] : 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int kb = tid * BPT + j;
    if (kb < nb0) {
      s_span[kb] = s0[j];
      s_flg[kb] = (uint8_t)f0[j];
    }
  }
  __syncthreads();
  auto span_at = [&](int b) { return b < nb0 ? s_span[b] : span[b]; };
  auto flg_at = [&](int b) { return b < nb0 ? (int)s_flg[b] : (int)flg[b]; };

  // ---- query tokens
  bool valid = tid < nq;
  int c = -1;
  if (valid) {
    c = cq;
    if (c < 0 || c >= L) {
      atomicOr(P.err, (uint32_t)MINIPIC_EW_QCTX);
      c = c < 0 ? 0 : L - 1;
      if (c < 0) valid = false;  // empty context: the row has nothing to attend
    }
  }
  const int bq = valid ? (c >> 4) : -1;
  int sp = 0, pd = 0;
  if (valid) {
    sp = span_at(bq);
    pd = (flg_at(bq) & MINIPIC_BLK_PDEP) ? 1 : 0;
  }
  if (tid < BQ) qblk[tid] = bq;
  __syncthreads();

  // ---- distinct query blocks ("entries")
  const bool first = valid && (tid == 0 || qblk[tid - 1] != bq);
  int n_e;
  const int idx = block_excl_scan_pred<NT>(first, tmp, &n_e);
  if (first) {
    e_bq[idx] = bq;
    e_span[idx] = sp;
    e_pdep[idx] = pd;
  }
  __syncthreads();

  // ---- run start of every non-PDep entry (wave 0): the first block of the
  // run of equal span ids that holds the entry's block. An entry in the block
  // right after the previous entry's, with the same span id, shares that
  // entry's run; every other entry searches backwards, 64 blocks per round.
  if (tid < 64) {
    int carry = 0;   // run start of the last searched entry of earlier chunks
    for (int e0 = 0; e0 < n_e; e0 += 64) {
      const int e = e0 + lane;
      bool need = false;
      if (e < n_e && !e_pdep[e])
        need = e == 0 || e_pdep[e - 1] || e_span[e] != e_span[e - 1] || e_bq[e] != e_bq[e - 1] + 1;
      const uint64_t nm = __ballot(need);
      uint64_t m = nm;
      int my_lo = 0;
      while (m) {
        const int k = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const int sm = e_span[e0 + k];
        int base = e_bq[e0 + k];
        int start;
        while (true) {
          const int b2 = base - 1 - lane;
          const bool stop = (b2 < 0) || (span_at(b2) != sm);
          const uint64_t sb = __ballot(stop);
          if (sb) {
            start = base - (__ffsll((unsigned long long)sb) - 1);
            break;
          }
          base -= 64;
        }
        if (lane == k) my_lo = start;
      }
      // an entry that shares a run takes the start of the nearest searched entry before it
      const uint64_t upto = nm & (lane == 63 ? ~0ull : ((2ull << lane) - 1));
      const int src = upto ? 63 - __clzll((long long)upto) : -1;
      const int inherited = __shfl(my_lo, src < 0 ? 0 : src, 64);
      const int lo_e = need ? my_lo : (src >= 0 ? inherited : carry);
      if (e < n_e) e_lo[e] = e_pdep[e] ? 0 : lo_e;
      if (nm) carry = __shfl(my_lo, 63 - __clzll((long long)nm), 64);
    }
  }
  __syncthreads();
  if (tid < BQ) P.toks[(int64_t)t * BQ + tid] = TokDesc{valid ? c : -1, sp, pd, valid ? e_lo[idx - (first ? 0 : 1)] : 0};

  // ---- key range (wave 0): lo = 0 if some row is PDep, else the earliest run start
  if (tid < 64) {
    int hi = -1, lo = INT_MAX, anyp = 0, phi = -1;
    for (int e = lane; e < n_e; e += 64) {
      const int b2 = e_bq[e];
      hi = max(hi, b2);
      lo = min(lo, e_lo[e]);
      if (e_pdep[e]) {
        anyp = 1;
        phi = max(phi, b2);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      hi = max(hi, __shfl_xor(hi, o, 64));
      lo = min(lo, __shfl_xor(lo, o, 64));
      anyp |= __shfl_xor(anyp, o, 64);
      phi = max(phi, __shfl_xor(phi, o, 64));
    }
    if (lane == 0) {
      s_hi = hi;
      s_lo = (anyp || lo == INT_MAX) ? 0 : lo;
      s_anyp = anyp;
      s_phi = phi;
    }
  }
  __syncthreads();
  const int lo = s_lo, hi = s_hi;

  // ---- compacted list, in block order: the GLOBAL blocks below lo (visible
  // to every row, below every query block) and the blocks of [lo, hi] some row
  // sees. A pass covers PASS blocks, each thread owning BPT consecutive ones,
  // so all loads of a pass are in flight together (the first pass's were
  // loaded at the start) and one scan places the visible blocks. A block that
  // carries a row's span id before the row's own run breaks the span-id
  // contract: it is not visible to that row, and the error word says so.
  BlkDesc* out = P.blist + (int64_t)t * P.max_blocks;
  int n = 0;
  bool broken = false;
  for (int base = 0; base <= hi; base += PASS) {
    int f[BPT], s[BPT];
    bool vis[BPT], full[BPT];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int kb = base + tid * BPT + j;
      f[j] = 0;
      s[j] = 0;
      vis[j] = false;
      full[j] = true;
      if (kb <= hi) {
        f[j] = base == 0 ? f0[j] : flg[kb];
        s[j] = base == 0 ? s0[j] : span[kb];
        const bool glob = (f[j] & MINIPIC_BLK_GLOBAL) != 0;
        // visible to some row (vis) / to every row, strictly below its own block (full)
        for (int e = 0; e < n_e; ++e) {
          const bool same = e_span[e] == s[j];
          const bool in_run = kb >= e_lo[e];
          const bool see = kb <= e_bq[e] && (e_pdep[e] || glob || (same && in_run));
          broken = broken || (same && !in_run && !glob);
          vis[j] = vis[j] || see;
          full[j] = full[j] && see && kb < e_bq[e];
        }
        vis[j] = vis[j] && (kb >= lo || glob);
      }
      cnt += vis[j] ? 1 : 0;
    }
    int tot;
    int off = block_excl_scan<NT>(cnt, tmp, &tot);
#pragma unroll
    for (int j = 0; j < BPT; ++j)
      if (vis[j]) {
        const int kb = base + tid * BPT + j;
        out[n + off++] = make_blk(P, base == 0 ? ph0[j] : btab[kb], lpos, L, kb, s[j], f[j], full[j] ? 1 : 0);
      }
    n += tot;
  }
  if (broken) atomicOr(P.err, (uint32_t)MINIPIC_EW_SPAN);
  if (tid == 0) *td = TileDesc{r, row0, nq, n, 0, -1, 0, 0};
}

// ---------------------------------------------------------------------------

template <int NT>
__device__ long long block_sum_ll(long long v, unsigned long long* red) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) red[w] = (unsigned long long)v;
  __syncthreads();
  long long s = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += (long long)red[i];
  __syncthreads();
  return s;
}

__device__ __forceinline__ int num_pieces(int n, int chunk) {
  if (n <= 0) return 0;
  const int ns = (n + chunk - 1) / chunk;
  return ns < kMaxSplits ? ns : kMaxSplits;
}

__device__ __forceinline__ int piece_start(int n, int ns, int s) { return (int)(((int64_t)s * n) / ns); }

// Queue of an item: items reading the same K/V blocks (same KV head, same
// first key block) land in the same queue. With a multiple of kQueues KV
// heads, queue = head; otherwise a hash of (request, head, first block).
__device__ __forceinline__ int item_queue(const PlanParams& P, int t, int g, int p0) {
  if (P.hkv % kQueues == 0) return g % kQueues;
  const int kb = P.blist[(int64_t)t * P.max_blocks + p0].kb;
  uint32_t h = (uint32_t)P.tiles[t].r * 0x9E3779B1u ^ (uint32_t)g * 0x85EBCA77u ^ (uint32_t)kb * 0xC2B2AE3Du;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  return (int)(h % kQueues);
}

// Counter of (queue, cost): queue-major, longest pieces first inside a queue.
__device__ __forceinline__ int bin_index(int q, int cost) {
  return q * kCostBins + (kCostBins - 1 - min(cost, kCostBins - 1));
}

__global__ void __launch_bounds__(kItemThreads) plan_items_kernel(PlanParams P) {
  constexpr int NT = kItemThreads;
  static_assert((kQueues * kCostBins) % NT == 0, "whole counters per thread");
  __shared__ unsigned long long red[NT / 64];
  __shared__ int tmp[NT / 64];
  __shared__ int bins[kQueues * kCostBins];
  // fields of the first kTileCache tiles, read or computed once: list length,
  // first item, request, first query row, first partial slot, query tokens |
  // pieces << 16
  __shared__ int s_nl[kTileCache];
  __shared__ int s_ioff[kTileCache];
  __shared__ int s_r[kTileCache];
  __shared__ int s_row0[kTileCache];
  __shared__ int s_slot0[kTileCache];
  __shared__ int s_nqns[kTileCache];
  const int tid = threadIdx.x;
  const int T = P.num_tiles;
  const int H = P.hkv;
  // list lengths of the tiles, read once (cached in LDS for up to kTileCache tiles)
  for (int t = tid; t < T && t < kTileCache; t += NT) {
    const TileDesc d = P.tiles[t];
    s_nl[t] = d.nlist;
    s_r[t] = d.r;
    s_row0[t] = d.row0;
    s_nqns[t] = d.nq;
  }
  __syncthreads();
  auto nlist = [&](int t) { return t < kTileCache ? s_nl[t] : P.tiles[t].nlist; };

  // ---- piece length: about one piece of work per persistent work-group,
  // never shorter than min_chunk, and few enough split tiles to fit the
  // partial-result slots. The work of a tile counts its key blocks plus the
  // fixed cost of starting an item (staging its list and query rows, filling
  // the load pipeline, storing its result), so pieces of long lists come out
  // longer where many short tiles share the grid.
  long long work = 0;
  for (int t = tid; t < T; t += NT) work += nlist(t) > 0 ? nlist(t) + kItemCostBlocks : 0;
  work = block_sum_ll<NT>(work, red) * H;
  const long long per = P.num_wg;
  long long cl = (work + per - 1) / per;
  int chunk = (int)(cl < (long long)P.min_chunk ? P.min_chunk : (cl > (1LL << 30) ? (1LL << 30) : cl));
  for (int iter = 0; iter < 40; ++iter) {
    long long slots = 0;
    for (int t = tid; t < T; t += NT) {
      const int ns = num_pieces(nlist(t), chunk);
      if (ns > 1) slots += (long long)ns * H;
    }
    slots = block_sum_ll<NT>(slots, red);
    if (slots <= P.max_slots || chunk >= (1 << 30)) break;
    chunk *= 2;
  }

  // ---- pieces, partial-result slots and first item (in tile order) per tile
  int slot_base = 0, item_base = 0;
  for (int t0 = 0; t0 < T; t0 += NT) {
    const int t = t0 + tid;
    const int ns = t < T ? num_pieces(nlist(t), chunk) : 0;
    int tot, itot;
    const int off = block_excl_scan<NT>(ns > 1 ? ns * H : 0, tmp, &tot);
    const int ioff = block_excl_scan<NT>(ns * H, tmp, &itot);
    if (t < T) {
      P.tiles[t].nsplit = ns;
      P.tiles[t].slot0 = ns > 1 ? slot_base + off : -1;
      P.tiles[t].item0 = item_base + ioff;
      if (t < kTileCache) {
        s_ioff[t] = item_base + ioff;
        s_slot0[t] = ns > 1 ? slot_base + off : -1;
        s_nqns[t] |= ns << 16;
      }
    }
    slot_base += tot;
    item_base += itot;
  }
  const int n_items = item_base;
  __syncthreads();
  auto item0 = [&](int t) { return t < kTileCache ? s_ioff[t] : P.tiles[t].item0; };
  // Items in tile order are numbered 0 .. n_items-1, (tile, piece, head) with
  // the head fastest; item i belongs to the last tile whose first item is <= i.
  auto item_tile = [&](int i) {
    int lo = 0, hi = T - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (item0(mid) <= i) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };

  // ---- bucket the items by (queue, length), longest first within a queue
  for (int f = tid; f < kQueues * kCostBins; f += NT) bins[f] = 0;
  __syncthreads();
  // Pieces are numbered in tile order (a tile's first piece is item0 / H).
  // Each thread takes a contiguous run of pieces: the tile of the first is
  // found by binary search, the following ones by walking forward; a piece's
  // bounds are computed once for its H items (one per KV head).
  const int n_pieces = n_items / H;
  const int per_thread = (n_pieces + NT - 1) / NT;
  const int q_begin = min(n_pieces, tid * per_thread);
  const int q_end = min(n_pieces, q_begin + per_thread);
  auto for_my_pieces = [&](auto&& fn) {
    if (q_begin >= q_end) return;
    int t = item_tile(q_begin * H);
    int first = item0(t) / H, n = nlist(t), ns = num_pieces(n, chunk);
    for (int q = q_begin; q < q_end; ++q) {
      while (q >= first + ns) {
        first += ns;
        ++t;
        n = nlist(t);
        ns = num_pieces(n, chunk);
      }
      const int s = q - first;
      const int p0 = ns == 1 ? 0 : piece_start(n, ns, s);
      const int p1 = ns == 1 ? n : piece_start(n, ns, s + 1);
      fn(t, s, ns, p0, p1);
    }
  };
  for_my_pieces([&](int t, int s, int ns, int p0, int p1) {
    const int cost_bin = bin_index(0, p1 - p0);
    for (int g = 0; g < H; ++g) atomicAdd(&bins[item_queue(P, t, g, p0) * kCostBins + cost_bin], 1);
  });
  __syncthreads();
  // exclusive scan of the kQueues * kCostBins counters, kFlat per thread
  constexpr int kFlat = kQueues * kCostBins / NT;
  int loc[kFlat];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kFlat; ++k) {
    loc[k] = bins[tid * kFlat + k];
    sum += loc[k];
  }
  int total;
  int run = block_excl_scan<NT>(sum, tmp, &total);
#pragma unroll
  for (int k = 0; k < kFlat; ++k) {
    const int f = tid * kFlat + k;
    bins[f] = run;
    if (f % kCostBins == 0) P.hdr->qstart[f / kCostBins] = (uint32_t)run;
    run += loc[k];
  }
  __syncthreads();
  if (tid < kQueues) {
    const uint32_t end = tid + 1 < kQueues ? (uint32_t)bins[(tid + 1) * kCostBins] : (uint32_t)total;
    P.hdr->qcount[tid] = end - (uint32_t)bins[tid * kCostBins];
    // tickets 0 .. (work-groups of the queue) - 1 are the work-groups' first
    // items, taken without an atomic (work-group b: ticket b / 8 of queue b % 8)
    P.hdr->next[tid] = first_tickets(P.num_wg, tid);
  }
  __syncthreads();
  int t_td = -1;
  TileDesc td{};
  for_my_pieces([&](int t, int s, int ns, int p0, int p1) {
    if (t != t_td) {
      if (t < kTileCache) {
        td.r = s_r[t];
        td.row0 = s_row0[t];
        td.nq = s_nqns[t] & 0xffff;
        td.slot0 = s_slot0[t];
      } else {
        td = P.tiles[t];
      }
      t_td = t;
    }
    const int cost_bin = bin_index(0, p1 - p0);
    for (int g = 0; g < H; ++g) {
      const int pos = atomicAdd(&bins[item_queue(P, t, g, p0) * kCostBins + cost_bin], 1);
      P.items[pos] = Item{t, p0, p1, pack_gsn(g, s, ns), td.r, td.row0, td.nq, td.slot0};
    }
  });

  // ---- split (tile, head) groups for the merge kernel
  int group_base = 0;
  for (int t0 = 0; t0 < T; t0 += NT) {
    const int t = t0 + tid;
    const int ns = t < T ? (t < kTileCache ? s_nqns[t] >> 16 : P.tiles[t].nsplit) : 0;
    int tot;
    const int off = block_excl_scan<NT>(ns > 1 ? H : 0, tmp, &tot);
    if (ns > 1) {
      const int slot0 = t < kTileCache ? s_slot0[t] : P.tiles[t].slot0;
      for (int g = 0; g < H; ++g) P.groups[group_base + off + g] = Group{t, g, ns, slot0 + g * ns};
    }
    group_base += tot;
  }
  if (tid == 0) {
    P.hdr->num_items = (uint32_t)total;
    P.hdr->chunk = (uint32_t)chunk;
    P.hdr->num_groups = (uint32_t)group_base;
    P.hdr->plan_key = P.plan_key;
  }
}

template <int NT>
static hipError_t launch_tiles(const PlanParams& p, int bq, hipStream_t s) {
  switch (bq) {
    case 8: hipLaunchKernelGGL((plan_tiles_kernel<8, NT>), dim3(p.num_tiles), dim3(NT), 0, s, p); break;
    case 16: hipLaunchKernelGGL((plan_tiles_kernel<16, NT>), dim3(p.num_tiles), dim3(NT), 0, s, p); break;
    case 32: hipLaunchKernelGGL((plan_tiles_kernel<32, NT>), dim3(p.num_tiles), dim3(NT), 0, s, p); break;
    case 64: hipLaunchKernelGGL((plan_tiles_kernel<64, NT>), dim3(p.num_tiles), dim3(NT), 0, s, p); break;
    case 128: hipLaunchKernelGGL((plan_tiles_kernel<128, NT>), dim3(p.num_tiles), dim3(NT), 0, s, p); break;
    case 256: hipLaunchKernelGGL((plan_tiles_kernel<256, NT>), dim3(p.num_tiles), dim3(NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_plan(const PlanParams& p, int bq, hipStream_t s) {
  // a request's blocks in one pass where possible; small work-groups for
  // short contexts (more of them resident per CU)
  hipError_t e = p.max_blocks <= kPlanBlocksPerThread * 256 ? launch_tiles<256>(p, bq, s)
                                                              : launch_tiles<kPlanThreads>(p, bq, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_items_kernel, dim3(1), dim3(kItemThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace minipic
