// bf16 position-free paged prefill attention on gfx950 MFMA.
//
// "MiniPIC: Flexible Position-Independent Caching in <100LOC", §3.2.2: the
// kernel loads each K tile UNROTATED from the paged cache, looks up cos/sin
// at the keys' logical positions pi(j), rotates the tile, and only then takes
// its dot products with the already-rotated queries; V is used as stored.
// §3.2.1 gives the score (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d).
//
// Persistent kernel: one work-group per CU takes work items (q tile, KV
// head, piece of the tile's visible-block list) from the per-XCD queues.
//
// One work item = 256 query rows = BQ query tokens x G query heads sharing
// KV head g (G = Hq/Hkv). A work-group has 12 waves in two roles, three per
// SIMD at 168 VGPRs each (waves w, w + 4 and w + 8 share a SIMD):
//   * 8 consumer waves, 32 query rows each (rows 32 w + (l % 32)): QK^T, the
//     online softmax and PV on MFMA;
//   * 4 producer waves: the global loads of the K tiles, their cos/sin rows
//     and the V tiles, the rotation of K, and the stores of both to LDS.
// Splitting the roles keeps the staging registers out of the consumers,
// which is what lets three waves share a SIMD (and two consumers
// alternate between MFMA and vector work while the producer streams).
//   * a pipeline step covers 32 keys = 2 cache blocks of the list.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: keys on the M side, queries on
//     the N side, so lane l holds 16 keys of ONE query and the row max / sum
//     stay in the lane (plus one exchange with l ^ 32).
//   * K rows sit in LDS with bits 2 and 3 of the key index swapped, so the
//     accumulator of lane l, element i, is key 16(i/8) + 8(l/32) + i%8; eight
//     consecutive elements then are the bf16x8 B operand of O^T += V^T P^T.
//   * V is cached transposed inside each block ([d][16]): the V^T A operand
//     is one 16-byte LDS read of 8 consecutive keys.
//   * The K and V fragments of a step are read from LDS through a small ring
//     that runs ahead of the MFMAs, in an order pinned by scheduling fences,
//     so an MFMA seldom waits for its operand.
//   * q is scaled by scale * log2(e) when it is loaded and the QK MFMA chain
//     starts from minus the running max, laid down by one small MFMA (ones
//     times -m, with m kept exact in bf16), so the scores leave the MFMA in
//     log2 units already shifted: P = exp2(S) needs no multiply-add per score,
//     and no vector instruction copies the shift into the accumulator.
//   * Software pipeline with one barrier per step: in step s the consumers
//     compute S(s+1) = K(s+1) Q^T and O += V(s) P(s) and the softmax of the
//     next scores, while the producers rotate and store K(s+2), store V(s+1)
//     (loaded two steps before) and issue the loads of K(s+4), cos/sin(s+4)
//     and V(s+3). The two consumers that share a SIMD take their parts in
//     opposite order, so one issues MFMAs while the other runs vector work.
//     The rotation (rotate-half, i <-> i + d/2) happens once per work item
//     and tile, between the global load and the LDS store, in fp32 with one
//     rounding to bf16.
//   * Global loads are buffer loads: a wave's keys always lie in one cache
//     block, so the block's base address is a scalar and an invalid block
//     becomes a zero-size buffer whose loads return zeros.
//   * The element-wise mask runs only on steps where some row does not see
//     every key (plan_tiles marks fully visible blocks); it is a uniform branch.
//   * Online softmax with a lazily raised running max: the accumulators are
//     rescaled only when a score exceeds the running max by more than 8 (in
//     log2 units), which is exact (numerator and denominator share the stale
//     max). The row sums add the same bf16 P the numerator uses, two at a time
//     with v_dot2_f32_bf16.
//   * q rows come in and the output goes out through an LDS row buffer, so
//     every global load or store instruction moves whole rows; both are
//     non-temporal accesses (each byte is touched once), which keeps them
//     from displacing the K/V lines that the XCD's work-groups share in L2.
//   * A piece of a split tile stores fp32 (O, m, l) to its slot (O in the
//     lanes' order); the merge kernel combines the pieces.
#include "common.h"

namespace minipic {

constexpr int kKT = 32;           // keys per pipeline step
constexpr int kListMax = 256;     // list entries staged in LDS per pass
// Sentinel entries after the last one of a pass (no block: loads return
// zeros, never visible, never full), so the look-ups of the steps past the
// end need no bounds test and the step body stays free of branches. Step s
// issues the K loads of step s + 4 and reads the list entries of the loads of
// step s + 1 (entries up to 2s + 11); with nsteps = ceil(n / 2) the last index
// reached is n + 10.
constexpr int kLoadAhead = 4;
constexpr int kListPad = 2 * kLoadAhead + 4;
constexpr int kClaimLate = -2;   // s_next: the claimed ticket is past its queue
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3 (gfx9, raw dword access)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// Combine a value with the one held by lane l ^ 32: v_permlane32_swap gives
// both operands' halves, so max / sum of the pair needs no LDS round trip.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work-group shape: NW waves of RB row blocks (32 query rows each), NT
// threads; each thread stages one K unit of CW rotate-half pairs (a key's
// elements [CW c, CW c + CW) and [d/2 + CW c, d/2 + CW c + CW)) and VU 16-byte
// V pieces per step.
constexpr int kRB = 1;    // row blocks per consumer wave
constexpr int kNC = 8;    // consumer waves: QK, softmax, PV of 32 query rows each
constexpr int kNP = 4;    // producer waves: K/V loads, rotation, LDS stores
constexpr int kNW = kNC + kNP;

template <int D, int RB>
struct Cfg {
  static constexpr int NT = 64 * kNW;
  static constexpr int PT = 64 * kNP;            // producer threads
  static constexpr int ROWS = 32 * RB * kNC;     // query rows per work item
  static constexpr int CW = 4 * D <= PT ? 4 : 8;
  static constexpr int KCH = (D / 2) / CW;       // K units per key
  static constexpr int KUNITS = kKT * KCH;
  static_assert(KUNITS == PT, "one K unit per producer thread");
  static constexpr int VUNITS = 2 * D * 2;       // 2 blocks x D rows x 2 halves of 8 keys
  static constexpr int VU = VUNITS / PT;
  static_assert(VU * PT == VUNITS, "whole V pieces per producer thread");
  static constexpr int KSTR = D + 8;             // bf16 per K row (16-byte pad: conflict-free MFMA reads)
  static constexpr int VSTR = kKT + 8;           // bf16 per V^T row
  static constexpr int KSZ = kKT * KSTR;
  static constexpr int VSZ = D * VSTR;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// The running-max shift of the scores, made by one small MFMA: with A = (1,
// 0, 0, 0) in lanes 0..31 (zeros in 32..63) and B = (-m, 0, 0, 0) in lane n
// (m the running max of query row n, exact in bf16), D[key][n] = -m for every
// key. The QK chain accumulates on top of it; the broadcast costs no vector
// instruction per step.
__device__ __forceinline__ f32x16 bias_mfma(const s16x4& ones, const s16x4& mb) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ones, mb, f32x16{}, 0, 0, 0);
}

// bf16 operand (-m, 0, 0, 0) for lanes 0..31, zero for lanes 32..63
__device__ __forceinline__ s16x4 bias_operand(float m, int lane) {
  const uint32_t b = (m == -INFINITY || lane >= 32) ? 0u : (__float_as_uint(-m) >> 16);
  return s16x4{(short)b, 0, 0, 0};
}

// smallest bf16 value >= x (x finite)
__device__ __forceinline__ float bf16_ceil(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0xffffu) == 0u) return x;
  return __uint_as_float(x > 0.f ? ((u + 0x10000u) & 0xffff0000u) : (u & 0xffff0000u));
}

__device__ __forceinline__ int key_perm(int k) {
  // swap bits 2 and 3 (an involution); bits 0, 1, 4 unchanged
  return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Registers of the loads in flight for one step.
template <int D, int RB>
struct Stage {
  static constexpr int CW = Cfg<D, RB>::CW;
  uint32_t ka[CW / 2], kb[CW / 2];   // CW bf16 of each half of the K unit
  float c[CW], s[CW];                // cos / sin of the unit's CW frequencies
  u32x4 v[Cfg<D, RB>::VU];
  int nv[Cfg<D, RB>::VU];            // keys inside the context in each V piece's block
};

// Per-pass state the step helpers need (all wave-uniform).
template <int D, int RB>
struct StepCtx {
  const BlkDesc* lst;   // LDS: list entries of this pass
  const int* pos_s;     // LDS: logical position of every key of the pass
  int n_l;              // entries in the pass
  const __bf16* kc;     // K cache + offset of head g inside a block group
  const __bf16* vc;     // V cache + offset of head g
  int64_t group;        // elements per physical block group (all heads)
  rsrc_t tab;           // cos/sin table
  __bf16* kl;           // LDS K buffers
  __bf16* vl;           // LDS V^T buffers
};

// The lane's query rows.
template <int RB>
struct RowInfo {
  int c[RB], bq[RB], span[RB], lo[RB];
  bool valid[RB], pdep[RB];
};

// List look-ups of one step's tile loads, read from LDS a step before the
// loads are issued (so no step waits on an LDS round trip for them): the
// physical block of the wave's K block and of each of its V pieces (uniform
// values, -1 past the list), and the logical position of the thread's key.
template <int D, int RB>
struct Pre {
  int ph_k, pos;
  int ph_v[Cfg<D, RB>::VU], nv_v[Cfg<D, RB>::VU];
};

template <int D, int RB, bool ROPE>
__device__ __forceinline__ void prefetch(const StepCtx<D, RB>& cx, int jk, int jv, Pre<D, RB>& pr, int tid) {
  using C = Cfg<D, RB>;
  const int t0 = __builtin_amdgcn_readfirstlane(tid);
  const int ek = __builtin_amdgcn_readfirstlane(2 * jk + t0 / (C::KCH * kBlock));
  pr.ph_k = cx.lst[ek].phys;
  if (ROPE) pr.pos = cx.pos_s[ek * kBlock + (tid / C::KCH) % kBlock];
#pragma unroll
  for (int u = 0; u < C::VU; ++u) {
    const int u0 = __builtin_amdgcn_readfirstlane(tid + u * C::PT);
    const int ev = __builtin_amdgcn_readfirstlane(2 * jv + u0 / (2 * D));
    pr.ph_v[u] = cx.lst[ev].phys;
    pr.nv_v[u] = cx.lst[ev].nvalid;
  }
}

// Global loads of a step's K unit and its cos/sin rows (list look-ups in
// pr). Past the list or for an invalid block the buffer is empty and the
// loads return zeros.
template <int D, int RB, bool ROPE>
__device__ __forceinline__ void load_k(const StepCtx<D, RB>& cx, const Pre<D, RB>& pr, Stage<D, RB>& st, int tid) {
  using C = Cfg<D, RB>;
  constexpr int CW = C::CW;
  const int key = tid / C::KCH, ch = tid % C::KCH;
  // a wave's K units lie in one block and are all active or all idle: derive
  // both from the wave's first thread so the buffer descriptor is scalar
  const int off = key % kBlock;
  const int ph = __builtin_amdgcn_readfirstlane(pr.ph_k);
  const int bytes = ph >= 0 ? kBlock * D * 2 : 0;
  const rsrc_t r = make_rsrc(cx.kc + (int64_t)(ph < 0 ? 0 : ph) * cx.group, bytes);
  const int row_b = (off * D + CW * ch) * 2;
  if constexpr (CW == 8) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, row_b, 0, 0));
    const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, row_b + D, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) { st.ka[i] = a[i]; st.kb[i] = b[i]; }
  } else {
    const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, row_b, 0, 0));
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, row_b + D, 0, 0));
#pragma unroll
    for (int i = 0; i < 2; ++i) { st.ka[i] = a[i]; st.kb[i] = b[i]; }
  }
  if (ROPE) {
    const int tb = (pr.pos * D + CW * ch) * 4;
#pragma unroll
    for (int q = 0; q < CW / 4; ++q) {
      const f32x4 cv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(cx.tab, tb + 16 * q, 0, 0));
      const f32x4 sv =
          __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(cx.tab, tb + D * 2 + 16 * q, 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) { st.c[4 * q + i] = cv[i]; st.s[4 * q + i] = sv[i]; }
    }
  }
}

template <int D, int RB>
__device__ __forceinline__ void load_v(const StepCtx<D, RB>& cx, const Pre<D, RB>& pr, Stage<D, RB>& st, int tid) {
  using C = Cfg<D, RB>;
#pragma unroll
  for (int u = 0; u < C::VU; ++u) {
    const int unit = tid + u * C::PT;   // a wave's pieces share one block
    const int rem = unit % (2 * D);
    const int ph = __builtin_amdgcn_readfirstlane(pr.ph_v[u]);
    const rsrc_t r = make_rsrc(cx.vc + (int64_t)(ph < 0 ? 0 : ph) * cx.group, ph >= 0 ? kBlock * D * 2 : 0);
    st.v[u] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, ((rem / 2) * kBlock + 8 * (rem % 2)) * 2, 0, 0));
    st.nv[u] = __builtin_amdgcn_readfirstlane(pr.nv_v[u]);
  }
}

// Rotate the staged K unit (rotate-half in fp32, one rounding to bf16) and
// store it to LDS buffer `buf` in the permuted row order.
template <int D, int RB, bool ROPE>
__device__ __forceinline__ void store_k(const StepCtx<D, RB>& cx, int buf, const Stage<D, RB>& st, int tid) {
  using C = Cfg<D, RB>;
  constexpr int CW = C::CW;
  const int key = tid / C::KCH, ch = tid % C::KCH;
  uint32_t ra[CW / 2], rb[CW / 2];
#pragma unroll
  for (int j = 0; j < CW / 2; ++j) {
    if (ROPE) {
      const float a0 = bf16_lo(st.ka[j]), a1 = bf16_hi(st.ka[j]);
      const float b0 = bf16_lo(st.kb[j]), b1 = bf16_hi(st.kb[j]);
      const float c0 = st.c[2 * j], c1 = st.c[2 * j + 1];
      const float s0 = st.s[2 * j], s1 = st.s[2 * j + 1];
      ra[j] = pack_bf16x2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
      rb[j] = pack_bf16x2(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
    } else {
      ra[j] = st.ka[j];
      rb[j] = st.kb[j];
    }
  }
  __bf16* dst = cx.kl + buf * C::KSZ + key_perm(key) * C::KSTR + CW * ch;
  if constexpr (CW == 8) {
    *(u32x4*)dst = u32x4{ra[0], ra[1], ra[2], ra[3]};
    *(u32x4*)(dst + D / 2) = u32x4{rb[0], rb[1], rb[2], rb[3]};
  } else {
    *(u32x2*)dst = u32x2{ra[0], ra[1]};
    *(u32x2*)(dst + D / 2) = u32x2{rb[0], rb[1]};
  }
}

template <int D, int RB>
__device__ __forceinline__ void store_v(const StepCtx<D, RB>& cx, int buf, const Stage<D, RB>& st, int tid) {
  using C = Cfg<D, RB>;
#pragma unroll
  for (int u = 0; u < C::VU; ++u) {
    const int unit = tid + u * C::PT;
    const int bk = unit / (2 * D);
    const int rem = unit % (2 * D);
    u32x4 val = st.v[u];
    if (st.nv[u] < kBlock) {
      // a ragged last block: its slots past the context hold no token (maybe
      // NaN); P is 0 there, but 0 * NaN would still reach O, so zero them
      const int k0 = 8 * (rem % 2);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int k = k0 + 2 * w;
        val[w] = k >= st.nv[u] ? 0u : (k + 1 >= st.nv[u] ? (val[w] & 0xffffu) : val[w]);
      }
    }
    *(u32x4*)(cx.vl + buf * C::VSZ + (rem / 2) * C::VSTR + kBlock * bk + 8 * (rem % 2)) = val;
  }
}

// S^T - m for the 32 keys in K buffer `buf`, all row blocks of the wave: the
// MFMA chain starts from the bias MFMA's -m (every element of a lane is minus
// the running max of the lane's query row), so the scores leave the MFMA
// already shifted.
template <int D, int RB>
__device__ __forceinline__ void qk(const StepCtx<D, RB>& cx, int buf, const bf16x8 (&qf)[RB][D / 16],
                                   const s16x4& ones, const s16x4 (&mb)[RB], f32x16 (&s)[RB]) {
  using C = Cfg<D, RB>;
  const int lane = threadIdx.x & 63;
  const __bf16* kb_ = cx.kl + buf * C::KSZ + (lane & 31) * C::KSTR + 8 * (lane >> 5);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) s[rb] = bias_mfma(ones, mb[rb]);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 a = *(const bf16x8*)(kb_ + 16 * ks);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[rb][ks], s[rb], 0, 0, 0);
  }
}

// S(s+1) = K Q^T from K buffer kbuf and O += V P from V buffer vbuf (one row
// block per wave): the LDS fragment reads run kRing ahead of the MFMAs in a
// ring (program order of the QK part pinned with scheduling fences), so an
// MFMA seldom waits on an LDS read.
constexpr int kRing = 2;
template <int D, int RB>
__device__ __forceinline__ void qk_pv(const StepCtx<D, RB>& cx, int kbuf, int vbuf, const bf16x8 (&qf)[RB][D / 16],
                                      const s16x4& ones, const s16x4 (&mb)[RB], f32x16 (&s)[RB], const bf16x8 (&pk)[RB][2],
                                      f32x16 (&o)[RB][D / 32]) {
  using C = Cfg<D, RB>;
  static_assert(RB == 1, "one row block per wave");
  const int lane = threadIdx.x & 63;
  const __bf16* kb_ = cx.kl + kbuf * C::KSZ + (lane & 31) * C::KSTR + 8 * (lane >> 5);
  const __bf16* vb_ = cx.vl + vbuf * C::VSZ + (lane & 31) * C::VSTR + 8 * (lane >> 5);
  constexpr int NK = D / 16, NV = 2 * (D / 32), N = NK + NV;
  auto addr = [&](int i) -> const bf16x8* {
    return i < NK ? (const bf16x8*)(kb_ + 16 * i)
                  : (const bf16x8*)(vb_ + 32 * ((i - NK) / 2) * C::VSTR + 16 * ((i - NK) % 2));
  };
  bf16x8 ring[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) ring[i] = *addr(i);
  s[0] = bias_mfma(ones, mb[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bf16x8 a = ring[i % kRing];
    if (i < NK) s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0][i], s[0], 0, 0, 0);
    else o[0][(i - NK) / 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[0][(i - NK) % 2], o[0][(i - NK) / 2], 0, 0, 0);
    if (i + kRing < N) ring[i % kRing] = *addr(i + kRing);
    // the QK part in a pinned order; the PV part left to the scheduler, which
    // may move the wave's other work between its MFMAs
    if (i < NK) __builtin_amdgcn_sched_barrier(0);
  }
}

// Bit j: every row of the tile sees every key of step j. One bit per step of
// a pass (at most 128), built once per pass by a ballot over the list.
template <int D, int RB>
__device__ __forceinline__ void full_steps(const StepCtx<D, RB>& cx, int nsteps, uint64_t (&fm)[2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = 64 * h + lane;
    const bool f = j < nsteps && (cx.lst[2 * j].full & cx.lst[2 * j + 1].full) != 0;
    fm[h] = __ballot(f);
  }
}

// element-wise mask of step j: block visibility and the causal diagonal
template <int D, int RB>
__device__ __forceinline__ void apply_mask(const StepCtx<D, RB>& cx, int j, const RowInfo<RB>& rows, f32x16 (&s)[RB]) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    const BlkDesc bd = cx.lst[2 * j + bk];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool vis = rows.valid[rb] && block_visible(bd.kb, bd.span, bd.flags, rows.bq[rb], rows.span[rb],
                                                       rows.pdep[rb], rows.lo[rb]);
      const int lim = rows.c[rb] - bd.kb * kBlock - 8 * h;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (!(vis && r <= lim)) s[rb][8 * bk + r] = -INFINITY;
    }
  }
}

// P = exp2(S - m) rounded to bf16 in the B-operand layout of the PV MFMA
// (the scores are already in log2 units and shifted by the running max). The
// lane's share of the row sum adds the same bf16 values the numerator uses,
// two per v_dot2_f32_bf16 against (1, 1). (The packed word goes to the dot
// product before it is inserted into the vector: taking it back out of the
// vector made hipcc read the first word of the quad four times.)
template <int RB>
__device__ __forceinline__ void softmax_p(const f32x16 (&s)[RB], bf16x8 (&pk)[RB][2], float (&lsum)[RB]) {
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      u32x4 u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(s[rb][8 * sh + 2 * j]), __builtin_amdgcn_exp2f(s[rb][8 * sh + 2 * j + 1]));
        lsum[rb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one2, lsum[rb], false);
        u[j] = w;
      }
      pk[rb][sh] = __builtin_bit_cast(bf16x8, u);
    }
}

// max of the lane's 16 shifted scores (one half of its query row)
__device__ __forceinline__ float lane_max(const f32x16& s) {
  float m = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int i = 3; i + 1 < 16; i += 2) m = fmaxf(fmaxf(m, s[i]), s[i + 1]);
  return fmaxf(m, s[15]);
}

// Running-max state of the lane's query rows. The max is raised lazily: only
// when a shifted score exceeds `thr` (2^8 while the row has a max; -inf
// before its first visible key, when the shift is 0).
template <int RB>
struct MaxState {
  float m[RB];        // running max in log2 units (-inf: no visible key yet)
  float thr[RB];
  s16x4 mb[RB];       // B operand of the bias MFMA: -m (exact in bf16), or 0 while m is -inf
};

// Shift the rows whose scores crossed the threshold to their new max: the
// scores of this step, the bias of the next ones, O and the row sums.
template <int D, int RB>
__device__ __forceinline__ void raise_max(const float (&mx)[RB], MaxState<RB>& ms, f32x16 (&sc)[RB],
                                          float (&lsum)[RB], f32x16 (&o)[RB][D / 32], int lane) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float rm = xor32_max(mx[rb]);           // shifted row max
    const bool up = rm > ms.thr[rb];
    const float m_old = ms.m[rb];
    const float base = m_old == -INFINITY ? 0.f : m_old;
    // the new max is rounded up to a bf16 value (the bias MFMA takes it in
    // bf16); the shift of this step's scores is the exact difference
    const float m_new = up ? bf16_ceil(base + rm) : m_old;
    const float delta = up ? m_new - base : 0.f;
    const float alpha = up ? exp2f(m_old - m_new) : 1.f;   // 0 for a first max (O, l are zero)
#pragma unroll
    for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[rb][dg][i] *= alpha;
    lsum[rb] *= alpha;

#pragma unroll
    for (int i = 0; i < 16; ++i) sc[rb][i] -= delta;
    if (up) {
      ms.m[rb] = m_new;
      ms.thr[rb] = 8.0f;
      ms.mb[rb] = bias_operand(m_new, lane);
    }
  }
}

// Work item i through the constant address space: with a uniform index the
// fields arrive by scalar loads (the list was written by an earlier launch).
__device__ __forceinline__ Item load_item(const Item* items, int i) {
  typedef const __attribute__((address_space(4))) int32_t CI;
  const CI* f = (const CI*)(items + i);
  Item t;
  t.tile = f[0];
  t.p0 = f[1];
  t.p1 = f[2];
  t.gsn = (uint32_t)f[3];
  t.r = f[4];
  t.row0 = f[5];
  t.nq = f[6];
  t.slot0 = f[7];
  return t;
}

// Role of a wave, as a type: the two roles run the item loop as separate
// instances, so that neither keeps the other's registers live.
template <bool B>
struct Role {
  static constexpr bool prod = B;
};

template <int D, int G, bool ROPE, int RB>
__global__ void __launch_bounds__(64 * kNW, 1) attn_bf16_kernel(AttnParams P) {
  using C = Cfg<D, RB>;
  using St = Stage<D, RB>;
  constexpr int NT = C::NT;
  constexpr int BQ = C::ROWS / G;
  constexpr int NKS = D / 16;             // k-steps of QK^T
  constexpr int NDG = D / 32;             // 32-row d blocks of O^T
  __shared__ __attribute__((aligned(16))) BlkDesc lst[kListMax + kListPad];
  __shared__ __attribute__((aligned(16))) int pos_s[ROPE ? (kListMax + kListPad) * kBlock : 4];
  __shared__ int s_first, s_next, s_late;
  __shared__ uint32_t s_qs[kQueues], s_qc[kQueues];
  __shared__ __attribute__((aligned(16))) __bf16 kl[2 * C::KSZ];
  __shared__ __attribute__((aligned(16))) __bf16 vl[2 * C::VSZ];
  // the query rows of the work item, bf16, one padded row each: q passes
  // through it on the way in and the normalised output on the way out, so
  // that every global load or store instruction moves whole rows (each
  // wave uses only its own rows)
  __shared__ __attribute__((aligned(16))) __bf16 rowbuf[C::ROWS * C::KSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  // waves w, w + 4 and w + 8 share a SIMD: consumers w < 4 lead, w + 4
  // trail (see the step loop), w + 8 produces
  const bool producer = w >= kNC;
  const bool lead = w < 4;
  const int pt = tid - 64 * kNC;   // producer thread index

  const __bf16* kc = (const __bf16*)P.k_cache;
  const __bf16* vc = (const __bf16*)P.v_cache;
  const float sl2 = P.scale_log2;
  const rsrc_t tab = make_rsrc(P.cos_sin, P.max_pos * D * 4);

  // a run needs the plan of its own configuration in the workspace
  if (P.hdr->plan_key != P.plan_key) {   // uniform (one scalar load)
    if (blockIdx.x == 0 && tid == 0) atomicOr(P.err, (uint32_t)MINIPIC_EW_PLAN);
    return;
  }
  if (blockIdx.x == 0 && tid == 0) {   // measurement: clock stamps of work-group 0
    P.hdr->clk_start = clock64();
    P.hdr->rt_start = wall_clock64();
  }
  if (tid < kQueues) {
    s_qs[tid] = P.hdr->qstart[tid];
    s_qc[tid] = P.hdr->qcount[tid];
  }
  int q_cur = blockIdx.x % kQueues;   // queue being drained (thread 0)
  __syncthreads();
  // the first item is the work-group's own ticket (the planner starts each
  // queue's counter past the work-groups that drain it)
  if (tid == 0) s_first = resolve_ticket(P.hdr, s_qs, s_qc, q_cur, blockIdx.x / kQueues);
  __syncthreads();
  // the two roles run the same items and barriers in loops of their own
  // (so that neither keeps the other's registers live)
  auto run = [&](auto role) {
  constexpr bool prod = decltype(role)::prod;
  int it = __builtin_amdgcn_readfirstlane(s_first);
  Item item{};
  if (it >= 0) item = load_item(P.items, it);
  while (it >= 0) {
    // Claim the following item now. Thread 0 publishes the ticket's item
    // (when it falls inside the current queue) just before the prologue's
    // first barrier, long after the atomic has returned, and every wave reads
    // s_next after the prologue's second barrier; s_next is written again
    // only in the next item's prologue, after that item's staging barrier, so
    // the item needs no barrier at its end, and the following item's fields
    // are read during this one (scalar loads). A ticket past its queue is
    // resolved at the end of the item (the queue walk, with a barrier), off
    // the critical path of the item.
    uint32_t ticket = 0;
    int nxt = -1;
    Item nitem = item;
    const int g = item.gsn & 0xff;
    const int sp = (item.gsn >> 8) & 0xfff;
    const int ns = item.gsn >> 20;
    const int32_t* lpos = P.logical_pos + (int64_t)item.r * P.max_blocks * kBlock;
    const BlkDesc* blist = P.blist + (int64_t)item.tile * P.max_blocks;
    const int64_t kv_head = (int64_t)g * kBlock * D;   // offset of head g inside a block group

    // ---- the list of the first pass is fetched before the rows, so that its
    // loads and those of q are in flight together
    // (entries past the piece are sentinels: above every query block, so
    // never visible, no block, never full)
    constexpr int LI = (kListMax + kListPad + NT - 1) / NT;
    u32x4 bdv[LI][2];
    auto fetch_list = [&](int c0, int n_l) {
#pragma unroll
      for (int k = 0; k < LI; ++k) {
        const int i = tid + k * NT;
        const u32x4* src = (const u32x4*)(blist + c0 + (i < n_l ? i : 0));
        bdv[k][0] = i < n_l ? src[0] : u32x4{1u << 26, 0xffffffffu, 0xffffffffu, 0u};
        bdv[k][1] = i < n_l ? src[1] : u32x4{0u, 0u, 0u, 0u};
      }
    };
    // The thread that holds entry i also writes the logical positions of its
    // 16 keys: its base position plus the key offset, or (positions that do
    // not run consecutively) the request's positions, clamped to the table.
    auto store_list = [&](int n_l) {
#pragma unroll
      for (int k = 0; k < LI; ++k) {
        const int i = tid + k * NT;
        if (i < n_l + kListPad) {
          u32x4* dst = (u32x4*)(lst + i);
          dst[0] = bdv[k][0];
          dst[1] = bdv[k][1];
          if (ROPE) {
            const int kb = (int)bdv[k][0][0];
            const int pos0 = (int)bdv[k][1][0];
            u32x4* pd = (u32x4*)(pos_s + i * kBlock);
            if (pos0 >= 0) {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                pd[q] = u32x4{(uint32_t)(pos0 + 4 * q), (uint32_t)(pos0 + 4 * q + 1), (uint32_t)(pos0 + 4 * q + 2),
                              (uint32_t)(pos0 + 4 * q + 3)};
            } else {
              const int nvalid = (int)bdv[k][1][2];
              for (int o2 = 0; o2 < kBlock; ++o2) {
                // keys past the context hold no token: any row of the table will do
                int pos = o2 < nvalid ? lpos[kb * kBlock + o2] : 0;
                if (pos < 0 || pos >= P.max_pos) {
                  atomicOr(P.err, (uint32_t)MINIPIC_EW_POS);
                  pos = pos < 0 ? 0 : P.max_pos - 1;
                }
                pos_s[i * kBlock + o2] = pos;
              }
            }
          }
        }
      }
    };
    // The claim goes out first: its answer is needed only at the prologue's
    // second barrier. The list and q loads behind it retire after it (loads
    // retire in issue order), which costs little: an atomic at L2 usually
    // returns before loads that go to HBM.
    if (tid == 0) ticket = atomicAdd(&P.hdr->next[q_cur], 1u);
    fetch_list(item.p0, min(kListMax, item.p1 - item.p0));

    // ---- the lane's query rows
    RowInfo<RB> rows;
    bf16x8 qf[RB][NKS];
    // q rows of the wave: lane i loads 16-byte piece i % CPR of row i / CPR
    // (+ RPI per round), so a load instruction reads RPI whole rows; they go
    // to the wave's rows of rowbuf. A row past the tile's end is read from
    // its last token (an address inside q) and zeroed below, so the loads do
    // not wait for the row descriptors. All of the wave's q loads and its
    // rows' descriptors are in flight together (one round trip).
    constexpr int CPR = D / 8;          // 16-byte pieces per row
    constexpr int RPI = 64 / CPR;       // rows per load instruction
    constexpr int QLD = 32 * RB / RPI;  // load instructions per lane
    // (the lane index is made opaque here so that the row and buffer
    // addresses derived from it, the same for every item, are computed when
    // used instead of being kept across the item loop, where they would
    // not fit in the registers and would go to scratch)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int l32 = ln & 31;
    const int h = ln >> 5;
    if constexpr (!prod) {
      u32x4 qv[QLD];
#pragma unroll
      for (int k = 0; k < QLD; ++k) {
        const int rw = 32 * RB * w + RPI * k + ln / CPR;
        const int tq = rw / G;
        const int tq_in = tq < item.nq ? tq : item.nq - 1;
        // read once: non-temporal, so q does not displace K/V lines that
        // other work-groups of the XCD still stream through its L2
        qv[k] = __builtin_nontemporal_load((const u32x4*)((const __bf16*)P.q +
                                                          (((int64_t)item.row0 + tq_in) * P.hq + g * G + rw % G) * D +
                                                          8 * (ln % CPR)));
      }
      TokDesc tk[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) tk[rb] = P.toks[(int64_t)item.tile * BQ + (32 * RB * w + 32 * rb + l32) / G];
#pragma unroll
      for (int k = 0; k < QLD; ++k)
        *(u32x4*)(rowbuf + (32 * RB * w + RPI * k + ln / CPR) * C::KSTR + 8 * (ln % CPR)) = qv[k];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = 32 * RB * w + 32 * rb + l32;
        const int tok = row / G;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[rb][ks] = *(const bf16x8*)(rowbuf + row * C::KSTR + 16 * ks + 8 * h);
        const bool valid = tok < item.nq && tk[rb].c >= 0;
        rows.valid[rb] = valid;
        rows.c[rb] = valid ? tk[rb].c : -1;
        rows.bq[rb] = valid ? (tk[rb].c >> 4) : -1;
        rows.span[rb] = tk[rb].span;
        rows.lo[rb] = tk[rb].lo;
        rows.pdep[rb] = valid && tk[rb].pdep;
      }
    }
    store_list(min(kListMax, item.p1 - item.p0));
    if constexpr (!prod)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool valid = rows.valid[rb];
      if (!valid) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[rb][ks] = bf16x8{};
      }
      // q is scaled by scale * log2(e) here, so that the MFMA gives the scores in
      // log2 units (rounded to bf16 once with the rotation below)
      if (!(P.flags & MINIPIC_FLAG_ROTATE_Q)) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          u32x4 u = __builtin_bit_cast(u32x4, qf[rb][ks]);
#pragma unroll
          for (int j = 0; j < 4; ++j) u[j] = pack_bf16x2(bf16_lo(u[j]) * sl2, bf16_hi(u[j]) * sl2);
          qf[rb][ks] = __builtin_bit_cast(bf16x8, u);
        }
      } else if (valid) {
        int pos = lpos[rows.c[rb]];
        if (pos < 0 || pos >= P.max_pos) {
          atomicOr(P.err, (uint32_t)MINIPIC_EW_POS);
          pos = pos < 0 ? 0 : P.max_pos - 1;
        }
        const float* cs = P.cos_sin + (int64_t)pos * D;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const u32x4 a = __builtin_bit_cast(u32x4, qf[rb][ks]);
          const u32x4 b = __builtin_bit_cast(u32x4, qf[rb][ks + D / 32]);
          u32x4 ra, rbv;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i0 = 16 * ks + 8 * h + 2 * j;
            const float c_0 = cs[i0] * sl2, c_1 = cs[i0 + 1] * sl2;
            const float s_0 = cs[D / 2 + i0] * sl2, s_1 = cs[D / 2 + i0 + 1] * sl2;
            const float a0 = bf16_lo(a[j]), a1 = bf16_hi(a[j]);
            const float b0 = bf16_lo(b[j]), b1 = bf16_hi(b[j]);
            ra[j] = pack_bf16x2(a0 * c_0 - b0 * s_0, a1 * c_1 - b1 * s_1);
            rbv[j] = pack_bf16x2(b0 * c_0 + a0 * s_0, b1 * c_1 + a1 * s_1);
          }
          qf[rb][ks] = __builtin_bit_cast(bf16x8, ra);
          qf[rb][ks + D / 32] = __builtin_bit_cast(bf16x8, rbv);
        }
      }
    }


    f32x16 o[RB][NDG];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < NDG; ++i) o[rb][i] = f32x16{};
    MaxState<RB> mst;
    // A operand of the bias MFMA: (1, 0, 0, 0) in lanes 0..31
    const s16x4 ones = (threadIdx.x & 32) ? s16x4{0, 0, 0, 0} : s16x4{(short)0x3f80, 0, 0, 0};
    float lsum[RB];        // the lane's share of the running row sums (lanes l, l ^ 32 add up to row l % 32)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      mst.m[rb] = -INFINITY;
      mst.thr[rb] = -INFINITY;
      mst.mb[rb] = s16x4{0, 0, 0, 0};
      lsum[rb] = 0.f;
    }

    for (int c0 = item.p0; c0 < item.p1; c0 += kListMax) {
      const int n_l = min(kListMax, item.p1 - c0);
      const int nsteps = (n_l + 1) / 2;
      // ---- stage the list piece (the first pass was staged with the rows)
      if (c0 != item.p0) {
        fetch_list(c0, n_l);
        store_list(n_l);
      }
      __syncthreads();

      StepCtx<D, RB> cx;
      cx.lst = lst;
      cx.pos_s = pos_s;
      cx.n_l = n_l;
      cx.kc = kc + kv_head;
      cx.vc = vc + kv_head;
      cx.group = (int64_t)P.hkv * kBlock * D;
      cx.tab = tab;
      cx.kl = kl;
      cx.vl = vl;

      // ---- prologue: K(0), V(0), K(1) in LDS; S(0) (and for the leading
      // waves P(0)); loads of K(2), V(1) (stage sa) and K(3), V(2) (stage sb)
      // in flight. Step s stores the stage it loaded two steps before, so each
      // load has two steps to arrive.
      St sa, sb;
      Pre<D, RB> pr;
      if constexpr (prod) {
        prefetch<D, RB, ROPE>(cx, 0, 0, pr, pt);
        load_k<D, RB, ROPE>(cx, pr, sa, pt);
        load_v<D, RB>(cx, pr, sa, pt);
        prefetch<D, RB, ROPE>(cx, 1, 1, pr, pt);
        load_k<D, RB, ROPE>(cx, pr, sb, pt);
        store_k<D, RB, ROPE>(cx, 0, sa, pt);
        store_v<D, RB>(cx, 0, sa, pt);
        prefetch<D, RB, ROPE>(cx, 2, 1, pr, pt);
        load_k<D, RB, ROPE>(cx, pr, sa, pt);
        load_v<D, RB>(cx, pr, sa, pt);
        store_k<D, RB, ROPE>(cx, 1, sb, pt);
        prefetch<D, RB, ROPE>(cx, 3, 2, pr, pt);
        load_k<D, RB, ROPE>(cx, pr, sb, pt);
        load_v<D, RB>(cx, pr, sb, pt);
        prefetch<D, RB, ROPE>(cx, kLoadAhead, kLoadAhead - 1, pr, pt);   // the loads of step 0
      }
      uint64_t fm[2];
      full_steps(cx, nsteps, fm);
      if (c0 == item.p0 && tid == 0) s_next = ticket < s_qc[q_cur] ? (int)(s_qs[q_cur] + ticket) : kClaimLate;
      __syncthreads();
      f32x16 sc[RB];         // scores S of one step
      bf16x8 pk[RB][2];      // probabilities P of one step (B operand of the PV MFMA)
      // S(j) in sc -> P(j) in pk: mask where the step is not full, raise the
      // running max where a score crossed the threshold, exponentiate
      auto softmax_step = [&](int j) {
        if ((((j < 64 ? fm[0] : fm[1]) >> (j & 63)) & 1) == 0) apply_mask(cx, j, rows, sc);
        float mx[RB];
        bool up = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          mx[rb] = lane_max(sc[rb]);
          up |= mx[rb] > mst.thr[rb];
        }
        if (__any(up)) raise_max<D, RB>(mx, mst, sc, lsum, o, (int)(threadIdx.x & 63));
        softmax_p<RB>(sc, pk, lsum);
      };
      // the work-group's share of the tile traffic of step s: rotate and store
      // K(s+2), store V(s+1) (stage st, loaded in step s-2), issue the loads
      // of K(s+4), V(s+3) into the same stage, read the list entries of the
      // next step's loads
      auto tiles = [&](int s, St& st) {
        store_k<D, RB, ROPE>(cx, s & 1, st, pt);
        store_v<D, RB>(cx, (s + 1) & 1, st, pt);
        load_k<D, RB, ROPE>(cx, pr, st, pt);
        load_v<D, RB>(cx, pr, st, pt);
        prefetch<D, RB, ROPE>(cx, s + 1 + kLoadAhead, s + kLoadAhead, pr, pt);
      };
      // S(s+1) = K(s+1) Q^T and O += V(s) P(s), with the row sums of P(s)
      auto mfma = [&](int s) {
        qk_pv<D, RB>(cx, (s + 1) & 1, s & 1, qf, ones, mst.mb, sc, pk, o);
      };
      if constexpr (!prod) {
        qk<D, RB>(cx, 0, qf, ones, mst.mb, sc);
        if (lead) softmax_step(0);
      }
      __syncthreads();   // K(0) read by every wave before step 0 reuses its buffer
      if (c0 == item.p0) {
        nxt = __builtin_amdgcn_readfirstlane(s_next);
        if (nxt >= 0) nitem = load_item(P.items, nxt);
      }

      // Steps. The two waves sharing a SIMD work in opposite order inside a
      // step, so that one issues its MFMAs while the other runs its vector
      // ALU work: a leading wave does the MFMA part of step s first, then the
      // softmax of S(s+1) and its share of the tile traffic; a trailing wave
      // does the softmax of S(s) and the tile traffic first, then the MFMAs.
      // (This is program order: the compiler is free to interleave the
      // independent instructions of the parts, which measured faster than
      // fencing them.)
      // Both read K(s+1), V(s) and write K(s+2), V(s+1) (other buffers) in
      // step s; one barrier ends each step.
      // The stages alternate with the step's parity, so the loop runs two
      // steps per iteration.
      // Consumers compute, producers stage the tiles two steps ahead; one
      // barrier ends each step of every wave.
      if constexpr (prod) {
        int s = 0;
        for (; s + 1 < nsteps; s += 2) {
          tiles(s, sa);
          __syncthreads();
          tiles(s + 1, sb);
          __syncthreads();
        }
        if (s < nsteps) {
          tiles(s, sa);
          __syncthreads();
        }
      } else if (lead) {
        for (int s = 0; s < nsteps; ++s) {
          mfma(s);
          if (s + 1 < nsteps) softmax_step(s + 1);
          __syncthreads();
        }
      } else {
        for (int s = 0; s < nsteps; ++s) {
          softmax_step(s);
          mfma(s);
          __syncthreads();
        }
      }
    }

    // ---- epilogue (the lane's row and buffer addresses are derived again
    // from an opaque lane index, so none of them stays live across the steps)
    ln = lane;
    asm volatile("" : "+v"(ln));
    const int l32e = ln & 31;
    const int he = ln >> 5;
    if constexpr (prod) {
    } else if (ns == 1) {
      // out = O / l in bf16: the wave's rows go to rowbuf, then every store
      // instruction writes RPI whole rows of out (rows past the tile's end
      // or without keys are not written)
      uint32_t vmask[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float inv = 1.f / xor32_sum(lsum[rb]);
        vmask[rb] = (uint32_t)__ballot(rows.valid[rb]);
        __bf16* rp = rowbuf + (32 * RB * w + 32 * rb + l32e) * C::KSTR + 4 * he;
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            u32x2 u;
            u[0] = pack_bf16x2(o[rb][dg][4 * j] * inv, o[rb][dg][4 * j + 1] * inv);
            u[1] = pack_bf16x2(o[rb][dg][4 * j + 2] * inv, o[rb][dg][4 * j + 3] * inv);
            *(u32x2*)(rp + 32 * dg + 8 * j) = u;
          }
      }
#pragma unroll
      for (int k = 0; k < 32 * RB / RPI; ++k) {
        const int rr = RPI * k + ln / CPR;   // row within the wave's rows
        const u32x4 v = *(const u32x4*)(rowbuf + (32 * RB * w + rr) * C::KSTR + 8 * (ln % CPR));
        if ((vmask[rr / 32] >> (rr % 32)) & 1u) {
          const int rw = 32 * RB * w + rr;
          // written once and not read by this launch: non-temporal as well
          __builtin_nontemporal_store(v, (u32x4*)((__bf16*)P.out + (((int64_t)item.row0 + rw / G) * P.hq + g * G + rw % G) * D +
                                                  8 * (ln % CPR)));
        }
      }
    } else {
      // a piece of a split tile: fp32 (O, m, l) to its slot, merged by
      // merge_kernel. O is stored in the lanes' own order: the 32-row block
      // of a wave is [d/32][(d%32)/8][lane][4] with lane = row + 32 ((d%8)/4),
      // so every store instruction writes 1 KiB in one piece.
      const int slot = item.slot0 + g * ns + sp;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float l_tot = xor32_sum(lsum[rb]);
        float* po = P.part_o + ((int64_t)slot * C::ROWS + 32 * (RB * w + rb)) * D + 4 * ln;
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 u = {o[rb][dg][4 * j], o[rb][dg][4 * j + 1], o[rb][dg][4 * j + 2], o[rb][dg][4 * j + 3]};
            *(f32x4*)(po + (dg * 4 + j) * 256) = u;
          }
        if (he == 0 && rows.valid[rb])
          P.part_ml[(int64_t)slot * C::ROWS + 32 * RB * w + 32 * rb + l32e] = make_float2(mst.m[rb], l_tot);
      }
    }
    if (nxt == kClaimLate) {
      if (tid == 0) s_late = resolve_ticket(P.hdr, s_qs, s_qc, q_cur, ticket);
      __syncthreads();
      nxt = __builtin_amdgcn_readfirstlane(s_late);
      if (nxt >= 0) nitem = load_item(P.items, nxt);
    }
    it = nxt;
    item = nitem;
  }
  };
  if (producer) run(Role<true>{});
  else run(Role<false>{});
  if (blockIdx.x == 0 && tid == 0) {
    P.hdr->clk_end = clock64();
    P.hdr->rt_end = wall_clock64();
  }
}


template <int D, int G, bool ROPE>
static hipError_t launch_one(const AttnParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, G, ROPE, kRB>), dim3((unsigned)grid), dim3(64 * kNW), 0, s, p);
  return hipGetLastError();
}

template <int D, bool ROPE>
static hipError_t launch_g(const AttnParams& p, int G, int grid, hipStream_t s) {
  switch (G) {
    case 1: return launch_one<D, 1, ROPE>(p, grid, s);
    case 2: return launch_one<D, 2, ROPE>(p, grid, s);
    case 4: return launch_one<D, 4, ROPE>(p, grid, s);
    case 8: return launch_one<D, 8, ROPE>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

// Query rows per work item and threads per work-group of the built kernels.
int attn_bf16_rows() { return 32 * kRB * kNC; }
int attn_bf16_threads() { return 64 * kNW; }

hipError_t launch_attn_bf16(const AttnParams& p, int D, int G, bool rope, int grid, hipStream_t s) {
  if (D == 128) return rope ? launch_g<128, true>(p, G, grid, s) : launch_g<128, false>(p, G, grid, s);
  if (D == 64) return rope ? launch_g<64, true>(p, G, grid, s) : launch_g<64, false>(p, G, grid, s);
  return hipErrorInvalidValue;
}

// Occupancy of one attention configuration (work-groups per CU), for sizing
// the persistent grid.
int attn_bf16_blocks_per_cu(int D, int G, bool rope) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
#define MINIPIC_OCC(DD, GG, RR)                                                                          \
  if (D == DD && G == GG && rope == RR)                                                                 \
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<DD, GG, RR, kRB>, 64 * kNW, 0);
  MINIPIC_OCC(128, 1, true) MINIPIC_OCC(128, 2, true) MINIPIC_OCC(128, 4, true) MINIPIC_OCC(128, 8, true)
  MINIPIC_OCC(128, 1, false) MINIPIC_OCC(128, 2, false) MINIPIC_OCC(128, 4, false) MINIPIC_OCC(128, 8, false)
  MINIPIC_OCC(64, 1, true) MINIPIC_OCC(64, 2, true) MINIPIC_OCC(64, 4, true) MINIPIC_OCC(64, 8, true)
  MINIPIC_OCC(64, 1, false) MINIPIC_OCC(64, 2, false) MINIPIC_OCC(64, 4, false) MINIPIC_OCC(64, 8, false)
#undef MINIPIC_OCC
  return (e == hipSuccess && n > 0) ? n : 1;
}

}  // namespace minipic
