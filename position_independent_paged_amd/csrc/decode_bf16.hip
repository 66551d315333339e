// Decode-phase position-free paged attention (gfx950): one query token per
// request attends to its request's visible keys, with the key rotation done
// in-kernel from the unrotated cache ("MiniPIC: Flexible Position-Independent
// Caching in <100LOC", §3.2.1 score equation and §3.2.2 rotation of each K
// tile after a cos/sin lookup at pi(j); the visibility rule of §3.1.1 /
// §3.3.1 as restated in common.h). A generated token belongs to the PDep
// segment that follows the spans, so it usually sees every earlier key; the
// kernel applies the general rule from the query's block descriptors.
//
// Decode reads every visible K/V block once per KV head for a single query
// row: it is bound by HBM bandwidth, not by the MFMA. Work split:
//   * one wave per (request r, KV head g, split s): the split covers a
//     contiguous run of the request's key blocks (host-chosen length);
//     invisible blocks are skipped before any K/V load;
//   * per 16-key block: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with keys on
//     M and the G query heads of KV head g on N (columns >= G are zero), after
//     rotating K in fp32 in registers (lane (key, slice j) holds the rotate-half
//     pairs d and d + D/2 of its slice); P = exp2(S * scale log2 e - m) with a
//     lazily raised running max; O^T += V^T P^T on v_mfma_f32_16x16x16bf16_1k,
//     whose B operand layout is the S accumulator's, and whose A operand is an
//     8-byte read of the [d][16] V block;
//   * the block table, span ids and flags are read through the scalar cache
//     (the block index is wave-uniform; a PDep query, the usual decode case,
//     sees every block up to its own and skips the scan), and each block's
//     cos/sin rows are requested before the next block's K/V: the waits for a
//     block's data never wait for the following block's loads, so one block
//     stays in flight behind the one being computed. The K/V and position
//     loads are buffer loads issued on every path (a descriptor without
//     records reads zeros with no memory request past the split or for an
//     invalid block): a load issued on one path only would make the
//     compiler's wait at the join count it and wait for everything;
//   * every wave writes its (O, m, l) partial (m in log2 units); a merge
//     kernel combines the splits of a (request, query head) in split order.
#include "common.h"

namespace minipic {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer resource on gfx9 (32-bit data, no swizzle, no
// index stride). A load at an offset past num_records returns zeros and
// sends no request to memory.
constexpr int kBufWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufWord3);
}

template <int D, int G, bool ROPE>
__global__ void __launch_bounds__(64) decode_bf16_kernel(DecodeParams P) {
  static_assert(G >= 1 && G <= 16, "query heads per KV head fit the 16 MFMA columns");
  constexpr int NC = D / 32;     // 32-wide d chunks of the QK MFMA
  constexpr int NH = D / 64;     // chunks in each rotate-half
  constexpr int NM = D / 16;     // 16-row d blocks of the PV MFMA
  const int l = threadIdx.x;
  const int n = l & 15;          // MFMA column: query head n of this KV head / key row of K
  const int j = l >> 4;          // lane group: d slice 8j..8j+7 of a chunk (QK), keys 4j..4j+3 (S, PV)
  // Wave u runs on XCD u mod 8. The KV heads of one (request, split) are
  // numbered so that they run on one XCD at about the same time and share
  // the cos/sin rows of their keys in its L2: u = ((rs / 8) Hkv + g) 8 + rs mod 8.
  const int u = blockIdx.x;
  const int rs = (u / (kQueues * P.hkv)) * kQueues + u % kQueues;
  if (rs >= P.num_reqs * P.nsplit) return;   // padding of the last group of 8
  const int g = (u / kQueues) % P.hkv;
  const int s = rs % P.nsplit;
  const int r = rs / P.nsplit;
  const int64_t pslot = ((int64_t)(r * P.hkv + g) * P.nsplit + s) * G;

  // ---- the query's context index, block and descriptors (wave-uniform)
  const int Lmax = P.max_blocks * kBlock;
  int L = P.ctx_len[r];
  if (L > Lmax || L < 0) {
    if (l == 0 && s == 0 && g == 0) atomicOr(P.err, (uint32_t)MINIPIC_EW_CTX);
    L = L < 0 ? 0 : Lmax;
  }
  int c = P.q_ctx_idx[r];
  if (c < 0 || c >= L) {
    if (l == 0 && s == 0 && g == 0) atomicOr(P.err, (uint32_t)MINIPIC_EW_QCTX);
    c = c < 0 ? 0 : L - 1;
  }
  const int32_t* span = P.span_id + (int64_t)r * P.max_blocks;
  const uint8_t* flg = P.blk_flags + (int64_t)r * P.max_blocks;
  const int32_t* btab = P.block_table + (int64_t)r * P.max_blocks;
  const int32_t* lpos = P.logical_pos + (int64_t)r * Lmax;
  const int bq = c >> 4;
  const int b0 = s * P.split_blocks;
  const int b1 = min(bq + 1, b0 + P.split_blocks);
  float m_run = -INFINITY;       // running max of this lane's head (log2 units)
  float l_run = 0.f;             // this lane's share of the row sum (keys 4j..4j+3 of each block)
  f32x4 o[NM];
#pragma unroll
  for (int i = 0; i < NM; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (L > 0 && b0 < b1) {
    const int span_q = span[bq];
    const bool pdep_q = (flg[bq] & MINIPIC_BLK_PDEP) != 0;
    // first block of the query's span run (the span test compares runs; a
    // block with the query's span id before it breaks the span-id contract)
    int lo_q = 0;
    if (!pdep_q) {
      int base = bq;
      while (true) {
        const int b2 = base - 1 - l;
        const uint64_t sb = __ballot(b2 < 0 || span[b2] != span_q);
        if (sb) {
          lo_q = base - (__ffsll((unsigned long long)sb) - 1);
          break;
        }
        base -= 64;
      }
    }
    // Q^T operand: lane (n, j) holds d = 32 t + 8 j + [0, 8) of query head g G + n
    bf16x8 qf[NC];
    {
      const bool hv = n < G;
      const __bf16* qp = (const __bf16*)P.q + ((int64_t)r * P.hq + g * G + (hv ? n : 0)) * D + 8 * j;
#pragma unroll
      for (int t = 0; t < NC; ++t) qf[t] = hv ? *(const bf16x8*)(qp + 32 * t) : bf16x8{};
    }
    const int64_t group = (int64_t)P.hkv * kBlock * D;
    const __bf16* kc = (const __bf16*)P.k_cache + (int64_t)g * kBlock * D;
    const __bf16* vc = (const __bf16*)P.v_cache + (int64_t)g * kBlock * D;
    const float sl2 = P.scale_log2;
    // rotation by this lane's key offset n within a block: cos(n theta_i),
    // sin(n theta_i) for the lane's first-half elements i (rows n of the table)
    float cd[ROPE ? NH * 8 : 1], sd[ROPE ? NH * 8 : 1];
    const bool delta_ok = ROPE && P.max_pos >= kBlock;
    if (delta_ok) {
      const float* cs = P.cos_sin + (int64_t)n * D + 8 * j;
#pragma unroll
      for (int t = 0; t < NH; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          cd[8 * t + e] = cs[32 * t + e];
          sd[8 * t + e] = cs[D / 2 + 32 * t + e];
        }
    }
    // Block descriptors through the scalar cache: the block index is uniform,
    // and scalar loads leave the vector memory counter, which paces the K/V
    // stream, alone.
    typedef const __attribute__((address_space(4))) int32_t CI;
    auto span_at = [&](int b) { return ((const CI*)span)[b]; };
    auto flg_at = [&](int b) {
      const uintptr_t a = (uintptr_t)(flg + b);
      return (int)((((const CI*)(a & ~(uintptr_t)3))[0] >> (8 * (a & 3))) & 0xff);
    };
    // the next block of the split the query sees, or b1
    auto next_visible = [&](int b) {
      b = __builtin_amdgcn_readfirstlane(b);
      if (pdep_q) return b;   // a PDep query sees every block up to its own
      bool broken = false;
      for (; b < b1; ++b) {
        const bool glob = (flg_at(b) & MINIPIC_BLK_GLOBAL) != 0;
        const bool same = span_at(b) == span_q;
        broken = broken || (!pdep_q && !glob && same && b < lo_q);
        if (pdep_q || glob || (same && b >= lo_q)) break;
      }
      if (broken && l == 0 && g == 0) atomicOr(P.err, (uint32_t)MINIPIC_EW_SPAN);
      return b;
    };
    // K rows: lane (n, j) = key n of the block, d slices 8 j of every chunk;
    // V^T operand: lane (n, j) = d row 16 mt + n, keys 4 j .. 4 j + 3; the
    // key's logical position. An invalid block reads as zeros.
    auto load_block = [&](int b, bf16x8 (&ka)[NC], s16x4 (&va)[NM], int& pos) {
      // Every load is issued, whatever the block: past the split or for an
      // invalid block the buffer descriptors have no records, the loads
      // read zeros without a memory request, and the waits for the next
      // block count the same loads on every path.
      const bool in = b < b1;
      int ph = in ? ((const CI*)btab)[b] : -1;
      if (in && (ph < 0 || (int64_t)ph >= P.num_blocks)) {
        if (l == 0) atomicOr(P.err, (uint32_t)MINIPIC_EW_BLOCK);
        ph = -1;
      }
      // a key past the context holds no token: its position is not read (the
      // lane then follows the block's run of positions, or reads row 0). It
      // is loaded first, so that waiting for it waits for no K/V load.
      if (ROPE) {
        const int live = __builtin_amdgcn_readfirstlane(in ? min(max(L - b * kBlock, 0), kBlock) : 0);
        const __amdgpu_buffer_rsrc_t rp = buf_rsrc(lpos + (live > 0 ? (int64_t)b * kBlock : 0), 4 * live);
        pos = __builtin_amdgcn_raw_buffer_load_b32(rp, 4 * n, 0, 0);
      } else {
        pos = 0;
      }
      ph = __builtin_amdgcn_readfirstlane(ph);   // uniform: the descriptors live in scalar registers
      const int64_t off = ph >= 0 ? (int64_t)ph * group : 0;
      const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kc + off, ph >= 0 ? kBlock * D * 2 : 0);
      const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vc + off, ph >= 0 ? kBlock * D * 2 : 0);
#pragma unroll
      for (int t = 0; t < NC; ++t)
        ka[t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, 2 * (n * D + 8 * j + 32 * t), 0, 0));
#pragma unroll
      for (int mt = 0; mt < NM; ++mt)
        va[mt] = __builtin_bit_cast(s16x4, __builtin_amdgcn_raw_buffer_load_b64(rv, 2 * (n * kBlock + 4 * j + 16 * mt * kBlock), 0, 0));
    };
    // one block in flight ahead of the one being computed
    bf16x8 ka_n[NC];
    s16x4 va_n[NM];
    int pos_n = 0;
    int b = next_visible(b0);
    load_block(b, ka_n, va_n, pos_n);
    while (b < b1) {
      bf16x8 ka[NC];
      s16x4 va[NM];
#pragma unroll
      for (int t = 0; t < NC; ++t) ka[t] = ka_n[t];
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) va[mt] = va_n[mt];
      int pos = pos_n;
      const int bc = b;
      // the cos/sin rows of this block are requested before the next block's
      // K/V, so that waiting for them never waits for the next block
      f32x4 cw[ROPE ? NH : 1][4];
      bool cons = false;
      if (ROPE) {
        const bool past = bc * kBlock + n >= L;   // lane 0 (key 0) never is
        if (!past && (pos < 0 || pos >= P.max_pos)) {
          atomicOr(P.err, (uint32_t)MINIPIC_EW_POS);
          pos = pos < 0 ? 0 : P.max_pos - 1;
        }
        // consecutive positions p0 .. p0+15 (the usual case): read only row
        // p0, shared by the block's 16 keys, and add the angle n theta_i;
        // otherwise read each key's own row
        const int p0 = __builtin_amdgcn_readfirstlane(pos);   // lane 0 holds key 0
        cons = delta_ok && __all(past || pos == p0 + n);
        const float* cs = P.cos_sin + (int64_t)(cons ? p0 : pos) * D + 8 * j;
#pragma unroll
        for (int t = 0; t < NH; ++t) {
          cw[t][0] = *(const f32x4*)(cs + 32 * t);
          cw[t][1] = *(const f32x4*)(cs + 32 * t + 4);
          cw[t][2] = *(const f32x4*)(cs + D / 2 + 32 * t);
          cw[t][3] = *(const f32x4*)(cs + D / 2 + 32 * t + 4);
        }
      }
      b = next_visible(b + 1);
      load_block(b, ka_n, va_n, pos_n);
      if (ROPE) {
        // rotate-half at the key's logical position: element i (first half)
        // with element i + D/2, in fp32, one rounding to bf16
#pragma unroll
        for (int t = 0; t < NH; ++t) {
          const f32x4 c0 = cw[t][0], c1 = cw[t][1], s0 = cw[t][2], s1 = cw[t][3];
          float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
          float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
          if (cons) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float cb = cv[e], sb = sv[e];
              cv[e] = cb * cd[8 * t + e] - sb * sd[8 * t + e];
              sv[e] = sb * cd[8 * t + e] + cb * sd[8 * t + e];
            }
          }
          const u32x4 ua = __builtin_bit_cast(u32x4, ka[t]);
          const u32x4 ub = __builtin_bit_cast(u32x4, ka[t + NH]);
          u32x4 ra, rb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a0 = bf16_lo(ua[e]), a1 = bf16_hi(ua[e]);
            const float x0 = bf16_lo(ub[e]), x1 = bf16_hi(ub[e]);
            const float c_0 = cv[2 * e], c_1 = cv[2 * e + 1], s_0 = sv[2 * e], s_1 = sv[2 * e + 1];
            ra[e] = pack_bf16x2(a0 * c_0 - x0 * s_0, a1 * c_1 - x1 * s_1);
            rb[e] = pack_bf16x2(x0 * c_0 + a0 * s_0, x1 * c_1 + a1 * s_1);
          }
          ka[t] = __builtin_bit_cast(bf16x8, ra);
          ka[t + NH] = __builtin_bit_cast(bf16x8, rb);
        }
      }
      // ---- S^T = K Q^T: acc[i] = score of key 4 j + i for head n
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NC; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t], qf[t], acc, 0, 0, 0);
      if (bc == bq) {   // causal diagonal: keys after the query
        const int lim = c - bq * kBlock - 4 * j;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i > lim) acc[i] = -INFINITY;
      }
      // ---- online softmax of head n over this block's 16 keys
      float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      mx *= sl2;
      if (__any(mx > m_run + 8.0f)) {   // lazy raise (exact: numerator and sum share the stale max)
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) o[mt] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(acc[i], sl2, -m_use));
      const uint32_t p01 = pack_bf16x2(p[0], p[1]), p23 = pack_bf16x2(p[2], p[3]);
      // the row sum of the bf16 values the numerator uses
      l_run += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
      const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{p01, p23});
      if (bc == bq) {
        // keys after the query: P is 0, and slots past the context may hold
        // anything (NaN) that 0 * V would still carry into O; zero them
        const int lim = c - bq * kBlock - 4 * j;
#pragma unroll
        for (int mt = 0; mt < NM; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i > lim) va[mt][i] = 0;
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[mt], pb, o[mt], 0, 0, 0);
    }
  }
  // ---- partial of this split: lane (n, j) holds O^T[d = 16 mt + 4 j + i][head n]
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (n < G) {
    float* po = P.part_o + (pslot + n) * D + 4 * j;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) *(f32x4*)(po + 16 * mt) = o[mt];
    if (j == 0) P.part_ml[pslot + n] = make_float2(m_run, l_run);
  }
}

// Merge of the splits of one (request, query head): O = sum_s 2^(m_s - m*) O_s /
// sum_s 2^(m_s - m*) l_s, m* = max_s m_s. One 256-thread work-group per
// (request, query head, slice of 32 E elements of d): E = D / 32 (whole
// rows) for batches of many requests, E = 1 where few (request, head) pairs
// would leave most of the GPU idle. The (m, l) pairs of the splits go to LDS
// in one pass; the first batch of partial outputs is requested right after
// them, so its latency passes while the max, the weights and the denominator
// are formed. The eight 32-lane groups sum splits g, g + 8, ... of the slice
// (E consecutive elements per lane, 32 / E splits in flight per lane), and
// the eight partial sums are added in group order.
template <int D, int E>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeParams P, int G) {
  constexpr int NDC = D / (32 * E);   // slices of d
  constexpr int UNR = 32 / E;         // splits per lane and batch
  __shared__ float2 ml_s[kDecodeMaxSplits];
  __shared__ float red[256 / 64][2];
  __shared__ float part[8][32 * E];
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int grp = tid >> 5, e = tid & 31;
  const int dc = blockIdx.x % NDC;
  const int h = (blockIdx.x / NDC) % P.hq;
  const int r = blockIdx.x / (NDC * P.hq);
  const int g = h / G, n = h % G;
  const int ns = P.nsplit;
  const int64_t base = (int64_t)(r * P.hkv + g) * ns * G + n;   // split s at base + s G
  float mloc = -INFINITY;
  for (int s = tid; s < ns; s += 256) {
    const float2 ml = P.part_ml[base + (int64_t)s * G];
    ml_s[s] = ml;
    mloc = fmaxf(mloc, ml.x);
  }
  const float* po = P.part_o + base * D + 32 * E * dc + E * e;
  float v[UNR][E];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int s = s0 + 8 * k;
#pragma unroll
      for (int i = 0; i < E; ++i) v[k][i] = s < ns ? po[(int64_t)s * G * D + i] : 0.f;
    }
  };
  load_batch(grp);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o, 64));
  if (l == 0) red[w][0] = mloc;
  __syncthreads();
  const float mstar = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
  float dloc = 0.f;
  for (int s = tid; s < ns; s += 256) {
    const float2 ml = ml_s[s];
    const float wt = ml.x == -INFINITY ? 0.f : exp2f(ml.x - mstar);
    ml_s[s].x = wt;
    dloc += wt * ml.y;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) dloc += __shfl_xor(dloc, o, 64);
  if (l == 0) red[w][1] = dloc;
  __syncthreads();
  const float den = (red[0][1] + red[1][1]) + (red[2][1] + red[3][1]);
  float num[E];
#pragma unroll
  for (int i = 0; i < E; ++i) num[i] = 0.f;
  for (int s0 = grp; s0 < ns; s0 += 8 * UNR) {
    if (s0 != grp) load_batch(s0);
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int s = s0 + 8 * k;
      const float wt = s < ns ? ml_s[s].x : 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) num[i] += wt * v[k][i];
    }
  }
#pragma unroll
  for (int i = 0; i < E; ++i) part[grp][E * e + i] = num[i];
  __syncthreads();
  for (int x = tid; x < 32 * E; x += 256) {
    float t = part[0][x];
#pragma unroll
    for (int k = 1; k < 8; ++k) t += part[k][x];
    ((__bf16*)P.out)[((int64_t)r * P.hq + h) * D + 32 * E * dc + x] = (__bf16)(t / den);
  }
}

template <int D, bool ROPE>
static hipError_t launch_dec_g(const DecodeParams& p, int G, hipStream_t s) {
  const int64_t groups = ((int64_t)p.num_reqs * p.nsplit + kQueues - 1) / kQueues;
  const dim3 grid((unsigned)(groups * kQueues * p.hkv));
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_bf16_kernel<D, 1, ROPE>), grid, dim3(64), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_bf16_kernel<D, 2, ROPE>), grid, dim3(64), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_bf16_kernel<D, 4, ROPE>), grid, dim3(64), 0, s, p); break;
    case 8: hipLaunchKernelGGL((decode_bf16_kernel<D, 8, ROPE>), grid, dim3(64), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeParams& p, int D, int G, bool rope, hipStream_t s) {
  if (D == 128) return rope ? launch_dec_g<128, true>(p, G, s) : launch_dec_g<128, false>(p, G, s);
  if (D == 64) return rope ? launch_dec_g<64, true>(p, G, s) : launch_dec_g<64, false>(p, G, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const DecodeParams& p, int D, int G, hipStream_t s) {
  // whole rows per work-group once the (request, head) pairs fill the GPU
  const int64_t heads = (int64_t)p.num_reqs * p.hq;
  const bool rows = heads >= 256;
  const dim3 grid((unsigned)(heads * (rows ? 1 : D / 32)));
  if (D == 128 && rows) hipLaunchKernelGGL((decode_merge_kernel<128, 4>), grid, dim3(256), 0, s, p, G);
  else if (D == 128) hipLaunchKernelGGL((decode_merge_kernel<128, 1>), grid, dim3(256), 0, s, p, G);
  else if (D == 64 && rows) hipLaunchKernelGGL((decode_merge_kernel<64, 2>), grid, dim3(256), 0, s, p, G);
  else if (D == 64) hipLaunchKernelGGL((decode_merge_kernel<64, 1>), grid, dim3(256), 0, s, p, G);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace minipic
