// bf16 position-free paged prefill attention on gfx950 MFMA.
//
// "MiniPIC: Flexible Position-Independent Caching in <100LOC", §3.2.2: the
// kernel loads each K tile UNROTATED from the paged cache, looks up cos/sin
// at the keys' logical positions pi(j), rotates the tile, and only then takes
// its dot products with the already-rotated queries; V is used as stored.
// §3.2.1 gives the score (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d).
//
// Persistent kernel: about one work-group per CU; each work-group takes work
// items (q tile, KV head, piece of the tile's visible-block list) from an
// atomic counter until none are left.
//
// Layout of one item (one work-group = 8 waves = 256 query rows):
//   * rows = BQ query tokens x G query heads sharing KV head g (G = Hq/Hkv);
//     wave w owns rows 32w .. 32w+31, one row per lane pair (l, l+32).
//   * key tiles of 64 keys = 4 cache blocks from the tile's block list.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: keys on the M side, queries on
//     the N side, so lane l holds 16 keys of ONE query per 32x32 block and the
//     row max / row sum stay inside the lane (plus one exchange with l^32).
//   * K rows are written to LDS in a permuted order (bits 2 and 3 of the key
//     index swapped) so that the accumulator of lane l, element i, is key
//     16(i/8) + 8(l/32) + i%8 of the 32-key block; eight consecutive
//     accumulator elements then form exactly the bf16x8 B operand of the PV
//     MFMA O^T += V^T P^T, with no data movement.
//   * V is cached transposed inside each block ([d][16]), so the V^T A operand
//     is one 16-byte LDS read of 8 consecutive keys.
//   * The rotation (rotate-half pairing i <-> i + d/2) is applied once per
//     work-group per tile, in registers between the global load and the LDS
//     store, and the next tile's loads are in flight during the current
//     tile's MFMAs (two LDS buffers, one barrier per tile).
//   * Online softmax in log2 units with a lazily updated running max: the
//     accumulators are rescaled only when a row max grows by more than 2^8,
//     which is exact (numerator and denominator share the stale max).
//   * A tile whose list was cut into pieces: every piece stores (O, m, l) in
//     fp32 to its slot; merge_kernel combines them afterwards.
#include "common.h"

namespace minipic {

constexpr int kNT = 512;          // threads per work-group
constexpr int kRows = 256;        // query rows per work-group
constexpr int kKT = 64;           // keys per tile
constexpr int kListMax = 512;     // list entries staged in LDS at a time

template <int D>
struct Lds {
  static constexpr int KSTR = D + 8;     // bf16 elements per K row (16-byte pad)
  static constexpr int VSTR = kKT + 8;   // bf16 elements per V^T row
  static constexpr int KSZ = kKT * KSTR;
  static constexpr int VSZ = D * VSTR;
};

__device__ __forceinline__ int key_perm(int k) {
  // swap bits 2 and 3 (an involution); bits 0, 1, 4, 5 unchanged
  return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D, bool ROPE>
struct Stage {
  static constexpr int KUNITS = kKT * (D / 16);       // (key, chunk pair)
  static constexpr int KU = (KUNITS + kNT - 1) / kNT;
  static constexpr int VUNITS = 4 * D * 2;            // (block, d row, half)
  static constexpr int VU = VUNITS / kNT;
  u32x4 ka[KU], kb[KU];
  f32x4 c0[KU], c1[KU], s0[KU], s1[KU];
  u32x4 v[VU];
};

template <int D, int G, bool ROPE>
__global__ void __launch_bounds__(kNT, 1) attn_bf16_kernel(AttnParams P) {
  constexpr int BQ = kRows / G;
  using L = Lds<D>;
  using St = Stage<D, ROPE>;
  __shared__ BlkDesc lst[kListMax];
  __shared__ int s_next;
  __shared__ __attribute__((aligned(16))) __bf16 kl[2 * L::KSZ];
  __shared__ __attribute__((aligned(16))) __bf16 vl[2 * L::VSZ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int row = 32 * w + l32;   // this lane's query row within the item
  const int tok = row / G;
  const int hig = row % G;

  const __bf16* kc = (const __bf16*)P.k_cache;
  const __bf16* vc = (const __bf16*)P.v_cache;
  const float sl2 = P.scale_log2;
  int it = next_item(P.hdr, &s_next);
  while (it >= 0) {
    if (tid == 0) s_next = claim_item(P.hdr);  // the following item
    const Item item = P.items[it];
    const int g = item.gsn & 0xff;
    const int sp = (item.gsn >> 8) & 0xfff;
    const int ns = item.gsn >> 20;
    const TileDesc td = P.tiles[item.tile];
    const TokDesc tk = P.toks[(int64_t)item.tile * BQ + tok];
    const bool rvalid = tok < td.nq && tk.c >= 0;
    const int c_row = rvalid ? tk.c : -1;
    const int bq_row = rvalid ? (c_row >> 4) : -1;
    const int span_row = tk.span;
    const bool pdep_row = rvalid && tk.pdep;
    const int head = g * G + hig;
    const int64_t qrow = (int64_t)td.row0 + tok;
    const int32_t* lpos = P.logical_pos + (int64_t)td.r * P.max_blocks * kBlock;
    const BlkDesc* blist = P.blist + (int64_t)item.tile * P.max_blocks;

    // ---- this lane's query row (B operand of S^T = K Q^T)
    bf16x8 qf[D / 16];
    {
      const __bf16* qp = (const __bf16*)P.q + (qrow * P.hq + head) * D;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        if (rvalid) qf[ks] = *(const bf16x8*)(qp + 16 * ks + 8 * h);
        else qf[ks] = bf16x8{};
      }
      if ((P.flags & MINIPIC_FLAG_ROTATE_Q) && rvalid) {
        int pos = lpos[c_row];
        if (pos < 0 || pos >= P.max_pos) {
          atomicOr(&P.hdr->err, (uint32_t)MINIPIC_EW_POS);
          pos = pos < 0 ? 0 : P.max_pos - 1;
        }
        const float* cs = P.cos_sin + (int64_t)pos * D;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const u32x4 a = __builtin_bit_cast(u32x4, qf[ks]);
          const u32x4 b = __builtin_bit_cast(u32x4, qf[ks + D / 32]);
          u32x4 ra, rb;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i0 = 16 * ks + 8 * h + 2 * j;
            const float c_0 = cs[i0], c_1 = cs[i0 + 1];
            const float s_0 = cs[D / 2 + i0], s_1 = cs[D / 2 + i0 + 1];
            const float a0 = bf16_lo(a[j]), a1 = bf16_hi(a[j]);
            const float b0 = bf16_lo(b[j]), b1 = bf16_hi(b[j]);
            ra[j] = pack_bf16x2(a0 * c_0 - b0 * s_0, a1 * c_1 - b1 * s_1);
            rb[j] = pack_bf16x2(b0 * c_0 + a0 * s_0, b1 * c_1 + a1 * s_1);
          }
          qf[ks] = __builtin_bit_cast(bf16x8, ra);
          qf[ks + D / 32] = __builtin_bit_cast(bf16x8, rb);
        }
      }
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
    float m_run = -INFINITY;   // running max of scaled scores (log2 units)
    float l_run = 0.f;         // this half-lane's share of the row sum

    for (int c0 = item.p0; c0 < item.p1; c0 += kListMax) {
      const int n_l = min(kListMax, item.p1 - c0);
      for (int i = tid; i < n_l; i += kNT) lst[i] = blist[c0 + i];
      __syncthreads();
      const int ntiles = (n_l + 3) / 4;

      auto load = [&](int ti, St& st) {
#pragma unroll
        for (int u = 0; u < St::KU; ++u) {
          const int unit = tid + u * kNT;
          st.ka[u] = u32x4{}; st.kb[u] = u32x4{};
          if (ROPE) { st.c0[u] = f32x4{}; st.c1[u] = f32x4{}; st.s0[u] = f32x4{}; st.s1[u] = f32x4{}; }
          if (unit < St::KUNITS) {
            const int key = unit / (D / 16);
            const int cp = unit % (D / 16);
            const int e = 4 * ti + key / kBlock;
            const int off = key % kBlock;
            const int ph = e < n_l ? lst[e].phys : -1;
            if (ph >= 0) {
              const __bf16* kr = kc + (((int64_t)ph * P.hkv + g) * kBlock + off) * D;
              st.ka[u] = *(const u32x4*)(kr + 8 * cp);
              st.kb[u] = *(const u32x4*)(kr + D / 2 + 8 * cp);
              if (ROPE) {
                const int pos0 = lst[e].pos0;
                int pos = pos0 >= 0 ? pos0 + off : lpos[lst[e].kb * kBlock + off];
                if (pos < 0 || pos >= P.max_pos) {
                  atomicOr(&P.hdr->err, (uint32_t)MINIPIC_EW_POS);
                  pos = pos < 0 ? 0 : P.max_pos - 1;
                }
                const float* cs = P.cos_sin + (int64_t)pos * D + 8 * cp;
                st.c0[u] = *(const f32x4*)(cs);
                st.c1[u] = *(const f32x4*)(cs + 4);
                st.s0[u] = *(const f32x4*)(cs + D / 2);
                st.s1[u] = *(const f32x4*)(cs + D / 2 + 4);
              }
            }
          }
        }
#pragma unroll
        for (int u = 0; u < St::VU; ++u) {
          const int unit = tid + u * kNT;
          const int b = unit / (2 * D);
          const int rem = unit % (2 * D);
          const int e = 4 * ti + b;
          const int ph = e < n_l ? lst[e].phys : -1;
          st.v[u] = u32x4{};
          if (ph >= 0)
            st.v[u] = *(const u32x4*)(vc + (((int64_t)ph * P.hkv + g) * D + rem / 2) * kBlock + 8 * (rem % 2));
        }
      };

      auto store = [&](int buf, const St& st) {
        __bf16* kb_ = kl + buf * L::KSZ;
        __bf16* vb_ = vl + buf * L::VSZ;
#pragma unroll
        for (int u = 0; u < St::KU; ++u) {
          const int unit = tid + u * kNT;
          if (unit < St::KUNITS) {
            const int key = unit / (D / 16);
            const int cp = unit % (D / 16);
            u32x4 ra = st.ka[u], rb = st.kb[u];
            if (ROPE) {
              const float cc[8] = {st.c0[u][0], st.c0[u][1], st.c0[u][2], st.c0[u][3],
                                   st.c1[u][0], st.c1[u][1], st.c1[u][2], st.c1[u][3]};
              const float ss[8] = {st.s0[u][0], st.s0[u][1], st.s0[u][2], st.s0[u][3],
                                   st.s1[u][0], st.s1[u][1], st.s1[u][2], st.s1[u][3]};
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float a0 = bf16_lo(st.ka[u][j]), a1 = bf16_hi(st.ka[u][j]);
                const float b0 = bf16_lo(st.kb[u][j]), b1 = bf16_hi(st.kb[u][j]);
                const float c_0 = cc[2 * j], c_1 = cc[2 * j + 1];
                const float s_0 = ss[2 * j], s_1 = ss[2 * j + 1];
                ra[j] = pack_bf16x2(a0 * c_0 - b0 * s_0, a1 * c_1 - b1 * s_1);
                rb[j] = pack_bf16x2(b0 * c_0 + a0 * s_0, b1 * c_1 + a1 * s_1);
              }
            }
            __bf16* dst = kb_ + key_perm(key) * L::KSTR + 8 * cp;
            *(u32x4*)dst = ra;
            *(u32x4*)(dst + D / 2) = rb;
          }
        }
#pragma unroll
        for (int u = 0; u < St::VU; ++u) {
          const int unit = tid + u * kNT;
          const int b = unit / (2 * D);
          const int rem = unit % (2 * D);
          *(u32x4*)(vb_ + (rem / 2) * L::VSTR + kBlock * b + 8 * (rem % 2)) = st.v[u];
        }
      };

      St st;
      load(0, st);
      store(0, st);
      __syncthreads();
      for (int ti = 0; ti < ntiles; ++ti) {
        const int buf = ti & 1;
        const bool more = ti + 1 < ntiles;
        if (more) load(ti + 1, st);

        // ---- S^T = K Q^T for the 64-key tile
        const __bf16* kb_ = kl + buf * L::KSZ;
        f32x16 sacc[2];
#pragma unroll
        for (int kb32 = 0; kb32 < 2; ++kb32) {
          sacc[kb32] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 a = *(const bf16x8*)(kb_ + (32 * kb32 + l32) * L::KSTR + 16 * ks + 8 * h);
            sacc[kb32] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kb32], 0, 0, 0);
          }
        }

        // ---- block mask (block-granular + causal diagonal)
        bool vis[4];
        int lim[4];
        bool full = true;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int e = 4 * ti + b;
          const bool ev = e < n_l;
          const BlkDesc bd = ev ? lst[e] : BlkDesc{0, -1, 0, 0, -1, 0, 0, 0};
          vis[b] = ev && rvalid && block_visible(bd.kb, bd.span, bd.flags, bq_row, span_row, pdep_row);
          lim[b] = c_row - bd.kb * kBlock - 8 * h;
          full = full && vis[b] && lim[b] >= 7;
        }
        if (!__all(full)) {
#pragma unroll
          for (int kb32 = 0; kb32 < 2; ++kb32)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int b = 2 * kb32 + i / 8;
              if (!(vis[b] && (i % 8) <= lim[b])) sacc[kb32][i] = -INFINITY;
            }
        }

        // ---- online softmax (log2 units, lazy rescale)
        float mx = sacc[0][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[0][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[1][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float ms = mx * sl2;
        if (__any(ms > m_run + 8.0f)) {
          const float m_new = fmaxf(m_run, ms);
          const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
#pragma unroll
          for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dg][i] *= alpha;
          l_run *= alpha;
          m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        bf16x8 pk[2][2];
#pragma unroll
        for (int kb32 = 0; kb32 < 2; ++kb32)
#pragma unroll
          for (int sh = 0; sh < 2; ++sh) {
            u32x4 u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb32][8 * sh + 2 * j], sl2, -m_use));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb32][8 * sh + 2 * j + 1], sl2, -m_use));
              u[j] = pack_bf16x2(p0, p1);
              l_run += p0 + p1;
            }
            pk[kb32][sh] = __builtin_bit_cast(bf16x8, u);
          }

        // ---- O^T += V^T P^T
        const __bf16* vb_ = vl + buf * L::VSZ;
#pragma unroll
        for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
          for (int kb32 = 0; kb32 < 2; ++kb32)
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
              const bf16x8 a = *(const bf16x8*)(vb_ + (32 * dg + l32) * L::VSTR + 32 * kb32 + 16 * sh + 8 * h);
              o[dg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kb32][sh], o[dg], 0, 0, 0);
            }

        if (more) store(buf ^ 1, st);
        __syncthreads();
      }
    }

    // ---- epilogue
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    __bf16* op = (__bf16*)P.out + (qrow * P.hq + head) * D;
    if (ns == 1) {
      if (rvalid) {
        const float inv = 1.f / l_tot;
#pragma unroll
        for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            u32x2 u;
            u[0] = pack_bf16x2(o[dg][4 * j] * inv, o[dg][4 * j + 1] * inv);
            u[1] = pack_bf16x2(o[dg][4 * j + 2] * inv, o[dg][4 * j + 3] * inv);
            *(u32x2*)(op + 32 * dg + 8 * j + 4 * h) = u;
          }
      }
    } else if (rvalid) {
      // a piece of a split tile: fp32 partial result to its slot (merged by merge_kernel)
      const int64_t pr = (int64_t)(td.slot0 + g * ns + sp) * kRows + row;
      float* po = P.part_o + pr * D;
#pragma unroll
      for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 u = {o[dg][4 * j], o[dg][4 * j + 1], o[dg][4 * j + 2], o[dg][4 * j + 3]};
          *(f32x4*)(po + 32 * dg + 8 * j + 4 * h) = u;
        }
      if (h == 0) P.part_ml[pr] = make_float2(m_run, l_tot);
    }
    __syncthreads();
    it = __builtin_amdgcn_readfirstlane(s_next);
    __syncthreads();
  }
}

template <int D, int G, bool ROPE>
static hipError_t launch_one(const AttnParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, G, ROPE>), dim3((unsigned)grid), dim3(kNT), 0, s, p);
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
#define MINIPIC_OCC(DD, GG, RR)                                                                   \
  if (D == DD && G == GG && rope == RR)                                                          \
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<DD, GG, RR>, kNT, 0);
  MINIPIC_OCC(128, 1, true) MINIPIC_OCC(128, 2, true) MINIPIC_OCC(128, 4, true) MINIPIC_OCC(128, 8, true)
  MINIPIC_OCC(128, 1, false) MINIPIC_OCC(128, 2, false) MINIPIC_OCC(128, 4, false) MINIPIC_OCC(128, 8, false)
  MINIPIC_OCC(64, 1, true) MINIPIC_OCC(64, 2, true) MINIPIC_OCC(64, 4, true) MINIPIC_OCC(64, 8, true)
  MINIPIC_OCC(64, 1, false) MINIPIC_OCC(64, 2, false) MINIPIC_OCC(64, 4, false) MINIPIC_OCC(64, 8, false)
#undef MINIPIC_OCC
  return (e == hipSuccess && n > 0) ? n : 1;
}

}  // namespace minipic
